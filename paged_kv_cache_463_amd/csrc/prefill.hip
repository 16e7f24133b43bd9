// Chunked causal prefill over the paged cache on gfx950 matrix cores.
//
// The pages name the chunked-prefill switch only (page "vLLM推理引擎深度实战"
// §5.3); the attention itself is that of page "vLLM推理引擎深度解析" §五
// (scores q·k/sqrt(d) against the K rows the block table names, softmax,
// weighted sum of V). Reading implemented: sequence b's chunk holds its last
// q_len positions, query i sits at absolute position seq_len - q_len + i and
// sees keys 0 .. that position.
//
// Tiling (one workgroup of 4 waves, two workgroups per CU):
//   * a workgroup owns one (sequence, kv head) and 128 "columns" = (query
//     position, query head of the group) pairs: BQ = 128/G consecutive chunk
//     positions for all G heads of the group, so every K/V tile it stages is
//     shared by G heads. Wave w owns columns 32w .. 32w+31, one 32-wide MFMA
//     N-tile, which keeps its accumulators, scores and query operand within
//     half the register file (two waves per SIMD: one wave's softmax overlaps
//     the other's matrix work).
//   * keys advance in tiles of 64 (four 16-token blocks gathered through the
//     block table). K is staged in LDS row-major [key][d] (pitch D+8
//     elements), V transposed [d][key] (pitch 68 elements) so both MFMA
//     operands read contiguous 16-byte / 8-byte runs; the V thread mapping
//     makes the transposed writes bank-conflict free. Software pipeline: while
//     the VALU turns the scores of tile t into P, the matrix cores already
//     compute the scores of tile t+1; K runs one tile ahead of V through two
//     LDS buffers each, fetched into registers a tile ahead; one barrier per
//     tile.
//   * S^T = K Q^T on v_mfma_f32_32x32x16 (A = K rows from LDS, B = Q from
//     registers, loaded once). In this layout a lane holds 16 keys of ONE
//     query column, so the softmax max/sum are in-lane plus one exchange with
//     lane ^ 32.
//   * online softmax in log2 units with a per-column reference max that only
//     moves when a score exceeds it by more than 8; P is rounded to the input
//     type, summed for the normaliser from the rounded values (packed dot2
//     against ones), and fed as the B operand of O^T += V^T P^T. The key order
//     inside each 16-key MFMA step follows the S^T register order; the V^T
//     reads use the same order, so the contraction is unchanged.
//   * masking (only in tiles that reach the causal diagonal or the end of the
//     keys): keys past the causal limit get score -inf (select, never a
//     multiply), and V rows of keys outside [0, kend) are written to LDS as
//     zeros, so stale NaN in unused slots never meets P = 0. Columns past the
//     chunk's end carry a zero query and are never stored.
//   * XCD-aware order: workgroups of one (sequence, kv head) share its K/V
//     through L2, so they are placed on the same XCD (linear id i runs on XCD
//     i % 8); within a pair the tiles with the most keys start first.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kCols = 32 * kWaves;           // columns per workgroup
constexpr int kBK = 64;                      // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.0f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <DT dt> struct Mfma;
template <> struct Mfma<DT::BF16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x16 run(const vec& a, const vec& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
  }
  static __device__ __forceinline__ float sum2(uint32_t pk, float acc) {   // acc + lo + hi
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                          __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
  }
};
template <> struct Mfma<DT::F16> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x16 run(const vec& a, const vec& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
  }
  static __device__ __forceinline__ float sum2(uint32_t pk, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), __builtin_bit_cast(f16x2, 0x3C003C00u), acc,
                                  false);
  }
};

template <typename V>
__device__ __forceinline__ V as_vec(const u32x4& u) { return __builtin_bit_cast(V, u); }

}  // namespace

// F8: K and V come from an FP8 (e4m3) cache. Each wave then loads its block of
// the tile into registers with ordinary 16-byte loads (issued where the 16-bit
// path issues its direct global->LDS loads), widens the codes to the query
// type (exact) and writes them into LDS in the same swizzled 16-bit layout,
// so everything after the landing is shared with the 16-bit path. Inside the
// loop the widening runs under the second half of the tile's P.V products
// (the destination buffers are free by then, and the loads have had the
// score phase to land), not before the barrier. k_scale[g] joins the score
// scale and v_scale[g] the output.
template <DT dt, int D, int G, bool F8>
__global__ __launch_bounds__(64 * kWaves, 2)
void prefill_kernel(PrefillParams p, int tiles_per_pair, int xcd_mapped, const float* k_scale,
                    const float* v_scale) {
  using M = Mfma<dt>;
  using vec = typename M::vec;
  constexpr int BQ = kCols / G;              // chunk positions per workgroup
  constexpr int CH = D * 2 / 16;             // 16-byte chunks per K/V row
  constexpr int DS = D / 16;                 // MFMA k-steps over head_dim
  constexpr int MD = D / 32;                 // 32-row tiles of head_dim in O^T
  constexpr int RB = D * 2;                  // bytes of one K/V row in LDS (unpadded, swizzled)
  constexpr int NI = kBlockSize * RB / 1024; // 1 KB DMA instructions per wave per tile (4 or 2)
  constexpr int NL8 = D / 64;                // FP8: 16-byte loads per lane per block (2 or 1)
  constexpr int NPARTS = F8 ? 2 * NL8 : 2 * NI;   // load instructions per wave per tile

  // K and V tiles, row-major, two buffers each, filled by direct global->LDS
  // loads. 16-byte granule c of row r sits at position c ^ kswz(r) (K) or
  // c ^ vswz(r) (V), chosen (by bank-conflict counts) so that the 16-byte K
  // reads of 16 consecutive rows and the transposing 8-byte V reads of two
  // 16-lane groups over 4 consecutive rows hit distinct banks.
  __shared__ __attribute__((aligned(1024))) uint8_t sK[2][kBK * RB];
  __shared__ __attribute__((aligned(1024))) uint8_t sV[2][kBK * RB];

  // ---- which (sequence, kv head, tile) -----------------------------------
  const int npairs = p.num_seqs * p.num_kv_heads;
  int pair, tile;
  {
    const int lin = __builtin_amdgcn_workgroup_id_x();   // builtins: this unit is built with the
                                                        // IEEE bit off, which keeps library calls out of line
    if (xcd_mapped) {                        // all tiles of a pair on one XCD
      const int xcd = lin & 7, k = lin >> 3;
      pair = xcd + 8 * (k / tiles_per_pair);
      tile = tiles_per_pair - 1 - (k % tiles_per_pair);
    } else {
      pair = lin / tiles_per_pair;
      tile = tiles_per_pair - 1 - (lin % tiles_per_pair);
    }
  }
  if (pair >= npairs) return;
  const int b = pair / p.num_kv_heads;
  const int g = pair % p.num_kv_heads;
  // chunk rows stay inside [0, num_q_tokens) and a chunk never claims more
  // positions than the sequence has keys: both are preconditions, the clamps
  // only keep a violating call inside its buffers
  const int64_t nq = p.num_q_tokens;
  const int L = p.seq_lens[b];
  const int cu0 = (int)min((int64_t)max(p.cu_q_lens[b], 0), nq);
  const int qlen = min((int)min((int64_t)max(p.cu_q_lens[b + 1], cu0), nq) - cu0, max(L, 0));
  const int q0 = tile * BQ;                  // first chunk position of this workgroup
  if (q0 >= qlen || L <= 0) return;
  const int s0 = L - qlen;                   // absolute position of chunk position 0
  const int q1 = min(qlen, q0 + BQ);
  const int kend = p.causal ? min(L, s0 + q1) : L;   // keys [0, kend) can be visible
  const int nkt = (kend + kBK - 1) / kBK;
  const int nblk_valid = min((kend + kBlockSize - 1) / kBlockSize, p.block_table_stride);

  const int tid = __builtin_amdgcn_workitem_id_x();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;                  // which half of the 32x32 operand
  const int col = lane & 31;

  // ---- this lane's query column (one N-tile per wave) ---------------------
  const int cidx = wave * 32 + col;
  const int hl = cidx / BQ;
  const int qpos = q0 + cidx % BQ;
  const bool cvalid = qpos < qlen;
  const int pabs = cvalid ? s0 + qpos : -1;
  vec qreg[DS];
  {
    const char* qrow = static_cast<const char*>(p.query) +
                       (((int64_t)(cu0 + (cvalid ? qpos : 0)) * p.num_q_heads + g * G + hl) * D) * 2;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4 u = cvalid ? load16(qrow + (ds * 16 + 8 * hi) * 2) : u32x4{0u, 0u, 0u, 0u};
      qreg[ds] = as_vec<vec>(u);
    }
  }

  // ---- tile loads: direct global -> LDS ----------------------------------
  // Wave w loads logical block 4t+w of tile t (16 keys): DMA instruction n of a
  // wave writes 1 KB at LDS offset 16w*RB + 1024n, 16 bytes per lane, and each
  // lane fetches the global granule whose swizzled position that is.
  // the table is read-only for the kernel's lifetime: read it through the
  // constant address space so the uniform lookups stay scalar loads
  const __attribute__((address_space(4))) int32_t* tbl =
      (const __attribute__((address_space(4))) int32_t*)(p.block_tables + (int64_t)b * p.block_table_stride);
  const char* kc = static_cast<const char*>(p.k_cache);
  const char* vc = static_cast<const char*>(p.v_cache);
  const int64_t prow = (int64_t)p.num_kv_heads * D * (F8 ? 1 : 2);   // bytes of one pool row (all kv heads)
  auto kswz = [](int r) { return RB == 256 ? (r & 15) : ((r >> 1) & 7); };
  auto vswz = [](int r) { return RB == 256 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
  uint32_t k_src[NI], v_src[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int r = (n * 1024 + 16 * lane) / RB;               // row inside the wave's block
    const int gp = lane % (RB / 16);                         // granule position inside the row
    const uint32_t row_off = (uint32_t)(r * prow + (int64_t)g * D * 2);
    k_src[n] = row_off + ((gp ^ kswz(r)) << 4);     // the swizzles use the row's low 4 bits only
    v_src[n] = row_off + ((gp ^ vswz(r)) << 4);
  }
  // FP8: lane l loads row l/4 of the wave's block, bytes (l%4)*D/4 .. +D/4 of
  // the head's row, as NL8 16-byte loads; load i holds elements e0 .. e0+15,
  // e0 = (l%4)*D/4 + 16i, which are 16-bit granules e0/8 and e0/8 + 1
  const int r8 = lane >> 2, q8 = lane & 3;
  uint32_t f8_src[NL8];
#pragma unroll
  for (int i = 0; i < NL8; ++i)
    f8_src[i] = (uint32_t)(r8 * prow + (int64_t)g * D + q8 * (D / 4) + 16 * i);
  u32x4 k8[NL8], v8[NL8];                    // FP8: this wave's loads of the tile in flight
  const uint8_t* pend_kd = nullptr;          // FP8: their LDS destinations
  const uint8_t* pend_vd = nullptr;
  // table entry of this wave's logical block in tile t (scalar: the index is
  // uniform), and the byte offset of its physical block; blocks past the
  // visible keys read block 0
  auto entry = [&](int t) -> int {
    return tbl[min(min(t, nkt - 1) * (kBK / kBlockSize) + wave, nblk_valid - 1)];
  };
  auto block_base = [&](int t, int bid) -> int64_t {
    const int blk = min(t, nkt - 1) * (kBK / kBlockSize) + wave;
    bid = (blk < nblk_valid && bid >= 0 && bid < p.num_blocks) ? bid : 0;
    return (int64_t)bid * p.block_stride_bytes;
  };
  // Blocks of tile t (bit k: logical block 4t+k) that hold visible keys but have
  // no valid table entry (an id outside the pool, or past the table's stride):
  // they are read as block 0, so their scores are masked and their V rows
  // zeroed, as for keys past the end. A precondition violation; this only
  // keeps other sequences' rows out of the result.
  auto tile_bad = [&](int t) -> int {
    int bad = 0;
#pragma unroll
    for (int k = 0; k < kBK / kBlockSize; ++k) {
      const int blk = t * (kBK / kBlockSize) + k;
      if (blk * kBlockSize < kend) {
        const int bid = blk < p.block_table_stride ? tbl[blk] : -1;
        if (bid < 0 || bid >= p.num_blocks) bad |= 1 << k;
      }
    }
    return bad;
  };
  // One direct global -> LDS load of 16 bytes per lane: M0 holds the LDS
  // destination of lane 0 (lane i writes 16 bytes further per lane), the
  // global address is a scalar block base plus a 32-bit lane offset. Issued as
  // inline assembly: the completion of these loads is waited for explicitly
  // (s_waitcnt vmcnt(0) and a barrier, once per tile), and the buffers read
  // while they are in flight are never their destinations.
  auto lds_load16 = [&](const char* base, uint32_t off, const uint8_t* lds_dst) {
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) uint8_t*)lds_dst);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(m0), "v"(off), "s"(base) : "memory", "m0");
  };
  // the loads of K tile tk (table entry kbid) into sK[kb] and V tile tv
  // (entry vbid) into sV[vb]: 2*NI instructions, issued one at a time by
  // dma_part (a burst of them stalls the wave behind the address unit); tiles
  // past the end re-read the last tile, so every wave issues the same loads
  struct DmaJob { const char* ks; const char* vs; const uint8_t* kd; const uint8_t* vd; };
  auto dma_job = [&](int tk, int kbid, int kb, int tv, int vbid, int vb) -> DmaJob {
    return {kc + block_base(tk, kbid), vc + block_base(tv, vbid), &sK[kb][wave * kBlockSize * RB],
            &sV[vb][wave * kBlockSize * RB]};
  };
  // this wave's block of V tile tv is a valid pool block (else its rows are zeroed on landing)
  auto v_ok = [&](int tv, int vbid) -> bool {
    const int blk = min(tv, nkt - 1) * (kBK / kBlockSize) + wave;
    return blk >= p.block_table_stride || blk * kBlockSize >= kend || (vbid >= 0 && vbid < p.num_blocks);
  };
  auto dma_part = [&](const DmaJob& j, int n) {      // n in [0, NPARTS)
    if constexpr (F8) {
      if (n == 0) {
        pend_kd = j.kd;
        pend_vd = j.vd;
      }
      if (n < NL8) k8[n] = load16(j.ks + f8_src[n]);
      else v8[n - NL8] = load16(j.vs + f8_src[n - NL8]);
    } else {
      if (n < NI) lds_load16(j.ks, k_src[n], j.kd + n * 1024);
      else lds_load16(j.vs, v_src[n - NI], j.vd + (n - NI) * 1024);
    }
  };
  auto dma = [&](int tk, int kbid, int kb, int tv, int vbid, int vb) {
    const DmaJob j = dma_job(tk, kbid, kb, tv, vbid, vb);
#pragma unroll
    for (int n = 0; n < NPARTS; ++n) dma_part(j, n);
  };
  // wait for this wave's loads; in the last V tile zero the rows of keys past
  // kend (stale slots) in this wave's block, and all rows of a block without a
  // valid table entry, then make everything visible
  // FP8: widen-and-write unit u (0 .. 4*NL8-1) of this wave's landed rows:
  // load u/4, K or V, first or second 16-bit granule pair
  auto widen_unit = [&](int u) {
    const int i = u >> 2, kv = (u >> 1) & 1, h = u & 1;
    const int g0 = (q8 * (D / 4) + 16 * i) / 8 + h;
    const u32x4 w = kv ? v8[i] : k8[i];
    uint8_t* dst = const_cast<uint8_t*>(kv ? pend_vd : pend_kd) + r8 * RB;
    const int sw = kv ? vswz(r8) : kswz(r8);
    *reinterpret_cast<u32x4*>(dst + ((g0 ^ sw) << 4)) = widen_fp8<dt>(u32x2{w[2 * h], w[2 * h + 1]});
  };
  auto land = [&](int tv, int vb, bool vok, bool widened = false) {
    if constexpr (F8) {                      // widen this wave's rows into the 16-bit layout
      if (!widened) {
#pragma unroll
        for (int u = 0; u < 4 * NL8; ++u) widen_unit(u);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const bool blk_ok = vok && tv * (kBK / kBlockSize) + wave < p.block_table_stride;
    if (tv < nkt && (tv * kBK + kBK > kend || !blk_ok)) {
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const int r = (n * 1024 + 16 * lane) / RB;
        if (tv * kBK + wave * kBlockSize + r >= kend || !blk_ok)
          *reinterpret_cast<u32x4*>(&sV[vb][wave * kBlockSize * RB + n * 1024 + 16 * lane]) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    __syncthreads();
  };

  // ---- accumulators --------------------------------------------------------
  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[md][r] = 0.f;
  float mref = -INFINITY;
  float lsum = 0.f;
  const float sl2 = p.scale * kLog2e * (F8 ? k_scale[g] : 1.f);

  // Software pipeline over key tiles: iteration t computes the scores of tile
  // t+1 on the matrix cores while the VALU turns the scores of tile t into P,
  // then accumulates P V of tile t. K runs one tile ahead of V in LDS: during
  // iteration t the wave reads K(t+1) and V(t) and the workgroup writes K(t+2)
  // and V(t+1) into the other two buffers; one barrier per tile.
  f32x16 sa[2], sb[2];                       // scores of two consecutive tiles
  dma(0, entry(0), 0, 0, entry(0), 0);
  // Does any block with visible keys lack a valid table entry? Checked once,
  // with vector loads that complete with the first tile's, so that only a
  // workgroup that has such a block pays the per-tile lookups of tile_bad.
  bool any_bad = (kend + kBlockSize - 1) / kBlockSize > p.block_table_stride;
  {
    int bad = 0;
    const int32_t* row = p.block_tables + (int64_t)b * p.block_table_stride;
    for (int i = lane; i < nblk_valid; i += 64) {
      const int bid = row[i];
      bad |= (bid < 0 || bid >= p.num_blocks);
    }
    any_bad = any_bad || __any(bad);
  }
  land(0, 0, v_ok(0, entry(0)));
  dma(1, entry(1), 1, nkt, entry(nkt), 1);    // K(1); the V part re-reads tile nkt-1 into sV[1]
  // table entries for the loads of the next iteration, read a tile ahead
  int kbid_next = entry(2), vbid_next = entry(1);
  int bad_cur = any_bad ? tile_bad(0) : 0;   // blocks of the scored tile without a valid entry
  {
    const uint8_t* K0 = sK[0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const f32x16 z = {};
      sa[kt] = z;
      const int r = kt * 32 + col;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        sa[kt] = M::run(as_vec<vec>(*reinterpret_cast<const u32x4*>(&K0[r * RB + (((2 * ds + hi) ^ kswz(r)) << 4)])),
                        qreg[ds], sa[kt]);
    }
  }
  land(nkt, 1, true);

  // one tile; sc holds the scores of tile t, sn receives those of tile t+1.
  // The loop below runs two tiles per trip with the two score arrays trading
  // roles, so no copy from sn to sc is needed.
  auto key_tile = [&](const int t, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    const int key0 = t * kBK;
    const DmaJob job = dma_job(t + 2, kbid_next, t & 1, t + 1, vbid_next, (t + 1) & 1);
    const bool vok_next = v_ok(t + 1, vbid_next);

    // scale; mask (uniform: only tiles that reach the causal diagonal or the
    // end of the keys); tile max of the column; rare rescale
    const bool edge = (key0 + kBK > kend) || (p.causal && key0 + kBK - 1 > s0 + q0);
    if (edge) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool vis = key < kend && (!p.causal || key <= pabs);
          sc[kt][r] = vis ? sc[kt][r] : -INFINITY;
        }
    }
    if (bad_cur) {                            // uniform and rare: blocks without a valid entry
#pragma unroll
      for (int k = 0; k < kBK / kBlockSize; ++k)
        if ((bad_cur >> k) & 1)               // block k of the tile = registers 8(k&1).. of half k>>1
#pragma unroll
          for (int r = 0; r < 8; ++r) sc[k >> 1][8 * (k & 1) + r] = -INFINITY;
    }
    // tile max of the column (raw scores, scale > 0) by a balanced tree of
    // 3-input maxima; rare rescale
    float tmax;
    {
      auto v = [&](int j) { return sc[j >> 4][j & 15]; };
      auto mx3 = [](float a, float b, float c) { return fmaxf(fmaxf(a, b), c); };
      float l1[11];
#pragma unroll
      for (int i = 0; i < 10; ++i) l1[i] = mx3(v(3 * i), v(3 * i + 1), v(3 * i + 2));
      l1[10] = fmaxf(v(30), v(31));
      tmax = fmaxf(mx3(mx3(l1[0], l1[1], l1[2]), mx3(l1[3], l1[4], l1[5]), mx3(l1[6], l1[7], l1[8])),
                   fmaxf(l1[9], l1[10]));
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * sl2;
    if (__any(tmax > mref + kSlack)) {
      const float mn = fmaxf(mref, tmax);
      const float corr = (mref == -INFINITY) ? 0.f : fast_exp2(mref - mn);
      lsum *= corr;
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[md][r] *= corr;
      mref = mn;
    }
    const float mu = (mref == -INFINITY) ? 0.f : mref;

    // P = 2^(s - m) rounded to the input type, normaliser from the rounded
    // values; pair pr (0..15) of this lane's scores is (kt, ss, e2).
    u32x4 pk[2][2];                           // [kt][16-key step]: packed P pairs
    auto make_p = [&](int pr) {
      const int kt = pr >> 3, ss = (pr >> 2) & 1, e2 = pr & 3;
      const float p0 = fast_exp2(fmaf(sc[kt][8 * ss + 2 * e2], sl2, -mu));
      const float p1 = fast_exp2(fmaf(sc[kt][8 * ss + 2 * e2 + 1], sl2, -mu));
      pk[kt][ss][e2] = M::pack(p0, p1);
      lsum = M::sum2(pk[kt][ss][e2], lsum);
    };
    // Scores of tile t+1 (matrix cores) interleaved with the P of keys 0..31
    // of tile t (VALU); the P of keys 32..63 is made during the first half of
    // the P.V products below, which only use keys 0..31, so both phases carry
    // vector work for the matrix cores to overlap. Step ds issues the two
    // MFMAs of k-step ds and its share of the pairs; a scheduling barrier
    // closes each step so the matrix and vector streams stay interleaved. The
    // last iteration computes scores it never uses (its buffer holds an older
    // tile).
    {
      constexpr int PPS = 8 / DS;             // pairs of keys 0..31 per k-step
      const uint8_t* Kn = sK[(t + 1) & 1];
      auto kfrag = [&](int kt, int ds) {
        const int r = kt * 32 + col;
        return as_vec<vec>(*reinterpret_cast<const u32x4*>(&Kn[r * RB + (((2 * ds + hi) ^ kswz(r)) << 4)]));
      };
      vec ka[2][2];
      ka[0][0] = kfrag(0, 0);
      ka[0][1] = kfrag(1, 0);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        if (ds + 1 < DS) {
          ka[(ds + 1) & 1][0] = kfrag(0, ds + 1);
          ka[(ds + 1) & 1][1] = kfrag(1, ds + 1);
        }
        // this tile's global -> LDS loads, spread over the k-steps
#pragma unroll
        for (int n = ds * NPARTS / DS; n < (ds + 1) * NPARTS / DS; ++n) dma_part(job, n);
        if (ds == 0) {
          const f32x16 z = {};
          sn[0] = M::run(ka[0][0], qreg[0], z);
          sn[1] = M::run(ka[0][1], qreg[0], z);
        } else {
          sn[0] = M::run(ka[ds & 1][0], qreg[ds], sn[0]);
          sn[1] = M::run(ka[ds & 1][1], qreg[ds], sn[1]);
        }
#pragma unroll
        for (int j = 0; j < PPS; ++j) make_p(ds * PPS + j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // O^T += V^T P^T over V(t). The A operand (32 head-dim rows x 16 keys) is
    // read from row-major V with two transposing 8-byte reads: in each group of
    // 16 lanes, lane 4j+q names key j of the read at columns 4q..4q+3 and lane
    // i receives column i of the 4 named keys. Read 0 covers keys 4h..4h+3 and
    // read 1 keys 8+4h..8+4h+3 of the 16-key step (h = lane / 32), which is the
    // key order of the P^T operand.
    {
      const uint8_t* Vc = sV[t & 1];
      const int vg = lane >> 4, vj = (lane >> 2) & 3, vq = lane & 3, vh = lane >> 5;
      auto vfrag = [&](int md, int kt, int ss) {
        const int d = md * 32 + 16 * (vg & 1) + 4 * vq;
        const int key0 = kt * 32 + 16 * ss + 4 * vh + vj;
        const int key1 = key0 + 8;
        const uint32_t gr = (uint32_t)(d >> 3), lo8 = (uint32_t)((d & 7) << 1);
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
        const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(Vc + key0 * RB + (((gr ^ vswz(key0)) << 4) | lo8)));
        const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(Vc + key1 * RB + (((gr ^ vswz(key1)) << 4) | lo8)));
        const u32x2 a0 = __builtin_bit_cast(u32x2, r0), a1 = __builtin_bit_cast(u32x2, r1);
        return as_vec<vec>(u32x4{a0[0], a0[1], a1[0], a1[1]});
      };
      // step i: key step ks = i / MD of the 64 keys, output tile md = i % MD, so
      // consecutive MFMAs accumulate into different tiles
      constexpr int NV = MD * 4;
      constexpr int PPV = 8 / (NV / 2);       // pairs of keys 32..63 per step of the first half
      auto vstep = [&](int i) { return vfrag(i % MD, (i / MD) >> 1, (i / MD) & 1); };
      vec va[3];
      va[0] = vstep(0);
      va[1] = vstep(1);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (i + 2 < NV) va[(i + 2) % 3] = vstep(i + 2);
        const int md = i % MD, ks = i / MD;
        if (i < NV / 2) {
#pragma unroll
          for (int j = 0; j < PPV; ++j) make_p(8 + i * PPV + j);
        }
        const vec pbk = as_vec<vec>(pk[ks >> 1][ks & 1]);
        o[md] = M::run(va[i % 3], pbk, o[md]);
        // FP8: the next tiles' rows (loaded during the scores above) are
        // widened into LDS under the second half of the products
        if constexpr (F8) {
          constexpr int U = 4 * NL8, H = NV / 2;
          if (i >= H) {
#pragma unroll
            for (int u = (i - H) * U / H; u < (i - H + 1) * U / H; ++u) widen_unit(u);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    kbid_next = entry(t + 3);                 // after this tile's LDS reads: the scalar
    vbid_next = entry(t + 2);                 // loads complete during the wait below
    bad_cur = (any_bad && t + 1 < nkt) ? tile_bad(t + 1) : 0;
    land(t + 1, (t + 1) & 1, vok_next, true);
  };
  int t = 0;
  for (; t + 1 < nkt; t += 2) {
    key_tile(t, sa, sb);
    key_tile(t + 1, sb, sa);
  }
  if (t < nkt) key_tile(t, sa, sb);

  // ---- normalise and store ------------------------------------------------
  const float l = lsum + __shfl_xor(lsum, 32);
  if (!cvalid) return;
  const float inv = (l > 0.f ? 1.f / l : 0.f) * (F8 ? v_scale[g] : 1.f);
  uint16_t* orow = static_cast<uint16_t*>(p.out) + ((int64_t)(cu0 + qpos) * p.num_q_heads + g * G + hl) * D;
#pragma unroll
  for (int md = 0; md < MD; ++md) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = md * 32 + 8 * j + 4 * hi;
      u32x2 pk;
      pk[0] = M::pack(o[md][4 * j] * inv, o[md][4 * j + 1] * inv);
      pk[1] = M::pack(o[md][4 * j + 2] * inv, o[md][4 * j + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + d) = pk;
    }
  }
}

template <DT dt, int D, bool F8>
static hipError_t launch_dg(const PrefillParams& p, const float* ks, const float* vs, hipStream_t s) {
  const int G = p.num_q_heads / p.num_kv_heads;
  const int BQ = kCols / G;
  const int tiles = (p.max_q_len + BQ - 1) / BQ;
  const int npairs = p.num_seqs * p.num_kv_heads;
  const int xcd = (npairs % 8 == 0) ? 1 : 0;
  const int64_t nwg = (int64_t)tiles * npairs;
  if (nwg <= 0) return hipSuccess;
  dim3 grid((unsigned)nwg), block(64 * kWaves);
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_kernel<dt, D, 1, F8>), grid, block, 0, s, p, tiles, xcd, ks, vs); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<dt, D, 2, F8>), grid, block, 0, s, p, tiles, xcd, ks, vs); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<dt, D, 4, F8>), grid, block, 0, s, p, tiles, xcd, ks, vs); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<dt, D, 8, F8>), grid, block, 0, s, p, tiles, xcd, ks, vs); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool F8>
static hipError_t launch_any(const PrefillParams& p, const float* ks, const float* vs, hipStream_t s) {
  const DT dt = static_cast<DT>(p.dtype);
  if (p.head_dim == 128) {
    if (dt == DT::BF16) return launch_dg<DT::BF16, 128, F8>(p, ks, vs, s);
    if (dt == DT::F16) return launch_dg<DT::F16, 128, F8>(p, ks, vs, s);
  } else if (p.head_dim == 64) {
    if (dt == DT::BF16) return launch_dg<DT::BF16, 64, F8>(p, ks, vs, s);
    if (dt == DT::F16) return launch_dg<DT::F16, 64, F8>(p, ks, vs, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) { return launch_any<false>(p, nullptr, nullptr, s); }
hipError_t launch_prefill_fp8(const PrefillParams& p, const float* k_scale, const float* v_scale, hipStream_t s) {
  return launch_any<true>(p, k_scale, v_scale, s);
}

}  // namespace pa
