// Chunked causal prefill over the paged cache on gfx950 matrix cores.
//
// The pages name the chunked-prefill switch only (page "vLLM推理引擎深度实战"
// §5.3); the attention itself is that of page "vLLM推理引擎深度解析" §五
// (scores q·k/sqrt(d) against the K rows the block table names, softmax,
// weighted sum of V). Reading implemented: sequence b's chunk holds its last
// q_len positions, query i sits at absolute position seq_len - q_len + i and
// sees keys 0 .. that position.
//
// Tiling (one workgroup of 4 waves):
//   * a workgroup owns one (sequence, kv head) and 256 "columns" = (query
//     position, query head of the group) pairs: BQ = 256/G consecutive chunk
//     positions for all G heads of the group, so every K/V tile it stages is
//     shared by G heads. Wave w owns columns 64w .. 64w+63 as two 32-column
//     N-tiles.
//   * keys advance in tiles of 64 (four 16-token blocks gathered through the
//     block table). K is staged in LDS row-major [key][d] (pitch D+8 elements),
//     V transposed [d][key] (pitch 68 elements) so both MFMA operands read
//     16-byte / 8-byte contiguous runs without bank conflicts on the K side.
//     Two LDS stages: tile t+1 is fetched into registers while tile t is
//     computed, then written to the other stage; one barrier per tile.
//   * S^T = K Q^T on v_mfma_f32_32x32x16 (A = K rows from LDS, B = Q from
//     registers, loaded once). In this layout a lane holds 16 keys of ONE
//     query column, so the softmax max/sum are in-lane plus one exchange with
//     lane ^ 32.
//   * online softmax in log2 units with a per-column reference max that only
//     moves when a score exceeds it by more than 8; P is rounded to the input
//     type and fed as the B operand of O^T += V^T P^T. The key order inside
//     each 16-key MFMA step follows the S^T register order; the V^T reads use
//     the same order, so the contraction is unchanged.
//   * masking: keys past the causal limit get score -inf (select, never a
//     multiply), and V rows of keys outside [0, kend) are written to LDS as
//     zeros, so stale NaN in unused slots never meets P = 0.
//   * XCD-aware order: workgroups of one (sequence, kv head) share its K/V
//     through L2, so they are placed on the same XCD (linear id i runs on XCD
//     i % 8); within a pair the tiles with the most keys start first.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kCols = 256;                   // columns per workgroup
constexpr int kBK = 64;                      // keys per tile
constexpr int kVtPitch = kBK + 4;            // V^T row pitch (elements)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.0f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <DT dt> struct Mfma;
template <> struct Mfma<DT::BF16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x16 run(const vec& a, const vec& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t bits(float x) { return to_bf16_bits(x); }
};
template <> struct Mfma<DT::F16> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x16 run(const vec& a, const vec& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t bits(float x) { return to_f16_bits(x); }
};

template <typename V>
__device__ __forceinline__ V as_vec(const u32x4& u) { return __builtin_bit_cast(V, u); }

}  // namespace

template <DT dt, int D, int G>
__global__ __launch_bounds__(64 * kWaves)
void prefill_kernel(PrefillParams p, int tiles_per_pair, int xcd_mapped) {
  using M = Mfma<dt>;
  using vec = typename M::vec;
  constexpr int BQ = kCols / G;              // chunk positions per workgroup
  constexpr int KPitch = D + 8;              // K row pitch (elements)
  constexpr int CH = D * 2 / 16;             // 16-byte chunks per K/V row
  constexpr int KPT = kBK * CH / (64 * kWaves);   // keys per thread per tile (2 or 4)
  constexpr int DS = D / 16;                 // MFMA k-steps over head_dim
  constexpr int MD = D / 32;                 // 32-row tiles of head_dim in O^T
  static_assert(KPT == 2 || KPT == 4, "tile mapping");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBK * KPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2][D * kVtPitch];

  // ---- which (sequence, kv head, tile) -----------------------------------
  const int npairs = p.num_seqs * p.num_kv_heads;
  int pair, tile;
  {
    const int lin = blockIdx.x;
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
  const int cu0 = p.cu_q_lens[b];
  const int qlen = p.cu_q_lens[b + 1] - cu0;
  const int L = p.seq_lens[b];
  const int q0 = tile * BQ;                  // first chunk position of this workgroup
  if (q0 >= qlen || L <= 0) return;
  const int s0 = L - qlen;                   // absolute position of chunk position 0
  const int q1 = min(qlen, q0 + BQ);
  const int kend = p.causal ? min(L, s0 + q1) : L;   // keys [0, kend) can be visible
  const int nkt = (kend + kBK - 1) / kBK;
  const int nblk_valid = min((kend + kBlockSize - 1) / kBlockSize, p.block_table_stride);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;                  // which half of the 32x32 operand
  const int col = lane & 31;

  // ---- this lane's query columns (two N-tiles) ---------------------------
  int qpos[2], pabs[2];
  bool cvalid[2];
  vec qreg[2][DS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int c = (2 * wave + nt) * 32 + col;
    const int hl = c / BQ;
    qpos[nt] = q0 + c % BQ;
    cvalid[nt] = qpos[nt] < qlen;
    pabs[nt] = cvalid[nt] ? s0 + qpos[nt] : -1;
    const char* qrow = static_cast<const char*>(p.query) +
                       (((int64_t)(cu0 + (cvalid[nt] ? qpos[nt] : 0)) * p.num_q_heads + g * G + hl) * D) * 2;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4 u = cvalid[nt] ? load16(qrow + (ds * 16 + 8 * hi) * 2) : u32x4{0u, 0u, 0u, 0u};
      qreg[nt][ds] = as_vec<vec>(u);
    }
  }

  // ---- cooperative tile fetch: thread -> (key group, 16-byte chunk) -------
  const int dchunk = tid % CH;
  const int kg = tid / CH;                   // keys kg*KPT .. kg*KPT+KPT-1 of the tile
  const int32_t* tbl = p.block_tables + (int64_t)b * p.block_table_stride;
  const char* kc = static_cast<const char*>(p.k_cache);
  const char* vc = static_cast<const char*>(p.v_cache);
  const int64_t row_bytes = (int64_t)p.num_kv_heads * D * 2;
  u32x4 kreg[KPT], vreg[KPT];

  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int key = t * kBK + kg * KPT + i;
      const int blk = key / kBlockSize;
      int bid = blk < nblk_valid ? tbl[blk] : 0;
      bid = (bid >= 0 && bid < p.num_blocks) ? bid : 0;
      const int64_t off = (int64_t)bid * p.block_stride_bytes + (key % kBlockSize) * row_bytes +
                          (int64_t)g * D * 2 + dchunk * 16;
      kreg[i] = load16(kc + off);
      vreg[i] = load16(vc + off);
    }
  };
  auto stage = [&](int t, int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int key = kg * KPT + i;
      *reinterpret_cast<u32x4*>(&sK[buf][key * KPitch + dchunk * 8]) = kreg[i];
    }
    // V^T: KPT consecutive keys of one column packed together; keys outside
    // [0, kend) are zeroed so stale slots never reach the MFMA
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int key = t * kBK + kg * KPT + i;
      if (key >= kend) vreg[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = dchunk * 8 + e;
      uint16_t v16[KPT];
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint32_t w = vreg[i][e >> 1];
        v16[i] = (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xFFFFu);
      }
      uint16_t* dst = &sVt[buf][d * kVtPitch + kg * KPT];
      if constexpr (KPT == 4) {
        u32x2 pk = {(uint32_t)v16[0] | ((uint32_t)v16[1] << 16), (uint32_t)v16[2] | ((uint32_t)v16[3] << 16)};
        *reinterpret_cast<u32x2*>(dst) = pk;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = (uint32_t)v16[0] | ((uint32_t)v16[1] << 16);
      }
    }
  };

  // ---- accumulators --------------------------------------------------------
  f32x16 o[MD][2];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[md][nt][r] = 0.f;
  float mref[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};
  const float sl2 = p.scale * kLog2e;

  fetch(0);
  stage(0, 0);
  __syncthreads();

  for (int t = 0; t < nkt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nkt) fetch(t + 1);
    const uint16_t* K_ = sK[buf];
    const uint16_t* Vt = sVt[buf];
    const int key0 = t * kBK;

    // S^T for 2 key sub-tiles x 2 column tiles
    f32x16 s[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][nt][r] = 0.f;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const vec a = as_vec<vec>(*reinterpret_cast<const u32x4*>(&K_[(kt * 32 + col) * KPitch + ds * 16 + 8 * hi]));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) s[kt][nt] = M::run(a, qreg[nt][ds], s[kt][nt]);
      }
    }

    // scale, mask, tile max per column
    const bool edge = (key0 + kBK > kend) || (p.causal && key0 + kBK - 1 > s0 + q0);
    float tmax[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kt][nt][r] * sl2;
          if (edge || !cvalid[nt]) {
            const int key = key0 + kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool vis = cvalid[nt] && key < kend && (!p.causal || key <= pabs[nt]);
            x = vis ? x : -INFINITY;
          }
          s[kt][nt][r] = x;
          tmax[nt] = fmaxf(tmax[nt], x);
        }
      }
      tmax[nt] = fmaxf(tmax[nt], __shfl_xor(tmax[nt], 32));
    }
    const bool need = (tmax[0] > mref[0] + kSlack) || (tmax[1] > mref[1] + kSlack);
    if (__any(need)) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float mn = fmaxf(mref[nt], tmax[nt]);
        const float corr = (mref[nt] == -INFINITY) ? 0.f : fast_exp2(mref[nt] - mn);
        lsum[nt] *= corr;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[md][nt][r] *= corr;
        mref[nt] = mn;
      }
    }

    // P (rounded to the input type) as B operands, row sums
    vec pb[2][2][2];                          // [kt][nt][half of the 32 keys]
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float mu = (mref[nt] == -INFINITY) ? 0.f : mref[nt];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          u32x4 pk;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float p0 = fast_exp2(s[kt][nt][8 * ss + 2 * e2] - mu);
            const float p1 = fast_exp2(s[kt][nt][8 * ss + 2 * e2 + 1] - mu);
            lsum[nt] += p0 + p1;
            pk[e2] = (uint32_t)M::bits(p0) | ((uint32_t)M::bits(p1) << 16);
          }
          pb[kt][nt][ss] = as_vec<vec>(pk);
        }
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const uint16_t* vrow = &Vt[(md * 32 + col) * kVtPitch];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          const int kb = kt * 32 + 16 * ss + 4 * hi;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(&vrow[kb]);
          const u32x2 up = *reinterpret_cast<const u32x2*>(&vrow[kb + 8]);
          const vec a = as_vec<vec>(u32x4{lo[0], lo[1], up[0], up[1]});
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) o[md][nt] = M::run(a, pb[kt][nt][ss], o[md][nt]);
        }
      }
    }

    if (t + 1 < nkt) stage(t + 1, buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store ------------------------------------------------
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float l = lsum[nt] + __shfl_xor(lsum[nt], 32);
    if (!cvalid[nt]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int c = (2 * wave + nt) * 32 + col;
    const int hl = c / BQ;
    uint16_t* orow = static_cast<uint16_t*>(p.out) +
                     ((int64_t)(cu0 + qpos[nt]) * p.num_q_heads + g * G + hl) * D;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = md * 32 + 8 * j + 4 * hi;
        u32x2 pk;
        pk[0] = (uint32_t)M::bits(o[md][nt][4 * j] * inv) | ((uint32_t)M::bits(o[md][nt][4 * j + 1] * inv) << 16);
        pk[1] = (uint32_t)M::bits(o[md][nt][4 * j + 2] * inv) | ((uint32_t)M::bits(o[md][nt][4 * j + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(orow + d) = pk;
      }
    }
  }
}

template <DT dt, int D>
static hipError_t launch_dg(const PrefillParams& p, hipStream_t s) {
  const int G = p.num_q_heads / p.num_kv_heads;
  const int BQ = kCols / G;
  const int tiles = (p.max_q_len + BQ - 1) / BQ;
  const int npairs = p.num_seqs * p.num_kv_heads;
  const int xcd = (npairs % 8 == 0) ? 1 : 0;
  const int64_t nwg = (int64_t)tiles * npairs;
  if (nwg <= 0) return hipSuccess;
  dim3 grid((unsigned)nwg), block(64 * kWaves);
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_kernel<dt, D, 1>), grid, block, 0, s, p, tiles, xcd); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<dt, D, 2>), grid, block, 0, s, p, tiles, xcd); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<dt, D, 4>), grid, block, 0, s, p, tiles, xcd); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<dt, D, 8>), grid, block, 0, s, p, tiles, xcd); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
  const DT dt = static_cast<DT>(p.dtype);
  if (p.head_dim == 128) {
    if (dt == DT::BF16) return launch_dg<DT::BF16, 128>(p, s);
    if (dt == DT::F16) return launch_dg<DT::F16, 128>(p, s);
  } else if (p.head_dim == 64) {
    if (dt == DT::BF16) return launch_dg<DT::BF16, 64>(p, s);
    if (dt == DT::F16) return launch_dg<DT::F16, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
