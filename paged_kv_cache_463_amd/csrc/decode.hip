// Paged decode attention for gfx950: one query token per sequence attends over
// the K/V rows its block table names (page "vLLM推理引擎深度解析" §五,
// PagedAttention.forward: per sequence look up the block table, read K and V
// from the physical blocks in place, score q·k/sqrt(d), softmax, weight V).
//
// Work mapping (one workgroup = one (sequence, kv head), or one token partition
// of it in the split-KV variant; W waves split the workgroup's blocks into
// contiguous ranges):
//   * A token row of one head is D*e bytes (256 B for 16-bit D=128 or fp32 D=64).
//     LPR = D*e/16 lanes cover a row with one 16-byte load each; a wave covers
//     ROWS = 64/LPR rows per load, so a 16-token block is TPL = 16/ROWS loads of
//     K and TPL of V per lane, all 16-byte, each row segment fully used.
//   * The G query heads of the group share every K/V row: each lane keeps its
//     16-byte slice of all G query vectors in registers and computes G partial
//     dot products per row (packed dot2 for 16-bit types), reduced across the
//     LPR lanes of the row with DPP (no LDS).
//   * Online softmax with a wave-uniform reference max per head: scores are
//     kept in log2 units (scale*log2 e folded in), p = 2^(s - m_ref). m_ref only
//     moves when some score exceeds it by more than 8 (ballot, uniform branch),
//     which bounds p by 256 and makes the rescale of the accumulators rare. The
//     softmax is unchanged by the choice of reference, which cancels in o/l.
//   * Every lane accumulates p*V for its own columns and tokens; rows are
//     summed once at the end, then waves are merged through LDS with the usual
//     max-rescale.
//   * Masking: only the last block of a sequence can hold dead rows (they may
//     hold stale NaN); their scores become -inf and their V slices are zeroed
//     before use, so 0 * NaN never happens.
//   * Block ids are wave-uniform (scalar loads); the next block's K/V loads are
//     issued before the current block is computed.
//
// Split-KV: workgroup (kv head, sequence, partition) covers logical tokens
// [partition_size*p, partition_size*(p+1)) and writes, per query head, the
// unnormalised output row plus (max, normaliser) to the workspace; a second
// kernel merges partitions by log-sum-exp.
#include <math.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;   // log2 units: p <= 2^8 between rescales
constexpr int kDecodeWaves = 4;

template <DT dt, int D, int G, int W, bool SPLIT>
__global__ __launch_bounds__(64 * W)
void decode_kernel(DecodeParams p) {
  constexpr int E = Elem<dt>::bytes;
  constexpr int EPL = 16 / E;               // elements per lane per load
  constexpr int LPR = D / EPL;              // lanes per token row
  constexpr int ROWS = 64 / LPR;            // rows per wave load
  constexpr int TPL = kBlockSize / ROWS;    // tokens per lane per block
  static_assert(LPR >= 8 && LPR <= 32 && TPL >= 1, "unsupported head_dim/dtype");

  __shared__ float s_acc[W][G][D];
  __shared__ float s_m[W][G];
  __shared__ float s_l[W][G];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPR;
  const int c = lane % LPR;
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int part = SPLIT ? (int)blockIdx.z : 0;
  const int hq0 = g * G;

  const int L = max(p.context_lens[b], 0);
  const int nblk = min((L + kBlockSize - 1) / kBlockSize, p.block_table_stride);
  int lo = 0, hi = nblk;
  if constexpr (SPLIT) {
    lo = part * p.partition_blocks;
    if (lo >= nblk) return;                 // whole workgroup: partition past the end
    hi = min(nblk, lo + p.partition_blocks);
  }
  const int per = (hi - lo + W - 1) / W;
  const int my_lo = lo + wave * per;
  const int my_hi = min(hi, my_lo + per);

  // this lane's 16-byte slice of the G query vectors
  u32x4 q[G];
  {
    const char* qb = static_cast<const char*>(p.query) +
                     (((int64_t)b * p.num_q_heads + hq0) * D + c * EPL) * E;
#pragma unroll
    for (int h = 0; h < G; ++h) q[h] = load16(qb + (int64_t)h * D * E);
  }
  // byte offsets of this lane's rows inside a physical block
  uint32_t off[TPL];
#pragma unroll
  for (int j = 0; j < TPL; ++j)
    off[j] = (uint32_t)((((r + ROWS * j) * p.num_kv_heads + g) * D) * E + c * 16);

  const float sl2 = p.scale * kLog2e;
  const int32_t* tbl = p.block_tables + (int64_t)b * p.block_table_stride;
  const char* kc = static_cast<const char*>(p.k_cache);
  const char* vc = static_cast<const char*>(p.v_cache);

  float m_ref[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_ref[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  u32x4 kcur[TPL], vcur[TPL], knxt[TPL], vnxt[TPL];
  bool ok_cur = true, ok_nxt = true;

  auto fetch = [&](int i, u32x4* kd, u32x4* vd, bool& ok) {
    int bid = tbl[i];
    ok = (bid >= 0) && (bid < p.num_blocks);
    bid = ok ? bid : 0;                      // never address outside the pool
    const char* kb = kc + (int64_t)bid * p.block_stride_bytes;
    const char* vb = vc + (int64_t)bid * p.block_stride_bytes;
#pragma unroll
    for (int j = 0; j < TPL; ++j) kd[j] = load16(kb + off[j]);
#pragma unroll
    for (int j = 0; j < TPL; ++j) vd[j] = load16(vb + off[j]);
  };

  if (my_lo < my_hi) fetch(my_lo, kcur, vcur, ok_cur);
  for (int i = my_lo; i < my_hi; ++i) {
    if (i + 1 < my_hi) fetch(i + 1, knxt, vnxt, ok_nxt);

    float s[TPL][G];
#pragma unroll
    for (int j = 0; j < TPL; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) s[j][h] = group_sum<LPR>(dot16<dt>(q[h], kcur[j], 0.f)) * sl2;

    const int tok0 = i * kBlockSize;
    if (!ok_cur || tok0 + kBlockSize > L) {  // uniform: only a sequence's last block
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        if (!ok_cur || tok0 + r + ROWS * j >= L) {
#pragma unroll
          for (int h = 0; h < G; ++h) s[j][h] = -INFINITY;
          vcur[j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }

    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < TPL; ++j) need |= s[j][h] > m_ref[h] + kRescaleSlack;
    if (__any(need)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = s[0][h];
#pragma unroll
        for (int j = 1; j < TPL; ++j) mx = fmaxf(mx, s[j][h]);
        const float mn = fmaxf(m_ref[h], wave_max(mx));
        const float corr = (m_ref[h] == -INFINITY) ? 0.f : fast_exp2(m_ref[h] - mn);
        l[h] *= corr;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= corr;
        m_ref[h] = mn;
      }
    }

#pragma unroll
    for (int j = 0; j < TPL; ++j) {
      float vf[EPL];
      unpack<dt>(vcur[j], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pj = fast_exp2(s[j][h] - m_ref[h]);
        l[h] += pj;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pj, vf[e], acc[h][e]);
      }
    }

#pragma unroll
    for (int j = 0; j < TPL; ++j) { kcur[j] = knxt[j]; vcur[j] = vnxt[j]; }
    ok_cur = ok_nxt;
  }

  // sum the ROWS row-streams of the wave (all lanes of a row hold equal l)
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      l[h] += __shfl_xor(l[h], o);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], o);
    }
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][h][c * EPL + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) { s_m[wave][h] = m_ref[h]; s_l[wave][h] = l[h]; }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += 64 * W) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = s_m[w][h];
      const float sc = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      num = fmaf(sc, s_acc[w][h][d], num);
      den = fmaf(sc, s_l[w][h], den);
    }
    const int64_t row = (int64_t)b * p.num_q_heads + hq0 + h;
    if constexpr (!SPLIT) {
      store_elem<dt>(p.out, row * D + d, den > 0.f ? num / den : 0.f);
    } else {
      const int64_t pr = row * p.max_parts + part;
      p.ws_acc[pr * D + d] = num;
      if (d == 0) { p.ws_ml[2 * pr] = M; p.ws_ml[2 * pr + 1] = den; }
    }
  }
}

// Log-sum-exp merge of the split-KV partials: one wave per (query head, sequence).
template <DT dt, int D>
__global__ __launch_bounds__(64)
void splitkv_merge_kernel(DecodeParams p) {
  constexpr int CPL = D / 64;
  const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int L = max(p.context_lens[b], 0);
  const int nblk = min((L + kBlockSize - 1) / kBlockSize, p.block_table_stride);
  const int np = min((nblk + p.partition_blocks - 1) / p.partition_blocks, p.max_parts);
  const int64_t row = (int64_t)b * p.num_q_heads + hq;
  const float* ml = p.ws_ml + row * p.max_parts * 2;
  const float* pa_ = p.ws_acc + row * p.max_parts * D;

  float M = -INFINITY;
  for (int i = lane; i < np; i += 64) M = fmaxf(M, ml[2 * i]);
  M = wave_max(M);
  float num[CPL], den = 0.f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) num[k] = 0.f;
  for (int i = 0; i < np; ++i) {
    const float mi = ml[2 * i], li = ml[2 * i + 1];
    const float w = (mi == -INFINITY) ? 0.f : fast_exp2(mi - M);
    den = fmaf(w, li, den);
#pragma unroll
    for (int k = 0; k < CPL; ++k) num[k] = fmaf(w, pa_[(int64_t)i * D + lane + 64 * k], num[k]);
  }
#pragma unroll
  for (int k = 0; k < CPL; ++k)
    store_elem<dt>(p.out, row * D + lane + 64 * k, den > 0.f ? num[k] / den : 0.f);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <DT dt, int D, bool SPLIT>
static hipError_t launch_g(const DecodeParams& p, hipStream_t s) {
  const int G = p.num_q_heads / p.num_kv_heads;
  dim3 grid(p.num_kv_heads, p.num_seqs, SPLIT ? p.max_parts : 1);
  dim3 block(64 * kDecodeWaves);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_kernel<dt, D, 1, kDecodeWaves, SPLIT>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<dt, D, 2, kDecodeWaves, SPLIT>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<dt, D, 4, kDecodeWaves, SPLIT>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<dt, D, 8, kDecodeWaves, SPLIT>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !SPLIT) return e;
  hipLaunchKernelGGL((splitkv_merge_kernel<dt, D>), dim3(p.num_q_heads, p.num_seqs), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <bool SPLIT>
static hipError_t launch_any(const DecodeParams& p, hipStream_t s) {
  const DT dt = static_cast<DT>(p.dtype);
  if (p.head_dim == 128) {
    if (dt == DT::F32) return launch_g<DT::F32, 128, SPLIT>(p, s);
    if (dt == DT::F16) return launch_g<DT::F16, 128, SPLIT>(p, s);
    if (dt == DT::BF16) return launch_g<DT::BF16, 128, SPLIT>(p, s);
  } else if (p.head_dim == 64) {
    if (dt == DT::F32) return launch_g<DT::F32, 64, SPLIT>(p, s);
    if (dt == DT::F16) return launch_g<DT::F16, 64, SPLIT>(p, s);
    if (dt == DT::BF16) return launch_g<DT::BF16, 64, SPLIT>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) { return launch_any<false>(p, s); }
hipError_t launch_decode_splitkv(const DecodeParams& p, hipStream_t s) { return launch_any<true>(p, s); }

}  // namespace pa
