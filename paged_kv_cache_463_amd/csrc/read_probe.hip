// Read-bandwidth calibration for the decode walks: the K and V rows that a
// decode call reads (every cached token's row of every kv head, reached
// through the block tables), read with the same 16-byte non-temporal loads and
// no arithmetic. It measures what the memory system delivers for exactly that
// access set, the practical ceiling the attention kernels are judged against.
//
// Two walks, as the attention calls:
//   * partition_size > 0 (the split-KV walk): one wave per (kv head,
//     sequence, partition) item, items numbered kv head fastest and then the
//     existing (sequence, partition) pairs densely, four waves per workgroup;
//   * partition_size == 0 (the single-pass walk): one workgroup of four waves
//     per (kv head, sequence), the waves taking its blocks round-robin; grid
//     row r takes the sequence of rank r in descending length (ties by
//     index), the dispatch order of the single-pass decode, found here by a
//     direct count (batches above 1024 sequences keep grid order).
// Each wave keeps two blocks of loads in flight and folds the words it read
// into an XOR that it stores into sink, so no load can be dropped.
#include <algorithm>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kProbeWaves = 4;
constexpr int kProbeMaxSeqs = 1024;        // dense item numbering / ranking in LDS up to this batch

// The sequence of rank r (descending length, ties by index) among B <= 1024:
// keys in LDS, then every thread counts, for its candidates, the keys larger
// than theirs; the candidate with count r is the one.
__device__ int probe_sequence_of_rank(const int32_t* lens, int B, int r, int* s_key) {
  __shared__ int s_pick;
  for (int t = threadIdx.x; t < B; t += 64 * kProbeWaves)
    s_key[t] = (min(max(lens[t], 0), (1 << 21) - 1) << 10) | (1023 - t);
  __syncthreads();
  for (int t = threadIdx.x; t < B; t += 64 * kProbeWaves) {
    const int key = s_key[t];
    int rank = 0;
    for (int u = 0; u < B; ++u) rank += s_key[u] > key;
    if (rank == r) s_pick = t;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(s_pick);
}

template <int TPL>
__global__ __launch_bounds__(64 * kProbeWaves)
void read_probe_kernel(ReadProbeParams p) {
  __shared__ int s_pre[kProbeMaxSeqs + 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int LPR = p.row_bytes / 16;          // lanes per token row of one head
  const int ROWS = 64 / LPR;                 // rows per wave load
  const int r = lane / LPR, c = lane % LPR;
  const int B = p.num_seqs;

  int g, b, lo, hi, step;
  if (p.partition_blocks > 0) {              // split-KV walk: one item per wave
    for (int t = threadIdx.x; t < B; t += 64 * kProbeWaves) {
      const int nb = min((max(p.context_lens[t], 0) + kBlockSize - 1) / kBlockSize, p.block_table_stride);
      s_pre[t] = (nb + p.partition_blocks - 1) / p.partition_blocks;
    }
    __syncthreads();
    if (threadIdx.x < 64) {                  // exclusive prefix sums: a run of sequences per lane
      const int per = (B + 63) / 64;
      const int t0 = min(lane * per, B), t1 = min(t0 + per, B);
      int run = 0;
      for (int t = t0; t < t1; ++t) run += s_pre[t];
      int inc = run;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
      }
      int acc = inc - run;
      for (int t = t0; t < t1; ++t) {
        const int n = s_pre[t];
        s_pre[t] = acc;
        acc += n;
      }
      if (lane == 63) s_pre[B] = inc;
    }
    __syncthreads();
    const int ticket = blockIdx.x * kProbeWaves + wave;
    g = ticket % p.num_kv_heads;
    const int item = ticket / p.num_kv_heads;
    if (item >= __builtin_amdgcn_readfirstlane(s_pre[B])) return;
    int l = 0, h = B - 1;                    // last sequence whose first item is <= item
    while (l < h) {
      const int mid = (l + h + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(s_pre[mid]) <= item) l = mid; else h = mid - 1;
    }
    b = l;
    const int part = item - __builtin_amdgcn_readfirstlane(s_pre[l]);
    const int nb = min((max(p.context_lens[b], 0) + kBlockSize - 1) / kBlockSize, p.block_table_stride);
    lo = part * p.partition_blocks;
    hi = min(nb, lo + p.partition_blocks);
    step = 1;
  } else {                                   // single-pass walk: one workgroup per (kv head, sequence)
    g = blockIdx.x;
    b = B <= kProbeMaxSeqs ? probe_sequence_of_rank(p.context_lens, B, blockIdx.y, s_pre) : blockIdx.y;
    const int nb = min((max(p.context_lens[b], 0) + kBlockSize - 1) / kBlockSize, p.block_table_stride);
    lo = wave;
    hi = nb;
    step = kProbeWaves;
  }

  const int32_t* tbl = p.block_tables + (int64_t)b * p.block_table_stride;
  const char* kc = static_cast<const char*>(p.k_cache);
  const char* vc = static_cast<const char*>(p.v_cache);
  uint32_t off[TPL];
#pragma unroll
  for (int j = 0; j < TPL; ++j)
    off[j] = (uint32_t)(((r + ROWS * j) * p.num_kv_heads + g) * p.row_bytes + c * 16);
  auto fetch = [&](int i, u32x4* kd, u32x4* vd) {
    int bid = i < hi ? tbl[i] : 0;
    bid = (bid >= 0 && bid < p.num_blocks) ? bid : 0;
    const char* kb = kc + (int64_t)bid * p.block_stride_bytes;
    const char* vb = vc + (int64_t)bid * p.block_stride_bytes;
#pragma unroll
    for (int j = 0; j < TPL; ++j) kd[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + off[j]));
#pragma unroll
    for (int j = 0; j < TPL; ++j) vd[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + off[j]));
  };
  uint32_t x = 0;
  auto fold = [&](const u32x4* kd, const u32x4* vd) {
#pragma unroll
    for (int j = 0; j < TPL; ++j) x ^= kd[j][0] ^ kd[j][1] ^ kd[j][2] ^ kd[j][3] ^ vd[j][0] ^ vd[j][1] ^ vd[j][2] ^ vd[j][3];
  };
  u32x4 k0[TPL], v0[TPL], k1[TPL], v1[TPL];
  int i = lo;
  if (i < hi) fetch(i, k0, v0);
  if (i + step < hi) fetch(i + step, k1, v1);
  for (; i < hi; i += 2 * step) {            // two blocks in flight
    fold(k0, v0);
    if (i + 2 * step < hi) fetch(i + 2 * step, k0, v0);
    if (i + step < hi) {
      fold(k1, v1);
      if (i + 3 * step < hi) fetch(i + 3 * step, k1, v1);
    }
  }
  // one word per wave (the XOR of every lane's words), so no load can be removed
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x ^= __shfl_xor(x, o);
  const int64_t w = ((int64_t)(blockIdx.y * gridDim.x + blockIdx.x) * kProbeWaves + wave) % p.sink_words;
  if (lane == 0) p.sink[w] = x;
}

}  // namespace

hipError_t launch_read_probe(const ReadProbeParams& p, hipStream_t s) {
  const int tpl = kBlockSize * p.row_bytes / 1024;   // tokens per lane per block
  auto kernel = tpl == 4 ? read_probe_kernel<4> : tpl == 2 ? read_probe_kernel<2>
              : tpl == 8 ? read_probe_kernel<8> : tpl == 1 ? read_probe_kernel<1> : nullptr;
  if (!kernel) return hipErrorInvalidValue;
  dim3 grid;
  if (p.partition_blocks > 0) {
    if (p.num_seqs > kProbeMaxSeqs) return hipErrorInvalidValue;
    const int64_t items = (int64_t)p.num_kv_heads * p.num_seqs * p.max_parts;
    grid = dim3((unsigned)std::max<int64_t>((items + kProbeWaves - 1) / kProbeWaves, 1));
  } else {
    if (p.num_seqs > 65535) return hipErrorInvalidValue;
    grid = dim3(p.num_kv_heads, p.num_seqs);
  }
  hipLaunchKernelGGL(kernel, grid, dim3(64 * kProbeWaves), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa
