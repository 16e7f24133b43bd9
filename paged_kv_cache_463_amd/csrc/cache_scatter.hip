// reshape_and_cache: copy each new token's K and V row into the slot the block
// manager chose for it. Page "vLLM推理引擎深度解析" §三 (append_token) decides the
// slot — the last block while it has room, else a fresh one — and §五 leaves the
// write to the manager. Slot s is row s % 16 of physical block s / 16; a row is
// [num_kv_heads][head_dim] contiguous elements. The copy moves raw 16-byte
// chunks, so it is bit-exact for every dtype.
//
// Mapping: a token's row is cut into slices of 64 * U units (16-byte chunks of
// a 16-bit row, 8-element groups of an FP8 one); one wave copies one slice of
// K and of V, lane l taking units l, l + 64, ..., four waves per 256-thread
// workgroup. The host picks U: 1 while the batch fills fewer than
// kScatterMinWaves waves (a decode step scatters few tokens, so each row is
// spread over several waves), more for large scatters (a prefill chunk), where
// fewer, longer waves move the same bytes with less per-wave work. HBM-bound:
// 2 * row_bytes read and written per token.
#include <algorithm>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kScatterWaves = 4;

constexpr int64_t kScatterMinWaves = 2048;

// waves per token row: slices of 64 * u units of `unit_bytes`
__host__ __device__ inline int64_t scatter_slices(int64_t row_bytes, int unit_bytes, int u) {
  return (row_bytes / unit_bytes + 64 * u - 1) / (64 * u);
}

__global__ __launch_bounds__(64 * kScatterWaves)
void reshape_and_cache_kernel(ScatterParams p, int u) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * kScatterWaves + (threadIdx.x >> 6);
  const int64_t per = scatter_slices(p.row_bytes, 16, u);
  const int64_t t = w / per;
  if (t >= p.num_tokens) return;
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.num_slots) return;       // padding, or out of range: skip
  const int64_t blk = slot / kBlockSize, row = slot % kBlockSize;
  const char* ksrc = static_cast<const char*>(p.key) + t * p.token_stride_bytes;
  const char* vsrc = static_cast<const char*>(p.value) + t * p.token_stride_bytes;
  char* kdst = static_cast<char*>(p.k_cache) + blk * p.block_stride_bytes + row * (int64_t)p.row_bytes;
  char* vdst = static_cast<char*>(p.v_cache) + blk * p.block_stride_bytes + row * (int64_t)p.row_bytes;
  const int chunks = p.row_bytes >> 4;
  const int c1 = min(chunks, (int)(w % per + 1) * 64 * u);
  for (int c = (int)(w % per) * 64 * u + lane; c < c1; c += 64) {   // this lane's 16-byte chunks
    const u32x4 kv = load16(ksrc + 16 * c);
    const u32x4 vv = load16(vsrc + 16 * c);
    *reinterpret_cast<u32x4*>(kdst + 16 * c) = kv;
    *reinterpret_cast<u32x4*>(vdst + 16 * c) = vv;
  }
}

// units per lane and grid: one unit per lane while the batch fills fewer than
// kScatterMinWaves waves, else as many as keep it at kScatterMinWaves or more
static hipError_t scatter_grid(const ScatterParams& p, int unit_bytes, int& u, dim3& grid) {
  const int64_t slices1 = scatter_slices(p.row_bytes, unit_bytes, 1);
  u = (int)std::max<int64_t>(1, std::min<int64_t>(slices1, p.num_tokens * slices1 / kScatterMinWaves));
  const int64_t waves = p.num_tokens * scatter_slices(p.row_bytes, unit_bytes, u);
  const int64_t wgs = (waves + kScatterWaves - 1) / kScatterWaves;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  grid = dim3((unsigned)wgs);
  return hipSuccess;
}

hipError_t launch_reshape_and_cache(const ScatterParams& p, hipStream_t s) {
  dim3 grid;
  int u;
  if (scatter_grid(p, 16, u, grid) != hipSuccess) return hipErrorInvalidValue;
  hipLaunchKernelGGL(reshape_and_cache_kernel, grid, dim3(64 * kScatterWaves), 0, s, p, u);
  return hipGetLastError();
}

// reshape_and_cache into an FP8 (e4m3) cache: the same slots, but each element
// x of head h is stored as the e4m3 code nearest to x / scale[h] (one
// correctly rounded fp32 division, ties to the even mantissa, saturating at
// +-448; the pages list FP8 among the supported quantisation schemes, page
// "vLLM推理引擎深度实战", introduction). A lane converts 8 consecutive elements
// (16 or 32 input bytes) into one 8-byte store; 8 divides head_dim, so the 8
// share one head and one scale. A wave takes a slice of 64 such groups of one
// token's row (a correctly rounded division and an encode per element make
// this work VALU-bound, so the rows are spread over as many waves as they fill).
template <DT dt>
__global__ __launch_bounds__(64 * kScatterWaves)
void reshape_and_cache_fp8_kernel(ScatterParams p, int u) {
  constexpr int E = Elem<dt>::bytes;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * kScatterWaves + (threadIdx.x >> 6);
  const int64_t per = scatter_slices(p.row_bytes, 8, u);
  const int64_t t = w / per;
  if (t >= p.num_tokens) return;
  const int groups = p.row_bytes >> 3;                  // 8 elements a group
  const int c0 = (int)(w % per) * 64 * u, c1 = min(groups, c0 + 64 * u);
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.num_slots) return;
  const int64_t blk = slot / kBlockSize, row = slot % kBlockSize;
  const int64_t dst = blk * p.block_stride_bytes + row * (int64_t)p.row_bytes;
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const char* src = static_cast<const char*>(kv ? p.value : p.key) + t * p.token_stride_bytes;
    char* out = static_cast<char*>(kv ? p.v_cache : p.k_cache) + dst;
    const float* sc = kv ? p.v_scale : p.k_scale;
    for (int c = c0 + lane; c < c1; c += 64) {        // this lane's groups of the row
      float x[8];
      if constexpr (dt == DT::F32) {
        unpack<dt>(load16(src + 32 * c), x);
        unpack<dt>(load16(src + 32 * c + 16), x + 4);
      } else {
        unpack<dt>(load16(src + 16 * c), x);
      }
      const float s = sc[(8 * c) / p.head_dim];
      uint32_t code[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) code[i >> 2] |= e4m3_encode(x[i] / s) << (8 * (i & 3));
      *reinterpret_cast<u32x2*>(out + 8 * c) = u32x2{code[0], code[1]};
    }
  }
}

hipError_t launch_reshape_and_cache_fp8(const ScatterParams& p, hipStream_t s) {
  dim3 grid;
  int u;
  if (scatter_grid(p, 8, u, grid) != hipSuccess) return hipErrorInvalidValue;
  const dim3 block(64 * kScatterWaves);
  switch (static_cast<DT>(p.in_dtype)) {
    case DT::F32: hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT::F32>, grid, block, 0, s, p, u); break;
    case DT::F16: hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT::F16>, grid, block, 0, s, p, u); break;
    case DT::BF16: hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT::BF16>, grid, block, 0, s, p, u); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
