// reshape_and_cache: copy each new token's K and V row into the slot the block
// manager chose for it. Page "vLLM推理引擎深度解析" §三 (append_token) decides the
// slot — the last block while it has room, else a fresh one — and §五 leaves the
// write to the manager. Slot s is row s % 16 of physical block s / 16; a row is
// [num_kv_heads][head_dim] contiguous elements. The copy moves raw 16-byte
// chunks, so it is bit-exact for every dtype.
//
// Mapping: one wave per token, lanes stride over the row's 16-byte chunks; four
// tokens per 256-thread workgroup. HBM-bound: 2 * row_bytes read and written per
// token.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kScatterWaves = 4;

__global__ __launch_bounds__(64 * kScatterWaves)
void reshape_and_cache_kernel(ScatterParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kScatterWaves + (threadIdx.x >> 6);
  if (t >= p.num_tokens) return;
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.num_slots) return;       // padding, or out of range: skip
  const int64_t blk = slot / kBlockSize, row = slot % kBlockSize;
  const int64_t dst = blk * p.block_stride_bytes + row * (int64_t)p.row_bytes;
  const char* ksrc = static_cast<const char*>(p.key) + t * p.token_stride_bytes;
  const char* vsrc = static_cast<const char*>(p.value) + t * p.token_stride_bytes;
  char* kdst = static_cast<char*>(p.k_cache) + dst;
  char* vdst = static_cast<char*>(p.v_cache) + dst;
  const int chunks = p.row_bytes >> 4;
  for (int c = lane; c < chunks; c += 64) {
    const u32x4 kv = load16(ksrc + 16 * c);
    const u32x4 vv = load16(vsrc + 16 * c);
    *reinterpret_cast<u32x4*>(kdst + 16 * c) = kv;
    *reinterpret_cast<u32x4*>(vdst + 16 * c) = vv;
  }
}

hipError_t launch_reshape_and_cache(const ScatterParams& p, hipStream_t s) {
  const int64_t groups = (p.num_tokens + kScatterWaves - 1) / kScatterWaves;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)groups), dim3(64 * kScatterWaves), 0, s, p);
  return hipGetLastError();
}

// reshape_and_cache into an FP8 (e4m3) cache: the same slots, but each element
// x of head h is stored as the e4m3 code nearest to x / scale[h] (one
// correctly rounded fp32 division, ties to the even mantissa, saturating at
// +-448; the pages list FP8 among the supported quantisation schemes, page
// "vLLM推理引擎深度实战", introduction). A lane converts 8 consecutive elements
// (16 or 32 input bytes) into one 8-byte store; 8 divides head_dim, so the 8
// share one head and one scale.
template <DT dt>
__global__ __launch_bounds__(64 * kScatterWaves)
void reshape_and_cache_fp8_kernel(ScatterParams p) {
  constexpr int E = Elem<dt>::bytes;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kScatterWaves + (threadIdx.x >> 6);
  if (t >= p.num_tokens) return;
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.num_slots) return;
  const int64_t blk = slot / kBlockSize, row = slot % kBlockSize;
  const int64_t dst = blk * p.block_stride_bytes + row * (int64_t)p.row_bytes;
  const int groups = p.row_bytes >> 3;                  // 8 elements a group
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const char* src = static_cast<const char*>(kv ? p.value : p.key) + t * p.token_stride_bytes;
    char* out = static_cast<char*>(kv ? p.v_cache : p.k_cache) + dst;
    const float* sc = kv ? p.v_scale : p.k_scale;
    for (int c = lane; c < groups; c += 64) {
      float x[8];
      if constexpr (dt == DT::F32) {
        unpack<dt>(load16(src + 32 * c), x);
        unpack<dt>(load16(src + 32 * c + 16), x + 4);
      } else {
        unpack<dt>(load16(src + 16 * c), x);
      }
      const float s = sc[(8 * c) / p.head_dim];
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i >> 2] |= e4m3_encode(x[i] / s) << (8 * (i & 3));
      *reinterpret_cast<u32x2*>(out + 8 * c) = u32x2{w[0], w[1]};
    }
  }
}

hipError_t launch_reshape_and_cache_fp8(const ScatterParams& p, hipStream_t s) {
  const int64_t groups = (p.num_tokens + kScatterWaves - 1) / kScatterWaves;
  const dim3 grid((unsigned)groups), block(64 * kScatterWaves);
  switch (static_cast<DT>(p.in_dtype)) {
    case DT::F32: hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT::F32>, grid, block, 0, s, p); break;
    case DT::F16: hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT::F16>, grid, block, 0, s, p); break;
    case DT::BF16: hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT::BF16>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
