// Device-side building blocks shared by the paged-attention kernels (gfx950,
// wave64): element traits, 16-byte vectors, DPP row reductions, conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// F32, F16 and BF16 name both query/output and cache types; FP8 (OCP e4m3)
// names a cache type only.
enum class DT : int { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };

constexpr int kBlockSize = 16;   // tokens per physical block

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <DT dt> struct Elem;
template <> struct Elem<DT::F32>  { static constexpr int bytes = 4; };
template <> struct Elem<DT::F16>  { static constexpr int bytes = 2; };
template <> struct Elem<DT::BF16> { static constexpr int bytes = 2; };
template <> struct Elem<DT::FP8>  { static constexpr int bytes = 1; };

// ---------------------------------------------------------------------------
// DPP lane exchanges inside a row of 16 lanes.
//   0xB1 quad_perm [1,0,3,2]  (lane ^ 1)
//   0x4E quad_perm [2,3,0,1]  (lane ^ 2)
//   0x141 row_half_mirror     (lane i <-> 7-i within 8)
//   0x140 row_mirror          (lane i <-> 15-i within 16)
// After the quad exchanges every lane of a quad holds the quad's value, so the
// mirrors pair each lane with one of the other quad / other half.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in {1,2,4,8,16,32,64}); every lane of a
// group ends with the same, bit-identical sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f<0xB1>(v);
  if constexpr (N >= 4) v += dpp_f<0x4E>(v);
  if constexpr (N >= 8) v += dpp_f<0x141>(v);
  if constexpr (N >= 16) v += dpp_f<0x140>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// 16-byte vector <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(half2v, w).x;
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(half2v, w).y;
}

// Unpack the 16 bytes a lane loaded into EPL fp32 values.
template <DT dt>
__device__ __forceinline__ void unpack(const u32x4& v, float* f) {
  if constexpr (dt == DT::F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  } else if constexpr (dt == DT::F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = f16lo(v[i]); f[2 * i + 1] = f16hi(v[i]); }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16lo(v[i]); f[2 * i + 1] = bf16hi(v[i]); }
  }
}

// Partial dot product of two 16-byte vectors (same dtype), fp32 accumulation.
// 16-bit types use the packed dot2 instructions (two products per lane op).
template <DT dt>
__device__ __forceinline__ float dot16(const u32x4& a, const u32x4& b, float acc) {
  if constexpr (dt == DT::F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), acc);
  } else if constexpr (dt == DT::F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // copy the lanes out first: bit-casting a vector element in place reads element 0
      const uint32_t x = a[i], y = b[i];
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, x), __builtin_bit_cast(half2v, y), acc, false);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = a[i], y = b[i];
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162v, x), __builtin_bit_cast(bf162v, y),
                                            acc, false);
    }
  }
  return acc;
}

// fp32 -> storage bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <DT dt>
__device__ __forceinline__ void store_elem(void* base, int64_t idx, float x) {
  if constexpr (dt == DT::F32) {
    reinterpret_cast<float*>(base)[idx] = x;
  } else if constexpr (dt == DT::F16) {
    reinterpret_cast<uint16_t*>(base)[idx] = to_f16_bits(x);
  } else {
    reinterpret_cast<uint16_t*>(base)[idx] = to_bf16_bits(x);
  }
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 load8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// ---------------------------------------------------------------------------
// FP8 e4m3 (OCP 8-bit floating point E4M3: bias 7, 3 mantissa bits,
// subnormals, no infinities, NaN = S.1111.111, largest finite 448)
// ---------------------------------------------------------------------------
// Nearest code of a float, ties to the even mantissa; finite values past
// +-448 and infinities saturate to +-448; NaN stays NaN; the sign of zero is
// kept. Below 2^-6 the codes are the subnormal steps of 2^-9, so the code is
// |y| * 2^9 rounded to an integer (8 is the smallest normal); above it the
// float's mantissa is rounded to 3 bits in place and the exponent rebased.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;                 // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;                // >= 448 (inf included)
  if (a < 0x3C800000u)                                      // < 2^-6
    return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);       // round 23 -> 3 mantissa bits
  return sign | (((r >> 20) - (120u << 3)) & 0x7Fu);        // exponent bias 127 -> 7
}

// Four e4m3 codes of one dword -> two dwords of packed 16-bit values (the
// query type), byte pairs (0,1) and (2,3). Every e4m3 value is exact in f16
// and bf16; the conversion scale is 1.
template <DT dt, bool HI>
__device__ __forceinline__ uint32_t widen_fp8_pair(uint32_t w) {
  if constexpr (dt == DT::BF16)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

template <DT dt>
__device__ __forceinline__ u32x4 widen_fp8(const u32x2& w) {
  const uint32_t w0 = w[0], w1 = w[1];
  return u32x4{widen_fp8_pair<dt, false>(w0), widen_fp8_pair<dt, true>(w0),
               widen_fp8_pair<dt, false>(w1), widen_fp8_pair<dt, true>(w1)};
}

}  // namespace pa
