// Device-side building blocks for the gfx950 KDA kernels: vector types, the
// two MFMA shapes used (bf16 16x16x32 and fp32 16x16x4) behind one
// "32-wide reduction block" interface, and fragment conversion helpers.
//
// MFMA lane layouts on gfx950 (lane l, g = l >> 4, i = l & 15):
//   v_mfma_f32_16x16x32_bf16: a[t] = A[i][8g + t], b[t] = B[8g + t][i],
//                             c[r] = C[4g + r][i]
//   v_mfma_f32_16x16x4_f32:   a = A[i][g], b = B[g][i], c[r] = C[4g + r][i]
//
// A "frag8" is the 8 operand values one lane supplies for a 32-wide block of
// the reduction index. Element t of lane group g stands for the physical
// reduction index phys(g, t) (4g + t, then 16 + 4g + t - 4). For bf16 that
// is a single MFMA (virtual index 8g + t <-> phys(g, t)); for fp32 it is 8
// MFMAs, MFMA s taking element s. Because two 16x16 accumulator tiles stacked
// along the reduction index hold exactly rows phys(g, 0..7) in lane group g,
// an accumulator pair becomes a B operand with no data movement.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

template <typename T> struct Vec;
template <> struct Vec<bf16> { typedef bf16x8 x8; typedef bf16x4 x4; };
template <> struct Vec<float> { typedef floatx8 x8; typedef floatx4 x4; };

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// acc += A(16 x 32) * B(32 x 16) with both operands given as frag8.
__device__ __forceinline__ floatx4 mma32(floatx4 acc, const bf16x8& a, const bf16x8& b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma32(floatx4 acc, const floatx8& a, const floatx8& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
  return acc;
}

// fp32 16x16x4 step with a 16-wide reduction: element s of a / b is the
// reduction index 4g + s. Used by the fp32 triangular solve.
__device__ __forceinline__ floatx4 mma16_f32(floatx4 acc, const floatx4& a, const floatx4& b) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
  return acc;
}

// conversions between fp32 and the stored element type
__device__ __forceinline__ void cvt8(const floatx8& x, bf16x8& y) { y = __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ void cvt8(const floatx8& x, floatx8& y) { y = x; }
__device__ __forceinline__ void cvt4(const floatx4& x, bf16x4& y) { y = __builtin_convertvector(x, bf16x4); }
__device__ __forceinline__ void cvt4(const floatx4& x, floatx4& y) { y = x; }
__device__ __forceinline__ floatx4 widen4(const bf16x4& x) { return __builtin_convertvector(x, floatx4); }
__device__ __forceinline__ floatx4 widen4(const floatx4& x) { return x; }
__device__ __forceinline__ floatx8 widen8(const bf16x8& x) { return __builtin_convertvector(x, floatx8); }
__device__ __forceinline__ floatx8 widen8(const floatx8& x) { return x; }

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

// stack two accumulator tiles into one frag8 (top tile = phys rows 0..15)
template <typename T>
__device__ __forceinline__ typename Vec<T>::x8 stack8(const typename Vec<T>::x4& top,
                                                      const typename Vec<T>::x4& bot) {
  typename Vec<T>::x8 r;
  r[0] = top[0]; r[1] = top[1]; r[2] = top[2]; r[3] = top[3];
  r[4] = bot[0]; r[5] = bot[1]; r[6] = bot[2]; r[7] = bot[3];
  return r;
}

__device__ __forceinline__ floatx8 stackf(const floatx4& top, const floatx4& bot) {
  floatx8 r;
  r[0] = top[0]; r[1] = top[1]; r[2] = top[2]; r[3] = top[3];
  r[4] = bot[0]; r[5] = bot[1]; r[6] = bot[2]; r[7] = bot[3];
  return r;
}

// 2^x on the transcendental unit (no denormal fix-up; inputs are bounded)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// load 4 consecutive elements of type T from global memory as fp32
__device__ __forceinline__ floatx4 load4_f32(const bf16* p) {
  return widen4(*reinterpret_cast<const bf16x4*>(p));
}
__device__ __forceinline__ floatx4 load4_f32(const float* p) {
  return *reinterpret_cast<const floatx4*>(p);
}

}  // namespace kda
