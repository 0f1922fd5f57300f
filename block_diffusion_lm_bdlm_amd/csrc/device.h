// device.h — gfx950 building blocks shared by the kernels.
//
// Matrix-core tile used everywhere: v_mfma_f32_32x32x16_{bf16,f16}.  For
// C[32x32] += A[32x16] * B[16x32] a lane l (64 per wave) supplies
//   A[m = l%32][k = (l/32)*8 .. +8]   and   B[k = (l/32)*8 .. +8][n = l%32]
// and receives C[m][n = l%32] for m = (i/4)*8 + (l/32)*4 + i%4, i = 0..15.
//
// The C tile can feed the next product's B operand directly when the next
// contraction runs over C's row index m: register i = 8*s + e (k-step s,
// element e) holds row m = 16*s + (e/4)*8 + (l/32)*4 + e%4.  The other
// operand must list its contraction index in the same order, so transposed
// operands are stored with every aligned group of 16 rows permuted by
// kPerm16 (slot j holds row kPerm16[j]; the permutation is an involution).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int perm16(int j) {
  // slots 4..7 <-> rows 8..11
  return (j >= 4 && j < 8) ? j + 4 : ((j >= 8 && j < 12) ? j - 4 : j);
}

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T ld16(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Reductions over lanes l and l ^ 32.  v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second; given
// x twice, every lane receives x of both lanes of its pair (in some order),
// with no LDS round trip.
__device__ __forceinline__ float wave_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// MFMA C-tile row index of register i for lane half hh.
__device__ __forceinline__ int crow(int i, int hh) { return (i >> 2) * 8 + hh * 4 + (i & 3); }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return *reinterpret_cast<uint16_t*>(&b);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float((uint32_t)u << 16);
}

// Largest finite fp16 value.
constexpr float kHalfMax = 65504.f;

// Eight bf16 values (as loaded, two per dword), times `mul` (a power of two),
// to fp16 through fp32 with round-to-nearest-even: exact for products in
// the half range above its subnormals.  A product outside [-65504, 65504]
// (or NaN) sets `bad`; finite ones are clamped to the half range.
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(const u32x4& v, float mul, bool& bad) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x = bf16_to_f32((uint16_t)(v[e >> 1] >> (16 * (e & 1)))) * mul;
    bad |= !(fabsf(x) <= kHalfMax);
    if (fabsf(x) > kHalfMax) x = copysignf(kHalfMax, x);
    r[e] = (_Float16)x;
  }
  return r;
}

}  // namespace bd
