// Device-side helpers shared by the P-EAGLE draft-forward kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace peagle {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// 32x32x16 bf16 MFMA: D[32x32] += A[32x16] * B[16x32]. Lane l supplies row l%32 of A and
// column l%32 of B, each as 8 consecutive k; it receives column l%32 of D, rows
// 8*(r/4) + 4*(l/32) + r%4 for accumulator register r.
__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __builtin_bit_cast(float, b16 << 16);
}

// Index of the last element <= x in the non-decreasing array a[0..len) (or -1).
__device__ __forceinline__ int upper_index(const int32_t* a, int len, int32_t x) {
  int lo = 0, hi = len;  // first element > x
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid + 1; else hi = mid;
  }
  return lo - 1;
}

// Number of elements < x in the non-decreasing array a[0..len).
__device__ __forceinline__ int lower_count(const int32_t* a, int len, int32_t x) {
  int lo = 0, hi = len;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

}  // namespace peagle
