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

// ---- LDS DMA (global_load_lds_dwordx4, buffer_load_dwordx4 ... lds) and scheduling helpers ----

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left at their maxima (N < 16): at most N of
// this wave's vector-memory operations (here: LDS-DMA tile loads) are still outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
__device__ __forceinline__ void wait_dma() { wait_vm<0>(); }

// A wave-uniform pointer the optimiser cannot follow across loop iterations: it stays one
// scalar register pair (the DMA uses the scalar-base + 32-bit lane offset form) instead of
// being strength-reduced into a 64-bit pointer per lane and per source.
__device__ __forceinline__ const char* uniform_opaque(const char* p) {
  asm("" : "+s"(p));
  return p;
}

// A 32-bit lane offset kept 32-bit at its use (not hoisted as a 64-bit extension).
__device__ __forceinline__ uint32_t lane_opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ void dma16(const void* src, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// The same LDS DMA in its buffer form (buffer_load_dwordx4 ... lds): lane l moves 16 bytes
// from the range's byte voff to lds_wave_base + 16 l. The compiler's wait-count pass treats
// the global form as a flat access that may touch LDS, and while one is outstanding it
// makes every LDS read wait with lgkmcnt(0), draining the reads issued ahead of the MFMAs;
// the buffer form it tracks on vmcnt alone. The range is a raw buffer resource (gfx9
// descriptor, no stride) over [base, base + bytes): a lane offset at or past bytes loads
// zeros instead of reading outside it. base is wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_range(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t range, uint32_t voff,
                                          char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      range, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, 0, 0, 0);
}

// Scheduling pattern for a run of N groups of R LDS reads, each group feeding M MFMAs: the
// first PF groups of reads go first, then one MFMA group and one read group alternate,
// then the last PF MFMA groups.
constexpr int kSchedDsRead = 0x100, kSchedMfma = 0x008;
template <int N, int PF, int M, int R = 1>
__device__ __forceinline__ void sched_reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, PF * R, 0);
#pragma unroll
  for (int i = 0; i < N - PF; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, M, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, PF * M, 0);
}

}  // namespace peagle
