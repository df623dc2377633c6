// Depth-weighted cross-entropy of the draft rows and its gradient, gfx950.
//
// NeMo Automodel PR 2376 (description): the P-EAGLE trainer shares EAGLE-3's draft-vocab
// projection and its 0.8**d weighted-mean loss schedule; its validation run starts near
// ln(draft vocab), and out-of-draft-vocab targets are masked. Read as: the loss of depth d
// is the mean cross-entropy lse(x) - x[label] over the depth's rows with a label in
// [0, V); the total is sum_d decay^d L_d / sum_d decay^d over the depths that have such a
// row; d total / d x = decay^d / (W n_d) (softmax(x) - onehot(label)) on those rows, 0 on
// masked rows.
//
// Kernels (HBM-bound: the logits are read once for the statistics and once more, mostly
// from cache, for the gradient, which is written in bf16):
//   ce_count_kernel   unmasked rows per depth (a workgroup per depth).
//   ce_rows_kernel    a workgroup per row: online max / sum of exp over 16-byte chunks,
//                     the row's loss, and the row's gradient (a second read of the row);
//                     ce_rows_reg_kernel for V <= 16384 with V % 8 == 0 gives each wave a
//                     row, keeps it in registers and reads it once.
//   ce_reduce_kernel  one workgroup: per-depth means in a fixed order (fp64) and the
//                     weighted total, so the scalar is the same on every run.
#include <algorithm>

#include "bwd.h"
#include "common.h"

namespace peagle {

namespace {

constexpr int kCeThreads = 256;

__device__ __forceinline__ float depth_weight(float decay, int d) {
  float w = 1.f;
  for (int e = 0; e < d; ++e) w *= decay;
  return w;
}

__global__ __launch_bounds__(kCeThreads) void ce_count_kernel(const int32_t* __restrict__ labels,
                                                              const int32_t* __restrict__ depth_off,
                                                              int T, int V,
                                                              int32_t* __restrict__ cnt) {
  __shared__ int part[kCeThreads / 64];
  const int d = blockIdx.x, tid = threadIdx.x;
  const int a = min(max(depth_off[d], 0), T), b = min(max(depth_off[d + 1], a), T);
  int c = 0;
  for (int r = a + tid; r < b; r += kCeThreads) c += (labels[r] >= 0 && labels[r] < V) ? 1 : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if ((tid & 63) == 0) part[tid >> 6] = c;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int w = 0; w < kCeThreads / 64; ++w) s += part[w];
    cnt[d] = s;
  }
}

// Merge (m2, s2) into the running (max, sum of exp(x - max)) pair.
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  const float mn = fmaxf(m, m2);
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}

// Logits t .. t+7 of a row (bf16 -> fp32); past V: -inf. kVec: one 16-byte load (V % 8 == 0).
template <bool kVec>
__device__ __forceinline__ void load8(const uint16_t* row, int t, int V, float (&x)[8]) {
  if constexpr (kVec) {
    if (t < V) {
      const bf16x8 b = as_bf16x8(*reinterpret_cast<const u32x4*>(row + t));
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (float)b[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = -INFINITY;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = t + e < V ? bf16_bits_to_f32(row[t + e]) : -INFINITY;
  }
}

template <bool kVec>
__global__ __launch_bounds__(kCeThreads) void ce_rows_kernel(
    const uint16_t* __restrict__ logits, const int32_t* __restrict__ labels,
    const int32_t* __restrict__ depth_off, const int32_t* __restrict__ cnt, int K, int T, int V,
    float decay, float* __restrict__ row_loss, uint16_t* __restrict__ dlogits) {
  __shared__ float sm[kCeThreads / 64], ss[kCeThreads / 64];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* row = logits + (size_t)r * V;
  constexpr int kStep = kCeThreads * 8;
  float m = -INFINITY, s = 0.f;
  for (int t = tid * 8; t < V; t += kStep) {
    float x[8];
    load8<kVec>(row, t, V, x);
    float cm = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, x[e]);
    if (cm == -INFINITY) continue;
    float cs = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) cs += __expf(x[e] - cm);
    ms_merge(m, s, cm, cs);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    ms_merge(m, s, m2, s2);
  }
  if (lane == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  m = sm[0];
  s = ss[0];
#pragma unroll
  for (int w = 1; w < kCeThreads / 64; ++w) ms_merge(m, s, sm[w], ss[w]);
  const float lse = m + __logf(s);
  const int label = labels[r];
  const bool valid = label >= 0 && label < V;
  if (tid == 0) row_loss[r] = valid ? lse - bf16_bits_to_f32(row[label]) : 0.f;
  if (dlogits == nullptr) return;

  const int d = min(max(upper_index(depth_off, K + 1, r), 0), K - 1);
  float W = 0.f;
  for (int e = 0; e < K; ++e)
    if (cnt[e] > 0) W += depth_weight(decay, e);
  const float c = (valid && cnt[d] > 0) ? depth_weight(decay, d) / (W * (float)cnt[d]) : 0.f;
  uint16_t* grow = dlogits + (size_t)r * V;
  for (int t = tid * 8; t < V; t += kStep) {
    float x[8];
    load8<kVec>(row, t, V, x);
    float g[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = c * (__expf(x[e] - lse) - (t + e == label ? 1.f : 0.f));
    if constexpr (kVec) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)g[e];
      *reinterpret_cast<bf16x8*>(grow + t) = o;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (t + e < V) grow[t + e] = f32_to_bf16_bits(g[e]);
    }
  }
}

// The same for V % 8 == 0 and V <= 512 NCH, one wave per row (4 rows per workgroup, no LDS
// or barrier): the row is read once into registers (NCH 16-byte chunks per lane) and the
// gradient is formed from them.
template <int NCH>
__global__ __launch_bounds__(kCeThreads) void ce_rows_reg_kernel(
    const uint16_t* __restrict__ logits, const int32_t* __restrict__ labels,
    const int32_t* __restrict__ depth_off, const int32_t* __restrict__ cnt, int K, int T, int V,
    float decay, float* __restrict__ row_loss, uint16_t* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (kCeThreads / 64) + (threadIdx.x >> 6);
  if (r >= T) return;
  const uint16_t* row = logits + (size_t)r * V;
  constexpr int kStep = 64 * 8;
  u32x4 raw[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int t = lane * 8 + c * kStep;
    raw[c] = t < V ? *reinterpret_cast<const u32x4*>(row + t) : u32x4{0u, 0u, 0u, 0u};
  }
  float m = -INFINITY, s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (lane * 8 + c * kStep >= V) continue;
    const bf16x8 b = as_bf16x8(raw[c]);
    float cm = (float)b[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, (float)b[e]);
    float cs = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) cs += __expf((float)b[e] - cm);
    ms_merge(m, s, cm, cs);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    ms_merge(m, s, m2, s2);
  }
  const float lse = m + __logf(s);
  const int label = labels[r];
  const bool valid = label >= 0 && label < V;
  if (lane == 0) row_loss[r] = valid ? lse - bf16_bits_to_f32(row[label]) : 0.f;
  if (dlogits == nullptr) return;

  const int d = min(max(upper_index(depth_off, K + 1, r), 0), K - 1);
  float W = 0.f;
  for (int e = 0; e < K; ++e)
    if (cnt[e] > 0) W += depth_weight(decay, e);
  const float cf = (valid && cnt[d] > 0) ? depth_weight(decay, d) / (W * (float)cnt[d]) : 0.f;
  uint16_t* grow = dlogits + (size_t)r * V;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int t = lane * 8 + c * kStep;
    if (t >= V) continue;
    const bf16x8 b = as_bf16x8(raw[c]);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      o[e] = (__bf16)(cf * (__expf((float)b[e] - lse) - (t + e == label ? 1.f : 0.f)));
    *reinterpret_cast<bf16x8*>(grow + t) = o;
  }
}

__global__ __launch_bounds__(1024) void ce_reduce_kernel(const float* __restrict__ row_loss,
                                                         const int32_t* __restrict__ depth_off,
                                                         const int32_t* __restrict__ cnt, int K,
                                                         int T, float decay,
                                                         float* __restrict__ loss_out,
                                                         float* __restrict__ depth_loss) {
  __shared__ double part[16];
  const int tid = threadIdx.x;
  double num = 0.0, den = 0.0;
  for (int d = 0; d < K; ++d) {
    const int a = min(max(depth_off[d], 0), T), b = min(max(depth_off[d + 1], a), T);
    double acc = 0.0;
    for (int r = a + tid; r < b; r += 1024) acc += (double)row_loss[r];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if ((tid & 63) == 0) part[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
      double sum = 0.0;
      for (int w = 0; w < 16; ++w) sum += part[w];
      const int n = cnt[d];
      const double ld = n > 0 ? sum / n : 0.0;
      if (depth_loss != nullptr) depth_loss[d] = n > 0 ? (float)ld : __builtin_nanf("");
      if (n > 0) {
        const double w = (double)depth_weight(decay, d);
        num += w * ld;
        den += w;
      }
    }
    __syncthreads();
  }
  if (tid == 0) loss_out[0] = den > 0.0 ? (float)(num / den) : 0.f;
}

}  // namespace

size_t depth_ce_workspace_bytes(int64_t T, int32_t K) {
  return ((size_t)T * 4 + 255) / 256 * 256 + ((size_t)K * 4 + 255) / 256 * 256;
}

hipError_t launch_depth_ce(int64_t T, int32_t K, int32_t V, const int32_t* depth_off,
                           const uint16_t* logits, const int32_t* labels, float decay,
                           float* loss_out, float* depth_loss, uint16_t* dlogits, char* ws,
                           hipStream_t stream) {
  float* row_loss = reinterpret_cast<float*>(ws);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + ((size_t)T * 4 + 255) / 256 * 256);
  hipLaunchKernelGGL(ce_count_kernel, dim3(K), dim3(kCeThreads), 0, stream, labels, depth_off,
                     (int)T, V, cnt);
  const bool vec = V % 8 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0 &&
                   (dlogits == nullptr || (reinterpret_cast<uintptr_t>(dlogits) & 15) == 0);
  const int nch = (V + 64 * 8 - 1) / (64 * 8);  // 16-byte chunks per lane, a wave per row
  const dim3 wgrid((unsigned)((T + kCeThreads / 64 - 1) / (kCeThreads / 64)));
#define PEAGLE_CE_REG(N)                                                                      \
  hipLaunchKernelGGL(ce_rows_reg_kernel<N>, wgrid, dim3(kCeThreads), 0, stream, logits,      \
                     labels, depth_off, cnt, K, (int)T, V, decay, row_loss, dlogits)
  if (vec && nch <= 2)
    PEAGLE_CE_REG(2);
  else if (vec && nch <= 4)
    PEAGLE_CE_REG(4);
  else if (vec && nch <= 8)
    PEAGLE_CE_REG(8);
  else if (vec && nch <= 16)
    PEAGLE_CE_REG(16);
  else if (vec && nch <= 32)
    PEAGLE_CE_REG(32);
#undef PEAGLE_CE_REG
  else if (vec)
    hipLaunchKernelGGL(ce_rows_kernel<true>, dim3((unsigned)T), dim3(kCeThreads), 0, stream,
                       logits, labels, depth_off, cnt, K, (int)T, V, decay, row_loss, dlogits);
  else
    hipLaunchKernelGGL(ce_rows_kernel<false>, dim3((unsigned)T), dim3(kCeThreads), 0, stream,
                       logits, labels, depth_off, cnt, K, (int)T, V, decay, row_loss, dlogits);
  hipLaunchKernelGGL(ce_reduce_kernel, dim3(1), dim3(1024), 0, stream, row_loss, depth_off, cnt,
                     K, (int)T, decay, loss_out, depth_loss);
  return hipGetLastError();
}

}  // namespace peagle
