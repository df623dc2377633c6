// Attention inputs of the first draft decoder layer, gfx950.
//
// snxtyle/P_Eagle README, "How Speculative Decoding Works", step 3: the drafter's input is
// the concatenation [embeddings ⊕ hidden]; speculators P-EAGLE guide, "Architecture": the
// projected hidden states pass through Llama-style decoder layers. Per draft row:
//   x = [rms(emb; w_emb) ⊕ rms(hidden; w_hidden)]   (RMSNorm: x / sqrt(mean x^2 + eps) w)
//   [q | k | v] = x W_qkv^T                            (bias-free, W_qkv output-major)
//
// NeMo Automodel PR 2376, changelog: every depth >= 1 row takes the projected mask_hidden
// and the ptd embedding, so in this first layer all depth >= 1 rows have the same x and the
// same q, k, v before RoPE. Draft rows are depth-major and depth 0 keeps every position:
// rows 0 .. n-1 are the depth-0 rows and row n (when T > n) is the first depth-1 row. The
// projection therefore runs on n + 1 rows instead of T, and rows n+1 .. T-1 copy row n.
//
// Kernels: layer1_norm_kernel (one wave per row: both RMSNorms, the concatenation, bf16
// into the workspace), the DMA-fed GEMM of gemm.h with an epilogue that splits the
// columns into q, k and v (bf16), and layer1_broadcast_kernel (16-byte copies of row n).
//
// Layers stacked after the first (speculators P-EAGLE guide, "Key Parameters": the number
// of decoder layers is a parameter) take the first layer's output h as their residual
// stream: x = rms(h; w_norm) and [q | k | v] = x W_qkv^T on every row, the depth >= 1 rows
// having diverged in the first layer's attention.
#include <algorithm>

#include "common.h"
#include "gemm.h"
#include "layer.h"

namespace peagle {

namespace {

// x[r] = [rms(embed[r]) * w_emb, rms(hidden[r]) * w_hidden] in bf16; fp32 arithmetic.
__global__ __launch_bounds__(256) void layer1_norm_kernel(const float* __restrict__ hidden,
                                                          const uint16_t* __restrict__ embed,
                                                          const uint16_t* __restrict__ w_emb,
                                                          const uint16_t* __restrict__ w_hid,
                                                          uint16_t* __restrict__ x, int M, int H,
                                                          float eps) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= M) return;
  const uint16_t* e = embed + (size_t)r * H;
  const float* h = hidden + (size_t)r * H;
  float se = 0.f, sh = 0.f;
  for (int j = lane * 8; j < H; j += 512) {
    const bf16x8 ev = as_bf16x8(*reinterpret_cast<const u32x4*>(e + j));
    const floatx4 h0 = *reinterpret_cast<const floatx4*>(h + j);
    const floatx4 h1 = *reinterpret_cast<const floatx4*>(h + j + 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = (float)ev[i], b = i < 4 ? h0[i] : h1[i - 4];
      se = fmaf(a, a, se);
      sh = fmaf(b, b, sh);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    se += __shfl_xor(se, o, 64);
    sh += __shfl_xor(sh, o, 64);
  }
  const float ie = 1.f / sqrtf(se / (float)H + eps), ih = 1.f / sqrtf(sh / (float)H + eps);
  uint16_t* xr = x + (size_t)r * 2 * H;
  for (int j = lane * 8; j < H; j += 512) {
    const bf16x8 ev = as_bf16x8(*reinterpret_cast<const u32x4*>(e + j));
    const bf16x8 we = as_bf16x8(*reinterpret_cast<const u32x4*>(w_emb + j));
    const bf16x8 wh = as_bf16x8(*reinterpret_cast<const u32x4*>(w_hid + j));
    const floatx4 h0 = *reinterpret_cast<const floatx4*>(h + j);
    const floatx4 h1 = *reinterpret_cast<const floatx4*>(h + j + 4);
    bf16x8 oe, oh;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      oe[i] = (__bf16)((float)ev[i] * ie * (float)we[i]);
      oh[i] = (__bf16)((i < 4 ? h0[i] : h1[i - 4]) * ih * (float)wh[i]);
    }
    *reinterpret_cast<bf16x8*>(xr + j) = oe;
    *reinterpret_cast<bf16x8*>(xr + H + j) = oh;
  }
}

// Column c of the projection goes to q (c < nq), k (next nk) or v (last nk), bf16.
struct StoreQKV {
  static constexpr bool kWaveTile = false;
  static constexpr bool kBlock = true;
  uint16_t* q;
  uint16_t* k;
  uint16_t* v;
  int nq, nk;
  // nq and nk are multiples of 64, so each 32-column MFMA tile of the wave lies inside one
  // of q, k, v: the destination is chosen once per tile, not per element
  template <int NI, int NJ>
  __device__ __forceinline__ void wave_tile(const floatx16 (&acc)[NI][NJ], int row0, int col0,
                                            int lane, int M, int N) const {
    const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int cb = col0 + 32 * j;
      if (cb >= N) continue;
      uint16_t* dst;
      int width, c0;
      if (cb < nq) {
        dst = q, width = nq, c0 = cb;
      } else if (cb < nq + nk) {
        dst = k, width = nk, c0 = cb - nq;
      } else {
        dst = v, width = nk, c0 = cb - nq - nk;
      }
      dst += c0 + r32;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
          if (row < M) dst[(size_t)row * width] = f32_to_bf16_bits(acc[i][j][r]);
        }
    }
  }
};

// Rows n+1 .. T-1 of q, k and v copy row n; one 16-byte chunk per thread step.
__global__ __launch_bounds__(256) void layer1_broadcast_kernel(uint16_t* __restrict__ q,
                                                               uint16_t* __restrict__ k,
                                                               uint16_t* __restrict__ v, int n,
                                                               int T, int nq, int nk) {
  const int cq = nq / 8, ck = nk / 8, per_row = cq + 2 * ck;
  const size_t total = (size_t)(T - n - 1) * per_row;
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < total;
       t += (size_t)gridDim.x * blockDim.x) {
    const size_t row = n + 1 + t / per_row;
    const int c = (int)(t % per_row);
    uint16_t* base;
    int width, cc;
    if (c < cq) {
      base = q, width = nq, cc = c;
    } else if (c < cq + ck) {
      base = k, width = nk, cc = c - cq;
    } else {
      base = v, width = nk, cc = c - cq - ck;
    }
    *reinterpret_cast<u32x4*>(base + row * width + cc * 8) =
        *reinterpret_cast<const u32x4*>(base + (size_t)n * width + cc * 8);
  }
}

}  // namespace

size_t layer1_workspace_bytes(int64_t n, int64_t T, int32_t H) {
  const int64_t M = T > n ? n + 1 : n;
  return ((size_t)M * 2 * H * 2 + 255) & ~(size_t)255;
}

hipError_t launch_layer1_qkv(const Layer1Args& a, const float* hidden, const uint16_t* embed,
                             const uint16_t* w_emb, const uint16_t* w_hid, const uint16_t* w_qkv,
                             uint16_t* q, uint16_t* k, uint16_t* v, char* ws, hipStream_t stream) {
  const int M = a.T > a.n ? a.n + 1 : a.n;
  const int K = 2 * a.H, nq = a.Hq * a.D, nk = a.Hkv * a.D, N = nq + 2 * nk;
  uint16_t* x = reinterpret_cast<uint16_t*>(ws);
  hipLaunchKernelGGL(layer1_norm_kernel, dim3((M + 3) / 4), dim3(256), 0, stream, hidden, embed,
                     w_emb, w_hid, x, M, a.H, a.eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = gemm::launch_dma_gemm(x, w_qkv, M, N, K, StoreQKV{q, k, v, nq, nk}, stream);
  if (e != hipSuccess) return e;
  if (a.T > a.n + 1) {
    const size_t work = (size_t)(a.T - a.n - 1) * (N / 8);
    const unsigned blocks = (unsigned)std::min<size_t>((work + 255) / 256, 65536);
    hipLaunchKernelGGL(layer1_broadcast_kernel, dim3(blocks), dim3(256), 0, stream, q, k, v, a.n,
                       a.T, nq, nk);
  }
  return hipGetLastError();
}

size_t layer_qkv_workspace_bytes(int64_t T, int32_t H) {
  return ((size_t)T * H * 2 + 255) & ~(size_t)255;
}

hipError_t launch_layer_qkv(const LayerArgs& a, const float* h, const uint16_t* w_norm,
                            const uint16_t* w_qkv, uint16_t* q, uint16_t* k, uint16_t* v,
                            char* ws, hipStream_t stream) {
  const int nq = a.Hq * a.D, nk = a.Hkv * a.D, N = nq + 2 * nk;
  uint16_t* x = reinterpret_cast<uint16_t*>(ws);
  hipError_t e = launch_rms_rows(h, w_norm, x, a.T, a.H, a.eps, stream);
  if (e != hipSuccess) return e;
  return gemm::launch_dma_gemm(x, w_qkv, a.T, N, a.H, StoreQKV{q, k, v, nq, nk}, stream);
}

}  // namespace peagle
