// Fused input stage of the draft forward.
//
// NeMo Automodel PR 2376 (description): depth 0 takes the real token embedding and the
// fc projection of the concatenated target aux hidden states; depths >= 1 take the
// embedding of the reserved ptd_token_id and the fc projection of the learnable
// mask_hidden [1, 3*H_target]. The speculators P-EAGLE guide ("Architecture") says the
// selected target hidden states are concatenated and projected.
//
// Draft rows are depth-major and depth 0 keeps every position, so draft row p of depth
// 0 is anchor p: the projection of aux row p lands directly in hidden_out[p]. The
// projected mask_hidden is one extra GEMM row (row n) and lands in hidden_out[n], the
// first depth-1 row; the fill kernel copies it to the remaining depth >= 1 rows and
// gathers the embedding rows.
//
// The projection runs on the wide DMA-fed GEMM of gemm.h (256 x 320 or 256 x 256 tiles)
// when 3 H_target is a multiple of 128, H a multiple of 320 or 256 and the grid fills the
// chip; else on the 256 x 128 DMA-fed GEMM when 3 H_target is a multiple of 192. Otherwise fc_gemm, register-staged: C[M,N] = A[M,K] * B[N,K]^T, bf16 in, fp32
// accumulate and out, on v_mfma_f32_32x32x16_bf16. Workgroup tile 256x128x64, 4 waves in
// 2x2, wave tile 128x64 (4x2 MFMA tiles). Both operands are K-contiguous, so each MFMA operand is one
// 16-byte LDS read; LDS rows are 128 B with the 16-byte chunk index XOR-swizzled by
// (row >> 1) & 7. The LDS has 64 banks (256 B per bank row, so two tile rows share one)
// and serves 16 lanes of a 16-byte read per cycle: rows 2i and 2i+1 fill the two halves
// of a bank row, and the swizzle gives the 8 even (odd) rows of a 16-row group 8
// different chunk slots.
#include <algorithm>

#include "common.h"
#include "gemm.h"
#include "kernels.h"
#include "variants.h"

namespace peagle {

namespace {

using gemm::BM;
using gemm::BN;
using gemm::kThreads;
using gemm::xcd_tile;
constexpr int BK = 64;
constexpr int kAChunks = BM * BK / 8 / kThreads;  // 16-byte chunks per thread
constexpr int kBChunks = BN * BK / 8 / kThreads;

__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK * 2 + ((chunk ^ swz_key(row)) << 4); }

// Workgroup tiles are remapped over the XCDs as in gemm.h (xcd_tile).
__global__ __launch_bounds__(kThreads) void fc_gemm_kernel(
    const uint16_t* __restrict__ aux, const uint16_t* __restrict__ mask_hidden,
    const uint16_t* __restrict__ W, float* __restrict__ C, int n, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) char As[BM * BK * 2];
  __shared__ __attribute__((aligned(16))) char Bs[BN * BK * 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (N + BN - 1) / BN;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile / ntn) * BM, n0 = (tile % ntn) * BN;

  u32x4 ra[kAChunks], rb[kBChunks];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int q = tid + i * kThreads, row = q >> 3, c = q & 7;
      const int m = m0 + row, k = k0 + c * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m < M && k < K) {
        const uint16_t* src = (m < n) ? aux + (size_t)m * K : mask_hidden;
        v = *reinterpret_cast<const u32x4*>(src + k);
      }
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const int q = tid + i * kThreads, row = q >> 3, c = q & 7;
      const int col = n0 + row, k = k0 + c * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (col < N && k < K) v = *reinterpret_cast<const u32x4*>(W + (size_t)col * K + k);
      rb[i] = v;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int q = tid + i * kThreads;
      *reinterpret_cast<u32x4*>(As + swz(q >> 3, q & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const int q = tid + i * kThreads;
      *reinterpret_cast<u32x4*>(Bs + swz(q >> 3, q & 7)) = rb[i];
    }
  };

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int r32 = lane & 31, half = lane >> 5;
  load_tile(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (k0 + BK < K) load_tile(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + r32;
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(As + swz(row, ks * 2 + half)));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + j * 32 + r32;
        bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(Bs + swz(row, ks * 2 + half)));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + r32;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < M) C[(size_t)row * N + col] = acc[i][j][r];
      }
    }
}

// The projected mask_hidden (one row): out[h] = sum_k x[k] W[h][k], one wave per output,
// fp32 accumulation of the exact bf16 products; block b of 256 threads takes outputs
// 4 b .. 4 b + 3.
__device__ __forceinline__ void fc_row_block(const uint16_t* __restrict__ x,
                                             const uint16_t* __restrict__ W,
                                             float* __restrict__ out, int N, int K, int b) {
  const int lane = threadIdx.x & 63;
  const int h = b * 4 + (threadIdx.x >> 6);
  if (h >= N) return;
  const uint16_t* w = W + (size_t)h * K;
  float acc = 0.f;
  for (int k = lane * 8; k < K; k += 64 * 8) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(x + k);
    const u32x4 b = *reinterpret_cast<const u32x4*>(w + k);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc = fmaf(bf16_bits_to_f32((a[e >> 1] >> (16 * (e & 1))) & 0xFFFFu),
                 bf16_bits_to_f32((b[e >> 1] >> (16 * (e & 1))) & 0xFFFFu), acc);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) out[h] = acc;
}

__global__ __launch_bounds__(256) void fc_row_kernel(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ W,
                                                    float* __restrict__ out, int N, int K) {
  fc_row_block(x, W, out, N, K, blockIdx.x);
}

// Depth >= 1 rows: hidden = projected mask_hidden (row n), embedding of ptd_token_id.
// Depth 0 rows (r < n, anchor r): embedding of tokens[r]. One thread per 16 bytes.
__global__ __launch_bounds__(256) void fuse_fill_kernel(
    const int32_t* __restrict__ tokens, const uint16_t* __restrict__ embed,
    float* __restrict__ hidden, uint16_t* __restrict__ embed_out, int n, int T, int H, int vocab,
    int ptd) {
  const int ech = H / 8, hch = H / 4;  // 16-byte chunks per embed / hidden row
  const size_t total_e = (size_t)T * ech;
  const size_t total_h = (T > n + 1) ? (size_t)(T - n - 1) * hch : 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < total_e + total_h; t += stride) {
    if (t < total_e) {
      const int r = (int)(t / ech), c = (int)(t % ech);
      int tok = (r < n) ? tokens[r] : ptd;
      tok = min(max(tok, 0), vocab - 1);
      *reinterpret_cast<u32x4*>(embed_out + (size_t)r * H + c * 8) =
          *reinterpret_cast<const u32x4*>(embed + (size_t)tok * H + c * 8);
    } else {
      const size_t u = t - total_e;
      const int r = n + 1 + (int)(u / hch), c = (int)(u % hch);
      *reinterpret_cast<floatx4*>(hidden + (size_t)r * H + c * 4) =
          *reinterpret_cast<const floatx4*>(hidden + (size_t)n * H + c * 4);
    }
  }
}

// The K-split fc GEMM's closing steps in one launch. Blocks [0, nsum) sum the partials in
// a fixed order, in place: out = (out + p1) + p2 (p2 may be null), over `count` float4s.
// Blocks past nsum project the mask row into row_out (hidden_out row n, which neither the
// sum nor the partials touch), so that latency-bound product overlaps the sum.
__global__ __launch_bounds__(256) void split_close_kernel(
    float* __restrict__ out, const float* __restrict__ p1, const float* __restrict__ p2,
    size_t count, int nsum, const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
    float* __restrict__ row_out, int N, int K) {
  if ((int)blockIdx.x >= nsum) {
    fc_row_block(x, W, row_out, N, K, (int)blockIdx.x - nsum);
    return;
  }
  const size_t stride = (size_t)nsum * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count; i += stride) {
    floatx4 o = reinterpret_cast<const floatx4*>(out)[i];
    const floatx4 b = reinterpret_cast<const floatx4*>(p1)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] += b[e];
    if (p2 != nullptr) {
      const floatx4 c = reinterpret_cast<const floatx4*>(p2)[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += c[e];
    }
    reinterpret_cast<floatx4*>(out)[i] = o;
  }
}

// Ranges of the reduction the fc GEMM is cut into: 1, or up to 3 when its 256x128 tile grid
// leaves at least half the chip idle. Partial 0 goes to hidden_out rows [0, n); partials 1
// and 2 to space the call writes only afterwards: hidden_out rows n+1 .. (the depth >= 1
// copies) and embed_out, when each holds n x H floats. Each range must be a whole number of
// 64-wide k steps.
int fc_splits(const FuseArgs& a, int cus) {
  const int tiles = (int)gemm::grid_tiles(a.n, a.H);
  if (gemm::wide_width(a.n, a.H, a.aux_dim) != 0 || a.aux_dim % gemm::kDmaK != 0 ||
      2 * tiles > cus)
    return 1;
  const size_t part = (size_t)a.n * a.H * sizeof(float);
  const bool in_hidden = (int64_t)a.T - a.n - 1 >= a.n;
  const bool in_embed = (size_t)a.T * a.H * sizeof(uint16_t) >= part;
  const int nks = a.aux_dim / gemm::kDmaK;
  int s = std::min(1 + (int)in_hidden + (int)in_embed, (cus + tiles - 1) / tiles);
  while (s > 1 && nks % s != 0) --s;
  return s;
}

// fc_norm: x[r] = x[r] / sqrt(mean(x[r]^2) + eps) * w in place; one wave per row.
__global__ __launch_bounds__(256) void rms_inplace_kernel(float* __restrict__ x,
                                                          const uint16_t* __restrict__ w,
                                                          int64_t rows, int H, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float* xr = x + r * H;
  float s = 0.f;
  for (int j = lane * 4; j < H; j += 256) {
    const floatx4 v = *reinterpret_cast<const floatx4*>(xr + j);
    s = fmaf(v[0], v[0], fmaf(v[1], v[1], fmaf(v[2], v[2], fmaf(v[3], v[3], s))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  const float inv = 1.f / sqrtf(s / (float)H + eps);
  for (int j = lane * 4; j < H; j += 256) {
    floatx4 v = *reinterpret_cast<const floatx4*>(xr + j);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = v[i] * inv * bf16_bits_to_f32(w[j + i]);
    *reinterpret_cast<floatx4*>(xr + j) = v;
  }
}

}  // namespace

hipError_t launch_rms_inplace(float* x, const uint16_t* w, int64_t rows, int32_t H, float eps,
                              hipStream_t stream) {
  hipLaunchKernelGGL(rms_inplace_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, x,
                     w, rows, H, eps);
  return hipGetLastError();
}

hipError_t launch_fuse(const FuseArgs& a, const int32_t* idx, const uint16_t* aux,
                       const uint16_t* fc_weight, const uint16_t* mask_hidden,
                       const int32_t* tokens, const uint16_t* embed, float* hidden_out,
                       uint16_t* embed_out, hipStream_t stream) {
  (void)idx;  // depth-0 row r is anchor r; depth >= 1 rows need no anchor
  hipError_t e;
  int cus = 256;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int splits = fc_splits(a, cus);
  if (splits > 1) {
    // the reduction in `splits` ranges of K, one workgroup per (tile, range), then the
    // partials summed in order into hidden_out rows [0, n)
    float* p1 = hidden_out + (size_t)(a.n + 1) * a.H;
    float* p2 = splits > 2 ? reinterpret_cast<float*>(embed_out) : nullptr;
    const gemm::StoreF32Parts parts{{hidden_out, p1, p2 != nullptr ? p2 : p1}, a.H};
    const int klen = a.aux_dim / splits;
    const dim3 grid(gemm::grid_tiles(a.n, a.H) * splits);
    if ((klen / gemm::kDmaK) % gemm::kStages == 0)
      hipLaunchKernelGGL((gemm::dma_gemm_kernel<gemm::kDmaK, gemm::StoreF32Parts, false, true>),
                         grid, dim3(gemm::kThreads), 0, stream, aux, fc_weight, (int)a.n, a.H,
                         klen, parts, a.aux_dim);
    else
      hipLaunchKernelGGL((gemm::dma_gemm_kernel<gemm::kDmaK, gemm::StoreF32Parts, true, true>),
                         grid, dim3(gemm::kThreads), 0, stream, aux, fc_weight, (int)a.n, a.H,
                         klen, parts, a.aux_dim);
    const size_t count = (size_t)a.n * a.H / 4;
    const int nsum = (int)std::min<size_t>((count + 255) / 256, 8192);
    const int nrow = a.T > a.n ? (a.H + 3) / 4 : 0;
    hipLaunchKernelGGL(split_close_kernel, dim3((unsigned)(nsum + nrow)), dim3(256), 0, stream,
                       hidden_out, p1, p2, count, nsum, mask_hidden, fc_weight,
                       hidden_out + (size_t)a.n * a.H, a.H, a.aux_dim);
  } else if (gemm::wide_width(a.n, a.H, a.aux_dim) != 0 ||
             a.aux_dim % (gemm::kStages * gemm::kDmaK) == 0) {
    // depth-0 rows on a DMA-fed kernel, the mask row (first depth-1 row) on its own
    e = gemm::launch_dma_gemm(aux, fc_weight, (int)a.n, a.H, a.aux_dim,
                              gemm::StoreF32{hidden_out, a.H}, stream);
    if (e != hipSuccess) return e;
    if (a.T > a.n)
      hipLaunchKernelGGL(fc_row_kernel, dim3((a.H + 3) / 4), dim3(256), 0, stream, mask_hidden,
                         fc_weight, hidden_out + (size_t)a.n * a.H, a.H, a.aux_dim);
  } else {
    // other K: register-staged kernel, the mask row as GEMM row n
    const int M = (a.T > a.n) ? a.n + 1 : a.n;
    const dim3 grid(((a.H + BN - 1) / BN) * ((M + BM - 1) / BM));
    hipLaunchKernelGGL(fc_gemm_kernel, grid, dim3(kThreads), 0, stream, aux, mask_hidden,
                       fc_weight, hidden_out, a.n, M, a.H, a.aux_dim);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t work = (size_t)a.T * (a.H / 8) + (size_t)(a.T > a.n + 1 ? a.T - a.n - 1 : 0) * (a.H / 4);
  const int blocks = (int)((work + 255) / 256 < 65536 ? (work + 255) / 256 : 65536);
  if (blocks > 0)
    hipLaunchKernelGGL(fuse_fill_kernel, dim3(blocks), dim3(256), 0, stream, tokens, embed,
                       hidden_out, embed_out, a.n, a.T, a.H, a.vocab, a.ptd);
  return hipGetLastError();
}

}  // namespace peagle
