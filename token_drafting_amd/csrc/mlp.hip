// Second half of the first draft decoder layer and the draft-vocab head, gfx950.
//
// speculators P-EAGLE guide, "Architecture": Llama-style decoder layers; "Key Parameters":
// a flag that disables normalization before the residual connection (so by default the
// residual stream starts from the normalised hidden state). NeMo Automodel PR 2376: the
// P-EAGLE trainer shares EAGLE-3's draft-vocab projection. Per draft row:
//   r  = rms(hidden; w_hidden)  (or hidden when normalization before the residual is off)
//   h1 = r + o W_o^T                       o = attention output, heads flattened
//   h2 = h1 + W_down (silu(W_gate m) * (W_up m)),   m = rms(h1; w_post)
//   token = argmax_v rms(h2; w_final) . W_head[v]  (lowest index on ties)
//
// Every product runs on the DMA-fed GEMM of gemm.h with its own epilogue:
//   o_proj   A = o in bf16 (cast kernel), epilogue adds the residual, h1 in fp32;
//   gate/up  B = W_gate and W_up interleaved by 32 rows (pack kernel), so a lane holds
//            gate and up of the same intermediate column in two neighbouring 32-wide
//            MFMA tiles: the epilogue writes silu(gate) * up in bf16 and the pair never
//            exists in memory;
//   down     epilogue adds h1, h2 in fp32;
//   head     epilogue folds each wave's 64 columns into one order-preserving 64-bit key
//            per row (value bits, then the inverted column), a second kernel takes the
//            largest key of each row: the logits never reach HBM.
#include <algorithm>

#include "common.h"
#include "gemm.h"
#include "layer.h"

namespace peagle {

namespace {

// 1 / sqrt(mean(x^2) + eps) of rows [0, rows) of x [rows, H] (fp32); one wave per row.
__global__ __launch_bounds__(256) void row_inv_rms_kernel(const float* __restrict__ x,
                                                          float* __restrict__ inv, int rows, int H,
                                                          float eps) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float* xr = x + (size_t)r * H;
  float s = 0.f;
  for (int j = lane * 4; j < H; j += 256) {
    const floatx4 v = *reinterpret_cast<const floatx4*>(xr + j);
    s = fmaf(v[0], v[0], fmaf(v[1], v[1], fmaf(v[2], v[2], fmaf(v[3], v[3], s))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) inv[r] = 1.f / sqrtf(s / (float)H + eps);
}

// y[r] = bf16(x[r] / sqrt(mean(x[r]^2) + eps) * w) for fp32 rows; one wave per row.
__global__ __launch_bounds__(256) void rms_rows_kernel(const float* __restrict__ x,
                                                       const uint16_t* __restrict__ w,
                                                       uint16_t* __restrict__ y, int rows, int H,
                                                       float eps) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float* xr = x + (size_t)r * H;
  float s = 0.f;
  for (int j = lane * 8; j < H; j += 512) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(xr + j);
    const floatx4 b = *reinterpret_cast<const floatx4*>(xr + j + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) s = fmaf(a[i], a[i], fmaf(b[i], b[i], s));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  const float inv = 1.f / sqrtf(s / (float)H + eps);
  uint16_t* yr = y + (size_t)r * H;
  for (int j = lane * 8; j < H; j += 512) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(xr + j);
    const floatx4 b = *reinterpret_cast<const floatx4*>(xr + j + 4);
    const bf16x8 wv = as_bf16x8(*reinterpret_cast<const u32x4*>(w + j));
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (__bf16)((i < 4 ? a[i] : b[i - 4]) * inv * (float)wv[i]);
    *reinterpret_cast<bf16x8*>(yr + j) = o;
  }
}

// fp32 -> bf16 (round to nearest even), 8 elements per thread step.
__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ x,
                                                        uint16_t* __restrict__ y, size_t n8) {
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < n8;
       t += (size_t)gridDim.x * blockDim.x) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(x + t * 8);
    const floatx4 b = *reinterpret_cast<const floatx4*>(x + t * 8 + 4);
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (__bf16)(i < 4 ? a[i] : b[i - 4]);
    *reinterpret_cast<bf16x8*>(y + t * 8) = o;
  }
}

// Rows of W_gate and W_up [I, H] interleaved by 32: packed row 64 j + t is gate row
// 32 j + t for t < 32, up row 32 j + t - 32 otherwise (one 32-wide MFMA tile of gate
// columns, then the up tile of the same outputs). 16 bytes per thread step.
__global__ __launch_bounds__(256) void pack_gate_up_kernel(const uint16_t* __restrict__ gate,
                                                           const uint16_t* __restrict__ up,
                                                           uint16_t* __restrict__ out, int I,
                                                           int H) {
  const int per_row = H / 8;
  const size_t total = (size_t)2 * I * per_row;
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < total;
       t += (size_t)gridDim.x * blockDim.x) {
    const int prow = (int)(t / per_row), c = (int)(t % per_row);
    const int j = prow >> 6, tt = prow & 63;
    const uint16_t* src = tt < 32 ? gate + (size_t)(32 * j + tt) * H : up + (size_t)(32 * j + tt - 32) * H;
    *reinterpret_cast<u32x4*>(out + (size_t)prow * H + c * 8) =
        *reinterpret_cast<const u32x4*>(src + c * 8);
  }
}

// out = acc + src (fp32, row stride N) over a wave's tile, with src scaled by inv[min(row,
// n)] * w[col] when kNorm. Rows past M and columns past N load clamped addresses and store
// nothing; the restrict-qualified pointers let the compiler move loads above stores.
//   - Plain residual: the MFMA tiles are visited in turn and the src values of tile t + 1
//     are loaded before tile t is stored, so a tile's loads are in flight while the
//     previous tile stores (loaded and stored one tile at a time, every tile waited for its
//     loads from memory in full).
//   - kNorm: each MFMA tile loads all its src values (and its rows' scales, once per row
//     block) before it stores; the pipelined form needs more registers than the tile has.
template <int NI, int NJ, bool kNorm>
__device__ __forceinline__ void add_tile(const floatx16 (&acc)[NI][NJ], float* __restrict__ out,
                                         const float* __restrict__ src,
                                         const float* __restrict__ inv,
                                         const uint16_t* __restrict__ w, int N, int n, int row0,
                                         int col0, int lane, int M) {
  const int r32 = lane & 31, half = lane >> 5;
  if constexpr (!kNorm) {
    constexpr int NT = NI * NJ;
    float buf[2][16];
    auto load = [&](int t, float (&d)[16]) {
      const int i = t / NJ, j = t % NJ;
      const int colc = min(col0 + 32 * j + r32, N - 1);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = min(row0 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3), M - 1);
        d[r] = src[(size_t)row * N + colc];
      }
    };
    load(0, buf[0]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t + 1 < NT) load(t + 1, buf[(t + 1) & 1]);
      const int i = t / NJ, j = t % NJ;
      const int col = col0 + 32 * j + r32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < M && col < N) out[(size_t)row * N + col] = acc[i][j][r] + buf[t & 1][r];
      }
      __builtin_amdgcn_sched_barrier(0);  // one tile of loads ahead, no more
    }
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float rs[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = min(row0 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3), M - 1);
        rs[r] = inv[min(row, n)];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = col0 + 32 * j + r32;
        const int colc = min(col, N - 1);
        const float wc = bf16_bits_to_f32(w[colc]);
        float pre[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = min(row0 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3), M - 1);
          pre[r] = src[(size_t)row * N + colc] * rs[r] * wc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
          if (row < M && col < N) out[(size_t)row * N + col] = acc[i][j][r] + pre[r];
        }
      }
    }
  }
}

// h1 = residual + acc: the residual is hidden (or, kNorm, rms(hidden) w_hidden, with the
// row's 1/rms from inv; rows past n share row n's input). The choice is a template
// argument so that the plain residual carries no normalisation registers.
template <bool kNorm>
struct StoreResidual {
  static constexpr bool kWaveTile = false;
  static constexpr bool kBlock = true;
  float* out;
  const float* hidden;
  const float* inv;
  const uint16_t* w;
  int N, n;
  template <int NI, int NJ>
  __device__ __forceinline__ void wave_tile(const floatx16 (&acc)[NI][NJ], int row0, int col0,
                                            int lane, int M, int) const {
    add_tile<NI, NJ, kNorm>(acc, out, hidden, inv, w, N, n, row0, col0, lane, M);
  }
};

// out = acc + add (fp32).
struct StoreAdd {
  static constexpr bool kWaveTile = false;
  static constexpr bool kBlock = true;
  float* out;
  const float* add;
  int N;
  template <int NI, int NJ>
  __device__ __forceinline__ void wave_tile(const floatx16 (&acc)[NI][NJ], int row0, int col0,
                                            int lane, int M, int) const {
    add_tile<NI, NJ, false>(acc, out, add, nullptr, nullptr, N, 0, row0, col0, lane, M);
  }
};

// silu(gate) * up from the interleaved columns, bf16 into act [M, I].
struct StoreSwiGLU {
  static constexpr bool kWaveTile = true;
  uint16_t* act;
  int I;
  // acc[i][j]: the 32x32 MFMA tile at rows row0 + 32 i, columns col0 + 32 j. The packed
  // columns come in blocks of 64 (32 gate, then 32 up for the same outputs) and a wave's
  // columns start on a block, so tiles 2c and 2c + 1 give each lane the gate and up value
  // of one output column: no lane exchange, and all 32 lanes of a row store.
  template <int NI, int NJ>
  __device__ __forceinline__ void wave_tile(const floatx16 (&acc)[NI][NJ], int row0, int col0,
                                            int lane, int M, int N) const {
    static_assert(NJ % 2 == 0, "gate and up tiles in pairs");
    const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int c = 0; c < NJ / 2; ++c) {
        const int colb = col0 + 64 * c;  // first packed column of the block
        const int out_col = (colb >> 6) * 32 + r32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float g = acc[i][2 * c][r], u = acc[i][2 * c + 1][r];
          const int row = row0 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
          if (colb < N && row < M)
            act[(size_t)row * I + out_col] = f32_to_bf16_bits(g / (1.f + __expf(-g)) * u);
        }
      }
  }
};

// Order-preserving 32-bit image of a float (larger float -> larger unsigned).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __builtin_bit_cast(uint32_t, f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Per row and per 64-column chunk: the largest (value, lowest column) as one 64-bit key,
// keys [M, ceil(N / 64)]. A wave tile is NJ / 2 whole chunks (col0 a multiple of 64).
struct StoreArgmaxKeys {
  static constexpr bool kWaveTile = true;
  uint64_t* keys;
  int nchunks;
  // Per 64-column chunk a lane holds one key per row it covers (the larger of its two
  // columns), V0 = 16 NI rows. The 32 lanes of a half-wave reduce them by a transposing
  // butterfly: at the exchange with lane l ^ o, each lane keeps the half of its keys that
  // bit o of its lane selects and takes the max with the partner's copy of that half, so
  // the key count halves at every exchange (V0 - V0 / 32 exchanges per lane instead of
  // 5 V0) and lane l ends with the rows V0 / 32 (l % 32) .. + V0 / 32 - 1.
  template <int NI, int NJ>
  __device__ __forceinline__ void wave_tile(const floatx16 (&acc)[NI][NJ], int row0, int col0,
                                            int lane, int M, int N) const {
    static_assert(NJ % 2 == 0, "whole 64-column chunks");
    constexpr int V0 = 16 * NI, VF = V0 / 32;
    static_assert(V0 % 32 == 0, "whole rows per lane after the exchanges");
    const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int c = 0; c < NJ / 2; ++c) {
      const int cc = col0 + 64 * c;  // this chunk's first column
      uint64_t k[V0];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          uint64_t best = 0;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = cc + 32 * j + r32;
            const uint64_t key = col < N ? ((uint64_t)order_key(acc[i][2 * c + j][r]) << 32) |
                                               (uint64_t)(0xFFFFFFFFu - (uint32_t)col)
                                         : 0;
            best = key > best ? key : best;
          }
          k[16 * i + r] = best;
        }
#pragma unroll
      for (int e = 0; e < 5; ++e) {
        const int o = 16 >> e, v = V0 >> (e + 1);  // partner offset, keys kept
        const bool up = (lane & o) != 0;
#pragma unroll
        for (int q = 0; q < v; ++q) {
          const uint64_t send = up ? k[q] : k[q + v];
          const uint64_t keep = up ? k[q + v] : k[q];
          const uint32_t lo = __shfl_xor((uint32_t)send, o, 64);
          const uint32_t hi = __shfl_xor((uint32_t)(send >> 32), o, 64);
          const uint64_t got = ((uint64_t)hi << 32) | lo;
          k[q] = got > keep ? got : keep;
        }
      }
#pragma unroll
      for (int q = 0; q < VF; ++q) {
        const int x = VF * r32 + q, i = x >> 4, r = x & 15;
        const int row = row0 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        // a chunk whose 64 columns all lie past N (the last tile) has no key
        if (row < M && cc < N) keys[(size_t)row * nchunks + (cc >> 6)] = k[q];
      }
    }
  }
};

// token[r] = the column of the largest key of row r.
__global__ __launch_bounds__(256) void argmax_keys_kernel(const uint64_t* __restrict__ keys,
                                                          int32_t* __restrict__ tokens, int rows,
                                                          int nchunks) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  uint64_t best = 0;
  for (int c = 0; c < nchunks; ++c) {
    const uint64_t k = keys[(size_t)r * nchunks + c];
    best = k > best ? k : best;
  }
  tokens[r] = (int32_t)(0xFFFFFFFFu - (uint32_t)best);
}

template <typename Epi>
hipError_t gemm_launch(const uint16_t* A, const uint16_t* W, int M, int N, int K, const Epi& epi,
                       hipStream_t stream) {
  return gemm::launch_dma_gemm(A, W, M, N, K, epi, stream);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct PostLayout {
  size_t a_bf16, h1, m, act, wgu, inv, total;
};

PostLayout post_layout(int64_t n, int64_t T, int32_t H, int32_t QW, int32_t I) {
  PostLayout l;
  l.a_bf16 = 0;
  l.h1 = l.a_bf16 + align256((size_t)T * QW * 2);
  l.m = l.h1 + align256((size_t)T * H * 4);
  l.act = l.m + align256((size_t)T * H * 2);
  l.wgu = l.act + align256((size_t)T * I * 2);
  l.inv = l.wgu + align256((size_t)2 * I * H * 2);
  l.total = l.inv + align256((size_t)(n + 1) * 4);
  return l;
}

unsigned blocks_for(size_t work) {
  return (unsigned)std::max<size_t>(1, std::min<size_t>((work + 255) / 256, 65536));
}

}  // namespace

size_t layer1_post_workspace_bytes(int64_t n, int64_t T, int32_t H, int32_t QW, int32_t I) {
  return post_layout(n, T, H, QW, I).total;
}

hipError_t launch_layer1_post(const Layer1PostArgs& a, const float* attn, const float* hidden,
                              const uint16_t* w_hid, const uint16_t* w_o, const uint16_t* w_post,
                              const uint16_t* w_gate, const uint16_t* w_up,
                              const uint16_t* w_down, float* h2, char* ws, hipStream_t stream) {
  const PostLayout lay = post_layout(a.n, a.T, a.H, a.QW, a.I);
  uint16_t* a_bf16 = reinterpret_cast<uint16_t*>(ws + lay.a_bf16);
  float* h1 = reinterpret_cast<float*>(ws + lay.h1);
  uint16_t* m = reinterpret_cast<uint16_t*>(ws + lay.m);
  uint16_t* act = reinterpret_cast<uint16_t*>(ws + lay.act);
  uint16_t* wgu = reinterpret_cast<uint16_t*>(ws + lay.wgu);
  float* inv = reinterpret_cast<float*>(ws + lay.inv);
  const int rows_in = a.T > a.n ? a.n + 1 : a.n;  // distinct hidden rows
  if (a.norm_before_residual)
    hipLaunchKernelGGL(row_inv_rms_kernel, dim3((rows_in + 3) / 4), dim3(256), 0, stream, hidden,
                       inv, rows_in, a.H, a.eps);
  const size_t n8 = (size_t)a.T * a.QW / 8;
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(blocks_for(n8)), dim3(256), 0, stream, attn, a_bf16,
                     n8);
  hipLaunchKernelGGL(pack_gate_up_kernel, dim3(blocks_for((size_t)2 * a.I * a.H / 8)), dim3(256),
                     0, stream, w_gate, w_up, wgu, a.I, a.H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = a.norm_before_residual
          ? gemm_launch(a_bf16, w_o, a.T, a.H, a.QW,
                        StoreResidual<true>{h1, hidden, inv, w_hid, a.H, a.n}, stream)
          : gemm_launch(a_bf16, w_o, a.T, a.H, a.QW,
                        StoreResidual<false>{h1, hidden, inv, w_hid, a.H, a.n}, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rms_rows_kernel, dim3((a.T + 3) / 4), dim3(256), 0, stream, h1, w_post, m,
                     a.T, a.H, a.eps);
  e = gemm_launch(m, wgu, a.T, 2 * a.I, a.H, StoreSwiGLU{act, a.I}, stream);
  if (e != hipSuccess) return e;
  return gemm_launch(act, w_down, a.T, a.H, a.I, StoreAdd{h2, h1, a.H}, stream);
}

hipError_t launch_rms_rows(const float* x, const uint16_t* w, uint16_t* y, int32_t rows,
                           int32_t H, float eps, hipStream_t stream) {
  hipLaunchKernelGGL(rms_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, x,
                     w, y, rows, H, eps);
  return hipGetLastError();
}

size_t draft_head_workspace_bytes(int64_t T, int32_t H, int32_t V) {
  return align256((size_t)T * H * 2) + align256((size_t)T * ((V + 63) / 64) * 8);
}

hipError_t launch_draft_head(int64_t T, int32_t H, int32_t V, float eps, const float* h,
                             const uint16_t* w_final, const uint16_t* w_head, int32_t* tokens,
                             char* ws, hipStream_t stream) {
  uint16_t* xn = reinterpret_cast<uint16_t*>(ws);
  uint64_t* keys = reinterpret_cast<uint64_t*>(ws + align256((size_t)T * H * 2));
  const int nchunks = (V + 63) / 64;
  hipLaunchKernelGGL(rms_rows_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, h,
                     w_final, xn, (int)T, H, eps);
  hipError_t e = gemm_launch(xn, w_head, (int)T, V, H, StoreArgmaxKeys{keys, nchunks}, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(argmax_keys_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, stream,
                     keys, tokens, (int)T, nchunks);
  return hipGetLastError();
}

}  // namespace peagle
