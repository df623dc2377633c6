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
// fc_gemm: C[M,N] = A[M,K] * B[N,K]^T, bf16 in, fp32 accumulate and out, on
// v_mfma_f32_32x32x16_bf16. Workgroup tile 256x128x64, 4 waves in 2x2, wave tile
// 128x64 (4x2 MFMA tiles). Both operands are K-contiguous, so each MFMA operand is one
// 16-byte LDS read; LDS rows are 128 B with the 16-byte chunk index XOR-swizzled by
// (row >> 1) & 7. The LDS has 64 banks (256 B per bank row, so two tile rows share one)
// and serves 16 lanes of a 16-byte read per cycle: rows 2i and 2i+1 fill the two halves
// of a bank row, and the swizzle gives the 8 even (odd) rows of a 16-row group 8
// different chunk slots.
#include "common.h"
#include "kernels.h"

namespace peagle {

namespace {

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kAChunks = BM * BK / 8 / kThreads;  // 16-byte chunks per thread
constexpr int kBChunks = BN * BK / 8 / kThreads;

__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK * 2 + ((chunk ^ swz_key(row)) << 4); }

// Workgroups are handed to the 8 XCDs round-robin by linear id, and each XCD has its own
// L2. The linear id b is remapped so that XCD b % 8 runs a contiguous range of tile ids,
// and tile ids enumerate the N tiles of one M block together: the N tiles that share an
// A block run at the same time on one XCD and fetch that A block from HBM once.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_tile(int b, int tiles) {
  const int q = tiles / kXcds, r = tiles % kXcds, x = b % kXcds;
  return x * q + min(x, r) + b / kXcds;
}

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

// fc_gemm_dma<DK>: the same tile (256x128, 4 waves of 128x64) fed by LDS DMA through a
// three-stage ring of DK-wide k steps, for K a multiple of 3 * DK: stage k+2 streams in
// while stage k is computed, one barrier per k step, and the fragments of the next
// 16-wide sub-step are read from LDS while the current sub-step's 8 MFMAs run. DK = 64
// takes 144 KB of LDS (one workgroup, one wave per SIMD); DK = 32 takes 72 KB (two
// workgroups, two waves per SIMD). The DMA writes each wave's 1 KB linearly, so the
// swizzle moves to the source: LDS slot (row, c) is filled from global chunk
// c ^ dswz_key(row). Rows past M and columns past N read the last valid row (never
// stored).
constexpr int kStages = 3;
constexpr int kWaves = kThreads / 64;
constexpr int kDmaK = 64;  // k-step width of the DMA-fed kernel (32: two workgroups per CU, measured no faster)

// rows of DK bf16 (2*DK bytes): 256 / (2*DK) rows share one 64-bank row, so the chunk
// slots are XOR-ed with the bank-row index (mod the chunks per row): the 16 rows one LDS
// cycle reads then cover all 64 banks.
template <int DK>
__device__ __forceinline__ int dswz_key(int row) { return (row / (128 / DK)) & (DK / 8 - 1); }
template <int DK>
__device__ __forceinline__ int dswz(int row, int chunk) {
  return row * DK * 2 + ((chunk ^ dswz_key<DK>(row)) << 4);
}

template <int DK>
__global__ __launch_bounds__(kThreads) void fc_gemm_dma_kernel(const uint16_t* __restrict__ A,
                                                               const uint16_t* __restrict__ W,
                                                               float* __restrict__ C, int M, int N,
                                                               int K) {
  constexpr int kABytes = BM * DK * 2, kBBytes = BN * DK * 2;
  constexpr int kADma = kABytes / 1024 / kWaves, kBDma = kBBytes / 1024 / kWaves;  // per wave
  static_assert(kABytes % (1024 * kWaves) == 0 && kBBytes % (1024 * kWaves) == 0, "DMA split");
  constexpr int kRowsPerDma = 1024 / (DK * 2), kChunks = DK / 8;
  __shared__ __attribute__((aligned(1024))) char As0[kABytes];
  __shared__ __attribute__((aligned(1024))) char As1[kABytes];
  __shared__ __attribute__((aligned(1024))) char As2[kABytes];
  __shared__ __attribute__((aligned(1024))) char Bs0[kBBytes];
  __shared__ __attribute__((aligned(1024))) char Bs1[kBBytes];
  __shared__ __attribute__((aligned(1024))) char Bs2[kBBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (N + BN - 1) / BN;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile / ntn) * BM, n0 = (tile % ntn) * BN;
  const int r32 = lane & 31, half = lane >> 5;

  // source byte offsets of this lane's DMA chunks, relative to the tile's (row, k) origin
  uint32_t aoff[kADma], boff[kBDma];
#pragma unroll
  for (int j = 0; j < kADma; ++j) {
    const int row = (wave + j * kWaves) * kRowsPerDma + lane / kChunks;
    const int g = (lane % kChunks) ^ dswz_key<DK>(row);
    aoff[j] = (uint32_t)(((size_t)(min(m0 + row, M - 1) - m0) * K + g * 8) * 2);
  }
#pragma unroll
  for (int j = 0; j < kBDma; ++j) {
    const int row = (wave + j * kWaves) * kRowsPerDma + lane / kChunks;
    const int g = (lane % kChunks) ^ dswz_key<DK>(row);
    boff[j] = (uint32_t)(((size_t)(min(n0 + row, N - 1) - n0) * K + g * 8) * 2);
  }
  auto issue = [&](int ks, char* Ad, char* Bd) {
    const char* ab = uniform_opaque(reinterpret_cast<const char*>(A + (size_t)m0 * K + (size_t)ks * DK));
    const char* bb = uniform_opaque(reinterpret_cast<const char*>(W + (size_t)n0 * K + (size_t)ks * DK));
#pragma unroll
    for (int j = 0; j < kADma; ++j) dma16(ab + lane_opaque(aoff[j]), Ad + (wave + j * kWaves) * 1024);
#pragma unroll
    for (int j = 0; j < kBDma; ++j) dma16(bb + lane_opaque(boff[j]), Bd + (wave + j * kWaves) * 1024);
  };

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](const char* As, const char* Bs) {
    constexpr int SUB = DK / 16;
    bf16x8 af[SUB][4], bfr[SUB][2];
#pragma unroll
    for (int ks = 0; ks < SUB; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[ks][i] = as_bf16x8(*reinterpret_cast<const u32x4*>(As + dswz<DK>(wm * 128 + i * 32 + r32, ks * 2 + half)));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[ks][j] = as_bf16x8(*reinterpret_cast<const u32x4*>(Bs + dswz<DK>(wn * 64 + j * 32 + r32, ks * 2 + half)));
    }
#pragma unroll
    for (int ks = 0; ks < SUB; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[ks][i], bfr[ks][j], acc[i][j]);
    // the 6 fragments of sub-step ks+1 are read while the 8 MFMAs of sub-step ks run
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
#pragma unroll
    for (int ks = 0; ks < SUB - 1; ++ks) {
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 0);
  };

  const int nk = K / DK;
  // stage s of the ring holds k step s, s+3, ...; before step ks a wave lets the DMAs of
  // step ks+1 (kADma + kBDma of them) stay in flight
  auto step = [&](int ks, const char* Ac, const char* Bc, char* An, char* Bn) {
    if (ks + 1 < nk) wait_vm<kADma + kBDma>(); else wait_vm<0>();
    __syncthreads();  // step ks landed for every wave; the stage of step ks-1 is free
    if (ks + 2 < nk) issue(ks + 2, An, Bn);
    compute(Ac, Bc);
  };
  issue(0, As0, Bs0);
  if (nk > 1) issue(1, As1, Bs1);
  for (int ks = 0; ks < nk; ks += kStages) {  // nk is a multiple of kStages
    step(ks, As0, Bs0, As2, Bs2);
    step(ks + 1, As1, Bs1, As0, Bs0);
    step(ks + 2, As2, Bs2, As1, Bs1);
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
// fp32 accumulation of the exact bf16 products.
__global__ __launch_bounds__(256) void fc_row_kernel(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ W,
                                                    float* __restrict__ out, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
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

}  // namespace

hipError_t launch_fuse(const FuseArgs& a, const int32_t* idx, const uint16_t* aux,
                       const uint16_t* fc_weight, const uint16_t* mask_hidden,
                       const int32_t* tokens, const uint16_t* embed, float* hidden_out,
                       uint16_t* embed_out, hipStream_t stream) {
  (void)idx;  // depth-0 row r is anchor r; depth >= 1 rows need no anchor
  hipError_t e;
  if (a.aux_dim % (kStages * kDmaK) == 0) {
    // depth-0 rows on the DMA-fed kernel, the mask row (first depth-1 row) on its own
    const dim3 grid(((a.H + BN - 1) / BN) * ((a.n + BM - 1) / BM));
    hipLaunchKernelGGL(fc_gemm_dma_kernel<kDmaK>, grid, dim3(kThreads), 0, stream, aux, fc_weight,
                       hidden_out, (int)a.n, a.H, a.aux_dim);
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
