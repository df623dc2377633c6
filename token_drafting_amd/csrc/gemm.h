// DMA-fed bf16 GEMM shared by the draft-layer stages (gfx950).
//
// C[M,N] = A[M,K] * B[N,K]^T: bf16 operands, both K-contiguous (B in linear-layer layout,
// output-major), fp32 accumulation on v_mfma_f32_32x32x16_bf16; the epilogue functor
// receives every (row, col, value) of the tile that lies inside [M) x [N).
//
// Workgroup tile 256x128, 4 waves of 128x64 (4x2 MFMA tiles). Operands stream into LDS
// by LDS DMA (global_load_lds_dwordx4) through a three-stage ring of DK-wide k steps:
// step k+2 streams in while step k is computed, one barrier per k step, and the
// fragments of the next 16-wide sub-step are read from LDS while the current sub-step's
// 8 MFMAs run. K must be a multiple of 3 DK, or with kTail a multiple of DK (the ring
// then ends with a tail of one or two steps; a separate instantiation, since the tail
// costs the main loop accumulator moves between AGPRs and VGPRs). DK = 64 takes 144 KB of LDS (one workgroup, one wave per SIMD).
//
// The DMA writes each wave's 1 KB linearly, so the LDS swizzle moves to the source: LDS
// slot (row, c) is filled from global chunk c ^ dswz_key(row). Rows past M and columns
// past N read the last valid row and are never stored.
//
// Workgroups go to the 8 XCDs round-robin by linear id, each XCD with its own L2; the
// id is remapped so that XCD b % 8 runs a contiguous range of tile ids, and tile ids
// enumerate the N tiles of one M block together: the N tiles that share an A block run
// at the same time on one XCD and fetch that block from HBM once. The wide variant with
// N tiles in multiples of 8 instead gives each XCD a fixed eighth of the N tiles (below).
#pragma once

#include <type_traits>

#include "common.h"

namespace peagle {
namespace gemm {

// Epilogues with kBlock = true take the wave's whole tile through wave_tile() without
// combining lanes, so any tile width suits them; kWaveTile ones combine lanes.
template <typename E, typename = void>
struct takes_block : std::false_type {};
template <typename E>
struct takes_block<E, std::void_t<decltype(E::kBlock)>> : std::bool_constant<E::kBlock> {};

constexpr int BM = 256, BN = 128;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kStages = 3;
constexpr int kDmaK = 64;  // k-step width (32: two workgroups per CU, measured no faster)
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_tile(int b, int tiles) {
  const int q = tiles / kXcds, r = tiles % kXcds, x = b % kXcds;
  return x * q + min(x, r) + b / kXcds;
}

// rows of DK bf16 (2*DK bytes): 256 / (2*DK) rows share one 64-bank row, so the chunk
// slots are XOR-ed with the bank-row index (mod the chunks per row): the 16 rows one LDS
// cycle reads then cover all 64 banks.
template <int DK>
__device__ __forceinline__ int dswz_key(int row) { return (row / (128 / DK)) & (DK / 8 - 1); }
template <int DK>
__device__ __forceinline__ int dswz(int row, int chunk) {
  return row * DK * 2 + ((chunk ^ dswz_key<DK>(row)) << 4);
}

// Grid for an M x N problem.
inline unsigned grid_tiles(int M, int N) {
  return (unsigned)(((N + BN - 1) / BN) * ((M + BM - 1) / BM));
}

// kSplitK: the reduction is cut into gridDim.x / tiles equal ranges of K columns (K is then
// one range's length, lda the operands' row stride); range s goes to epilogue epi.part(s).
template <int DK, typename Epi, bool kTail, bool kSplitK = false>
__global__ __launch_bounds__(kThreads) void dma_gemm_kernel(const uint16_t* __restrict__ A,
                                                            const uint16_t* __restrict__ W, int M,
                                                            int N, int K, Epi epi, int lda = 0) {
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
  // with a split, consecutive ids (one XCD) take the N tiles of one M block and K range
  const int vt = xcd_tile(blockIdx.x, gridDim.x);
  const int tiles = kSplitK ? ntn * ((M + BM - 1) / BM) : (int)gridDim.x;
  const int tile = kSplitK ? vt % tiles : vt;
  const int split = kSplitK ? vt / tiles : 0;
  const int ld = kSplitK ? lda : K;
  const size_t kbase = (size_t)split * K;  // first K column of this block's range
  const int m0 = (tile / ntn) * BM, n0 = (tile % ntn) * BN;
  const int r32 = lane & 31, half = lane >> 5;

  // source byte offsets of this lane's DMA chunks, relative to the tile's (row, k) origin
  uint32_t aoff[kADma], boff[kBDma];
#pragma unroll
  for (int j = 0; j < kADma; ++j) {
    const int row = (wave + j * kWaves) * kRowsPerDma + lane / kChunks;
    const int g = (lane % kChunks) ^ dswz_key<DK>(row);
    aoff[j] = (uint32_t)(((size_t)(min(m0 + row, M - 1) - m0) * ld + g * 8) * 2);
  }
#pragma unroll
  for (int j = 0; j < kBDma; ++j) {
    const int row = (wave + j * kWaves) * kRowsPerDma + lane / kChunks;
    const int g = (lane % kChunks) ^ dswz_key<DK>(row);
    boff[j] = (uint32_t)(((size_t)(min(n0 + row, N - 1) - n0) * ld + g * 8) * 2);
  }
  auto issue = [&](int ks, char* Ad, char* Bd) {
    const char* ab = uniform_opaque(reinterpret_cast<const char*>(A + (size_t)m0 * ld + kbase + (size_t)ks * DK));
    const char* bb = uniform_opaque(reinterpret_cast<const char*>(W + (size_t)n0 * ld + kbase + (size_t)ks * DK));
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
  if constexpr (!kTail) {
    for (int ks = 0; ks < nk; ks += kStages) {  // nk is a multiple of kStages
      step(ks, As0, Bs0, As2, Bs2);
      step(ks + 1, As1, Bs1, As0, Bs0);
      step(ks + 2, As2, Bs2, As1, Bs1);
    }
  } else {
    int ks = 0;
    for (; ks + kStages <= nk; ks += kStages) {
      step(ks, As0, Bs0, As2, Bs2);
      step(ks + 1, As1, Bs1, As0, Bs0);
      step(ks + 2, As2, Bs2, As1, Bs1);
    }
    if (ks < nk) step(ks, As0, Bs0, As2, Bs2);  // tail: nk % 3 steps
    if (ks + 1 < nk) step(ks + 1, As1, Bs1, As0, Bs0);
  }

  if constexpr (Epi::kWaveTile || takes_block<Epi>::value) {
    // an epilogue that combines lanes, or reads before it writes, gets the wave's whole
    // 128x64 tile, all lanes active
    epi.wave_tile(acc, m0 + wm * 128, n0 + wn * 64, lane, M, N);
  } else {
    const auto out = [&] {
      if constexpr (kSplitK) return epi.part(split); else return epi;
    }();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + j * 32 + r32;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (row < M) out(row, col, acc[i][j][r]);
        }
      }
  }
}

// Wide variant: workgroup tile 256 x BNW (BNW = 256 or 320; N a multiple of BNW), 8 waves
// of 64 x BNW/2 (2 x BNW/64 MFMA tiles), two waves per SIMD. A 64-wide k step moves
// (256 + BNW) x 128 bytes for 2 x 256 x BNW x 64 FLOP: 1.5x (BNW = 256) to 1.66x (320)
// fewer bytes per FLOP than the 256x128 tile. That is what bounds these projections: the
// operand stream a CU can keep in flight (~16 B per clock measured), not the MFMA pipe. The
// LDS holds a two-stage ring (144 KB at BNW = 320): step k+1 streams in while step k is
// computed, one barrier per step. K must be a multiple of 2 x 64. Epilogues that combine
// lanes get the wave's 64 x BNW/2 tile (acc[2][BNW/64]); they need BNW = 256, so that a
// wave's columns are whole 64-column chunks.
constexpr int kWideThreads = 512, kWideWaves = kWideThreads / 64, kWideDK = 64;

template <int BNW, typename Epi>
__global__ __launch_bounds__(kWideThreads) void dma_gemm_wide_kernel(const uint16_t* __restrict__ A,
                                                                     const uint16_t* __restrict__ W,
                                                                     int M, int N, int K, Epi epi) {
  static_assert(!Epi::kWaveTile || BNW == 256, "lane-combining epilogues take 64-column chunks");
  constexpr int DK = kWideDK;
  constexpr int kABytes = BM * DK * 2, kBBytes = BNW * DK * 2;
  constexpr int kADma = kABytes / 1024 / kWideWaves, kBDma = kBBytes / 1024 / kWideWaves;
  static_assert(kABytes % (1024 * kWideWaves) == 0 && kBBytes % (1024 * kWideWaves) == 0, "DMA split");
  constexpr int kRowsPerDma = 1024 / (DK * 2), kChunks = DK / 8;
  constexpr int NI = 2, NJ = BNW / 64, WN = BNW / 2;  // MFMA tiles per wave, wave columns
  __shared__ __attribute__((aligned(1024))) char As0[kABytes];
  __shared__ __attribute__((aligned(1024))) char As1[kABytes];
  __shared__ __attribute__((aligned(1024))) char Bs0[kBBytes];
  __shared__ __attribute__((aligned(1024))) char Bs1[kBBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = N / BNW;
  // With N tiles in multiples of the XCD count (wide outputs: the draft head, the gate/up
  // projection, the 4096-wide fc), XCD x runs N tiles [x nx, (x + 1) nx) of every M block,
  // so its slice of W stays in its L2 while the A blocks, re-read by the 8 XCDs, come from
  // the last-level cache. Else an XCD runs all N tiles of a range of M blocks (W small).
  int mblk, ntile;
  if (ntn % kXcds == 0) {
    const int nx = ntn / kXcds, i = blockIdx.x / kXcds;
    mblk = i / nx;
    ntile = (blockIdx.x % kXcds) * nx + i % nx;
  } else {
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    mblk = tile / ntn;
    ntile = tile % ntn;
  }
  const int m0 = mblk * BM, n0 = ntile * BNW;
  const int r32 = lane & 31, half = lane >> 5;

  uint32_t aoff[kADma], boff[kBDma];
#pragma unroll
  for (int j = 0; j < kADma; ++j) {
    const int row = (wave + j * kWideWaves) * kRowsPerDma + lane / kChunks;
    const int g = (lane % kChunks) ^ dswz_key<DK>(row);
    aoff[j] = (uint32_t)(((size_t)(min(m0 + row, M - 1) - m0) * K + g * 8) * 2);
  }
#pragma unroll
  for (int j = 0; j < kBDma; ++j) {
    const int row = (wave + j * kWideWaves) * kRowsPerDma + lane / kChunks;
    const int g = (lane % kChunks) ^ dswz_key<DK>(row);
    boff[j] = (uint32_t)(((size_t)(min(n0 + row, N - 1) - n0) * K + g * 8) * 2);
  }
  auto issue = [&](int ks, char* Ad, char* Bd) {
    const char* ab = uniform_opaque(reinterpret_cast<const char*>(A + (size_t)m0 * K + (size_t)ks * DK));
    const char* bb = uniform_opaque(reinterpret_cast<const char*>(W + (size_t)n0 * K + (size_t)ks * DK));
#pragma unroll
    for (int j = 0; j < kADma; ++j) dma16(ab + lane_opaque(aoff[j]), Ad + (wave + j * kWideWaves) * 1024);
#pragma unroll
    for (int j = 0; j < kBDma; ++j) dma16(bb + lane_opaque(boff[j]), Bd + (wave + j * kWideWaves) * 1024);
  };

  floatx16 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](const char* As, const char* Bs) {
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks) {
      bf16x8 af[NI], bfr[NJ];
#pragma unroll
      for (int i = 0; i < NI; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(As + dswz<DK>(wm * 64 + i * 32 + r32, ks * 2 + half)));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(Bs + dswz<DK>(wn * WN + j * 32 + r32, ks * 2 + half)));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < NI; ++i) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
  };

  const int nk = K / DK;  // even
  issue(0, As0, Bs0);
  for (int ks = 0; ks < nk; ks += 2) {
    wait_vm<0>();
    __syncthreads();  // step ks landed in stage 0; stage 1 is free
    issue(ks + 1, As1, Bs1);
    compute(As0, Bs0);
    wait_vm<0>();
    __syncthreads();  // step ks+1 landed in stage 1; stage 0 is free
    if (ks + 2 < nk) issue(ks + 2, As0, Bs0);
    compute(As1, Bs1);
  }

  if constexpr (Epi::kWaveTile || takes_block<Epi>::value) {
    epi.wave_tile(acc, m0 + wm * 64, n0 + wn * WN, lane, M, N);
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = n0 + wn * WN + j * 32 + r32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (row < M) epi(row, col, acc[i][j][r]);
        }
      }
  }
}

// Width of the wide variant for an M x N x K problem, or 0 if it does not apply: K a
// multiple of 128, N of 320 or 256, and a full round of workgroups (256 CUs; with fewer,
// the 256x128 tile's larger grid is faster, e.g. 4096 x 640: 32 wide tiles against 80).
// Epilogues that combine lanes (wave_tile) take only the 256-wide tile.
constexpr int kWideMinTiles = 256;
inline int wide_width(int M, int N, int K, bool lane_combining = false) {
  if (K % (2 * kWideDK) != 0 || N <= 0 || M <= 0) return 0;
  const int w = (N % 320 == 0 && !lane_combining) ? 320 : N % 256 == 0 ? 256 : 0;
  if (w == 0 || (long long)(N / w) * ((M + BM - 1) / BM) < kWideMinTiles) return 0;
  return w;
}

// C = A W^T through the fastest DMA-fed kernel that applies: the wide tile (see
// wide_width), else the 256x128 tile (K a multiple of 64; with a tail step when K / 64 is
// not a multiple of 3).
template <typename Epi>
hipError_t launch_dma_gemm(const uint16_t* A, const uint16_t* W, int M, int N, int K,
                           const Epi& epi, hipStream_t stream) {
  const int wide = wide_width(M, N, K, Epi::kWaveTile);
  if (wide != 0) {
    const dim3 grid((unsigned)((N / wide) * ((M + BM - 1) / BM)));
    if constexpr (!Epi::kWaveTile) {
      if (wide == 320) {
        hipLaunchKernelGGL((dma_gemm_wide_kernel<320, Epi>), grid, dim3(kWideThreads), 0, stream,
                           A, W, M, N, K, epi);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((dma_gemm_wide_kernel<256, Epi>), grid, dim3(kWideThreads), 0, stream, A,
                       W, M, N, K, epi);
    return hipGetLastError();
  }
  const dim3 grid(grid_tiles(M, N));
  if ((K / kDmaK) % kStages == 0)
    hipLaunchKernelGGL((dma_gemm_kernel<kDmaK, Epi, false>), grid, dim3(kThreads), 0, stream, A,
                       W, M, N, K, epi);
  else
    hipLaunchKernelGGL((dma_gemm_kernel<kDmaK, Epi, true>), grid, dim3(kThreads), 0, stream, A, W,
                       M, N, K, epi);
  return hipGetLastError();
}

// Epilogues are called per element (row, col, value) inside [M) x [N), or, with
// kWaveTile, once per wave with the wave's accumulators: acc[i][j] is the 32x32 MFMA tile
// at rows row0 + 32 i, columns col0 + 32 j; lane l holds column l % 32 of it, rows
// 8 (r / 4) + 4 (l / 32) + r % 4 in register r.

// fp32 row-major stores of the K ranges of a split GEMM: range s into C[s] (up to 3).
struct StoreF32Parts {
  static constexpr bool kWaveTile = false;
  float* C[3];
  int N;
  struct Part {
    static constexpr bool kWaveTile = false;
    float* C;
    int N;
    __device__ __forceinline__ void operator()(int row, int col, float v) const {
      C[(size_t)row * N + col] = v;
    }
  };
  __device__ __forceinline__ Part part(int s) const {
    return Part{s == 0 ? C[0] : s == 1 ? C[1] : C[2], N};
  }
};

// fp32 row-major store.
struct StoreF32 {
  static constexpr bool kWaveTile = false;
  float* C;
  int N;
  __device__ __forceinline__ void operator()(int row, int col, float v) const {
    C[(size_t)row * N + col] = v;
  }
};

}  // namespace gemm
}  // namespace peagle
