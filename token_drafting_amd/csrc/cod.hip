// COD (Conditional Drop-token) index builder.
//
// Follows the speculators P-EAGLE guide, section "COD Sampling": depth 0 keeps every
// position, depth d keeps about n*r^d (floor n*r_min). Depth d keeps the m_d buffer
// indices p with the smallest SplitMix64(seed XOR p), compared as unsigned 64-bit words
// (SplitMix64 as published by Steele, Lea and Flood, OOPSLA 2014: add the golden gamma,
// then the variant-13 mixer). Taking the m_d smallest of one ranking nests the sets.
// The hash is a bijection, so the m_d-th smallest hash is a unique threshold and depth d
// keeps exactly the p with hash <= threshold.
//
// One workgroup of 1024 threads per block of 1024 positions. The thresholds are cheap
// (a few passes of hashing over n), so every workgroup derives them itself and no
// workgroup waits on another:
//   1. a 12-bit histogram of the hashes locates, for every depth, the bin that holds the
//      m_d-th smallest hash; the handful of hashes in that bin are ranked directly (an
//      8-bit radix select is the fallback for a bin with more than 1024 hashes);
//   2. the workgroup counts the kept positions of every depth before its block;
//   3. ordered compaction of its own block with wave ballots (coalesced idx / row_of);
//   4. cu_seqlens_d for the sequence starts inside its block.
#include "common.h"
#include "kernels.h"

namespace peagle {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Exclusive scan of one value per thread over the 1024-thread block (wave shuffles, then
// the 16 wave totals through LDS). Returns the prefix; *total receives the block sum.
__device__ int block_scan_excl(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int c = sh[w];
    if (w < wave) before += c;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// The rank-th smallest (1-based) hash, by MSB-first radix select with 8-bit digits.
// Slow path, taken only when a 12-bit bin of the fast path holds too many hashes.
__device__ uint64_t radix_select(const CodArgs& a, int rank, uint32_t* hist, uint64_t* s_prefix,
                                 int* s_rank) {
  const int tid = threadIdx.x, n = a.n;
  uint64_t prefix = 0, pmask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int p = tid; p < n; p += kThreads) {
      const uint64_t h = splitmix64(a.seed ^ (uint64_t)p);
      if ((h & pmask) == prefix) atomicAdd(&hist[(h >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int before = 0, b = 0;
      for (; b < 255; ++b) {
        if (before + (int)hist[b] >= rank) break;
        before += hist[b];
      }
      *s_rank = rank - before;
      *s_prefix = prefix | ((uint64_t)b << shift);
    }
    __syncthreads();
    prefix = *s_prefix;
    rank = *s_rank;
    pmask |= 0xFFull << shift;
  }
  return prefix;
}

__global__ __launch_bounds__(kThreads) void cod_select_kernel(
    CodArgs a, const int32_t* __restrict__ cu, int32_t* __restrict__ idx,
    int32_t* __restrict__ depth_off, int32_t* __restrict__ cu_d, int32_t* __restrict__ row_of) {
  constexpr int kBinBits = 12, kBins = 1 << kBinBits, kPerThread = kBins / kThreads;
  constexpr int kCand = 1024;
  __shared__ uint32_t hist[kBins];
  __shared__ uint64_t cand[kCand];
  __shared__ uint64_t thr[kMaxDepths];
  __shared__ int32_t bin_of[kMaxDepths], rank_in_bin[kMaxDepths];
  __shared__ uint64_t wmask[kMaxDepths][kWaves];
  __shared__ int32_t wsum[8][kWaves];
  __shared__ int32_t before_blk[kMaxDepths];
  __shared__ int32_t sh[kWaves];
  __shared__ uint64_t s_prefix;
  __shared__ int32_t s_rank, s_count;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = a.n, K = a.K;

  // 1. thresholds: keep p at depth d iff hash(p) <= thr[d] (m_d == 0 keeps nothing).
  //    One histogram of the top 12 hash bits serves every depth: its prefix sums give the
  //    bin holding the m_d-th smallest hash and the rank inside that bin; the bin's few
  //    hashes (n / 4096 on average) are then ranked directly.
  for (int b = tid; b < kBins; b += kThreads) hist[b] = 0;
  __syncthreads();
  for (int p = tid; p < n; p += kThreads)
    atomicAdd(&hist[splitmix64(a.seed ^ (uint64_t)p) >> (64 - kBinBits)], 1u);
  __syncthreads();
  {
    uint32_t mine[kPerThread];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      mine[i] = hist[tid * kPerThread + i];
      sum += mine[i];
    }
    int total;
    int before = block_scan_excl(sum, sh, &total);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int b = tid * kPerThread + i;
      for (int d = 0; d < K; ++d) {
        const int m = a.m[d];
        if (m > before && m <= before + (int)mine[i]) {
          bin_of[d] = b;
          rank_in_bin[d] = m - before;
        }
      }
      before += mine[i];
    }
  }
  __syncthreads();
  for (int d = 0; d < K; ++d) {
    const int m = a.m[d];
    if (m >= n || m == 0) {
      if (tid == 0) thr[d] = ~0ull;
      continue;
    }
    if (d > 0 && a.m[d - 1] == m) {  // same count, same threshold
      if (tid == 0) thr[d] = thr[d - 1];
      continue;
    }
    const uint32_t b = (uint32_t)bin_of[d];
    if (hist[b] > (uint32_t)kCand) {  // pathological bin: full radix select
      const uint64_t t = radix_select(a, m, hist + 0, &s_prefix, &s_rank);
      if (tid == 0) thr[d] = t;
      __syncthreads();
      // the histogram was overwritten: rebuild it for the depths still to come
      for (int i = tid; i < kBins; i += kThreads) hist[i] = 0;
      __syncthreads();
      for (int p = tid; p < n; p += kThreads)
        atomicAdd(&hist[splitmix64(a.seed ^ (uint64_t)p) >> (64 - kBinBits)], 1u);
      __syncthreads();
      continue;
    }
    if (tid == 0) s_count = 0;
    __syncthreads();
    for (int p = tid; p < n; p += kThreads) {
      const uint64_t h = splitmix64(a.seed ^ (uint64_t)p);
      if ((h >> (64 - kBinBits)) == b) cand[atomicAdd(&s_count, 1)] = h;
    }
    __syncthreads();
    const int c = s_count, want = rank_in_bin[d] - 1;
    for (int i = tid; i < c; i += kThreads) {
      const uint64_t h = cand[i];
      int smaller = 0;
      for (int j = 0; j < c; ++j) smaller += cand[j] < h;
      if (smaller == want) thr[d] = h;  // hashes are distinct: exactly one writer
    }
    __syncthreads();
  }
  __syncthreads();

  // 2. kept positions of every depth before this workgroup's block: one pass over
  //    [0, base), eight depths per pass, reduced over the workgroup.
  const int base = blockIdx.x * kThreads;
  for (int d0 = 0; d0 < K; d0 += 8) {
    int c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = 0;
    for (int p = tid; p < base; p += kThreads) {
      const uint64_t h = splitmix64(a.seed ^ (uint64_t)p);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (d0 + j < K) c[j] += (a.m[d0 + j] > 0 && h <= thr[d0 + j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int v = c[j];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
      if (lane == 0) wsum[j][wave] = v;
    }
    __syncthreads();
    if (tid < 8 && d0 + tid < K) {
      int v = 0;
      for (int w = 0; w < kWaves; ++w) v += wsum[tid][w];
      before_blk[d0 + tid] = v;
    }
    __syncthreads();
  }

  // 3. ordered compaction of the block [base, base + 1024): a wave ballot per depth gives
  //    each lane its rank inside the wave, the wave masks in LDS give the rank inside
  //    the block.
  const int p = base + tid;
  const bool inside = p < n;
  const uint64_t h = splitmix64(a.seed ^ (uint64_t)p);
  for (int d = 0; d < K; ++d) {
    const bool keep = inside && a.m[d] > 0 && h <= thr[d];
    const uint64_t ball = __ballot(keep);
    if (lane == 0) wmask[d][wave] = ball;
  }
  __syncthreads();
  for (int d = 0; d < K; ++d) {
    const uint64_t ball = wmask[d][wave];
    const bool keep = (ball >> lane) & 1ull;
    int r = a.off[d] + before_blk[d] + __popcll(ball & ((1ull << lane) - 1ull));
    for (int w = 0; w < wave; ++w) r += __popcll(wmask[d][w]);
    if (inside) {
      row_of[(size_t)d * n + p] = keep ? r : -1;
      if (keep && r < a.off[d + 1]) idx[r] = p;
    }
  }

  // 4. kept anchors of depth d before each sequence start that falls in this block (the
  //    last block also owns cu = n).
  for (int t = tid; t < K * (a.S + 1); t += kThreads) {
    const int d = t / (a.S + 1), s = t % (a.S + 1);
    const int x = cu[s];
    const bool mine = (x >= base && x < base + kThreads && x < n) ||
                      (x >= n && blockIdx.x == gridDim.x - 1);
    if (!mine) continue;
    int v;
    if (x >= n) {
      v = a.m[d];
    } else {
      const int off = x - base, w = off >> 6, l = off & 63;
      v = before_blk[d] + __popcll(wmask[d][w] & ((1ull << l) - 1ull));
      for (int j = 0; j < w; ++j) v += __popcll(wmask[d][j]);
    }
    cu_d[t] = v;
  }
  if (blockIdx.x == 0 && tid <= K) depth_off[tid] = a.off[tid];
}

}  // namespace

hipError_t launch_cod_select(const CodArgs& a, const int32_t* cu_seqlens, int32_t* idx,
                             int32_t* depth_off, int32_t* cu_seqlens_d, int32_t* row_of,
                             hipStream_t stream) {
  hipLaunchKernelGGL(cod_select_kernel, dim3((a.n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, a, cu_seqlens, idx, depth_off, cu_seqlens_d, row_of);
  return hipGetLastError();
}

}  // namespace peagle
