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
// Two launches, each hash computed where it is needed (re-hashing is cheaper than
// storing 8 bytes per position):
//   cod_threshold_kernel (one workgroup of 1024 threads, O(n)):
//     1. a 12-bit histogram of all n hashes locates, for every depth, the bin that holds
//        the m_d-th smallest hash; the handful of hashes in that bin (n / 4096 on
//        average) are ranked directly (an 8-bit radix select is the fallback for a bin
//        with more than 1024 hashes);
//     2. one more pass counts, for every 1024-position block, the positions each depth
//        keeps there, and writes the exclusive prefix of those counts over the blocks;
//     thresholds and prefixes go to the caller's workspace.
//   cod_compact_kernel (one workgroup per block of 1024 positions):
//     3. ordered compaction of its block with wave ballots (coalesced idx / row_of);
//     4. cu_seqlens_d for the sequence starts inside its block.
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace peagle {

// Scratch of the allocation-free entry point: thresholds and per-block prefixes, the same
// layout as a caller's workspace. Each device holds its own copy for the life of the
// process; host code reaches it only through the address hipGetSymbolAddress returns.
__device__ __align__(256) char scratch[kCodNoAllocScratchBytes];

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

constexpr int kBinBits = 12, kBins = 1 << kBinBits;
constexpr int kCand = 1024;    // candidate hashes held at once (all depths together)
constexpr int kCache = 32768;  // positions whose hash's top 32 bits stay in LDS

// Depth d needs its own threshold search: it keeps some but not all positions, and not the
// same number as depth d - 1 (equal counts give equal thresholds).
__device__ __forceinline__ bool own_search(const CodArgs& a, int d) {
  const int m = a.m[d];
  return m > 0 && m < a.n && (d == 0 || a.m[d - 1] != m);
}

__global__ __launch_bounds__(kThreads) void cod_threshold_kernel(
    CodArgs a, uint64_t* __restrict__ thr_out, int32_t* __restrict__ before_out) {
  constexpr int kPerThread = kBins / kThreads;
  __shared__ uint32_t hist[kBins];  // 12-bit histogram; later the per-block kept counts
  __shared__ uint64_t cand[kCand];
  __shared__ uint32_t hcache[kCache];
  __shared__ uint64_t thr[kMaxDepths];
  __shared__ int32_t bin_of[kMaxDepths], rank_in_bin[kMaxDepths];
  __shared__ int32_t cbase[kMaxDepths + 1], cfill[kMaxDepths];
  __shared__ int32_t sh[kWaves];
  __shared__ uint64_t s_prefix;
  __shared__ int32_t s_rank, s_count;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = a.n, K = a.K;
  const int ncache = min(n, kCache);
  auto hash_of = [&](int p) { return splitmix64(a.seed ^ (uint64_t)p); };
  auto top32 = [&](int p) -> uint32_t {
    return p < ncache ? hcache[p] : (uint32_t)(hash_of(p) >> 32);
  };
  // Depth d's parameters sit in lane d of every wave (K <= 64) and are broadcast with
  // readlane inside the loops, instead of indexing the kernel arguments there.
  auto bcast = [](int v, int d) { return __builtin_amdgcn_readlane(v, d); };
  const int m_v = lane < K ? a.m[lane] : 0;
  const bool own_v = lane < K && own_search(a, lane);

  // 1. thresholds: keep p at depth d iff hash(p) <= thr[d] (m_d == 0 keeps nothing).
  //    One histogram of the top 12 hash bits serves every depth: its prefix sums give the
  //    bin holding the m_d-th smallest hash and the rank inside that bin. The top 32 bits
  //    of the first kCache hashes stay in LDS for the later passes.
  for (int b = tid; b < kBins; b += kThreads) hist[b] = 0;
  __syncthreads();
  for (int p = tid; p < n; p += kThreads) {
    const uint64_t h = hash_of(p);
    if (p < ncache) hcache[p] = (uint32_t)(h >> 32);
    atomicAdd(&hist[h >> (64 - kBinBits)], 1u);
  }
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
        const int m = bcast(m_v, d);
        if (m > before && m <= before + (int)mine[i]) {
          bin_of[d] = b;
          rank_in_bin[d] = m - before;
        }
      }
      before += mine[i];
    }
  }
  __syncthreads();
  // candidate regions of the depths with their own search, one pool for all of them
  if (tid == 0) {
    int c = 0;
    for (int d = 0; d < K; ++d) {
      cbase[d] = c;
      cfill[d] = 0;
      if (own_search(a, d)) c += (int)hist[bin_of[d]];
    }
    cbase[K] = c;
  }
  __syncthreads();
  if (cbase[K] <= kCand) {
    // one pass gathers every depth's candidates, then each candidate ranks itself inside
    // its depth's region (the region's hashes are distinct: exactly one has the rank)
    const int bin_v = own_v ? bin_of[lane] : -1;
    for (int p = tid; p < n; p += kThreads) {
      const int t = (int)(top32(p) >> (32 - kBinBits));
      for (int d = 0; d < K; ++d)
        if (t == bcast(bin_v, d)) cand[cbase[d] + atomicAdd(&cfill[d], 1)] = hash_of(p);
    }
    __syncthreads();
    for (int i = tid; i < cbase[K]; i += kThreads) {
      int d = 0;
      while (cbase[d + 1] <= i) ++d;
      const uint64_t h = cand[i];
      int smaller = 0;
      for (int j = cbase[d]; j < cbase[d + 1]; ++j) smaller += cand[j] < h;
      if (smaller == rank_in_bin[d] - 1) thr[d] = h;
    }
    __syncthreads();
  } else {
    // depth by depth: the bin's hashes ranked directly, or a radix select for a bin with
    // more than kCand hashes
    for (int d = 0; d < K; ++d) {
      if (!own_search(a, d)) continue;
      const uint32_t b = (uint32_t)bin_of[d];
      if (hist[b] > (uint32_t)kCand) {
        const uint64_t t = radix_select(a, a.m[d], reinterpret_cast<uint32_t*>(cand), &s_prefix,
                                        &s_rank);
        if (tid == 0) thr[d] = t;
        __syncthreads();
        continue;
      }
      if (tid == 0) s_count = 0;
      __syncthreads();
      for (int p = tid; p < n; p += kThreads)
        if ((top32(p) >> (32 - kBinBits)) == b) cand[atomicAdd(&s_count, 1)] = hash_of(p);
      __syncthreads();
      const int c = s_count, want = rank_in_bin[d] - 1;
      for (int i = tid; i < c; i += kThreads) {
        const uint64_t h = cand[i];
        int smaller = 0;
        for (int j = 0; j < c; ++j) smaller += cand[j] < h;
        if (smaller == want) thr[d] = h;
      }
      __syncthreads();
    }
  }
  if (tid == 0)
    for (int d = 0; d < K; ++d)
      if (!own_search(a, d)) thr[d] = (a.m[d] >= n || a.m[d] == 0 || d == 0) ? ~0ull : thr[d - 1];
  __syncthreads();

  // 2. kept positions of every depth in each block of kThreads positions: a wave per
  //    block, one ballot per depth and 64 positions; lane d carries depth d's count. The
  //    full hash is needed only where the top 32 bits tie a threshold's. The counts go to
  //    LDS (the histogram's space, no longer needed) when they fit, else to before_out.
  const int nb = (n + kThreads - 1) / kThreads;
  const bool in_lds = nb * K <= kBins;
  int32_t* const cnt = in_lds ? reinterpret_cast<int32_t*>(hist) : before_out;
  const uint32_t thr_hi_v = lane < K ? (uint32_t)(thr[lane] >> 32) : 0u;
  const uint32_t thr_lo_v = lane < K ? (uint32_t)thr[lane] : 0u;
  for (int b = wave; b < nb; b += kWaves) {
    int c = 0;
    for (int j = 0; j < kThreads; j += kWave) {
      const int p = b * kThreads + j + lane;
      const bool inside = p < n;
      const uint32_t t = inside ? top32(p) : 0u;
      for (int d = 0; d < K; ++d) {
        const uint32_t th = (uint32_t)bcast((int)thr_hi_v, d);
        bool keep = inside && bcast(m_v, d) > 0 && t <= th;
        if (keep && t == th)
          keep = (uint32_t)hash_of(p) <= (uint32_t)bcast((int)thr_lo_v, d);
        const uint64_t ball = __ballot(keep);
        if (lane == d) c += __popcll(ball);
      }
    }
    if (lane < K) cnt[(size_t)b * K + lane] = c;
  }
  __syncthreads();
  // exclusive prefix over the blocks, per depth, into before_out
  for (int d = 0; d < K; ++d) {
    int carry = 0;
    for (int b0 = 0; b0 < nb; b0 += kThreads) {
      const int b = b0 + tid;
      const int v = b < nb ? cnt[(size_t)b * K + d] : 0;
      int total;
      const int ex = block_scan_excl(v, sh, &total);
      if (b < nb) before_out[(size_t)b * K + d] = carry + ex;
      carry += total;
    }
  }
  if (tid < K) thr_out[tid] = thr[tid];
}

__global__ __launch_bounds__(kThreads) void cod_compact_kernel(
    CodArgs a, const int32_t* __restrict__ cu, const uint64_t* __restrict__ thr_in,
    const int32_t* __restrict__ before_in, int32_t* __restrict__ idx,
    int32_t* __restrict__ depth_off, int32_t* __restrict__ cu_d, int32_t* __restrict__ row_of) {
  __shared__ uint64_t thr[kMaxDepths];
  __shared__ uint64_t wmask[kMaxDepths][kWaves];
  __shared__ int32_t before_blk[kMaxDepths];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = a.n, K = a.K;
  const int base = blockIdx.x * kThreads;
  if (tid < K) {
    thr[tid] = thr_in[tid];
    before_blk[tid] = before_in[(size_t)blockIdx.x * K + tid];
  }
  __syncthreads();

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

// Workspace: the kMaxDepths thresholds, then the [blocks][K] exclusive prefixes.
size_t cod_workspace_bytes(int64_t n, int32_t K) {
  const size_t nb = (size_t)((n + kThreads - 1) / kThreads);
  const size_t bytes = (size_t)kMaxDepths * sizeof(uint64_t) + nb * (size_t)K * sizeof(int32_t);
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_cod_select(const CodArgs& a, const int32_t* cu_seqlens, int32_t* idx,
                             int32_t* depth_off, int32_t* cu_seqlens_d, int32_t* row_of,
                             void* workspace, hipStream_t stream) {
  uint64_t* thr = static_cast<uint64_t*>(workspace);
  int32_t* before = reinterpret_cast<int32_t*>(thr + kMaxDepths);
  hipLaunchKernelGGL(cod_threshold_kernel, dim3(1), dim3(kThreads), 0, stream, a, thr, before);
  hipLaunchKernelGGL(cod_compact_kernel, dim3((a.n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, a, cu_seqlens, thr, before, idx, depth_off, cu_seqlens_d, row_of);
  return hipGetLastError();
}

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

// Device address of `scratch` on the current device, looked up on the first call there
// (concurrent first calls look up and store the same address).
hipError_t cod_noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace peagle
