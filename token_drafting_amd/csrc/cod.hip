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
// Up to 64 blocks of 1024 positions, a hash pass and a select pass (below, before the
// workspace sizes). Beyond, two launches, each hash computed where it is needed
// (re-hashing is cheaper than storing 8 bytes per position):
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

// The per-depth parameters in LDS: kernel arguments indexed by a depth in a loop cost a
// serialized scalar load per iteration, LDS reads do not.
struct DepthLds {
  int32_t m[kMaxDepths];
  int32_t off[kMaxDepths + 1];
  int8_t own[kMaxDepths];  // own_search
};

// Threads 0 .. K fill dl (callers order it with a barrier before use).
__device__ __forceinline__ void load_depths(const CodArgs& a, DepthLds& dl) {
  const int t = threadIdx.x;
  if (t < a.K) {
    dl.m[t] = a.m[t];
    dl.off[t] = a.off[t];
    dl.own[t] = own_search(a, t) ? 1 : 0;
  }
  if (t == a.K) dl.off[t] = a.off[t];
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
  __shared__ int8_t bin_depth[kBins];  // the depth whose candidate bin this is, -1, or -2 (several)
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
    // its depth's region (the region's hashes are distinct: exactly one has the rank). A
    // byte map of the bins tells a position in one lookup whether it is a candidate.
    for (int b = tid; b < kBins; b += kThreads) bin_depth[b] = -1;
    __syncthreads();
    if (tid == 0)
      for (int d = 0; d < K; ++d)
        if (own_search(a, d)) bin_depth[bin_of[d]] = bin_depth[bin_of[d]] == -1 ? (int8_t)d : (int8_t)-2;
    __syncthreads();
    for (int p = tid; p < n; p += kThreads) {
      const int t = (int)(top32(p) >> (32 - kBinBits));
      const int bd = bin_depth[t];
      if (bd >= 0) {
        cand[cbase[bd] + atomicAdd(&cfill[bd], 1)] = hash_of(p);
      } else if (bd == -2) {  // a bin shared by several depths
        for (int d = 0; d < K; ++d)
          if (own_search(a, d) && bin_of[d] == t) cand[cbase[d] + atomicAdd(&cfill[d], 1)] = hash_of(p);
      }
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
  //    block holds the block's top hash bits in registers and, depth after depth (each
  //    threshold a wave-uniform value), counts them with one ballot per 64 positions;
  //    the full hash is needed only where the top 32 bits tie the threshold's. The counts
  //    go to LDS (the histogram's space, no longer needed) when they fit, else to
  //    before_out.
  const int nb = (n + kThreads - 1) / kThreads;
  const bool in_lds = nb * K <= kBins;
  int32_t* const cnt = in_lds ? reinterpret_cast<int32_t*>(hist) : before_out;
  constexpr int kPer = kThreads / kWave;  // positions of a block per lane
  for (int b = wave; b < nb; b += kWaves) {
    uint32_t t[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = b * kThreads + j * kWave + lane;
      t[j] = p < n ? top32(p) : 0xFFFFFFFFu;
    }
    for (int d = 0; d < K; ++d) {
      int c = 0;
      if (a.m[d] > 0) {
        const uint64_t th = thr[d];
        const uint32_t hi = (uint32_t)(th >> 32);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int p = b * kThreads + j * kWave + lane;
          // positions past n carry top bits of all ones: they reach the tie branch at most,
          // which rejects them
          bool keep = t[j] <= hi;
          if (__ballot(t[j] == hi) != 0ull && t[j] == hi)  // rare: compare the low bits
            keep = p < n && hash_of(p) <= th;
          c += __popcll(__ballot(keep));
        }
      }
      if (lane == 0) cnt[(size_t)b * K + d] = c;
    }
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

// Steps 3-4 for the block [base, base + kThreads), given every depth's threshold and this
// block's exclusive prefix of kept positions (LDS), and this thread's hash h:
//   3. ordered compaction with wave ballots: a lane's rank inside its wave, the wave masks in
//      LDS give the rank inside the block (coalesced idx / row_of);
//   4. kept anchors of depth d before each sequence start that falls in this block (the
//      last block also owns cu = n).
__device__ void compact_block(const CodArgs& a, const DepthLds& dl, const int32_t* __restrict__ cu,
                              int cu_first, const uint64_t* thr, const int32_t* before_blk,
                              uint64_t (*wmask)[kWaves], int32_t (*wpre)[kWaves], uint64_t h,
                              int32_t* __restrict__ idx,
                              int32_t* __restrict__ depth_off, int32_t* __restrict__ cu_d,
                              int32_t* __restrict__ row_of) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n = a.n, K = a.K;
  const int base = blockIdx.x * kThreads;
  const int p = base + tid;
  const bool inside = p < n;
  for (int d = 0; d < K; ++d) {
    const bool keep = inside && dl.m[d] > 0 && h <= thr[d];
    const uint64_t ball = __ballot(keep);
    if (lane == 0) wmask[d][wave] = ball;
  }
  __syncthreads();
  // kept positions of the waves before each wave, per depth (lane w of wave d sums the
  // popcounts of waves 0..w-1)
  for (int d = wave; d < K; d += kWaves) {
    const int c = lane < kWaves ? __popcll(wmask[d][lane]) : 0;
    int x = c;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      const int y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    if (lane < kWaves) wpre[d][lane] = x - c;
  }
  __syncthreads();
  for (int d = 0; d < K; ++d) {
    const uint64_t ball = wmask[d][wave];
    const bool keep = (ball >> lane) & 1ull;
    const int r = dl.off[d] + before_blk[d] + wpre[d][wave] + __popcll(ball & ((1ull << lane) - 1ull));
    if (inside) {
      row_of[(size_t)d * n + p] = keep ? r : -1;
      if (keep && r < dl.off[d + 1]) idx[r] = p;
    }
  }
  for (int t = tid; t < K * (a.S + 1); t += kThreads) {
    const int d = t / (a.S + 1), s = t % (a.S + 1);
    const int x = t == tid ? cu_first : cu[s];
    const bool mine = (x >= base && x < base + kThreads && x < n) ||
                      (x >= n && blockIdx.x == gridDim.x - 1);
    if (!mine) continue;
    int v;
    if (x >= n) {
      v = dl.m[d];
    } else {
      const int off = x - base, w = off >> 6, l = off & 63;
      v = before_blk[d] + wpre[d][w] + __popcll(wmask[d][w] & ((1ull << l) - 1ull));
    }
    cu_d[t] = v;
  }
  if (blockIdx.x == 0 && tid <= K) depth_off[tid] = dl.off[tid];
}

__global__ __launch_bounds__(kThreads) void cod_compact_kernel(
    CodArgs a, const int32_t* __restrict__ cu, const uint64_t* __restrict__ thr_in,
    const int32_t* __restrict__ before_in, int32_t* __restrict__ idx,
    int32_t* __restrict__ depth_off, int32_t* __restrict__ cu_d, int32_t* __restrict__ row_of) {
  __shared__ uint64_t thr[kMaxDepths];
  __shared__ uint64_t wmask[kMaxDepths][kWaves];
  __shared__ int32_t wpre[kMaxDepths][kWaves];
  __shared__ int32_t before_blk[kMaxDepths];
  __shared__ DepthLds dl;
  const int tid = threadIdx.x;
  load_depths(a, dl);
  if (tid < a.K) {
    thr[tid] = thr_in[tid];
    before_blk[tid] = before_in[(size_t)blockIdx.x * a.K + tid];
  }
  __syncthreads();
  const int p = blockIdx.x * kThreads + tid;
  const int cu_first = tid < a.K * (a.S + 1) ? cu[tid % (a.S + 1)] : 0;
  compact_block(a, dl, cu, cu_first, thr, before_blk, wmask, wpre,
                splitmix64(a.seed ^ (uint64_t)p), idx, depth_off, cu_d, row_of);
}

// ---- one-pass path for buffers of at most kSmallBlocks blocks ----
// cod_hash_kernel: a workgroup per block hashes its positions and stores them sorted by
// the hash's top 8 bits (a counting sort in LDS: the block's hashes and positions grouped
// by that byte, with each group's count and start). cod_select_small_kernel: every
// workgroup rebuilds, from the counts, the global histogram and each depth's bin and rank;
// loads only those bins' groups (a few hundred hashes per depth at these sizes); finds each
// threshold by a second 8-bit histogram over the candidates and a rank among the few that
// share the threshold's sub-bin; counts its own prefix of kept positions; then compacts
// its block. Two launches, no single-workgroup stage.
constexpr int kSmallBlocks = 64;
constexpr int kCoarseBins = 256;
constexpr int kPool = 4096;  // candidate hashes held at once

struct SmallWs {
  uint64_t* shash;  // [blocks][kThreads] hashes grouped by top byte
  int32_t* spos;    // their positions
  uint32_t* group;  // [blocks][kCoarseBins] group size | group start inside the block << 16
};

__host__ __device__ inline SmallWs small_ws(void* ws, int nb) {
  char* b = static_cast<char*>(ws);
  SmallWs w;
  w.shash = reinterpret_cast<uint64_t*>(b);
  b += (size_t)nb * kThreads * sizeof(uint64_t);
  w.spos = reinterpret_cast<int32_t*>(b);
  b += (size_t)nb * kThreads * sizeof(int32_t);
  w.group = reinterpret_cast<uint32_t*>(b);
  return w;
}

// Orders this wave's LDS accesses before and after it (the lanes of one wave exchange data
// through LDS without a workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, kWave);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, kWave);
  return ((uint64_t)hi << 32) | lo;
}

__global__ __launch_bounds__(kThreads) void cod_hash_kernel(CodArgs a, SmallWs w) {
  __shared__ uint32_t h8[kCoarseBins];
  __shared__ uint32_t st[kCoarseBins];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int blk = blockIdx.x, p = blk * kThreads + tid;
  if (tid < kCoarseBins) h8[tid] = 0;
  __syncthreads();
  const bool inside = p < a.n;
  uint64_t h = 0;
  int t = 0;
  uint32_t slot = 0;
  if (inside) {
    h = splitmix64(a.seed ^ (uint64_t)p);
    t = (int)(h >> 56);
    slot = atomicAdd(&h8[t], 1u);
  }
  __syncthreads();
  // exclusive scan of the group sizes by wave 0 (4 bins per lane)
  if (tid < kWave) {
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = h8[4 * lane + i];
      sum += c[i];
    }
    uint32_t x = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    x -= sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st[4 * lane + i] = x;
      w.group[(size_t)blk * kCoarseBins + 4 * lane + i] = c[i] | (x << 16);
      x += c[i];
    }
  }
  __syncthreads();
  if (inside) {
    const size_t o = (size_t)blk * kThreads + st[t] + slot;
    w.shash[o] = h;
    w.spos[o] = p;
  }
}

__global__ __launch_bounds__(kThreads) void cod_select_small_kernel(
    CodArgs a, const int32_t* __restrict__ cu, const SmallWs w, int32_t* __restrict__ idx,
    int32_t* __restrict__ depth_off, int32_t* __restrict__ cu_d, int32_t* __restrict__ row_of) {
  __shared__ uint32_t ghist[kCoarseBins];  // all blocks
  __shared__ uint32_t phist[kCoarseBins];  // the blocks before this one
  __shared__ uint64_t cand[kPool];
  __shared__ int32_t cpos[kPool];
  __shared__ int32_t goff[kMaxDepths][kSmallBlocks + 1];  // a depth's candidates before block j
  __shared__ uint32_t gst[kMaxDepths][kSmallBlocks];      // start of the bin's group in block j
  __shared__ uint32_t hist2[kWaves][kCoarseBins];         // second-level histograms
  __shared__ uint64_t sub_list[kWaves][kWave];
  __shared__ uint64_t thr[kMaxDepths];
  __shared__ int32_t bin_of[kMaxDepths], rank_in_bin[kMaxDepths], below[kMaxDepths];
  __shared__ int32_t cbase[kMaxDepths + 1];
  __shared__ int32_t before_blk[kMaxDepths];
  __shared__ uint64_t wmask[kMaxDepths][kWaves];
  __shared__ int32_t wpre[kMaxDepths][kWaves];
  __shared__ int32_t sh[kWaves];
  __shared__ uint64_t s_prefix;
  __shared__ int32_t s_rank;
  __shared__ DepthLds dl;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int n = a.n, K = a.K, nb = gridDim.x, blk = blockIdx.x;
  const int base = blk * kThreads;
  constexpr int kParts = kThreads / kCoarseBins;  // threads per bin for the sums
  constexpr int kPerPart = kSmallBlocks / kParts;

  // the compaction's sequence starts, loaded now so that their latency is hidden
  const int ncu = K * (a.S + 1);
  const int cu_first = tid < ncu ? cu[tid % (a.S + 1)] : 0;

  // global histogram of the top 8 bits, and that of the blocks before this one: each bin
  // summed by kParts threads over interleaved blocks (the group words stay in registers
  // for the candidate bins)
  if (tid < kCoarseBins) {
    ghist[tid] = 0;
    phist[tid] = 0;
  }
  load_depths(a, dl);
  __syncthreads();
  const int x = tid % kCoarseBins, part = tid / kCoarseBins;
  uint32_t gw[kPerPart];
  {
#pragma unroll
    for (int i = 0; i < kPerPart; ++i) {
      const int j = part + i * kParts;
      gw[i] = j < nb ? w.group[(size_t)j * kCoarseBins + x] : 0u;
    }
    uint32_t all = 0, pre = 0;
#pragma unroll
    for (int i = 0; i < kPerPart; ++i) {
      const uint32_t v = gw[i] & 0xFFFFu;
      all += v;
      pre += part + i * kParts < blk ? v : 0u;
    }
    atomicAdd(&ghist[x], all);
    atomicAdd(&phist[x], pre);
  }
  __syncthreads();
  // inclusive prefix sums of both histograms over the bins, by wave 0 (4 bins per lane)
  if (tid < kWave) {
    uint32_t g[4], q[4], gsum = 0, qsum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g[i] = ghist[4 * lane + i];
      q[i] = phist[4 * lane + i];
      gsum += g[i];
      qsum += q[i];
    }
    uint32_t gx = gsum, qx = qsum;  // inclusive scan over the lanes
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t gy = __shfl_up(gx, o, kWave), qy = __shfl_up(qx, o, kWave);
      if (lane >= o) {
        gx += gy;
        qx += qy;
      }
    }
    gx -= gsum;
    qx -= qsum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gx += g[i];
      qx += q[i];
      ghist[4 * lane + i] = gx;  // now inclusive prefixes
      phist[4 * lane + i] = qx;
    }
  }
  __syncthreads();
  // depth d: the bin holding the m_d-th smallest hash (prefix before < m_d <= prefix through
  // it), the rank inside it, and the positions before this block in the bins below it (all
  // kept at depth d)
  if (tid < kCoarseBins) {
    const uint32_t gin = ghist[tid], gex = tid > 0 ? ghist[tid - 1] : 0u;
    const uint32_t pex = tid > 0 ? phist[tid - 1] : 0u;
    for (int d = 0; d < K; ++d) {
      const uint32_t m = (uint32_t)dl.m[d];
      if (m > gex && m <= gin) {
        bin_of[d] = tid;
        rank_in_bin[d] = (int)(m - gex);
        below[d] = (int)pex;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int c = 0;
    for (int d = 0; d < K; ++d) {
      cbase[d] = c;
      if (dl.own[d]) {
        const int b = bin_of[d];
        c += (int)(ghist[b] - (b > 0 ? ghist[b - 1] : 0u));
      }
    }
    cbase[K] = c;
  }
  // the threads of each depth's bin leave its group sizes and starts per block
  for (int d = 0; d < K; ++d) {
    if (!dl.own[d] || bin_of[d] != x) continue;
#pragma unroll
    for (int i = 0; i < kPerPart; ++i) {
      const int j = part + i * kParts;
      if (j < nb) {
        goff[d][j + 1] = (int)(gw[i] & 0xFFFFu);
        gst[d][j] = gw[i] >> 16;
      }
    }
  }
  __syncthreads();
  const int ctot = cbase[K];
  if (ctot <= kPool) {
    // a wave per depth with its own search, no workgroup barriers: the depth's candidates,
    // its threshold, and its kept positions before this block
    for (int d = wave; d < K; d += kWaves) {
      if (!dl.own[d]) continue;
      const int j0 = cbase[d], cnt = cbase[d + 1] - j0;
      // 1. the bin's candidates before each block (exclusive prefix over the blocks)
      {
        const int c = lane < nb ? goff[d][lane + 1] : 0;
        int y = c;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int z = __shfl_up(y, o, kWave);
          if (lane >= o) y += z;
        }
        if (lane < nb) goff[d][lane + 1] = y;
        if (lane == 0) goff[d][0] = 0;
      }
      wave_lds_sync();
      // 2. candidate c is entry c - goff[j] of the bin's group in the block j with
      //    goff[j] <= c < goff[j + 1]; four loads in flight per lane
      constexpr int kBatch = 4;
      for (int c0 = 0; c0 < cnt; c0 += kBatch * kWave) {
        size_t src[kBatch];
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
          const int c = c0 + e * kWave + lane;
          src[e] = 0;
          if (c < cnt) {
            int lo = 0, hi = nb - 1;  // the last block whose prefix is <= c
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (goff[d][mid] <= c) lo = mid;
              else hi = mid - 1;
            }
            src[e] = (size_t)lo * kThreads + gst[d][lo] + (c - goff[d][lo]);
          }
        }
        uint64_t hv[kBatch];
        int32_t pv[kBatch];
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
          const bool ok = c0 + e * kWave + lane < cnt;
          hv[e] = ok ? w.shash[src[e]] : 0ull;
          pv[e] = ok ? w.spos[src[e]] : 0;
        }
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
          const int c = c0 + e * kWave + lane;
          if (c < cnt) {
            cand[j0 + c] = hv[e];
            cpos[j0 + c] = pv[e];
          }
        }
      }
      // 3. histogram of the next 8 bits over the candidates: the sub-bin holding the rank
      uint32_t* h2 = hist2[wave];
      for (int b = lane; b < kCoarseBins; b += kWave) h2[b] = 0;
      wave_lds_sync();
      for (int c = lane; c < cnt; c += kWave) atomicAdd(&h2[(cand[j0 + c] >> 48) & 255u], 1u);
      wave_lds_sync();
      const uint32_t r = (uint32_t)rank_in_bin[d];
      int sb = 0, r2 = 0;
      {
        uint32_t hc[4], sum = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          hc[k] = h2[4 * lane + k];
          sum += hc[k];
        }
        uint32_t y = sum;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const uint32_t z = __shfl_up(y, o, kWave);
          if (lane >= o) y += z;
        }
        y -= sum;
        int my_sb = -1, my_r2 = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (r > y && r <= y + hc[k]) {
            my_sb = 4 * lane + k;
            my_r2 = (int)(r - y);
          }
          y += hc[k];
        }
        const int src = __ffsll((unsigned long long)__ballot(my_sb >= 0)) - 1;
        sb = __shfl(my_sb, src, kWave);
        r2 = __shfl(my_r2, src, kWave);
      }
      // 4. the sub-bin's members, compacted by ballot
      int m = 0;
      for (int c0 = 0; c0 < cnt; c0 += kWave) {
        const int c = c0 + lane;
        const uint64_t h = c < cnt ? cand[j0 + c] : 0ull;
        const bool mine = c < cnt && (int)((h >> 48) & 255u) == sb;
        const uint64_t ball = __ballot(mine);
        const int slot = m + __popcll(ball & ((1ull << lane) - 1ull));
        if (mine && slot < kWave) sub_list[wave][slot] = h;
        m += __popcll(ball);
      }
      wave_lds_sync();
      // 5. the member of rank r2 among them (every candidate of the depth if a wave's worth
      //    or more share the sub-bin)
      uint64_t thr_d = 0;
      if (m <= kWave) {
        const uint64_t h = lane < m ? sub_list[wave][lane] : 0ull;
        int smaller = 0;
        for (int k = 0; k < m; ++k) smaller += sub_list[wave][k] < h;
        const uint64_t sel = __ballot(lane < m && smaller == r2 - 1);
        thr_d = lane_u64(h, __ffsll((unsigned long long)sel) - 1);
      } else {
        for (int c0 = 0; c0 < cnt; c0 += kWave) {
          const int c = c0 + lane;
          const uint64_t h = c < cnt ? cand[j0 + c] : 0ull;
          int smaller = 0;
          for (int j = 0; j < cnt; ++j) smaller += cand[j0 + j] < h;
          const uint64_t sel = __ballot(c < cnt && smaller == (int)r - 1);
          if (sel) thr_d = lane_u64(h, __ffsll((unsigned long long)sel) - 1);
        }
      }
      // 6. kept positions before this block: those in the bins below, and the bin's
      //    candidates from the blocks before it that do not exceed the threshold
      const int nbefore = goff[d][blk];
      int kept = 0;
      for (int c0 = 0; c0 < nbefore; c0 += kWave) {
        const int c = c0 + lane;
        kept += __popcll(__ballot(c < nbefore && cand[j0 + c] <= thr_d));
      }
      if (lane == 0) {
        thr[d] = thr_d;
        before_blk[d] = below[d] + kept;
      }
    }
  } else {
    // a bin too full for the pool (not expected at these sizes): radix select over every
    // hash, then count the kept positions before the block
    for (int d = 0; d < K; ++d) {
      if (!dl.own[d]) continue;
      const uint64_t t = radix_select(a, dl.m[d], reinterpret_cast<uint32_t*>(cand), &s_prefix, &s_rank);
      int c = 0;
      for (int p = tid; p < base; p += kThreads) c += splitmix64(a.seed ^ (uint64_t)p) <= t;
      int total;
      (void)block_scan_excl(c, sh, &total);
      if (tid == 0) {
        thr[d] = t;
        before_blk[d] = total;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  if (tid == 0)
    for (int d = 0; d < K; ++d) {
      if (dl.own[d]) continue;
      const bool all = dl.m[d] >= n || d == 0, none = dl.m[d] == 0;
      thr[d] = (all || none) ? ~0ull : thr[d - 1];
      before_blk[d] = none ? 0 : all ? base : before_blk[d - 1];
    }
  __syncthreads();
  const int p = base + tid;
  compact_block(a, dl, cu, cu_first, thr, before_blk, wmask, wpre,
                p < n ? splitmix64(a.seed ^ (uint64_t)p) : 0ull, idx, depth_off, cu_d, row_of);
}

}  // namespace

// Workspace: up to kSmallBlocks blocks, the one-pass path's grouped hashes and positions,
// then the per-block group words (size and start); else the kMaxDepths thresholds, then the
// [blocks][K] exclusive prefixes.
size_t cod_workspace_bytes(int64_t n, int32_t K) {
  const size_t nb = (size_t)((n + kThreads - 1) / kThreads);
  const size_t bytes = nb <= (size_t)kSmallBlocks
                           ? nb * kThreads * (sizeof(uint64_t) + sizeof(int32_t)) +
                                 nb * kCoarseBins * sizeof(uint32_t)
                           : (size_t)kMaxDepths * sizeof(uint64_t) + nb * (size_t)K * sizeof(int32_t);
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_cod_select(const CodArgs& a, const int32_t* cu_seqlens, int32_t* idx,
                             int32_t* depth_off, int32_t* cu_seqlens_d, int32_t* row_of,
                             void* workspace, hipStream_t stream) {
  const int nb = (a.n + kThreads - 1) / kThreads;
  if (nb <= kSmallBlocks) {
    const SmallWs w = small_ws(workspace, nb);
    hipLaunchKernelGGL(cod_hash_kernel, dim3(nb), dim3(kThreads), 0, stream, a, w);
    hipLaunchKernelGGL(cod_select_small_kernel, dim3(nb), dim3(kThreads), 0, stream, a, cu_seqlens,
                       w, idx, depth_off, cu_seqlens_d, row_of);
    return hipGetLastError();
  }
  uint64_t* thr = static_cast<uint64_t*>(workspace);
  int32_t* before = reinterpret_cast<int32_t*>(thr + kMaxDepths);
  hipLaunchKernelGGL(cod_threshold_kernel, dim3(1), dim3(kThreads), 0, stream, a, thr, before);
  hipLaunchKernelGGL(cod_compact_kernel, dim3(nb), dim3(kThreads), 0, stream, a, cu_seqlens, thr,
                     before, idx, depth_off, cu_seqlens_d, row_of);
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
