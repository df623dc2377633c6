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
__device__ void compact_block(const CodArgs& a, const int32_t* __restrict__ cu,
                              const uint64_t* thr, const int32_t* before_blk,
                              uint64_t (*wmask)[kWaves], uint64_t h, int32_t* __restrict__ idx,
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

__global__ __launch_bounds__(kThreads) void cod_compact_kernel(
    CodArgs a, const int32_t* __restrict__ cu, const uint64_t* __restrict__ thr_in,
    const int32_t* __restrict__ before_in, int32_t* __restrict__ idx,
    int32_t* __restrict__ depth_off, int32_t* __restrict__ cu_d, int32_t* __restrict__ row_of) {
  __shared__ uint64_t thr[kMaxDepths];
  __shared__ uint64_t wmask[kMaxDepths][kWaves];
  __shared__ int32_t before_blk[kMaxDepths];
  const int tid = threadIdx.x;
  if (tid < a.K) {
    thr[tid] = thr_in[tid];
    before_blk[tid] = before_in[(size_t)blockIdx.x * a.K + tid];
  }
  __syncthreads();
  const int p = blockIdx.x * kThreads + tid;
  compact_block(a, cu, thr, before_blk, wmask, splitmix64(a.seed ^ (uint64_t)p), idx, depth_off,
                cu_d, row_of);
}

// ---- one-pass path for buffers of at most kSmallBlocks blocks ----
// cod_hash_kernel: a workgroup per block stores its positions' hashes and the histogram of
// their top 8 bits. cod_select_small_kernel: every workgroup rebuilds, from those, the
// global histogram, each depth's bin and rank, the candidates and thresholds (the same in
// every workgroup: a few hundred hashes per depth at these sizes), and its own prefix of
// kept positions, then compacts its block. Two launches, no single-workgroup stage.
constexpr int kSmallBlocks = 64;
constexpr int kCoarseBins = 256;
constexpr int kPool = 4096;  // candidate hashes held at once

__global__ __launch_bounds__(kThreads) void cod_hash_kernel(CodArgs a, uint64_t* __restrict__ hashes,
                                                           uint32_t* __restrict__ bhist) {
  __shared__ uint32_t h8[kCoarseBins];
  const int tid = threadIdx.x, p = blockIdx.x * kThreads + tid;
  if (tid < kCoarseBins) h8[tid] = 0;
  __syncthreads();
  if (p < a.n) {
    const uint64_t h = splitmix64(a.seed ^ (uint64_t)p);
    hashes[p] = h;
    atomicAdd(&h8[h >> 56], 1u);
  }
  __syncthreads();
  if (tid < kCoarseBins) bhist[(size_t)blockIdx.x * kCoarseBins + tid] = h8[tid];
}

__global__ __launch_bounds__(kThreads) void cod_select_small_kernel(
    CodArgs a, const int32_t* __restrict__ cu, const uint64_t* __restrict__ hashes,
    const uint32_t* __restrict__ bhist, int32_t* __restrict__ idx, int32_t* __restrict__ depth_off,
    int32_t* __restrict__ cu_d, int32_t* __restrict__ row_of) {
  __shared__ uint32_t ghist[kCoarseBins];  // all blocks
  __shared__ uint32_t phist[kCoarseBins];  // the blocks before this one
  __shared__ uint64_t cand[kPool];
  __shared__ int32_t cpos[kPool];
  __shared__ int32_t csmall[kPool];  // candidates of the same depth below each candidate
  __shared__ uint64_t thr[kMaxDepths];
  __shared__ int32_t bin_of[kMaxDepths], rank_in_bin[kMaxDepths], below[kMaxDepths];
  __shared__ int32_t cbase[kMaxDepths + 1], cfill[kMaxDepths];
  __shared__ int32_t before_blk[kMaxDepths], kept_cnt[kMaxDepths];
  __shared__ int8_t bin_depth[kCoarseBins];
  __shared__ uint64_t wmask[kMaxDepths][kWaves];
  __shared__ int32_t sh[kWaves];
  __shared__ uint64_t s_prefix;
  __shared__ int32_t s_rank;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int n = a.n, K = a.K, nb = gridDim.x, blk = blockIdx.x;
  const int base = blk * kThreads;
  constexpr int kParts = kThreads / kCoarseBins;  // threads per bin for the sums

  // global histogram of the top 8 bits, and that of the blocks before this one: each bin
  // summed by kParts threads over interleaved blocks
  if (tid < kCoarseBins) {
    ghist[tid] = 0;
    phist[tid] = 0;
    bin_depth[tid] = -1;
  }
  if (tid < kMaxDepths) kept_cnt[tid] = 0;
  for (int i = tid; i < kPool; i += kThreads) csmall[i] = 0;
  __syncthreads();
  {
    const int x = tid % kCoarseBins, part = tid / kCoarseBins;
    constexpr int kPerPart = kSmallBlocks / kParts;  // all of a thread's loads in flight at once
    uint32_t v[kPerPart];
#pragma unroll
    for (int i = 0; i < kPerPart; ++i) {
      const int j = part + i * kParts;
      v[i] = j < nb ? bhist[(size_t)j * kCoarseBins + x] : 0u;
    }
    uint32_t all = 0, pre = 0;
#pragma unroll
    for (int i = 0; i < kPerPart; ++i) {
      all += v[i];
      pre += part + i * kParts < blk ? v[i] : 0u;
    }
    atomicAdd(&ghist[x], all);
    atomicAdd(&phist[x], pre);
  }
  __syncthreads();
  // inclusive prefix sums of both histograms over the bins, by wave 0 (4 bins per lane)
  if (tid < kWave) {
    uint32_t g[4], q[4], gs = 0, qs = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g[i] = ghist[4 * lane + i];
      q[i] = phist[4 * lane + i];
      gs += g[i];
      qs += q[i];
    }
    uint32_t gx = gs, qx = qs;  // inclusive scan over the lanes
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t gy = __shfl_up(gx, o, kWave), qy = __shfl_up(qx, o, kWave);
      if (lane >= o) {
        gx += gy;
        qx += qy;
      }
    }
    gx -= gs;
    qx -= qs;
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
      const uint32_t m = (uint32_t)a.m[d];
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
      cfill[d] = 0;
      if (own_search(a, d)) {
        c += (int)(ghist[bin_of[d]] - (bin_of[d] > 0 ? ghist[bin_of[d] - 1] : 0u));
        bin_depth[bin_of[d]] = bin_depth[bin_of[d]] == -1 ? (int8_t)d : (int8_t)-2;
      }
    }
    cbase[K] = c;
  }
  __syncthreads();
  if (cbase[K] <= kPool) {
    // candidates of every depth with its own search, with their positions; the hashes are
    // loaded sixteen at a time before any is examined
    constexpr int kBatch = 16;
    for (int p0 = tid; p0 < n; p0 += kBatch * kThreads) {
      uint64_t hb[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int p = p0 + i * kThreads;
        hb[i] = p < n ? hashes[p] : 0ull;
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int p = p0 + i * kThreads;
        if (p >= n) break;
        const uint64_t h = hb[i];
        const int t = (int)(h >> 56);
        const int bd = bin_depth[t];
        if (bd >= 0) {
          const int slot = cbase[bd] + atomicAdd(&cfill[bd], 1);
          cand[slot] = h;
          cpos[slot] = p;
        } else if (bd == -2) {  // a bin shared by several depths
          for (int d = 0; d < K; ++d)
            if (own_search(a, d) && bin_of[d] == t) {
              const int slot = cbase[d] + atomicAdd(&cfill[d], 1);
              cand[slot] = h;
              cpos[slot] = p;
            }
        }
      }
    }
    __syncthreads();
    // each candidate ranks itself inside its depth's region (distinct hashes: one match);
    // `per` threads share one candidate's comparisons, eight reads in flight each
    const int ctot = cbase[K];
    const int per = max(1, kThreads / max(ctot, 1));
    for (int t = tid; t < ctot * per; t += kThreads) {
      const int i = t / per, part = t - i * per;
      int d = 0;
      while (cbase[d + 1] <= i) ++d;
      const uint64_t h = cand[i];
      const int j1 = cbase[d + 1];
      int smaller = 0;
      int j = cbase[d] + part;
      for (; j + 7 * per < j1; j += 8 * per) {
        uint64_t c[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) c[e] = cand[j + e * per];
#pragma unroll
        for (int e = 0; e < 8; ++e) smaller += c[e] < h;
      }
      for (; j < j1; j += per) smaller += cand[j] < h;
      atomicAdd(&csmall[i], smaller);
    }
    __syncthreads();
    for (int i = tid; i < ctot; i += kThreads) {
      int d = 0;
      while (cbase[d + 1] <= i) ++d;
      if (csmall[i] == rank_in_bin[d] - 1) thr[d] = cand[i];
    }
    __syncthreads();
    // kept positions before this block: those in the bins below, and the candidates of the
    // depth's bin before the block that do not exceed its threshold
    for (int i = tid; i < cbase[K]; i += kThreads) {
      int d = 0;
      while (cbase[d + 1] <= i) ++d;
      if (cpos[i] < base && cand[i] <= thr[d]) atomicAdd(&kept_cnt[d], 1);
    }
    __syncthreads();
    if (tid < K && own_search(a, tid)) before_blk[tid] = below[tid] + kept_cnt[tid];
  } else {
    // a bin too full for the pool (not expected at these sizes): radix select over every
    // hash, then count the kept positions before the block
    for (int d = 0; d < K; ++d) {
      if (!own_search(a, d)) continue;
      const uint64_t t = radix_select(a, a.m[d], reinterpret_cast<uint32_t*>(cand), &s_prefix, &s_rank);
      int c = 0;
      for (int p = tid; p < base; p += kThreads) c += hashes[p] <= t;
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
      if (own_search(a, d)) continue;
      const bool all = a.m[d] >= n || d == 0, none = a.m[d] == 0;
      thr[d] = (all || none) ? ~0ull : thr[d - 1];
      before_blk[d] = none ? 0 : all ? base : before_blk[d - 1];
    }
  __syncthreads();
  const int p = base + tid;
  compact_block(a, cu, thr, before_blk, wmask, p < n ? hashes[p] : 0ull, idx, depth_off, cu_d,
                row_of);
}

}  // namespace

// Workspace: up to kSmallBlocks blocks, the n hashes then the per-block histograms of the
// one-pass path; else the kMaxDepths thresholds, then the [blocks][K] exclusive prefixes.
size_t cod_workspace_bytes(int64_t n, int32_t K) {
  const size_t nb = (size_t)((n + kThreads - 1) / kThreads);
  const size_t bytes = nb <= (size_t)kSmallBlocks
                           ? (size_t)n * sizeof(uint64_t) + nb * kCoarseBins * sizeof(uint32_t)
                           : (size_t)kMaxDepths * sizeof(uint64_t) + nb * (size_t)K * sizeof(int32_t);
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_cod_select(const CodArgs& a, const int32_t* cu_seqlens, int32_t* idx,
                             int32_t* depth_off, int32_t* cu_seqlens_d, int32_t* row_of,
                             void* workspace, hipStream_t stream) {
  const int nb = (a.n + kThreads - 1) / kThreads;
  if (nb <= kSmallBlocks) {
    uint64_t* hashes = static_cast<uint64_t*>(workspace);
    uint32_t* bhist = reinterpret_cast<uint32_t*>(hashes + a.n);
    hipLaunchKernelGGL(cod_hash_kernel, dim3(nb), dim3(kThreads), 0, stream, a, hashes, bhist);
    hipLaunchKernelGGL(cod_select_small_kernel, dim3(nb), dim3(kThreads), 0, stream, a, cu_seqlens,
                       hashes, bhist, idx, depth_off, cu_seqlens_d, row_of);
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
