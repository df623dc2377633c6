// Greedy verification: draft argmax vs target argmax, longest accepted prefix.
//
// Speculators P-EAGLE guide, "Inference Process": the target verifies all draft tokens in
// one forward pass and the longest correct prefix is accepted. With greedy decoding a
// draft token is correct iff it equals the target's argmax at the same depth; draft and
// target share one vocabulary here. Ties go to the lowest index.
//
// One workgroup (4 waves) per draft. Each wave scans whole [V] rows with streaming loads,
// four in flight per lane. Every lane folds its 16-byte chunks into one integer key that
// orders like (value, -index), so the argmax with the lowest-index tie rule is a plain
// unsigned max; a butterfly across the wave finishes it. The bf16 value is mapped to an
// order-preserving 16-bit code (sign-magnitude to offset binary, -0 folded onto +0 so
// that equal values tie). Then wave 0 takes one ballot over the K match bits; the
// accepted length is the number of trailing ones of that mask.
#include <algorithm>

#include "common.h"
#include "variants.h"
#include "kernels.h"

namespace peagle {

namespace {

__device__ __forceinline__ uint32_t order16(uint32_t b) {
  b = (b == 0x8000u) ? 0u : b;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

// Key type: value code above, bit-inverted index below (smaller index -> larger key).
template <typename Key>
struct ArgKey;
template <>
struct ArgKey<uint32_t> {
  __device__ static uint32_t make(uint32_t bits, uint32_t i) { return (order16(bits) << 16) | (0xFFFFu - i); }
  __device__ static uint32_t index(uint32_t k) { return 0xFFFFu - (k & 0xFFFFu); }
  __device__ static uint32_t shfl(uint32_t k, int m) { return (uint32_t)__shfl_xor((int)k, m, 64); }
};
template <>
struct ArgKey<uint64_t> {
  __device__ static uint64_t make(uint32_t bits, uint32_t i) {
    return ((uint64_t)order16(bits) << 32) | (uint64_t)(0xFFFFFFFFu - i);
  }
  __device__ static uint32_t index(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }
  __device__ static uint64_t shfl(uint64_t k, int m) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)k, m, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(k >> 32), m, 64);
    return ((uint64_t)hi << 32) | lo;
  }
};

template <typename Key>
__device__ uint32_t row_argmax(const uint16_t* __restrict__ row, int V, bool vec, int lane) {
  Key best = 0;
  int done = 0;
  if (vec) {
    const int nch = V / 8;
    const u32x4* src = reinterpret_cast<const u32x4*>(row);
    auto fold = [&](const u32x4& w, int c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const Key k = ArgKey<Key>::make(bits, (uint32_t)(c * 8 + e));
        best = k > best ? k : best;
      }
    };
    // kUnroll independent 16-byte loads in flight per lane before any is folded
    constexpr int kUnroll = 4;
    int c = lane;
    for (; c + 64 * (kUnroll - 1) < nch; c += 64 * kUnroll) {
      u32x4 w[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) w[u] = __builtin_nontemporal_load(src + c + 64 * u);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) fold(w[u], c + 64 * u);
    }
    for (; c < nch; c += 64) fold(__builtin_nontemporal_load(src + c), c);
    done = nch * 8;
  }
  for (int i = done + lane; i < V; i += 64) {
    const Key k = ArgKey<Key>::make(row[i], (uint32_t)i);
    best = k > best ? k : best;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const Key o = ArgKey<Key>::shfl(best, m);
    best = o > best ? o : best;
  }
  return ArgKey<Key>::index(best);
}

// One workgroup per draft: the 2K row argmaxes (draft rows of Vd, target rows of Vt),
// then one ballot over the K matches. With kMap the draft token's target id is
// d2t[draft token] (a draft vocabulary smaller than the target's).
template <typename Key, bool kMap>
__global__ __launch_bounds__(256) void accept_kernel(const uint16_t* __restrict__ draft,
                                                     const uint16_t* __restrict__ target,
                                                     const int32_t* __restrict__ d2t,
                                                     int32_t* __restrict__ dtok,
                                                     int32_t* __restrict__ ttok,
                                                     int32_t* __restrict__ alen, int K, int Vd,
                                                     int Vt, bool vec) {
  __shared__ int32_t toks[2][kMaxDepths];
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int r = wave; r < 2 * K; r += 4) {
    const int which = r / K, d = r % K;
    const int V = which ? Vt : Vd;
    const uint16_t* row = (which ? target : draft) + ((size_t)i * K + d) * V;
    const int32_t tok = (int32_t)row_argmax<Key>(row, V, vec, lane);
    if (lane == 0) {
      toks[which][d] = (kMap && which == 0) ? d2t[tok] : tok;
      (which ? ttok : dtok)[(size_t)i * K + d] = tok;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const bool match = lane < K && toks[0][lane] == toks[1][lane];
    const uint64_t mask = __ballot(match);
    if (lane == 0) {
      const uint64_t miss = ~mask;
      int L = (miss == 0) ? 64 : (int)__builtin_ctzll(miss);
      alen[i] = L < K ? L : K;
    }
  }
}

}  // namespace

hipError_t launch_accept_map(int32_t N, int32_t K, int32_t Vd, int32_t Vt,
                             const uint16_t* draft, const uint16_t* target, const int32_t* d2t,
                             int32_t* draft_tok, int32_t* target_tok, int32_t* accept_len,
                             hipStream_t stream) {
  const bool vec = (Vd % 8 == 0) && (Vt % 8 == 0) &&
                   ((reinterpret_cast<uintptr_t>(draft) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(target) & 15) == 0);
  const bool wide = std::max(Vd, Vt) > 65536;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(N), dim3(256), 0, stream, draft, target, d2t, draft_tok,
                       target_tok, accept_len, K, Vd, Vt, vec);
  };
  if (d2t == nullptr) {
    if (!wide) go(accept_kernel<uint32_t, false>); else go(accept_kernel<uint64_t, false>);
  } else {
    if (!wide) go(accept_kernel<uint32_t, true>); else go(accept_kernel<uint64_t, true>);
  }
  return hipGetLastError();
}

hipError_t launch_accept(int32_t N, int32_t K, int32_t V, const uint16_t* draft,
                         const uint16_t* target, int32_t* draft_tok, int32_t* target_tok,
                         int32_t* accept_len, hipStream_t stream) {
  return launch_accept_map(N, K, V, V, draft, target, nullptr, draft_tok, target_tok, accept_len,
                           stream);
}

}  // namespace peagle
