// Sampling acceptance of the drafts, gfx950.
//
// snxtyle/P_Eagle README, "How Speculative Decoding Works", step 6: accepted tokens are
// used, rejected tokens resampled. Read as speculative sampling: with p = softmax(target
// logits / tau) and q = softmax(draft logits / tau) at each depth, the drafter's token x_d
// is accepted while u_d < p(x_d) / q(x_d); at the first rejected depth j the next token is
// the smallest t whose cumulative residual max(0, p_j - q_j) exceeds w * Z (Z the
// residual's total). All K accepted: the next token is -1, or, given a K+1-th target row
// (kBonus), the bonus token drawn from p_K = softmax(target row K / tau) by the same
// inverse CDF with w.
//
// One workgroup (4 waves) per draft; the logits are read as chunks of 8 consecutive
// tokens a lane (16-byte loads when V % 8 == 0):
//   1. the 2K rows are swept once, waves taking rows in turn; each lane keeps an online
//      (max, sum of exp) pair, merged across the wave;
//   2. wave 0 forms the K ratios and finds the first rejection with one ballot;
//   3. at that depth only, the residual is summed over 4 contiguous segments (a wave
//      each), and the wave whose segment holds w * Z walks it again, 512 tokens a step,
//      with a wave prefix sum to find the token.
// fp32 arithmetic throughout; the decisions match a float64 evaluation except within its
// rounding of the thresholds.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "variants.h"

namespace peagle {

namespace {

constexpr int kSpecWaves = 4;
constexpr int kChunk = 8;                     // consecutive tokens a lane holds
constexpr int kStride = 64 * kChunk;          // tokens a wave covers per step

// Tokens j .. j+7 of a logit row, scaled by 1 / tau; tokens at or past `end` read -inf.
// kVec: 16-byte loads (V % 8 == 0, so a chunk never straddles `end`).
template <bool kVec>
__device__ __forceinline__ void load_chunk(const uint16_t* row, int j, int end, float inv_tau,
                                           float (&x)[kChunk]) {
  if constexpr (kVec) {
    if (j < end) {
      const bf16x8 b = as_bf16x8(*reinterpret_cast<const u32x4*>(row + j));
#pragma unroll
      for (int e = 0; e < kChunk; ++e) x[e] = (float)b[e] * inv_tau;
    } else {
#pragma unroll
      for (int e = 0; e < kChunk; ++e) x[e] = -INFINITY;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kChunk; ++e)
      x[e] = j + e < end ? bf16_bits_to_f32(row[j + e]) * inv_tau : -INFINITY;
  }
}

// Merge (m2, s2) into the running (max, sum of exp(x - max)) state (m, s).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  const float mn = fmaxf(m, m2);
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);  // exp(-inf) = 0 covers m = -inf
  m = mn;
}

// (max, sum of exp) of one row of V logits / tau, reduced over the wave.
template <bool kVec>
__device__ __forceinline__ void row_stats(const uint16_t* row, int V, float inv_tau, int lane,
                                          float& m, float& s) {
  constexpr int kDeep = 4;  // chunks loaded before any is used
  m = -INFINITY;
  s = 0.f;
  for (int j0 = lane * kChunk; j0 < V; j0 += kDeep * kStride) {
    float x[kDeep][kChunk];
#pragma unroll
    for (int c = 0; c < kDeep; ++c) load_chunk<kVec>(row, j0 + c * kStride, V, inv_tau, x[c]);
#pragma unroll
    for (int c = 0; c < kDeep; ++c) {
      float cm = x[c][0];
#pragma unroll
      for (int e = 1; e < kChunk; ++e) cm = fmaxf(cm, x[c][e]);
      if (cm == -INFINITY) continue;
      float cs = 0.f;
#pragma unroll
      for (int e = 0; e < kChunk; ++e) cs += __expf(x[c][e] - cm);
      lse_merge(m, s, cm, cs);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    lse_merge(m, s, m2, s2);
  }
}

// Residual weights max(0, p_t - q_t) of tokens j .. j+7 (0 past `end`); with drow == NULL
// (the bonus row) the weights are p_t alone.
template <bool kVec>
__device__ __forceinline__ void resid_chunk(const uint16_t* trow, const uint16_t* drow, int j,
                                            int end, float inv_tau, float mp, float isp,
                                            float mq, float isq, float (&r)[kChunk]) {
  float xt[kChunk];
  load_chunk<kVec>(trow, j, end, inv_tau, xt);
  if (drow == nullptr) {
#pragma unroll
    for (int e = 0; e < kChunk; ++e) r[e] = __expf(xt[e] - mp) * isp;
    return;
  }
  float xd[kChunk];
  load_chunk<kVec>(drow, j, end, inv_tau, xd);
#pragma unroll
  for (int e = 0; e < kChunk; ++e)
    r[e] = fmaxf(__expf(xt[e] - mp) * isp - __expf(xd[e] - mq) * isq, 0.f);
}

// kBonus: target holds K + 1 rows per draft (row K: the bonus distribution).
template <bool kVec, bool kBonus>
__global__ __launch_bounds__(64 * kSpecWaves) void spec_accept_kernel(
    const uint16_t* __restrict__ draft, const uint16_t* __restrict__ target,
    const int32_t* __restrict__ dtok, const float* __restrict__ u, const float* __restrict__ w,
    float inv_tau, int K, int V, int32_t* __restrict__ alen, int32_t* __restrict__ next) {
  __shared__ float st_m[2][kMaxDepths + 1], st_s[2][kMaxDepths + 1];
  __shared__ float seg_sum[kSpecWaves];
  __shared__ int s_L;
  const int i = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int KT = K + (kBonus ? 1 : 0);  // target rows per draft
  const uint16_t* tdraft = target + (size_t)i * KT * V;  // this draft's target rows

  // 1. (max, sum) of every draft row (which = 0) and target row (which = 1), a wave per row
  for (int r = wave; r < K + KT; r += kSpecWaves) {
    const int which = r < K ? 0 : 1, d = which ? r - K : r;
    float m, s;
    row_stats<kVec>(which ? tdraft + (size_t)d * V : draft + ((size_t)i * K + d) * V, V, inv_tau,
                    lane, m, s);
    if (lane == 0) {
      st_m[which][d] = m;
      st_s[which][d] = s;
    }
  }
  __syncthreads();

  // 2. accept depth d while u_d q(x_d) < p(x_d); the first miss ends the prefix
  if (wave == 0) {
    bool ok = false;
    if (lane < K) {
      const size_t rd = (size_t)i * K + lane;
      const int x = dtok[rd];
      if (x >= 0 && x < V) {  // a token outside the vocabulary is rejected
        const float p = __expf(bf16_bits_to_f32(tdraft[(size_t)lane * V + x]) * inv_tau -
                               st_m[1][lane]) / st_s[1][lane];
        const float q = __expf(bf16_bits_to_f32(draft[rd * V + x]) * inv_tau - st_m[0][lane]) /
                        st_s[0][lane];
        ok = u[rd] * q < p;
      }
    }
    const uint64_t miss = ~__ballot(ok);  // lanes >= K count as misses, so miss != 0
    if (lane == 0) {
      const int L = min((int)__builtin_ctzll(miss), K);
      alen[i] = L;
      s_L = L;
      if (L == K && !kBonus) next[i] = -1;
    }
  }
  __syncthreads();
  const int L = s_L;
  if (L >= K && !kBonus) return;  // the same for every wave of the workgroup

  // 3. inverse-CDF draw from the residual at depth L (or from the bonus row's p_K when all
  //    K are accepted). Segment totals first (wave q sums tokens [q * seg, (q + 1) * seg),
  //    seg a multiple of the chunk), then the wave whose segment holds w * Z walks its
  //    chunks in order with a wave prefix sum.
  const uint16_t* trow = tdraft + (size_t)L * V;
  const uint16_t* drow = L < K ? draft + ((size_t)i * K + L) * V : nullptr;
  const float mp = st_m[1][L], isp = 1.f / st_s[1][L];
  const float mq = L < K ? st_m[0][L] : 0.f, isq = L < K ? 1.f / st_s[0][L] : 0.f;
  const int seg = (V + kSpecWaves * kChunk - 1) / (kSpecWaves * kChunk) * kChunk;
  const int s0 = min(wave * seg, V), s1 = min(s0 + seg, V);
  float part = 0.f;
  for (int j = s0 + lane * kChunk; j < s1; j += kStride) {
    float r[kChunk];
    resid_chunk<kVec>(trow, drow, j, s1, inv_tau, mp, isp, mq, isq, r);
#pragma unroll
    for (int e = 0; e < kChunk; ++e) part += r[e];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
  if (lane == 0) seg_sum[wave] = part;
  __syncthreads();

  float Z = 0.f;
#pragma unroll
  for (int q = 0; q < kSpecWaves; ++q) Z += seg_sum[q];
  const float theta = w[i] * Z;
  // owner: the first segment whose cumulative total exceeds theta; should rounding leave
  // theta at or past Z, the last segment with weight, whose walk then ends on its last
  // token with weight
  int owner = -1, last = -1;
  float off = 0.f, acc = 0.f, off_last = 0.f;
#pragma unroll
  for (int q = 0; q < kSpecWaves; ++q) {
    if (owner < 0 && theta < acc + seg_sum[q]) owner = q, off = acc;
    if (seg_sum[q] > 0.f) last = q, off_last = acc;
    acc += seg_sum[q];
  }
  if (owner < 0) owner = last, off = off_last;
  if (owner < 0) {  // no residual weight at fp32 (p == q at depth L): keep the draft token
    // (a bonus row always has weight: its largest logit gives p = 1 / sum >= 1 / V)
    if (threadIdx.x == 0) next[i] = L < K ? dtok[(size_t)i * K + L] : 0;
    return;
  }
  if (wave != owner) return;
  const float rel = theta - off;  // the threshold measured from the segment's start
  float run = 0.f;
  int last_pos = -1;
  for (int b0 = s0; b0 < s1; b0 += kStride) {
    float r[kChunk], cs = 0.f;
    const int j = b0 + lane * kChunk;
    resid_chunk<kVec>(trow, drow, j, s1, inv_tau, mp, isp, mq, isq, r);
#pragma unroll
    for (int e = 0; e < kChunk; ++e) {
      cs += r[e];
      if (r[e] > 0.f) last_pos = j + e;
    }
    float incl = cs;  // inclusive prefix over the lanes' chunk totals
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    float excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.f;
    const uint64_t hit = __ballot(run + incl > rel);
    if (hit != 0) {
      // the first such lane: its exclusive prefix is the previous lane's inclusive one,
      // which did not exceed rel, so its chunk holds the crossing
      if (lane == (int)__builtin_ctzll(hit)) {
        float c = run + excl;
        int tok = -1, pos = -1;
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          c += r[e];
          if (r[e] > 0.f) pos = j + e;
          if (tok < 0 && c > rel) tok = j + e;
        }
        next[i] = tok >= 0 ? tok : pos;  // pos: the lane's last token with weight
      }
      return;
    }
    run += __shfl(incl, 63, 64);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) last_pos = max(last_pos, __shfl_xor(last_pos, o, 64));
  if (lane == 0) next[i] = last_pos;
}

}  // namespace

hipError_t launch_accept_sampled(int32_t N, int32_t K, int32_t V, const uint16_t* draft,
                                 const uint16_t* target, const int32_t* draft_tok,
                                 const float* u, const float* w, float temperature, bool bonus,
                                 int32_t* accept_len, int32_t* next_tok, hipStream_t stream) {
  const bool vec = V % kChunk == 0 && (reinterpret_cast<uintptr_t>(draft) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(target) & 15) == 0;
  const dim3 grid(N), block(64 * kSpecWaves);
  const float inv_tau = 1.f / temperature;
#define PEAGLE_SPEC(VEC, BONUS)                                                                \
  hipLaunchKernelGGL((spec_accept_kernel<VEC, BONUS>), grid, block, 0, stream, draft, target,  \
                     draft_tok, u, w, inv_tau, K, V, accept_len, next_tok)
  if (vec) {
    if (bonus) PEAGLE_SPEC(true, true); else PEAGLE_SPEC(true, false);
  } else {
    if (bonus) PEAGLE_SPEC(false, true); else PEAGLE_SPEC(false, false);
  }
#undef PEAGLE_SPEC
  return hipGetLastError();
}

}  // namespace peagle
