// Draft attention at inference (the decode shape), gfx950.
//
// NeMo Automodel PR 2376, parity section: at inference vLLM runs one flat parallel
// forward over [context, mask_1, ..., mask_{K-1}]; speculators P-EAGLE guide, "Inference
// Process": all depths are drafted in one pass and drafting repeats from the last
// accepted token. Request b has L_b context tokens in the KV cache (keys rotated at their
// positions 0 .. L_b - 1) and K new rows at positions L_b + d (d = 0: the anchor, the
// last accepted token; d >= 1: the mask rows). New row d attends to every cache key of
// its request and to new rows 0 .. d: the forward's predicate with a single anchor.
//
// Layouts:
//   k_cache  [Ltot, Hkv, D] bf16, rotated, natural order.
//   V tiles  [Hkv][ntiles][D][32] bf16 (decode_pack_v_kernel): tile (cu[b] >> 5) + b + j
//            of a kv head holds keys 32 j .. 32 j + 31 of request b (zeros past L_b),
//            dim-major, slot s of a dim row holding key dec_key(s). That is the order in
//            which a lane's two 16-key score accumulators hand their weights to the
//            P^T operand of O^T = V^T P^T, so P^T needs no data movement and every V^T
//            operand is one 16-byte load. The base (cu[b] >> 5) + b never overlaps the
//            previous request and needs no prefix sum.
//
// Kernels (all on the caller's stream):
//   decode_prep     one thread per rotation pair or element: q rotated at L_b + d, the new
//                   rows' keys rotated at L_b + e as one extra 32-key tile per (request, kv
//                   head) (zero rows past K), and their values as that tile's V^T. Its last
//                   workgroup lays out the work split (below).
//   decode_attn     split-KV over a compact tile space: request b takes nt_b =
//                   max(1, ceil(L_b / 32)) consecutive tile slots (one at least, for its new
//                   rows), and the space is cut into P equal ranges, one per workgroup and
//                   (kv head group, column group), P sized so that every workgroup is
//                   resident at once. A range may cross request boundaries: it leaves one
//                   partial (O, max, sum) per request it touches, in slot range + request,
//                   which no other (range, request) pair shares since both are ordered.
//                   Every workgroup streams the same number of cache bytes, so the launch
//                   ends without a tail of late workgroups. A wave holds 16 or 32 query
//                   columns (column c of a kv head: q head g*G + c / K, depth c % K) and
//                   computes S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 with
//                   an online softmax in base 2 (scale folded into one FMA) that rescales
//                   only when the running max grows by more than 2^8; the weights enter PV
//                   as a hi + lo bf16 pair. The range holding a request's first slot also
//                   takes its new rows' tile.
//   decode_combine  merges the partials of each (request, kv head, column).
// The path is HBM-bound: every cache byte is read once.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "variants.h"

namespace peagle {

namespace {

constexpr int kDecWaves = 4;  // waves per workgroup
constexpr int kDecTile = 32;  // keys per tile
constexpr float kDecRescaleLog2 = 8.f;
// Bound on the workgroups of one launch that the workspace provides partials for; the
// launch takes one workgroup per CU.
constexpr int kDecMaxWorkgroups = 1024;

// 16x16x32 bf16 MFMA: D[16x16] += A[16x32] * B[32x16]. Lane l supplies row l%16 of A and
// column l%16 of B, 8 values each at the same k positions for both operands; it
// receives column l%16 of D, rows 4*(l/16) + r for accumulator register r.
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Key held by slot s (0..31) of a V^T tile row: lane group q of the P^T operand holds
// keys 4q .. 4q + 3 (first score block) then 16 + 4q .. 16 + 4q + 3 (second).
__host__ __device__ constexpr int dec_key(int s) {
  return (s & 7) < 4 ? 4 * (s >> 3) + (s & 7) : 16 + 4 * (s >> 3) + (s & 7) - 4;
}

struct DecodeParams {
  const int32_t* cu;
  const int32_t* lens;  // current lengths inside the capacities, or null
  const uint16_t* kc;  // [Ltot, Hkv, D] rotated
  const uint16_t* vt;  // V tiles
  const uint16_t* qr;    // rotated q [B, K, Hq, D]
  const uint16_t* knew;  // rotated new keys [B, Hkv, 32, D], zero rows past K
  const uint16_t* vnew;  // new values as a V^T tile [B, Hkv, D, 32]
  const int32_t* rstart;  // [B + 1] first tile slot of each request, then the total S
  const int32_t* rfirst;  // [P] request holding the first slot of each range
  const int32_t* rlen;    // tile slots per range
  float* part_o;       // [P + B, Hkv, NCg, PC, D]
  float* part_ml;      // [P + B, Hkv, NCg, PC, 2]: max (base 2) and sum
  int B, K, Hq, Hkv, G, GK, NCg, max_ctx;
  int64_t total_ctx, ntiles;
  float c_log2;
};

// Cache start, capacity and context length of request b: cu gives the starts and
// capacities (cu[b + 1] - cu[b]); lens, when given, the current lengths inside them (a
// cache that grows in place), else a request fills its capacity. Trusted device data,
// clamped so that every access stays inside the cache.
__device__ __forceinline__ void request_extent(const int32_t* cu, const int32_t* lens, int b,
                                               int64_t total_ctx, int max_ctx, int64_t& c0,
                                               int& L, int& cap) {
  c0 = std::min<int64_t>(std::max(cu[b], 0), total_ctx);
  cap = (int)std::min<int64_t>(std::max<int64_t>((int64_t)cu[b + 1] - c0, 0),
                               std::min<int64_t>(max_ctx, total_ctx - c0));
  L = lens != nullptr ? std::min(std::max(lens[b], 0), cap) : cap;
}
__device__ __forceinline__ void request_extent(const int32_t* cu, const int32_t* lens, int b,
                                               int64_t total_ctx, int max_ctx, int64_t& c0,
                                               int& L) {
  int cap;
  request_extent(cu, lens, b, total_ctx, max_ctx, c0, L, cap);
}

// Rotate-half RoPE of dims j0 .. j0 + 7 and their partners j0 + D/2 .. of one pre-RoPE bf16
// row at position pos, rounded to bf16 (fp32 arithmetic; cos/sin from the table).
__device__ __forceinline__ void rope8(const uint16_t* src, uint16_t* dst, int j0, int H, int pos,
                                      const float* cs, const float* sn) {
  const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(src + j0));
  const bf16x8 b = as_bf16x8(*reinterpret_cast<const u32x4*>(src + j0 + H));
  const floatx4* cp = reinterpret_cast<const floatx4*>(cs + (size_t)pos * H + j0);
  const floatx4* sp = reinterpret_cast<const floatx4*>(sn + (size_t)pos * H + j0);
  const floatx4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
  bf16x8 lo, hi;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = (float)a[e], y = (float)b[e];
    const float c = e < 4 ? c0[e] : c1[e - 4], s = e < 4 ? s0[e] : s1[e - 4];
    lo[e] = (__bf16)(x * c - y * s);
    hi[e] = (__bf16)(y * c + x * s);
  }
  *reinterpret_cast<bf16x8*>(dst + j0) = lo;
  *reinterpret_cast<bf16x8*>(dst + j0 + H) = hi;
}

// Tile slots of request b: max(1, ceil(L_b / 32)).
__device__ __forceinline__ int request_slots(const int32_t* cu, const int32_t* lens, int b,
                                             int64_t total_ctx, int max_ctx) {
  int64_t c0;
  int L;
  request_extent(cu, lens, b, total_ctx, max_ctx, c0, L);
  return std::max(1, (L + kDecTile - 1) / kDecTile);
}

// The work split, by one workgroup of 256 threads: rstart[b] = sum of the slots of the
// requests before b (rstart[B] = S), len = ceil(S / P) slots per range, and rfirst[r] = the
// request holding slot r len, for every range with r len < S (the others hold nothing).
// Thread i takes ceil(B / 256) consecutive requests; their totals are scanned in LDS.
__device__ void decode_ranges(const int32_t* __restrict__ cu, const int32_t* __restrict__ lens,
                              int B, int64_t total_ctx, int max_ctx, int P,
                              int32_t* __restrict__ rstart, int32_t* __restrict__ rfirst,
                              int32_t* __restrict__ rlen) {
  __shared__ int scan[256];
  const int tid = threadIdx.x;
  const int per = (B + 255) / 256;
  const int lo = std::min(tid * per, B), hi = std::min(lo + per, B);
  int sum = 0;
  for (int b = lo; b < hi; ++b) sum += request_slots(cu, lens, b, total_ctx, max_ctx);
  scan[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  const int S = scan[255];  // >= B >= 1
  const int len = (S + P - 1) / P;
  int run = scan[tid] - sum;
  for (int b = lo; b < hi; ++b) {
    const int end = run + request_slots(cu, lens, b, total_ctx, max_ctx);
    rstart[b] = run;
    // ranges whose first slot lies in [run, end)
    for (int r = (run + len - 1) / len; (int64_t)r * len < end; ++r) rfirst[r] = b;
    run = end;
  }
  if (tid == 0) {
    rstart[B] = S;
    *rlen = len;
  }
}

// Flat grid, 8 outputs per thread, over three ranges: q (B K Hq rows, D/16 threads a row),
// new keys (B Hkv 32 rows, D/16 threads a row), new V^T (B Hkv D rows of 32 slots, 4
// threads a row); one more workgroup, the last, lays out the work split.
__global__ __launch_bounds__(256) void decode_prep_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ lens,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ cs, const float* __restrict__ sn,
    uint16_t* __restrict__ qr, uint16_t* __restrict__ knew, uint16_t* __restrict__ vnew, int B,
    int K, int Hq, int Hkv, int D, int max_ctx, int max_pos, int64_t total_ctx, int P,
    int32_t* __restrict__ rstart, int32_t* __restrict__ rfirst, int32_t* __restrict__ rlen) {
  if (blockIdx.x == gridDim.x - 1) {
    decode_ranges(cu, lens, B, total_ctx, max_ctx, P, rstart, rfirst, rlen);
    return;
  }
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int H = D / 2, per_row = D / 16;
  const int64_t nq = (int64_t)B * K * Hq * per_row, nk = (int64_t)B * Hkv * kDecTile * per_row;
  const int64_t nv = (int64_t)B * Hkv * D * (kDecTile / 8);
  int64_t c0;
  int L;
  if (t < nq) {
    const int j0 = (int)(t % per_row) * 8;
    const int64_t row = t / per_row;  // (b, d, h)
    const int d = (int)((row / Hq) % K), b = (int)(row / ((int64_t)Hq * K));
    request_extent(cu, lens, b, total_ctx, max_ctx, c0, L);
    rope8(q + row * D, qr + row * D, j0, H, std::min(L + d, max_pos), cs, sn);
  } else if (t < nq + nk) {
    const int64_t u = t - nq;
    const int j0 = (int)(u % per_row) * 8;
    const int64_t row = u / per_row;  // (b, g, e)
    const int e = (int)(row % kDecTile);
    const int64_t bg = row / kDecTile;
    const int g = (int)(bg % Hkv), b = (int)(bg / Hkv);
    uint16_t* dst = knew + row * D;
    if (e < K) {
      request_extent(cu, lens, b, total_ctx, max_ctx, c0, L);
      rope8(k + (((size_t)b * K + e) * Hkv + g) * D, dst, j0, H, std::min(L + e, max_pos), cs, sn);
    } else {
      *reinterpret_cast<u32x4*>(dst + j0) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(dst + j0 + H) = u32x4{0u, 0u, 0u, 0u};
    }
  } else if (t < nq + nk + nv) {
    const int64_t u = t - nq - nk;
    const int s0 = (int)(u % (kDecTile / 8)) * 8;
    const int64_t drow = u / (kDecTile / 8);  // (b, g, dim)
    const int dim = (int)(drow % D);
    const int64_t bg = drow / D;
    const int g = (int)(bg % Hkv), b = (int)(bg / Hkv);
    bf16x8 out;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = dec_key(s0 + i);
      const uint16_t bits =
          v[(((size_t)b * K + std::min(e, K - 1)) * Hkv + g) * D + dim];
      out[i] = __builtin_bit_cast(__bf16, e < K ? bits : (uint16_t)0);
    }
    *reinterpret_cast<bf16x8*>(vnew + drow * kDecTile + s0) = out;
  }
}

template <int D, int NCW>
struct DecodeWave {
  static constexpr int DK = D / 32, MT = D / 16;
  bf16x8 qf[NCW][DK];
  floatx4 o[NCW][MT];
  float m_run[NCW], l_run[NCW];
};

// Scores, online softmax and PV of one 32-key tile held in registers: kf[h] are the A
// fragments of keys 16 h .. 16 h + 15, vf the V^T fragments; column group c keeps the
// keys below lim[c].
template <int D, int NCW>
__device__ __forceinline__ void decode_tile_math(DecodeWave<D, NCW>& w,
                                                 const bf16x8 (&kf)[2][D / 32],
                                                 const bf16x8 (&vf)[D / 16],
                                                 const int (&lim)[NCW], float c_log2, int grp) {
  constexpr int DK = D / 32, MT = D / 16;
#pragma unroll
  for (int c = 0; c < NCW; ++c) {
    floatx4 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) s[h] = mfma16(kf[h][kk], w.qf[c][kk], s[h]);
    }
    if (lim[c] < kDecTile) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * h + 4 * grp + r >= lim[c]) s[h][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c_log2;
    const float m_new = fmaxf(w.m_run[c], mx);
    if (__any(m_new > w.m_run[c] + kDecRescaleLog2)) {
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(w.m_run[c] - m_new);
      w.l_run[c] *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) w.o[c][mt] *= alpha;
      w.m_run[c] = m_new;
    }
    // P^T as a bf16 pair (hi + lo): about 16 significant bits instead of 8 for two MFMAs
    // per V^T fragment, which cost nothing next to the cache reads
    const float mu = w.m_run[c] == -INFINITY ? 0.f : w.m_run[c];
    bf16x8 ph, pl;
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pr = __builtin_amdgcn_exp2f(fmaf(s[i >> 2][i & 3], c_log2, -mu));
      ls += pr;
      ph[i] = (__bf16)pr;
      pl[i] = (__bf16)(pr - (float)ph[i]);
    }
    w.l_run[c] += ls;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      w.o[c][mt] = mfma16(vf[mt], ph, w.o[c][mt]);
      w.o[c][mt] = mfma16(vf[mt], pl, w.o[c][mt]);
    }
  }
}

// One cache tile in registers: kf[h] the A fragments of keys 16 h .. 16 h + 15, vf the V^T
// fragments.
template <int D>
struct CacheTile {
  bf16x8 kf[2][D / 32];
  bf16x8 vf[D / 16];
};

// Issue the loads of one cache tile: rows [0, rows) of kbase (row stride kstride elements;
// rows past the end repeat the last one and are masked) and its V^T tile. Every cache byte
// is read once per call, so the loads are nontemporal: they stream past the caches instead
// of evicting lines that are still wanted (measured 8% faster). kbase and vtile are
// wave-uniform: the loads go through raw buffer resources over the tile's bytes (scalar
// registers) with 32-bit lane offsets (the row stride, Hkv D < 2^24 elements, keeps them
// below 2^31). Per-lane 64-bit addresses had pushed the two-tile loop past its registers:
// a spilled address reloaded from scratch once per tile, and its vmcnt wait drained the
// next tile's loads.
constexpr int kLoadNT = 2;  // cache policy of the buffer loads: nontemporal
template <int D, bool kIssueAll>
__device__ __forceinline__ void load_cache_tile(CacheTile<D>& t, const uint16_t* kbase,
                                                size_t kstride, int rows,
                                                const uint16_t* vtile, int l16, int grp) {
  constexpr int DK = D / 32, MT = D / 16;
  const int rows_c = std::min(rows, kDecTile);
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(kbase), 0, (int)(((size_t)(rows_c - 1) * kstride + D) * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vtile), 0, D * kDecTile * 2, 0x00020000);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = std::min(16 * h + l16, rows_c - 1);
    const uint32_t ko = (uint32_t)((size_t)row * kstride + 8 * grp) * 2;
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
      t.kf[h][kk] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(kr, ko + 64 * kk, 0, kLoadNT));
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    t.vf[mt] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(
        vr, (uint32_t)((16 * mt + l16) * kDecTile + 8 * grp) * 2, 0, kLoadNT));
  // kIssueAll: every load of the tile is issued before the first wait on any of them, one
  // memory round trip per tile instead of one for K and then one for V (without this
  // barrier the compiler sinks the V loads below the scores under register pressure: 18%
  // slower). With a second tile in flight the compiler's own order measured 1.5% faster.
  if constexpr (kIssueAll) __builtin_amdgcn_sched_barrier(0);
}

// Work split. A workgroup job is (range r of the tile slots, column group, group of HEADS
// kv heads), the head group fastest. HEADS = 4 (Hkv a multiple of 4): wave w takes kv head
// 4 gg + w and every tile of the range, so the four waves read neighbouring head segments
// of the same cache rows, and each wave writes its partials. HEADS = 1: the four waves take
// the tiles of each request segment in turn (neighbouring tiles at the same time) and merge
// through LDS into one partial per segment. Segment bounds are uniform over the workgroup,
// so every barrier is reached by all waves.
template <int D, int NCW, int HEADS>
__global__ __launch_bounds__(64 * kDecWaves, HEADS == 1 ? 1 : 2) void decode_attn_kernel(
    const DecodeParams p) {
  constexpr int DK = D / 32, MT = D / 16, PC = 16 * NCW;
  constexpr bool kMerge = HEADS == 1;
  constexpr int kRedWaves = kMerge ? kDecWaves : 1;
  __shared__ float red_o[kRedWaves][kMerge ? PC : 1][kMerge ? D : 1];
  __shared__ float red_ml[kRedWaves][kMerge ? PC : 1][2];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, grp = lane >> 4;
  const int K = p.K, Hkv = p.Hkv;
  const int ngg = Hkv / HEADS;
  const int gg = (int)(blockIdx.x % ngg);
  const int r1 = (int)(blockIdx.x / ngg);
  const int cg = r1 % p.NCg;
  const int r = r1 / p.NCg;
  const int g = HEADS == 1 ? gg : gg * HEADS + wave;
  const int len = *p.rlen, S = p.rstart[p.B];
  const int t0 = r * len;
  if (t0 >= S) return;  // uniform: ranges past the last slot hold nothing
  const int t1 = std::min(t0 + len, S);

  for (int b = p.rfirst[r]; b < p.B; ++b) {
    const int sb = p.rstart[b];
    if (sb >= t1) break;
    const int eb = p.rstart[b + 1];
    int64_t c0;
    int L;
    request_extent(p.cu, p.lens, b, p.total_ctx, p.max_ctx, c0, L);
    const int j0 = std::max(t0, sb) - sb, j1 = std::min(t1, eb) - sb;  // tiles of b here

    DecodeWave<D, NCW> w;
    int dcol[NCW];
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
      const int col = std::min((cg * NCW + c) * 16 + l16, p.GK - 1);
      const int d = col % K, head = g * p.G + col / K;
      dcol[c] = d;
      const uint16_t* qrow = p.qr + (((size_t)b * K + d) * p.Hq + head) * D + 8 * grp;
#pragma unroll
      for (int kk = 0; kk < DK; ++kk)
        w.qf[c][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 32 * kk));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) w.o[c][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      w.m_run[c] = -INFINITY;
      w.l_run[c] = 0.f;
    }

    // the new rows' tile (laid out by decode_prep), with the request's first slot: row d
    // keeps new keys e <= d
    if (j0 == 0 && (HEADS > 1 || wave == 0)) {
      const size_t bg = (size_t)b * Hkv + g;
      const uint16_t* kbase = p.knew + bg * kDecTile * D;
      const uint16_t* vtile = p.vnew + bg * D * kDecTile;
      bf16x8 kf[2][DK];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
          kf[h][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(kbase + (16 * h + l16) * D + 32 * kk + 8 * grp));
      bf16x8 vf[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        vf[mt] = as_bf16x8(*reinterpret_cast<const u32x4*>(vtile + (16 * mt + l16) * kDecTile + 8 * grp));
      int lim[NCW];
#pragma unroll
      for (int c = 0; c < NCW; ++c) lim[c] = dcol[c] + 1;
      decode_tile_math<D, NCW>(w, kf, vf, lim, p.c_log2, grp);
    }
    // the segment's cache tiles (a request with no context has one slot and no tile)
    const int j_end = std::min(j1, (L + kDecTile - 1) / kDecTile);
    const uint16_t* vbase = p.vt + (((size_t)g * p.ntiles + (c0 >> 5) + b) * D) * kDecTile;
    // HEADS = 1: two tiles in registers, the loads of the next tile in flight while this
    // one is computed (one wave per SIMD leaves the registers for it; measured 7% faster at
    // D = 256). HEADS = 4 keeps one tile a wave: four waves of one CU already stream four
    // heads of the same keys, and the second buffer measured 1.5% slower there.
    const int j_step = HEADS == 1 ? kDecWaves : 1;
    const int j_first = j0 + (HEADS == 1 ? wave : 0);
    auto issue = [&](CacheTile<D>& t, int j) {
      const int key0 = j * kDecTile;
      load_cache_tile<D, HEADS != 1>(t, p.kc + ((size_t)(c0 + key0) * Hkv + g) * D,
                                     (size_t)Hkv * D, L - key0,
                                     vbase + (size_t)j * D * kDecTile, l16, grp);
    };
    auto compute = [&](const CacheTile<D>& t, int j) {
      int lim[NCW];
#pragma unroll
      for (int c = 0; c < NCW; ++c) lim[c] = L - j * kDecTile;
      decode_tile_math<D, NCW>(w, t.kf, t.vf, lim, p.c_log2, grp);
    };
    if constexpr (HEADS != 1) {
      for (int j = j_first; j < j_end; ++j) {
        CacheTile<D> t;
        issue(t, j);
        compute(t, j);
      }
    } else if (j_first < j_end) {
      CacheTile<D> ta, tb;
      issue(ta, j_first);
      for (int j = j_first; j < j_end; j += 2 * j_step) {
        const int jn = j + j_step;
        if (jn < j_end) issue(tb, jn);
        compute(ta, j);
        if (jn >= j_end) break;
        if (jn + j_step < j_end) issue(ta, jn + j_step);
        compute(tb, jn);
      }
    }

    const size_t part = ((size_t)(r + b) * Hkv + g) * p.NCg + cg;
    if constexpr (!kMerge) {
      // the wave's partial: O^T columns (the lane holds dims 16 mt + 4 grp + r of column
      // l16), running max and sum
#pragma unroll
      for (int c = 0; c < NCW; ++c) {
        float lt = w.l_run[c] + __shfl_xor(w.l_run[c], 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        float* po = p.part_o + (part * PC + c * 16 + l16) * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *reinterpret_cast<floatx4*>(po + 16 * mt + 4 * grp) = w.o[c][mt];
        if (grp == 0) {
          p.part_ml[(part * PC + c * 16 + l16) * 2] = w.m_run[c];
          p.part_ml[(part * PC + c * 16 + l16) * 2 + 1] = lt;
        }
      }
    } else {
      // merge the four waves through LDS; the workgroup writes one partial
#pragma unroll
      for (int c = 0; c < NCW; ++c) {
        float lt = w.l_run[c] + __shfl_xor(w.l_run[c], 16, 64);
        lt += __shfl_xor(lt, 32, 64);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *reinterpret_cast<floatx4*>(&red_o[wave][c * 16 + l16][16 * mt + 4 * grp]) = w.o[c][mt];
        if (grp == 0) {
          red_ml[wave][c * 16 + l16][0] = w.m_run[c];
          red_ml[wave][c * 16 + l16][1] = lt;
        }
      }
      __syncthreads();
      for (int t = threadIdx.x; t < PC * (D / 4); t += 64 * kDecWaves) {
        const int col = t / (D / 4), d4 = (t % (D / 4)) * 4;
        float M = -INFINITY;
#pragma unroll
        for (int q = 0; q < kDecWaves; ++q) M = fmaxf(M, red_ml[q][col][0]);
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;
#pragma unroll
        for (int q = 0; q < kDecWaves; ++q) {
          const float mq = red_ml[q][col][0];
          const float f = mq == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mq - M);
          acc += f * *reinterpret_cast<const floatx4*>(&red_o[q][col][d4]);
          lsum += f * red_ml[q][col][1];
        }
        *reinterpret_cast<floatx4*>(p.part_o + (part * PC + col) * D + d4) = acc;
        if (d4 == 0) {
          p.part_ml[(part * PC + col) * 2] = M;
          p.part_ml[(part * PC + col) * 2 + 1] = lsum;
        }
      }
      __syncthreads();  // the LDS is written again by the next segment
    }
  }
}

// Merge the partials of each (request, kv head, column): request b's slots [s_b, e_b)
// meet ranges r0 = s_b / len .. (e_b - 1) / len, whose partials sit in slots r + b.
// out = sum_r 2^(m_r - M) O_r / sum_r 2^(m_r - M) l_r and lse = (M + log2 of that sum) ln 2,
// M the largest m_r. One thread per output (column, 4 dims), dims fastest: a wave reads whole
// partial rows; up to 8 partials are loaded before any is used.
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const int32_t* __restrict__ rstart, const int32_t* __restrict__ rlen,
    const float* __restrict__ part_o, const float* __restrict__ part_ml, float* __restrict__ out,
    float* __restrict__ lse, int K, int Hq, int Hkv, int G, int GK, int NCg, int PC, int D,
    int64_t n) {
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= n) return;
  const int per_col = D / 4;
  const int d4 = (int)(o % per_col) * 4;
  const int c = (int)((o / per_col) % PC);
  const int64_t item = o / ((int64_t)per_col * PC);  // (b, g, cg)
  const int cg = (int)(item % NCg);
  const int col = cg * PC + c;
  if (col >= GK) return;
  const int64_t bg = item / NCg;
  const int b = (int)(bg / Hkv), g = (int)(bg % Hkv);
  const int len = *rlen, sb = rstart[b], eb = rstart[b + 1];
  const int r0 = sb / len, nparts = (eb - 1) / len - r0 + 1;
  const size_t slot_stride = (size_t)Hkv * NCg;  // partial units per slot
  const size_t base = ((size_t)(r0 + b) * Hkv + g) * NCg + cg;
  float M = -INFINITY, lsum = 0.f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < nparts; q0 += 8) {
    float mq[8], lq[8];
    floatx4 oq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mq[i] = -INFINITY;
      lq[i] = 0.f;
      oq[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (q0 + i < nparts) {  // uniform over the threads of one (request, head, column)
        const size_t u = (base + (size_t)(q0 + i) * slot_stride) * PC + c;
        mq[i] = part_ml[u * 2];
        lq[i] = part_ml[u * 2 + 1];
        oq[i] = *reinterpret_cast<const floatx4*>(part_o + u * D + d4);
      }
    }
    float Mr = M;
#pragma unroll
    for (int i = 0; i < 8; ++i) Mr = fmaxf(Mr, mq[i]);
    if (Mr == -INFINITY) continue;
    const float fa = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mr);
    acc *= fa;
    lsum *= fa;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float f = mq[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mq[i] - Mr);
      acc += f * oq[i];
      lsum += f * lq[i];
    }
    M = Mr;
  }
  const int d = col % K, head = g * G + col / K;
  *reinterpret_cast<floatx4*>(out + (((size_t)b * K + d) * Hq + head) * D + d4) = acc / lsum;
  if (lse != nullptr && d4 == 0)
    lse[((size_t)b * K + d) * Hq + head] = (M + __log2f(lsum)) * 0.69314718055994531f;
}

// Natural V [Ltot, Hkv, D] -> V tiles (layout in the header comment). One workgroup per
// (tile j of request b, kv head g); tiles past the request's end write nothing.
template <int D>
__global__ __launch_bounds__(256) void decode_pack_v_kernel(const int32_t* __restrict__ cu,
                                                            const int32_t* __restrict__ lens,
                                                            const uint16_t* __restrict__ v,
                                                            uint16_t* __restrict__ vt,
                                                            int64_t total_ctx, int max_ctx,
                                                            int64_t ntiles, int Hkv) {
  __shared__ uint16_t tile[kDecTile][D + 8];
  const int j = blockIdx.x, b = blockIdx.y, g = blockIdx.z, tid = threadIdx.x;
  int64_t c0;
  int L, cap;
  request_extent(cu, lens, b, total_ctx, max_ctx, c0, L, cap);
  if (j * kDecTile >= cap) return;  // tiles up to the capacity; zeros past the length
  constexpr int cpr = D / 8;
  for (int q = tid; q < kDecTile * cpr; q += 256) {
    const int key = q / cpr, c = q % cpr, pos = j * kDecTile + key;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (pos < L) val = *reinterpret_cast<const u32x4*>(v + ((size_t)(c0 + pos) * Hkv + g) * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[key][c * 8 + 2 * e] = (uint16_t)(val[e] & 0xFFFFu);
      tile[key][c * 8 + 2 * e + 1] = (uint16_t)(val[e] >> 16);
    }
  }
  __syncthreads();
  uint16_t* dst = vt + (((size_t)g * ntiles + (c0 >> 5) + b + j) * D) * kDecTile;
  for (int q = tid; q < D * kDecTile; q += 256) dst[q] = tile[dec_key(q % kDecTile)][q / kDecTile];
}

template <typename F>
hipError_t for_dim(int D, F&& f) {
  switch (D) {
    case 64: f(std::integral_constant<int, 64>{}); break;
    case 128: f(std::integral_constant<int, 128>{}); break;
    case 256: f(std::integral_constant<int, 256>{}); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct DecodeLayout {
  size_t qr, knew, vnew, part_o, part_ml, rstart, rfirst, rlen, total;
};

DecodeLayout decode_layout(int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D,
                           const DecodePlan& pl) {
  DecodeLayout l;
  const size_t parts = (size_t)pl.nslots * Hkv * pl.ncg * pl.pc;
  l.qr = 0;
  l.knew = l.qr + align256((size_t)B * K * Hq * D * 2);
  l.vnew = l.knew + align256((size_t)B * Hkv * kDecTile * D * 2);
  l.part_o = l.vnew + align256((size_t)B * Hkv * D * kDecTile * 2);
  l.part_ml = l.part_o + align256(parts * D * 4);
  l.rstart = l.part_ml + align256(parts * 2 * 4);
  l.rfirst = l.rstart + align256(((size_t)B + 1) * 4);
  l.rlen = l.rfirst + align256((size_t)pl.max_ranges * 4);
  l.total = l.rlen + 256;
  return l;
}

// Position of key x (0..31) in a V^T tile row: the inverse of dec_key.
__device__ __forceinline__ int dec_slot(int x) {
  return x < 16 ? 8 * (x >> 2) + (x & 3) : 8 * ((x - 16) >> 2) + 4 + (x & 3);
}

// A cache that grows in place (speculators P-EAGLE guide, "Inference Process": drafting
// repeats from the last accepted token, so the newly committed tokens join the context).
// Request b takes m_b = n_new[b] + n_add rows j = 0 .. m_b - 1 of k_new / v_new
// [B, max_new, Hkv, D] (pre-RoPE) at positions L_b + j: k rotated at that position into
// cache row c0 + L_b + j, v into slot dec_slot((L_b + j) & 31) of the request's V tile
// (L_b + j) >> 5. Rows past the capacity are dropped; lens_out[b] = min(L_b + m_b, cap).
// Flat grid over three ranges: k (D/16 threads a row), v (D/8 threads a row), lengths.
__global__ __launch_bounds__(256) void decode_append_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ lens_in,
    const int32_t* __restrict__ n_new, int n_add, int max_new, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const float* __restrict__ cs, const float* __restrict__ sn,
    int max_pos, uint16_t* __restrict__ kc, uint16_t* __restrict__ vt,
    int32_t* __restrict__ lens_out, int B, int Hkv, int D, int max_ctx, int64_t total_ctx,
    int64_t ntiles) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int H = D / 2;
  const int64_t rows = (int64_t)B * max_new * Hkv;
  const int64_t nk = rows * (D / 16), nv = rows * (D / 8);
  int64_t c0;
  int L, cap;
  if (t < nk + nv) {
    const bool is_k = t < nk;
    const int64_t u = is_k ? t : t - nk;
    const int per_row = is_k ? D / 16 : D / 8;
    const int c = (int)(u % per_row);
    const int64_t row = u / per_row;  // (b, j, g)
    const int g = (int)(row % Hkv);
    const int j = (int)((row / Hkv) % max_new);
    const int b = (int)(row / ((int64_t)Hkv * max_new));
    request_extent(cu, lens_in, b, total_ctx, max_ctx, c0, L, cap);
    const int m = std::min(std::max(n_new[b] + n_add, 0), max_new);
    if (j >= m || L + j >= cap) return;
    const int key = L + j;
    const uint16_t* src = (is_k ? k_new : v_new) + (size_t)row * D;
    if (is_k) {
      rope8(src, kc + ((size_t)(c0 + key) * Hkv + g) * D, c * 8, H, std::min(key, max_pos), cs, sn);
    } else {
      const u32x4 val = *reinterpret_cast<const u32x4*>(src + c * 8);
      uint16_t* tile = vt + (((size_t)g * ntiles + (c0 >> 5) + b + (key >> 5)) * D) * kDecTile;
      const int slot = dec_slot(key & 31);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        tile[(size_t)(c * 8 + e) * kDecTile + slot] = (uint16_t)((val[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    }
  } else if (t < nk + nv + B) {
    const int b = (int)(t - nk - nv);
    request_extent(cu, lens_in, b, total_ctx, max_ctx, c0, L, cap);
    const int m = std::min(std::max(n_new[b] + n_add, 0), max_new);
    lens_out[b] = std::min(L + m, cap);
  }
}

}  // namespace

int64_t decode_ntiles(int64_t total_ctx, int32_t B) { return (total_ctx >> 5) + B + 1; }

DecodePlan decode_plan(int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D,
                       int64_t total_ctx, int32_t max_ctx) {
  (void)max_ctx;
  DecodePlan pl;
  const int gk = (Hq / Hkv) * K;
  // two column groups per wave where the registers allow it (D <= 128)
  pl.ncw = (D <= 128 && gk > 16) ? 2 : 1;
  pl.pc = 16 * pl.ncw;
  pl.ncg = (gk + pl.pc - 1) / pl.pc;
  // Four kv heads per workgroup where Hkv allows it; otherwise the waves share a range.
  pl.heads = Hkv % 4 == 0 ? 4 : 1;
  pl.wg_per_range = pl.ncg * (Hkv / pl.heads);
  // The launch picks the range count for the device (every workgroup resident at once);
  // the workspace holds up to kDecMaxWorkgroups workgroups' worth, and no more ranges than
  // the (total_ctx / 32 + B bounded) tile slots.
  const int64_t slots_max = (total_ctx >> 5) + B;
  pl.max_ranges = (int)std::max<int64_t>(
      1, std::min<int64_t>(slots_max, std::max(1, kDecMaxWorkgroups / pl.wg_per_range)));
  pl.nslots = pl.max_ranges + B;
  return pl;
}

size_t decode_workspace_bytes(int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D,
                              int64_t total_ctx, int32_t max_ctx) {
  return decode_layout(B, K, Hq, Hkv, D, decode_plan(B, K, Hq, Hkv, D, total_ctx, max_ctx)).total;
}

hipError_t launch_decode_pack_v(const int32_t* cu, int32_t B, int64_t total_ctx, int32_t max_ctx,
                                const uint16_t* v, int32_t Hkv, int32_t D, uint16_t* vt,
                                hipStream_t stream) {
  return launch_decode_pack_v_lens(cu, nullptr, B, total_ctx, max_ctx, v, Hkv, D, vt, stream);
}

hipError_t launch_decode_pack_v_lens(const int32_t* cu, const int32_t* lens, int32_t B,
                                     int64_t total_ctx, int32_t max_ctx, const uint16_t* v,
                                     int32_t Hkv, int32_t D, uint16_t* vt, hipStream_t stream) {
  const int tiles_max = (max_ctx + kDecTile - 1) / kDecTile;
  if (tiles_max == 0) return hipSuccess;
  const int64_t ntiles = decode_ntiles(total_ctx, B);
  return for_dim(D, [&](auto dc) {
    constexpr int DD = decltype(dc)::value;
    hipLaunchKernelGGL(decode_pack_v_kernel<DD>, dim3(tiles_max, B, Hkv), dim3(256), 0, stream, cu,
                       lens, v, vt, total_ctx, max_ctx, ntiles, Hkv);
  });
}

hipError_t launch_decode_attn(const DecodeArgs& a, const int32_t* cu, const uint16_t* kc,
                              const uint16_t* vt, const uint16_t* qn, const uint16_t* kn,
                              const uint16_t* vn, const float* cs, const float* sn, float* out,
                              float* lse, char* ws, hipStream_t stream) {
  return launch_decode_attn_lens(a, cu, nullptr, kc, vt, qn, kn, vn, cs, sn, out, lse, ws, stream);
}


hipError_t launch_decode_attn_lens(const DecodeArgs& a, const int32_t* cu, const int32_t* lens,
                                   const uint16_t* kc, const uint16_t* vt, const uint16_t* qn,
                                   const uint16_t* kn, const uint16_t* vn, const float* cs,
                                   const float* sn, float* out, float* lse, char* ws,
                                   hipStream_t stream) {
  const DecodePlan pl = decode_plan(a.B, a.K, a.Hq, a.Hkv, a.D, a.total_ctx, a.max_ctx);
  const DecodeLayout lay = decode_layout(a.B, a.K, a.Hq, a.Hkv, a.D, pl);
  DecodeParams p;
  p.cu = cu;
  p.lens = lens;
  p.kc = kc;
  p.vt = vt;
  p.qr = reinterpret_cast<const uint16_t*>(ws + lay.qr);
  p.knew = reinterpret_cast<const uint16_t*>(ws + lay.knew);
  p.vnew = reinterpret_cast<const uint16_t*>(ws + lay.vnew);
  p.rstart = reinterpret_cast<const int32_t*>(ws + lay.rstart);
  p.rfirst = reinterpret_cast<const int32_t*>(ws + lay.rfirst);
  p.rlen = reinterpret_cast<const int32_t*>(ws + lay.rlen);
  p.part_o = reinterpret_cast<float*>(ws + lay.part_o);
  p.part_ml = reinterpret_cast<float*>(ws + lay.part_ml);
  p.B = a.B;
  p.K = a.K;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.G = a.Hq / a.Hkv;
  p.GK = p.G * a.K;
  p.NCg = pl.ncg;
  p.max_ctx = a.max_ctx;
  p.total_ctx = a.total_ctx;
  p.ntiles = decode_ntiles(a.total_ctx, a.B);
  p.c_log2 = a.scale * 1.4426950408889634f;

  // ranges: one workgroup per CU, all resident at once and each with the same number of
  // cache bytes. Measured on 256 CUs: one workgroup per CU is 5-7% faster than two (half
  // the partials, and the same bandwidth from fewer streams), 1.5 or 0.5 far slower.
  const int64_t want = (int64_t)device_cus() / pl.wg_per_range;
  const int P = (int)std::max<int64_t>(1, std::min<int64_t>(want, pl.max_ranges));

  const int64_t nprep = (int64_t)a.B * a.K * a.Hq * (a.D / 16) +
                        (int64_t)a.B * a.Hkv * kDecTile * (a.D / 16) +
                        (int64_t)a.B * a.Hkv * a.D * (kDecTile / 8);
  hipLaunchKernelGGL(decode_prep_kernel, dim3((unsigned)((nprep + 255) / 256 + 1)), dim3(256), 0,
                     stream, cu, lens, qn, kn, vn, cs, sn, reinterpret_cast<uint16_t*>(ws + lay.qr),
                     reinterpret_cast<uint16_t*>(ws + lay.knew),
                     reinterpret_cast<uint16_t*>(ws + lay.vnew), a.B, a.K, a.Hq, a.Hkv, a.D,
                     a.max_ctx, a.max_pos, a.total_ctx, P,
                     reinterpret_cast<int32_t*>(ws + lay.rstart),
                     reinterpret_cast<int32_t*>(ws + lay.rfirst),
                     reinterpret_cast<int32_t*>(ws + lay.rlen));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = for_dim(a.D, [&](auto dc) {
    constexpr int DD = decltype(dc)::value;
    const dim3 grid((unsigned)((int64_t)P * pl.wg_per_range));
    const dim3 block(64 * kDecWaves);
    if (pl.ncw == 2) {
      if constexpr (DD <= 128) {
        if (pl.heads == 4) hipLaunchKernelGGL((decode_attn_kernel<DD, 2, 4>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((decode_attn_kernel<DD, 2, 1>), grid, block, 0, stream, p);
      }
    } else {
      if (pl.heads == 4) hipLaunchKernelGGL((decode_attn_kernel<DD, 1, 4>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((decode_attn_kernel<DD, 1, 1>), grid, block, 0, stream, p);
    }
  });
  if (e != hipSuccess) return e;
  const int64_t nout = (int64_t)a.B * a.Hkv * pl.ncg * pl.pc * (a.D / 4);
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)((nout + 255) / 256)), dim3(256), 0,
                     stream, p.rstart, p.rlen, p.part_o, p.part_ml, out, lse, a.K, a.Hq, a.Hkv,
                     p.G, p.GK, pl.ncg, pl.pc, a.D, nout);
  return hipGetLastError();
}

}  // namespace peagle

namespace peagle {

hipError_t launch_decode_append(const int32_t* cu, const int32_t* lens_in, const int32_t* n_new,
                                int32_t n_add, int32_t max_new, const uint16_t* k_new,
                                const uint16_t* v_new, const float* cs, const float* sn,
                                int32_t max_pos, uint16_t* kc, uint16_t* vt, int32_t* lens_out,
                                int32_t B, int32_t Hkv, int32_t D, int32_t max_ctx,
                                int64_t total_ctx, hipStream_t stream) {
  const int64_t rows = (int64_t)B * max_new * Hkv;
  const int64_t work = rows * (D / 16) + rows * (D / 8) + B;
  hipLaunchKernelGGL(decode_append_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0,
                     stream, cu, lens_in, n_new, n_add, max_new, k_new, v_new, cs, sn, max_pos, kc,
                     vt, lens_out, B, Hkv, D, max_ctx, total_ctx, decode_ntiles(total_ctx, B));
  return hipGetLastError();
}

}  // namespace peagle
