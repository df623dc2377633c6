// Multi-depth draft attention forward (flash-style, GQA), gfx950.
//
// NeMo Automodel PR 2376 (description): P-EAGLE reuses EAGLE-3's cache_hidden
// "diagonal extension" attention; its parity section equates it with a flat causal
// forward over [context, mask_1, ..., mask_{K-1}]. The snxtyle/P_Eagle README isolates
// packed conversations with cu_seqlens. So the query of draft row (d, p) sees
//   - the depth-0 keys p' of its own sequence with p' <= p (causal context), and
//   - its own anchor's depth-e rows for 1 <= e <= d (the diagonal extension).
//
// Work decomposition. Rows are visited in anchor-major order (all depths of anchor 0,
// then of anchor 1, ...; built by qlist_kernel). A workgroup owns a chunk of up to
// QR = 256/G consecutive rows of that list, never crossing a packed sequence, for all G
// q heads of one kv head: 256 query slots in 8 waves of 32, roughly 25 anchors and all
// their depths at K=4, G=4. Every row of the chunk reads a prefix of the same depth-0
// K/V, so each K/V tile is loaded to LDS once and used by all 256 slots (all depths, all
// heads of the group); halving the workgroup to 128 slots was measured 1.5x slower. Tiles wholly inside every row's range run unmasked; the one or
// two at the chunk's edge are masked per element; tiles past the last anchor are never
// visited. The diagonal keys of the chunk's anchors are a short contiguous run of the
// anchor-major list, processed as extra masked tiles.
//
// Staging. K and V^T tiles go global -> LDS by LDS DMA in its buffer form
// (buffer_load_dwordx4 ... lds, no register round trip) into two LDS buffers: tile t+1
// streams in while tile t is computed, one barrier per tile. The loop is unrolled by two so
// each buffer is a distinct static array and the compiler does not make LDS reads wait on
// the other buffer's loads; the buffer form (not global_load_lds) lets the LDS reads issued
// ahead of the MFMAs wait for themselves alone.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16). Scores are computed transposed,
// S^T = K * Q^T, so a lane holds one query column and 16 of the 32 keys of a tile: the
// softmax state is per lane and one cross-half exchange per tile gives the tile max.
// P^T stays in registers as the B operand of O^T = V^T * P^T: the 16 keys a lane holds
// for one 16-key step are exactly the 8+8 it must supply once the keys of each 16-key
// group are taken in the order (0-3, 8-11 | 4-7, 12-15); V^T tiles are stored in that
// order (v_transpose_kernel), so each PV operand is one 16-byte LDS read.
//
// Softmax: base-2 exponent with the 1/sqrt(D)*log2(e) factor folded into one FMA. The
// main kernel fixes each row's reference max m at its first tile (which holds the first
// key of the row's sequence, so it is finite) and never rescales: P = 2^(s - m) may grow
// above 1 but stays far from fp32/bf16 overflow as long as the row's softmax sum stays
// below 2^64, and floating point keeps the same relative precision at any scale. The O
// accumulators are then touched only by MFMAs inside the loop and stay in AGPRs. A row
// whose sum exceeds 2^64 (a later score more than ~40 above the first tile's maximum,
// in base-2 units) marks its chunk, which is then recomputed on the exact path with a
// rescaling online softmax: by the same workgroup when the key range is not split, else
// by a redo launch after the segments are merged.
//
// Precision. Rounding q', k' and P to bf16 perturbs each score by ~1e-3 and each weight
// by up to 2^-9; for a row whose output mixes only a handful of keys that moves it by
// up to ~1e-2 (outputs there reach |v| ~ 5). Chunks whose context span is short
// (<= kShortSpan keys: the first anchors of each sequence) take the exact path, which
// carries k' = k_hi + k_lo (k_lo from the RoPE kernel, two MFMAs per step of S^T) and
// P = P_hi + P_lo (two MFMAs per step of PV); q' stays bf16. Rows with many keys average
// the rounding out and take the plain path. Both paths live in one kernel: the short
// chunks are its last blocks (they fill the tail behind the long chunks).
//
// LDS layouts. K tiles: one 16-byte-padded row per key (stride 2D + 16 bytes), so the
// 32 keys a half-wave reads at one head-dim offset fall in distinct bank groups and a
// lane's 16 k-step reads share one base address. V^T tiles: rows of 32 keys (64 bytes),
// 16-byte chunk index XOR ((d >> 2) & 3).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace peagle {

namespace {

constexpr int KT = 32;  // keys per tile
constexpr int kMainNT = 1;   // query columns of 32 per wave in the main kernel
constexpr int kExactNT = 1;  // and in the exact / redo kernel
constexpr float kRescaleLog2 = 8.f;
constexpr float kSumLimit = 18446744073709551616.f;  // 2^64: above it a row is redone

template <int D, int NT>
struct Cfg {
  static constexpr int WAVES = kAttnSlots / (32 * NT);
  static constexpr int TH = 64 * WAVES;
  static constexpr int KROW = D * 2 + 16;         // padded K row
  static constexpr int KBUF = (KT * KROW + 1023) / 1024 * 1024;  // whole DMA blocks
  static constexpr int VBYTES = D * KT * 2;       // V^T tile: D rows x 32 keys
  static constexpr int KCH = KT * (D / 8);        // 16-byte chunks of a K tile
  static constexpr int DK = D / 16;               // k-steps of S^T
  static constexpr int MT = D / 32;               // 32-row M tiles of O^T
};

// V^T row d is 64 bytes (4 chunks of 8 keys); the chunk index is XOR-ed with bits 2-3 of
// d so the 16 rows read in one LDS cycle cover all 16 sixteen-byte slots of the 64 banks.
__device__ __forceinline__ int v_off(int d, int chunk) {
  return d * (KT * 2) + ((chunk ^ ((d >> 2) & 3)) << 4);
}

// Read-ahead depths (D = 256, 2 waves per SIMD): 2 K fragments and 3 V fragments are what
// fits in the 256-register budget beside O (128), Q (64) and S (16); one more spills a Q
// fragment to scratch inside the loop, whose reload then waits on the tile DMA. The split
// variant keeps its segment bounds live as well and reads V one fragment less ahead.
// D = 128 has registers to spare: 4 K and 6 V fragments ahead (measured ~2% faster than
// 2 / 3 at 55266 rows, 32/8 heads; 8 / 8 gained less).
constexpr int kPrefetchK = 2, kPrefetchV = 3;
template <int D> constexpr int prefetch_k() { return D == 128 ? 4 : kPrefetchK; }
template <int D> constexpr int prefetch_v() { return D == 128 ? 6 : kPrefetchV; }

struct AttnParams {
  const int4* qinfo;
  const int32_t* qstart;
  const int2* chunks;
  const int4* cmeta;  // [2 chunk], [2 chunk + 1]: the chunk's entries, key range, diagonal
  const int32_t* nchunks;
  const int32_t* seq_chunk;
  int32_t* flags;  // [chunk * Hkv + g]: the main kernel asks for a redo
  const uint16_t* qr;
  const uint16_t* kr;
  const uint16_t* kr_lo;
  const uint16_t* vt;
  const uint16_t* v;
  float* out;
  float* lse;
  int32_t* segs;  // [chunk * Hkv + g]: segments of the chunk (1: not split)
  int2* items;    // split main kernel's work list: (chunk * Hkv + g, segment | nseg << 8)
  int32_t* nitems;
  float* part;    // [segment - 1][T][Hq][D]: unnormalised O of segments 1.. of split chunks
  float2* ml;     // [segment][Hq][T]: (reference max, sum) of each segment of split chunks
  int n, T, S, Hq, Hkv, G, QR, ntiles, exact_per_seq, max_chunks, nsplit;
  int budget;  // work items the split main kernel runs at once (one round)
  int main_blocks;  // unsplit launch: blocks of the main path (chunk bound x kv heads)
  float c_log2;
};

// Key range of a chunk (rows j0 .. j0 + jn - 1 of the anchor-major list, one sequence):
// every row sees keys from k_lo (the sequence start) up to its own anchor, so the range is
// [k_lo, k_hi] and keys [full_lo, full_hi] are seen by every row (the prepare stage's
// chunk metadata holds them).
struct ChunkKeys {
  int k_lo, k_hi, full_lo, full_hi, p_first, p_last;
};

// Key-range split of a chunk's context tiles [t_first, t_last] into nseg segments. Segment
// j > 0 starts at tile b_j, a tile wholly inside [full_lo, full_hi]: every row sees all its
// keys, so each segment's first tile fixes a finite reference max for every row. A chunk
// with no such tile past its first is not split (splittable = false).
struct SegPlan {
  int t_first, t_last, ntl, bmin, bmax;
  bool splittable;
  __device__ int bound(int j, int nseg) const {
    return min(max(t_first + (int)((int64_t)j * ntl / nseg), bmin), bmax);
  }
};
__device__ __forceinline__ SegPlan seg_plan(const ChunkKeys& c) {
  SegPlan s;
  s.t_first = c.k_lo / KT;
  s.t_last = c.k_hi / KT;
  s.ntl = s.t_last - s.t_first + 1;
  s.bmin = max(s.t_first + 1, (c.full_lo + KT - 1) / KT);
  s.bmax = min(s.t_last, (c.full_hi + 1) / KT - 1);
  s.splittable = s.bmin <= s.bmax;
  return s;
}
// Segments of a chunk for a segment length of L tiles, at most nsplit.
__device__ __forceinline__ int seg_count(int ntl, int L, int nsplit) {
  return max(1, min(nsplit, (ntl + L - 1) / L));
}
constexpr int kMinSplitTiles = 8;  // shorter segments do not pay for their partial's merge
constexpr int kItemsMaxEntries = 4096;  // (chunk, kv head) entries the length search holds

// LDS of one workgroup, shared by the main and the exact paths: double-buffered K, V^T and
// (exact path) k_lo tiles, plus the chunk's key range and the diagonal keys' metadata.
template <int D>
struct AttnLds {
  using C = Cfg<D, 1>;
  alignas(1024) char Ks0[C::KBUF];
  alignas(1024) char Ks1[C::KBUF];
  alignas(1024) char Vs0[C::VBYTES];
  alignas(1024) char Vs1[C::VBYTES];
  alignas(1024) char Kl0[C::KBUF];
  alignas(1024) char Kl1[C::KBUF];
  int kp[KT], kd[KT];
  int bad;  // main path: some row's fixed-reference sum left the safe range
};

// One (chunk, kv head) of the attention, or one segment of it (SPLIT). EXACT = false: the
// main path, chunks with a long context span (a short chunk returns at once); it sets
// L.bad when a row's sum overflowed. EXACT = true: chunks with a short span (k' and P
// split into bf16 pairs), or with `redo` a chunk the main path flagged (rescaling online
// softmax on k' alone). Every thread of the workgroup calls it with the same arguments.
template <int D, bool EXACT, bool SPLIT>
__device__ __forceinline__ void attn_chunk(const AttnParams& p, AttnLds<D>& L, int chunk, int g,
                                           int seg, int nseg, bool redo) {
  constexpr int NT = EXACT ? kExactNT : kMainNT;
  using C = Cfg<D, NT>;
  char* const Ks0 = L.Ks0;
  char* const Ks1 = L.Ks1;
  char* const Vs0 = L.Vs0;
  char* const Vs1 = L.Vs1;
  char* const Kl0 = L.Kl0;
  char* const Kl1 = L.Kl1;
  int* const s_kp = L.kp;
  int* const s_kd = L.kd;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, half = lane >> 5;
  const int n = p.n, T = p.T, Hkv = p.Hkv;
  // the chunk's metadata, laid out by the prepare stage: one uniform load
  const int4 cm0 = p.cmeta[2 * chunk], cm1 = p.cmeta[2 * chunk + 1];
  const int j0 = cm0.x, jn = cm0.y;
  const int k_lo = cm0.z, k_hi = cm0.w;          // first and last key of any row
  const int full_lo = cm1.x, full_hi = cm1.y;    // keys every row sees
  const int dg_lo = cm1.z, dg_hi = cm1.w;        // list entries of the chunk's anchors
  if (tid == 0) L.bad = 0;
  __syncthreads();
  const bool is_short = (k_hi - k_lo + 1) <= kShortSpan;  // uniform over the workgroup
  if (EXACT ? (!is_short && !redo) : is_short) return;


  // Query slots of this lane: NT columns of 32 (lanes l and l+32 share a column, each
  // holding 16 of the 32 keys of a tile); loaded once the first tile's DMA is in flight.
  int q_row[NT], q_head[NT], q_p[NT], q_d[NT], q_lo[NT];
  bool q_on[NT];
  bf16x8 qf[NT][C::DK];
  // D = 256 on the main path: the last k-step's q fragment of each lane is kept in LDS (the
  // k_lo buffer, which this path does not use) and read with the tile's K fragments. At the
  // 256-register limit the compiler otherwise spills one to scratch and reloads it every
  // tile behind the next tile's DMA, whose completion the reload's vmcnt wait then awaits.
  constexpr bool kQInLds = !EXACT && D == 256;
  char* const q_lds = Kl0 + tid * 16 * NT;

  floatx16 o[NT][C::MT];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[nt][mt][r] = 0.f;
  }

  // One tile: S^T = K Q^T -> mask -> softmax weights -> O^T += V^T P^T.
  // mode 0: no mask, 1: context range, 2: diagonal keys (meta in s_kp / s_kd).
  // SET_MAX: the main kernel's first tile fixes the reference max.
  auto compute = [&](const char* Ks, const char* Kl, const char* Vs, int mode, int key0,
                     bool set_max) {
    floatx16 s[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nt][r] = 0.f;
    const char* kbase = Ks + r32 * C::KROW + half * 16;
    if constexpr (!EXACT) {
      // K fragments are read prefetch_k<D>() steps ahead of the MFMA that uses them, so LDS
      // latency overlaps the MFMA chain instead of stalling each step.
      bf16x8 kf[C::DK];
#pragma unroll
      for (int kk = 0; kk < C::DK; ++kk)
        kf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(kbase + kk * 32));
      bf16x8 ql[NT];
      if constexpr (kQInLds) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) ql[nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(q_lds + nt * 16));
      }
#pragma unroll
      for (int kk = 0; kk < C::DK; ++kk)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          s[nt] = mfma32(kf[kk], kQInLds && kk == C::DK - 1 ? ql[nt] : qf[nt][kk], s[nt]);
      if constexpr (kQInLds) {
        // the q read goes with the first read-ahead group
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, prefetch_k<D>() + NT, 0);
#pragma unroll
        for (int i = 0; i < C::DK - prefetch_k<D>(); ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, NT, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, prefetch_k<D>() * NT, 0);
      } else {
        sched_reads_ahead<C::DK, prefetch_k<D>(), NT>();
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < C::DK; ++kk) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(kbase + kk * 32));
        const bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4*>(Kl + (kbase - Ks) + kk * 32));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          s[nt] = mfma32(a, qf[nt][kk], s[nt]);
          s[nt] = mfma32(al, qf[nt][kk], s[nt]);
        }
      }
    }
    if (mode == 1) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key < q_lo[nt] || key > q_p[nt]) s[nt][r] = -INFINITY;
        }
    } else if (mode == 2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = 8 * (r >> 2) + 4 * half + (r & 3);
        const int kp = s_kp[kl], kd = s_kd[kl];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          if (kp != q_p[nt] || kd < 1 || kd > q_d[nt]) s[nt][r] = -INFINITY;
      }
    }
    if (EXACT || set_max) {
      float m_new[NT];
      bool need = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float mx = fmaxf(s[nt][0], s[nt][1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[nt][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        m_new[nt] = fmaxf(m_run[nt], mx * p.c_log2);
        need |= m_new[nt] > m_run[nt] + kRescaleLog2;
      }
      if constexpr (EXACT) {
        if (__any(need)) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const float alpha = (m_new[nt] == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[nt] - m_new[nt]);
            l_run[nt] *= alpha;
#pragma unroll
            for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[nt][mt][r] *= alpha;
            m_run[nt] = m_new[nt];
          }
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) m_run[nt] = m_new[nt];  // O is still zero
      }
    }
    bf16x8 pb[NT][2];
    [[maybe_unused]] bf16x8 pl[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mu = (m_run[nt] == -INFINITY) ? 0.f : m_run[nt];
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[nt][r], p.c_log2, -mu));
        ls += pr;
        pb[nt][r >> 3][r & 7] = (__bf16)pr;
        if constexpr (EXACT) pl[nt][r >> 3][r & 7] = (__bf16)(pr - (float)pb[nt][r >> 3][r & 7]);
      }
      l_run[nt] += ls;
    }
    if constexpr (!EXACT) {
      bf16x8 vf[C::MT][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
          vf[mt][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(Vs + v_off(mt * 32 + r32, ks * 2 + half)));
      // k-step outer: the two MFMAs into one O tile are MT apart, not back to back
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[nt][mt] = mfma32(vf[mt][ks], pb[nt][ks], o[nt][mt]);
      sched_reads_ahead<2 * C::MT, SPLIT ? prefetch_v<D>() - 1 : prefetch_v<D>(), NT>();
    } else {
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(Vs + v_off(mt * 32 + r32, ks * 2 + half)));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            o[nt][mt] = mfma32(a, pb[nt][ks], o[nt][mt]);
            o[nt][mt] = mfma32(a, pl[nt][ks], o[nt][mt]);
          }
        }
    }
  };

  // ---- causal context: depth-0 key tiles, streamed by LDS DMA ----
  // A wave moves 1 KB per instruction: lane i fills bytes [16 i, 16 i + 16) of that KB.
  // Each lane's source offset inside a tile does not depend on the tile, so it is computed
  // once; the tile base is uniform (scalar registers). The last tile may reach up to 31
  // rows past key n - 1: the K regions carry that many rows of padding, and such keys are
  // always masked.
  constexpr int KI = (C::KBUF / 1024 + C::WAVES - 1) / C::WAVES;  // K blocks per wave
  constexpr int VI = (C::VBYTES / 1024 + C::WAVES - 1) / C::WAVES;
  uint32_t koff[KI], voff[VI];
#pragma unroll
  for (int j = 0; j < KI; ++j) {
    const int P = (wave + j * C::WAVES) * 1024 + lane * 16;
    const int key = P / C::KROW, off = P - key * C::KROW;
    const bool real = key < KT && off < D * 2;  // else padding: any valid source
    koff[j] = real ? (uint32_t)(key * Hkv * D * 2 + off) : 0u;
  }
#pragma unroll
  for (int j = 0; j < VI; ++j) {
    const int P = (wave + j * C::WAVES) * 1024 + lane * 16;
    const int d = P >> 6, c = ((P >> 4) & 3) ^ ((d >> 2) & 3);
    voff[j] = (uint32_t)((d * KT + c * 8) * 2);
  }
  auto dma_k = [&](const uint16_t* src, int t, char* dst) {
    // the tile's KT rows of kv head g, Hkv * D apart
    const auto range = dma_range(uniform_opaque(reinterpret_cast<const char*>(src + ((size_t)t * KT * Hkv + g) * D)),
                                 (uint32_t)(((KT - 1) * Hkv + 1) * D * 2));
#pragma unroll
    for (int j = 0; j < KI; ++j) {
      const int i = wave + j * C::WAVES;
      if (i < C::KBUF / 1024) dma16_buf(range, koff[j], dst + i * 1024);
    }
  };
  auto dma_v = [&](int t, char* dst) {
    const auto range = dma_range(uniform_opaque(reinterpret_cast<const char*>(p.vt + ((size_t)g * p.ntiles + t) * (size_t)(D * KT))),
                                 (uint32_t)(D * KT * 2));
#pragma unroll
    for (int j = 0; j < VI; ++j) {
      const int i = wave + j * C::WAVES;
      if (i < C::VBYTES / 1024) dma16_buf(range, voff[j], dst + i * 1024);
    }
  };
  auto issue = [&](int t, char* Kd, char* Kld, char* Vd) {
    dma_k(p.kr, t, Kd);
    if (EXACT && !redo) dma_k(p.kr_lo, t, Kld);
    dma_v(t, Vd);
  };

  // Context tiles of this workgroup: all of [t_first, t_last], or one segment of them. The
  // last segment also takes the masked edge tiles and the diagonal keys.
  const int t_first = k_lo / KT, t_last = k_hi / KT;
  int t_begin = t_first, t_end = t_last;
  if constexpr (SPLIT) {  // segment seg of the nseg the work list chose for this chunk
    const SegPlan sp = seg_plan(ChunkKeys{k_lo, k_hi, full_lo, full_hi, 0, 0});
    if (seg > 0) t_begin = sp.bound(seg, nseg);
    if (seg < nseg - 1) t_end = sp.bound(seg + 1, nseg) - 1;
  }
  if constexpr (EXACT) {
    // k_lo exists only for the first kShortSpan positions of each sequence (the short
    // chunks). A chunk redone for its softmax sum is past them: it runs on k' alone, its
    // k_lo buffers held at zero (the first barrier below orders these stores).
    if (redo)
      for (int q = tid; q < C::KBUF / 16; q += C::TH) {
        *reinterpret_cast<u32x4*>(Kl0 + q * 16) = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(Kl1 + q * 16) = u32x4{0u, 0u, 0u, 0u};
      }
  }
  if (!SPLIT || t_begin <= t_end) issue(t_begin, Ks0, Kl0, Vs0);
  // The diagonal keys' data of the first kPreDiag tiles (D <= 128, where registers are to
  // spare): the list entry of this thread's key, then its K (and k_lo) and V chunk, loaded
  // beside the query fragments' own two round trips and held through the context loop, so
  // the diagonal phase after it does not wait on them.
  const int jd0 = seg == nseg - 1 ? dg_lo : dg_hi;  // first diagonal tile
  constexpr int kPreDiag = D <= 128 ? 2 : 0;
  constexpr int kPreSlots = kPreDiag > 0 ? kPreDiag : 1;
  int4 pre_e[kPreSlots];  // entry jb + tid, for s_kp / s_kd (threads below KT)
  u32x4 pre_k[kPreSlots], pre_v[kPreSlots], pre_l[kPreSlots];
  if constexpr (kPreDiag > 0) {
    int pre_row[kPreSlots];
#pragma unroll
    for (int i = 0; i < kPreDiag; ++i) {
      const int jb = jd0 + i * KT;
      const int jk = jb + tid / (D / 8);
      pre_e[i] = tid < KT && jb + tid < dg_hi ? p.qinfo[jb + tid] : int4{-1, 0, 0, 0};
      pre_row[i] = tid < C::KCH && jk < dg_hi ? min(max(p.qinfo[jk].x, 0), T - 1) : -1;
    }
#pragma unroll
    for (int i = 0; i < kPreDiag; ++i) {
      const int c = tid % (D / 8);
      pre_k[i] = pre_v[i] = pre_l[i] = u32x4{0u, 0u, 0u, 0u};
      if (pre_row[i] >= 0) {
        const size_t at = ((size_t)pre_row[i] * Hkv + g) * D + c * 8;
        pre_k[i] = *reinterpret_cast<const u32x4*>(p.kr + at);
        pre_v[i] = *reinterpret_cast<const u32x4*>(p.v + at);
        if (EXACT && !redo) pre_l[i] = *reinterpret_cast<const u32x4*>(p.kr_lo + at);
      }
    }
  }
  // the query fragments: the row list entry, then the rotated q row (two round trips that
  // overlap the first tile's)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int slot = wave * 32 * NT + nt * 32 + r32;
    const int rl = slot % p.QR, hl = slot / p.QR;
    q_on[nt] = rl < jn;
    const int4 qi = p.qinfo[j0 + min(rl, jn - 1)];
    q_row[nt] = min(max(qi.x, 0), T - 1);
    q_p[nt] = min(max(qi.y, 0), n - 1);
    q_d[nt] = qi.z;
    q_lo[nt] = min(max(qi.w, 0), q_p[nt]);
    q_head[nt] = g * p.G + hl;
    const uint16_t* qrow = p.qr + ((size_t)q_row[nt] * p.Hq + q_head[nt]) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < C::DK; ++kk)
      qf[nt][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + kk * 16));
    if constexpr (kQInLds) *reinterpret_cast<bf16x8*>(q_lds + nt * 16) = qf[nt][C::DK - 1];
  }
  for (int t = t_begin; t <= t_end; t += 2) {
    wait_dma();
    __syncthreads();  // tile t landed in buffer 0; buffer 1 is free
    if (t + 1 <= t_end) issue(t + 1, Ks1, Kl1, Vs1);
    {
      const int key0 = t * KT;
      const bool full = key0 >= full_lo && key0 + KT - 1 <= full_hi;
      compute(Ks0, Kl0, Vs0, full ? 0 : 1, key0, t == t_begin);
    }
    if (t + 1 > t_end) break;
    wait_dma();
    __syncthreads();  // tile t+1 landed in buffer 1; buffer 0 is free
    if (t + 2 <= t_end) issue(t + 2, Ks0, Kl0, Vs0);
    {
      const int key0 = (t + 1) * KT;
      const bool full = key0 >= full_lo && key0 + KT - 1 <= full_hi;
      compute(Ks1, Kl1, Vs1, full ? 0 : 1, key0, false);
    }
  }

  // ---- diagonal extension: depth >= 1 rows of the chunk's anchors ----
  for (int jb = jd0; jb < dg_hi; jb += KT) {
    __syncthreads();
    const int di = (jb - jd0) / KT;  // diagonal tile index: the first kPreDiag are loaded
    if (tid < KT) {
      const int jk = jb + tid;
      int kp = -1, kd = 0;
      if (di < kPreDiag) {
#pragma unroll
        for (int i = 0; i < kPreDiag; ++i)
          if (i == di) {
            kp = jk < dg_hi ? pre_e[i].y : -1;
            kd = jk < dg_hi ? pre_e[i].z : 0;
          }
      } else if (jk < dg_hi) {
        const int4 e = p.qinfo[jk];
        kp = e.y;
        kd = e.z;
      }
      s_kp[tid] = kp;
      s_kd[tid] = kd;
    }
    for (int q = tid; q < C::KCH; q += C::TH) {
      const int key = q / (D / 8), c = q % (D / 8), jk = jb + key;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u}, kl = {0u, 0u, 0u, 0u};
      if (di < kPreDiag && q == tid) {
#pragma unroll
        for (int i = 0; i < kPreDiag; ++i)
          if (i == di) {
            kv = pre_k[i];
            vv = pre_v[i];
            kl = pre_l[i];
          }
      } else if (jk < dg_hi) {
        const int row = min(max(p.qinfo[jk].x, 0), T - 1);
        kv = *reinterpret_cast<const u32x4*>(p.kr + ((size_t)row * Hkv + g) * D + c * 8);
        vv = *reinterpret_cast<const u32x4*>(p.v + ((size_t)row * Hkv + g) * D + c * 8);
        if (EXACT && !redo) kl = *reinterpret_cast<const u32x4*>(p.kr_lo + ((size_t)row * Hkv + g) * D + c * 8);
      }
      *reinterpret_cast<u32x4*>(Ks0 + key * C::KROW + c * 16) = kv;
      if constexpr (EXACT) *reinterpret_cast<u32x4*>(Kl0 + key * C::KROW + c * 16) = kl;
      // scatter the 8 d-values of this key into the V^T tile (key order as in v_transpose)
      const int vchunk = 2 * (key >> 4) + ((key & 7) >> 2);
      const int elem = 4 * ((key & 15) >> 3) + (key & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = c * 8 + e;
        *reinterpret_cast<uint16_t*>(Vs0 + v_off(d, vchunk) + elem * 2) =
            (uint16_t)((vv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      }
    }
    __syncthreads();
    // Entries are anchor-major, so the tile's anchors run from s_kp[0] to that of its last
    // entry. A wave none of whose rows has its anchor in that run (or a depth >= 1) would
    // get only -inf scores from the tile, zero weights and an unchanged O: it skips it.
    bool sees = false;
    {
      const int a_lo = s_kp[0], a_hi = s_kp[min(KT, dg_hi - jb) - 1];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sees |= q_d[nt] >= 1 && q_p[nt] >= a_lo && q_p[nt] <= a_hi;
    }
    if (__any(sees)) compute(Ks0, Kl0, Vs0, 2, 0, false);
  }

  // ---- epilogue: O / l, lse; the main kernel flags rows whose sum left the safe range ----
  // A segment of a split chunk stores its unnormalised O (segment 0 into out, segment j
  // into part[j - 1]) and its (reference max, sum); the combine kernel merges them.
  const bool partial = SPLIT && nseg > 1;
  bool bad = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = l_run[nt] + __shfl_xor(l_run[nt], 32, 64);
    if constexpr (!EXACT) bad |= q_on[nt] && !(lt <= kSumLimit);
    const float inv = partial ? 1.f : 1.f / lt;
    if (q_on[nt]) {
      float* dst = (SPLIT && seg > 0 ? p.part + (size_t)(seg - 1) * T * p.Hq * D : p.out) +
                   ((size_t)q_row[nt] * p.Hq + q_head[nt]) * D;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          floatx4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = o[nt][mt][4 * i + j] * inv;
          *reinterpret_cast<floatx4*>(dst + mt * 32 + 8 * i + 4 * half) = w;
        }
      if (partial) {
        if (half == 0)
          p.ml[((size_t)seg * p.Hq + q_head[nt]) * T + q_row[nt]] = make_float2(m_run[nt], lt);
      } else if (p.lse != nullptr && half == 0) {
        p.lse[(size_t)q_head[nt] * T + q_row[nt]] = (m_run[nt] + __log2f(lt)) * 0.69314718055994531f;
      }
    }
  }
  if constexpr (!EXACT) {
    if (__any(bad) && lane == 0) L.bad = 1;
  }
}

// Roles of the attention launches.
//   kRoleMain  (the key range is not split): blocks [0, main_blocks) take the chunks
//              heaviest first on the main path, and redo their own chunk with the exact
//              path when a row's sum overflowed; the blocks after them take the short
//              chunks, so those fill the tail of the launch.
//   kRoleSplit (key-range split): blocks [0, short_blocks) take the short chunks, the rest
//              the (chunk, segment) work list; an overflow flags the chunk.
//   kRoleRedo  (after the split's merge): the flagged chunks, exact path.
enum { kRoleMain = 0, kRoleSplit = 1, kRoleRedo = 2 };

template <int D, int ROLE>
__global__ __launch_bounds__(2 * kAttnSlots) void attn_core_kernel(const AttnParams p) {
  static_assert(kMainNT == kExactNT, "one LDS layout for both paths");
  __shared__ AttnLds<D> L;
  const int bid = blockIdx.x;
  const int short_blocks = p.S * p.exact_per_seq * p.Hkv;
  if constexpr (ROLE == kRoleRedo) {
    const int chunk = bid / p.Hkv, g = bid % p.Hkv;
    if (chunk >= min(*p.nchunks, p.max_chunks) || p.flags[chunk * p.Hkv + g] == 0) return;
    attn_chunk<D, true, false>(p, L, chunk, g, 0, 1, true);
    if (threadIdx.x == 0) p.flags[chunk * p.Hkv + g] = 0;
    return;
  }
  const int sb = ROLE == kRoleMain ? bid - p.main_blocks : bid;
  int chunk, g;
  bool redo = false;
  if (sb >= 0 && sb < short_blocks) {  // one of the first chunks of a sequence
    const int r = sb / p.Hkv;
    const int s = r / p.exact_per_seq, j = r % p.exact_per_seq;
    g = sb % p.Hkv;
    chunk = p.seq_chunk[s] + j;
    if (chunk >= p.seq_chunk[s + 1]) return;
  } else if constexpr (ROLE == kRoleMain) {
    // Chunks are listed sequence by sequence, anchors ascending: the last ones have the
    // longest prefixes, so they are dispatched first. The grid is sized for the largest
    // possible chunk count; blocks past the actual count exit.
    chunk = *p.nchunks - 1 - bid / p.Hkv;
    g = bid % p.Hkv;
    if (chunk < 0) return;
    attn_chunk<D, false, false>(p, L, chunk, g, 0, 1, false);
    __syncthreads();
    if (!L.bad) return;
    __syncthreads();  // every wave has read L.bad before the redo clears it
    redo = true;
  } else {
    // the work list of the split, in the same heaviest-first order
    const int item = sb - short_blocks;
    if (item >= *p.nitems) return;
    const int2 it = p.items[item];
    g = it.x % p.Hkv;
    chunk = it.x / p.Hkv;
    attn_chunk<D, false, true>(p, L, chunk, g, it.y & 255, max(it.y >> 8, 1), false);
    __syncthreads();
    if (threadIdx.x == 0 && L.bad) p.flags[chunk * p.Hkv + g] = 1;
    return;
  }
  attn_chunk<D, true, false>(p, L, chunk, g, 0, 1, redo);
}

// Work list of the split main kernel, one workgroup. Every (chunk, kv head) entry, heaviest
// chunks first, gets one item per segment; chunks with a short span (run by the exact
// kernel) get none. The segment length L is chosen from the chunks' actual spans: the
// smallest L (>= kMinSplitTiles) whose item count fits p.budget, the workgroups that run at
// once, so the split finishes in one round bounded by the longest segment. The candidates
// are 1024 evenly spaced lengths; the item count does not grow with L, so the first that
// fits is bracketed in three rounds (strides 64, 4, 1), each wave counting one candidate
// over all entries. If none fits, nothing is split. Also writes each entry's segment count
// for the merge.
__global__ __launch_bounds__(1024) void attn_items_kernel(const AttnParams p) {
  __shared__ int s_ntl[kItemsMaxEntries];  // tiles (splittable), -1 (not splittable), 0 (short)
  __shared__ int s_wave[16];
  __shared__ int s_fits[16];
  __shared__ int s_carry, s_best, s_maxntl;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nc = min(max(*p.nchunks, 0), p.max_chunks);
  const int total = nc * p.Hkv;
  const bool search = total <= kItemsMaxEntries;
  if (tid == 0) {
    s_carry = 0;
    s_best = 1 << 30;  // no split
    s_maxntl = 0;
  }
  __syncthreads();
  auto entry = [&](int i, int& key, SegPlan& sp) {
    const int chunk = nc - 1 - i / p.Hkv, g = i % p.Hkv;
    key = chunk * p.Hkv + g;
    const int4 cm0 = p.cmeta[2 * chunk], cm1 = p.cmeta[2 * chunk + 1];
    const ChunkKeys c{cm0.z, cm0.w, cm1.x, cm1.y, 0, 0};
    sp = seg_plan(c);
    return c.k_hi - c.k_lo + 1 > kShortSpan;  // else short
  };
  if (search) {
    int mx = 0;
    for (int i = tid; i < total; i += 1024) {
      int key;
      SegPlan sp;
      const bool on = entry(i, key, sp);
      const int v = !on ? 0 : (sp.splittable ? sp.ntl : -1);
      s_ntl[i] = v;
      mx = max(mx, v);
    }
    atomicMax(&s_maxntl, mx);
    __syncthreads();
    const int lo = kMinSplitTiles, hi = max(s_maxntl, lo);
    const int step = (hi - lo + 1024) / 1024;
    const int ng = min(1024, (hi - lo) / step + 1);  // candidates lo + i * step, i < ng
    // fits(i): candidate i's item count is within the budget (true past the last one)
    auto fits = [&](int i) {
      if (i >= ng) return true;
      const int L = lo + i * step;
      // seg_count for every entry, with ceil(v / L) from a float reciprocal corrected to
      // the exact integer (v + L - 1 < 2^24): integer division is a long instruction
      // sequence
      const float inv = 1.f / (float)L;
      int cnt = 0;
      for (int e = lane; e < total; e += 64) {
        const int v = s_ntl[e];
        const int x = v + L - 1;
        int q = (int)((float)x * inv);
        q -= q * L > x ? 1 : 0;
        q += (q + 1) * L <= x ? 1 : 0;
        cnt += v > 0 ? max(1, min(p.nsplit, q)) : (v < 0 ? 1 : 0);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
      return cnt <= p.budget;
    };
    // The first fitting index lies in [base, base + 16 * stride) (1024 when none does);
    // wave w tests the last index of its sub-range, and the first wave whose test fits
    // narrows the range to that sub-range. Strides 64, 4, 1: the last range holds 4
    // indices, and the waves past them test indices that fit whenever the range's last one
    // does.
    int base = 0;
    for (int stride = 64;; stride = stride == 64 ? 4 : 1) {
      const int probe = base + (wave + 1) * stride - 1;
      const bool f = (stride > 1 || wave < 4) ? fits(probe) : true;
      if (lane == 0) s_fits[wave] = f ? 1 : 0;
      __syncthreads();
      int w = 0;
      while (w < 16 && !s_fits[w]) ++w;
      base += w * stride;
      __syncthreads();
      if (stride == 1) break;
    }
    if (tid == 0 && base < ng) s_best = lo + base * step;
    __syncthreads();
  }
  const int L = s_best;
  for (int base = 0; base < total; base += 1024) {
    const int i = base + tid;
    int nseg = 0, key = 0;
    SegPlan sp;
    if (i < total) {
      if (entry(i, key, sp)) nseg = sp.splittable ? seg_count(sp.ntl, L, p.nsplit) : 1;
      p.segs[key] = max(nseg, 1);
    }
    // exclusive scan of nseg over the block
    int incl = nseg;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int before = s_carry;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    const int at = before + incl - nseg;
    for (int j = 0; j < nseg; ++j) p.items[at + j] = make_int2(key, j | (nseg << 8));
    __syncthreads();
    if (tid == 1023) s_carry = at + nseg;
    __syncthreads();
  }
  if (tid == 0) *p.nitems = s_carry;
}

// Merge of the segments of split chunks. Slot (row, head) of a chunk cut into nseg
// segments: M = max_j m_j, w_j = 2^(m_j - M), out = sum_j w_j O_j / sum_j w_j l_j,
// lse = (M + log2 sum_j w_j l_j) ln 2. One wave per slot, D / 64 floats per lane; blocks
// (chunk * Hkv + g, 4 of the chunk's 256 slots), so every slot's loads are in flight at
// once. Chunks flagged for a redo are skipped: the exact kernel rewrites them afterwards.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnParams p) {
  constexpr int VW = D / 64;
  const int g = blockIdx.x % p.Hkv;
  const int chunk = blockIdx.x / p.Hkv;
  if (chunk >= min(*p.nchunks, p.max_chunks)) return;
  const int nseg = min(p.segs[chunk * p.Hkv + g], p.nsplit);
  if (nseg <= 1 || p.flags[chunk * p.Hkv + g] != 0) return;
  const int2 ch = p.chunks[chunk];
  const int j0 = min(max(ch.x, 0), p.T - 1);
  const int jn = min(max(ch.y, 1), p.T - j0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t seg_stride = (size_t)p.T * p.Hq * D;
  const int s = blockIdx.y * 4 + wave;
  if (s < jn * p.G) {
    const int rl = s % jn, h = g * p.G + s / jn;
    const int row = min(max(p.qinfo[j0 + rl].x, 0), p.T - 1);
    float2 ml[kMaxAttnSplit];
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxAttnSplit; ++j)
      if (j < nseg) {
        ml[j] = p.ml[((size_t)j * p.Hq + h) * p.T + row];
        M = fmaxf(M, ml[j].x);
      }
    float L = 0.f, acc[VW];
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[e] = 0.f;
    const size_t off = ((size_t)row * p.Hq + h) * D + lane * VW;
#pragma unroll
    for (int j = 0; j < kMaxAttnSplit; ++j)
      if (j < nseg) {
        const float w = ml[j].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[j].x - M);
        L += w * ml[j].y;
        const float* src = (j == 0 ? p.out : p.part + (size_t)(j - 1) * seg_stride) + off;
#pragma unroll
        for (int e = 0; e < VW; ++e) acc[e] += w * src[e];
      }
    const float inv = 1.f / L;
    float* dst = p.out + off;
#pragma unroll
    for (int e = 0; e < VW; ++e) dst[e] = acc[e] * inv;
    if (p.lse != nullptr && lane == 0)
      p.lse[(size_t)h * p.T + row] = (M + __log2f(L)) * 0.69314718055994531f;
  }
}

}  // namespace

constexpr int kMaxDevices = 64;

// Compute units of the current device, cached per device (every thread that fills an
// entry stores the same value, so relaxed atomics suffice).
int device_cus() {
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

hipError_t launch_attn_core(const AttnArgs& a, const uint16_t* v, float* out, float* lse,
                            const char* ws, hipStream_t stream) {
  const AttnLayout L = attn_layout(a.n, a.T, a.Hq, a.Hkv, a.D);
  AttnParams p;
  p.qinfo = reinterpret_cast<const int4*>(ws + L.qinfo);
  p.qstart = reinterpret_cast<const int32_t*>(ws + L.qstart);
  p.chunks = reinterpret_cast<const int2*>(ws + L.chunks);
  p.cmeta = reinterpret_cast<const int4*>(ws + L.cmeta);
  p.nchunks = reinterpret_cast<const int32_t*>(ws + L.nchunks);
  p.seq_chunk = reinterpret_cast<const int32_t*>(ws + L.seq_chunk);
  p.flags = reinterpret_cast<int32_t*>(const_cast<char*>(ws) + L.flags);
  p.qr = reinterpret_cast<const uint16_t*>(ws + L.qrot);
  p.kr = reinterpret_cast<const uint16_t*>(ws + L.krot);
  p.kr_lo = reinterpret_cast<const uint16_t*>(ws + L.krot_lo);
  p.vt = reinterpret_cast<const uint16_t*>(ws + L.vt);
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.segs = reinterpret_cast<int32_t*>(const_cast<char*>(ws) + L.segs);
  p.items = reinterpret_cast<int2*>(const_cast<char*>(ws) + L.items);
  p.nitems = reinterpret_cast<int32_t*>(const_cast<char*>(ws) + L.nitems);
  p.part = reinterpret_cast<float*>(const_cast<char*>(ws) + L.part);
  p.ml = reinterpret_cast<float2*>(const_cast<char*>(ws) + L.ml);
  p.nsplit = attn_split_plan(a.n, a.T, a.Hq, a.Hkv).nsplit;
  p.n = a.n;
  p.T = a.T;
  p.S = a.S;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.G = a.Hq / a.Hkv;
  p.QR = kAttnSlots / p.G;
  p.ntiles = (a.n + 31) / 32;
  p.exact_per_seq = attn_exact_chunks_per_seq(a.K, p.QR);
  p.max_chunks = L.max_chunks;
  p.c_log2 = a.scale * 1.4426950408889634f;
  // Unsplit: one launch, the main path's blocks heaviest chunk first, then the short chunks
  // (exact path) filling the tail; a chunk whose sums overflow is redone by its own block.
  // Split: the work list, one launch of the short chunks and the segments, the merge, then
  // the redo of flagged chunks. All on the caller's stream: the library keeps no streams or
  // events of its own.
  // chunk count <= ceil(T / QR) + S (each sequence adds at most one partial chunk)
  const int chunk_bound = std::min(L.max_chunks, (a.T + p.QR - 1) / p.QR + a.S);
  const int short_blocks = a.S * p.exact_per_seq * a.Hkv;
  p.main_blocks = chunk_bound * a.Hkv;
  const dim3 main_grid(p.main_blocks + short_blocks);
  const dim3 split_grid(short_blocks + chunk_bound * a.Hkv * p.nsplit);
  const dim3 combine_grid(chunk_bound * a.Hkv, kAttnSlots / 4);
  const dim3 redo_grid(chunk_bound * a.Hkv);
  const dim3 block(2 * kAttnSlots);
  if (p.nsplit > 1) {
    // one round of the split launch: its resident workgroups over the chip, less the short
    // chunks' workgroups that run beside the segments
    int per_cu = 1;
    hipError_t eo = hipErrorInvalidValue;
#define PEAGLE_OCC(DD)                                                                      \
  eo = hipOccupancyMaxActiveBlocksPerMultiprocessor(                                        \
      &per_cu, reinterpret_cast<const void*>(&attn_core_kernel<DD, kRoleSplit>),            \
      2 * kAttnSlots, 0)
    switch (a.D) {
      case 64: PEAGLE_OCC(64); break;
      case 128: PEAGLE_OCC(128); break;
      case 256: PEAGLE_OCC(256); break;
      default: break;
    }
#undef PEAGLE_OCC
    if (eo != hipSuccess) per_cu = 1;
    p.budget = std::max(1, std::max(1, per_cu) * device_cus() - short_blocks);
  }
#define PEAGLE_CORE(DD)                                                                       \
  do {                                                                                        \
    if (p.nsplit > 1) {                                                                       \
      hipLaunchKernelGGL(attn_items_kernel, dim3(1), dim3(1024), 0, stream, p);               \
      hipLaunchKernelGGL((attn_core_kernel<DD, kRoleSplit>), split_grid, block, 0, stream, p); \
      hipLaunchKernelGGL((attn_combine_kernel<DD>), combine_grid, dim3(256), 0, stream, p);   \
      hipLaunchKernelGGL((attn_core_kernel<DD, kRoleRedo>), redo_grid, block, 0, stream, p);  \
    } else {                                                                                  \
      hipLaunchKernelGGL((attn_core_kernel<DD, kRoleMain>), main_grid, block, 0, stream, p);  \
    }                                                                                         \
  } while (0)
  switch (a.D) {
    case 64: PEAGLE_CORE(64); break;
    case 128: PEAGLE_CORE(128); break;
    case 256: PEAGLE_CORE(256); break;
    default: return hipErrorInvalidValue;
  }
#undef PEAGLE_CORE
  return hipGetLastError();
}

}  // namespace peagle
