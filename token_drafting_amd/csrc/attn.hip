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
// Staging. K and V^T tiles go global -> LDS with global_load_lds_dwordx4 (no register
// round trip) into two LDS buffers: tile t+1 streams in while tile t is computed, one
// barrier per tile. The loop is unrolled by two so each buffer is a distinct static
// array and the compiler does not make LDS reads wait on the other buffer's loads.
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
// in base-2 units) flags its chunk, and the second kernel recomputes the chunk with a
// rescaling online softmax.
//
// Precision. Rounding q', k' and P to bf16 perturbs each score by ~1e-3 and each weight
// by up to 2^-9; for a row whose output mixes only a handful of keys that moves it by
// up to ~1e-2 (outputs there reach |v| ~ 5). Chunks whose context span is short
// (<= kShortSpan keys: the first anchors of each sequence) run in the second kernel,
// which also carries k' = k_hi + k_lo (k_lo from the RoPE kernel, two MFMAs per step of
// S^T) and P = P_hi + P_lo (two MFMAs per step of PV); q' stays bf16. Rows with many
// keys average the rounding out and take the plain path.
//
// LDS layouts. K tiles: one 16-byte-padded row per key (stride 2D + 16 bytes), so the
// 32 keys a half-wave reads at one head-dim offset fall in distinct bank groups and a
// lane's 16 k-step reads share one base address. V^T tiles: rows of 32 keys (64 bytes),
// 16-byte chunk index XOR ((d >> 2) & 3).
#include <algorithm>
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
// fragment to scratch inside the loop, whose reload then waits on the tile DMA.
constexpr int kPrefetchK = 2, kPrefetchV = 3;

struct AttnParams {
  const int4* qinfo;
  const int32_t* qstart;
  const int2* chunks;
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
  int n, T, S, Hq, Hkv, G, QR, ntiles, exact_per_seq, max_chunks;
  float c_log2;
};

// EXACT = false: the main kernel, every chunk with a long context span. EXACT = true:
// chunks with a short span, and chunks the main kernel flagged for a redo.
template <int D, bool EXACT>
__global__ __launch_bounds__(2 * kAttnSlots / (EXACT ? kExactNT : kMainNT)) void attn_core_kernel(
    const AttnParams p) {
  constexpr int NT = EXACT ? kExactNT : kMainNT;
  using C = Cfg<D, NT>;
  __shared__ __attribute__((aligned(1024))) char Ks0[C::KBUF];
  __shared__ __attribute__((aligned(1024))) char Ks1[C::KBUF];
  __shared__ __attribute__((aligned(1024))) char Vs0[C::VBYTES];
  __shared__ __attribute__((aligned(1024))) char Vs1[C::VBYTES];
  __shared__ __attribute__((aligned(1024))) char Kl0[EXACT ? C::KBUF : 16];
  __shared__ __attribute__((aligned(1024))) char Kl1[EXACT ? C::KBUF : 16];
  __shared__ int s_range[6];
  __shared__ int s_kp[KT], s_kd[KT];
  __shared__ int s_redo;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, half = lane >> 5;
  const int bid = blockIdx.x;
  const int g = bid % p.Hkv;
  int chunk;
  bool redo = false;
  if constexpr (EXACT) {
    const int r = bid / p.Hkv;
    const int n_short = p.S * p.exact_per_seq;
    if (r < n_short) {  // one of the first chunks of a sequence
      const int s = r / p.exact_per_seq, j = r % p.exact_per_seq;
      chunk = p.seq_chunk[s] + j;
      if (chunk >= p.seq_chunk[s + 1]) return;
    } else {            // a chunk the main kernel flagged
      chunk = r - n_short;
      if (chunk >= *p.nchunks || p.flags[chunk * p.Hkv + g] == 0) return;
      redo = true;
    }
  } else {
    // Chunks are listed sequence by sequence, anchors ascending: the last ones have the
    // longest prefixes, so they are dispatched first. The grid is sized for the largest
    // possible chunk count; blocks past the actual count exit.
    chunk = *p.nchunks - 1 - bid / p.Hkv;
    if (chunk < 0) return;
  }
  const int n = p.n, T = p.T, Hkv = p.Hkv;
  const int2 ch = p.chunks[chunk];
  const int j0 = min(max(ch.x, 0), T - 1);
  const int jn = min(max(ch.y, 1), T - j0);

  if (tid == 0) {
    const int4 first = p.qinfo[j0], last = p.qinfo[j0 + jn - 1];
    const int p_first = min(max(first.y, 0), n - 1), p_last = min(max(last.y, 0), n - 1);
    const int lo_first = min(max(first.w, 0), p_first), lo_last = min(max(last.w, 0), p_last);
    s_range[0] = lo_first;  // first key of any row
    s_range[1] = p_last;    // last key of any row
    s_range[2] = lo_last;   // keys in [lo_last, p_first] are seen by every row
    s_range[3] = p_first;
    s_range[4] = min(max(p.qstart[p_first], 0), T);     // diagonal keys: entries of the
    s_range[5] = min(max(p.qstart[p_last + 1], 0), T);  // chunk's anchors in the list
    s_redo = 0;
  }
  __syncthreads();
  const int k_lo = s_range[0], k_hi = s_range[1], full_lo = s_range[2], full_hi = s_range[3];
  const int dg_lo = s_range[4], dg_hi = s_range[5];
  const bool is_short = (k_hi - k_lo + 1) <= kShortSpan;  // uniform over the workgroup
  if (EXACT ? (!is_short && !redo) : is_short) return;

  // Query slots of this lane: NT columns of 32 (lanes l and l+32 share a column, each
  // holding 16 of the 32 keys of a tile).
  int q_row[NT], q_head[NT], q_p[NT], q_d[NT], q_lo[NT];
  bool q_on[NT];
  bf16x8 qf[NT][C::DK];
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
  }

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
      // K fragments are read kPrefetchK steps ahead of the MFMA that uses them, so LDS
      // latency overlaps the MFMA chain instead of stalling each step.
      bf16x8 kf[C::DK];
#pragma unroll
      for (int kk = 0; kk < C::DK; ++kk)
        kf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(kbase + kk * 32));
#pragma unroll
      for (int kk = 0; kk < C::DK; ++kk)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[nt] = mfma32(kf[kk], qf[nt][kk], s[nt]);
      sched_reads_ahead<C::DK, kPrefetchK, NT>();
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
      sched_reads_ahead<2 * C::MT, kPrefetchV, NT>();
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
    const char* base = uniform_opaque(reinterpret_cast<const char*>(src + ((size_t)t * KT * Hkv + g) * D));
#pragma unroll
    for (int j = 0; j < KI; ++j) {
      const int i = wave + j * C::WAVES;
      if (i < C::KBUF / 1024) dma16(base + lane_opaque(koff[j]), dst + i * 1024);
    }
  };
  auto dma_v = [&](int t, char* dst) {
    const char* base = uniform_opaque(reinterpret_cast<const char*>(p.vt + ((size_t)g * p.ntiles + t) * (size_t)(D * KT)));
#pragma unroll
    for (int j = 0; j < VI; ++j) {
      const int i = wave + j * C::WAVES;
      if (i < C::VBYTES / 1024) dma16(base + lane_opaque(voff[j]), dst + i * 1024);
    }
  };
  auto issue = [&](int t, char* Kd, char* Kld, char* Vd) {
    dma_k(p.kr, t, Kd);
    if constexpr (EXACT) dma_k(p.kr_lo, t, Kld);
    dma_v(t, Vd);
  };

  const int t_first = k_lo / KT, t_last = k_hi / KT;
  issue(t_first, Ks0, Kl0, Vs0);
  for (int t = t_first; t <= t_last; t += 2) {
    wait_dma();
    __syncthreads();  // tile t landed in buffer 0; buffer 1 is free
    if (t + 1 <= t_last) issue(t + 1, Ks1, Kl1, Vs1);
    {
      const int key0 = t * KT;
      const bool full = key0 >= full_lo && key0 + KT - 1 <= full_hi;
      compute(Ks0, Kl0, Vs0, full ? 0 : 1, key0, t == t_first);
    }
    if (t + 1 > t_last) break;
    wait_dma();
    __syncthreads();  // tile t+1 landed in buffer 1; buffer 0 is free
    if (t + 2 <= t_last) issue(t + 2, Ks0, Kl0, Vs0);
    {
      const int key0 = (t + 1) * KT;
      const bool full = key0 >= full_lo && key0 + KT - 1 <= full_hi;
      compute(Ks1, Kl1, Vs1, full ? 0 : 1, key0, false);
    }
  }

  // ---- diagonal extension: depth >= 1 rows of the chunk's anchors ----
  for (int jb = dg_lo; jb < dg_hi; jb += KT) {
    __syncthreads();
    if (tid < KT) {
      const int jk = jb + tid;
      int kp = -1, kd = 0;
      if (jk < dg_hi) {
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
      if (jk < dg_hi) {
        const int row = min(max(p.qinfo[jk].x, 0), T - 1);
        kv = *reinterpret_cast<const u32x4*>(p.kr + ((size_t)row * Hkv + g) * D + c * 8);
        vv = *reinterpret_cast<const u32x4*>(p.v + ((size_t)row * Hkv + g) * D + c * 8);
        if constexpr (EXACT) kl = *reinterpret_cast<const u32x4*>(p.kr_lo + ((size_t)row * Hkv + g) * D + c * 8);
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
    compute(Ks0, Kl0, Vs0, 2, 0, false);
  }

  // ---- epilogue: O / l, lse; the main kernel flags rows whose sum left the safe range ----
  bool bad = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = l_run[nt] + __shfl_xor(l_run[nt], 32, 64);
    if constexpr (!EXACT) bad |= q_on[nt] && !(lt <= kSumLimit);
    const float inv = 1.f / lt;
    if (q_on[nt]) {
      float* dst = p.out + ((size_t)q_row[nt] * p.Hq + q_head[nt]) * D;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          floatx4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = o[nt][mt][4 * i + j] * inv;
          *reinterpret_cast<floatx4*>(dst + mt * 32 + 8 * i + 4 * half) = w;
        }
      if (p.lse != nullptr && half == 0)
        p.lse[(size_t)q_head[nt] * T + q_row[nt]] = (m_run[nt] + __log2f(lt)) * 0.69314718055994531f;
    }
  }
  if constexpr (!EXACT) {
    if (__any(bad) && lane == 0) s_redo = 1;
    __syncthreads();
    if (tid == 0 && s_redo) p.flags[chunk * Hkv + g] = 1;
  } else {
    if (redo && tid == 0) p.flags[chunk * Hkv + g] = 0;
  }
}

}  // namespace

hipError_t launch_attn_core(const AttnArgs& a, const uint16_t* v, float* out, float* lse,
                            const char* ws, hipStream_t stream) {
  const AttnLayout L = attn_layout(a.n, a.T, a.Hq, a.Hkv, a.D);
  AttnParams p;
  p.qinfo = reinterpret_cast<const int4*>(ws + L.qinfo);
  p.qstart = reinterpret_cast<const int32_t*>(ws + L.qstart);
  p.chunks = reinterpret_cast<const int2*>(ws + L.chunks);
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
  // main kernel first (it may flag chunks), then short and flagged chunks
  // chunk count <= ceil(T / QR) + S (each sequence adds at most one partial chunk)
  const int chunk_bound = std::min(L.max_chunks, (a.T + p.QR - 1) / p.QR + a.S);
  const dim3 main_grid(chunk_bound * a.Hkv);
  const dim3 exact_grid((a.S * p.exact_per_seq + chunk_bound) * a.Hkv);
#define PEAGLE_CORE(DD)                                                                       \
  do {                                                                                        \
    hipLaunchKernelGGL((attn_core_kernel<DD, false>), main_grid, dim3(Cfg<DD, kMainNT>::TH), \
                       0, stream, p);                                                         \
    hipLaunchKernelGGL((attn_core_kernel<DD, true>), exact_grid, dim3(Cfg<DD, kExactNT>::TH), \
                       0, stream, p);                                                         \
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
