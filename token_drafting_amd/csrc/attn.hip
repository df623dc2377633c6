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
// q heads of one kv head: 256 query slots, roughly 25 anchors and all their depths at
// K=4, G=4. Every row of the chunk reads a
// prefix of the same depth-0 K/V, so each K/V tile is loaded to LDS once and used by
// all 256 slots (all depths, all heads of the group). Tiles wholly inside every row's
// range run unmasked; the few at the chunk's edge are masked per element; tiles past
// the last anchor are never visited. The diagonal keys of the chunk's anchors are a
// short contiguous run of the anchor-major list, processed as extra masked tiles.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16). Scores are computed transposed,
// S^T = K * Q^T, so a lane holds one query column and 16 of the 32 keys of a tile: the
// softmax state is per lane and one cross-half exchange per tile gives the tile max.
// P^T stays in registers as the B operand of O^T = V^T * P^T: the 16 keys a lane holds
// for one 16-key step are exactly the 8+8 it must supply once the keys of each 16-key
// group are taken in the order (0-3, 8-11 | 4-7, 12-15); V^T tiles are stored in that
// order (v_transpose_kernel), so each PV operand is one 16-byte LDS read.
//
// Softmax: base-2 exponent with the 1/sqrt(D)*log2(e) factor folded into one FMA; the
// running max is only raised (and O, l rescaled) when a tile's max exceeds it by more
// than 8, so P <= 2^8 and the rescale of the large O accumulator is rare.
//
// Precision. Rounding q', k' and P to bf16 perturbs each score by ~1e-3 and each weight
// by up to 2^-9; for a row whose output mixes only a handful of keys that moves it by
// up to ~1e-2 (outputs there reach |v| ~ 5). Chunks whose context span is short
// (<= kShortSpan keys, the first anchors of each sequence) therefore run an exact-split
// variant: q' = q_hi + q_lo and k' = k_hi + k_lo in bf16 (three MFMAs per step for
// S^T), P = P_hi + P_lo (two MFMAs for PV), with q', k' rotated in fp32 from the
// pre-RoPE inputs. Rows with many keys average the rounding out and take the plain path.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace peagle {

namespace {

constexpr int KT = 32;             // keys per tile
constexpr float kRescaleLog2 = 8.f;
constexpr int kShortSpan = 96;     // context span (keys) up to which a chunk runs exact-split

template <int D, int NT>
struct Cfg {
  static constexpr int kThreads = 512 / NT;          // 256 query slots per workgroup
  static constexpr int KROW = D * 2;                 // bytes of one K row in LDS
  static constexpr int KBYTES = KT * KROW;
  static constexpr int VBYTES = D * KT * 2;          // V^T tile: D rows x 32 keys
  static constexpr int KCH = KT * (D / 8);           // 16-byte chunks of a K tile
  static constexpr int VCH = D * (KT / 8);           // 16-byte chunks of a V^T tile
  static constexpr int NKC = (KCH + kThreads - 1) / kThreads;  // per thread (last may idle)
  static constexpr int NVC = (VCH + kThreads - 1) / kThreads;
  static constexpr int DK = D / 16;                  // k-steps of S^T
  static constexpr int MT = D / 32;                  // 32-row M tiles of O^T
};

__device__ __forceinline__ int k_off(int key, int chunk, int krow) {
  return key * krow + ((chunk ^ (key & 7)) << 4);
}
__device__ __forceinline__ int v_off(int d, int chunk) {
  return d * (KT * 2) + ((chunk ^ ((d >> 1) & 3)) << 4);
}

__device__ __forceinline__ float bf16_elem(const u32x4& w, int e) {
  return bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
}

// fp32 RoPE of the 8 head-dim elements [d0, d0+8) of one pre-RoPE bf16 head row at
// position pos (rotate-half: element j pairs with j + D/2).
template <int D>
__device__ __forceinline__ void rope8(const uint16_t* __restrict__ row, const float* __restrict__ cosT,
                                      const float* __restrict__ sinT, int pos, int d0, float out[8]) {
  constexpr int H2 = D / 2;
  const bool first = d0 < H2;
  const int j0 = first ? d0 : d0 - H2;
  const u32x4 x = *reinterpret_cast<const u32x4*>(row + d0);
  const u32x4 y = *reinterpret_cast<const u32x4*>(row + (first ? d0 + H2 : d0 - H2));
  const floatx4* cp = reinterpret_cast<const floatx4*>(cosT + (size_t)pos * H2 + j0);
  const floatx4* sp = reinterpret_cast<const floatx4*>(sinT + (size_t)pos * H2 + j0);
  const floatx4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float a = bf16_elem(x, e), b = bf16_elem(y, e);
    const float cs = e < 4 ? c0[e] : c1[e - 4], sn = e < 4 ? s0[e] : s1[e - 4];
    out[e] = first ? a * cs - b * sn : a * cs + b * sn;
  }
}

// EXACT = false runs the chunks with a long context span, EXACT = true the short ones;
// each returns at once for the other kind, so the two launches together cover all.
template <int D, int NT, bool EXACT>
__global__ __launch_bounds__(512 / NT) void attn_core_kernel(
    const int4* __restrict__ qinfo, const int32_t* __restrict__ qstart,
    const int2* __restrict__ chunks, const int32_t* __restrict__ nchunks_dev,
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ vt, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ q_in, const uint16_t* __restrict__ k_in,
    const float* __restrict__ cosT, const float* __restrict__ sinT, float* __restrict__ out,
    float* __restrict__ lse, int n, int T, int Hq, int Hkv, int G, int QR, int ntiles,
    int max_pos, float c_log2) {
  using C = Cfg<D, NT>;
  constexpr int TH = C::kThreads;
  __shared__ __attribute__((aligned(16))) char Ks[C::KBYTES];
  __shared__ __attribute__((aligned(16))) char Kl[EXACT ? C::KBYTES : 16];  // k_lo (exact split)
  __shared__ __attribute__((aligned(16))) char Vs[C::VBYTES];
  __shared__ int s_range[6];
  __shared__ int s_kp[KT], s_kd[KT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, half = lane >> 5;
  const int bid = blockIdx.x;
  // Chunks are listed sequence by sequence, anchors ascending: the last ones have the
  // longest prefixes, so they are dispatched first. The grid is sized for the largest
  // possible chunk count; blocks past the actual count exit.
  const int chunk = *nchunks_dev - 1 - bid / Hkv;
  if (chunk < 0) return;
  const int g = bid % Hkv;
  const int2 ch = chunks[chunk];
  const int j0 = min(max(ch.x, 0), T - 1);
  const int jn = min(max(ch.y, 1), T - j0);

  if (tid == 0) {
    const int4 first = qinfo[j0], last = qinfo[j0 + jn - 1];
    const int p_first = min(max(first.y, 0), n - 1), p_last = min(max(last.y, 0), n - 1);
    const int lo_first = min(max(first.w, 0), p_first), lo_last = min(max(last.w, 0), p_last);
    s_range[0] = lo_first;                // first key of any row
    s_range[1] = p_last;                  // last key of any row
    s_range[2] = lo_last;                 // keys in [lo_last, p_first] are seen by every row
    s_range[3] = p_first;
    s_range[4] = min(max(qstart[p_first], 0), T);      // diagonal keys: entries of the
    s_range[5] = min(max(qstart[p_last + 1], 0), T);   // chunk's anchors in the list
  }

  // Query slots of this lane: NT columns of 32.
  int q_row[NT], q_head[NT], q_p[NT], q_d[NT], q_lo[NT];
  bool q_on[NT];
  bf16x8 qf[NT][C::DK];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int slot = wave * 32 * NT + nt * 32 + r32;
    const int rl = slot % QR, hl = slot / QR;
    q_on[nt] = rl < jn;
    const int4 qi = qinfo[j0 + min(rl, jn - 1)];
    q_row[nt] = min(max(qi.x, 0), T - 1);
    q_p[nt] = min(max(qi.y, 0), n - 1);
    q_d[nt] = qi.z;
    q_lo[nt] = min(max(qi.w, 0), q_p[nt]);
    q_head[nt] = g * G + hl;
    const uint16_t* qrow = qr + ((size_t)q_row[nt] * Hq + q_head[nt]) * D + half * 8;
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
  __syncthreads();
  const int k_lo = s_range[0], k_hi = s_range[1], full_lo = s_range[2], full_hi = s_range[3];
  const int dg_lo = s_range[4], dg_hi = s_range[5];
  const bool precise = (k_hi - k_lo + 1) <= kShortSpan;   // uniform over the workgroup
  if (precise != EXACT) return;

  // One tile of scores -> online softmax -> PV. mode 0: no mask, 1: context range,
  // 2: diagonal keys (meta in s_kp / s_kd). `exact`: hi/lo split products.
  auto compute = [&](int mode, int key0) {
    constexpr bool exact = EXACT;
    floatx16 s[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nt][r] = 0.f;
    if constexpr (!exact) {
#pragma unroll
      for (int kk = 0; kk < C::DK; ++kk) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(Ks + k_off(r32, kk * 2 + half, C::KROW)));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[nt] = mfma32(a, qf[nt][kk], s[nt]);
      }
    } else {
      for (int kk = 0; kk < C::DK; ++kk) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(Ks + k_off(r32, kk * 2 + half, C::KROW)));
        const bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4*>(Kl + k_off(r32, kk * 2 + half, C::KROW)));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float qv[8];
          const int qpos = min(q_p[nt] - q_lo[nt] + q_d[nt], max_pos);
          rope8<D>(q_in + ((size_t)q_row[nt] * Hq + q_head[nt]) * D, cosT, sinT, qpos,
                   kk * 16 + half * 8, qv);
          bf16x8 ql;
#pragma unroll
          for (int e = 0; e < 8; ++e) ql[e] = (__bf16)(qv[e] - (float)qf[nt][kk][e]);
          s[nt] = mfma32(a, qf[nt][kk], s[nt]);
          s[nt] = mfma32(al, qf[nt][kk], s[nt]);
          s[nt] = mfma32(a, ql, s[nt]);
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
    float m_new[NT];
    bool need = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = s[nt][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[nt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      m_new[nt] = fmaxf(m_run[nt], mx * c_log2);
      need |= m_new[nt] > m_run[nt] + kRescaleLog2;
    }
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
    bf16x8 pb[NT][2];
    float pf[NT][16];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mu = (m_run[nt] == -INFINITY) ? 0.f : m_run[nt];
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[nt][r], c_log2, -mu));
        ls += pr;
        pf[nt][r] = pr;
        pb[nt][r >> 3][r & 7] = (__bf16)pr;
      }
      l_run[nt] += ls;
    }
    if constexpr (!exact) {
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(Vs + v_off(mt * 32 + r32, ks * 2 + half)));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[nt][mt] = mfma32(a, pb[nt][ks], o[nt][mt]);
        }
    } else {
      bf16x8 pl[NT][2];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) pl[nt][r >> 3][r & 7] = (__bf16)(pf[nt][r] - (float)pb[nt][r >> 3][r & 7]);
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

  // ---- causal context: depth-0 key tiles ----
  u32x4 rk[C::NKC], rv[C::NVC];
  auto load_ctx = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::NKC; ++i) {
      const int q = tid + i * TH, key = q / (D / 8), c = q % (D / 8), pos = t * KT + key;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (q < C::KCH && pos < n) val = *reinterpret_cast<const u32x4*>(kr + ((size_t)pos * Hkv + g) * D + c * 8);
      rk[i] = val;
    }
    const uint16_t* vsrc = vt + ((size_t)g * ntiles + t) * (size_t)(D * KT);
#pragma unroll
    for (int i = 0; i < C::NVC; ++i) {
      const int q = tid + i * TH;
      if (q < C::VCH) rv[i] = *reinterpret_cast<const u32x4*>(vsrc + q * 8);
    }
  };
  auto store_ctx = [&]() {
#pragma unroll
    for (int i = 0; i < C::NKC; ++i) {
      const int q = tid + i * TH;
      if (q < C::KCH) *reinterpret_cast<u32x4*>(Ks + k_off(q / (D / 8), q % (D / 8), C::KROW)) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < C::NVC; ++i) {
      const int q = tid + i * TH;
      if (q < C::VCH) *reinterpret_cast<u32x4*>(Vs + v_off(q >> 2, q & 3)) = rv[i];
    }
  };
  // Exact-split staging: k' rotated in fp32 from the pre-RoPE k at the key's own
  // position, stored as bf16 hi (Ks) and lo (Kl). `row_pos` gives (row, position) of key
  // slot `key` or row -1 for an empty slot.
  auto stage_k_split = [&](auto row_pos) {
    for (int q = tid; q < C::KCH; q += TH) {
      const int key = q / (D / 8), c = q % (D / 8);
      const int2 rp = row_pos(key);
      u32x4 hi = {0u, 0u, 0u, 0u}, lo = {0u, 0u, 0u, 0u};
      if (rp.x >= 0) {
        float kv[8];
        rope8<D>(k_in + ((size_t)rp.x * Hkv + g) * D, cosT, sinT, rp.y, c * 8, kv);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t h2 = 0, l2 = 0;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float x = kv[2 * w + e];
            const uint16_t hb = f32_to_bf16_bits(x);
            h2 |= (uint32_t)hb << (16 * e);
            l2 |= (uint32_t)f32_to_bf16_bits(x - bf16_bits_to_f32(hb)) << (16 * e);
          }
          hi[w] = h2;
          lo[w] = l2;
        }
      }
      *reinterpret_cast<u32x4*>(Ks + k_off(key, c, C::KROW)) = hi;
      *reinterpret_cast<u32x4*>(Kl + k_off(key, c, C::KROW)) = lo;
    }
  };

  const int t_first = k_lo / KT, t_last = k_hi / KT;
  if constexpr (!EXACT) {
    load_ctx(t_first);
    for (int t = t_first; t <= t_last; ++t) {
      __syncthreads();
      store_ctx();
      __syncthreads();
      if (t < t_last) load_ctx(t + 1);
      const int key0 = t * KT;
      const bool full = key0 >= full_lo && key0 + KT - 1 <= full_hi;
      compute(full ? 0 : 1, key0);
    }
  } else {
    const int p_first = full_hi, lo_first = k_lo;
    for (int t = t_first; t <= t_last; ++t) {
      __syncthreads();
      load_ctx(t);
      store_ctx();  // V^T tile (and plain K, overwritten below)
      __syncthreads();
      stage_k_split([&](int key) {
        const int pos = t * KT + key;
        if (pos < k_lo || pos > k_hi) return make_int2(-1, 0);
        const int start = pos < p_first ? lo_first : min(max(qinfo[min(max(qstart[pos], 0), T - 1)].w, 0), pos);
        return make_int2(pos, min(pos - start, max_pos));
      });
      __syncthreads();
      compute(1, t * KT);
    }
  }

  // ---- diagonal extension: depth >= 1 rows of the chunk's anchors ----
  for (int jb = dg_lo; jb < dg_hi; jb += KT) {
    __syncthreads();
    if (tid < KT) {
      const int jk = jb + tid;
      int kp = -1, kd = 0;
      if (jk < dg_hi) {
        const int4 qi = qinfo[jk];
        kp = qi.y;
        kd = qi.z;
      }
      s_kp[tid] = kp;
      s_kd[tid] = kd;
    }
    for (int q = tid; q < C::KCH; q += TH) {
      const int key = q / (D / 8), c = q % (D / 8), jk = jb + key;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (jk < dg_hi) {
        const int row = min(max(qinfo[jk].x, 0), T - 1);
        kv = *reinterpret_cast<const u32x4*>(kr + ((size_t)row * Hkv + g) * D + c * 8);
        vv = *reinterpret_cast<const u32x4*>(v + ((size_t)row * Hkv + g) * D + c * 8);
      }
      *reinterpret_cast<u32x4*>(Ks + k_off(key, c, C::KROW)) = kv;
      // scatter the 8 d-values of this key into the V^T tile (key order as in v_transpose)
      const int vchunk = 2 * (key >> 4) + ((key & 7) >> 2);
      const int elem = 4 * ((key & 15) >> 3) + (key & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = c * 8 + e;
        const uint16_t val = (uint16_t)((vv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        *reinterpret_cast<uint16_t*>(Vs + v_off(d, vchunk) + elem * 2) = val;
      }
    }
    if constexpr (EXACT) {
      __syncthreads();
      stage_k_split([&](int key) {
        const int jk = jb + key;
        if (jk >= dg_hi) return make_int2(-1, 0);
        const int4 qi = qinfo[jk];
        const int p = min(max(qi.y, 0), n - 1);
        const int pos = min(max(p - min(max(qi.w, 0), p) + qi.z, 0), max_pos);
        return make_int2(min(max(qi.x, 0), T - 1), pos);
      });
    }
    __syncthreads();
    compute(2, 0);
  }

  // ---- epilogue: O / l, lse ----
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = l_run[nt] + __shfl_xor(l_run[nt], 32, 64);
    const float inv = 1.f / lt;
    if (q_on[nt]) {
      float* dst = out + ((size_t)q_row[nt] * Hq + q_head[nt]) * D;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          floatx4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = o[nt][mt][4 * i + j] * inv;
          *reinterpret_cast<floatx4*>(dst + mt * 32 + 8 * i + 4 * half) = w;
        }
      if (lse != nullptr && half == 0)
        lse[(size_t)q_head[nt] * T + q_row[nt]] = (m_run[nt] + __log2f(lt)) * 0.69314718055994531f;
    }
  }
}

}  // namespace

hipError_t launch_attn_core(const AttnArgs& a, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const float* rope_cos, const float* rope_sin,
                            float* out, float* lse, const char* ws, hipStream_t stream) {
  const AttnLayout L = attn_layout(a.n, a.T, a.Hq, a.Hkv, a.D);
  const int4* qinfo = reinterpret_cast<const int4*>(ws + L.qinfo);
  const int32_t* qstart = reinterpret_cast<const int32_t*>(ws + L.qstart);
  const uint16_t* qr = reinterpret_cast<const uint16_t*>(ws + L.qrot);
  const uint16_t* kr = reinterpret_cast<const uint16_t*>(ws + L.krot);
  const uint16_t* vt = reinterpret_cast<const uint16_t*>(ws + L.vt);
  const int2* chunks = reinterpret_cast<const int2*>(ws + L.chunks);
  const int32_t* nchunks = reinterpret_cast<const int32_t*>(ws + L.nchunks);
  const int G = a.Hq / a.Hkv;
  const int QR = 256 / G;
  const int ntiles = (a.n + 31) / 32;
  const float c_log2 = a.scale * 1.4426950408889634f;
  const dim3 grid(L.max_chunks * a.Hkv);
#define PEAGLE_CORE(DD, NN)                                                                    \
  do {                                                                                         \
    hipLaunchKernelGGL((attn_core_kernel<DD, NN, true>), grid, dim3(Cfg<DD, NN>::kThreads), 0, \
                       stream, qinfo, qstart, chunks, nchunks, qr, kr, vt, v, q, k, rope_cos,      \
                       rope_sin, out, lse, a.n, a.T, a.Hq, a.Hkv, G, QR, ntiles, a.max_pos, c_log2);      \
    hipLaunchKernelGGL((attn_core_kernel<DD, NN, false>), grid, dim3(Cfg<DD, NN>::kThreads), 0, \
                       stream, qinfo, qstart, chunks, nchunks, qr, kr, vt, v, q, k, rope_cos,      \
                       rope_sin, out, lse, a.n, a.T, a.Hq, a.Hkv, G, QR, ntiles, a.max_pos, c_log2);      \
  } while (0)
  switch (a.D) {
    case 64: PEAGLE_CORE(64, 1); break;
    case 128: PEAGLE_CORE(128, 1); break;
    case 256: PEAGLE_CORE(256, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef PEAGLE_CORE
  return hipGetLastError();
}

}  // namespace peagle
