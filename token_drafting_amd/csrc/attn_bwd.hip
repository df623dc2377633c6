// Multi-depth draft attention backward (flash-style, GQA), gfx950.
//
// NeMo Automodel PR 2376 (description): the P-EAGLE trainer runs the masked-depth loss
// through the EAGLE-3 cache_hidden attention, so the drafter's attention is trained through
// the same predicate as its forward: row (d, p) sees the depth-0 keys p' <= p of its own
// packed sequence and its own anchor's depth-e rows, 1 <= e <= d. With P the softmax of
// S = q' k'^T * scale (q', k' rotated by RoPE at the rows' positions), lse from the forward
// and Delta = rowsum(dO * O):
//   dP = dO V^T,  dS = P * (dP - Delta),  dq' = scale dS k',  dk' = scale dS^T q',
//   dV = P^T dO,
// summed over the q heads of a kv head; dq and dk are dq', dk' rotated back (RoPE is an
// orthogonal map, so its transpose is the rotation by the opposite angle).
//
// Work decomposition:
//   dq   query-major, like the forward: a workgroup takes half of one chunk's 256 query
//        slots (8 waves of 16) and streams the chunk's depth-0 key tiles through LDS, then
//        the chunk's diagonal keys. Per 32-key tile, on 16x16x32 MFMAs: S^T = K Q^T and
//        dP^T = V dO^T (the lane holds one query column and 8 keys), P and dS in
//        registers, then dq'^T += K'^T dS^T with K'^T read from the row-major key tile by
//        LDS transpose reads.
//   dk, dv of depth-0 keys: key-major. A workgroup owns 128 consecutive keys (8 waves of
//        16) of one kv head and streams every query tile that can see them: the query
//        slots (anchor-major rows x G heads) of the anchors from the block's first key to
//        the end of its last key's sequence, pre-cut into 32-slot row tiles. Per tile, on
//        16x16x32 MFMAs: S = Q K^T and dP = dO V^T (the lane holds one key column and 8
//        slots), then dV^T += dO^T P and dK^T += Q^T dS with the lane's own P and dS as
//        the B operands and dO^T, Q^T read from the row tiles by LDS transpose reads.
//   dk, dv of depth >= 1 keys: a depth-e row is seen only by its own anchor's rows of
//        depth >= e (at most K - e rows x G heads): one wave per key row and kv head on
//        the vector units.
// Tiles move global -> LDS by LDS DMA in its buffer form (buffer_load_dwordx4 ... lds)
// into two buffers (tile t+1 streams while tile t is computed). Operands are bf16 (q', k',
// v, dO, P, dS) with fp32 accumulation; P is exact up to rounding because lse is the
// forward's. Every path uses the same bf16-rounded dO, Delta included.
#include <algorithm>

#include "bwd.h"
#include "common.h"
#include "kernels.h"

namespace peagle {

namespace {

constexpr int KT = 32;  // keys (or query slots) per tile
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BCfg {
  // Rows padded by 32 bytes: a row starts 8 of the 64 LDS banks after the previous one, so
  // the transpose reads (four consecutive rows, 32 bytes each, per 16 lanes) and the
  // 16-byte row reads (16 rows per 16 lanes) are both free of bank conflicts; with 16 bytes
  // the transpose reads of neighbouring rows overlapped by 4 banks.
  static constexpr int KROW = D * 2 + 32;
  static constexpr int KBUF = (KT * KROW + 1023) / 1024 * 1024;  // whole DMA blocks
};

// 16x16x32 bf16 MFMA: lane l supplies row l%16 of A and column l%16 of B, 8 values each at
// k positions 8 (l/16) .. + 7; it receives column l%16 of D, rows 4 (l/16) + r.
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr int kBwdWaves = 8;               // waves of the key-major pass, 16 keys each
constexpr int kBwdThreads = 64 * kBwdWaves;

__device__ __forceinline__ bf16x8 ld8(const void* p) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
}

// ds_read_b64_tr_b16 (LDS transpose read). Within each 16-lane group, lane i receives
// element i % 4 of the 8 bytes addressed by lanes i / 4, 4 + i / 4, 8 + i / 4 and
// 12 + i / 4 (measured with an index-coded matrix). So if lane j of a group addresses row
// r0 + j / 4, columns c0 + 4 (j % 4) .. + 3 of a row-major 16-bit matrix, lane i gets
// column c0 + i of rows r0 .. r0 + 3.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v4i16 ld_tr16(const char* lds) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)lds);
}

struct BwdParams {
  const int4* qinfo;        // anchor-major list: (row, anchor, depth, sequence start)
  const int32_t* qstart;    // first list entry of each anchor [n + 1]
  const int32_t* cu;        // cu_seqlens [S + 1]
  const int2* chunks;
  const int32_t* nchunks;
  const uint16_t* qr;       // q' [T, Hq, D]
  const uint16_t* kr;       // k' [T + 32, Hkv, D]
  const uint16_t* v;        // v  [T, Hkv, D]
  const uint16_t* vpad;     // depth-0 v [n + 32, Hkv, D], zero past n
  const uint16_t* dob;      // bf16 dO [T, Hq, D]
  const float* lse;         // [Hq, T], natural log
  const float* dlt;         // Delta [Hq, T]
  const uint16_t* qtr;      // query tiles, rows [Hkv][ntq][32][D]
  const uint16_t* dtr;
  const int4* smeta;        // per slot: (anchor, sequence start, lse * log2 e, Delta)
  float* dq;
  float* dk;
  float* dv;
  float* part;              // per-segment dK'^T, dV^T partials [nseg][2][n][Hkv][D]
  int n, T, S, Hq, Hkv, G, QR;
  int nkb, seg_len;  // key blocks; query tiles per segment of a key block's range
  int64_t ntq;
  float scale, c_log2;
};

// dO rounded to bf16 and Delta[h, row] = sum_d bf16(dO) * O in fp32. Delta takes the same
// rounded dO as dP = dO V^T, so that each row of dS = P (dP - Delta) still sums to zero (a
// Delta from the unrounded dO leaves a bias in every dS row that dominates dq on rows with
// thousands of keys). A group of D/8 threads per (row, head), 8 elements each.
template <int D>
__global__ __launch_bounds__(256) void bwd_dout_kernel(const float* __restrict__ dout,
                                                       const float* __restrict__ out,
                                                       uint16_t* __restrict__ dob,
                                                       float* __restrict__ dlt, int T, int Hq) {
  constexpr int CPR = D / 8;
  const size_t item = blockIdx.x * (size_t)256 + threadIdx.x;
  const size_t total = (size_t)T * Hq * CPR;
  const bool on = item < total;
  const size_t pair = item / CPR;
  const int c = (int)(item % CPR);
  float acc = 0.f;
  if (on) {
    const float* a = dout + pair * D + c * 8;
    const float* b = out + pair * D + c * 8;
    const floatx4 a0 = *reinterpret_cast<const floatx4*>(a);
    const floatx4 a1 = *reinterpret_cast<const floatx4*>(a + 4);
    const floatx4 b0 = *reinterpret_cast<const floatx4*>(b);
    const floatx4 b1 = *reinterpret_cast<const floatx4*>(b + 4);
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = (__bf16)a0[i];
      o[i + 4] = (__bf16)a1[i];
      acc = fmaf((float)o[i], b0[i], acc);
      acc = fmaf((float)o[i + 4], b1[i], acc);
    }
    *reinterpret_cast<bf16x8*>(dob + pair * D + c * 8) = o;
  }
#pragma unroll
  for (int o = CPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (on && c == 0) {
    const size_t row = pair / Hq, h = pair % Hq;
    dlt[h * T + row] = acc;
  }
}

// vpad rows [0, n + 32): v's depth-0 rows, then 32 rows of zeros (the last key tile).
__global__ __launch_bounds__(256) void vpad_kernel(const uint16_t* __restrict__ v,
                                                   uint16_t* __restrict__ vpad, int n, int Hkv,
                                                   int D) {
  const size_t per_row = (size_t)Hkv * D / 8, total = (size_t)(n + KT) * per_row;
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < total;
       t += (size_t)gridDim.x * blockDim.x) {
    const size_t row = t / per_row;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (row < (size_t)n) val = *reinterpret_cast<const u32x4*>(v + t * 8);
    *reinterpret_cast<u32x4*>(vpad + t * 8) = val;
  }
}

// Query tile t of kv head g: slots 32t .. 32t+31 of the list (entry s / G, head
// g G + s % G). Writes q' and dO of each slot in row layout, and the slot's metadata. Slots
// past the list get zero data and anchor -1 (never visible).
template <int D>
__global__ __launch_bounds__(256) void qtile_kernel(const BwdParams p, uint16_t* __restrict__ qtr,
                                                    uint16_t* __restrict__ dtr,
                                                    int4* __restrict__ smeta) {
  const int64_t t = blockIdx.x;
  const int g = blockIdx.y, tid = threadIdx.x;
  constexpr int CPR = D / 8;
  const size_t tb = (size_t)g * p.ntq + t;
  for (int q = tid; q < KT * CPR; q += 256) {
    const int x = q / CPR, c = q % CPR;
    const int64_t s = t * KT + x, e = s / p.G;
    const int h = g * p.G + (int)(s % p.G);
    u32x4 vq = {0u, 0u, 0u, 0u}, vd = {0u, 0u, 0u, 0u};
    if (e < p.T) {
      const int row = min(max(p.qinfo[e].x, 0), p.T - 1);
      const size_t off = ((size_t)row * p.Hq + h) * D + c * 8;
      vq = *reinterpret_cast<const u32x4*>(p.qr + off);
      vd = *reinterpret_cast<const u32x4*>(p.dob + off);
    }
    *reinterpret_cast<u32x4*>(qtr + (tb * KT + x) * D + c * 8) = vq;
    *reinterpret_cast<u32x4*>(dtr + (tb * KT + x) * D + c * 8) = vd;
  }
  if (tid < KT) {
    const int64_t s = t * KT + tid, e = s / p.G;
    int4 m = make_int4(-1, -1, 0, 0);
    if (e < p.T) {
      const int4 qi = p.qinfo[e];
      const int row = min(max(qi.x, 0), p.T - 1);
      const size_t li = (size_t)(g * p.G + (int)(s % p.G)) * p.T + row;
      m = make_int4(qi.y, qi.w, __float_as_int(p.lse[li] * kLog2e), __float_as_int(p.dlt[li]));
    }
    smeta[tb * KT + tid] = m;
  }
}

// Query tiles [a, b) of one kv head's tile list that can see depth-0 keys [k0, k1]: the
// slots of the anchors from k0 to the end of k1's sequence (all their depths and heads).
__device__ __forceinline__ void key_block_tiles(const BwdParams& p, int k0, int k1, int64_t& a,
                                                int64_t& b) {
  const int s1 = min(max(upper_index(p.cu, p.S + 1, k1), 0), p.S - 1);
  const int end = min(max(p.cu[s1 + 1], k1 + 1), p.n);
  const int64_t e0 = min(max(p.qstart[k0], 0), p.T);
  const int64_t e1 = min(max((int64_t)p.qstart[end], e0), (int64_t)p.T);
  a = e0 * p.G / KT;
  b = (e1 * p.G + KT - 1) / KT;
}

// dk' and dv of the depth-0 keys [k0, k0 + 128) of kv head g, from the
// query tiles that see them inside one absolute segment of seg_len tiles of the list.
// Workgroups are ordered segment-major, so those running at the same time stream the same
// few segments and the tiles come from HBM about once per segment (later blocks hit the
// caches), instead of once per key block; and no workgroup takes more than seg_len tiles
// (the first key blocks are seen by nearly every tile, the last by few). Each segment
// stores its partial sums in its own slab of the workspace; dkdv_sum_kernel adds a key
// block's segments in a fixed order, so the result does not depend on timing.
//
// v_mfma_f32_16x16x32_bf16 with 16 keys per wave and 8 waves: a lane holds the k' and v
// fragments of one key for half of a 32-key wave's registers, so the pass keeps two waves
// per SIMD. Per 32-slot tile: S = Q K^T and dP = dO V^T as two 16-slot blocks (the lane
// holds key l%16, slots 16 mi + 4 (l/16) + r), then dV^T += dO^T P and dK^T += Q^T dS with
// the lane's 8 weights as the B operand: positions 8 (l/16) .. + 7 of a k-step are slots
// 4 (l/16) .. + 3 and 16 + 4 (l/16) .. + 3. The A operands (dO^T, Q^T) are read from the
// row-major tiles by LDS transpose reads, so a stage holds only the row tiles (35 KB at
// D = 256 instead of 67 KB with transposed copies; 7% faster).
template <int D>
__global__ __launch_bounds__(kBwdThreads) void dkdv_kernel(const BwdParams p) {
  using C = BCfg<D>;
  constexpr int DS = D / 32;  // k-steps of S and dP over D
  constexpr int MB = D / 16;  // 16-row blocks of dK^T and dV^T
  constexpr int kPfS = 4;     // S / dP row reads in flight ahead of their MFMAs
  constexpr int kPfT = 3;     // dV^T / dK^T MFMAs whose transpose reads are in flight
  // LDS regions of one stage, only those the pass reads
  // q' rows, dO rows (both row-major, padded rows), slot metadata; the transposed operands
  // of dV^T and dK^T are read from the row tiles by LDS transpose reads
  constexpr int RQ = 0;
  constexpr int RD = RQ + C::KBUF;
  constexpr int RM = RD + C::KBUF;
  constexpr int STAGE = RM + 1024;
  constexpr int NR = C::KBUF / 1024;
  __shared__ __attribute__((aligned(1024))) char buf0[STAGE];
  __shared__ __attribute__((aligned(1024))) char buf1[STAGE];
  __shared__ int s_rng[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int g = blockIdx.x % p.Hkv, rest = blockIdx.x / p.Hkv;
  const int kb = rest % p.nkb, seg = rest / p.nkb;
  const int k0 = kb * kBwdKeys;
  if (k0 >= p.n) return;
  const int k1 = min(k0 + kBwdKeys, p.n) - 1;
  if (tid == 0) {
    // this block's tiles [a, b) within absolute segment seg of the tile list
    int64_t a, b;
    key_block_tiles(p, k0, k1, a, b);
    const int64_t ts = (int64_t)seg * p.seg_len;
    s_rng[0] = (int)std::max(a, ts);
    s_rng[1] = (int)std::min(b, ts + p.seg_len);
  }
  __syncthreads();
  const int t0 = s_rng[0], t1 = s_rng[1];
  if (t0 >= t1) return;  // an empty segment (the same for the whole workgroup)

  const int key = k0 + wave * 16 + l16;
  const bool key_on = key <= k1;
  const int kc = min(key, k1);
  const int key_lo = p.qinfo[min(max(p.qstart[kc], 0), p.T - 1)].w;
  bf16x8 kf[DS], vf[DS];
  {
    const uint16_t* krow = p.kr + ((size_t)kc * p.Hkv + g) * D + q4 * 8;
    const uint16_t* vrow = p.v + ((size_t)kc * p.Hkv + g) * D + q4 * 8;
#pragma unroll
    for (int kk = 0; kk < DS; ++kk) {
      kf[kk] = ld8(krow + kk * 32);
      vf[kk] = ld8(vrow + kk * 32);
    }
  }
  floatx4 dkt[MB], dvt[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) dkt[mb] = dvt[mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int t, char* dst) {
    const size_t tb = (size_t)g * p.ntq + t;
    const auto rq = dma_range(uniform_opaque(reinterpret_cast<const char*>(p.qtr + tb * KT * D)), KT * D * 2);
    const auto rd = dma_range(uniform_opaque(reinterpret_cast<const char*>(p.dtr + tb * KT * D)), KT * D * 2);
#pragma unroll
    for (int j = 0; j < (NR + kBwdWaves - 1) / kBwdWaves; ++j) {
      const int b = wave + kBwdWaves * j;
      if (b < NR) {
        const int P = b * 1024 + lane * 16;
        const int x = P / C::KROW, off = P - x * C::KROW;
        const uint32_t o = (x < KT && off < D * 2) ? (uint32_t)(x * D * 2 + off) : 0u;
        dma16_buf(rq, o, dst + RQ + b * 1024);
        dma16_buf(rd, o, dst + RD + b * 1024);
      }
    }
    if (wave == 0)
      dma16_buf(dma_range(uniform_opaque(reinterpret_cast<const char*>(p.smeta + tb * KT)), KT * 16),
                (uint32_t)(lane & 31) * 16, dst + RM);
  };

  auto compute = [&](const char* B) {
    // S = Q K^T and dP = dO V^T for the two 16-slot halves: four independent chains, one
    // 16-byte row read per MFMA, interleaved so that no MFMA waits on its predecessor
    floatx4 s[2], dp[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) s[mi] = dp[mi] = floatx4{0.f, 0.f, 0.f, 0.f};
    const char* qb = B + RQ + l16 * C::KROW + q4 * 16;
    const char* db = B + RD + l16 * C::KROW + q4 * 16;
#pragma unroll
    for (int kk = 0; kk < DS; ++kk) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        s[mi] = mfma16(ld8(qb + 16 * mi * C::KROW + kk * 64), kf[kk], s[mi]);
        dp[mi] = mfma16(ld8(db + 16 * mi * C::KROW + kk * 64), vf[kk], dp[mi]);
      }
    }
    // One 16-byte metadata read per weight and a branch-free mask: a short-circuit test
    // compiles to nested branches, each reading one field and waiting for it.
    const int4* meta = reinterpret_cast<const int4*>(B + RM);
    int4 m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = meta[16 * (e >> 2) + 4 * q4 + (e & 3)];
    bf16x8 pb, sb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int mi = e >> 2, r = e & 3;
      const bool ok = key_on & (m[e].y == key_lo) & (m[e].x >= key);
      const float ex = __builtin_amdgcn_exp2f(fmaf(s[mi][r], p.c_log2, -__int_as_float(m[e].z)));
      const float pr = ok ? ex : 0.f;
      pb[e] = (__bf16)pr;
      sb[e] = (__bf16)(pr * (dp[mi][r] - __int_as_float(m[e].w)));
    }
    // A operands of dV^T += dO^T P and dK^T += Q^T dS: dims 16 mb + l16 of slots
    // 4 q4 .. 4 q4 + 3 and 16 + 4 q4 .. (the order of the lane's weights), two transpose
    // reads from the row tile each
    auto tr_frag = [&](const char* rows, int mb) {
      const char* a = rows + (4 * q4 + (l16 >> 2)) * C::KROW + (16 * mb + 4 * (l16 & 3)) * 2;
      const v4i16 lo = ld_tr16(a), hi = ld_tr16(a + 16 * C::KROW);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      dvt[mb] = mfma16(tr_frag(B + RD, mb), pb, dvt[mb]);
      dkt[mb] = mfma16(tr_frag(B + RQ, mb), sb, dkt[mb]);
    }
    // LDS reads ahead of the MFMAs that take them: the S and dP row reads kPfS MFMAs
    // ahead, the metadata behind the last of them, the transpose reads (two per MFMA)
    // kPfT MFMAs ahead
    sched_reads_ahead<4 * DS, kPfS, 1>();
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
    sched_reads_ahead<2 * MB, kPfT, 1, 2>();
  };

  // two tiles per iteration over two static buffers, one loop exit, odd last tile after
  // the loop (as in dq_kernel)
  issue(t0, buf0);
  int t = t0;
  for (; t + 1 < t1; t += 2) {
    wait_dma();
    __syncthreads();  // tile t landed in buffer 0; buffer 1 is free
    issue(t + 1, buf1);
    compute(buf0);
    wait_dma();
    __syncthreads();  // tile t+1 landed in buffer 1; buffer 0 is free
    if (t + 2 < t1) issue(t + 2, buf0);
    compute(buf1);
  }
  if (t < t1) {
    wait_dma();
    __syncthreads();
    compute(buf0);
  }

  if (key_on) {
    const size_t plane = (size_t)p.n * p.Hkv * D;  // one of dK', dV of one segment
    float* dkr = p.part + 2 * (size_t)seg * plane + ((size_t)key * p.Hkv + g) * D;
    float* dvr = dkr + plane;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int d = 16 * mb + 4 * q4;
      *reinterpret_cast<floatx4*>(dkr + d) = dkt[mb];
      *reinterpret_cast<floatx4*>(dvr + d) = dvt[mb];
    }
  }
}

// dk' and dv of the depth-0 keys: the sum of the partials of the segments that hold tiles
// seeing the key's block, in segment order; dk' takes the softmax scale. One thread per
// (key, kv head, 4 of D).
template <int D>
__global__ __launch_bounds__(256) void dkdv_sum_kernel(const BwdParams p) {
  const size_t total = (size_t)p.n * p.Hkv * (D / 4);
  const size_t plane = (size_t)p.n * p.Hkv * D;
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < total;
       t += (size_t)gridDim.x * blockDim.x) {
    const int key = (int)(t / ((size_t)p.Hkv * (D / 4)));
    const int k0 = key / kBwdKeys * kBwdKeys;
    const int k1 = min(k0 + kBwdKeys, p.n) - 1;
    int64_t a, b;
    key_block_tiles(p, k0, k1, a, b);
    floatx4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
    if (a < b) {
      const int s0 = (int)(a / p.seg_len), s1 = (int)((b - 1) / p.seg_len);
      for (int sg = s0; sg <= s1; ++sg) {
        const float* base = p.part + 2 * (size_t)sg * plane + 4 * t;
        const floatx4 k = *reinterpret_cast<const floatx4*>(base);
        const floatx4 v = *reinterpret_cast<const floatx4*>(base + plane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sk[e] += k[e];
          sv[e] += v[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sk[e] *= p.scale;
    *reinterpret_cast<floatx4*>(p.dk + 4 * t) = sk;
    *reinterpret_cast<floatx4*>(p.dv + 4 * t) = sv;
  }
}

// dk' and dv of the depth >= 1 rows: wave per (row j, kv head g); lane holds d = lane + 64 i.
template <int D>
__global__ __launch_bounds__(256) void diag_kernel(const BwdParams p, const int32_t* __restrict__ idx,
                                                   const int32_t* __restrict__ depth_off, int K) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = blockIdx.x * (int64_t)4 + (threadIdx.x >> 6);
  if (w >= (int64_t)(p.T - p.n) * p.Hkv) return;
  const int j = p.n + (int)(w / p.Hkv), g = (int)(w % p.Hkv);
  const int e = min(max(upper_index(depth_off, K + 1, j), 1), K - 1);  // depth of row j
  const int anchor = min(max(idx[j], 0), p.n - 1);
  const int q0 = min(max(p.qstart[anchor], 0), p.T);
  const int q1 = min(max(p.qstart[anchor + 1], q0), p.T);
  float kv[E], vv[E], dk[E], dv[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const size_t o = ((size_t)j * p.Hkv + g) * D + lane + 64 * i;
    kv[i] = bf16_bits_to_f32(p.kr[o]);
    vv[i] = bf16_bits_to_f32(p.v[o]);
    dk[i] = dv[i] = 0.f;
  }
  for (int ent = q0 + e; ent < q1; ++ent) {  // the anchor's rows of depth >= e
    const int row = min(max(p.qinfo[ent].x, 0), p.T - 1);
    for (int hl = 0; hl < p.G; ++hl) {
      const int h = g * p.G + hl;
      float qv[E], dov[E], sd = 0.f, pd = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const size_t o = ((size_t)row * p.Hq + h) * D + lane + 64 * i;
        qv[i] = bf16_bits_to_f32(p.qr[o]);
        dov[i] = bf16_bits_to_f32(p.dob[o]);  // the rounded dO that Delta was formed with
        sd = fmaf(qv[i], kv[i], sd);
        pd = fmaf(dov[i], vv[i], pd);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        sd += __shfl_xor(sd, o, 64);
        pd += __shfl_xor(pd, o, 64);
      }
      const size_t li = (size_t)h * p.T + row;
      const float pr = __expf(sd * p.scale - p.lse[li]);
      const float ds = pr * (pd - p.dlt[li]) * p.scale;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        dv[i] = fmaf(pr, dov[i], dv[i]);
        dk[i] = fmaf(ds, qv[i], dk[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const size_t o = ((size_t)j * p.Hkv + g) * D + lane + 64 * i;
    p.dk[o] = dk[i];
    p.dv[o] = dv[i];
  }
}

// dq' of half of a chunk's query slots, eight waves of 16 slots on 16x16x32 MFMAs. A
// wave holds its slots' q' and dO fragments (the B operands of S^T = K Q^T and
// dP^T = V dO^T, rows of K and V the A operands from LDS) and dq'^T (16 dims x 16 slots per
// tile of the accumulator): 128 registers at D = 256 where 32 slots a wave take 256, so two
// waves share a SIMD. The A operand of dq'^T += K'^T dS^T comes from the row-major K tile by
// LDS transpose reads, in the key order of the lane's dS weights (4 q4 .. 4 q4 + 3, then
// 16 + 4 q4 ..), so no transposed copy of K is needed.
template <int D>
__global__ __launch_bounds__(512, D <= 128 ? 2 : 1) void dq_kernel(const BwdParams p) {
  using C = BCfg<D>;
  constexpr int DS = D / 32;  // k-steps of S^T and dP^T
  constexpr int MB = D / 16;  // 16-dim tiles of dq'^T
  constexpr int NR = C::KBUF / 1024;
  constexpr int kW = 8;
  __shared__ __attribute__((aligned(1024))) char Ks0[C::KBUF];
  __shared__ __attribute__((aligned(1024))) char Ks1[C::KBUF];
  __shared__ __attribute__((aligned(1024))) char Vs0[C::KBUF];
  __shared__ __attribute__((aligned(1024))) char Vs1[C::KBUF];
  __shared__ int s_range[6];
  __shared__ int s_kp[KT], s_kd[KT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int hs = blockIdx.x & 1, rest = blockIdx.x >> 1;
  const int g = rest % p.Hkv;
  const int chunk = *p.nchunks - 1 - rest / p.Hkv;  // longest prefixes first
  if (chunk < 0) return;
  const int n = p.n, T = p.T, Hkv = p.Hkv;
  const int2 ch = p.chunks[chunk];
  const int j0 = min(max(ch.x, 0), T - 1);
  const int jn = min(max(ch.y, 1), T - j0);
  if (tid == 0) {
    const int4 first = p.qinfo[j0], last = p.qinfo[j0 + jn - 1];
    const int p_first = min(max(first.y, 0), n - 1), p_last = min(max(last.y, 0), n - 1);
    const int lo_first = min(max(first.w, 0), p_first), lo_last = min(max(last.w, 0), p_last);
    s_range[0] = lo_first;
    s_range[1] = p_last;
    s_range[2] = lo_last;
    s_range[3] = p_first;
    s_range[4] = min(max(p.qstart[p_first], 0), T);
    s_range[5] = min(max(p.qstart[p_last + 1], 0), T);
  }
  __syncthreads();
  const int k_lo = s_range[0], k_hi = s_range[1], full_lo = s_range[2], full_hi = s_range[3];
  const int dg_lo = s_range[4], dg_hi = s_range[5];

  const int slot = hs * 128 + wave * 16 + l16;
  const int rl = slot % p.QR, hl = slot / p.QR;
  const bool q_on = rl < jn;
  const int4 qi = p.qinfo[j0 + min(rl, jn - 1)];
  const int q_row = min(max(qi.x, 0), T - 1);
  const int q_p = min(max(qi.y, 0), n - 1);
  const int q_d = qi.z;
  const int q_lo = min(max(qi.w, 0), q_p);
  const int q_head = g * p.G + hl;
  bf16x8 qf[DS], df[DS];
  {
    const size_t o = ((size_t)q_row * p.Hq + q_head) * D + 8 * q4;
#pragma unroll
    for (int kk = 0; kk < DS; ++kk) {
      qf[kk] = ld8(p.qr + o + 32 * kk);
      df[kk] = ld8(p.dob + o + 32 * kk);
    }
  }
  const size_t li = (size_t)q_head * T + q_row;
  const float lse2 = p.lse[li] * kLog2e, delta = p.dlt[li];
  floatx4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // mode 0: no mask, 1: context range, 2: diagonal keys (meta in s_kp / s_kd)
  auto compute = [&](const char* Ks, const char* Vs, int mode, int key0) {
    floatx4 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
      dp[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
      const char* kr = Ks + (16 * kb + l16) * C::KROW + q4 * 16;
      const char* vr = Vs + (16 * kb + l16) * C::KROW + q4 * 16;
#pragma unroll
      for (int kk = 0; kk < DS; ++kk) {
        s[kb] = mfma16(ld8(kr + kk * 64), qf[kk], s[kb]);
        dp[kb] = mfma16(ld8(vr + kk * 64), df[kk], dp[kb]);
      }
    }
    bf16x8 sb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kb = e >> 2, r = e & 3;
      const int kl = 16 * kb + 4 * q4 + r;
      // branch-free: the weight is computed for every key and masked by a select
      bool ok = true;
      if (mode == 1) {
        const int key = key0 + kl;
        ok = (key >= q_lo) & (key <= q_p);
      } else if (mode == 2) {
        const int kp = s_kp[kl], kd = s_kd[kl];
        ok = (kp == q_p) & (kd >= 1) & (kd <= q_d);
      }
      const float ex = __builtin_amdgcn_exp2f(fmaf(s[kb][r], p.c_log2, -lse2));
      const float pr = ok ? ex : 0.f;
      sb[e] = (__bf16)(pr * (dp[kb][r] - delta));
    }
    // A operand: dims 16 mb + l16 of keys 4 q4 .. 4 q4 + 3 and 16 + 4 q4 .. (two transpose
    // reads from the row-major K tile)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const char* a = Ks + (4 * q4 + (l16 >> 2)) * C::KROW + (16 * mb + 4 * (l16 & 3)) * 2;
      const v4i16 lo = ld_tr16(a), hi = ld_tr16(a + 16 * C::KROW);
      acc[mb] = mfma16(__builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)),
                       sb, acc[mb]);
    }
  };

  // ---- causal context: depth-0 key tiles ----
  auto issue = [&](int t, char* Kd, char* Vd) {
    // a tile's rows of kv head g: KT rows Hkv * D apart
    const uint32_t span = (uint32_t)(((KT - 1) * Hkv + 1) * D * 2);
    const auto rk = dma_range(uniform_opaque(reinterpret_cast<const char*>(p.kr + ((size_t)t * KT * Hkv + g) * D)), span);
    const auto rv = dma_range(uniform_opaque(reinterpret_cast<const char*>(p.vpad + ((size_t)t * KT * Hkv + g) * D)), span);
#pragma unroll
    for (int j = 0; j < (NR + kW - 1) / kW; ++j) {
      const int b = wave + kW * j;
      if (b < NR) {
        const int P = b * 1024 + lane * 16;
        const int x = P / C::KROW, off = P - x * C::KROW;
        const uint32_t o = (x < KT && off < D * 2) ? (uint32_t)(x * Hkv * D * 2 + off) : 0u;
        dma16_buf(rk, o, Kd + b * 1024);
        dma16_buf(rv, o, Vd + b * 1024);
      }
    }
  };
  const int t_first = k_lo / KT, t_last = k_hi / KT;
  auto full_tile = [&](int key0) { return key0 >= full_lo && key0 + KT - 1 <= full_hi; };
  issue(t_first, Ks0, Vs0);
  int t = t_first;
  for (; t + 1 <= t_last; t += 2) {
    wait_dma();
    __syncthreads();  // tile t landed in buffer 0; buffer 1 is free
    issue(t + 1, Ks1, Vs1);
    compute(Ks0, Vs0, full_tile(t * KT) ? 0 : 1, t * KT);
    wait_dma();
    __syncthreads();  // tile t+1 landed in buffer 1; buffer 0 is free
    if (t + 2 <= t_last) issue(t + 2, Ks0, Vs0);
    compute(Ks1, Vs1, full_tile((t + 1) * KT) ? 0 : 1, (t + 1) * KT);
  }
  if (t == t_last) {
    wait_dma();
    __syncthreads();
    compute(Ks0, Vs0, full_tile(t * KT) ? 0 : 1, t * KT);
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
    for (int q = tid; q < KT * (D / 8); q += 64 * kW) {
      const int x = q / (D / 8), c = q % (D / 8), jk = jb + x;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (jk < dg_hi) {
        const int row = min(max(p.qinfo[jk].x, 0), T - 1);
        kv = *reinterpret_cast<const u32x4*>(p.kr + ((size_t)row * Hkv + g) * D + c * 8);
        vv = *reinterpret_cast<const u32x4*>(p.v + ((size_t)row * Hkv + g) * D + c * 8);
      }
      *reinterpret_cast<u32x4*>(Ks0 + x * C::KROW + c * 16) = kv;
      *reinterpret_cast<u32x4*>(Vs0 + x * C::KROW + c * 16) = vv;
    }
    __syncthreads();
    compute(Ks0, Vs0, 2, 0);
  }

  if (q_on) {
    float* dst = p.dq + ((size_t)q_row * p.Hq + q_head) * D + 4 * q4;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) *reinterpret_cast<floatx4*>(dst + 16 * mb) = acc[mb] * p.scale;
  }
}

// dq = R^T dq', dk = R^T dk' in place (R: the RoPE rotation at the row's position). A
// thread takes 4 consecutive dims j .. j + 3 < D/2 of one (entry, head) and their partners
// j + D/2 .. (16-byte accesses). Index is uint32_t when the item count, T (Hq + Hkv) D / 8,
// fits 32 bits (cheap divisions), else uint64_t.
template <int D, typename Index>
__global__ __launch_bounds__(256) void unrotate_kernel(const int4* __restrict__ qinfo,
                                                       const float* __restrict__ cs,
                                                       const float* __restrict__ sn,
                                                       float* __restrict__ dq,
                                                       float* __restrict__ dk, int T, int Hq,
                                                       int Hkv, int max_pos) {
  constexpr int hd = D / 2, Q = hd / 4;  // float4 groups per half
  const int H = Hq + Hkv;
  const Index total = (Index)T * (Index)H * Q;
  for (Index t = (Index)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (Index)gridDim.x * blockDim.x) {
    const Index eh = t / Q;
    const int j = (int)(t % Q) * 4;
    const int e = (int)(eh / (Index)H), h = (int)(eh % (Index)H);
    const int4 qi = qinfo[e];
    const int row = min(max(qi.x, 0), T - 1);
    const int pos = min(max(qi.y - qi.w + qi.z, 0), max_pos);
    const floatx4 c = *reinterpret_cast<const floatx4*>(cs + (size_t)pos * hd + j);
    const floatx4 s = *reinterpret_cast<const floatx4*>(sn + (size_t)pos * hd + j);
    float* x = h < Hq ? dq + ((size_t)row * Hq + h) * D : dk + ((size_t)row * Hkv + (h - Hq)) * D;
    const floatx4 a = *reinterpret_cast<const floatx4*>(x + j);
    const floatx4 b = *reinterpret_cast<const floatx4*>(x + j + hd);
    floatx4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = a[i] * c[i] + b[i] * s[i];
      hi[i] = b[i] * c[i] - a[i] * s[i];
    }
    *reinterpret_cast<floatx4*>(x + j) = lo;
    *reinterpret_cast<floatx4*>(x + j + hd) = hi;
  }
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename F>
hipError_t for_d(int D, F&& f) {
  switch (D) {
    case 64: return f(std::integral_constant<int, 64>{});
    case 128: return f(std::integral_constant<int, 128>{});
    case 256: return f(std::integral_constant<int, 256>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

AttnBwdLayout attn_bwd_layout(int64_t n, int64_t T, int32_t Hq, int32_t Hkv, int32_t D) {
  AttnBwdLayout L;
  const int64_t G = Hq / std::max(1, Hkv);
  L.ntq = (T * G + KT - 1) / KT;
  const size_t tile_bytes = (size_t)Hkv * L.ntq * KT * D * 2;
  size_t off = attn_layout(n, T, Hq, Hkv, D).total;
  L.fwd = 0;
  L.dob = off;   off += al256((size_t)T * Hq * D * 2);
  L.dlt = off;   off += al256((size_t)T * Hq * 4);
  L.vpad = off;  off += al256((size_t)(n + KT) * Hkv * D * 2);
  L.qtr = off;   off += al256(tile_bytes);
  L.dtr = off;   off += al256(tile_bytes);
  L.smeta = off; off += al256((size_t)Hkv * L.ntq * KT * 16);
  // absolute segments of the tile list: about 16 for large lists, 32 to 512 tiles each
  L.seg_len = (int)std::min<int64_t>(512, std::max<int64_t>(32, (L.ntq + 15) / 16));
  L.nseg = (int)((L.ntq + L.seg_len - 1) / L.seg_len);
  L.part = off;  off += al256((size_t)L.nseg * 2 * n * Hkv * D * 4);
  L.total = off;
  return L;
}

hipError_t launch_attn_bwd(const AttnArgs& a, const int32_t* idx, const int32_t* depth_off,
                           const int32_t* cu_seqlens, const uint16_t* v, const float* out,
                           const float* lse, const float* dout, const float* rope_cos,
                           const float* rope_sin, float* dq, float* dk, float* dv, char* ws,
                           hipStream_t stream) {
  const AttnLayout F = attn_layout(a.n, a.T, a.Hq, a.Hkv, a.D);
  const AttnBwdLayout L = attn_bwd_layout(a.n, a.T, a.Hq, a.Hkv, a.D);
  BwdParams p;
  p.qinfo = reinterpret_cast<const int4*>(ws + F.qinfo);
  p.qstart = reinterpret_cast<const int32_t*>(ws + F.qstart);
  p.cu = cu_seqlens;
  p.chunks = reinterpret_cast<const int2*>(ws + F.chunks);
  p.nchunks = reinterpret_cast<const int32_t*>(ws + F.nchunks);
  p.qr = reinterpret_cast<const uint16_t*>(ws + F.qrot);
  p.kr = reinterpret_cast<const uint16_t*>(ws + F.krot);
  p.v = v;
  p.vpad = reinterpret_cast<const uint16_t*>(ws + L.vpad);
  p.dob = reinterpret_cast<const uint16_t*>(ws + L.dob);
  p.lse = lse;
  p.dlt = reinterpret_cast<const float*>(ws + L.dlt);
  p.qtr = reinterpret_cast<const uint16_t*>(ws + L.qtr);
  p.dtr = reinterpret_cast<const uint16_t*>(ws + L.dtr);
  p.smeta = reinterpret_cast<const int4*>(ws + L.smeta);
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.part = reinterpret_cast<float*>(ws + L.part);
  p.n = a.n;
  p.T = a.T;
  p.S = a.S;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.G = a.Hq / a.Hkv;
  p.QR = kAttnSlots / p.G;
  p.ntq = L.ntq;
  p.nkb = (a.n + kBwdKeys - 1) / kBwdKeys;
  p.seg_len = L.seg_len;
  const int nseg = L.nseg;
  p.scale = a.scale;
  p.c_log2 = a.scale * kLog2e;
  uint16_t* dob = reinterpret_cast<uint16_t*>(ws + L.dob);
  float* dlt = reinterpret_cast<float*>(ws + L.dlt);
  const int chunk_bound = std::min(F.max_chunks, (a.T + p.QR - 1) / p.QR + a.S);
  const int nkb = (a.n + kBwdKeys - 1) / kBwdKeys;

  return for_d(a.D, [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    const size_t items = (size_t)a.T * a.Hq * (D / 8);
    hipLaunchKernelGGL(bwd_dout_kernel<D>, dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                       stream, dout, out, dob, dlt, a.T, a.Hq);
    {
      const size_t work = (size_t)(a.n + KT) * a.Hkv * D / 8;
      const unsigned blocks = (unsigned)std::min<size_t>((work + 255) / 256, 65536);
      hipLaunchKernelGGL(vpad_kernel, dim3(blocks), dim3(256), 0, stream, v,
                         const_cast<uint16_t*>(p.vpad), a.n, a.Hkv, D);
    }
    hipLaunchKernelGGL(qtile_kernel<D>, dim3((unsigned)L.ntq, a.Hkv), dim3(256), 0, stream, p,
                       const_cast<uint16_t*>(p.qtr), const_cast<uint16_t*>(p.dtr),
                       const_cast<int4*>(p.smeta));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 kgrid((unsigned)((int64_t)nkb * a.Hkv * nseg));
    hipLaunchKernelGGL((dkdv_kernel<D>), kgrid, dim3(kBwdThreads), 0, stream, p);
    {
      const size_t count4 = (size_t)a.n * a.Hkv * D / 4;  // depth-0 rows of dk and dv
      const unsigned sb = (unsigned)std::min<size_t>((count4 + 255) / 256, 65536);
      hipLaunchKernelGGL(dkdv_sum_kernel<D>, dim3(sb), dim3(256), 0, stream, p);
    }
    if (a.T > a.n) {
      const int64_t waves = (int64_t)(a.T - a.n) * a.Hkv;
      hipLaunchKernelGGL(diag_kernel<D>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream,
                         p, idx, depth_off, a.K);
    }
    hipLaunchKernelGGL(dq_kernel<D>, dim3(chunk_bound * a.Hkv * 2), dim3(512), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t work = (size_t)a.T * (a.Hq + a.Hkv) * (D / 8);
    const unsigned blocks = (unsigned)std::min<size_t>((work + 255) / 256, 1 << 20);
    if (work + (size_t)blocks * 256 < ((size_t)1 << 32))
      hipLaunchKernelGGL((unrotate_kernel<D, uint32_t>), dim3(blocks), dim3(256), 0, stream,
                         p.qinfo, rope_cos, rope_sin, dq, dk, a.T, a.Hq, a.Hkv, a.max_pos);
    else
      hipLaunchKernelGGL((unrotate_kernel<D, uint64_t>), dim3(blocks), dim3(256), 0, stream,
                         p.qinfo, rope_cos, rope_sin, dq, dk, a.T, a.Hq, a.Hkv, a.max_pos);
    return hipGetLastError();
  });
}

}  // namespace peagle
