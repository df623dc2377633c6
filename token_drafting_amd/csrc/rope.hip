// RoPE gathered by position value, plus the layout preparation of the draft attention.
//
// NeMo Automodel PR 2376, commit message of the RoPE fix: cos/sin are gathered by the
// actual position values (not sliced by sequence length), from a cache sized to the
// highest requested position, which exceeds the sequence length for the per-depth
// offsets. Draft row (d, p) sits at position p - a_s + d, a_s being the start of p's
// packed sequence (the speculators guide, "Architecture": depth d at anchor + d; the
// snxtyle/P_Eagle README: packed sequences separated by cu_seqlens). Llama rotate-half
// convention, frequencies theta^(-2j/D); applied to q and k, not v.
//
// Kernels:
//   rope_table_kernel    cos/sin [max_pos+1, D/2] fp32, angles and cos/sin in fp64
//                        (direct sincos every 16th position of a thread, fp64 angle
//                        addition between).
//   qcount/qlist_kernel  anchor-major list of draft rows (all depths of anchor 0, then
//                        of anchor 1, ...) with per-row (row, anchor, depth, seq start),
//                        and qstart[p] = first entry of anchor p.
//   chunk_count/fill     the attention's chunk table (chunks never cross a sequence).
//   rope_rotate_kernel   q' and k' of every draft row, bf16, draft-row order.
//   v_transpose_kernel   depth-0 v as 32-key tiles laid out [d][32 keys], keys permuted
//                        inside each 16-key group as (0-3, 8-11, 4-7, 12-15) so that a
//                        16-byte read is the PV operand of one MFMA half-wave.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace peagle {

namespace {

// One thread per (frequency j, position residue p0 < P): the inverse frequency once, then
// positions p0, p0 + P, ... advance by the fp64 rotation through P theta_j (angle
// addition), re-anchored with a direct sincos every kRopeAnchor steps; the rotation's
// rounding (~1e-16 per step) stays far below the fp32 table's. Consecutive threads take
// consecutive j, so each position's row is written contiguously.
constexpr int kRopeAnchor = 16;
__global__ __launch_bounds__(256) void rope_table_kernel(float* __restrict__ cos_out,
                                                         float* __restrict__ sin_out, int half,
                                                         int D, double theta, int max_pos, int P) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int j = (int)(t % half);
  const int64_t p0 = t / half;
  if (p0 >= P || p0 > max_pos) return;
  const double inv = pow(theta, -2.0 * (double)j / (double)D);
  double step_s, step_c, sn = 0.0, cs = 1.0;
  sincos((double)P * inv, &step_s, &step_c);
  int k = 0;
  for (int64_t pos = p0; pos <= max_pos; pos += P, ++k) {
    if (k % kRopeAnchor == 0) {
      sincos((double)pos * inv, &sn, &cs);
    } else {
      const double c2 = fma(cs, step_c, -sn * step_s);
      sn = fma(sn, step_c, cs * step_s);
      cs = c2;
    }
    cos_out[pos * half + j] = (float)cs;
    sin_out[pos * half + j] = (float)sn;
  }
}

constexpr int kScanThreads = 1024;

// Exclusive scan of one value per thread over the 1024-thread block; returns the
// exclusive prefix and writes the block total to *total.
__device__ int block_exclusive_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kScanThreads / 64; ++w) {
    const int c = sh[w];
    if (w < wave) before += c;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// Kept depths of every anchor (depth sets are nested, so anchor p owns list entries for
// depths 0 .. c(p)-1); per block of 1024 anchors, the block total.
__device__ __forceinline__ int kept_depths(const int32_t* __restrict__ row_of, int n, int K, int p) {
  int c = 0;
  if (p < n)
    for (int d = 0; d < K; ++d) c += row_of[(size_t)d * n + p] >= 0;
  return c;
}

__global__ __launch_bounds__(kScanThreads) void qcount_kernel(const int32_t* __restrict__ row_of,
                                                              int n, int K,
                                                              int32_t* __restrict__ blocksum) {
  __shared__ int sh[kScanThreads / 64];
  int total;
  block_exclusive_scan(kept_depths(row_of, n, K, blockIdx.x * kScanThreads + threadIdx.x), sh, &total);
  if (threadIdx.x == 0) blocksum[blockIdx.x] = total;
}

// Anchor-major list: entry qstart[p] + d is draft row (d, p), stored with its anchor, its
// depth and the start of its sequence. Each block adds up the totals of the blocks before
// it, then scans its own anchors.
__global__ __launch_bounds__(kScanThreads) void qlist_kernel(
    const int32_t* __restrict__ row_of, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ blocksum, int n, int K, int S, int T, int4* __restrict__ qinfo,
    int32_t* __restrict__ qstart) {
  __shared__ int sh[kScanThreads / 64];
  __shared__ int s_off;
  const int b = blockIdx.x, p = b * kScanThreads + threadIdx.x;
  if (threadIdx.x < 64) {
    int v = 0;
    for (int j = threadIdx.x; j < b; j += 64) v += blocksum[j];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (threadIdx.x == 0) s_off = v;
  }
  const int c = kept_depths(row_of, n, K, p);
  int total;
  const int excl = block_exclusive_scan(c, sh, &total);  // its barriers also publish s_off
  const int start = s_off + excl;
  if (p < n) {
    qstart[p] = start;
    const int s = min(max(upper_index(cu, S + 1, p), 0), S);
    const int lo = cu[s];
    for (int d = 0; d < c; ++d)
      if (start + d < T) qinfo[start + d] = make_int4(row_of[(size_t)d * n + p], p, d, lo);
  }
  if (b == gridDim.x - 1 && threadIdx.x == 0) qstart[n] = min(s_off + total, T);
}

// Chunks of at most QR consecutive list entries that never cross a sequence, numbered
// sequence after sequence: seq_chunk[s] = first chunk of sequence s (a scan of the
// per-sequence chunk counts), seq_chunk[S] = *nchunks. One workgroup.
__global__ __launch_bounds__(kScanThreads) void chunk_count_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ qstart, int n, int S, int QR,
    int max_chunks, int32_t* __restrict__ nchunks, int32_t* __restrict__ seq_chunk) {
  __shared__ int sh[kScanThreads / 64];
  int ccarry = 0;
  for (int base = 0; base < S; base += kScanThreads) {
    const int s = base + threadIdx.x;
    int cnt = 0;
    if (s < S) {
      const int a = min(max(cu[s], 0), n), e = min(max(cu[s + 1], 0), n);
      const int rows = max(qstart[e] - qstart[a], 0);
      cnt = (rows + QR - 1) / QR;
    }
    int total;
    const int at = ccarry + block_exclusive_scan(cnt, sh, &total);
    if (s < S) seq_chunk[s] = min(at, max_chunks);
    ccarry += total;
  }
  if (threadIdx.x == 0) {
    *nchunks = min(ccarry, max_chunks);
    seq_chunk[S] = min(ccarry, max_chunks);
  }
}

// Chunk table entries (first list entry, entry count), one thread per chunk: the chunk's
// sequence is the last s with seq_chunk[s] <= c (empty sequences share their successor's
// start, so the last one is the non-empty sequence). Also clears the per-(chunk, kv head)
// redo flags, and writes the chunk's key metadata, which the attention workgroups then
// read in one load instead of a chain of dependent ones:
//   cmeta[2c]     = (j0, jn, k_lo, k_hi): the chunk's list entries (clamped to the list) and
//                   its key range (rows see keys from their sequence start up to their
//                   own anchor: k_lo = the first row's sequence start, k_hi = the last
//                   row's anchor);
//   cmeta[2c + 1] = (full_lo, full_hi, dg_lo, dg_hi): keys every row sees, and the list
//                   entries of the chunk's anchors (their depth >= 1 rows are the
//                   diagonal keys).
__global__ __launch_bounds__(256) void chunk_fill_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ qstart,
    const int4* __restrict__ qinfo, const int32_t* __restrict__ seq_chunk,
    const int32_t* __restrict__ nchunks, int n, int T, int S, int QR, int max_chunks,
    int2* __restrict__ chunks, int4* __restrict__ cmeta, int32_t* __restrict__ flags,
    int nflags) {
  const int nc = min(max(*nchunks, 0), max_chunks);
  const int stride = gridDim.x * blockDim.x;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nflags; i += stride) flags[i] = 0;
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < nc; c += stride) {
    const int s = min(max(upper_index(seq_chunk, S + 1, c), 0), S - 1);
    const int j = c - seq_chunk[s];
    const int a = min(max(cu[s], 0), n), e = min(max(cu[s + 1], 0), n);
    const int first = qstart[a], rows = max(qstart[e] - first, 0);
    const int2 ch = make_int2(first + j * QR, min(QR, rows - j * QR));
    chunks[c] = ch;
    const int j0 = min(max(ch.x, 0), T - 1);
    const int jn = min(max(ch.y, 1), T - j0);
    const int4 qa = qinfo[j0], qb = qinfo[j0 + jn - 1];
    const int p_first = min(max(qa.y, 0), n - 1), p_last = min(max(qb.y, 0), n - 1);
    cmeta[2 * c] = make_int4(j0, jn, min(max(qa.w, 0), p_first), p_last);
    cmeta[2 * c + 1] = make_int4(min(max(qb.w, 0), p_last), p_first,
                                 min(max(qstart[p_first], 0), T),
                                 min(max(qstart[p_last + 1], 0), T));
  }
}

// One thread per (list entry, head, 8-wide chunk of the first half of the head
// dimension). The anchor-major list entry gives the draft row, its anchor, depth and
// sequence start, so the position value is one load away. Idx is 32-bit unless the
// work count needs 64 bits.
template <typename Idx>
__global__ __launch_bounds__(256) void rope_rotate_kernel(
    const int4* __restrict__ qinfo, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ cosT, const float* __restrict__ sinT, uint16_t* __restrict__ qr,
    uint16_t* __restrict__ kr, uint16_t* __restrict__ kr_lo, int n, int T, int Hq, int Hkv, int D,
    int max_pos) {
  const int half = D / 2, cpr = half / 8;  // chunks per head
  const Idx heads = (Idx)(Hq + Hkv), per_entry = heads * (Idx)cpr;
  const Idx total = (Idx)T * per_entry;
  for (Idx t = (Idx)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (Idx)gridDim.x * blockDim.x) {
    const Idx j = t / per_entry, rem = t - j * per_entry;
    const int h = (int)(rem / (Idx)cpr), c = (int)(rem - (Idx)h * cpr);
    const int4 e = qinfo[j];
    const int r = min(max(e.x, 0), T - 1);
    const int p = min(max(e.y, 0), n - 1);
    const int offset = p - min(max(e.w, 0), p);  // anchor's offset in its sequence
    const int pos = min(max(offset + e.z, 0), max_pos);
    const uint16_t* src = (h < Hq) ? q + ((size_t)r * Hq + h) * D : k + ((size_t)r * Hkv + (h - Hq)) * D;
    uint16_t* dst = (h < Hq) ? qr + ((size_t)r * Hq + h) * D : kr + ((size_t)r * Hkv + (h - Hq)) * D;
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(src + c * 8);
    const u32x4 x2 = *reinterpret_cast<const u32x4*>(src + half + c * 8);
    const floatx4* cp = reinterpret_cast<const floatx4*>(cosT + (size_t)pos * half + c * 8);
    const floatx4* sp = reinterpret_cast<const floatx4*>(sinT + (size_t)pos * half + c * 8);
    const floatx4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
    u32x4 y1, y2, z1, z2;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t o1 = 0, o2 = 0, l1 = 0, l2 = 0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int j = w * 2 + e;
        const float a = bf16_bits_to_f32((x1[w] >> (16 * e)) & 0xFFFFu);
        const float b = bf16_bits_to_f32((x2[w] >> (16 * e)) & 0xFFFFu);
        const float cs = (j < 4) ? c0[j] : c1[j - 4];
        const float sn = (j < 4) ? s0[j] : s1[j - 4];
        const float r1 = a * cs - b * sn, r2 = b * cs + a * sn;
        const uint16_t h1 = f32_to_bf16_bits(r1), h2 = f32_to_bf16_bits(r2);
        o1 |= (uint32_t)h1 << (16 * e);
        o2 |= (uint32_t)h2 << (16 * e);
        l1 |= (uint32_t)f32_to_bf16_bits(r1 - bf16_bits_to_f32(h1)) << (16 * e);
        l2 |= (uint32_t)f32_to_bf16_bits(r2 - bf16_bits_to_f32(h2)) << (16 * e);
      }
      y1[w] = o1;
      y2[w] = o2;
      z1[w] = l1;
      z2[w] = l2;
    }
    *reinterpret_cast<u32x4*>(dst + c * 8) = y1;
    *reinterpret_cast<u32x4*>(dst + half + c * 8) = y2;
    // k rows of a sequence's first anchors also keep the rounding residual (k_lo) for the
    // attention's exact-split chunks
    if (h >= Hq && offset < kShortSpan) {
      uint16_t* lo = kr_lo + ((size_t)r * Hkv + (h - Hq)) * D;
      *reinterpret_cast<u32x4*>(lo + c * 8) = z1;
      *reinterpret_cast<u32x4*>(lo + half + c * 8) = z2;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void v_transpose_kernel(const uint16_t* __restrict__ v,
                                                          uint16_t* __restrict__ vt, int n, int Hkv,
                                                          int ntiles) {
  __shared__ uint16_t tile[32][D + 8];
  const int t = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  constexpr int cpr = D / 8;
  for (int q = tid; q < 32 * cpr; q += 256) {
    const int key = q / cpr, c = q % cpr, pos = t * 32 + key;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (pos < n) val = *reinterpret_cast<const u32x4*>(v + ((size_t)pos * Hkv + g) * D + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      tile[key][c * 8 + 2 * w] = (uint16_t)(val[w] & 0xFFFFu);
      tile[key][c * 8 + 2 * w + 1] = (uint16_t)(val[w] >> 16);
    }
  }
  __syncthreads();
  uint16_t* out = vt + ((size_t)g * ntiles + t) * D * 32;
  for (int q = tid; q < D * 4; q += 256) {
    const int d = q >> 2, chunk = q & 3;
    uint16_t vals[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // element e of chunk (2*g16 + h) holds key 16*g16 + 8*(e/4) + 4*h + e%4
      const int g16 = chunk >> 1, h = chunk & 1;
      const int key = 16 * g16 + 8 * (e >> 2) + 4 * h + (e & 3);
      vals[e] = tile[key][d];
    }
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = (uint32_t)vals[2 * w] | ((uint32_t)vals[2 * w + 1] << 16);
    *reinterpret_cast<u32x4*>(out + (size_t)d * 32 + chunk * 8) = o;
  }
}

template <typename F>
hipError_t launch_for_d(int D, F&& f) {
  switch (D) {
    case 64: return f(std::integral_constant<int, 64>{});
    case 128: return f(std::integral_constant<int, 128>{});
    case 256: return f(std::integral_constant<int, 256>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_rope_table(int32_t head_dim, double theta, int32_t max_pos, float* cos_out,
                             float* sin_out, hipStream_t stream) {
  const int half = head_dim / 2;
  // position stride: ~128K threads, each taking every P-th position
  const int P = (int)std::min<int64_t>((int64_t)max_pos + 1,
                                       std::max<int64_t>(1, ((int64_t)1 << 17) / half));
  const int64_t threads = (int64_t)P * half;
  const int blocks = (int)((threads + 255) / 256);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, stream, cos_out, sin_out, half,
                     head_dim, theta, max_pos, P);
  return hipGetLastError();
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Upper bound on the chunk count: every sequence adds at most one partial chunk, and a
// sequence holds at least one anchor, so S <= n.
int attn_max_chunks(int64_t n, int64_t T, int32_t Hq, int32_t Hkv) {
  const int QR = kAttnSlots / std::max(1, Hq / std::max(1, Hkv));
  return (int)((T + QR - 1) / QR + n);
}

// Enough workgroups for two per CU (256 CUs) need no split; below that, up to
// kMaxAttnSplit segments per chunk. A chunk spans at most n keys: with fewer than
// kSplitMinTiles 32-key tiles none can be cut into two segments of the work list's
// 8-tile minimum, and the split's extra launches would be pure overhead.
constexpr int kSplitBlocks = 512, kSplitMinTiles = 16;

AttnSplit attn_split_plan(int64_t n, int64_t T, int32_t Hq, int32_t Hkv) {
  const int64_t QR = kAttnSlots / std::max(1, Hq / std::max(1, Hkv));
  const int64_t blocks = std::max<int64_t>(1, (T + QR - 1) / QR) * std::max(1, Hkv);
  const bool split = blocks < kSplitBlocks && (n + 31) / 32 >= kSplitMinTiles;
  return AttnSplit{split ? kMaxAttnSplit : 1};
}

AttnLayout attn_layout(int64_t n, int64_t T, int32_t Hq, int32_t Hkv, int32_t D) {
  AttnLayout L;
  const size_t ntiles = (size_t)((n + 31) / 32);
  size_t off = 0;
  L.qinfo = off;  off += align256((size_t)T * sizeof(int4));
  L.qstart = off; off += align256((size_t)(n + 1) * sizeof(int32_t));
  L.qrot = off;   off += align256((size_t)T * Hq * D * 2);
  // K regions: 32 rows of padding so the last 32-key tile of depth-0 keys stays inside
  L.krot = off;   off += align256((size_t)(T + 32) * Hkv * D * 2);
  L.krot_lo = off; off += align256((size_t)(T + 32) * Hkv * D * 2);
  L.vt = off;     off += align256(ntiles * 32 * Hkv * D * 2);
  L.max_chunks = attn_max_chunks(n, T, Hq, Hkv);
  L.chunks = off; off += align256((size_t)L.max_chunks * sizeof(int2));
  L.cmeta = off;  off += align256((size_t)L.max_chunks * 2 * sizeof(int4));
  L.nchunks = off; off += 256;
  L.seq_chunk = off; off += align256((size_t)(n + 1) * sizeof(int32_t));
  L.flags = off;  off += align256((size_t)L.max_chunks * Hkv * sizeof(int32_t));
  L.blocksum = off; off += align256((size_t)((n + 1023) / 1024) * sizeof(int32_t));
  // split attention: segment count per (chunk, kv head), the work list of (chunk, segment)
  // items; partial O of segments 1.. (segment 0 keeps its partial in the output);
  // per-segment (reference max, sum) of every row
  const AttnSplit sp = attn_split_plan(n, T, Hq, Hkv);
  L.segs = off;   off += align256((size_t)L.max_chunks * Hkv * sizeof(int32_t));
  L.items = off;  off += align256((size_t)L.max_chunks * Hkv * sp.nsplit * sizeof(int2));
  L.nitems = off; off += 256;
  L.part = off;   off += align256((size_t)(sp.nsplit - 1) * T * Hq * D * sizeof(float));
  L.ml = off;     off += sp.nsplit > 1 ? align256((size_t)sp.nsplit * Hq * T * 2 * sizeof(float)) : 0;
  L.total = off;
  return L;
}

hipError_t launch_attn_prepare(const AttnArgs& a, const int32_t* idx, const int32_t* depth_off,
                               const int32_t* row_of, const int32_t* cu_seqlens,
                               const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const float* rope_cos, const float* rope_sin, char* ws,
                               hipStream_t stream) {
  const AttnLayout L = attn_layout(a.n, a.T, a.Hq, a.Hkv, a.D);
  int4* qinfo = reinterpret_cast<int4*>(ws + L.qinfo);
  int32_t* qstart = reinterpret_cast<int32_t*>(ws + L.qstart);
  uint16_t* qr = reinterpret_cast<uint16_t*>(ws + L.qrot);
  uint16_t* kr = reinterpret_cast<uint16_t*>(ws + L.krot);
  uint16_t* kr_lo = reinterpret_cast<uint16_t*>(ws + L.krot_lo);
  uint16_t* vt = reinterpret_cast<uint16_t*>(ws + L.vt);

  int2* chunks = reinterpret_cast<int2*>(ws + L.chunks);
  int32_t* nchunks = reinterpret_cast<int32_t*>(ws + L.nchunks);
  int32_t* seq_chunk = reinterpret_cast<int32_t*>(ws + L.seq_chunk);
  int32_t* blocksum = reinterpret_cast<int32_t*>(ws + L.blocksum);
  const int nblk = (a.n + kScanThreads - 1) / kScanThreads;
  hipLaunchKernelGGL(qcount_kernel, dim3(nblk), dim3(kScanThreads), 0, stream, row_of, a.n, a.K,
                     blocksum);
  hipLaunchKernelGGL(qlist_kernel, dim3(nblk), dim3(kScanThreads), 0, stream, row_of, cu_seqlens,
                     blocksum, a.n, a.K, a.S, a.T, qinfo, qstart);
  const int QR = kAttnSlots / (a.Hq / a.Hkv);
  hipLaunchKernelGGL(chunk_count_kernel, dim3(1), dim3(kScanThreads), 0, stream, cu_seqlens, qstart,
                     a.n, a.S, QR, L.max_chunks, nchunks, seq_chunk);
  {
    // chunk count <= ceil(T / QR) + S; the flags cover max_chunks * Hkv entries
    const int64_t work = std::max<int64_t>((int64_t)(a.T + QR - 1) / QR + a.S,
                                           (int64_t)L.max_chunks * a.Hkv);
    const int blocks = (int)std::min<int64_t>((work + 255) / 256, 2048);
    hipLaunchKernelGGL(chunk_fill_kernel, dim3(blocks), dim3(256), 0, stream, cu_seqlens, qstart,
                       qinfo, seq_chunk, nchunks, a.n, a.T, a.S, QR, L.max_chunks, chunks,
                       reinterpret_cast<int4*>(ws + L.cmeta),
                       reinterpret_cast<int32_t*>(ws + L.flags), L.max_chunks * a.Hkv);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const size_t work = (size_t)a.T * (a.Hq + a.Hkv) * (a.D / 16);
  const int blocks = (int)std::min<size_t>((work + 255) / 256, 1 << 20);
  if (work < (size_t)UINT32_MAX)
    hipLaunchKernelGGL(rope_rotate_kernel<uint32_t>, dim3(blocks), dim3(256), 0, stream, qinfo, q, k,
                       rope_cos, rope_sin, qr, kr, kr_lo, a.n, a.T, a.Hq, a.Hkv, a.D, a.max_pos);
  else
    hipLaunchKernelGGL(rope_rotate_kernel<size_t>, dim3(blocks), dim3(256), 0, stream, qinfo, q, k,
                       rope_cos, rope_sin, qr, kr, kr_lo, a.n, a.T, a.Hq, a.Hkv, a.D, a.max_pos);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int ntiles = (a.n + 31) / 32;
  return launch_for_d(a.D, [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    hipLaunchKernelGGL(v_transpose_kernel<D>, dim3(ntiles, a.Hkv), dim3(256), 0, stream, v, vt,
                       a.n, a.Hkv, ntiles);
    return hipGetLastError();
  });
}

}  // namespace peagle
