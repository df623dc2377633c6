// C entry points of libpeagle: host-side validation, then the kernel launchers.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "peagle.h"
#include "kernels.h"
#include "layer.h"
#include "bwd.h"
#include "variants.h"

using namespace peagle;

namespace {

constexpr int64_t kMaxI32 = 0x7FFFFFFF;

int status_of(hipError_t e) { return e == hipSuccess ? PEAGLE_OK : PEAGLE_ERR_HIP; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// COD counts [speculators P-EAGLE guide, "COD Sampling"]: depth d keeps
// max(round(n r^d), round(n r_min)) positions, rounding half up, capped at n.
int counts(int64_t n, int32_t K, double r, double r_min, int64_t* m, int64_t* T) {
  if (n < 1 || n > kMaxI32 || K < 1 || K > PEAGLE_MAX_DEPTHS) return PEAGLE_ERR_ARG;
  if (!std::isfinite(r) || !(r > 0.0) || r > 1.0) return PEAGLE_ERR_ARG;
  if (!std::isfinite(r_min) || r_min < 0.0 || r_min > 1.0) return PEAGLE_ERR_ARG;
  const double nd = (double)n;
  const int64_t floor_count = (int64_t)std::floor(nd * r_min + 0.5);
  int64_t total = 0;
  for (int d = 0; d < K; ++d) {
    int64_t md = (int64_t)std::floor(nd * std::pow(r, (double)d) + 0.5);
    if (md < floor_count) md = floor_count;
    if (md > n) md = n;
    if (m) m[d] = md;
    total += md;
  }
  if (T) *T = total;
  return PEAGLE_OK;
}

// Attention shapes the kernels take: every product behind the workspace layout stays far
// inside size_t ((T + 32) Hq D elements at most 2^44).
int attn_shape(int64_t n, int64_t T, int32_t Hq, int32_t Hkv, int32_t D) {
  if (n < 1 || n > kMaxI32 || T < n || T > kMaxI32) return PEAGLE_ERR_ARG;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return PEAGLE_ERR_ARG;
  if (D != 64 && D != 128 && D != 256) return PEAGLE_ERR_UNSUPPORTED;
  if (kAttnSlots % (Hq / Hkv) != 0) return PEAGLE_ERR_UNSUPPORTED;
  // the kernels address a 32-row tile of kv rows (Hkv D bf16 apart) with 32-bit offsets
  if ((int64_t)Hkv * D > ((int64_t)1 << 25)) return PEAGLE_ERR_UNSUPPORTED;
  if ((double)(T + 32) * (double)Hq * (double)D > (double)((int64_t)1 << 44)) return PEAGLE_ERR_ARG;
  return PEAGLE_OK;
}

struct AttnCall {
  AttnArgs a;
  const int32_t *idx, *depth_off, *row_of, *cu;
  const uint16_t *q, *k, *v;
  const float *cs, *sn;
  float *out, *lse;
  char* ws;
  hipStream_t stream;
};

int attn_check(int64_t n, int32_t K, int64_t T, const int32_t* idx, const int32_t* depth_off,
               const int32_t* row_of, const int32_t* cu, int32_t S, const peagle_bf16* q,
               const peagle_bf16* k, const peagle_bf16* v, int32_t Hq, int32_t Hkv, int32_t D,
               float scale, const float* cs, const float* sn, int32_t max_pos, float* out,
               float* lse, void* ws, size_t ws_bytes, void* stream, AttnCall* call) {
  if (K < 1 || K > PEAGLE_MAX_DEPTHS) return PEAGLE_ERR_ARG;
  const int shape = attn_shape(n, T, Hq, Hkv, D);
  if (shape != PEAGLE_OK) return shape;
  if (T > (int64_t)K * n) return PEAGLE_ERR_ARG;
  if (S < 1 || S > n) return PEAGLE_ERR_ARG;
  if (!(scale > 0.f) || !std::isfinite(scale)) return PEAGLE_ERR_ARG;
  if ((int64_t)max_pos < n + K - 2) return PEAGLE_ERR_ARG;
  if (ws_bytes < attn_layout(n, T, Hq, Hkv, D).total) return PEAGLE_ERR_WORKSPACE;
  if (!idx || !depth_off || !row_of || !cu || !q || !k || !v || !cs || !sn || !out || !ws)
    return PEAGLE_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(cs) ||
      !aligned16(sn) || (reinterpret_cast<uintptr_t>(ws) & 255) != 0)
    return PEAGLE_ERR_ARG;
  call->a = AttnArgs{(int32_t)n, K, (int32_t)T, S, Hq, Hkv, D, max_pos, scale};
  call->idx = idx;
  call->depth_off = depth_off;
  call->row_of = row_of;
  call->cu = cu;
  call->q = q;
  call->k = k;
  call->v = v;
  call->cs = cs;
  call->sn = sn;
  call->out = out;
  call->lse = lse;
  call->ws = static_cast<char*>(ws);
  call->stream = static_cast<hipStream_t>(stream);
  return PEAGLE_OK;
}

int run_prepare(const AttnCall& c) {
  return status_of(launch_attn_prepare(c.a, c.idx, c.depth_off, c.row_of, c.cu, c.q, c.k, c.v,
                                       c.cs, c.sn, c.ws, c.stream));
}

int run_core(const AttnCall& c) {
  return status_of(launch_attn_core(c.a, c.v, c.out, c.lse, c.ws, c.stream));
}

bool decode_dims_ok(int32_t B, int32_t Hkv, int32_t D) {
  return B >= 1 && B <= 65535 && Hkv >= 1 && Hkv <= 65535 && (D == 64 || D == 128 || D == 256);
}

size_t v_tiles_bytes(int64_t total_ctx, int32_t B, int32_t Hkv, int32_t D) {
  return (size_t)decode_ntiles(total_ctx, B) * Hkv * D * 32 * sizeof(uint16_t);
}

}  // namespace

extern "C" {

const char* peagle_status_string(int status) {
  switch (status) {
    case PEAGLE_OK: return "ok";
    case PEAGLE_ERR_ARG: return "invalid argument";
    case PEAGLE_ERR_UNSUPPORTED: return "unsupported shape";
    case PEAGLE_ERR_HIP: return "HIP launch failure";
    case PEAGLE_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

int peagle_version(void) { return 100; }

int peagle_cod_counts(int64_t n, int32_t K, double r, double r_min, int64_t* m, int64_t* T) {
  return counts(n, K, r, r_min, m, T);
}

size_t peagle_cod_workspace_bytes(int64_t n, int32_t K) {
  if (n < 1 || n > kMaxI32 || K < 1 || K > PEAGLE_MAX_DEPTHS) return 0;
  return cod_workspace_bytes(n, K);
}

static int cod_select_entry(int64_t n, int32_t K, double r, double r_min, uint64_t seed,
                            const int32_t* cu_seqlens, int32_t num_seqs, int32_t* idx,
                            int32_t* depth_off, int32_t* cu_seqlens_d, int32_t* row_of,
                            void* workspace, size_t workspace_bytes, bool noalloc, void* stream) {
  int64_t m[PEAGLE_MAX_DEPTHS], T = 0;
  const int st = counts(n, K, r, r_min, m, &T);
  if (st != PEAGLE_OK) return st;
  if (T > kMaxI32 || (int64_t)K * n > ((int64_t)1 << 40)) return PEAGLE_ERR_ARG;
  if (num_seqs < 1 || num_seqs > n) return PEAGLE_ERR_ARG;
  if (!cu_seqlens || !idx || !depth_off || !cu_seqlens_d || !row_of) return PEAGLE_ERR_ARG;
  if (noalloc) {
    static_assert(kCodNoAllocScratchBytes == PEAGLE_COD_NOALLOC_SCRATCH_BYTES, "scratch size");
    if (cod_workspace_bytes(n, K) > kCodNoAllocScratchBytes) return PEAGLE_ERR_WORKSPACE;
    if (cod_noalloc_scratch(&workspace) != hipSuccess) return PEAGLE_ERR_HIP;
  } else {
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return PEAGLE_ERR_ARG;
    if (workspace_bytes < cod_workspace_bytes(n, K)) return PEAGLE_ERR_WORKSPACE;
  }
  CodArgs a{};
  a.n = (int32_t)n;
  a.K = K;
  a.S = num_seqs;
  a.seed = seed;
  a.off[0] = 0;
  for (int d = 0; d < K; ++d) {
    a.m[d] = (int32_t)m[d];
    a.off[d + 1] = a.off[d] + (int32_t)m[d];
  }
  return status_of(launch_cod_select(a, cu_seqlens, idx, depth_off, cu_seqlens_d, row_of,
                                     workspace, static_cast<hipStream_t>(stream)));
}

int peagle_cod_select(int64_t n, int32_t K, double r, double r_min, uint64_t seed,
                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t* idx,
                      int32_t* depth_off, int32_t* cu_seqlens_d, int32_t* row_of,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return cod_select_entry(n, K, r, r_min, seed, cu_seqlens, num_seqs, idx, depth_off,
                          cu_seqlens_d, row_of, workspace, workspace_bytes, false, stream);
}

int peagle_cod_select_noalloc(int64_t n, int32_t K, double r, double r_min, uint64_t seed,
                              const int32_t* cu_seqlens, int32_t num_seqs, int32_t* idx,
                              int32_t* depth_off, int32_t* cu_seqlens_d, int32_t* row_of,
                              void* stream) {
  return cod_select_entry(n, K, r, r_min, seed, cu_seqlens, num_seqs, idx, depth_off,
                          cu_seqlens_d, row_of, nullptr, 0, true, stream);
}

int peagle_fuse_inputs(int64_t n, int32_t K, int64_t T, const int32_t* idx,
                       const peagle_bf16* aux, int32_t aux_dim, const peagle_bf16* fc_weight,
                       const peagle_bf16* mask_hidden, const int32_t* tokens,
                       const peagle_bf16* embed, int32_t vocab, int32_t ptd_token_id, int32_t H,
                       float* hidden_out, peagle_bf16* embed_out, void* stream) {
  if (n < 1 || n > kMaxI32 || K < 1 || K > PEAGLE_MAX_DEPTHS) return PEAGLE_ERR_ARG;
  if (T < n || T > (int64_t)K * n || T > kMaxI32) return PEAGLE_ERR_ARG;
  if (aux_dim < 8 || aux_dim % 8 != 0 || H < 8 || H % 8 != 0 || vocab < 1) return PEAGLE_ERR_ARG;
  if (ptd_token_id < 0 || ptd_token_id >= vocab) return PEAGLE_ERR_ARG;
  if (!idx || !aux || !fc_weight || !mask_hidden || !tokens || !embed || !hidden_out || !embed_out)
    return PEAGLE_ERR_ARG;
  if (!aligned16(aux) || !aligned16(fc_weight) || !aligned16(mask_hidden) || !aligned16(embed) ||
      !aligned16(hidden_out) || !aligned16(embed_out))
    return PEAGLE_ERR_ARG;
  FuseArgs a{(int32_t)n, (int32_t)T, aux_dim, H, vocab, ptd_token_id};
  return status_of(launch_fuse(a, idx, aux, fc_weight, mask_hidden, tokens, embed, hidden_out,
                               embed_out, static_cast<hipStream_t>(stream)));
}

int peagle_fuse_inputs_fc_norm(int64_t n, int32_t K, int64_t T, const int32_t* idx,
                               const peagle_bf16* aux, int32_t aux_dim,
                               const peagle_bf16* fc_weight, const peagle_bf16* mask_hidden,
                               const int32_t* tokens, const peagle_bf16* embed, int32_t vocab,
                               int32_t ptd_token_id, int32_t H, const peagle_bf16* fc_norm_weight,
                               float eps, float* hidden_out, peagle_bf16* embed_out,
                               void* stream) {
  if (!fc_norm_weight || !aligned16(fc_norm_weight) || !(eps > 0.f) || !std::isfinite(eps))
    return PEAGLE_ERR_ARG;
  const int st = peagle_fuse_inputs(n, K, T, idx, aux, aux_dim, fc_weight, mask_hidden, tokens,
                                    embed, vocab, ptd_token_id, H, hidden_out, embed_out, stream);
  if (st != PEAGLE_OK) return st;
  return status_of(
      launch_rms_inplace(hidden_out, fc_norm_weight, T, H, eps, static_cast<hipStream_t>(stream)));
}

int peagle_rope_table(int32_t head_dim, double theta, int32_t max_pos, float* cos_out,
                      float* sin_out, void* stream) {
  if (head_dim < 2 || head_dim % 2 != 0 || max_pos < 0) return PEAGLE_ERR_ARG;
  if (!std::isfinite(theta) || !(theta > 0.0)) return PEAGLE_ERR_ARG;
  if (((int64_t)max_pos + 1) * (head_dim / 2) > kMaxI32) return PEAGLE_ERR_ARG;
  if (!cos_out || !sin_out) return PEAGLE_ERR_ARG;
  return status_of(
      launch_rope_table(head_dim, theta, max_pos, cos_out, sin_out, static_cast<hipStream_t>(stream)));
}

size_t peagle_draft_attn_workspace_bytes(int64_t n, int64_t T, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim) {
  if (attn_shape(n, T, num_q_heads, num_kv_heads, head_dim) != PEAGLE_OK) return 0;
  return attn_layout(n, T, num_q_heads, num_kv_heads, head_dim).total;
}

#define PEAGLE_ATTN_ARGS                                                                       \
  int64_t n, int32_t K, int64_t T, const int32_t *idx, const int32_t *depth_off,              \
      const int32_t *row_of, const int32_t *cu_seqlens, int32_t num_seqs, const peagle_bf16 *q, \
      const peagle_bf16 *k, const peagle_bf16 *v, int32_t num_q_heads, int32_t num_kv_heads,    \
      int32_t head_dim, float softmax_scale, const float *rope_cos, const float *rope_sin,     \
      int32_t rope_max_pos, float *out, float *lse, void *workspace, size_t workspace_bytes,   \
      void *stream
#define PEAGLE_ATTN_FWD                                                                         \
  n, K, T, idx, depth_off, row_of, cu_seqlens, num_seqs, q, k, v, num_q_heads, num_kv_heads,   \
      head_dim, softmax_scale, rope_cos, rope_sin, rope_max_pos, out, lse, workspace,          \
      workspace_bytes, stream

int peagle_draft_attn_prepare(PEAGLE_ATTN_ARGS) {
  AttnCall c;
  const int st = attn_check(PEAGLE_ATTN_FWD, &c);
  return st != PEAGLE_OK ? st : run_prepare(c);
}

int peagle_draft_attn_core(PEAGLE_ATTN_ARGS) {
  AttnCall c;
  const int st = attn_check(PEAGLE_ATTN_FWD, &c);
  return st != PEAGLE_OK ? st : run_core(c);
}

int peagle_draft_attn_fwd(PEAGLE_ATTN_ARGS) {
  AttnCall c;
  int st = attn_check(PEAGLE_ATTN_FWD, &c);
  if (st != PEAGLE_OK) return st;
  st = run_prepare(c);
  return st != PEAGLE_OK ? st : run_core(c);
}

size_t peagle_draft_attn_bwd_workspace_bytes(int64_t n, int64_t T, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim) {
  if (attn_shape(n, T, num_q_heads, num_kv_heads, head_dim) != PEAGLE_OK) return 0;
  return attn_bwd_layout(n, T, num_q_heads, num_kv_heads, head_dim).total;
}

int peagle_draft_attn_bwd(int64_t n, int32_t K, int64_t T, const int32_t* idx,
                          const int32_t* depth_off, const int32_t* row_of,
                          const int32_t* cu_seqlens, int32_t num_seqs, const peagle_bf16* q,
                          const peagle_bf16* k, const peagle_bf16* v, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                          const float* rope_cos, const float* rope_sin, int32_t rope_max_pos,
                          const float* out, const float* lse, const float* dout, float* dq,
                          float* dk, float* dv, void* workspace, size_t workspace_bytes,
                          void* stream) {
  AttnCall c;
  int st = attn_check(n, K, T, idx, depth_off, row_of, cu_seqlens, num_seqs, q, k, v,
                      num_q_heads, num_kv_heads, head_dim, softmax_scale, rope_cos, rope_sin,
                      rope_max_pos, const_cast<float*>(out), const_cast<float*>(lse), workspace,
                      workspace_bytes, stream, &c);
  if (st != PEAGLE_OK) return st;
  if (!lse || !dout || !dq || !dk || !dv) return PEAGLE_ERR_ARG;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(lse))
    return PEAGLE_ERR_ARG;
  const AttnBwdLayout L = attn_bwd_layout(n, T, num_q_heads, num_kv_heads, head_dim);
  if (workspace_bytes < L.total) return PEAGLE_ERR_WORKSPACE;
  if (L.ntq > kMaxI32) return PEAGLE_ERR_ARG;
  st = run_prepare(c);
  if (st != PEAGLE_OK) return st;
  return status_of(launch_attn_bwd(c.a, idx, depth_off, cu_seqlens, v, out, lse, dout, rope_cos,
                                   rope_sin, dq, dk, dv, c.ws, c.stream));
}

size_t peagle_depth_ce_workspace_bytes(int64_t T, int32_t K) {
  if (T < 1 || T > kMaxI32 || K < 1 || K > PEAGLE_MAX_DEPTHS) return 0;
  return depth_ce_workspace_bytes(T, K);
}

int peagle_depth_ce(int64_t T, int32_t K, int32_t vocab, const int32_t* depth_off,
                    const peagle_bf16* logits, const int32_t* labels, float decay,
                    float* loss_out, float* depth_loss, peagle_bf16* dlogits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (T < 1 || T > kMaxI32 || K < 1 || K > PEAGLE_MAX_DEPTHS || vocab < 1) return PEAGLE_ERR_ARG;
  if (!(decay > 0.f) || !(decay <= 1.f)) return PEAGLE_ERR_ARG;
  if (!depth_off || !logits || !labels || !loss_out || !workspace) return PEAGLE_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return PEAGLE_ERR_ARG;
  if (workspace_bytes < depth_ce_workspace_bytes(T, K)) return PEAGLE_ERR_WORKSPACE;
  return status_of(launch_depth_ce(T, K, vocab, depth_off, logits, labels, decay, loss_out,
                                   depth_loss, dlogits, static_cast<char*>(workspace),
                                   static_cast<hipStream_t>(stream)));
}

int peagle_accept_prefix(int32_t num_drafts, int32_t K, int32_t vocab,
                         const peagle_bf16* draft_logits, const peagle_bf16* target_logits,
                         int32_t* draft_tok, int32_t* target_tok, int32_t* accept_len,
                         void* stream) {
  if (num_drafts < 0 || K < 1 || K > PEAGLE_MAX_DEPTHS || vocab < 1) return PEAGLE_ERR_ARG;
  if (!draft_logits || !target_logits || !draft_tok || !target_tok || !accept_len)
    return PEAGLE_ERR_ARG;
  if (num_drafts == 0) return PEAGLE_OK;
  return status_of(launch_accept(num_drafts, K, vocab, draft_logits, target_logits, draft_tok,
                                 target_tok, accept_len, static_cast<hipStream_t>(stream)));
}

size_t peagle_decode_v_tiles_bytes(int64_t total_ctx, int32_t num_reqs, int32_t num_kv_heads,
                                   int32_t head_dim) {
  if (total_ctx < 0 || total_ctx > kMaxI32 || !decode_dims_ok(num_reqs, num_kv_heads, head_dim))
    return 0;
  return v_tiles_bytes(total_ctx, num_reqs, num_kv_heads, head_dim);
}

int peagle_decode_pack_v(int32_t num_reqs, const int32_t* cu_ctx, int64_t total_ctx,
                         int32_t max_ctx, const peagle_bf16* v_cache, int32_t num_kv_heads,
                         int32_t head_dim, peagle_bf16* v_tiles, size_t v_tiles_bytes_given,
                         void* stream) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PEAGLE_ERR_UNSUPPORTED;
  if (!decode_dims_ok(num_reqs, num_kv_heads, head_dim)) return PEAGLE_ERR_ARG;
  if (total_ctx < 0 || total_ctx > kMaxI32 || max_ctx < 0 || max_ctx > total_ctx)
    return PEAGLE_ERR_ARG;
  if (!cu_ctx) return PEAGLE_ERR_ARG;
  if (total_ctx == 0) return PEAGLE_OK;
  if (!v_cache || !v_tiles || !aligned16(v_cache) || !aligned16(v_tiles)) return PEAGLE_ERR_ARG;
  if (v_tiles_bytes_given < v_tiles_bytes(total_ctx, num_reqs, num_kv_heads, head_dim))
    return PEAGLE_ERR_WORKSPACE;
  return status_of(launch_decode_pack_v(cu_ctx, num_reqs, total_ctx, max_ctx, v_cache,
                                        num_kv_heads, head_dim, v_tiles,
                                        static_cast<hipStream_t>(stream)));
}

size_t peagle_draft_decode_workspace_bytes(int32_t num_reqs, int32_t K, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int64_t total_ctx, int32_t max_ctx) {
  if (!decode_dims_ok(num_reqs, num_kv_heads, head_dim) || K < 1 || K > 32 || max_ctx < 0 ||
      total_ctx < max_ctx || total_ctx > kMaxI32 || num_q_heads < 1 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  return decode_workspace_bytes(num_reqs, K, num_q_heads, num_kv_heads, head_dim, total_ctx,
                                max_ctx);
}

static int decode_attn_entry(int32_t num_reqs, int32_t K, const int32_t* cu_ctx,
                             const int32_t* lens, int64_t total_ctx, int32_t max_ctx,
                             const peagle_bf16* k_cache, const peagle_bf16* v_tiles,
                             size_t v_tiles_bytes_given, const peagle_bf16* q,
                             const peagle_bf16* k, const peagle_bf16* v, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                             const float* rope_cos, const float* rope_sin, int32_t rope_max_pos,
                             float* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PEAGLE_ERR_UNSUPPORTED;
  if (K > 32) return PEAGLE_ERR_UNSUPPORTED;
  if (!decode_dims_ok(num_reqs, num_kv_heads, head_dim) || K < 1) return PEAGLE_ERR_ARG;
  if (num_q_heads < 1 || num_q_heads % num_kv_heads != 0) return PEAGLE_ERR_ARG;
  if ((int64_t)num_kv_heads * ((num_q_heads / num_kv_heads * K + 31) / 32) > 65535)
    return PEAGLE_ERR_UNSUPPORTED;
  // the combine kernel runs one thread per (request, kv head, column, 4 dims)
  if ((int64_t)num_reqs * num_kv_heads * ((num_q_heads / num_kv_heads * K + 31) / 32 * 32) *
          (head_dim / 4) > kMaxI32)
    return PEAGLE_ERR_UNSUPPORTED;
  if (total_ctx < 0 || total_ctx > kMaxI32 || max_ctx < 0 || max_ctx > total_ctx)
    return PEAGLE_ERR_ARG;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return PEAGLE_ERR_ARG;
  if (rope_max_pos < 0 || (int64_t)rope_max_pos < (int64_t)max_ctx + K - 1) return PEAGLE_ERR_ARG;
  if (!cu_ctx || !q || !k || !v || !rope_cos || !rope_sin || !out || !workspace)
    return PEAGLE_ERR_ARG;
  if (total_ctx > 0 && (!k_cache || !v_tiles || !aligned16(k_cache) || !aligned16(v_tiles)))
    return PEAGLE_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(rope_cos) ||
      !aligned16(rope_sin) || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return PEAGLE_ERR_ARG;
  if (total_ctx > 0 &&
      v_tiles_bytes_given < v_tiles_bytes(total_ctx, num_reqs, num_kv_heads, head_dim))
    return PEAGLE_ERR_WORKSPACE;
  if (workspace_bytes <
      decode_workspace_bytes(num_reqs, K, num_q_heads, num_kv_heads, head_dim, total_ctx, max_ctx))
    return PEAGLE_ERR_WORKSPACE;
  DecodeArgs a{num_reqs, K, num_q_heads, num_kv_heads, head_dim, max_ctx, rope_max_pos,
               total_ctx, softmax_scale};
  return status_of(launch_decode_attn_lens(a, cu_ctx, lens, k_cache, v_tiles, q, k, v, rope_cos,
                                           rope_sin, out, lse, static_cast<char*>(workspace),
                                           static_cast<hipStream_t>(stream)));
}

int peagle_draft_decode_attn(int32_t num_reqs, int32_t K, const int32_t* cu_ctx,
                             int64_t total_ctx, int32_t max_ctx, const peagle_bf16* k_cache,
                             const peagle_bf16* v_tiles, size_t v_tiles_bytes_given,
                             const peagle_bf16* q, const peagle_bf16* k, const peagle_bf16* v,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             float softmax_scale, const float* rope_cos, const float* rope_sin,
                             int32_t rope_max_pos, float* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return decode_attn_entry(num_reqs, K, cu_ctx, nullptr, total_ctx, max_ctx, k_cache, v_tiles,
                           v_tiles_bytes_given, q, k, v, num_q_heads, num_kv_heads, head_dim,
                           softmax_scale, rope_cos, rope_sin, rope_max_pos, out, lse, workspace,
                           workspace_bytes, stream);
}

int peagle_draft_decode_attn_lens(int32_t num_reqs, int32_t K, const int32_t* cu_cap,
                                  const int32_t* lens, int64_t total_cap, int32_t max_cap,
                                  const peagle_bf16* k_cache, const peagle_bf16* v_tiles,
                                  size_t v_tiles_bytes_given, const peagle_bf16* q,
                                  const peagle_bf16* k, const peagle_bf16* v,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  float softmax_scale, const float* rope_cos,
                                  const float* rope_sin, int32_t rope_max_pos, float* out,
                                  float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (!lens) return PEAGLE_ERR_ARG;
  return decode_attn_entry(num_reqs, K, cu_cap, lens, total_cap, max_cap, k_cache, v_tiles,
                           v_tiles_bytes_given, q, k, v, num_q_heads, num_kv_heads, head_dim,
                           softmax_scale, rope_cos, rope_sin, rope_max_pos, out, lse, workspace,
                           workspace_bytes, stream);
}

int peagle_decode_pack_v_lens(int32_t num_reqs, const int32_t* cu_cap, const int32_t* lens,
                              int64_t total_cap, int32_t max_cap, const peagle_bf16* v_cache,
                              int32_t num_kv_heads, int32_t head_dim, peagle_bf16* v_tiles,
                              size_t v_tiles_bytes_given, void* stream) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PEAGLE_ERR_UNSUPPORTED;
  if (!decode_dims_ok(num_reqs, num_kv_heads, head_dim)) return PEAGLE_ERR_ARG;
  if (total_cap < 0 || total_cap > kMaxI32 || max_cap < 0 || max_cap > total_cap)
    return PEAGLE_ERR_ARG;
  if (!cu_cap || !lens) return PEAGLE_ERR_ARG;
  if (total_cap == 0) return PEAGLE_OK;
  if (!v_cache || !v_tiles || !aligned16(v_cache) || !aligned16(v_tiles)) return PEAGLE_ERR_ARG;
  if (v_tiles_bytes_given < v_tiles_bytes(total_cap, num_reqs, num_kv_heads, head_dim))
    return PEAGLE_ERR_WORKSPACE;
  return status_of(launch_decode_pack_v_lens(cu_cap, lens, num_reqs, total_cap, max_cap, v_cache,
                                             num_kv_heads, head_dim, v_tiles,
                                             static_cast<hipStream_t>(stream)));
}

int peagle_decode_append(int32_t num_reqs, const int32_t* cu_cap, const int32_t* lens_in,
                         const int32_t* n_new, int32_t n_add, int32_t max_new,
                         const peagle_bf16* k_new, const peagle_bf16* v_new,
                         int32_t num_kv_heads, int32_t head_dim, const float* rope_cos,
                         const float* rope_sin, int32_t rope_max_pos, int64_t total_cap,
                         int32_t max_cap, peagle_bf16* k_cache, peagle_bf16* v_tiles,
                         size_t v_tiles_bytes_given, int32_t* lens_out, void* stream) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PEAGLE_ERR_UNSUPPORTED;
  if (!decode_dims_ok(num_reqs, num_kv_heads, head_dim)) return PEAGLE_ERR_ARG;
  if (max_new < 1 || n_add < 0 || n_add > max_new) return PEAGLE_ERR_ARG;
  if ((int64_t)num_reqs * max_new * num_kv_heads * (head_dim / 16 + head_dim / 8) + num_reqs >
      kMaxI32)
    return PEAGLE_ERR_UNSUPPORTED;
  if (total_cap < 1 || total_cap > kMaxI32 || max_cap < 1 || max_cap > total_cap)
    return PEAGLE_ERR_ARG;
  if (rope_max_pos < 0 || rope_max_pos < max_cap - 1) return PEAGLE_ERR_ARG;
  if (!cu_cap || !lens_in || !n_new || !k_new || !v_new || !rope_cos || !rope_sin || !k_cache ||
      !v_tiles || !lens_out || lens_out == lens_in)
    return PEAGLE_ERR_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_tiles) ||
      !aligned16(rope_cos) || !aligned16(rope_sin))
    return PEAGLE_ERR_ARG;
  if (v_tiles_bytes_given < v_tiles_bytes(total_cap, num_reqs, num_kv_heads, head_dim))
    return PEAGLE_ERR_WORKSPACE;
  return status_of(launch_decode_append(cu_cap, lens_in, n_new, n_add, max_new, k_new, v_new,
                                        rope_cos, rope_sin, rope_max_pos, k_cache, v_tiles,
                                        lens_out, num_reqs, num_kv_heads, head_dim, max_cap,
                                        total_cap, static_cast<hipStream_t>(stream)));
}

size_t peagle_layer1_qkv_workspace_bytes(int64_t n, int64_t T, int32_t H) {
  if (n < 1 || T < n || T > kMaxI32 || H < 1) return 0;
  return layer1_workspace_bytes(n, T, H);
}

int peagle_layer1_qkv(int64_t n, int32_t K, int64_t T, const float* hidden,
                      const peagle_bf16* embed, int32_t H, const peagle_bf16* w_norm_emb,
                      const peagle_bf16* w_norm_hidden, float eps, const peagle_bf16* w_qkv,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      peagle_bf16* q, peagle_bf16* k, peagle_bf16* v, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (n < 1 || n > kMaxI32 || K < 1 || K > PEAGLE_MAX_DEPTHS) return PEAGLE_ERR_ARG;
  if (T < n || T > (int64_t)K * n || T > kMaxI32) return PEAGLE_ERR_ARG;
  if (H < 1 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 ||
      head_dim < 1)
    return PEAGLE_ERR_ARG;
  if (H % 32 != 0 || head_dim % 8 != 0) return PEAGLE_ERR_UNSUPPORTED;
  if ((int64_t)(num_q_heads + 2 * num_kv_heads) * head_dim > kMaxI32) return PEAGLE_ERR_ARG;
  if (!(eps > 0.f) || !std::isfinite(eps)) return PEAGLE_ERR_ARG;
  if (!hidden || !embed || !w_norm_emb || !w_norm_hidden || !w_qkv || !q || !k || !v ||
      !workspace)
    return PEAGLE_ERR_ARG;
  if (!aligned16(hidden) || !aligned16(embed) || !aligned16(w_norm_emb) ||
      !aligned16(w_norm_hidden) || !aligned16(w_qkv) || !aligned16(q) || !aligned16(k) ||
      !aligned16(v) || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return PEAGLE_ERR_ARG;
  if (workspace_bytes < layer1_workspace_bytes(n, T, H)) return PEAGLE_ERR_WORKSPACE;
  Layer1Args a{(int32_t)n, K, (int32_t)T, H, num_q_heads, num_kv_heads, head_dim, eps};
  return status_of(launch_layer1_qkv(a, hidden, embed, w_norm_emb, w_norm_hidden, w_qkv, q, k, v,
                                     static_cast<char*>(workspace),
                                     static_cast<hipStream_t>(stream)));
}

size_t peagle_layer1_post_workspace_bytes(int64_t n, int64_t T, int32_t H, int32_t QW,
                                          int32_t I) {
  if (n < 1 || T < n || T > kMaxI32 || H < 1 || QW < 1 || I < 1) return 0;
  return layer1_post_workspace_bytes(n, T, H, QW, I);
}

int peagle_layer1_post(int64_t n, int32_t K, int64_t T, const float* attn_out, int32_t QW,
                       const float* hidden, int32_t H, const peagle_bf16* w_norm_hidden,
                       int32_t norm_before_residual, const peagle_bf16* w_o,
                       const peagle_bf16* w_post, const peagle_bf16* w_gate,
                       const peagle_bf16* w_up, int32_t I, const peagle_bf16* w_down, float eps,
                       float* h2_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (n < 1 || n > kMaxI32 || K < 1 || K > PEAGLE_MAX_DEPTHS) return PEAGLE_ERR_ARG;
  if (T < n || T > (int64_t)K * n || T > kMaxI32) return PEAGLE_ERR_ARG;
  if (H < 1 || QW < 1 || I < 1) return PEAGLE_ERR_ARG;
  if (H % 64 != 0 || QW % 64 != 0 || I % 64 != 0) return PEAGLE_ERR_UNSUPPORTED;
  if ((int64_t)2 * I > kMaxI32 || (int64_t)T * (QW > H ? QW : H) > ((int64_t)1 << 40))
    return PEAGLE_ERR_ARG;
  if (!(eps > 0.f) || !std::isfinite(eps)) return PEAGLE_ERR_ARG;
  if (!attn_out || !hidden || (norm_before_residual && !w_norm_hidden) || !w_o || !w_post ||
      !w_gate || !w_up || !w_down || !h2_out || !workspace)
    return PEAGLE_ERR_ARG;
  if (!aligned16(attn_out) || !aligned16(hidden) ||
      (norm_before_residual && !aligned16(w_norm_hidden)) || !aligned16(w_o) ||
      !aligned16(w_post) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(h2_out) || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return PEAGLE_ERR_ARG;
  if (workspace_bytes < layer1_post_workspace_bytes(n, T, H, QW, I)) return PEAGLE_ERR_WORKSPACE;
  Layer1PostArgs a{(int32_t)n, (int32_t)T, H, QW, I, norm_before_residual ? 1 : 0, eps};
  return status_of(launch_layer1_post(a, attn_out, hidden, w_norm_hidden, w_o, w_post, w_gate,
                                      w_up, w_down, h2_out, static_cast<char*>(workspace),
                                      static_cast<hipStream_t>(stream)));
}

size_t peagle_layer_qkv_workspace_bytes(int64_t T, int32_t H) {
  if (T < 1 || T > kMaxI32 || H < 1) return 0;
  return layer_qkv_workspace_bytes(T, H);
}

int peagle_layer_qkv(int64_t T, const float* h, int32_t H, const peagle_bf16* w_norm, float eps,
                     const peagle_bf16* w_qkv, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, peagle_bf16* q, peagle_bf16* k, peagle_bf16* v,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 1 || T > kMaxI32) return PEAGLE_ERR_ARG;
  if (H < 1 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 ||
      head_dim < 1)
    return PEAGLE_ERR_ARG;
  if (H % 64 != 0 || head_dim % 8 != 0) return PEAGLE_ERR_UNSUPPORTED;
  if ((int64_t)(num_q_heads + 2 * num_kv_heads) * head_dim > kMaxI32) return PEAGLE_ERR_ARG;
  if (!(eps > 0.f) || !std::isfinite(eps)) return PEAGLE_ERR_ARG;
  if (!h || !w_norm || !w_qkv || !q || !k || !v || !workspace) return PEAGLE_ERR_ARG;
  if (!aligned16(h) || !aligned16(w_norm) || !aligned16(w_qkv) || !aligned16(q) ||
      !aligned16(k) || !aligned16(v) || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return PEAGLE_ERR_ARG;
  if (workspace_bytes < layer_qkv_workspace_bytes(T, H)) return PEAGLE_ERR_WORKSPACE;
  LayerArgs a{(int32_t)T, H, num_q_heads, num_kv_heads, head_dim, eps};
  return status_of(launch_layer_qkv(a, h, w_norm, w_qkv, q, k, v, static_cast<char*>(workspace),
                                    static_cast<hipStream_t>(stream)));
}

size_t peagle_layer_post_workspace_bytes(int64_t T, int32_t H, int32_t QW, int32_t I) {
  if (T < 1 || T > kMaxI32 || H < 1 || QW < 1 || I < 1) return 0;
  return layer1_post_workspace_bytes(T, T, H, QW, I);
}

int peagle_layer_post(int64_t T, const float* attn_out, int32_t QW, const float* h, int32_t H,
                      const peagle_bf16* w_o, const peagle_bf16* w_post,
                      const peagle_bf16* w_gate, const peagle_bf16* w_up, int32_t I,
                      const peagle_bf16* w_down, float eps, float* h2_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (T < 1 || T > kMaxI32 || H < 1 || QW < 1 || I < 1) return PEAGLE_ERR_ARG;
  if (H % 64 != 0 || QW % 64 != 0 || I % 64 != 0) return PEAGLE_ERR_UNSUPPORTED;
  if ((int64_t)2 * I > kMaxI32 || T * (QW > H ? QW : H) > ((int64_t)1 << 40))
    return PEAGLE_ERR_ARG;
  if (!(eps > 0.f) || !std::isfinite(eps)) return PEAGLE_ERR_ARG;
  if (!attn_out || !h || !w_o || !w_post || !w_gate || !w_up || !w_down || !h2_out ||
      !workspace)
    return PEAGLE_ERR_ARG;
  if (!aligned16(attn_out) || !aligned16(h) || !aligned16(w_o) || !aligned16(w_post) ||
      !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(h2_out) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return PEAGLE_ERR_ARG;
  if (workspace_bytes < layer1_post_workspace_bytes(T, T, H, QW, I)) return PEAGLE_ERR_WORKSPACE;
  // the first layer's second half with every row distinct and the raw residual stream
  Layer1PostArgs a{(int32_t)T, (int32_t)T, H, QW, I, 0, eps};
  return status_of(launch_layer1_post(a, attn_out, h, nullptr, w_o, w_post, w_gate, w_up, w_down,
                                      h2_out, static_cast<char*>(workspace),
                                      static_cast<hipStream_t>(stream)));
}

size_t peagle_draft_head_workspace_bytes(int64_t T, int32_t H, int32_t V) {
  if (T < 1 || T > kMaxI32 || H < 1 || V < 1) return 0;
  return draft_head_workspace_bytes(T, H, V);
}

int peagle_draft_head(int64_t T, const float* h, int32_t H, const peagle_bf16* w_final,
                      const peagle_bf16* w_head, int32_t V, float eps, int32_t* tokens,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 1 || T > kMaxI32 || H < 1 || V < 1) return PEAGLE_ERR_ARG;
  if (H % 64 != 0) return PEAGLE_ERR_UNSUPPORTED;
  if (!(eps > 0.f) || !std::isfinite(eps)) return PEAGLE_ERR_ARG;
  if (!h || !w_final || !w_head || !tokens || !workspace) return PEAGLE_ERR_ARG;
  if (!aligned16(h) || !aligned16(w_final) || !aligned16(w_head) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return PEAGLE_ERR_ARG;
  if (workspace_bytes < draft_head_workspace_bytes(T, H, V)) return PEAGLE_ERR_WORKSPACE;
  return status_of(launch_draft_head(T, H, V, eps, h, w_final, w_head, tokens,
                                     static_cast<char*>(workspace),
                                     static_cast<hipStream_t>(stream)));
}

int peagle_accept_prefix_d2t(int32_t num_drafts, int32_t K, int32_t draft_vocab,
                             int32_t target_vocab, const peagle_bf16* draft_logits,
                             const peagle_bf16* target_logits, const int32_t* d2t,
                             int32_t* draft_tok, int32_t* target_tok, int32_t* accept_len,
                             void* stream) {
  if (num_drafts < 0 || K < 1 || K > PEAGLE_MAX_DEPTHS || draft_vocab < 1 || target_vocab < 1)
    return PEAGLE_ERR_ARG;
  if (!draft_logits || !target_logits || !d2t || !draft_tok || !target_tok || !accept_len)
    return PEAGLE_ERR_ARG;
  if (num_drafts == 0) return PEAGLE_OK;
  return status_of(launch_accept_map(num_drafts, K, draft_vocab, target_vocab, draft_logits,
                                     target_logits, d2t, draft_tok, target_tok, accept_len,
                                     static_cast<hipStream_t>(stream)));
}

static int accept_sampled_entry(int32_t num_drafts, int32_t K, int32_t vocab,
                                const peagle_bf16* draft_logits, const peagle_bf16* target_logits,
                                const int32_t* draft_tok, const float* u, const float* w,
                                float temperature, bool bonus, int32_t* accept_len,
                                int32_t* next_tok, void* stream) {
  if (num_drafts < 0 || K < 1 || K > PEAGLE_MAX_DEPTHS || vocab < 1) return PEAGLE_ERR_ARG;
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return PEAGLE_ERR_ARG;
  if (num_drafts == 0) return PEAGLE_OK;  // nothing is read: empty tensors may be null
  if (!draft_logits || !target_logits || !draft_tok || !u || !w || !accept_len || !next_tok)
    return PEAGLE_ERR_ARG;
  return status_of(launch_accept_sampled(num_drafts, K, vocab, draft_logits, target_logits,
                                         draft_tok, u, w, temperature, bonus, accept_len,
                                         next_tok, static_cast<hipStream_t>(stream)));
}

int peagle_accept_sampled(int32_t num_drafts, int32_t K, int32_t vocab,
                          const peagle_bf16* draft_logits, const peagle_bf16* target_logits,
                          const int32_t* draft_tok, const float* u, const float* w,
                          float temperature, int32_t* accept_len, int32_t* next_tok,
                          void* stream) {
  return accept_sampled_entry(num_drafts, K, vocab, draft_logits, target_logits, draft_tok, u, w,
                              temperature, false, accept_len, next_tok, stream);
}

int peagle_accept_sampled_bonus(int32_t num_drafts, int32_t K, int32_t vocab,
                                const peagle_bf16* draft_logits, const peagle_bf16* target_logits,
                                const int32_t* draft_tok, const float* u, const float* w,
                                float temperature, int32_t* accept_len, int32_t* next_tok,
                                void* stream) {
  return accept_sampled_entry(num_drafts, K, vocab, draft_logits, target_logits, draft_tok, u, w,
                              temperature, true, accept_len, next_tok, stream);
}

}  // extern "C"
