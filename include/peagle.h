/*
 * peagle.h -- C ABI of libpeagle, the MI355X (gfx950) draft forward of P-EAGLE
 * parallel drafting: all K prediction depths of an EAGLE-3 style drafter in one pass.
 *
 * Sources (the pages that describe the method):
 *   [G]  speculators documentation, user guide "P-EAGLE": sections "Architecture",
 *        "COD Sampling", "Inference Process", "Key Parameters".
 *   [N]  NeMo Automodel pull request 2376, "feat(speculative): add P-EAGLE
 *        parallel-drafting training for EAGLE-3 drafts": the PR description
 *        (implementation, checkpoint contract, parity section) and the commit message
 *        of the RoPE fix.
 *   [R]  snxtyle/P_Eagle README: packed conversations isolated by cu_seqlens; section
 *        "How Speculative Decoding Works" (accepted tokens kept, rejected ones resampled).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host). The caller owns all memory;
 *     the library never allocates, frees or synchronises. Work is enqueued
 *     asynchronously on `stream` (a hipStream_t passed as void*, NULL = null stream).
 *   - Tensors are dense, row-major, and bf16 tensors are raw bit patterns (uint16_t).
 *     Device pointers must be 16-byte aligned.
 *   - Arguments are checked on the host before anything is enqueued. A bad argument
 *     returns PEAGLE_ERR_ARG (or PEAGLE_ERR_UNSUPPORTED for a valid but unimplemented
 *     shape) and enqueues nothing. A launch failure returns PEAGLE_ERR_HIP. Faults inside
 *     a kernel surface at the caller's next synchronisation.
 *   - Integer arrays that are device data (cu_seqlens, idx, row_of, tokens) are trusted:
 *     the kernels clamp indices derived from them so a malformed array cannot make them
 *     read or write out of bounds, but the results are then meaningless.
 *   - Notation: n tokens in the packed buffer, S packed sequences, K depths, T draft
 *     rows. Draft rows are depth-major; inside a depth they ascend by anchor. Depth 0
 *     keeps every position, so draft row p of depth 0 is anchor p.
 *   - The library keeps no state beyond a per-device cache of the compute-unit count,
 *     creates no streams or events, and is safe to call from several threads (calls
 *     that share an output or workspace buffer must not overlap).
 */
#ifndef PEAGLE_H_
#define PEAGLE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t peagle_bf16; /* raw bfloat16 bits */

enum {
  PEAGLE_OK = 0,
  PEAGLE_ERR_ARG = -1,         /* invalid argument; nothing enqueued */
  PEAGLE_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head_dim 96) */
  PEAGLE_ERR_HIP = -3,         /* the HIP runtime rejected a launch */
  PEAGLE_ERR_WORKSPACE = -4    /* workspace smaller than the *_workspace_bytes result */
};

#define PEAGLE_MAX_DEPTHS 64

/* Human-readable name of a status code (static string). */
const char *peagle_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int peagle_version(void);

/*
 * peagle_cod_counts -- host arithmetic of COD sampling [G, "COD Sampling"]: depth 0
 * keeps all n positions, depth d keeps about n*r^d, never fewer than about n*r_min.
 *   m[d] = min(n, max(floor(n*r^d + 1/2), floor(n*r_min + 1/2)))  for d in [0, K)
 *   *T   = sum of m[d]
 * n >= 1, 1 <= K <= PEAGLE_MAX_DEPTHS, 0 < r <= 1, 0 <= r_min <= 1.
 * m: (host) int64[K]; T: (host) int64. Either may be NULL when not wanted.
 */
int peagle_cod_counts(int64_t n, int32_t K, double r, double r_min, int64_t *m, int64_t *T);

/*
 * peagle_cod_select -- COD index builder [G, "COD Sampling"]. Depth d keeps the m[d]
 * buffer indices p with the smallest SplitMix64(seed XOR p) (first output of the
 * SplitMix64 generator from state seed^p, compared as unsigned 64-bit words), p being
 * the index in the whole packed buffer. The sets are nested: R_d within R_{d-1}.
 *   cu_seqlens    int32[S+1]       packed-sequence starts, 0 = cu[0] <= ... <= cu[S] = n
 *   idx           int32[T]   out   anchors, depth-major, ascending within a depth
 *   depth_off     int32[K+1] out   first draft row of each depth (prefix sum of m)
 *   cu_seqlens_d  int32[K*(S+1)] out  [d][s] = kept anchors of depth d below cu[s]
 *   row_of        int32[K*n] out   [d][p] = draft row of (d, p), or -1 if not kept
 *   workspace     >= peagle_cod_workspace_bytes(n, K) bytes of device memory, 256-byte
 *                 aligned (up to n = 65536 the hashes grouped by their top byte per block
 *                 of 1024 positions, with the groups' sizes; beyond, per-depth thresholds
 *                 and per-block kept counts); its contents are scratch and need no
 *                 initialisation
 * Requires n < 2^31 and T as given by peagle_cod_counts. Work is O(n K) in two launches:
 * up to n = 65536 a hash pass and a select pass, each a workgroup per 1024 positions;
 * beyond, one workgroup finds the thresholds and per-block counts, then a workgroup per
 * 1024 positions compacts its block.
 */
size_t peagle_cod_workspace_bytes(int64_t n, int32_t K); /* 0 on bad arguments */
int peagle_cod_select(int64_t n, int32_t K, double r, double r_min, uint64_t seed,
                      const int32_t *cu_seqlens, int32_t num_seqs, int32_t *idx,
                      int32_t *depth_off, int32_t *cu_seqlens_d, int32_t *row_of,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * peagle_cod_select_noalloc -- peagle_cod_select for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and outputs without the workspace. Its scratch (the
 * thresholds and per-block counts) is a static device array of
 * PEAGLE_COD_NOALLOC_SCRATCH_BYTES per GPU, held from the library's load until the process
 * ends; the call allocates and frees nothing. The first call on a device looks up the
 * array's address there (hipGetSymbolAddress). Limit: peagle_cod_workspace_bytes(n, K) must
 * not exceed PEAGLE_COD_NOALLOC_SCRATCH_BYTES (every n up to 65536; then e.g. n <= 33.5M at
 * K = 8), else
 * PEAGLE_ERR_WORKSPACE and nothing is enqueued. All calls on one GPU share the array: calls
 * that may overlap on that GPU (other streams, other threads) race and must be ordered by
 * the caller. The scratch needs no clearing: every call writes what it reads.
 */
#define PEAGLE_COD_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)
int peagle_cod_select_noalloc(int64_t n, int32_t K, double r, double r_min, uint64_t seed,
                              const int32_t *cu_seqlens, int32_t num_seqs, int32_t *idx,
                              int32_t *depth_off, int32_t *cu_seqlens_d, int32_t *row_of,
                              void *stream);

/*
 * peagle_fuse_inputs -- fused input stage [N, description; G, "Architecture"]. Depth 0
 * rows take fc(aux[p]) and the embedding of tokens[p]; depth >= 1 rows take
 * fc(mask_hidden) and the embedding of ptd_token_id. fc is a bias-free linear layer
 * run as a bf16 MFMA GEMM with fp32 accumulation; no fc_norm.
 *   idx           int32[T]            from peagle_cod_select
 *   aux           bf16[n, aux_dim]    concatenated target aux hidden states (3 x H_target)
 *   fc_weight     bf16[H, aux_dim]    linear-layer layout (output-major)
 *   mask_hidden   bf16[aux_dim]       the learnable placeholder
 *   tokens        int32[n]            token of each position
 *   embed         bf16[vocab, H]      input embedding table
 *   hidden_out    fp32[T, H]   out
 *   embed_out     bf16[T, H]   out
 * aux_dim and H must be multiples of 8. ptd_token_id must lie in [0, vocab)
 * (required and range-checked, as in [N]'s recipe arguments). hidden_out and embed_out are
 * written in full; before its final writes the call may keep partial sums of the fc
 * reduction in them (their previous contents are ignored).
 */
int peagle_fuse_inputs(int64_t n, int32_t K, int64_t T, const int32_t *idx,
                       const peagle_bf16 *aux, int32_t aux_dim, const peagle_bf16 *fc_weight,
                       const peagle_bf16 *mask_hidden, const int32_t *tokens,
                       const peagle_bf16 *embed, int32_t vocab, int32_t ptd_token_id, int32_t H,
                       float *hidden_out, peagle_bf16 *embed_out, void *stream);

/*
 * peagle_fuse_inputs_fc_norm -- peagle_fuse_inputs with the RMSNorm after fc [N,
 * description: mask_hidden is projected "through fc/fc_norm", after EAGLE-3.1's toggle]:
 * every hidden_out row (the projections of aux and of mask_hidden alike) becomes
 *   row / sqrt(mean(row^2) + eps) * fc_norm_weight,
 * in fp32. fc_norm_weight bf16[H]; eps > 0 (Llama: 1e-6); other arguments as for
 * peagle_fuse_inputs. H must be a multiple of 8 (as there).
 */
int peagle_fuse_inputs_fc_norm(int64_t n, int32_t K, int64_t T, const int32_t *idx,
                               const peagle_bf16 *aux, int32_t aux_dim,
                               const peagle_bf16 *fc_weight, const peagle_bf16 *mask_hidden,
                               const int32_t *tokens, const peagle_bf16 *embed, int32_t vocab,
                               int32_t ptd_token_id, int32_t H, const peagle_bf16 *fc_norm_weight,
                               float eps, float *hidden_out, peagle_bf16 *embed_out,
                               void *stream);

/*
 * peagle_rope_table -- cos/sin cache indexed by position value [N, RoPE-fix commit]:
 *   cos_out[pos][j] = cos(pos * theta^(-2j/D)), sin_out likewise, j < D/2,
 * angles and cos/sin evaluated in float64, stored fp32, for pos in [0, max_pos].
 *   cos_out, sin_out  fp32[max_pos+1, head_dim/2]  out
 * head_dim even, theta > 0, max_pos >= 0.
 */
int peagle_rope_table(int32_t head_dim, double theta, int32_t max_pos, float *cos_out,
                      float *sin_out, void *stream);

/* Bytes of workspace peagle_draft_attn_* need for these sizes (0 on bad arguments). */
size_t peagle_draft_attn_workspace_bytes(int64_t n, int64_t T, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim);

/*
 * peagle_draft_attn_fwd -- multi-depth draft attention forward [N, description and
 * parity section; R; G, "Architecture"]. The query of draft row (d, p), head h, sees
 *   - depth-0 keys p' of the same packed sequence with p' <= p, and
 *   - its own anchor's depth-e rows for 1 <= e <= d (the diagonal extension),
 * on RoPE-rotated q and k at positions p - a_s + d (a_s = start of p's sequence; cos/sin
 * gathered by position value, [N, RoPE-fix commit]); q head h reads kv head
 * floor(h / (Hq/Hkv)). Softmax in fp32, QK^T and PV on bf16 MFMA.
 *   idx, depth_off, row_of   from peagle_cod_select
 *   cu_seqlens       int32[S+1]
 *   q                bf16[T, Hq, D]   pre-RoPE
 *   k, v             bf16[T, Hkv, D]  pre-RoPE
 *   softmax_scale    usually 1/sqrt(D)
 *   rope_cos/sin     fp32[rope_max_pos+1, D/2] from peagle_rope_table;
 *                    rope_max_pos >= n + K - 2 (the largest position any row can take)
 *   out              fp32[T, Hq, D]   out
 *   lse              fp32[Hq, T]      out, natural-log softmax denominators; may be NULL
 *   workspace        >= peagle_draft_attn_workspace_bytes(n, T, Hq, Hkv, D) bytes,
 *                    device memory, 256-byte aligned; its contents are scratch
 * head_dim in {64, 128, 256}; Hq % Hkv == 0 and 256 % (Hq/Hkv) == 0; Hkv * head_dim
 * at most 2^25 (a 32-row key tile then stays below 2^31 bytes).
 * Equal to peagle_draft_attn_prepare followed by peagle_draft_attn_core.
 * Streams: every kernel goes on `stream` alone, ordered after earlier work on it and
 * before later work on it; the call creates no streams or events and takes no locks, so
 * it can be recorded into a HIP graph. Two calls that share a workspace must not overlap.
 * T is checked only against n <= T <= K*n: the call takes no r / r_min, so the caller
 * must pass the T that peagle_cod_counts gave for the idx / depth_off / row_of in use.
 */
int peagle_draft_attn_fwd(int64_t n, int32_t K, int64_t T, const int32_t *idx,
                          const int32_t *depth_off, const int32_t *row_of,
                          const int32_t *cu_seqlens, int32_t num_seqs, const peagle_bf16 *q,
                          const peagle_bf16 *k, const peagle_bf16 *v, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                          const float *rope_cos, const float *rope_sin, int32_t rope_max_pos,
                          float *out, float *lse, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * The two halves of peagle_draft_attn_fwd, same arguments, for callers that time them
 * apart: _prepare rotates q and k by position value into the workspace (RoPE), lays
 * the depth-0 v out in attention tiles and builds the anchor-major row list; _core runs
 * the attention itself from that workspace, which must hold what a _prepare call with
 * the same arguments wrote (stream order suffices).
 */
int peagle_draft_attn_prepare(int64_t n, int32_t K, int64_t T, const int32_t *idx,
                              const int32_t *depth_off, const int32_t *row_of,
                              const int32_t *cu_seqlens, int32_t num_seqs,
                              const peagle_bf16 *q, const peagle_bf16 *k, const peagle_bf16 *v,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              float softmax_scale, const float *rope_cos, const float *rope_sin,
                              int32_t rope_max_pos, float *out, float *lse, void *workspace,
                              size_t workspace_bytes, void *stream);
int peagle_draft_attn_core(int64_t n, int32_t K, int64_t T, const int32_t *idx,
                           const int32_t *depth_off, const int32_t *row_of,
                           const int32_t *cu_seqlens, int32_t num_seqs, const peagle_bf16 *q,
                           const peagle_bf16 *k, const peagle_bf16 *v, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                           const float *rope_cos, const float *rope_sin, int32_t rope_max_pos,
                           float *out, float *lse, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * peagle_draft_attn_bwd -- gradients of peagle_draft_attn_fwd [N, description: the
 * P-EAGLE trainer backpropagates its masked-depth loss through the same cache_hidden
 * attention]. Same layout arguments as the forward, plus its results and dL/d out:
 *   out, lse         fp32[T, Hq, D], fp32[Hq, T]  from peagle_draft_attn_fwd on the same
 *                    inputs (lse required)
 *   dout             fp32[T, Hq, D]   dL/d out
 *   dq               fp32[T, Hq, D]   out  dL/dq  (pre-RoPE q)
 *   dk, dv           fp32[T, Hkv, D]  out  dL/dk, dL/dv (pre-RoPE k)
 *   workspace        >= peagle_draft_attn_bwd_workspace_bytes(n, T, Hq, Hkv, D), 256-byte
 *                    aligned; the forward's preparation is redone at its head
 * With P the masked softmax: dV = P^T dO, dS = P * (dO V^T - rowsum(dO * O)),
 * dq' = scale dS k', dk' = scale dS^T q', summed over the q heads of each kv head, and
 * dq, dk rotated back from the RoPE frame. Products on bf16 MFMA (q', k', v, dO, P and dS
 * rounded to bf16) with fp32 accumulation; the diagonal-extension keys' dk, dv in fp32.
 * Every element of dq, dk and dv is written. Shapes as for the forward.
 */
size_t peagle_draft_attn_bwd_workspace_bytes(int64_t n, int64_t T, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim);
int peagle_draft_attn_bwd(int64_t n, int32_t K, int64_t T, const int32_t *idx,
                          const int32_t *depth_off, const int32_t *row_of,
                          const int32_t *cu_seqlens, int32_t num_seqs, const peagle_bf16 *q,
                          const peagle_bf16 *k, const peagle_bf16 *v, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                          const float *rope_cos, const float *rope_sin, int32_t rope_max_pos,
                          const float *out, const float *lse, const float *dout, float *dq,
                          float *dk, float *dv, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * peagle_depth_ce -- depth-weighted cross-entropy of the draft rows and its gradient
 * [N, description: the parallel masked-depth loss with the 0.8**d weighted-mean schedule
 * and the draft-vocab projection; validation: starting loss ~ ln(draft vocab);
 * out-of-draft-vocab masking]. Per depth d, L_d = mean over the depth's rows whose label
 * lies in [0, V) of lse(logits) - logits[label]; the loss is
 * sum_d decay^d L_d / sum_d decay^d over the depths with at least one such row.
 *   depth_off   int32[K+1]   (device) first row of each depth, depth_off[K] = T
 *   logits      bf16[T, V]   draft-vocab logits of the draft rows
 *   labels      int32[T]     draft-vocab id each row should predict; -1 (or any id outside
 *                            [0, V)) masks the row
 *   decay       in (0, 1]    0.8 in the pages' schedule
 *   loss_out    fp32[1] out
 *   depth_loss  fp32[K] out or NULL; NaN for a depth with no unmasked row
 *   dlogits     bf16[T, V] out or NULL: d loss / d logits (zero rows where masked)
 *   workspace   >= peagle_depth_ce_workspace_bytes(T, K), 256-byte aligned
 * Row statistics in fp32, the reductions over rows in fp64 in a fixed order: the same
 * inputs give the same loss bit for bit.
 */
size_t peagle_depth_ce_workspace_bytes(int64_t T, int32_t K);
int peagle_depth_ce(int64_t T, int32_t K, int32_t vocab, const int32_t *depth_off,
                    const peagle_bf16 *logits, const int32_t *labels, float decay,
                    float *loss_out, float *depth_loss, peagle_bf16 *dlogits, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * peagle_accept_prefix -- greedy verification [G, "Inference Process"]: the target
 * checks every draft token in one pass and the longest correct prefix is accepted.
 *   draft_logits, target_logits  bf16[N, K, V]; row [i, d] of target_logits scores the
 *                                token that draft depth d proposes; shared vocabulary
 *   draft_tok, target_tok        int32[N, K] out  argmax per row (lowest index on ties)
 *   accept_len                   int32[N]    out  leading d with draft_tok == target_tok
 * 1 <= K <= PEAGLE_MAX_DEPTHS, V >= 1. NaN logits give unspecified tokens.
 */
int peagle_accept_prefix(int32_t num_drafts, int32_t K, int32_t vocab,
                         const peagle_bf16 *draft_logits, const peagle_bf16 *target_logits,
                         int32_t *draft_tok, int32_t *target_tok, int32_t *accept_len,
                         void *stream);

/*
 * peagle_accept_prefix_d2t -- greedy verification with a draft vocabulary smaller than the
 * target's [N: draft vocabulary 8192 in the validation run; out-of-draft-vocab masking]:
 * the draft head scores Vd draft ids, d2t[draft id] is the id in the target's vocabulary,
 * and a draft token is correct iff d2t[its argmax] equals the target's argmax over Vt. A
 * target argmax outside d2t's image never matches.
 *   draft_logits   bf16[N, K, Vd];  target_logits bf16[N, K, Vt]
 *   d2t            int32[Vd]   (device; values are only compared, never used as addresses)
 *   draft_tok      int32[N, K] out  draft ids (lowest index on ties)
 *   target_tok     int32[N, K] out  target ids
 *   accept_len     int32[N]    out
 */
int peagle_accept_prefix_d2t(int32_t num_drafts, int32_t K, int32_t draft_vocab,
                             int32_t target_vocab, const peagle_bf16 *draft_logits,
                             const peagle_bf16 *target_logits, const int32_t *d2t,
                             int32_t *draft_tok, int32_t *target_tok, int32_t *accept_len,
                             void *stream);

/*
 * peagle_accept_sampled -- verification of sampled drafts [R, "How Speculative Decoding
 * Works", step 6: accepted draft tokens are kept, a rejected one is resampled], read as
 * speculative sampling. At depth d, p = softmax(target_logits[i, d] / tau) and
 * q = softmax(draft_logits[i, d] / tau); the drafter's token x_d is accepted while
 * u[i, d] * q(x_d) < p(x_d) (u < p / q), and accept_len[i] is the number of leading
 * accepted depths. At the first rejected depth L the next token is drawn from the
 * residual r = max(0, p - q): the smallest t whose running sum r_0 + .. + r_t exceeds
 * w[i] * (r_0 + .. + r_{V-1}). With all K accepted, next_tok[i] = -1.
 *   draft_logits, target_logits  bf16[N, K, V]  shared vocabulary
 *   draft_tok     int32[N, K]   the drafter's sampled tokens; one outside [0, V) is
 *                               rejected
 *   u             fp32[N, K]    uniforms in [0, 1), one per depth (acceptance)
 *   w             fp32[N]       uniforms in [0, 1), one per draft (the residual draw)
 *   temperature   tau > 0 (host)
 *   accept_len    int32[N] out
 *   next_tok      int32[N] out  the resampled token, or -1
 * Arithmetic is fp32: a decision whose float64 margin (|u q - p|, or the distance of
 * w * Z to a boundary of the running sum) is below fp32 rounding may differ from a
 * float64 evaluation; the resampled token always has positive fp32 residual weight.
 * 1 <= K <= PEAGLE_MAX_DEPTHS, V >= 1; with num_drafts = 0 nothing is read and the
 * pointers may be NULL.
 */
int peagle_accept_sampled(int32_t num_drafts, int32_t K, int32_t vocab,
                          const peagle_bf16 *draft_logits, const peagle_bf16 *target_logits,
                          const int32_t *draft_tok, const float *u, const float *w,
                          float temperature, int32_t *accept_len, int32_t *next_tok,
                          void *stream);

/*
 * peagle_accept_sampled_bonus -- peagle_accept_sampled with the bonus token [R, "How
 * Speculative Decoding Works": the target verifies every drafted token in one pass, which
 * also gives its distribution after the last one]. target_logits holds K + 1 rows per
 * draft, bf16[N, K + 1, V]: rows 0 .. K-1 verify the K depths as in peagle_accept_sampled;
 * when all K are accepted, next_tok[i] is drawn from p_K = softmax(target row K / tau): the
 * smallest t whose running sum p_0 + .. + p_t exceeds w[i] * (p_0 + .. + p_{V-1}). Every
 * draft thus yields accept_len[i] + 1 tokens and next_tok is never -1. Other arguments,
 * arithmetic and limits as for peagle_accept_sampled.
 */
int peagle_accept_sampled_bonus(int32_t num_drafts, int32_t K, int32_t vocab,
                                const peagle_bf16 *draft_logits, const peagle_bf16 *target_logits,
                                const int32_t *draft_tok, const float *u, const float *w,
                                float temperature, int32_t *accept_len, int32_t *next_tok,
                                void *stream);

/*
 * The first draft decoder layer's attention inputs [R, "How Speculative Decoding Works",
 * step 3: the drafter input concatenates embeddings and hidden states; G, "Architecture":
 * Llama-style decoder layers; N, changelog: depths >= 1 take the ptd token and the
 * projected mask_hidden]. For every draft row:
 *   x = [rms(embed) * w_norm_emb, rms(hidden) * w_norm_hidden]   (width 2H, embedding first;
 *        rms(y) = y / sqrt(mean(y^2) + eps))
 *   [q | k | v] = x W_qkv^T                                      (bias-free)
 * All depth >= 1 rows share x, so the projection runs on rows 0 .. n (row n = the first
 * depth-1 row) and rows n+1 .. T-1 receive row n's q, k and v.
 *   hidden         fp32[T, H]  from peagle_fuse_inputs (hidden_out); rows 0 .. n are read
 *   embed          bf16[T, H]  from peagle_fuse_inputs (embed_out); rows 0 .. n are read
 *   w_norm_emb, w_norm_hidden  bf16[H]
 *   eps            > 0 (Llama: 1e-6)
 *   w_qkv          bf16[(Hq + 2 Hkv) D, 2H]  the q, k and v projections stacked by output
 *                  row (linear-layer layout)
 *   q              bf16[T, Hq, D]   out, pre-RoPE (the input of peagle_draft_attn_*)
 *   k, v           bf16[T, Hkv, D]  out
 *   workspace      >= peagle_layer1_qkv_workspace_bytes(n, T, H) bytes, 256-byte aligned
 * H a multiple of 32 and head_dim a multiple of 8 (else PEAGLE_ERR_UNSUPPORTED);
 * Hq % Hkv == 0. The projection runs as bf16 MFMA with fp32 accumulation on the
 * normalised rows rounded to bf16.
 */
size_t peagle_layer1_qkv_workspace_bytes(int64_t n, int64_t T, int32_t H);
int peagle_layer1_qkv(int64_t n, int32_t K, int64_t T, const float *hidden,
                      const peagle_bf16 *embed, int32_t H, const peagle_bf16 *w_norm_emb,
                      const peagle_bf16 *w_norm_hidden, float eps, const peagle_bf16 *w_qkv,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      peagle_bf16 *q, peagle_bf16 *k, peagle_bf16 *v, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * The rest of the first draft layer [G, "Architecture": Llama-style decoder layers; G,
 * "Key Parameters": normalization before the residual connection unless disabled].
 * Per draft row, with o the attention output (heads flattened, width QW = Hq D):
 *   r  = norm_before_residual ? rms(hidden) * w_norm_hidden : hidden
 *   h1 = r + o W_o^T
 *   h2 = h1 + W_down (silu(W_gate m) * (W_up m)),  m = rms(h1) * w_post
 *   attn_out       fp32[T, QW]        from peagle_draft_attn_fwd (out)
 *   hidden         fp32[T, H]         from peagle_fuse_inputs (hidden_out)
 *   w_norm_hidden  bf16[H]            as for peagle_layer1_qkv (read if norm_before_residual)
 *   w_o            bf16[H, QW];  w_post bf16[H]
 *   w_gate, w_up   bf16[I, H];   w_down bf16[H, I]
 *   h2_out         fp32[T, H]   out
 *   workspace      >= peagle_layer1_post_workspace_bytes(n, T, H, QW, I), 256-byte aligned
 * H, QW and I multiples of 64 (else PEAGLE_ERR_UNSUPPORTED). Every product is a bf16 MFMA
 * GEMM with fp32 accumulation on operands rounded to bf16; h1 and h2 stay fp32.
 */
size_t peagle_layer1_post_workspace_bytes(int64_t n, int64_t T, int32_t H, int32_t QW,
                                          int32_t I);
int peagle_layer1_post(int64_t n, int32_t K, int64_t T, const float *attn_out, int32_t QW,
                       const float *hidden, int32_t H, const peagle_bf16 *w_norm_hidden,
                       int32_t norm_before_residual, const peagle_bf16 *w_o,
                       const peagle_bf16 *w_post, const peagle_bf16 *w_gate,
                       const peagle_bf16 *w_up, int32_t I, const peagle_bf16 *w_down, float eps,
                       float *h2_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Stacked draft layers (the 2nd and later) [G, "Key Parameters": the number of decoder
 * layers is a parameter; G, "Architecture": Llama-style decoder layers]. The residual
 * stream h is the previous layer's output (h2_out); there is no concatenation and no
 * separate embedding input. Per draft row:
 *   x = rms(h) * w_norm;  [q | k | v] = x W_qkv^T                  (peagle_layer_qkv)
 *   h1 = h + o W_o^T;  h2 = h1 + W_down (silu(W_gate m) * (W_up m)),
 *   m = rms(h1) * w_post                                           (peagle_layer_post)
 * with o this layer's attention output from peagle_draft_attn_fwd on its q, k, v (the
 * same rows, positions and predicate as the first layer).
 *   h              fp32[T, H]
 *   w_norm, w_post bf16[H];  w_qkv bf16[(Hq + 2 Hkv) D, H];  w_o bf16[H, QW]
 *   w_gate, w_up   bf16[I, H];  w_down bf16[H, I]
 *   q              bf16[T, Hq, D] out;  k, v bf16[T, Hkv, D] out  (before RoPE)
 *   attn_out       fp32[T, QW];  h2_out fp32[T, H] out (may be h itself: h is consumed by
 *                  the first product, h2_out written by the last, in stream order)
 *   workspace      >= the matching *_workspace_bytes, 256-byte aligned
 * H, QW and I multiples of 64 and D a multiple of 8 (else PEAGLE_ERR_UNSUPPORTED).
 * Products are bf16 MFMA GEMMs with fp32 accumulation on operands rounded to bf16.
 */
size_t peagle_layer_qkv_workspace_bytes(int64_t T, int32_t H);
int peagle_layer_qkv(int64_t T, const float *h, int32_t H, const peagle_bf16 *w_norm, float eps,
                     const peagle_bf16 *w_qkv, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, peagle_bf16 *q, peagle_bf16 *k, peagle_bf16 *v,
                     void *workspace, size_t workspace_bytes, void *stream);
size_t peagle_layer_post_workspace_bytes(int64_t T, int32_t H, int32_t QW, int32_t I);
int peagle_layer_post(int64_t T, const float *attn_out, int32_t QW, const float *h, int32_t H,
                      const peagle_bf16 *w_o, const peagle_bf16 *w_post,
                      const peagle_bf16 *w_gate, const peagle_bf16 *w_up, int32_t I,
                      const peagle_bf16 *w_down, float eps, float *h2_out, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * peagle_draft_head -- the draft-vocab head and its argmax [N, description: the P-EAGLE
 * trainer shares EAGLE-3's draft-vocab projection]:
 *   token[r] = argmax_v (rms(h[r]) * w_final) . w_head[v]   (lowest v on ties)
 *   h        fp32[T, H]   (e.g. h2_out of peagle_layer1_post)
 *   w_final  bf16[H];  w_head bf16[V, H]
 *   tokens   int32[T]   out
 *   workspace >= peagle_draft_head_workspace_bytes(T, H, V), 256-byte aligned
 * The logits are reduced inside the projection (per row and 64 columns) and never stored.
 * H a multiple of 64 (else PEAGLE_ERR_UNSUPPORTED); V >= 1. The argmax is taken on fp32
 * logits of bf16 operands: rows whose top two logits are closer than that rounding may
 * pick either.
 */
size_t peagle_draft_head_workspace_bytes(int64_t T, int32_t H, int32_t V);
int peagle_draft_head(int64_t T, const float *h, int32_t H, const peagle_bf16 *w_final,
                      const peagle_bf16 *w_head, int32_t V, float eps, int32_t *tokens,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Draft attention at inference (the decode shape) [N, parity section: at inference one
 * flat parallel forward over [context, mask_1, ..., mask_{K-1}]; G, "Inference Process":
 * all depths drafted in one pass, drafting repeats from the last accepted token].
 *
 * Request b (of B) has L_b = cu_ctx[b+1] - cu_ctx[b] context tokens in the KV cache and
 * K new rows: row d sits at position L_b + d (d = 0 the anchor, the last accepted token;
 * d >= 1 the mask rows). Row d attends to every cache key of its request and to new rows
 * 0 .. d, i.e. causal attention over the flat sequence: the forward's predicate with a
 * single anchor. Cache keys are stored already rotated at their positions 0 .. L_b - 1.
 *
 * The V cache is kept in attention tiles, one tile per 32 keys of a request:
 *   v_tiles  bf16[Hkv][ntiles][D][32], ntiles = floor(total_ctx / 32) + B + 1;
 *            tile floor(cu_ctx[b] / 32) + b + j of a kv head holds keys 32j .. 32j + 31
 *            of request b transposed (dim-major), zero past L_b, the keys of each group
 *            of 16 stored in the order 0-3, 8-11, 4-7, 12-15.
 * peagle_decode_pack_v writes that layout from a natural V cache.
 */

/* Bytes of the V tile layout for a cache of total_ctx keys over num_reqs requests. */
size_t peagle_decode_v_tiles_bytes(int64_t total_ctx, int32_t num_reqs, int32_t num_kv_heads,
                                   int32_t head_dim);

/*
 * peagle_decode_pack_v -- V cache (natural layout) -> V tiles.
 *   cu_ctx     int32[B+1]  request starts in the cache, 0 = cu[0] <= ... <= cu[B] = total_ctx
 *   max_ctx    (host) >= every L_b; bounds the launch
 *   v_cache    bf16[total_ctx, Hkv, D]
 *   v_tiles    bf16, v_tiles_bytes >= peagle_decode_v_tiles_bytes(...)   out
 * Tiles of a request are written in full (zero padded); the spare tiles between
 * requests are left untouched. head_dim in {64, 128, 256}; 1 <= B <= 65535.
 */
int peagle_decode_pack_v(int32_t num_reqs, const int32_t *cu_ctx, int64_t total_ctx,
                         int32_t max_ctx, const peagle_bf16 *v_cache, int32_t num_kv_heads,
                         int32_t head_dim, peagle_bf16 *v_tiles, size_t v_tiles_bytes,
                         void *stream);

/* Bytes of workspace peagle_draft_decode_attn needs for these sizes (0 on bad arguments). */
size_t peagle_draft_decode_workspace_bytes(int32_t num_reqs, int32_t K, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int64_t total_ctx, int32_t max_ctx);

/*
 * peagle_draft_decode_attn -- the decode-shaped draft attention. Split-KV: the cache
 * tiles of all requests are cut into equal ranges, one workgroup per CU, and a last
 * kernel merges the partial softmax states a range leaves for each request it touches
 * (three launches, all enqueued on `stream`; nothing is allocated or synchronized).
 *   cu_ctx         int32[B+1]          as for peagle_decode_pack_v
 *   total_ctx      (host) cu_ctx[B];   max_ctx (host) >= every L_b
 *   k_cache        bf16[total_ctx, Hkv, D]   rotated keys
 *   v_tiles        from peagle_decode_pack_v (same cu_ctx)
 *   q              bf16[B, K, Hq, D]   pre-RoPE
 *   k, v           bf16[B, K, Hkv, D]  pre-RoPE k of the new rows; v
 *   softmax_scale  usually 1/sqrt(D)
 *   rope_cos/sin   fp32[rope_max_pos+1, D/2] from peagle_rope_table;
 *                  rope_max_pos >= max_ctx + K - 1
 *   out            fp32[B, K, Hq, D]   out
 *   lse            fp32[B, K, Hq]      out, natural-log softmax denominators; may be NULL
 *   workspace      >= peagle_draft_decode_workspace_bytes(B, K, Hq, Hkv, D, total_ctx,
 *                  max_ctx)
 *                  bytes, 256-byte aligned scratch
 * head_dim in {64, 128, 256}; Hq % Hkv == 0; 1 <= K <= 32; 1 <= B <= 65535.
 * total_ctx = 0 (every request empty) is allowed; k_cache and v_tiles may then be NULL.
 */
int peagle_draft_decode_attn(int32_t num_reqs, int32_t K, const int32_t *cu_ctx,
                             int64_t total_ctx, int32_t max_ctx, const peagle_bf16 *k_cache,
                             const peagle_bf16 *v_tiles, size_t v_tiles_bytes,
                             const peagle_bf16 *q, const peagle_bf16 *k, const peagle_bf16 *v,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             float softmax_scale, const float *rope_cos, const float *rope_sin,
                             int32_t rope_max_pos, float *out, float *lse, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * The decode loop over a cache that grows in place [G, "Inference Process": drafting
 * repeats from the last accepted token]: each request owns a capacity in the cache and
 * a current length inside it, and after verification the newly committed tokens' keys
 * and values are appended where they belong instead of repacking the cache.
 *   cu_cap      int32[B+1]  (device) starts and capacities: request b owns cache rows
 *                           [cu_cap[b], cu_cap[b+1]) and V tiles laid out as for
 *                           peagle_decode_pack_v over those capacities
 *   lens        int32[B]    (device) current context lengths, 0 <= lens[b] <= capacity
 *   total_cap = cu_cap[B];  max_cap >= every capacity (it bounds the work split)
 * peagle_decode_pack_v_lens: V tiles of the first lens[b] rows of each request, zeros in
 *   the rest of each capacity (appended rows and masked slots then never meet stale data).
 * peagle_draft_decode_attn_lens: peagle_draft_decode_attn with L_b = lens[b]; the new rows
 *   sit at positions lens[b] + d. rope_max_pos >= max_cap + K - 1.
 * peagle_decode_append: request b takes m_b = n_new[b] + n_add new rows (rows 0 .. m_b - 1
 *   of k_new, v_new bf16[B, max_new, Hkv, D], pre-RoPE) at positions lens_in[b] + j: keys
 *   rotated at those positions into k_cache, values into their V-tile slots. Rows past the
 *   capacity are dropped. lens_out[b] = min(lens_in[b] + m_b, capacity) (lens_out and
 *   lens_in distinct). With n_new = accept_len from verification and n_add = 1, the
 *   accepted drafts and the next anchor join the context. rope_max_pos >= max_cap - 1.
 */
int peagle_decode_pack_v_lens(int32_t num_reqs, const int32_t *cu_cap, const int32_t *lens,
                              int64_t total_cap, int32_t max_cap, const peagle_bf16 *v_cache,
                              int32_t num_kv_heads, int32_t head_dim, peagle_bf16 *v_tiles,
                              size_t v_tiles_bytes, void *stream);
int peagle_draft_decode_attn_lens(int32_t num_reqs, int32_t K, const int32_t *cu_cap,
                                  const int32_t *lens, int64_t total_cap, int32_t max_cap,
                                  const peagle_bf16 *k_cache, const peagle_bf16 *v_tiles,
                                  size_t v_tiles_bytes, const peagle_bf16 *q,
                                  const peagle_bf16 *k, const peagle_bf16 *v,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  float softmax_scale, const float *rope_cos,
                                  const float *rope_sin, int32_t rope_max_pos, float *out,
                                  float *lse, void *workspace, size_t workspace_bytes,
                                  void *stream);
int peagle_decode_append(int32_t num_reqs, const int32_t *cu_cap, const int32_t *lens_in,
                         const int32_t *n_new, int32_t n_add, int32_t max_new,
                         const peagle_bf16 *k_new, const peagle_bf16 *v_new,
                         int32_t num_kv_heads, int32_t head_dim, const float *rope_cos,
                         const float *rope_sin, int32_t rope_max_pos, int64_t total_cap,
                         int32_t max_cap, peagle_bf16 *k_cache, peagle_bf16 *v_tiles,
                         size_t v_tiles_bytes, int32_t *lens_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PEAGLE_H_ */
