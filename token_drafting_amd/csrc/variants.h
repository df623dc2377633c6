// Host-side launchers of the variants of the path: verification with a draft vocabulary
// smaller than the target's, the RMSNorm after fc, verification of sampled drafts, and
// the decode attention over a cache that grows in place. Internal to libpeagle: arguments
// are validated by the C entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace peagle {

// Draft rows of Vd logits, target rows of Vt; d2t[draft id] = target id (nullptr: the
// identity, Vd == Vt).
hipError_t launch_accept_map(int32_t N, int32_t K, int32_t Vd, int32_t Vt,
                             const uint16_t* draft, const uint16_t* target, const int32_t* d2t,
                             int32_t* draft_tok, int32_t* target_tok, int32_t* accept_len,
                             hipStream_t stream);

// In-place RMSNorm (fp32 rows, bf16 weight) of rows [0, rows) of x [rows, H].
hipError_t launch_rms_inplace(float* x, const uint16_t* w, int64_t rows, int32_t H, float eps,
                              hipStream_t stream);

// Speculative-sampling acceptance: accept_len[i] and the resampled next_tok[i] (-1 when all
// K depths are accepted); temperature > 0.
hipError_t launch_accept_sampled(int32_t N, int32_t K, int32_t V, const uint16_t* draft,
                                 const uint16_t* target, const int32_t* draft_tok,
                                 const float* u, const float* w, float temperature, bool bonus,
                                 int32_t* accept_len, int32_t* next_tok, hipStream_t stream);

// Decode over a cache with per-request capacities (cu: starts and capacities) and current
// lengths lens (null: every request fills its capacity, the packed layout).
hipError_t launch_decode_pack_v_lens(const int32_t* cu, const int32_t* lens, int32_t B,
                                     int64_t total_ctx, int32_t max_ctx, const uint16_t* v,
                                     int32_t Hkv, int32_t D, uint16_t* vt, hipStream_t stream);
hipError_t launch_decode_attn_lens(const DecodeArgs& a, const int32_t* cu, const int32_t* lens,
                                   const uint16_t* kc, const uint16_t* vt, const uint16_t* qn,
                                   const uint16_t* kn, const uint16_t* vn, const float* cs,
                                   const float* sn, float* out, float* lse, char* ws,
                                   hipStream_t stream);
// Append n_new[b] + n_add rows per request (pre-RoPE k, v [B, max_new, Hkv, D]) at the end of
// each request's context; lens_out = the new lengths (lens_in and lens_out distinct).
hipError_t launch_decode_append(const int32_t* cu, const int32_t* lens_in, const int32_t* n_new,
                                int32_t n_add, int32_t max_new, const uint16_t* k_new,
                                const uint16_t* v_new, const float* cs, const float* sn,
                                int32_t max_pos, uint16_t* kc, uint16_t* vt, int32_t* lens_out,
                                int32_t B, int32_t Hkv, int32_t D, int32_t max_ctx,
                                int64_t total_ctx, hipStream_t stream);

}  // namespace peagle
