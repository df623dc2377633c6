// Host-side launchers of the variants of the path: verification with a draft vocabulary
// smaller than the target's, the RMSNorm after fc, and verification of sampled drafts. Internal to libpeagle: arguments
// are validated by the C entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
                                 const float* u, const float* w, float temperature,
                                 int32_t* accept_len, int32_t* next_tok, hipStream_t stream);

}  // namespace peagle
