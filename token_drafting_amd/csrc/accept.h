// Host-side launcher of the verification with a draft vocabulary smaller than the
// target's. Internal to libpeagle: arguments are validated by the C entry point.
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

}  // namespace peagle
