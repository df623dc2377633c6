// Host-side launchers of the training side: the draft attention backward and the
// depth-weighted cross-entropy. Internal to libpeagle: arguments are validated by the C
// entry points; the backward's runs the forward's preparation (rotated q and k,
// anchor-major row list, chunk table) into the head of the same workspace first.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kernels.h"

namespace peagle {

// Query slots of one kv head (draft rows of the anchor-major list x its G q heads) are cut
// into tiles of this many slots for the key-major pass.
constexpr int kBwdSlots = 32;
// Depth-0 keys per workgroup of the key-major pass (8 waves of 16).
constexpr int kBwdKeys = 128;

// The backward's own workspace regions, after the forward's (offsets from the start).
struct AttnBwdLayout {
  size_t fwd, dob, dlt, vpad, qtr, dtr, smeta, part, total;
  int64_t ntq;   // query tiles per kv head
  int seg_len;   // query tiles per segment of the key-major pass
  int nseg;      // segments of the tile list
};
AttnBwdLayout attn_bwd_layout(int64_t n, int64_t T, int32_t Hq, int32_t Hkv, int32_t D);

hipError_t launch_attn_bwd(const AttnArgs& a, const int32_t* idx, const int32_t* depth_off,
                           const int32_t* cu_seqlens, const uint16_t* v, const float* out,
                           const float* lse, const float* dout, const float* rope_cos,
                           const float* rope_sin, float* dq, float* dk, float* dv, char* ws,
                           hipStream_t stream);

// Depth-weighted cross-entropy: workspace holds the per-row losses (fp32 [T]) and the
// per-depth counts of unmasked rows (int32 [K]).
size_t depth_ce_workspace_bytes(int64_t T, int32_t K);
hipError_t launch_depth_ce(int64_t T, int32_t K, int32_t V, const int32_t* depth_off,
                           const uint16_t* logits, const int32_t* labels, float decay,
                           float* loss_out, float* depth_loss, uint16_t* dlogits, char* ws,
                           hipStream_t stream);

}  // namespace peagle
