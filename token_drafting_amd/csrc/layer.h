// Host-side launchers of the draft decoder layers and the draft-vocab head. Internal to
// libpeagle: arguments are validated by the C entry points before they run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace peagle {

struct Layer1Args {
  int32_t n, K, T, H, Hq, Hkv, D;
  float eps;
};

// Workspace: the normalised, concatenated rows 0 .. n (bf16, 2H wide).
size_t layer1_workspace_bytes(int64_t n, int64_t T, int32_t H);

hipError_t launch_layer1_qkv(const Layer1Args& a, const float* hidden, const uint16_t* embed,
                             const uint16_t* w_emb, const uint16_t* w_hid, const uint16_t* w_qkv,
                             uint16_t* q, uint16_t* k, uint16_t* v, char* ws, hipStream_t stream);

// Second half of the first layer: output projection and residual, RMSNorm, SwiGLU MLP and
// residual. QW = Hq * D (width of the attention output), I = intermediate size.
struct Layer1PostArgs {
  int32_t n, T, H, QW, I, norm_before_residual;
  float eps;
};
size_t layer1_post_workspace_bytes(int64_t n, int64_t T, int32_t H, int32_t QW, int32_t I);
hipError_t launch_layer1_post(const Layer1PostArgs& a, const float* attn, const float* hidden,
                              const uint16_t* w_hid, const uint16_t* w_o, const uint16_t* w_post,
                              const uint16_t* w_gate, const uint16_t* w_up,
                              const uint16_t* w_down, float* h2, char* ws, hipStream_t stream);

// Attention inputs of a stacked layer (2nd and later): one RMSNorm of the fp32 residual
// stream, then the QKV projection of every draft row (rows no longer coincide).
struct LayerArgs {
  int32_t T, H, Hq, Hkv, D;
  float eps;
};
// Workspace: the normalised rows (bf16, H wide).
size_t layer_qkv_workspace_bytes(int64_t T, int32_t H);
hipError_t launch_layer_qkv(const LayerArgs& a, const float* h, const uint16_t* w_norm,
                            const uint16_t* w_qkv, uint16_t* q, uint16_t* k, uint16_t* v,
                            char* ws, hipStream_t stream);

// y = bf16(rms(x) * w) for fp32 rows x [rows, H] (H % 8 == 0).
hipError_t launch_rms_rows(const float* x, const uint16_t* w, uint16_t* y, int32_t rows,
                           int32_t H, float eps, hipStream_t stream);

// Draft-vocab head: final RMSNorm, projection to V logits, argmax per row (fused).
size_t draft_head_workspace_bytes(int64_t T, int32_t H, int32_t V);
hipError_t launch_draft_head(int64_t T, int32_t H, int32_t V, float eps, const float* h,
                             const uint16_t* w_final, const uint16_t* w_head, int32_t* tokens,
                             char* ws, hipStream_t stream);

}  // namespace peagle
