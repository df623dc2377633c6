// Host-side launcher of the first draft layer's attention inputs. Internal to libpeagle:
// arguments are validated by the C entry point before it runs.
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

}  // namespace peagle
