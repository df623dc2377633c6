// Host-side launchers of the P-EAGLE draft-forward kernels. Internal to libpeagle:
// arguments are validated by the C entry points before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace peagle {

constexpr int kMaxDepths = 64;

struct CodArgs {
  int32_t n, K, S;
  uint64_t seed;
  int32_t m[kMaxDepths];
  int32_t off[kMaxDepths + 1];
};

size_t cod_workspace_bytes(int64_t n, int32_t K);
// Size of the static device scratch used by the allocation-free COD entry point.
constexpr size_t kCodNoAllocScratchBytes = (size_t)1 << 20;
hipError_t cod_noalloc_scratch(void** ptr);
hipError_t launch_cod_select(const CodArgs& a, const int32_t* cu_seqlens, int32_t* idx,
                             int32_t* depth_off, int32_t* cu_seqlens_d, int32_t* row_of,
                             void* workspace, hipStream_t stream);

struct FuseArgs {
  int32_t n, T, aux_dim, H, vocab, ptd;
};

hipError_t launch_fuse(const FuseArgs& a, const int32_t* idx, const uint16_t* aux,
                       const uint16_t* fc_weight, const uint16_t* mask_hidden,
                       const int32_t* tokens, const uint16_t* embed, float* hidden_out,
                       uint16_t* embed_out, hipStream_t stream);

hipError_t launch_rope_table(int32_t head_dim, double theta, int32_t max_pos, float* cos_out,
                             float* sin_out, hipStream_t stream);

// Workspace of the draft attention, carved from one caller-provided buffer.
struct AttnLayout {
  size_t qinfo, qstart, qrot, krot, krot_lo, vt, chunks, cmeta, nchunks, seq_chunk, flags,
      blocksum, segs, items, nitems, part, ml, total;
  int max_chunks;
};
AttnLayout attn_layout(int64_t n, int64_t T, int32_t Hq, int32_t Hkv, int32_t D);
int attn_max_chunks(int64_t n, int64_t T, int32_t Hq, int32_t Hkv);

// Key-range split of the attention's main kernel, for grids that would not fill the chip:
// a chunk's context tiles are cut into at most nsplit segments, each run by its own
// workgroup (the segment length is chosen on the device from the chunks' spans); a merge
// kernel combines their partial softmax states. nsplit = 1 when there are enough chunks.
constexpr int kMaxAttnSplit = 4;
struct AttnSplit {
  int nsplit;
};
AttnSplit attn_split_plan(int64_t n, int64_t T, int32_t Hq, int32_t Hkv);

// Query slots (rows x q heads of one kv head) per attention workgroup: a chunk holds
// kAttnSlots / G consecutive rows of the anchor-major list.
constexpr int kAttnSlots = 256;

// Attention chunks whose context span is at most this many keys (the first anchors of
// each sequence) run the exact-split variant; the RoPE kernel stores k_lo for the rows
// of those anchors.
constexpr int kShortSpan = 96;
// Chunks per sequence that can be short: their rows belong to the first kShortSpan
// anchors, which own at most kShortSpan * K list entries.
inline int attn_exact_chunks_per_seq(int K, int QR) { return (kShortSpan * K + QR - 1) / QR; }

struct AttnArgs {
  int32_t n, K, T, S, Hq, Hkv, D, max_pos;
  float scale;
};

hipError_t launch_attn_prepare(const AttnArgs& a, const int32_t* idx, const int32_t* depth_off,
                               const int32_t* row_of, const int32_t* cu_seqlens,
                               const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const float* rope_cos, const float* rope_sin, char* ws,
                               hipStream_t stream);

hipError_t launch_attn_core(const AttnArgs& a, const uint16_t* v, float* out, float* lse,
                            const char* ws, hipStream_t stream);

hipError_t launch_accept(int32_t N, int32_t K, int32_t V, const uint16_t* draft,
                         const uint16_t* target, int32_t* draft_tok, int32_t* target_tok,
                         int32_t* accept_len, hipStream_t stream);

// Draft attention at inference: K new rows per request over a KV cache.
struct DecodeArgs {
  int32_t B, K, Hq, Hkv, D, max_ctx, max_pos;
  int64_t total_ctx;
  float scale;
};
// Split of the decode attention: a wave holds ncw groups of 16 query columns (pc = 16 ncw
// columns); ncg column groups per kv head; heads kv heads per workgroup, so wg_per_range
// workgroups per range of tile slots; up to max_ranges ranges, and nslots = max_ranges + B
// partial slots per (kv head, column group).
struct DecodePlan {
  int ncw, pc, ncg, heads, wg_per_range, max_ranges, nslots;
};
DecodePlan decode_plan(int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D,
                       int64_t total_ctx, int32_t max_ctx);
size_t decode_workspace_bytes(int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D,
                              int64_t total_ctx, int32_t max_ctx);
// Compute units of the current device (cached per device; 256 if the runtime cannot say).
int device_cus();
// V tiles per kv head of a cache of total_ctx keys over B requests.
int64_t decode_ntiles(int64_t total_ctx, int32_t B);

hipError_t launch_decode_pack_v(const int32_t* cu, int32_t B, int64_t total_ctx, int32_t max_ctx,
                                const uint16_t* v, int32_t Hkv, int32_t D, uint16_t* vt,
                                hipStream_t stream);
hipError_t launch_decode_attn(const DecodeArgs& a, const int32_t* cu, const uint16_t* kc,
                              const uint16_t* vt, const uint16_t* qn, const uint16_t* kn,
                              const uint16_t* vn, const float* cs, const float* sn, float* out,
                              float* lse, char* ws, hipStream_t stream);

}  // namespace peagle
