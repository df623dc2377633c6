// Host-side robustness driver for the C entry points' argument validation, built with
// AddressSanitizer and UndefinedBehaviorSanitizer around abi.cpp (see test_host_sanitizers.py).
//
// Every call below passes NULL for every pointer argument, with sizes drawn from a mix of
// valid, boundary and hostile values (0, negatives, INT32/INT64 extremes, powers of two +- 1,
// NaN and infinities). Such a call must be refused on the host: it may return PEAGLE_OK only
// where the arguments describe no work, and must never reach the HIP runtime (which, on a
// machine without a GPU, would answer PEAGLE_ERR_HIP). Signed overflow or an out-of-bounds
// access anywhere in the validation aborts the run through the sanitizers.
//
// Also checked: peagle_cod_counts writes exactly K counts into a heap array of exactly K
// elements (none when it refuses), the size queries never fault on extreme arguments, and
// peagle_status_string returns a string for every status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "peagle.h"

namespace {

uint64_t g_state = 0x243F6A8885A308D3ull;

uint64_t next_u64() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545F4914F6CDD1Dull;
}

int64_t chaos_i64() {
  static const int64_t fixed[] = {0,
                                  1,
                                  -1,
                                  2,
                                  3,
                                  4,
                                  7,
                                  8,
                                  16,
                                  31,
                                  32,
                                  63,
                                  64,
                                  65,
                                  96,
                                  127,
                                  128,
                                  255,
                                  256,
                                  1000,
                                  1024,
                                  4096,
                                  32768,
                                  65535,
                                  65536,
                                  1 << 20,
                                  (int64_t)1 << 31,
                                  ((int64_t)1 << 31) - 1,
                                  -((int64_t)1 << 31),
                                  (int64_t)1 << 32,
                                  (int64_t)1 << 40,
                                  (int64_t)1 << 62,
                                  std::numeric_limits<int64_t>::max(),
                                  std::numeric_limits<int64_t>::min(),
                                  std::numeric_limits<int64_t>::max() - 1};
  const uint64_t pick = next_u64() % 4;
  if (pick == 0) return fixed[next_u64() % (sizeof(fixed) / sizeof(fixed[0]))];
  if (pick == 1) return (int64_t)(next_u64() % 70000);
  if (pick == 2) return (int64_t)(next_u64() % 300) - 30;
  return (int64_t)next_u64();
}

int32_t chaos_i32() {
  const int64_t v = chaos_i64();
  if (next_u64() % 3 == 0) return (int32_t)(uint32_t)(uint64_t)v;  // wraps on purpose
  if (v > std::numeric_limits<int32_t>::max()) return std::numeric_limits<int32_t>::max();
  if (v < std::numeric_limits<int32_t>::min()) return std::numeric_limits<int32_t>::min();
  return (int32_t)v;
}

double chaos_f64() {
  static const double fixed[] = {0.0, -0.0, 1.0, -1.0, 0.5, 0.7, 0.2, 1e-300, 1e300, 2.0,
                                 10000.0, 1e6, std::numeric_limits<double>::quiet_NaN(),
                                 std::numeric_limits<double>::infinity(),
                                 -std::numeric_limits<double>::infinity(),
                                 std::numeric_limits<double>::denorm_min()};
  if (next_u64() % 2 == 0) return fixed[next_u64() % (sizeof(fixed) / sizeof(fixed[0]))];
  return (double)(next_u64() % 2000001) / 1000000.0 - 0.5;
}

float chaos_f32() { return (float)chaos_f64(); }

size_t chaos_size() {
  switch (next_u64() % 4) {
    case 0: return 0;
    case 1: return std::numeric_limits<size_t>::max();
    case 2: return (size_t)(next_u64() % (1ull << 34));
    default: return (size_t)next_u64();
  }
}

long g_calls = 0, g_ok = 0, g_bad = 0;

void check(const char* name, int rc) {
  ++g_calls;
  if (rc == PEAGLE_OK && ++g_ok <= 5) std::printf("note: %s accepted (no work to enqueue)\n", name);
  const bool allowed = rc == PEAGLE_OK || rc == PEAGLE_ERR_ARG || rc == PEAGLE_ERR_UNSUPPORTED ||
                       rc == PEAGLE_ERR_WORKSPACE;
  if (!allowed) {
    ++g_bad;
    if (g_bad <= 20) std::printf("FAIL %s returned %d with NULL pointers\n", name, rc);
  }
}

#define N nullptr

void fuzz_calls(int reps) {
  for (int it = 0; it < reps; ++it) {
    check("cod_select", peagle_cod_select(chaos_i64(), chaos_i32(), chaos_f64(), chaos_f64(),
                                          next_u64(), N, chaos_i32(), N, N, N, N, N, chaos_size(), N));
    check("cod_select_noalloc",
          peagle_cod_select_noalloc(chaos_i64(), chaos_i32(), chaos_f64(), chaos_f64(), next_u64(), N,
                                    chaos_i32(), N, N, N, N, N));
    check("fuse_inputs", peagle_fuse_inputs(chaos_i64(), chaos_i32(), chaos_i64(), N, N, chaos_i32(), N,
                                            N, N, N, chaos_i32(), chaos_i32(), chaos_i32(), N, N, N));
    check("fuse_inputs_fc_norm",
          peagle_fuse_inputs_fc_norm(chaos_i64(), chaos_i32(), chaos_i64(), N, N, chaos_i32(), N, N, N,
                                     N, chaos_i32(), chaos_i32(), chaos_i32(), N, chaos_f32(), N, N, N));
    check("rope_table", peagle_rope_table(chaos_i32(), chaos_f64(), chaos_i32(), N, N, N));
    check("draft_attn_fwd",
          peagle_draft_attn_fwd(chaos_i64(), chaos_i32(), chaos_i64(), N, N, N, N, chaos_i32(), N, N, N,
                                chaos_i32(), chaos_i32(), chaos_i32(), chaos_f32(), N, N, chaos_i32(), N,
                                N, N, chaos_size(), N));
    check("draft_attn_prepare",
          peagle_draft_attn_prepare(chaos_i64(), chaos_i32(), chaos_i64(), N, N, N, N, chaos_i32(), N, N,
                                    N, chaos_i32(), chaos_i32(), chaos_i32(), chaos_f32(), N, N,
                                    chaos_i32(), N, N, N, chaos_size(), N));
    check("draft_attn_core",
          peagle_draft_attn_core(chaos_i64(), chaos_i32(), chaos_i64(), N, N, N, N, chaos_i32(), N, N, N,
                                 chaos_i32(), chaos_i32(), chaos_i32(), chaos_f32(), N, N, chaos_i32(), N,
                                 N, N, chaos_size(), N));
    check("draft_attn_bwd",
          peagle_draft_attn_bwd(chaos_i64(), chaos_i32(), chaos_i64(), N, N, N, N, chaos_i32(), N, N, N,
                                chaos_i32(), chaos_i32(), chaos_i32(), chaos_f32(), N, N, chaos_i32(), N,
                                N, N, N, N, N, N, chaos_size(), N));
    check("depth_ce", peagle_depth_ce(chaos_i64(), chaos_i32(), chaos_i32(), N, N, N, chaos_f32(), N, N,
                                      N, N, chaos_size(), N));
    check("accept_prefix",
          peagle_accept_prefix(chaos_i32(), chaos_i32(), chaos_i32(), N, N, N, N, N, N));
    check("accept_prefix_d2t", peagle_accept_prefix_d2t(chaos_i32(), chaos_i32(), chaos_i32(),
                                                        chaos_i32(), N, N, N, N, N, N, N));
    check("accept_sampled", peagle_accept_sampled(chaos_i32(), chaos_i32(), chaos_i32(), N, N, N, N, N,
                                                  chaos_f32(), N, N, N));
    check("accept_sampled_bonus",
          peagle_accept_sampled_bonus(chaos_i32(), chaos_i32(), chaos_i32(), N, N, N, N, N, chaos_f32(),
                                      N, N, N));
    check("layer1_qkv", peagle_layer1_qkv(chaos_i64(), chaos_i32(), chaos_i64(), N, N, chaos_i32(), N, N,
                                          chaos_f32(), N, chaos_i32(), chaos_i32(), chaos_i32(), N, N, N,
                                          N, chaos_size(), N));
    check("layer1_post",
          peagle_layer1_post(chaos_i64(), chaos_i32(), chaos_i64(), N, chaos_i32(), N, chaos_i32(), N,
                             chaos_i32(), N, N, N, N, chaos_i32(), N, chaos_f32(), N, N, chaos_size(),
                             N));
    check("layer_qkv", peagle_layer_qkv(chaos_i64(), N, chaos_i32(), N, chaos_f32(), N, chaos_i32(),
                                        chaos_i32(), chaos_i32(), N, N, N, N, chaos_size(), N));
    check("layer_post", peagle_layer_post(chaos_i64(), N, chaos_i32(), N, chaos_i32(), N, N, N, N,
                                          chaos_i32(), N, chaos_f32(), N, N, chaos_size(), N));
    check("draft_head", peagle_draft_head(chaos_i64(), N, chaos_i32(), N, N, chaos_i32(), chaos_f32(),
                                          N, N, chaos_size(), N));
    check("decode_pack_v", peagle_decode_pack_v(chaos_i32(), N, chaos_i64(), chaos_i32(), N,
                                                chaos_i32(), chaos_i32(), N, chaos_size(), N));
    check("draft_decode_attn",
          peagle_draft_decode_attn(chaos_i32(), chaos_i32(), N, chaos_i64(), chaos_i32(), N, N,
                                   chaos_size(), N, N, N, chaos_i32(), chaos_i32(), chaos_i32(),
                                   chaos_f32(), N, N, chaos_i32(), N, N, N, chaos_size(), N));
    check("decode_pack_v_lens", peagle_decode_pack_v_lens(chaos_i32(), N, N, chaos_i64(), chaos_i32(),
                                                          N, chaos_i32(), chaos_i32(), N, chaos_size(),
                                                          N));
    check("draft_decode_attn_lens",
          peagle_draft_decode_attn_lens(chaos_i32(), chaos_i32(), N, N, chaos_i64(), chaos_i32(), N, N,
                                        chaos_size(), N, N, N, chaos_i32(), chaos_i32(), chaos_i32(),
                                        chaos_f32(), N, N, chaos_i32(), N, N, N, chaos_size(), N));
    check("decode_append",
          peagle_decode_append(chaos_i32(), N, N, N, chaos_i32(), chaos_i32(), N, N, chaos_i32(),
                               chaos_i32(), N, N, chaos_i32(), chaos_i64(), chaos_i32(), N, N,
                               chaos_size(), N, N));
  }
}

#undef N

// Size queries on hostile arguments: no fault, no signed overflow; 0 is the refusal.
void fuzz_sizes(int reps) {
  volatile size_t sink = 0;
  for (int it = 0; it < reps; ++it) {
    sink += peagle_cod_workspace_bytes(chaos_i64(), chaos_i32());
    sink += peagle_draft_attn_workspace_bytes(chaos_i64(), chaos_i64(), chaos_i32(), chaos_i32(),
                                              chaos_i32());
    sink += peagle_draft_attn_bwd_workspace_bytes(chaos_i64(), chaos_i64(), chaos_i32(), chaos_i32(),
                                                  chaos_i32());
    sink += peagle_depth_ce_workspace_bytes(chaos_i64(), chaos_i32());
    sink += peagle_layer1_qkv_workspace_bytes(chaos_i64(), chaos_i64(), chaos_i32());
    sink += peagle_layer1_post_workspace_bytes(chaos_i64(), chaos_i64(), chaos_i32(), chaos_i32(),
                                               chaos_i32());
    sink += peagle_layer_qkv_workspace_bytes(chaos_i64(), chaos_i32());
    sink += peagle_layer_post_workspace_bytes(chaos_i64(), chaos_i32(), chaos_i32(), chaos_i32());
    sink += peagle_draft_head_workspace_bytes(chaos_i64(), chaos_i32(), chaos_i32());
    sink += peagle_decode_v_tiles_bytes(chaos_i64(), chaos_i32(), chaos_i32(), chaos_i32());
    sink += peagle_draft_decode_workspace_bytes(chaos_i32(), chaos_i32(), chaos_i32(), chaos_i32(),
                                                chaos_i32(), chaos_i64(), chaos_i32());
  }
  (void)sink;
}

// peagle_cod_counts into a heap array of exactly K elements (a zero-length one when K is
// out of range): a write past it, or any write on refusal, is caught by the sanitizer.
bool fuzz_counts(int reps) {
  bool ok = true;
  for (int it = 0; it < reps; ++it) {
    const int64_t n = chaos_i64();
    const int32_t K = next_u64() % 4 == 0 ? chaos_i32() : (int32_t)(next_u64() % 70);
    const double r = chaos_f64(), r_min = chaos_f64();
    const bool in_range = K >= 1 && K <= PEAGLE_MAX_DEPTHS;
    int64_t* m = new int64_t[in_range ? K : 0];
    int64_t T = -12345;
    const int rc = peagle_cod_counts(n, K, r, r_min, m, &T);
    if (rc == PEAGLE_OK) {
      int64_t sum = 0;
      bool good = in_range;
      for (int d = 0; good && d < K; ++d) {
        good = m[d] >= 0 && m[d] <= n && (d == 0 || m[d] <= m[d - 1]) && m[0] == n;
        sum += m[d];
      }
      if (!good || sum != T) {
        ok = false;
        std::printf("FAIL cod_counts(n=%lld, K=%d, r=%g, r_min=%g) accepted, counts inconsistent\n",
                    (long long)n, K, r, r_min);
      }
    } else if (rc != PEAGLE_ERR_ARG) {
      ok = false;
      std::printf("FAIL cod_counts returned %d\n", rc);
    } else if (T != -12345) {
      ok = false;
      std::printf("FAIL cod_counts wrote T on refusal\n");
    }
    delete[] m;
  }
  return ok;
}

}  // namespace

int main(int argc, char** argv) {
  const int reps = argc > 1 ? std::atoi(argv[1]) : 2000;
  for (int s = -64; s <= 64; ++s) {
    const char* str = peagle_status_string(s);
    if (str == nullptr || std::strlen(str) == 0) {
      std::printf("FAIL status_string(%d)\n", s);
      return 1;
    }
  }
  if (peagle_version() <= 0) {
    std::printf("FAIL version\n");
    return 1;
  }
  fuzz_sizes(reps * 10);
  const bool counts_ok = fuzz_counts(reps * 20);
  fuzz_calls(reps);
  std::printf("calls %ld accepted-as-no-op %ld refused-wrongly %ld counts %s\n", g_calls, g_ok, g_bad,
              counts_ok ? "ok" : "FAIL");
  return (g_bad == 0 && counts_ok) ? 0 : 1;
}
