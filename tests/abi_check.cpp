// Host check of the C ABI's argument validation (attn_api.hip), built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code: every
// call below must be rejected with its status before anything would be
// enqueued, so the kernel launchers are stubs that abort if reached, and the
// workspace-size functions are exercised at their overflow edges.  No GPU is
// touched.  Test infrastructure; prints one line and exits non-zero on the
// first violation.
#include <math.h>
#include <stdint.h>

#include <cstdio>
#include <cstdlib>

#include "attn.h"
#include "attn_launch.hpp"

namespace attn {
// Validation must return before any of these is called.
#define STUB(name, T)                                            \
  hipError_t name(const T&) {                                    \
    std::printf("FAIL: %s reached past validation\n", #name);    \
    std::abort();                                                \
  }
STUB(launch_fwd, FwdArgs)
STUB(launch_rope, RopeArgs)
STUB(launch_fwd_small, FwdArgs)
STUB(launch_bwd_dq, BwdArgs)
STUB(launch_bwd_dkdv, BwdArgs)
STUB(launch_bwd_prep, BwdArgs)
}  // namespace attn

static int fails = 0;
#define EXPECT(expr, want)                                                            \
  do {                                                                                \
    const int got_ = (int)(expr);                                                     \
    if (got_ != (int)(want)) {                                                        \
      std::printf("FAIL line %d: %s returned %d, expected %d\n", __LINE__, #expr, got_, \
                  (int)(want));                                                       \
      ++fails;                                                                        \
    }                                                                                 \
  } while (0)

int main() {
  void* const P = reinterpret_cast<void*>(0x10000);  // aligned, never dereferenced
  void* const M = reinterpret_cast<void*>(0x10008);  // 8-byte aligned only
  float* const L = static_cast<float*>(P);
  const float s = 0.125f;
  const attn_status_t INV = ATTN_ERR_INVALID_ARG, UNS = ATTN_ERR_UNSUPPORTED, WS = ATTN_ERR_WORKSPACE;

  // forward
  EXPECT(attn_fwd(ATTN_F32, nullptr, P, P, P, L, 1, 1, 8, 64, 1, s, nullptr), INV);
  EXPECT(attn_fwd(ATTN_F32, P, P, M, P, L, 1, 1, 8, 64, 1, s, nullptr), INV);
  EXPECT(attn_fwd(ATTN_F32, P, P, P, P, static_cast<float*>(M), 1, 1, 8, 64, 1, s, nullptr), INV);
  EXPECT(attn_fwd(ATTN_F32, P, P, P, P, L, 0, 1, 8, 64, 1, s, nullptr), INV);
  EXPECT(attn_fwd(ATTN_F32, P, P, P, P, L, 1, 1, 8, 64, 2, s, nullptr), INV);
  EXPECT(attn_fwd(ATTN_F32, P, P, P, P, L, 1, 1, 8, 64, 1, NAN, nullptr), INV);
  EXPECT(attn_fwd(ATTN_F32, P, P, P, P, L, 1, 1, 8, 64, 1, -s, nullptr), INV);
  EXPECT(attn_fwd(ATTN_F32, P, P, P, P, L, 1, 1, 8, 48, 1, s, nullptr), UNS);
  EXPECT(attn_fwd((attn_dtype_t)7, P, P, P, P, L, 1, 1, 8, 64, 1, s, nullptr), UNS);
  EXPECT(attn_fwd(ATTN_F32, P, P, P, P, L, 1 << 16, 1 << 16, 8, 64, 1, s, nullptr), INV);
  EXPECT(attn_fwd(ATTN_F32, P, P, P, P, L, 1, 1, 1 << 26, 64, 1, s, nullptr), INV);
  EXPECT(attn_fwd(ATTN_BF16, P, P, P, P, L, 0x7fffffff, 0x7fffffff, 0x7fffffff, 128, 1, s,
                  nullptr), INV);
  // backward (every pointer misaligned in turn, the workspace, the sizes)
  for (int i = 0; i < 10; ++i) {
    void* p[10];
    for (int j = 0; j < 10; ++j) p[j] = j == i ? M : P;
    EXPECT(attn_bwd(ATTN_F32, p[0], p[1], p[2], p[3], p[4], static_cast<float*>(p[5]), p[6],
                    p[7], p[8], p[9], 1 << 20, 1, 1, 8, 64, 1, s, nullptr),
           INV);
  }
  EXPECT(attn_bwd(ATTN_F32, P, P, P, P, P, L, P, P, P, P, 2 * 8 * 4 - 1, 1, 1, 8, 64, 1, s,
                  nullptr), WS);
  EXPECT(attn_bwd(ATTN_BF16, P, P, P, P, P, L, P, P, P, P, 1 << 20, 1, 1, 8, 96, 1, s, nullptr),
         UNS);
  EXPECT(attn_bwd_prep(ATTN_F32, P, P, L, P, 16, 1, 1, 8, 64, nullptr), WS);
  EXPECT(attn_bwd_dkdv(ATTN_F32, P, P, P, P, P, P, P, 16, 1, 1, 8, 64, 1, s, nullptr), WS);
  EXPECT(attn_bwd_dq(ATTN_F32, P, P, P, P, P, P, 16, 1, 1, 8, 64, 1, s, nullptr), WS);
  EXPECT(attn_bwd_noalloc(ATTN_F32, P, P, P, P, P, L, P, P, M, 1, 1, 8, 64, 1, s, nullptr), INV);
  EXPECT(attn_bwd_noalloc(ATTN_F32, P, P, P, P, P, L, P, P, P, 1, 256, 65537, 64, 1, s, nullptr),
         WS);
  // cross-attention and strided layouts
  const int* const kv = static_cast<const int*>(P);
  EXPECT(attn_fwd_cross(ATTN_F32, P, P, P, P, L, 1, 1, 8, 0, 64, kv, 1, s, nullptr), INV);
  EXPECT(attn_fwd_cross(ATTN_F32, P, P, P, P, L, 1, 1, 8, 8, 64,
                        reinterpret_cast<const int*>(0x10002), 1, s, nullptr), INV);
  long long st[24];
  for (int t = 0; t < 8; ++t) {
    st[3 * t] = 8 * 64;
    st[3 * t + 1] = 8 * 64;
    st[3 * t + 2] = 64;
  }
  st[2] = 12;  // not a multiple of 8 elements
  EXPECT(attn_fwd_strided(ATTN_F32, P, P, P, P, L, 1, 1, 8, 8, 64, nullptr, st, 1, s, nullptr),
         INV);
  st[2] = 64;
  st[3 * 5 + 2] = 0;  // dq rows overlap
  EXPECT(attn_bwd_strided(ATTN_F32, P, P, P, P, P, L, P, P, P, P, 1 << 20, 1, 1, 8, 8, 64,
                          nullptr, st, 1, s, nullptr), INV);
  st[3 * 5 + 2] = 1LL << 40;  // row stride beyond the kernels' 32-bit offsets
  EXPECT(attn_bwd_strided(ATTN_F32, P, P, P, P, P, L, P, P, P, P, 1 << 20, 1, 1, 8, 8, 64,
                          nullptr, st, 1, s, nullptr), INV);
  EXPECT(attn_fwd_strided(ATTN_F32, P, P, P, P, L, 1, 1, 8, 8, 64, nullptr, nullptr, 1, s,
                          nullptr), INV);
  // RoPE pass
  long long rs[3] = {8 * 64, 8 * 64, 64};
  EXPECT(attn_rope_copy(ATTN_F32, P, rs, P, rs, L, nullptr, 8, 0, 1, 1, 8, 64, 0, nullptr), INV);
  EXPECT(attn_rope_copy(ATTN_F32, P, rs, P, rs, L, L, 8, 1, 1, 1, 8, 64, 0, nullptr), INV);
  EXPECT(attn_rope_copy(ATTN_F32, P, rs, P, rs, nullptr, nullptr, 0, 0, 1, 1, 8, 64, 2, nullptr),
         INV);
  // fused RoPE entry points: tables, qk_rot and the internal [B,H,S,D] strides
  const float* const T = L;
  for (int i = 0; i < 24; ++i) st[i] = (i % 3 == 0) ? 8 * 64 : 64;  // B = H = 1, rows of 64
  EXPECT(attn_fwd_rope(ATTN_F32, P, P, P, P, L, nullptr, 1, 1, 8, 64, st, T, T, 8, 0, 1, s,
                       nullptr), INV);
  EXPECT(attn_fwd_rope(ATTN_F32, P, P, P, P, L, P, 1, 1, 8, 64, st, T, nullptr, 8, 0, 1, s,
                       nullptr), INV);
  EXPECT(attn_fwd_rope(ATTN_F32, P, P, P, P, L, P, 1, 1, 8, 64, st, T, T, 8, 1, 1, s, nullptr),
         INV);
  EXPECT(attn_fwd_rope(ATTN_F32, P, P, P, P, L, P, 1, 1, 8, 64, st, static_cast<const float*>(M),
                       T, 8, 0, 1, s, nullptr), INV);
  EXPECT(attn_bwd_rope(ATTN_F32, P, P, P, P, L, P, P, P, P, 1 << 20, 1, 1, 8, 64, st, T, T, 7, 0,
                       1, s, nullptr), INV);
  EXPECT(attn_bwd_rope(ATTN_F32, M, P, P, P, L, P, P, P, P, 1 << 20, 1, 1, 8, 64, st, T, T, 8, 0,
                       1, s, nullptr), INV);
  EXPECT(attn_bwd_rope(ATTN_F32, P, P, P, P, L, P, P, P, P, 16, 1, 1, 8, 64, st, T, T, 8, 0, 1, s,
                       nullptr), WS);
  EXPECT(attn_bwd_rope(ATTN_BF16, P, P, P, P, L, P, P, P, P, 1 << 20, 1, 1, 8, 96, st, T, T, 8, 0,
                       1, s, nullptr), UNS);
  // workspace sizes: 0 for rejected shapes, monotone and overflow-free at the edges
  EXPECT(attn_bwd_workspace_size(ATTN_F32, 1, 1, 8, 48, 1), 0);
  EXPECT(attn_bwd_workspace_size_min(ATTN_F32, 0, 1, 8, 64, 1), 0);
  // beyond the cap on the dS/dP layout the recommendation falls back to the minimum
  const size_t big = attn_bwd_workspace_size(ATTN_F32, 1, 1, 1 << 20, 128, 1);
  const size_t bigmin = attn_bwd_workspace_size_min(ATTN_F32, 1, 1, 1 << 20, 128, 1);
  if (!(big == bigmin && bigmin == 2u * (1u << 20) * 4u)) {
    std::printf("FAIL: workspace sizes at S = 2^20: %zu, %zu\n", big, bigmin);
    ++fails;
  }
  const size_t mid = attn_bwd_workspace_size(ATTN_F32, 1, 16, 2048, 128, 1);
  const size_t midmin = attn_bwd_workspace_size_min(ATTN_F32, 1, 16, 2048, 128, 1);
  if (!(mid > midmin && mid - midmin <= (size_t)ATTN_DS_WORKSPACE_CAP)) {
    std::printf("FAIL: workspace sizes at S = 2048: %zu, %zu\n", mid, midmin);
    ++fails;
  }
  if (attn_bwd_cross_workspace_size(ATTN_BF16, 2, 8, 4096, 77, 64, 0) <=
      attn_bwd_cross_workspace_size_min(ATTN_BF16, 2, 8, 4096, 77, 64, 0)) {
    std::printf("FAIL: cross workspace sizes\n");
    ++fails;
  }
  std::printf(fails ? "FAILED (%d)\n" : "OK\n", fails);
  return fails ? 1 : 0;
}
