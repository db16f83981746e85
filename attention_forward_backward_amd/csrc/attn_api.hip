// attn_api.hip -- the C ABI declared in include/attn.h.
//
// Validates every argument on the host before anything is enqueued, then
// hands a launch descriptor to the kernel launchers.  Stateless: nothing is
// allocated, cached or retained between calls.
#include <math.h>
#include <stdint.h>

#include "../../include/attn.h"
#include "attn_launch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

attn_status_t check_shape(attn_dtype_t dtype, int batch, int heads, int seq, int head_dim,
                          int causal, float scale, bool check_scale) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (batch <= 0 || heads <= 0 || seq <= 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (check_scale && !(isfinite(scale) && scale > 0.f)) return ATTN_ERR_INVALID_ARG;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  // Element counts must fit the kernels' index arithmetic: B*H within the
  // grid's x dimension, S*D within int, and the whole tensor within int64.
  const int64_t bh = (int64_t)batch * heads;
  if (bh > 0x7fffffffLL) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)seq * head_dim > 0x7fffffffLL) return ATTN_ERR_INVALID_ARG;
  if (bh * seq > 0x7fffffffLL) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

attn_status_t check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs) {
    if (p == nullptr || !aligned16(p)) return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

size_t delta_bytes(int batch, int heads, int seq) {
  // D, then LSE * log2(e), one float each per query row
  const size_t b = 2 * (size_t)batch * heads * seq * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

attn_status_t from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

attn::BwdArgs make_bwd(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                       const void* o, const void* dout, const float* lse, void* dq, void* dk,
                       void* dv, void* ws, int batch, int heads, int seq, int head_dim,
                       int causal, float scale, void* stream) {
  attn::BwdArgs a;
  a.bf16 = dtype == ATTN_BF16;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.delta = static_cast<float*>(ws);
  a.BH = batch * heads; a.S = seq; a.D = head_dim;
  a.causal = causal != 0; a.scale = scale;
  a.stream = static_cast<hipStream_t>(stream);
  return a;
}

}  // namespace

extern "C" {

attn_status_t attn_fwd(attn_dtype_t dtype, const void* q, const void* k, const void* v, void* o,
                       float* lse, int batch, int heads, int seq, int head_dim, int causal,
                       float scale, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if ((st = check_ptrs({q, k, v, o, lse})) != ATTN_OK) return st;
  attn::FwdArgs a;
  a.bf16 = dtype == ATTN_BF16;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.BH = batch * heads; a.S = seq; a.D = head_dim;
  a.causal = causal != 0; a.scale = scale;
  a.stream = static_cast<hipStream_t>(stream);
  return from_hip(attn::launch_fwd(a));
}

size_t attn_bwd_workspace_size(attn_dtype_t dtype, int batch, int heads, int seq, int head_dim,
                               int causal) {
  if (check_shape(dtype, batch, heads, seq, head_dim, causal, 1.f, false) != ATTN_OK) return 0;
  return delta_bytes(batch, heads, seq);
}

attn_status_t attn_bwd_dq(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                          const void* o, const void* dout, const float* lse, void* dq,
                          void* workspace, size_t workspace_bytes, int batch, int heads, int seq,
                          int head_dim, int causal, float scale, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if ((st = check_ptrs({q, k, v, o, dout, lse, dq, workspace})) != ATTN_OK) return st;
  if (workspace_bytes < delta_bytes(batch, heads, seq)) return ATTN_ERR_WORKSPACE;
  const attn::BwdArgs a = make_bwd(dtype, q, k, v, o, dout, lse, dq, nullptr, nullptr, workspace,
                                   batch, heads, seq, head_dim, causal, scale, stream);
  return from_hip(attn::launch_bwd_dq(a));
}

attn_status_t attn_bwd_dkdv(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                            const void* dout, const float* lse, void* dk, void* dv,
                            const void* workspace, size_t workspace_bytes, int batch, int heads,
                            int seq, int head_dim, int causal, float scale, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if ((st = check_ptrs({q, k, v, dout, lse, dk, dv, workspace})) != ATTN_OK) return st;
  if (workspace_bytes < delta_bytes(batch, heads, seq)) return ATTN_ERR_WORKSPACE;
  const attn::BwdArgs a =
      make_bwd(dtype, q, k, v, nullptr, dout, lse, nullptr, dk, dv, const_cast<void*>(workspace),
               batch, heads, seq, head_dim, causal, scale, stream);
  return from_hip(attn::launch_bwd_dkdv(a));
}

attn_status_t attn_bwd(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                       const void* o, const void* dout, const float* lse, void* dq, void* dk,
                       void* dv, void* workspace, size_t workspace_bytes, int batch, int heads,
                       int seq, int head_dim, int causal, float scale, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if ((st = check_ptrs({q, k, v, o, dout, lse, dq, dk, dv, workspace})) != ATTN_OK) return st;
  if (workspace_bytes < delta_bytes(batch, heads, seq)) return ATTN_ERR_WORKSPACE;
  const attn::BwdArgs a = make_bwd(dtype, q, k, v, o, dout, lse, dq, dk, dv, workspace, batch,
                                   heads, seq, head_dim, causal, scale, stream);
  if ((st = from_hip(attn::launch_bwd_dq(a))) != ATTN_OK) return st;
  return from_hip(attn::launch_bwd_dkdv(a));
}

const char* attn_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head_dim or dtype";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

const char* attn_version(void) { return "0.1.0"; }

}  // extern "C"
