// attn_api.hip -- the C ABI declared in include/attn.h.
//
// Validates every argument on the host before anything is enqueued, then
// hands a launch descriptor to the kernel launchers.  No call allocates
// device memory and no pointer is retained between calls (the launchers
// cache only occupancy figures and schedule patterns, on the host); the one
// device buffer of the library is the static scratch array of the
// allocation-free backward.
#include <math.h>

#include <mutex>
#include <utility>
#include <stdint.h>

#include "../../include/attn.h"
#include "attn_launch.hpp"

// The allocation-free backward (attn_bwd_noalloc) takes its workspace from
// this device array: one copy per GPU, resident while the process runs.  In
// host code `scratch` names a host-side stand-in, never the device memory;
// scratch_base() gives the device address.
constexpr size_t kScratchBytes = ATTN_BWD_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of this GPU's scratch array, looked up once per device
// (with that device current) and kept; null if the lookup fails.
void* scratch_base() {
  static std::mutex mu;
  static void* base[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (base[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    base[dev] = p;
  }
  return base[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

attn_status_t check_shape(attn_dtype_t dtype, int batch, int heads, int sq, int sk, int head_dim,
                          int causal, float scale, bool check_scale) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_F32_BF16FWD) return ATTN_ERR_UNSUPPORTED;
  if (batch <= 0 || heads <= 0 || sq <= 0 || sk <= 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (check_scale && !(isfinite(scale) && scale > 0.f)) return ATTN_ERR_INVALID_ARG;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  // Element counts must fit the kernels' index arithmetic: B*H within the
  // grid's x dimension, S*D within int, and the whole tensor within int64.
  const int64_t bh = (int64_t)batch * heads;
  if (bh > 0x7fffffffLL) return ATTN_ERR_INVALID_ARG;
  for (const int s : {sq, sk}) {
    if ((int64_t)s * head_dim > 0x7fffffffLL) return ATTN_ERR_INVALID_ARG;
    if (bh * s > 0x7fffffffLL) return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

attn_status_t check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs) {
    if (p == nullptr || !aligned16(p)) return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Minimum workspace: D, then LSE * log2(e), one float each per query row.
size_t ws_min_bytes(int batch, int heads, int sq) {
  return round256(2 * (size_t)batch * heads * sq * sizeof(float));
}

// Stride of the stored dS: a length rounded up to the largest tile.
int ds_stride(int s) { return (s + 127) / 128 * 128; }

// Full workspace: the minimum plus dS^T [B*H][ds_stride(sk)][ds_stride(sq)] in dtype.
size_t ws_full_bytes(attn_dtype_t dtype, int batch, int heads, int sq, int sk) {
  const size_t esize = dtype == ATTN_BF16 ? 2 : 4;
  return ws_min_bytes(batch, heads, sq) +
         round256((size_t)batch * heads * ds_stride(sk) * ds_stride(sq) * esize);
}

// dK, dV partials of the query-chunk split, [2][nqs][B*H][Sk][D] f32 (none
// when the shape needs no split; the backward arithmetic is f32 unless the
// tensors are bf16).
size_t ws_part_bytes(attn_dtype_t dtype, int batch, int heads, int sq, int sk, int head_dim) {
  const int nqs =
      attn::dkdv_query_chunks(dtype == ATTN_BF16, (long long)batch * heads, sq, sk, head_dim);
  return nqs > 1 ? round256(2 * (size_t)nqs * batch * heads * sk * head_dim * sizeof(float)) : 0;
}

// Recommended workspace: the dS path while its dS^T buffer fits
// ATTN_DS_WORKSPACE_CAP bytes, else the minimum (so the recommended size is
// O(S) for long sequences), plus, for shapes with few key tiles per head,
// room for the dK, dV partials.
size_t ws_rec_bytes(attn_dtype_t dtype, int batch, int heads, int sq, int sk, int head_dim) {
  const size_t full = ws_full_bytes(dtype, batch, heads, sq, sk);
  const size_t mn = ws_min_bytes(batch, heads, sq);
  return (full - mn <= (size_t)ATTN_DS_WORKSPACE_CAP ? full : mn) +
         ws_part_bytes(dtype, batch, heads, sq, sk, head_dim);
}

attn_status_t from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Backward launch descriptor.  The dS path is taken iff the workspace holds
// the minimum plus dS^T; the dK+dV query split iff it also holds the
// partials (after dS^T, or after the minimum without the dS path).
attn::BwdArgs make_bwd(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                       const void* o, const void* dout, const float* lse, void* dq, void* dk,
                       void* dv, void* ws, size_t ws_bytes, int batch, int heads, int sq, int sk,
                       int head_dim, const int* kvlen, int causal, float scale, void* stream,
                       const attn::Layout* layout = nullptr) {
  attn::BwdArgs a;
  a.bf16 = dtype == ATTN_BF16;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.delta = static_cast<float*>(ws);
  const size_t wmin = ws_min_bytes(batch, heads, sq);
  const size_t wfull = ws_full_bytes(dtype, batch, heads, sq, sk);
  const size_t wpart = ws_part_bytes(dtype, batch, heads, sq, sk, head_dim);
  const bool full = ws_bytes >= wfull;
  const bool split = wpart > 0 && ws_bytes >= (full ? wfull : wmin) + wpart;
  a.ds = full ? static_cast<char*>(ws) + wmin : nullptr;
  a.part = split ? reinterpret_cast<float*>(static_cast<char*>(ws) + (full ? wfull : wmin))
                 : nullptr;
  a.nqs = split ? attn::dkdv_query_chunks(dtype == ATTN_BF16, (long long)batch * heads, sq, sk,
                                           head_dim)
                : 1;
  a.SPq = ds_stride(sq); a.SPk = ds_stride(sk);
  a.BH = batch * heads; a.H = heads; a.Sq = sq; a.Sk = sk; a.D = head_dim;
  a.kvlen = kvlen;
  a.cross = sq != sk || kvlen != nullptr || layout != nullptr;
  a.causal = causal != 0; a.scale = scale;
  a.stream = static_cast<hipStream_t>(stream);
  a.layout = layout;
  return a;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Strides (batch, head, row) of one tensor of extents (B, H, S) x D:
// non-negative multiples of 8 elements (16-byte rows), below 2^31 (the
// kernels hold them in 32 bits), a row stride of at most 2^24 (their 32-bit
// lane offsets), and the farthest element within int64.
// Outputs must also not overlap themselves: sorted by stride, each stride is
// at least the span of the dimensions below it (the D elements of a row
// first).
bool check_strides(const long long* st, int B, int H, int S, int D, bool output) {
  const int ext[3] = {B, H, S};
  double far = D;
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0 || st[i] % 8 != 0) return false;
    far += (double)st[i] * (ext[i] - 1);
  }
  if (st[0] > 0x7fffffffLL || st[1] > 0x7fffffffLL || st[2] > (1LL << 24) || far > 4.0e18)
    return false;
  if (!output) return true;
  int ord[3] = {0, 1, 2};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (st[ord[j]] < st[ord[i]]) std::swap(ord[i], ord[j]);
  long long span = D;
  for (int i = 0; i < 3; ++i) {
    const int d = ord[i];
    if (ext[d] == 1) continue;
    if (st[d] < span) return false;
    span = st[d] * ext[d];
  }
  return true;
}

attn::Str3 str3(const long long* st) {
  return attn::Str3{(int)st[0], (int)st[1], (int)st[2]};
}

// RoPE tables: both given, 16-byte aligned, rows pos_offset .. pos_offset +
// seq - 1 inside [0, table_rows).
bool check_tables(const float* cos_table, const float* sin_table, int table_rows, int pos_offset,
                  int seq) {
  if (cos_table == nullptr || sin_table == nullptr) return false;
  if (!aligned16(cos_table) || !aligned16(sin_table)) return false;
  return pos_offset >= 0 && table_rows >= 0 && (int64_t)pos_offset + seq <= table_rows;
}

// Workspace of the key-split forward: unnormalised O partials [nch][B*H][Sp][D]
// and (m, l) pairs [nch][B*H][Sp][2], float32; 0 when the shape is not split.
size_t fwd_ws_bytes(attn_dtype_t dtype, int batch, int heads, int seq, int head_dim, int causal) {
  if (seq <= (dtype == ATTN_BF16 ? ATTN_FWD_SMALL_MAXQ_BF16 : ATTN_FWD_SMALL_MAXQ_F32)) return 0;
  int nch = 1, kc = 0;
  const bool bf16 = dtype == ATTN_BF16;
  if (!attn::fwd_key_split(bf16, (long long)batch * heads, seq, head_dim, causal != 0, nch, kc))
    return 0;
  const int br = attn::fwd_query_tile(bf16, head_dim);
  const size_t sp = (size_t)(seq + br - 1) / br * br;
  return round256((size_t)nch * batch * heads * sp * (head_dim + 2) * sizeof(float));
}

attn_status_t fwd_impl(attn_dtype_t dtype, const void* q, const void* k, const void* v, void* o,
                       float* lse, int batch, int heads, int sq, int sk, int head_dim,
                       const int* kvlen, int causal, float scale, void* stream,
                       const attn::Layout* layout = nullptr, float* part = nullptr,
                       const attn::RopeTab* rope = nullptr) {
  attn_status_t st = check_shape(dtype, batch, heads, sq, sk, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if ((st = check_ptrs({q, k, v, o})) != ATTN_OK) return st;
  if (lse != nullptr && !aligned16(lse)) return ATTN_ERR_INVALID_ARG;  // NULL: no LSE
  if (kvlen != nullptr && !aligned4(kvlen)) return ATTN_ERR_INVALID_ARG;
  attn::FwdArgs a;
  a.bf16 = dtype == ATTN_BF16;
  a.bf16_operands = dtype == ATTN_F32_BF16FWD;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.BH = batch * heads; a.H = heads; a.Sq = sq; a.Sk = sk; a.D = head_dim;
  a.kvlen = kvlen;
  a.cross = sq != sk || kvlen != nullptr || layout != nullptr;
  a.causal = causal != 0; a.scale = scale;
  a.stream = static_cast<hipStream_t>(stream);
  a.layout = layout;
  a.part = part;
  if (rope != nullptr) a.rope = *rope;
  return from_hip(attn::launch_fwd(a));
}

attn_status_t bwd_impl(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                       const void* o, const void* dout, const float* lse, void* dq, void* dk,
                       void* dv, void* workspace, size_t workspace_bytes, int batch, int heads,
                       int sq, int sk, int head_dim, const int* kvlen, int causal, float scale,
                       void* stream, const attn::Layout* layout = nullptr,
                       const attn::RopeTab* rope = nullptr) {
  attn_status_t st = check_shape(dtype, batch, heads, sq, sk, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if ((st = check_ptrs({q, k, v, o, dout, lse, dq, dk, dv, workspace})) != ATTN_OK) return st;
  if (kvlen != nullptr && !aligned4(kvlen)) return ATTN_ERR_INVALID_ARG;
  if (workspace_bytes < ws_min_bytes(batch, heads, sq)) return ATTN_ERR_WORKSPACE;
  attn::BwdArgs a = make_bwd(dtype, q, k, v, o, dout, lse, dq, dk, dv, workspace,
                             workspace_bytes, batch, heads, sq, sk, head_dim, kvlen, causal, scale,
                             stream, layout);
  if (rope != nullptr) a.rope = *rope;
  a.dfused = attn::dkdv_dfused(a);
  if (!a.dfused && (st = from_hip(attn::launch_bwd_prep(a))) != ATTN_OK) return st;
  if ((st = from_hip(attn::launch_bwd_dkdv(a))) != ATTN_OK) return st;
  return from_hip(attn::launch_bwd_dq(a));
}

}  // namespace

extern "C" {

attn_status_t attn_fwd(attn_dtype_t dtype, const void* q, const void* k, const void* v, void* o,
                       float* lse, int batch, int heads, int seq, int head_dim, int causal,
                       float scale, void* stream) {
  return fwd_impl(dtype, q, k, v, o, lse, batch, heads, seq, seq, head_dim, nullptr, causal, scale,
                  stream);
}

size_t attn_fwd_workspace_size(attn_dtype_t dtype, int batch, int heads, int seq, int head_dim,
                               int causal) {
  if (check_shape(dtype, batch, heads, seq, seq, head_dim, causal, 1.f, false) != ATTN_OK) return 0;
  return fwd_ws_bytes(dtype, batch, heads, seq, head_dim, causal);
}

attn_status_t attn_fwd_ws(attn_dtype_t dtype, const void* q, const void* k, const void* v, void* o,
                          float* lse, void* workspace, size_t workspace_bytes, int batch,
                          int heads, int seq, int head_dim, int causal, float scale,
                          void* stream) {
  if (workspace != nullptr && !aligned16(workspace)) return ATTN_ERR_INVALID_ARG;
  const size_t need = check_shape(dtype, batch, heads, seq, seq, head_dim, causal, scale, true) ==
                              ATTN_OK
                          ? fwd_ws_bytes(dtype, batch, heads, seq, head_dim, causal)
                          : 0;
  float* part = (need > 0 && workspace != nullptr && workspace_bytes >= need)
                    ? static_cast<float*>(workspace)
                    : nullptr;
  return fwd_impl(dtype, q, k, v, o, lse, batch, heads, seq, seq, head_dim, nullptr, causal, scale,
                  stream, nullptr, part);
}

attn_status_t attn_fwd_cross(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                             void* o, float* lse, int batch, int heads, int seq_q, int seq_k,
                             int head_dim, const int* kv_len, int causal, float scale,
                             void* stream) {
  return fwd_impl(dtype, q, k, v, o, lse, batch, heads, seq_q, seq_k, head_dim, kv_len, causal,
                  scale, stream);
}

size_t attn_bwd_workspace_size(attn_dtype_t dtype, int batch, int heads, int seq, int head_dim,
                               int causal) {
  if (check_shape(dtype, batch, heads, seq, seq, head_dim, causal, 1.f, false) != ATTN_OK) return 0;
  return ws_rec_bytes(dtype, batch, heads, seq, seq, head_dim);
}

size_t attn_bwd_workspace_size_min(attn_dtype_t dtype, int batch, int heads, int seq,
                                   int head_dim, int causal) {
  if (check_shape(dtype, batch, heads, seq, seq, head_dim, causal, 1.f, false) != ATTN_OK) return 0;
  return ws_min_bytes(batch, heads, seq);
}

size_t attn_bwd_cross_workspace_size(attn_dtype_t dtype, int batch, int heads, int seq_q,
                                     int seq_k, int head_dim, int causal) {
  if (check_shape(dtype, batch, heads, seq_q, seq_k, head_dim, causal, 1.f, false) != ATTN_OK)
    return 0;
  return ws_rec_bytes(dtype, batch, heads, seq_q, seq_k, head_dim);
}

size_t attn_bwd_cross_workspace_size_min(attn_dtype_t dtype, int batch, int heads, int seq_q,
                                         int seq_k, int head_dim, int causal) {
  if (check_shape(dtype, batch, heads, seq_q, seq_k, head_dim, causal, 1.f, false) != ATTN_OK)
    return 0;
  return ws_min_bytes(batch, heads, seq_q);
}

attn_status_t attn_bwd_prep(attn_dtype_t dtype, const void* o, const void* dout,
                            const float* lse, void* workspace, size_t workspace_bytes, int batch,
                            int heads, int seq, int head_dim, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq, seq, head_dim, 0, 1.f, false);
  if (st != ATTN_OK) return st;
  if ((st = check_ptrs({o, dout, lse, workspace})) != ATTN_OK) return st;
  if (workspace_bytes < ws_min_bytes(batch, heads, seq)) return ATTN_ERR_WORKSPACE;
  const attn::BwdArgs a = make_bwd(dtype, nullptr, nullptr, nullptr, o, dout, lse, nullptr, nullptr,
                                   nullptr, workspace, workspace_bytes, batch, heads, seq, seq,
                                   head_dim, nullptr, 0, 1.f, stream);
  return from_hip(attn::launch_bwd_prep(a));
}

attn_status_t attn_bwd_dkdv(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                            const void* dout, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, int batch, int heads, int seq, int head_dim,
                            int causal, float scale, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq, seq, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if ((st = check_ptrs({q, k, v, dout, dk, dv, workspace})) != ATTN_OK) return st;
  if (workspace_bytes < ws_min_bytes(batch, heads, seq)) return ATTN_ERR_WORKSPACE;
  const attn::BwdArgs a = make_bwd(dtype, q, k, v, nullptr, dout, nullptr, nullptr, dk, dv,
                                   workspace, workspace_bytes, batch, heads, seq, seq, head_dim,
                                   nullptr, causal, scale, stream);
  return from_hip(attn::launch_bwd_dkdv(a));
}

attn_status_t attn_bwd_dq(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                          const void* dout, void* dq, const void* workspace,
                          size_t workspace_bytes, int batch, int heads, int seq, int head_dim,
                          int causal, float scale, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq, seq, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if ((st = check_ptrs({q, k, v, dout, dq, workspace})) != ATTN_OK) return st;
  if (workspace_bytes < ws_min_bytes(batch, heads, seq)) return ATTN_ERR_WORKSPACE;
  const attn::BwdArgs a = make_bwd(dtype, q, k, v, nullptr, dout, nullptr, dq, nullptr, nullptr,
                                   const_cast<void*>(workspace), workspace_bytes, batch, heads,
                                   seq, seq, head_dim, nullptr, causal, scale, stream);
  return from_hip(attn::launch_bwd_dq(a));
}

attn_status_t attn_bwd(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                       const void* o, const void* dout, const float* lse, void* dq, void* dk,
                       void* dv, void* workspace, size_t workspace_bytes, int batch, int heads,
                       int seq, int head_dim, int causal, float scale, void* stream) {
  return bwd_impl(dtype, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, batch,
                  heads, seq, seq, head_dim, nullptr, causal, scale, stream);
}

attn_status_t attn_bwd_noalloc(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                               const void* o, const void* dout, const float* lse, void* dq,
                               void* dk, void* dv, int batch, int heads, int seq, int head_dim,
                               int causal, float scale, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq, seq, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if ((st = check_ptrs({q, k, v, o, dout, lse, dq, dk, dv})) != ATTN_OK) return st;
  if (ws_min_bytes(batch, heads, seq) > kScratchBytes) return ATTN_ERR_WORKSPACE;
  void* ws = scratch_base();
  if (ws == nullptr) return ATTN_ERR_HIP;
  // The largest workspace layout the array holds (make_bwd picks the dS
  // path and the query split by size, as for a caller's workspace).
  const size_t bytes = std::min(kScratchBytes, ws_rec_bytes(dtype, batch, heads, seq, seq, head_dim));
  return bwd_impl(dtype, q, k, v, o, dout, lse, dq, dk, dv, ws, bytes, batch, heads, seq, seq,
                  head_dim, nullptr, causal, scale, stream);
}

attn_status_t attn_bwd_cross(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse, void* dq,
                             void* dk, void* dv, void* workspace, size_t workspace_bytes,
                             int batch, int heads, int seq_q, int seq_k, int head_dim,
                             const int* kv_len, int causal, float scale, void* stream) {
  return bwd_impl(dtype, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, batch,
                  heads, seq_q, seq_k, head_dim, kv_len, causal, scale, stream);
}

attn_status_t attn_fwd_strided(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                               void* o, float* lse, int batch, int heads, int seq_q, int seq_k,
                               int head_dim, const int* kv_len, const long long* strides,
                               int causal, float scale, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq_q, seq_k, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if (strides == nullptr) return ATTN_ERR_INVALID_ARG;
  const int rows[4] = {seq_q, seq_k, seq_k, seq_q};
  for (int t = 0; t < 4; ++t)
    if (!check_strides(strides + 3 * t, batch, heads, rows[t], head_dim, t == 3))
      return ATTN_ERR_INVALID_ARG;
  attn::Layout lay{};
  lay.q = str3(strides);
  lay.k = str3(strides + 3);
  lay.v = str3(strides + 6);
  lay.o = str3(strides + 9);
  return fwd_impl(dtype, q, k, v, o, lse, batch, heads, seq_q, seq_k, head_dim, kv_len, causal,
                  scale, stream, &lay);
}

attn_status_t attn_bwd_strided(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                               const void* o, const void* dout, const float* lse, void* dq,
                               void* dk, void* dv, void* workspace, size_t workspace_bytes,
                               int batch, int heads, int seq_q, int seq_k, int head_dim,
                               const int* kv_len, const long long* strides, int causal,
                               float scale, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq_q, seq_k, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if (strides == nullptr) return ATTN_ERR_INVALID_ARG;
  // q, k, v, o, dout, dq, dk, dv
  const int rows[8] = {seq_q, seq_k, seq_k, seq_q, seq_q, seq_q, seq_k, seq_k};
  for (int t = 0; t < 8; ++t)
    if (!check_strides(strides + 3 * t, batch, heads, rows[t], head_dim, t >= 5))
      return ATTN_ERR_INVALID_ARG;
  attn::Layout lay{};
  lay.q = str3(strides);
  lay.k = str3(strides + 3);
  lay.v = str3(strides + 6);
  lay.o = str3(strides + 9);
  lay.dout = str3(strides + 12);
  lay.dq = str3(strides + 15);
  lay.dk = str3(strides + 18);
  lay.dv = str3(strides + 21);
  return bwd_impl(dtype, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, batch,
                  heads, seq_q, seq_k, head_dim, kv_len, causal, scale, stream, &lay);
}

attn_status_t attn_fwd_rope(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                            void* o, float* lse, void* qk_rot, int batch, int heads, int seq,
                            int head_dim, const long long* strides, const float* cos_table,
                            const float* sin_table, int table_rows, int pos_offset, int causal,
                            float scale, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq, seq, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if ((st = check_ptrs({q, k, v, o, qk_rot})) != ATTN_OK) return st;
  if (lse != nullptr && !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  if (strides == nullptr) return ATTN_ERR_INVALID_ARG;
  for (int t = 0; t < 4; ++t)
    if (!check_strides(strides + 3 * t, batch, heads, seq, head_dim, t == 3))
      return ATTN_ERR_INVALID_ARG;
  if (!check_tables(cos_table, sin_table, table_rows, pos_offset, seq)) return ATTN_ERR_INVALID_ARG;
  const size_t esz = dtype == ATTN_BF16 ? 2 : 4;
  const long long sd = (long long)seq * head_dim;
  const long long rs[3] = {heads * sd, sd, head_dim};  // [B, H, S, D] row-major
  if (!check_strides(rs, batch, heads, seq, head_dim, true)) return ATTN_ERR_INVALID_ARG;
  attn::Layout lay{};
  lay.q = str3(strides);
  lay.k = str3(strides + 3);
  lay.v = str3(strides + 6);
  lay.o = str3(strides + 9);
  // Q and K are turned inside the forward kernel as their tiles arrive; it
  // stores them turned into qk_rot for the backward
  attn::RopeTab rt;
  rt.cos = cos_table;
  rt.sin = sin_table;
  rt.pos = pos_offset;
  rt.out = qk_rot;
  rt.kout = static_cast<char*>(qk_rot) + (size_t)batch * heads * sd * esz;
  return fwd_impl(dtype, q, k, v, o, lse, batch, heads, seq, seq, head_dim, nullptr, causal,
                  scale, stream, &lay, nullptr, &rt);
}

attn_status_t attn_bwd_rope(attn_dtype_t dtype, const void* qk_rot, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes, int batch, int heads, int seq,
                            int head_dim, const long long* strides, const float* cos_table,
                            const float* sin_table, int table_rows, int pos_offset, int causal,
                            float scale, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq, seq, head_dim, causal, scale, true);
  if (st != ATTN_OK) return st;
  if (qk_rot == nullptr || !aligned16(qk_rot) || strides == nullptr) return ATTN_ERR_INVALID_ARG;
  // v, o, dout, dq, dk, dv
  for (int t = 0; t < 6; ++t)
    if (!check_strides(strides + 3 * t, batch, heads, seq, head_dim, t >= 3))
      return ATTN_ERR_INVALID_ARG;
  if (!check_tables(cos_table, sin_table, table_rows, pos_offset, seq)) return ATTN_ERR_INVALID_ARG;
  const size_t esz = dtype == ATTN_BF16 ? 2 : 4;
  const long long sd = (long long)seq * head_dim;
  const long long rs[3] = {heads * sd, sd, head_dim};
  if (!check_strides(rs, batch, heads, seq, head_dim, true)) return ATTN_ERR_INVALID_ARG;
  const void* krot = static_cast<const char*>(qk_rot) + (size_t)batch * heads * sd * esz;
  attn::Layout lay{};
  lay.q = str3(rs);
  lay.k = str3(rs);
  lay.v = str3(strides);
  lay.o = str3(strides + 3);
  lay.dout = str3(strides + 6);
  lay.dq = str3(strides + 9);
  lay.dk = str3(strides + 12);
  lay.dv = str3(strides + 15);
  attn::RopeTab rt;
  rt.cos = cos_table;
  rt.sin = sin_table;
  rt.pos = pos_offset;
  return bwd_impl(dtype, qk_rot, krot, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
                  batch, heads, seq, seq, head_dim, nullptr, causal, scale, stream, &lay, &rt);
}

attn_status_t attn_rope_copy(attn_dtype_t dtype, const void* src, const long long* src_strides,
                             void* dst, const long long* dst_strides, const float* cos_table,
                             const float* sin_table, int table_rows, int pos_offset, int batch,
                             int heads, int seq, int head_dim, int transpose, void* stream) {
  attn_status_t st = check_shape(dtype, batch, heads, seq, seq, head_dim, 0, 1.f, false);
  if (st != ATTN_OK) return st;
  if ((st = check_ptrs({src, dst})) != ATTN_OK) return st;
  if (src_strides == nullptr || dst_strides == nullptr) return ATTN_ERR_INVALID_ARG;
  if (transpose != 0 && transpose != 1) return ATTN_ERR_INVALID_ARG;
  if ((cos_table == nullptr) != (sin_table == nullptr)) return ATTN_ERR_INVALID_ARG;
  if (cos_table != nullptr) {
    if (!aligned16(cos_table) || !aligned16(sin_table)) return ATTN_ERR_INVALID_ARG;
    if (pos_offset < 0 || table_rows < 0 || (int64_t)pos_offset + seq > table_rows)
      return ATTN_ERR_INVALID_ARG;
  }
  // strides in elements: non-negative multiples of 8 (16-byte accesses),
  // and the farthest element within int64
  const int dims[3] = {batch, heads, seq};
  for (const long long* str : {src_strides, dst_strides}) {
    double far = head_dim;
    for (int i = 0; i < 3; ++i) {
      if (str[i] < 0 || str[i] % 8 != 0 || str[i] > (1LL << 48)) return ATTN_ERR_INVALID_ARG;
      far += (double)str[i] * (dims[i] - 1);
    }
    if (far > 4.0e18) return ATTN_ERR_INVALID_ARG;
  }
  attn::RopeArgs a;
  a.bf16 = dtype == ATTN_BF16;
  a.src = src;
  a.dst = dst;
  for (int i = 0; i < 3; ++i) {
    a.ss[i] = src_strides[i];
    a.ds[i] = dst_strides[i];
  }
  a.cos = cos_table;
  a.sin = sin_table;
  a.pos_offset = cos_table != nullptr ? pos_offset : 0;
  a.B = batch; a.H = heads; a.S = seq; a.D = head_dim;
  a.transpose = transpose != 0;
  a.stream = static_cast<hipStream_t>(stream);
  return from_hip(attn::launch_rope(a));
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

const char* attn_version(void) { return "0.8.0"; }

}  // extern "C"
