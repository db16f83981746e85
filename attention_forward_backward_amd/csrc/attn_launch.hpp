// attn_launch.hpp -- host-side launch descriptors passed from the C ABI
// (attn_api.hip) to the per-kernel launchers.  Arguments are validated by
// the caller; launchers only pick the compiled variant and enqueue it.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

// Launch shapes per kernel and contract: NW waves per workgroup, NSPLIT
// waves sharing each 32-row block (splitting its inner loop), KPW 32-row
// blocks per wave per staged tile, NST LDS stages in the tile ring.  Defaults come from measurements on
// MI355X; a build may override them with -D for tuning sweeps.
#ifndef ATTN_FWD_NW_F32
#define ATTN_FWD_NW_F32 4
#endif
#ifndef ATTN_FWD_NSPLIT_F32
#define ATTN_FWD_NSPLIT_F32 2
#endif
#ifndef ATTN_FWD_KPW_F32
#define ATTN_FWD_KPW_F32 1
#endif
#ifndef ATTN_FWD_NW_BF16
#define ATTN_FWD_NW_BF16 4
#endif
#ifndef ATTN_FWD_NSPLIT_BF16
#define ATTN_FWD_NSPLIT_BF16 2
#endif
#ifndef ATTN_FWD_KPW_BF16
#define ATTN_FWD_KPW_BF16 1
#endif
#ifndef ATTN_DQ_NW_F32
#define ATTN_DQ_NW_F32 4
#endif
#ifndef ATTN_DQ_NSPLIT_F32
#define ATTN_DQ_NSPLIT_F32 2
#endif
#ifndef ATTN_DQ_KPW_F32
#define ATTN_DQ_KPW_F32 1
#endif
#ifndef ATTN_DQ_NW_BF16
#define ATTN_DQ_NW_BF16 4
#endif
#ifndef ATTN_DQ_NSPLIT_BF16
#define ATTN_DQ_NSPLIT_BF16 2
#endif
#ifndef ATTN_DQ_KPW_BF16
#define ATTN_DQ_KPW_BF16 1
#endif
#ifndef ATTN_DKDV_NW_F32
#define ATTN_DKDV_NW_F32 4
#endif
#ifndef ATTN_DKDV_NSPLIT_F32
#define ATTN_DKDV_NSPLIT_F32 2
#endif
#ifndef ATTN_DKDV_KPW_F32
#define ATTN_DKDV_KPW_F32 1
#endif
#ifndef ATTN_DKDV_NW_BF16
#define ATTN_DKDV_NW_BF16 4
#endif
#ifndef ATTN_DKDV_NSPLIT_BF16
#define ATTN_DKDV_NSPLIT_BF16 2
#endif
#ifndef ATTN_DKDV_KPW_BF16
#define ATTN_DKDV_KPW_BF16 1
#endif
#ifndef ATTN_FWD_NST_F32
#define ATTN_FWD_NST_F32 2
#endif
#ifndef ATTN_FWD_NST_BF16
#define ATTN_FWD_NST_BF16 3
#endif
#ifndef ATTN_DQ_NST_F32
#define ATTN_DQ_NST_F32 2
#endif
#ifndef ATTN_DQ_NST_BF16
#define ATTN_DQ_NST_BF16 3
#endif
#ifndef ATTN_DKDV_NST_F32
#define ATTN_DKDV_NST_F32 2
#endif
#ifndef ATTN_DKDV_NST_BF16
#define ATTN_DKDV_NST_BF16 3
#endif
// Workgroups per CU the f32 dK+dV kernel (D <= 64) must fit: 2 holds its
// registers to 256, so two of its single-wave-per-SIMD workgroups share a CU.
#ifndef ATTN_DKDV_MINW_F32
#define ATTN_DKDV_MINW_F32 2
#endif

namespace attn {

struct FwdArgs {
  bool bf16;
  const void *q, *k, *v;
  void* o;
  float* lse;
  int BH, S, D;
  bool causal;
  float scale;
  hipStream_t stream;
};

struct BwdArgs {
  bool bf16;
  const void *q, *k, *v, *o, *dout;
  const float* lse;
  void *dq, *dk, *dv;
  float* delta;  // workspace: D [B*H*S] f32, then LSE*log2(e) [B*H*S] f32
  void* ds;      // workspace dS^T [B*H][SP][SP] (dtype), or null: dQ recomputes
  int SP;        // row stride of dS (S rounded up to the key tile)
  int BH, S, D;
  bool causal;
  float scale;
  hipStream_t stream;
};

// Workgroups of kernel Kern (launched with `threads` threads and no dynamic
// LDS) that the current device holds at once: CUs x resident workgroups per
// CU.  Persistent kernels launch this many (or fewer) workgroups.  Queried
// once per device and cached; falls back to one per CU if a query fails.
template <auto Kern>
inline int resident_workgroups(int threads) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int ncu = 0, nb = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    ncu = 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(Kern), threads, 0) !=
          hipSuccess ||
      nb <= 0)
    nb = 1;
  v = ncu * nb;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_prep(const BwdArgs& a);

}  // namespace attn
