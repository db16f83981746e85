// attn_launch.hpp -- host-side launch descriptors passed from the C ABI
// (attn_api.hip) to the per-kernel launchers.  Arguments are validated by
// the caller; launchers only pick the compiled variant and enqueue it.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "attn_device.hpp"

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
#define ATTN_FWD_NST_BF16 2
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
// the bf16 dK+dV that forms D itself (dkdv_dfused): 2 stages
#ifndef ATTN_DKDV_NST_BF16_DF
#define ATTN_DKDV_NST_BF16_DF 2
#endif
// The dQ GEMM (dS K with the stored dS^T): waves per workgroup, waves
// sharing each 32-query block, LDS stages.  At B8 H12 S512 D64 causal the
// f32 defaults took 23.4 us against 27.9 with 3 stages, 26.3 with 8 waves
// and 29.5 without the split; bf16 measured the same with 2 stages as 3.
#ifndef ATTN_DQG_NW_F32
#define ATTN_DQG_NW_F32 4
#endif
#ifndef ATTN_DQG_NSPLIT_F32
#define ATTN_DQG_NSPLIT_F32 2
#endif
#ifndef ATTN_DQG_NST_F32
#define ATTN_DQG_NST_F32 2
#endif
#ifndef ATTN_DQG_NW_BF16
#define ATTN_DQG_NW_BF16 4
#endif
#ifndef ATTN_DQG_NSPLIT_BF16
#define ATTN_DQG_NSPLIT_BF16 2
#endif
#ifndef ATTN_DQG_NST_BF16
#define ATTN_DQG_NST_BF16 3
#endif
// Workgroups per CU the f32 dK+dV kernel (D <= 64) must fit: 2 holds its
// registers to 256, so two of its single-wave-per-SIMD workgroups share a CU.
#ifndef ATTN_DKDV_MINW_F32
#define ATTN_DKDV_MINW_F32 2
#endif
// Row steps each wave of the prep pass loads before its arithmetic.  At
// B8 H12 S512 D64 the prep kernel took 5.6 / 5.8 / 6.0 / 7.0 us (f32) and
// 4.1 / 3.9 / 4.4 / 5.3 us (bf16) with 2 / 1 / 4 / 8 steps: more, smaller
// waves start loading sooner.
#ifndef ATTN_PREP_UNR_F32
#define ATTN_PREP_UNR_F32 2
#endif
#ifndef ATTN_PREP_UNR_BF16
#define ATTN_PREP_UNR_BF16 1
#endif
// Work estimates of the static schedule, in quarter tile-steps: an item of
// the forward costs 4 per key tile plus ATTN_FWD_ITEM_COST (merge, epilogue
// and stores), an item of dK+dV 4 per query tile plus ATTN_DKDV_ITEM_COST
// (its header tile, merge and stores).
#ifndef ATTN_FWD_ITEM_COST_F32
#define ATTN_FWD_ITEM_COST_F32 0
#endif
#ifndef ATTN_FWD_ITEM_COST_BF16
#define ATTN_FWD_ITEM_COST_BF16 0
#endif
#ifndef ATTN_DKDV_ITEM_COST_F32
#define ATTN_DKDV_ITEM_COST_F32 4
#endif
#ifndef ATTN_DKDV_ITEM_COST_BF16
#define ATTN_DKDV_ITEM_COST_BF16 4
#endif
// Largest dS^T buffer the recommended backward workspace holds: 256 MiB,
// the size of the last-level cache.  Measured on MI355X (backward, causal),
// the dS path beat recomputing the scores at every length tried (f32 by
// 20-30% up to S = 8192; bf16 by 5-15% up to S = 4096 at head_dim 64 and
// 8192 at 128, and lost at S = 8192, head_dim 64); past this size the S^2
// buffer costs more memory than the gain is worth, and the recommended
// workspace becomes the O(S) minimum.
#ifndef ATTN_DS_WORKSPACE_CAP
#define ATTN_DS_WORKSPACE_CAP (256u << 20)
#endif
// Query-chunk split of the dK+dV pass (dkdv_query_chunks): shapes with
// fewer (key tile, head) items than these are split.  At B1 H16 S1024 D128
// causal (256 items, the longest walking 16 query tiles) two chunks took the
// f32 backward from 220 to 168 us; bf16 measured 58.4 us unsplit, 60.3 with
// two chunks and 77.6 with four, so it keeps the lower bound.
#ifndef ATTN_DKDV_SPLIT_BELOW_F32
#define ATTN_DKDV_SPLIT_BELOW_F32 512
#endif
#ifndef ATTN_DKDV_SPLIT_BELOW_BF16
#define ATTN_DKDV_SPLIT_BELOW_BF16 256
#endif
#ifndef ATTN_DKDV_SPLIT_TARGET
#define ATTN_DKDV_SPLIT_TARGET 512
#endif
#ifndef ATTN_DKDV_QCHUNK_MIN
#define ATTN_DKDV_QCHUNK_MIN 4
#endif
// Forward of heads with few queries: the VALU kernel of attn_fwd_small.hip
// takes heads of at most ATTN_FWD_SMALL_MAXQ_F32 queries with float32
// storage and ATTN_FWD_SMALL_MAXQ_BF16 with bf16 storage; longer ones run on
// the MFMA kernel.  One-query heads use ATTN_FWD_SMALL_NW1 waves per
// workgroup and ATTN_FWD_SMALL_U1 keys per lane row and iteration, groups
// of four queries ATTN_FWD_SMALL_NW4 and ATTN_FWD_SMALL_U4 (at D = 128 a
// half and a quarter of those keys).  Measured on MI355X at B8 H12 Sk512
// D64 causal: the VALU kernel wins at Sq = 1 in both storage types (f32
// 4.6 us, bf16 4.8 us, against 28.7 and 9.5 on the MFMA kernel) and up to
// Sq = 8 with float32 storage; 16 waves of 4 keys per row are best at
// Sq = 1, 8 waves of 16 at Sq = 4 (16 waves there exceed 128 registers per
// lane and spill).
#ifndef ATTN_FWD_SMALL_MAXQ_F32
#define ATTN_FWD_SMALL_MAXQ_F32 8
#endif
#ifndef ATTN_FWD_SMALL_MAXQ_BF16
#define ATTN_FWD_SMALL_MAXQ_BF16 1
#endif
#ifndef ATTN_FWD_SMALL_NW1
#define ATTN_FWD_SMALL_NW1 16
#endif
#ifndef ATTN_FWD_SMALL_U1
#define ATTN_FWD_SMALL_U1 4
#endif
#ifndef ATTN_FWD_SMALL_NW4
#define ATTN_FWD_SMALL_NW4 8
#endif
#ifndef ATTN_FWD_SMALL_U4
#define ATTN_FWD_SMALL_U4 16
#endif

namespace attn {

struct FwdArgs {
  bool bf16;           // bf16 storage and operands
  bool bf16_operands;  // f32 storage, bf16 MFMA operands
  const void *q, *k, *v;
  void* o;
  float* lse;  // null: not stored
  int BH, H, Sq, Sk, D;
  const int* kvlen;  // valid keys per batch (device), or null: all Sk
  bool cross;        // Sq != Sk or kvlen given: the general (cross-attention) kernels
  bool causal;
  float scale;
  hipStream_t stream;
  const Layout* layout = nullptr;  // strides of q, k, v, o; null: [B, H, S, D] row-major
  float* part = nullptr;  // key-split partials (fwd_key_split), or null: no split
  RopeTab rope;           // rope.cos null: no RoPE; else Q turned on load (strided
                          // self-attention) and stored turned to rope.out
};

struct BwdArgs {
  bool bf16;
  const void *q, *k, *v, *o, *dout;
  const float* lse;
  void *dq, *dk, *dv;
  float* delta;  // workspace: D [B*H*Sq] f32, then LSE*log2(e) [B*H*Sq] f32
  void* ds;      // workspace dS^T [B*H][SPk][SPq] (dtype), or null: dQ recomputes
  float* part;   // workspace dK, dV partials [2][nqs][B*H][Sk][D] f32, or null
  int nqs;       // query chunks of the dK+dV pass (1: no partials)
  const Layout* layout = nullptr;  // strides of every tensor; null: [B, H, S, D] row-major
  int SPq, SPk;  // query stride and key rows per head of dS^T (rounded up to the tile)
  int BH, H, Sq, Sk, D;
  const int* kvlen;
  bool cross;
  bool causal;
  float scale;
  hipStream_t stream;
  RopeTab rope;  // rope.cos null: no RoPE; else dQ and dK leave turned back
                 // (transposed rotation, query / key i at table row rope.pos + i)
  bool dfused = false;  // dK+dV forms D and LSE*log2(e) itself from O, dO and
                        // the LSE (no prep pass; the workspace's D part unused)
};

// The bf16 backward on the dS path, plain layout and no padded keys, query
// chunks or RoPE forms D inside dK+dV (its step is instruction-bound, so the
// few dot products per query tile cost less than the prep pass they replace;
// f32 keeps the pass: the O rows would not fit its register budget).
inline bool dkdv_dfused(const BwdArgs& a) {
  return a.bf16 && a.ds != nullptr && a.layout == nullptr && !a.cross &&
         !(a.part != nullptr && a.nqs > 1) && a.rope.cos == nullptr;
}

// Rotary embedding / layout pass: dst rows = R(src rows) (or R^T, or a plain
// copy without tables); element (b, h, s, d) of a tensor at
// b*strides[0] + h*strides[1] + s*strides[2] + d.
struct RopeArgs {
  bool bf16;
  const void* src;
  long long ss[3];
  void* dst;
  long long ds[3];
  const float* cos;  // [rows][D/2] f32, or null: no rotation
  const float* sin;
  int pos_offset;    // table row of sequence position 0
  int B, H, S, D;
  bool transpose;
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

// CUs per XCD of the current device (8 XCDs), cached per device.
inline int cus_per_xcd() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 8)
    ncu = 8;
  v = ncu / 8;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// The pattern of a persistent launch of G workgroups over BH heads whose
// items fall in ncls work classes (class c has one item per head, of work
// works[c]), for an XCD of cux CUs.  Items are placed largest first on the
// XCD's CU with the least total work (ties: lowest CU), on that CU's
// least-loaded slot; slots j and j + cux of an XCD share a CU (the
// dispatcher fills every CU once before it gives any a second workgroup).
// M = 0 when the pattern does not apply or fit (the kernels then use the
// snake order).  Pure host function.
inline Sched build_sched(int G, int BH, const std::vector<int>& works, int cux) {
  Sched s;
  s.M = 0;
  s.R = 0;
  const int ncls = (int)works.size();
  if (G % 8 || BH % 8 || G <= 0 || ncls <= 0) return s;
  const int M = G / 8, hx = BH / 8;
  if (M > kSchedSlots || hx > 255 || ncls > 255) return s;
  if (cux <= 0 || M % cux) cux = M;  // fewer workgroups than CUs: one per CU
  const int spc = M / cux;
  std::vector<int> order(ncls);
  for (int c = 0; c < ncls; ++c) order[c] = c;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return works[a] > works[b]; });
  std::vector<long> load(M, 0);
  std::vector<std::vector<uint16_t>> lists(M);
  for (int c : order) {
    if (works[c] <= 0) continue;  // a class without work has no items
    for (int u = 0; u < hx; ++u) {
      int bcu = 0;
      long bsum = -1;
      for (int cu = 0; cu < cux; ++cu) {
        long sum = 0;
        for (int t = 0; t < spc; ++t) sum += load[cu + cux * t];
        if (bsum < 0 || sum < bsum) { bsum = sum; bcu = cu; }
      }
      int bj = bcu;
      for (int t = 1; t < spc; ++t)
        if (load[bcu + cux * t] < load[bj]) bj = bcu + cux * t;
      load[bj] += works[c];
      lists[bj].push_back((uint16_t)((c << 8) | u));
    }
  }
  size_t R = 0;
  for (const auto& l : lists) R = std::max(R, l.size());
  if ((R - 1) * M > (size_t)kSchedEntries) return s;
  for (int j = 0; j < M; ++j) s.first[j] = lists[j].empty() ? 0xffff : lists[j][0];
  for (size_t r = 1; r < R; ++r)
    for (int j = 0; j < M; ++j) s.ent[(r - 1) * M + j] = r < lists[j].size() ? lists[j][r] : 0xffff;
  s.M = M;
  s.R = (int)R;
  return s;
}

// build_sched for the current device, cached per argument set.
inline Sched make_sched(int G, int BH, const std::vector<int>& works) {
  const int cux = cus_per_xcd();
  struct Entry { int G, BH, cux; std::vector<int> works; Sched s; };
  static std::mutex mu;
  static std::vector<Entry> cache;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : cache)
    if (e.G == G && e.BH == BH && e.cux == cux && e.works == works) return e.s;
  const Sched s = build_sched(G, BH, works, cux);
  if (cache.size() >= 32) cache.erase(cache.begin());
  cache.push_back(Entry{G, BH, cux, works, s});
  return s;
}

// Launch shape of one kernel for an element type and head_dim: NW waves per
// workgroup, NSPLIT waves sharing each 32-row block, KPW 32-row blocks per
// wave per staged tile, NST ring stages (the macros above).  head_dim-32
// tiles hold half the bytes of head_dim-64 ones: with more than 4 waves or
// 2-way splits a wave's share of a tile, or a merge's partials, would not
// fill whole 1 KiB loads or one stage, so head_dim 32 keeps 4 waves, 2-way
// splits and one block per wave.
struct LShape {
  int nw, nsplit, kpw, nst;
};
constexpr LShape small_d_shape(int nst) { return LShape{4, 2, 1, nst}; }
constexpr LShape fwd_shape(bool bf16, int D) {
  return bf16 ? (D < 64 ? small_d_shape(ATTN_FWD_NST_BF16)
                        : LShape{ATTN_FWD_NW_BF16, ATTN_FWD_NSPLIT_BF16, ATTN_FWD_KPW_BF16,
                                 ATTN_FWD_NST_BF16})
              : (D < 64 ? small_d_shape(ATTN_FWD_NST_F32)
                        : LShape{ATTN_FWD_NW_F32, ATTN_FWD_NSPLIT_F32, ATTN_FWD_KPW_F32,
                                 ATTN_FWD_NST_F32});
}
constexpr LShape dkdv_shape(bool bf16, int D) {
  return bf16 ? (D < 64 ? small_d_shape(ATTN_DKDV_NST_BF16)
                        : LShape{ATTN_DKDV_NW_BF16, ATTN_DKDV_NSPLIT_BF16, ATTN_DKDV_KPW_BF16,
                                 ATTN_DKDV_NST_BF16})
              : (D < 64 ? small_d_shape(ATTN_DKDV_NST_F32)
                        : LShape{ATTN_DKDV_NW_F32, ATTN_DKDV_NSPLIT_F32, ATTN_DKDV_KPW_F32,
                                 ATTN_DKDV_NST_F32});
}
constexpr LShape dq_shape(bool bf16, int D) {  // dQ with recomputed scores
  return bf16 ? (D < 64 ? small_d_shape(ATTN_DQ_NST_BF16)
                        : LShape{ATTN_DQ_NW_BF16, ATTN_DQ_NSPLIT_BF16, ATTN_DQ_KPW_BF16,
                                 ATTN_DQ_NST_BF16})
              : (D < 64 ? small_d_shape(ATTN_DQ_NST_F32)
                        : LShape{ATTN_DQ_NW_F32, ATTN_DQ_NSPLIT_F32, ATTN_DQ_KPW_F32,
                                 ATTN_DQ_NST_F32});
}
constexpr LShape dqg_shape(bool bf16, int D) {  // dQ GEMM over the stored dS^T
  return bf16 ? (D < 64 ? small_d_shape(ATTN_DQG_NST_BF16)
                        : LShape{ATTN_DQG_NW_BF16, ATTN_DQG_NSPLIT_BF16, 1, ATTN_DQG_NST_BF16})
              : (D < 64 ? small_d_shape(ATTN_DQG_NST_F32)
                        : LShape{ATTN_DQG_NW_F32, ATTN_DQG_NSPLIT_F32, 1, ATTN_DQG_NST_F32});
}

// Tiles of the forward kernel: queries per item, keys per staged tile.
constexpr int fwd_query_tile(bool bf16, int D) {
  return 32 * (fwd_shape(bf16, D).nw / fwd_shape(bf16, D).nsplit);
}
constexpr int fwd_key_tile(bool bf16, int D) {
  return 32 * fwd_shape(bf16, D).nsplit * fwd_shape(bf16, D).kpw;
}

// Key split of the forward for causal or non-causal self-attention whose
// longest query tile walks far more key tiles than a balanced share (few
// long heads): with W the key tiles of all items, the share of one of 256
// CUs is ceil(W / 256) tiles; when the longest query tile has more than 1.5
// shares, every query tile with more than kc = 3/4 of a share (at least 2)
// key tiles is cut into ceil(n / kc) chunks of equal size (nch = the most
// chunks), each its own
// item with partial results, merged afterwards.  A function of the shape
// alone, so that the workspace size and the launch agree; false (nch = 1):
// no split.  The chunk items need the static schedule's table, which pins
// heads to XCDs, so B*H must be a multiple of 8.
inline bool fwd_key_split(bool bf16, long long BH, int S, int D, bool causal, int& nch, int& kc) {
  nch = 1;
  kc = 1 << 30;
  if (BH % 8 != 0) return false;
  const int BR = fwd_query_tile(bf16, D), BK = fwd_key_tile(bf16, D);
  const int nqt = (S + BR - 1) / BR;
  long long W = 0;
  int longest = 0;
  for (int qt = 0; qt < nqt; ++qt) {
    const int kend = causal ? std::min(S, qt * BR + BR) : S;
    const int n = (kend + BK - 1) / BK;
    W += n;
    longest = std::max(longest, n);
  }
  W *= BH;
  const long long share0 = (W + 255) / 256;
  if (share0 < 2 || 2LL * longest <= 3 * share0 || share0 >= longest) return false;
  // chunks of three quarters of a share: more, shorter items than one share
  // each (B1 H16 S1024 D128 causal, f32: forward 69.2 -> 65.2 us; half a
  // share measured slower, 70.2)
  const long long share = std::max<long long>(2, share0 * 3 / 4);
  kc = (int)share;
  nch = (longest + kc - 1) / kc;
  return nch > 1;
}

// Tiles of the dK+dV kernel: keys per item, queries per staged tile.
constexpr int dkdv_key_tile(bool bf16, int D) {
  return 32 * (dkdv_shape(bf16, D).nw / dkdv_shape(bf16, D).nsplit);
}
constexpr int dkdv_query_tile(bool bf16, int D) {
  return 32 * dkdv_shape(bf16, D).nsplit * dkdv_shape(bf16, D).kpw;
}

// Query chunks of the dK+dV pass for a shape (a function of the shape
// alone, so that workspace sizes and launches agree).  With fewer than
// ATTN_DKDV_SPLIT_BELOW (key tile, head) items the chip would idle (many
// queries over few keys: the text cross-attention); the query tiles are then
// cut into chunks of at least ATTN_DKDV_QCHUNK_MIN tiles, towards
// ATTN_DKDV_SPLIT_TARGET items, and the chunks' partial sums are added up
// afterwards.
inline int dkdv_query_chunks(bool bf16, long long BH, int Sq, int Sk, int D) {
  const long long nkt = (Sk + dkdv_key_tile(bf16, D) - 1) / dkdv_key_tile(bf16, D);
  const int nqt = (Sq + dkdv_query_tile(bf16, D) - 1) / dkdv_query_tile(bf16, D);
  const long long items = BH * nkt;
  if (items >= (bf16 ? ATTN_DKDV_SPLIT_BELOW_BF16 : ATTN_DKDV_SPLIT_BELOW_F32)) return 1;
  long long n = (ATTN_DKDV_SPLIT_TARGET + items - 1) / items;
  n = std::min<long long>(n, nqt / ATTN_DKDV_QCHUNK_MIN);
  n = std::min<long long>(n, 64);
  if (n <= 1) return 1;
  const int qpc = (int)((nqt + n - 1) / n);
  return (nqt + qpc - 1) / qpc;  // no empty chunk
}

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_rope(const RopeArgs& a);
hipError_t launch_fwd_small(const FwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_prep(const BwdArgs& a);

}  // namespace attn
