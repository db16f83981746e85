// attn_bwd_dq.hip -- the dQ stage of the attention backward for gfx950.
//
// The pages ("Meganeura: Portable GPU Training and Inference through Vulkan
// and Metal", arXiv 2608.01563) lower the attention derivative to a dQ
// kernel and a fused dK+dV kernel (Section 3.3; profiled as FlashGradQ and
// FlashGradKV in Section 7.3).  This file holds the two ways to form
//   dQ_i = scale * sum_j dS_ij K_j,   dS_ij = P_ij (dO_i.V_j - D_i)
// without atomics or partial sums in device memory:
//  * bwd_dq_gemm_kernel: when the workspace can hold dS (stored transposed,
//    dS^T [key][query], by the dK+dV kernel), dQ is a causal-blocked GEMM;
//  * bwd_dq_kernel: otherwise the dQ kernel recomputes P (from the LSE) and
//    dP per key tile, as the pages' separate dQ kernel does; a workgroup
//    owns its query rows outright.  The price is recomputing the two
//    score-shaped products that the dK+dV kernel also forms.
// D_i and LSE_i*log2(e) come from the workspace (the prep kernel).
//
// Recompute kernel work split: one workgroup per (query tile of 32*RB rows,
// batch*head); each
// 32-query block is owned by NSPLIT waves that split the key blocks between
// them and sum their partial dQ through LDS at the end.  K and V stream
// through an NST-stage ring of LDS tiles filled by direct global->LDS loads
// issued NST-1 tiles ahead (one barrier per tile).  Per 32-key block a wave
// forms S^T = K Q^T and dP^T = V dO^T (keys x queries; each lane holds one
// query, so LSE_i and D_i are one register each), then
// dS^T = P^T o (dP^T - D) in registers, which is the B operand of
// dQ^T (d x queries) += K^T dS^T with K read back from the same LDS tile:
// each lane accumulates the d values of its own query, so dQ leaves in
// 16-byte (f32) or 8-byte (bf16) row stores.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {

template <class E, int D, int NW, int NSPLIT, int KPW, int NST, bool CAUSAL, bool CROSS, bool STR,
          bool ROPE>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    typename E::T* __restrict__ dQ, const float* __restrict__ Dws, int Sq, int Sk_, int Lws,
    float c, float scale, int H, const int* __restrict__ kvlen, const Layout lay,
    const RopeTab rope) {
  // STR: Q, K, V, dO, dQ are laid out by `lay` (else [B, H, S, D] row-major).
  // ROPE (STR): Q and K hold RoPE-turned rows; dQ leaves turned back by the
  // transposed rotation of query i (table row rope.pos + i).
  // Queries Sq, keys Sk (one length in self-attention, CROSS = false); key j
  // is visible from query i iff j < L and, when causal, j <= i + off
  // (head_keys).  Lws: offset of LSE*log2(e) in the workspace (B*H*Sq).
  using T = typename E::T;
  using TL = Tile<E, D>;
  constexpr int RB = NW / NSPLIT;        // 32-query blocks per workgroup
  constexpr int BR = 32 * RB;
  constexpr int BK = 32 * NSPLIT * KPW;  // keys per staged tile
  constexpr int NDB = D / 32;
  using LD = StageLoader<E, D, BK, NW>;
  constexpr int TILEB = BK * TL::ROWB;  // one matrix tile; V follows K in a stage
  constexpr int COMB = RB * (NSPLIT - 1) * 16 * NDB * 64 * 4;
  constexpr int SMEM = NST * LD::BYTES > COMB ? NST * LD::BYTES : COMB;
  static_assert(NW % NSPLIT == 0 && NST >= 2 && NST <= 4, "launch shape");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar
  const int qb = w / NSPLIT, sp = w % NSPLIT;
  const int bh = blockIdx.x;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;
  const int Sk = CROSS ? Sk_ : Sq;
  const size_t base = (size_t)bh * Sq * D;
  const T* k = K + head_off<STR, D>(lay.k, bh, H, Sk);
  const T* v = V + head_off<STR, D>(lay.v, bh, H, Sk);
  const int ldk = row_ld<STR, D>(lay.k), ldv = row_ld<STR, D>(lay.v);
  int L, off;
  head_keys<CROSS>(kvlen, bh, H, Sq, Sk, L, off);
  const int krows = CROSS ? max(L, 1) : Sk;  // key rows the loads may read

  const int q0 = qt * BR + qb * 32;
  const int qi = q0 + n;
  const bool wave_active = q0 < Sq;
  const bool qvalid = qi < Sq;
  const size_t qrow = base + (size_t)min(qi, Sq - 1) * D + h * (D / 2);

  RowFrag<E, D> qf, dof;
  if constexpr (STR) {
    const size_t r = (size_t)min(qi, Sq - 1);
    load_row_frag<E, D>(qf, Q + head_off<STR, D>(lay.q, bh, H, Sq) + r * lay.q.s + h * (D / 2),
                        qvalid);
    load_row_frag<E, D>(dof,
                        dO + head_off<STR, D>(lay.dout, bh, H, Sq) + r * lay.dout.s + h * (D / 2),
                        qvalid);
  } else {
    load_row_frag<E, D>(qf, Q + qrow, qvalid);
    load_row_frag<E, D>(dof, dO + qrow, qvalid);
  }
  // D_i and LSE_i*log2(e), written by the prep kernel
  const float di = qvalid ? Dws[(size_t)bh * Sq + qi] : 0.f;
  const float lse2 = qvalid ? Dws[(size_t)Lws + (size_t)bh * Sq + qi] : 0.f;

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = zero16();

  const int kend = CAUSAL ? min(L, qt * BR + BR + off) : L;
  const int nkt = max((kend + BK - 1) / BK, 0);

  const unsigned lo = STR ? 0u : LD::lane_offset(w, lane);
  auto issue_kv = [&](char* st, int row0) __attribute__((always_inline)) {
    if constexpr (STR)
      LD::issue_ld(st, k, ldk, v, ldv, row0, krows, w, lane);
    else
      LD::issue(st, k, v, row0, krows, w, lane, lo, lo);
  };
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nkt) issue_kv(smem + s * LD::BYTES, s * BK);

  // One staged tile of keys.  When the stages' LDS addresses fit 16-bit
  // offsets, the loop is unrolled by NST with the stage index constant.
  auto step = [&](const int kt, auto sc) __attribute__((always_inline)) {
    const int si = sc;  // kt % NST
    wait_tiles<LD::NLOADS>(min(NST - 2, nkt - 1 - kt));
    lds_barrier();  // tile kt is in LDS; every wave is done with tile kt-1
    if (kt + NST - 1 < nkt) issue_kv(smem + ((kt + NST - 1) % NST) * LD::BYTES, (kt + NST - 1) * BK);
    if (!wave_active) return;
    const char* Kt = smem + si * LD::BYTES;
    const char* Vt = Kt + TILEB;

#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int kb = sp + NSPLIT * j;
      const int kk0 = kt * BK + kb * 32;
      if (!(kk0 < L && (!CAUSAL || kk0 <= q0 + 31 + off))) continue;  // wave-uniform
      const int arow = kb * 32 + pi32(n);
      f32x16 st = dot_tile<E, D>(Kt, arow, h, qf, zero16());
      f32x16 dpt = dot_tile<E, D>(Vt, arow, h, dof, zero16());
      if (kk0 + 32 > L || (CAUSAL && kk0 + 31 > q0 + off)) {
        // key(r) = kk0 + 8h + (16*(r/8) + r%8); visible iff key < L and key <= qi + off
        const int lim = min(L - 1, CAUSAL ? qi + off : L - 1) - kk0 - 8 * h;
        // -inf where 16*(r/8) + r%8 > lim, built arithmetically (no
        // per-element compare masks in scalar registers); the whole vector
        // is bit-cast (a bit_cast of one ext_vector element is not reliable)
        u32x16 sb = __builtin_bit_cast(u32x16, st);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const unsigned out = (unsigned)((lim - (16 * (r >> 3) + (r & 7))) >> 31);
          sb[r] = (sb[r] & ~out) | (0xff800000u & out);
        }
        st = __builtin_bit_cast(f32x16, sb);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // 0 where masked (a row with no visible key has lse2 = 0 from the
        // prep pass and only masked keys)
        const float p = fast_exp2(fmaf(st[r], c, -lse2));
        st[r] = p * (dpt[r] - di);                            // dS^T
      }
      RegOperand<E> dS;
      dS.set(st);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = second_tile<E, D, false>(dS, Kt, kb * 32, db * 32, lane, acc[db]);
    }
  };
  if constexpr (NST * LD::BYTES <= 65536) {
    for_stages<NST>(nkt, step);
  } else {
    for (int kt = 0; kt < nkt; ++kt) step(kt, kt % NST);
  }

  // Sum the NSPLIT partial dQ of each query block through LDS.
  if constexpr (NSPLIT > 1) {
    float* cb = reinterpret_cast<float*>(smem);
    lds_barrier();  // every wave is done with the tiles (no loads pending)
    // four values per 16-byte LDS access: group q of lane l at float (q * 64 + l) * 4
    if (sp != 0 && wave_active) {
      f32x4* dst = reinterpret_cast<f32x4*>(cb + ((qb * (NSPLIT - 1) + sp - 1) * 16 * NDB) * 64) + lane;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          dst[(db * 4 + j) * 64] =
              f32x4{acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2], acc[db][4 * j + 3]};
    }
    lds_barrier();
    if (sp != 0) return;
    if (wave_active) {
#pragma unroll
      for (int p = 0; p < NSPLIT - 1; ++p) {
        const f32x4* src =
            reinterpret_cast<const f32x4*>(cb + ((qb * (NSPLIT - 1) + p) * 16 * NDB) * 64) + lane;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 x = src[(db * 4 + j) * 64];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[db][4 * j + e] += x[e];
          }
      }
    }
  }
  if (!wave_active) return;
  // acc[db] holds dQ^T: element r is query q0 + n, column db*32 + out_row(r, h),
  // so elements 4j .. 4j+3 are four consecutive columns (one store)
  T* dq = STR ? dQ + head_off<STR, D>(lay.dq, bh, H, Sq) : dQ + base;
  const int lddq = row_ld<STR, D>(lay.dq);
  if (qvalid) {
    float qs = scale;
    if constexpr (ROPE) {  // dQ of the turned rows, scaled, then turned back in f32
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= scale;
      const size_t tr = (size_t)(rope.pos + qi) * (D / 2);
      rope_back_acc<D>(acc, rope.cos + tr, rope.sin + tr, h);
      qs = 1.f;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store4<T>(dq + (size_t)qi * lddq + db * 32 + 8 * j + 4 * h, acc[db][4 * j] * qs,
                  acc[db][4 * j + 1] * qs, acc[db][4 * j + 2] * qs, acc[db][4 * j + 3] * qs);
  }
}

// dQ = scale * dS K from the stored dS^T.  One workgroup per (query tile of
// 32*RB rows, batch*head); each 32-query block is owned by NSPLIT waves that
// split the key blocks and sum their partials through LDS.  A staged tile is
// the dS^T block [32*NSPLIT*KPW keys x queries] and the matching K rows; both
// operands are read in the k-slot layout (keys on k) the second products of
// the other kernels use.
// Blocks with no visible key (above the causal diagonal, or past S) are
// skipped; the dK+dV kernel wrote exact zeros for every masked entry and
// every key past S inside the blocks it processed.
template <class E, int D, int NW, int NSPLIT, int KPW, int NST, bool CAUSAL, bool CROSS, bool STR,
          bool ROPE>
__global__ __launch_bounds__(NW * 64) void bwd_dq_gemm_kernel(
    const typename E::T* __restrict__ K, const typename E::T* __restrict__ dST,
    typename E::T* __restrict__ dQ, int Sq, int Sk_, int SPq, int SPk, float scale, int H,
    const int* __restrict__ kvlen, const Layout lay, const RopeTab rope) {
  // STR: K and dQ are laid out by `lay` (dS^T is the packed workspace).
  // ROPE: as in bwd_dq_kernel.
  using T = typename E::T;
  constexpr int RB = NW / NSPLIT;
  constexpr int BR = 32 * RB;
  constexpr int BK = 32 * NSPLIT * KPW;
  constexpr int NDB = D / 32;
  using LDS_ = TileLoader<E, BR, BK, NW>;  // dS^T block: BK keys x BR queries
  using LDK = TileLoader<E, D, BK, NW>;    // K rows:   BK keys x D
  constexpr int STAGE = LDS_::BYTES + LDK::BYTES;
  constexpr int NL = LDS_::NLOADS + LDK::NLOADS;
  constexpr int COMB = RB * (NSPLIT - 1) * 16 * NDB * 64 * 4;
  constexpr int SMEM = NST * STAGE > COMB ? NST * STAGE : COMB;
  static_assert(NW % NSPLIT == 0 && NST >= 2 && NST <= 4, "launch shape");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar
  const int qb = w / NSPLIT, sp = w % NSPLIT;
  const int bh = blockIdx.x;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;
  const int Sk = CROSS ? Sk_ : Sq;
  const T* k = K + head_off<STR, D>(lay.k, bh, H, Sk);
  const int ldk = row_ld<STR, D>(lay.k);
  const T* dst_ = dST + (size_t)bh * SPk * SPq;
  int L, off;  // key j is visible from query i iff j < L and (causal) j <= i + off
  head_keys<CROSS>(kvlen, bh, H, Sq, Sk, L, off);
  const int krows = CROSS ? max(L, 1) : Sk;  // key rows the loads may read
  const int qw0 = qt * BR;         // first query of the workgroup
  const int q0 = qw0 + qb * 32;    // first query of this wave's block
  const bool wave_active = q0 < Sq;
  RopeAccRow<D> rrow;  // (ROPE) angles of query q0 + n, fetched ahead of the tiles
  if constexpr (ROPE) {
    const size_t tr = (size_t)(rope.pos + min(q0 + n, Sq - 1)) * (D / 2);
    rrow.load(rope.cos + tr, rope.sin + tr, h);
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = zero16();

  const int kend = CAUSAL ? min(L, qw0 + BR + off) : L;
  const int nkt = max((kend + BK - 1) / BK, 0);
  const unsigned los = LDS_::lane_offset(SPq, w, lane), lok = LDK::lane_offset(ldk, w, lane);
  auto issue = [&](int t) __attribute__((always_inline)) {
    char* st = smem + (t % NST) * STAGE;
    LDS_::issue(st, dst_, SPq, t * BK, SPk, qw0, w, lane, los);
    LDK::issue(st + LDS_::BYTES, k, ldk, t * BK, krows, 0, w, lane, lok);
  };
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nkt) issue(s);

  auto step = [&](const int kt, auto sc) __attribute__((always_inline)) {
    const int si = sc;  // kt % NST
    wait_tiles<NL>(min(NST - 2, nkt - 1 - kt));
    lds_barrier();
    // The next tile's loads go out after the first product of the step is
    // issued, and the products run at raised wave priority: together (not
    // either alone) 23.0 -> 22.3 us for f32 at B8 H12 S512 D64 causal.
    bool issued = false;
    if (!wave_active) {
      if (kt + NST - 1 < nkt) issue(kt + NST - 1);
      return;
    }
    const char* St = smem + si * STAGE;
    const char* Kt = St + LDS_::BYTES;
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int kb = sp + NSPLIT * j;
      const int kk0 = kt * BK + kb * 32;
      if (!(kk0 < L && (!CAUSAL || kk0 <= q0 + 31 + off))) continue;  // wave-uniform
      RegOperand<E> R;  // dS[q0 + n][keys]: k-slots from the dS^T rows
      read_kslot_operand<E, BR>(R, St, kb * 32, qb * 32, lane);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        acc[db] = second_tile<E, D, false>(R, Kt, kb * 32, db * 32, lane, acc[db]);
        if (db == 0 && !issued) {
          __builtin_amdgcn_sched_barrier(0);
          if (kt + NST - 1 < nkt) issue(kt + NST - 1);
          __builtin_amdgcn_sched_barrier(0);
          issued = true;
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
    if (!issued && kt + NST - 1 < nkt) issue(kt + NST - 1);
  };
  if constexpr (NST * STAGE <= 65536) {
    for_stages<NST>(nkt, step);
  } else {
    for (int kt = 0; kt < nkt; ++kt) step(kt, kt % NST);
  }

  if constexpr (NSPLIT > 1) {
    float* cb = reinterpret_cast<float*>(smem);
    lds_barrier();
    // four values per 16-byte LDS access: group q of lane l at float (q * 64 + l) * 4
    if (sp != 0 && wave_active) {
      f32x4* dst = reinterpret_cast<f32x4*>(cb + ((qb * (NSPLIT - 1) + sp - 1) * 16 * NDB) * 64) + lane;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          dst[(db * 4 + j) * 64] =
              f32x4{acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2], acc[db][4 * j + 3]};
    }
    lds_barrier();
    if (sp != 0) return;
    if (wave_active) {
#pragma unroll
      for (int p = 0; p < NSPLIT - 1; ++p) {
        const f32x4* src =
            reinterpret_cast<const f32x4*>(cb + ((qb * (NSPLIT - 1) + p) * 16 * NDB) * 64) + lane;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 x = src[(db * 4 + j) * 64];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[db][4 * j + e] += x[e];
          }
      }
    }
  }
  if (!wave_active) return;
  // acc[db] holds dQ^T: element r is query q0 + n, column db*32 + out_row(r, h)
  T* dq = dQ + head_off<STR, D>(lay.dq, bh, H, Sq);
  const int lddq = row_ld<STR, D>(lay.dq);
  const int qi = q0 + n;
  if (qi < Sq) {
    float qs = scale;
    if constexpr (ROPE) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= scale;
      rrow.apply(acc);
      qs = 1.f;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store4<T>(dq + (size_t)qi * lddq + db * 32 + 8 * j + 4 * h, acc[db][4 * j] * qs,
                  acc[db][4 * j + 1] * qs, acc[db][4 * j + 2] * qs, acc[db][4 * j + 3] * qs);
  }
}

template <class E, int D, bool CAUSAL, bool CROSS, bool STR, bool ROPE = false>
static hipError_t launch_gemm(const BwdArgs& a) {
  constexpr LShape SH = dqg_shape(is_bf16<E>(), D);
  constexpr int NW = SH.nw, NSPLIT = SH.nsplit, KPW = SH.kpw, NST = SH.nst;
  using T = typename E::T;
  constexpr int BR = 32 * (NW / NSPLIT);
  const int nqt = (a.Sq + BR - 1) / BR;
  dim3 grid(a.BH, nqt);
  hipLaunchKernelGGL((bwd_dq_gemm_kernel<E, D, NW, NSPLIT, KPW, NST, CAUSAL, CROSS, STR, ROPE>),
                     grid, dim3(NW * 64), 0, a.stream, (const T*)a.k, (const T*)a.ds, (T*)a.dq,
                     a.Sq, a.Sk, a.SPq, a.SPk, a.scale, a.H, a.kvlen,
                     a.layout != nullptr ? *a.layout : Layout{}, a.rope);
  return hipGetLastError();
}

template <class E, int D, bool CAUSAL, bool CROSS, bool STR, bool ROPE = false>
static hipError_t launch(const BwdArgs& a) {
  constexpr LShape SH = dq_shape(is_bf16<E>(), D);
  constexpr int NW = SH.nw, NSPLIT = SH.nsplit, KPW = SH.kpw, NST = SH.nst;
  using T = typename E::T;
  constexpr int BR = 32 * (NW / NSPLIT);
  const int nqt = (a.Sq + BR - 1) / BR;
  dim3 grid(a.BH, nqt);
  hipLaunchKernelGGL((bwd_dq_kernel<E, D, NW, NSPLIT, KPW, NST, CAUSAL, CROSS, STR, ROPE>), grid,
                     dim3(NW * 64), 0, a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                     (const T*)a.dout, (T*)a.dq, a.delta, a.Sq, a.Sk, a.BH * a.Sq,
                     a.scale * kLog2e, a.scale, a.H, a.kvlen,
                     a.layout != nullptr ? *a.layout : Layout{}, a.rope);
  return hipGetLastError();
}

// (strided layouts run the cross-attention instantiation)
template <class E, int D, bool CAUSAL>
static hipError_t launch_x(const BwdArgs& a) {
  if (a.rope.cos != nullptr)
    return a.ds != nullptr ? launch_gemm<E, D, CAUSAL, true, true, true>(a)
                           : launch<E, D, CAUSAL, true, true, true>(a);
  if (a.ds != nullptr) {
    if (a.layout != nullptr) return launch_gemm<E, D, CAUSAL, true, true>(a);
    return a.cross ? launch_gemm<E, D, CAUSAL, true, false>(a)
                   : launch_gemm<E, D, CAUSAL, false, false>(a);
  }
  if (a.layout != nullptr) return launch<E, D, CAUSAL, true, true>(a);
  return a.cross ? launch<E, D, CAUSAL, true, false>(a) : launch<E, D, CAUSAL, false, false>(a);
}

template <class E, int D>
static hipError_t launch_c(const BwdArgs& a) {
  return a.causal ? launch_x<E, D, true>(a) : launch_x<E, D, false>(a);
}

template <class E>
static hipError_t launch_d(const BwdArgs& a) {
  switch (a.D) {
    case 32: return launch_c<E, 32>(a);
    case 64: return launch_c<E, 64>(a);
    case 128: return launch_c<E, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_dq(const BwdArgs& a) {
  return a.bf16 ? launch_d<EBF16>(a) : launch_d<EF32>(a);
}

}  // namespace attn
