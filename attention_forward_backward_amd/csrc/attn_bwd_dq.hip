// attn_bwd_dq.hip -- first backward kernel for gfx950: D and dQ.
//
// The pages ("Meganeura: Portable GPU Training and Inference through Vulkan
// and Metal", arXiv 2608.01563) lower the attention derivative to a dQ
// kernel and a fused dK+dV kernel (Section 3.3; profiled as FlashGradQ and
// FlashGradKV in Section 7.3).  This is the dQ kernel:
//   D_i  = sum_d dO_id O_id                      (written to the workspace)
//   P_ij = exp(scale * Q_i.K_j - LSE_i)          (recomputed from the LSE)
//   dQ_i = scale * sum_j P_ij (dO_i.V_j - D_i) K_j
// It owns its query rows outright, so dQ needs no atomics and no partial
// sums: the price is recomputing the two score-shaped products that the
// dK+dV kernel also forms.
//
// Work split: one workgroup per (query tile of 32*NW rows, batch*head), one
// wave per 32 queries, key tiles of BK keys staged in LDS and shared.  Per
// 32-key block a wave forms S^T = K Q^T and dP^T = V dO^T (keys x queries;
// each lane holds one query, so LSE_i and D_i are one register each), then
// dS^T = P^T o (dP^T - D) in registers, which is the A operand of
// dQ (queries x d) += dS K with K read back from the same LDS tile.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {

template <class E, int D, int NW, int BK, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ O,
    const typename E::T* __restrict__ dO, const float* __restrict__ LSE,
    typename E::T* __restrict__ dQ, float* __restrict__ Dws, int S, float c, float scale) {
  using T = typename E::T;
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;
  constexpr int NDB = D / 32;
  constexpr int NKB = BK / 32;
  constexpr int STR = row_stride<E, D>();
  constexpr int STRT = tr_stride<BK>();
  constexpr int T_ELEMS = BK * STR;
  constexpr int KT_ELEMS = is_bf16<E>() ? D * STRT : 0;
  __shared__ __attribute__((aligned(16))) T smem[2 * T_ELEMS + KT_ELEMS];
  T* Ks = smem;                 // [key][d]
  T* Vs = smem + T_ELEMS;       // [key][d]
  T* KsT = smem + 2 * T_ELEMS;  // bf16 only: [d][key]

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, n = lane & 31;
  const int bh = blockIdx.x;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;
  const size_t base = (size_t)bh * S * D;
  const T* k = K + base;
  const T* v = V + base;

  const int q0 = qt * BR + w * 32;
  const int qi = q0 + n;
  const bool wave_active = q0 < S;
  const bool qvalid = qi < S;
  const size_t qrow = base + (size_t)min(qi, S - 1) * D + h * (D / 2);

  RowFrag<E, D> qf, dof;
  load_row_frag<E, D>(qf, Q + qrow, qvalid);
  load_row_frag<E, D>(dof, dO + qrow, qvalid);

  // D_i = sum_d dO_id O_id: this lane's half row, then the other half.
  float di = 0.f;
  {
    RowFrag<E, D> of;
    load_row_frag<E, D>(of, O + qrow, qvalid);
#pragma unroll
    for (int s = 0; s < RowFrag<E, D>::NS; ++s) {
      if constexpr (is_bf16<E>()) {
#pragma unroll
        for (int t = 0; t < 8; ++t) di += (float)dof.f[s][t] * (float)of.f[s][t];
      } else {
        di += dof.f[s] * of.f[s];
      }
    }
    di += xhalf(di);
  }
  if (qvalid && h == 0) Dws[(size_t)bh * S + qi] = di;
  const float lse2 = qvalid ? LSE[(size_t)bh * S + qi] * kLog2e : 0.f;

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = zero16();

  const int kend = CAUSAL ? min(S, qt * BR + BR) : S;
  const int nkt = (kend + BK - 1) / BK;

  TileRegs<T, BK, D, NT> kr, vr;
  kr.load(k, 0, S, tid);
  vr.load(v, 0, S, tid);

  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    kr.template store<STR>(Ks, tid);
    vr.template store<STR>(Vs, tid);
    if constexpr (is_bf16<E>()) kr.template store_t<STRT>(KsT, tid);
    __syncthreads();
    if (kt + 1 < nkt) {
      kr.load(k, (kt + 1) * BK, S, tid);
      vr.load(v, (kt + 1) * BK, S, tid);
    }
    if (!wave_active) continue;

#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int kk0 = kt * BK + kb * 32;
      if (!(kk0 < S && (!CAUSAL || kk0 <= q0 + 31))) continue;  // wave-uniform
      const int arow = (kb * 32 + pi32(n)) * STR + h * (D / 2);
      f32x16 st = dot_rows<E, D>(Ks + arow, qf, zero16());
      f32x16 dpt = dot_rows<E, D>(Vs + arow, dof, zero16());
      if (kk0 + 32 > S || (CAUSAL && kk0 + 31 > q0)) {
        // key(r) = kk0 + 8h + (16*(r/8) + r%8); visible iff key < S and key <= qi
        const int lim = min(S - 1, CAUSAL ? qi : S - 1) - kk0 - 8 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * (r >> 3) + (r & 7) > lim) st[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(st[r], c, -lse2));  // 0 where masked
        st[r] = p * (dpt[r] - di);                            // dS^T
      }
      RegOperand<E> dS;
      dS.set(st);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = second_product<E, STR, STRT, true>(dS, Ks, KsT, kb * 32, db * 32 + n, h, acc[db]);
    }
  }

  if (!wave_active) return;
  // acc[db] element r: dQ[q0 + out_row(r, h)][db*32 + n]
  T* dq = dQ + base;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = q0 + out_row(r, h);
    if (row < S) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) dq[(size_t)row * D + db * 32 + n] = (T)(acc[db][r] * scale);
    }
  }
}

template <class E, int D, bool CAUSAL>
static hipError_t launch(const BwdArgs& a) {
  constexpr int NW = 4;
  constexpr int BK = D == 128 ? 32 : 64;
  using T = typename E::T;
  const int nqt = (a.S + NW * 32 - 1) / (NW * 32);
  dim3 grid(a.BH, nqt);
  hipLaunchKernelGGL((bwd_dq_kernel<E, D, NW, BK, CAUSAL>), grid, dim3(NW * 64), 0, a.stream,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.o,
                     (const T*)a.dout, a.lse, (T*)a.dq, a.delta, a.S, a.scale * kLog2e, a.scale);
  return hipGetLastError();
}

template <class E, int D>
static hipError_t launch_c(const BwdArgs& a) {
  return a.causal ? launch<E, D, true>(a) : launch<E, D, false>(a);
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
