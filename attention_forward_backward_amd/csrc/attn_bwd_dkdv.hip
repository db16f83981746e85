// attn_bwd_dkdv.hip -- fused dK+dV backward kernel for gfx950.
//
// The pages ("Meganeura: Portable GPU Training and Inference through Vulkan
// and Metal", arXiv 2608.01563) make one fused dK+dV kernel the invariant
// for the attention derivative (Section 8; kernel list in Section 3.3,
// FlashGradKV in the Section 7.3 profile).  For each key row j:
//   P_ij  = exp(scale * Q_i.K_j - LSE_i)
//   dV_j  = sum_i P_ij dO_i
//   dK_j  = scale * sum_i P_ij (dO_i.V_j - D_i) Q_i
// with D_i from the workspace (written by the dQ kernel).
//
// Work split: one workgroup per (key tile of 32*NW rows, batch*head), one
// wave per 32 keys whose K and V rows stay in registers, and dK, dV
// accumulated in registers over all query tiles (BQ queries each, staged in
// LDS with their LSE and D and shared by the waves).  Per 32-query block a
// wave forms S = Q K^T and dP = dO V^T (queries x keys; each lane holds one
// key), then P^T and dS^T are the register A operands of
// dV (keys x d) += P^T dO and dK += dS^T Q, with dO and Q read back from LDS.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {

template <class E, int D, int NW, int BQ, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dws,
    typename E::T* __restrict__ dK, typename E::T* __restrict__ dV, int S, float c,
    float scale) {
  using T = typename E::T;
  constexpr int NT = NW * 64;
  constexpr int BKV = NW * 32;
  constexpr int NDB = D / 32;
  constexpr int NQB = BQ / 32;
  constexpr int STR = row_stride<E, D>();
  constexpr int STRT = tr_stride<BQ>();
  constexpr int T_ELEMS = BQ * STR;
  constexpr int TT_ELEMS = is_bf16<E>() ? D * STRT : 0;
  __shared__ __attribute__((aligned(16))) T smem[2 * T_ELEMS + 2 * TT_ELEMS];
  __shared__ __attribute__((aligned(16))) float stat[2 * BQ];
  T* Qs = smem;                                // [query][d]
  T* dOs = smem + T_ELEMS;                     // [query][d]
  T* QsT = smem + 2 * T_ELEMS;                 // bf16 only: [d][query]
  T* dOsT = smem + 2 * T_ELEMS + TT_ELEMS;     // bf16 only: [d][query]
  float* lse2s = stat;                         // LSE * log2(e); +inf past S
  float* Ds = stat + BQ;                       // D; 0 past S

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, n = lane & 31;
  const int bh = blockIdx.x;
  const int kt = blockIdx.y;  // causal: tile 0 has the most queries, dispatched first
  const size_t base = (size_t)bh * S * D;
  const T* q = Q + base;
  const T* dout = dO + base;
  const float* lse = LSE + (size_t)bh * S;
  const float* dws = Dws + (size_t)bh * S;

  const int k0 = kt * BKV + w * 32;
  const int kj = k0 + n;
  const bool wave_active = k0 < S;
  const size_t krow = base + (size_t)min(kj, S - 1) * D + h * (D / 2);

  RowFrag<E, D> kf, vf;
  load_row_frag<E, D>(kf, K + krow, kj < S);
  load_row_frag<E, D>(vf, V + krow, kj < S);

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dkacc[i] = zero16();
    dvacc[i] = zero16();
  }

  const int nqt = (S + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? (kt * BKV) / BQ : 0;

  TileRegs<T, BQ, D, NT> qr, dor;
  float st_lse = 0.f, st_d = 0.f;
  auto load_tile = [&](int qt) {
    qr.load(q, qt * BQ, S, tid);
    dor.load(dout, qt * BQ, S, tid);
    if (tid < BQ) {
      const int qi = qt * BQ + tid;
      st_lse = qi < S ? lse[qi] * kLog2e : INFINITY;
      st_d = qi < S ? dws[qi] : 0.f;
    }
  };
  if (qt0 < nqt) load_tile(qt0);

  for (int qt = qt0; qt < nqt; ++qt) {
    __syncthreads();
    qr.template store<STR>(Qs, tid);
    dor.template store<STR>(dOs, tid);
    if constexpr (is_bf16<E>()) {
      qr.template store_t<STRT>(QsT, tid);
      dor.template store_t<STRT>(dOsT, tid);
    }
    if (tid < BQ) {
      lse2s[tid] = st_lse;
      Ds[tid] = st_d;
    }
    __syncthreads();
    if (qt + 1 < nqt) load_tile(qt + 1);
    if (!wave_active) continue;

#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qq0 = qt * BQ + qb * 32;
      if (!(qq0 < S && (!CAUSAL || qq0 + 31 >= k0))) continue;  // wave-uniform
      const int arow = (qb * 32 + pi32(n)) * STR + h * (D / 2);
      f32x16 s = dot_rows<E, D>(Qs + arow, kf, zero16());
      f32x16 dp = dot_rows<E, D>(dOs + arow, vf, zero16());
      if (CAUSAL && qq0 < k0 + 31) {
        // query(r) = qq0 + 8h + (16*(r/8) + r%8) sees key kj iff query >= kj
        const int lim = kj - qq0 - 8 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * (r >> 3) + (r & 7) < lim) s[r] = -INFINITY;
      }
      // LSE*log2(e) and D of this lane's 16 queries: two runs of 8 at rho(0, h)
      // and rho(8, h).  Queries past S carry LSE = +inf, so their P is 0.
      float lq[16], dq_[16];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v4 = 0; v4 < 2; ++v4) {
          const int off = qb * 32 + 16 * u + 8 * h + 4 * v4;
          const f32x4 a = *reinterpret_cast<const f32x4*>(lse2s + off);
          const f32x4 b = *reinterpret_cast<const f32x4*>(Ds + off);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lq[8 * u + 4 * v4 + e] = a[e];
            dq_[8 * u + 4 * v4 + e] = b[e];
          }
        }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[r], c, -lq[r]));
        s[r] = p;
        dp[r] = p * (dp[r] - dq_[r]);
      }
      RegOperand<E> P, dS;
      P.set(s);
      dS.set(dp);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dvacc[db] = second_product<E, STR, STRT, true>(P, dOs, dOsT, qb * 32, db * 32 + n, h, dvacc[db]);
        dkacc[db] = second_product<E, STR, STRT, true>(dS, Qs, QsT, qb * 32, db * 32 + n, h, dkacc[db]);
      }
    }
  }

  if (!wave_active) return;
  // element r of acc[db]: row k0 + out_row(r, h), column db*32 + n
  T* dk = dK + base;
  T* dv = dV + base;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = k0 + out_row(r, h);
    if (row < S) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dk[(size_t)row * D + db * 32 + n] = (T)(dkacc[db][r] * scale);
        dv[(size_t)row * D + db * 32 + n] = (T)dvacc[db][r];
      }
    }
  }
}

template <class E, int D, bool CAUSAL>
static hipError_t launch(const BwdArgs& a) {
  constexpr int NW = 4;
  constexpr int BQ = D == 128 ? 32 : 64;
  using T = typename E::T;
  const int nkt = (a.S + NW * 32 - 1) / (NW * 32);
  dim3 grid(a.BH, nkt);
  hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, NW, BQ, CAUSAL>), grid, dim3(NW * 64), 0, a.stream,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout, a.lse,
                     a.delta, (T*)a.dk, (T*)a.dv, a.S, a.scale * kLog2e, a.scale);
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

hipError_t launch_bwd_dkdv(const BwdArgs& a) {
  return a.bf16 ? launch_d<EBF16>(a) : launch_d<EF32>(a);
}

}  // namespace attn
