// attn_fwd.hip -- tiled attention forward for gfx950.
//
// The forward of the attention node ("Meganeura: Portable GPU Training and
// Inference through Vulkan and Metal", arXiv 2608.01563, Section 3.3, tiled
// attention forward kernel): O = softmax(scale * Q K^T, masked) V and the row
// LSE, with the softmax taken online over key tiles so that no S x S matrix
// exists.
//
// Work split: one workgroup per (query tile of 32*NW rows, batch*head); each
// wave owns 32 queries.  The workgroup walks the key tiles (BK keys) in
// order; K and V of each tile are staged once in LDS and shared by all
// waves, with the next tile's global loads in flight during the math.
//
// Per wave and 32-key block the scores are computed transposed,
// S^T = K Q^T (32 keys x 32 queries): each lane then holds one query and 16
// of the block's keys, so the row max and row sum are 16 in-lane operations
// plus one exchange between the two lane halves, and the O accumulator of a
// lane (O^T, d x query) belongs to that same query and is rescaled by one
// factor.  P^T stays in registers as the B operand of O^T += V^T P^T.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {

template <class E, int D, int NW, int BK, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, typename E::T* __restrict__ O,
    float* __restrict__ LSE, int S, float c) {
  using T = typename E::T;
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;
  constexpr int NDB = D / 32;
  constexpr int NKB = BK / 32;
  constexpr int STR = row_stride<E, D>();
  constexpr int STRT = tr_stride<BK>();
  constexpr int K_ELEMS = BK * STR;
  constexpr int V_ELEMS = is_bf16<E>() ? D * STRT : BK * STR;
  __shared__ __attribute__((aligned(16))) T smem[K_ELEMS + V_ELEMS];
  T* Ks = smem;
  T* Vs = smem + K_ELEMS;  // f32: row-major [key][d]; bf16: transposed [d][key]

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, n = lane & 31;
  const int bh = blockIdx.x;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;  // longest causal tiles first
  const size_t base = (size_t)bh * S * D;
  const T* q = Q + base;
  const T* k = K + base;
  const T* v = V + base;

  const int q0 = qt * BR + w * 32;
  const int qi = q0 + n;
  const bool wave_active = q0 < S;

  RowFrag<E, D> qf;
  load_row_frag<E, D>(qf, q + (size_t)min(qi, S - 1) * D + h * (D / 2), qi < S);

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
  float m = -INFINITY;  // running max of c * score (log2 domain)
  float l = 0.f;        // this half's running sum of exp2(c*score - m)

  const int kend = CAUSAL ? min(S, qt * BR + BR) : S;
  const int nkt = (kend + BK - 1) / BK;

  TileRegs<T, BK, D, NT> kr, vr;
  kr.load(k, 0, S, tid);
  vr.load(v, 0, S, tid);

  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    kr.template store<STR>(Ks, tid);
    if constexpr (is_bf16<E>()) vr.template store_t<STRT>(Vs, tid);
    else vr.template store<STR>(Vs, tid);
    __syncthreads();
    if (kt + 1 < nkt) {
      kr.load(k, (kt + 1) * BK, S, tid);
      vr.load(v, (kt + 1) * BK, S, tid);
    }
    if (!wave_active) continue;

    // Scores of the tile's 32-key blocks.  A block is skipped when no key in
    // it is visible from any of the wave's queries, and masked only when
    // some but not all of it is (the causal diagonal, the ragged end).
    f32x16 sacc[NKB];
    bool blk[NKB], part[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int kk0 = kt * BK + kb * 32;
      blk[kb] = kk0 < S && (!CAUSAL || kk0 <= q0 + 31);
      part[kb] = kk0 + 32 > S || (CAUSAL && kk0 + 31 > q0);
      if (blk[kb]) sacc[kb] = dot_rows<E, D>(Ks + (kb * 32 + pi32(n)) * STR + h * (D / 2), qf, zero16());
    }
    float mx = -INFINITY;  // max of the raw (unscaled) visible scores
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (!blk[kb]) continue;
      if (part[kb]) {
        const int kk0 = kt * BK + kb * 32;
        // key(r) = kk0 + 8h + (16*(r/8) + r%8); visible iff key < S and key <= qi
        const int lim = min(S - 1, CAUSAL ? qi : S - 1) - kk0 - 8 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * (r >> 3) + (r & 7) > lim) sacc[kb][r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[kb][r], sacc[kb][r + 1]));
    }
    mx = fmaxf(mx, xhalf(mx));
    // Lazy rescaling: exponents are taken against a reference m that may lag
    // the running max by up to 2^8, so O and l are rescaled only when some
    // row's max grows past that (and never on the first tile, where they are 0).
    const float mc = mx * c;
    if (__any(mc > m + 8.f)) {
      const float mnew = fmaxf(m, mc);
      const float alpha = fast_exp2(m - mnew);  // 0 on the first tile (m = -inf)
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (blk[kb]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[kb][r], c, -m));
          sacc[kb][r] = p;
          rs += p;
        }
      }
    }
    l += rs;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (blk[kb]) {
        RegOperand<E> P;
        P.set(sacc[kb]);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = second_product<E, STR, STRT, false>(P, Vs, Vs, kb * 32, db * 32 + n, h, oacc[db]);
      }
    }
  }

  if (!wave_active) return;
  const float ltot = l + xhalf(l);
  const float inv = 1.f / ltot;
  if (qi < S) {
    T* orow = O + base + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = db * 32 + 8 * j + 4 * h;
        store4<T>(orow + d, oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv,
                  oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
      }
    if (h == 0) LSE[(size_t)bh * S + qi] = (m + __log2f(ltot)) * kLn2;
  }
}

template <class E, int D, bool CAUSAL>
static hipError_t launch(const FwdArgs& a) {
  constexpr int NW = 4;
  constexpr int BK = D == 128 ? 32 : 64;
  using T = typename E::T;
  const int nqt = (a.S + NW * 32 - 1) / (NW * 32);
  dim3 grid(a.BH, nqt);
  hipLaunchKernelGGL((fwd_kernel<E, D, NW, BK, CAUSAL>), grid, dim3(NW * 64), 0, a.stream,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.o, a.lse, a.S,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <class E, int D>
static hipError_t launch_c(const FwdArgs& a) {
  return a.causal ? launch<E, D, true>(a) : launch<E, D, false>(a);
}

template <class E>
static hipError_t launch_d(const FwdArgs& a) {
  switch (a.D) {
    case 32: return launch_c<E, 32>(a);
    case 64: return launch_c<E, 64>(a);
    case 128: return launch_c<E, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd(const FwdArgs& a) {
  return a.bf16 ? launch_d<EBF16>(a) : launch_d<EF32>(a);
}

}  // namespace attn
