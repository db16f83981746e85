// attn_fwd_small.hip -- attention forward for heads with very few queries.
//
// The same operation as attn_fwd.hip ("Meganeura: Portable GPU Training and
// Inference through Vulkan and Metal", arXiv 2608.01563, Section 3.3, tiled
// attention forward), for the one-token and few-token queries of the pages'
// minimal-latency cell (Section 4.3).  With one query row per head the work
// is a pair of matrix-vector products over the head's K and V: the kernel is
// bound by the HBM read of K and V, and a 32-row MFMA tile would leave 31 of
// its rows empty.  So the products run on the VALU, laid out for coalesced
// loads, and the key range of a head is split over every wave of the
// workgroup (flash-decoding style), with the partial softmax states merged
// in LDS at the end.
//
// Work split: one workgroup per (head, group of QG queries).  A wave is four
// rows of 16 lanes; each row takes one key at a time and lane c of the row
// holds elements [c*DV, c*DV + DV) of that key's K and V rows (DV = D/16), so
// one load instruction reads four whole rows.  A score is a 16-lane sum
// (DPP row rotations).  Wave w takes keys w*KB .. w*KB + KB-1, then
// (w + NW)*KB ..., KB = 4*U keys per iteration (U keys per row; the file is
// built with the ILP-first scheduler, which issues every load of an
// iteration before the first use).  Each (wave, row) keeps a running max,
// sum and O slice per query; rows merge across the wave by lane exchanges,
// waves merge through LDS.  Workgroup g runs on XCD g % 8; the queries of
// one head stay on one XCD, so its K and V come from HBM once.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {

// DV consecutive elements of T at p (aligned to their size, up to 16 bytes)
// as floats.
template <class T, int DV>
__device__ inline void load_slice(const T* __restrict__ p, float (&x)[DV]) {
  if constexpr (sizeof(T) == 4) {
    if constexpr (DV == 2) {
      const float2 v = *reinterpret_cast<const float2*>(p);
      x[0] = v.x;
      x[1] = v.y;
    } else {
#pragma unroll
      for (int e = 0; e < DV; e += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p + e);
#pragma unroll
        for (int t = 0; t < 4; ++t) x[e + t] = v[t];
      }
    }
  } else {
    constexpr int NWD = DV / 2;  // 32-bit words (two bf16 each)
    uint32_t w[NWD];
    if constexpr (NWD == 1) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else if constexpr (NWD == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x;
      w[1] = v.y;
    } else {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = v[t];
    }
#pragma unroll
    for (int k = 0; k < NWD; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
}

__device__ inline float round_bf16(float x) { return (float)(__bf16)x; }

// Sum over the 16 lanes of each row of the wave (every lane gets its row's
// sum): DPP row rotations by 8, 4, 2, 1.
__device__ inline float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));
  return x;
}

template <class E, int D, int NW, int QG, int U, bool CAUSAL, bool CROSS, bool STR>
__global__ __launch_bounds__(NW * 64) void fwd_small_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, typename E::T* __restrict__ O, float* __restrict__ LSE,
    int Sq, int Sk, float c, int BH, int H, const int* __restrict__ kvlen, int nqg,
    const Layout lay) {
  using T = typename E::T;
  constexpr int DV = D / 16;
  constexpr int KB = 4 * U;
  constexpr bool RQKV = mma_bf16<E>() && !is_bf16<E>();  // round f32 Q, K, V to bf16
  constexpr bool RP = mma_bf16<E>();                      // round P to bf16 before PV
  __shared__ float ms[NW][QG];
  __shared__ float ls[NW][QG];
  __shared__ float os[NW][QG][D];

  const int g = blockIdx.x;
  const int s = g >> 3;
  const int bh = (s / nqg) * 8 + (g & 7);
  const int qg = s % nqg;
  if (bh >= BH) return;  // whole workgroup, before any barrier
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int rg = lane >> 4, cc = lane & 15;

  int L, off;
  head_keys<CROSS>(kvlen, bh, H, Sq, Sk, L, off);
  const int q0 = qg * QG;
  const int qlast = min(Sq - 1, q0 + QG - 1);
  // keys 0 .. kend-1 are the ones some query of the group may see
  const int kend = CAUSAL ? min(L, qlast + 1 + off) : L;

  float q[QG][DV];
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    if (q0 + i < Sq) {
      load_slice<T, DV>(Q + head_off<STR, D>(lay.q, bh, H, Sq) +
                            (size_t)(q0 + i) * row_ld<STR, D>(lay.q) + cc * DV,
                        q[i]);
    } else {
#pragma unroll
      for (int e = 0; e < DV; ++e) q[i][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < DV; ++e)
      if constexpr (RQKV) q[i][e] = round_bf16(q[i][e]);
  }
  float m[QG], l[QG], o[QG][DV];
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < DV; ++e) o[i][e] = 0.f;
  }

  const T* Kh = K + head_off<STR, D>(lay.k, bh, H, Sk) + cc * DV;
  const T* Vh = V + head_off<STR, D>(lay.v, bh, H, Sk) + cc * DV;
  const int ldk = row_ld<STR, D>(lay.k), ldv = row_ld<STR, D>(lay.v);
  for (int base = w * KB; base < kend; base += NW * KB) {
    float kr[U][DV], vr[U][DV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // rows past kend are clamped to the last one the group may see (their
      // scores are masked): no row at or past the valid keys is read
      const int row = min(base + 4 * u + rg, kend - 1);
      load_slice<T, DV>(Kh + (size_t)row * ldk, kr[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = min(base + 4 * u + rg, kend - 1);
      load_slice<T, DV>(Vh + (size_t)row * ldv, vr[u]);
    }
    if constexpr (RQKV) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < DV; ++e) {
          kr[u][e] = round_bf16(kr[u][e]);
          vr[u][e] = round_bf16(vr[u][e]);
        }
    }
#pragma unroll
    for (int i = 0; i < QG; ++i) {
      // last key query q0+i sees (CROSS/causal: the aligned diagonal)
      const int lim = (q0 + i < Sq) ? (CAUSAL ? min(L - 1, q0 + i + off) : L - 1) : -1;
      float sc[U];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < DV; ++e) part = fmaf(q[i][e], kr[u][e], part);
        const float sv = row16_sum(part) * c;
        sc[u] = (base + 4 * u + rg <= lim) ? sv : -INFINITY;
        mx = fmaxf(mx, sc[u]);
      }
      const float mnew = fmaxf(m[i], mx);
      // a row with no visible key yet keeps m = -inf, l = 0, O = 0
      const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m[i] - mnew);
      const float mref = (mnew == -INFINITY) ? 0.f : mnew;
      m[i] = mnew;
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < DV; ++e) o[i][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = fast_exp2(sc[u] - mref);
        rs += p;
        const float pv = RP ? round_bf16(p) : p;
#pragma unroll
        for (int e = 0; e < DV; ++e) o[i][e] = fmaf(pv, vr[u][e], o[i][e]);
      }
      l[i] = fmaf(l[i], alpha, rs);
    }
  }

  // Merge the four rows of the wave (each row saw its own keys).
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    float M = fmaxf(m[i], __shfl_xor(m[i], 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float a = (m[i] == -INFINITY) ? 0.f : fast_exp2(m[i] - M);
    float li = l[i] * a;
    li += __shfl_xor(li, 16);
    li += __shfl_xor(li, 32);
#pragma unroll
    for (int e = 0; e < DV; ++e) {
      float x = o[i][e] * a;
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      o[i][e] = x;
    }
    m[i] = M;
    l[i] = li;
  }
  if (rg == 0) {
#pragma unroll
    for (int i = 0; i < QG; ++i) {
#pragma unroll
      for (int e = 0; e < DV; ++e) os[w][i][cc * DV + e] = o[i][e];
      if (cc == 0) {
        ms[w][i] = m[i];
        ls[w][i] = l[i];
      }
    }
  }
  __syncthreads();

  // Merge the waves and store O and the LSE (a row with no visible key:
  // O = 0, LSE = -inf).
  for (int t = threadIdx.x; t < QG * D; t += NW * 64) {
    const int i = t / D, d = t % D;
    const int qi = q0 + i;
    if (qi >= Sq) continue;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, ms[v][i]);
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float a = (ms[v][i] == -INFINITY) ? 0.f : fast_exp2(ms[v][i] - M);
      lsum = fmaf(ls[v][i], a, lsum);
      acc = fmaf(os[v][i][d], a, acc);
    }
    const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
    O[head_off<STR, D>(lay.o, bh, H, Sq) + (size_t)qi * row_ld<STR, D>(lay.o) + d] =
        (T)(acc * inv);
    if (d == 0 && LSE != nullptr)
      LSE[(size_t)bh * Sq + qi] = (lsum > 0.f) ? (M + __log2f(lsum)) * kLn2 : -INFINITY;
  }
}

template <class E, int D, int QG, bool CAUSAL, bool CROSS, bool STR>
static hipError_t launch_small(const FwdArgs& a) {
  constexpr int NW = QG == 1 ? ATTN_FWD_SMALL_NW1 : ATTN_FWD_SMALL_NW4;
  constexpr int U0 = QG == 1 ? ATTN_FWD_SMALL_U1 : ATTN_FWD_SMALL_U4;
  // (D = 128: twice the registers per key row; a quarter of the keys for a
  // query group, which also holds four O slices)
  constexpr int UD = D == 128 ? (QG == 1 ? U0 / 2 : U0 / 4) : U0;
  constexpr int U = UD > 0 ? UD : 1;
  using T = typename E::T;
  const int nqg = (a.Sq + QG - 1) / QG;
  // heads in blocks of 8 (one per XCD), then query groups, then the block
  const long long grid = (long long)((a.BH + 7) / 8) * 8 * nqg;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_small_kernel<E, D, NW, QG, U, CAUSAL, CROSS, STR>),
                     dim3((unsigned)grid), dim3(NW * 64), 0, a.stream, (const T*)a.q,
                     (const T*)a.k, (const T*)a.v, (T*)a.o, a.lse, a.Sq, a.Sk, a.scale * kLog2e,
                     a.BH, a.H, a.kvlen, nqg, a.layout != nullptr ? *a.layout : Layout{});
  return hipGetLastError();
}

template <class E, int D, int QG>
static hipError_t launch_small_g(const FwdArgs& a) {
  if (a.layout != nullptr)  // (strided: the cross-attention instantiation)
    return a.causal ? launch_small<E, D, QG, true, true, true>(a)
                    : launch_small<E, D, QG, false, true, true>(a);
  if (a.cross)
    return a.causal ? launch_small<E, D, QG, true, true, false>(a)
                    : launch_small<E, D, QG, false, true, false>(a);
  return a.causal ? launch_small<E, D, QG, true, false, false>(a)
                  : launch_small<E, D, QG, false, false, false>(a);
}

template <class E, int D>
static hipError_t launch_small_q(const FwdArgs& a) {
  return a.Sq == 1 ? launch_small_g<E, D, 1>(a) : launch_small_g<E, D, 4>(a);
}

template <class E>
static hipError_t launch_small_d(const FwdArgs& a) {
  switch (a.D) {
    case 32: return launch_small_q<E, 32>(a);
    case 64: return launch_small_q<E, 64>(a);
    case 128: return launch_small_q<E, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_small(const FwdArgs& a) {
  if (a.bf16) return launch_small_d<EBF16>(a);
  return a.bf16_operands ? launch_small_d<EF32B>(a) : launch_small_d<EF32>(a);
}

}  // namespace attn
