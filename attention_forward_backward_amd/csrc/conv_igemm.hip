// conv_igemm.hip -- 2-D convolution and its two derivatives as implicit
// GEMMs on the MFMA units (gfx950), and their C ABI (include/conv.h).
//
// "Meganeura: Portable GPU Training and Inference through Vulkan and Metal"
// (arXiv 2608.01563): convolution is a graph node with local input and weight
// derivatives (Section 3.1), lowered to implicit-GEMM kernels (Section 3.3);
// its weight-gradient, small weight-gradient and input-gradient kernels were
// most of a ResNet-50 training step (Section 7.3).  The operation is the
// deep-learning cross-correlation with zero padding and a stride, NHWC:
//   y[n,p,q,k]  = sum_{r,s,c} x[n, p*sh+r-ph, q*sw+s-pw, c] w[k,r,s,c]
//   dx[n,h,w,c] = sum_{p,q,r,s,k : p*sh+r-ph = h, q*sw+s-pw = w} dy[n,p,q,k] w[k,r,s,c]
//   dw[k,r,s,c] = sum_{n,p,q} dy[n,p,q,k] x[n, p*sh+r-ph, q*sw+s-pw, c]
// Each is one GEMM out[M][NC] = sum_kk A[m][kk] B[kk][j] whose operands are
// gathered from the tensors on the fly (no im2col buffer):
//   forward      M = N*P*Q (n,p,q)  NC = K          KD = R*S*C (r,s,c)
//                A = x at the tap's input pixel, B[kk][k] = w[k][kk]
//   data grad    M = N*H*W (n,h,w)  NC = C          KD = R*S*K (r,s,k)
//                A = dy at the output pixel that tap (r,s) maps onto (h,w),
//                zero where none does (stride), B[kk][c] = w[k,r,s,c]
//   filter grad  M = K              NC = R*S*C      KD = N*P*Q (n,p,q)
//                A[k][kk] = dy[kk][k], B[kk][(r,s,c)] = x at the tap's pixel
// so the output is row-major [M][NC] in every case: y [N,P,Q,K], dx
// [N,H,W,C], dw [K,R,S,C].  The filter gradient's reduction (N*P*Q) is long
// and its output small, so it is split over gridDim.z slices whose float32
// partials a second kernel adds in slice order (deterministic).
//
// Work split: a workgroup of 4 waves computes a 64 x 64 output tile, wave
// (wm, wn) one 32 x 32 MFMA block.  The reduction runs in chunks of KC
// values: every thread gathers its share of the A and B chunk into
// registers (the next chunk's loads are in flight while the current chunk
// is multiplied out of LDS), then stores them to LDS as rows of the output
// index with the reduction index contiguous, which is the operand layout of
// both MFMA shapes (strict f32: one value per lane and k-step; bf16: eight).
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "attn.h"
#include "attn_device.hpp"
#include "conv.h"

namespace attn {

enum ConvMode { CONV_FWD = 0, CONV_DATA = 1, CONV_FILTER = 2 };

// Division of indices below 2^31 by an invariant divisor d >= 1 as a
// multiply-high, add and shift (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l.  The
// sum stays below 2^32 because n < 2^31.
struct FastDiv {
  unsigned d, m;
  int l;
  __host__ static FastDiv make(unsigned d) {
    int l = 0;
    while ((1ull << l) < d) ++l;
    const unsigned m = (unsigned)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    return FastDiv{d, m, l};
  }
  __device__ inline int div(int n) const {
    return (int)((__umulhi((unsigned)n, m) + (unsigned)n) >> l);
  }
  // n = q d + r with 0 <= r < d
  __device__ inline int divmod(int n, int& r) const {
    const int q = div(n);
    r = n - q * (int)d;
    return q;
  }
};

struct ConvShape {
  int N, H, W, C, K, R, S, P, Q, sh, sw, ph, pw;
  int M, NC, KD;  // the GEMM's rows, columns and reduction length
  FastDiv dC, dK, dS, dP, dQ, dH, dW, dsh, dsw;
};

constexpr int CT = 64;  // output tile rows and columns
// Reduction values per chunk (between two workgroup barriers), per element
// type: a bf16 MFMA consumes 16 per instruction, an f32 one 2.
#ifndef ATTN_CONV_KC_F32
#define ATTN_CONV_KC_F32 32
#endif
#ifndef ATTN_CONV_KC_BF16
#define ATTN_CONV_KC_BF16 32
#endif
// Chunks gathered ahead of the one being multiplied (1 or 2).  On the
// ResNet-50 layers of the benchmark two were slower everywhere but the bf16
// 1x1 forward (3x3 f32 forward 98 -> 103 us, stem bf16 forward 174 -> 218;
// 1x1 bf16 forward 21.7 -> 18.9), so one is the default.
#ifndef ATTN_CONV_PREFETCH
#define ATTN_CONV_PREFETCH 1
#endif
static_assert(ATTN_CONV_PREFETCH == 1 || ATTN_CONV_PREFETCH == 2, "prefetch depth 1 or 2");
// bf16 with both operands gathered as 16-byte vectors: 64 values per chunk
// (1x1 C1024->256 forward at 14x14, batch 32: 21.8 -> 18.0 us; 3x3 C64->64
// data derivative 46.9 -> 45.2; 128 helped the 1x1 forward further but not
// the 3x3 layer, and with element gathers larger chunks doubled the stem's
// forward, so those keep 32).
#ifndef ATTN_CONV_KC_BF16_VEC
#define ATTN_CONV_KC_BF16_VEC 64
#endif

// A[m][kk] of the GEMM (zero outside the tensors and past KD).
template <class T, int MODE>
__device__ inline float a_val(const T* __restrict__ a, const ConvShape& s, int m, int kk) {
  if (m >= s.M || kk >= s.KD) return 0.f;
  if constexpr (MODE == CONV_FWD) {
    int q, p, c, ss;
    const int n = s.dP.divmod(s.dQ.divmod(m, q), p);
    const int r = s.dS.divmod(s.dC.divmod(kk, c), ss);
    const int ih = p * s.sh + r - s.ph, iw = q * s.sw + ss - s.pw;
    if (ih < 0 || ih >= s.H || iw < 0 || iw >= s.W) return 0.f;
    return (float)a[(((size_t)n * s.H + ih) * s.W + iw) * s.C + c];
  } else if constexpr (MODE == CONV_DATA) {
    int w, h, k, ss;
    const int n = s.dH.divmod(s.dW.divmod(m, w), h);
    const int r = s.dS.divmod(s.dK.divmod(kk, k), ss);
    const int ph = h + s.ph - r, pw = w + s.pw - ss;  // p*sh and q*sw
    if (ph < 0 || pw < 0) return 0.f;
    int rh, rw;
    const int p = s.dsh.divmod(ph, rh), q = s.dsw.divmod(pw, rw);
    if (rh != 0 || rw != 0 || p >= s.P || q >= s.Q) return 0.f;
    return (float)a[(((size_t)n * s.P + p) * s.Q + q) * s.K + k];
  } else {
    return (float)a[(size_t)kk * s.K + m];  // dy[(n,p,q)][k]
  }
}

// B[kk][j] of the GEMM (zero outside the tensors and past KD).
template <class T, int MODE>
__device__ inline float b_val(const T* __restrict__ b, const ConvShape& s, int kk, int j) {
  if (j >= s.NC || kk >= s.KD) return 0.f;
  if constexpr (MODE == CONV_FWD) {
    return (float)b[(size_t)j * s.KD + kk];  // w[k][(r,s,c)]
  } else if constexpr (MODE == CONV_DATA) {
    int k;
    const int u = s.dK.divmod(kk, k);  // u = r*S + s
    return (float)b[((size_t)k * s.R * s.S + u) * s.C + j];  // w[k,r,s,c]
  } else {
    int q, p, c, ss;
    const int n = s.dP.divmod(s.dQ.divmod(kk, q), p);
    const int r = s.dS.divmod(s.dC.divmod(j, c), ss);
    const int ih = p * s.sh + r - s.ph, iw = q * s.sw + ss - s.pw;
    if (ih < 0 || ih >= s.H || iw < 0 || iw >= s.W) return 0.f;
    return (float)b[(((size_t)n * s.H + ih) * s.W + iw) * s.C + c];
  }
}

// How an operand is gathered: one element per load, or 16-byte vectors of
// V = 16 / sizeof(T) consecutive elements along the reduction index (the
// channels of x and dy, the rows of w) or along the output index (the
// channels of w in the data derivative, dy and x in the filter derivative).  The host takes a vector gather only where
// every group of V is contiguous and 16-byte aligned (channel counts and
// reduction lengths multiples of V, aligned base pointers).
enum Gather { G_SCALAR = 0, G_ALONG_K = 1, G_ALONG_ROW = 2 };

// Reduction values per chunk of a kernel with gathers GA, GB.
template <class E, int GA, int GB>
__host__ __device__ constexpr int conv_kc() {
  if constexpr (is_bf16<E>())
    return GA != G_SCALAR && GB != G_SCALAR ? ATTN_CONV_KC_BF16_VEC : ATTN_CONV_KC_BF16;
  else
    return ATTN_CONV_KC_F32;
}

// The V values of operand WHICH (0: A, 1: B) at output index row (the first
// of V rows with G_ALONG_ROW) and reduction index kk (the first of V with
// G_ALONG_K), zero outside the tensors: one index decomposition, one load.
template <class T, int MODE, int WHICH>
__device__ inline u32x4 vec_val(const T* __restrict__ src, const ConvShape& s, int row, int kk) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
  if (kk >= s.KD) return zero;
  if constexpr (WHICH == 0 && MODE == CONV_FWD) {  // x channels c .. c+V-1 of the tap's pixel
    if (row >= s.M) return zero;
    int q, p, c, ss;
    const int n = s.dP.divmod(s.dQ.divmod(row, q), p);
    const int r = s.dS.divmod(s.dC.divmod(kk, c), ss);
    const int ih = p * s.sh + r - s.ph, iw = q * s.sw + ss - s.pw;
    if (ih < 0 || ih >= s.H || iw < 0 || iw >= s.W) return zero;
    return *reinterpret_cast<const u32x4*>(src + (((size_t)n * s.H + ih) * s.W + iw) * s.C + c);
  } else if constexpr (WHICH == 1 && MODE == CONV_FWD) {  // w[k][kk .. kk+V-1]
    if (row >= s.NC) return zero;
    return *reinterpret_cast<const u32x4*>(src + (size_t)row * s.KD + kk);
  } else if constexpr (WHICH == 0 && MODE == CONV_DATA) {  // dy channels k .. k+V-1
    if (row >= s.M) return zero;
    int w, h, k, ss;
    const int n = s.dH.divmod(s.dW.divmod(row, w), h);
    const int r = s.dS.divmod(s.dK.divmod(kk, k), ss);
    const int ph = h + s.ph - r, pw = w + s.pw - ss;
    if (ph < 0 || pw < 0) return zero;
    int rh, rw;
    const int p = s.dsh.divmod(ph, rh), q = s.dsw.divmod(pw, rw);
    if (rh != 0 || rw != 0 || p >= s.P || q >= s.Q) return zero;
    return *reinterpret_cast<const u32x4*>(src + (((size_t)n * s.P + p) * s.Q + q) * s.K + k);
  } else if constexpr (WHICH == 1 && MODE == CONV_DATA) {  // w[k, r, s, c .. c+V-1]
    if (row >= s.NC) return zero;
    int k;
    const int u = s.dK.divmod(kk, k);  // u = r*S + s
    return *reinterpret_cast<const u32x4*>(src + ((size_t)k * s.R * s.S + u) * s.C + row);
  } else if constexpr (WHICH == 0 && MODE == CONV_FILTER) {  // dy[kk][k .. k+V-1]
    if (row >= s.M) return zero;
    return *reinterpret_cast<const u32x4*>(src + (size_t)kk * s.K + row);
  } else {  // B of the filter derivative: x channels c .. c+V-1 of tap (r, s)
    static_assert(WHICH == 1 && MODE == CONV_FILTER, "no vector gather for this operand");
    if (row >= s.NC) return zero;
    int q, p, c, ss;
    const int n = s.dP.divmod(s.dQ.divmod(kk, q), p);
    const int r = s.dS.divmod(s.dC.divmod(row, c), ss);
    const int ih = p * s.sh + r - s.ph, iw = q * s.sw + ss - s.pw;
    if (ih < 0 || ih >= s.H || iw < 0 || iw >= s.W) return zero;
    return *reinterpret_cast<const u32x4*>(src + (((size_t)n * s.H + ih) * s.W + iw) * s.C + c);
  }
}

template <class E, int MODE, int GA, int GB>
__global__ __launch_bounds__(256) void conv_igemm_kernel(const typename E::T* __restrict__ A,
                                                         const typename E::T* __restrict__ B,
                                                         typename E::T* __restrict__ out,
                                                         float* __restrict__ part, int kspan,
                                                         const ConvShape s) {
  // out (or, with part != null, part[blockIdx.z]) = A B over the reduction
  // range [blockIdx.z * kspan, min(KD, +kspan)) for the 64 x 64 tile
  // (blockIdx.y, blockIdx.x); GA, GB: how A and B are gathered (Gather).
  using T = typename E::T;
  constexpr int V = 16 / (int)sizeof(T);            // elements per vector gather
  constexpr int KC = conv_kc<E, GA, GB>();
  constexpr int PER = CT * KC / 256;                // values of one operand per thread per chunk
  constexpr int NV = CT * KC / V / 256;             // vector groups per thread per chunk
  constexpr int LDK = KC + (is_bf16<E>() ? 8 : 1);  // padded LDS row (bf16: 16-byte reads)
  // bf16 operands gathered along the output index are held transposed: KC
  // reduction rows of CT output values in the swizzled tile layout of the
  // attention kernels (one 16-byte store per gathered group instead of eight
  // 2-byte ones), read back with transposed LDS reads
  constexpr bool TA = is_bf16<E>() && GA == G_ALONG_ROW;
  constexpr bool TB = is_bf16<E>() && GB == G_ALONG_ROW;
  using TT = Tile<E, CT>;
  static_assert(!is_bf16<E>() || KC % 32 == 0, "bf16 chunks of whole MFMA pairs");
  static_assert(KC * TT::ROWB <= CT * LDK * (int)sizeof(T), "transposed tile fits the buffer");
  __shared__ __attribute__((aligned(16))) T As[CT * LDK];
  __shared__ __attribute__((aligned(16))) T Bs[CT * LDK];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const int m0 = blockIdx.y * CT, j0 = blockIdx.x * CT;
  const int k0 = blockIdx.z * kspan, k1 = min(s.KD, k0 + kspan);
  // Element-gather pattern: the filter gradient walks the output index
  // fastest (its A and B rows are contiguous along it); the others the
  // reduction index.
  auto slot = [&](int i, int& row, int& kk) __attribute__((always_inline)) {
    const int e = i * 256 + tid;
    if constexpr (MODE == CONV_FILTER) {
      row = e % CT;
      kk = e / CT;
    } else {
      row = e / KC;
      kk = e % KC;
    }
  };
  // Vector-group pattern (first row and reduction index of group g).
  auto vslot = [&](int g, int mode, int& row, int& kk) __attribute__((always_inline)) {
    const int e = g * 256 + tid;
    if (mode == G_ALONG_K) {
      row = e / (KC / V);
      kk = (e % (KC / V)) * V;
    } else {
      kk = e / (CT / V);
      row = (e % (CT / V)) * V;
    }
  };
  // Register sets of gathered chunks (ATTN_CONV_PREFETCH chunks in flight).
  constexpr int NS = ATTN_CONV_PREFETCH;
  float sa_[NS][GA == G_SCALAR ? PER : 1], sb_[NS][GB == G_SCALAR ? PER : 1];
  u32x4 va_[NS][GA == G_SCALAR ? 1 : NV], vb_[NS][GB == G_SCALAR ? 1 : NV];
  // The part of a vector group's x address that its output index fixes,
  // computed once: the forward's A (output pixel n, p, q: image row base and
  // the window's top-left input coordinate; a pixel past M gets a row that no
  // tap brings inside the image) and the filter derivative's B (tap r, s and
  // channel c).  Per chunk only the reduction index is decomposed.
  constexpr bool XA = MODE == CONV_FWD && GA == G_ALONG_K;
  constexpr bool XB = MODE == CONV_FILTER && GB == G_ALONG_ROW;
  constexpr bool XD = MODE == CONV_DATA && GA == G_ALONG_K;  // dy, likewise
  constexpr bool XANY = XA || XB || XD;
  int xh[XANY ? NV : 1], xw[XANY ? NV : 1], xc[XANY ? NV : 1];
  if constexpr (XANY) {
#pragma unroll
    for (int g = 0; g < NV; ++g) {
      int row, kk;
      vslot(g, XB ? GB : GA, row, kk);
      if constexpr (XD) {
        // input pixel n, h, w: dy image base and the padded coordinates
        const int m = m0 + row;
        int w, h;
        const int n = s.dH.divmod(s.dW.divmod(min(m, s.M - 1), w), h);
        xc[g] = n * s.P;
        xh[g] = m < s.M ? h + s.ph : -(1 << 28);
        xw[g] = w + s.pw;
      } else if constexpr (XA) {
        const int m = m0 + row;
        int q, p;
        const int n = s.dP.divmod(s.dQ.divmod(min(m, s.M - 1), q), p);
        xc[g] = n * s.H;                                   // image n's first row
        xh[g] = m < s.M ? p * s.sh - s.ph : -(1 << 28);    // top input row of the window
        xw[g] = q * s.sw - s.pw;
      } else {
        const int j = j0 + row;
        int c, ss;
        const int r = s.dS.divmod(s.dC.divmod(min(j, s.NC - 1), c), ss);
        xh[g] = j < s.NC ? r - s.ph : -(1 << 28);          // tap offsets, padding folded in
        xw[g] = ss - s.pw;
        xc[g] = c;
      }
    }
  }
  // The same for x gathered element by element (the 3-channel stem): in the
  // forward a thread's PER elements share one reduction index (tid % KC) and
  // have PER output pixels, decomposed once here, so a chunk decomposes its
  // reduction index once; in the filter derivative they share one tap and
  // channel (tid % CT).
  constexpr bool SA = MODE == CONV_FWD && GA == G_SCALAR;
  constexpr bool SB = MODE == CONV_FILTER && GB == G_SCALAR;
  static_assert(256 % KC == 0 && 256 % CT == 0, "element slots keep their index across i");
  int sxh[SA ? PER : 1], sxw[SA ? PER : 1], sxc[SA ? PER : 1];
  int fr = 0, fs = 0, fc = 0;
  if constexpr (SA) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int row, kk;
      slot(i, row, kk);
      const int m = m0 + row;
      int q, p;
      const int n = s.dP.divmod(s.dQ.divmod(min(m, s.M - 1), q), p);
      sxc[i] = n * s.H;
      sxh[i] = m < s.M ? p * s.sh - s.ph : -(1 << 28);
      sxw[i] = q * s.sw - s.pw;
    }
  }
  if constexpr (SB) {
    int row, kk;
    slot(0, row, kk);
    const int j = j0 + row;
    int c, ss;
    const int r = s.dS.divmod(s.dC.divmod(min(j, s.NC - 1), c), ss);
    fr = j < s.NC ? r - s.ph : -(1 << 28);
    fs = ss - s.pw;
    fc = c;
  }
  // (k1 and every group boundary are multiples of V on the vector paths, so
  // a group is either wholly inside the chunk range or wholly outside)
  auto gather = [&](int kc, auto setc) __attribute__((always_inline)) {
    constexpr int st = decltype(setc)::value;
    float* sa = sa_[st];
    float* sb = sb_[st];
    u32x4* va = va_[st];
    u32x4* vb = vb_[st];
    if constexpr (SA) {
      int row0, kk0;
      slot(0, row0, kk0);  // (every i has this reduction index)
      const int k = kc + kk0;
      int c, ss;
      const int r = s.dS.divmod(s.dC.divmod(min(k, s.KD - 1), c), ss);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int ih = sxh[i] + r, iw = sxw[i] + ss;
        const bool in = k < k1 && (unsigned)ih < (unsigned)s.H && (unsigned)iw < (unsigned)s.W;
        sa[i] = in ? (float)A[((size_t)(sxc[i] + ih) * s.W + iw) * s.C + c] : 0.f;
      }
    } else if constexpr (GA == G_SCALAR) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int row, kk;
        slot(i, row, kk);
        sa[i] = kc + kk < k1 ? a_val<T, MODE>(A, s, m0 + row, kc + kk) : 0.f;
      }
    } else {
#pragma unroll
      for (int g = 0; g < NV; ++g) {
        int row, kk;
        vslot(g, GA, row, kk);
        if constexpr (XD) {
          // dy channels k .. k+V-1 of the output pixel that tap (r, ss) of
          // the group's input pixel comes from (none between strides)
          const int kx = kc + kk;
          int k, ss;
          const int r = s.dS.divmod(s.dK.divmod(kx, k), ss);
          const int ph = xh[g] - r, pw = xw[g] - ss;
          int rh, rw;
          const int p = s.dsh.divmod(max(ph, 0), rh), q = s.dsw.divmod(max(pw, 0), rw);
          const bool in = kx < k1 && ph >= 0 && pw >= 0 && rh == 0 && rw == 0 && p < s.P &&
                          q < s.Q;
          va[g] = in ? *reinterpret_cast<const u32x4*>(A + ((size_t)(xc[g] + p) * s.Q + q) * s.K + k)
                     : u32x4{0u, 0u, 0u, 0u};
        } else if constexpr (XA) {
          // x channels c .. c+V-1 of tap (r, ss) of the group's output pixel
          const int k = kc + kk;
          int c, ss;
          const int r = s.dS.divmod(s.dC.divmod(k, c), ss);
          const int ih = xh[g] + r, iw = xw[g] + ss;
          const bool in = k < k1 && (unsigned)ih < (unsigned)s.H && (unsigned)iw < (unsigned)s.W;
          va[g] = in ? *reinterpret_cast<const u32x4*>(A + ((size_t)(xc[g] + ih) * s.W + iw) * s.C + c)
                     : u32x4{0u, 0u, 0u, 0u};
        } else {
          va[g] = kc + kk < k1 ? vec_val<T, MODE, 0>(A, s, m0 + row, kc + kk) : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    if constexpr (SB) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int row, kk;
        slot(i, row, kk);
        const int k = kc + kk;
        int q, p;
        const int n = s.dP.divmod(s.dQ.divmod(min(k, s.KD - 1), q), p);
        const int ih = p * s.sh + fr, iw = q * s.sw + fs;
        const bool in = k < k1 && (unsigned)ih < (unsigned)s.H && (unsigned)iw < (unsigned)s.W;
        sb[i] = in ? (float)B[(((size_t)n * s.H + ih) * s.W + iw) * s.C + fc] : 0.f;
      }
    } else if constexpr (GB == G_SCALAR) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int row, kk;
        slot(i, row, kk);
        sb[i] = kc + kk < k1 ? b_val<T, MODE>(B, s, kc + kk, j0 + row) : 0.f;
      }
    } else {
#pragma unroll
      for (int g = 0; g < NV; ++g) {
        int row, kk;
        vslot(g, GB, row, kk);
        if constexpr (XB) {
          // x channels c .. c+V-1 of the group's tap at output pixel kc + kk
          const int k = kc + kk;
          int q, p;
          const int n = s.dP.divmod(s.dQ.divmod(k, q), p);
          const int ih = p * s.sh + xh[g], iw = q * s.sw + xw[g];
          const bool in = k < k1 && (unsigned)ih < (unsigned)s.H && (unsigned)iw < (unsigned)s.W;
          vb[g] = in ? *reinterpret_cast<const u32x4*>(B + (((size_t)n * s.H + ih) * s.W + iw) * s.C + xc[g])
                     : u32x4{0u, 0u, 0u, 0u};
        } else {
          vb[g] = kc + kk < k1 ? vec_val<T, MODE, 1>(B, s, j0 + row, kc + kk) : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  // The gathered chunk into LDS rows (output index) with the reduction index
  // contiguous.
  auto put = [&](T* dst, const float* sv, const u32x4* vv, auto modec) __attribute__((always_inline)) {
    constexpr int mode = decltype(modec)::value;
    if constexpr (mode == G_SCALAR) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int row, kk;
        slot(i, row, kk);
        dst[row * LDK + kk] = (T)sv[i];
      }
    } else {
#pragma unroll
      for (int g = 0; g < NV; ++g) {
        int row, kk;
        vslot(g, mode, row, kk);
        if constexpr (mode == G_ALONG_K && is_bf16<E>()) {
          *reinterpret_cast<u32x4*>(dst + row * LDK + kk) = vv[g];  // 16-byte aligned row part
        } else if constexpr (mode == G_ALONG_ROW && is_bf16<E>()) {
          // the group is one 16-byte chunk of reduction row kk of the
          // transposed tile
          *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dst) + TT::off(kk, row)) = vv[g];
        } else {
          const T* e = reinterpret_cast<const T*>(&vv[g]);
#pragma unroll
          for (int u = 0; u < V; ++u) {
            if constexpr (mode == G_ALONG_K)
              dst[row * LDK + kk + u] = e[u];
            else
              dst[(row + u) * LDK + kk] = e[u];
          }
        }
      }
    }
  };
  f32x16 acc = zero16();
  // One chunk: its registers into LDS, the gather of the chunk NS ahead into
  // the same registers, the products out of LDS.
  auto chunk = [&](int kc, auto setc) __attribute__((always_inline)) {
    constexpr int st = decltype(setc)::value;
    put(As, sa_[st], va_[st], std::integral_constant<int, GA>{});
    put(Bs, sb_[st], vb_[st], std::integral_constant<int, GB>{});
    __syncthreads();
    if (kc + NS * KC < k1) gather(kc + NS * KC, setc);  // in flight during later chunks
    const T* ar = As + (wm * 32 + n) * LDK;
    const T* br = Bs + (wn * 32 + n) * LDK;
    if constexpr (is_bf16<E>()) {
      // per 32 reduction values, two MFMAs; an operand held transposed is
      // read in the same k-slot form (8 consecutive reduction values of the
      // lane's row) with transposed LDS reads
#pragma unroll
      for (int t = 0; t < KC / 32; ++t) {
        RegOperand<E> xa, xb;
        if constexpr (TA) {
          read_kslot_operand<E, CT>(xa, reinterpret_cast<const char*>(As), 32 * t, wm * 32, lane);
        } else {
#pragma unroll
          for (int u = 0; u < 2; ++u)
            xa.v[u] = *reinterpret_cast<const bf16x8*>(ar + 32 * t + 16 * u + 8 * h);
        }
        if constexpr (TB) {
          read_kslot_operand<E, CT>(xb, reinterpret_cast<const char*>(Bs), 32 * t, wn * 32, lane);
        } else {
#pragma unroll
          for (int u = 0; u < 2; ++u)
            xb.v[u] = *reinterpret_cast<const bf16x8*>(br + 32 * t + 16 * u + 8 * h);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) acc = E::mma(xa.v[u], xb.v[u], acc);
      }
    } else {
#pragma unroll
      for (int t = 0; t < KC / 2; ++t) acc = E::mma(ar[2 * t + h], br[2 * t + h], acc);
    }
    __syncthreads();
  };
  gather(k0, std::integral_constant<int, 0>{});
  if constexpr (NS == 2) {
    if (k0 + KC < k1) gather(k0 + KC, std::integral_constant<int, 1>{});
    for (int kc = k0; kc < k1; kc += 2 * KC) {
      chunk(kc, std::integral_constant<int, 0>{});
      if (kc + KC >= k1) break;
      chunk(kc + KC, std::integral_constant<int, NS - 1>{});
    }
  } else {
    for (int kc = k0; kc < k1; kc += KC) chunk(kc, std::integral_constant<int, 0>{});
  }
  // element r: row m0 + 32 wm + out_row(r, h), column j0 + 32 wn + n
  const int j = j0 + wn * 32 + n;
  if (j >= s.NC) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + wm * 32 + out_row(r, h);
    if (m < s.M) {
      if (part != nullptr)
        part[((size_t)blockIdx.z * s.M + m) * s.NC + j] = acc[r];
      else
        out[(size_t)m * s.NC + j] = (T)acc[r];
    }
  }
}

// out[i] = sum over the z slices of part[z][i] in a fixed order: a
// workgroup takes 64 outputs, its wave g sums the slices z = g (mod 4) of
// each in eight running sums (z = g + 4u mod 32), added pairwise, and the
// four wave sums are added pairwise through LDS (deterministic; four waves
// per output keep more loads in flight than one thread per output did).
template <class T>
__global__ __launch_bounds__(256) void conv_split_reduce_kernel(const float* __restrict__ part,
                                                                T* __restrict__ out, int total,
                                                                int nz) {
  __shared__ float red[4][64];
  const int g = threadIdx.x >> 6, o = threadIdx.x & 63;
  const int i = blockIdx.x * 64 + o;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (i < total) {
    const float* p = part + i;
    int z = g;
    for (; z + 28 < nz; z += 32) {
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] += p[(size_t)(z + 4 * u) * total];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (z + 4 * u < nz) a[u] += p[(size_t)(z + 4 * u) * total];
  }
  red[g][o] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  __syncthreads();
  if (g == 0 && i < total) out[i] = (T)((red[0][o] + red[1][o]) + (red[2][o] + red[3][o]));
}

}  // namespace attn

namespace {

using attn::ConvShape;

// Reduction slices of the filter gradient: enough 64 x 64 tiles x slices to
// fill the chip (about 1024 workgroups), each slice at least 512 long.
int filter_slices(const ConvShape& s) {
  const long long tiles = (long long)((s.M + 63) / 64) * ((s.NC + 63) / 64);
  long long z = (1024 + tiles - 1) / tiles;
  z = std::min<long long>(z, (s.KD + 511) / 512);
  return (int)std::max<long long>(1, std::min<long long>(z, 256));
}

// Checks the shape and fills s; false on any invalid value.
bool make_shape(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                ConvShape& s) {
  if (N <= 0 || H <= 0 || W <= 0 || C <= 0 || K <= 0 || R <= 0 || S <= 0) return false;
  if (sh <= 0 || sw <= 0 || ph < 0 || pw < 0) return false;
  const long long P = ((long long)H + 2LL * ph - R) / sh + 1;
  const long long Q = ((long long)W + 2LL * pw - S) / sw + 1;
  if ((long long)H + 2LL * ph < R || (long long)W + 2LL * pw < S || P <= 0 || Q <= 0) return false;
  const long long lim = 1LL << 31;
  // every tensor and every GEMM extent indexed in 32 bits
  if ((long long)N * H * W * C >= lim || (long long)K * R * S * C >= lim ||
      (long long)N * P * Q * K >= lim || (long long)N * P * Q >= lim)
    return false;
  s = ConvShape{N, H, W, C, K, R, S, (int)P, (int)Q, sh, sw, ph, pw, 0, 0, 0, {}, {}, {}, {}, {}, {},
                {}, {}, {}};
  using attn::FastDiv;
  s.dC = FastDiv::make(C); s.dK = FastDiv::make(K); s.dS = FastDiv::make(S);
  s.dP = FastDiv::make((unsigned)P); s.dQ = FastDiv::make((unsigned)Q);
  s.dH = FastDiv::make(H); s.dW = FastDiv::make(W);
  s.dsh = FastDiv::make(sh); s.dsw = FastDiv::make(sw);
  return true;
}

template <class E, int MODE, int GA, int GB>
void launch_g(const void* a, const void* b, void* out, float* part, int nz, dim3 grid,
              const ConvShape& s, hipStream_t st) {
  using T = typename E::T;
  // each of the nz reduction slices a whole number of chunks
  constexpr int KC = attn::conv_kc<E, GA, GB>();
  const int kspan = ((s.KD + nz - 1) / nz + KC - 1) / KC * KC;
  hipLaunchKernelGGL((attn::conv_igemm_kernel<E, MODE, GA, GB>), grid, dim3(256), 0, st,
                     (const T*)a, (const T*)b, (T*)out, part, kspan, s);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <class E, int MODE>
hipError_t launch(const void* a, const void* b, void* out, float* part, int nz, ConvShape s,
                  hipStream_t st) {
  using T = typename E::T;
  constexpr int V = 16 / (int)sizeof(T);
  if (MODE == attn::CONV_FWD) {
    s.M = s.N * s.P * s.Q; s.NC = s.K; s.KD = s.R * s.S * s.C;
  } else if (MODE == attn::CONV_DATA) {
    s.M = s.N * s.H * s.W; s.NC = s.C; s.KD = s.R * s.S * s.K;
  } else {
    s.M = s.K; s.NC = s.R * s.S * s.C; s.KD = s.N * s.P * s.Q;
  }
  dim3 grid((s.NC + 63) / 64, (s.M + 63) / 64, nz);
  // Vector gathers where every group of V is contiguous and aligned.
  using namespace attn;
  if (MODE == CONV_FWD) {
    const bool va = s.C % V == 0 && aligned16(a), vb = s.KD % V == 0 && aligned16(b);
    if (va && vb) launch_g<E, CONV_FWD, G_ALONG_K, G_ALONG_K>(a, b, out, part, nz, grid, s, st);
    else if (va) launch_g<E, CONV_FWD, G_ALONG_K, G_SCALAR>(a, b, out, part, nz, grid, s, st);
    else if (vb) launch_g<E, CONV_FWD, G_SCALAR, G_ALONG_K>(a, b, out, part, nz, grid, s, st);
    else launch_g<E, CONV_FWD, G_SCALAR, G_SCALAR>(a, b, out, part, nz, grid, s, st);
  } else if (MODE == CONV_DATA) {
    const bool va = s.K % V == 0 && aligned16(a), vb = s.C % V == 0 && aligned16(b);
    if (va && vb) launch_g<E, CONV_DATA, G_ALONG_K, G_ALONG_ROW>(a, b, out, part, nz, grid, s, st);
    else if (va) launch_g<E, CONV_DATA, G_ALONG_K, G_SCALAR>(a, b, out, part, nz, grid, s, st);
    else if (vb) launch_g<E, CONV_DATA, G_SCALAR, G_ALONG_ROW>(a, b, out, part, nz, grid, s, st);
    else launch_g<E, CONV_DATA, G_SCALAR, G_SCALAR>(a, b, out, part, nz, grid, s, st);
  } else {
    const bool va = s.K % V == 0 && aligned16(a), vb = s.C % V == 0 && aligned16(b);
    if (va && vb) launch_g<E, CONV_FILTER, G_ALONG_ROW, G_ALONG_ROW>(a, b, out, part, nz, grid, s, st);
    else if (va) launch_g<E, CONV_FILTER, G_ALONG_ROW, G_SCALAR>(a, b, out, part, nz, grid, s, st);
    else if (vb) launch_g<E, CONV_FILTER, G_SCALAR, G_ALONG_ROW>(a, b, out, part, nz, grid, s, st);
    else launch_g<E, CONV_FILTER, G_SCALAR, G_SCALAR>(a, b, out, part, nz, grid, s, st);
  }
  if (part != nullptr) {
    const int total = s.M * s.NC;
    hipLaunchKernelGGL((attn::conv_split_reduce_kernel<T>), dim3((total + 63) / 64), dim3(256),
                       0, st, (const float*)part, (T*)out, total, nz);
  }
  return hipGetLastError();
}

attn_status_t status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

attn_status_t conv2d_fwd(attn_dtype_t dtype, const void* x, const void* w, void* y, int batch,
                         int height, int width, int channels, int filters, int kh, int kw,
                         int stride_h, int stride_w, int pad_h, int pad_w, void* stream) {
  ConvShape s;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!x || !w || !y) return ATTN_ERR_INVALID_ARG;
  const size_t es = dtype == ATTN_BF16 ? 2 : 4;
  if (!aligned(x, es) || !aligned(w, es) || !aligned(y, es)) return ATTN_ERR_INVALID_ARG;
  if (!make_shape(batch, height, width, channels, filters, kh, kw, stride_h, stride_w, pad_h,
                  pad_w, s))
    return ATTN_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return status(dtype == ATTN_BF16
                    ? launch<attn::EBF16, attn::CONV_FWD>(x, w, y, nullptr, 1, s, st)
                    : launch<attn::EF32, attn::CONV_FWD>(x, w, y, nullptr, 1, s, st));
}

attn_status_t conv2d_bwd_data(attn_dtype_t dtype, const void* dy, const void* w, void* dx,
                              int batch, int height, int width, int channels, int filters,
                              int kh, int kw, int stride_h, int stride_w, int pad_h, int pad_w,
                              void* stream) {
  ConvShape s;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!dy || !w || !dx) return ATTN_ERR_INVALID_ARG;
  const size_t es = dtype == ATTN_BF16 ? 2 : 4;
  if (!aligned(dy, es) || !aligned(w, es) || !aligned(dx, es)) return ATTN_ERR_INVALID_ARG;
  if (!make_shape(batch, height, width, channels, filters, kh, kw, stride_h, stride_w, pad_h,
                  pad_w, s))
    return ATTN_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return status(dtype == ATTN_BF16
                    ? launch<attn::EBF16, attn::CONV_DATA>(dy, w, dx, nullptr, 1, s, st)
                    : launch<attn::EF32, attn::CONV_DATA>(dy, w, dx, nullptr, 1, s, st));
}

size_t conv2d_bwd_filter_workspace_size(attn_dtype_t dtype, int batch, int height, int width,
                                        int channels, int filters, int kh, int kw, int stride_h,
                                        int stride_w, int pad_h, int pad_w) {
  ConvShape s;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return 0;
  if (!make_shape(batch, height, width, channels, filters, kh, kw, stride_h, stride_w, pad_h,
                  pad_w, s))
    return 0;
  s.M = s.K; s.NC = s.R * s.S * s.C; s.KD = s.N * s.P * s.Q;
  const int nz = filter_slices(s);
  return nz > 1 ? ((size_t)nz * s.M * s.NC * sizeof(float) + 255) / 256 * 256 : 0;
}

attn_status_t conv2d_bwd_filter(attn_dtype_t dtype, const void* x, const void* dy, void* dw,
                                void* workspace, size_t workspace_bytes, int batch, int height,
                                int width, int channels, int filters, int kh, int kw,
                                int stride_h, int stride_w, int pad_h, int pad_w, void* stream) {
  ConvShape s;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!x || !dy || !dw) return ATTN_ERR_INVALID_ARG;
  const size_t es = dtype == ATTN_BF16 ? 2 : 4;
  if (!aligned(x, es) || !aligned(dy, es) || !aligned(dw, es)) return ATTN_ERR_INVALID_ARG;
  if (!make_shape(batch, height, width, channels, filters, kh, kw, stride_h, stride_w, pad_h,
                  pad_w, s))
    return ATTN_ERR_INVALID_ARG;
  const size_t need = conv2d_bwd_filter_workspace_size(dtype, batch, height, width, channels,
                                                       filters, kh, kw, stride_h, stride_w,
                                                       pad_h, pad_w);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16)))
    return ATTN_ERR_WORKSPACE;
  ConvShape g = s;
  g.M = g.K; g.NC = g.R * g.S * g.C; g.KD = g.N * g.P * g.Q;
  const int nz = need > 0 ? filter_slices(g) : 1;
  float* part = need > 0 ? static_cast<float*>(workspace) : nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return status(dtype == ATTN_BF16
                    ? launch<attn::EBF16, attn::CONV_FILTER>(dy, x, dw, part, nz, s, st)
                    : launch<attn::EF32, attn::CONV_FILTER>(dy, x, dw, part, nz, s, st));
}

}  // extern "C"
