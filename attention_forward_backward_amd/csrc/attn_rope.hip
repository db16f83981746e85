// attn_rope.hip -- rotary position embedding and row-layout change, in one
// memory-bound pass.
//
// The pages ("Meganeura: Portable GPU Training and Inference through Vulkan
// and Metal", arXiv 2608.01563) use axial RoPE in front of attention in their
// DinoVision case study (Section 5.2) and rewrite projections into packed
// forms (Section 3.2).  The attention kernels read [B, H, S, D] row-major
// tensors; this pass brings Q and K (rotated) and V from any layout whose
// head dimension is contiguous -- [B, S, H, D], a packed [B, S, 3, H, D]
// projection -- into that layout, and takes the gradients back (rotated by
// the transpose).  Rotation, rotate-half arrangement: pair (i, i + D/2) of
// row s is turned by the angle whose cosine and sine are row
// pos_offset + s, column i of the caller's tables.
//
// Thread t handles PV consecutive pairs of one row: PV elements of the lower
// half and the PV elements D/2 later, 16 bytes each, and the PV table
// entries.  Reads and writes of a pair happen in the same thread, so the
// pass may run in place.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {

template <class T, int N>
struct alignas(16) Vec {
  T v[N];
};

template <class T, int D, bool ROT, bool TRANSPOSE>
__global__ __launch_bounds__(256) void rope_copy_kernel(
    const T* __restrict__ src, long long sb, long long sh, long long ss, T* __restrict__ dst,
    long long db, long long dh, long long ds, const float* __restrict__ cosT,
    const float* __restrict__ sinT, int pos_offset, int H, int S, long long nthreads) {
  constexpr int PV = 16 / sizeof(T);  // pairs per thread
  constexpr int TPR = D / 2 / PV;     // threads per row
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= nthreads) return;
  const long long row = t / TPR;
  const int j = (int)(t % TPR) * PV;  // first pair
  const int s = (int)(row % S);
  const long long bh = row / S;
  const long long b = bh / H, h = bh % H;
  const T* x = src + b * sb + h * sh + s * ss + j;
  T* y = dst + b * db + h * dh + s * ds + j;
  const Vec<T, PV> lo = *reinterpret_cast<const Vec<T, PV>*>(x);
  const Vec<T, PV> hi = *reinterpret_cast<const Vec<T, PV>*>(x + D / 2);
  Vec<T, PV> olo, ohi;
  if constexpr (ROT) {
    const float* cp = cosT + (size_t)(pos_offset + s) * (D / 2) + j;
    const float* sp = sinT + (size_t)(pos_offset + s) * (D / 2) + j;
    float c[PV], sn[PV];
#pragma unroll
    for (int e = 0; e < PV; e += 4) {
      const f32x4 cv = *reinterpret_cast<const f32x4*>(cp + e);
      const f32x4 sv = *reinterpret_cast<const f32x4*>(sp + e);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        c[e + u] = cv[u];
        sn[e + u] = TRANSPOSE ? -sv[u] : sv[u];
      }
    }
#pragma unroll
    for (int e = 0; e < PV; ++e) {
      float ylo, yhi;
      rope_pair((float)lo.v[e], (float)hi.v[e], c[e], sn[e], ylo, yhi);
      olo.v[e] = (T)ylo;
      ohi.v[e] = (T)yhi;
    }
  } else {
    olo = lo;
    ohi = hi;
  }
  *reinterpret_cast<Vec<T, PV>*>(y) = olo;
  *reinterpret_cast<Vec<T, PV>*>(y + D / 2) = ohi;
}

template <class T, int D>
static hipError_t launch_rope_t(const RopeArgs& a) {
  constexpr int PV = 16 / sizeof(T);
  const long long nthreads = (long long)a.B * a.H * a.S * (D / 2 / PV);
  const long long blocks = (nthreads + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const T* src = static_cast<const T*>(a.src);
  T* dst = static_cast<T*>(a.dst);
  const dim3 grid((unsigned)blocks), block(256);
  if (a.cos == nullptr) {
    hipLaunchKernelGGL((rope_copy_kernel<T, D, false, false>), grid, block, 0, a.stream, src,
                       a.ss[0], a.ss[1], a.ss[2], dst, a.ds[0], a.ds[1], a.ds[2], a.cos, a.sin,
                       a.pos_offset, a.H, a.S, nthreads);
  } else if (a.transpose) {
    hipLaunchKernelGGL((rope_copy_kernel<T, D, true, true>), grid, block, 0, a.stream, src,
                       a.ss[0], a.ss[1], a.ss[2], dst, a.ds[0], a.ds[1], a.ds[2], a.cos, a.sin,
                       a.pos_offset, a.H, a.S, nthreads);
  } else {
    hipLaunchKernelGGL((rope_copy_kernel<T, D, true, false>), grid, block, 0, a.stream, src,
                       a.ss[0], a.ss[1], a.ss[2], dst, a.ds[0], a.ds[1], a.ds[2], a.cos, a.sin,
                       a.pos_offset, a.H, a.S, nthreads);
  }
  return hipGetLastError();
}

template <class T>
static hipError_t launch_rope_d(const RopeArgs& a) {
  switch (a.D) {
    case 32: return launch_rope_t<T, 32>(a);
    case 64: return launch_rope_t<T, 64>(a);
    case 128: return launch_rope_t<T, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rope(const RopeArgs& a) {
  return a.bf16 ? launch_rope_d<__bf16>(a) : launch_rope_d<float>(a);
}

}  // namespace attn
