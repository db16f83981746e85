// attn_bwd_prep.hip -- per-query-row statistics the backward kernels share.
//
// For the attention derivative ("Meganeura: Portable GPU Training and
// Inference through Vulkan and Metal", arXiv 2608.01563, Section 3.1 --
// attention's local derivative rule; Section 3.3 -- dQ and fused dK+dV
// kernels), every query row i needs
//   D_i      = sum_d dO_id O_id        (dS_ij = P_ij (dP_ij - D_i))
//   LSE_i * log2(e)                     (P_ij = exp2(scale*log2(e)*S_ij - LSE_i*log2(e)))
// This memory-bound pass writes both to the workspace once, so the
// compute kernels read two floats per query instead of recomputing them.
//
// Layout: a wave covers 64*16 bytes of consecutive rows per step (coalesced
// 16-byte loads); the CPR lanes that share a row reduce their partial dot
// products with cross-lane adds.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {

template <class E, int D, int UNR, bool STR>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const typename E::T* __restrict__ O,
                                                        const typename E::T* __restrict__ dO,
                                                        const float* __restrict__ LSE,
                                                        float* __restrict__ ws, int L, int Sq,
                                                        int H, const Layout lay) {
  // Rows are the B*H*Sq query rows in [B, H, Sq] order; STR: O and dO are
  // laid out by `lay`.
  using T = typename E::T;
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;              // chunks per row (<= 32)
  constexpr int RPW = 64 / CPR;             // rows per wave step
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int chunk = lane % CPR;
  u32x4 a[UNR], b[UNR];
#pragma unroll
  for (int i = 0; i < UNR; ++i) {  // all loads first, then the arithmetic
    const int row = min((wave * UNR + i) * RPW + lane / CPR, L - 1);
    if constexpr (STR) {
      const int bh = row / Sq, s = row % Sq;
      a[i] = *reinterpret_cast<const u32x4*>(O + head_off<STR, D>(lay.o, bh, H, Sq) +
                                              (size_t)s * lay.o.s + chunk * EPC);
      b[i] = *reinterpret_cast<const u32x4*>(dO + head_off<STR, D>(lay.dout, bh, H, Sq) +
                                              (size_t)s * lay.dout.s + chunk * EPC);
    } else {
      a[i] = *reinterpret_cast<const u32x4*>(O + (size_t)row * D + chunk * EPC);
      b[i] = *reinterpret_cast<const u32x4*>(dO + (size_t)row * D + chunk * EPC);
    }
  }
#pragma unroll
  for (int i = 0; i < UNR; ++i) {
    const int row = (wave * UNR + i) * RPW + lane / CPR;
    float acc = 0.f;
    if constexpr (is_bf16<E>()) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, a[i]), y = __builtin_bit_cast(bf16x8, b[i]);
#pragma unroll
      for (int t = 0; t < 8; ++t) acc += (float)x[t] * (float)y[t];
    } else {
      const f32x4 x = __builtin_bit_cast(f32x4, a[i]), y = __builtin_bit_cast(f32x4, b[i]);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc += x[t] * y[t];
    }
    // sum over the CPR lanes of the row (aligned groups of CPR lanes)
#pragma unroll
    for (int o = 1; o < CPR; o <<= 1) acc += __shfl_xor(acc, o);
    if (row < L && chunk == 0) {
      ws[row] = acc;
      // A row with no visible key (LSE = -inf; only with padded keys or
      // more queries than keys) stores 0: its keys are all masked, so
      // exp2(-inf - 0) = 0 is its P everywhere, where -inf - (-inf) would
      // not be.
      const float lse = LSE[row];
      ws[(size_t)L + row] = lse == -INFINITY ? 0.f : lse * kLog2e;
    }
  }
}

template <class E, int D, bool STR>
static hipError_t launch(const BwdArgs& a) {
  constexpr int EPC = 16 / (int)sizeof(typename E::T);
  constexpr int RPW = 64 / (D / EPC);
  constexpr int UNR = is_bf16<E>() ? ATTN_PREP_UNR_BF16 : ATTN_PREP_UNR_F32;
  const int L = a.BH * a.Sq;
  const int waves = (L + RPW * UNR - 1) / (RPW * UNR);
  const int blocks = (waves + 3) / 4;
  using T = typename E::T;
  hipLaunchKernelGGL((bwd_prep_kernel<E, D, UNR, STR>), dim3(blocks), dim3(256), 0, a.stream,
                     (const T*)a.o, (const T*)a.dout, a.lse, a.delta, L, a.Sq, a.H,
                     a.layout != nullptr ? *a.layout : Layout{});
  return hipGetLastError();
}

template <class E>
static hipError_t launch_d(const BwdArgs& a) {
  switch (a.D) {
    case 32: return a.layout ? launch<E, 32, true>(a) : launch<E, 32, false>(a);
    case 64: return a.layout ? launch<E, 64, true>(a) : launch<E, 64, false>(a);
    case 128: return a.layout ? launch<E, 128, true>(a) : launch<E, 128, false>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_prep(const BwdArgs& a) {
  return a.bf16 ? launch_d<EBF16>(a) : launch_d<EF32>(a);
}

}  // namespace attn
