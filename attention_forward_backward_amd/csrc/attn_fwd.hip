// attn_fwd.hip -- tiled attention forward for gfx950.
//
// The forward of the attention node ("Meganeura: Portable GPU Training and
// Inference through Vulkan and Metal", arXiv 2608.01563, Section 3.3, tiled
// attention forward kernel): O = softmax(scale * Q K^T, masked) V and the row
// LSE, with the softmax taken online over key tiles so that no S x S matrix
// exists.
//
// Work split: one workgroup per (query tile of 32*RB rows, batch*head).  Each
// 32-query block is owned by NSPLIT waves that split the key range between
// them (block kb of every staged tile goes to wave kb % NSPLIT); each keeps
// its own running max, sum and O, and the NSPLIT partial results are merged
// through LDS at the end.
//
// K and V stream through an NST-stage ring of LDS tiles (32*NSPLIT*KPW keys
// each) filled by direct global->LDS loads issued NST-1 tiles ahead, with one
// workgroup barrier per tile.
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

template <class E, int D, int NW, int NSPLIT, int KPW, int NST, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, typename E::T* __restrict__ O,
    float* __restrict__ LSE, int S, float c) {
  using T = typename E::T;
  using TL = Tile<E, D>;
  constexpr int RB = NW / NSPLIT;        // 32-query blocks per workgroup
  constexpr int BR = 32 * RB;            // queries per workgroup
  constexpr int BK = 32 * NSPLIT * KPW;  // keys per staged tile
  constexpr int NDB = D / 32;
  using LD = StageLoader<E, D, BK, NW>;
  constexpr int TILEB = BK * TL::ROWB;  // one matrix tile; V follows K in a stage
  constexpr int NV = 16 * NDB + 2;      // floats per lane in a partial result
  constexpr int COMB = RB * (NSPLIT - 1) * NV * 64 * 4;
  constexpr int SMEM = NST * LD::BYTES > COMB ? NST * LD::BYTES : COMB;
  static_assert(NW % NSPLIT == 0 && NST >= 2 && NST <= 4, "launch shape");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar
  const int qb = w / NSPLIT, sp = w % NSPLIT;
  const int bh = blockIdx.x;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;  // longest causal tiles first
  const size_t base = (size_t)bh * S * D;
  const T* k = K + base;
  const T* v = V + base;

  const int q0 = qt * BR + qb * 32;
  const int qi = q0 + n;
  const bool wave_active = q0 < S;

  RowFrag<E, D> qf;
  load_row_frag<E, D>(qf, Q + base + (size_t)min(qi, S - 1) * D + h * (D / 2), qi < S);

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
  float m = -INFINITY;  // exponent reference (log2 domain), lags the row max by < 2^8
  float l = 0.f;        // this half's running sum of exp2(c*score - m)

  const int kend = CAUSAL ? min(S, qt * BR + BR) : S;
  const int nkt = (kend + BK - 1) / BK;

  const unsigned lo = LD::lane_offset(w, lane);
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nkt) LD::issue(smem + s * LD::BYTES, k, v, s * BK, S, w, lane, lo);

  // One staged tile of keys.  When the stages' LDS addresses fit 16-bit
  // offsets, the loop is unrolled by NST with the stage index constant.
  auto step = [&](const int kt, auto sc) __attribute__((always_inline)) {
    const int si = sc;  // kt % NST
    wait_tiles<LD::NLOADS>(min(NST - 2, nkt - 1 - kt));
    lds_barrier();  // tile kt is in LDS; every wave is done with tile kt-1
    if (kt + NST - 1 < nkt)
      LD::issue(smem + ((kt + NST - 1) % NST) * LD::BYTES, k, v, (kt + NST - 1) * BK, S, w, lane, lo);
    if (!wave_active) return;
    const char* Kt = smem + si * LD::BYTES;
    const char* Vt = Kt + TILEB;

      // This wave's 32-key blocks of the tile.  A block is skipped when no key
      // in it is visible from any of the wave's queries, and masked only when
      // some but not all of it is (the causal diagonal, the ragged end).  Every
      // processed block has at least one visible key for every query (block
      // starts are multiples of 32), so row maxima are finite.
  #pragma unroll
      for (int j = 0; j < KPW; ++j) {
        const int kb = sp + NSPLIT * j;
        const int kk0 = kt * BK + kb * 32;
        if (!(kk0 < S && (!CAUSAL || kk0 <= q0 + 31))) continue;  // wave-uniform
        f32x16 sacc = dot_tile<E, D>(Kt, kb * 32 + pi32(n), h, qf, zero16());
        if (kk0 + 32 > S || (CAUSAL && kk0 + 31 > q0)) {
          // key(r) = kk0 + 8h + (16*(r/8) + r%8); visible iff key < S and key <= qi
          const int lim = min(S - 1, CAUSAL ? qi : S - 1) - kk0 - 8 * h;
          // -inf where 16*(r/8) + r%8 > lim, built arithmetically (no
          // per-element compare masks in scalar registers); the whole vector
          // is bit-cast (a bit_cast of one ext_vector element is not reliable)
          u32x16 sb = __builtin_bit_cast(u32x16, sacc);
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const unsigned out = (unsigned)((lim - (16 * (r >> 3) + (r & 7))) >> 31);
            sb[r] = (sb[r] & ~out) | (0xff800000u & out);
          }
          sacc = __builtin_bit_cast(f32x16, sb);
        }
        float mx = -INFINITY;  // max of the raw (unscaled) visible scores
  #pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[r], sacc[r + 1]));
        mx = fmaxf(mx, xhalf(mx));
        // Lazy rescaling: exponents are taken against a reference m that may
        // lag the running max by up to 2^8, so O and l are rescaled only when
        // some row's max grows past that (on a wave's first block they are 0).
        const float mc = mx * c;
        if (__any(mc > m + 8.f)) {
          const float mnew = fmaxf(m, mc);
          const float alpha = fast_exp2(m - mnew);
          m = mnew;
          l *= alpha;
  #pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        }
        float rs = 0.f;
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[r], c, -m));
          sacc[r] = p;
          rs += p;
        }
        l += rs;
        RegOperand<E> P;
        P.set(sacc);
  #pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = second_tile<E, D, false>(P, Vt, kb * 32, db * 32, lane, oacc[db]);
      }
  };
  if constexpr (NST * LD::BYTES <= 65536) {
    for_stages<NST>(nkt, step);
  } else {
    for (int kt = 0; kt < nkt; ++kt) step(kt, kt % NST);
  }

  // Merge the NSPLIT partial (m, l, O) of each query block through LDS.
  l += xhalf(l);
  if constexpr (NSPLIT > 1) {
    float* cb = reinterpret_cast<float*>(smem);
    lds_barrier();  // every wave is done with the K/V tiles (no loads pending)
    if (sp != 0 && wave_active) {
      float* dst = cb + ((qb * (NSPLIT - 1) + sp - 1) * NV) * 64 + lane;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(db * 16 + r) * 64] = oacc[db][r];
      dst[(16 * NDB) * 64] = m;
      dst[(16 * NDB + 1) * 64] = l;
    }
    lds_barrier();
    if (sp != 0 || !wave_active) return;
#pragma unroll
    for (int p = 0; p < NSPLIT - 1; ++p) {
      const float* src = cb + ((qb * (NSPLIT - 1) + p) * NV) * 64 + lane;
      const float mp = src[(16 * NDB) * 64];
      const float lp = src[(16 * NDB + 1) * 64];
      const float mnew = fmaxf(m, mp);  // finite: split 0 always sees key 0
      const float a0 = fast_exp2(m - mnew), a1 = fast_exp2(mp - mnew);
      l = l * a0 + lp * a1;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = oacc[db][r] * a0 + src[(db * 16 + r) * 64] * a1;
      m = mnew;
    }
  } else {
    if (!wave_active) return;
  }

  const float inv = 1.f / l;
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
    if (h == 0) LSE[(size_t)bh * S + qi] = (m + __log2f(l)) * kLn2;
  }
}

template <class E, int D, bool CAUSAL>
static hipError_t launch(const FwdArgs& a) {
  constexpr int NW = is_bf16<E>() ? ATTN_FWD_NW_BF16 : ATTN_FWD_NW_F32;
  constexpr int NSPLIT = is_bf16<E>() ? ATTN_FWD_NSPLIT_BF16 : ATTN_FWD_NSPLIT_F32;
  constexpr int KPW = is_bf16<E>() ? ATTN_FWD_KPW_BF16 : ATTN_FWD_KPW_F32;
  constexpr int NST = is_bf16<E>() ? ATTN_FWD_NST_BF16 : ATTN_FWD_NST_F32;
  using T = typename E::T;
  constexpr int BR = 32 * (NW / NSPLIT);
  const int nqt = (a.S + BR - 1) / BR;
  dim3 grid(a.BH, nqt);
  hipLaunchKernelGGL((fwd_kernel<E, D, NW, NSPLIT, KPW, NST, CAUSAL>), grid, dim3(NW * 64), 0,
                     a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.o, a.lse, a.S,
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
