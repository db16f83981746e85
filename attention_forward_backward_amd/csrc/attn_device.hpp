// attn_device.hpp -- device-side building blocks shared by the attention
// kernels (gfx950 / CDNA4, 64-lane wavefronts).
//
// Every contraction runs on the 32x32 MFMA shapes:
//   strict f32 : v_mfma_f32_32x32x2_f32   (per lane one f32 of A and of B)
//   bf16       : v_mfma_f32_32x32x16_bf16 (per lane eight bf16 of A and of B)
// For both, lane l (n = l % 32, h = l / 32) feeds row n of A and column n of
// B with the k-slots of half h, and receives output rows
//   m(r, h) = 8*(r/4) + 4*h + (r%4),  r = 0..15,  column n.
//
// Attention chains two contractions: a score-like product whose 32x32
// output stays in registers, then a product that consumes those registers as
// an operand with the 32 output rows as its k dimension.  To make the
// hand-over free, A-operand row m of the first product is loaded from
// logical row pi32(m) = 16*(j/2) + 8*hh + 4*(j%2) + i, where m = 8j + 4hh + i
// (a bijection on 0..31), so that output element r of a lane in half h
// belongs to logical row
//   rho(r, h) = 16*(r/8) + 8*h + (r%8).
// A lane then owns two runs of eight consecutive logical rows, which is
// exactly the k-slot pattern of the second product (slot (h, t) of MFMA u is
// logical row 16u + 8h + t for bf16; slot h of step w is rho(w, h) for f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ element types
struct EF32 {
  using T = float;
  static constexpr int KL = 1;  // k elements per lane per MFMA operand
  using Frag = float;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

struct EBF16 {
  using T = __bf16;
  static constexpr int KL = 8;
  using Frag = bf16x8;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <class E> constexpr bool is_bf16() { return E::KL == 8; }

// Row stride (elements) of a row-major tile with D columns in LDS: pads each
// row by 16 bytes so that 16 lanes reading 16-byte chunks from 16 different
// rows, and 32 lanes reading one row while 32 read the row 8 further on,
// touch disjoint banks.
template <class E, int D> constexpr int row_stride() {
  return is_bf16<E>() ? D + 8 : D + 4;
}
// Row stride of a transposed bf16 tile [column][row] holding N rows.
template <int N> constexpr int tr_stride() { return N + 8; }

// ------------------------------------------------------------------ lane maps
__device__ inline int pi32(int m) {
  // A-operand row m of the score product reads logical row pi32(m).
  const int j = m >> 3, hh = (m >> 2) & 1, i = m & 3;
  return ((j >> 1) << 4) + (hh << 3) + ((j & 1) << 2) + i;
}
__host__ __device__ constexpr int rho(int r, int h) {
  // Logical row of output element r in lane half h (see header comment).
  return 16 * (r >> 3) + 8 * h + (r & 7);
}
__host__ __device__ constexpr int out_row(int r, int h) {
  // Physical MFMA output row of element r in lane half h.
  return 8 * (r >> 2) + 4 * h + (r & 3);
}

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ inline float xhalf(float x) { return __shfl_xor(x, 32); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <class T> __device__ inline float to_f32(T x) { return (float)x; }

// ------------------------------------------------------------------ row fragments
// The register-resident operand of a score product: lane (n, h) holds
// elements [h*D/2, h*D/2 + D/2) of one row (its query or key), as KL-wide
// MFMA fragments in d order.
template <class E, int D>
struct RowFrag {
  static constexpr int NS = D / (2 * E::KL);  // MFMA steps over d
  typename E::Frag f[NS];
};

template <class E, int D>
__device__ inline void load_row_frag(RowFrag<E, D>& rf, const typename E::T* p, bool valid) {
  // p points at element h*D/2 of the row; reads D/2 contiguous elements.
  constexpr int NCH = (D / 2) * (int)sizeof(typename E::T) / 16;
  const u32x4* src = reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    u32x4 x = valid ? src[c] : u32x4{0u, 0u, 0u, 0u};
    if constexpr (is_bf16<E>()) {
      rf.f[c] = __builtin_bit_cast(bf16x8, x);
    } else {
      // bit-cast the whole vector: a bit_cast of one ext_vector element is
      // not reliable here (it read element 0 for every e)
      const f32x4 xf = __builtin_bit_cast(f32x4, x);
#pragma unroll
      for (int e = 0; e < 4; ++e) rf.f[4 * c + e] = xf[e];
    }
  }
}

// acc += A * B where A row (this lane's) is the LDS row `arow` (already
// offset by h*D/2) and B column is the register fragment `b`.
template <class E, int D>
__device__ inline f32x16 dot_rows(const typename E::T* arow, const RowFrag<E, D>& b, f32x16 acc) {
  constexpr int NCH = (D / 2) * (int)sizeof(typename E::T) / 16;
  const u32x4* src = reinterpret_cast<const u32x4*>(arow);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const u32x4 x = src[c];
    if constexpr (is_bf16<E>()) {
      acc = E::mma(__builtin_bit_cast(bf16x8, x), b.f[c], acc);
    } else {
      const f32x4 xf = __builtin_bit_cast(f32x4, x);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = E::mma(xf[e], b.f[4 * c + e], acc);
    }
  }
  return acc;
}

// Same as dot_rows with the operands swapped: the register fragment is A
// (this lane's row) and the LDS row is B (this lane's column).
template <class E, int D>
__device__ inline f32x16 dot_rows_swapped(const RowFrag<E, D>& a, const typename E::T* brow, f32x16 acc) {
  constexpr int NCH = (D / 2) * (int)sizeof(typename E::T) / 16;
  const u32x4* src = reinterpret_cast<const u32x4*>(brow);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const u32x4 x = src[c];
    if constexpr (is_bf16<E>()) {
      acc = E::mma(a.f[c], __builtin_bit_cast(bf16x8, x), acc);
    } else {
      const f32x4 xf = __builtin_bit_cast(f32x4, x);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = E::mma(a.f[4 * c + e], xf[e], acc);
    }
  }
  return acc;
}

// ------------------------------------------------------------------ second product
// The register operand of the second product: the 16 f32 values of one 32x32
// output block of the first product (logical rows rho(r, h)), rounded to the
// MFMA operand type.
template <class E>
struct RegOperand;

template <>
struct RegOperand<EF32> {
  float v[16];
  __device__ inline void set(const f32x16& x) {
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = x[r];
  }
};

template <>
struct RegOperand<EBF16> {
  bf16x8 v[2];
  __device__ inline void set(const f32x16& x) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < 8; ++t) v[u][t] = (__bf16)x[8 * u + t];  // round to nearest even
  }
};

// acc += R^T-side product over 32 logical rows of a tile in LDS.
//   REG_IS_A = true : acc[m][n] += sum_k R[m = this lane's row][k] * X[k][col0 + n]
//   REG_IS_A = false: acc[m][n] += sum_k X[k][col0 + m] * R[k][n = this lane's column]
// where k runs over the 32 logical rows row0 .. row0+31 of X, and R's k-slots
// are the lane's rho rows.  X is read from
//   f32 : the row-major tile `x` (stride STR): element [row][col]
//   bf16: the transposed tile `xt` (stride STRT): element [col][row]
template <class E, int STR, int STRT, bool REG_IS_A>
__device__ inline f32x16 second_product(const RegOperand<E>& R, const typename E::T* x,
                                        const typename E::T* xt, int row0, int col, int h,
                                        f32x16 acc) {
  if constexpr (is_bf16<E>()) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 o = *reinterpret_cast<const bf16x8*>(xt + col * STRT + row0 + 16 * u + 8 * h);
      acc = REG_IS_A ? E::mma(R.v[u], o, acc) : E::mma(o, R.v[u], acc);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const float o = x[(row0 + rho(w, h)) * STR + col];
      acc = REG_IS_A ? E::mma(R.v[w], o, acc) : E::mma(o, R.v[w], acc);
    }
  }
  return acc;
}

// ------------------------------------------------------------------ tile staging
// A ROWS x D tile of a row-major [S x D] matrix, held in registers as 16-byte
// chunks between the global load and the LDS store (so the next tile's loads
// are in flight while the current tile is being used).  Rows >= S read as 0.
template <class T, int ROWS, int D, int NT>
struct TileRegs {
  static constexpr int CH = 16 / (int)sizeof(T);
  static constexpr int CPR = D / CH;           // chunks per row
  static constexpr int TOTAL = ROWS * CPR;     // chunks per tile
  static constexpr int N = (TOTAL + NT - 1) / NT;
  u32x4 c[N];

  __device__ inline void load(const T* base, int r0, int S, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / CPR, col = (idx % CPR) * CH;
      const bool ok = (TOTAL % NT == 0 || idx < TOTAL) && (r0 + row < S);
      // the address is clamped into the matrix even when the value is unused
      const int srow = min(r0 + row, S - 1);
      const int scol = (TOTAL % NT == 0 || idx < TOTAL) ? col : 0;
      c[i] = ok ? *reinterpret_cast<const u32x4*>(base + (size_t)srow * D + scol)
                : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // Row-major into LDS with row stride STR (elements).
  template <int STR>
  __device__ inline void store(T* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + i * NT;
      if (TOTAL % NT == 0 || idx < TOTAL) {
        const int row = idx / CPR, col = (idx % CPR) * CH;
        *reinterpret_cast<u32x4*>(lds + row * STR + col) = c[i];
      }
    }
  }
  // Transposed into LDS: element [row][col] goes to lds[col * STRT + row].
  template <int STRT>
  __device__ inline void store_t(T* lds, int tid) const {
    static_assert(sizeof(T) == 2, "transposed staging is for 16-bit elements");
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + i * NT;
      if (TOTAL % NT == 0 || idx < TOTAL) {
        const int row = idx / CPR, col = (idx % CPR) * CH;
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&c[i]);
        uint16_t* dst = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
        for (int t = 0; t < CH; ++t) dst[(col + t) * STRT + row] = e[t];
      }
    }
  }
};

// Store the 4 consecutive values x[4j .. 4j+3] of a lane's output block to
// p[0..3] (converted to T).
template <class T>
__device__ inline void store4(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
  } else {
    bf16x4 v;
    v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
    *reinterpret_cast<bf16x4*>(p) = v;
  }
}

}  // namespace attn
