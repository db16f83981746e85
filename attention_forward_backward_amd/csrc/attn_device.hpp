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

#include <type_traits>
#include <stdint.h>

namespace attn {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

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

// f32 storage with bf16 MFMA operands: the forward of the pages' practical
// contract ("Meganeura", Section 4.2: eligible forward matrix and attention
// inputs rounded locally to reduced precision, f32 accumulation, f32
// stores).  Tiles stay f32 in LDS; Q, K and V are rounded to bf16
// (nearest-even) as they become MFMA operands, and P as in EBF16.
struct EF32B {
  using T = float;
  static constexpr int KL = 8;
  using Frag = bf16x8;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// Storage (tile layout, loads, stores) is bf16.
template <class E> __host__ __device__ constexpr bool is_bf16() { return sizeof(typename E::T) == 2; }
// MFMA operands are bf16 (8 k-values per lane).
template <class E> __host__ __device__ constexpr bool mma_bf16() { return E::KL == 8; }

// Four floats rounded to bf16 (nearest-even) into elements 4j .. 4j+3 of v.
__device__ inline void put_bf16x4(bf16x8& v, int j, f32x4 x) {
#pragma unroll
  for (int e = 0; e < 4; ++e) v[4 * j + e] = (__bf16)x[e];
}

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

// ------------------------------------------------------------------ row fragments
// The register-resident operand of a score product: lane (n, h) holds
// elements [h*D/2, h*D/2 + D/2) of one row (its query or key), as KL-wide
// MFMA fragments in d order.
template <class E, int D>
struct RowFrag {
  static constexpr int NS = D / (2 * E::KL);  // MFMA steps over d
  typename E::Frag f[NS];
};

// Store 16 bytes (chunk c of the lane's half row) into the fragment.
template <class E, int D>
__device__ inline void set_frag_chunk(RowFrag<E, D>& rf, int c, u32x4 x) {
  if constexpr (is_bf16<E>()) {
    rf.f[c] = __builtin_bit_cast(bf16x8, x);
  } else if constexpr (mma_bf16<E>()) {
    // f32 storage, bf16 operands: chunk c is half (c & 1) of fragment c / 2
    put_bf16x4(rf.f[c >> 1], c & 1, __builtin_bit_cast(f32x4, x));
  } else {
    // bit-cast the whole vector: a bit_cast of one ext_vector element is
    // not reliable here (it read element 0 for every e)
    const f32x4 xf = __builtin_bit_cast(f32x4, x);
#pragma unroll
    for (int e = 0; e < 4; ++e) rf.f[4 * c + e] = xf[e];
  }
}

template <class E, int D>
__device__ inline void load_row_frag(RowFrag<E, D>& rf, const typename E::T* p, bool valid) {
  // p points at element h*D/2 of the row; reads D/2 contiguous elements.
  constexpr int NCH = (D / 2) * (int)sizeof(typename E::T) / 16;
  const u32x4* src = reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int c = 0; c < NCH; ++c) set_frag_chunk(rf, c, valid ? src[c] : u32x4{0u, 0u, 0u, 0u});
}

// ------------------------------------------------------------------ LDS tiles
// Tiles live in LDS row-major and unpadded (D elements per row), filled by
// direct global->LDS 16-byte loads, with the 16-byte chunks of each row
// permuted by an XOR swizzle so that every read pattern below is free of bank
// conflicts:
//   (A) score operand: 16 lanes read the same chunk of 16 different rows
//       (ds_read_b128);
//   (B) f32 second operand: 32 lanes read 32 consecutive floats of one row
//       while the other 32 read the row 8 further on (ds_read_b32);
//   (C) bf16 second operand: transposed reads of 4 consecutive rows x 32
//       columns per half wave (ds_read_b64_tr_b16).
// Every swizzle depends on row % 16 only, so offsets of 16-row aligned blocks
// are additive.  (f32 with D = 32 keeps a 2-way conflict on pattern B: the
// two rows 8 apart share a bank half whatever the swizzle.)
// KS selects a second f32 layout for tiles read only by pattern B: chunk c of
// row r sits at c ^ (8 * bit 3 of r), which is all pattern B needs (its two
// half waves read rows 8 apart and land in opposite bank halves), and which
// leaves the 16 rows of one read sequence a fixed distance apart, so a lane
// forms their addresses from one base with immediate offsets instead of one
// XOR per read.  bf16 storage ignores KS.
template <class E, int D, bool KS = false>
struct Tile {
  using T = typename E::T;
  static constexpr int ROWB = D * (int)sizeof(T);  // bytes per row
  static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
  static constexpr int EPC = 16 / (int)sizeof(T);  // elements per chunk
  __host__ __device__ static constexpr int swz(int row) {
    if constexpr (is_bf16<E>()) {
      if constexpr (CPR == 4) return (row >> 2) & 3;
      else if constexpr (CPR == 8) return ((row >> 1) & 7) ^ (((row >> 1) & 1) << 2);
      else return ((row & 3) << 2) | ((row >> 2) & 3);
    } else if constexpr (KS) {
      return CPR >= 16 ? ((row >> 3) & 1) << 3 : 0;
    } else {
      if constexpr (CPR == 8) return (row >> 1) & 7;
      else return row & 15;
    }
  }
  // Byte offset of element (row, col) in the tile.
  __host__ __device__ static constexpr int off(int row, int col) {
    return row * ROWB + (((col / EPC) ^ swz(row)) << 4) + (col % EPC) * (int)sizeof(T);
  }
};

// The row fragment of tile row `row` (this lane's key or query), read from a
// swizzled LDS tile: half h of the row, 16 bytes at a time (read pattern A).
// Rows that are not valid read as zero.
template <class E, int D>
__device__ inline void load_row_frag_lds(RowFrag<E, D>& rf, const char* tile, int row, int h,
                                         bool valid) {
  using TL = Tile<E, D>;
  constexpr int NCH = TL::CPR / 2;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const u32x4 x =
        *reinterpret_cast<const u32x4*>(tile + row * TL::ROWB + (((h * NCH + c) ^ TL::swz(row)) << 4));
    set_frag_chunk(rf, c, valid ? x : u32x4{0u, 0u, 0u, 0u});
  }
}

// ------------------------------------------------------------------ rotary embedding
// Rotate-half RoPE (the axial RoPE of "Meganeura", Section 5.2, applied to Q
// and K in front of the attention; 1-D and axial positions differ only in
// the angle tables): pair (x_i, x_{i+D/2}) of a row is turned by the angle
// of cosine c and sine s,
//   y_i = x_i c - x_{i+D/2} s,   y_{i+D/2} = x_{i+D/2} c + x_i s,
// and with s negated by the transposed rotation (the map of the gradient
// with respect to the turned row back to the row).  Every site that turns
// rows -- the rotation pass, the forward's Q operand, the dQ and dK stores --
// rounds the same way: each output is fma(own, c, -+(other * s)).
__device__ inline void rope_pair(float lo, float hi, float c, float s, float& ylo, float& yhi) {
  ylo = fmaf(lo, c, -(hi * s));
  yhi = fmaf(hi, c, lo * s);
}

// 16-byte LDS read and write through restrict pointers: with the alias-scope
// metadata they carry, the compiler's wait insertion does not take them for
// accesses to LDS that a direct global->LDS load in flight may write (it
// would put a vmcnt(0) before them, draining the ring's prefetched tiles).
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
__device__ __attribute__((always_inline)) inline u32x4 lds_read16(const lds_u32x4* __restrict__ p) {
  return *p;
}
__device__ __attribute__((always_inline)) inline void lds_write16(lds_u32x4* __restrict__ p,
                                                                  u32x4 v) {
  *p = v;
}

// RoPE on a [BR x D] tile of rows in LDS (swizzled as Tile<E, D>) filled by
// the direct loads of TileLoader / StageLoader over NW waves: 1 KiB slot s of
// the tile holds rows s*RPS .. s*RPS + RPS - 1 (every chunk of them) and is
// loaded by wave s % NW, so once a wave's own loads are complete it can turn
// the rows of its slots in place with no barrier.  Unit u of a wave = (row,
// chunk ch of the lower half) turns the chunk's columns i with their
// partners i + D/2; a slot has RPS * D/2 / EPC = 32 units.  load() fetches
// the angles of a lane's units (float32 tables [rows][D/2]; row r of the
// tile is sequence position pos0 + r, clamped to the last valid one);
// apply() turns the units, rounds to the storage type as a rotation pass
// would, writes them back and, when out is not null, stores rows below
// `rows` to out + r * D (the turned rows).
template <class E, int D, int BR, int NW>
struct TileRope {
  using TL = Tile<E, D>;
  using T = typename E::T;
  static constexpr int NCH = TL::CPR / 2;  // 16-byte chunks per half row
  static constexpr int EPC = TL::EPC;
  static constexpr int RPS = 64 / TL::CPR;             // rows per slot
  static constexpr int SPW = BR * TL::CPR / 64 / NW;   // slots per wave
  static constexpr int UNITS = SPW * 32;               // units per wave
  static constexpr int UPT = (UNITS + 63) / 64;        // units per lane (the last may idle)
  static_assert(BR * TL::CPR % (64 * NW) == 0 && RPS * NCH == 32, "tile slots split over waves");
  f32x4 c[UPT * EPC / 4], s[UPT * EPC / 4];

  __device__ static inline void unit(int k, int w, int lane, int& r, int& ch) {
    const int u = k * 64 + lane;
    const int slot = w + (u / 32) * NW, v = u % 32;
    r = slot * RPS + v / NCH;
    ch = v % NCH;
  }

  __device__ inline void load(const float* __restrict__ cs, const float* __restrict__ sn, int pos0,
                              int rows, int w, int lane) {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      if (UNITS % 64 != 0 && k * 64 + lane >= UNITS) break;
      int r, ch;
      unit(k, w, lane, r, ch);
      const size_t t = (size_t)(pos0 + min(r, rows - 1)) * (D / 2) + ch * EPC;
#pragma unroll
      for (int v = 0; v < EPC / 4; ++v) {
        c[k * (EPC / 4) + v] = *reinterpret_cast<const f32x4*>(cs + t + 4 * v);
        s[k * (EPC / 4) + v] = *reinterpret_cast<const f32x4*>(sn + t + 4 * v);
      }
    }
  }

  // An empty use of the angles: the compiler's wait for their loads goes
  // here (placed where no load the ring prefetches is in flight), so that
  // apply() later needs none.
  __device__ inline void ready() const {
#pragma unroll
    for (int k = 0; k < UPT * EPC / 4; ++k) asm volatile("" ::"v"(c[k]), "v"(s[k]));
  }

  __device__ inline void apply(char* tile, T* out, int rows, int w, int lane) const {
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      if (UNITS % 64 != 0 && k * 64 + lane >= UNITS) break;
      int r, ch;
      unit(k, w, lane, r, ch);
      lds_u32x4* plo = (lds_u32x4*)(tile + r * TL::ROWB + ((ch ^ TL::swz(r)) << 4));
      lds_u32x4* phi = (lds_u32x4*)(tile + r * TL::ROWB + (((ch + NCH) ^ TL::swz(r)) << 4));
      u32x4 lo = lds_read16(plo), hi = lds_read16(phi);
      if constexpr (sizeof(T) == 4) {
        f32x4 a = __builtin_bit_cast(f32x4, lo), b = __builtin_bit_cast(f32x4, hi);
        const f32x4 cc = c[k], ss = s[k];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float ylo, yhi;
          rope_pair(a[e], b[e], cc[e], ss[e], ylo, yhi);
          a[e] = ylo;
          b[e] = yhi;
        }
        lo = __builtin_bit_cast(u32x4, a);
        hi = __builtin_bit_cast(u32x4, b);
      } else {
        bf16x8 a = __builtin_bit_cast(bf16x8, lo), b = __builtin_bit_cast(bf16x8, hi);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float ylo, yhi;
          rope_pair((float)a[e], (float)b[e], c[2 * k + e / 4][e % 4], s[2 * k + e / 4][e % 4], ylo,
                    yhi);
          a[e] = (__bf16)ylo;
          b[e] = (__bf16)yhi;
        }
        lo = __builtin_bit_cast(u32x4, a);
        hi = __builtin_bit_cast(u32x4, b);
      }
      lds_write16(plo, lo);
      lds_write16(phi, hi);
      if (out != nullptr && r < rows) {
        T* o = out + (size_t)r * D + ch * EPC;
        *reinterpret_cast<u32x4*>(o) = lo;
        *reinterpret_cast<u32x4*>(o + D / 2) = hi;
      }
    }
  }
};

// The transposed rotation applied to a row held in MFMA output
// accumulators: element 4j+e of acc[db] is column db*32 + 8j + 4h + e of the
// lane's row (the dK^T and dQ^T accumulators), so both columns of every
// pair (i, i + D/2) are in the lane.  load() fetches the row's angles at the
// lane's lower-half columns (cs, sn point at the row), apply() turns acc.
template <int D>
struct RopeAccRow {
  static constexpr int NDB = D / 32;
  static constexpr int NG = D >= 64 ? 2 * NDB : 2;  // groups of 4 lower-half columns
  f32x4 c[NG], s[NG];
  // group g: lower column block lb, group j in it; the partner is D/2 on
  __device__ static constexpr int lb(int g) { return D >= 64 ? g / 4 : 0; }
  __device__ static constexpr int jj(int g) { return D >= 64 ? g % 4 : g; }
  __device__ inline void load(const float* __restrict__ cs, const float* __restrict__ sn, int h) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int i = lb(g) * 32 + 8 * jj(g) + 4 * h;
      c[g] = *reinterpret_cast<const f32x4*>(cs + i);
      s[g] = *reinterpret_cast<const f32x4*>(sn + i);
    }
  }
  __device__ inline void apply(f32x16 (&acc)[NDB]) const {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int l = lb(g), j = jj(g);
      const int hb = D >= 64 ? l + NDB / 2 : 0, hj = D >= 64 ? j : j + 2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float ylo, yhi;
        rope_pair(acc[l][4 * j + e], acc[hb][4 * hj + e], c[g][e], -s[g][e], ylo, yhi);
        acc[l][4 * j + e] = ylo;
        acc[hb][4 * hj + e] = yhi;
      }
    }
  }
};
template <int D>
__device__ inline void rope_back_acc(f32x16 (&acc)[D / 32], const float* __restrict__ cs,
                                     const float* __restrict__ sn, int h) {
  RopeAccRow<D> r;
  r.load(cs, sn, h);
  r.apply(acc);
}

// Run f(t, stage) for t = 0 .. n-1, where stage = t % NST is passed as a
// compile-time constant (std::integral_constant): the loop is unrolled by
// NST so that each stage's LDS base folds into the reads' 16-bit immediate
// offsets, and the loop-carried state flows from one stage's body into the
// next.
template <int NST, class F>
__device__ inline void for_stages(int n, F&& f) {
  for (int t0 = 0; t0 < n; t0 += NST) {
    f(t0, std::integral_constant<int, 0>{});
    if constexpr (NST >= 2) {
      if (t0 + 1 < n) f(t0 + 1, std::integral_constant<int, 1>{});
    }
    if constexpr (NST >= 3) {
      if (t0 + 2 < n) f(t0 + 2, std::integral_constant<int, 2>{});
    }
    if constexpr (NST >= 4) {
      if (t0 + 3 < n) f(t0 + 3, std::integral_constant<int, 3>{});
    }
  }
}

// Static persistent schedule: in round r workgroup g of G takes item
// r*G + g (r even) or r*G + g' (r odd), where g' reverses the order of the
// workgroups that share g's residue mod 8 (items are numbered in order of
// decreasing work, so the reversal evens out the per-workgroup totals).
// Workgroups are dispatched round-robin over the 8 XCDs, so keeping the
// residue keeps every item of a head on one XCD and its L2.  Item numbers
// grow with r, so a workgroup stops at its first number >= the count.
__host__ __device__ inline int snake_item(int r, int g, int G) {
  if (!(r & 1)) return r * G + g;
  const int gr = (G % 8 == 0) ? g % 8 + 8 * (G / 8 - 1 - g / 8) : G - 1 - g;
  return r * G + gr;
}

// Keys of batch*head bh that exist for the softmax: the first L of Sk, and
// the causal offset off, so that key j is visible from query i iff j < L
// and, when causal, j <= i + off (off = L - Sq aligns the causal diagonal
// with the end of the valid keys).  Self-attention (CROSS = false): L = Sk,
// off = 0.  kvlen (valid keys per batch, device memory) may be null; its
// values are clamped to [0, Sk].
template <bool CROSS>
__device__ inline void head_keys(const int* __restrict__ kvlen, int bh, int H, int Sq, int Sk,
                                 int& L, int& off) {
  if constexpr (!CROSS) {
    L = Sk;
    off = 0;
  } else {
    L = Sk;
    if (kvlen != nullptr) L = min(max(kvlen[bh / H], 0), Sk);
    off = L - Sq;
  }
}

// Element strides (batch, head, row) of a tensor indexed [B, H, S, D] whose
// head dimension is contiguous, and the layout of every tensor of a call
// (strided entry points; the other entry points use [B, H, S, D] row-major).
struct Str3 {
  int b, h, s;  // (the host checks each is below 2^31)
};
struct Layout {
  Str3 q, k, v, o, dout, dq, dk, dv;
};

// RoPE of a fused call: row p of the float32 tables cos, sin [rows][D/2]
// holds the angles of sequence position p - pos; out, kout: where the
// forward stores the turned Q and K rows ([B, H, S, D] row-major, the
// storage type).
struct RopeTab {
  const float* cos = nullptr;
  const float* sin = nullptr;
  int pos = 0;
  void* out = nullptr;
  void* kout = nullptr;
};

// First element of head bh's rows: with STR from the strides, else in the
// row-major [B, H, rows, D] layout.
template <bool STR, int D>
__device__ inline size_t head_off(const Str3& st, int bh, int H, int rows) {
  if constexpr (STR)
    return (size_t)(bh / H) * (unsigned)st.b + (size_t)(bh % H) * (unsigned)st.h;
  else
    return (size_t)bh * rows * D;
}
// Elements between consecutive rows.
template <bool STR, int D>
__device__ inline int row_ld(const Str3& st) {
  if constexpr (STR)
    return (int)st.s;
  else
    return D;
}

// Static schedule of a persistent launch, computed on the host and passed by
// value in the kernel arguments.  Workgroups are dispatched round-robin over
// the 8 XCDs, so workgroup g runs on XCD g % 8 as its slot g / 8.  When the
// head count is a multiple of 8, head b is kept on XCD b % 8 and every XCD
// runs the same pattern: slot j takes first[j] in round 0 and
// ent[(r-1) * M + j] in round r >= 1 (0xffff: none, and none after it), each
// naming (work class c, local head u) as (c << 8) | u, which is item
// c * BH + 8u + g % 8.  Every lookup is one load at an address that needs
// no other load (round 0's not even M), so a workgroup's first item is known
// one scalar-load latency after it starts.  M = 0: no pattern, the snake
// order applies.
constexpr int kSchedSlots = 256;
constexpr int kSchedEntries = 1280;
struct Sched {
  int M;  // slots per XCD, or 0
  int R;  // rounds in the table
  alignas(4) uint16_t first[kSchedSlots];
  alignas(4) uint16_t ent[kSchedEntries];
};

// Item of round r of workgroup g (a value >= every item count once g has no
// more items).
// The 16-bit entries are read as the 32-bit words that hold them: with a
// wave-uniform index those are scalar loads, while a 16-bit read would be a
// vector load (and a vector-memory wait that also drains the tile loads).
__host__ __device__ inline int sched_entry(const uint16_t* a, int i) {
  const uint32_t v = reinterpret_cast<const uint32_t*>(a)[i >> 1];
  return (int)((i & 1) ? v >> 16 : v & 0xffffu);
}
__host__ __device__ inline int sched_item(const Sched& s, int r, int g, int G, int BH) {
  const int e0 = sched_entry(s.first, (g >> 3) & (kSchedSlots - 1));
  if (s.M == 0) return snake_item(r, g, G);
  if (r >= s.R) return 0x7fffffff;
  const int e = r == 0 ? e0 : sched_entry(s.ent, (r - 1) * s.M + (g >> 3));
  if (e == 0xffff) return 0x7fffffff;
  return (e >> 8) * BH + 8 * (e & 255) + (g & 7);
}

// Wait until at most N vector-memory operations of this wave are pending.
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait until at most n (clamped to 0..63) vector-memory operations of this
// wave are pending, for a wave-uniform n known only at run time: a binary
// search over the immediate forms.
template <int LO, int HI>
__device__ inline void wait_vmem_range(int n) {
  if constexpr (LO == HI) {
    wait_vmem<LO>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID) wait_vmem_range<MID, HI>(n);
    else wait_vmem_range<LO, MID - 1>(n);
  }
}
__device__ inline void wait_vmem_dyn(int n) { wait_vmem_range<0, 63>(n < 0 ? 0 : n); }

// Wait for the oldest staged tile when `newer` younger tiles (NL loads each)
// may stay in flight, and after them `blocks` groups of NS stores each
// (vmcnt counts stores as well as loads, and vector memory operations retire
// in issue order, so the stores issued after the younger tiles' loads are
// the ones that may stay outstanding).
template <int NL, int NS = 0>
__device__ inline void wait_tiles(int newer, int blocks = 0) {
  if (blocks >= 2) {
    if (newer >= 2) wait_vmem<2 * NL + 2 * NS>();
    else if (newer == 1) wait_vmem<NL + 2 * NS>();
    else wait_vmem<2 * NS>();
  } else if (blocks == 1) {
    if (newer >= 2) wait_vmem<2 * NL + NS>();
    else if (newer == 1) wait_vmem<NL + NS>();
    else wait_vmem<NS>();
  } else {
    if (newer >= 2) wait_vmem<2 * NL>();
    else if (newer == 1) wait_vmem<NL>();
    else wait_vmem<0>();
  }
}
// The issue count just after the loads of the tile in each slot of an
// NST-stage ring (see the kernels' wait rule), as separate scalars: a small
// array indexed by a run-time slot would be placed in LDS by the compiler.
template <int NST>
struct RingMarks {
  int m0 = 0, m1 = 0, m2 = 0, m3 = 0;
  __host__ __device__ inline void set(int slot, int v) {
    if (slot == 0) m0 = v;
    if (NST > 1 && slot == 1) m1 = v;
    if (NST > 2 && slot == 2) m2 = v;
    if (NST > 3 && slot == 3) m3 = v;
  }
  __host__ __device__ inline int get(int slot) const {
    int v = m0;
    if (NST > 1 && slot == 1) v = m1;
    if (NST > 2 && slot == 2) v = m2;
    if (NST > 3 && slot == 3) v = m3;
    return v;
  }
};

// Workgroup barrier that orders LDS accesses without waiting for pending
// global loads (those are waited for explicitly with wait_vmem).
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Address of a direct load: a wave-uniform base plus this lane's byte
// offset.  The base is passed through an empty asm statement so the
// compiler keeps it in SGPRs and adds the one lane offset per load, instead
// of hoisting base+offset pairs into loop-invariant VGPRs.
__device__ inline const void* lane_addr(const void* base, unsigned lane_bytes) {
  unsigned long long b = reinterpret_cast<unsigned long long>(base);
  asm volatile("" : "+s"(b));
  return reinterpret_cast<const void*>(b + lane_bytes);
}

// The direct loads of one staged tile: rows row0 .. row0+BT-1 of two
// row-major [S x D] matrices (src0, src1) into two consecutive swizzled
// tiles at `stage`, the second in the KS1 layout of Tile.  Rows past S read
// row S-1 (finite; the caller masks them).  Each wave issues NLOADS
// instructions, each filling 1 KiB of LDS.
//
// A wave's consecutive loads are RS rows apart.  The swizzle repeats every
// 16 rows, so when RS and BT are multiples of 16 every load of a wave into
// one matrix has the same lane offset from its (wave-uniform) first row:
// lane_offset() is then computed once per kernel per matrix and a whole tile
// costs one address add per load.  The clamped per-lane form remains for
// tiles that cross S.
template <class E, int D, int BT, int NW, bool KS1 = false>
struct StageLoader {
  using T = typename E::T;
  using TL = Tile<E, D>;
  using TL1 = Tile<E, D, KS1>;
  static constexpr int CH_PER = BT * TL::CPR;            // chunks per matrix
  static constexpr int NLOADS = 2 * CH_PER / (NW * 64);  // per wave
  static constexpr int BYTES = 2 * BT * TL::ROWB;
  static constexpr int RPS = 64 / TL::CPR;               // rows per 1 KiB slot
  static constexpr int RS = NW * RPS;                    // rows between a wave's loads
  static constexpr int SPM = CH_PER / 64;                // 1 KiB slots per matrix
  static constexpr bool FAST = RS % 16 == 0 && BT % 16 == 0;
  static_assert((2 * CH_PER) % (NW * 64) == 0, "tile must split into whole wave loads");
  static_assert(CH_PER % 64 == 0, "a 1 KiB slot lies in one matrix");
  // The matrix of load i of wave w (wave-uniform; a compile-time constant
  // when a matrix holds whole rounds of the NW waves' loads).
  __device__ static inline int mat_of(int i, int w) {
    return SPM % NW == 0 ? i * NW / SPM : (i * NW + w) / SPM;
  }
  __host__ __device__ static constexpr int swz(int mat, int row) {
    return mat == 0 ? TL::swz(row) : TL1::swz(row);
  }
  // Byte offset of this lane's chunk of matrix `mat` from the first row of
  // the wave's first load (valid for every load of the wave into that
  // matrix when FAST).
  __device__ static inline unsigned lane_offset(int w, int lane, int mat = 0) {
    const int row = w * RPS + lane / TL::CPR;
    return (unsigned)((row * D + ((lane % TL::CPR) ^ swz(mat, row)) * TL::EPC) * sizeof(T));
  }
  __device__ static inline void issue(char* stage, const T* src0, const T* src1, int row0, int S,
                                      int w, int lane, unsigned lo, unsigned lo1) {
    if constexpr (FAST) {
      if (row0 + BT <= S) {
#pragma unroll
        for (int i = 0; i < NLOADS; ++i) {
          const int slot = i * NW + w;  // 1 KiB slot of the stage (wave-uniform)
          const int mat = mat_of(i, w);
          const T* base = (mat == 0 ? src0 : src1) + (size_t)(row0 + i * RS - mat * BT) * D;
          __builtin_amdgcn_global_load_lds(lane_addr(base, mat == 0 ? lo : lo1),
                                           stage + slot * 1024, 16, 0, 0);
        }
        return;
      }
      // The tile crosses S: the same lane pattern with the global row clamped.
      const int lrow = lo / (D * (int)sizeof(T));  // tile row of the lane in the first load
      const unsigned col = lo - lrow * D * (int)sizeof(T);
      const unsigned col1 = lo1 - lrow * D * (int)sizeof(T);
#pragma unroll
      for (int i = 0; i < NLOADS; ++i) {
        const int slot = i * NW + w;
        const int mat = mat_of(i, w);
        const int grow = min(row0 + i * RS - mat * BT + lrow, S - 1);
        const char* src = reinterpret_cast<const char*>(mat == 0 ? src0 : src1) +
                          (size_t)grow * D * sizeof(T) + (mat == 0 ? col : col1);
        __builtin_amdgcn_global_load_lds(src, stage + slot * 1024, 16, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NLOADS; ++i) {
      const int slot = i * NW + w;
      const int chunk = slot * 64 + lane;  // physical chunk in the stage
      const int mat = chunk / CH_PER;
      const int pc = chunk - mat * CH_PER;
      const int row = pc / TL::CPR;
      const int logical = (pc % TL::CPR) ^ swz(mat, row);
      const T* src = (mat == 0 ? src0 : src1) + (size_t)min(row0 + row, S - 1) * D + logical * TL::EPC;
      __builtin_amdgcn_global_load_lds(src, stage + slot * 1024, 16, 0, 0);
    }
  }

  // The same loads from matrices whose rows are ld0 and ld1 elements apart
  // (strided layouts).  A lane keeps only its row in the wave's first load
  // and its chunk's byte column (with FAST both hold for every load) and
  // forms each address from them; rows past S read row S-1.
  __device__ static inline void issue_ld(char* stage, const T* src0, int ld0, const T* src1,
                                         int ld1, int row0, int S, int w, int lane) {
    if constexpr (FAST) {
      const int lrow = w * RPS + lane / TL::CPR;
      const int lcolb0 = ((lane % TL::CPR) ^ swz(0, lrow)) * TL::EPC * (int)sizeof(T);
      const int lcolb1 = ((lane % TL::CPR) ^ swz(1, lrow)) * TL::EPC * (int)sizeof(T);
      const int lim = row0 + BT <= S ? 0x7fffffff : S - 1;
#pragma unroll
      for (int i = 0; i < NLOADS; ++i) {
        const int slot = i * NW + w;
        const int mat = mat_of(i, w);
        const size_t grow = (size_t)min(row0 + i * RS - mat * BT + lrow, lim);
        const char* src = mat == 0
                              ? reinterpret_cast<const char*>(src0) + grow * ld0 * sizeof(T)
                              : reinterpret_cast<const char*>(src1) + grow * ld1 * sizeof(T);
        __builtin_amdgcn_global_load_lds(src + (mat == 0 ? lcolb0 : lcolb1), stage + slot * 1024,
                                         16, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NLOADS; ++i) {
      const int slot = i * NW + w;
      const int chunk = slot * 64 + lane;
      const int mat = chunk / CH_PER;
      const int pc = chunk - mat * CH_PER;
      const int row = pc / TL::CPR;
      const int logical = (pc % TL::CPR) ^ swz(mat, row);
      const size_t r = (size_t)min(row0 + row, S - 1);
      const T* src = mat == 0 ? src0 + r * ld0 : src1 + r * ld1;
      __builtin_amdgcn_global_load_lds(src + logical * TL::EPC, stage + slot * 1024, 16, 0, 0);
    }
  }
};

// The direct loads of one swizzled tile of a single row-major matrix:
// rows row0 .. row0+BT-1 (rows past `rows` read row rows-1), columns
// col0 .. col0+COLS-1 of a matrix with row stride `ld` elements.  Same
// uniform-step fast path as StageLoader.
template <class E, int COLS, int BT, int NW>
struct TileLoader {
  using T = typename E::T;
  using TL = Tile<E, COLS>;
  static constexpr int CH = BT * TL::CPR;        // chunks in the tile
  static constexpr int NLOADS = CH / (NW * 64);  // per wave
  static constexpr int BYTES = BT * TL::ROWB;
  static constexpr int RPS = 64 / TL::CPR;
  static constexpr int RS = NW * RPS;
  static constexpr bool FAST = RS % 16 == 0;
  static_assert(CH % (NW * 64) == 0, "tile must split into whole wave loads");
  __device__ static inline unsigned lane_offset(size_t ld, int w, int lane) {
    const int row = w * RPS + lane / TL::CPR;
    return (unsigned)(((size_t)row * ld + ((lane % TL::CPR) ^ TL::swz(row)) * TL::EPC) * sizeof(T));
  }
  __device__ static inline void issue(char* dst, const T* src, size_t ld, int row0, int rows,
                                      int col0, int w, int lane, unsigned lo) {
    if constexpr (FAST) {
      if (row0 + BT <= rows) {
#pragma unroll
        for (int i = 0; i < NLOADS; ++i) {
          const int slot = i * NW + w;
          const T* base = src + (size_t)(row0 + i * RS) * ld + col0;
          __builtin_amdgcn_global_load_lds(lane_addr(base, lo), dst + slot * 1024, 16, 0, 0);
        }
        return;
      }
      // The tile crosses `rows`: the same lane pattern with the row clamped.
      const int lrow = w * RPS + lane / TL::CPR;
      const int lcol = ((lane % TL::CPR) ^ TL::swz(lrow)) * TL::EPC;
#pragma unroll
      for (int i = 0; i < NLOADS; ++i) {
        const int slot = i * NW + w;
        const T* g = src + (size_t)min(row0 + i * RS + lrow, rows - 1) * ld + col0 + lcol;
        __builtin_amdgcn_global_load_lds(g, dst + slot * 1024, 16, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NLOADS; ++i) {
      const int slot = i * NW + w;
      const int pc = slot * 64 + lane;
      const int row = pc / TL::CPR;
      const int logical = (pc % TL::CPR) ^ TL::swz(row);
      const T* g = src + (size_t)min(row0 + row, rows - 1) * ld + col0 + logical * TL::EPC;
      __builtin_amdgcn_global_load_lds(g, dst + slot * 1024, 16, 0, 0);
    }
  }
};

// Per-query statistics of a staged query tile for the dK+dV kernel: BT
// values of LSE*log2(e), then BT values of D, with one direct 4-byte load per
// wave (2*BT/NW active lanes).  Queries past S read query S-1.
template <int BT, int NW>
__device__ inline void issue_stats(float* dst, const float* lse2, const float* dlt, int q0, int S,
                                   int w, int lane) {
  constexpr int PER = 2 * BT / NW;
  static_assert(PER <= 64 && (2 * BT) % NW == 0, "stats split");
  if (lane < PER) {
    const int e = w * PER + lane;
    const float* src = e < BT ? lse2 + min(q0 + e, S - 1) : dlt + min(q0 + e - BT, S - 1);
    __builtin_amdgcn_global_load_lds(src, dst + w * PER, 4, 0, 0);
  }
}

// acc += A*B over the D/2 columns of this lane's half, where the A row is
// row `row` of a swizzled LDS tile and B is the register fragment.
template <class E, int D>
__device__ inline f32x16 dot_tile(const char* tile, int row, int h, const RowFrag<E, D>& b,
                                  f32x16 acc) {
  using TL = Tile<E, D>;
  constexpr int NCH = TL::CPR / 2;
  if constexpr (!is_bf16<E>() && mma_bf16<E>()) {
    // f32 tile, bf16 operands: two 16-byte chunks (8 d-values) per MFMA
#pragma unroll
    for (int cc = 0; cc < NCH / 2; ++cc) {
      bf16x8 a;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int chunk = h * NCH + 2 * cc + j;
        put_bf16x4(a, j, *reinterpret_cast<const f32x4*>(tile + row * TL::ROWB +
                                                          ((chunk ^ TL::swz(row)) << 4)));
      }
      acc = E::mma(a, b.f[cc], acc);
    }
    return acc;
  }
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    const int chunk = h * NCH + cc;
    const u32x4 x =
        *reinterpret_cast<const u32x4*>(tile + row * TL::ROWB + ((chunk ^ TL::swz(row)) << 4));
    if constexpr (is_bf16<E>()) {
      acc = E::mma(__builtin_bit_cast(bf16x8, x), b.f[cc], acc);
    } else {
      const f32x4 xf = __builtin_bit_cast(f32x4, x);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = E::mma(xf[e], b.f[4 * cc + e], acc);
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

template <>
struct RegOperand<EF32B> : RegOperand<EBF16> {};

// acc += product over the 32 logical rows row0 .. row0+31 of an LDS tile X:
//   REG_IS_A = true : acc[m][n] += sum_k R[m = this lane's row][k] * X[k][col0 + n]
//   REG_IS_A = false: acc[m][n] += sum_k X[k][col0 + m] * R[k][n = this lane's column]
// R's k-slots are the lane's rho rows.  The X operand (read_kslot_operand)
// needs, per lane, the k-slot rows of one column: f32 reads one element per
// MFMA; bf16 reads 8 consecutive rows of one column with two transposed LDS
// reads
// (ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives
// element e of the 8-byte row read of lane 4e + i/4, position i%4; so lanes
// that read rows kbase + r/4, columns colbase + 4(r%4) .. +3 hand lane i
// rows kbase .. kbase+3 of column colbase + i).
// One transposed LDS read (ds_read_b64_tr_b16).  The pointer goes through a
// __restrict__ parameter of an inlined function so that the read carries
// alias-scope metadata: without any, the compiler's wait insertion assumes
// it may read LDS that a direct global->LDS load still in flight writes,
// and puts a vmcnt(0) before it, which also waits for every tile the ring
// is prefetching.  The tile it reads has been waited for explicitly.
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __attribute__((always_inline)) inline s16x4 ds_read_tr(
    const lds_s16x4* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4*>(p));
}

template <class E, int COLS, bool KS = false>
__device__ inline void read_kslot_operand(RegOperand<E>& X, const char* tile, int row0, int col0,
                                          int lane) {
  // X in the k-slot layout of RegOperand: for this lane's column col0 + n,
  // the k-slot rows row0 + rho(w, h) (f32) or row0 + 16u + 8h + t (bf16).
  using TL = Tile<E, COLS, KS>;
  const int h = lane >> 5, n = lane & 31;
  if constexpr (KS && !is_bf16<E>()) {
    // k-slot layout (row0 and col0 multiples of 16 and 32): every k-slot row
    // of the lane is row0 + 8h plus a constant, all with the lane's chunk
    // XOR 8h, so one base address serves all 16 reads.
    static_assert(TL::EPC == 4, "f32 tile");
    const int sw = TL::CPR >= 16 ? 8 * h : 0;
    const char* p = tile + (row0 + 8 * h) * TL::ROWB + ((((col0 >> 2) ^ sw) + (n >> 2)) << 4) +
                    (n & 3) * 4;
    if constexpr (mma_bf16<E>()) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          X.v[u][t] = (__bf16)*reinterpret_cast<const float*>(p + (16 * u + t) * TL::ROWB);
    } else {
#pragma unroll
      for (int w = 0; w < 16; ++w)
        X.v[w] = *reinterpret_cast<const float*>(p + (rho(w, 0)) * TL::ROWB);
    }
  } else if constexpr (is_bf16<E>()) {
    const int g = lane >> 4, r = lane & 15;
    const int col = col0 + 16 * (g & 1) + 4 * (r & 3);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s16x4 part[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = row0 + 16 * u + 8 * h + 4 * j + (r >> 2);
        part[j] = ds_read_tr((const lds_s16x4*)(tile + TL::off(row, col)));
      }
      const s16x8 all = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
      X.v[u] = __builtin_bit_cast(bf16x8, all);
    }
  } else if constexpr (mma_bf16<E>()) {
    // f32 tile, bf16 operands: the 8 k-slot rows of column col0 + n, one
    // element each, rounded
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        X.v[u][t] = (__bf16)*reinterpret_cast<const float*>(
            tile + TL::off(row0 + 16 * u + 8 * h + t, col0 + n));
  } else {
#pragma unroll
    for (int w = 0; w < 16; ++w)
      X.v[w] = *reinterpret_cast<const float*>(tile + TL::off(row0 + rho(w, h), col0 + n));
  }
}

template <class E, int D, bool REG_IS_A, bool KS = false>
__device__ inline f32x16 second_tile(const RegOperand<E>& R, const char* tile, int row0, int col0,
                                     int lane, f32x16 acc) {
  RegOperand<E> X;
  read_kslot_operand<E, D, KS>(X, tile, row0, col0, lane);
  constexpr int NU = 16 / E::KL;
#pragma unroll
  for (int u = 0; u < NU; ++u) acc = REG_IS_A ? E::mma(R.v[u], X.v[u], acc) : E::mma(X.v[u], R.v[u], acc);
  return acc;
}

// ------------------------------------------------------------------ stores
// Store the 4 consecutive values of a lane's output block to p[0..3]
// (converted to T).
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
