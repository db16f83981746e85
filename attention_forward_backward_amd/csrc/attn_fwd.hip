// attn_fwd.hip -- tiled attention forward for gfx950.
//
// The forward of the attention node ("Meganeura: Portable GPU Training and
// Inference through Vulkan and Metal", arXiv 2608.01563, Section 3.3, tiled
// attention forward kernel): O = softmax(scale * Q K^T, masked) V and the row
// LSE, with the softmax taken online over key tiles so that no S x S matrix
// exists.
//
// Work split (persistent): an item is (query tile of BR = 32*RB rows,
// batch*head), numbered in order of decreasing causal work; the launch puts
// about one workgroup on every resident slot and each walks the items a
// static schedule gives it (sched_item: balanced over the CUs, each head's
// items on one XCD).  Each 32-query block of an item is owned by
// NSPLIT waves that split the key range between them (block kb of every
// staged tile goes to wave kb % NSPLIT); each keeps its own running max, sum
// and O, and the NSPLIT partial results are merged through LDS when the item
// ends.
//
// K and V stream through an NST-stage ring of LDS tiles (32*NSPLIT*KPW keys
// each) filled by direct global->LDS loads issued NST-1 tiles ahead, with one
// workgroup barrier per tile.  The stream runs across item boundaries, so the
// next item's first keys load while the current item finishes; the next
// item's Q tile loads into its own LDS buffer one item ahead, and each wave
// reads its Q rows into registers when its item starts.
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

template <class E, int D, int NW, int NSPLIT, int KPW, int NST, bool CAUSAL, bool CROSS,
          bool STR, bool KS, bool ROPE>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, typename E::T* __restrict__ O,
    float* __restrict__ LSE, int Sq, int Sk_, float c, int BH, int H,
    const int* __restrict__ kvlen, int nitems, const Sched sched, const Layout lay, int nch,
    int kc, float* __restrict__ part, int Sp, const RopeTab rope) {
  // LSE may be null (an inference-only forward stores no LSE).  Queries Sq,
  // keys Sk (one length in self-attention, CROSS = false); per batch*head the
  // first L keys exist and key j is visible from query i iff j < L and, when
  // causal, j <= i + off (head_keys).  STR: Q, K, V, O are laid out by `lay`
  // (else [B, H, S, D] row-major).
  // KS (key split, self-attention only): the key tiles a query tile sees are
  // cut into at most nch chunks of at most kc tiles (fwd_key_split); item
  // it = (query tile, chunk) * BH + head, and an item of a query tile with
  // more than one chunk stores its unnormalised O (f32) and its (m, l) in
  // `part` -- [nch][BH][Sp][D] then [nch][BH][Sp][2] -- for fwd_merge_kernel.
  // ROPE (self-attention, STR; query and key i at table row rope.pos + i):
  // Q and K tiles are turned by RoPE in LDS (TileRope) once they arrive,
  // each wave turning the rows it loaded, each K tile by every item that
  // reads it; the turned rows are stored once, Q by its item and key tile t
  // by the item of query tile t (same tile height), to rope.out and
  // rope.kout for the backward.
  using T = typename E::T;
  using TL = Tile<E, D>;
  constexpr int RB = NW / NSPLIT;        // 32-query blocks per item
  constexpr int BR = 32 * RB;            // queries per item
  constexpr int BK = 32 * NSPLIT * KPW;  // keys per staged tile
  constexpr int NDB = D / 32;
  using LD = StageLoader<E, D, BK, NW, true>;  // V in the k-slot layout (read by PV only)
  constexpr int STAGE = LD::BYTES;
  constexpr int TILEB = BK * TL::ROWB;  // one matrix tile; V follows K in a stage
  using QL = TileLoader<E, D, BR, NW>;
  static_assert(NW % NSPLIT == 0 && NST >= 2 && NST <= 4, "launch shape");
  // (ROPE: a tile's angles are fetched on the step before it is consumed,
  // the one that issues it; the diagonal store needs square tiles)
  static_assert(!ROPE || (NST == 2 && BK == BR && !KS), "RoPE launch shape");
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE + QL::BYTES];
  char* const qtile = smem + NST * STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar
  const int qb = w / NSPLIT, sp = w % NSPLIT;
  const int g = blockIdx.x, G = gridDim.x;
  const int Sk = CROSS ? Sk_ : Sq;
  const int nqt = (Sq + BR - 1) / BR;
  const int ldk = row_ld<STR, D>(lay.k), ldv = row_ld<STR, D>(lay.v);
  const int ldq = row_ld<STR, D>(lay.q), ldo = row_ld<STR, D>(lay.o);
  const unsigned lo = STR ? 0u : LD::lane_offset(w, lane);
  const unsigned lo1 = STR ? 0u : LD::lane_offset(w, lane, 1);
  const unsigned qlo = QL::lane_offset(ldq, w, lane);
  auto item_qt = [&](int it) { return nqt - 1 - (KS ? it / BH / nch : it / BH); };
  // Key tiles of item it's query tile: those holding a key visible from one
  // of its queries; an item none of whose queries sees a key still takes one
  // tile (processed fully masked), so that its zero rows are stored.
  auto qt_nkt = [&](int it) {
    int L, off;
    head_keys<CROSS>(kvlen, it % BH, H, Sq, Sk, L, off);
    const int kend = CAUSAL ? min(L, item_qt(it) * BR + BR + off) : L;
    const int n = (kend + BK - 1) / BK;
    return CROSS ? max(n, 1) : n;
  };
  // With KS, the chunk of item it: its first key tile kb0, its tile count
  // and whether its query tile has more than one chunk (partial results).
  auto item_chunk = [&](int it, int& kb0, int& ntl, bool& partial) {
    const int full = qt_nkt(it);
    if constexpr (KS) {
      const int nq = (full + kc - 1) / kc;
      const int csz = (full + nq - 1) / nq;
      kb0 = (it / BH % nch) * csz;
      ntl = min(csz, full - kb0);
      partial = nq > 1;
    } else {
      kb0 = 0;
      ntl = full;
      partial = false;
    }
  };
  auto item_nkt = [&](int it) {
    int kb0, ntl;
    bool partial;
    item_chunk(it, kb0, ntl, partial);
    return ntl;
  };
  // Rows a key tile may read: past them the loads read the last valid row
  // (finite, and masked), so padded rows are never read.
  auto key_rows = [&](int it) {
    int L, off;
    head_keys<CROSS>(kvlen, it % BH, H, Sq, Sk, L, off);
    return CROSS ? max(L, 1) : Sk;
  };
  if (sched_item(sched, 0, g, G, BH) >= nitems) return;  // (the launch never makes more workgroups than items)

  // Vector-memory instructions this wave has issued (loads, and the stores
  // counted by the rule below), and the count just after the loads of each
  // tile in the ring and of the prefetched Q rows.  Waiting until at most
  // vm - mark operations are pending completes everything up to that mark
  // (vmcnt counts loads and stores, and they retire in issue order);
  // counting fewer operations than issued (the stores of partial waves, and
  // with ROPE the angle loads and turned-row stores) only makes a wait
  // stricter.
  int vm = 0, qmark = 0;
  RingMarks<NST> mk;

  // Loader cursor: tile lkt (of lnkt, from key tile lkb) of item lit is the
  // next one to issue.
  int lr = 0, lit = sched_item(sched, 0, g, G, BH), lkt = 0, lnkt, lkb;
  bool lpart;
  item_chunk(lit, lkb, lnkt, lpart);
  int lrows = key_rows(lit);
  size_t kbase = head_off<STR, D>(lay.k, lit % BH, H, Sk);
  size_t vbase = head_off<STR, D>(lay.v, lit % BH, H, Sk);
  // While tiles remain, the tile issued at stream position pos goes to ring
  // slot (pos + NST - 1) % NST, a constant of the unrolled step.
  auto issue_next = [&](const int slot) __attribute__((always_inline)) {
    if (lit >= nitems) return;
    if constexpr (STR)
      LD::issue_ld(smem + slot * STAGE, K + kbase, ldk, V + vbase, ldv, (lkb + lkt) * BK, lrows,
                   w, lane);
    else
      LD::issue(smem + slot * STAGE, K + kbase, V + vbase, (lkb + lkt) * BK, lrows, w, lane, lo,
                lo1);
    vm += LD::NLOADS;
    mk.set(slot, vm);
    if (++lkt == lnkt) {
      lit = sched_item(sched, ++lr, g, G, BH);
      lkt = 0;
      if (lit < nitems) {
        item_chunk(lit, lkb, lnkt, lpart);
        lrows = key_rows(lit);
        kbase = head_off<STR, D>(lay.k, lit % BH, H, Sk);
        vbase = head_off<STR, D>(lay.v, lit % BH, H, Sk);
      }
    }
  };
  // The Q tile of item it (rows past Sq read row Sq-1) into its LDS buffer.
  auto load_q = [&](int it) __attribute__((always_inline)) {
    QL::issue(qtile, Q + head_off<STR, D>(lay.q, it % BH, H, Sq), ldq, item_qt(it) * BR, Sq, 0, w,
              lane, qlo);
    vm += QL::NLOADS;
    qmark = vm;
  };
  RowFrag<E, D> qf;

  // Consumer state: item cit (round cr), its tile kt of nkt.  (Taken before
  // the first issues, which may move the loader cursor past the first item.)
  int cr = 0, cit = lit, kt = 0, nkt = lnkt, ckb = lkb;
  bool cpart = lpart;
  load_q(lit);
  // (ROPE) angles of this lane's share of the next Q tile and of the K tile
  // the loader issues next
  TileRope<E, D, BR, NW> qrope;
  TileRope<E, D, BK, NW> krope;
  if constexpr (ROPE) {
    const int qrow0 = item_qt(lit) * BR;
    qrope.load(rope.cos, rope.sin, rope.pos + qrow0, Sq - qrow0, w, lane);
    const int krow0 = (lkb + lkt) * BK;
    krope.load(rope.cos, rope.sin, rope.pos + krow0, Sk - krow0, w, lane);
  }
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) issue_next(s);
  int bh = cit % BH, q0 = item_qt(cit) * BR + qb * 32;
  int cL, coff;  // the current item's valid keys and causal offset
  head_keys<CROSS>(kvlen, bh, H, Sq, Sk, cL, coff);
  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
  float m = -INFINITY;  // exponent reference (log2 domain), lags the row max by < 2^8
  float l = 0.f;        // this half's running sum of exp2(c*score - m)

  // Merge the NSPLIT partial (m, l, O) of each query block through the LDS
  // stage at `buf` (no load targets it), in passes of as many d-blocks as
  // the stage holds: the first pass also carries m and l, from which every
  // partial's factor exp2(m_p - max m) is formed once.
  auto merge = [&](char* buf, bool active) __attribute__((always_inline)) {
    if constexpr (NSPLIT > 1) {
      // Values go through LDS four at a time (group q of lane l at float
      // (q * 64 + l) * 4: 1 KiB per wave access, no bank conflicts); the
      // first pass leads with one group (m, l, -, -).
      constexpr int HELP = RB * (NSPLIT - 1);
      constexpr int PERDB = HELP * 16 * 64 * 4;
      constexpr int MLB = HELP * 4 * 64 * 4;
      constexpr int DB0 = (STAGE - MLB) / PERDB < NDB ? (STAGE - MLB) / PERDB : NDB;
      constexpr int DBN = STAGE / PERDB < NDB ? STAGE / PERDB : NDB;
      static_assert(DBN >= 1, "a d-block of partials fits one stage");
      constexpr int NPASS = 1 + (NDB - DB0 + DBN - 1) / DBN;
      f32x4* cb = reinterpret_cast<f32x4*>(buf);
      float a0 = 1.f, ap[NSPLIT - 1];
#pragma unroll
      for (int pass = 0; pass < NPASS; ++pass) {
        const int dlo = pass == 0 ? 0 : DB0 + (pass - 1) * DBN;
        const int dhi = pass == 0 ? DB0 : (dlo + DBN < NDB ? dlo + DBN : NDB);
        const int ov = pass == 0 ? 1 : 0;          // leading (m, l) group
        const int ng = ov + 4 * (dhi - dlo);       // groups per lane per helper
        lds_barrier();  // every wave is done reading the stage (or the previous pass)
        if (sp != 0 && active) {
          f32x4* dst = cb + ((qb * (NSPLIT - 1) + sp - 1) * ng) * 64 + lane;
          if (pass == 0) dst[0] = f32x4{m, l, 0.f, 0.f};
#pragma unroll
          for (int db = dlo; db < dhi; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              dst[(ov + (db - dlo) * 4 + j) * 64] =
                  f32x4{oacc[db][4 * j], oacc[db][4 * j + 1], oacc[db][4 * j + 2], oacc[db][4 * j + 3]};
        }
        lds_barrier();
        if (sp == 0 && active) {
          if (pass == 0) {
            float mp[NSPLIT - 1], lp[NSPLIT - 1];
            // In self-attention split 0 always sees key 0, so mx is finite;
            // with CROSS a row may have seen no key in any split (mx = -inf:
            // every factor is then 0 and the row stays empty).
            float mx = m;
#pragma unroll
            for (int p = 0; p < NSPLIT - 1; ++p) {
              const f32x4 ml = cb[((qb * (NSPLIT - 1) + p) * ng) * 64 + lane];
              mp[p] = ml[0];
              lp[p] = ml[1];
              mx = fmaxf(mx, mp[p]);
            }
            const float mxs = (CROSS && mx == -INFINITY) ? 0.f : mx;
            a0 = fast_exp2(m - mxs);
            l *= a0;
#pragma unroll
            for (int p = 0; p < NSPLIT - 1; ++p) {
              ap[p] = fast_exp2(mp[p] - mxs);  // 0 for a split that saw no key
              l += lp[p] * ap[p];
            }
            m = mx;
          }
#pragma unroll
          for (int db = dlo; db < dhi; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              f32x4 o = f32x4{oacc[db][4 * j], oacc[db][4 * j + 1], oacc[db][4 * j + 2],
                              oacc[db][4 * j + 3]} * a0;
#pragma unroll
              for (int p = 0; p < NSPLIT - 1; ++p)
                o += cb[((qb * (NSPLIT - 1) + p) * ng + ov + (db - dlo) * 4 + j) * 64 + lane] * ap[p];
#pragma unroll
              for (int e = 0; e < 4; ++e) oacc[db][4 * j + e] = o[e];
            }
        }
      }
    }
  };

  // One staged tile of keys at stream position pos (ring slot sc when
  // constant).  When the stages' LDS addresses fit 16-bit offsets, the loop
  // is unrolled by NST with the slot constant.
  auto step = [&](const int pos, auto sc) __attribute__((always_inline)) {
    const int si = sc;  // pos % NST
    int mark = mk.get(si);
    if (kt == 0) mark = max(mark, qmark);  // the item's Q rows too
    wait_vmem_dyn(vm - mark);
    if constexpr (ROPE) {
      // This wave's own rows of the tile (and on an item's first tile of its
      // Q tile) are in LDS: the wave turns them in place before the barrier,
      // storing the turned Q rows, and the turned K rows on the item's
      // diagonal tile.  The angles were fetched on the previous step; no
      // load the ring prefetches is in flight here, so the compiler's wait
      // for them stalls on nothing.
      krope.ready();
      if (kt == 0) {
        qrope.ready();
        const int qrow0 = item_qt(cit) * BR;
        qrope.apply(qtile, static_cast<T*>(rope.out) + ((size_t)bh * Sq + qrow0) * D,
                    Sq - qrow0, w, lane);
      }
      const int krow0 = (ckb + kt) * BK;
      T* kout = item_qt(cit) == ckb + kt
                    ? static_cast<T*>(rope.kout) + ((size_t)bh * Sk + krow0) * D
                    : nullptr;
      krope.apply(smem + si * STAGE, kout, Sk - krow0, w, lane);
    }
    lds_barrier();  // tile pos (and on an item's first tile its Q) is in LDS;
                    // every wave is done with tile pos-1
    if constexpr (ROPE) {  // the angles of the tile issued below
      if (lit < nitems) {
        const int r0 = (lkb + lkt) * BK;
        krope.load(rope.cos, rope.sin, rope.pos + r0, Sk - r0, w, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    issue_next((si + NST - 1) % NST);
    if (kt == 0) {
      // This wave's Q rows, then the next item's Q tile (if any) once every
      // wave has read its rows.
      load_row_frag_lds<E, D>(qf, qtile, qb * 32 + n, h, true);
      const int nit = sched_item(sched, cr + 1, g, G, BH);
      if (nit < nitems) {
        lds_barrier();
        load_q(nit);
        if constexpr (ROPE) {  // the angles of that tile
          const int qrow0 = item_qt(nit) * BR;
          qrope.load(rope.cos, rope.sin, rope.pos + qrow0, Sq - qrow0, w, lane);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the counts above assume this issue order
    const int qi = q0 + n;
    const bool wave_active = q0 < Sq;
    if (wave_active) {
      const char* Kt = smem + si * STAGE;
      const char* Vt = Kt + TILEB;
      // This wave's 32-key blocks of the tile.  A block is skipped when no
      // key in it is visible from any of the wave's queries, and masked only
      // when some but not all of it is (the causal diagonal, the ragged end,
      // padded keys).  In self-attention every processed block has at least
      // one visible key for every query (block starts are multiples of 32),
      // so row maxima are finite; with CROSS a row may see none in a block,
      // or at all (handled where noted).
#pragma unroll
      for (int j = 0; j < KPW; ++j) {
        const int kb = sp + NSPLIT * j;
        const int kk0 = (ckb + kt) * BK + kb * 32;
        if (!(kk0 < cL && (!CAUSAL || kk0 <= q0 + 31 + coff))) continue;  // wave-uniform
        // The products run at raised wave priority, so that while one wave
        // of a SIMD works through its softmax the other's MFMAs issue first
        // (f32: forward 40.2 -> 39.3 us at B8 H12 S512 D64; bf16 unchanged).
        __builtin_amdgcn_s_setprio(1);
        f32x16 sacc = dot_tile<E, D>(Kt, kb * 32 + pi32(n), h, qf, zero16());
        __builtin_amdgcn_s_setprio(0);
        if (kk0 + 32 > cL || (CAUSAL && kk0 + 31 > q0 + coff)) {
          // key(r) = kk0 + 8h + (16*(r/8) + r%8); visible iff key < L and key <= qi + off
          const int lim = min(cL - 1, CAUSAL ? qi + coff : cL - 1) - kk0 - 8 * h;
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
          // (CROSS: a row with no visible key yet keeps m = mnew = -inf)
          const float alpha = (CROSS && mnew == -INFINITY) ? 1.f : fast_exp2(m - mnew);
          m = mnew;
          l *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        }
        // exponent reference: m, or 0 for a row with no visible key yet
        // (its scores are all -inf, so every p is 0)
        const float mref = (CROSS && m == -INFINITY) ? 0.f : m;
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sacc[r], c, -mref));
          sacc[r] = p;
          rs += p;
        }
        l += rs;
        RegOperand<E> P;
        P.set(sacc);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = second_tile<E, D, false, true>(P, Vt, kb * 32, db * 32, lane, oacc[db]);
        __builtin_amdgcn_s_setprio(0);
      }
    }
    if (++kt < nkt) return;

    // The item is done: merge the splits through the stage just consumed
    // (the tiles in flight are the next NST-1), then store O and the LSE.
    l += xhalf(l);
    merge(smem + si * STAGE, wave_active);
    if (KS && cpart && sp == 0 && wave_active) {
      // one chunk of a split query tile: O unnormalised (relative to m), and
      // (m, l), for the merge kernel
      if (qi < Sq) {
        const size_t row = ((size_t)(cit / BH % nch) * BH + bh) * Sp + qi;
        float* prow = part + row * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            store4<float>(prow + db * 32 + 8 * j + 4 * h, oacc[db][4 * j], oacc[db][4 * j + 1],
                          oacc[db][4 * j + 2], oacc[db][4 * j + 3]);
        if (h == 0)
          *reinterpret_cast<float2*>(part + (size_t)nch * BH * Sp * D + row * 2) =
              make_float2(m, l);
      }
      if (q0 + 31 < Sq) vm += 4 * NDB;
    } else if (sp == 0 && wave_active) {
      // (CROSS: a row with no visible key has l = 0: O = 0, LSE = -inf)
      const float inv = (CROSS && !(l > 0.f)) ? 0.f : 1.f / l;
      if (qi < Sq) {
        T* orow;
        if constexpr (STR)
          orow = O + head_off<STR, D>(lay.o, bh, H, Sq) + (size_t)qi * ldo;
        else
          orow = O + ((size_t)bh * Sq + qi) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = db * 32 + 8 * j + 4 * h;
            store4<T>(orow + d, oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv,
                      oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
          }
        if (h == 0 && LSE != nullptr) LSE[(size_t)bh * Sq + qi] = (m + __log2f(l)) * kLn2;
      }
      // Only the O stores of a wave whose every lane stores are counted.
      if (q0 + 31 < Sq) vm += 4 * NDB;
    }
    // Next item.
    cit = sched_item(sched, ++cr, g, G, BH);
    kt = 0;
    if (cit < nitems) {
      item_chunk(cit, ckb, nkt, cpart);
      bh = cit % BH;
      q0 = item_qt(cit) * BR + qb * 32;
      head_keys<CROSS>(kvlen, bh, H, Sq, Sk, cL, coff);
    }
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
    m = -INFINITY;
    l = 0.f;
  };

  // Tiles this workgroup consumes: the key tiles of all its items.
  int ntiles = 0;
  for (int r = 0;; ++r) {
    const int it = sched_item(sched, r, g, G, BH);
    if (it >= nitems) break;
    ntiles += item_nkt(it);
  }
  if constexpr (NST * STAGE <= 65536) {
    for_stages<NST>(ntiles, step);
  } else {
    for (int pos = 0; pos < ntiles; ++pos) step(pos, pos % NST);
  }
}

// The chunks of split query tiles merged in chunk order (deterministic):
// with m* the largest chunk reference, O = sum_c 2^(m_c - m*) O_c / l and
// l = sum_c 2^(m_c - m*) l_c, LSE = (m* + log2 l) ln 2.  One thread per four
// columns of a query row; rows of query tiles with one chunk were written by
// the forward kernel and are skipped.
template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const float* __restrict__ part,
                                                        T* __restrict__ O, float* __restrict__ LSE,
                                                        int BH, int Sq, int Sp, int nch, int kc,
                                                        int BR, int BK) {
  constexpr int NG = D / 4;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = i / NG;
  const int gcol = (int)(i % NG) * 4;
  if (row >= (long long)BH * Sq) return;
  const int bh = (int)(row / Sq), q = (int)(row % Sq);
  const int qt = q / BR;
  const int kend = CAUSAL ? min(Sq, qt * BR + BR) : Sq;
  const int full = (kend + BK - 1) / BK;
  const int nq = (full + kc - 1) / kc;
  if (nq <= 1) return;
  const float2* ml = reinterpret_cast<const float2*>(part + (size_t)nch * BH * Sp * D);
  float mx = -INFINITY;
  for (int ch = 0; ch < nq; ++ch) mx = fmaxf(mx, ml[((size_t)ch * BH + bh) * Sp + q].x);
  float l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int ch = 0; ch < nq; ++ch) {
    const size_t r = ((size_t)ch * BH + bh) * Sp + q;
    const float2 mlc = ml[r];
    const float wgt = fast_exp2(mlc.x - mx);
    l += mlc.y * wgt;
    const f32x4 oc = *reinterpret_cast<const f32x4*>(part + r * D + gcol);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] += oc[e] * wgt;
  }
  const float inv = 1.f / l;
  store4<T>(O + (size_t)row * D + gcol, o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
  if (gcol == 0 && LSE != nullptr) LSE[row] = (mx + __log2f(l)) * kLn2;
}

template <class E, int D, bool CAUSAL, bool CROSS, bool STR, bool KS, bool ROPE = false>
static hipError_t launch(const FwdArgs& a) {
  constexpr LShape SH = fwd_shape(is_bf16<E>(), D);
  constexpr int NW = SH.nw, NSPLIT = SH.nsplit, KPW = SH.kpw, NST = SH.nst;
  using T = typename E::T;
  constexpr auto kern = fwd_kernel<E, D, NW, NSPLIT, KPW, NST, CAUSAL, CROSS, STR, KS, ROPE>;
  constexpr int BR = 32 * (NW / NSPLIT);
  constexpr int BK = 32 * NSPLIT * KPW;
  static_assert(BR == fwd_query_tile(is_bf16<E>(), D) && BK == fwd_key_tile(is_bf16<E>(), D),
                "tiles of the key-split choice");
  const int nqt = (a.Sq + BR - 1) / BR;
  // Key split (self-attention with a workspace): chunks of at most kc key
  // tiles, nch chunk classes per query tile (class = query tile * nch + chunk).
  int nch = 1, kc = 1 << 30;
  if (KS) fwd_key_split(is_bf16<E>(), a.BH, a.Sq, D, CAUSAL, nch, kc);
  const int nitems = a.BH * nqt * nch;
  const int grid = std::min(nitems, resident_workgroups<kern>(NW * 64));
  // work of each class: its key tiles (with every key valid: the per-batch
  // counts live on the device); classes of chunks a query tile does not
  // have get no work and no items
  std::vector<int> works(nqt * nch);
  for (int c = 0; c < nqt * nch; ++c) {
    const int qt = nqt - 1 - c / nch, ch = c % nch;
    const int kend = CAUSAL ? std::min(a.Sk, qt * BR + BR + a.Sk - a.Sq) : a.Sk;
    const int full = std::max((kend + BK - 1) / BK, 1);
    const int nq = (full + kc - 1) / kc, csz = (full + nq - 1) / nq;
    const int ntl = ch < nq ? std::min(csz, full - ch * csz) : 0;
    works[c] = ntl > 0 ? 4 * ntl + (is_bf16<E>() ? ATTN_FWD_ITEM_COST_BF16 : ATTN_FWD_ITEM_COST_F32)
                       : 0;
  }
  const Sched sched = make_sched(grid, a.BH, works);
  // The chunk items exist only in a schedule table; when none can be built
  // for this launch (grid or table size), run the forward unsplit.
  if constexpr (KS) {
    if (sched.M == 0) return launch<E, D, CAUSAL, CROSS, STR, false>(a);
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), 0, a.stream, (const T*)a.q, (const T*)a.k,
                     (const T*)a.v, (T*)a.o, a.lse, a.Sq, a.Sk, a.scale * kLog2e, a.BH, a.H,
                     a.kvlen, nitems, sched, a.layout != nullptr ? *a.layout : Layout{}, nch, kc,
                     a.part, nqt * BR, a.rope);
  if (KS) {
    const long long threads = (long long)a.BH * a.Sq * (D / 4);
    hipLaunchKernelGGL((fwd_merge_kernel<T, D, CAUSAL>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, a.stream, a.part, (T*)a.o, a.lse, a.BH, a.Sq, nqt * BR, nch,
                       kc, BR, BK);
  }
  return hipGetLastError();
}

// (strided layouts run the cross-attention instantiation, which handles any
// lengths)
template <class E, int D>
static hipError_t launch_c(const FwdArgs& a) {
  if (a.rope.cos != nullptr)  // (strided self-attention)
    return a.causal ? launch<E, D, true, true, true, false, true>(a)
                    : launch<E, D, false, true, true, false, true>(a);
  if (a.layout != nullptr)
    return a.causal ? launch<E, D, true, true, true, false>(a)
                    : launch<E, D, false, true, true, false>(a);
  if (a.cross)
    return a.causal ? launch<E, D, true, true, false, false>(a)
                    : launch<E, D, false, true, false, false>(a);
  if (a.part != nullptr)  // (the caller checked that the shape is split)
    return a.causal ? launch<E, D, true, false, false, true>(a)
                    : launch<E, D, false, false, false, true>(a);
  return a.causal ? launch<E, D, true, false, false, false>(a)
                  : launch<E, D, false, false, false, false>(a);
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
  if (a.rope.cos == nullptr && a.Sq <= (a.bf16 ? ATTN_FWD_SMALL_MAXQ_BF16 : ATTN_FWD_SMALL_MAXQ_F32))
    return launch_fwd_small(a);
  if (a.bf16) return launch_d<EBF16>(a);
  return a.bf16_operands ? launch_d<EF32B>(a) : launch_d<EF32>(a);
}

}  // namespace attn
