// attn_bwd_dkdv.hip -- fused dK+dV backward kernel for gfx950.
//
// The pages ("Meganeura: Portable GPU Training and Inference through Vulkan
// and Metal", arXiv 2608.01563) make one fused dK+dV kernel the invariant
// for the attention derivative (Section 8; kernel list in Section 3.3,
// FlashGradKV in the Section 7.3 profile).  For each key row j:
//   P_ij  = exp(scale * Q_i.K_j - LSE_i)
//   dV_j  = sum_i P_ij dO_i
//   dK_j  = scale * sum_i P_ij (dO_i.V_j - D_i) Q_i
// with D_i and LSE_i*log2(e) read from the workspace (the prep kernel).  When
// the workspace holds room for it, the kernel also stores dS^T (the values it
// feeds its own dK product), from which dQ = scale * dS K is a plain GEMM.
//
// Work split (persistent): an item is (key tile of BKV = 32*RB rows,
// batch*head), numbered in order of decreasing causal work; the launch puts
// about one workgroup on every resident slot and each walks its items in the
// static schedule (sched_item: balanced over the CUs, each head's items on
// one XCD).  Each 32-key block of an item is owned by
// NSPLIT waves that keep its K and V rows in registers, split the query
// blocks between them, accumulate dK and dV in registers and sum their
// partials through LDS when the item ends.
//
// Tiles stream through an NST-stage ring of LDS tiles filled by direct
// global->LDS loads issued NST-1 tiles ahead.  The stream runs across item
// boundaries: per item, a header tile (the item's K and V rows, read into
// registers from LDS) and then its query tiles (Q, dO, and the queries' LSE
// and D), so the next item's rows and first queries load while the current
// item finishes.  Per 32-query block a wave forms S = Q K^T and dP = dO V^T
// (queries x keys; each lane holds one key), then P and dS are the register
// B operands of dV^T (d x keys) += dO^T P and dK^T += Q^T dS, with dO and Q
// read back from LDS: each lane accumulates the d values of its own key, so
// dK and dV leave in 16-byte (f32) or 8-byte (bf16) row stores.
#include "attn_device.hpp"
#include "attn_launch.hpp"

namespace attn {

template <class E, int D, int NW, int NSPLIT, int KPW, int NST, bool CAUSAL, bool WDS, bool CROSS,
          bool QSPLIT, bool STR, bool ROPE, bool DF = false>
__global__ __launch_bounds__(NW * 64, !is_bf16<E>() && D <= 64 ? ATTN_DKDV_MINW_F32 : 1) void bwd_dkdv_kernel(
    const typename E::T* __restrict__ Q, const typename E::T* __restrict__ K,
    const typename E::T* __restrict__ V, const typename E::T* __restrict__ dO,
    const float* __restrict__ Dws, typename E::T* __restrict__ dK, typename E::T* __restrict__ dV,
    typename E::T* __restrict__ dSout, int SPq, int SPk, int Sq, int Sk_, int Lws, float c,
    float scale, int BH, int H, const int* __restrict__ kvlen, float* __restrict__ part, int nqs_,
    int qpc_, int nitems, const Sched sched, const Layout lay, const RopeTab rope,
    const typename E::T* __restrict__ Oin, const float* __restrict__ LSEin) {
  // Queries Sq, keys Sk (one length in self-attention, CROSS = false); per
  // batch*head the first L keys exist and key j is visible from query i iff
  // j < L and, when causal, j <= i + off (head_keys).  Lws: offset of the
  // LSE*log2(e) vector in the workspace (B*H*Sq).
  // Query chunks: item (class c, head bh) is key tile c / nqs over query
  // tiles [(c % nqs) * qpc, (c % nqs + 1) * qpc); with nqs > 1 it stores
  // its dK (scaled) and dV sums as float32 partials, part[qc][bh][Sk][D]
  // then part[nqs + qc][bh][Sk][D], which a second kernel adds up.  Without
  // QSPLIT there is one chunk of every query tile and dK, dV are stored.
  // STR: Q, K, V, dO, dK, dV are laid out by `lay` (else [B, H, S, D]
  // row-major; the workspace is always packed).
  // ROPE (STR): Q and K hold RoPE-turned rows; dK leaves turned back by the
  // transposed rotation of key j (table row rope.pos + j) -- here, or with
  // QSPLIT in the reduce kernel.
  // DF (bf16, dS stored, plain layout): no prep pass ran; D and LSE*log2(e)
  // of each query tile are formed here from O (Oin, whose rows follow Q and
  // dO in a stage), dO and the LSE (LSEin): the statistics of a stage hold
  // the raw LSE (loaded twice, to keep the load count), then LSE*log2(e) and
  // D written by the waves.
  using T = typename E::T;
  using TL = Tile<E, D>;
  constexpr int RB = NW / NSPLIT;        // 32-key blocks per item
  constexpr int BKV = 32 * RB;           // keys per item
  constexpr int BQ = 32 * NSPLIT * KPW;  // queries per staged tile
  constexpr int NDB = D / 32;
  using LD = StageLoader<E, D, BQ, NW>;
  constexpr int TILEB = BQ * TL::ROWB;                            // dO follows Q in a stage
  using OL = TileLoader<E, D, BQ, NW>;                            // DF: O follows dO
  // A ring stage holds the tiles only (its LDS addresses then fit the read
  // instructions' 16-bit offsets); the per-stage statistics (LSE*log2e, D)
  // follow all the stages.
  constexpr int STAGE = LD::BYTES + (DF ? OL::BYTES : 0);
  constexpr int SQF = (DF ? 4 : 2) * BQ;  // floats of statistics per stage
  constexpr int STATS = SQF * 4;
  constexpr int NL = LD::NLOADS + (DF ? OL::NLOADS : 0) + 1;      // loads per wave per tile
  static_assert(!DF || (is_bf16<E>() && WDS && !STR && !CROSS && !QSPLIT && !ROPE),
                "D formed in dK+dV: bf16 on the dS path, plain layout only");
  // Partials of the NSPLIT-1 helper waves of every key block, one matrix
  // (dK or dV): summed through the stage just consumed, in one pass when it
  // holds both matrices, else in two.
  constexpr int PART = RB * (NSPLIT - 1) * 16 * NDB * 64 * 4;
  constexpr int NPASS = 2 * PART <= STAGE ? 1 : 2;
  static_assert(PART * (3 - NPASS) <= STAGE, "split partials must fit one stage");
  static_assert(BKV == BQ, "a K/V header tile has the shape of a query tile");
  static_assert(NW % NSPLIT == 0 && NST >= 2 && NST <= 4, "launch shape");
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE + NST * STATS];
  float* const stats0 = reinterpret_cast<float*>(smem + NST * STAGE);

  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar
  const int kbk = w / NSPLIT, sp = w % NSPLIT;
  const int g = blockIdx.x, G = gridDim.x;
  const int Sk = CROSS ? Sk_ : Sq;
  const int nqt = (Sq + BQ - 1) / BQ;
  const int nqs = QSPLIT ? nqs_ : 1;
  const int qpc = QSPLIT ? qpc_ : nqt;
  const unsigned lane_off = STR ? 0u : LD::lane_offset(w, lane);
  const unsigned o_off = DF ? OL::lane_offset(D, w, lane) : 0u;
  const int ldq = row_ld<STR, D>(lay.q), ldk = row_ld<STR, D>(lay.k);
  const int ldv = row_ld<STR, D>(lay.v), lddo = row_ld<STR, D>(lay.dout);
  // First query tile with a query that sees a key of key tile kt (nqt: none).
  auto first_qt = [&](int kt, int L, int off) {
    if constexpr (!CROSS) {
      return CAUSAL ? (kt * BKV) / BQ : 0;
    } else {
      if (kt * BKV >= L) return nqt;
      return CAUSAL ? min(nqt, max(0, kt * BKV - off) / BQ) : 0;
    }
  };

  // Loader cursor: the next stream tile to issue (lqt < 0: the header of
  // item lit, whose K and V rows it stages; else query tile lqt).  Every
  // stream tile is NL loads per wave (the header also loads statistics it
  // does not use, to keep that count).
  int lr = 0, lit = sched_item(sched, 0, g, G, BH), lqt = -1, lkt = lit / BH / nqs;
  int lqc = lit / BH % nqs, lqend = nqt;
  size_t lhq = (size_t)(lit % BH) * Sq, lhk = (size_t)(lit % BH) * Sk;  // first rows of the head
  int lL, loff;
  head_keys<CROSS>(kvlen, lit % BH, H, Sq, Sk, lL, loff);
  int nissued = 0;
  auto next_item = [&]() {
    lit = sched_item(sched, ++lr, g, G, BH);
    lqt = -1;
    lkt = lit / BH / nqs;
    lqc = lit / BH % nqs;
    lhq = (size_t)(lit % BH) * Sq;
    lhk = (size_t)(lit % BH) * Sk;
    head_keys<CROSS>(kvlen, lit % BH, H, Sq, Sk, lL, loff);
  };
  auto issue_next = [&]() {
    if (lit >= nitems) return;
    char* st = smem + (nissued % NST) * STAGE;
    const bool head = lqt < 0;
    if (head) {
      // K and V rows; past the valid keys the loads read the last valid row
      // (finite, and masked), so padded rows are never read.
      if constexpr (STR) {
        const int bhl = lit % BH;
        LD::issue_ld(st, K + head_off<STR, D>(lay.k, bhl, H, Sk), ldk,
                     V + head_off<STR, D>(lay.v, bhl, H, Sk), ldv, lkt * BKV,
                     CROSS ? max(lL, 1) : Sk, w, lane);
      } else {
        LD::issue(st, K + lhk * D, V + lhk * D, lkt * BKV, CROSS ? max(lL, 1) : Sk, w, lane,
                  lane_off, lane_off);
        // (DF: the head's first O rows, unused, so every tile has NL loads)
        if constexpr (DF) OL::issue(st + LD::BYTES, Oin + lhq * D, D, 0, Sq, 0, w, lane, o_off);
      }
    } else {
      if constexpr (STR) {
        const int bhl = lit % BH;
        LD::issue_ld(st, Q + head_off<STR, D>(lay.q, bhl, H, Sq), ldq,
                     dO + head_off<STR, D>(lay.dout, bhl, H, Sq), lddo, lqt * BQ, Sq, w, lane);
      } else {
        LD::issue(st, Q + lhq * D, dO + lhq * D, lqt * BQ, Sq, w, lane, lane_off, lane_off);
        if constexpr (DF)
          OL::issue(st + LD::BYTES, Oin + lhq * D, D, lqt * BQ, Sq, 0, w, lane, o_off);
      }
    }
    issue_stats<BQ, NW>(stats0 + (nissued % NST) * SQF, DF ? LSEin + lhq : Dws + Lws + lhq,
                        DF ? LSEin + lhq : Dws + lhq, head ? 0 : lqt * BQ, Sq, w, lane);
    ++nissued;
    if (head) {
      lqt = first_qt(lkt, lL, loff);
      if constexpr (QSPLIT) {
        lqt = max(lqt, lqc * qpc);
        lqend = min(nqt, (lqc + 1) * qpc);
      }
      if (lqt >= (QSPLIT ? lqend : nqt)) next_item();  // (an item that no query of its chunk sees)
    } else if (++lqt == (QSPLIT ? lqend : nqt)) {
      next_item();
    }
  };

  if (sched_item(sched, 0, g, G, BH) >= nitems) return;  // (the launch never makes more workgroups than items)
#pragma unroll
  for (int i = 0; i < NST - 1; ++i) issue_next();

  // dS^T store instructions per stored block: 16 values of T in 16-byte stores
  constexpr int NSTORE = WDS ? 16 * (int)sizeof(T) / 16 : 0;
  f32x16 dkacc[NDB], dvacc[NDB];
  RowFrag<E, D> kf, vf;
  // Sum the NSPLIT partial dK, dV of each key block of the item through
  // `buf` (an LDS stage no load targets), then store dK and dV.
  // Returns the store instructions counted for the tile waits: only rows that
  // every lane writes, so the count never exceeds the instructions issued.
  auto merge_store = [&](char* buf, int bh, int qc, int k0, bool active) -> int {
    if constexpr (NSPLIT > 1) {
      float* cb = reinterpret_cast<float*>(buf);
      constexpr int PER = (NPASS == 1 ? 2 : 1) * 16 * NDB;  // floats per lane per helper wave
      constexpr int VOFF = NPASS == 1 ? 16 * NDB : 0;       // dV after dK in one pass
#pragma unroll
      for (int pass = 0; pass < NPASS; ++pass) {
        const bool withk = NPASS == 1 || pass == 0, withv = NPASS == 1 || pass == 1;
        lds_barrier();  // every wave is done reading the stage (or the previous pass)
        // Partials go through LDS four at a time: value group q of lane l at
        // float (q * 64 + l) * 4, so each 16-byte write or read of a wave
        // covers 1 KiB without bank conflicts.
        if (sp != 0 && active) {
          f32x4* dst = reinterpret_cast<f32x4*>(cb + ((kbk * (NSPLIT - 1) + sp - 1) * PER) * 64) + lane;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (withk)
                dst[(db * 4 + j) * 64] = f32x4{dkacc[db][4 * j], dkacc[db][4 * j + 1],
                                               dkacc[db][4 * j + 2], dkacc[db][4 * j + 3]};
              if (withv)
                dst[(VOFF / 4 + db * 4 + j) * 64] = f32x4{dvacc[db][4 * j], dvacc[db][4 * j + 1],
                                                          dvacc[db][4 * j + 2], dvacc[db][4 * j + 3]};
            }
        }
        lds_barrier();
        if (sp == 0 && active) {
#pragma unroll
          for (int p = 0; p < NSPLIT - 1; ++p) {
            const f32x4* src =
                reinterpret_cast<const f32x4*>(cb + ((kbk * (NSPLIT - 1) + p) * PER) * 64) + lane;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                if (withk) {
                  const f32x4 x = src[(db * 4 + j) * 64];
#pragma unroll
                  for (int e = 0; e < 4; ++e) dkacc[db][4 * j + e] += x[e];
                }
                if (withv) {
                  const f32x4 x = src[(VOFF / 4 + db * 4 + j) * 64];
#pragma unroll
                  for (int e = 0; e < 4; ++e) dvacc[db][4 * j + e] += x[e];
                }
              }
          }
        }
      }
    }
    int nstores = 0;
    if (sp == 0 && active) {
      // The accumulators hold dK^T and dV^T: element r of acc[db] is key
      // k0 + n, column db*32 + out_row(r, h), so elements 4j .. 4j+3 are four
      // consecutive columns of one key row and go out in one store.
      const int key = k0 + n;
      if constexpr (!QSPLIT) {
        T* dk = dK + head_off<STR, D>(lay.dk, bh, H, Sk);
        T* dv = dV + head_off<STR, D>(lay.dv, bh, H, Sk);
        const int lddk = row_ld<STR, D>(lay.dk), lddv = row_ld<STR, D>(lay.dv);
        if (key < Sk) {
          float ks = scale;
          if constexpr (ROPE) {
            // dK of the turned rows, scaled, then turned back in f32
#pragma unroll
            for (int db = 0; db < NDB; ++db) dkacc[db] *= scale;
            const size_t tr = (size_t)(rope.pos + key) * (D / 2);
            rope_back_acc<D>(dkacc, rope.cos + tr, rope.sin + tr, h);
            ks = 1.f;
          }
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int d = db * 32 + 8 * j + 4 * h;
              store4<T>(dk + (size_t)key * lddk + d, dkacc[db][4 * j] * ks,
                        dkacc[db][4 * j + 1] * ks, dkacc[db][4 * j + 2] * ks,
                        dkacc[db][4 * j + 3] * ks);
              store4<T>(dv + (size_t)key * lddv + d, dvacc[db][4 * j], dvacc[db][4 * j + 1],
                        dvacc[db][4 * j + 2], dvacc[db][4 * j + 3]);
            }
        }
      } else {
        float* pk = part + ((size_t)qc * BH + bh) * Sk * D;
        float* pv = part + ((size_t)(nqs + qc) * BH + bh) * Sk * D;
        if (key < Sk) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int d = db * 32 + 8 * j + 4 * h;
              store4<float>(pk + (size_t)key * D + d, dkacc[db][4 * j] * scale,
                            dkacc[db][4 * j + 1] * scale, dkacc[db][4 * j + 2] * scale,
                            dkacc[db][4 * j + 3] * scale);
              store4<float>(pv + (size_t)key * D + d, dvacc[db][4 * j], dvacc[db][4 * j + 1],
                            dvacc[db][4 * j + 2], dvacc[db][4 * j + 3]);
            }
        }
      }
      // (counted only when every lane's key exists, so that every lane stores)
      if (k0 + 31 < Sk) nstores = 2 * 4 * NDB;
    }
    return nstores;
  };

  // Vector-memory operations this wave issued in the previous iteration after
  // the loads of every tile still in flight: dS^T stores (NSTORE per stored
  // block) and dK, dV stores.  A tile waits until no more than those and the
  // younger tiles' loads are pending (vmcnt counts stores too, and vector
  // memory retires in issue order).
  int stored = 0, estores = 0;
  int pos = 0;  // stream position of the tile being consumed
  for (int cr = 0;; ++cr) {
    const int cit = sched_item(sched, cr, g, G, BH);
    if (cit >= nitems) break;
    const int kt = cit / BH / nqs, qc = cit / BH % nqs, bh = cit % BH;
    const int k0 = kt * BKV + kbk * 32;
    const int kj = k0 + n;
    const bool wave_active = k0 < Sk;
    int cL, coff;  // the item's valid keys and causal offset
    head_keys<CROSS>(kvlen, bh, H, Sq, Sk, cL, coff);

    // Header: this wave's K, V rows into registers.
    wait_vmem_dyn(NL * (nissued - pos - 1) + NSTORE * stored + estores);
    stored = 0;
    estores = 0;
    lds_barrier();  // the header is in LDS; every wave is done with the tile before
    issue_next();
    __builtin_amdgcn_sched_barrier(0);  // the counts above assume this issue order
    const char* hst = smem + (pos % NST) * STAGE;
    load_row_frag_lds<E, D>(kf, hst, kbk * 32 + n, h, kj < Sk);
    load_row_frag_lds<E, D>(vf, hst + TILEB, kbk * 32 + n, h, kj < Sk);
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
      dkacc[i] = zero16();
      dvacc[i] = zero16();
    }
    ++pos;

    const int qbeg = QSPLIT ? max(first_qt(kt, cL, coff), qc * qpc) : first_qt(kt, cL, coff);
    const int qend = QSPLIT ? min(nqt, (qc + 1) * qpc) : nqt;
    for (int qt = qbeg; qt < qend; ++qt, ++pos) {
      if (estores == 0) wait_tiles<NL, NSTORE>(nissued - pos - 1, stored);
      else wait_vmem_dyn(NL * (nissued - pos - 1) + NSTORE * stored + estores);
      stored = 0;
      estores = 0;
      lds_barrier();  // tile pos is in LDS; every wave is done with the one before
      // f32 issues the next tile's loads after this step's first products,
      // so that their issue overlaps those MFMAs (dK+dV at B8 H12 S512 D64
      // causal: 70.9 -> 70.4 us); bf16 measured slower so and issues first.
      // Either way they precede the step's stores, as the waits assume.
      bool issued = false;
      if (is_bf16<E>() || !wave_active) {
        issue_next();
        issued = true;
      }
      __builtin_amdgcn_sched_barrier(0);
      if (!wave_active) continue;
      const int si = pos % NST;
      const char* Qt = smem + si * STAGE;
      const char* dOt = Qt + TILEB;
      float* const stw = stats0 + si * SQF + (DF ? 2 * BQ : 0);  // LSE*log2(e), then D
      const float* lse2s = stw;
      const float* Ds = lse2s + BQ;

#pragma unroll
      for (int j = 0; j < KPW; ++j) {
        const int qbl = sp + NSPLIT * j;  // query block within the tile
        const int qq0 = qt * BQ + qbl * 32;
        if (!(qq0 < Sq && (!CAUSAL || qq0 + 31 >= k0 - coff) && (!CROSS || k0 < cL)))
          continue;  // wave-uniform
        const int arow = qbl * 32 + pi32(n);
        // f32 runs the products at raised wave priority, so that while one
        // wave of a SIMD is in its softmax the other's MFMAs issue first
        // (70.4 -> 69.2 us at B8 H12 S512 D64 causal; bf16 measured slower)
        if constexpr (!is_bf16<E>()) __builtin_amdgcn_s_setprio(1);
        f32x16 s = dot_tile<E, D>(Qt, arow, h, kf, zero16());
        f32x16 dp = dot_tile<E, D>(dOt, arow, h, vf, zero16());
        if constexpr (!is_bf16<E>()) __builtin_amdgcn_s_setprio(0);
        if (!issued) {
          __builtin_amdgcn_sched_barrier(0);
          issue_next();
          __builtin_amdgcn_sched_barrier(0);
          issued = true;
        }
        if constexpr (DF) {
          // D and LSE*log2(e) of the block's 32 queries: lane (h, n) dots
          // half h of query row qbl*32 + n of dO and O, the halves add, and
          // every lane stores its row's pair (both halves, and the other wave
          // of this query block, store the same bits), read back below.
          const int qr = qbl * 32 + n;
          RowFrag<E, D> fd, fo;
          load_row_frag_lds<E, D>(fd, dOt, qr, h, true);
          load_row_frag_lds<E, D>(fo, dOt + TILEB, qr, h, true);
          float dsum = 0.f;
#pragma unroll
          for (int c = 0; c < RowFrag<E, D>::NS; ++c) {
            const bf16x8 x = fd.f[c], y = fo.f[c];
            dsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1),
                                                   __builtin_shufflevector(y, y, 0, 1), dsum, false);
            dsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3),
                                                   __builtin_shufflevector(y, y, 2, 3), dsum, false);
            dsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5),
                                                   __builtin_shufflevector(y, y, 4, 5), dsum, false);
            dsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7),
                                                   __builtin_shufflevector(y, y, 6, 7), dsum, false);
          }
          dsum += __shfl_xor(dsum, 32);
          stw[qr] = stw[qr - 2 * BQ] * kLog2e;
          stw[BQ + qr] = dsum;
        }
        if ((CAUSAL && qq0 < k0 + 31 - coff) || qq0 + 32 > Sq || k0 + 32 > (CROSS ? cL : Sk)) {
          // query(r) = qq0 + 8h + (16*(r/8) + r%8) sees key kj iff
          // kj - off <= query < Sq and kj < L (L = Sk without CROSS); a key
          // past them gets P = 0 and dS = 0 exactly (its K, V registers
          // hold finite values: zeros, or a copy of the last valid row), so
          // blocks of valid keys need no select
          int lo = CAUSAL ? kj - coff - qq0 - 8 * h : -64;
          if (kj >= (CROSS ? cL : Sk)) lo = 64;
          const int hi = Sq - 1 - qq0 - 8 * h;
          // all-ones where o < lo or o > hi, built without per-element
          // compare masks (which would hold 16 scalar register pairs); the
          // whole vector is bit-cast (a bit_cast of one element of an
          // ext_vector is not reliable in this toolchain)
          u32x16 sb = __builtin_bit_cast(u32x16, s);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int o = 16 * (r >> 3) + (r & 7);
            const unsigned out = (unsigned)(((o - lo) | (hi - o)) >> 31);
            sb[r] = (sb[r] & ~out) | (0xff800000u & out);
          }
          s = __builtin_bit_cast(f32x16, sb);
        }
        // LSE*log2(e) and D of this lane's 16 queries: two runs of 8 at rho(0, h)
        // and rho(8, h), handled one run at a time to keep registers down.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int off = qbl * 32 + 16 * u + 8 * h;
          const f32x4 l0 = *reinterpret_cast<const f32x4*>(lse2s + off);
          const f32x4 l1 = *reinterpret_cast<const f32x4*>(lse2s + off + 4);
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(Ds + off);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(Ds + off + 4);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int r = 8 * u + t;
            const float lq = t < 4 ? l0[t] : l1[t - 4];
            const float dq = t < 4 ? d0[t] : d1[t - 4];
            const float p = fast_exp2(fmaf(s[r], c, -lq));  // 0 where masked
            s[r] = p;
            dp[r] = p * (dp[r] - dq);
          }
        }
        if constexpr (WDS) {
          ++stored;
          // dS^T for the dQ GEMM, row kj: this lane's 16 values are queries
          // qq0 + 8h + {0..7} and qq0 + 16 + 8h + {0..7} (exact zeros where
          // masked, for queries past Sq and for keys past Sk).
          T* row = dSout + ((size_t)bh * SPk + kj) * SPq + qq0 + 8 * h;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            if constexpr (is_bf16<E>()) {
              bf16x8 o;
#pragma unroll
              for (int t = 0; t < 8; ++t) o[t] = (__bf16)dp[8 * u + t];
              *reinterpret_cast<bf16x8*>(row + 16 * u) = o;
            } else {
#pragma unroll
              for (int v4 = 0; v4 < 2; ++v4) {
                f32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = dp[8 * u + 4 * v4 + e];
                *reinterpret_cast<f32x4*>(row + 16 * u + 4 * v4) = o;
              }
            }
          }
        }
        RegOperand<E> P, dS;
        P.set(s);
        dS.set(dp);
        if constexpr (!is_bf16<E>()) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          // dV^T (d x keys) += dO^T P and dK^T += Q^T dS: the register
          // operand is the B side, so a lane accumulates its own key's row
          dvacc[db] = second_tile<E, D, false>(P, dOt, qbl * 32, db * 32, lane, dvacc[db]);
          dkacc[db] = second_tile<E, D, false>(dS, Qt, qbl * 32, db * 32, lane, dkacc[db]);
        }
        if constexpr (!is_bf16<E>()) __builtin_amdgcn_s_setprio(0);
      }
      if (!issued) issue_next();  // (no block of the tile was visible)
    }

    // The item is done: merge through the stage of its last tile (the tiles
    // in flight are the next NST-1, so no load targets it).
    estores = merge_store(smem + ((pos - 1) % NST) * STAGE, bh, qc, k0, wave_active);
  }
}

// dK = sum over the query chunks of the float32 partials, and dV likewise,
// in chunk order (deterministic); four elements per thread, 64 threads per
// workgroup (a small tensor spread over the CUs), the loads of eight chunks
// issued before their sums.
template <class T, int D, bool STR, bool ROPE>
__global__ __launch_bounds__(64) void bwd_dkdv_reduce_kernel(const float* __restrict__ part,
                                                             T* __restrict__ dK,
                                                             T* __restrict__ dV, int nqs,
                                                             long long nel4, int Sk, int H,
                                                             const Layout lay, const RopeTab rope) {
  // (partials are [B*H][Sk][D] packed; STR: dK, dV are laid out by `lay`)
  // ROPE: thread i sums the four columns it would own and the four D/2 on
  // (the pairs of the rotation), turns dK back, and stores both; the
  // launch covers half the groups.
  if constexpr (ROPE) {
    const long long i = (long long)blockIdx.x * 64 + threadIdx.x;
    if (i >= nel4 / 2) return;
    const long long row = i / (D / 8);
    const int col = (int)(i % (D / 8)) * 4;
    const long long lo4 = (row * D + col) / 4, hi4 = lo4 + D / 8;
    const f32x4* pk = reinterpret_cast<const f32x4*>(part);
    const f32x4* pv = pk + (size_t)nqs * nel4;
    f32x4 kl = {0.f, 0.f, 0.f, 0.f}, kh = kl, vl = kl, vh = kl;
    for (int qc = 0; qc < nqs; ++qc) {
      kl += pk[(size_t)qc * nel4 + lo4];
      kh += pk[(size_t)qc * nel4 + hi4];
      vl += pv[(size_t)qc * nel4 + lo4];
      vh += pv[(size_t)qc * nel4 + hi4];
    }
    const int bh = (int)(row / Sk), r = (int)(row % Sk);
    const size_t tr = (size_t)(rope.pos + r) * (D / 2) + col;
    const f32x4 c = *reinterpret_cast<const f32x4*>(rope.cos + tr);
    const f32x4 sv = *reinterpret_cast<const f32x4*>(rope.sin + tr);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float ylo, yhi;
      rope_pair(kl[e], kh[e], c[e], -sv[e], ylo, yhi);
      kl[e] = ylo;
      kh[e] = yhi;
    }
    T* dk = dK + head_off<STR, D>(lay.dk, bh, H, Sk) + (size_t)r * row_ld<STR, D>(lay.dk) + col;
    T* dv = dV + head_off<STR, D>(lay.dv, bh, H, Sk) + (size_t)r * row_ld<STR, D>(lay.dv) + col;
    store4<T>(dk, kl[0], kl[1], kl[2], kl[3]);
    store4<T>(dk + D / 2, kh[0], kh[1], kh[2], kh[3]);
    store4<T>(dv, vl[0], vl[1], vl[2], vl[3]);
    store4<T>(dv + D / 2, vh[0], vh[1], vh[2], vh[3]);
    return;
  }
  const long long i = (long long)blockIdx.x * 64 + threadIdx.x;
  if (i >= nel4) return;
  const f32x4* pk = reinterpret_cast<const f32x4*>(part) + i;
  const f32x4* pv = pk + (size_t)nqs * nel4;
  f32x4 ak = {0.f, 0.f, 0.f, 0.f}, av = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < nqs; q0 += 8) {
    f32x4 xk[8], xv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int qc = min(q0 + u, nqs - 1);  // (past the last chunk: loaded, not added)
      xk[u] = pk[(size_t)qc * nel4];
      xv[u] = pv[(size_t)qc * nel4];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (q0 + u < nqs) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ak[e] += xk[u][e];
          av[e] += xv[u][e];
        }
      }
    }
  }
  if constexpr (STR) {
    const long long e = 4 * i;
    const int bh = (int)(e / ((long long)Sk * D));
    const int rem = (int)(e - (long long)bh * Sk * D);
    const int row = rem / D, d = rem % D;
    store4<T>(dK + head_off<STR, D>(lay.dk, bh, H, Sk) + (size_t)row * lay.dk.s + d, ak[0], ak[1],
              ak[2], ak[3]);
    store4<T>(dV + head_off<STR, D>(lay.dv, bh, H, Sk) + (size_t)row * lay.dv.s + d, av[0], av[1],
              av[2], av[3]);
  } else {
    store4<T>(dK + 4 * i, ak[0], ak[1], ak[2], ak[3]);
    store4<T>(dV + 4 * i, av[0], av[1], av[2], av[3]);
  }
}

template <class E, int D, bool CAUSAL, bool WDS, bool CROSS, bool QSPLIT, bool STR, bool ROPE,
          bool DF = false>
static hipError_t launch(const BwdArgs& a) {
  constexpr LShape SH = dkdv_shape(is_bf16<E>(), D);
  constexpr int NW = SH.nw, NSPLIT = SH.nsplit, KPW = SH.kpw;
  constexpr int NST = DF ? ATTN_DKDV_NST_BF16_DF : SH.nst;
  using T = typename E::T;
  constexpr auto kern =
      bwd_dkdv_kernel<E, D, NW, NSPLIT, KPW, NST, CAUSAL, WDS, CROSS, QSPLIT, STR, ROPE, DF>;
  const Layout lay = a.layout != nullptr ? *a.layout : Layout{};
  constexpr int BKV = 32 * (NW / NSPLIT);
  constexpr int BQ = 32 * NSPLIT * KPW;
  static_assert(BKV == dkdv_key_tile(is_bf16<E>(), D) && BQ == dkdv_query_tile(is_bf16<E>(), D),
                "tile sizes of the query-chunk choice");
  const int nkt = (a.Sk + BKV - 1) / BKV;
  const int nqt = (a.Sq + BQ - 1) / BQ;
  const int nqs = QSPLIT ? a.nqs : 1;
  const int qpc = (nqt + nqs - 1) / nqs;
  const int nitems = a.BH * nkt * nqs;
  const int grid = std::min(nitems, resident_workgroups<kern>(NW * 64));
  // work of class c = (key tile c / nqs, query chunk c % nqs): its header
  // tile and the query tiles it visits (with every key valid: the per-batch
  // counts live on the device)
  const int off = a.Sk - a.Sq;
  std::vector<int> works(nkt * nqs);
  for (int c = 0; c < nkt * nqs; ++c) {
    const int kt = c / nqs, qc = c % nqs;
    const int fq = CAUSAL ? std::min(nqt, std::max(0, kt * BKV - off) / BQ) : 0;
    const int lo = std::max(fq, qc * qpc), hi = std::min(nqt, (qc + 1) * qpc);
    works[c] = 4 * std::max(0, hi - lo) +
               (is_bf16<E>() ? ATTN_DKDV_ITEM_COST_BF16 : ATTN_DKDV_ITEM_COST_F32);
  }
  const Sched sched = make_sched(grid, a.BH, works);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), 0, a.stream, (const T*)a.q, (const T*)a.k,
                     (const T*)a.v, (const T*)a.dout, a.delta, (T*)a.dk, (T*)a.dv, (T*)a.ds, a.SPq,
                     a.SPk, a.Sq, a.Sk, a.BH * a.Sq, a.scale * kLog2e, a.scale, a.BH, a.H, a.kvlen,
                     QSPLIT ? a.part : nullptr, nqs, qpc, nitems, sched, lay, a.rope,
                     DF ? (const T*)a.o : nullptr, DF ? a.lse : nullptr);
  if (QSPLIT) {
    const long long nel4 = (long long)a.BH * a.Sk * D / 4;
    const long long nthr = ROPE ? nel4 / 2 : nel4;
    hipLaunchKernelGGL((bwd_dkdv_reduce_kernel<T, D, STR, ROPE>), dim3((unsigned)((nthr + 63) / 64)),
                       dim3(64), 0, a.stream, a.part, (T*)a.dk, (T*)a.dv, nqs, nel4, a.Sk, a.H,
                       lay, a.rope);
  }
  return hipGetLastError();
}

template <class E, int D, bool CAUSAL, bool WDS, bool CROSS, bool STR, bool ROPE = false>
static hipError_t launch_s(const BwdArgs& a) {
  if constexpr (is_bf16<E>() && WDS && !CROSS && !STR && !ROPE) {
    if (a.dfused) return launch<E, D, CAUSAL, WDS, CROSS, false, STR, ROPE, true>(a);
  }
  if (a.dfused) return hipErrorInvalidValue;  // (dkdv_dfused admits only the case above)
  if (a.part != nullptr && a.nqs > 1) return launch<E, D, CAUSAL, WDS, CROSS, true, STR, ROPE>(a);
  return launch<E, D, CAUSAL, WDS, CROSS, false, STR, ROPE>(a);
}

// (strided layouts run the cross-attention instantiation)
template <class E, int D, bool CAUSAL, bool WDS>
static hipError_t launch_x(const BwdArgs& a) {
  if (a.rope.cos != nullptr) return launch_s<E, D, CAUSAL, WDS, true, true, true>(a);
  if (a.layout != nullptr) return launch_s<E, D, CAUSAL, WDS, true, true>(a);
  return a.cross ? launch_s<E, D, CAUSAL, WDS, true, false>(a)
                 : launch_s<E, D, CAUSAL, WDS, false, false>(a);
}

template <class E, int D>
static hipError_t launch_c(const BwdArgs& a) {
  if (a.ds != nullptr) return a.causal ? launch_x<E, D, true, true>(a) : launch_x<E, D, false, true>(a);
  return a.causal ? launch_x<E, D, true, false>(a) : launch_x<E, D, false, false>(a);
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
