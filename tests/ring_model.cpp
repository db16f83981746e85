// Host model of the vector-memory wait protocol of the persistent attention
// kernels (fwd_kernel in attn_fwd.hip, bwd_dkdv_kernel in attn_bwd_dkdv.hip).
//
// Each wave of those kernels streams tiles through an NST-stage LDS ring with
// direct global->LDS loads, and before consuming a tile it waits until at
// most N of its vector-memory operations are pending (s_waitcnt vmcnt(N)),
// where N comes from a count the kernel keeps of what it issued after that
// tile (loads of younger tiles, and stores).  vmcnt counts loads and stores
// alike and they retire in issue order, so the wait is right iff every
// operation of the tile is older than the N youngest pending ones.
//
// This program replays, per wave, the exact sequence of vector-memory
// instructions the kernels issue for a launch -- the same static schedule
// (build_sched / sched_item), the same per-tile load counts (the loaders'
// NLOADS constants for the launch shape of each element type and head_dim),
// the same store instructions (with the partial-wave stores that the kernels
// do not count) -- into an in-order queue of pending operations (at most 63
// pending, as the hardware counter allows), applies the kernels' wait
// formulas to that queue, and checks at every consumed tile that
//   * every load of the tile (and, in the forward, of the item's Q tile) has
//     retired,
//   * the ring slot holds the tile the consumer expects (the loader and the
//     consumer agree on the stream, also across items shorter than the ring),
//   * no slot is reloaded before its tile was consumed.
// It covers causal and non-causal self-attention, cross-attention with
// padded keys (empty rows, items no query sees), the query-chunk split, every
// head_dim and both storage types, and shapes whose items have fewer tiles
// than the ring is deep.  Test infrastructure; prints one line per case and
// exits non-zero on the first violation.
#include "attn_launch.hpp"

#include <cstdio>
#include <cstdlib>
#include <deque>
#include <string>
#include <vector>

using namespace attn;

namespace {

int fails = 0;
// A planted mistake (command-line argument; 0: none) that the checks must
// catch, so that a pass of the model means something:
//   1 forward: the consumer takes its first item after the prologue issues
//     (the loader cursor has then moved past a short first item)
//   2 forward: a tile waits with the mark of the next ring slot
//   3 forward: O stores are counted for a wave whose queries all lie past the
//     end (it stores nothing)
//   4 dK+dV: the header wait counts the item-end stores twice
//   5 dK+dV: the item-end stores are counted for the helper waves too (they
//     store nothing)
//   6 dK+dV: a tile waits as if one more tile had been issued after it
int plant = 0;
#define CHECK(c, ...)                                  \
  do {                                                 \
    if (!(c)) {                                        \
      std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
      std::printf(__VA_ARGS__);                        \
      std::printf("\n");                               \
      if (++fails > 5) std::exit(1);                   \
      return false;                                    \
    }                                                  \
  } while (0)

// The pending vector-memory operations of one wave, oldest first.
struct Queue {
  struct Op {
    long tag;  // what the operation belongs to (a tile's stream position, ...)
  };
  std::deque<Op> q;
  void issue(long tag) {
    if (q.size() == 63) q.pop_front();  // the counter is full: issue stalls until one retires
    q.push_back(Op{tag});
  }
  void wait(int n) {  // s_waitcnt vmcnt(n), n clamped as wait_vmem_dyn does
    if (n < 0) n = 0;
    if (n > 63) n = 63;
    while ((int)q.size() > n) q.pop_front();
  }
  bool pending(long tag) const {
    for (const Op& o : q)
      if (o.tag == tag) return true;
    return false;
  }
};

constexpr long kStore = -1;          // tag of store instructions
constexpr long kQBase = 1L << 40;    // forward Q tiles: kQBase + round
constexpr long kAngle = -2;          // tag of the RoPE angle loads (counted by no wait)

// ---------------------------------------------------------------- forward
struct FwdCase {
  bool bf16;
  int D, BH, H, Sq, Sk;
  bool causal, cross;
  std::vector<int> kvlen;  // per batch (cross only; empty: all Sk)
  bool lse;
  bool ks = false;  // key split (fwd_key_split), self-attention only
  bool rope = false;  // RoPE turned in the kernel (attn_fwd_rope), self-attention only
};

template <class E, int D>
bool model_fwd(const FwdCase& c, int G) {
  constexpr LShape SH = fwd_shape(is_bf16<E>(), D);
  constexpr int NW = SH.nw, NSPLIT = SH.nsplit, KPW = SH.kpw, NST = SH.nst;
  constexpr int RB = NW / NSPLIT, BR = 32 * RB, BK = 32 * NSPLIT * KPW, NDB = D / 32;
  using LD = StageLoader<E, D, BK, NW>;
  using QL = TileLoader<E, D, BR, NW>;
  // RoPE: the kernel's per-wave angle loads of one Q or K tile and its
  // turned-row stores, none of them in its count
  constexpr int NANG = 2 * TileRope<E, D, BK, NW>::UPT * (TileRope<E, D, BK, NW>::EPC / 4);
  constexpr int NTST = 2 * TileRope<E, D, BK, NW>::UPT;
  static_assert(BR == BK, "the RoPE forward turns square tiles");
  const int Sq = c.Sq, Sk = c.cross ? c.Sk : c.Sq, BH = c.BH, H = c.H;
  const int nqt = (Sq + BR - 1) / BR;
  int nch = 1, kc = 1 << 30;
  if (c.ks && !fwd_key_split(is_bf16<E>(), BH, Sq, D, c.causal, nch, kc)) return true;
  const int nitems = BH * nqt * nch;
  G = std::min(G, nitems);
  std::vector<int> works(nqt * nch);
  for (int cc = 0; cc < nqt * nch; ++cc) {
    const int qt = nqt - 1 - cc / nch, ch = cc % nch;
    const int kend = c.causal ? std::min(Sk, qt * BR + BR + Sk - Sq) : Sk;
    const int full = std::max((kend + BK - 1) / BK, 1);
    const int nq = (full + kc - 1) / kc, csz = (full + nq - 1) / nq;
    const int ntl = ch < nq ? std::min(csz, full - ch * csz) : 0;
    works[cc] = ntl > 0 ? 4 * ntl + (is_bf16<E>() ? ATTN_FWD_ITEM_COST_BF16 : ATTN_FWD_ITEM_COST_F32)
                        : 0;
  }
  const Sched sched = build_sched(G, BH, works, 32);
  if (c.ks && sched.M == 0) {  // the launcher then runs the forward unsplit
    FwdCase u = c;
    u.ks = false;
    return model_fwd<E, D>(u, G);
  }
  auto keys = [&](int bh, int& L, int& off) {
    L = Sk;
    off = 0;
    if (c.cross) {
      if (!c.kvlen.empty()) L = std::min(std::max(c.kvlen[bh / H], 0), Sk);
      off = L - Sq;
    }
  };
  auto item_qt = [&](int it) { return nqt - 1 - it / BH / nch; };
  auto item_nkt = [&](int it) {  // (the chunk's tiles, as the kernel's item_chunk)
    int L, off;
    keys(it % BH, L, off);
    const int kend = c.causal ? std::min(L, item_qt(it) * BR + BR + off) : L;
    const int n = (kend + BK - 1) / BK;
    const int full = c.cross ? std::max(n, 1) : n;
    const int nq = (full + kc - 1) / kc, csz = (full + nq - 1) / nq;
    const int kb0 = (it / BH % nch) * csz;
    return std::min(csz, full - kb0);
  };
  for (int g = 0; g < G; ++g) {
    if (sched_item(sched, 0, g, G, BH) >= nitems) continue;
    for (int w = 0; w < NW; ++w) {
      const int qb = w / NSPLIT, sp = w % NSPLIT;
      Queue Q;
      int vm = 0, qmark = 0;
      RingMarks<NST> mk;
      std::vector<long> slot_tile(NST, -1);   // stream position held by each slot
      std::vector<bool> consumed(NST, true);
      std::vector<std::pair<int, int>> stream;  // (item, key tile) of each stream position
      long qtile = -1;                           // round whose Q tile the Q buffer holds
      int lr = 0, lit = sched_item(sched, 0, g, G, BH), lkt = 0, lnkt = item_nkt(lit);
      long issued = 0;
      auto issue_next = [&](int slot) -> bool {
        if (lit >= nitems) return true;
        CHECK(consumed[slot], "fwd g%d w%d: slot %d reloaded before its tile was consumed", g, w,
              slot);
        for (int i = 0; i < LD::NLOADS; ++i) Q.issue(issued);
        vm += LD::NLOADS;
        mk.set(slot, vm);
        slot_tile[slot] = issued;
        consumed[slot] = false;
        stream.push_back({lit, lkt});
        ++issued;
        if (++lkt == lnkt) {
          lit = sched_item(sched, ++lr, g, G, BH);
          lkt = 0;
          if (lit < nitems) lnkt = item_nkt(lit);
        }
        return true;
      };
      auto load_q = [&](int round) {
        for (int i = 0; i < QL::NLOADS; ++i) Q.issue(kQBase + round);
        vm += QL::NLOADS;
        qmark = vm;
        qtile = round;
      };
      int cr = 0, cit = lit, kt = 0, nkt = lnkt;
      load_q(0);
      if (c.rope)  // angles of the first Q tile and of the first K tile
        for (int i = 0; i < 2 * NANG; ++i) Q.issue(kAngle);
      for (int s = 0; s < NST - 1; ++s)
        if (!issue_next(s)) return false;
      if (plant == 1) {
        cit = lit;
        nkt = lit < nitems ? item_nkt(lit) : 0;
      }
      int q0 = item_qt(cit) * BR + qb * 32;
      int ntiles = 0;
      for (int r = 0;; ++r) {
        const int it = sched_item(sched, r, g, G, BH);
        if (it >= nitems) break;
        ntiles += item_nkt(it);
      }
      for (int pos = 0; pos < ntiles; ++pos) {
        const int si = pos % NST;
        int mark = mk.get(plant == 2 ? (si + 1) % NST : si);
        if (kt == 0) mark = std::max(mark, qmark);
        Q.wait(vm - mark);
        CHECK(slot_tile[si] == pos, "fwd g%d w%d pos %d: slot %d holds stream tile %ld", g, w,
              pos, si, slot_tile[si]);
        CHECK(!Q.pending(pos), "fwd g%d w%d pos %d: tile consumed before its loads retired", g, w,
              pos);
        CHECK(stream[pos].first == cit && stream[pos].second == kt,
              "fwd g%d w%d pos %d: loader issued (item %d, tile %d), consumer expects (%d, %d)", g,
              w, pos, stream[pos].first, stream[pos].second, cit, kt);
        consumed[si] = true;
        if (c.rope) {
          // the wave turns its rows of the K tile (and on an item's first
          // tile of its Q tile) before the barrier; the compiler's wait for
          // the angles (taken as vmcnt(0)); turned-row stores; then the
          // angles of the tile issued next
          if (kt == 0)
            CHECK(qtile == cr && !Q.pending(kQBase + cr),
                  "fwd g%d w%d: item round %d turned its Q tile before it arrived", g, w, cr);
          Q.wait(0);
          for (int i = 0; i < (kt == 0 ? 2 : 1) * NTST; ++i) Q.issue(kStore);
          if (lit < nitems)
            for (int i = 0; i < NANG; ++i) Q.issue(kAngle);
        }
        if (!issue_next((si + NST - 1) % NST)) return false;
        if (kt == 0) {
          CHECK(qtile == cr && !Q.pending(kQBase + cr),
                "fwd g%d w%d: item round %d read its Q tile before it arrived", g, w, cr);
          if (sched_item(sched, cr + 1, g, G, BH) < nitems) {
            load_q(cr + 1);
            if (c.rope)
              for (int i = 0; i < NANG; ++i) Q.issue(kAngle);
          }
        }
        if (++kt < nkt) continue;
        // item done: O stores (and the LSE store) of the waves that own the block
        const bool active = q0 < Sq;
        if (sp == 0 && active) {
          for (int i = 0; i < 4 * NDB + (c.lse ? 1 : 0); ++i) Q.issue(kStore);
          if (q0 + 31 < Sq) vm += 4 * NDB;
        } else if (plant == 3 && sp == 0) {
          vm += 4 * NDB;
        }
        cit = sched_item(sched, ++cr, g, G, BH);
        kt = 0;
        if (cit < nitems) {
          nkt = item_nkt(cit);
          q0 = item_qt(cit) * BR + qb * 32;
        }
      }
      CHECK(cit >= nitems && lit >= nitems && issued == ntiles,
            "fwd g%d w%d: loader issued %ld tiles, consumer took %d", g, w, issued, ntiles);
    }
  }
  return true;
}

// ---------------------------------------------------------------- dK + dV
struct BwdCase {
  bool bf16;
  int D, BH, H, Sq, Sk;
  bool causal, cross, wds;
  std::vector<int> kvlen;
  int nqs;          // query chunks (1: no split)
  bool df = false;  // bf16 with D formed in the kernel: O rows in every tile, its own ring depth
};

template <class E, int D, bool DF = false>
bool model_dkdv(const BwdCase& c, int G) {
  constexpr LShape SH = dkdv_shape(is_bf16<E>(), D);
  constexpr int NW = SH.nw, NSPLIT = SH.nsplit, KPW = SH.kpw;
  constexpr int NST = DF ? ATTN_DKDV_NST_BF16_DF : SH.nst;
  constexpr int RB = NW / NSPLIT, BKV = 32 * RB, BQ = 32 * NSPLIT * KPW, NDB = D / 32;
  using LD = StageLoader<E, D, BQ, NW>;
  constexpr int NL = LD::NLOADS + (DF ? TileLoader<E, D, BQ, NW>::NLOADS : 0) + 1;
  constexpr int NSTORE = 16 * (int)sizeof(typename E::T) / 16;
  const int nstore = c.wds ? NSTORE : 0;
  const int Sq = c.Sq, Sk = c.cross ? c.Sk : c.Sq, BH = c.BH, H = c.H;
  const int nkt = (Sk + BKV - 1) / BKV, nqt = (Sq + BQ - 1) / BQ;
  const int nqs = c.nqs, qpc = (nqt + nqs - 1) / nqs, nitems = BH * nkt * nqs;
  G = std::min(G, nitems);
  const int offw = Sk - Sq;
  std::vector<int> works(nkt * nqs);
  for (int cc = 0; cc < nkt * nqs; ++cc) {
    const int kt = cc / nqs, qc = cc % nqs;
    const int fq = c.causal ? std::min(nqt, std::max(0, kt * BKV - offw) / BQ) : 0;
    const int lo = std::max(fq, qc * qpc), hi = std::min(nqt, (qc + 1) * qpc);
    works[cc] = 4 * std::max(0, hi - lo) +
                (is_bf16<E>() ? ATTN_DKDV_ITEM_COST_BF16 : ATTN_DKDV_ITEM_COST_F32);
  }
  const Sched sched = build_sched(G, BH, works, 32);
  auto keys = [&](int bh, int& L, int& off) {
    L = Sk;
    off = 0;
    if (c.cross) {
      if (!c.kvlen.empty()) L = std::min(std::max(c.kvlen[bh / H], 0), Sk);
      off = L - Sq;
    }
  };
  auto first_qt = [&](int kt, int L, int off) {
    if (!c.cross) return c.causal ? (kt * BKV) / BQ : 0;
    if (kt * BKV >= L) return nqt;
    return c.causal ? std::min(nqt, std::max(0, kt * BKV - off) / BQ) : 0;
  };
  for (int g = 0; g < G; ++g) {
    if (sched_item(sched, 0, g, G, BH) >= nitems) continue;
    for (int w = 0; w < NW; ++w) {
      const int kbk = w / NSPLIT, sp = w % NSPLIT;
      Queue Q;
      std::vector<long> slot_tile(NST, -1);
      std::vector<bool> consumed(NST, true);
      std::vector<std::pair<int, int>> stream;  // (item, query tile or -1 for the header)
      int lr = 0, lit = sched_item(sched, 0, g, G, BH), lqt = -1;
      int lkt = lit / BH / nqs, lqc = lit / BH % nqs, lqend = nqt;
      int lL, loff;
      keys(lit % BH, lL, loff);
      long nissued = 0;
      auto next_item = [&]() {
        lit = sched_item(sched, ++lr, g, G, BH);
        lqt = -1;
        lkt = lit / BH / nqs;
        lqc = lit / BH % nqs;
        keys(lit % BH, lL, loff);
      };
      auto issue_next = [&]() -> bool {
        if (lit >= nitems) return true;
        const int slot = (int)(nissued % NST);
        CHECK(consumed[slot], "dkdv g%d w%d: slot %d reloaded before its tile was consumed", g,
              w, slot);
        for (int i = 0; i < NL; ++i) Q.issue(nissued);
        slot_tile[slot] = nissued;
        consumed[slot] = false;
        stream.push_back({lit, lqt});
        ++nissued;
        if (lqt < 0) {
          lqt = first_qt(lkt, lL, loff);
          if (nqs > 1) {
            lqt = std::max(lqt, lqc * qpc);
            lqend = std::min(nqt, (lqc + 1) * qpc);
          }
          if (lqt >= (nqs > 1 ? lqend : nqt)) next_item();
        } else if (++lqt == (nqs > 1 ? lqend : nqt)) {
          next_item();
        }
        return true;
      };
      for (int i = 0; i < NST - 1; ++i)
        if (!issue_next()) return false;
      int stored = 0, estores = 0;
      long pos = 0;
      for (int cr = 0;; ++cr) {
        const int cit = sched_item(sched, cr, g, G, BH);
        if (cit >= nitems) break;
        const int kt = cit / BH / nqs, qc = cit / BH % nqs, bh = cit % BH;
        const int k0 = kt * BKV + kbk * 32;
        const bool active = k0 < Sk;
        int cL, coff;
        keys(bh, cL, coff);
        // header
        Q.wait((int)(NL * (nissued - pos - 1) + nstore * stored + (plant == 4 ? 2 : 1) * estores));
        stored = estores = 0;
        {
          const int si = (int)(pos % NST);
          CHECK(slot_tile[si] == pos && !Q.pending(pos) && stream[pos].first == cit &&
                    stream[pos].second == -1,
                "dkdv g%d w%d: header of item %d (stream %ld) not ready or not the item's", g, w,
                cit, pos);
          consumed[si] = true;
        }
        if (!issue_next()) return false;
        ++pos;
        const int qbeg = nqs > 1 ? std::max(first_qt(kt, cL, coff), qc * qpc) : first_qt(kt, cL, coff);
        const int qend = nqs > 1 ? std::min(nqt, (qc + 1) * qpc) : nqt;
        for (int qt = qbeg; qt < qend; ++qt, ++pos) {
          const long newer = nissued - pos - 1 + (plant == 6 ? 1 : 0);
          if (estores == 0) {
            // wait_tiles<NL, NSTORE>(newer, stored): newer clamped to 2
            const int nw = newer >= 2 ? 2 : (int)newer;
            Q.wait(nw * NL + (stored >= 2 ? 2 : stored) * nstore);
          } else {
            Q.wait((int)(NL * newer + nstore * stored + estores));
          }
          stored = estores = 0;
          const int si = (int)(pos % NST);
          CHECK(slot_tile[si] == pos && !Q.pending(pos),
                "dkdv g%d w%d: query tile %d of item %d consumed before its loads retired", g, w,
                qt, cit);
          CHECK(stream[pos].first == cit && stream[pos].second == qt,
                "dkdv g%d w%d pos %ld: loader issued (item %d, tile %d), consumer expects (%d, %d)",
                g, w, pos, stream[pos].first, stream[pos].second, cit, qt);
          consumed[si] = true;
          if (!issue_next()) return false;
          if (!active) continue;
          for (int j = 0; j < KPW; ++j) {
            const int qbl = sp + NSPLIT * j;
            const int qq0 = qt * BQ + qbl * 32;
            if (!(qq0 < Sq && (!c.causal || qq0 + 31 >= k0 - coff) && (!c.cross || k0 < cL)))
              continue;
            if (c.wds) {
              ++stored;
              for (int i = 0; i < NSTORE; ++i) Q.issue(kStore);
            }
          }
        }
        // merge_store: dK and dV of the wave that owns the block (4 stores per
        // 32 columns each), counted when every lane's key exists
        if (sp == 0 && active) {
          for (int i = 0; i < 2 * 4 * NDB; ++i) Q.issue(kStore);
          if (k0 + 31 < Sk) estores = 2 * 4 * NDB;
        } else if (plant == 5 && active) {
          estores = 2 * 4 * NDB;
        }
      }
      CHECK(lit >= nitems && nissued == pos, "dkdv g%d w%d: loader issued %ld, consumer took %ld",
            g, w, nissued, pos);
    }
  }
  return true;
}

template <class E>
bool fwd_d(const FwdCase& c, int G) {
  switch (c.D) {
    case 32: return model_fwd<E, 32>(c, G);
    case 64: return model_fwd<E, 64>(c, G);
    default: return model_fwd<E, 128>(c, G);
  }
}
template <class E>
bool dkdv_d(const BwdCase& c, int G) {
  if (c.df) {
    switch (c.D) {
      case 32: return model_dkdv<E, 32, true>(c, G);
      case 64: return model_dkdv<E, 64, true>(c, G);
      default: return model_dkdv<E, 128, true>(c, G);
    }
  }
  switch (c.D) {
    case 32: return model_dkdv<E, 32>(c, G);
    case 64: return model_dkdv<E, 64>(c, G);
    default: return model_dkdv<E, 128>(c, G);
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc > 1) plant = std::atoi(argv[1]);
  // Resident workgroup counts to model: the launch uses min(items, resident);
  // several values exercise long and short per-workgroup item lists.
  const int grids[] = {512, 256, 64, 8, 1};
  int cases = 0;
  for (const bool bf16 : {false, true})
    for (const int D : {32, 64, 128})
      for (const int S : {1, 5, 17, 33, 64, 65, 130, 197, 512})
        for (const bool causal : {true, false})
          for (const int G : grids) {
            const int BH = S >= 512 ? 16 : 24;
            FwdCase f{bf16, D, BH, 4, S, S, causal, false, {}, true};
            BwdCase b{bf16, D, BH, 4, S, S, causal, false, true, {}, 1};
            const bool ok = (bf16 ? fwd_d<EBF16>(f, G) : fwd_d<EF32>(f, G)) &&
                            (bf16 ? dkdv_d<EBF16>(b, G) : dkdv_d<EF32>(b, G));
            bool ok3 = true;
            if (bf16) {  // (the D-fused bf16 dK+dV: dS stored, self-attention)
              b.df = true;
              ok3 = dkdv_d<EBF16>(b, G);
              b.df = false;
            }
            b.wds = false;
            const bool ok2 = (bf16 ? dkdv_d<EBF16>(b, G) : dkdv_d<EF32>(b, G)) && ok3;
            ++cases;
            if (!ok || !ok2) {
              std::printf("case: %s D%d S%d causal%d G%d\n", bf16 ? "bf16" : "f32", D, S, causal, G);
              return 1;
            }
          }
  std::printf("self-attention: %d cases ok\n", cases);
  // key split: few long heads (every chunked shape the rule produces for
  // these lengths), both storage types, every head_dim
  int kcases = 0;
  for (const bool bf16 : {false, true})
    for (const int D : {32, 64, 128})
      for (const int S : {1000, 1024, 1500, 2048})
        for (const int BH : {1, 2, 8, 16})
          for (const bool causal : {true, false})
            for (const int G : {512, 256, 64}) {
              FwdCase f{bf16, D, BH, BH, S, S, causal, false, {}, true, true};
              const bool ok = bf16 ? fwd_d<EBF16>(f, G) : fwd_d<EF32>(f, G);
              ++kcases;
              if (!ok) {
                std::printf("case: key split %s D%d BH%d S%d causal%d G%d\n", bf16 ? "bf16" : "f32",
                            D, BH, S, causal, G);
                return 1;
              }
            }
  std::printf("key split: %d cases ok\n", kcases);
  // RoPE turned in the forward: angle loads and turned-row stores that no
  // wait counts, in every self-attention shape above
  int rcases = 0;
  for (const bool bf16 : {false, true})
    for (const int D : {32, 64, 128})
      for (const int S : {1, 5, 17, 33, 64, 65, 130, 197, 512})
        for (const bool causal : {true, false})
          for (const int G : grids) {
            const int BH = S >= 512 ? 16 : 24;
            FwdCase f{bf16, D, BH, 4, S, S, causal, false, {}, true, false, true};
            const bool ok = bf16 ? fwd_d<EBF16>(f, G) : fwd_d<EF32>(f, G);
            ++rcases;
            if (!ok) {
              std::printf("case: rope %s D%d S%d causal%d G%d\n", bf16 ? "bf16" : "f32", D, S,
                          causal, G);
              return 1;
            }
          }
  std::printf("rope forward: %d cases ok\n", rcases);
  // cross-attention: separate lengths, padded keys (0, short, full), causal
  // alignment at the end of the valid keys, query-chunk split
  struct X { int Sq, Sk; std::vector<int> kv; int nqs; };
  const X xs[] = {{256, 77, {}, 1},        {256, 77, {77, 50}, 1},   {200, 130, {130, 97}, 1},
                  {96, 300, {300, 250}, 1}, {197, 197, {197, 120}, 1}, {2048, 77, {}, 8},
                  {1024, 200, {150, 3}, 4}, {1536, 100, {100, 61}, 6}, {64, 512, {512, 1}, 1},
                  {130, 64, {0, 64}, 1},   {5, 300, {300, 3}, 1}};
  int xc = 0;
  for (const bool bf16 : {false, true})
    for (const int D : {32, 64, 128})
      for (const bool causal : {true, false})
        for (const X& x : xs)
          for (const int G : grids) {
            FwdCase f{bf16, D, 8, 4, x.Sq, x.Sk, causal, true, x.kv, true};
            BwdCase b{bf16, D, 8, 4, x.Sq, x.Sk, causal, true, true, x.kv, x.nqs};
            const bool ok = (bf16 ? fwd_d<EBF16>(f, G) : fwd_d<EF32>(f, G)) &&
                            (bf16 ? dkdv_d<EBF16>(b, G) : dkdv_d<EF32>(b, G));
            ++xc;
            if (!ok) {
              std::printf("case: cross %s D%d Sq%d Sk%d causal%d nqs%d G%d\n",
                          bf16 ? "bf16" : "f32", D, x.Sq, x.Sk, causal, x.nqs, G);
              return 1;
            }
          }
  std::printf("cross-attention: %d cases ok\n", xc);
  std::printf("OK\n");
  return 0;
}
