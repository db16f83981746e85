// Host check of the LDS tile layouts of attn_device.hpp (Tile, StageLoader):
//   * Tile<E, D, KS>::off places every element of a row in that row's bytes,
//     each 16-byte chunk in its own slot (a permutation of the row's chunks),
//     with a swizzle that depends on row % 16 only (so offsets of 16-row
//     aligned blocks add);
//   * f32 storage: the second product's column reads (32 lanes read 32
//     consecutive floats of one row, the other 32 the row 8 further on) hit
//     64 distinct 4-byte banks for D >= 64 in both layouts (D = 32: at most
//     two lanes per bank);
//   * the k-slot layout (KS): a lane's 16 k-slot rows row0 + rho(w, h) all
//     carry the chunk XOR 8h, so their addresses are one base plus
//     rho(w, 0) rows, the form the k-slot operand read uses;
//   * StageLoader: with the per-matrix lane offsets, the chunk a lane fetches
//     on every load of every wave is the one Tile::off places at that lane's
//     direct-load destination, for both matrices and both layouts.
// Test infrastructure; prints one line per case and exits non-zero on the
// first violation.
#include "attn_launch.hpp"

#include <cstdio>
#include <set>

using namespace attn;

static int g_fail = 0;

#define CHECK(cond, ...)              \
  do {                                \
    if (!(cond)) {                    \
      std::printf("FAIL: ");          \
      std::printf(__VA_ARGS__);       \
      std::printf("\n");              \
      g_fail = 1;                     \
      return;                         \
    }                                 \
  } while (0)

template <class E, int D, bool KS>
static void check_tile(const char* name) {
  using TL = Tile<E, D, KS>;
  using T = typename E::T;
  for (int row = 0; row < 64; ++row) {
    CHECK(TL::swz(row) == TL::swz(row % 16), "%s swizzle of row %d", name, row);
    std::set<int> slots;
    for (int c = 0; c < TL::CPR; ++c) {
      const int o = TL::off(row, c * TL::EPC);
      CHECK(o / TL::ROWB == row && o % 16 == 0, "%s chunk %d of row %d at %d", name, c, row, o);
      slots.insert(o);
      for (int e = 0; e < TL::EPC; ++e)
        CHECK(TL::off(row, c * TL::EPC + e) == o + e * (int)sizeof(T), "%s element %d", name, e);
    }
    CHECK((int)slots.size() == TL::CPR, "%s row %d chunks collide", name, row);
  }
  if constexpr (!is_bf16<E>()) {
    for (int row0 = 0; row0 < 64; row0 += 32)
      for (int col0 = 0; col0 < D; col0 += 32)
        for (int w = 0; w < 16; ++w) {
          int per_bank[64] = {};
          for (int lane = 0; lane < 64; ++lane) {
            const int h = lane >> 5, n = lane & 31;
            const int addr = TL::off(row0 + rho(w, h), col0 + n);
            ++per_bank[(addr / 4) % 64];
            if constexpr (KS) {
              const int sw = TL::CPR >= 16 ? 8 * h : 0;
              CHECK(TL::swz(row0 + rho(w, h)) == sw, "%s k-slot swizzle w %d h %d", name, w, h);
              const int base = (row0 + 8 * h) * TL::ROWB +
                               ((((col0 >> 2) ^ sw) + (n >> 2)) << 4) + (n & 3) * 4;
              CHECK(addr == base + rho(w, 0) * TL::ROWB, "%s k-slot base w %d lane %d", name, w,
                    lane);
            }
          }
          for (int b = 0; b < 64; ++b)
            CHECK(per_bank[b] <= (D >= 64 ? 1 : 2), "%s bank %d read %d times (w %d col0 %d)",
                  name, b, per_bank[b], w, col0);
        }
  }
  std::printf("tile %-24s ok\n", name);
}

template <class E, int D, int BT, int NW, bool KS1>
static void check_stage(const char* name) {
  using LD = StageLoader<E, D, BT, NW, KS1>;
  using TL = typename LD::TL;
  for (int w = 0; w < NW; ++w)
    for (int lane = 0; lane < 64; ++lane)
      for (int i = 0; i < LD::NLOADS; ++i) {
        const int slot = i * NW + w;
        int mat, src_row, lchunk;
        if constexpr (LD::FAST) {
          // lane_offset(w, lane, mat): the lane's row in the wave's first
          // load and its logical chunk, kept for every load of the matrix
          mat = LD::SPM % NW == 0 ? i * NW / LD::SPM : (i * NW + w) / LD::SPM;
          CHECK(mat == slot / LD::SPM, "%s matrix of load %d wave %d", name, i, w);
          const int lrow = w * LD::RPS + lane / TL::CPR;
          lchunk = (lane % TL::CPR) ^ LD::swz(mat, lrow);
          src_row = i * LD::RS - mat * BT + lrow;
        } else {
          // the per-lane form
          const int chunk = slot * 64 + lane;
          mat = chunk / LD::CH_PER;
          const int pc = chunk - mat * LD::CH_PER;
          src_row = pc / TL::CPR;
          lchunk = (pc % TL::CPR) ^ LD::swz(mat, src_row);
        }
        const int dst = slot * 1024 + lane * 16 - mat * BT * TL::ROWB;
        const int placed = mat == 0 ? Tile<E, D>::off(src_row, lchunk * TL::EPC)
                                    : Tile<E, D, KS1>::off(src_row, lchunk * TL::EPC);
        CHECK(mat >= 0 && mat < 2 && src_row >= 0 && src_row < BT && placed == dst,
              "%s load %d wave %d lane %d matrix %d: row %d chunk %d placed at %d, lands at %d",
              name, i, w, lane, mat, src_row, lchunk, placed, dst);
      }
  std::printf("stage %-23s ok%s\n", name, LD::FAST ? "" : " (per-lane form)");
}

int main() {
  check_tile<EF32, 32, false>("f32 D32");
  check_tile<EF32, 64, false>("f32 D64");
  check_tile<EF32, 128, false>("f32 D128");
  check_tile<EF32, 32, true>("f32 D32 k-slot");
  check_tile<EF32, 64, true>("f32 D64 k-slot");
  check_tile<EF32, 128, true>("f32 D128 k-slot");
  check_tile<EF32B, 64, true>("f32b D64 k-slot");
  check_tile<EF32B, 128, true>("f32b D128 k-slot");
  check_tile<EBF16, 32, false>("bf16 D32");
  check_tile<EBF16, 64, false>("bf16 D64");
  check_tile<EBF16, 128, false>("bf16 D128");
  check_tile<EBF16, 64, true>("bf16 D64 (k-slot ignored)");
  // the forward's stage (K, then V in the k-slot layout) and the backward's
  check_stage<EF32, 32, 64, 4, true>("fwd f32 D32");
  check_stage<EF32, 64, 64, 4, true>("fwd f32 D64");
  check_stage<EF32, 128, 64, 4, true>("fwd f32 D128");
  check_stage<EF32B, 64, 64, 4, true>("fwd f32b D64");
  check_stage<EBF16, 64, 64, 4, true>("fwd bf16 D64");
  check_stage<EBF16, 128, 64, 4, true>("fwd bf16 D128");
  check_stage<EF32, 64, 64, 4, false>("bwd f32 D64");
  check_stage<EBF16, 64, 64, 4, false>("bwd bf16 D64");
  if (g_fail) return 1;
  std::printf("OK\n");
  return 0;
}
