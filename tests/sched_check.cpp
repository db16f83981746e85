// Host check of the static schedule of the persistent kernels (build_sched):
// every item exactly once, each head's items on one XCD, slots ordered by
// decreasing work, the per-CU load bound, and the decode that sched_item
// applies on the device.  Test infrastructure; prints one line per case and
// exits non-zero on the first violation.
#include "attn_launch.hpp"

#include <cstdio>
#include <vector>

using attn::Sched;

static int decode(const Sched& s, int r, int g, int BH) {  // sched_item with a table
  if (r >= s.R) return -1;
  const int e = r == 0 ? s.first[g >> 3] : s.ent[(r - 1) * s.M + (g >> 3)];
  if (e == 0xffff) return -1;
  return (e >> 8) * BH + 8 * (e & 255) + (g & 7);
}

int main() {
  struct Case { int G, BH, n, cux; bool causal; long cu_bound; };
  const Case cases[] = {
      {512, 96, 8, 32, true, 14},    // decoder step: 2 workgroups per CU, ideal 13.5
      {512, 96, 8, 32, false, 24},   // non-causal, equal items
      {256, 16, 16, 32, true, 16},   // long context: one workgroup per CU, largest item 16
      {768, 256, 4, 32, false, 16},  // ragged encoder, 3 per CU, ideal 16
      {64, 8, 8, 32, true, 8},       // fewer workgroups than CUs
      {1024, 96, 8, 32, true, 14},   // 4 per CU
      {512, 8, 1, 32, false, 1},     // one item per head
  };
  for (const Case& c : cases) {
    std::vector<int> works(c.n);
    for (int k = 0; k < c.n; ++k) works[k] = c.causal ? c.n - k : c.n;
    const Sched s = attn::build_sched(c.G, c.BH, works, c.cux);
    if (s.M != c.G / 8) { printf("FAIL G=%d BH=%d: no pattern\n", c.G, c.BH); return 1; }
    const int nitems = c.BH * c.n, M = s.M;
    const int cux = M % c.cux ? M : c.cux;
    std::vector<int> seen(nitems, 0);
    std::vector<long> cu_load(8 * cux, 0);
    for (int g = 0; g < c.G; ++g) {
      int prev_work = 1 << 30;
      for (int r = 0;; ++r) {
        const int it = decode(s, r, g, c.BH);
        if (it < 0) break;
        if (it >= nitems) { printf("FAIL item %d out of range\n", it); return 1; }
        ++seen[it];
        if ((it % c.BH) % 8 != g % 8) { printf("FAIL head %d off its XCD\n", it % c.BH); return 1; }
        const int w = works[it / c.BH];
        if (w > prev_work) { printf("FAIL slot order\n"); return 1; }
        prev_work = w;
        cu_load[(g % 8) * cux + (g / 8) % cux] += w;
      }
    }
    for (int it = 0; it < nitems; ++it)
      if (seen[it] != 1) { printf("FAIL item %d taken %d times\n", it, seen[it]); return 1; }
    long mx = 0;
    for (long l : cu_load) mx = l > mx ? l : mx;
    printf("G=%d BH=%d classes=%d causal=%d: %d items once each, max CU load %ld (bound %ld)\n",
           c.G, c.BH, c.n, (int)c.causal, nitems, mx, c.cu_bound);
    if (mx > c.cu_bound) { printf("FAIL balance\n"); return 1; }
  }
  // shapes outside the pattern fall back (M = 0)
  if (attn::build_sched(512, 12, {8, 7}, 32).M != 0) { printf("FAIL BH %% 8\n"); return 1; }
  if (attn::build_sched(500, 96, {8, 7}, 32).M != 0) { printf("FAIL G %% 8\n"); return 1; }
  printf("OK\n");
  return 0;
}
