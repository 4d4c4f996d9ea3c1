// Host check of the work-group tables the backward's one-launch schedule runs
// on (plan_runs, make_tables and the decode unit_of from the library sources):
// for random sets of runs, every (run, block, batch row * kv head) unit is
// decoded from exactly one work-group of exactly one launch, blocks stay in
// range, launches are cut at kMaxRuns runs and kMaxEnt ranges, and the units
// of a launch go out longest first.  Prints "ok" and exits 0 on success.
#include <climits>
#include <cstdio>
#include <map>
#include <random>
#include <tuple>
#include <vector>

#include "tg_attn.h"

using namespace tg;

static int fail(const char *what, int trial) {
  std::printf("FAIL %s (trial %d)\n", what, trial);
  return 1;
}

int main() {
  std::mt19937 rng(12345);
  long units = 0;
  for (int trial = 0; trial < 1500; ++trial) {
    const int nr = 1 + (int)(rng() % 24), Hkv = 1 << (rng() % 4), G = 1 << (rng() % 3), Hq = Hkv * G;
    std::vector<RunRow> runs;
    int off = 0;
    for (int i = 0; i < nr; ++i) {
      const int n = 1 + (int)(rng() % 4), M = 1 + (int)(rng() % (trial % 3 == 0 ? 6000 : 600));
      runs.push_back(RunRow{off, 0, n, M, 0, 0});
      off += n * M;
    }
    plan_runs(runs.data(), nr, Hq, Hkv, 128);
    // padded offsets: each run's sequences rounded up to 32 tokens
    int64_t pexp = 0;
    for (const RunRow &r : runs) {
      if (r.poff != pexp) return fail("poff", trial);
      pexp += (int64_t)r.n * ((r.M + 31) / 32 * 32);
    }
    const int BQ = 256 / G;
    for (int r0 = 0; r0 < nr; r0 += kMaxRuns) {
      const int cnt = nr - r0 < kMaxRuns ? nr - r0 : kMaxRuns;
      for (int kind = 0; kind < 2; ++kind) {  // query blocks (dq), key blocks (dk, dv)
        std::vector<Level> lv;
        long expect = 0;
        for (int i = 0; i < cnt; ++i) {
          const RunRow &r = runs[r0 + i];
          const int nb = kind == 0 ? (r.M + BQ - 1) / BQ : (r.M + 127) / 128, ntq = (r.M + 31) / 32;
          for (int b = 0; b < nb; ++b) {
            const int qe = (b + 1) * BQ < r.M ? (b + 1) * BQ : r.M;
            const int64_t cost = kind == 0 ? (int64_t)((qe + 31) / 32) + 6 : (int64_t)G * (ntq - 4 * b) + 2;
            lv.push_back(Level{i, b, cost});
          }
          expect += (long)nb * r.n * Hkv;
        }
        std::vector<Level> sorted = lv;
        std::vector<RunTable> tabs;
        std::vector<unsigned> grids;
        make_tables(sorted, runs.data() + r0, cnt, Hkv, tabs, grids);
        std::map<std::tuple<int, int, int>, int> seen;
        std::map<std::pair<int, int>, int64_t> costof;
        for (const Level &L : lv) costof[{L.run, L.blk}] = L.cost;
        long got = 0;
        int64_t prev = INT64_MAX;
        for (size_t t = 0; t < tabs.size(); ++t) {
          int ne = 0;
          while (ne < kMaxEnt && tabs[t].start[ne] != INT_MAX) ++ne;
          if (ne == 0 || tabs[t].start[0] != 0) return fail("first range", trial);
          for (unsigned w = 0; w < grids[t]; ++w) {
            const Unit u = unit_of(tabs[t], (int)w, Hkv);
            if (u.run < 0 || u.run >= cnt) return fail("run index", trial);
            const RunRow &R = tabs[t].run[u.run];
            if (R.M != runs[r0 + u.run].M || R.n != runs[r0 + u.run].n || R.off != runs[r0 + u.run].off)
              return fail("run row", trial);
            const int nb = kind == 0 ? (R.M + BQ - 1) / BQ : (R.M + 127) / 128;
            if (u.blk < 0 || u.blk >= nb || u.bh < 0 || u.bh >= R.n * Hkv) return fail("unit range", trial);
            if (seen[{u.run, u.blk, u.bh}]++) return fail("unit twice", trial);
            const int64_t c = costof[{u.run, u.blk}];
            if (c > prev) return fail("longest first", trial);
            prev = c;
            ++got;
          }
        }
        if (got != expect) return fail("unit count", trial);
        units += got;
      }
    }
  }
  std::printf("ok %ld units\n", units);
  return 0;
}
