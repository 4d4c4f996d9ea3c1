// Host check of the work-group tables the one-launch schedules over packed
// runs run on (plan_runs, make_tables, make_fwd_tables and the backward's
// decode unit_of from the library sources).  Backward: for random sets of
// runs, every (run, block, batch row * kv head) unit is decoded from exactly
// one work-group of exactly one launch, blocks stay in range, launches are cut
// at kMaxRuns runs and kMaxEnt ranges, and the units of a launch go out
// longest first.  Forward: the tables decoded as their layout states (ranges
// down one run's blocks with all their pieces, or across runs at one block)
// give every (run, block, piece, batch row * kv head) exactly once, pieces of
// split blocks get distinct record slots numbered from the run's top block,
// the runs of a group share one C, and split blocks go out first, then the
// rest longest first.  Prints "ok" and exits 0 on success.
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

// The forward's pieces: block qb of a run of length M holds ceil(min((qb+1) BQ, M) / 32)
// key tiles, cut into ceil(tiles / C) pieces.
static int ntiles(int qb, int BQ, int M) {
  const int qe = (qb + 1) * BQ < M ? (qb + 1) * BQ : M;
  return (qe + 31) / 32;
}
static int npieces(int nt, int C) { return (nt + C - 1) / C; }

static int check_fwd(const RunRow *runs, int cnt, int Hq, int Hkv, int trial, long &units) {
  const int BQ = 256 / (Hq / Hkv), C = runs[0].C;
  for (int i = 0; i < cnt; ++i)
    if (runs[i].C != C || C < 8) return fail("fwd: one C per group", trial);
  if (cnt == 1 && fwd_sched(runs[0].n, runs[0].M, Hq, Hkv).C != C) return fail("fwd: C of one run", trial);
  std::vector<RunTable> tabs;
  std::vector<unsigned> grids;
  if (!make_fwd_tables(runs, cnt, Hq, Hkv, tabs, grids)) return fail("fwd: make_fwd_tables", trial);
  std::map<std::tuple<int, int, int, int>, int> seen;
  std::map<std::tuple<int, int, int>, int> recs;
  long got = 0, expect = 0;
  for (int i = 0; i < cnt; ++i)
    for (int qb = 0; qb * BQ < runs[i].M; ++qb)
      expect += (long)npieces(ntiles(qb, BQ, runs[i].M), C) * runs[i].n * Hkv;
  bool in_split = true;
  int prev_cost = INT_MAX;
  for (size_t t = 0; t < tabs.size(); ++t) {
    const RunTable &T = tabs[t];
    if (T.start[0] != 0) return fail("fwd: first range", trial);
    for (unsigned w = 0; w < grids[t]; ++w) {
      int e = 0;
      while (e + 1 < kMaxEnt && T.start[e + 1] <= (int)w) ++e;
      const unsigned code = (unsigned)T.code[e];
      int ri = code & 0xFF, loc = (int)w - T.start[e];
      const int blk0 = (code >> 8) & 0x3FFFFF;
      int qb = blk0, p = 0, np = 1, pfirst = 0, bh;
      if ((code >> 30) & 1) {
        while (ri < cnt && loc >= T.run[ri].n * Hkv) loc -= T.run[ri++].n * Hkv;
        if (ri >= cnt) return fail("fwd: across range past the runs", trial);
        bh = loc;
        if (npieces(ntiles(qb, BQ, T.run[ri].M), C) != 1) return fail("fwd: split block in an across range", trial);
      } else {
        const int nbh = T.run[ri].n * Hkv;
        bh = loc % nbh;
        int rem = loc / nbh, base = 0;
        for (qb = blk0; qb >= 0; --qb) {
          np = npieces(ntiles(qb, BQ, T.run[ri].M), C);
          if (rem < np) break;
          rem -= np;
          base += np;
        }
        if (qb < 0) return fail("fwd: range past block 0", trial);
        p = rem;
        pfirst = base;
      }
      if (ri >= cnt) return fail("fwd: run index", trial);
      const RunRow &R = runs[ri];
      if (T.run[ri].off != R.off || T.run[ri].M != R.M || T.run[ri].n != R.n || T.run[ri].C != C)
        return fail("fwd: run row", trial);
      const int nqb = (R.M + BQ - 1) / BQ;
      if (qb >= nqb || bh < 0 || bh >= R.n * Hkv) return fail("fwd: unit range", trial);
      if (seen[{ri, qb, p, bh}]++) return fail("fwd: unit twice", trial);
      const int nt = ntiles(qb, BQ, R.M);
      if (npieces(nt, C) != np) return fail("fwd: pieces", trial);
      if (np > 1) {
        int above = 0;
        for (int q = nqb - 1; q > qb; --q) above += npieces(ntiles(q, BQ, R.M), C);
        if (pfirst != above) return fail("fwd: record slots from the top block", trial);
        const FwdSched f = fwd_sched_c(R.n, R.M, Hq, Hkv, C);
        if (pfirst + p >= f.nmulti) return fail("fwd: record slot range", trial);
        if (recs[{ri, pfirst + p, bh}]++) return fail("fwd: record slot twice", trial);
        if (!in_split) return fail("fwd: split blocks first", trial);
      } else {
        if (in_split) in_split = false;
        if (nt > prev_cost) return fail("fwd: longest first", trial);
        prev_cost = nt;
      }
      ++got;
    }
  }
  if (got != expect) return fail("fwd: unit count", trial);
  units += got;
  return 0;
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
      runs.push_back(RunRow{off, 0, n, M, 0, 0, 0});
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
      if (check_fwd(runs.data() + r0, cnt, Hq, Hkv, trial, units)) return 1;
    }
  }
  std::printf("ok %ld units\n", units);
  return 0;
}
