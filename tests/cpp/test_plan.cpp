// Unit test of the library's host placement logic (csrc/plan.cpp), built on
// the CPU on its own with AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Part 1 prints the first placement and the tier counts of a grid of cases
// ("Not All Thoughts Need HBM", gist.science summary, Method §1 budgets);
// the Python driver compares them with the oracle's tiering.
// Part 2 checks make_plan on random reassignments (Method §4: only changed
// rows move) by simulating what the plan does to the T0 pool, the arenas
// and the location table, and comparing with the state make_plan leaves.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <string>
#include <vector>

#include "../../decode_attention_tkv_amd/csrc/plan.hpp"

using namespace tkvd;

static int g_fail = 0;
#define CHECK(cond, ...)                                        \
  do {                                                          \
    if (!(cond)) {                                              \
      std::fprintf(stderr, "CHECK failed: %s: ", #cond);        \
      std::fprintf(stderr, __VA_ARGS__);                        \
      std::fprintf(stderr, "\n");                               \
      if (++g_fail > 20) std::exit(1);                          \
    }                                                           \
  } while (0)

static void print_cases() {
  const int ns[] = {1, 7, 12, 40, 301};
  const double hs[] = {0.0, 0.3, 0.5, 0.7, 1.0};
  for (int n : ns)
    for (double h : hs)
      for (int prot = 0; prot < 3; ++prot)
        for (int no_t1 = 0; no_t1 < 2; ++no_t1) {
          const int prompt = prot == 1 ? n / 3 : 0, sinks = prot ? 2 : 0, recent = prot == 2 ? n / 2 : 3;
          const auto t = first_placement(n, prompt, sinks, recent, h, no_t1 != 0);
          std::printf("first %d %d %d %d %.3f %d :", n, prompt, sinks, recent, h, no_t1);
          for (uint8_t x : t) std::printf(" %d", x);
          std::printf("\n");
        }
  for (int n : ns)
    for (int np = 0; np <= n; np += (n / 3 > 0 ? n / 3 : 1))
      for (int nev = 0; nev + np <= n; nev += (n / 4 > 0 ? n / 4 : 1))
        for (double h : hs)
          for (double e : {0.0, 0.03, 0.5})
            for (double t2 : {0.0, 0.2})
              for (int no_t1 = 0; no_t1 < 2; ++no_t1) {
                const CutCounts c = cut_counts(n, np, nev, h, e, t2, no_t1 != 0);
                std::printf("cut %d %d %d %.3f %.3f %.3f %d : %lld %lld %lld\n", n, np, nev, h, e, t2, no_t1,
                            (long long)c.n3, (long long)c.n0c, (long long)c.n2);
              }
}

static void check_compact(std::mt19937& rng) {
  for (int rep = 0; rep < 500; ++rep) {
    const int n = rng() % 40;
    std::vector<int32_t> own(n);
    std::vector<char> vac(n);
    for (int i = 0; i < n; ++i) {
      own[i] = 1000 + i;
      vac[i] = (rng() % 3) == 0;
    }
    const std::vector<int32_t> before = own;
    uint32_t m = 0;
    std::vector<std::pair<uint32_t, uint32_t>> moves;
    compact(own, vac, &m, &moves);
    std::multiset<int32_t> kept, got(own.begin(), own.end());
    for (int i = 0; i < n; ++i)
      if (!vac[i]) kept.insert(before[i]);
    CHECK(m == own.size() && kept == got, "compact keeps exactly the kept rows (n %d)", n);
    std::set<uint32_t> dsts;
    for (auto& mv : moves) {
      CHECK(mv.first >= m && mv.second < m && vac[mv.second] && !vac[mv.first], "move %u -> %u, m %u", mv.first,
            mv.second, m);
      CHECK(dsts.insert(mv.second).second, "destination %u twice", mv.second);
    }
    for (uint32_t i = 0; i < m; ++i)
      if (!vac[i]) CHECK(own[i] == before[i], "kept row %u moved", i);
  }
}

// One random reassignment of a consistent placement, checked against a
// simulation of its moves.
static void check_plan(std::mt19937& rng, bool positional, bool shared) {
  const int B = 1 + rng() % 3, nmax = 64, n = 10 + rng() % 54;
  const int cap1 = nmax, cap2 = nmax;
  const int cap0 = positional ? nmax : (shared ? B * nmax : nmax);
  std::vector<uint8_t> tier((size_t)B * nmax, kUnused);
  std::vector<uint32_t> loc((size_t)B * nmax, kNoLoc), aidx((size_t)B * nmax, kNoLoc);
  std::vector<std::vector<int32_t>> free0(shared ? 1 : B), own1(B), own2(B), free1(B), free2(B);
  std::vector<int32_t> nlive(B);
  // a consistent starting placement with random tiers
  std::vector<std::vector<int32_t>> used(shared ? 1 : B);
  std::vector<int32_t> all;
  for (int i = 0; i < cap0; ++i) all.push_back(i);
  for (auto& f : free0) {
    f = all;
    std::shuffle(f.begin(), f.end(), rng);
  }
  for (int b = 0; b < B; ++b) {
    auto& fl = free0[shared ? 0 : b];
    for (int p = 0; p < n; ++p) {
      const uint8_t x = rng() % 4;
      const size_t at = (size_t)b * nmax + p;
      tier[at] = x;
      if (x == TKV_T3) continue;
      if (positional) {
        loc[at] = p;
        if (x == TKV_T1) aidx[at] = own1[b].size(), own1[b].push_back(p);
        if (x == TKV_T2) aidx[at] = own2[b].size(), own2[b].push_back(p);
      } else if (x == TKV_T0) {
        loc[at] = fl.back();
        fl.pop_back();
      } else if (x == TKV_T1) {
        loc[at] = cap0 + own1[b].size();
        own1[b].push_back(p);
      } else {
        loc[at] = cap0 + cap1 + own2[b].size();
        own2[b].push_back(p);
      }
    }
  }
  // simulated contents: a tag per slot and arena index (the position it holds)
  std::map<std::pair<int, uint32_t>, int32_t> pool;  // (seq or 0, slot) -> position
  std::vector<std::vector<int32_t>> ar1(B), ar2(B);
  for (int b = 0; b < B; ++b) {
    ar1[b] = own1[b];
    ar2[b] = own2[b];
    for (int p = 0; p < n; ++p)
      if (!positional && tier[(size_t)b * nmax + p] == TKV_T0) pool[{shared ? 0 : b, loc[(size_t)b * nmax + p]}] = p;
  }
  // new tiers: T3 stays; others anything
  std::vector<uint8_t> neu(tier);
  std::vector<int32_t> counts(2 * B);
  std::vector<tkv_delta> pro((size_t)B * nmax), dem((size_t)B * nmax);
  for (int b = 0; b < B; ++b) {
    int np = 0, nd = 0;
    for (int p = 0; p < n; ++p) {
      const size_t at = (size_t)b * nmax + p;
      if (tier[at] != TKV_T3 && rng() % 3 == 0) neu[at] = rng() % 4;
      const tkv_delta d{(uint32_t)p, tier[at], neu[at], 0};
      if (neu[at] < tier[at]) pro[(size_t)b * nmax + np++] = d;
      if (neu[at] > tier[at]) dem[(size_t)b * nmax + nd++] = d;
    }
    counts[2 * b] = np;
    counts[2 * b + 1] = nd;
  }
  const std::vector<uint32_t> loc_before = loc, aidx_before = aidx;
  const std::vector<uint8_t> tier_before = tier;
  PlanConfig cfg{B, nmax, n, cap0, cap1, cap2, positional, shared};
  PlanState st{&tier, &loc, &aidx, &free0, &own1, &own2, &free1, &free2, &nlive};
  PlanResult r;
  std::string err;
  const int rc = make_plan(cfg, st, counts.data(), pro.data(), dem.data(), &r, &err);
  CHECK(rc == TKV_OK, "make_plan: %s", err.c_str());
  if (rc) return;
  // the simulated moves: T0 promotions into their slots, arena compaction, entrants
  int64_t e1 = 0, e2 = 0, p0 = 0;
  for (int b = 0; b < B; ++b) {
    const SeqPlan& sp = r.seq[b];
    for (size_t k = 0; k < sp.promo.size(); ++k) pool[{shared ? 0 : b, sp.promo_slot[k]}] = (int32_t)sp.promo[k].pos;
    CHECK(sp.dst1.size() == sp.ent1.size() && sp.dst2.size() == sp.ent2.size(), "entrant destinations");
    if (positional) {
      // rows leaving an arena free their index; entrants land at their destinations
      for (int p = 0; p < n; ++p) {
        const size_t at = (size_t)b * nmax + p;
        if (tier_before[at] == TKV_T1 && neu[at] != TKV_T1) ar1[b][aidx_before[at]] = -1;
        if (tier_before[at] == TKV_T2 && neu[at] != TKV_T2) ar2[b][aidx_before[at]] = -1;
      }
      CHECK(sp.mov1.empty() && sp.mov2.empty(), "positional arenas are not compacted");
    } else {
      for (auto& mv : sp.mov1) ar1[b][mv.second] = ar1[b][mv.first];
      for (auto& mv : sp.mov2) ar2[b][mv.second] = ar2[b][mv.first];
      ar1[b].resize(sp.m1);
      ar2[b].resize(sp.m2);
    }
    for (size_t e = 0; e < sp.ent1.size(); ++e) {
      const uint32_t d = sp.dst1[e];
      CHECK(d < (uint32_t)cap1, "T1 destination past the arena");
      if (d >= ar1[b].size()) ar1[b].resize(d + 1, -1);
      CHECK(ar1[b][d] == -1, "T1 entrant onto a live row (seq %d index %u)", b, d);
      ar1[b][d] = (int32_t)sp.ent1[e].pos;
    }
    for (size_t e = 0; e < sp.ent2.size(); ++e) {
      const uint32_t d = sp.dst2[e];
      CHECK(d < (uint32_t)cap2, "T2 destination past the arena");
      if (d >= ar2[b].size()) ar2[b].resize(d + 1, -1);
      CHECK(ar2[b][d] == -1, "T2 entrant onto a live row (seq %d index %u)", b, d);
      ar2[b][d] = (int32_t)sp.ent2[e].pos;
    }
    CHECK(sp.e1off == e1 && sp.e2off == e2 && sp.poff == p0, "F offsets");
    e1 += sp.ent1.size();
    e2 += sp.ent2.size();
    p0 += sp.promo.size();
    if (positional) CHECK(sp.promo.empty(), "positional staging moves no promoted row");
  }
  CHECK(r.e1 == e1 && r.e2 == e2 && r.p == p0, "totals");
  // the location table: the updates applied to the old one give the new one
  std::vector<uint32_t> applied = loc_before;
  for (auto& u : r.upd) applied[(size_t)u.b * nmax + u.pos] = u.code;
  for (int b = 0; b < B; ++b) {
    int live = 0;
    CHECK(ar1[b] == own1[b] && ar2[b] == own2[b], "simulated arenas equal the owners (seq %d)", b);
    if (positional) {  // every live T1/T2 row owns exactly one index; the rest are free, each listed once
      for (int w = 0; w < 2; ++w) {
        const auto& own = w ? own2[b] : own1[b];
        const auto& fr = w ? free2[b] : free1[b];
        std::set<int32_t> fs(fr.begin(), fr.end());
        CHECK(fs.size() == fr.size(), "free index twice");
        int holes = 0, rows = 0;
        for (size_t i = 0; i < own.size(); ++i) {
          if (own[i] < 0) {
            ++holes;
            CHECK(fs.count((int32_t)i) == 1, "free index not listed");
          } else {
            ++rows;
            CHECK(neu[(size_t)b * nmax + own[i]] == (w ? TKV_T2 : TKV_T1), "arena row of another tier");
          }
        }
        int in_tier = 0;
        for (int p = 0; p < n; ++p) in_tier += neu[(size_t)b * nmax + p] == (w ? TKV_T2 : TKV_T1);
        CHECK(holes == (int)fr.size() && rows == in_tier, "arena rows %d vs tier %d", rows, in_tier);
      }
    }
    for (int p = 0; p < n; ++p) {
      const size_t at = (size_t)b * nmax + p;
      CHECK(tier[at] == neu[at], "tier mirror");
      live += neu[at] != TKV_T3;
      if (neu[at] == TKV_T3) {
        CHECK(loc[at] == kNoLoc, "evicted row keeps a location");
        continue;
      }
      if (positional) {
        CHECK(loc[at] == (uint32_t)p, "positional location");
        if (neu[at] == TKV_T1) CHECK(own1[b][aidx[at]] == p, "T1 arena index");
        if (neu[at] == TKV_T2) CHECK(own2[b][aidx[at]] == p, "T2 arena index");
        continue;
      }
      CHECK(applied[at] == loc[at], "location updates (seq %d pos %d)", b, p);
      if (neu[at] == TKV_T0) {
        auto it = pool.find({shared ? 0 : b, loc[at]});
        CHECK(it != pool.end() && it->second == p, "T0 slot holds its row (seq %d pos %d)", b, p);
      } else if (neu[at] == TKV_T1) {
        CHECK(loc[at] >= (uint32_t)cap0 && own1[b][loc[at] - cap0] == p, "T1 location");
      } else {
        CHECK(loc[at] >= (uint32_t)(cap0 + cap1) && own2[b][loc[at] - cap0 - cap1] == p, "T2 location");
      }
    }
    CHECK(nlive[b] == live, "live rows");
  }
  if (!positional) {  // free slots and T0 slots partition each slot space
    for (size_t q = 0; q < free0.size(); ++q) {
      std::set<int32_t> seen(free0[q].begin(), free0[q].end());
      CHECK(seen.size() == free0[q].size(), "free slot twice");
      for (int b = 0; b < B; ++b) {
        if (!shared && (size_t)b != q) continue;
        for (int p = 0; p < n; ++p)
          if (neu[(size_t)b * nmax + p] == TKV_T0) CHECK(seen.insert((int32_t)loc[(size_t)b * nmax + p]).second, "slot twice");
      }
      CHECK((int)seen.size() == cap0, "slots lost: %zu of %d", seen.size(), cap0);
    }
  }
}

int main(int argc, char** argv) {
  if (argc > 1 && std::string(argv[1]) == "cases") {
    print_cases();
    return 0;
  }
  std::mt19937 rng(12345);
  check_compact(rng);
  for (int rep = 0; rep < 400; ++rep) check_plan(rng, rep % 3 == 0, rep % 3 == 2);
  std::printf("plan checks: %d failures\n", g_fail);
  return g_fail ? 1 : 0;
}
