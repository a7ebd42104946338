// Host placement logic of the tiers (see plan.hpp).  No HIP in this file.
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <functional>

namespace tkvd {

int64_t floor_ratio(double r, int64_t n) { return (int64_t)std::floor(r * (double)n); }

std::vector<uint8_t> first_placement(int n, int prompt, int sinks, int recent, double hbm, bool no_t1) {
  std::vector<uint8_t> tier(n, TKV_T1);
  int64_t np = 0;
  for (int i = 0; i < n; ++i)
    if (protected_at(i, n, prompt, sinks, recent)) {
      tier[i] = TKV_T0;
      ++np;
    }
  const int64_t ncand = n - np;
  int64_t room = std::min<int64_t>(ncand, std::max<int64_t>(0, floor_ratio(hbm, n) - np));
  for (int i = 0; i < n && room > 0; ++i)
    if (tier[i] == TKV_T1) {
      tier[i] = TKV_T0;
      --room;
    }
  if (no_t1)
    for (auto& x : tier)
      if (x == TKV_T1) x = TKV_T3;
  return tier;
}

CutCounts cut_counts(int64_t n, int64_t np, int64_t nev, double hbm, double evict, double t2, bool no_t1) {
  const int64_t ncand = n - np - nev;
  CutCounts c{};
  if (no_t1) {
    c.n0c = std::min<int64_t>(ncand, std::max<int64_t>(0, floor_ratio(hbm, n) - np));
    c.n2 = std::min<int64_t>(ncand - c.n0c, floor_ratio(t2, n));
    c.n3 = ncand - c.n0c - c.n2;
    return c;
  }
  c.n3 = std::min<int64_t>(ncand, std::max<int64_t>(0, floor_ratio(evict, n) - nev));
  c.n0c = std::min<int64_t>(ncand - c.n3, std::max<int64_t>(0, floor_ratio(hbm, n) - np));
  c.n2 = std::min<int64_t>(ncand - c.n3 - c.n0c, floor_ratio(t2, n));
  return c;
}

void compact(std::vector<int32_t>& own, const std::vector<char>& vac, uint32_t* m,
             std::vector<std::pair<uint32_t, uint32_t>>* moves) {
  const uint32_t n = (uint32_t)own.size();
  uint32_t kept = 0;
  for (uint32_t i = 0; i < n; ++i) kept += vac[i] ? 0 : 1;
  std::vector<uint32_t> holes, srcs;
  for (uint32_t i = 0; i < kept; ++i)
    if (vac[i]) holes.push_back(i);
  for (uint32_t i = kept; i < n; ++i)
    if (!vac[i]) srcs.push_back(i);
  for (size_t k = 0; k < holes.size(); ++k) {
    moves->emplace_back(srcs[k], holes[k]);
    own[holes[k]] = own[srcs[k]];
  }
  own.resize(kept);
  *m = kept;
}

int make_plan(const PlanConfig& cfg, PlanState& st, const int32_t* counts, const tkv_delta* promote,
              const tkv_delta* demote, PlanResult* out, std::string* err) {
  const int B = cfg.batch, n = cfg.n;
  const size_t nmax = (size_t)cfg.nmax;
  const uint32_t c1 = (uint32_t)cfg.cap0, c2 = (uint32_t)(cfg.cap0 + cfg.cap1);
  auto free_list = [&](int b) -> std::vector<int32_t>& { return (*st.free0)[cfg.shared ? 0 : b]; };
  PlanResult& r = *out;
  r = PlanResult{};
  r.seq.resize(B);
  std::vector<std::vector<char>> vac1s(B), vac2s(B);
  // pass 1: who leaves which place; every freed T0 slot goes back to its free
  // list before any promotion takes one (the lists are shared by the batch
  // when the HBM budget is)
  for (int b = 0; b < B; ++b) {
    SeqPlan& sp = r.seq[b];
    uint8_t* tr = &(*st.tier)[b * nmax];
    uint32_t* lc = &(*st.loc)[b * nmax];
    auto& vac1 = vac1s[b];
    auto& vac2 = vac2s[b];
    vac1.assign((*st.own1)[b].size(), 0);
    vac2.assign((*st.own2)[b].size(), 0);
    std::vector<uint32_t> freed;
    uint32_t* ai = cfg.positional ? &(*st.aidx)[b * nmax] : nullptr;
    auto source = [&](uint32_t pos, uint8_t old) -> Move {
      if (cfg.positional) {
        // the row's values are at its own slot whatever its tier; a T1/T2
        // row's departure leaves a hole in its arena
        if (old == TKV_T1) vac1[ai[pos]] = 1;
        if (old == TKV_T2) vac2[ai[pos]] = 1;
        return {pos, kFromPool, pos};
      }
      if (old == TKV_T0) return {pos, kFromPool, lc[pos]};
      if (old == TKV_T1) {
        vac1[lc[pos] - c1] = 1;
        return {pos, kFromT1, lc[pos] - c1};
      }
      vac2[lc[pos] - c2] = 1;
      return {pos, kFromT2, lc[pos] - c2};
    };
    auto take = [&](const tkv_delta* list, int count) {
      for (int k = 0; k < count; ++k) {
        const tkv_delta& d = list[k];
        const Move mv = source(d.pos, d.old_tier);
        if (d.old_tier == TKV_T0 && !cfg.positional) freed.push_back(mv.idx);
        switch (d.new_tier) {
          case TKV_T0: sp.promo.push_back(mv); break;
          case TKV_T1: sp.ent1.push_back(mv); break;
          case TKV_T2: sp.ent2.push_back(mv); break;
          default:
            lc[d.pos] = kNoLoc;
            r.upd.push_back({b, d.pos, kNoLoc});
            ++r.evictions;
        }
        tr[d.pos] = d.new_tier;
      }
    };
    const int cp = counts[2 * b], cd = counts[2 * b + 1];
    take(demote + b * nmax, cd);
    take(promote + b * nmax, cp);
    r.promotions += cp;
    r.demotions += cd;
    auto by_pos = [](const Move& x, const Move& y) { return x.pos < y.pos; };
    std::sort(sp.ent1.begin(), sp.ent1.end(), by_pos);
    std::sort(sp.ent2.begin(), sp.ent2.end(), by_pos);
    for (auto it = freed.rbegin(); it != freed.rend(); ++it) free_list(b).push_back((int32_t)*it);
  }
  // pass 2: promotions take T0 slots; arenas compact and take their entrants
  for (int b = 0; b < B; ++b) {
    SeqPlan& sp = r.seq[b];
    uint8_t* tr = &(*st.tier)[b * nmax];
    uint32_t* lc = &(*st.loc)[b * nmax];
    auto& own1 = (*st.own1)[b];
    auto& own2 = (*st.own2)[b];
    if (cfg.positional) sp.promo.clear();  // promoted rows stay where they are
    for (const Move& mv : sp.promo) {
      if (free_list(b).empty()) {
        *err = "T0 pool full while promoting";
        return TKV_ECAPACITY;
      }
      const uint32_t slot = (uint32_t)free_list(b).back();
      free_list(b).pop_back();
      sp.promo_slot.push_back(slot);
      lc[mv.pos] = slot;
      r.upd.push_back({b, mv.pos, slot});
    }
    uint32_t* ai = cfg.positional ? &(*st.aidx)[b * nmax] : nullptr;
    if (cfg.positional) {
      // arenas nothing reads on the decode path: vacated indices are freed
      // and the entrants take the lowest free ones, then new ones
      auto place = [&](std::vector<int32_t>& own, std::vector<int32_t>& fr, const std::vector<char>& vac,
                       const std::vector<Move>& ent, std::vector<uint32_t>& dst, int cap) -> bool {
        for (size_t i = 0; i < vac.size(); ++i)
          if (vac[i]) {
            own[i] = -1;
            fr.push_back((int32_t)i);
          }
        std::sort(fr.begin(), fr.end(), std::greater<int32_t>());
        for (const Move& mv : ent) {
          uint32_t idx;
          if (!fr.empty()) {
            idx = (uint32_t)fr.back();
            fr.pop_back();
            own[idx] = (int32_t)mv.pos;
          } else {
            if (own.size() >= (size_t)cap) return false;
            idx = (uint32_t)own.size();
            own.push_back((int32_t)mv.pos);
          }
          dst.push_back(idx);
          ai[mv.pos] = idx;
        }
        return true;
      };
      if (!place(own1, (*st.free1)[b], vac1s[b], sp.ent1, sp.dst1, cfg.cap1)) {
        *err = "T1 arena full";
        return TKV_ECAPACITY;
      }
      if (!place(own2, (*st.free2)[b], vac2s[b], sp.ent2, sp.dst2, cfg.cap2)) {
        *err = "T2 arena full";
        return TKV_ECAPACITY;
      }
      sp.e1off = r.e1;
      sp.e2off = r.e2;
      sp.poff = r.p;
      r.e1 += (int64_t)sp.ent1.size();
      r.e2 += (int64_t)sp.ent2.size();
      int32_t evicted_b = 0;
      for (int p = 0; p < n; ++p) evicted_b += tr[p] == TKV_T3 ? 1 : 0;
      (*st.nlive)[b] = n - evicted_b;
      continue;
    }
    // dense arenas: compaction, then the entrants at the end
    compact(own1, vac1s[b], &sp.m1, &sp.mov1);
    compact(own2, vac2s[b], &sp.m2, &sp.mov2);
    for (auto& mv : sp.mov1) {
      lc[own1[mv.second]] = c1 + mv.second;
      r.upd.push_back({b, (uint32_t)own1[mv.second], c1 + mv.second});
    }
    for (auto& mv : sp.mov2) {
      lc[own2[mv.second]] = c2 + mv.second;
      r.upd.push_back({b, (uint32_t)own2[mv.second], c2 + mv.second});
    }
    if (sp.m1 + sp.ent1.size() > (size_t)cfg.cap1) {
      *err = "T1 arena full";
      return TKV_ECAPACITY;
    }
    if (sp.m2 + sp.ent2.size() > (size_t)cfg.cap2) {
      *err = "T2 arena full";
      return TKV_ECAPACITY;
    }
    for (size_t e = 0; e < sp.ent1.size(); ++e) {
      own1.push_back((int32_t)sp.ent1[e].pos);
      sp.dst1.push_back(sp.m1 + (uint32_t)e);
      lc[sp.ent1[e].pos] = c1 + sp.m1 + (uint32_t)e;
      r.upd.push_back({b, sp.ent1[e].pos, c1 + sp.m1 + (uint32_t)e});
    }
    for (size_t e = 0; e < sp.ent2.size(); ++e) {
      own2.push_back((int32_t)sp.ent2[e].pos);
      sp.dst2.push_back(sp.m2 + (uint32_t)e);
      lc[sp.ent2[e].pos] = c2 + sp.m2 + (uint32_t)e;
      r.upd.push_back({b, sp.ent2[e].pos, c2 + sp.m2 + (uint32_t)e});
    }
    sp.e1off = r.e1;
    sp.e2off = r.e2;
    sp.poff = r.p;
    r.e1 += (int64_t)sp.ent1.size();
    r.e2 += (int64_t)sp.ent2.size();
    r.p += (int64_t)sp.promo.size();
    int32_t evicted_b = 0;
    for (int p = 0; p < n; ++p) evicted_b += tr[p] == TKV_T3 ? 1 : 0;
    (*st.nlive)[b] = n - evicted_b;
  }
  return TKV_OK;
}

}  // namespace tkvd
