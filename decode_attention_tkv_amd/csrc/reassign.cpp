// tkv_reassign: score-ranked re-placement of every sequence's rows
// ("Not All Thoughts Need HBM", gist.science technical summary, Method §1
// four tiers and §4 periodic reassignment where only changed rows move).
//
// Device: rank + label (radix select on the GPU's fp32 scores) and the
// changed-row lists (prefix-scan compaction).  Host: one synchronisation to
// read the lists, then a placement plan per sequence:
//   * the T1 and T2 arenas of a sequence stay dense: rows that leave leave
//     holes, the last remaining rows move into the holes, rows that enter are
//     appended (one contiguous block per layer and kv head);
//   * T0 slots freed by demotions are reused by promotions.
// Data movement:
//   phase 1   every moved row's value lands in the fetch pack F (from the T0
//             pool, the resident staging, or -- stream mode -- the pinned
//             arenas, 8-bit rows dequantised on the GPU);
//   phase 2a  promotions F -> T0 slots; compaction moves inside the staging;
//   phase 2b  rows entering T1: F -> staging; rows entering T2: quantised
//             from F on the GPU (codes + scale out, dequantised values into
//             the staging).
// Positional resident staging (every live row at its own position in the
// pool) moves no row inside HBM: phase 1 gathers only the rows entering T1
// or T2, for their write-back, and T2 entrants get their dequantised values
// in their own slots; phases 2a and 2b are empty.  T1/T2 rows keep a
// host-side arena index per position.
// Rows entering T1/T2 reach their pinned home through one write-back copy per
// pack on a stream of their own; a host job (never waited for by the GPU)
// compacts the arenas and files them.  Every area is head-major.
#include <algorithm>
#include <chrono>
#include <cstring>
#include <memory>
#include <thread>

#include "handle.hpp"
#include "host_util.hpp"

using namespace tkvd;

namespace {

// Largest changed-row block read back whole (one copy, one wait); a few tens
// of microseconds over PCIe, about one synchronisation round trip.
constexpr size_t kOneCopyDeltaBytes = 1u << 20;

enum SrcKind : uint8_t { kFromPool, kFromT1, kFromT2 };

struct Move {
  uint32_t pos;
  SrcKind kind;
  uint32_t idx;  // pool slot, T1 index or T2 index
};

struct SeqPlan {
  std::vector<Move> ent1, ent2, promo;  // rows entering T1, T2 and T0
  std::vector<uint32_t> promo_slot;
  std::vector<std::pair<uint32_t, uint32_t>> mov1, mov2;  // arena (src, dst)
  uint32_t m1 = 0, m2 = 0;              // arena rows kept before the entrants
  int64_t e1off = 0, e2off = 0, poff = 0;  // offsets within the F segments
};

int grow_device(tkv* t, void** p, size_t* cap, size_t need) {
  if (need <= *cap) return TKV_OK;
  if (*p) HIP_TRY(t, hipFree(*p));
  *p = nullptr;
  *cap = 0;
  const size_t bytes = std::max(need, (size_t)4096) * 2;
  HIP_TRY(t, hipMalloc(p, bytes));
  *cap = bytes;
  return TKV_OK;
}

int grow_pinned(tkv* t, void** p, size_t* cap, size_t need) {
  if (need <= *cap) return TKV_OK;
  if (*p) HIP_TRY(t, hipHostFree(*p));
  *p = nullptr;
  *cap = 0;
  const size_t bytes = std::max(need, (size_t)4096) * 2;
  HIP_TRY(t, hipHostMalloc(p, bytes, hipHostMallocDefault));
  *cap = bytes;
  return TKV_OK;
}

// Dense-arena compaction: indices marked vacated leave; the kept rows above
// the new size m move down into the holes below it, in order.
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

}  // namespace

// Batch-shared HBM budget: how many candidates of each sequence the joint
// ranking puts in T0.  Per sequence the n3 lowest-ranked candidates are set
// aside (eviction keeps its own budget); the rest of the batch is ranked by
// (fp32 score descending, sequence ascending, position ascending) -- the
// kernel's keys, extended by the sequence -- and the best
// min(remaining, B * floor(hN) - sum |P|) go to T0.  T2 then takes its own
// budget from what each sequence has left.
static int shared_t0_counts(tkv* t, hipStream_t st, const std::vector<int64_t>& ncand, const std::vector<int64_t>& nprot,
                     std::vector<CutCounts>* cuts) {
  const int B = t->B, n = t->n;
  const size_t nmax = t->nmax;
  std::vector<float> s((size_t)B * nmax);
  HIP_TRY(t, hipMemcpyAsync(s.data(), t->s, s.size() * 4, hipMemcpyDeviceToHost, st));
  HIP_TRY(t, hipStreamSynchronize(st));
  struct Key {
    uint32_t bits;  // fp32 score bits: scores are >= 0, so the bits order as the values
    int32_t b, pos;
  };
  auto better = [](const Key& x, const Key& y) {
    if (x.bits != y.bits) return x.bits > y.bits;
    if (x.b != y.b) return x.b < y.b;
    return x.pos < y.pos;
  };
  std::vector<Key> remaining;
  int64_t budget = 0;
  for (int b = 0; b < B; ++b) {
    std::vector<Key> cand;
    cand.reserve(ncand[b]);
    for (int p = 0; p < n; ++p) {
      const uint8_t x = t->h_tier[(size_t)b * nmax + p];
      if (x == TKV_T3 || is_protected(*t, p, n)) continue;
      uint32_t bits;
      std::memcpy(&bits, &s[(size_t)b * nmax + p], 4);
      cand.push_back({bits, b, p});
    }
    std::sort(cand.begin(), cand.end(), better);
    cand.resize(cand.size() - (size_t)(*cuts)[b].n3);  // the lowest n3 are evicted
    remaining.insert(remaining.end(), cand.begin(), cand.end());
    budget += floor_ratio(t->hbm, n) - nprot[b];
  }
  const int64_t take = std::min<int64_t>((int64_t)remaining.size(), std::max<int64_t>(0, budget));
  std::vector<int64_t> n0c(B, 0);
  if (take > 0) {
    std::nth_element(remaining.begin(), remaining.begin() + (take - 1), remaining.end(), better);
    const Key last = remaining[take - 1];
    for (const Key& k : remaining)
      if (!better(last, k)) n0c[k.b] += 1;  // k is at least as good as the last one taken
  }
  for (int b = 0; b < B; ++b) {
    CutCounts& c = (*cuts)[b];
    c.n0c = n0c[b];
    c.n2 = std::min<int64_t>(ncand[b] - c.n3 - c.n0c, floor_ratio(t->t2, n));
  }
  return TKV_OK;
}

static int reassign_impl(tkv_t* t, tkv_stream_t stream) {
  if (!t) return tkv_fail(nullptr, TKV_EINVAL, "handle is NULL");
  if (t->state == TkvState::InStep) return tkv_fail(t, TKV_ESTATE, "reassign between the layer groups of a step");
  if (t->n == 0) return TKV_OK;
  const auto wall0 = std::chrono::steady_clock::now();
  hipStream_t st = (hipStream_t)stream;
  if (int rc = tkv_flush_score(t, st)) return rc;  // ranking reads s
  const int B = t->B, L = t->L, n = t->n, H = t->Hkv, D = t->D;
  const size_t nmax = t->nmax;
  const size_t hb = (size_t)D * t->esz;  // bytes of one head's row
  // The host arenas and the pinned packs may still be in use by the previous
  // reassignment's host job and copies.
  if (t->arena_job.valid()) {
    const int rc = t->arena_job.get();
    if (rc) return tkv_fail(t, rc, "host arena work of the last reassignment failed");
  }
  HIP_TRY(t, hipStreamSynchronize(t->side));
  if (t->side_v) HIP_TRY(t, hipStreamSynchronize(t->side_v));
  HIP_TRY(t, hipEventSynchronize(t->ev_arena));

  // ---- cut points from the host mirror of the tiers
  RankArgs ra{};
  ra.s = t->s;
  ra.tier_old = t->tier;
  ra.tier_new = t->tier_alt;
  ra.nmax = t->nmax;
  ra.n = n;
  ra.prompt = t->prompt;
  ra.sinks = t->sinks;
  ra.recent = t->recent;
  std::vector<CutCounts> cuts(B);
  std::vector<int64_t> ncands(B), nprots(B);
  for (int b = 0; b < B; ++b) {
    int64_t np = 0, nev = 0;
    const uint8_t* tr = &t->h_tier[b * nmax];
    for (int p = 0; p < n; ++p) {
      if (tr[p] == TKV_T3)
        ++nev;
      else if (is_protected(*t, p, n))
        ++np;
    }
    ncands[b] = n - np - nev;
    nprots[b] = np;
    cuts[b] = cut_counts(*t, n, np, nev);
  }
  if (t->shared_hbm) {
    int rc = shared_t0_counts(t, st, ncands, nprots, &cuts);
    if (rc) return rc;
  }
  for (int b = 0; b < B; ++b) {
    const int64_t ncand = ncands[b], n3 = cuts[b].n3, n0c = cuts[b].n0c, n2 = cuts[b].n2;
    ra.ncand[b] = (int32_t)ncand;
    ra.rank[b][0] = (int32_t)n3;
    ra.rank[b][1] = (int32_t)(n3 + n2);
    ra.rank[b][2] = (int32_t)(ncand - n0c);
  }
  HIP_TRY(t, launch_rank_label(ra, B, st));
  DeltaArgs da{};
  da.tier_old = t->tier;
  da.tier_new = t->tier_alt;
  da.promote = t->d_promote;
  da.demote = t->d_demote;
  da.counts = t->d_counts;
  da.nmax = t->nmax;
  da.n = n;
  HIP_TRY(t, launch_deltas(da, B, st));
  // Counts and lists in one copy and one wait while the block is small;
  // otherwise the counts first, then only the filled part of each list.
  if (t->delta_block_bytes <= kOneCopyDeltaBytes) {
    HIP_TRY(t, hipMemcpyAsync(t->h_counts, t->d_counts, t->delta_block_bytes, hipMemcpyDeviceToHost, st));
    HIP_TRY(t, hipStreamSynchronize(st));
  } else {
    HIP_TRY(t, hipMemcpyAsync(t->h_counts, t->d_counts, (size_t)B * 2 * 4, hipMemcpyDeviceToHost, st));
    HIP_TRY(t, hipStreamSynchronize(st));
    for (int b = 0; b < B; ++b) {
      const size_t np = t->h_counts[2 * b], nd = t->h_counts[2 * b + 1];
      if (np) HIP_TRY(t, hipMemcpyAsync(t->h_promote + b * nmax, t->d_promote + b * nmax, np * sizeof(tkv_delta),
                                        hipMemcpyDeviceToHost, st));
      if (nd) HIP_TRY(t, hipMemcpyAsync(t->h_demote + b * nmax, t->d_demote + b * nmax, nd * sizeof(tkv_delta),
                                        hipMemcpyDeviceToHost, st));
    }
    HIP_TRY(t, hipStreamSynchronize(st));
  }
  std::swap(t->tier, t->tier_alt);  // device labels are now the new ones

  // ---- placement plan
  std::vector<SeqPlan> plan(B);
  std::vector<LocUpdate> upd;
  int64_t E1 = 0, E2 = 0, P = 0, n_evict = 0, n_prom = 0, n_dem = 0;
  const uint32_t c1 = (uint32_t)t->cap0, c2 = (uint32_t)(t->cap0 + t->cap1);
  std::vector<std::vector<char>> vac1s(B), vac2s(B);
  // pass 1: who leaves which place; every freed T0 slot goes back to its free
  // list before any promotion takes one (the lists are shared by the batch
  // when the HBM budget is)
  for (int b = 0; b < B; ++b) {
    SeqPlan& sp = plan[b];
    uint8_t* tr = &t->h_tier[b * nmax];
    uint32_t* lc = &t->h_loc[b * nmax];
    auto& vac1 = vac1s[b];
    auto& vac2 = vac2s[b];
    vac1.assign(t->t1_owner[b].size(), 0);
    vac2.assign(t->t2_owner[b].size(), 0);
    std::vector<uint32_t> freed;
    uint32_t* ai = t->positional ? &t->h_aidx[b * nmax] : nullptr;
    auto source = [&](uint32_t pos, uint8_t old) -> Move {
      if (t->positional) {
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
        if (d.old_tier == TKV_T0 && !t->positional) freed.push_back(mv.idx);
        switch (d.new_tier) {
          case TKV_T0: sp.promo.push_back(mv); break;
          case TKV_T1: sp.ent1.push_back(mv); break;
          case TKV_T2: sp.ent2.push_back(mv); break;
          default:
            lc[d.pos] = kNoLoc;
            upd.push_back({b, d.pos, kNoLoc});
            ++n_evict;
        }
        tr[d.pos] = d.new_tier;
      }
    };
    const int cp = t->h_counts[2 * b], cd = t->h_counts[2 * b + 1];
    take(t->h_demote + b * nmax, cd);
    take(t->h_promote + b * nmax, cp);
    n_prom += cp;
    n_dem += cd;
    auto by_pos = [](const Move& x, const Move& y) { return x.pos < y.pos; };
    std::sort(sp.ent1.begin(), sp.ent1.end(), by_pos);
    std::sort(sp.ent2.begin(), sp.ent2.end(), by_pos);
    for (auto it = freed.rbegin(); it != freed.rend(); ++it) t->free_list(b).push_back((int32_t)*it);
  }
  // pass 2: promotions take T0 slots; arenas compact and take their entrants
  for (int b = 0; b < B; ++b) {
    SeqPlan& sp = plan[b];
    uint8_t* tr = &t->h_tier[b * nmax];
    uint32_t* lc = &t->h_loc[b * nmax];
    auto& own1 = t->t1_owner[b];
    auto& own2 = t->t2_owner[b];
    if (t->positional) sp.promo.clear();  // promoted rows stay where they are
    for (const Move& mv : sp.promo) {
      if (t->free_list(b).empty()) return tkv_fail(t, TKV_ECAPACITY, "T0 pool full while promoting");
      const uint32_t slot = (uint32_t)t->free_list(b).back();
      t->free_list(b).pop_back();
      sp.promo_slot.push_back(slot);
      lc[mv.pos] = slot;
      upd.push_back({b, mv.pos, slot});
    }
    // arenas: compaction, then the entrants at the end
    compact(own1, vac1s[b], &sp.m1, &sp.mov1);
    compact(own2, vac2s[b], &sp.m2, &sp.mov2);
    uint32_t* ai = t->positional ? &t->h_aidx[b * nmax] : nullptr;
    for (auto& mv : sp.mov1) {
      if (ai) {
        ai[own1[mv.second]] = mv.second;
        continue;
      }
      lc[own1[mv.second]] = c1 + mv.second;
      upd.push_back({b, (uint32_t)own1[mv.second], c1 + mv.second});
    }
    for (auto& mv : sp.mov2) {
      if (ai) {
        ai[own2[mv.second]] = mv.second;
        continue;
      }
      lc[own2[mv.second]] = c2 + mv.second;
      upd.push_back({b, (uint32_t)own2[mv.second], c2 + mv.second});
    }
    if (sp.m1 + sp.ent1.size() > (size_t)t->cap1) return tkv_fail(t, TKV_ECAPACITY, "T1 arena full");
    if (sp.m2 + sp.ent2.size() > (size_t)t->cap2) return tkv_fail(t, TKV_ECAPACITY, "T2 arena full");
    for (size_t e = 0; e < sp.ent1.size(); ++e) {
      own1.push_back((int32_t)sp.ent1[e].pos);
      if (ai) {
        ai[sp.ent1[e].pos] = sp.m1 + (uint32_t)e;
        continue;
      }
      lc[sp.ent1[e].pos] = c1 + sp.m1 + (uint32_t)e;
      upd.push_back({b, sp.ent1[e].pos, c1 + sp.m1 + (uint32_t)e});
    }
    for (size_t e = 0; e < sp.ent2.size(); ++e) {
      own2.push_back((int32_t)sp.ent2[e].pos);
      if (ai) {
        ai[sp.ent2[e].pos] = sp.m2 + (uint32_t)e;
        continue;
      }
      lc[sp.ent2[e].pos] = c2 + sp.m2 + (uint32_t)e;
      upd.push_back({b, sp.ent2[e].pos, c2 + sp.m2 + (uint32_t)e});
    }
    sp.e1off = E1;
    sp.e2off = E2;
    sp.poff = P;
    E1 += (int64_t)sp.ent1.size();
    E2 += (int64_t)sp.ent2.size();
    P += (int64_t)sp.promo.size();
    int32_t evicted_b = 0;
    for (int p = 0; p < n; ++p) evicted_b += tr[p] == TKV_T3 ? 1 : 0;
    t->nlive[b] = n - evicted_b;
  }

  // ---- F layout: [rows entering T1 | rows entering T2 | promotions]
  const int64_t F = E1 + E2 + P;
  const size_t f_bytes = (size_t)L * H * F * hb;  // per K|V
  {
    int rc = grow_device(t, &t->fpack, &t->fpack_bytes, 2 * f_bytes);
    if (rc) return rc;
  }
  FPack fp{t->fpack, (char*)t->fpack + f_bytes, F};

  // ---- phase 1 sources
  std::vector<RowOp> ops1, ops2a, ops2b;
  std::vector<DequantOp> dq1;
  std::vector<QuantOp> q2;
  // stream mode: rows that live only on the host are packed there first
  std::vector<std::pair<int, uint32_t>> host_t1, host_t2;  // (sequence, arena index) in pack order
  auto fetch = [&](int b, const Move& mv, uint32_t frow) {
    if (mv.kind == kFromPool) {
      ops1.push_back({kAreaPool, kAreaPackOut, (uint16_t)b, mv.idx, frow});
    } else if (t->resident) {
      const uint32_t sidx = mv.kind == kFromT1 ? mv.idx : (uint32_t)t->cap1 + mv.idx;
      ops1.push_back({kAreaStage, kAreaPackOut, (uint16_t)b, sidx, frow});
    } else if (mv.kind == kFromT1) {
      ops1.push_back({kAreaPackIn, kAreaPackOut, (uint16_t)b, (uint32_t)host_t1.size(), frow});
      host_t1.emplace_back(b, mv.idx);
    } else {
      dq1.push_back({(uint16_t)b, (uint32_t)host_t2.size(), frow});
      host_t2.emplace_back(b, mv.idx);
    }
  };
  for (int b = 0; b < B; ++b) {
    const SeqPlan& sp = plan[b];
    for (size_t e = 0; e < sp.ent1.size(); ++e) fetch(b, sp.ent1[e], (uint32_t)(sp.e1off + e));
    for (size_t e = 0; e < sp.ent2.size(); ++e) fetch(b, sp.ent2[e], (uint32_t)(E1 + sp.e2off + e));
    for (size_t p = 0; p < sp.promo.size(); ++p) fetch(b, sp.promo[p], (uint32_t)(E1 + E2 + sp.poff + p));
    // phase 2a: promotions into T0 slots, compaction inside the resident staging
    for (size_t p = 0; p < sp.promo.size(); ++p)
      ops2a.push_back({kAreaPackOut, kAreaPool, (uint16_t)b, (uint32_t)(E1 + E2 + sp.poff + p), sp.promo_slot[p]});
    if (t->resident && !t->positional) {
      for (auto& mv : sp.mov1) ops2a.push_back({kAreaStage, kAreaStage, (uint16_t)b, mv.first, mv.second});
      for (auto& mv : sp.mov2)
        ops2a.push_back({kAreaStage, kAreaStage, (uint16_t)b, (uint32_t)t->cap1 + mv.first,
                         (uint32_t)t->cap1 + mv.second});
      // phase 2b: entrants into the resident staging
      for (size_t e = 0; e < sp.ent1.size(); ++e)
        ops2b.push_back({kAreaPackOut, kAreaStage, (uint16_t)b, (uint32_t)(sp.e1off + e), sp.m1 + (uint32_t)e});
    }
    // the dequantised values go to the row's location: its own slot
    // (positional), its new staging place (resident), or nowhere (stream)
    for (size_t e = 0; e < sp.ent2.size(); ++e)
      q2.push_back({(uint16_t)b, (uint32_t)(E1 + sp.e2off + e), (uint32_t)(sp.e2off + e),
                    t->positional ? sp.ent2[e].pos
                    : t->resident ? c2 + sp.m2 + (uint32_t)e : kNoLoc});
  }

  // ---- stream mode: host-resident sources packed and sent
  const int64_t NF1 = (int64_t)host_t1.size(), NF2 = (int64_t)host_t2.size();
  auto a1row = [&](int which, int l, int b, int h, uint32_t idx) -> char* {
    return (char*)(which ? t->arena1_v : t->arena1_k) + ((((size_t)l * B + b) * H + h) * t->cap1 + idx) * hb;
  };
  const size_t qrow = (size_t)D;  // bytes of one head's int8 row
  if (NF1 > 0) {
    const size_t half = (size_t)L * H * NF1 * hb;
    int rc = grow_pinned(t, &t->h_pack_in, &t->h_pack_in_bytes, 2 * half);
    if (!rc) rc = grow_device(t, &t->fin, &t->fin_bytes, 2 * half);
    if (rc) return rc;
    for (int64_t i = 0; i < NF1; ++i)
      for (int which = 0; which < 2; ++which)
        for (int l = 0; l < L; ++l)
          for (int h = 0; h < H; ++h)
            std::memcpy((char*)t->h_pack_in + ((((size_t)which * L + l) * H + h) * NF1 + i) * hb,
                        a1row(which, l, host_t1[i].first, h, host_t1[i].second), hb);
    HIP_TRY(t, hipMemcpyAsync(t->fin, t->h_pack_in, 2 * half, hipMemcpyHostToDevice, st));
    t->st.h2d_bytes += 2 * (int64_t)half;
  }
  QPack qin{};
  if (NF2 > 0) {
    const size_t codes_half = (size_t)L * H * NF2 * qrow, sc_half = (size_t)L * NF2 * t->sh * 4;
    const size_t bytes = 2 * codes_half + 2 * sc_half;
    int rc = grow_pinned(t, &t->h_qin, &t->h_qin_bytes, bytes);
    if (!rc) rc = grow_device(t, &t->qin, &t->qin_bytes, bytes);
    if (rc) return rc;
    char* hc = (char*)t->h_qin;
    float* hs = (float*)(hc + 2 * codes_half);
    for (int64_t i = 0; i < NF2; ++i) {
      const int b = host_t2[i].first;
      const uint32_t idx = host_t2[i].second;
      for (int which = 0; which < 2; ++which)
        for (int l = 0; l < L; ++l) {
          for (int h = 0; h < H; ++h)
            std::memcpy(hc + ((((size_t)which * L + l) * H + h) * NF2 + i) * qrow,
                        (which ? t->arena2_v : t->arena2_k) + ((((size_t)l * B + b) * H + h) * t->cap2 + idx) * qrow,
                        qrow);
          for (int k = 0; k < t->sh; ++k)
            hs[(((size_t)which * L + l) * NF2 + i) * t->sh + k] =
                (which ? t->ascale_v : t->ascale_k)[(((size_t)l * B + b) * t->cap2 + idx) * t->sh + k];
        }
    }
    HIP_TRY(t, hipMemcpyAsync(t->qin, t->h_qin, bytes, hipMemcpyHostToDevice, st));
    t->st.h2d_bytes += (int64_t)bytes;
    qin = QPack{(int8_t*)t->qin, (float*)((char*)t->qin + 2 * codes_half), NF2};
  }

  // ---- ops and location updates to the device
  const size_t nops = ops1.size() + ops2a.size() + ops2b.size();
  const size_t bytes = nops * sizeof(RowOp) + dq1.size() * sizeof(DequantOp) + q2.size() * sizeof(QuantOp) +
                       upd.size() * sizeof(LocUpdate);
  const RowOp* d_ops1 = nullptr;
  const RowOp* d_ops2a = nullptr;
  const RowOp* d_ops2b = nullptr;
  const DequantOp* d_dq1 = nullptr;
  const QuantOp* d_q2 = nullptr;
  const LocUpdate* d_upd = nullptr;
  if (bytes > 0) {
    int rc = grow_pinned(t, &t->h_ops, &t->h_ops_bytes, bytes);
    if (!rc) rc = grow_device(t, &t->d_ops, &t->d_ops_bytes, bytes);
    if (rc) return rc;
    char* h = (char*)t->h_ops;
    char* d = (char*)t->d_ops;
    size_t off = 0;
    auto put = [&](const void* src, size_t sz) -> const void* {
      if (sz) std::memcpy(h + off, src, sz);
      const void* dev_ptr = d + off;
      off += sz;
      return dev_ptr;
    };
    d_ops1 = (const RowOp*)put(ops1.data(), ops1.size() * sizeof(RowOp));
    d_ops2a = (const RowOp*)put(ops2a.data(), ops2a.size() * sizeof(RowOp));
    d_ops2b = (const RowOp*)put(ops2b.data(), ops2b.size() * sizeof(RowOp));
    d_dq1 = (const DequantOp*)put(dq1.data(), dq1.size() * sizeof(DequantOp));
    d_q2 = (const QuantOp*)put(q2.data(), q2.size() * sizeof(QuantOp));
    d_upd = (const LocUpdate*)put(upd.data(), upd.size() * sizeof(LocUpdate));
    HIP_TRY(t, hipMemcpyAsync(t->d_ops, t->h_ops, bytes, hipMemcpyHostToDevice, st));
  }

  // ---- device phases
  CopyArgs ca{};
  ca.rows = t->rowspace();
  ca.kv_heads = H;
  ca.head_bytes = (int32_t)hb;
  ca.elem_bytes = t->esz;
  ca.pack_out_k = fp.k;  // F
  ca.pack_out_v = fp.v;
  ca.pack_out_rows = F;
  ca.pack_in_k = t->fin;  // FI
  ca.pack_in_v = t->fin ? (char*)t->fin + (size_t)L * H * NF1 * hb : nullptr;
  ca.pack_in_rows = NF1;
  HIP_TRY(t, launch_copy_rows(ca, d_ops1, (int)ops1.size(), L, st));
  DequantArgs dqa{qin, fp, H, D, t->esz, (t->flags & TKV_FLAG_T2_FP8) ? 1 : 0, t->sh};
  HIP_TRY(t, launch_dequant_rows(dqa, d_dq1, (int)dq1.size(), L, st));
  HIP_TRY(t, launch_copy_rows(ca, d_ops2a, (int)ops2a.size(), L, st));
  HIP_TRY(t, launch_copy_rows(ca, d_ops2b, (int)ops2b.size(), L, st));
  QPack qout{};
  if (E2 > 0) {
    const size_t codes_half = (size_t)L * H * E2 * qrow, sc_half = (size_t)L * E2 * t->sh * 4;
    int rc = grow_device(t, &t->qout, &t->qout_bytes, 2 * codes_half + 2 * sc_half);
    if (rc) return rc;
    qout = QPack{(int8_t*)t->qout, (float*)((char*)t->qout + 2 * codes_half), E2};
    QuantArgs qa{t->rowspace(), fp, qout, H, D, t->esz, (t->flags & TKV_FLAG_T2_FP8) ? 1 : 0, t->sh};
    HIP_TRY(t, launch_quant_rows(qa, d_q2, (int)q2.size(), L, st));
  }
  HIP_TRY(t, launch_set_loc(d_upd, (int)upd.size(), t->loc, t->nmax, st));
  LiveArgs la{};
  la.tier = t->tier;
  la.loc = t->loc;
  la.live_pos = t->live_pos;
  la.live_loc = t->live_loc;
  la.nmax = t->nmax;
  la.n = n;
  HIP_TRY(t, launch_build_live(la, B, st));
  HIP_TRY(t, hipEventRecord(t->ev_gathered, st));

  // ---- write-back of the entrants, on its own stream
  if (E1 > 0 || E2 > 0) HIP_TRY(t, hipStreamWaitEvent(t->wb, t->ev_gathered, 0));
  if (E1 > 0) {
    const size_t half = (size_t)L * H * E1 * hb;
    int rc = grow_pinned(t, &t->h_pack_out, &t->h_pack_out_bytes, 2 * half);
    if (rc) return rc;
    for (int which = 0; which < 2; ++which)
      HIP_TRY(t, hipMemcpy2DAsync((char*)t->h_pack_out + which * half, E1 * hb, which ? fp.v : fp.k, F * hb, E1 * hb,
                                  (size_t)L * H, hipMemcpyDeviceToHost, t->wb));
    t->st.d2h_bytes += 2 * (int64_t)half;
  }
  if (E2 > 0) {
    const size_t qbytes = 2 * (size_t)L * H * E2 * qrow + 2 * (size_t)L * E2 * t->sh * 4;
    int rc = grow_pinned(t, &t->h_qout, &t->h_qout_bytes, qbytes);
    if (rc) return rc;
    HIP_TRY(t, hipMemcpyAsync(t->h_qout, t->qout, qbytes, hipMemcpyDeviceToHost, t->wb));
    t->st.d2h_bytes += (int64_t)qbytes;
  }
  HIP_TRY(t, hipEventRecord(t->ev_pack, t->wb));
  HIP_TRY(t, hipEventRecord(t->ev_arena, st));
  t->arena_pending = true;

  // ---- host job: compact the arenas, file the entrants
  bool any_host_work = E1 > 0 || E2 > 0;
  for (int b = 0; b < B && !any_host_work; ++b) any_host_work = !plan[b].mov1.empty() || !plan[b].mov2.empty();
  if (any_host_work) {
    struct Job {
      std::vector<SeqPlan> plan;
      char *a1k, *a1v;
      int8_t *a2k, *a2v;
      float *s2k, *s2v;
      const char* pack1;  // [2][L][H][E1][D] cache type
      const char* pack2;  // codes [2][L][H][E2][D], scales [2][L][E2][SH]
      hipEvent_t ev;
      int L, B, H, D, SH;
      size_t cap1, cap2, hb;
      int64_t E1, E2;
    };
    auto job = std::make_shared<Job>(Job{std::move(plan), (char*)t->arena1_k, (char*)t->arena1_v, t->arena2_k,
                                         t->arena2_v, t->ascale_k, t->ascale_v, (const char*)t->h_pack_out,
                                         (const char*)t->h_qout, t->ev_pack, L, B, H, D, t->sh, (size_t)t->cap1,
                                         (size_t)t->cap2, hb, E1, E2});
    t->arena_job = t->worker.submit([job]() -> int {
     try {
      const Job& j = *job;
      auto r1 = [&](int which, int l, int b, int h, uint32_t idx) -> char* {
        return (which ? j.a1v : j.a1k) + ((((size_t)l * j.B + b) * j.H + h) * j.cap1 + idx) * j.hb;
      };
      auto r2 = [&](int which, int l, int b, int h, uint32_t idx) -> int8_t* {
        return (which ? j.a2v : j.a2k) + ((((size_t)l * j.B + b) * j.H + h) * j.cap2 + idx) * j.D;
      };
      auto s2 = [&](int which, int l, int b, uint32_t idx) -> float* {
        return (which ? j.s2v : j.s2k) + (((size_t)l * j.B + b) * j.cap2 + idx) * j.SH;
      };
      auto moves = [&](int l0, int l1) {
        for (int l = l0; l < l1; ++l)
          for (int b = 0; b < j.B; ++b)
            for (int which = 0; which < 2; ++which) {
              for (auto& mv : j.plan[b].mov1)
                for (int h = 0; h < j.H; ++h) std::memcpy(r1(which, l, b, h, mv.second), r1(which, l, b, h, mv.first), j.hb);
              for (auto& mv : j.plan[b].mov2) {
                for (int h = 0; h < j.H; ++h) std::memcpy(r2(which, l, b, h, mv.second), r2(which, l, b, h, mv.first), j.D);
                std::memcpy(s2(which, l, b, mv.second), s2(which, l, b, mv.first), j.SH * 4);
              }
            }
      };
      auto file = [&](int l0, int l1) {
        const size_t c2half = (size_t)j.L * j.H * j.E2 * j.D;
        const float* sc = (const float*)(j.pack2 + 2 * c2half);
        for (int l = l0; l < l1; ++l)
          for (int b = 0; b < j.B; ++b)
            for (int which = 0; which < 2; ++which) {
              const SeqPlan& sp = j.plan[b];
              const size_t n1 = sp.ent1.size(), n2 = sp.ent2.size();
              for (int h = 0; h < j.H && n1; ++h)
                std::memcpy(r1(which, l, b, h, sp.m1),
                            j.pack1 + ((((size_t)which * j.L + l) * j.H + h) * j.E1 + sp.e1off) * j.hb, n1 * j.hb);
              for (int h = 0; h < j.H && n2; ++h)
                std::memcpy(r2(which, l, b, h, sp.m2),
                            j.pack2 + ((((size_t)which * j.L + l) * j.H + h) * j.E2 + sp.e2off) * j.D, n2 * j.D);
              if (n2)
                std::memcpy(s2(which, l, b, sp.m2), sc + (((size_t)which * j.L + l) * j.E2 + sp.e2off) * j.SH,
                            n2 * j.SH * 4);
            }
      };
      const int nth = std::min(4, j.L);
      auto split = [&](const std::function<void(int, int)>& f) {
        std::vector<std::thread> th;
        for (int i = 1; i < nth; ++i) th.emplace_back(f, j.L * i / nth, j.L * (i + 1) / nth);
        f(0, j.L / nth);
        for (auto& x : th) x.join();
      };
      split(moves);
      if (j.E1 > 0 || j.E2 > 0) {
        if (hipEventSynchronize(j.ev) != hipSuccess) return TKV_EHIP;
        split(file);
      }
      return TKV_OK;
     } catch (const std::bad_alloc&) {  // the job reports, never throws
      return TKV_ENOMEM;
     } catch (...) {
      return TKV_EHIP;
     }
    });
  }

  t->st.promotions += n_prom;
  t->st.demotions += n_dem;
  t->st.evictions += n_evict;
  t->st.reassigns += 1;
  t->st.reassign_ms +=
      std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - wall0).count();
  return TKV_OK;
}
extern "C" int tkv_reassign(tkv_t* t, tkv_stream_t stream) {
  return guarded(t, [&] { return reassign_impl(t, stream); });
}
