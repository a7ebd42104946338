// tkv_reassign: score-ranked re-placement of every sequence's rows
// ("Not All Thoughts Need HBM", gist.science technical summary, Method §1
// four tiers and §4 periodic reassignment with differential movement).
//
// Device: rank + label (radix select on the GPU's fp32 scores), changed-row
// lists by prefix-scan compaction.  Host: one synchronisation to read the
// lists, then a placement plan per sequence:
//   * the T1 arena of a sequence stays dense: rows leaving T1 leave holes,
//     the last remaining rows move into the holes, rows entering T1 are
//     appended (so they land in one contiguous block per layer);
//   * T0 slots freed by demotions are reused by promotions.
// Rows move in three dependent phases of one copy kernel: (1) rows that
// leave their home are gathered into pack buffers, (2a) arena compaction in
// the staging mirror and promotions into T0 slots, (2b) entrants into the
// staging mirror.  Entrants leave the GPU as one contiguous copy per K|V into
// a pinned pack; a host job (never waited for by the GPU) compacts the
// pinned arena and files the entrants.  In stream mode promoted rows come
// from the host arena.  Every area is head-major, [..][kv_head][row][d].
#include <chrono>
#include <cstring>
#include <memory>
#include <thread>

#include "handle.hpp"
#include "host_util.hpp"

using namespace tkvd;

namespace {

struct SeqPlan {
  std::vector<uint32_t> entrant_pos, entrant_slot;    // T0 -> T1: position, old T0 slot
  std::vector<uint32_t> promo_pos, promo_idx, promo_slot;  // T1 -> T0: position, old arena index, new slot
  std::vector<std::pair<uint32_t, uint32_t>> movers;  // arena (src, dst)
  uint32_t m = 0;                                     // arena rows before the entrants
  int64_t eoff = 0, poff = 0;                         // offsets in the pack buffers
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

int grow_packs(tkv* t, int64_t E, int64_t P) {
  const size_t lrb = (size_t)t->L * t->row_bytes;
  if ((size_t)E > t->pack_out_cap) {
    const size_t rows = std::max<size_t>((size_t)E * 2, 64);
    for (void** p : {&t->pack_out_k, &t->pack_out_v}) {
      if (*p) HIP_TRY(t, hipFree(*p));
      *p = nullptr;
      HIP_TRY(t, hipMalloc(p, rows * lrb));
    }
    t->pack_out_cap = rows;
  }
  if ((size_t)P > t->pack_in_cap) {
    const size_t rows = std::max<size_t>((size_t)P * 2, 64);
    for (void** p : {&t->pack_in_k, &t->pack_in_v}) {
      if (*p) HIP_TRY(t, hipFree(*p));
      *p = nullptr;
      HIP_TRY(t, hipMalloc(p, rows * lrb));
    }
    t->pack_in_cap = rows;
  }
  return TKV_OK;
}

}  // namespace

extern "C" int tkv_reassign(tkv_t* t, tkv_stream_t stream) {
  if (!t) return tkv_fail(nullptr, TKV_EINVAL, "handle is NULL");
  if (t->state == TkvState::InStep) return tkv_fail(t, TKV_ESTATE, "reassign between the layer groups of a step");
  if (t->n == 0) return TKV_OK;
  const auto wall0 = std::chrono::steady_clock::now();
  hipStream_t st = (hipStream_t)stream;
  const int B = t->B, L = t->L, n = t->n;
  const size_t nmax = t->nmax;
  // The host arena and the pinned staging buffers may still be read or
  // written by the previous reassignment's host job and copies.
  if (t->arena_job.valid()) {
    const int rc = t->arena_job.get();
    if (rc) return rc;
  }
  HIP_TRY(t, hipStreamSynchronize(t->side));
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
  for (int b = 0; b < B; ++b) {
    int64_t np = 0, nev = 0;
    const uint8_t* tr = &t->h_tier[b * nmax];
    for (int p = 0; p < n; ++p) {
      if (tr[p] == TKV_T3)
        ++nev;
      else if (is_protected(*t, p, n))
        ++np;
    }
    const int64_t ncand = n - np - nev;
    const int64_t n3 = std::min<int64_t>(ncand, std::max<int64_t>(0, floor_ratio(t->evict, n) - nev));
    const int64_t n0c = std::min<int64_t>(ncand - n3, std::max<int64_t>(0, floor_ratio(t->hbm, n) - np));
    const int64_t n2 = std::min<int64_t>(ncand - n3 - n0c, floor_ratio(t->t2, n));
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
  std::swap(t->tier, t->tier_alt);  // device labels are now the new ones

  // ---- placement plan
  std::vector<SeqPlan> plan(B);
  std::vector<LocUpdate> upd;
  int64_t E = 0, P = 0, n_evict = 0, n_prom = 0, n_dem = 0;
  for (int b = 0; b < B; ++b) {
    SeqPlan& sp = plan[b];
    auto& own = t->t1_owner[b];
    uint8_t* tr = &t->h_tier[b * nmax];
    uint32_t* lc = &t->h_loc[b * nmax];
    std::vector<char> vacated(own.size(), 0);
    std::vector<uint32_t> freed;
    const tkv_delta* pro = t->h_promote + b * nmax;
    const tkv_delta* dem = t->h_demote + b * nmax;
    const int cp = t->h_counts[2 * b], cd = t->h_counts[2 * b + 1];
    for (int k = 0; k < cd; ++k) {
      const tkv_delta& d = dem[k];
      if (d.old_tier == TKV_T0) {
        freed.push_back(lc[d.pos]);
        if (d.new_tier == TKV_T1) {
          sp.entrant_pos.push_back(d.pos);
          sp.entrant_slot.push_back(lc[d.pos]);
        }
      } else if (d.old_tier == TKV_T1) {
        vacated[lc[d.pos] - t->cap0] = 1;
      } else {
        return tkv_fail(t, TKV_ESTATE, "unexpected demotion from tier %d", d.old_tier);
      }
      if (d.new_tier == TKV_T3) {
        lc[d.pos] = kNoLoc;
        upd.push_back({b, d.pos, kNoLoc});
        ++n_evict;
      } else if (d.new_tier == TKV_T2) {
        return tkv_fail(t, TKV_ESTATE, "8-bit tier rows are not supported by this build");
      }
      tr[d.pos] = d.new_tier;
    }
    for (int k = 0; k < cp; ++k) {
      const tkv_delta& d = pro[k];
      if (d.old_tier != TKV_T1 || d.new_tier != TKV_T0)
        return tkv_fail(t, TKV_ESTATE, "unexpected promotion %d -> %d", d.old_tier, d.new_tier);
      const uint32_t idx = lc[d.pos] - t->cap0;
      vacated[idx] = 1;
      sp.promo_pos.push_back(d.pos);
      sp.promo_idx.push_back(idx);
      tr[d.pos] = d.new_tier;
    }
    n_prom += cp;
    n_dem += cd;
    // T0 slots: freed ones first go back, then promotions take slots
    for (auto it = freed.rbegin(); it != freed.rend(); ++it) t->free0[b].push_back((int32_t)*it);
    for (size_t k = 0; k < sp.promo_pos.size(); ++k) {
      if (t->free0[b].empty()) return tkv_fail(t, TKV_ECAPACITY, "T0 pool full while promoting");
      const uint32_t slot = (uint32_t)t->free0[b].back();
      t->free0[b].pop_back();
      sp.promo_slot.push_back(slot);
      lc[sp.promo_pos[k]] = slot;
      upd.push_back({b, sp.promo_pos[k], slot});
    }
    // arena compaction: the last kept rows fill the holes below m
    const uint32_t n1 = (uint32_t)own.size();
    uint32_t kept = 0;
    for (uint32_t i = 0; i < n1; ++i) kept += vacated[i] ? 0 : 1;
    sp.m = kept;
    std::vector<uint32_t> holes, srcs;
    for (uint32_t i = 0; i < sp.m; ++i)
      if (vacated[i]) holes.push_back(i);
    for (uint32_t i = sp.m; i < n1; ++i)
      if (!vacated[i]) srcs.push_back(i);
    if (holes.size() != srcs.size()) return tkv_fail(t, TKV_ESTATE, "arena compaction mismatch");
    for (size_t k = 0; k < holes.size(); ++k) {
      sp.movers.emplace_back(srcs[k], holes[k]);
      own[holes[k]] = own[srcs[k]];
      lc[own[holes[k]]] = (uint32_t)t->cap0 + holes[k];
      upd.push_back({b, (uint32_t)own[holes[k]], (uint32_t)t->cap0 + holes[k]});
    }
    own.resize(sp.m);
    for (size_t e = 0; e < sp.entrant_pos.size(); ++e) {
      const uint32_t idx = sp.m + (uint32_t)e;
      if (idx >= (uint32_t)t->cap1) return tkv_fail(t, TKV_ECAPACITY, "T1 arena full");
      own.push_back((int32_t)sp.entrant_pos[e]);
      lc[sp.entrant_pos[e]] = (uint32_t)t->cap0 + idx;
      upd.push_back({b, sp.entrant_pos[e], (uint32_t)t->cap0 + idx});
    }
    sp.eoff = E;
    sp.poff = P;
    E += (int64_t)sp.entrant_pos.size();
    P += (int64_t)sp.promo_pos.size();
    int32_t evicted_b = 0;
    for (int p = 0; p < n; ++p) evicted_b += tr[p] == TKV_T3 ? 1 : 0;
    t->nlive[b] = n - evicted_b;
  }

  // ---- host arena: promoted rows out first (stream mode), then compaction
  const size_t rb = t->row_bytes;
  const size_t hb = (size_t)t->D * t->esz;
  const int H = t->Hkv;
  auto arena_row = [&](int which, int l, int b, int h, uint32_t idx) -> char* {
    return (char*)(which ? t->arena1_v : t->arena1_k) + ((((size_t)l * B + b) * H + h) * t->cap1 + idx) * hb;
  };
  if (!t->resident && P > 0) {
    int rc = grow_pinned(t, &t->h_pack_in, &t->h_pack_in_bytes, 2 * (size_t)L * P * rb);
    if (rc) return rc;
    for (int b = 0; b < B; ++b)
      for (size_t p = 0; p < plan[b].promo_idx.size(); ++p)
        for (int which = 0; which < 2; ++which)
          for (int l = 0; l < L; ++l)
            for (int h = 0; h < H; ++h)
              std::memcpy((char*)t->h_pack_in + ((((size_t)which * L + l) * H + h) * P + plan[b].poff + p) * hb,
                          arena_row(which, l, b, h, plan[b].promo_idx[p]), hb);
  }

  // ---- row-copy ops
  std::vector<RowOp> ops1, ops2a, ops2b;
  for (int b = 0; b < B; ++b) {
    const SeqPlan& sp = plan[b];
    for (size_t e = 0; e < sp.entrant_pos.size(); ++e) {
      ops1.push_back({kAreaPool, kAreaPackOut, (uint16_t)b, sp.entrant_slot[e], (uint32_t)(sp.eoff + e)});
      if (t->resident)
        ops2b.push_back({kAreaPackOut, kAreaStage, (uint16_t)b, (uint32_t)(sp.eoff + e), sp.m + (uint32_t)e});
    }
    for (size_t p = 0; p < sp.promo_pos.size(); ++p) {
      if (t->resident) ops1.push_back({kAreaStage, kAreaPackIn, (uint16_t)b, sp.promo_idx[p], (uint32_t)(sp.poff + p)});
      ops2a.push_back({kAreaPackIn, kAreaPool, (uint16_t)b, (uint32_t)(sp.poff + p), sp.promo_slot[p]});
    }
    if (t->resident)
      for (auto& mv : sp.movers) ops2a.push_back({kAreaStage, kAreaStage, (uint16_t)b, mv.first, mv.second});
  }
  const size_t nops = ops1.size() + ops2a.size() + ops2b.size();
  const size_t bytes = nops * sizeof(RowOp) + upd.size() * sizeof(LocUpdate);
  if (bytes > 0) {
    int rc = grow_pinned(t, &t->h_ops, &t->h_ops_bytes, bytes);
    if (!rc) rc = grow_device(t, &t->d_ops, &t->d_ops_bytes, bytes);
    if (rc) return rc;
    char* h = (char*)t->h_ops;
    std::memcpy(h, ops1.data(), ops1.size() * sizeof(RowOp));
    std::memcpy(h + ops1.size() * sizeof(RowOp), ops2a.data(), ops2a.size() * sizeof(RowOp));
    std::memcpy(h + (ops1.size() + ops2a.size()) * sizeof(RowOp), ops2b.data(), ops2b.size() * sizeof(RowOp));
    std::memcpy(h + nops * sizeof(RowOp), upd.data(), upd.size() * sizeof(LocUpdate));
    HIP_TRY(t, hipMemcpyAsync(t->d_ops, t->h_ops, bytes, hipMemcpyHostToDevice, st));
  }
  const RowOp* d_ops1 = (const RowOp*)t->d_ops;
  const RowOp* d_ops2a = d_ops1 + ops1.size();
  const RowOp* d_ops2b = d_ops2a + ops2a.size();
  const LocUpdate* d_upd = (const LocUpdate*)(d_ops1 + nops);

  CopyArgs ca{};
  ca.rows = t->rowspace();
  ca.kv_heads = H;
  ca.head_bytes = (int32_t)hb;
  ca.elem_bytes = t->esz;
  ca.pack_out_rows = E;
  ca.pack_in_rows = P;
  {
    int rc = grow_packs(t, E, P);
    if (rc) return rc;
  }
  ca.pack_out_k = t->pack_out_k;
  ca.pack_out_v = t->pack_out_v;
  ca.pack_in_k = t->pack_in_k;
  ca.pack_in_v = t->pack_in_v;
  HIP_TRY(t, launch_copy_rows(ca, d_ops1, (int)ops1.size(), L, st));
  HIP_TRY(t, hipEventRecord(t->ev_gathered, st));
  if (!t->resident && P > 0) {
    HIP_TRY(t, hipMemcpyAsync(ca.pack_in_k, t->h_pack_in, (size_t)L * P * rb, hipMemcpyHostToDevice, st));
    HIP_TRY(t, hipMemcpyAsync(ca.pack_in_v, (char*)t->h_pack_in + (size_t)L * P * rb, (size_t)L * P * rb,
                              hipMemcpyHostToDevice, st));
    t->st.h2d_bytes += 2 * (int64_t)L * P * rb;
  }
  HIP_TRY(t, launch_copy_rows(ca, d_ops2a, (int)ops2a.size(), L, st));
  HIP_TRY(t, launch_copy_rows(ca, d_ops2b, (int)ops2b.size(), L, st));
  HIP_TRY(t, launch_set_loc(d_upd, (int)upd.size(), t->loc, t->nmax, st));
  LiveArgs la{};
  la.tier = t->tier;
  la.loc = t->loc;
  la.live_pos = t->live_pos;
  la.live_loc = t->live_loc;
  la.nmax = t->nmax;
  la.n = n;
  HIP_TRY(t, launch_build_live(la, B, st));
  // entrants leave the GPU as one contiguous copy per K|V into a pinned pack;
  // a host job then compacts the arena and files the entrants at [m, m + E_b)
  if (E > 0) {
    int rc = grow_pinned(t, &t->h_pack_out, &t->h_pack_out_bytes, 2 * (size_t)L * E * rb);
    if (rc) return rc;
    // on the write-back stream, so the decode steps that follow do not wait for it
    HIP_TRY(t, hipStreamWaitEvent(t->wb, t->ev_gathered, 0));
    HIP_TRY(t, hipMemcpyAsync(t->h_pack_out, t->pack_out_k, (size_t)L * E * rb, hipMemcpyDeviceToHost, t->wb));
    HIP_TRY(t, hipMemcpyAsync((char*)t->h_pack_out + (size_t)L * E * rb, t->pack_out_v, (size_t)L * E * rb,
                              hipMemcpyDeviceToHost, t->wb));
    t->st.d2h_bytes += 2 * (int64_t)L * E * rb;
  }
  HIP_TRY(t, hipEventRecord(t->ev_pack, t->wb));
  HIP_TRY(t, hipEventRecord(t->ev_arena, st));
  t->arena_pending = true;
  bool any_host_work = E > 0;
  for (int b = 0; b < B && !any_host_work; ++b) any_host_work = !plan[b].movers.empty();
  if (any_host_work) {
    struct Job {
      std::vector<SeqPlan> plan;
      char* ak;
      char* av;
      const char* pack;
      hipEvent_t ev;
      int L, B, H;
      size_t cap1, hb;
      int64_t E;
    };
    auto job = std::make_shared<Job>(Job{std::move(plan), (char*)t->arena1_k, (char*)t->arena1_v,
                                         (const char*)t->h_pack_out, t->ev_pack, L, B, H, (size_t)t->cap1, hb, E});
    t->arena_job = std::async(std::launch::async, [job]() -> int {
      const Job& j = *job;
      auto row = [&](int which, int l, int b, int h, uint32_t idx) -> char* {
        return (which ? j.av : j.ak) + ((((size_t)l * j.B + b) * j.H + h) * j.cap1 + idx) * j.hb;
      };
      // layers split over a few threads; each layer's rows are independent
      auto work = [&](int l0, int l1) {
        for (int l = l0; l < l1; ++l)
          for (int b = 0; b < j.B; ++b)
            for (auto& mv : j.plan[b].movers)
              for (int which = 0; which < 2; ++which)
                for (int h = 0; h < j.H; ++h)
                  std::memcpy(row(which, l, b, h, mv.second), row(which, l, b, h, mv.first), j.hb);
      };
      // pack_out is [K|V][layer][kv head][entrant][head_dim]
      auto file = [&](int l0, int l1) {
        for (int l = l0; l < l1; ++l)
          for (int b = 0; b < j.B; ++b) {
            const size_t ne = j.plan[b].entrant_pos.size();
            if (!ne) continue;
            for (int which = 0; which < 2; ++which)
              for (int h = 0; h < j.H; ++h)
                std::memcpy(row(which, l, b, h, j.plan[b].m),
                            j.pack + ((((size_t)which * j.L + l) * j.H + h) * j.E + j.plan[b].eoff) * j.hb, ne * j.hb);
          }
      };
      const int nth = std::min(4, j.L);
      auto split = [&](const std::function<void(int, int)>& f) {
        std::vector<std::thread> th;
        for (int i = 1; i < nth; ++i) th.emplace_back(f, j.L * i / nth, j.L * (i + 1) / nth);
        f(0, j.L / nth);
        for (auto& x : th) x.join();
      };
      split(work);
      if (j.E > 0) {
        if (hipEventSynchronize(j.ev) != hipSuccess) return TKV_EHIP;
        split(file);
      }
      return TKV_OK;
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
