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
//             pool, the resident staging, or -- stream staging -- the pinned
//             arenas, read by the kernels over PCIe; 8-bit rows dequantised
//             on the way);
//   phase 2a  promotions F -> T0 slots; compaction moves inside the staging;
//   phase 2b  rows entering T1: F -> staging; rows entering T2: quantised
//             from F on the GPU (codes + scale out, dequantised values into
//             the staging).
// Positional resident staging (every live row at its own position in the
// pool) moves no row inside HBM: phase 1 gathers only the rows entering T1
// or T2, for their write-back, and T2 entrants get their dequantised values
// in their own slots; phases 2a and 2b are empty.  T1/T2 rows keep a
// host-side arena index per position.
// Where the arenas change:
//   * stream staging: the kernels compact the pinned arenas and write the
//     entrants (codes and scales for T2) straight into them, on the caller's
//     stream, before the next step's copies read them (an event gates the
//     copy streams).  No host thread touches a row.
//   * resident staging: nothing reads the arenas on the decode path, so
//     rows leaving them free their index and entrants take the lowest free
//     ones (no compaction); the rows entering T1 are copied from their own
//     HBM slots into the mapped arena by a few work-groups on the write-back
//     stream, beside the next decode steps, and T2 entrants' codes and
//     scales are written there by the quantiser.
// Every allocation a reassignment may need is made before the device labels
// change; a failure after that point marks the handle failed (every later
// call but tkv_destroy, tkv_last_error and tkv_stats returns TKV_ESTATE).
// Every area is head-major.
#include <algorithm>
#include <chrono>
#include <cstring>

#include "handle.hpp"
#include "host_util.hpp"

using namespace tkvd;

namespace {

// Largest changed-row block read back whole (one copy, one wait); a few tens
// of microseconds over PCIe, about one synchronisation round trip.
constexpr size_t kOneCopyDeltaBytes = 1u << 20;

// Grow a reassignment buffer to hold `need` bytes (twice that, when the
// handle's memory cap allows, so that it rarely grows again).  Failure
// (TKV_ENOMEM) leaves the buffer empty.
int grow_buffer(tkv* t, void** p, size_t* cap, size_t need, bool pinned) {
  if (need <= *cap) return TKV_OK;
  if (*p) {
    if (pinned)
      HIP_TRY(t, hipHostFree(*p));
    else
      HIP_TRY(t, hipFree(*p));
  }
  t->mem_held -= (int64_t)*cap;
  *p = nullptr;
  *cap = 0;
  size_t bytes = std::max(need, (size_t)4096) * 2;
  if (!within_cap(*t, bytes)) bytes = need;
  if (!within_cap(*t, bytes))
    return tkv_fail(t, TKV_ENOMEM, "memory cap (%lld bytes) reached: a reassignment needs %zu more bytes",
                    (long long)t->mem_cap, need);
  const hipError_t e = pinned ? hipHostMalloc(p, bytes, hipHostMallocDefault) : hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    return tkv_fail(t, TKV_ENOMEM, "%s(%zu bytes) failed: %s", pinned ? "hipHostMalloc" : "hipMalloc", bytes,
                    hipGetErrorString(e));
  }
  *cap = bytes;
  t->mem_held += (int64_t)bytes;
  return TKV_OK;
}
int grow_device(tkv* t, void** p, size_t* cap, size_t need) { return grow_buffer(t, p, cap, need, false); }
int grow_pinned(tkv* t, void** p, size_t* cap, size_t need) { return grow_buffer(t, p, cap, need, true); }

}  // namespace

// Counts of a reassignment's changed rows, known from the lists alone (before
// any host state changes): rows entering T1, T2 and T0, evictions.
struct DeltaTotals {
  int64_t e1 = 0, e2 = 0, p = 0, evict = 0, all = 0;
};
static DeltaTotals delta_totals(const tkv* t) {
  DeltaTotals d{};
  for (int b = 0; b < t->B; ++b)
    for (int which = 0; which < 2; ++which) {
      const tkv_delta* list = (which ? t->h_demote : t->h_promote) + (size_t)b * t->nmax;
      const int cnt = t->h_counts[2 * b + which];
      d.all += cnt;
      for (int k = 0; k < cnt; ++k) {
        switch (list[k].new_tier) {
          case TKV_T0: d.p += 1; break;
          case TKV_T1: d.e1 += 1; break;
          case TKV_T2: d.e2 += 1; break;
          default: d.evict += 1;
        }
      }
    }
  return d;
}

// use_static: the fetch pack F and the ops block live in the library's static
// device scratch (no allocation); a reassignment that needs more returns
// TKV_ECAPACITY before any state changes, and the call returns only once no
// kernel reads the scratch any more.
static int reassign_impl(tkv_t* t, tkv_stream_t stream, bool use_static) {
  if (!t) return tkv_fail(nullptr, TKV_EINVAL, "handle is NULL");
  for (const tkv* p : t->parts) t->failed = t->failed || p->failed;
  if (t->failed) return tkv_fail(t, TKV_ESTATE, "handle unusable: an earlier reassignment failed part way");
  if (t->state == TkvState::InStep) return tkv_fail(t, TKV_ESTATE, "reassign between the layer groups of a step");
  if (t->n == 0) return TKV_OK;
  if (!t->parts.empty()) {
    // Per-layer budgets: each part ranks the scores of all layers, so every
    // part's pending Eq. 1 increment goes in first; then each part re-places
    // its layers with its own ratio.  A part that fails after an earlier one
    // was re-placed leaves the parts disagreeing: the handle is then failed.
    if (int rc = tkv_flush_score(t, (hipStream_t)stream)) return rc;
    for (size_t i = 0; i < t->parts.size(); ++i) {
      const int rc = reassign_impl(t->parts[i], stream, use_static);
      if (rc != TKV_OK) {
        t->err = t->parts[i]->err;
        t->failed = t->failed || i > 0 || t->parts[i]->failed;
        return rc;
      }
    }
    return TKV_OK;
  }
  const auto wall0 = std::chrono::steady_clock::now();
  hipStream_t st = (hipStream_t)stream;
  if (int rc = tkv_flush_score(t, st)) return rc;  // ranking reads s
  const int B = t->B, L = t->L, n = t->n, H = t->Hkv, D = t->D;
  const size_t nmax = t->nmax;
  const size_t hb = (size_t)D * t->esz;  // bytes of one head's row
  const bool stream_mode = !t->resident;
  // The ops buffers may still be read by the last reassignment's kernels.
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
  for (int b = 0; b < B; ++b) {
    const int64_t ncand = ncands[b], n3 = cuts[b].n3, n0c = cuts[b].n0c, n2 = cuts[b].n2;
    ra.ncand[b] = (int32_t)ncand;
    ra.rank[b][0] = (int32_t)n3;
    ra.rank[b][1] = (int32_t)(n3 + n2);
    ra.rank[b][2] = (int32_t)(ncand - n0c);
  }
  if (t->shared_hbm) {
    // Batch-shared budget, all on the GPU: each sequence's eviction cut
    // (select-only pass), the joint select of the batch's best remaining
    // candidates, then the labels with each sequence's share of T0.
    int64_t remaining = 0, budget = 0;
    for (int b = 0; b < B; ++b) {
      remaining += ncands[b] - cuts[b].n3;
      budget += floor_ratio(t->hbm, n) - nprots[b];
      ra.rank[b][1] = ra.rank[b][2] = ra.ncand[b];  // no other cut in the select-only pass
    }
    ra.cuts_out = t->d_cuts;
    HIP_TRY(t, launch_rank_label(ra, B, st));
    JointArgs ja{};
    ja.s = t->s;
    ja.tier_old = t->tier;
    ja.cuts = t->d_cuts;
    ja.n0c = t->d_n0c;
    ja.nmax = t->nmax;
    ja.n = n;
    ja.prompt = t->prompt;
    ja.sinks = t->sinks;
    ja.recent = t->recent;
    ja.batch = B;
    ja.remaining = remaining;
    ja.take = std::min<int64_t>(remaining, std::max<int64_t>(0, budget));
    HIP_TRY(t, launch_joint_select(ja, st));
    ra.cuts_out = nullptr;
    ra.n0c = t->d_n0c;
    ra.t2cap = (int32_t)std::min<int64_t>(floor_ratio(t->t2, n), INT32_MAX);
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

  // ---- every buffer this reassignment can need, before any state changes:
  // F holds every moved row once; the ops block is bounded by a few ops per
  // changed row; the resident write-back packs hold the entrants.
  const DeltaTotals tot = delta_totals(t);
  void* fbase = nullptr;    // F
  char* d_opsbuf = nullptr;  // ops block, device
  char* h_opsbuf = nullptr;  // its host staging
  size_t ops_cap = 0;
  std::vector<char> h_pageable;  // host staging of the static variant (no pinned allocation)
  {
    // positional staging: every moved row is read where it sits, F is not needed
    const int64_t Fmax = t->positional ? 0 : tot.e1 + tot.e2 + tot.p;
    const size_t f_need = 2 * (size_t)L * H * Fmax * hb;
    const size_t ops_max = (size_t)tot.all * (4 * sizeof(RowOp) + sizeof(DequantOp) + sizeof(QuantOp) +
                                              3 * sizeof(LocUpdate) + sizeof(RowOp));
    if (use_static) {
      void* base = nullptr;
      size_t cap = 0;
      if (int rc = static_scratch(t, &base, &cap)) return rc;
      const size_t f_al = (f_need + 255) / 256 * 256;
      if (f_al + ops_max > cap)
        return tkv_fail(t, TKV_ECAPACITY,
                        "reassignment needs %zu bytes of scratch; the static scratch holds %zu (use tkv_reassign)",
                        f_al + ops_max, cap);
      fbase = base;
      d_opsbuf = (char*)base + f_al;
      ops_cap = ops_max;
      h_pageable.resize(ops_max);
      h_opsbuf = h_pageable.data();
    } else {
      int rc = grow_device(t, &t->fpack, &t->fpack_bytes, f_need);
      if (!rc && ops_max) rc = grow_pinned(t, &t->h_ops, &t->h_ops_bytes, ops_max);
      if (!rc && ops_max) rc = grow_device(t, &t->d_ops, &t->d_ops_bytes, ops_max);
      if (rc) return rc;  // nothing has changed: the handle stays as it was
      fbase = t->fpack;
      d_opsbuf = (char*)t->d_ops;
      h_opsbuf = (char*)t->h_ops;
      ops_cap = std::min(t->h_ops_bytes, t->d_ops_bytes);
    }
  }
  std::swap(t->tier, t->tier_alt);  // device labels are now the new ones
  // from here on a failure leaves device and host state apart
  struct Poison {
    tkv* t;
    bool done = false;
    ~Poison() {
      if (!done) t->failed = true;
    }
  } poison{t};

  // ---- placement plan (host mirror of tiers, locations, free slots, arenas)
  PlanConfig pc{B, t->nmax, n, t->cap0, t->cap1, t->cap2, t->positional, t->shared_hbm};
  PlanState ps{&t->h_tier,  &t->h_loc,    &t->h_aidx,  &t->free0, &t->t1_owner,
               &t->t2_owner, &t->t1_free, &t->t2_free, &t->nlive};
  PlanResult pr;
  {
    std::string why;
    const int rc = make_plan(pc, ps, t->h_counts, t->h_promote, t->h_demote, &pr, &why);
    if (rc) return tkv_fail(t, rc, "%s", why.c_str());
  }
  const std::vector<SeqPlan>& plan = pr.seq;
  const std::vector<LocUpdate>& upd = pr.upd;
  const int64_t E1 = pr.e1, E2 = pr.e2, P = pr.p;
  const uint32_t c2 = (uint32_t)(t->cap0 + t->cap1);

  // ---- F layout: [rows entering T1 | rows entering T2 | promotions]
  const int64_t F = E1 + E2 + P;
  const size_t f_bytes = (size_t)L * H * F * hb;  // per K|V
  FPack fp{fbase, (char*)fbase + f_bytes, F};

  // ---- ops
  // ops1: phase 1 fetch into F; ops2a: promotions (+ resident staging
  // compaction); ops2b: resident staging entrants; am1/am2: arena compaction
  // (T1, T2); ae1: T1 entrants into the arena; q2: T2 entrants quantised into
  // the arena
  std::vector<RowOp> ops1, ops2a, ops2b, am1, am2, ae1;
  std::vector<DequantOp> dq1;
  std::vector<QuantOp> q2;
  auto fetch = [&](int b, const Move& mv, uint32_t frow) {
    if (mv.kind == kFromPool) {
      ops1.push_back({kAreaPool, kAreaPackOut, (uint16_t)b, mv.idx, frow});
    } else if (t->resident) {
      const uint32_t sidx = mv.kind == kFromT1 ? mv.idx : (uint32_t)t->cap1 + mv.idx;
      ops1.push_back({kAreaStage, kAreaPackOut, (uint16_t)b, sidx, frow});
    } else if (mv.kind == kFromT1) {
      ops1.push_back({kAreaArena1, kAreaPackOut, (uint16_t)b, mv.idx, frow});  // over PCIe
    } else {
      dq1.push_back({(uint16_t)b, mv.idx, frow});  // 8-bit row over PCIe, dequantised
    }
  };
  for (int b = 0; b < B; ++b) {
    const SeqPlan& sp = plan[b];
    if (t->positional) {
      // rows stay at their positions: entrants go to their arenas from there
      for (size_t e = 0; e < sp.ent1.size(); ++e)
        ae1.push_back({kAreaPool, kAreaArena1, (uint16_t)b, sp.ent1[e].pos, sp.dst1[e]});
      for (size_t e = 0; e < sp.ent2.size(); ++e)
        q2.push_back({(uint16_t)b, sp.ent2[e].pos, sp.dst2[e], sp.ent2[e].pos});
      continue;
    }
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
    // the pinned arenas: compaction, then the entrants at the end
    for (auto& mv : sp.mov1) am1.push_back({kAreaArena1, kAreaArena1, (uint16_t)b, mv.first, mv.second});
    for (auto& mv : sp.mov2) am2.push_back({0, 0, (uint16_t)b, mv.first, mv.second});
    for (size_t e = 0; e < sp.ent1.size(); ++e)
      ae1.push_back({kAreaPackOut, kAreaArena1, (uint16_t)b, (uint32_t)(sp.e1off + e), sp.dst1[e]});
    // T2 entrants: codes and scales into the arena; the dequantised values go
    // to the row's new staging place (resident) or nowhere (stream)
    for (size_t e = 0; e < sp.ent2.size(); ++e)
      q2.push_back({(uint16_t)b, (uint32_t)(E1 + sp.e2off + e), sp.dst2[e],
                    t->resident ? c2 + sp.dst2[e] : kNoLoc});
  }

  // ---- ops and location updates to the device (buffers grown above)
  const size_t bytes = (ops1.size() + ops2a.size() + ops2b.size() + am1.size() + am2.size() + ae1.size()) *
                           sizeof(RowOp) +
                       dq1.size() * sizeof(DequantOp) + q2.size() * sizeof(QuantOp) + upd.size() * sizeof(LocUpdate);
  if (bytes > ops_cap)
    return tkv_fail(t, TKV_EHIP, "internal error: reassignment ops (%zu bytes) exceed their buffer", bytes);
  const RowOp *d_ops1 = nullptr, *d_ops2a = nullptr, *d_ops2b = nullptr, *d_am1 = nullptr, *d_am2 = nullptr,
              *d_ae1 = nullptr;
  const DequantOp* d_dq1 = nullptr;
  const QuantOp* d_q2 = nullptr;
  const LocUpdate* d_upd = nullptr;
  if (bytes > 0) {
    char* h = h_opsbuf;
    char* d = d_opsbuf;
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
    d_am1 = (const RowOp*)put(am1.data(), am1.size() * sizeof(RowOp));
    d_am2 = (const RowOp*)put(am2.data(), am2.size() * sizeof(RowOp));
    d_ae1 = (const RowOp*)put(ae1.data(), ae1.size() * sizeof(RowOp));
    d_dq1 = (const DequantOp*)put(dq1.data(), dq1.size() * sizeof(DequantOp));
    d_q2 = (const QuantOp*)put(q2.data(), q2.size() * sizeof(QuantOp));
    d_upd = (const LocUpdate*)put(upd.data(), upd.size() * sizeof(LocUpdate));
    HIP_TRY(t, hipMemcpyAsync(d_opsbuf, h_opsbuf, bytes, hipMemcpyHostToDevice, st));
  }

  // ---- device phases.  The caller's stream first waits for the last
  // reassignment's arena work (it read F, which phase 1 overwrites).
  if (t->arena_pending) HIP_TRY(t, hipStreamWaitEvent(st, t->ev_arena, 0));
  const ArenaSpace arena = t->arenaspace();
  CopyArgs ca{};
  ca.rows = t->rowspace();
  ca.arena = arena;
  ca.kv_heads = H;
  ca.head_bytes = (int32_t)hb;
  ca.elem_bytes = t->esz;
  ca.pack_out_k = fp.k;  // F
  ca.pack_out_v = fp.v;
  ca.pack_out_rows = F;
  const int fp8 = (t->flags & TKV_FLAG_T2_FP8) ? 1 : 0;
  HIP_TRY(t, launch_copy_rows(ca, d_ops1, (int)ops1.size(), L, 0, st));
  DequantArgs dqa{arena, fp, H, D, t->esz, fp8, t->sh};
  HIP_TRY(t, launch_dequant_rows(dqa, d_dq1, (int)dq1.size(), L, st));
  HIP_TRY(t, launch_copy_rows(ca, d_ops2a, (int)ops2a.size(), L, 0, st));
  HIP_TRY(t, launch_copy_rows(ca, d_ops2b, (int)ops2b.size(), L, 0, st));
  // The T2 arena on this stream: compaction (every fetch from it is done; a
  // move's source, a kept row past the new size, is no op's destination),
  // then the entrants past the kept rows, whose dequantised values the next
  // step reads.
  HIP_TRY(t, launch_arena2_moves(arena, d_am2, (int)am2.size(), L, D, kArenaBlocks, st));
  if (E2 > 0) {
    QuantArgs qa{t->rowspace(), fp, arena, H, D, t->esz, fp8, t->sh, t->positional ? 1 : 0};
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
  // The T1 arena the same way.  Stream staging: on this stream, before the
  // next step's copies read it.  Resident staging (no kernel reads the
  // arena): on the write-back stream, beside the next steps, from a few
  // work-groups that loop over the rows.
  hipStream_t as = st;
  if (!stream_mode) {
    HIP_TRY(t, hipEventRecord(t->ev_gathered, st));
    HIP_TRY(t, hipStreamWaitEvent(t->wb, t->ev_gathered, 0));
    as = t->wb;
  }
  const int wblocks = stream_mode ? kArenaBlocks : kWritebackBlocks;
  HIP_TRY(t, launch_copy_rows(ca, d_am1, (int)am1.size(), L, wblocks, as));
  HIP_TRY(t, launch_copy_rows(ca, d_ae1, (int)ae1.size(), L, wblocks, as));
  HIP_TRY(t, hipEventRecord(t->ev_arena, as));
  t->arena_pending = true;
  {
    const size_t qrow = (size_t)D;  // bytes of one head's 8-bit row
    int64_t h2d = 0;
    for (const RowOp& o : ops1) h2d += o.src_area == kAreaArena1 ? 2 * (int64_t)L * H * hb : 0;
    h2d += (int64_t)dq1.size() * 2 * L * (H * qrow + t->sh * 4);
    t->st.h2d_bytes += h2d;
    t->st.d2h_bytes += 2 * (int64_t)L * H * (E1 * hb + E2 * qrow) + 2 * (int64_t)L * E2 * t->sh * 4;
  }

  if (use_static) HIP_TRY(t, hipEventSynchronize(t->ev_arena));  // nothing reads the scratch after return
  poison.done = true;
  t->st.promotions += pr.promotions;
  t->st.demotions += pr.demotions;
  t->st.evictions += pr.evictions;
  t->st.reassigns += 1;
  t->st.reassign_ms +=
      std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - wall0).count();
  return TKV_OK;
}
extern "C" int tkv_reassign(tkv_t* t, tkv_stream_t stream) {
  return guarded(t, [&] { return reassign_impl(t, stream, false); });
}

extern "C" int tkv_reassign_static(tkv_t* t, tkv_stream_t stream) {
  return guarded(t, [&] { return reassign_impl(t, stream, true); });
}
