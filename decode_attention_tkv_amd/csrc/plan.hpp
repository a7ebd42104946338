// Host placement logic of the tiers, free of HIP: tier budgets, the first
// placement, and the plan of a reassignment ("Not All Thoughts Need HBM",
// gist.science technical summary, Method §1 four tiers with the prompt,
// sinks and recent window always in T0; Method §4 periodic re-placement
// where only changed rows move).  The library calls it; the CPU unit test
// (tests/cpp/test_plan.cpp) builds it on its own, with sanitizers.
#pragma once

#include <cstdint>
#include <string>
#include <utility>
#include <vector>

#include "../../include/tkv.h"

namespace tkvd {

constexpr uint32_t kNoLoc = 0xFFFFFFFFu;  // loc code of evicted / unused positions
constexpr uint8_t kUnused = 255;           // tier code of positions not appended yet

// floor(ratio * n) in fp64: the tier budgets of Method §1.
int64_t floor_ratio(double r, int64_t n);

// Protected positions of a sequence holding n positions: [0, prompt),
// [0, sinks) and the last `recent` (Method §1: prompt, sinks, recent window).
inline bool protected_at(int64_t i, int64_t n, int prompt, int sinks, int recent) {
  return i < prompt || i < sinks || i >= n - recent;
}

// Placement of a freshly filled cache before any score exists: protected
// rows plus the lowest positions in T0 up to floor(hbm * n), the rest T1
// (evicted instead of T1 under the eviction-only policy).
std::vector<uint8_t> first_placement(int n, int prompt, int sinks, int recent, double hbm, bool no_t1);

// Candidates newly evicted (n3), kept in T0 (n0c) and put in T2 (n2) at one
// reassignment of a sequence with n positions, np protected and nev already
// evicted (Method §1 budgets as floor(ratio * n)).
struct CutCounts {
  int64_t n3, n0c, n2;
};
CutCounts cut_counts(int64_t n, int64_t np, int64_t nev, double hbm, double evict, double t2, bool no_t1);

// One row update of the location table (position pos of sequence b -> code).
struct LocUpdate {
  int32_t b;
  uint32_t pos;
  uint32_t code;
};

enum SrcKind : uint8_t { kFromPool, kFromT1, kFromT2 };

struct Move {
  uint32_t pos;
  SrcKind kind;
  uint32_t idx;  // pool slot, T1 index or T2 index
};

// What a reassignment does to one sequence.
struct SeqPlan {
  std::vector<Move> ent1, ent2, promo;  // rows entering T1, T2 and T0
  std::vector<uint32_t> promo_slot;
  std::vector<uint32_t> dst1, dst2;     // arena index of each entrant
  std::vector<std::pair<uint32_t, uint32_t>> mov1, mov2;  // arena compaction (src, dst)
  uint32_t m1 = 0, m2 = 0;              // dense arenas: rows kept before the entrants
  int64_t e1off = 0, e2off = 0, poff = 0;  // offsets within the F segments
};

// Dense-arena compaction: indices marked vacated leave; the kept rows above
// the new size m move down into the holes below it, in order.
void compact(std::vector<int32_t>& own, const std::vector<char>& vac, uint32_t* m,
             std::vector<std::pair<uint32_t, uint32_t>>* moves);

struct PlanConfig {
  int batch, nmax, n;     // sequences, position capacity, positions appended
  int cap0, cap1, cap2;   // T0 pool slots (per sequence, or of the batch when shared), arena capacities
  bool positional;        // every live row at its own position (resident staging)
  bool shared;            // one T0 slot space for the batch
};

// The host mirror of the placement, updated in place by make_plan.
// Arenas: dense (index < size holds a row) except under positional staging,
// where nothing reads them on the decode path and rows entering take freed
// indices (own = -1 there; free1/free2 list them, back() = lowest) instead
// of the arena being compacted.
struct PlanState {
  std::vector<uint8_t>* tier;                  // [batch][nmax]
  std::vector<uint32_t>* loc;                  // [batch][nmax] location codes
  std::vector<uint32_t>* aidx;                 // [batch][nmax] arena index (positional only)
  std::vector<std::vector<int32_t>>* free0;    // free T0 slots, back() next ([1] when shared)
  std::vector<std::vector<int32_t>>* own1;     // [batch] T1 arena index -> position (-1: free)
  std::vector<std::vector<int32_t>>* own2;     // [batch] T2 arena index -> position (-1: free)
  std::vector<std::vector<int32_t>>* free1;    // [batch] freed T1 arena indices (positional only)
  std::vector<std::vector<int32_t>>* free2;    // [batch] freed T2 arena indices (positional only)
  std::vector<int32_t>* nlive;                 // [batch] live rows
};

struct PlanResult {
  std::vector<SeqPlan> seq;
  std::vector<LocUpdate> upd;
  int64_t e1 = 0, e2 = 0, p = 0, evictions = 0, promotions = 0, demotions = 0;
};

// Plan a reassignment from its changed-row lists (counts [batch][2] =
// {promote, demote}; lists [batch][nmax], ascending by position): every
// freed T0 slot returns to its free list before any promotion takes one;
// promotions take T0 slots (none under positional staging, where rows stay
// put); dense arenas compact and take their entrants at the end, in
// position order (positional staging: entrants take the lowest freed
// indices, then new ones); the location updates follow.  TKV_OK, or TKV_ECAPACITY (with *err)
// when the T0 pool or an arena overflows -- the state is then partly
// updated.
int make_plan(const PlanConfig& cfg, PlanState& st, const int32_t* counts, const tkv_delta* promote,
              const tkv_delta* demote, PlanResult* out, std::string* err);

}  // namespace tkvd
