// The tkv handle: configuration, device buffers, host-side placement state.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "tkv_internal.hpp"

enum class TkvState { Empty, Ready, InStep };

struct tkv {
  // ---- configuration
  int L = 0, Hq = 0, Hkv = 0, D = 0, B = 0, nmax = 0, dtype = 0, esz = 0, group = 0;
  int delta = 0, chunk = 256, S = 0;  // S = staging slots (== L when resident)
  bool resident = true;
  bool vector_pass = false;  // bf16 grouped-query heads on the vector units (TKV_FLAG_VECTOR_PASS)
  double hbm = 0, evict = 0, t2 = 0;
  int prompt = 0, sinks = 0, recent = 0;
  uint64_t flags = 0;
  int device = 0;        // the GPU current when the handle was created
  int64_t mem_cap = 0;   // most device + pinned bytes the handle may hold (0: no cap)
  int64_t mem_held = 0;  // device + pinned bytes held now
  int cap0 = 0, cap1 = 0, cap2 = 0, capS = 0, max_chunks = 0;  // capS: staging rows per slot
  int sh = 1;  // T2 scales per row: Hkv with per-head scales, else 1
  int lstride = 0;  // logits row stride: nmax rounded up to whole lines
  int64_t row_elems = 0, row_bytes = 0;

  // ---- device buffers (owned)
  void* pool_k = nullptr;  // [L][B][Hkv][cap0][D], or [L][Hkv][cap0][D] when the batch shares it
  void* pool_v = nullptr;
  void* stage_k = nullptr;  // [S][B][Hkv][capS][D]: T1 rows, then (resident) T2 values
  void* stage_v = nullptr;
  uint32_t* live_loc = nullptr;  // [B][nmax]
  int32_t* live_pos = nullptr;   // [B][nmax]
  uint8_t* tier = nullptr;       // [B][nmax]
  uint32_t* loc = nullptr;       // [B][nmax]
  float* s = nullptr;            // [B][nmax]
  float* logits = nullptr;       // [L][B][Hq][lstride]
  float* part_ml = nullptr;      // [L][B][Hq][max_chunks][2]
  float* part_o = nullptr;       // [L][B][Hq][max_chunks][D]
  float* layer_score = nullptr;  // [L][B][lstride]
  uint8_t* tier_alt = nullptr;   // [B][nmax] labels being computed by a reassignment
  uint64_t* d_cuts = nullptr;    // batch-shared budget: [B][3] cut keys of the select-only pass
  int32_t* d_n0c = nullptr;      // batch-shared budget: [B] T0 share from the joint select
  // changed rows of a reassignment, one block: counts [B][2] (padded to 16 B),
  // then promote [B][nmax], then demote [B][nmax]; mirrored in pinned host memory
  int32_t* d_counts = nullptr;
  tkv_delta* d_promote = nullptr;
  tkv_delta* d_demote = nullptr;
  size_t delta_block_bytes = 0;
  std::vector<void*> device_allocs;

  // growable device / pinned scratch of the reassignment
  void* d_ops = nullptr;
  size_t d_ops_bytes = 0;
  void* h_ops = nullptr;  // pinned staging of ops + loc updates
  size_t h_ops_bytes = 0;
  // device pack, persistent, grown on demand
  void* fpack = nullptr;       // F: every moved row's value, K then V, [L][Hkv][rows][D] each
  size_t fpack_bytes = 0;

  // ---- pinned host arenas (owned)
  void* arena1_k = nullptr;  // [L][B][Hkv][cap1][D]: T1 rows, dense per (layer, seq, head)
  void* arena1_v = nullptr;
  int8_t* arena2_k = nullptr;  // [L][B][Hkv][cap2][D]: T2 codes, dense per (layer, seq, head)
  int8_t* arena2_v = nullptr;
  float* ascale_k = nullptr;   // [L][B][cap2]: T2 scales
  float* ascale_v = nullptr;
  std::vector<void*> host_allocs;
  // the same arenas as the GPU addresses them (hipHostGetDevicePointer)
  void* d_arena1_k = nullptr;
  void* d_arena1_v = nullptr;
  int8_t* d_arena2_k = nullptr;
  int8_t* d_arena2_v = nullptr;
  float* d_ascale_k = nullptr;
  float* d_ascale_v = nullptr;
  // stream staging: one layer's 8-bit rows per slot, as they crossed PCIe; the
  // attention pass reads the codes directly
  int8_t* qstage_k = nullptr;  // [S][B][Hkv][cap2][D]
  int8_t* qstage_v = nullptr;
  float* qsscale_k = nullptr;  // [S][B][cap2][sh]
  float* qsscale_v = nullptr;

  // ---- host-side placement state
  int n = 0;  // positions appended per sequence
  int64_t step = 0;
  int layers_done = 0;
  TkvState state = TkvState::Empty;
  // A reassignment failed after the device labels changed: host and device
  // placement state disagree, so every call but tkv_destroy, tkv_last_error
  // and tkv_stats returns TKV_ESTATE.
  bool failed = false;
  // The last completed step's Eq. 1 update of s, not yet applied: it runs
  // in the next append's launch, or before anything else reads or writes s.
  bool score_pending = false;
  tkvd::ScoreArgs pending_score{};
  int pending_tiles = 0;
  // Deferred Eq. 1 (bf16 on the matrix cores, resident staging): a step's
  // weights are recomputed, from its queries and its heads' (M, 1/L), by a
  // later step's attention launch, which streams the same K rows anyway, and
  // folded into s by that step's merge pass.  The logits tile and the
  // forming launch's extra tiles have room for kmax = defer_max_pending(g)
  // pending steps beside the running one (15 at g = 1, 11 at g = 4, 8 at
  // g = 5, 5 at g = 8), so a launch forms the pending steps' weights once
  // kmax are pending and writes one sum per row and kv head for all of them;
  // the launches in between form none.  A
  // reassignment first runs a score-only pass over K for the pending steps
  // and folds them into s; a score read folds them into a copy of s only, so
  // that reads never change which steps are summed together.  No logits are
  // stored.
  bool defer = false;
  int kmax = 1;                     // pending steps per forming launch
  int pend = 0;                     // steps whose weights are not in s yet (0..kmax)
  std::vector<int32_t> prev_nlive;  // [B] live rows of the last of them
  // rings of kmax + 1 slots: the last completed step's queries and (M, 1/L)
  // at slot qcur, the one before it at qcur - 1 (mod ring); the running
  // step's go to (qcur + 1) mod ring
  int ring = 2, qcur = 0;
  void* qring = nullptr;     // [ring][L][B][Hq][D]
  float* mlring = nullptr;   // [ring][L][B][Hq][2]
  float* spart = nullptr;              // [L][Hkv][B][lstride]
  float* s_view = nullptr;             // [B][nmax]: s with the pending steps folded in, for reads
  std::vector<int32_t> nlive;                 // [B] live rows
  std::vector<std::vector<int32_t>> free0;    // [B] free T0 slots (back = next to use); [1] when shared
  bool shared_hbm = false;                    // one T0 slot space and budget for the batch
  // Positional resident staging: every live row, whatever its tier, sits in
  // the pool at its own position (location code = position), so the pass
  // reads each region in order and a reassignment moves no row inside HBM.
  // T1/T2 rows keep their pinned homes; h_aidx holds their arena index.
  bool positional = false;
  std::vector<uint32_t> h_aidx;               // [B][nmax] (positional only)
  std::vector<int32_t>& free_list(int b) { return free0[shared_hbm ? 0 : b]; }
  std::vector<uint8_t> h_tier;                // [B][nmax]
  std::vector<uint32_t> h_loc;                // [B][nmax]
  std::vector<std::vector<int32_t>> t1_owner; // [B]: T1 arena index -> position (-1: free, positional only)
  std::vector<std::vector<int32_t>> t2_owner; // [B]: T2 arena index -> position (-1: free, positional only)
  std::vector<std::vector<int32_t>> t1_free;  // [B]: freed T1 arena indices (positional only)
  std::vector<std::vector<int32_t>> t2_free;  // [B]: freed T2 arena indices (positional only)

  // ---- last reassignment's changed rows (pinned host copy of the device block)
  int32_t* h_counts = nullptr;     // [B][2]
  tkv_delta* h_promote = nullptr;  // [B][nmax]
  tkv_delta* h_demote = nullptr;   // [B][nmax]

  // ---- streams and events
  hipStream_t side = nullptr;           // host->device row traffic of the stream mode (K rows, 8-bit rows)
  hipStream_t side_v = nullptr;         // the same for V rows: two copy queues overlap their gaps (stream staging only)
  hipStream_t wb = nullptr;             // resident staging: the T1 arena's reassignment kernels
  hipEvent_t ev_gathered = nullptr;     // resident staging: rows entering T1 are in F
  std::vector<hipEvent_t> ev_h2d;       // [S] staging slot filled (side)
  std::vector<hipEvent_t> ev_h2d_v;     // [S] its V rows filled (side_v)
  std::vector<hipEvent_t> ev_comp;      // [S] attention done reading the slot
  std::vector<char> comp_recorded;      // [S]
  hipEvent_t ev_arena = nullptr;        // the last reassignment's arena kernels are done
  bool arena_pending = false;
  int next_issue = 0;                   // next layer whose staging copy is to be issued this step

  // ---- stats and timing
  tkv_stats_t st{};
  std::vector<hipEvent_t> ev_free;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev_pending;

  std::string err;

  // ---- per-layer HBM budgets
  // The handle the caller holds: one part per group of consecutive layers with
  // one ratio, each a whole handle over its layers (empty otherwise).  The
  // parts share this handle's score array s.
  std::vector<tkv*> parts;
  std::vector<int> part_l0;   // first layer of each part
  // In a part: s belongs to the handle of the parts (not freed here), and
  // Eq. 1 averages over score_layers layers (all of that handle's).
  bool s_shared = false;
  int score_layers = 0;
  // Eq. 1's 1 / (layers * q_heads) over the layers the scores average over
  double inv_lh() const { return 1.0 / ((double)(score_layers ? score_layers : L) * Hq); }

  tkvd::ArenaSpace arenaspace() const {
    tkvd::ArenaSpace a{};
    a.a1_k = d_arena1_k;
    a.a1_v = d_arena1_v;
    a.a2_k = d_arena2_k;
    a.a2_v = d_arena2_v;
    a.s2_k = d_ascale_k;
    a.s2_v = d_ascale_v;
    a.batch = B;
    a.kv_heads = Hkv;
    a.cap1 = cap1;
    a.cap2 = cap2;
    a.sh = sh;
    return a;
  }

  tkvd::RowSpace rowspace() const {
    tkvd::RowSpace r{};
    r.pool_k = pool_k;
    r.pool_v = pool_v;
    r.stage_k = stage_k;
    r.stage_v = stage_v;
    r.pool_hstride = (int64_t)cap0 * D;
    r.pool_bstride = shared_hbm ? 0 : r.pool_hstride * Hkv;
    r.pool_lstride = r.pool_hstride * Hkv * (shared_hbm ? 1 : B);
    r.stage_hstride = (int64_t)capS * D;
    r.stage_bstride = r.stage_hstride * Hkv;
    r.stage_lstride = r.stage_bstride * B;
    r.q_k = qstage_k;
    r.q_v = qstage_v;
    r.qs_k = qsscale_k;
    r.qs_v = qsscale_v;
    r.q_hstride = (int64_t)cap2 * D;
    r.q_bstride = r.q_hstride * Hkv;
    r.q_lstride = r.q_bstride * B;
    r.qs_bstride = (int64_t)cap2 * sh;
    r.qs_lstride = (int64_t)cap2 * sh * B;
    r.cap0 = cap0;
    r.cap1 = cap1;
    r.cap2 = cap2;
    r.stage_slots = S;
    r.q_fp8 = (flags & TKV_FLAG_T2_FP8) ? 1 : 0;
    r.q_sh = sh;
    return r;
  }
};
