// Internal declarations of the tkv library: handle state, kernel argument
// blocks and kernel launchers.  Host code (api.cpp, reassign.cpp) and the
// HIP kernels (attn.hip, reassign.hip, move.hip) include this.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/tkv.h"
#include "plan.hpp"

namespace tkvd {

constexpr int kMaxBatch = 64;
constexpr int kMaxQHeads = 256;

// ---- kernel argument blocks (passed by value) ------------------------------

// Where the K/V rows live.  Every area is head-major:
// [..][batch][kv_heads][cap][head_dim], so the rows of one kv head are
// contiguous (head_dim elements apart).  A live row's location code `loc` is
// a T0 pool slot when loc < cap0, else index (loc - cap0) of the staging area
// of slot (layer % stage_slots): T1 rows first, then (resident staging) the
// T2 rows' dequantised values from index cap1.  Stream staging instead
// carries a layer's T2 rows as the 8-bit codes and scales that crossed PCIe
// (q_k != nullptr): codes >= cap0 + cap1 are rows of that area, and the
// attention pass dequantises them as it reads them.
struct RowSpace {
  const void* pool_k;
  const void* pool_v;
  const void* stage_k;
  const void* stage_v;
  int8_t* q_k;  // stream staging: T2 codes [stage_slots][batch][kv_heads][cap2][head_dim]; else null
  int8_t* q_v;
  float* qs_k;  // T2 scales [stage_slots][batch][cap2][q_sh]
  float* qs_v;
  int64_t pool_lstride, pool_bstride, pool_hstride;     // elements per layer / sequence / kv head
  int64_t stage_lstride, stage_bstride, stage_hstride;  // elements per slot / sequence / kv head
  int64_t q_lstride, q_bstride, q_hstride;              // T2 codes per slot / sequence / kv head
  int64_t qs_lstride, qs_bstride;                       // T2 scales per slot / sequence
  int32_t cap0, cap1, cap2;
  int32_t stage_slots;
  int32_t q_fp8;  // T2 codes are FP8 E4M3 (else int8)
  int32_t q_sh;   // T2 scales per row: kv_heads (one per head) or 1
};

// T2 area offsets: codes of row idx (kv head h) of layer l's slot, and its scale.
__host__ __device__ inline int64_t q_codes_at(const RowSpace& r, int l, int b, int h, uint32_t idx, int d) {
  return (int64_t)(l % r.stage_slots) * r.q_lstride + (int64_t)b * r.q_bstride + (int64_t)h * r.q_hstride +
         (int64_t)idx * d;
}
__host__ __device__ inline int64_t q_scale_at(const RowSpace& r, int l, int b, uint32_t idx) {
  return (int64_t)(l % r.stage_slots) * r.qs_lstride + (int64_t)b * r.qs_bstride + (int64_t)idx * r.q_sh;
}

// Logits and per-layer score rows are padded to kLogitAlign floats, so every
// chunk's stores start on a line boundary.
constexpr int kLogitAlign = 64;

// Deferred Eq. 1 on the matrix cores: a 16-row logits tile holds 16 / g
// steps' query heads (g per step).  The running step's tile holds it and
// 16 / g - 1 pending steps; a launch that forms pending steps (or a
// score-only pass) adds defer_extra_tiles(g) more tiles of 16 / g pending
// steps each, their queries staged in LDS, so that with few steps per tile
// the weight sums are still written only once per several steps.
constexpr int defer_steps_per_tile(int g) { return 16 / g; }
constexpr int defer_extra_tiles(int g) { return g >= 4 ? 2 : 0; }
constexpr int defer_max_pending(int g) { return defer_steps_per_tile(g) * (1 + defer_extra_tiles(g)) - 1; }

struct AttnArgs {
  RowSpace rows;
  const uint32_t* live_loc;  // [batch][nmax] loc code of live index j (ascending position)
  const void* q;             // [layer_count][batch][q_heads][head_dim]
  float* logits;             // [layers][batch][q_heads][lstride], log2-scaled q.k/sqrt(d)
  float* part_ml;            // [layers][batch][q_heads][max_chunks][2] chunk (max, sum)
  float* part_o;             // [layers][batch][q_heads][max_chunks][head_dim]
  float qscale;              // log2(e) / sqrt(head_dim)
  int32_t layer_begin, batch, q_heads, kv_heads, nmax, max_chunks, lstride;
  // Deferred Eq. 1 (matrix-core path, resident staging): the weights of the
  // last prev_steps steps are recomputed from their queries while this launch
  // streams K.
  //   prev_mode 0: none; 1: this step's launch, the last pending step's rows
  //   are live indices < nlive - 1; 2: score only (flush), rows < nlive, no
  //   attention.  Each earlier pending step has one row fewer.
  // Queries and (M, 1/L) of recent steps sit in rings of `ring` slots: the
  // last completed step in slot qcur, the one before it in qcur - 1 (mod
  // ring), and so on; the merge pass puts this step's in slot
  // (qcur + 1) mod ring.
  int32_t prev_mode, prev_steps;
  int32_t ring, qcur;
  void* qring;          // [ring][layers][batch][q_heads][head_dim]
  float* mlring;        // [ring][layers][batch][q_heads][2], log2 units
  int64_t qslot, mlslot; // elements per slot
  float* spart;         // [layers][kv_heads][batch][lstride]: sum over the pending heads of alpha
  int32_t nlive[kMaxBatch];
};

struct FinalizeArgs {
  const float* logits;
  const float* part_ml;
  const float* part_o;
  float* out;     // [layer_count][batch][q_heads][head_dim] fp32
  float* layer_score;  // [layers][batch][lstride]: sum over heads of alpha, per live index
  int32_t layer_begin, batch, q_heads, nmax, max_chunks, chunk, lstride;
  int32_t tiles_grid;  // score blocks in the grid (tiles of the longest sequence; set by the launcher)
  float* mlprev;       // deferred Eq. 1: (M, 1/L) of every head kept for later steps (a ring slot), or null
  const void* q;       // deferred Eq. 1: the step's queries [layer_count][batch][q_heads][head_dim] (bf16)
  void* qsave;         // deferred Eq. 1: their ring slot [layers][batch][q_heads][head_dim], or null
  int32_t fold_tiles;  // deferred Eq. 1: tiles of the fold of `fold` run by layer-0 blocks (0: none)
  int32_t nlive[kMaxBatch];
};

struct ScoreArgs {
  const float* layer_score;  // [layers][batch][lstride]
  const int32_t* live_pos;   // [batch][nmax]
  float* s;                  // [batch][nmax] by position
  float inv_lh;              // 1 / (layers * q_heads)
  int32_t layers, batch, nmax, lstride;
  int32_t parts;             // deferred fold: partial sums per row (4, or 16 for lists over 640 rows)
  int32_t nlive[kMaxBatch];
};

struct AppendArgs {
  RowSpace rows;
  const void* k;  // [layers][batch][kv_heads][head_dim]
  const void* v;
  uint32_t* live_loc;
  int32_t* live_pos;
  uint8_t* tier;
  uint32_t* loc;
  float* s;
  int32_t layers, batch, kv_heads, head_dim, elem_bytes, nmax, pos;
  int32_t slot[kMaxBatch];
  int32_t nlive[kMaxBatch];
};

// The append and the pending Eq. 1 update, carried out by the attention launch
// of a whole step (resident staging only).  The new token's row is live index
// nlive - 1 of every sequence; the attention blocks read it from k / v and
// the block whose chunk holds it also writes it to T0 slot slot[b].  With
// fold set, blocks (chunk, kv head 0, layer 0) apply `f` to the 256-row tiles
// that start in their chunk.  k == nullptr: neither (a plain attention launch).
struct StepArgs {
  const void* k;  // [layers][batch][kv_heads][head_dim]
  const void* v;
  uint32_t* live_loc;
  int32_t* live_pos;
  uint8_t* tier;
  uint32_t* loc;
  float* s;
  int32_t pos;
  int32_t fold;
  ScoreArgs f;
  int32_t slot[kMaxBatch];
};

// Location code that stands for the row being appended in a step launch.
constexpr uint32_t kNewRow = 0xFFFFFFFEu;

// Place input rows [layers][batch][n_tokens][row] at their location codes
// (codes [batch][n_tokens]; kNoLoc = skip).
struct PlaceArgs {
  RowSpace rows;
  const void* k;
  const void* v;
  const uint32_t* codes;
  int32_t batch, n_tokens, kv_heads, head_bytes, elem_bytes;
};

// ---- reassignment (reassign.hip) ---------------------------------------------
struct RankArgs {
  const float* s;
  const uint8_t* tier_old;
  uint8_t* tier_new;
  int32_t nmax, n, prompt, sinks, recent;
  int32_t ncand[kMaxBatch];    // candidates (live, unprotected) per sequence
  int32_t rank[kMaxBatch][3];  // ascending-rank cut points: first non-T3, first non-T2, first T0
  // cuts_out set: only find the cut keys and store them ([batch][3]); no labels
  uint64_t* cuts_out;
  // batch-shared HBM budget: the T0 count of each sequence comes from the
  // joint select on the device; then rank[b][1] = n3 + min(ncand - n3 - n0c,
  // t2cap) and rank[b][2] = ncand - n0c, with n3 = rank[b][0]
  const int32_t* n0c;
  int32_t t2cap;
};

// Batch-shared HBM budget: one select over the remaining candidates of every
// sequence (per-sequence key at or above cut3[b], the sequence's lowest
// kept key), ordered by the joint key (bits(s) << 32) | ((63 - b) << 26) |
// (2^26 - 1 - position): best score first, then lower sequence, then lower
// position.  The `take` best go to T0; n0c[b] counts those of sequence b.
struct JointArgs {
  const float* s;
  const uint8_t* tier_old;
  const uint64_t* cuts;  // [batch][3] from the select-only rank pass; [b][0] = cut3
  int32_t* n0c;          // [batch] out
  int32_t nmax, n, prompt, sinks, recent, batch;
  int64_t remaining, take;
};

struct DeltaArgs {
  const uint8_t* tier_old;
  const uint8_t* tier_new;
  tkv_delta* promote;  // [batch][nmax]
  tkv_delta* demote;   // [batch][nmax]
  int32_t* counts;     // [batch][2]
  int32_t nmax, n;
};

struct LiveArgs {
  const uint8_t* tier;
  const uint32_t* loc;
  int32_t* live_pos;
  uint32_t* live_loc;
  int32_t nmax, n;
};

// The pinned host arenas (the home of T1 and T2 rows) as kernels address
// them.  With stream staging a reassignment reads rows leaving an arena and
// writes rows entering it straight over PCIe, in stream order, so no host
// thread copies rows and no host pack is needed.
struct ArenaSpace {
  void* a1_k;   // T1 rows [layers][batch][kv_heads][cap1][head_dim], cache type
  void* a1_v;
  int8_t* a2_k; // T2 codes [layers][batch][kv_heads][cap2][head_dim]
  int8_t* a2_v;
  float* s2_k;  // T2 scales [layers][batch][cap2][sh]
  float* s2_v;
  int32_t batch, kv_heads, cap1, cap2, sh;
};

// Row areas of a copy op.  Packs are [layers][kv_heads][rows][head_dim].
enum : uint8_t { kAreaPool = 0, kAreaStage = 1, kAreaPackOut = 2, kAreaArena1 = 3 };

struct RowOp {
  uint8_t src_area, dst_area;
  uint16_t b;
  uint32_t src, dst;
};

struct CopyArgs {
  RowSpace rows;
  ArenaSpace arena;
  void* pack_out_k;
  void* pack_out_v;
  int64_t pack_out_rows;
  int32_t kv_heads, head_bytes, elem_bytes;  // head_bytes = head_dim * elem_bytes
};

// ---- 8-bit host tier codec (codec.hip) ---------------------------------------
// Fetch pack F: every moved row's value, [layers][kv_heads][rows][head_dim]
struct FPack {
  void* k;
  void* v;
  int64_t rows;
};

struct QuantOp {
  uint16_t b;
  uint32_t src;    // F row
  uint32_t dst;    // T2 arena index
  uint32_t stage;  // location code that receives the dequantised values (pool slot, or cap0 +
                   // staging index), or kNoLoc
};

// Rows entering T2: F row src (from_pool: pool slot src of sequence b)
// quantised into T2 arena index dst of sequence b (codes [layers][batch]
// [kv_heads][cap2][head_dim], scales [layers][batch][cap2][sh]).
struct QuantArgs {
  RowSpace rows;
  FPack f;
  ArenaSpace arena;
  int32_t kv_heads, head_dim, elem_bytes;
  int32_t fp8;  // FP8 E4M3 codes (else int8)
  int32_t sh;   // scales per row: kv_heads or 1
  int32_t from_pool;
};

// T2 arena row src of sequence b -> cache-type values in F row dst.
struct DequantOp {
  uint16_t b;
  uint32_t src;
  uint32_t dst;
};

struct DequantArgs {
  ArenaSpace arena;
  FPack f;
  int32_t kv_heads, head_dim, elem_bytes;
  int32_t fp8;
  int32_t sh;
};

// Scored prefill: inputs k [layers][batch][n][kv_heads][d], q [layers][batch][n][q_heads][d]
// (cache type); scratch row_max, row_inv, colsum [layers][batch][q_heads][n] fp32; the
// scores s[b][j] (row stride nmax) are set for j < n.
struct PrefillScoreArgs {
  const void* k;
  const void* q;
  float* row_max;
  float* row_inv;
  float* colsum;
  float* s;
  float qscale;  // log2(e) / sqrt(head_dim)
  float inv_lh;  // 1 / (layers * q_heads)
  int32_t layers, batch, q_heads, kv_heads, n, nmax;
};

// ---- launchers (prefill.hip) ------------------------------------------------
hipError_t launch_prefill_scores(const PrefillScoreArgs& a, int dtype, int head_dim, hipStream_t s);

// ---- launchers (attn.hip) -------------------------------------------------
// fold != nullptr: the same launch also applies a pending Eq. 1 update
// (fold_tiles tiles of 256 live rows per sequence); the two touch disjoint data.
hipError_t launch_append(const AppendArgs& a, const ScoreArgs* fold, int fold_tiles, hipStream_t s);
// step: the fused append and Eq. 1 update of a whole-step launch, or k == nullptr.
// e0, e1 (may be null): events that take the kernel's own start and end times.
// vector_pass: bf16 grouped-query heads on the vector units instead of the matrix cores.
hipError_t launch_attn(const AttnArgs& a, const StepArgs& step, int dtype, int head_dim, int group, int chunk,
                       bool vector_pass, int layer_count, int chunks_now, hipEvent_t e0, hipEvent_t e1,
                       hipStream_t s);
// max_live: live rows of the longest sequence; the launcher sets tiles_grid.
// fold (or null): the deferred Eq. 1 sums to add to the scores, fold_tiles tiles of 64 rows per sequence
hipError_t launch_finalize(const FinalizeArgs& a, const ScoreArgs* fold, int fold_tiles, int head_dim,
                           int layer_count, int max_live, hipStream_t s);
hipError_t launch_score(const ScoreArgs& a, int tiles_now, hipStream_t s);
// deferred Eq. 1 fold (a.layers rows [layer][kv head]), tiles of 64 live rows
// Deferred fold of a.layer_score into s: tiles of 256 / a.parts live rows.
hipError_t launch_fold(const ScoreArgs& a, int tiles, hipStream_t s);

// ---- launchers (move.hip) -------------------------------------------------
hipError_t launch_place_rows(const PlaceArgs& a, int layers, hipStream_t s);
// A bounded delay on a stream (test hook): one wave sleeps `iters` times, then exits.
constexpr int kTestDelayIters = 200;  // about half a millisecond
hipError_t launch_delay(int iters, hipStream_t s);

// ---- launchers (reassign.hip) -----------------------------------------------
hipError_t launch_rank_label(const RankArgs& a, int batch, hipStream_t s);
hipError_t launch_joint_select(const JointArgs& a, hipStream_t s);
hipError_t launch_deltas(const DeltaArgs& a, int batch, hipStream_t s);
hipError_t launch_set_loc(const LocUpdate* u, int n, uint32_t* loc, int nmax, hipStream_t s);
hipError_t launch_build_live(const LiveArgs& a, int batch, hipStream_t s);
// max_blocks: at most this many work-groups, each looping over (op, layer, K|V)
// items (0: one per item).  Copies over PCIe into the pinned arenas use a few:
// their rate is PCIe's, and the fewer work-groups they hold, the more the
// attention running beside them keeps.
constexpr int kArenaBlocks = 32;     // on the caller's stream (stream staging)
constexpr int kWritebackBlocks = 8;  // beside the decode steps (resident staging)
hipError_t launch_copy_rows(const CopyArgs& a, const RowOp* ops, int n_ops, int layers, int max_blocks,
                            hipStream_t s);

// ---- launchers (codec.hip) --------------------------------------------------
hipError_t launch_quant_rows(const QuantArgs& a, const QuantOp* ops, int n_ops, int layers, hipStream_t s);
hipError_t launch_dequant_rows(const DequantArgs& a, const DequantOp* ops, int n_ops, int layers, hipStream_t s);
// T2 arena rows moved within the arena (codes and scales; ops' src/dst are arena indices)
hipError_t launch_arena2_moves(const ArenaSpace& a, const RowOp* ops, int n_ops, int layers, int head_dim,
                               int max_blocks, hipStream_t s);

}  // namespace tkvd
