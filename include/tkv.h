/*
 * tkv.h -- tiered-KV decode attention with cumulative attention scoring,
 * for AMD Instinct MI355X (gfx950).
 *
 * The method is the semantics-aware KV-cache hierarchy of "Not All Thoughts
 * Need HBM: Semantics-Aware Memory Hierarchy for LLM Reasoning" (arXiv
 * 2605.09490; gist.science technical summary and the arXiv abstract):
 *   - Method §1: every cache position sits in one of four tiers -- T0 (HBM;
 *     always holds the prompt, the attention sinks and the recent window),
 *     T1 (host DDR at full precision, brought to the GPU before attention),
 *     T2 (host, 8-bit), T3 (evicted for good).
 *   - Method §2, Eq. 1: per decode step, s_i += mean over layers and heads of
 *     the attention weight alpha_{l,h}[i].
 *   - Method §3, Proposition 1: T1 rows take part in attention at full
 *     precision, so outputs depend only on the evicted set, never on the
 *     T0/T1 split.  Here that holds bit for bit: the reduction order follows
 *     logical position, not where a row is stored.
 *   - Method §4: re-placement every Delta (default 64) steps; only rows whose
 *     tier changed are moved.
 *
 * Conventions for every call:
 *   - Return TKV_OK (0) or a negative tkv_status.  Nothing throws across the
 *     boundary.  tkv_last_error() gives the message of the last failure on a
 *     handle (or of the last failed tkv_create when passed NULL).
 *   - "device" pointers are HIP device memory (e.g. a torch tensor's
 *     data_ptr()); "host" pointers are ordinary CPU memory.  The caller owns
 *     every pointer it passes; the library owns everything it allocates.
 *   - Work is ordered on the caller's `stream` (a hipStream_t; NULL is the
 *     null stream).  Device buffers passed in must stay valid until that
 *     stream's work has completed.  Calls that return host data synchronise
 *     the stream.
 *   - A handle is used from one host thread at a time.
 *   - Layouts are dense row-major; element type is the handle's dtype (bf16
 *     bit patterns or fp32) unless stated.
 */
#ifndef TKV_H
#define TKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tkv tkv_t;
typedef void* tkv_stream_t; /* a hipStream_t */

typedef enum {
  TKV_OK = 0,
  TKV_EINVAL = -1,    /* bad argument: shape, ratio outside [0,1], delta <= 0, NULL pointer,
                         a device buffer (k, v, q, out) not 16-byte aligned */
  TKV_ECAPACITY = -2, /* more positions than max_tokens, the T0 pool is full, or a reassignment
                         needs more than the static scratch (tkv_reassign_static) */
  TKV_ENOMEM = -3,    /* device or pinned-host allocation failed, or past mem_cap_bytes */
  TKV_ESTATE = -4,    /* call out of order (e.g. reassign between layer groups of a step), or the
                         handle is marked failed after a reassignment failed part way */
  TKV_EHIP = -5       /* a HIP runtime call failed; see tkv_last_error */
} tkv_status;

typedef enum { TKV_BF16 = 0, TKV_F32 = 1 } tkv_dtype;
typedef enum { TKV_T0 = 0, TKV_T1 = 1, TKV_T2 = 2, TKV_T3 = 3 } tkv_tier;

/* Model and batch shape.  q_heads must be a multiple of kv_heads (query head
 * h reads kv head h / (q_heads / kv_heads)); head_dim is 64 or 128; batch is
 * 1..64; q_heads <= 256. */
typedef struct {
  int32_t layers, q_heads, kv_heads, head_dim, batch, max_tokens;
  int32_t dtype; /* tkv_dtype */
} tkv_shape;

/* Always-T0 positions of every sequence: [0, prompt), [0, sinks) and the
 * last `recent` positions (Method §1). */
typedef struct {
  int32_t prompt, sinks, recent;
} tkv_protect;

typedef struct {
  double t2_ratio;        /* share of positions held 8-bit on the host (T2); 0 = no T2 */
  int32_t staging_layers; /* S: HBM staging slots for T1/T2 rows.  0 or >= layers:
                             "resident": every live row stays in HBM, at its own position
                             (with TKV_FLAG_SHARED_HBM: T0 slots plus a staging mirror of
                             T1/T2), and only changed rows cross to or from the host.
                             2..layers-1: "stream": each step copies a layer's T1/T2 rows
                             from pinned host memory into slot (layer mod S), ahead of the
                             attention that reads it (S - 1 layers ahead at most; with an
                             even S >= 4, S/2 consecutive layers per copy). */
  int32_t chunk;          /* split-K rows per work-group: 128, 256, 512 or 1024 (1024 on
                             the matrix-core path only: bf16 with 1 or >= 4 query heads
                             per kv head, no TKV_FLAG_VECTOR_PASS; TKV_EINVAL otherwise);
                             0 = 1024 for bf16 with q_heads >= 4 * kv_heads (512 with
                             TKV_FLAG_VECTOR_PASS or fp32), else 256 */
  uint64_t flags;         /* TKV_FLAG_* */
  int64_t mem_cap_bytes;  /* most device + pinned host bytes the handle may hold (pools,
                             arenas, scratch, the buffers a reassignment grows); an
                             allocation past it fails with TKV_ENOMEM as a failed hipMalloc
                             would.  0 = no cap. */
  const double* layer_hbm; /* per-layer HBM budgets: `layers` ratios in [0,1] (host
                             memory, read during tkv_create only), or NULL for hbm_ratio
                             in every layer.  See "Per-layer HBM budgets" below. */
} tkv_options;

/* Per-layer HBM budgets (the budget variant in the spirit of ARKV's per-layer
 * ratios, gist.science ARKV summary, Method; tiers and budgets from "Not All
 * Thoughts Need HBM", Method §1): layer l keeps floor(layer_hbm[l] * N) rows
 * in HBM.  Consecutive layers with the same ratio form a group, and each group
 * places its rows by Method §1 with its own ratio: its T0 holds the protected
 * rows and its best candidates.  Every group ranks by the one Eq. 1 score,
 * averaged over all layers, and shares evict_ratio and t2_ratio.  So every
 * group evicts the same rows and the outputs do not depend on the ratios
 * (Method §3, Proposition 1).  A group's T2 count can be smaller than
 * floor(t2_ratio * N) when its HBM share leaves fewer candidates.  Each group
 * holds its own T0 pool, staging and arenas, sized by its own ratio; with
 * stream staging every group needs more than staging_layers layers.  Calls take
 * every layer as usual (each group runs on its own slice, in layer order, on
 * the caller's stream); tkv_read_tiers and tkv_read_deltas report layer 0's
 * group, tkv_read_layer_tiers any layer's.  hbm_ratio is then unused; one
 * distinct ratio is the same as no layer_hbm.  Deferred Eq. 1 defers as many
 * steps as without groups (the groups run in step); tkv_read_scores folds
 * every group's pending steps into one copy of the scores.  A reassignment
 * first applies every group's pending Eq. 1 increment, then re-places each
 * group.  Not with TKV_FLAG_NO_T1 or
 * TKV_FLAG_SHARED_HBM (TKV_EINVAL).  mem_cap_bytes is split over the groups
 * by their layer counts.  tkv_stats sums pools and traffic over the groups;
 * tier_count then counts (layer, position) rows of the batch. */

/* Record HIP events around the attention kernels; tkv_stats reports their time. */
#define TKV_FLAG_TIME_KERNELS 1ull
/* Eviction-only baseline on the same engine (the heavy-hitter eviction policies
 * the gist.science summary compares against, Results): no T1.  Each
 * reassignment keeps the protected rows plus the floor(hbm_ratio*N) - |P|
 * best-ranked candidates in T0, puts the next floor(t2_ratio*N) in T2 and
 * evicts every other candidate; evict_ratio plays no part.  The first
 * placement evicts the rows the tiered policy would put in T1.  With
 * hbm_ratio 0 and prompt 0 this is the sinks-plus-recent-window policy: only
 * the attention sinks and the recent window are ever live.  (Without the flag,
 * hbm_ratio 0, evict_ratio 1 and prompt 0 reach the same set at every
 * reassignment, keeping the other rows in T1 until the first one.) */
#define TKV_FLAG_NO_T1 2ull
/* T2 rows as FP8 instead of int8 (the "FP8 etc." low-precision formats the
 * ARKV summary names): OCP E4M3 ("FN": bias 7, largest finite 448), one fp32
 * scale per (layer, position, K|V) row, scale = amax / 448 (1 for a zero
 * row), code = nearest E4M3 of clamp(x / scale, -448, 448) with ties to even,
 * value = fp32(decode(code) * scale) rounded to the cache type.  Codes and
 * scales have the int8 format's sizes; tkv_read_t2 returns the E4M3 bytes. */
#define TKV_FLAG_T2_FP8 4ull
/* Budget variant: one HBM budget for the whole batch (the batch projection of
 * the summary's Results).  The T0 pool is one slot space shared by the
 * sequences; at each reassignment the protected rows stay in T0, eviction and
 * T2 follow each sequence's own budgets as usual, and the remaining
 * batch * floor(hbm_ratio*N) - sum |P| T0 slots go to the best candidates of
 * the whole batch, ranked jointly by score (ties: lower sequence, then lower
 * position).  The first placement is per sequence (no scores yet).  Not
 * combinable with TKV_FLAG_NO_T1 (TKV_EINVAL). */
#define TKV_FLAG_SHARED_HBM 8ull
/* T2 with one fp32 scale per kv head of a row (each from that head's own
 * amax) instead of one per row: heads of small values keep their precision
 * next to heads of large ones.  Combines with TKV_FLAG_T2_FP8.  tkv_read_t2
 * then returns kv_heads scales for K followed by kv_heads for V. */
#define TKV_FLAG_T2_HEAD_SCALES 16ull
/* bf16 caches with one, or 4 or more, query heads per kv head: run the
 * split-K pass on the vector units (as for 2 heads per kv head and fp32)
 * instead of the matrix cores; the logits are then stored and Eq. 1 is never
 * deferred.  Outputs agree with the matrix-core pass to rounding.  Not with an
 * 8-bit tier in stream staging (TKV_EINVAL).  No effect on other shapes. */
#define TKV_FLAG_VECTOR_PASS 32ull
/* Test hooks, off in normal use.  TKV_FLAG_TEST_DELAY_COPIES: stream staging
 * enqueues a bounded delay kernel (a fixed number of sleep iterations, then
 * it exits) on each copy stream before every layer's staging copy, so the
 * copies land late against the attention that waits for them; results must
 * not change.  TKV_FLAG_TEST_SHUFFLE_SLOTS: free T0 pool slots (stream
 * staging, and the batch-shared budget) are handed out in a seeded
 * pseudo-random order instead of lowest first, so rows sit in scattered
 * slots; results must not change (Method §3, Proposition 1). */
#define TKV_FLAG_TEST_DELAY_COPIES 256ull
#define TKV_FLAG_TEST_SHUFFLE_SLOTS 512ull

/* One changed row of a reassignment (Method §4). */
typedef struct {
  uint32_t pos;     /* logical position */
  uint8_t old_tier; /* tkv_tier */
  uint8_t new_tier; /* tkv_tier */
  uint16_t reserved;
} tkv_delta;

typedef struct {
  int64_t step;              /* decode steps completed */
  int64_t n_tokens;          /* positions appended per sequence (incl. evicted) */
  int64_t tier_count[4];     /* positions per tier, summed over the batch (with per-layer
                                budgets: (layer, position) rows) */
  int64_t hbm_bytes;         /* K/V bytes allocated in HBM (T0 pool + staging) */
  int64_t host_bytes;        /* pinned host K/V bytes (T1 + T2 arenas) */
  int64_t full_cache_bytes;  /* K/V bytes an all-HBM cache of max_tokens would take */
  int64_t promotions, demotions, evictions, reassigns;
  int64_t h2d_bytes, d2h_bytes; /* K/V rows moved host<->device since create */
  double attn_kernel_ms;     /* with TKV_FLAG_TIME_KERNELS: summed split-K kernel time */
  int64_t attn_kernel_launches;
  int64_t attn_kv_bytes;     /* with TKV_FLAG_TIME_KERNELS: K/V bytes of the live rows those
                                launches had to read (the algorithmic traffic) */
  double reassign_ms;        /* host wall time inside tkv_reassign */
  int64_t mem_bytes;         /* device + pinned host bytes the handle holds now (what
                                tkv_options.mem_cap_bytes caps) */
} tkv_stats_t;

/* Create a handle and allocate every pool (on the current device, with
 * synchronous allocations: no stream is involved, and the handle's own
 * streams are created here).  delta: reassignment period (Method §4);
 * hbm_ratio / evict_ratio in [0,1] give the T0 and T3 shares floor(ratio * N)
 * of the N positions appended so far (Method §1).  opts may be NULL.  On
 * failure *out is NULL and tkv_last_error(NULL) explains. */
int tkv_create(const tkv_shape* shape, int32_t delta, double hbm_ratio, double evict_ratio,
               tkv_protect protect, const tkv_options* opts, tkv_t** out);

/* Synchronise the library's own streams and free everything.  NULL is a no-op. */
int tkv_destroy(tkv_t* t);

/* Message of the last failure on t (NULL: of the last failed tkv_create). */
const char* tkv_last_error(const tkv_t* t);

/* Fill an empty cache with n_tokens positions (the prompt and the reasoning
 * chain so far: every token adds a K/V row, problem statement of the
 * summary).  k, v: device [layers][batch][n_tokens][kv_heads][head_dim].
 * Scores start at 0.  The pages place rows by score and have none yet
 * (Method §1, §4); the reading taken: the protected set plus the lowest
 * positions in T0 up to floor(hbm_ratio * n_tokens), the rest in T1, nothing
 * evicted and nothing in T2.  T1 rows are copied to their pinned home.
 * Allocates temporaries from the stream's allocator.  Synchronises
 * `stream`. */
int tkv_prefill(tkv_t* t, const void* k, const void* v, int32_t n_tokens, tkv_stream_t stream);

/* Scored prefill (the step before the decode path): fill an empty cache as
 * tkv_prefill does, then give the prompt the scores its own causal attention
 * earns -- every position t attends to positions 0..t with its query and adds
 * its weights, averaged over layers and query heads, to the scores (Eq. 1 of
 * Method §2, applied to the prompt as to decode steps) -- and re-place every
 * row by those scores with the full tier rules, as tkv_reassign does
 * (counted as one reassignment).  q: device [layers][batch][n_tokens]
 * [q_heads][head_dim] (handle dtype); k, v as for tkv_prefill.  Scratch of
 * 12 * layers * batch * q_heads * n_tokens bytes is taken from the stream's
 * allocator and returned before the call ends.  Errors as tkv_prefill, plus
 * those of tkv_reassign.  Synchronises `stream`. */
int tkv_prefill_scored(tkv_t* t, const void* k, const void* v, const void* q, int32_t n_tokens,
                       tkv_stream_t stream);

/* Start a decode step: append one position to every sequence (each decoded
 * token adds a K/V row, problem statement of the summary; the recent window
 * is always in T0, Method §1).  k, v: device [layers][batch][kv_heads]
 * [head_dim].  The new row enters T0 with score 0.
 * The copy out of k, v is enqueued on `stream` by this call, so the caller may
 * reuse them in stream order right after it returns.
 * TKV_ECAPACITY at max_tokens, or (stream staging, or a batch-shared budget)
 * when the T0 pool is full (reassign first). */
int tkv_append(tkv_t* t, const void* k, const void* v, tkv_stream_t stream);

/* Attention of layers [layer_begin, layer_begin + layer_count) of the
 * current step (Method §3): every non-evicted row of every tier takes part.
 * q: device [layer_count][batch][q_heads][head_dim] (handle dtype);
 * out: device fp32 [layer_count][batch][q_heads][head_dim].  Layer groups of
 * one step must be called in order and cover every layer once.  The step's
 * Eq. 1 increment of the scores (Method §2) is applied in stream order before
 * anything that reads them: it runs inside the next tkv_append's launch, or
 * first thing in tkv_reassign or tkv_read_scores on the stream given to that
 * call.  bf16 caches with one, or 4 or more, query heads per kv head and
 * resident staging (staging_layers 0 or layers) defer it further: a later
 * step's attention launch recomputes the pending steps' weights from their
 * queries while it streams the same K rows, and that step's last layer group
 * adds them; it does so once 15 steps are pending at g = 1 (g query heads per
 * kv head), 11 at g = 4, 8 at g = 5 and 5 at g = 8 (the running step's logits
 * tile holds 16/g - 1 of them, and a forming launch adds two tiles of 16/g
 * steps each at g >= 4).  tkv_reassign first runs a score-only pass over K (half a
 * step's reads) for the steps still pending and adds them; tkv_read_scores
 * does the same into a copy that it returns, leaving them pending, so reads
 * never change the scores' bits.  tkv_write_scores replaces the scores and
 * drops every pending increment. */
int tkv_decode_attn(tkv_t* t, int32_t layer_begin, int32_t layer_count, const void* q, float* out,
                    tkv_stream_t stream);

/* One whole decode step: tkv_append(k, v) followed by tkv_decode_attn over
 * every layer, with identical results (bit for bit) and the same errors and
 * state rules (no step may be open).  k, v as for tkv_append; q, out as for
 * tkv_decode_attn with layer_count = layers.  With resident staging the
 * append and the pending Eq. 1 update run inside the attention launch (the
 * new row is read straight from k, v), so the step takes two launches
 * instead of three; with stream staging it is exactly the two calls.  k, v,
 * q are read by work enqueued on `stream` by this call. */
int tkv_decode_step(tkv_t* t, const void* k, const void* v, const void* q, float* out, tkv_stream_t stream);

/* Re-place every sequence's rows by score (Method §1, §4): protected rows to
 * T0; of the other live rows, ranked by score descending then position
 * ascending, the lowest go to T3 (up to floor(evict_ratio*N) evicted in
 * total), the highest fill T0 up to floor(hbm_ratio*N), the next lowest
 * floor(t2_ratio*N) go to T2 and the rest to T1.  Only changed rows move:
 * the kernels read rows leaving the pinned arenas and write rows entering
 * them over PCIe.  Call between steps, normally when the step count is a
 * multiple of delta.  Synchronises `stream` once (to read the change
 * counts); may grow its scratch with hipMalloc / hipHostMalloc.  Errors
 * before the new labels take effect (TKV_ENOMEM, TKV_ECAPACITY) leave the
 * handle as it was; a failure after that marks it failed: every later call
 * but tkv_destroy, tkv_last_error and tkv_stats returns TKV_ESTATE. */
int tkv_reassign(tkv_t* t, tkv_stream_t stream);

/* For callers that cannot allocate memory -- code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc: tkv_reassign with the
 * reassignment's scratch (the pack of moved rows and the row-copy plan) in
 * the library's static device array, 64 MiB per GPU, instead of buffers that
 * tkv_reassign grows with hipMalloc / hipHostMalloc.  Same results as
 * tkv_reassign, bit for bit.  A reassignment needing more than the array
 * holds -- 2 * layers * kv_heads * head_dim * element bytes per moved row
 * (rows entering T1 or T2; promotions too outside positional staging) plus
 * about 100 bytes per changed row -- returns TKV_ECAPACITY and changes
 * nothing (with per-layer budgets the layer groups are re-placed one after
 * another, each within the array; if a later group does not fit, the earlier
 * ones are already re-placed and the handle is marked failed).  The array is
 * shared by every handle on that GPU and keeps the last call's contents:
 * calls that overlap on one GPU (other host threads) race.  The call returns
 * only once no kernel reads the array any more. */
int tkv_reassign_static(tkv_t* t, tkv_stream_t stream);

/* Counters and sizes (the HBM the tiers save and the traffic they cost: the
 * summary's Results, system overhead and HBM savings); synchronises the
 * library's streams.  Never fails on a handle marked failed. */
int tkv_stats(tkv_t* t, tkv_stats_t* out);

/* Test and inspection hooks (synchronise `stream`).  Arrays are host
 * [batch][max_tokens]; entries at positions >= n_tokens are unspecified.
 * tkv_read_scores returns the scores with every completed step's Eq. 1
 * increment in them; tkv_write_scores replaces them (pending increments are
 * dropped). */
int tkv_read_scores(tkv_t* t, float* scores, tkv_stream_t stream);
int tkv_write_scores(tkv_t* t, const float* scores, tkv_stream_t stream);
int tkv_read_tiers(tkv_t* t, uint8_t* tiers, tkv_stream_t stream);
/* The tiers of layer `layer`'s rows (host [batch][max_tokens]); with
 * per-layer budgets each layer group has its own, otherwise every layer has
 * the handle's.  TKV_EINVAL for a layer out of range. */
int tkv_read_layer_tiers(tkv_t* t, int32_t layer, uint8_t* tiers, tkv_stream_t stream);
/* Changed rows of the last tkv_reassign: promote/demote are host
 * [batch][max_tokens], ascending by position per sequence; counts is host
 * [batch][2] = {promotions, demotions}. */
int tkv_read_deltas(tkv_t* t, tkv_delta* promote, tkv_delta* demote, int32_t* counts);

/* The values attention reads for one live row: host k, v [kv_heads][head_dim]
 * (handle dtype).  For a T2 row these are its dequantised values.  TKV_ESTATE
 * for an evicted or unused position, and for a T2 row in stream staging (its
 * values then exist only as 8-bit codes; see tkv_read_t2). */
int tkv_read_kv(tkv_t* t, int32_t layer, int32_t seq, int32_t pos, void* k, void* v, tkv_stream_t stream);

/* The 8-bit host copy of one T2 row: host k_codes, v_codes [kv_heads][head_dim]
 * (int8, or E4M3 bytes with TKV_FLAG_T2_FP8) and the fp32 scales: {K, V}, or
 * with TKV_FLAG_T2_HEAD_SCALES the kv_heads K scales then the kv_heads V
 * scales.  TKV_ESTATE if the row is not in T2. */
int tkv_read_t2(tkv_t* t, int32_t layer, int32_t seq, int32_t pos, int8_t* k_codes, int8_t* v_codes,
                float* scales);

#ifdef __cplusplus
}
#endif

#endif /* TKV_H */
