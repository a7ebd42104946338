// Decode-step kernels: append, split-K attention over the tiered cache,
// chunk merge + per-layer score sums, and the Eq. 1 score update.
//
// "Not All Thoughts Need HBM" (gist.science technical summary):
//   Method §3 -- every live row (T0 pool or T1/T2 staging) contributes
//   exactly the same terms; rows are walked in logical-position order through
//   a location table, so the arithmetic never depends on where a row sits.
//   Method §2, Eq. 1 -- s_i += (1/|L|) sum_l (1/H) sum_h alpha_{l,h}[i].
//
// Work decomposition (gfx950, wave64):
//   k_attn_chunk  one work-group (4 waves) per (chunk of CHUNK live rows,
//                 kv head, layer x sequence).  A K or V row of head_dim
//                 elements is read as 16-byte pieces by LPR consecutive lanes,
//                 so a wave covers 64/LPR rows per load instruction.  Each row
//                 is loaded once for all G query heads of its kv head.  The
//                 dot products reduce over the LPR lanes with DPP butterflies
//                 (quad_perm, row_half_mirror, row_mirror), the chunk max and
//                 sums with DPP + LDS in a fixed order.  Phase 1 keeps the
//                 log2-scaled logits in LDS; phase 2 forms p = 2^(z - m_chunk)
//                 once per (head, row) and accumulates p * V.  bf16 caches
//                 with G >= 4 or G == 1 do both contractions on the matrix
//                 cores instead.  The block's outputs (logits, chunk
//                 max/sum, partial o) leave last, written through to memory:
//                 writes mixed into the read stream cost the HBM far more
//                 than their size, so the kernel writes only what Eq. 1 and
//                 the merge need.
//   k_finalize    one work-group per (256 live rows, sequence, layer): merges
//                 the chunk partials in chunk order into M, 1/sum and out, and
//                 sums alpha over the layer's heads for its rows.
//   k_score       one thread per live row: adds the layers' sums (layer
//                 order) times 1/(L*H) to s.  The same code normally runs in
//                 the next step's append launch, saving a launch per step.
//   Deferred Eq. 1 (the matrix-core path over resident staging): no
//                 logits are stored; a later step's k_attn_chunk recomputes
//                 the pending steps' weights in the padded rows of its logits
//                 tile (and, with G >= 4, in two more tiles of pending
//                 queries held in LDS, against the same K fragments) and
//                 writes their sum over the pending heads, and its
//                 k_finalize folds those sums into s (k_fold when a
//                 score-only pass applies pending steps).
//                 No atomics anywhere, so every result is bitwise
//                 reproducible.
#include <hip/hip_ext.h>

#include <type_traits>

#include "tkv_internal.hpp"

namespace tkvd {
namespace {

typedef uint16_t bf16_t;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in 1..64); every lane of a group
// gets the identical value (each step adds a pair in both orders).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<0xB1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<0x4E>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<0x140>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// A result the merge pass or Eq. 1 reads later, written through to memory
// (a relaxed store at system scope: global_store sc0 sc1) rather than held
// dirty in L2.  Measured on MI355X against non-temporal stores over the same
// steps: split-K launch 201.1 vs 206.1 us at 7B (-2.4%), 7177 vs 7258 us at
// 70B, 572 vs 575 us at 14B.
__device__ __forceinline__ void store_through(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  const u32x4 v = {u.x, u.y, u.z, u.w};
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ uint4 load16nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T>
__device__ __forceinline__ void unpack(const uint4& u, float* f);

template <>
__device__ __forceinline__ void unpack<bf16_t>(const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void unpack<float>(const uint4& u, float* f) {
  f[0] = __uint_as_float(u.x);
  f[1] = __uint_as_float(u.y);
  f[2] = __uint_as_float(u.z);
  f[3] = __uint_as_float(u.w);
}

// One 16-byte piece (EPL elements of the cache type) of a T2 row, from its
// 8-bit codes (int8, or FP8 E4M3 when fp8): value = fp32(code value * scale),
// rounded to the cache type (bf16 round-to-nearest-even) -- the same values
// the codec defines for the tier.
template <typename T>
__device__ __forceinline__ uint4 deq_piece(const int8_t* codes, float scale, int fp8);

// the four E4M3 bytes of w as floats (exact)
__device__ __forceinline__ void e4m3x4(uint32_t w, float* f) {
  f[0] = __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
  f[1] = __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
  f[2] = __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
  f[3] = __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
}

__device__ __forceinline__ uint32_t bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even (finite values)
  return u >> 16;
}

// signed byte `byte` of w as a float
__device__ __forceinline__ float code_at(uint32_t w, int byte) {
  return (float)((int32_t)(w << (24 - 8 * byte)) >> 24);
}

template <>
__device__ __forceinline__ uint4 deq_piece<bf16_t>(const int8_t* codes, float scale, int fp8) {
  const uint2 c = *reinterpret_cast<const uint2*>(codes);
  float v[8];
  if (fp8) {
    e4m3x4(c.x, v);
    e4m3x4(c.y, v + 4);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = code_at(c.x, k);
      v[4 + k] = code_at(c.y, k);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = bf16_bits(v[2 * i] * scale) | (bf16_bits(v[2 * i + 1] * scale) << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <>
__device__ __forceinline__ uint4 deq_piece<float>(const int8_t* codes, float scale, int fp8) {
  const uint32_t x = *reinterpret_cast<const uint32_t*>(codes);
  float v[4];
  if (fp8) {
    e4m3x4(x, v);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = code_at(x, k);
  }
  return make_uint4(__float_as_uint(v[0] * scale), __float_as_uint(v[1] * scale), __float_as_uint(v[2] * scale),
                    __float_as_uint(v[3] * scale));
}

// Eq. 1 update for live rows [256 tile, 256 tile + 256) of sequence b:
// s[pos(j)] += (sum over layers, in order) * 1/(L*H).
__device__ __forceinline__ void score_rows(const ScoreArgs& a, int tile, int b) {
  const int j = tile * 256 + threadIdx.x;
  if (j >= a.nlive[b]) return;
  float acc = 0.f;
#pragma unroll 8
  for (int l = 0; l < a.layers; ++l) acc += a.layer_score[((int64_t)l * a.batch + b) * a.lstride + j];
  const int64_t p = (int64_t)b * a.nmax + a.live_pos[(int64_t)b * a.nmax + j];
  a.s[p] += acc * a.inv_lh;
}

// Deferred Eq. 1 fold for live rows [R tile, R tile + R) of sequence b,
// R = 256 / P: s[pos(j)] += (sum over the f.layers rows [layer][kv head] of
// f.layer_score) * 1/(L*H).  P partial sums per row: partial k adds every
// P-th entry of the row's list from k, in order, and the P partials are then
// added in order.  The lists are long (layers x kv heads), so one thread per
// row would wait on one long load chain; P = 4 (64 rows per block, each load
// reading 256 contiguous bytes) up to 640 entries, 16 beyond that (16 rows
// per block, 64 entries per thread at 1024).  Every thread of the block calls it.
template <int P>
__device__ __forceinline__ void fold_rows(const ScoreArgs& f, int tile, int b, float* red) {
  constexpr int R = 256 / P;
  const int r = threadIdx.x % R, k = threadIdx.x / R;
  const int j = tile * R + r;
  const bool live = j < f.nlive[b];
  float acc = 0.f;
  if (live) {
    const float* p = f.layer_score + (int64_t)b * f.lstride + j;
    const int64_t step = (int64_t)f.batch * f.lstride;
#pragma unroll 16
    for (int l = k; l < f.layers; l += P) acc += p[l * step];
  }
  red[k * R + r] = acc;
  __syncthreads();
  if (k == 0 && live) {
    float t = red[r];
#pragma unroll
    for (int q = 1; q < P; ++q) t += red[q * R + r];
    const int64_t pos = (int64_t)b * f.nmax + f.live_pos[(int64_t)b * f.nmax + j];
    f.s[pos] += t * f.inv_lh;
  }
}

__device__ __forceinline__ void fold_tile(const ScoreArgs& f, int tile, int b, float* red) {
  if (f.parts == 16)
    fold_rows<16>(f, tile, b, red);
  else
    fold_rows<4>(f, tile, b, red);
}

// ---------------------------------------------------------------------------
// Append: copy the new token's K/V rows of every (layer, sequence) into its
// T0 slot and extend the live list.  Blocks [0, 2*layers*batch) copy (one per
// (layer, sequence, K|V)); the fold_tiles*batch blocks after them apply the
// previous step's Eq. 1 update, which reads only positions and live indices
// below the ones the append writes.  Block 256.
__global__ __launch_bounds__(256) void k_append(const AppendArgs a, const ScoreArgs f, int fold_tiles) {
  const int nappend = 2 * a.layers * a.batch;
  if ((int)blockIdx.x >= nappend) {
    const int y = blockIdx.x - nappend;
    score_rows(f, y % fold_tiles, y / fold_tiles);
    return;
  }
  const int lb = blockIdx.x >> 1;
  const int b = lb % a.batch;
  const int l = lb / a.batch;
  const int which = blockIdx.x & 1;
  const int head_bytes = a.head_dim * a.elem_bytes;
  const int row_bytes = a.kv_heads * head_bytes;
  const char* src = (const char*)(which ? a.v : a.k) + (int64_t)lb * row_bytes;
  char* dst = (char*)(which ? a.rows.pool_v : a.rows.pool_k) +
              ((int64_t)l * a.rows.pool_lstride + (int64_t)b * a.rows.pool_bstride) * a.elem_bytes +
              (int64_t)a.slot[b] * head_bytes;
  const int64_t hstride = a.rows.pool_hstride * a.elem_bytes;
  for (int off = threadIdx.x * 16; off < row_bytes; off += 256 * 16) {
    const int h = off / head_bytes, w = off % head_bytes;
    *reinterpret_cast<uint4*>(dst + h * hstride + w) = load16(src + off);
  }
  if (l == 0 && which == 0 && threadIdx.x == 0) {
    const int64_t j = (int64_t)b * a.nmax + a.nlive[b];
    const int64_t p = (int64_t)b * a.nmax + a.pos;
    a.live_loc[j] = (uint32_t)a.slot[b];
    a.live_pos[j] = a.pos;
    a.tier[p] = 0;
    a.loc[p] = (uint32_t)a.slot[b];
    a.s[p] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Split-K attention, pass 1.  grid (chunks, kv_heads, layer_count*batch).
// With n.k set (a whole-step launch over resident staging) the new token's
// row, live index nlive - 1, is read from n.k / n.v through the location
// code kNewRow; the block holding it stores it into its T0 slot after its
// own reads, and the (chunk, kv head 0, layer 0) blocks apply n.f to the
// live-row tiles starting in their chunk.  Nothing else in the launch reads
// what these writes touch: the slot was free, and the fold only reads
// positions and live indices below the new row's.
//
// DEF (matrix-core path, resident staging): Eq. 1 for pending steps runs
// here instead of from stored logits.  The 16-row logits tile holds this
// step's G query heads in rows 0..G-1; pending step s (1 = the last completed
// step) fills rows sG..sG+G-1, up to 16/G - 1 steps.  Each K tile thus gives
// every step's logits in the same MFMAs; with each pending step's (M, 1/L) a
// row's weights are summed over all pending heads, and one value per row and
// kv head leaves the block, in place of G logits per step.  The host asks for
// 16/G - 1 steps once that many are pending (15 at G = 1, 3 at G = 4, 2 at
// G = 5, 1 at G = 8) and for none in between.  Chunk-0 blocks keep this
// step's queries for later.
//
// At least four waves per SIMD: without that bound the compiler puts the
// matrix-core accumulators in AGPRs and, at G = 5 with pending steps,
// needs 132 registers, one wave fewer; with it, the same code fits in VGPRs
// alone (no spills).  The vector path's allocation is unchanged.
template <typename T, int D, int G, int CHUNK, bool MK, bool QT, bool DEF, int XT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void k_attn_chunk(const AttnArgs a, const StepArgs n) {
  constexpr int LPR = D * (int)sizeof(T) / 16;  // lanes per row
  constexpr int EPL = 16 / (int)sizeof(T);      // elements per lane
  constexpr int RPI = 64 / LPR;                 // rows per wave load
  constexpr int NW = 4;
  constexpr int RPW = CHUNK / NW;               // rows per wave
  constexpr int ITERS = RPW / RPI;
  // loads in flight per lane per batch: 16 for one query head per kv head
  // (1.2% faster than 8 at the 7B shape, though it leaves 5 waves per SIMD
  // instead of 8), fewer as the G query heads' accumulators take registers
  constexpr int UB = (G == 1) ? 16 : (G == 2) ? 8 : 4;
  constexpr int U = ITERS < UB ? ITERS : UB;    // loads in flight per lane per batch
  static_assert(RPW % RPI == 0 && ITERS % U == 0, "chunk shape");

  // logits (log2 units), kept to the end unless Eq. 1 is deferred; then the
  // per-wave partial outputs reuse their space once p is formed (one more
  // work-group per CU at G = 8)
  constexpr bool OSUM_IN_ZS = DEF && NW * D <= CHUNK;
  __shared__ __attribute__((aligned(16))) float zs_store[G * CHUNK + (OSUM_IN_ZS ? 0 : NW * G * D)];
  float (*zs)[CHUNK] = reinterpret_cast<float (*)[CHUNK]>(zs_store);
  float (*osum)[G][D] = reinterpret_cast<float (*)[G][D]>(zs_store + (OSUM_IN_ZS ? 0 : G * CHUNK));
  __shared__ float ps[MK ? 1 : G][MK ? 1 : CHUNK];     // p = 2^(z - m) of the vector path
  __shared__ float red[NW][G];
  __shared__ uint32_t codes_s[CHUNK];
  // deferred Eq. 1: the previous step's weight sums of the chunk's rows, held
  // here until the block's last barrier is behind it (a global store ahead of
  // a barrier holds the wave there until the store is acknowledged)
  __shared__ float es[DEF ? CHUNK : 1];
  // matrix-core p.V: each wave's sums of p per head (the lanes form p from
  // the logits as they build the MFMA operands)
  __shared__ float redL[MK ? NW : 1][MK ? G : 1];
  // deferred Eq. 1, forming launches: XT more logits tiles of pending steps,
  // each lane's A operand (tile row l % 16, elements 32 kc + 8 (l / 16) ..+7)
  // and each tile row's (M, 1/L)
  constexpr int XQ = (MK && DEF) ? XT : 0;
  constexpr int SPT = 16 / G;  // steps per tile
  __shared__ uint4 qx[XQ ? XQ : 1][XQ ? D / 32 : 1][XQ ? 64 : 1];
  __shared__ float2 mlx[XQ ? XQ : 1][XQ ? 16 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = lane % LPR, rg = lane / LPR;
  const int c = blockIdx.x, kvh = blockIdx.y;
  const int b = blockIdx.z % a.batch, ll = blockIdx.z / a.batch;
  const int l = a.layer_begin + ll;
  const int nl = a.nlive[b];
  const int j0 = c * CHUNK;
  if (j0 >= nl) return;
  const int nrows = min(CHUNK, nl - j0);

  constexpr int64_t rs = D;  // elements between consecutive rows of one kv head
  const int64_t poff = (int64_t)l * a.rows.pool_lstride + (int64_t)b * a.rows.pool_bstride +
                       (int64_t)kvh * a.rows.pool_hstride + part * EPL;
  const int64_t soff = (int64_t)(l % a.rows.stage_slots) * a.rows.stage_lstride +
                       (int64_t)b * a.rows.stage_bstride + (int64_t)kvh * a.rows.stage_hstride + part * EPL;
  const T* poolK = (const T*)a.rows.pool_k + poff;
  const T* poolV = (const T*)a.rows.pool_v + poff;
  const T* stageK = (const T*)a.rows.stage_k + soff;
  const T* stageV = (const T*)a.rows.stage_v + soff;
  const uint32_t cap0 = (uint32_t)a.rows.cap0;
  // T2 rows (codes >= qbase): row 0 of this (slot, sequence, kv head) in the 8-bit area
  const uint32_t qbase = cap0 + (uint32_t)a.rows.cap1;
  const int8_t* qK = nullptr;
  const int8_t* qV = nullptr;
  const float* qsK = nullptr;
  const float* qsV = nullptr;
  if constexpr (QT) {
    qK = a.rows.q_k + q_codes_at(a.rows, l, b, kvh, 0, D);
    qV = a.rows.q_v + q_codes_at(a.rows, l, b, kvh, 0, D);
    qsK = a.rows.qs_k + q_scale_at(a.rows, l, b, 0) + (a.rows.q_sh > 1 ? kvh : 0);  // row qi: [qi * q_sh]
    qsV = a.rows.qs_v + q_scale_at(a.rows, l, b, 0) + (a.rows.q_sh > 1 ? kvh : 0);
  }
  // the appended row of a step launch: read from the caller's k / v
  const int jn = n.k ? nl - 1 : -1;
  const int64_t noff = (((int64_t)l * a.batch + b) * a.kv_heads + kvh) * D + part * EPL;
  const T* newK = n.k ? (const T*)n.k + noff : poolK;
  const T* newV = n.k ? (const T*)n.v + noff : poolV;
  const uint32_t* locs = a.live_loc + (int64_t)b * a.nmax + j0;
  // Set-up: every global load of the block is issued before the first LDS
  // store, so their latencies overlap (a store that waits on its load ahead
  // of the next load would serialise them): the chunk's location codes and,
  // on the matrix cores, the tile's queries, the pending steps' (M, 1/L) and
  // the extra tiles' queries.
  constexpr int CPT = (CHUNK + 255) / 256;  // codes per thread
  uint32_t cr[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int r = tid + 256 * k;
    cr[k] = (r < CHUNK && r < nrows) ? (j0 + r == jn ? kNewRow : locs[r]) : 0u;
  }
  // matrix cores: lane l feeds tile row l % 16 (pending step (l % 16) / G,
  // 0 = this step, head (l % 16) % G; zeros past the steps formed here) and
  // receives rows 4 (l / 16) .. +3
  constexpr int KQ = MK ? D / 32 : 1;
  const int mprev = (MK && DEF) ? a.prev_mode : 0;
  const int mnps = mprev != 0 ? a.prev_steps : 0;  // pending steps formed here
  auto slot = [&](int st) {  // ring slot of pending step st (0: this step)
    const int x = (a.qcur + 1 - st) % a.ring;
    return x < 0 ? x + a.ring : x;
  };
  const int64_t qrow = ((int64_t)l * a.batch + b) * a.q_heads + kvh * G;  // head 0 of the group, layer l
  uint4 qu[KQ];
  float pM[4], piL[4];
  if constexpr (MK) {
    const int hl = lane & 15, kq = lane >> 4, qs = hl / G, qh = hl % G;
    const T* qsrc = nullptr;
    if (qs == 0 && mprev != 2)
      qsrc = (const T*)a.q + (((int64_t)ll * a.batch + b) * a.q_heads + kvh * G + qh) * D;
    else if (qs >= 1 && qs <= mnps && qs < SPT)
      qsrc = (const T*)a.qring + slot(qs) * a.qslot + (qrow + qh) * D;
#pragma unroll
    for (int kc = 0; kc < KQ; ++kc) qu[kc] = qsrc ? load16(qsrc + 32 * kc + 8 * kq) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * kq + i, st = h / G;
      const bool on = st >= 1 && st <= mnps && st < SPT;
      const float* ml = a.mlring + (on ? slot(st) * a.mlslot + (qrow + h % G) * 2 : 0);
      pM[i] = on ? ml[0] : 0.f;
      piL[i] = on ? ml[1] : 0.f;
    }
  }
  // extra tile x, row h: head h % G of pending step SPT (x + 1) + h / G, if
  // that step is formed here; zeros otherwise
  constexpr int XPT = XQ ? (XQ * (D / 32) * 64 + 255) / 256 : 1;  // A-operand pieces per thread
  uint4 xr[XPT];
  float2 xm = make_float2(0.f, 0.f);
  if constexpr (XQ > 0) {
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
      const int i = tid + 256 * k;
      const int x = i / ((D / 32) * 64), kc = (i / 64) % (D / 32), ln = i % 64;
      const int h = ln & 15, st = SPT * (x + 1) + h / G;
      xr[k] = make_uint4(0, 0, 0, 0);
      if (i < XQ * (D / 32) * 64 && h < SPT * G && st <= mnps)
        xr[k] = load16((const T*)a.qring + slot(st) * a.qslot + (qrow + h % G) * D + 32 * kc + 8 * (ln >> 4));
    }
    const int x = tid / 16, h = tid % 16, st = SPT * (x + 1) + h / G;
    if (tid < XQ * 16 && h < SPT * G && st <= mnps) {
      const float* ml = a.mlring + slot(st) * a.mlslot + (qrow + h % G) * 2;
      xm = make_float2(ml[0], ml[1]);
    }
  }
#pragma unroll
  for (int k = 0; k < CPT; ++k)
    if (tid + 256 * k < CHUNK) codes_s[tid + 256 * k] = cr[k];
  if constexpr (XQ > 0) {
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
      const int i = tid + 256 * k;
      if (i < XQ * (D / 32) * 64) qx[i / ((D / 32) * 64)][(i / 64) % (D / 32)][i % 64] = xr[k];
    }
    if (tid < XQ * 16) mlx[tid / 16][tid % 16] = xm;
  }
  __syncthreads();

  float mc[G];
  if constexpr (MK) {
    // deferred Eq. 1 (DEF): prev_mode 1, the last pending step's rows are the
    // live indices below the new row's; 2, score only over every live row.
    // Pending step s (1 = the last completed step) had s - 1 rows fewer (each
    // step appends one row per sequence and nothing leaves between
    // reassignments); its queries fill tile rows sG..sG+G-1 for s < 16 / G,
    // else rows of the extra tiles (XT of them, forming launches only).
    const int prev = mprev;
    const int nprev = prev == 1 ? nl - 1 : nl;
    const int nps = mnps;
    // ---- phase 1 on the matrix cores: Z[16 heads x 16 rows] += Q[16 x 32] K^T[32 x 16],
    // D/32 steps per tile of 16 rows (v_mfma_f32_16x16x32_bf16).  Lane l feeds
    // head / row (l % 16) and the 8 elements 8*(l/16) of each 32-wide slice;
    // it receives Z for heads 4*(l/16)..+3 of row (l % 16).  Heads >= G are 0.
    constexpr int KC = D / 32;
    constexpr int TILES = RPW / 16;
    const int hl = lane & 15, kq = lane >> 4;
    // the tile's queries (loaded in the set-up) and, in pM / piL, the pending
    // steps' (M, 1/L) of the tile rows this lane receives
    bf16x8 qa[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qa[kc] = as_bf16x8(qu[kc]);
    float* sp = DEF ? a.spart + (((int64_t)l * a.kv_heads + kvh) * a.batch + b) * a.lstride + j0 : nullptr;
    float mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = -INFINITY;
    const T* pK = poolK - part * EPL + 8 * kq;  // this lane's 8-element slice of a row
    const T* sK = stageK - part * EPL + 8 * kq;
    const T* nK = newK - part * EPL + 8 * kq;
#pragma unroll
    for (int t0 = 0; t0 < TILES; t0 += 2) {
      uint4 kd[2][KC];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int r = wave * RPW + (t0 + tt) * 16 + hl;
        const bool ok = t0 + tt < TILES && r < nrows;
        const uint32_t code = ok ? codes_s[r] : 0u;
        if (QT && ok && code >= qbase) {
          const uint32_t qi = code - qbase;
          const float sc = qsK[(int64_t)qi * a.rows.q_sh];
          const int8_t* qp = qK + (int64_t)qi * D + 8 * kq;
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) kd[tt][kc] = deq_piece<T>(qp + 32 * kc, sc, a.rows.q_fp8);
        } else {
          const T* p = code < cap0 ? pK + (int64_t)code * rs
                       : code == kNewRow ? nK : sK + (int64_t)(code - cap0) * rs;
          // 64-byte pieces per row per load: a streaming (non-temporal) hint would let
          // the row's lines leave the cache before the neighbouring piece is read.
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) kd[tt][kc] = ok ? load16(p + 32 * kc) : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        if (t0 + tt >= TILES) break;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kc], as_bf16x8(kd[tt][kc]), acc, 0, 0, 0);
        const int r = wave * RPW + (t0 + tt) * 16 + hl;
        if (prev != 2 && r < nrows) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int h = 4 * kq + i;
            const float z = acc[i] * a.qscale;
            if (h < G) zs[h][r] = z;
            mx[i] = fmaxf(mx[i], z);
          }
        }
        if (DEF && prev != 0) {
          // sum of the pending steps' weights of row r over their heads: this
          // lane's four tile rows, then the four lanes that hold row r, in a
          // fixed order (pending step st holds live indices < nprev - (st - 1))
          float e = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int st = (4 * kq + i) / G;
            if (st >= 1 && st <= nps && st < SPT && j0 + r < nprev - (st - 1))
              e += exp2f(acc[i] * a.qscale - pM[i]) * piL[i];
          }
          if constexpr (XQ > 0) {
            // the extra tiles: the same K fragments against queries from LDS
#pragma unroll
            for (int x = 0; x < XQ; ++x) {
              f32x4 ax = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int kc = 0; kc < KC; ++kc)
                ax = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qx[x][kc][lane]), as_bf16x8(kd[tt][kc]), ax, 0, 0, 0);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int h = 4 * kq + i, st = SPT * (x + 1) + h / G;
                if (h < SPT * G && st <= nps && j0 + r < nprev - (st - 1)) {
                  const float2 m = mlx[x][h];
                  e += exp2f(ax[i] * a.qscale - m.x) * m.y;
                }
              }
            }
          }
          e += __shfl_xor(e, 16);
          e += __shfl_xor(e, 32);
          if (kq == 0) es[r] = e;
        }
      }
    }
    if (prev == 2) {  // score only: the sums leave, and so does the whole block
      __syncthreads();
      for (int r = tid; r < nrows && j0 + r < nprev; r += 256) store_through(sp + r, es[r]);
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float m = group_max<16>(mx[i]);
      if (hl == 0 && 4 * kq + i < G) red[wave][4 * kq + i] = m;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) mc[g] = fmaxf(fmaxf(red[0][g], red[1][g]), fmaxf(red[2][g], red[3][g]));
  } else {
    float qv[G][EPL];
  #pragma unroll
    for (int g = 0; g < G; ++g) {
      const T* qp = (const T*)a.q + (((int64_t)ll * a.batch + b) * a.q_heads + kvh * G + g) * D + part * EPL;
      unpack<T>(load16(qp), qv[g]);
  #pragma unroll
      for (int e = 0; e < EPL; ++e) qv[g][e] *= a.qscale;
    }

    // ---- phase 1: logits and the chunk max
    float mx[G];
  #pragma unroll
    for (int g = 0; g < G; ++g) mx[g] = -INFINITY;
    for (int it0 = 0; it0 < ITERS; it0 += U) {
      uint4 kd[U];
  #pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = wave * RPW + (it0 + u) * RPI + rg;
        kd[u] = make_uint4(0, 0, 0, 0);
        if (r < nrows) {
          const uint32_t code = codes_s[r];
          if (QT && code >= qbase) {
            const uint32_t qi = code - qbase;
            kd[u] = deq_piece<T>(qK + (int64_t)qi * D + part * EPL, qsK[(int64_t)qi * a.rows.q_sh], a.rows.q_fp8);
          } else {
            const T* p = code < cap0 ? poolK + (int64_t)code * rs
                         : code == kNewRow ? newK : stageK + (int64_t)(code - cap0) * rs;
            kd[u] = load16nt(p);
          }
        }
      }
  #pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = wave * RPW + (it0 + u) * RPI + rg;
        float kf[EPL];
        unpack<T>(kd[u], kf);
  #pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc = 0.f;
  #pragma unroll
          for (int e = 0; e < EPL; ++e) acc = fmaf(qv[g][e], kf[e], acc);
          const float z = group_sum<LPR>(acc);
          if (r < nrows) {
            if (part == 0) zs[g][r] = z;
            mx[g] = fmaxf(mx[g], z);
          }
        }
      }
    }
  #pragma unroll
    for (int g = 0; g < G; ++g) {
      float m = mx[g];
      for (int off = LPR; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
      if (lane == 0) red[wave][g] = m;
    }
    __syncthreads();
  #pragma unroll
    for (int g = 0; g < G; ++g) mc[g] = fmaxf(fmaxf(red[0][g], red[1][g]), fmaxf(red[2][g], red[3][g]));
  }

  // ---- p = 2^(z - m) and the chunk sums.  The logits go out at the very end:
  // a global store ahead of a barrier would hold every wave at that barrier
  // until the store is acknowledged.
  if constexpr (!MK) {
    float ls[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      ls[g] = 0.f;
      for (int r = tid; r < CHUNK; r += 256) {
        float p = 0.f;
        if (r < nrows) p = exp2f(zs[g][r] - mc[g]);
        ps[g][r] = p;
        ls[g] += p;
      }
    }
    // all reads of red[] (maxima) and of zs (when osum reuses it) are done
    // before either is written again below
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float s = group_sum<64>(ls[g]);
      if (lane == 0) red[wave][g] = s;
    }
  }

  // ---- phase 2: o = sum_r p_r * v_r
  if constexpr (MK) {
    // Matrix cores, O[16 heads][D] += P[16 x 32 rows] V[32 rows x D], no transpose:
    // lane (hl, kq) loads 16 B (d = 8hl..8hl+7) of rows 8kq..8kq+7 of a 32-row
    // sub-tile (every load instruction covers 4 full rows), and MFMA #j takes
    // element j of those 8 rows, so its output columns are d = 8n + j.
    // v_mfma_f32_16x16x32_bf16 takes V's bf16 values as they are (any range)
    // and P as its three bf16 terms, one MFMA each: the products are exact in
    // fp32 and the sum is accumulated in fp32.  Heads G..15 of the tile are
    // zero.  With head_dim 64 only lanes hl < 8 carry columns; the others
    // load zeros and their output columns are dropped.
    constexpr int ST = RPW / 32;
    const int hl = lane & 15, kq = lane >> 4;
    const bool col_ok = 8 * hl < D;
    const T* pV = poolV - part * EPL + 8 * hl;
    const T* sV = stageV - part * EPL + 8 * hl;
    const T* nV = newV - part * EPL + 8 * hl;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;  // this lane's p of head hl, over its rows
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      const int rb = wave * RPW + st * 32 + 8 * kq;
      uint4 vr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = rb + i;
        const bool ok = col_ok && r < nrows;
        const uint32_t code = ok ? codes_s[r] : 0u;
        if (QT && ok && code >= qbase) {
          const uint32_t qi = code - qbase;
          vr[i] = deq_piece<T>(qV + (int64_t)qi * D + 8 * hl, qsV[(int64_t)qi * a.rows.q_sh], a.rows.q_fp8);
        } else {
          const T* p = code < cap0 ? pV + (int64_t)code * rs
                       : code == kNewRow ? nV : sV + (int64_t)(code - cap0) * rs;
          vr[i] = ok ? load16nt(p) : make_uint4(0, 0, 0, 0);
        }
      }
      // P of head hl, rows rb..rb+7: p = 2^(z - m) = hi + mid + lo, each a
      // bf16 value (each term takes the next 8 of p's 24 significant bits; the
      // remainders are exact in fp32), so the bf16 matrix cores weigh V by p
      // itself, as the vector path does.  Each (head, row) is formed by one
      // lane only, which also adds p to its head's sum.
      uint32_t pw[3][4] = {};
      if (hl < G) {
        float mh = mc[0];
#pragma unroll
        for (int g = 1; g < G; ++g) mh = hl == g ? mc[g] : mh;
        const f32x4 z0 = *reinterpret_cast<const f32x4*>(&zs[hl][rb]);
        const f32x4 z1 = *reinterpret_cast<const f32x4*>(&zs[hl][rb + 4]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = rb + i < nrows ? exp2f((i < 4 ? z0[i] : z1[i - 4]) - mh) : 0.f;
          const uint32_t hi = bf16_bits(p);
          const float r1 = p - __uint_as_float(hi << 16);
          const uint32_t mid = bf16_bits(r1);
          const uint32_t lo = bf16_bits(r1 - __uint_as_float(mid << 16));
          pw[0][i >> 1] |= hi << (16 * (i & 1));
          pw[1][i >> 1] |= mid << (16 * (i & 1));
          pw[2][i >> 1] |= lo << (16 * (i & 1));
          lsum += p;
        }
      }
      bf16x8 pa[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) pa[k] = as_bf16x8(make_uint4(pw[k][0], pw[k][1], pw[k][2], pw[k][3]));
      uint32_t vh[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        vh[i][0] = vr[i].x;
        vh[i][1] = vr[i].y;
        vh[i][2] = vr[i].z;
        vh[i][3] = vr[i].w;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x4 bw;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t a0 = vh[2 * t][j >> 1], a1 = vh[2 * t + 1][j >> 1];
          bw[t] = (j & 1) ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
        }
        const bf16x8 vb = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
        for (int k = 0; k < 3; ++k) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[k], vb, acc[j], 0, 0, 0);
      }
    }
    // the wave's sum of p per head: the four lanes of head hl, in a fixed order
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (kq == 0 && hl < G) redL[wave][hl] = lsum;
    // every wave's reads of the logits are done before osum, which may share
    // their space, is written
    if constexpr (OSUM_IN_ZS) __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * kq + i;
      if (h < G && col_ok) {
#pragma unroll
        for (int j = 0; j < 8; ++j) osum[wave][h][8 * hl + j] = acc[j][i];
      }
    }
  } else {
    // ---- phase 2: o = sum_r p_r * v_r
    float o[G][EPL];
  #pragma unroll
    for (int g = 0; g < G; ++g)
  #pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] = 0.f;
    for (int it0 = 0; it0 < ITERS; it0 += U) {
      uint4 vd[U];
  #pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = wave * RPW + (it0 + u) * RPI + rg;
        vd[u] = make_uint4(0, 0, 0, 0);
        if (r < nrows) {
          const uint32_t code = codes_s[r];
          if (QT && code >= qbase) {
            const uint32_t qi = code - qbase;
            vd[u] = deq_piece<T>(qV + (int64_t)qi * D + part * EPL, qsV[(int64_t)qi * a.rows.q_sh], a.rows.q_fp8);
          } else {
            const T* p = code < cap0 ? poolV + (int64_t)code * rs
                         : code == kNewRow ? newV : stageV + (int64_t)(code - cap0) * rs;
            vd[u] = load16nt(p);
          }
        }
      }
  #pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = wave * RPW + (it0 + u) * RPI + rg;
        if (r < nrows) {
          float vf[EPL];
          unpack<T>(vd[u], vf);
  #pragma unroll
          for (int g = 0; g < G; ++g) {
            const float pg = ps[g][r];
  #pragma unroll
            for (int e = 0; e < EPL; ++e) o[g][e] = fmaf(pg, vf[e], o[g][e]);
          }
        }
      }
    }
  #pragma unroll
    for (int g = 0; g < G; ++g)
  #pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float x = o[g][e];
        for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off);
        if (rg == 0) osum[wave][g][part * EPL + e] = x;
      }
  }
  __syncthreads();
  const int64_t hbase = ((int64_t)l * a.batch + b) * a.q_heads + kvh * G;
  for (int t = tid; t < G * D; t += 256) {
    const int g = t / D, e = t % D;
    const float x = ((osum[0][g][e] + osum[1][g][e]) + osum[2][g][e]) + osum[3][g][e];
    store_through(a.part_o + ((hbase + g) * a.max_chunks + c) * D + e, x);
  }
  if (tid < 2 * G) {
    const int g = tid >> 1;
    float v = mc[g];
    if constexpr (MK) {
      if (tid & 1) v = ((redL[0][g] + redL[1][g]) + redL[2][g]) + redL[3][g];
    } else {
      if (tid & 1) v = ((red[0][g] + red[1][g]) + red[2][g]) + red[3][g];
    }
    store_through(a.part_ml + ((hbase + g) * a.max_chunks + c) * 2 + (tid & 1), v);
  }
  if constexpr (MK && DEF) {
    if (a.prev_mode != 0) {
      // the previous step's rows: live indices below the new row's (all of them in a score-only pass)
      const int nprev = a.prev_mode == 1 ? nl - 1 : nl;
      float* sp = a.spart + (((int64_t)l * a.kv_heads + kvh) * a.batch + b) * a.lstride + j0;
      for (int r = tid; r < nrows && j0 + r < nprev; r += 256) store_through(sp + r, es[r]);
    }
  }
  // logits, padded with zeros to the line that holds the chunk's last row
  // (none when Eq. 1 is deferred)
  const int nw = DEF ? 0 : min(CHUNK, (nrows + 31) / 32 * 32);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float* lg = a.logits + (hbase + g) * a.lstride + j0;
    for (int r = tid; r < nw; r += 256) store_through(lg + r, r < nrows ? zs[g][r] : 0.f);
  }
  if (jn >= j0 && jn < j0 + nrows) {
    // the appended row's K and V of this kv head into T0 slot n.slot[b]
    constexpr int PPR = D * (int)sizeof(T) / 16;  // 16-byte pieces per head row
    if (tid < 2 * PPR) {
      const int which = tid / PPR, piece = tid % PPR;
      const int64_t src = (((int64_t)l * a.batch + b) * a.kv_heads + kvh) * D + piece * EPL;
      const int64_t dst = (int64_t)l * a.rows.pool_lstride + (int64_t)b * a.rows.pool_bstride +
                          (int64_t)kvh * a.rows.pool_hstride + (int64_t)n.slot[b] * D + piece * EPL;
      const uint4 x = load16((const T*)(which ? n.v : n.k) + src);
      *reinterpret_cast<uint4*>((T*)(which ? a.rows.pool_v : a.rows.pool_k) + dst) = x;
    }
    if (kvh == 0 && l == 0 && tid == 0) {
      const int64_t j = (int64_t)b * a.nmax + jn;
      const int64_t p = (int64_t)b * a.nmax + n.pos;
      n.live_loc[j] = (uint32_t)n.slot[b];
      n.live_pos[j] = n.pos;
      n.tier[p] = 0;
      n.loc[p] = (uint32_t)n.slot[b];
      n.s[p] = 0.f;
    }
  }
  if (n.fold && kvh == 0 && l == 0)
    for (int y = (j0 + 255) / 256; y * 256 < j0 + CHUNK; ++y) score_rows(n.f, y, b);
}

// ---------------------------------------------------------------------------
// Merge chunk partials and sum alpha over heads.  grid (tiles + ceil(Hq /
// HPB), batch, layer_count), block 256.  Blocks x < tiles sum alpha over the
// layer's heads for RPT * 256 live rows, RPT consecutive rows per thread (one
// 16-byte load per head when RPT = 4); the other blocks merge the chunk
// partials of HPB = 256 / (D / RPT) heads into M, 1 / sum and the output
// rows, RPT elements per thread.  Both kinds merge the chunk (max, sum) pairs in
// chunk order, so they agree, and every sum runs in head order (rows) or chunk
// order (outputs) whatever RPT is.
//
// Deferred Eq. 1 (a.mlprev set): there are no score blocks (tiles_grid = 0);
// the output blocks also keep every head's (M, 1/L) for the next step, and
// blocks past the heads fold the previous step's per-group sums into the
// scores (a.fold_tiles tiles of 64 rows per sequence, dealt over the layer
// slices of the grid).
template <int D, int RPT>
__global__ __launch_bounds__(256) void k_finalize(const FinalizeArgs a, const ScoreArgs fold) {
  __shared__ float Ms[kMaxQHeads];
  __shared__ float iLs[kMaxQHeads];
  __shared__ float fold_red[256];
  constexpr int TILE = 256 * RPT;
  const int tid = threadIdx.x;
  const int x = blockIdx.x, b = blockIdx.y, ll = blockIdx.z;
  const int l = a.layer_begin + ll;
  const int nl = a.nlive[b];
  const int tiles = (nl + TILE - 1) / TILE;
  const int tiles_grid = a.tiles_grid;
  const int nch = (nl + a.chunk - 1) / a.chunk;
  const int64_t hbase = ((int64_t)l * a.batch + b) * a.q_heads;

  // M = max of the chunk maxima, L = sum over chunks, in chunk order, of
  // sum_c * 2^(max_c - M).  Up to MC chunks the pairs arrive in one batch of
  // loads and stay in registers; longer lists take two passes over memory.
  // Both forms add the same terms in the same order.
  constexpr int MC = 16;
  auto load_pairs = [&](int h, float2 (&v)[MC]) {
    const float2* ml = reinterpret_cast<const float2*>(a.part_ml + (hbase + h) * a.max_chunks * 2);
#pragma unroll
    for (int c = 0; c < MC; ++c) v[c] = c < nch ? ml[c] : make_float2(-INFINITY, 0.f);
  };
  auto merge_pairs = [&](const float2 (&v)[MC], float* M_out, float* iL_out) {
    float M = -INFINITY, L = 0.f;
#pragma unroll
    for (int c = 0; c < MC; ++c) M = fmaxf(M, v[c].x);
#pragma unroll
    for (int c = 0; c < MC; ++c)
      if (c < nch) L += v[c].y * exp2f(v[c].x - M);
    *M_out = M;
    *iL_out = 1.f / L;
  };
  auto merge_head = [&](int h, float* M_out, float* iL_out) {
    if (nch <= MC) {
      float2 v[MC];
      load_pairs(h, v);
      merge_pairs(v, M_out, iL_out);
      return;
    }
    const float* ml = a.part_ml + (hbase + h) * a.max_chunks * 2;
    float M = -INFINITY, L = 0.f;
#pragma unroll 8
    for (int c = 0; c < nch; ++c) M = fmaxf(M, ml[2 * c]);
#pragma unroll 8
    for (int c = 0; c < nch; ++c) L += ml[2 * c + 1] * exp2f(ml[2 * c] - M);
    *M_out = M;
    *iL_out = 1.f / L;
  };

  if (x >= tiles_grid) {
    // ---- output rows: D / RPT threads per head
    typedef float outv __attribute__((ext_vector_type(RPT)));
    constexpr int TPH = D / RPT;
    constexpr int HPB = 256 / TPH;
    const int hblocks = (a.q_heads + HPB - 1) / HPB;
    if (x >= tiles_grid + hblocks) {
      // fold tiles are dealt over the layer slices: ceil(fold_tiles / slices) per slice
      const int per = (a.fold_tiles + gridDim.z - 1) / gridDim.z;
      const int ft = ll * per + (x - tiles_grid - hblocks);
      if (ft < a.fold_tiles) fold_tile(fold, ft, b, fold_red);
      return;
    }
    const int h = (x - tiles_grid) * HPB + tid / TPH, ev = tid % TPH;
    if (h >= a.q_heads || nl == 0) return;
    if (a.qsave && ev < D / 8) {
      // deferred Eq. 1: the head's query row into the ring, for the later
      // launches that form this step's weights (bf16, 16 B per thread)
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                                        (((int64_t)ll * a.batch + b) * a.q_heads + h) * D);
      reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.qsave) + (hbase + h) * D)[ev] = src[ev];
    }
    const float* ml = a.part_ml + (hbase + h) * a.max_chunks * 2;
    const outv* po = reinterpret_cast<const outv*>(a.part_o + (hbase + h) * a.max_chunks * D) + ev;
    outv acc = {};
    if (nch <= MC) {
      // the partials' loads go out with the pairs', before M is known
      float2 v[MC];
      outv pv[MC];
      load_pairs(h, v);
#pragma unroll
      for (int c = 0; c < MC; ++c) pv[c] = c < nch ? po[(int64_t)c * (D / RPT)] : outv{};
      float M, iL;
      merge_pairs(v, &M, &iL);
      if (a.mlprev && ev == 0) {
        a.mlprev[(hbase + h) * 2] = M;
        a.mlprev[(hbase + h) * 2 + 1] = iL;
      }
#pragma unroll
      for (int c = 0; c < MC; ++c)
        if (c < nch) {
          const float w = exp2f(v[c].x - M);
#pragma unroll
          for (int k = 0; k < RPT; ++k) acc[k] += pv[c][k] * w;
        }
      outv o;
#pragma unroll
      for (int k = 0; k < RPT; ++k) o[k] = acc[k] * iL;
      reinterpret_cast<outv*>(a.out + (((int64_t)ll * a.batch + b) * a.q_heads + h) * D)[ev] = o;
      return;
    }
    float M, iL;
    merge_head(h, &M, &iL);
    if (a.mlprev && ev == 0) {
      a.mlprev[(hbase + h) * 2] = M;
      a.mlprev[(hbase + h) * 2 + 1] = iL;
    }
#pragma unroll 8
    for (int c = 0; c < nch; ++c) {
      const outv v = po[(int64_t)c * (D / RPT)];
      const float w = exp2f(ml[2 * c] - M);
#pragma unroll
      for (int k = 0; k < RPT; ++k) acc[k] += v[k] * w;
    }
    outv o;
#pragma unroll
    for (int k = 0; k < RPT; ++k) o[k] = acc[k] * iL;
    reinterpret_cast<outv*>(a.out + (((int64_t)ll * a.batch + b) * a.q_heads + h) * D)[ev] = o;
    return;
  }
  if (x >= tiles) return;
  // ---- per-layer score of RPT consecutive live rows per thread
  typedef float rowv __attribute__((ext_vector_type(RPT)));
  const int j0 = x * TILE + RPT * tid;
  const float* lg = a.logits + hbase * a.lstride + j0;
  constexpr int KP = 32 / RPT;  // this thread's first KP heads' logits are in flight during the merge
  rowv zr[KP];
#pragma unroll
  for (int h = 0; h < KP; ++h)
    zr[h] = (j0 < nl && h < a.q_heads) ? *reinterpret_cast<const rowv*>(lg + (int64_t)h * a.lstride) : rowv{};
  for (int h = tid; h < a.q_heads; h += 256) merge_head(h, &Ms[h], &iLs[h]);
  __syncthreads();
  float* ls_row = a.layer_score + ((int64_t)l * a.batch + b) * a.lstride;
  if (j0 < (nl + 31) / 32 * 32) {  // the rows past nl on the last line get 0
    float S[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) S[k] = 0.f;
#pragma unroll
    for (int h = 0; h < KP; ++h)
      if (h < a.q_heads) {
#pragma unroll
        for (int k = 0; k < RPT; ++k) S[k] += exp2f(zr[h][k] - Ms[h]) * iLs[h];
      }
#pragma unroll 4
    for (int h = KP; h < a.q_heads; ++h) {
      const rowv z = *reinterpret_cast<const rowv*>(lg + (int64_t)h * a.lstride);
#pragma unroll
      for (int k = 0; k < RPT; ++k) S[k] += exp2f(z[k] - Ms[h]) * iLs[h];
    }
    rowv o;
#pragma unroll
    for (int k = 0; k < RPT; ++k) o[k] = j0 + k < nl ? S[k] : 0.f;
    *reinterpret_cast<rowv*>(ls_row + j0) = o;
  }
}

// Eq. 1 update on its own: grid (tiles, batch).
__global__ __launch_bounds__(256) void k_score(const ScoreArgs a) { score_rows(a, blockIdx.x, blockIdx.y); }

// Deferred Eq. 1 fold on its own: grid (tiles of 256 / a.parts rows, batch).
__global__ __launch_bounds__(256) void k_fold(const ScoreArgs a) {
  __shared__ float red[256];
  fold_tile(a, blockIdx.x, blockIdx.y, red);
}

// Grouped-query heads (G >= 4) of bf16 caches take the matrix-core logits.
// Launched through hipExtLaunchKernel so that timing events (when given) take
// the dispatch's own start and end instead of packets of their own.
struct AttnLaunch {
  dim3 grid;
  hipEvent_t e0, e1;
  hipStream_t s;
};

template <typename T, int D, int G, bool QT, bool DEF, bool MK, int XT = 0>
const void* attn_fn(int chunk) {
  switch (chunk) {
    case 128: return (const void*)&k_attn_chunk<T, D, G, 128, MK, QT, DEF, XT>;
    case 256: return (const void*)&k_attn_chunk<T, D, G, 256, MK, QT, DEF, XT>;
    case 512: return (const void*)&k_attn_chunk<T, D, G, 512, MK, QT, DEF, XT>;
    case 1024:  // the matrix-core path only
      if constexpr (MK) return (const void*)&k_attn_chunk<T, D, G, 1024, MK, QT, DEF, XT>;
      return nullptr;
    default: return nullptr;
  }
}

// a.spart set: deferred Eq. 1, which only the matrix-core path without 8-bit
// staging has (the launcher checks this before it sets a.spart).  vec: bf16
// grouped-query heads on the vector path instead of the matrix cores (not
// with 8-bit staging).
template <typename T, int D, int G, bool QT>
hipError_t launch_attn_t(const AttnArgs& a, const StepArgs& n, int chunk, bool vec, const AttnLaunch& L) {
  // the matrix cores for bf16 with 4 or more query heads per kv head, and with
  // one (whose tile then has room for 15 pending steps of deferred Eq. 1)
  constexpr bool MK = std::is_same<T, bf16_t>::value && (G >= 4 || G == 1);
  const void* fn = nullptr;
  if constexpr (MK && !QT) {
    if (vec) {
      if (a.spart) return hipErrorInvalidValue;
      fn = attn_fn<T, D, G, QT, false, false>(chunk);
    } else {
      // launches that form pending steps (or score them only) take the
      // form with the extra logits tiles; the others the lean one
      constexpr int XT = defer_extra_tiles(G);
      if (!a.spart)
        fn = attn_fn<T, D, G, QT, false, true>(chunk);
      else if (a.prev_mode != 0)
        fn = attn_fn<T, D, G, QT, true, true, XT>(chunk);
      else
        fn = attn_fn<T, D, G, QT, true, true, 0>(chunk);
    }
  } else {
    if (a.spart || (vec && MK)) return hipErrorInvalidValue;
    fn = attn_fn<T, D, G, QT, false, MK>(chunk);
  }
  if (!fn) return hipErrorInvalidValue;
  AttnArgs ac = a;
  StepArgs nc = n;
  void* args[] = {&ac, &nc};
  return hipExtLaunchKernel(fn, L.grid, dim3(256), args, 0, L.s, L.e0, L.e1, 0);
}

template <typename T, int D, bool QT>
hipError_t launch_attn_g(const AttnArgs& a, const StepArgs& n, int group, int chunk, bool vec, const AttnLaunch& L) {
  switch (group) {
    case 1: return launch_attn_t<T, D, 1, QT>(a, n, chunk, vec, L);
    case 2: return launch_attn_t<T, D, 2, QT>(a, n, chunk, vec, L);
    case 4: return launch_attn_t<T, D, 4, QT>(a, n, chunk, vec, L);
    case 5: return launch_attn_t<T, D, 5, QT>(a, n, chunk, vec, L);
    case 8: return launch_attn_t<T, D, 8, QT>(a, n, chunk, vec, L);
    default: return hipErrorInvalidValue;
  }
}

// Stream staging with an 8-bit tier takes the variant that reads T2 rows as codes.
// A step launch (n.k set) never comes with 8-bit staging: kNewRow is above every T2 code.
template <typename T, int D>
hipError_t launch_attn_q(const AttnArgs& a, const StepArgs& n, int group, int chunk, bool vec, const AttnLaunch& L) {
  if (a.rows.q_k != nullptr) {
    if (n.k) return hipErrorInvalidValue;
    return launch_attn_g<T, D, true>(a, n, group, chunk, vec, L);
  }
  return launch_attn_g<T, D, false>(a, n, group, chunk, vec, L);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, const ScoreArgs* fold, int fold_tiles, hipStream_t s) {
  ScoreArgs f{};
  if (fold) f = *fold; else fold_tiles = 0;
  k_append<<<dim3(2 * a.layers * a.batch + fold_tiles * a.batch), 256, 0, s>>>(a, f, fold_tiles);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, const StepArgs& n, int dtype, int head_dim, int group, int chunk,
                       bool vector_pass, int layer_count, int chunks_now, hipEvent_t e0, hipEvent_t e1,
                       hipStream_t s) {
  const AttnLaunch L{dim3(chunks_now, a.kv_heads, layer_count * a.batch), e0, e1, s};
  if (dtype == TKV_BF16) {
    if (head_dim == 128) return launch_attn_q<bf16_t, 128>(a, n, group, chunk, vector_pass, L);
    if (head_dim == 64) return launch_attn_q<bf16_t, 64>(a, n, group, chunk, vector_pass, L);
  } else {
    if (head_dim == 128) return launch_attn_q<float, 128>(a, n, group, chunk, vector_pass, L);
    if (head_dim == 64) return launch_attn_q<float, 64>(a, n, group, chunk, vector_pass, L);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_finalize(const FinalizeArgs& a, const ScoreArgs* fold, int fold_tiles, int head_dim,
                           int layer_count, int max_live, hipStream_t s) {
  // four rows (or output elements) per thread once that still gives 512 or
  // more score blocks (long or batched caches); one per thread otherwise,
  // where the pass is a single round of short, latency-bound blocks
  const int wide_tiles = (max_live + 1023) / 1024;
  const bool wide = (int64_t)wide_tiles * a.batch * layer_count >= 512;
  FinalizeArgs f = a;
  ScoreArgs fa{};
  if (fold) fa = *fold; else fold_tiles = 0;
  f.tiles_grid = a.mlprev ? 0 : wide ? wide_tiles : (max_live + 255) / 256;
  f.fold_tiles = fold_tiles;
  const int hpb = 256 / (head_dim / (wide ? 4 : 1));
  const int fold_x = (fold_tiles + layer_count - 1) / layer_count;
  const dim3 grid(f.tiles_grid + (a.q_heads + hpb - 1) / hpb + fold_x, a.batch, layer_count);
  if (head_dim == 128 && wide)
    k_finalize<128, 4><<<grid, 256, 0, s>>>(f, fa);
  else if (head_dim == 128)
    k_finalize<128, 1><<<grid, 256, 0, s>>>(f, fa);
  else if (head_dim == 64 && wide)
    k_finalize<64, 4><<<grid, 256, 0, s>>>(f, fa);
  else if (head_dim == 64)
    k_finalize<64, 1><<<grid, 256, 0, s>>>(f, fa);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, int tiles_now, hipStream_t s) {
  k_score<<<dim3(tiles_now, a.batch), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fold(const ScoreArgs& a, int tiles, hipStream_t s) {
  if (a.parts != 4 && a.parts != 16) return hipErrorInvalidValue;
  k_fold<<<dim3(tiles, a.batch), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tkvd
