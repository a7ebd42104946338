// Reassignment kernels (Method §1 and §4 of "Not All Thoughts Need HBM",
// gist.science technical summary): score-ranked tier labels, the lists of
// changed rows, location-table updates, live-list rebuild and row copies.
//
// Ranking: candidates (not protected, not evicted) are ordered by the 64-bit
// key (bits(s) << 32) | (0xFFFFFFFF - position): s >= 0, so its fp32 bit
// pattern orders like the value, and a lower position wins a tie.  Keys are
// unique, so three order statistics (radix select, 8 passes of 8 bits, one
// work-group per sequence, LDS histograms with integer atomics) give the
// exact cut points between T3 | T2 | T1 | T0.  The batch-shared budget adds
// one joint select over the whole batch (the sequence as the second key).
#include <algorithm>

#include "tkv_internal.hpp"

namespace tkvd {
namespace {

constexpr int kBlock = 1024;

__device__ __forceinline__ uint64_t rank_key(float s, int i) {
  const uint32_t bits = s == 0.f ? 0u : __float_as_uint(s);
  return ((uint64_t)bits << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

__device__ __forceinline__ bool protected_pos(int i, int n, int prompt, int sinks, int recent) {
  return i < prompt || i < sinks || i >= n - recent;
}

// Radix select inside one work-group (1024 threads): the keys of K ascending
// ranks at once among the members of [0, count) (key_of(x, &key) is false
// for non-members; member keys are unique), 8 passes of 8 bits.  want[k] is
// the rank sought (>= members: none; its key is then ~0, above every key).
// Every thread calls it; on return cut[k] holds the results.  LDS
// histograms with integer atomics: the counts, and so the keys, do not
// depend on the order the atomics land in.
template <int K, typename KeyFn>
__device__ void block_select(KeyFn key_of, int count, const int32_t (&rank)[K], int32_t members, uint64_t (&cut)[K]) {
  __shared__ uint32_t hist[K][256];
  __shared__ uint64_t prefix[K];
  __shared__ int32_t want[K];
  const int tid = threadIdx.x;
  if (tid < K) {
    prefix[tid] = 0;
    want[tid] = rank[tid];
  }
  uint64_t mask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int x = tid; x < K * 256; x += kBlock) (&hist[0][0])[x] = 0;
    __syncthreads();
    for (int x = tid; x < count; x += kBlock) {
      uint64_t key;
      if (!key_of(x, &key)) continue;
      const uint32_t digit = (uint32_t)(key >> shift) & 255u;
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (want[k] < members && (key & mask) == prefix[k]) atomicAdd(&hist[k][digit], 1u);
    }
    __syncthreads();
    // digit of each cut: wave k scans the 256 bins of select k, 4 bins per lane
    const int wv = tid >> 6, lane = tid & 63;
    if (wv < K) {
      const int r = want[wv];
      if (r < members) {
        uint32_t c[4], sum4 = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          c[d] = hist[wv][4 * lane + d];
          sum4 += c[d];
        }
        uint32_t incl = sum4;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t y = __shfl_up(incl, off);
          if (lane >= off) incl += y;
        }
        uint32_t cum = incl - sum4;
        if ((uint32_t)r >= cum && (uint32_t)r < incl) {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            if ((uint32_t)r < cum + c[d]) {
              prefix[wv] |= (uint64_t)(4 * lane + d) << shift;
              want[wv] = r - (int)cum;
              break;
            }
            cum += c[d];
          }
        }
      }
    }
    mask |= (uint64_t)255u << shift;
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < K; ++k) cut[k] = rank[k] < members ? prefix[k] : ~0ull;
  __syncthreads();
}

// grid (batch), block 1024
__global__ __launch_bounds__(kBlock) void k_rank_label(const RankArgs a) {
  __shared__ int32_t ranks_s[3];
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* s = a.s + (int64_t)b * a.nmax;
  const uint8_t* old = a.tier_old + (int64_t)b * a.nmax;
  uint8_t* neu = a.tier_new + (int64_t)b * a.nmax;
  const int n = a.n, ncand = a.ncand[b];
  if (tid == 0) {
    int32_t r0 = a.rank[b][0], r1 = a.rank[b][1], r2 = a.rank[b][2];
    if (a.n0c) {  // batch-shared budget: T0 share from the joint select
      const int32_t n0c = a.n0c[b];
      r1 = r0 + min(ncand - r0 - n0c, a.t2cap);
      r2 = ncand - n0c;
    }
    ranks_s[0] = r0;
    ranks_s[1] = r1;
    ranks_s[2] = r2;
  }
  __syncthreads();
  const int32_t ranks[3] = {ranks_s[0], ranks_s[1], ranks_s[2]};
  auto key_of = [&](int i, uint64_t* key) {
    if (old[i] == TKV_T3 || protected_pos(i, n, a.prompt, a.sinks, a.recent)) return false;
    *key = rank_key(s[i], i);
    return true;
  };
  uint64_t cut[3];
  block_select<3>(key_of, n, ranks, ncand, cut);
  if (a.cuts_out) {
    if (tid < 3) a.cuts_out[(int64_t)b * 3 + tid] = cut[tid];
    return;
  }
  for (int i = tid; i < n; i += kBlock) {
    uint8_t t;
    if (old[i] == TKV_T3)
      t = TKV_T3;
    else if (protected_pos(i, n, a.prompt, a.sinks, a.recent))
      t = TKV_T0;
    else {
      const uint64_t key = rank_key(s[i], i);
      if (key < cut[0])
        t = TKV_T3;
      else if (key < cut[1])
        t = TKV_T2;
      else if (key >= cut[2])
        t = TKV_T0;
      else
        t = TKV_T1;
    }
    neu[i] = t;
  }
}

// Batch-shared HBM budget: the joint select over every sequence's remaining
// candidates (one work-group, block 1024), then the per-sequence T0 counts.
__global__ __launch_bounds__(kBlock) void k_joint_select(const JointArgs a) {
  __shared__ int32_t cnt[kMaxBatch];
  const int tid = threadIdx.x;
  const int n = a.n;
  for (int b = tid; b < a.batch; b += kBlock) cnt[b] = 0;
  // the take best of `remaining` keys: ascending rank remaining - take
  const int32_t rank[1] = {(int32_t)(a.remaining - a.take)};
  auto key_of = [&](int x, uint64_t* key) {
    const int b = x / n, i = x % n;
    const int64_t at = (int64_t)b * a.nmax + i;
    if (a.tier_old[at] == TKV_T3 || protected_pos(i, n, a.prompt, a.sinks, a.recent)) return false;
    const float sc = a.s[at];
    if (rank_key(sc, i) < a.cuts[(int64_t)b * 3]) return false;  // among the sequence's evicted
    const uint32_t bits = sc == 0.f ? 0u : __float_as_uint(sc);
    *key = ((uint64_t)bits << 32) | ((uint64_t)(63 - b) << 26) | (uint64_t)(0x3FFFFFFu - (uint32_t)i);
    return true;
  };
  uint64_t thr[1];
  if (a.take > 0) {
    block_select<1>(key_of, a.batch * n, rank, (int32_t)a.remaining, thr);
    for (int x = tid; x < a.batch * n; x += kBlock) {
      uint64_t key;
      if (key_of(x, &key) && key >= thr[0]) atomicAdd(&cnt[x / n], 1);
    }
  }
  __syncthreads();
  for (int b = tid; b < a.batch; b += kBlock) a.n0c[b] = cnt[b];
}

// Exclusive prefix sum over the block (1024 threads = 16 waves); returns
// the exclusive offset of this thread, *total = block sum.
__device__ int block_exclusive_scan(int x, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < 16; ++i) {
    if (i < w) base += wsum[i];
    tot += wsum[i];
  }
  __syncthreads();
  *total = tot;
  return base + incl - x;
}

// Changed rows, ascending by position.  grid (batch), block 1024.
__global__ __launch_bounds__(kBlock) void k_deltas(const DeltaArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint8_t* old = a.tier_old + (int64_t)b * a.nmax;
  const uint8_t* neu = a.tier_new + (int64_t)b * a.nmax;
  tkv_delta* pro = a.promote + (int64_t)b * a.nmax;
  tkv_delta* dem = a.demote + (int64_t)b * a.nmax;
  int np = 0, nd = 0;
  for (int i0 = 0; i0 < a.n; i0 += kBlock) {
    const int i = i0 + tid;
    uint8_t o = 0, w = 0;
    if (i < a.n) {
      o = old[i];
      w = neu[i];
    }
    const int fp = (i < a.n && w < o) ? 1 : 0;
    const int fd = (i < a.n && w > o) ? 1 : 0;
    int tp, td;
    const int op = block_exclusive_scan(fp, &tp);
    const int od = block_exclusive_scan(fd, &td);
    tkv_delta e;
    e.pos = (uint32_t)i;
    e.old_tier = o;
    e.new_tier = w;
    e.reserved = 0;
    if (fp) pro[np + op] = e;
    if (fd) dem[nd + od] = e;
    np += tp;
    nd += td;
  }
  if (tid == 0) {
    a.counts[2 * b] = np;
    a.counts[2 * b + 1] = nd;
  }
}

// loc[b][pos] = code for a list of updates.  grid (ceil(n/256)), block 256.
__global__ __launch_bounds__(256) void k_set_loc(const LocUpdate* u, int n, uint32_t* loc, int nmax) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k < n) loc[(int64_t)u[k].b * nmax + u[k].pos] = u[k].code;
}

// Live list = non-evicted positions in ascending order with their codes.
// grid (batch), block 1024.
__global__ __launch_bounds__(kBlock) void k_build_live(const LiveArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint8_t* tier = a.tier + (int64_t)b * a.nmax;
  const uint32_t* loc = a.loc + (int64_t)b * a.nmax;
  int base = 0;
  for (int i0 = 0; i0 < a.n; i0 += kBlock) {
    const int i = i0 + tid;
    const int f = (i < a.n && tier[i] != TKV_T3) ? 1 : 0;
    int tot;
    const int off = block_exclusive_scan(f, &tot);
    if (f) {
      a.live_pos[(int64_t)b * a.nmax + base + off] = i;
      a.live_loc[(int64_t)b * a.nmax + base + off] = loc[i];
    }
    base += tot;
  }
}

__device__ __forceinline__ char* area_row(const CopyArgs& a, int area, int which, int l, int b, int h, uint32_t idx) {
  const RowSpace& rs = a.rows;
  switch (area) {
    case kAreaPool: {
      char* base = (char*)(which ? rs.pool_v : rs.pool_k);
      return base + ((int64_t)l * rs.pool_lstride + (int64_t)b * rs.pool_bstride + (int64_t)h * rs.pool_hstride) *
                        a.elem_bytes +
             (int64_t)idx * a.head_bytes;
    }
    case kAreaStage: {
      char* base = (char*)(which ? rs.stage_v : rs.stage_k);
      return base + ((int64_t)(l % rs.stage_slots) * rs.stage_lstride + (int64_t)b * rs.stage_bstride +
                     (int64_t)h * rs.stage_hstride) *
                        a.elem_bytes +
             (int64_t)idx * a.head_bytes;
    }
    case kAreaPackOut: {
      char* base = (char*)(which ? a.pack_out_v : a.pack_out_k);
      return base + (((int64_t)l * a.kv_heads + h) * a.pack_out_rows + idx) * a.head_bytes;
    }
    default: {  // kAreaArena1: the pinned T1 arena, over PCIe
      char* base = (char*)(which ? a.arena.a1_v : a.arena.a1_k);
      return base + ((((int64_t)l * a.arena.batch + b) * a.kv_heads + h) * a.arena.cap1 + idx) * a.head_bytes;
    }
  }
}

// One op = one position of one sequence copied in every layer and kv head,
// K and V: work items (op, layer, K|V), one work-group each, in a
// grid-stride loop over the items.
__global__ __launch_bounds__(256) void k_copy_rows(const CopyArgs a, const RowOp* ops, int n_ops, int layers) {
  const int64_t items = (int64_t)n_ops * layers * 2;
  const int row_bytes = a.kv_heads * a.head_bytes;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int which = (int)(it & 1);
    const int64_t r = it >> 1;
    const int l = (int)(r % layers);
    const RowOp op = ops[r / layers];
    for (int off = threadIdx.x * 16; off < row_bytes; off += 256 * 16) {
      const int h = off / a.head_bytes, w = off % a.head_bytes;
      const char* src = area_row(a, op.src_area, which, l, op.b, h, op.src);
      char* dst = area_row(a, op.dst_area, which, l, op.b, h, op.dst);
      *reinterpret_cast<uint4*>(dst + w) = *reinterpret_cast<const uint4*>(src + w);
    }
  }
}

}  // namespace

hipError_t launch_rank_label(const RankArgs& a, int batch, hipStream_t s) {
  k_rank_label<<<batch, kBlock, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_joint_select(const JointArgs& a, hipStream_t s) {
  if (a.batch < 1 || a.batch > kMaxBatch || a.n >= (1 << 26) || (int64_t)a.batch * a.n >= INT32_MAX ||
      a.take > a.remaining)
    return hipErrorInvalidValue;
  k_joint_select<<<1, kBlock, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_deltas(const DeltaArgs& a, int batch, hipStream_t s) {
  k_deltas<<<batch, kBlock, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_set_loc(const LocUpdate* u, int n, uint32_t* loc, int nmax, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_set_loc<<<(n + 255) / 256, 256, 0, s>>>(u, n, loc, nmax);
  return hipGetLastError();
}

hipError_t launch_build_live(const LiveArgs& a, int batch, hipStream_t s) {
  k_build_live<<<batch, kBlock, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const CopyArgs& a, const RowOp* ops, int n_ops, int layers, int max_blocks,
                            hipStream_t s) {
  if (n_ops <= 0) return hipSuccess;
  const int64_t items = (int64_t)n_ops * layers * 2;
  const int64_t cap = max_blocks > 0 ? max_blocks : (1 << 20);
  k_copy_rows<<<(unsigned)std::min<int64_t>(items, cap), 256, 0, s>>>(a, ops, n_ops, layers);
  return hipGetLastError();
}

}  // namespace tkvd
