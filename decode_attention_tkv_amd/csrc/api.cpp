// C ABI of the tkv library (include/tkv.h): handle lifetime, prefill,
// append, decode attention, statistics and inspection hooks.  Reassignment
// lives in reassign.cpp.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "handle.hpp"
#include "host_util.hpp"

using namespace tkvd;

static thread_local std::string g_create_err;

int tkv_fail(tkv* t, int code, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  try {
    if (t)
      t->err = buf;
    else
      g_create_err = buf;
  } catch (...) {  // no room even for the message: the code still tells
  }
  return code;
}

static int device_alloc(tkv* t, void** p, size_t bytes) {
  if (bytes == 0) bytes = 256;
  if (!within_cap(*t, bytes)) {
    *p = nullptr;
    return tkv_fail(t, TKV_ENOMEM, "memory cap (%lld bytes) reached: %zu more device bytes asked",
                    (long long)t->mem_cap, bytes);
  }
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    return tkv_fail(t, TKV_ENOMEM, "hipMalloc(%zu bytes) failed: %s", bytes, hipGetErrorString(e));
  }
  t->device_allocs.push_back(*p);
  t->mem_held += (int64_t)bytes;
  return TKV_OK;
}

static int host_alloc(tkv* t, void** p, size_t bytes) {
  if (bytes == 0) bytes = 256;
  if (!within_cap(*t, bytes)) {
    *p = nullptr;
    return tkv_fail(t, TKV_ENOMEM, "memory cap (%lld bytes) reached: %zu more pinned bytes asked",
                    (long long)t->mem_cap, bytes);
  }
  hipError_t e = hipHostMalloc(p, bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    return tkv_fail(t, TKV_ENOMEM, "hipHostMalloc(%zu bytes) failed: %s", bytes, hipGetErrorString(e));
  }
  t->host_allocs.push_back(*p);
  t->mem_held += (int64_t)bytes;
  return TKV_OK;
}

static void release(tkv* t) {
  for (tkv* p : t->parts) {
    release(p);
    delete p;
  }
  t->parts.clear();
  if (t->side) (void)hipStreamSynchronize(t->side);
  if (t->side_v) (void)hipStreamSynchronize(t->side_v);
  if (t->wb) (void)hipStreamSynchronize(t->wb);
  for (void* p : t->device_allocs) (void)hipFree(p);
  for (void* p : t->host_allocs) (void)hipHostFree(p);
  if (t->d_ops) (void)hipFree(t->d_ops);
  if (t->h_ops) (void)hipHostFree(t->h_ops);
  if (t->fpack) (void)hipFree(t->fpack);
  t->fpack = nullptr;
  for (hipEvent_t e : t->ev_h2d) (void)hipEventDestroy(e);
  for (hipEvent_t e : t->ev_h2d_v) (void)hipEventDestroy(e);
  for (hipEvent_t e : t->ev_comp) (void)hipEventDestroy(e);
  if (t->ev_arena) (void)hipEventDestroy(t->ev_arena);
  if (t->side) (void)hipStreamDestroy(t->side);
  if (t->side_v) (void)hipStreamDestroy(t->side_v);
  if (t->wb) (void)hipStreamDestroy(t->wb);
  if (t->ev_gathered) (void)hipEventDestroy(t->ev_gathered);
  t->wb = nullptr;
  t->ev_gathered = nullptr;
  t->d_ops = t->h_ops = nullptr;
  t->ev_h2d.clear();
  t->ev_h2d_v.clear();
  t->ev_comp.clear();
  t->ev_arena = nullptr;
  t->side = nullptr;
  t->side_v = nullptr;
  for (hipEvent_t e : t->ev_free) (void)hipEventDestroy(e);
  for (auto& pr : t->ev_pending) {
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  t->device_allocs.clear();
  t->host_allocs.clear();
}

// Before the host reads the pinned arenas: the last reassignment's kernels,
// which write them, are done.
static int arena_settled(tkv* t) {
  HIP_TRY(t, hipEventSynchronize(t->ev_arena));
  return TKV_OK;
}

// A handle whose last reassignment failed part way is unusable (with
// per-layer budgets: any of its parts).
static int usable(tkv* t) {
  if (!t) return tkv_fail(nullptr, TKV_EINVAL, "handle is NULL");
  for (const tkv* p : t->parts) t->failed = t->failed || p->failed;
  if (t->failed) return tkv_fail(t, TKV_ESTATE, "handle unusable: an earlier reassignment failed part way");
  return TKV_OK;
}

// The result of a call on part i of a handle with per-layer budgets: its
// error message, and whether it left the part unusable, pass to the handle.
static int part_rc(tkv* t, size_t i, int rc) {
  if (rc != TKV_OK) {
    t->err = t->parts[i]->err;
    t->failed = t->failed || t->parts[i]->failed;
  }
  return rc;
}

// The part of a handle with per-layer budgets that holds `layer`.
static size_t part_of(const tkv* t, int layer) {
  size_t i = 0;
  while (i + 1 < t->parts.size() && t->part_l0[i + 1] <= layer) ++i;
  return i;
}

// The step state of a handle with per-layer budgets, from its parts: a step
// is in progress while any part has layers left.
static void mirror_parts(tkv* t) {
  const tkv* p0 = t->parts[0];
  t->n = p0->n;
  t->step = p0->step;
  t->state = p0->state;
  for (const tkv* p : t->parts)
    if (p->state == TkvState::InStep) t->state = TkvState::InStep;
}

// A layer's slice of a [layers][...] device array whose layers are
// `layer_bytes` apart.
static const void* layer_slice(const void* base, int layer, size_t layer_bytes) {
  return (const char*)base + (size_t)layer * layer_bytes;
}

extern "C" const char* tkv_last_error(const tkv_t* t) { return t ? t->err.c_str() : g_create_err.c_str(); }

// A part of a handle with per-layer budgets: the handle's score array and
// the layer count Eq. 1 averages over.
struct PartOf {
  float* s;
  int score_layers;
};

static int create_groups(const tkv_shape& s, int32_t delta, double evict_ratio, tkv_protect protect,
                         const tkv_options& o, tkv_t** out);

static int create_impl(const tkv_shape* shape, int32_t delta, double hbm_ratio, double evict_ratio,
                          tkv_protect protect, const tkv_options* opts, tkv_t** out, const PartOf* part = nullptr) {
  if (!out) return tkv_fail(nullptr, TKV_EINVAL, "out is NULL");
  *out = nullptr;
  if (!shape) return tkv_fail(nullptr, TKV_EINVAL, "shape is NULL");
  const tkv_shape& s = *shape;
  if (s.layers < 1 || s.q_heads < 1 || s.kv_heads < 1 || s.batch < 1 || s.max_tokens < 1)
    return tkv_fail(nullptr, TKV_EINVAL, "shape fields must be positive");
  if (s.q_heads % s.kv_heads) return tkv_fail(nullptr, TKV_EINVAL, "q_heads must be a multiple of kv_heads");
  const int group = s.q_heads / s.kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 5 && group != 8)
    return tkv_fail(nullptr, TKV_EINVAL, "q_heads/kv_heads = %d not supported (1, 2, 4, 5, 8)", group);
  if (s.head_dim != 64 && s.head_dim != 128) return tkv_fail(nullptr, TKV_EINVAL, "head_dim must be 64 or 128");
  if (s.batch > kMaxBatch) return tkv_fail(nullptr, TKV_EINVAL, "batch > %d", kMaxBatch);
  if (s.q_heads > kMaxQHeads) return tkv_fail(nullptr, TKV_EINVAL, "q_heads > %d", kMaxQHeads);
  if (s.max_tokens > (1 << 30)) return tkv_fail(nullptr, TKV_EINVAL, "max_tokens too large");
  if (s.dtype != TKV_BF16 && s.dtype != TKV_F32) return tkv_fail(nullptr, TKV_EINVAL, "unknown dtype");
  if (delta <= 0) return tkv_fail(nullptr, TKV_EINVAL, "delta must be > 0");
  auto ratio_ok = [](double r) { return std::isfinite(r) && r >= 0.0 && r <= 1.0; };
  if (!ratio_ok(hbm_ratio) || !ratio_ok(evict_ratio))
    return tkv_fail(nullptr, TKV_EINVAL, "hbm_ratio and evict_ratio must be in [0, 1]");
  if (protect.prompt < 0 || protect.sinks < 0 || protect.recent < 0)
    return tkv_fail(nullptr, TKV_EINVAL, "protect fields must be >= 0");
  tkv_options o{};
  if (opts) o = *opts;
  if (!ratio_ok(o.t2_ratio)) return tkv_fail(nullptr, TKV_EINVAL, "t2_ratio must be in [0, 1]");
  // grouped-query heads (q_heads >= 4 kv_heads) write more partials per row
  // read, so they take larger chunks: 1024 rows on the matrix cores (bf16),
  // whose logits tile needs no LDS for P, 512 on the vector path
  if (o.chunk == 0) {
    const bool mk = s.dtype == TKV_BF16 && (o.flags & TKV_FLAG_VECTOR_PASS) == 0;
    o.chunk = s.q_heads >= 4 * s.kv_heads ? (mk ? 1024 : 512) : 256;
  }
  if (o.chunk != 128 && o.chunk != 256 && o.chunk != 512 && o.chunk != 1024)
    return tkv_fail(nullptr, TKV_EINVAL, "chunk must be 128, 256, 512 or 1024");
  if (o.chunk == 1024 && !(s.dtype == TKV_BF16 && (s.q_heads == s.kv_heads || s.q_heads >= 4 * s.kv_heads) &&
                           (o.flags & TKV_FLAG_VECTOR_PASS) == 0))
    return tkv_fail(nullptr, TKV_EINVAL, "chunk 1024 needs the matrix-core path (bf16, 1 or >= 4 query heads per kv head)");
  if (o.mem_cap_bytes < 0) return tkv_fail(nullptr, TKV_EINVAL, "mem_cap_bytes must be >= 0");
  if (o.staging_layers < 0 || o.staging_layers == 1)
    return tkv_fail(nullptr, TKV_EINVAL, "staging_layers must be 0 or >= 2");
  if ((o.flags & TKV_FLAG_NO_T1) && (o.flags & TKV_FLAG_SHARED_HBM))
    return tkv_fail(nullptr, TKV_EINVAL, "TKV_FLAG_NO_T1 and TKV_FLAG_SHARED_HBM do not combine");
  if ((o.flags & TKV_FLAG_VECTOR_PASS) && o.t2_ratio > 0 && o.staging_layers != 0 && o.staging_layers < s.layers)
    return tkv_fail(nullptr, TKV_EINVAL, "TKV_FLAG_VECTOR_PASS does not combine with an 8-bit tier in stream staging");
  if ((o.flags & TKV_FLAG_SHARED_HBM) && s.max_tokens >= (1 << 26))
    return tkv_fail(nullptr, TKV_EINVAL, "TKV_FLAG_SHARED_HBM needs max_tokens < 2^26 (joint ranking keys)");
  if (o.layer_hbm) {
    // per-layer budgets: groups of consecutive layers with one ratio
    int groups = 1;
    for (int l = 0; l < s.layers; ++l) {
      if (!ratio_ok(o.layer_hbm[l])) return tkv_fail(nullptr, TKV_EINVAL, "layer_hbm[%d] must be in [0, 1]", l);
      if (l > 0 && o.layer_hbm[l] != o.layer_hbm[l - 1]) ++groups;
    }
    if (o.flags & (TKV_FLAG_NO_T1 | TKV_FLAG_SHARED_HBM))
      return tkv_fail(nullptr, TKV_EINVAL, "layer_hbm does not combine with TKV_FLAG_NO_T1 or TKV_FLAG_SHARED_HBM");
    if (groups > 1) return create_groups(s, delta, evict_ratio, protect, o, out);
    hbm_ratio = o.layer_hbm[0];  // one ratio: a plain handle
    o.layer_hbm = nullptr;
  }
  const bool resident = o.staging_layers == 0 || o.staging_layers >= s.layers;

  tkv* t = new tkv();
  // frees the half-built handle on every early return and on an exception
  struct Owner {
    tkv* t;
    ~Owner() {
      if (t) {
        release(t);
        delete t;
      }
    }
  } owner{t};
  t->L = s.layers;
  t->Hq = s.q_heads;
  t->Hkv = s.kv_heads;
  t->D = s.head_dim;
  t->B = s.batch;
  t->nmax = s.max_tokens;
  t->dtype = s.dtype;
  t->esz = s.dtype == TKV_BF16 ? 2 : 4;
  t->group = group;
  t->delta = delta;
  t->chunk = o.chunk;
  t->resident = resident;
  t->S = resident ? s.layers : o.staging_layers;
  t->hbm = hbm_ratio;
  t->evict = evict_ratio;
  t->t2 = o.t2_ratio;
  t->prompt = protect.prompt;
  t->sinks = protect.sinks;
  t->recent = protect.recent;
  t->flags = o.flags;
  t->mem_cap = o.mem_cap_bytes;
  {
    const hipError_t e = hipGetDevice(&t->device);
    if (e != hipSuccess) return tkv_fail(nullptr, TKV_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  }
  t->row_elems = (int64_t)s.kv_heads * s.head_dim;
  t->row_bytes = t->row_elems * t->esz;

  const int64_t nmax = s.max_tokens;
  const int64_t pmax = std::min<int64_t>(nmax, (int64_t)std::max(protect.prompt, protect.sinks) + protect.recent);
  const int64_t h_at_max = floor_ratio(hbm_ratio, nmax);
  t->shared_hbm = (o.flags & TKV_FLAG_SHARED_HBM) != 0;
  t->cap0 = (int)std::min<int64_t>(nmax, std::max(pmax, h_at_max) + delta + 1);
  if (t->shared_hbm) t->cap0 *= s.batch;  // slots of the whole batch in one space
  t->positional = resident && !t->shared_hbm;
  if (t->positional) t->cap0 = (int)nmax;  // one slot per position
  t->cap1 = (o.flags & TKV_FLAG_NO_T1) ? 1 : (int)std::max<int64_t>(1, std::min<int64_t>(nmax, nmax - h_at_max + 1));
  t->cap2 = o.t2_ratio > 0 ? (int)std::min<int64_t>(nmax, floor_ratio(o.t2_ratio, nmax) + 1) : 0;
  t->capS = t->positional ? 1 : resident ? t->cap1 + t->cap2 : t->cap1;  // positional: nothing lives there
  t->sh = (o.flags & TKV_FLAG_T2_HEAD_SCALES) ? s.kv_heads : 1;
  t->max_chunks = (int)((nmax + t->chunk - 1) / t->chunk);
  t->lstride = (int)((nmax + kLogitAlign - 1) / kLogitAlign * kLogitAlign);

  const size_t L = t->L, B = t->B, Hq = t->Hq;
  int rc = TKV_OK;
  auto dev = [&](void** p, size_t bytes) {
    if (rc == TKV_OK) rc = device_alloc(t, p, bytes);
  };
  const size_t pool_rows = (size_t)L * t->cap0 * (t->shared_hbm ? 1 : B);
  dev(&t->pool_k, pool_rows * t->row_bytes);
  dev(&t->pool_v, pool_rows * t->row_bytes);
  dev(&t->stage_k, (size_t)t->S * B * t->capS * t->row_bytes);
  dev(&t->stage_v, (size_t)t->S * B * t->capS * t->row_bytes);
  dev((void**)&t->live_loc, B * nmax * 4);
  dev((void**)&t->live_pos, B * nmax * 4);
  dev((void**)&t->tier, B * nmax);
  dev((void**)&t->loc, B * nmax * 4);
  if (part) {
    t->s = part->s;  // the handle of the parts holds the scores
    t->s_shared = true;
    t->score_layers = part->score_layers;
  } else {
    dev((void**)&t->s, B * nmax * 4);
  }
  t->vector_pass = (o.flags & TKV_FLAG_VECTOR_PASS) != 0 && s.dtype == TKV_BF16 && (group >= 4 || group == 1);
  // the matrix-core path (bf16, g >= 4 or g == 1) over resident staging
  t->defer = resident && s.dtype == TKV_BF16 && (group >= 4 || group == 1) && !t->vector_pass;
  if (t->defer) {
    // as many pending steps per forming launch as fit beside this step's
    // queries in the 16-row tile and in the forming launch's extra tiles (the
    // parts of a handle with per-layer budgets run in step, so they form the
    // same steps together)
    t->kmax = tkvd::defer_max_pending(group);
    t->ring = t->kmax + 1;
    dev(&t->qring, (size_t)t->ring * L * B * Hq * t->D * t->esz);
    dev((void**)&t->mlring, (size_t)t->ring * L * B * Hq * 2 * 4);
    dev((void**)&t->s_view, B * nmax * 4);
    dev((void**)&t->spart, L * t->Hkv * B * t->lstride * 4);
  } else {
    dev((void**)&t->logits, L * B * Hq * t->lstride * 4);
    dev((void**)&t->layer_score, L * B * t->lstride * 4);
  }
  dev((void**)&t->part_ml, L * B * Hq * t->max_chunks * 2 * 4);
  dev((void**)&t->part_o, L * B * Hq * t->max_chunks * t->D * 4);
  dev((void**)&t->tier_alt, B * nmax);
  if (t->shared_hbm) {
    dev((void**)&t->d_cuts, B * 3 * sizeof(uint64_t));
    dev((void**)&t->d_n0c, B * sizeof(int32_t));
  }
  const size_t counts_bytes = (B * 2 * 4 + 15) / 16 * 16;
  t->delta_block_bytes = counts_bytes + 2 * B * nmax * sizeof(tkv_delta);
  dev((void**)&t->d_counts, t->delta_block_bytes);
  if (t->d_counts) {
    t->d_promote = (tkv_delta*)((char*)t->d_counts + counts_bytes);
    t->d_demote = t->d_promote + B * nmax;
  }
  if (rc == TKV_OK) rc = host_alloc(t, &t->arena1_k, L * B * t->cap1 * t->row_bytes);
  if (rc == TKV_OK) rc = host_alloc(t, &t->arena1_v, L * B * t->cap1 * t->row_bytes);
  if (t->cap2 > 0) {
    const size_t codes = L * B * t->Hkv * (size_t)t->cap2 * t->D;
    if (rc == TKV_OK) rc = host_alloc(t, (void**)&t->arena2_k, codes);
    if (rc == TKV_OK) rc = host_alloc(t, (void**)&t->arena2_v, codes);
    if (rc == TKV_OK) rc = host_alloc(t, (void**)&t->ascale_k, L * B * t->cap2 * t->sh * 4);
    if (rc == TKV_OK) rc = host_alloc(t, (void**)&t->ascale_v, L * B * t->cap2 * t->sh * 4);
    if (!resident) {
      const size_t qc = (size_t)t->S * B * t->Hkv * t->cap2 * t->D;
      dev((void**)&t->qstage_k, qc);
      dev((void**)&t->qstage_v, qc);
      dev((void**)&t->qsscale_k, (size_t)t->S * B * t->cap2 * t->sh * 4);
      dev((void**)&t->qsscale_v, (size_t)t->S * B * t->cap2 * t->sh * 4);
    }
  }
  // the kernels of a stream-staging reassignment address the arenas directly
  auto map = [&](void* host, void** dev) {
    if (rc != TKV_OK || !host) return;
    const hipError_t e = hipHostGetDevicePointer(dev, host, 0);
    if (e != hipSuccess) rc = tkv_fail(t, TKV_EHIP, "hipHostGetDevicePointer: %s", hipGetErrorString(e));
  };
  map(t->arena1_k, &t->d_arena1_k);
  map(t->arena1_v, &t->d_arena1_v);
  map(t->arena2_k, (void**)&t->d_arena2_k);
  map(t->arena2_v, (void**)&t->d_arena2_v);
  map(t->ascale_k, (void**)&t->d_ascale_k);
  map(t->ascale_v, (void**)&t->d_ascale_v);
  if (rc == TKV_OK) rc = host_alloc(t, (void**)&t->h_counts, t->delta_block_bytes);
  if (rc == TKV_OK) {
    t->h_promote = (tkv_delta*)((char*)t->h_counts + counts_bytes);
    t->h_demote = t->h_promote + B * nmax;
  }
  if (rc == TKV_OK) {
    hipError_t e = hipStreamCreateWithFlags(&t->side, hipStreamNonBlocking);
    // stream staging only: resident handles keep the streams they had (an extra
    // stream per handle measurably slowed the resident pass, by ~1.5% at 7B)
    if (e == hipSuccess && !resident) e = hipStreamCreateWithFlags(&t->side_v, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&t->wb, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&t->ev_gathered, hipEventDisableTiming);
    t->ev_h2d.assign(t->S, nullptr);
    t->ev_h2d_v.assign(resident ? 0 : t->S, nullptr);
    t->ev_comp.assign(t->S, nullptr);
    t->comp_recorded.assign(t->S, 0);
    for (int i = 0; i < t->S && e == hipSuccess; ++i) {
      e = hipEventCreateWithFlags(&t->ev_h2d[i], hipEventDisableTiming);
      if (e == hipSuccess && !resident) e = hipEventCreateWithFlags(&t->ev_h2d_v[i], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&t->ev_comp[i], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipEventCreateWithFlags(&t->ev_arena, hipEventDisableTiming);
    if (e != hipSuccess) rc = tkv_fail(t, TKV_EHIP, "creating streams/events: %s", hipGetErrorString(e));
  }
  if (rc == TKV_OK) {
    hipError_t e = hipSuccess;
    if (e == hipSuccess) e = hipMemset(t->tier, kUnused, B * nmax);
    if (e == hipSuccess) e = hipMemset(t->tier_alt, kUnused, B * nmax);  // the two swap at each reassignment
    if (e == hipSuccess) e = hipMemset(t->loc, 0xFF, B * nmax * 4);
    if (e == hipSuccess && !t->s_shared) e = hipMemset(t->s, 0, B * nmax * 4);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) rc = tkv_fail(t, TKV_EHIP, "initialising device state: %s", hipGetErrorString(e));
  }
  if (rc != TKV_OK) {
    g_create_err = t->err;
    return rc;  // the owner frees the handle
  }
  t->nlive.assign(B, 0);
  t->prev_nlive.assign(B, 0);
  t->free0.resize(t->shared_hbm ? 1 : B);
  if (!t->positional)
    for (size_t q = 0; q < t->free0.size(); ++q) {
      auto& f = t->free0[q];
      f.resize(t->cap0);
      for (int i = 0; i < t->cap0; ++i) f[i] = t->cap0 - 1 - i;  // back() = lowest free slot
      if (t->flags & TKV_FLAG_TEST_SHUFFLE_SLOTS) {
        // seeded Fisher-Yates over the slots (splitmix64 words)
        uint64_t x = 0x5EEDull + q;
        for (int i = t->cap0 - 1; i > 0; --i) {
          uint64_t z = (x += 0x9E3779B97F4A7C15ull);
          z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
          z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
          z ^= z >> 31;
          std::swap(f[i], f[(size_t)(z % (uint64_t)(i + 1))]);
        }
      }
    }
  if (t->positional) t->h_aidx.assign((size_t)B * nmax, kNoLoc);
  t->h_tier.assign(B * nmax, kUnused);
  t->h_loc.assign(B * nmax, kNoLoc);
  t->t1_owner.resize(B);
  t->t2_owner.resize(B);
  t->t1_free.resize(B);
  t->t2_free.resize(B);
  std::memset(t->h_counts, 0, B * 2 * 4);
  t->st.hbm_bytes = (int64_t)(2 * (size_t)L * t->cap0 * (t->shared_hbm ? 1 : B) + 2 * (size_t)t->S * B * t->capS) *
                        t->row_bytes +
                    (resident ? 0 : (int64_t)(2 * (size_t)t->S * B * t->cap2) * (t->Hkv * t->D + 4 * t->sh));
  t->st.host_bytes = (int64_t)(2 * L * B * t->cap1) * t->row_bytes +
                     (int64_t)(2 * L * B * t->cap2) * (t->Hkv * t->D + 4 * t->sh);
  t->st.full_cache_bytes = (int64_t)(2 * L * B * nmax) * t->row_bytes;
  owner.t = nullptr;
  *out = t;
  return TKV_OK;
}
// Per-layer budgets: the handle the caller holds keeps the shape, the scores
// and the step state; each group of consecutive layers with one ratio is a
// part, a whole handle over its layers that shares those scores.  With stream
// staging each part streams its own layers, so each needs more layers than
// staging slots.  The memory cap is split over the parts by layer count.
static int create_groups(const tkv_shape& s, int32_t delta, double evict_ratio, tkv_protect protect,
                         const tkv_options& o, tkv_t** out) {
  std::vector<std::pair<int, int>> groups;  // [first layer, end)
  for (int l = 0; l < s.layers; ++l) {
    if (l > 0 && o.layer_hbm[l] == o.layer_hbm[l - 1])
      groups.back().second = l + 1;
    else
      groups.emplace_back(l, l + 1);
  }
  const bool stream = o.staging_layers >= 2 && o.staging_layers < s.layers;
  for (const auto& g : groups)
    if (stream && g.second - g.first <= o.staging_layers)
      return tkv_fail(nullptr, TKV_EINVAL,
                      "layer_hbm with stream staging: layer group [%d, %d) has no more layers than staging_layers %d",
                      g.first, g.second, o.staging_layers);
  tkv* t = new tkv();
  struct Owner {
    tkv* t;
    ~Owner() {
      if (t) {
        release(t);
        delete t;
      }
    }
  } owner{t};
  t->L = s.layers;
  t->Hq = s.q_heads;
  t->Hkv = s.kv_heads;
  t->D = s.head_dim;
  t->B = s.batch;
  t->nmax = s.max_tokens;
  t->dtype = s.dtype;
  t->esz = s.dtype == TKV_BF16 ? 2 : 4;
  t->group = s.q_heads / s.kv_heads;
  t->delta = delta;
  t->resident = !stream;
  t->evict = evict_ratio;
  t->t2 = o.t2_ratio;
  t->prompt = protect.prompt;
  t->sinks = protect.sinks;
  t->recent = protect.recent;
  t->flags = o.flags;
  t->mem_cap = o.mem_cap_bytes;
  t->row_elems = (int64_t)s.kv_heads * s.head_dim;
  t->row_bytes = t->row_elems * t->esz;
  {
    const hipError_t e = hipGetDevice(&t->device);
    if (e != hipSuccess) return tkv_fail(nullptr, TKV_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  }
  const size_t sbytes = (size_t)s.batch * s.max_tokens * 4;
  int rc = device_alloc(t, (void**)&t->s, sbytes);
  if (rc == TKV_OK) {
    hipError_t e = hipMemset(t->s, 0, sbytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) rc = tkv_fail(t, TKV_EHIP, "initialising the scores: %s", hipGetErrorString(e));
  }
  if (rc != TKV_OK) {
    g_create_err = t->err;
    return rc;
  }
  const PartOf pof{t->s, s.layers};
  for (const auto& g : groups) {
    tkv_shape ps = s;
    ps.layers = g.second - g.first;
    tkv_options po = o;
    po.layer_hbm = nullptr;
    if (o.mem_cap_bytes > 0) po.mem_cap_bytes = std::max<int64_t>(1, o.mem_cap_bytes / s.layers * ps.layers);
    tkv* part = nullptr;
    rc = create_impl(&ps, delta, o.layer_hbm[g.first], evict_ratio, protect, &po, &part, &pof);
    if (rc != TKV_OK) return rc;  // g_create_err holds the part's message
    t->parts.push_back(part);
    t->part_l0.push_back(g.first);
  }
  t->st.hbm_bytes = t->st.host_bytes = t->st.full_cache_bytes = 0;
  for (const tkv* p : t->parts) {
    t->st.hbm_bytes += p->st.hbm_bytes;
    t->st.host_bytes += p->st.host_bytes;
    t->st.full_cache_bytes += p->st.full_cache_bytes;
  }
  owner.t = nullptr;
  *out = t;
  return TKV_OK;
}

extern "C" int tkv_create(const tkv_shape* shape, int32_t delta, double hbm_ratio, double evict_ratio,
                          tkv_protect protect, const tkv_options* opts, tkv_t** out) {
  return guarded(nullptr, [&] { return create_impl(shape, delta, hbm_ratio, evict_ratio, protect, opts, out); });
}

static int destroy_impl(tkv_t* t) {
  if (!t) return TKV_OK;
  (void)hipDeviceSynchronize();
  release(t);
  delete t;
  return TKV_OK;
}
extern "C" int tkv_destroy(tkv_t* t) {
  return guarded(nullptr, [&] { return destroy_impl(t); });
}

static int prefill_impl(tkv_t* t, const void* k, const void* v, int32_t n_tokens, tkv_stream_t stream) {
  if (int rc = usable(t)) return rc;
  if (t->state != TkvState::Empty || t->n != 0) return tkv_fail(t, TKV_ESTATE, "prefill needs an empty cache");
  if (!k || !v) return tkv_fail(t, TKV_EINVAL, "k/v is NULL");
  if (misaligned(k) || misaligned(v)) return tkv_fail(t, TKV_EINVAL, "k/v not 16-byte aligned");
  if (n_tokens < 1) return tkv_fail(t, TKV_EINVAL, "n_tokens must be >= 1");
  if (n_tokens > t->nmax) return tkv_fail(t, TKV_ECAPACITY, "n_tokens %d > max_tokens %d", n_tokens, t->nmax);
  if (!t->parts.empty()) {
    // per-layer budgets: each part places its layers' rows by its own ratio
    const size_t lb = (size_t)t->B * n_tokens * t->row_bytes;  // one layer of k: [batch][n_tokens][kv_heads][head_dim]
    for (size_t i = 0; i < t->parts.size(); ++i) {
      const int l0 = t->part_l0[i];
      const int rc = prefill_impl(t->parts[i], layer_slice(k, l0, lb), layer_slice(v, l0, lb), n_tokens, stream);
      if (part_rc(t, i, rc)) return rc;
    }
    mirror_parts(t);
    return TKV_OK;
  }
  hipStream_t st = (hipStream_t)stream;
  const int n0 = n_tokens;

  // first placement: every score is 0, so candidates rank by position
  std::vector<uint8_t> first = first_placement(*t, n0);
  const int nt0 = (int)std::count(first.begin(), first.end(), (uint8_t)TKV_T0);
  const int nt1 = (int)std::count(first.begin(), first.end(), (uint8_t)TKV_T1);
  const int nt3 = n0 - nt0 - nt1;  // evicted at once (eviction-only baseline)
  if (nt0 * (t->shared_hbm ? t->B : 1) > t->cap0 || nt1 > t->cap1)
    return tkv_fail(t, TKV_ECAPACITY, "first placement does not fit (T0 %d/%d, T1 %d/%d)", nt0, t->cap0, nt1, t->cap1);

  std::vector<uint32_t> codes((size_t)t->B * n0);
  // positional staging: every live row at its position, and the T1 rows also
  // through a temporary [L][B][cap1] area on the way to their pinned home
  std::vector<uint32_t> codes1(t->positional ? (size_t)t->B * n0 : 0, kNoLoc);
  for (int b = 0; b < t->B; ++b) {
    auto& own = t->t1_owner[b];
    own.clear();
    for (int p = 0; p < n0; ++p) {
      uint32_t code;
      if (first[p] == TKV_T3) {
        code = kNoLoc;
      } else if (t->positional) {
        code = (uint32_t)p;
        if (first[p] == TKV_T1) {
          codes1[(size_t)b * n0 + p] = (uint32_t)(t->cap0 + own.size());
          t->h_aidx[(size_t)b * t->nmax + p] = (uint32_t)own.size();
          own.push_back(p);
        }
      } else if (first[p] == TKV_T0) {
        code = (uint32_t)t->free_list(b).back();
        t->free_list(b).pop_back();
      } else {
        code = (uint32_t)(t->cap0 + own.size());
        own.push_back(p);
      }
      codes[(size_t)b * n0 + p] = code;
      t->h_tier[(size_t)b * t->nmax + p] = first[p];
      t->h_loc[(size_t)b * t->nmax + p] = code;
    }
    t->nlive[b] = n0 - nt3;
  }
  t->st.evictions += (int64_t)nt3 * t->B;

  void* d_codes = nullptr;
  HIP_TRY(t, hipMallocAsync(&d_codes, codes.size() * 4 * (t->positional ? 2 : 1), st));
  HIP_TRY(t, hipMemcpyAsync(d_codes, codes.data(), codes.size() * 4, hipMemcpyHostToDevice, st));
  if (t->positional)
    HIP_TRY(t, hipMemcpyAsync((uint32_t*)d_codes + codes.size(), codes1.data(), codes1.size() * 4,
                              hipMemcpyHostToDevice, st));
  PlaceArgs pa{};
  pa.rows = t->rowspace();
  // T1 rows land in a staging area first: the resident staging itself, or (stream
  // mode, whose staging holds only S layers) a temporary [L][B][cap1] area.
  void* tmp_k = nullptr;
  void* tmp_v = nullptr;
  const size_t hb = (size_t)t->D * t->esz;  // bytes of one head's row
  size_t src_pitch = (size_t)t->capS * hb;
  // positional staging: when the T1 rows are one run of positions (the first
  // placement ranks candidates by position, so they normally are) their
  // pinned home fills straight from the pool
  int t1_first = -1;
  if (t->positional && nt1 > 0) {
    int lo = n0, hi = -1;
    for (int p = 0; p < n0; ++p)
      if (first[p] == TKV_T1) {
        lo = std::min(lo, p);
        hi = std::max(hi, p);
      }
    if (hi - lo + 1 == nt1) t1_first = lo;
  }
  if ((!t->resident || (t->positional && t1_first < 0)) && nt1 > 0) {
    const size_t bytes = (size_t)t->L * t->B * t->cap1 * t->row_bytes;
    HIP_TRY(t, hipMallocAsync(&tmp_k, bytes, st));
    HIP_TRY(t, hipMallocAsync(&tmp_v, bytes, st));
    pa.rows.stage_k = tmp_k;
    pa.rows.stage_v = tmp_v;
    pa.rows.stage_slots = t->L;
    pa.rows.stage_hstride = (int64_t)t->cap1 * t->D;
    pa.rows.stage_bstride = pa.rows.stage_hstride * t->Hkv;
    pa.rows.stage_lstride = pa.rows.stage_bstride * t->B;
    src_pitch = (size_t)t->cap1 * hb;
  }
  pa.k = k;
  pa.v = v;
  pa.codes = (const uint32_t*)d_codes;
  pa.batch = t->B;
  pa.n_tokens = n0;
  pa.kv_heads = t->Hkv;
  pa.head_bytes = (int32_t)hb;
  pa.elem_bytes = t->esz;
  const void* arena_src_k = pa.rows.stage_k;
  const void* arena_src_v = pa.rows.stage_v;
  if (t->positional) {
    // every live row at its position in the pool; the T1 rows also into the
    // temporary area unless they are one run of positions in the pool
    PlaceArgs pp = pa;
    pp.rows = t->rowspace();
    HIP_TRY(t, launch_place_rows(pp, t->L, st));
    if (nt1 > 0 && t1_first >= 0) {
      arena_src_k = (const char*)t->pool_k + (size_t)t1_first * hb;
      arena_src_v = (const char*)t->pool_v + (size_t)t1_first * hb;
      src_pitch = (size_t)t->cap0 * hb;
    } else if (nt1 > 0) {
      pa.codes = (const uint32_t*)d_codes + codes.size();
      HIP_TRY(t, launch_place_rows(pa, t->L, st));
    }
  } else {
    HIP_TRY(t, launch_place_rows(pa, t->L, st));
  }
  // T1 rows also go to their home in pinned host memory
  if (nt1 > 0) {
    const size_t width = (size_t)nt1 * hb;
    for (int which = 0; which < 2; ++which) {
      HIP_TRY(t, hipMemcpy2DAsync(which ? t->arena1_v : t->arena1_k, (size_t)t->cap1 * hb,
                                  which ? arena_src_v : arena_src_k, src_pitch, width,
                                  (size_t)t->L * t->B * t->Hkv, hipMemcpyDeviceToHost, st));
    }
    t->st.d2h_bytes += 2 * (int64_t)width * t->L * t->B * t->Hkv;
  }
  if (tmp_k) HIP_TRY(t, hipFreeAsync(tmp_k, st));
  if (tmp_v) HIP_TRY(t, hipFreeAsync(tmp_v, st));
  // per-position tables and the live list (the non-evicted positions, ascending)
  const int nl = n0 - nt3;
  std::vector<int32_t> pos((size_t)t->B * nl);
  std::vector<uint32_t> lloc((size_t)t->B * nl);
  for (int b = 0; b < t->B; ++b) {
    int j = 0;
    for (int p = 0; p < n0; ++p)
      if (first[p] != TKV_T3) {
        pos[(size_t)b * nl + j] = p;
        lloc[(size_t)b * nl + j] = codes[(size_t)b * n0 + p];
        ++j;
      }
  }
  for (int b = 0; b < t->B; ++b) {
    const size_t off = (size_t)b * t->nmax;
    HIP_TRY(t, hipMemcpyAsync(t->tier + off, &t->h_tier[off], n0, hipMemcpyHostToDevice, st));
    HIP_TRY(t, hipMemcpyAsync(t->loc + off, &t->h_loc[off], (size_t)n0 * 4, hipMemcpyHostToDevice, st));
    if (nl > 0) {
      HIP_TRY(t, hipMemcpyAsync(t->live_loc + off, &lloc[(size_t)b * nl], (size_t)nl * 4, hipMemcpyHostToDevice, st));
      HIP_TRY(t, hipMemcpyAsync(t->live_pos + off, &pos[(size_t)b * nl], (size_t)nl * 4, hipMemcpyHostToDevice, st));
    }
  }
  HIP_TRY(t, hipFreeAsync(d_codes, st));
  HIP_TRY(t, hipStreamSynchronize(st));
  t->n = n0;
  t->state = TkvState::Ready;
  return TKV_OK;
}
extern "C" int tkv_prefill(tkv_t* t, const void* k, const void* v, int32_t n_tokens, tkv_stream_t stream) {
  return guarded(t, [&] { return prefill_impl(t, k, v, n_tokens, stream); });
}

static int prefill_scored_impl(tkv_t* t, const void* k, const void* v, const void* q, int32_t n_tokens,
                                  tkv_stream_t stream) {
  if (!t) return tkv_fail(nullptr, TKV_EINVAL, "handle is NULL");
  if (!q) return tkv_fail(t, TKV_EINVAL, "q is NULL");
  if (misaligned(q)) return tkv_fail(t, TKV_EINVAL, "q not 16-byte aligned");
  if (int rc = tkv_prefill(t, k, v, n_tokens, stream)) return rc;
  hipStream_t st = (hipStream_t)stream;
  const size_t per = (size_t)t->L * t->B * t->Hq * n_tokens * 4;
  PrefillScoreArgs a{};
  HIP_TRY(t, hipMallocAsync((void**)&a.row_max, per, st));
  HIP_TRY(t, hipMallocAsync((void**)&a.row_inv, per, st));
  HIP_TRY(t, hipMallocAsync((void**)&a.colsum, per, st));
  a.k = k;
  a.q = q;
  a.s = t->s;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)t->D));
  a.inv_lh = (float)t->inv_lh();
  a.layers = t->L;
  a.batch = t->B;
  a.q_heads = t->Hq;
  a.kv_heads = t->Hkv;
  a.n = n_tokens;
  a.nmax = t->nmax;
  const hipError_t e = launch_prefill_scores(a, t->dtype, t->D, st);
  HIP_TRY(t, hipFreeAsync(a.row_max, st));
  HIP_TRY(t, hipFreeAsync(a.row_inv, st));
  HIP_TRY(t, hipFreeAsync(a.colsum, st));
  HIP_TRY(t, e);
  return tkv_reassign(t, stream);
}
extern "C" int tkv_prefill_scored(tkv_t* t, const void* k, const void* v, const void* q, int32_t n_tokens,
                                  tkv_stream_t stream) {
  return guarded(t, [&] { return prefill_scored_impl(t, k, v, q, n_tokens, stream); });
}

// Checks of an append; TKV_OK when a step may start.
static int append_check(tkv* t, const void* k, const void* v) {
  if (int rc = usable(t)) return rc;
  if (t->state == TkvState::InStep) return tkv_fail(t, TKV_ESTATE, "previous step has layers left");
  if (!k || !v) return tkv_fail(t, TKV_EINVAL, "k/v is NULL");
  if (misaligned(k) || misaligned(v)) return tkv_fail(t, TKV_EINVAL, "k/v not 16-byte aligned");
  if (t->n >= t->nmax) return tkv_fail(t, TKV_ECAPACITY, "max_tokens (%d) reached", t->nmax);
  if (t->positional) {
    // every position has its slot
  } else if (t->shared_hbm) {
    if ((int)t->free0[0].size() < t->B) return tkv_fail(t, TKV_ECAPACITY, "shared T0 pool full: reassign first");
  } else {
    for (int b = 0; b < t->B; ++b)
      if (t->free0[b].empty()) return tkv_fail(t, TKV_ECAPACITY, "T0 pool full (sequence %d): reassign first", b);
  }
  return TKV_OK;
}

// T0 slot of each sequence's new row (shared pool: the last B free slots;
// positional staging: its position).
static void append_slots(tkv* t, int32_t* slot) {
  if (t->positional) {
    for (int b = 0; b < t->B; ++b) slot[b] = t->n;
    return;
  }
  for (int b = 0; b < t->B; ++b)
    slot[b] = t->free_list(b)[t->free_list(b).size() - 1 - (t->shared_hbm ? b : 0)];
}

// Host side of an append whose launch has been enqueued.
static void append_commit(tkv* t, const int32_t* slot) {
  t->score_pending = false;
  for (int b = 0; b < t->B; ++b) {
    if (!t->positional) t->free_list(b).pop_back();  // shared: the B slots taken, from the back
    const size_t off = (size_t)b * t->nmax + t->n;
    t->h_tier[off] = TKV_T0;
    t->h_loc[off] = (uint32_t)slot[b];
    t->nlive[b] += 1;
  }
  t->n += 1;
  t->layers_done = 0;
  t->state = TkvState::InStep;
}

static int append_impl(tkv_t* t, const void* k, const void* v, tkv_stream_t stream) {
  if (t && !t->parts.empty()) {
    // per-layer budgets: every part must take the row before any does
    if (int rc = usable(t)) return rc;
    for (size_t i = 0; i < t->parts.size(); ++i)
      if (int rc = part_rc(t, i, append_check(t->parts[i], k, v))) return rc;
    const size_t lb = (size_t)t->B * t->row_bytes;  // one layer of k: [batch][kv_heads][head_dim]
    for (size_t i = 0; i < t->parts.size(); ++i) {
      const int l0 = t->part_l0[i];
      const int rc = append_impl(t->parts[i], layer_slice(k, l0, lb), layer_slice(v, l0, lb), stream);
      if (rc) {
        t->failed = i > 0;  // earlier parts hold the row already
        return part_rc(t, i, rc);
      }
    }
    t->layers_done = 0;
    mirror_parts(t);
    return TKV_OK;
  }
  int rc = append_check(t, k, v);
  if (rc) return rc;
  AppendArgs a{};
  a.rows = t->rowspace();
  a.k = k;
  a.v = v;
  a.live_loc = t->live_loc;
  a.live_pos = t->live_pos;
  a.tier = t->tier;
  a.loc = t->loc;
  a.s = t->s;
  a.layers = t->L;
  a.batch = t->B;
  a.kv_heads = t->Hkv;
  a.head_dim = t->D;
  a.elem_bytes = t->esz;
  a.nmax = t->nmax;
  a.pos = t->n;
  append_slots(t, a.slot);
  for (int b = 0; b < t->B; ++b) a.nlive[b] = t->nlive[b];
  HIP_TRY(t, launch_append(a, t->score_pending ? &t->pending_score : nullptr, t->pending_tiles,
                           (hipStream_t)stream));
  append_commit(t, a.slot);
  return TKV_OK;
}
extern "C" int tkv_append(tkv_t* t, const void* k, const void* v, tkv_stream_t stream) {
  return guarded(t, [&] { return append_impl(t, k, v, stream); });
}

// A timing event from the pool.  The launch binds it to its kernel's own start
// or end; no host reads device memory through it, so it carries no
// system-scope fence (which would write back the caches at every launch).
static int take_event(tkv* t, hipEvent_t* e) {
  if (t->ev_free.empty()) {
    hipEvent_t x;
    HIP_TRY(t, hipEventCreateWithFlags(&x, hipEventDisableSystemFence));
    t->ev_free.push_back(x);
  }
  *e = t->ev_free.back();
  t->ev_free.pop_back();
  return TKV_OK;
}

static int drain_events(tkv* t) {
  for (auto& pr : t->ev_pending) {
    HIP_TRY(t, hipEventSynchronize(pr.second));
    float ms = 0.f;
    HIP_TRY(t, hipEventElapsedTime(&ms, pr.first, pr.second));
    t->st.attn_kernel_ms += ms;
    t->st.attn_kernel_launches += 1;
    t->ev_free.push_back(pr.first);
    t->ev_free.push_back(pr.second);
  }
  t->ev_pending.clear();
  return TKV_OK;
}

// Deferred fold: partial sums per row, 16 when a row's list (layers x kv
// heads) is longer than 640 entries, else 4.
static int fold_parts(const tkv* t) { return t->L * t->Hkv > 640 ? 16 : 4; }

// Deferred Eq. 1: the fold of the pending steps' sums into s.
static ScoreArgs defer_fold_args(const tkv* t) {
  ScoreArgs sa{};
  sa.layer_score = t->spart;  // rows [layer][kv head], summed in that order
  sa.live_pos = t->live_pos;
  sa.s = t->s;
  sa.inv_lh = (float)t->inv_lh();
  sa.layers = t->L * t->Hkv;
  sa.batch = t->B;
  sa.nmax = t->nmax;
  sa.lstride = t->lstride;
  sa.parts = fold_parts(t);
  for (int b = 0; b < t->B; ++b) sa.nlive[b] = t->prev_nlive[b];
  return sa;
}

// tiles of the deferred fold (256 / parts rows each)
static int prev_tiles(const tkv* t) {
  int m = 0;
  for (int b = 0; b < t->B; ++b) m = std::max(m, t->prev_nlive[b]);
  const int rows = 256 / fold_parts(t);
  return (m + rows - 1) / rows;
}

// The deferral's ring arguments of an attention launch.
static void ring_args(const tkv* t, AttnArgs* a) {
  a->ring = t->ring;
  a->qcur = t->qcur;
  a->qring = t->qring;
  a->mlring = t->mlring;
  a->qslot = (int64_t)t->L * t->B * t->Hq * t->D;
  a->mlslot = (int64_t)t->L * t->B * t->Hq * 2;
  a->spart = t->spart;
}

// Deferred Eq. 1: how many pending steps the running step's launches form
// (and its merge pass folds): all of them once kmax are pending, else none.
// Fixed for the whole step: pend changes only when a step ends or a
// reassignment commits.
static int defer_now(const tkv* t) {
  if (!t->defer) return 0;
  return t->pend >= t->kmax ? t->pend : 0;
}

// Split-K attention + chunk merge for layers [lb, lb + lc) whose q/out start at q, out.
// step: the fused append + Eq. 1 update of a whole-step launch, or nullptr.
static int launch_layers(tkv* t, int lb, int lc, const void* q, float* out, int max_live, hipStream_t st,
                         const StepArgs* step = nullptr) {
  AttnArgs a{};
  const int now = defer_now(t);
  if (t->defer) {
    a.prev_mode = now ? 1 : 0;
    a.prev_steps = now;
    ring_args(t, &a);
  }
  a.rows = t->rowspace();
  a.live_loc = t->live_loc;
  a.q = q;
  a.logits = t->logits;
  a.part_ml = t->part_ml;
  a.part_o = t->part_o;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)t->D));
  a.layer_begin = lb;
  a.batch = t->B;
  a.q_heads = t->Hq;
  a.kv_heads = t->Hkv;
  a.nmax = t->nmax;
  a.max_chunks = t->max_chunks;
  a.lstride = t->lstride;
  for (int b = 0; b < t->B; ++b) a.nlive[b] = t->nlive[b];
  const int chunks_now = (max_live + t->chunk - 1) / t->chunk;
  const bool timed = (t->flags & TKV_FLAG_TIME_KERNELS) != 0 && chunks_now > 0;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (timed) {
    int rc = take_event(t, &e0);
    if (!rc) rc = take_event(t, &e1);
    if (rc) return rc;
  }
  StepArgs none{};
  if (chunks_now > 0)
    HIP_TRY(t, launch_attn(a, step ? *step : none, t->dtype, t->D, t->group, t->chunk, t->vector_pass, lc, chunks_now, e0, e1,
                           st));
  if (timed) {
    t->ev_pending.emplace_back(e0, e1);
    int64_t rows = 0;
    for (int b = 0; b < t->B; ++b) rows += t->nlive[b];
    t->st.attn_kv_bytes += rows * lc * 2 * t->row_bytes;
  }
  FinalizeArgs f{};
  f.logits = t->logits;
  f.part_ml = t->part_ml;
  f.part_o = t->part_o;
  f.out = out;
  f.layer_score = t->layer_score;
  f.layer_begin = lb;
  f.batch = t->B;
  f.q_heads = t->Hq;
  f.nmax = t->nmax;
  f.max_chunks = t->max_chunks;
  f.chunk = t->chunk;
  f.lstride = t->lstride;
  for (int b = 0; b < t->B; ++b) f.nlive[b] = t->nlive[b];
  // deferred Eq. 1: keep (M, 1/L) for the next step; the step's last layer
  // group also folds the pending step's sums, complete once every layer ran
  ScoreArgs fold{};
  int fold_tiles = 0;
  if (t->defer) {
    f.mlprev = t->mlring + (size_t)((t->qcur + 1) % t->ring) * t->L * t->B * t->Hq * 2;
    f.q = q;
    f.qsave = (char*)t->qring + (size_t)((t->qcur + 1) % t->ring) * t->L * t->B * t->Hq * t->D * t->esz;
    if (now && lb + lc == t->L) {
      fold = defer_fold_args(t);
      fold_tiles = prev_tiles(t);
    }
  }
  if (max_live > 0)
    HIP_TRY(t, launch_finalize(f, fold_tiles ? &fold : nullptr, fold_tiles, t->D, lc, max_live, st));
  return TKV_OK;
}

// Deferred Eq. 1 of the pending steps on their own: a score-only pass over
// their rows' K in every layer, then the fold, into s (commit: nothing is
// pending afterwards) or into a copy of s that a score read returns (the
// steps stay pending and are later formed and folded exactly as without the
// read).  view: the copy to fold into when not committing, already holding s
// (the parts of a handle with per-layer budgets fold into one), or nullptr
// for this handle's own copy.
static int flush_deferred(tkv* t, hipStream_t st, bool commit, float* view = nullptr) {
  AttnArgs a{};
  a.rows = t->rowspace();
  a.live_loc = t->live_loc;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)t->D));
  a.layer_begin = 0;
  a.batch = t->B;
  a.q_heads = t->Hq;
  a.kv_heads = t->Hkv;
  a.nmax = t->nmax;
  a.max_chunks = t->max_chunks;
  a.lstride = t->lstride;
  a.prev_mode = 2;
  a.prev_steps = t->pend;
  ring_args(t, &a);
  int m = 0;
  for (int b = 0; b < t->B; ++b) {
    a.nlive[b] = t->prev_nlive[b];  // the last pending step's rows (the live list only grew since)
    m = std::max(m, a.nlive[b]);
  }
  const int chunks = (m + t->chunk - 1) / t->chunk;
  StepArgs none{};
  ScoreArgs fold = defer_fold_args(t);
  if (!commit) {
    if (!view) {
      HIP_TRY(t, hipMemcpyAsync(t->s_view, t->s, (size_t)t->B * t->nmax * 4, hipMemcpyDeviceToDevice, st));
      view = t->s_view;
    }
    fold.s = view;
  }
  if (chunks > 0) {
    HIP_TRY(t, launch_attn(a, none, t->dtype, t->D, t->group, t->chunk, false, t->L, chunks, nullptr, nullptr, st));
    HIP_TRY(t, launch_fold(fold, prev_tiles(t), st));
  }
  if (commit) t->pend = 0;
  return TKV_OK;
}

// Stream mode: copy layers' T1 rows from the pinned arena into their staging
// slot (layer mod S) on the side streams (K rows and 8-bit rows on one, V rows
// on the other), up to layer `upto`, each after the attention that last read
// that slot.  With an even S >= 4 the layers go in groups of S / 2: layers
// x .. x + S/2 - 1 (x a multiple of S / 2) take slots x mod S onwards, which
// are adjacent, as their rows are in the arena, so one copy per area moves
// the group at one pitch (S / 2 times the rows, the same fixed costs).  The
// two halves of the slots alternate.  A group is issued once all its layers
// are within `upto`, so no slot is still waiting for the attention that last
// read it to be enqueued.
static int issue_prefetch(tkv* t, int upto) {
  if (t->arena_pending) {
    HIP_TRY(t, hipStreamWaitEvent(t->side, t->ev_arena, 0));
    HIP_TRY(t, hipStreamWaitEvent(t->side_v, t->ev_arena, 0));
    t->arena_pending = false;
  }
  size_t n1max = 0, n2max = 0;
  for (int b = 0; b < t->B; ++b) {
    n1max = std::max(n1max, t->t1_owner[b].size());
    n2max = std::max(n2max, t->t2_owner[b].size());
  }
  const int per_copy = (t->S >= 4 && t->S % 2 == 0) ? t->S / 2 : 1;
  while (t->next_issue <= upto && t->next_issue < t->L) {
    const int x = t->next_issue, slot = x % t->S;  // x is a multiple of per_copy
    const int nx = std::min(per_copy, t->L - x);  // layers in this copy; slots slot .. slot + nx - 1
    if (x + nx - 1 > upto) break;
    for (int k = 0; k < nx; ++k)
      if (t->comp_recorded[slot + k]) {
        HIP_TRY(t, hipStreamWaitEvent(t->side, t->ev_comp[slot + k], 0));
        HIP_TRY(t, hipStreamWaitEvent(t->side_v, t->ev_comp[slot + k], 0));
      }
    if (t->flags & TKV_FLAG_TEST_DELAY_COPIES) {
      HIP_TRY(t, launch_delay(kTestDelayIters, t->side));
      HIP_TRY(t, launch_delay(kTestDelayIters, t->side_v));
    }
    if (n1max > 0) {
      const size_t hb = (size_t)t->D * t->esz;
      const size_t width = n1max * hb;
      for (int which = 0; which < 2; ++which) {
        char* dst = (char*)(which ? t->stage_v : t->stage_k) + (size_t)slot * t->B * t->capS * t->row_bytes;
        const char* src = (const char*)(which ? t->arena1_v : t->arena1_k) + (size_t)x * t->B * t->cap1 * t->row_bytes;
        HIP_TRY(t, hipMemcpy2DAsync(dst, (size_t)t->capS * hb, src, (size_t)t->cap1 * hb, width,
                                    (size_t)nx * t->B * t->Hkv, hipMemcpyHostToDevice, which ? t->side_v : t->side));
      }
      t->st.h2d_bytes += 2 * (int64_t)width * nx * t->B * t->Hkv;
    }
    if (n2max > 0) {
      // 8-bit rows: codes and scales over PCIe into the slot's T2 area, which the
      // attention pass reads directly
      const size_t cw = n2max * t->D;
      const size_t c_layer = (size_t)t->B * t->Hkv * t->cap2 * t->D;
      const size_t s_layer = (size_t)t->B * t->cap2 * t->sh;
      for (int which = 0; which < 2; ++which) {
        int8_t* qd = (which ? t->qstage_v : t->qstage_k) + (size_t)slot * c_layer;
        float* sd = (which ? t->qsscale_v : t->qsscale_k) + (size_t)slot * s_layer;
        HIP_TRY(t, hipMemcpy2DAsync(qd, (size_t)t->cap2 * t->D, (which ? t->arena2_v : t->arena2_k) + (size_t)x * c_layer,
                                    (size_t)t->cap2 * t->D, cw, (size_t)nx * t->B * t->Hkv, hipMemcpyHostToDevice,
                                    t->side));
        HIP_TRY(t, hipMemcpy2DAsync(sd, (size_t)t->cap2 * t->sh * 4,
                                    (which ? t->ascale_v : t->ascale_k) + (size_t)x * s_layer, (size_t)t->cap2 * t->sh * 4,
                                    n2max * t->sh * 4, (size_t)nx * t->B, hipMemcpyHostToDevice, t->side));
      }
      t->st.h2d_bytes += 2 * (int64_t)nx * (cw * t->B * t->Hkv + n2max * t->sh * 4 * t->B);
    }
    for (int k = 0; k < nx; ++k) {
      HIP_TRY(t, hipEventRecord(t->ev_h2d[slot + k], t->side));
      HIP_TRY(t, hipEventRecord(t->ev_h2d_v[slot + k], t->side_v));
    }
    t->next_issue += nx;
  }
  return TKV_OK;
}

// Close a step whose every layer is enqueued: its Eq. 1 update becomes pending.
static void end_step(tkv* t, int max_live) {
  ScoreArgs sa{};
  sa.layer_score = t->layer_score;
  sa.live_pos = t->live_pos;
  sa.s = t->s;
  sa.inv_lh = (float)t->inv_lh();
  sa.layers = t->L;
  sa.batch = t->B;
  sa.nmax = t->nmax;
  sa.lstride = t->lstride;
  for (int b = 0; b < t->B; ++b) sa.nlive[b] = t->nlive[b];
  if (t->defer) {
    // computed and folded by the next step's launches (or by tkv_flush_score)
    t->pend = t->pend - defer_now(t) + (max_live > 0 ? 1 : 0);
    t->prev_nlive = t->nlive;
    t->qcur = (t->qcur + 1) % t->ring;
  } else {
    // applied by the next append's launch (or by tkv_flush_score)
    t->pending_score = sa;
    t->pending_tiles = (max_live + 255) / 256;
    t->score_pending = t->pending_tiles > 0;
  }
  t->step += 1;
  t->state = TkvState::Ready;
}

static int decode_attn_impl(tkv_t* t, int32_t layer_begin, int32_t layer_count, const void* q, float* out,
                               tkv_stream_t stream) {
  if (int rc = usable(t)) return rc;
  if (t->state != TkvState::InStep) return tkv_fail(t, TKV_ESTATE, "no step in progress (append first)");
  if (!q || !out) return tkv_fail(t, TKV_EINVAL, "q/out is NULL");
  if (misaligned(q) || misaligned(out)) return tkv_fail(t, TKV_EINVAL, "q/out not 16-byte aligned");
  if (layer_begin != t->layers_done)
    return tkv_fail(t, TKV_ESTATE, "layer groups must come in order: expected layer %d", t->layers_done);
  if (layer_count < 1 || layer_begin + layer_count > t->L) return tkv_fail(t, TKV_EINVAL, "bad layer range");
  if (!t->parts.empty()) {
    // per-layer budgets: each part runs its share of the range, in layer order
    const size_t ql = (size_t)t->B * t->Hq * t->D * t->esz, ol = (size_t)t->B * t->Hq * t->D;
    const int end = layer_begin + layer_count;
    for (size_t i = 0; i < t->parts.size(); ++i) {
      const int p0 = t->part_l0[i], p1 = p0 + t->parts[i]->L;
      const int a = std::max(layer_begin, p0), e = std::min(end, p1);
      if (a >= e) continue;
      const int rc = decode_attn_impl(t->parts[i], a - p0, e - a, layer_slice(q, a - layer_begin, ql),
                                      out + (size_t)(a - layer_begin) * ol, stream);
      if (part_rc(t, i, rc)) return rc;
    }
    t->layers_done += layer_count;
    mirror_parts(t);
    return TKV_OK;
  }
  hipStream_t st = (hipStream_t)stream;
  int max_live = 0;
  for (int b = 0; b < t->B; ++b) max_live = std::max(max_live, t->nlive[b]);

  if (t->resident) {
    int rc = launch_layers(t, layer_begin, layer_count, q, out, max_live, st);
    if (rc) return rc;
  } else {
    if (layer_begin == 0) t->next_issue = 0;
    const size_t q_layer = (size_t)t->B * t->Hq * t->D * t->esz;
    const size_t o_layer = (size_t)t->B * t->Hq * t->D;
    for (int i = 0; i < layer_count; ++i) {
      const int l = layer_begin + i, slot = l % t->S;
      int rc = issue_prefetch(t, l + t->S - 1);
      if (rc) return rc;
      HIP_TRY(t, hipStreamWaitEvent(st, t->ev_h2d[slot], 0));
      HIP_TRY(t, hipStreamWaitEvent(st, t->ev_h2d_v[slot], 0));
      rc = launch_layers(t, l, 1, (const char*)q + i * q_layer, out + i * o_layer, max_live, st);
      if (rc) return rc;
      HIP_TRY(t, hipEventRecord(t->ev_comp[slot], st));
      t->comp_recorded[slot] = 1;
    }
  }

  t->layers_done += layer_count;
  if (t->layers_done == t->L) end_step(t, max_live);
  return TKV_OK;
}
extern "C" int tkv_decode_attn(tkv_t* t, int32_t layer_begin, int32_t layer_count, const void* q, float* out,
                               tkv_stream_t stream) {
  return guarded(t, [&] { return decode_attn_impl(t, layer_begin, layer_count, q, out, stream); });
}

static int decode_step_impl(tkv_t* t, const void* k, const void* v, const void* q, float* out,
                               tkv_stream_t stream) {
  if (t && !t->parts.empty()) {
    // per-layer budgets: every part must take the row, then each runs its step
    if (int rc = usable(t)) return rc;
    if (!q || !out) return tkv_fail(t, TKV_EINVAL, "q/out is NULL");
    if (misaligned(q) || misaligned(out)) return tkv_fail(t, TKV_EINVAL, "q/out not 16-byte aligned");
    for (size_t i = 0; i < t->parts.size(); ++i)
      if (int rc = part_rc(t, i, append_check(t->parts[i], k, v))) return rc;
    const size_t kl = (size_t)t->B * t->row_bytes;
    const size_t ql = (size_t)t->B * t->Hq * t->D * t->esz, ol = (size_t)t->B * t->Hq * t->D;
    for (size_t i = 0; i < t->parts.size(); ++i) {
      const int l0 = t->part_l0[i];
      const int rc = decode_step_impl(t->parts[i], layer_slice(k, l0, kl), layer_slice(v, l0, kl),
                                      layer_slice(q, l0, ql), out + (size_t)l0 * ol, stream);
      if (rc) {
        t->failed = i > 0;  // earlier parts hold the row already
        return part_rc(t, i, rc);
      }
    }
    t->layers_done = 0;
    mirror_parts(t);
    return TKV_OK;
  }
  int rc = append_check(t, k, v);
  if (rc) return rc;
  if (!q || !out) return tkv_fail(t, TKV_EINVAL, "q/out is NULL");
  if (misaligned(q) || misaligned(out)) return tkv_fail(t, TKV_EINVAL, "q/out not 16-byte aligned");
  if (!t->resident) {
    rc = tkv_append(t, k, v, stream);
    return rc ? rc : tkv_decode_attn(t, 0, t->L, q, out, stream);
  }
  StepArgs n{};
  n.k = k;
  n.v = v;
  n.live_loc = t->live_loc;
  n.live_pos = t->live_pos;
  n.tier = t->tier;
  n.loc = t->loc;
  n.s = t->s;
  n.pos = t->n;
  n.fold = t->score_pending ? 1 : 0;
  n.f = t->pending_score;
  append_slots(t, n.slot);
  append_commit(t, n.slot);
  int max_live = 0;
  for (int b = 0; b < t->B; ++b) max_live = std::max(max_live, t->nlive[b]);
  rc = launch_layers(t, 0, t->L, q, out, max_live, (hipStream_t)stream, &n);
  if (rc) return rc;
  t->layers_done = t->L;
  end_step(t, max_live);
  return TKV_OK;
}
extern "C" int tkv_decode_step(tkv_t* t, const void* k, const void* v, const void* q, float* out,
                               tkv_stream_t stream) {
  return guarded(t, [&] { return decode_step_impl(t, k, v, q, out, stream); });
}

static int stats_impl(tkv_t* t, tkv_stats_t* out) {
  if (!t || !out) return tkv_fail(t, TKV_EINVAL, "NULL argument");
  if (!t->parts.empty()) {
    // per-layer budgets: pools, traffic and time summed over the parts; the
    // tier counts weighted by each part's layers; the evictions (the same rows
    // in every part) and the reassignments counted once
    tkv_stats_t a{};
    for (size_t i = 0; i < t->parts.size(); ++i) {
      tkv_stats_t ps{};
      if (int rc = part_rc(t, i, stats_impl(t->parts[i], &ps))) return rc;
      const int64_t lw = t->parts[i]->L;
      for (int x = 0; x < 4; ++x) a.tier_count[x] += ps.tier_count[x] * lw;
      a.hbm_bytes += ps.hbm_bytes;
      a.host_bytes += ps.host_bytes;
      a.full_cache_bytes += ps.full_cache_bytes;
      a.promotions += ps.promotions;
      a.demotions += ps.demotions;
      a.h2d_bytes += ps.h2d_bytes;
      a.d2h_bytes += ps.d2h_bytes;
      a.attn_kernel_ms += ps.attn_kernel_ms;
      a.attn_kernel_launches += ps.attn_kernel_launches;
      a.attn_kv_bytes += ps.attn_kv_bytes;
      a.reassign_ms += ps.reassign_ms;
      a.mem_bytes += ps.mem_bytes;
      if (i == 0) {
        a.step = ps.step;
        a.n_tokens = ps.n_tokens;
        a.evictions = ps.evictions;
        a.reassigns = ps.reassigns;
      }
    }
    a.mem_bytes += t->mem_held;
    *out = a;
    return TKV_OK;
  }
  if (int rc = arena_settled(t)) return rc;
  HIP_TRY(t, hipStreamSynchronize(t->side));
  if (t->side_v) HIP_TRY(t, hipStreamSynchronize(t->side_v));
  HIP_TRY(t, hipStreamSynchronize(t->wb));
  int rc = drain_events(t);
  if (rc) return rc;
  t->st.step = t->step;
  t->st.n_tokens = t->n;
  t->st.mem_bytes = t->mem_held;
  for (int i = 0; i < 4; ++i) t->st.tier_count[i] = 0;
  for (int b = 0; b < t->B; ++b)
    for (int p = 0; p < t->n; ++p) {
      const uint8_t x = t->h_tier[(size_t)b * t->nmax + p];
      if (x < 4) t->st.tier_count[x] += 1;
    }
  *out = t->st;
  return TKV_OK;
}
extern "C" int tkv_stats(tkv_t* t, tkv_stats_t* out) {
  return guarded(t, [&] { return stats_impl(t, out); });
}

int tkv_flush_score(tkv* t, hipStream_t stream) {
  for (size_t i = 0; i < t->parts.size(); ++i)  // per-layer budgets: every part's pending increment
    if (int rc = part_rc(t, i, tkv_flush_score(t->parts[i], stream))) return rc;
  if (t->defer) return t->pend ? flush_deferred(t, stream, true) : TKV_OK;
  if (!t->score_pending) return TKV_OK;
  HIP_TRY(t, launch_score(t->pending_score, t->pending_tiles, stream));
  t->score_pending = false;
  return TKV_OK;
}

static int read_scores_impl(tkv_t* t, float* scores, tkv_stream_t stream) {
  if (int rc = usable(t)) return rc;
  if (!scores) return tkv_fail(t, TKV_EINVAL, "NULL argument");
  const float* src = t->s;
  if (!t->parts.empty() && t->parts[0]->defer) {
    // per-layer budgets with deferred Eq. 1: every part's pending steps into
    // one copy of the shared s (the first part's), which the read returns
    tkv* p0 = t->parts[0];
    if (p0->pend) {
      HIP_TRY(t, hipMemcpyAsync(p0->s_view, t->s, (size_t)t->B * t->nmax * 4, hipMemcpyDeviceToDevice,
                                (hipStream_t)stream));
      for (size_t i = 0; i < t->parts.size(); ++i)
        if (t->parts[i]->pend)
          if (int rc = part_rc(t, i, flush_deferred(t->parts[i], (hipStream_t)stream, false, p0->s_view)))
            return rc;
      src = p0->s_view;
    }
  } else if (!t->parts.empty()) {
    // per-layer budgets with stored logits: each part's pending score launch
    // (one step's) goes into s, as the next launch would apply it
    if (int rc = tkv_flush_score(t, (hipStream_t)stream)) return rc;
  } else if (t->defer && t->pend) {
    // the pending steps into a copy of s: they stay pending, so a read never
    // changes which steps a later launch sums together
    if (int rc = flush_deferred(t, (hipStream_t)stream, false)) return rc;
    src = t->s_view;
  } else if (int rc = tkv_flush_score(t, (hipStream_t)stream)) {
    return rc;
  }
  HIP_TRY(t, hipMemcpyAsync(scores, src, (size_t)t->B * t->nmax * 4, hipMemcpyDeviceToHost, (hipStream_t)stream));
  HIP_TRY(t, hipStreamSynchronize((hipStream_t)stream));
  return TKV_OK;
}
extern "C" int tkv_read_scores(tkv_t* t, float* scores, tkv_stream_t stream) {
  return guarded(t, [&] { return read_scores_impl(t, scores, stream); });
}

static int write_scores_impl(tkv_t* t, const float* scores, tkv_stream_t stream) {
  if (int rc = usable(t)) return rc;
  if (!scores) return tkv_fail(t, TKV_EINVAL, "NULL argument");
  if (t->state == TkvState::InStep) return tkv_fail(t, TKV_ESTATE, "step in progress");
  // the written scores replace s with every pending update: those are dropped
  for (tkv* p : t->parts) {
    if (p->state == TkvState::InStep) return tkv_fail(t, TKV_ESTATE, "step in progress");
    p->pend = 0;
    p->score_pending = false;
  }
  if (t->defer) {
    t->pend = 0;
  } else {
    t->score_pending = false;
  }
  HIP_TRY(t, hipMemcpyAsync(t->s, scores, (size_t)t->B * t->nmax * 4, hipMemcpyHostToDevice, (hipStream_t)stream));
  HIP_TRY(t, hipStreamSynchronize((hipStream_t)stream));
  return TKV_OK;
}
extern "C" int tkv_write_scores(tkv_t* t, const float* scores, tkv_stream_t stream) {
  return guarded(t, [&] { return write_scores_impl(t, scores, stream); });
}

static int read_tiers_impl(tkv_t* t, uint8_t* tiers, tkv_stream_t stream) {
  if (int rc = usable(t)) return rc;
  if (!tiers) return tkv_fail(t, TKV_EINVAL, "NULL argument");
  if (!t->parts.empty()) return part_rc(t, 0, read_tiers_impl(t->parts[0], tiers, stream));  // layer 0's
  HIP_TRY(t, hipMemcpyAsync(tiers, t->tier, (size_t)t->B * t->nmax, hipMemcpyDeviceToHost, (hipStream_t)stream));
  HIP_TRY(t, hipStreamSynchronize((hipStream_t)stream));
  return TKV_OK;
}
extern "C" int tkv_read_tiers(tkv_t* t, uint8_t* tiers, tkv_stream_t stream) {
  return guarded(t, [&] { return read_tiers_impl(t, tiers, stream); });
}

static int read_layer_tiers_impl(tkv_t* t, int32_t layer, uint8_t* tiers, tkv_stream_t stream) {
  if (int rc = usable(t)) return rc;
  if (layer < 0 || layer >= t->L) return tkv_fail(t, TKV_EINVAL, "layer %d out of range", layer);
  if (t->parts.empty()) return read_tiers_impl(t, tiers, stream);
  const size_t i = part_of(t, layer);
  return part_rc(t, i, read_tiers_impl(t->parts[i], tiers, stream));
}
extern "C" int tkv_read_layer_tiers(tkv_t* t, int32_t layer, uint8_t* tiers, tkv_stream_t stream) {
  return guarded(t, [&] { return read_layer_tiers_impl(t, layer, tiers, stream); });
}

static int read_deltas_impl(tkv_t* t, tkv_delta* promote, tkv_delta* demote, int32_t* counts) {
  if (int rc = usable(t)) return rc;
  if (!promote || !demote || !counts) return tkv_fail(t, TKV_EINVAL, "NULL argument");
  if (!t->parts.empty()) return part_rc(t, 0, read_deltas_impl(t->parts[0], promote, demote, counts));
  const size_t nd = (size_t)t->B * t->nmax;
  std::memcpy(promote, t->h_promote, nd * sizeof(tkv_delta));
  std::memcpy(demote, t->h_demote, nd * sizeof(tkv_delta));
  std::memcpy(counts, t->h_counts, (size_t)t->B * 2 * sizeof(int32_t));
  return TKV_OK;
}
extern "C" int tkv_read_deltas(tkv_t* t, tkv_delta* promote, tkv_delta* demote, int32_t* counts) {
  return guarded(t, [&] { return read_deltas_impl(t, promote, demote, counts); });
}

static int read_kv_impl(tkv_t* t, int32_t layer, int32_t seq, int32_t pos, void* k, void* v,
                           tkv_stream_t stream) {
  if (int rc = usable(t)) return rc;
  if (!k || !v) return tkv_fail(t, TKV_EINVAL, "NULL argument");
  if (layer < 0 || layer >= t->L || seq < 0 || seq >= t->B || pos < 0 || pos >= t->n)
    return tkv_fail(t, TKV_EINVAL, "layer/seq/pos out of range");
  if (!t->parts.empty()) {
    const size_t i = part_of(t, layer);
    return part_rc(t, i, read_kv_impl(t->parts[i], layer - t->part_l0[i], seq, pos, k, v, stream));
  }
  if (int rc = arena_settled(t)) return rc;
  const size_t at = (size_t)seq * t->nmax + pos;
  const uint8_t tier = t->h_tier[at];
  const uint32_t code = t->h_loc[at];
  if (tier > TKV_T2) return tkv_fail(t, TKV_ESTATE, "position %d is not live", pos);
  hipStream_t st = (hipStream_t)stream;
  const size_t hb = (size_t)t->D * t->esz;
  const RowSpace rs = t->rowspace();
  if (tier == TKV_T0 || t->resident) {
    for (int which = 0; which < 2; ++which) {
      const char* base;
      size_t hstride;
      if (code < (uint32_t)t->cap0) {
        base = (const char*)(which ? t->pool_v : t->pool_k) +
               ((size_t)layer * rs.pool_lstride + (size_t)seq * rs.pool_bstride) * t->esz + (size_t)code * hb;
        hstride = (size_t)rs.pool_hstride * t->esz;
      } else {
        base = (const char*)(which ? t->stage_v : t->stage_k) +
               ((size_t)(layer % t->S) * rs.stage_lstride + (size_t)seq * rs.stage_bstride) * t->esz +
               (size_t)(code - t->cap0) * hb;
        hstride = (size_t)rs.stage_hstride * t->esz;
      }
      HIP_TRY(t, hipMemcpy2DAsync(which ? v : k, hb, base, hstride, hb, t->Hkv, hipMemcpyDeviceToHost, st));
    }
    HIP_TRY(t, hipStreamSynchronize(st));
    return TKV_OK;
  }
  if (tier == TKV_T2) return tkv_fail(t, TKV_ESTATE, "T2 rows of stream staging exist only as codes");
  HIP_TRY(t, hipStreamSynchronize(st));
  const uint32_t idx = code - t->cap0;
  for (int which = 0; which < 2; ++which)
    for (int h = 0; h < t->Hkv; ++h)
      std::memcpy((char*)(which ? v : k) + h * hb,
                  (const char*)(which ? t->arena1_v : t->arena1_k) +
                      ((((size_t)layer * t->B + seq) * t->Hkv + h) * t->cap1 + idx) * hb,
                  hb);
  return TKV_OK;
}
extern "C" int tkv_read_kv(tkv_t* t, int32_t layer, int32_t seq, int32_t pos, void* k, void* v,
                           tkv_stream_t stream) {
  return guarded(t, [&] { return read_kv_impl(t, layer, seq, pos, k, v, stream); });
}

static int read_t2_impl(tkv_t* t, int32_t layer, int32_t seq, int32_t pos, int8_t* k_codes, int8_t* v_codes,
                           float* scales) {
  if (int rc = usable(t)) return rc;
  if (!k_codes || !v_codes || !scales) return tkv_fail(t, TKV_EINVAL, "NULL argument");
  if (layer < 0 || layer >= t->L || seq < 0 || seq >= t->B || pos < 0 || pos >= t->n)
    return tkv_fail(t, TKV_EINVAL, "layer/seq/pos out of range");
  if (!t->parts.empty()) {
    const size_t i = part_of(t, layer);
    return part_rc(t, i, read_t2_impl(t->parts[i], layer - t->part_l0[i], seq, pos, k_codes, v_codes, scales));
  }
  if (int rc = arena_settled(t)) return rc;
  const size_t at = (size_t)seq * t->nmax + pos;
  if (t->h_tier[at] != TKV_T2) return tkv_fail(t, TKV_ESTATE, "position %d is not in T2", pos);
  const uint32_t idx = t->positional ? t->h_aidx[at] : t->h_loc[at] - (uint32_t)(t->cap0 + t->cap1);
  for (int which = 0; which < 2; ++which) {
    for (int h = 0; h < t->Hkv; ++h)
      std::memcpy((which ? v_codes : k_codes) + (size_t)h * t->D,
                  (which ? t->arena2_v : t->arena2_k) + ((((size_t)layer * t->B + seq) * t->Hkv + h) * t->cap2 + idx) * t->D,
                  t->D);
    for (int k = 0; k < t->sh; ++k)
      scales[which * t->sh + k] =
          (which ? t->ascale_v : t->ascale_k)[(((size_t)layer * t->B + seq) * t->cap2 + idx) * t->sh + k];
  }
  return TKV_OK;
}
extern "C" int tkv_read_t2(tkv_t* t, int32_t layer, int32_t seq, int32_t pos, int8_t* k_codes, int8_t* v_codes,
                           float* scales) {
  return guarded(t, [&] { return read_t2_impl(t, layer, seq, pos, k_codes, v_codes, scales); });
}
