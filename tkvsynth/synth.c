/*
 * Seeded, counter-based synthetic inputs for the tiered-KV decode workloads.
 *
 * This file holds no arithmetic of the attention / scoring / tiering method:
 * it only draws the q, K, V tensors that both the CPU oracle and the GPU
 * library consume.  Every element is a pure function of
 * (seed, tensor id, flat element index), so any slice can be produced on its
 * own and in parallel.
 *
 * Random words: the splitmix64 output function (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014) applied to a
 * per-tensor key plus a counter.  Two 53-bit uniforms per element feed the
 * Box-Muller transform (fp64) for one N(0,1) sample.  Values are then shifted
 * by the planted heavy-hitter direction and rounded once to bf16 (round to
 * nearest even) or to fp32.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math: log/cos/sqrt must be
 * the C library's).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of tensor `tid` under `seed`. */
static inline uint64_t stream_key(uint64_t seed, uint64_t tid) {
  return mix64(mix64(seed) ^ (tid * 0xD1B54A32D192ED03ULL));
}

static inline double normal_at(uint64_t key, uint64_t n) {
  uint64_t x = mix64(key + 2 * n);
  uint64_t y = mix64(key + 2 * n + 1);
  double u1 = ((double)(x >> 11) + 0.5) * 0x1.0p-53; /* (0, 1) */
  double u2 = (double)(y >> 11) * 0x1.0p-53;         /* [0, 1) */
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

/* fp64 -> bf16 bits, one rounding to nearest even (valid for 0 and for
 * magnitudes in bf16's normal range; Gaussian draws never leave it). */
static inline uint16_t bf16_bits(double x) {
  uint64_t b;
  memcpy(&b, &x, 8);
  uint64_t lsb = (b >> 45) & 1u;
  b += 0x00000FFFFFFFFFFFULL + lsb; /* 2^44 - 1 + lsb */
  b &= ~0x00001FFFFFFFFFFFULL;      /* keep 1 + 7 mantissa bits */
  double r;
  memcpy(&r, &b, 8);
  float f = (float)r; /* exact */
  uint32_t fb;
  memcpy(&fb, &f, 4);
  return (uint16_t)(fb >> 16);
}

static inline void store(void* out, int64_t idx, double x, int out_bf16) {
  if (out_bf16)
    ((uint16_t*)out)[idx] = bf16_bits(x);
  else
    ((float*)out)[idx] = (float)x;
}

/* Raw 64-bit words of tensor `tid`: out[k] = word(n0 + k). */
void tkvsynth_words(uint64_t seed, uint64_t tid, uint64_t n0, int64_t count, uint64_t* out) {
  uint64_t key = stream_key(seed, tid);
  for (int64_t k = 0; k < count; ++k) out[k] = mix64(key + n0 + (uint64_t)k);
}

/* Raw N(0,1) draws of tensor `tid`: out[k] = normal(n0 + k). */
void tkvsynth_normals(uint64_t seed, uint64_t tid, uint64_t n0, int64_t count, double* out) {
  uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < count; ++k) out[k] = normal_at(key, n0 + (uint64_t)k);
}

/*
 * K (which=0, tensor id 1) or V (which=1, tensor id 2) rows of cache
 * positions [pos0, pos0 + np), written as out[l][b][p - pos0][h][j].
 * Element flat index: (((b*L + l)*n_final + p)*H + h)*d + j.
 * K rows of heavy positions (heavy[b*n_final + p] != 0) get amp*u[j] added
 * before rounding; V rows never do.
 */
void tkvsynth_kv(uint64_t seed, int which, int L, int B, int H, int d, int64_t n_final, int64_t pos0,
                 int64_t np, const uint8_t* heavy, const double* u, double amp, int out_bf16, void* out) {
  uint64_t key = stream_key(seed, which == 0 ? 1u : 2u);
  int64_t rows = (int64_t)L * B * np;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    int64_t p = pos0 + r % np;
    int64_t lb = r / np;
    int64_t b = lb % B;
    int64_t l = lb / B;
    int hv = (which == 0 && heavy != NULL && heavy[b * n_final + p]) ? 1 : 0;
    uint64_t base = (uint64_t)((((b * L + l) * n_final + p) * H) * d);
    int64_t obase = r * H * d;
    for (int64_t e = 0; e < (int64_t)H * d; ++e) {
      double x = normal_at(key, base + (uint64_t)e);
      if (hv) x += amp * u[e % d];
      store(out, obase + e, x, out_bf16);
    }
  }
}

/*
 * q (tensor id 3) of decode steps [t0, t0 + nt) (0-based), written as
 * out[t - t0][l][b][h][j]; every row gets amp*u[j] added before rounding.
 * Element flat index: (((t*L + l)*B + b)*Hq + h)*d + j.
 */
void tkvsynth_q(uint64_t seed, int L, int B, int Hq, int d, int64_t t0, int64_t nt, const double* u,
                double amp, int out_bf16, void* out) {
  uint64_t key = stream_key(seed, 3u);
  int64_t rows = nt * L * B * Hq;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    uint64_t n = (uint64_t)((t0 * L * B * Hq + r) * d);
    for (int j = 0; j < d; ++j) {
      double x = normal_at(key, n + (uint64_t)j) + amp * u[j];
      store(out, r * d + j, x, out_bf16);
    }
  }
}
