/*
 * ORACLE (test infrastructure, not product code).  Plain fp64 softmax
 * attention of one decode step over the non-evicted cache rows.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this library.  It shares no code with the GPU library.
 *
 * What it follows:
 *  - "Not All Thoughts Need HBM" (gist.science summary), method section 3,
 *    zero-approximation-error offload: rows of T0 (HBM), T1 (host DDR) and
 *    T2 (host, 8-bit) all take part in every attention step with the values
 *    they hold; only T3 (evicted) rows are left out.  The tier of a live row
 *    never enters this computation, which is Proposition 1 by construction.
 *  - The pages never write the attention formula out; the plain reading is
 *    scaled dot-product softmax attention, softmax(q K^T / sqrt(d)) V, with
 *    query head h reading kv head floor(h / (Hq / Hkv)).
 *
 * Layouts (row-major, C order):
 *   K, V   float  [L][B][nmax][Hkv][d]   exact cache values (bf16/fp32 inputs
 *                                       and 8-bit dequantised values are all
 *                                       exactly representable in float)
 *   live   uint8  [B][nmax]             1 = position takes part (not evicted)
 *   q      double [L][B][Hq][d]
 *   out    double [L][B][Hq][d]
 *   alpha  double [L][B][Hq][nmax]      attention weights, 0 off the live set
 * Only positions [0, n) are looked at.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

void oracle_attend(int L, int B, int Hq, int Hkv, int d, int64_t nmax, int64_t n, const float* K,
                   const float* V, const uint8_t* live, const double* q, double* out, double* alpha) {
  const int group = Hq / Hkv;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  const int64_t units = (int64_t)L * B * Hq;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    const int h = (int)(u % Hq);
    const int b = (int)((u / Hq) % B);
    const int l = (int)(u / ((int64_t)Hq * B));
    const int g = h / group; /* kv head read by query head h */
    const double* qv = q + u * d;
    const uint8_t* lv = live + (int64_t)b * nmax;
    const int64_t row0 = ((int64_t)l * B + b) * nmax; /* first row of (l, b) */
    double* a = alpha + u * nmax;
    double* o = out + u * d;

    /* logits z_i = q . k_i / sqrt(d) and their maximum */
    double m = -INFINITY;
    for (int64_t i = 0; i < nmax; ++i) a[i] = 0.0;
    for (int64_t i = 0; i < n; ++i) {
      if (!lv[i]) continue;
      const float* k = K + ((row0 + i) * Hkv + g) * d;
      double z = 0.0;
      for (int j = 0; j < d; ++j) z += qv[j] * (double)k[j];
      z *= inv_sqrt_d;
      a[i] = z;
      if (z > m) m = z;
    }
    /* softmax over the live set */
    double sum = 0.0;
    for (int64_t i = 0; i < n; ++i) {
      if (!lv[i]) continue;
      a[i] = exp(a[i] - m);
      sum += a[i];
    }
    for (int64_t i = 0; i < n; ++i)
      if (lv[i]) a[i] /= sum;
    /* weighted sum of the value rows */
    for (int j = 0; j < d; ++j) o[j] = 0.0;
    for (int64_t i = 0; i < n; ++i) {
      if (!lv[i]) continue;
      const float* v = V + ((row0 + i) * Hkv + g) * d;
      for (int j = 0; j < d; ++j) o[j] += a[i] * (double)v[j];
    }
  }
}
