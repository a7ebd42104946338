/* Drives the oracle's C attention on random small inputs under
 * AddressSanitizer / UndefinedBehaviorSanitizer; checks that every
 * (layer, sequence, head) gets weights summing to 1 over its live rows and
 * zero elsewhere, and finite outputs. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_attend(int L, int B, int Hq, int Hkv, int d, int64_t nmax, int64_t n, const float* K, const float* V,
                   const uint8_t* live, const double* q, double* out, double* alpha);

int main(void) {
  srand(7);
  int fails = 0;
  for (int rep = 0; rep < 40; ++rep) {
    const int L = 1 + rand() % 3, B = 1 + rand() % 3, Hkv = 1 + rand() % 3, g = 1 + rand() % 4, d = 8 * (1 + rand() % 3);
    const int Hq = Hkv * g;
    const int64_t nmax = 1 + rand() % 50, n = 1 + rand() % nmax;
    const size_t kv = (size_t)L * B * nmax * Hkv * d;
    float* K = malloc(kv * sizeof(float));
    float* V = malloc(kv * sizeof(float));
    uint8_t* live = malloc((size_t)B * nmax);
    double* q = malloc((size_t)L * B * Hq * d * sizeof(double));
    double* out = malloc((size_t)L * B * Hq * d * sizeof(double));
    double* alpha = malloc((size_t)L * B * Hq * nmax * sizeof(double));
    for (size_t i = 0; i < kv; ++i) {
      K[i] = (float)rand() / RAND_MAX - 0.5f;
      V[i] = (float)rand() / RAND_MAX - 0.5f;
    }
    for (int64_t i = 0; i < (int64_t)B * nmax; ++i) live[i] = (rand() % 4) != 0;
    for (int b = 0; b < B; ++b) live[(int64_t)b * nmax] = 1; /* at least one live row */
    for (size_t i = 0; i < (size_t)L * B * Hq * d; ++i) q[i] = (double)rand() / RAND_MAX - 0.5;
    oracle_attend(L, B, Hq, Hkv, d, nmax, n, K, V, live, q, out, alpha);
    for (int64_t u = 0; u < (int64_t)L * B * Hq; ++u) {
      const int b = (int)((u / Hq) % B);
      double s = 0.0;
      for (int64_t i = 0; i < nmax; ++i) {
        const double a = alpha[u * nmax + i];
        if (i < n && live[(int64_t)b * nmax + i]) s += a;
        else if (a != 0.0) ++fails;
      }
      if (fabs(s - 1.0) > 1e-12) ++fails;
      for (int j = 0; j < d; ++j)
        if (!isfinite(out[u * d + j])) ++fails;
    }
    free(K); free(V); free(live); free(q); free(out); free(alpha);
  }
  printf("attend checks: %d failures\n", fails);
  return fails ? 1 : 0;
}
