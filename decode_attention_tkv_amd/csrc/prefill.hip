// Scored prefill: the prompt's causal attention weights added to the scores
// ("Not All Thoughts Need HBM", gist.science technical summary, Method §2:
// Eq. 1 accumulates every token's attention weight averaged over layers and
// heads; here position t of the prompt attends to positions 0..t and its
// weights are added exactly as a decode step's are).
//
//   k_prefill_rowstats  one thread per (query t, query head, layer x
//                       sequence): max and sum of 2^z over keys 0..t (z in
//                       log2 units, online over the keys in order);
//   k_prefill_colsum    one thread per (key j, query head, layer x
//                       sequence): sum over queries t >= j of 2^(z - m_t) / l_t;
//   k_prefill_sum       one thread per (position, sequence): the scores,
//                       layers then heads in a fixed order, times 1/(L*H).
// fp32 caches take these per-thread passes; bf16 caches take the matrix-core
// passes below.  Both passes compute every z = q_t . k_j the same way (the
// same fma chain, or the same MFMA tile), so every weight is at most 1 and
// the weights of a query sum to 1 up to rounding.
#include <type_traits>

#include "tkv_internal.hpp"

namespace tkvd {
namespace {

// A row of D cache-type values as floats, 16 bytes per load.
template <typename T, int D>
__device__ __forceinline__ void ld_row(const T* p, float* f);
template <int D>
__device__ __forceinline__ void ld_row_bf16(const uint16_t* p, float* f) {
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    const uint4 u = reinterpret_cast<const uint4*>(p)[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
      f[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
}
template <>
__device__ __forceinline__ void ld_row<uint16_t, 64>(const uint16_t* p, float* f) { ld_row_bf16<64>(p, f); }
template <>
__device__ __forceinline__ void ld_row<uint16_t, 128>(const uint16_t* p, float* f) { ld_row_bf16<128>(p, f); }
template <int D>
__device__ __forceinline__ void ld_row_f32(const float* p, float* f) {
#pragma unroll
  for (int i = 0; i < D / 4; ++i) {
    const float4 u = reinterpret_cast<const float4*>(p)[i];
    f[4 * i] = u.x;
    f[4 * i + 1] = u.y;
    f[4 * i + 2] = u.z;
    f[4 * i + 3] = u.w;
  }
}
template <>
__device__ __forceinline__ void ld_row<float, 64>(const float* p, float* f) { ld_row_f32<64>(p, f); }
template <>
__device__ __forceinline__ void ld_row<float, 128>(const float* p, float* f) { ld_row_f32<128>(p, f); }

// q . k as one sequential fma chain (the same order in both passes)
template <int D>
__device__ __forceinline__ float dot(const float* q, const float* k) {
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < D; ++e) acc = fmaf(q[e], k[e], acc);
  return acc;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_prefill_rowstats(const PrefillScoreArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y, lb = blockIdx.z;  // lb = layer * batch + sequence
  const int kvh = h / (a.q_heads / a.kv_heads);
  const int tmax = min(a.n, (int)(blockIdx.x + 1) * 256) - 1;  // last query of the block
  const T* K = (const T*)a.k + ((int64_t)lb * a.n * a.kv_heads + kvh) * D;
  float q[D];
  if (t < a.n) ld_row<T, D>((const T*)a.q + (((int64_t)lb * a.n + t) * a.q_heads + h) * D, q);
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j <= tmax; ++j) {  // the block walks keys together; each thread stops at its t
    if (t < a.n && j <= t) {
      float kj[D];
      ld_row<T, D>(K + (int64_t)j * a.kv_heads * D, kj);
      const float z = dot<D>(q, kj) * a.qscale;
      if (z > m) {
        l = l * exp2f(m - z) + 1.f;
        m = z;
      } else {
        l += exp2f(z - m);
      }
    }
  }
  if (t < a.n) {
    const int64_t o = ((int64_t)lb * a.q_heads + h) * a.n + t;
    a.row_max[o] = m;
    a.row_inv[o] = 1.f / l;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_prefill_colsum(const PrefillScoreArgs a) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y, lb = blockIdx.z;
  const int kvh = h / (a.q_heads / a.kv_heads);
  const int jmin = blockIdx.x * 256;  // first key of the block
  float k[D];
  if (j < a.n) ld_row<T, D>((const T*)a.k + (((int64_t)lb * a.n + j) * a.kv_heads + kvh) * D, k);
  const int64_t so = ((int64_t)lb * a.q_heads + h) * a.n;
  float c = 0.f;
  for (int t = jmin; t < a.n; ++t) {  // the block walks queries together from its first key
    if (j < a.n && t >= j) {
      float qt[D];
      ld_row<T, D>((const T*)a.q + (((int64_t)lb * a.n + t) * a.q_heads + h) * D, qt);
      const float z = dot<D>(qt, k) * a.qscale;  // the row pass's product, q first
      c += exp2f(z - a.row_max[so + t]) * a.row_inv[so + t];
    }
  }
  if (j < a.n) a.colsum[so + j] = c;
}

// ---- matrix-core passes (bf16 caches) ----------------------------------------
// Tiles of 16 query rows x 16 keys, z = q k^T by v_mfma_f32_16x16x32_bf16 over
// head_dim/32 slices.  Lane (r, s) = (lane % 16, lane / 16) feeds query / key
// row r with the 8 elements 8s.. of each 32-wide slice and receives z of
// query rows 4s..4s+3 at key r.  The row pass and the column pass form the
// same tiles from the same operands, so every z is bitwise the same in both.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const u32x4 v = {u.x, u.y, u.z, u.w};
  return __builtin_bit_cast(bf16x8, v);
}

template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// max / sum over the 16 lanes of a DPP row; every lane gets the result
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dppf<0xB1>(x));
  x = fmaxf(x, dppf<0x4E>(x));
  x = fmaxf(x, dppf<0x141>(x));
  return fmaxf(x, dppf<0x140>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dppf<0xB1>(x);
  x += dppf<0x4E>(x);
  x += dppf<0x141>(x);
  return x + dppf<0x140>(x);
}

template <int D>
__device__ __forceinline__ f32x4 tile_z(const bf16x8* qa, const bf16x8* kb) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < D / 32; ++kc) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kc], kb[kc], acc, 0, 0, 0);
  return acc;
}

// grid (ceil(n / 64), q_heads, layers * batch), block 256: wave w owns query
// rows 16w.. of the block's 64 and walks the keys 0..(its last row).
template <int D>
__global__ __launch_bounds__(256) void k_prefill_rowstats_mk(const PrefillScoreArgs a) {
  constexpr int KC = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, sgrp = lane >> 4;
  const int h = blockIdx.y, lb = blockIdx.z;
  const int kvh = h / (a.q_heads / a.kv_heads);
  const int t0 = blockIdx.x * 64 + 16 * wave;
  if (t0 >= a.n) return;  // no barriers in this kernel
  const uint16_t* Q = (const uint16_t*)a.q + ((int64_t)lb * a.n * a.q_heads + h) * D;
  const uint16_t* K = (const uint16_t*)a.k + ((int64_t)lb * a.n * a.kv_heads + kvh) * D;
  bf16x8 qa[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const int t = t0 + r;
    qa[kc] = t < a.n ? ld8(Q + (int64_t)t * a.q_heads * D + 32 * kc + 8 * sgrp) : bf16x8{};
  }
  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
  const int jend = min(a.n, t0 + 16);
  for (int j0 = 0; j0 < jend; j0 += 16) {
    const int j = j0 + r;
    bf16x8 kb[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      kb[kc] = j < a.n ? ld8(K + (int64_t)j * a.kv_heads * D + 32 * kc + 8 * sgrp) : bf16x8{};
    const f32x4 acc = tile_z<D>(qa, kb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * sgrp + i;
      if (t < a.n && j <= t) {
        const float z = acc[i] * a.qscale;
        const float mn = fmaxf(m[i], z);
        l[i] = l[i] * exp2f(m[i] - mn) + exp2f(z - mn);
        m[i] = mn;
      }
    }
  }
  const int64_t so = ((int64_t)lb * a.q_heads + h) * a.n;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float M = row16_max(m[i]);
    const float part = m[i] == -INFINITY ? 0.f : l[i] * exp2f(m[i] - M);
    const float L = row16_sum(part);
    const int t = t0 + 4 * sgrp + i;
    if (r == 0 && t < a.n) {
      a.row_max[so + t] = M;
      a.row_inv[so + t] = 1.f / L;
    }
  }
}

// grid (ceil(n / 64), q_heads, layers * batch), block 256: wave w owns keys
// 16w.. of the block's 64 and walks the queries from its first key to n.
template <int D>
__global__ __launch_bounds__(256) void k_prefill_colsum_mk(const PrefillScoreArgs a) {
  constexpr int KC = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, sgrp = lane >> 4;
  const int h = blockIdx.y, lb = blockIdx.z;
  const int kvh = h / (a.q_heads / a.kv_heads);
  const int j0 = blockIdx.x * 64 + 16 * wave;
  if (j0 >= a.n) return;  // no barriers in this kernel
  const uint16_t* Q = (const uint16_t*)a.q + ((int64_t)lb * a.n * a.q_heads + h) * D;
  const uint16_t* K = (const uint16_t*)a.k + ((int64_t)lb * a.n * a.kv_heads + kvh) * D;
  const int j = j0 + r;
  bf16x8 kb[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    kb[kc] = j < a.n ? ld8(K + (int64_t)j * a.kv_heads * D + 32 * kc + 8 * sgrp) : bf16x8{};
  const int64_t so = ((int64_t)lb * a.q_heads + h) * a.n;
  float c = 0.f;
  for (int t0 = j0; t0 < a.n; t0 += 16) {
    bf16x8 qa[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int t = t0 + r;
      qa[kc] = t < a.n ? ld8(Q + (int64_t)t * a.q_heads * D + 32 * kc + 8 * sgrp) : bf16x8{};
    }
    float mt[4], it[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * sgrp + i;
      mt[i] = t < a.n ? a.row_max[so + t] : 0.f;
      it[i] = t < a.n ? a.row_inv[so + t] : 0.f;
    }
    const f32x4 acc = tile_z<D>(qa, kb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * sgrp + i;
      if (t < a.n && t >= j) c += exp2f(acc[i] * a.qscale - mt[i]) * it[i];
    }
  }
  c += __shfl_xor(c, 16);
  c += __shfl_xor(c, 32);
  if (sgrp == 0 && j < a.n) a.colsum[so + j] = c;
}

__global__ __launch_bounds__(256) void k_prefill_sum(const PrefillScoreArgs a) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (j >= a.n) return;
  float acc = 0.f;
  for (int l = 0; l < a.layers; ++l) {
    const float* c = a.colsum + (((int64_t)l * a.batch + b) * a.q_heads) * a.n + j;
#pragma unroll 8
    for (int h = 0; h < a.q_heads; ++h) acc += c[(int64_t)h * a.n];
  }
  a.s[(int64_t)b * a.nmax + j] = acc * a.inv_lh;
}

template <typename T, int D>
hipError_t launch_t(const PrefillScoreArgs& a, hipStream_t s) {
  hipError_t e;
  if constexpr (std::is_same<T, uint16_t>::value) {
    const dim3 grid((a.n + 63) / 64, a.q_heads, a.layers * a.batch);
    k_prefill_rowstats_mk<D><<<grid, 256, 0, s>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_prefill_colsum_mk<D><<<grid, 256, 0, s>>>(a);
  } else {
    const dim3 grid((a.n + 255) / 256, a.q_heads, a.layers * a.batch);
    k_prefill_rowstats<T, D><<<grid, 256, 0, s>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_prefill_colsum<T, D><<<grid, 256, 0, s>>>(a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_prefill_sum<<<dim3((a.n + 255) / 256, a.batch), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_scores(const PrefillScoreArgs& a, int dtype, int head_dim, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  if (dtype == TKV_BF16) {
    if (head_dim == 128) return launch_t<uint16_t, 128>(a, s);
    if (head_dim == 64) return launch_t<uint16_t, 64>(a, s);
  } else {
    if (head_dim == 128) return launch_t<float, 128>(a, s);
    if (head_dim == 64) return launch_t<float, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tkvd
