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
// fp32 caches take these per-thread passes.  bf16 caches take the
// matrix-core passes below: the row statistics in one online pass (one
// exponential per weight: 2^-|z - m| serves both the rescale of a running
// sum and a new term), then the column sums.  Every pass computes each
// z = q_t . k_j the same way (the same fma chain, or the same MFMA tile), so
// every weight is at most 1 and the weights of a query sum to 1 up to
// rounding.
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
// 2^x by the hardware instruction alone: results below 2^-126 flush to zero
// instead of taking the denormal-scaling sequence (five more VALU operations
// per weight); such weights are below fp32's resolution of any sum they join.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Operand tiles of 32 rows (of one head, row stride `stride` elements) are
// staged in LDS once per block and shared by its 4 waves: rows padded by 16
// bytes so that the 16-byte reads of 16 rows at one offset hit distinct banks.
template <int D>
struct Tile {
  static constexpr int RB = 2 * D + 16;  // padded row bytes
  static constexpr int PR = D / 8;       // 16-byte pieces per row
  static constexpr int RPP = 256 / PR;   // rows per block-wide pass
  static constexpr int NP = 32 / RPP;    // passes per 32-row tile
};

template <int D>
__device__ __forceinline__ void tile_fetch(const uint16_t* base, int64_t stride, int row0, int n, uint4* reg) {
#pragma unroll
  for (int p = 0; p < Tile<D>::NP; ++p) {
    const int row = p * Tile<D>::RPP + (int)threadIdx.x / Tile<D>::PR, piece = (int)threadIdx.x % Tile<D>::PR;
    const int gr = row0 + row;
    reg[p] = gr < n ? *reinterpret_cast<const uint4*>(base + (int64_t)gr * stride + 8 * piece) : make_uint4(0, 0, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void tile_store(char* lds, const uint4* reg) {
#pragma unroll
  for (int p = 0; p < Tile<D>::NP; ++p) {
    const int row = p * Tile<D>::RPP + (int)threadIdx.x / Tile<D>::PR, piece = (int)threadIdx.x % Tile<D>::PR;
    *reinterpret_cast<uint4*>(lds + row * Tile<D>::RB + 16 * piece) = reg[p];
  }
}

// MFMA operand (8 elements 32kc + 8s..) of row `row` of an LDS tile
template <int D>
__device__ __forceinline__ bf16x8 tile_op(const char* lds, int row, int kc, int sgrp) {
  const uint4 u = *reinterpret_cast<const uint4*>(lds + row * Tile<D>::RB + 2 * (32 * kc + 8 * sgrp));
  const u32x4 v = {u.x, u.y, u.z, u.w};
  return __builtin_bit_cast(bf16x8, v);
}

// grid (ceil(n / 128), q_heads, layers * batch), block 256: the block owns
// query rows [128x, 128x + 128), wave w the 32 rows 32w.. (two 16-row tiles,
// operands in registers); key tiles of 32 rows come through LDS.  Each lane
// keeps a running (max, sum of 2^(z - max)) per row over its own keys (key
// index = lane mod 16); the 16 partial pairs of a row merge at the end.
template <int D>
__global__ __launch_bounds__(256) void k_prefill_rowstats_mk(const PrefillScoreArgs a) {
  constexpr int KC = D / 32;
  __shared__ __attribute__((aligned(16))) char kt_s[2][32 * Tile<D>::RB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, sgrp = lane >> 4;
  const int h = blockIdx.y, lb = blockIdx.z;
  const int kvh = h / (a.q_heads / a.kv_heads);
  const int T0 = blockIdx.x * 128, tw = T0 + 32 * wave;
  const uint16_t* Q = (const uint16_t*)a.q + ((int64_t)lb * a.n * a.q_heads + h) * D;
  const uint16_t* K = (const uint16_t*)a.k + ((int64_t)lb * a.n * a.kv_heads + kvh) * D;
  bf16x8 qa[2][KC];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int t = tw + 16 * qt + r;
      qa[qt][kc] = t < a.n ? ld8(Q + (int64_t)t * a.q_heads * D + 32 * kc + 8 * sgrp) : bf16x8{};
    }
  const int64_t so = ((int64_t)lb * a.q_heads + h) * a.n;
  float m[2][4], l[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[qt][i] = -INFINITY;
      l[qt][i] = 0.f;
    }
  const int jend = min(a.n, T0 + 128);  // keys the block's rows can see
  const int iters = (jend + 31) / 32;
  uint4 reg[Tile<D>::NP];
  tile_fetch<D>(K, (int64_t)a.kv_heads * D, 0, a.n, reg);
  tile_store<D>(kt_s[0], reg);
  __syncthreads();
  for (int it = 0; it < iters; ++it) {
    const bool more = it + 1 < iters;
    if (more) tile_fetch<D>(K, (int64_t)a.kv_heads * D, 32 * (it + 1), a.n, reg);
    const char* ks = kt_s[it & 1];
    // Branch-free tile body; MASKED drops (by selection) keys after a row's
    // query and rows past the prompt.
    auto body = [&](auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        bf16x8 kb[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) kb[kc] = tile_op<D>(ks, 16 * kt + r, kc, sgrp);
        const int j = 32 * it + 16 * kt + r;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const f32x4 acc = tile_z<D>(qa[qt], kb);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float z = acc[i] * a.qscale;
            const float e = exp2_hw(-fabsf(z - m[qt][i]));  // 0 for the first key (m = -inf)
            const bool up = z > m[qt][i];
            const float nl = up ? fmaf(l[qt][i], e, 1.f) : l[qt][i] + e;
            const float nm = up ? z : m[qt][i];
            if constexpr (MASKED) {
              const int t = tw + 16 * qt + 4 * sgrp + i;
              const bool ok = t < a.n && j <= t;
              l[qt][i] = ok ? nl : l[qt][i];
              m[qt][i] = ok ? nm : m[qt][i];
            } else {
              l[qt][i] = nl;
              m[qt][i] = nm;
            }
          }
        }
      }
    };
    // keys 32it..32it+31 all precede this wave's rows, which all exist: no masks
    if (32 * it + 31 <= tw && tw + 31 < a.n)
      body(std::false_type{});
    else
      body(std::true_type{});
    if (more) tile_store<D>(kt_s[(it + 1) & 1], reg);
    __syncthreads();
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tw + 16 * qt + 4 * sgrp + i;
      const float M = row16_max(m[qt][i]);
      // a lane that saw no key of this row holds (-inf, 0)
      const float L = row16_sum(m[qt][i] == -INFINITY ? 0.f : l[qt][i] * exp2_hw(m[qt][i] - M));
      if (r == 0 && t < a.n) {
        a.row_max[so + t] = M;
        a.row_inv[so + t] = 1.f / L;
      }
    }
}

// grid (ceil(n / 128), q_heads, layers * batch), block 256: the block owns
// keys [128x, 128x + 128), wave w the 32 keys 32w.. (operands in registers);
// query tiles of 32 rows and their row statistics come through LDS.
template <int D>
__global__ __launch_bounds__(256) void k_prefill_colsum_mk(const PrefillScoreArgs a) {
  constexpr int KC = D / 32;
  __shared__ __attribute__((aligned(16))) char qt_s[2][32 * Tile<D>::RB];
  __shared__ float ms[2][32], is[2][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, sgrp = lane >> 4;
  const int h = blockIdx.y, lb = blockIdx.z;
  const int kvh = h / (a.q_heads / a.kv_heads);
  const int J0 = blockIdx.x * 128, jw = J0 + 32 * wave;
  const uint16_t* Q = (const uint16_t*)a.q + ((int64_t)lb * a.n * a.q_heads + h) * D;
  const uint16_t* K = (const uint16_t*)a.k + ((int64_t)lb * a.n * a.kv_heads + kvh) * D;
  const int64_t so = ((int64_t)lb * a.q_heads + h) * a.n;
  bf16x8 kb[2][KC];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int j = jw + 16 * kt + r;
      kb[kt][kc] = j < a.n ? ld8(K + (int64_t)j * a.kv_heads * D + 32 * kc + 8 * sgrp) : bf16x8{};
    }
  float c[2] = {0.f, 0.f};
  const int iters = (a.n - J0 + 31) / 32;  // query tiles from the block's first key on
  uint4 reg[Tile<D>::NP];
  float sreg = 0.f;
  auto stat_fetch = [&](int t0) {
    const int t = t0 + (int)(threadIdx.x & 31);
    if (threadIdx.x < 64) sreg = t < a.n ? (threadIdx.x < 32 ? a.row_max[so + t] : a.row_inv[so + t]) : 0.f;
  };
  auto stat_store = [&](int buf) {
    if (threadIdx.x < 32) ms[buf][threadIdx.x] = sreg;
    else if (threadIdx.x < 64) is[buf][threadIdx.x - 32] = sreg;
  };
  tile_fetch<D>(Q, (int64_t)a.q_heads * D, J0, a.n, reg);
  stat_fetch(J0);
  tile_store<D>(qt_s[0], reg);
  stat_store(0);
  __syncthreads();
  for (int it = 0; it < iters; ++it) {
    const bool more = it + 1 < iters;
    const int t0 = J0 + 32 * it;
    if (more) {
      tile_fetch<D>(Q, (int64_t)a.q_heads * D, t0 + 32, a.n, reg);
      stat_fetch(t0 + 32);
    }
    const int p = it & 1;
    // Branch-free tile body; MASKED drops (by selection) queries before a key
    // and rows past the prompt.
    auto body = [&](auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        bf16x8 qa[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) qa[kc] = tile_op<D>(qt_s[p], 16 * qt + r, kc, sgrp);
        float mt[4], iv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          mt[i] = ms[p][16 * qt + 4 * sgrp + i];
          iv[i] = is[p][16 * qt + 4 * sgrp + i];
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const f32x4 acc = tile_z<D>(qa, kb[kt]);
          const int j = jw + 16 * kt + r;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float w = exp2_hw(acc[i] * a.qscale - mt[i]) * iv[i];
            if constexpr (MASKED) {
              const int t = t0 + 16 * qt + 4 * sgrp + i;
              c[kt] += (t < a.n && t >= j) ? w : 0.f;
            } else {
              c[kt] += w;
            }
          }
        }
      }
    };
    // queries t0..t0+31 all follow this wave's keys and all exist: no masks
    if (t0 >= jw + 31 && t0 + 31 < a.n)
      body(std::false_type{});
    else
      body(std::true_type{});
    if (more) {
      tile_store<D>(qt_s[(it + 1) & 1], reg);
      stat_store((it + 1) & 1);
    }
    __syncthreads();
  }
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    float x = c[kt];
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    const int j = jw + 16 * kt + r;
    if (sgrp == 0 && j < a.n) a.colsum[so + j] = x;
  }
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
    const dim3 grid((a.n + 127) / 128, a.q_heads, a.layers * a.batch);
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
