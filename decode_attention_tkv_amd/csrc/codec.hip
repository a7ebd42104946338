// The 8-bit host tier's codec on the GPU ("Not All Thoughts Need HBM",
// gist.science technical summary, Method §1: T2 keeps low-importance rows on
// the CPU at low precision, 8-bit as the example; results §4 its cost).
//
// Format (the pages fix none): one fp32 scale per (layer, position, K|V)
// over the position's kv_heads * head_dim values.  int8: scale = amax / 127
// (1 for an all-zero row), code = clamp(rne(x / scale), -127, 127).  FP8
// (OCP E4M3): scale = amax / 448, code = the hardware's round-to-nearest-even
// E4M3 of clamp(x / scale, -448, 448).  Both: the division in fp32, value =
// fp32(code value * scale) rounded to the cache type (bf16
// round-to-nearest-even).  A row that entered the tier keeps these values
// for good.
#include "tkv_internal.hpp"

namespace tkvd {
namespace {

// E4M3 byte of y (|y| <= 448 already), and back (exact)
__device__ __forceinline__ uint32_t e4m3_of(float y) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false) & 0xFFu;
}
__device__ __forceinline__ float e4m3_val(uint32_t byte) { return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0); }

// code (int8 or E4M3 byte) as the value it stands for
__device__ __forceinline__ float code_val(int8_t c, int fp8) {
  return fp8 ? e4m3_val((uint32_t)(uint8_t)c) : (float)c;
}

__device__ __forceinline__ float load_val(const void* base, int64_t idx, int elem_bytes) {
  if (elem_bytes == 2) return __uint_as_float((uint32_t)((const uint16_t*)base)[idx] << 16);
  return ((const float*)base)[idx];
}

__device__ __forceinline__ void store_val(void* base, int64_t idx, float v, int elem_bytes) {
  if (elem_bytes == 2) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even (finite values)
    ((uint16_t*)base)[idx] = (uint16_t)(u >> 16);
  } else {
    ((float*)base)[idx] = v;
  }
}

__device__ __forceinline__ int64_t stage_elem(const RowSpace& rs, int l, int b, int h, uint32_t idx, int d) {
  return (int64_t)(l % rs.stage_slots) * rs.stage_lstride + (int64_t)b * rs.stage_bstride +
         (int64_t)h * rs.stage_hstride + (int64_t)idx * d;
}

// grid (n_ops, layers, 2), block 256: quantise F rows straight into the
// pinned T2 arena (over PCIe) at index op.dst of sequence op.b, and
// (optionally) write their dequantised values into the pool or the staging
// area.
__global__ __launch_bounds__(256) void k_quant_rows(const QuantArgs a, const QuantOp* ops) {
  __shared__ float red[4];
  __shared__ uint32_t hmax[kMaxQHeads];  // per-head amax bits (non-negative floats order as their bits)
  const QuantOp op = ops[blockIdx.x];
  const int l = blockIdx.y, which = blockIdx.z;
  const int d = a.head_dim, n = a.kv_heads * d;
  // the row's values: F row op.src, or (from_pool) pool slot op.src of sequence op.b
  const void* f = a.from_pool ? (which ? a.rows.pool_v : a.rows.pool_k) : (which ? a.f.v : a.f.k);
  auto at = [&](int h, int j) -> int64_t {
    if (a.from_pool)
      return (int64_t)l * a.rows.pool_lstride + (int64_t)op.b * a.rows.pool_bstride + (int64_t)h * a.rows.pool_hstride +
             (int64_t)op.src * d + j;
    return (((int64_t)l * a.kv_heads + h) * a.f.rows + op.src) * d + j;
  };
  float amax = 0.f;
  for (int e = threadIdx.x; e < n; e += 256) {
    const int h = e / d, j = e % d;
    amax = fmaxf(amax, fabsf(load_val(f, at(h, j), a.elem_bytes)));
  }
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float qmax = a.fp8 ? 448.f : 127.f;
  const float row_scale = amax > 0.f ? amax / qmax : 1.f;
  if (a.sh > 1) {  // one scale per kv head, from that head's own amax
    for (int h = threadIdx.x; h < a.kv_heads; h += 256) hmax[h] = 0u;
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += 256) {
      const int h = e / d, j = e % d;
      const float x = load_val(f, at(h, j), a.elem_bytes);
      atomicMax(&hmax[h], __float_as_uint(fabsf(x)));
    }
    __syncthreads();
  }
  auto head_scale = [&](int h) {
    if (a.sh == 1) return row_scale;
    const float m = __uint_as_float(hmax[h]);
    return m > 0.f ? m / qmax : 1.f;
  };
  auto code_at = [&](int h) -> int8_t* {  // first code of head h of this op's row
    return (which ? a.arena.a2_v : a.arena.a2_k) +
           ((((int64_t)l * a.arena.batch + op.b) * a.kv_heads + h) * a.arena.cap2 + op.dst) * d;
  };
  for (int e = threadIdx.x; e < n; e += 256) {
    const int h = e / d, j = e % d;
    // from_pool with op.stage == op.src rewrites this very element below:
    // every thread reads its elements before it writes them, and the amax
    // passes above finished at a barrier
    const float x = load_val(f, at(h, j), a.elem_bytes);
    const float scale = head_scale(h);
    float c;
    int8_t code;
    if (a.fp8) {
      const uint32_t byte = e4m3_of(fminf(fmaxf(x / scale, -448.f), 448.f));
      code = (int8_t)(uint8_t)byte;
      c = e4m3_val(byte);
    } else {
      c = fminf(fmaxf(rintf(x / scale), -127.f), 127.f);
      code = (int8_t)c;
    }
    code_at(h)[j] = code;
    if (op.stage != kNoLoc) {
      if (op.stage < (uint32_t)a.rows.cap0) {
        void* pl = which ? (void*)a.rows.pool_v : (void*)a.rows.pool_k;
        const int64_t at = (int64_t)l * a.rows.pool_lstride + (int64_t)op.b * a.rows.pool_bstride +
                           (int64_t)h * a.rows.pool_hstride + (int64_t)op.stage * d;
        store_val(pl, at + j, c * scale, a.elem_bytes);
      } else {
        void* st = which ? (void*)a.rows.stage_v : (void*)a.rows.stage_k;
        store_val(st, stage_elem(a.rows, l, op.b, h, op.stage - (uint32_t)a.rows.cap0, d) + j, c * scale,
                  a.elem_bytes);
      }
    }
  }
  float* sc = (which ? a.arena.s2_v : a.arena.s2_k) + (((int64_t)l * a.arena.batch + op.b) * a.arena.cap2 + op.dst) * a.sh;
  for (int k = threadIdx.x; k < a.sh; k += 256) sc[k] = head_scale(k);
}

// grid (n_ops, layers, 2), block 256: T2 arena rows (codes and scales, read
// over PCIe) -> cache-type values in F.
__global__ __launch_bounds__(256) void k_dequant_rows(const DequantArgs a, const DequantOp* ops) {
  const DequantOp op = ops[blockIdx.x];
  const int l = blockIdx.y, which = blockIdx.z;
  const int d = a.head_dim, n = a.kv_heads * d;
  const int8_t* codes = (which ? a.arena.a2_v : a.arena.a2_k) +
                        (((int64_t)l * a.arena.batch + op.b) * a.kv_heads * a.arena.cap2 + op.src) * d;
  const float* scales = (which ? a.arena.s2_v : a.arena.s2_k) +
                        (((int64_t)l * a.arena.batch + op.b) * a.arena.cap2 + op.src) * a.sh;
  void* f = which ? a.f.v : a.f.k;
  for (int e = threadIdx.x; e < n; e += 256) {
    const int h = e / d, j = e % d;
    const float scale = scales[a.sh > 1 ? h : 0];
    const float c = code_val(codes[(int64_t)h * a.arena.cap2 * d + j], a.fp8);
    store_val(f, (((int64_t)l * a.kv_heads + h) * a.f.rows + op.dst) * d + j, c * scale, a.elem_bytes);
  }
}

// T2 arena row op.src -> op.dst of sequence op.b (codes of every kv head,
// then the scales), within the pinned arena: work items (op, layer, K|V) in
// a grid-stride loop.  No op's source is another op's destination.
__global__ __launch_bounds__(256) void k_arena2_moves(const ArenaSpace a, const RowOp* ops, int n_ops, int layers,
                                                      int d) {
  const int64_t items = (int64_t)n_ops * layers * 2;
  const int pieces = d / 16;  // 16-byte pieces per head row of codes
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int which = (int)(it & 1);
    const int64_t r = it >> 1;
    const int l = (int)(r % layers);
    const RowOp op = ops[r / layers];
    int8_t* base = (which ? a.a2_v : a.a2_k) + ((int64_t)l * a.batch + op.b) * a.kv_heads * a.cap2 * d;
    for (int x = threadIdx.x; x < a.kv_heads * pieces; x += 256) {
      const int h = x / pieces, w = (x % pieces) * 16;
      *reinterpret_cast<uint4*>(base + ((int64_t)h * a.cap2 + op.dst) * d + w) =
          *reinterpret_cast<const uint4*>(base + ((int64_t)h * a.cap2 + op.src) * d + w);
    }
    float* sc = (which ? a.s2_v : a.s2_k) + ((int64_t)l * a.batch + op.b) * a.cap2 * a.sh;
    for (int k = threadIdx.x; k < a.sh; k += 256) sc[(int64_t)op.dst * a.sh + k] = sc[(int64_t)op.src * a.sh + k];
  }
}

}  // namespace

hipError_t launch_quant_rows(const QuantArgs& a, const QuantOp* ops, int n_ops, int layers, hipStream_t s) {
  if (n_ops <= 0) return hipSuccess;
  k_quant_rows<<<dim3(n_ops, layers, 2), 256, 0, s>>>(a, ops);
  return hipGetLastError();
}

hipError_t launch_dequant_rows(const DequantArgs& a, const DequantOp* ops, int n_ops, int layers, hipStream_t s) {
  if (n_ops <= 0) return hipSuccess;
  k_dequant_rows<<<dim3(n_ops, layers, 2), 256, 0, s>>>(a, ops);
  return hipGetLastError();
}

hipError_t launch_arena2_moves(const ArenaSpace& a, const RowOp* ops, int n_ops, int layers, int head_dim,
                               int max_blocks, hipStream_t s) {
  if (n_ops <= 0) return hipSuccess;
  if (head_dim % 16 || max_blocks < 1) return hipErrorInvalidValue;
  const int64_t items = (int64_t)n_ops * layers * 2;
  k_arena2_moves<<<(unsigned)(items < max_blocks ? items : max_blocks), 256, 0, s>>>(a, ops, n_ops, layers, head_dim);
  return hipGetLastError();
}

}  // namespace tkvd
