// Row movement kernels: placing prefilled rows, gathering rows into a packed
// buffer and scattering packed rows to their new homes.  A "row" is one
// position's K (or V) for all kv heads of one layer of one sequence:
// kv_heads * head_dim contiguous elements.
#include "tkv_internal.hpp"

namespace tkvd {
namespace {

__device__ __forceinline__ char* head_row(const RowSpace& rs, int which, int l, int b, int h, uint32_t code,
                                          int head_bytes, int elem_bytes) {
  if (code < (uint32_t)rs.cap0) {
    char* base = (char*)(which ? rs.pool_v : rs.pool_k);
    return base + ((int64_t)l * rs.pool_lstride + (int64_t)b * rs.pool_bstride + (int64_t)h * rs.pool_hstride) *
                      elem_bytes +
           (int64_t)code * head_bytes;
  }
  char* base = (char*)(which ? rs.stage_v : rs.stage_k);
  return base + ((int64_t)(l % rs.stage_slots) * rs.stage_lstride + (int64_t)b * rs.stage_bstride +
                 (int64_t)h * rs.stage_hstride) *
                    elem_bytes +
         (int64_t)(code - rs.cap0) * head_bytes;
}

// grid (n_tokens, layers*batch, 2): input row (l, b, p) -> its location code.
__global__ __launch_bounds__(256) void k_place_rows(const PlaceArgs a) {
  const int p = blockIdx.x;
  const int lb = blockIdx.y;
  const int b = lb % a.batch, l = lb / a.batch;
  const int which = blockIdx.z;
  const uint32_t code = a.codes[(int64_t)b * a.n_tokens + p];
  if (code == kNoLoc) return;
  const int row_bytes = a.kv_heads * a.head_bytes;
  const char* src = (const char*)(which ? a.v : a.k) + (((int64_t)lb * a.n_tokens) + p) * row_bytes;
  for (int off = threadIdx.x * 16; off < row_bytes; off += 256 * 16) {
    const int h = off / a.head_bytes, w = off % a.head_bytes;
    char* dst = head_row(a.rows, which, l, b, h, code, a.head_bytes, a.elem_bytes);
    *reinterpret_cast<uint4*>(dst + w) = *reinterpret_cast<const uint4*>(src + off);
  }
}

// One wave sleeping a fixed number of times (each s_sleep 127 is 127 * 64
// clock cycles), then leaving: a delay on a stream that always ends.
__global__ __launch_bounds__(64) void k_delay(int iters) {
  for (int i = 0; i < iters; ++i) __builtin_amdgcn_s_sleep(127);
}

}  // namespace

hipError_t launch_delay(int iters, hipStream_t s) {
  k_delay<<<1, 64, 0, s>>>(iters);
  return hipGetLastError();
}

hipError_t launch_place_rows(const PlaceArgs& a, int layers, hipStream_t s) {
  if (a.n_tokens <= 0) return hipSuccess;
  k_place_rows<<<dim3(a.n_tokens, layers * a.batch, 2), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tkvd
