// Row movement kernels: placing prefilled rows, gathering rows into a packed
// buffer and scattering packed rows to their new homes.  A "row" is one
// position's K (or V) for all kv heads of one layer of one sequence:
// kv_heads * head_dim contiguous elements.
#include "tkv_internal.hpp"

namespace tkvd {
namespace {

__device__ __forceinline__ char* row_addr(const RowSpace& rs, int which, int l, int b, uint32_t code,
                                          int64_t row_bytes, int elem_bytes) {
  if (code < (uint32_t)rs.cap0) {
    char* base = (char*)(which ? rs.pool_v : rs.pool_k);
    return base + ((int64_t)l * rs.pool_lstride + (int64_t)b * rs.pool_bstride) * elem_bytes +
           (int64_t)code * row_bytes;
  }
  char* base = (char*)(which ? rs.stage_v : rs.stage_k);
  return base + ((int64_t)(l % rs.stage_slots) * rs.stage_lstride + (int64_t)b * rs.stage_bstride) * elem_bytes +
         (int64_t)(code - rs.cap0) * row_bytes;
}

__device__ __forceinline__ void copy_row(char* dst, const char* src, int64_t row_bytes) {
  for (int64_t off = (int64_t)threadIdx.x * 16; off < row_bytes; off += (int64_t)blockDim.x * 16)
    *reinterpret_cast<uint4*>(dst + off) = *reinterpret_cast<const uint4*>(src + off);
}

// grid (n_tokens, layers*batch, 2): input row (l, b, p) -> its location code.
__global__ __launch_bounds__(256) void k_place_rows(const PlaceArgs a) {
  const int p = blockIdx.x;
  const int lb = blockIdx.y;
  const int b = lb % a.batch, l = lb / a.batch;
  const int which = blockIdx.z;
  const uint32_t code = a.codes[(int64_t)b * a.n_tokens + p];
  if (code == kNoLoc) return;
  const char* src = (const char*)(which ? a.v : a.k) + (((int64_t)lb * a.n_tokens) + p) * a.row_bytes;
  copy_row(row_addr(a.rows, which, l, b, code, a.row_bytes, a.elem_bytes), src, a.row_bytes);
}

}  // namespace

hipError_t launch_place_rows(const PlaceArgs& a, int layers, hipStream_t s) {
  if (a.n_tokens <= 0) return hipSuccess;
  k_place_rows<<<dim3(a.n_tokens, layers * a.batch, 2), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace tkvd
