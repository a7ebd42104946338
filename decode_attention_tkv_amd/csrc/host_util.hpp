// Small host-side helpers shared by the C ABI files.
#pragma once

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <exception>
#include <new>
#include <vector>

#include "handle.hpp"

int tkv_fail(tkv* t, int code, const char* fmt, ...);

// Runs the body of a C ABI call: no C++ exception leaves the library; a host
// allocation failure becomes TKV_ENOMEM, anything else TKV_EHIP.
template <typename F>
int guarded(tkv* t, F&& f) noexcept {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return tkv_fail(t, TKV_ENOMEM, "host memory allocation failed");
  } catch (const std::exception& e) {
    return tkv_fail(t, TKV_EHIP, "internal error: %s", e.what());
  } catch (...) {
    return tkv_fail(t, TKV_EHIP, "internal error");
  }
}

// Apply a pending Eq. 1 update of s on `stream` (no-op when none is pending).
int tkv_flush_score(tkv* t, hipStream_t stream);

#define HIP_TRY(t, call)                                                                       \
  do {                                                                                         \
    hipError_t e_ = (call);                                                                    \
    if (e_ != hipSuccess) {                                                                    \
      (void)hipGetLastError();                                                                 \
      return tkv_fail((t), TKV_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));           \
    }                                                                                          \
  } while (0)

// The handle's memory cap: TKV_OK when `bytes` more may be held.
inline bool within_cap(const tkv& t, size_t bytes) {
  return t.mem_cap <= 0 || t.mem_held + (int64_t)bytes <= t.mem_cap;
}

// Device buffers handed over are read in 16-byte pieces.
inline bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

// The static device scratch of the handle's GPU (static_scratch.hip): its
// address there and its size.
int static_scratch(tkv* t, void** base, size_t* cap);

// The tier rules of plan.hpp with a handle's policy.
inline bool is_protected(const tkv& t, int64_t i, int64_t n) {
  return tkvd::protected_at(i, n, t.prompt, t.sinks, t.recent);
}
inline std::vector<uint8_t> first_placement(const tkv& t, int n) {
  return tkvd::first_placement(n, t.prompt, t.sinks, t.recent, t.hbm, (t.flags & TKV_FLAG_NO_T1) != 0);
}
inline tkvd::CutCounts cut_counts(const tkv& t, int64_t n, int64_t np, int64_t nev) {
  return tkvd::cut_counts(n, np, nev, t.hbm, t.evict, t.t2, (t.flags & TKV_FLAG_NO_T1) != 0);
}
