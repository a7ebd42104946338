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

// Device buffers handed over are read in 16-byte pieces.
inline bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

// floor(ratio * n) in fp64: the tier budgets of Method §1.
inline int64_t floor_ratio(double r, int64_t n) { return (int64_t)std::floor(r * (double)n); }

// Protected positions of a sequence holding n positions: [0, prompt),
// [0, sinks) and the last `recent` (Method §1: prompt, sinks, recent window).
inline bool is_protected(const tkv& t, int64_t i, int64_t n) {
  return i < t.prompt || i < t.sinks || i >= n - t.recent;
}

// Placement of a freshly filled cache before any score exists: protected
// rows plus the lowest positions in T0 up to floor(hbm * n), the rest T1.
inline std::vector<uint8_t> first_placement(const tkv& t, int n) {
  std::vector<uint8_t> tier(n, TKV_T1);
  int64_t np = 0;
  for (int i = 0; i < n; ++i)
    if (is_protected(t, i, n)) {
      tier[i] = TKV_T0;
      ++np;
    }
  const int64_t ncand = n - np;
  int64_t room = std::min<int64_t>(ncand, std::max<int64_t>(0, floor_ratio(t.hbm, n) - np));
  for (int i = 0; i < n && room > 0; ++i)
    if (tier[i] == TKV_T1) {
      tier[i] = TKV_T0;
      --room;
    }
  if (t.flags & TKV_FLAG_NO_T1)
    for (auto& x : tier)
      if (x == TKV_T1) x = TKV_T3;
  return tier;
}

// Candidates newly evicted (n3), kept in T0 (n0c) and put in T2 (n2) at one
// reassignment (Method §1 budgets as floor(ratio * n)).
struct CutCounts {
  int64_t n3, n0c, n2;
};
inline CutCounts cut_counts(const tkv& t, int64_t n, int64_t np, int64_t nev) {
  const int64_t ncand = n - np - nev;
  CutCounts c{};
  if (t.flags & TKV_FLAG_NO_T1) {
    c.n0c = std::min<int64_t>(ncand, std::max<int64_t>(0, floor_ratio(t.hbm, n) - np));
    c.n2 = std::min<int64_t>(ncand - c.n0c, floor_ratio(t.t2, n));
    c.n3 = ncand - c.n0c - c.n2;
    return c;
  }
  c.n3 = std::min<int64_t>(ncand, std::max<int64_t>(0, floor_ratio(t.evict, n) - nev));
  c.n0c = std::min<int64_t>(ncand - c.n3, std::max<int64_t>(0, floor_ratio(t.hbm, n) - np));
  c.n2 = std::min<int64_t>(ncand - c.n3 - c.n0c, floor_ratio(t.t2, n));
  return c;
}
