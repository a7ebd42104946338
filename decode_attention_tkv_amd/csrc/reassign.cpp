// Reassignment (Method §1, §4): rank, label, changed-row lists and moves.
#include "handle.hpp"
#include "host_util.hpp"

extern "C" int tkv_reassign(tkv_t* t, tkv_stream_t stream) {
  (void)stream;
  if (!t) return tkv_fail(nullptr, TKV_EINVAL, "handle is NULL");
  return tkv_fail(t, TKV_ESTATE, "reassignment is not available yet");
}
