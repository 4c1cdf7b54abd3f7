// Stub of the launch layer for the host-only sanitizer build of api.cpp: every launch
// reports that no device is present and no device is current, so the validation and
// planning code runs exactly as in the library and every valid call ends in
// SINK_ATTN_ERR_HIP instead of a kernel launch.
#include "sa_launch.h"

namespace sa {

int device_cu_count() { return 0; }

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  return hipErrorNoDevice;
}

hipError_t launch_prefill(const PrefillArgs&, int, int, const RopeArgs&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_decode_split(const DecodeArgs&, int, int, int, bool, const int32_t*,
                               const RopeArgs&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_kv_append(const AppendArgs&, int, int, int, const int32_t*, const RopeArgs&,
                            hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_rope_apply(void*, int64_t, int, int, int64_t, int64_t, const int32_t*,
                             const RopeArgs&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_decode_stream(const DecodeArgs&, int, const StreamPlan&, const RopeArgs&,
                                const int32_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_merge_stream(const DecodeArgs&, int, const StreamPlan&, int64_t, bool,
                               hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_merge(const float*, const float*, const int32_t*, int64_t, int, int, void*,
                        float*, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace sa
