// Link stubs for a host-only build of the planner and the C ABI (tests/c/plan_sanitize.cpp).
// The calls that driver makes never reach the kernel launchers or the HIP runtime; each
// stub aborts with its name if one ever does, so a stub cannot stand in for real work.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>

#include "ga_internal.h"

[[noreturn]] static void reached(const char* name) {
  std::fprintf(stderr, "stub reached: %s\n", name);
  std::abort();
}

namespace ga {
bool fwd_supported(ga_dtype, ga_score, const Geometry&) { reached(__func__); }
bool bwd_supported(ga_dtype, const Geometry&) { reached(__func__); }
bool reduce_supported(ga_dtype, int) { reached(__func__); }
int launch_fwd(ga_dtype, int, const Geometry&, const FwdArgs&, int64_t, void*, TimerHook) {
  reached(__func__);
}
int launch_bwd(ga_dtype, const Geometry&, const BwdArgs&, int64_t, void*, TimerHook) {
  reached(__func__);
}
int launch_bwd_gat(ga_dtype, const Geometry&, const BwdArgs&, void*, TimerHook) {
  reached(__func__);
}
int launch_bwd_gatv2(ga_dtype, const Geometry&, const BwdArgs&, void*, TimerHook) {
  reached(__func__);
}
int64_t gatv2_da_slots(const ga_plan*, const Geometry&) { reached(__func__); }
int64_t gatv2_row_partial_floats(int, int) { reached(__func__); }
int64_t gatv2_reduce_rows(int64_t) { reached(__func__); }
int launch_reduce(ga_dtype, bool, int, int, const RedArgs&, void*, TimerHook) {
  reached(__func__);
}
int launch_copy(void*, const void*, size_t, void*, TimerHook) { reached(__func__); }
int launch_gather_probe_rows(const ProbeLaunch&, void*, TimerHook) { reached(__func__); }
int launch_gather_probe_cols(const ProbeLaunch&, void*, TimerHook) { reached(__func__); }
int launch_gather_probe_random(int, const void*, int64_t, int64_t, uint64_t, void*, void*,
                               TimerHook) {
  reached(__func__);
}
}  // namespace ga

extern "C" {
hipError_t hipEventCreate(hipEvent_t*) { reached(__func__); }
hipError_t hipEventElapsedTime(float*, hipEvent_t, hipEvent_t) { reached(__func__); }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { reached(__func__); }
hipError_t hipEventSynchronize(hipEvent_t) { reached(__func__); }
hipError_t hipGetDevice(int*) { reached(__func__); }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  reached(__func__);
}
hipError_t hipStreamSynchronize(hipStream_t) { reached(__func__); }
}
