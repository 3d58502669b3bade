// Host-only stand-ins for the kernel launchers (test infrastructure): they
// count calls and launch nothing, so the C-ABI entry points' argument checks
// and dispatch can run under the host sanitizers on a machine without a GPU.
#include "moef_internal.h"

namespace moef {

int g_launches = 0;

hipError_t launch_finalize(const Routed&, uint16_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_finalize_rmsnorm(const Routed&, const uint16_t*, const uint16_t*, float,
                                   uint16_t*, uint16_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_finalize_quant(const Routed&, uint8_t*, uint8_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_packed_decode(const int32_t*, int64_t, int32_t*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_ep_combine(const uint16_t*, int32_t, const uint16_t*, uint16_t*, int64_t,
                             int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_allreduce_rmsnorm(const uint16_t* const*, int32_t, const uint16_t*,
                                    const uint16_t*, float, uint16_t*, uint16_t*, int64_t, int64_t,
                                    hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_act_quant(const uint16_t*, int64_t, int64_t, uint8_t*, uint8_t*, float*,
                            hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_topk_sigmoid_gate(const float*, int64_t, int32_t, int32_t, int32_t*, float*,
                                    int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}

}  // namespace moef

// Launches the stubs have seen, for callers that load this code as a shared
// library.
extern "C" int moef_stub_launch_count(void) { return moef::g_launches; }
