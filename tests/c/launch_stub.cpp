// Host-only stand-ins for the kernel launchers (test infrastructure): they
// count calls and launch nothing, so the C-ABI entry points' argument checks
// and dispatch can run under the host sanitizers on a machine without a GPU.
#include "moef_internal.h"

namespace moef {

int g_launches = 0;
int g_cus = 256;

// The CU count the staged-kernel planning sees (set by moef_test_set_cus).
int device_cus(hipStream_t) { return g_cus; }

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

// The staged kernels' launch plan (moef_internal.h), for CPU tests of its
// sizing: out[0] = launches, out[1] = items per launch.
extern "C" void moef_test_plan_staged(int64_t items, int ncu, int64_t per_wg_max, int64_t* out) {
  const moef::StagedPlan p = moef::plan_staged(items, ncu, per_wg_max);
  out[0] = p.launches;
  out[1] = p.per_launch;
}

// The staging capacities the launchers size with: units per workgroup in
// LDS and in register slots per wave, for the quant, plain and RMSNorm
// kernels, the waves per staged workgroup, and the staged-path thresholds in
// units per CU, the top_k the staged kernels take, and the quant kernel's tail
// percentage, the plain staged kernel's waves per workgroup, the units per CU
// from which the quant kernel takes tail workgroups, and the plain kernel's
// wide layout (waves, register slots) for grids the 16-wave one cannot hold.
extern "C" void moef_test_stage_caps(int64_t* out) {
  out[0] = moef::kStageUnits;
  out[1] = moef::kStageRegUnits;
  out[2] = moef::kStagePlainUnits;
  out[3] = moef::kStagePlainRegUnits;
  out[4] = moef::kStageRmsUnits;
  out[5] = moef::kStageWaves;
  out[6] = moef::kStagedFromUnitsPerCu;
  out[7] = moef::kStagedPlainFromUnitsPerCu;
  out[8] = moef::kStagedRmsFromUnitsPerCu;
  out[9] = moef::kStagedMaxTopK;
  out[10] = moef::kStagedTailPercent;
  out[11] = moef::kStagePlainWaves;
  out[12] = moef::kStagedTailFromUnitsPerCu;
  out[13] = moef::kStagePlainWideWaves;
  out[14] = moef::kStagePlainWideRegUnits;
}

// The staged quant kernel's token plan and its group count for `ncu` CUs:
// out[0] = launches, out[1] = tokens per launch, out[2] = groups.
extern "C" void moef_test_plan_staged_tokens(int64_t tokens, int64_t nchunks, int ncu,
                                             int64_t per_wg_max, int64_t* out) {
  const int groups = moef::staged_quant_groups(ncu);
  const moef::StagedPlan p = moef::plan_staged_tokens(tokens, nchunks, ncu, groups, per_wg_max);
  out[0] = p.launches;
  out[1] = p.per_launch;
  out[2] = groups;
}

// The CU count moe_finalize_describe_launch plans for in this build.
extern "C" void moef_test_set_cus(int ncu) { moef::g_cus = ncu; }
