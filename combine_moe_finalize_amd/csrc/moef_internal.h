// Internal interface between the C-ABI entry points (moef_api.hip) and the
// gfx950 kernels (finalize_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_finalize.h"

namespace moef {

// The routed half of every finalize call: gemm2_out rows, the [T, top_k]
// index map and weights, the optional shared-expert output and the routed
// scaling factor. Validated by the entry points before any launch.
struct Routed {
  const uint16_t* gemm2_out;  // bf16 [num_rows, hidden]
  int64_t num_rows;
  const int32_t* idx;         // int32 [T, top_k]
  const uint32_t* weights;    // fp32 bits or packed words [T, top_k]
  bool packed;                // true: (id << 16) | bf16 bits
  const uint16_t* shared;     // bf16 [T, hidden] or nullptr
  float rsf;
  int64_t tokens;
  int64_t hidden;
  int32_t top_k;
  int32_t* err_flag;          // optional device int32
};

hipError_t launch_finalize(const Routed& r, uint16_t* out, hipStream_t stream);

hipError_t launch_finalize_rmsnorm(const Routed& r, const uint16_t* residual,
                                   const uint16_t* gamma, float eps,
                                   uint16_t* residual_out, uint16_t* normed,
                                   hipStream_t stream);

hipError_t launch_finalize_quant(const Routed& r, uint8_t* out_e4m3,
                                 uint8_t* scale_e8m0, hipStream_t stream);

hipError_t launch_ep_combine(const uint16_t* partials, int32_t num_partials,
                             const uint16_t* shared, uint16_t* out, int64_t tokens,
                             int64_t hidden, hipStream_t stream);

hipError_t launch_allreduce_rmsnorm(const uint16_t* const* rank_outputs, int32_t num_ranks,
                                    const uint16_t* residual, const uint16_t* gamma, float eps,
                                    uint16_t* residual_out, uint16_t* normed, int64_t tokens,
                                    int64_t hidden, hipStream_t stream);

hipError_t launch_packed_decode(const int32_t* packed, int64_t n,
                                int32_t* expert_ids, float* weights,
                                hipStream_t stream);

// exactly one of scale_e8m0 (power-of-two policy) / scale_f32 (amax / 448)
hipError_t launch_act_quant(const uint16_t* x, int64_t tokens, int64_t hidden, uint8_t* out_q,
                            uint8_t* scale_e8m0, float* scale_f32, hipStream_t stream);

hipError_t launch_topk_sigmoid_gate(const float* logits, int64_t tokens, int32_t experts,
                                    int32_t top_k, int32_t* ids, float* weights,
                                    int32_t* packed, hipStream_t stream);

// Launch-shape limits the entry points enforce.
constexpr int kWaveLanes = 64;
constexpr int kVecElems = 8;                           // bf16 per 16-byte vector
constexpr int kChunkCols = kWaveLanes * kVecElems;     // columns per wave pass
constexpr int kWavesPerBlock = 4;                      // plain / quant kernels
constexpr int kNormMaxThreads = 1024;                  // RMSNorm: one block per token
constexpr int kNormMaxChunks = MOEF_MAX_HIDDEN_RMSNORM / (kVecElems * kWaveLanes);
constexpr int64_t kNormHalfWidthFrom = 1024;           // tokens: half-width RMSNorm blocks
constexpr int64_t kActQuantPairFrom = int64_t(1) << 21;  // act quant: 2 vectors per lane
// Occupancy cap for large launches: a launch may reserve LDS it does not use
// so that at most `blocks` workgroups are resident on a CU at once (gfx950:
// 160 KiB of LDS per CU). Returns the bytes to reserve: `blocks` workgroups
// fit, one more does not.
constexpr int kLdsPerCu = 160 * 1024;
constexpr size_t lds_for_blocks_per_cu(int blocks) {
  return (size_t)((kLdsPerCu / (blocks + 1) + 512) / 512 * 512);
}
// The finalize kernels with one wave per (token, chunk) and the EP combine
// hold at most 4 of their 4-wave workgroups (16 waves) per CU once a grid is
// twice what fits on the chip uncapped (16384 waves): fewer waves streaming
// at once lose less to reads and writes mixing at the DRAM. (The act-quant
// kernels measured slower with any cap and run uncapped.)
constexpr int kStreamCapBlocksPerCu = 4;
constexpr int64_t kStreamCapFromWaves = 16384;
constexpr size_t stream_cap_lds(int64_t waves) {
  return waves >= kStreamCapFromWaves ? lds_for_blocks_per_cu(kStreamCapBlocksPerCu) : 0;
}
// The UE8M0 finalize on large grids stages its output on chip and writes it
// after the gathers (finalize_quant_staged_kernel): one workgroup of
// kStageWaves waves per CU owns all 160 KiB of the CU's LDS, which holds the
// codes and scale bytes of kStageUnits (token, chunk) units (516 bytes each);
// each wave holds up to kStageRegUnits more in registers. A launch covers at
// most (kStageUnits + kStageWaves * kStageRegUnits) units per CU; larger
// grids take several launches. Used from kStagedFromUnitsPerCu units per CU
// (T = 1463 at H = 7168 on 256 CUs) and top_k <= 8; below that the
// one-wave-per-unit kernel is as fast or faster (its grid fits the chip in
// few rounds; measured equal at 70 units per CU, faster at 56).
constexpr int kStageWaves = 16;
constexpr int kStageThreads = kStageWaves * kWaveLanes;
constexpr int kStageUnitBytes = kChunkCols + 4;        // E4M3 codes + 4 scale bytes
constexpr int kStageUnits = (kLdsPerCu - 256) / kStageUnitBytes;   // 317
constexpr int kStageRegUnits = 12;
constexpr int64_t kStagedFromUnitsPerCu = 80;
constexpr int kStagedMaxTopK = 8;
static_assert(kStageUnits * kStageUnitBytes + 4 <= kLdsPerCu, "staging fits the CU's LDS");
// The plain finalize stages the same way: 1 KiB of bf16 output per unit, 159
// units in LDS and up to 8 more per wave in registers (four VGPRs each); used
// from 48 units per CU (T = 878 at H = 7168 on 256 CUs), top_k <= 8.
constexpr int kStagePlainUnitBytes = kChunkCols * 2;
constexpr int kStagePlainUnits = (kLdsPerCu - 256) / kStagePlainUnitBytes;   // 159
constexpr int kStagePlainRegUnits = 8;
constexpr int64_t kStagedPlainFromUnitsPerCu = 48;
static_assert(kStagePlainUnits * kStagePlainUnitBytes + 4 <= kLdsPerCu, "staging fits the LDS");
// The RMSNorm epilogue with two column vectors per lane holds at most 20
// waves per CU (5 per SIMD): measured faster at large T than the 24 its
// register use would allow.
constexpr int kNorm2MaxWavesPerCu = 20;
static_assert(lds_for_blocks_per_cu(kStreamCapBlocksPerCu) * kStreamCapBlocksPerCu <= kLdsPerCu &&
              lds_for_blocks_per_cu(kStreamCapBlocksPerCu) * (kStreamCapBlocksPerCu + 1) > kLdsPerCu &&
              lds_for_blocks_per_cu(kStreamCapBlocksPerCu) <= 65536, "cap reservation");
// A kernel dispatch packet states a 1-D grid's size in work-items in a 32-bit
// field, so one launch holds at most 2^32 - 1 work-items. kMaxGridItems is the
// largest multiple of 256 (every rounded-up grid here uses 256-lane
// workgroups) below that; a grid of at most kMaxUnits one-wave units, or of
// kMaxGridItems single-lane items, rounded up to whole workgroups, fits.
constexpr int64_t kMaxGridItems = (int64_t(1) << 32) - 256;
constexpr int64_t kMaxUnits = kMaxGridItems / kWaveLanes;   // 2^26 - 4 (token, chunk) pairs
static_assert(kMaxUnits % kWavesPerBlock == 0, "whole 4-wave workgroups");
static_assert(kMaxUnits == MOEF_MAX_UNITS && kMaxGridItems == MOEF_MAX_ITEMS, "header limits");

}  // namespace moef
