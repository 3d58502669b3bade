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
// RMSNorm, one workgroup per token: from this many tokens on, half as many
// waves with two vectors per lane (H = 7168, kernel-trace medians, one wave
// per chunk -> half width: T = 256 8.44 -> 8.36 us; 320 11.68 -> 11.20; 512
// 17.04 -> 15.68; 704 23.64 -> 21.36; at T <= 64 half width is slower: T = 16
// 4.36 -> 4.76).
constexpr int64_t kNormHalfWidthFrom = 288;
constexpr int64_t kActQuantPairFrom = int64_t(1) << 21;  // act quant: 2 vectors per lane
// Occupancy cap for large launches: a launch may reserve LDS it does not use
// so that at most `blocks` workgroups are resident on a CU at once (gfx950:
// 160 KiB of LDS per CU). Returns the bytes to reserve: `blocks` workgroups
// fit, one more does not.
constexpr int kLdsPerCu = 160 * 1024;
constexpr size_t lds_for_blocks_per_cu(int blocks) {
  return (size_t)((kLdsPerCu / (blocks + 1) + 512) / 512 * 512);
}
// The finalize kernels with one wave per (token, chunk) hold at most 4 of
// their 4-wave workgroups (16 waves) per CU once a grid is twice what fits
// on the chip uncapped (16384 waves): fewer waves streaming at once lose
// less to reads and writes mixing at the DRAM. (The act-quant kernels
// measured slower with any cap and run uncapped.)
constexpr int kStreamCapBlocksPerCu = 4;
constexpr int64_t kStreamCapFromWaves = 16384;
constexpr size_t stream_cap_lds(int64_t waves) {
  return waves >= kStreamCapFromWaves ? lds_for_blocks_per_cu(kStreamCapBlocksPerCu) : 0;
}
// The EP combine's cap follows its partial count R. A thread loads the
// ranks four at a time and the last R % 4 of them one at a time, so with
// few partials it has few loads in flight and more workgroups per CU keep
// the memory system busy: no reservation for R = 1 (kEpCapNone: 8 of its
// 4-wave workgroups, the 32 wave slots of a CU), 7 for R = 2, 5 for R = 3,
// and the finalize kernels' 4 from R = 4. Kernel-trace medians against a
// fixed cap of 4 (µs, H = 7168): T = 8192, R = 1 / 2 / 3: 62.1 / 84.0 /
// 107.9 -> 54.1 / 75.6 / 94.0; R = 2 at T = 4096 and 2048: 41.8 -> 38.5,
// 21.6 -> 20.0. Caps of 3 or 5-7 from R = 4 on were no better across sizes
// (3 gains 2-3% at T = 8192 for R = 8 and 16 but loses 1-3% at T = 2048-4096).
constexpr int kEpCapNone = 8;
constexpr int ep_cap_blocks(int partials) {
  return partials <= 1 ? kEpCapNone : partials == 2 ? 7 : partials == 3 ? 5 : kStreamCapBlocksPerCu;
}
constexpr size_t ep_cap_lds(int64_t waves, int partials) {
  return waves >= kStreamCapFromWaves && ep_cap_blocks(partials) < kEpCapNone
             ? lds_for_blocks_per_cu(ep_cap_blocks(partials))
             : 0;
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
// From kStagedTailFromUnitsPerCu units per CU, the last kStagedTailPercent of
// each group's units go to workgroups beyond the one per CU, one unit per
// wave, which the dispatcher starts on the CUs that finish their share first
// (finalize_quant_staged_kernel). Measured at H = 7168 (kernel-trace medians
// without -> with): T = 2048 (112 units per CU) 44.4 -> 44.8 us; T = 2560
// (140) 55.9 -> 55.8; T = 3072 (168) 65.9 -> 64.9; T = 3584 (196) 76.7 ->
// 74.9; T = 4096 (224) 88.3 -> 86.6; T = 6144 131.0 -> 128.0; T = 8192 (448)
// 172.9 -> 169.1.
constexpr int kStagedTailPercent = 5;
constexpr int64_t kStagedTailFromUnitsPerCu = 160;
constexpr int kStagedMaxTopK = 8;
static_assert(kStageUnits * kStageUnitBytes + 4 <= kLdsPerCu, "staging fits the CU's LDS");
// The plain finalize stages the same way: 1 KiB of bf16 output per unit, 159
// units in LDS and more in registers (four VGPRs a unit). Workgroups of 16
// waves hold 8 register slots a wave (287 units per CU); grids larger than
// that take workgroups of 12 waves, whose waves may use 168 VGPRs, room for
// 25 slots (459 units per CU: T = 8192 at H = 7168 in one launch, 180.4 us
// against 184.4 for two 16-wave launches; at 224 units per CU the 16-wave
// layout was 1% faster). Used from 48 units per CU (T = 878 at H = 7168 on
// 256 CUs), top_k <= 8.
constexpr int kStagePlainUnitBytes = kChunkCols * 2;
constexpr int kStagePlainUnits = (kLdsPerCu - 256) / kStagePlainUnitBytes;   // 159
constexpr int kStagePlainWaves = 16;
constexpr int kStagePlainRegUnits = 8;
constexpr int kStagePlainWideWaves = 12;
constexpr int kStagePlainWideRegUnits = 25;
constexpr int64_t kStagedPlainFromUnitsPerCu = 48;
static_assert(kStagePlainUnits * kStagePlainUnitBytes + 4 <= kLdsPerCu, "staging fits the LDS");
// The staged quant kernel deals tokens to groups of workgroups, one group per
// XCD, in blocks of kXcdTokenBlock tokens, so that all scale bytes of a block
// are written through one XCD's L2 (finalize_quant_staged_kernel). MI355X
// has 8 XCDs and hands workgroups to them round-robin; a CU count that 8
// does not divide (a partitioned device) takes one group.
constexpr int kXcds = 8;
constexpr int kXcdTokenBlock = 16;
inline int staged_quant_groups(int ncu) { return ncu % kXcds == 0 ? kXcds : 1; }

// The staged quant kernel's launch plan, in whole tokens: a launch over Tl
// tokens gives each of its `groups` groups of ncu / groups workgroups at most
// ceil(Tl / groups) tokens, so a workgroup holds at most
// ceil(ceil(Tl / groups) * nchunks / (ncu / groups)) units. Launches are as
// few as keep that within per_wg_max, and as long as a multiple of
// groups * kXcdTokenBlock tokens where that fits. No launch (0) when not one
// token per group fits.
struct StagedPlan;
inline StagedPlan plan_staged_tokens(int64_t tokens, int64_t nchunks, int ncu, int groups,
                                     int64_t per_wg_max);

// The residual + RMSNorm epilogue stages the same way
// (finalize_rmsnorm_staged_kernel): a workgroup owns whole tokens, and each
// of their (token, chunk) units keeps 1 KiB of bf16 residual_out plus its
// sum of squares in LDS (4 more bytes per unit hold the per-token 1 / rms),
// 158 units per workgroup and launch, 11 tokens at H = 7168; larger grids
// take several launches. Used from kStagedRmsFromUnitsPerCu units per CU,
// top_k <= 8.
constexpr int kStageRmsUnitBytes = kChunkCols * 2 + 8;
constexpr int kStageRmsUnits = (kLdsPerCu - 256) / kStageRmsUnitBytes;     // 158
constexpr int64_t kStagedRmsFromUnitsPerCu = 40;
// The all-reduce + RMSNorm share stages the same way from
// kStagedArFromUnitsPerCu units per CU (R = 8, H = 7168, kernel-trace
// medians, one workgroup per token -> staged: T = 256 7.20 -> 7.64 us;
// 384 10.16 -> 9.80; 512 12.88 -> 11.48; 640 16.44 -> 15.64).
constexpr int64_t kStagedArFromUnitsPerCu = 20;
static_assert(kStageRmsUnits * kStageRmsUnitBytes + 4 <= kLdsPerCu, "staging fits the LDS");
static_assert(kStageRmsUnits / (MOEF_MAX_HIDDEN_RMSNORM / kChunkCols) >= 1,
              "a workgroup holds at least one token of the largest hidden size");

// Launch plan of a staged kernel: `items` (units, or tokens for the RMSNorm
// epilogue) in as few launches as keep every workgroup within `per_wg_max`
// items, each launch a contiguous range [r * per_launch, min(items, (r + 1)
// * per_launch)) spread round-robin over `ncu` workgroups (item i of the
// range to workgroup i % ncu), so a workgroup holds at most
// ceil(per_launch / ncu) <= per_wg_max items.
struct StagedPlan {
  int64_t launches;
  int64_t per_launch;
};
inline StagedPlan plan_staged(int64_t items, int ncu, int64_t per_wg_max) {
  const int64_t cap = (int64_t)ncu * per_wg_max;
  const int64_t launches = (items + cap - 1) / cap;
  return StagedPlan{launches, launches > 0 ? (items + launches - 1) / launches : 0};
}

inline StagedPlan plan_staged_tokens(int64_t tokens, int64_t nchunks, int ncu, int groups,
                                     int64_t per_wg_max) {
  const int64_t wpx = ncu / groups;
  const int64_t round = (int64_t)groups * kXcdTokenBlock;
  int64_t tl_max = groups * ((per_wg_max * wpx) / nchunks);
  if (tl_max >= round) tl_max = tl_max / round * round;
  if (tl_max <= 0 || tokens <= 0) return StagedPlan{0, 0};
  const int64_t launches = (tokens + tl_max - 1) / tl_max;
  int64_t per = (tokens + launches - 1) / launches;
  if (tl_max >= round) {
    per = (per + round - 1) / round * round;
    if (per > tl_max) per = tl_max;
  }
  return StagedPlan{(tokens + per - 1) / per, per};
}

// ---------------------------------------------------------- launch plans
// The launchers' choices, shared with moe_finalize_describe_launch so that
// what it reports is what they do. `ncu` is the CU count of the stream's
// device; 0 (unknown) keeps every call on the one-wave-per-unit kernels.

// The kernel instantiation a top_k runs: exact for 1, 2, 4, 6, 8, else the
// next larger instantiation with a runtime bound (guarded).
struct TopKChoice {
  int kmax;
  bool exact;
};
inline TopKChoice top_k_choice(int k) {
  if (k == 1 || k == 2 || k == 4 || k == 6 || k == 8) return TopKChoice{k, true};
  return TopKChoice{k <= 4 ? 4 : (k <= 8 ? 8 : 16), false};
}

inline int64_t nchunks_of(int64_t hidden) { return (hidden / kVecElems + kWaveLanes - 1) / kWaveLanes; }

// The plain finalize: staged (16-wave layout, else the wide 12-wave one) or
// one wave per unit.
struct PlainChoice {
  bool staged;
  bool wide;
  StagedPlan plan;      // units per launch
};
inline PlainChoice plain_choice(int64_t tokens, int64_t hidden, int top_k, int ncu) {
  PlainChoice c{false, false, StagedPlan{1, 0}};
  const int64_t units = tokens * nchunks_of(hidden);
  if (top_k > kStagedMaxTopK || ncu <= 0 || units < kStagedPlainFromUnitsPerCu * ncu) return c;
  c.staged = true;
  c.wide = units > (int64_t)ncu * (kStagePlainUnits + kStagePlainWaves * kStagePlainRegUnits);
  c.plan = plan_staged(units, ncu, kStagePlainUnits + (c.wide ? kStagePlainWideWaves * kStagePlainWideRegUnits
                                                              : kStagePlainWaves * kStagePlainRegUnits));
  return c;
}

// The residual + RMSNorm epilogue: staged (whole tokens per workgroup) or
// one workgroup per token with `threads` lanes and cpt vectors per lane.
struct RmsChoice {
  bool staged;
  StagedPlan plan;      // tokens per launch
  int threads;
  int cpt;
};
inline RmsChoice rmsnorm_choice(int64_t tokens, int64_t hidden, int top_k, int ncu) {
  RmsChoice c{false, StagedPlan{1, 0}, 0, 0};
  const int64_t nch = nchunks_of(hidden);
  if (top_k <= kStagedMaxTopK && ncu > 0 && tokens * nch >= kStagedRmsFromUnitsPerCu * ncu) {
    c.staged = true;
    c.plan = plan_staged(tokens, ncu, kStageRmsUnits / nch);
    return c;
  }
  // One thread per 16-byte column vector (one wave per 512-column chunk) up
  // to 16 waves; from kNormHalfWidthFrom tokens on, half as many waves with
  // two vectors per thread when the chunk count is even.
  int threads = (int)nch * kWaveLanes;
  if (tokens >= kNormHalfWidthFrom && nch % 2 == 0) threads /= 2;
  if (threads > kNormMaxThreads) threads = kNormMaxThreads;
  c.threads = threads;
  c.cpt = (int)((hidden / kVecElems + threads - 1) / threads);   // 1 or 2 (hidden <= 16384)
  return c;
}

// The UE8M0 finalize: staged (token groups per XCD, whole-token launches) or
// one wave per unit.
struct QuantChoice {
  bool staged;
  int groups;
  StagedPlan plan;      // tokens per launch
};
inline QuantChoice quant_choice(int64_t tokens, int64_t hidden, int top_k, int ncu) {
  QuantChoice c{false, 1, StagedPlan{1, 0}};
  const int64_t nch = nchunks_of(hidden);
  if (top_k > kStagedMaxTopK || ncu <= 0 || tokens * nch < kStagedFromUnitsPerCu * ncu) return c;
  const int64_t cap = kStageUnits + kStageWaves * kStageRegUnits;
  c.groups = staged_quant_groups(ncu);
  c.plan = plan_staged_tokens(tokens, nch, ncu, c.groups, cap);
  if (c.plan.launches == 0 && c.groups > 1) {
    c.groups = 1;
    c.plan = plan_staged_tokens(tokens, nch, ncu, c.groups, cap);
  }
  c.staged = c.plan.launches > 0;
  return c;
}
// Of one staged quant launch over tl tokens: whether a workgroup can hold
// more units than the LDS slots (the kernel with register slots), and the
// tail percentage.
inline bool quant_launch_regs(int64_t tl, int64_t nchunks, int ncu, int groups) {
  const int64_t wpx = ncu / groups;
  return ((tl + groups - 1) / groups * nchunks + wpx - 1) / wpx > kStageUnits;
}
inline int quant_launch_tail_percent(int64_t tl, int64_t nchunks, int ncu) {
  return tl * nchunks >= kStagedTailFromUnitsPerCu * ncu ? kStagedTailPercent : 0;
}
inline int64_t quant_launch_tail_workgroups(int64_t tl, int64_t nchunks, int groups, int pct) {
  const int64_t group_units = (tl + groups - 1) / groups * nchunks;
  return groups * ((group_units * pct / 100 + kStageWaves - 1) / kStageWaves);
}

// Writes into buf (NUL-terminated, at most len bytes) the kernel a call of
// this shape launches on a device with ncu CUs, in the form profilers print
// template instances ("name<8, true, 12>"), with its launch count and grid.
// op: 0 moe_finalize, 1 moe_finalize_residual_rmsnorm, 2 moe_finalize_quant_ue8m0.
void describe_finalize(int op, int64_t tokens, int64_t hidden, int top_k, int ncu, char* buf,
                       int64_t len);

// CUs of the device that runs `stream` (the current device for the null
// stream), or 0 if the runtime cannot say.
int device_cus(hipStream_t stream);

// The RMSNorm epilogue with two column vectors per lane holds at most 20
// waves per CU (5 per SIMD): measured faster at large T than the 24 its
// register use would allow.
constexpr int kNorm2MaxWavesPerCu = 20;
static_assert(lds_for_blocks_per_cu(5) * 5 <= kLdsPerCu && lds_for_blocks_per_cu(5) * 6 > kLdsPerCu &&
              lds_for_blocks_per_cu(7) * 7 <= kLdsPerCu && lds_for_blocks_per_cu(7) * 8 > kLdsPerCu,
              "EP combine cap reservations");
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
