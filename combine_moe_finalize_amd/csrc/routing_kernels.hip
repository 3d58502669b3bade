// gfx950 routing front-end: the sigmoid top-k gate that produces the routing
// the deferred finalize consumes, in both formats: fp32 weights, and packed
// (expert_id << 16) | bf16(weight) words ("[Deepseek V4] Keep fp32 routing
// weights in the mxfp4 trtllm MoE", PR description: the gate yields fp32
// weights; packing them truncates to bf16).
//
// Readings (the pages give no formula): scores are sigmoid(logit); the top_k
// experts are the top_k logits (sigmoid is increasing, so the choice never
// depends on how sigmoid is evaluated); ties go to the lower expert id and NaN
// ranks below every number; outputs are ordered by descending logit; the
// weights are the chosen sigmoids divided by their sum, in fp32.
//
// One wavefront per token. A lane holds up to 8 of the token's E <= 512
// logits in registers as 32-bit order keys: an order-preserving image of the
// logit, with NaN mapped to 1 (below -inf) and "no candidate" to 0. Each of
// the top_k rounds takes
//  * every lane's largest live key;
//  * the maximum inside each 16-lane row, by four DPP rotate-and-max steps;
//  * the maximum of the four rows by two DPP row-broadcast steps, read from
//    the last lane into a scalar register.
// Equal keys are then told apart without memory traffic: one ballot per
// register slot j marks the lanes that hold the maximum, and the first slot
// with a mark, then its lowest lane, is the lowest expert id (expert =
// lane + 64 j), which is the tie rule. Lane r keeps round r's winner. Lanes
// 0..top_k-1 then evaluate their sigmoid, the wave sums them, and each writes
// its slot.

#include "device_common.h"
#include "moef_internal.h"

namespace moef {
namespace {

using namespace dev;

constexpr int kGateWaves = 4;

// Order-preserving 32-bit image of a logit: a larger value gives a larger
// key; -0 and +0 map together; NaN maps to 1, below -inf (0x007FFFFF);
// 0 is left for "no candidate".
__device__ __forceinline__ uint32_t gate_key(float v) {
  if (v != v) return 1u;
  const uint32_t u = v == 0.0f ? 0u : __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The logit a key came from (+0 for a zero, NaN for key 1).
__device__ __forceinline__ float key_value(uint32_t k) {
  if (k == 1u) return __builtin_nanf("");
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int EPL>
__global__ void __launch_bounds__(kGateWaves * kWaveLanes)
topk_sigmoid_gate_kernel(const float* __restrict__ logits, int tokens, int experts, int k,
                         int32_t* __restrict__ ids, float* __restrict__ weights,
                         int32_t* __restrict__ packed) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int t = (int)blockIdx.x * kGateWaves + wave;
  if (t >= tokens) return;                       // whole waves
  const float* row = logits + (int64_t)t * experts;

  uint32_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + j * kWaveLanes;
    key[j] = e < experts ? gate_key(row[e]) : 0u;
  }

  uint32_t my_key = 0;                           // lane r keeps round r's winner
  int my_id = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t b = key[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) b = max(b, key[j]);
    const uint32_t m = wave_max_u32(b);
    // k <= live candidates, so m >= 1 and some slot holds it
    int wj = EPL - 1;
    uint64_t hit = 0;
#pragma unroll
    for (int j = EPL - 1; j >= 0; --j) {         // ends on the first slot with a hit
      const uint64_t bj = __ballot(key[j] == m);
      if (bj != 0) { wj = j; hit = bj; }
    }
    const int wl = (int)__builtin_ctzll(hit);
    if (lane == r) { my_key = m; my_id = wl + wj * kWaveLanes; }
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (j == wj && lane == wl) key[j] = 0u;
  }

  const float my_v = key_value(my_key);
  const float s = lane < k ? 1.0f / (1.0f + expf(-my_v)) : 0.0f;
  const float sum = wave_sum(s);
  if (lane < k) {
    const float w = s / sum;
    const int64_t o = (int64_t)t * k + lane;
    ids[o] = my_id;
    if (weights != nullptr) weights[o] = w;
    if (packed != nullptr) {
      const uint32_t wb = bf16x2_rne(w, 0.0f) & 0xFFFFu;
      packed[o] = (int32_t)(((uint32_t)my_id << 16) | wb);
    }
  }
}

}  // namespace

hipError_t launch_topk_sigmoid_gate(const float* logits, int64_t tokens, int32_t experts,
                                    int32_t top_k, int32_t* ids, float* weights,
                                    int32_t* packed, hipStream_t stream) {
  const unsigned int blocks = (unsigned int)((tokens + kGateWaves - 1) / kGateWaves);
  const dim3 grid(blocks), block(kGateWaves * kWaveLanes);
  const int t = (int)tokens;
  if (experts <= 64)
    hipLaunchKernelGGL(topk_sigmoid_gate_kernel<1>, grid, block, 0, stream, logits, t, experts,
                       top_k, ids, weights, packed);
  else if (experts <= 128)
    hipLaunchKernelGGL(topk_sigmoid_gate_kernel<2>, grid, block, 0, stream, logits, t, experts,
                       top_k, ids, weights, packed);
  else if (experts <= 256)
    hipLaunchKernelGGL(topk_sigmoid_gate_kernel<4>, grid, block, 0, stream, logits, t, experts,
                       top_k, ids, weights, packed);
  else
    hipLaunchKernelGGL(topk_sigmoid_gate_kernel<8>, grid, block, 0, stream, logits, t, experts,
                       top_k, ids, weights, packed);
  return hipGetLastError();
}

}  // namespace moef
