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
// logits in registers, each as a 64-bit key (order-preserving image of the
// logit above the complemented expert id), so one unsigned compare implements
// the whole order. Each of the top_k rounds takes every lane's best live key,
// the maximum inside each 16-lane row by four DPP steps, and the four row
// maxima read into scalar registers: the winner is uniform with no LDS or
// memory traffic. Lane r keeps round r's winner. Lanes 0..top_k-1 then
// evaluate their sigmoid, the wave sums them, and each writes its slot.

#include "device_common.h"
#include "moef_internal.h"

namespace moef {
namespace {

using namespace dev;

constexpr int kGateWaves = 4;

// Order-preserving 32-bit image of a logit: larger value -> larger image;
// -0 and +0 map together; NaN maps to 0, below -inf.
__device__ __forceinline__ uint32_t order_bits(float v) {
  if (v != v) return 0u;
  const uint32_t u = v == 0.0f ? 0u : __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_bits for non-NaN images (0 -> NaN).
__device__ __forceinline__ float from_order_bits(uint32_t o) {
  if (o == 0u) return __builtin_nanf("");
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Candidate key: a larger key comes first (larger logit, then lower id).
// 0 means "no candidate".
__device__ __forceinline__ uint64_t cand_key(float v, int e) {
  return ((uint64_t)order_bits(v) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t dpp_max(uint64_t k, int ctrl_sel) {
  uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
  uint32_t olo, ohi;
  switch (ctrl_sel) {   // constant after unrolling
    case 0:
      olo = __builtin_amdgcn_mov_dpp((int)lo, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
      ohi = __builtin_amdgcn_mov_dpp((int)hi, 0xB1, 0xF, 0xF, false);
      break;
    case 1:
      olo = __builtin_amdgcn_mov_dpp((int)lo, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
      ohi = __builtin_amdgcn_mov_dpp((int)hi, 0x4E, 0xF, 0xF, false);
      break;
    case 2:
      olo = __builtin_amdgcn_mov_dpp((int)lo, 0x124, 0xF, 0xF, false);  // row_ror:4
      ohi = __builtin_amdgcn_mov_dpp((int)hi, 0x124, 0xF, 0xF, false);
      break;
    default:
      olo = __builtin_amdgcn_mov_dpp((int)lo, 0x128, 0xF, 0xF, false);  // row_ror:8
      ohi = __builtin_amdgcn_mov_dpp((int)hi, 0x128, 0xF, 0xF, false);
      break;
  }
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > k ? o : k;
}

// The largest key of the wave, uniform: DPP maxima inside each 16-lane row,
// then the four row maxima read into scalar registers.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
#pragma unroll
  for (int c = 0; c < 4; ++c) k = dpp_max(k, c);
  const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
  uint64_t best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t rk = ((uint64_t)__builtin_amdgcn_readlane(hi, 16 * r) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane(lo, 16 * r);
    best = rk > best ? rk : best;
  }
  return best;
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

  uint64_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + j * kWaveLanes;
    key[j] = e < experts ? cand_key(row[e], e) : 0u;
  }

  uint64_t mine = 0;                             // lane r keeps round r's winner
  for (int r = 0; r < k; ++r) {
    uint64_t b = key[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) b = key[j] > b ? key[j] : b;
    const uint64_t win = wave_max_key(b);        // uniform
    if (lane == r) mine = win;
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (key[j] == win) key[j] = 0u;            // keys are unique: one lane, one slot
  }

  const int my_id = (int)(0xFFFFFFFFu - (uint32_t)mine);
  const float my_v = from_order_bits((uint32_t)(mine >> 32));
  const float s = lane < k ? 1.0f / (1.0f + expf(-my_v)) : 0.0f;
  float sum = s;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
  sum = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sum)));
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
