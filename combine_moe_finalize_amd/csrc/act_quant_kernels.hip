// gfx950 standalone FP8 activation quantization, 1 x 128 blocks along hidden.
//
// "[FP8][MoE] Honor UE8M0 activation scales in Triton MoE" (Motivation, "More
// context"): the activations entering each expert linear layer are quantized
// to FP8 with FP32 block scales; the checkpoint's `scale_fmt: ue8m0` asks for
// power-of-two scales where the older path used the continuous amax / 448.
// Both policies are here (the second for comparison):
//  * power-of-two: e = least integer with amax <= 448 * 2^e, byte e + 127,
//    q = e4m3(x / 2^e) -- the same device code as the finalize epilogue;
//  * continuous: s = amax / 448 (one correctly rounded fp32 division; 1 for
//    an all-zero block), q = e4m3(x / s) (fp32 division, then the plain E4M3
//    converter, nearest even), the scale stored as float32.
//
// The continuous policy needs one correctly rounded fp32 quotient per element.
// The compiler's IEEE division is 11 VALU ops, which made this kernel
// ALU-bound. Here it is 5 FMA-unit ops per element: one IEEE reciprocal
// y = fl(1/s) per lane, then div_rn below (Markstein's refinement, P. W.
// Markstein, "Computation of elementary functions on the IBM RISC System/6000
// processor", IBM J. Res. Dev. 34(1), 1990). The result is bit-identical to
// the IEEE quotient whenever the operands and residuals are normal fp32
// numbers. Outside that, |x| < 2^-100 with s >= 2^-60, so both quotients are
// below 2^-40 and encode to the same signed zero. The scale itself,
// fl(amax / 448), takes the same sequence with the constant fl(1/448). Blocks
// whose scale falls outside [2^-60, 2^60] keep the IEEE divisions. Each code
// takes its sign from its input (one byte permute per four codes), which
// also restores the sign of a zero quotient.
//
// The input is read as a flat run of 16-byte vectors (8 bf16 each). Since
// hidden is a multiple of 128, every aligned group of 16 vectors is one
// 1 x 128 block of one token, so a 16-lane DPP row is one block wherever a
// wave starts. A wave takes 64 U consecutive vectors, U = 1 or 2, and issues
// all U loads of a lane before any arithmetic: a lane with a single 16-byte
// load in flight leaves too few bytes in flight to cover HBM latency once
// every wave slot is busy. HBM-bound: 2 bytes read and 1 byte written per
// element, plus the scales.

#include <type_traits>

#include "device_common.h"
#include "moef_internal.h"

namespace moef {
namespace {

using namespace dev;

// fl(x / s), the correctly rounded quotient, given y = fl(1 / s) and s in
// [2^-60, 2^60]:
//  * q1 = fl(x y) is within 1.5 ulp of x/s;
//  * one residual step makes q2 faithful (within 1 ulp);
//  * with y within half an ulp of 1/s and q2 faithful, the residual
//    x - s q2 is exact and fl(q2 + (x - s q2) y) = fl(x/s) (Markstein).
// A zero quotient of a negative x may come out as +0 (a cancelling final
// sum); the caller takes the signs from the inputs.
__device__ __forceinline__ float div_rn(float x, float s, float y) {
  const float q1 = x * y;
  const float q2 = __builtin_fmaf(__builtin_fmaf(-s, q1, x), y, q1);
  return __builtin_fmaf(__builtin_fmaf(-s, q2, x), y, q2);
}

// bf16 bits of the block maxima 1.75 * 2^-52 and 1.75 * 2^68, between which
// s = amax / 448 lies in [2^-60, 2^60].
constexpr uint32_t kAmaxDivLo = (75u << 7) | 0x60u;
constexpr uint32_t kAmaxDivHi = (195u << 7) | 0x60u;
// fl(1 / 448), the reciprocal div_rn takes for the scale.
constexpr float kRcp448 = 1.0f / 448.0f;

// Eight fp32 values -> eight E4M3 codes, nearest even (the plain converter),
// two per op, in column order.
__device__ __forceinline__ u32x2 e4m3x8(const float f[8]) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
  return u32x2{(uint32_t)lo, (uint32_t)hi};
}

// The sign bits of the four bf16 values in (a, b), as bit 7 of bytes 0..3
// (byte j holds the code of value j: a's low and high halves, then b's).
__device__ __forceinline__ uint32_t signs4(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07050301u) & 0x80808080u;
}

// Quantizes one lane's 8 values (vector vi of the flat [T, H/8] view); the
// lane's 16-lane DPP row is one 1 x 128 block. Whole rows share `active`.
template <bool POW2>
__device__ __forceinline__ void quant_vector(const u32x4 v, bool active, int64_t vi, int lane,
                                             u32x2* __restrict__ out_q,
                                             uint8_t* __restrict__ scale_e8m0,
                                             float* __restrict__ scale_f32) {
  const uint32_t amax = row16_max(active ? absmax8_bits(v) : 0u);
  u32x2 q;
  if (POW2) {
    const int ex = ue8m0_exponent(amax);
    q = e4m3x8_scaled(v, ue8m0_scale(ex));
    if (active && (lane & 15) == 0) scale_e8m0[vi >> 4] = (uint8_t)(ex + 127);
  } else {
    float f[8];
    unpack8(v, f);
    float s;
    if (amax >= kAmaxDivLo && amax <= kAmaxDivHi) {    // block-uniform: whole 16-lane rows
      s = div_rn(__uint_as_float(amax << 16), 448.0f, kRcp448);
      const float y = 1.0f / s;
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = div_rn(f[e], s, y);
    } else {
      const float a = __uint_as_float(amax << 16);
      s = a > 0.0f ? a / 448.0f : 1.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = f[e] / s;
    }
    q = e4m3x8(f);
    q.x |= signs4(v.x, v.y);
    q.y |= signs4(v.z, v.w);
    if (active && (lane & 15) == 0) scale_f32[vi >> 4] = s;
  }
  if (active) __builtin_nontemporal_store(q, out_q + vi);
}

template <bool POW2, int U>
__global__ void __launch_bounds__(kWavesPerBlock * kWaveLanes)
act_quant_kernel(const u32x4* __restrict__ x, int64_t n, u32x2* __restrict__ out_q,
                 uint8_t* __restrict__ scale_e8m0, float* __restrict__ scale_f32) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * (kWaveLanes * U);
  if (base >= n) return;                                        // whole waves
  u32x4 v[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int64_t vi = base + i * kWaveLanes + lane;
    v[i] = __builtin_nontemporal_load(x + (vi < n ? vi : n - 1));
  }
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int64_t vi = base + i * kWaveLanes + lane;
    quant_vector<POW2>(v[i], vi < n, vi, lane, out_q, scale_e8m0, scale_f32);
  }
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* x, int64_t tokens, int64_t hidden, uint8_t* out_q,
                            uint8_t* scale_e8m0, float* scale_f32, hipStream_t stream) {
  const int64_t n = tokens * (hidden / kVecElems);            // a multiple of 16
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  u32x2* q = reinterpret_cast<u32x2*>(out_q);
  const dim3 block(kWavesPerBlock * kWaveLanes);
  auto go = [&](auto u) {
    constexpr int U = decltype(u)::value;
    const int64_t per_block = (int64_t)kWavesPerBlock * kWaveLanes * U;
    const dim3 grid((unsigned int)((n + per_block - 1) / per_block));
    if (scale_e8m0 != nullptr)
      hipLaunchKernelGGL((act_quant_kernel<true, U>), grid, block, 0, stream, xv, n, q,
                         scale_e8m0, scale_f32);
    else
      hipLaunchKernelGGL((act_quant_kernel<false, U>), grid, block, 0, stream, xv, n, q,
                         scale_e8m0, scale_f32);
    return hipGetLastError();
  };
  // Two vectors per lane once the input reaches 32 MiB (2^21 vectors): enough
  // waves remain to fill the chip, and each has twice the bytes in flight.
  // Below that, one vector per lane keeps more waves.
  if (n >= kActQuantPairFrom) return go(std::integral_constant<int, 2>{});
  return go(std::integral_constant<int, 1>{});
}

}  // namespace moef
