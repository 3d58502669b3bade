// Device helpers shared by the gfx950 kernels of this library: bf16 and
// FP8 E4M3 conversions (gfx950 hardware converters), 16-byte vector packing,
// wavefront reductions, the RMSNorm of a row held by one workgroup, and the
// 1 x 128 block power-of-two (UE8M0) scale rule.
// Internal; included by the kernel translation units only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moef {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ bf16 helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 values -> one word of two bf16 (lo in bits 0..15), round to nearest
// even, by gfx950's packed converter (NaN stays a quiet NaN with its sign).
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ void unpack8(const u32x4 v, float x[8]) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// Eight fp32 values -> eight bf16 in one 16-byte vector (one rounding each).
__device__ __forceinline__ u32x4 pack8_rne(const float x[8]) {
  u32x4 v;
  v.x = bf16x2_rne(x[0], x[1]);
  v.y = bf16x2_rne(x[2], x[3]);
  v.z = bf16x2_rne(x[4], x[5]);
  v.w = bf16x2_rne(x[6], x[7]);
  return v;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_fadd(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                           false));
}

// Sum over the wave, uniform, in a fixed order and without LDS traffic: each
// 16-lane row by four DPP rotate-and-add steps, then row_bcast:15 and
// row_bcast:31 add the row sums into the last row, and lane 63 holds the
// total (the other rows are left partial and are not read).
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_fadd<0x128, 0xF>(v);   // row_ror:8
  v = dpp_fadd<0x124, 0xF>(v);   // row_ror:4
  v = dpp_fadd<0x122, 0xF>(v);   // row_ror:2
  v = dpp_fadd<0x121, 0xF>(v);   // row_ror:1
  v = dpp_fadd<0x142, 0xA>(v);   // row_bcast:15
  v = dpp_fadd<0x143, 0xC>(v);   // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// ------------------------------------------------ kernel argument loads

// Makes the compiler load a kernel argument no later than this point: left
// alone, it defers the load of an output pointer (or of a scalar used after a
// barrier) to its use, which puts one more dependent memory round trip at
// the end of a short kernel. The empty asm reads the value in scalar
// registers; it counts as a memory access, so callers place it after their
// last load (a load after it could no longer be a scalar load).
template <typename T>
__device__ __forceinline__ void load_now(T v) {
  asm volatile("" ::"s"(v));
}

// ------------------------------------------------ workgroup work counter

// The next unit of the calling wave from a workgroup's LDS counter (which
// starts at 0): lane 0 adds one and the old value is broadcast, so the
// result is wave-uniform. A loop around this fetch must not end its body
// with a store made by lane 0 alone: the optimizer can then send lanes
// 1..63 from that store straight back to the broadcast, which the compiled
// code turns into an inner loop they only leave once lane 0's (stale) value
// reaches the loop bound, and the wave never finishes. Callers bound their
// loop by the unit count and stop on any value outside [0, n).
// (ds_append would fetch without a lane-0 branch, but it takes the counter's
// address from the low 16 bits of M0, so it cannot reach a counter placed
// after 64 KiB of staging arrays.)
__device__ __forceinline__ int next_unit(int* counter) {
  int j = 0;
  if ((threadIdx.x & 63) == 0) j = atomicAdd(counter, 1);
  return __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(j, 0));
}

// ---------------------------------------------------- RMSNorm of one row
// One workgroup holds one row; lane t of it owns the 16-byte column vectors
// t + i * blockDim.x, i < CPT, so wave w's vector i is 512-column chunk
// w + i * (blockDim.x / 64).

// Records the sum of squares of vector i of every lane of this wave (one
// 512-column chunk) in partial[chunk]. Called once per vector, as soon as
// that vector's sum is known.
__device__ __forceinline__ void put_chunk_sum(float ss, int i, float* partial) {
  const float v = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) partial[(threadIdx.x >> 6) + i * (blockDim.x >> 6)] = v;
}

// 1 / sqrt(sum / hidden + eps) of the row, from the chunk sums put_chunk_sum
// recorded, added in chunk order, so the value does not depend on how many
// waves share the row. Every lane gets the same value. Contains the
// workgroup barrier that makes the chunk sums visible.
template <int CPT>
__device__ __forceinline__ float row_inv_rms(const float* partial, float inv_hidden, float eps) {
  __syncthreads();
  const int nchunks = (blockDim.x >> 6) * CPT;
  float tot = 0.0f;
  for (int c = 0; c < nchunks; ++c) tot = tot + partial[c];
  return rsqrtf(tot * inv_hidden + eps);
}

// normed = bf16((x * inv) * gamma) for the lane's CPT vectors of the row,
// x being the stored bf16 values (fp32 math); vectors past h8 are skipped.
template <int CPT>
__device__ __forceinline__ void store_normed(const float x[CPT][8], const u32x4 gv[CPT],
                                             float inv, int h8, u32x4* __restrict__ normed_row) {
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int colv = threadIdx.x + i * blockDim.x;
    if (colv < h8) {
      float g[8];
      unpack8(gv[i], g);
      float n[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) n[e] = (x[i][e] * inv) * g[e];
      __builtin_nontemporal_store(pack8_rne(n), normed_row + colv);
    }
  }
}

// ------------------------------------------- 1 x 128 block quantization

// max(v, the value DPP control `ctrl` moves into this lane). Lanes whose row
// `row_mask` leaves out get 0, the identity of an unsigned max, so they keep
// v; the compiler folds the move into one v_max_u32 with a DPP source.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false));
}

// Largest value across the 16 lanes of a DPP row (every lane gets it).
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = dpp_umax<0x128, 0xF>(v);   // row_ror:8
  v = dpp_umax<0x124, 0xF>(v);   // row_ror:4
  v = dpp_umax<0x122, 0xF>(v);   // row_ror:2
  v = dpp_umax<0x121, 0xF>(v);   // row_ror:1
  return v;
}

// Largest value across the wave, uniform. After the row maxima, row_bcast:15
// folds each row's lane 15 into the next row (rows 1 and 3) and row_bcast:31
// folds lane 31 into rows 2 and 3, so lane 63 holds the maximum of all four.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row16_max(v);
  v = dpp_umax<0x142, 0xA>(v);   // row_bcast:15
  v = dpp_umax<0x143, 0xC>(v);   // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Largest |y| of the eight bf16 values in v, as bf16 bits: with the sign
// cleared, bf16 bit patterns order like their magnitudes (NaN above inf).
__device__ __forceinline__ uint32_t absmax8_bits(const u32x4 v) {
  const u16x2 a = __builtin_elementwise_max(__builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu),
                                            __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu));
  const u16x2 b = __builtin_elementwise_max(__builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu),
                                            __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu));
  const u16x2 m = __builtin_elementwise_max(a, b);
  return m.x > m.y ? m.x : m.y;
}

// Least e with amax <= 448 * 2^e, clamped to [-127, 127], from the bf16 bits
// of amax >= 0. With amax = 2^E * 1.f and 448 = 2^8 * 1.75: e = E - 8, plus one
// when 1.f > 1.75 (7-bit fraction above 0x60). Zero and subnormal amax clamp to
// -127 (every subnormal is below 448 * 2^-127); inf / NaN give 127.
__device__ __forceinline__ int ue8m0_exponent(uint32_t amax_bf16) {
  const int ef = (int)(amax_bf16 >> 7);
  if (ef == 0) return -127;
  if (ef >= 255) return 127;
  const int e = ef - 135 + ((amax_bf16 & 0x7Fu) > 0x60u ? 1 : 0);
  return e < -127 ? -127 : e;
}

// 2^e as an fp32 scale operand; 2^-127 is the subnormal 0x00400000.
__device__ __forceinline__ float ue8m0_scale(int e) {
  return __uint_as_float(e > -127 ? (uint32_t)(e + 127) << 23 : 0x00400000u);
}

// Eight bf16 values y -> eight OCP E4M3 codes of y / 2^e (round to nearest
// even, subnormals and the sign of zero kept, beyond 448 / NaN -> NaN code),
// two per gfx950 scaled fp32 converter op, in column order. (The scale only
// ever is an exact power of two, so the division is exact.)
__device__ __forceinline__ u32x2 e4m3x8_scaled(const u32x4 y, float scale) {
  float f[8];
  unpack8(y, f);
  s16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((s16x2){0, 0}, f[0], f[1], scale, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, f[2], f[3], scale, true);
  s16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((s16x2){0, 0}, f[4], f[5], scale, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, f[6], f[7], scale, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}


}  // namespace dev
}  // namespace moef
