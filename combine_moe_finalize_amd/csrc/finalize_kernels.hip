// gfx950 kernels of the deferred MoE finalize.
//
// What they compute ("Support deferred MoE finalize for MXFP4 and FP8
// block-scale", Motivation and Modifications item 2; "[Kimi K2.5] Fuse
// deferred MoE finalize into next-layer AR + residual + RMSNorm", Key
// modifications and "Numerics & speed"): for every token t and column h,
//   acc = +0;  for k ascending: acc = acc + w'[t,k] * x[perm[t,k], h]
//   acc = acc + shared[t,h];  [acc = acc + residual[t,h]]
// with w' = fp32(w * routed_scaling_factor), every operation rounded to fp32
// (this file is built with fp-contract off: no fused multiply-add), then one
// round-to-nearest-even to bf16.
//
// Work decomposition. The path is a gather-reduce bound by HBM bandwidth, not
// a contraction, so there is no MFMA here. One wavefront owns one
// (token, 512-column chunk): each of its 64 lanes owns 8 consecutive bf16
// columns and moves them with one 16-byte load per gathered row. The token's
// top_k indices and weights are wave-uniform and land in scalar registers;
// the weight (times the routed scaling factor) stays in a register for the
// whole chunk. The shared / residual (and gamma) loads are issued first, since
// they do not depend on the routing, then all top_k row loads, all before the
// first add: a lane has up to (top_k + 2) x 16 bytes in flight.
// Gathered rows are read exactly once and outputs are written once, so both
// use non-temporal loads and stores (measured: the streaming stores alone take
// the prefill launch from 195 to 183 microseconds, kernel-trace medians).
//
// Epilogues:
//  * RMSNorm: one workgroup per token (up to 16 waves), the row stays in
//    registers; the sum of squares of each 512-column chunk by DPP row
//    reductions, then the chunk sums through LDS in chunk order, so every
//    lane sees the same value and the result does not depend on the
//    workgroup width. From 288 tokens on, a token takes half as many waves
//    with two column vectors per lane (measured faster there, slower at
//    decode sizes); larger grids stage whole tokens per CU
//    (finalize_rmsnorm_staged_kernel).
//  * UE8M0 quant: a 1 x 128 block is 16 lanes x 8 columns, one DPP row; its
//    absolute maximum is taken on bf16 bit patterns (packed 16-bit integer
//    max, then four DPP row rotations), the power-of-two exponent comes from
//    the maximum's bit fields, and gfx950's scaled fp32 converter divides each
//    value by 2^e and rounds it to OCP E4M3 (nearest even), one op per pair.
//  * bf16 rounding uses gfx950's packed fp32 -> bf16 converter (nearest even).
//    ("[FP8][MoE] Honor UE8M0 activation scales in Triton MoE", Motivation
//    and "More context".)

#include <atomic>

#include "device_common.h"
#include "moef_internal.h"

namespace moef {
namespace {

using namespace dev;


// Kernel-side view of one routed call.
struct GatherArgs {
  const u32x4* g2;        // gemm2_out as 16-byte vectors, row stride h8
  int32_t num_rows;       // <= 2^31 - 1: rows are named by int32 indices
  const int32_t* idx;     // [T, k]
  const uint32_t* w;      // [T, k] fp32 bits or packed words
  const u32x4* shared;    // [T, h8] or nullptr
  float rsf;
  int32_t packed;
  int32_t tokens;
  int32_t h8;             // hidden / 8
  int32_t k;
  int32_t nchunks;        // ceil(h8 / 64)
  int32_t* err;
};

// The one-wave-per-unit kernels take the routed call as separate parameters,
// ordered for kernel-argument preload: the first 14 dwords (the index and
// row pointers, the sizes that address them, rsf, then the shared and weight
// pointers) arrive in SGPRs at wave start, so the index load that opens the
// decode call's dependent chain waits for no kernel-argument load; the
// output, error-flag and format arguments, needed later, are loaded from
// memory meanwhile.
#define MOEF_ROUTED_PARAMS                                                            \
  const int32_t *r_idx, const u32x4 *r_g2, int32_t r_h8, int32_t r_k, int32_t r_rows,  \
      int32_t r_nchunks, int32_t r_tokens, float r_rsf, const u32x4 *r_shared,         \
      const uint32_t *r_w, int32_t r_packed, int32_t *r_err
#define MOEF_ROUTED_ARGS(a)                                                           \
  (a).idx, (a).g2, (a).h8, (a).k, (a).num_rows, (a).nchunks, (a).tokens, (a).rsf,     \
      (a).shared, (a).w, (a).packed, (a).err
#define MOEF_ROUTED_GATHER_ARGS                                                       \
  routed_args(r_idx, r_g2, r_h8, r_k, r_rows, r_nchunks, r_tokens, r_rsf, r_shared, r_w, \
              r_packed, r_err)

__device__ __forceinline__ GatherArgs routed_args(MOEF_ROUTED_PARAMS) {
  GatherArgs a;
  a.g2 = r_g2;
  a.num_rows = r_rows;
  a.idx = r_idx;
  a.w = r_w;
  a.shared = r_shared;
  a.rsf = r_rsf;
  a.packed = r_packed;
  a.tokens = r_tokens;
  a.h8 = r_h8;
  a.k = r_k;
  a.nchunks = r_nchunks;
  a.err = r_err;
  return a;
}

// (bf16 / E4M3 conversion and packing helpers: device_common.h)

// ------------------------------------------------------------- gather core

// A call's latency at decode sizes is a chain of dependent round trips, so
// the helpers below are called in an order that keeps it short: the
// routing-independent operands (shared, residual) first, then the token's
// row indices, then the row loads they address, and only then the weights,
// which the compiler can fetch while the rows are in flight. Nothing
// branches between the index load and the row loads, nor between the loads
// and the adds: a skipped slot loads zeros through an empty buffer range and
// adds -0 (an out-of-range index is reported after the store, by
// report_out_of_range).

// The token's gathered rows, or -1 where a slot is skipped: an index < 0
// names an expert that is not local, one >= num_rows is out of range (the
// return value says whether one was). Wave-uniform scalar loads.
template <int KMAX, bool EXACT>
__device__ __forceinline__ bool load_rows(const GatherArgs& a, int t, int32_t row[KMAX]) {
  const int64_t base = (int64_t)t * a.k;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    row[j] = -1;
    if (EXACT || j < a.k) row[j] = a.idx[base + j];
  }
  bool oob = false;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    oob = oob || row[j] >= a.num_rows;
    row[j] = row[j] >= a.num_rows ? -1 : row[j];
  }
  return oob;
}

// Word 3 of a gfx9-family buffer resource for untyped loads (32-bit data
// format, no swizzle, no index stride), and the non-temporal cache policy.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kBufferNonTemporal = 2;

// One 16-byte vector of gathered row `row` (wave-uniform) at column vector
// col < h8, non-temporal. The load goes through a buffer resource that spans
// exactly that row, or nothing when row < 0: the hardware's range check then
// returns zeros without a memory access, so a skipped slot costs no branch.
__device__ __forceinline__ u32x4 load_row_vector(const u32x4* g2, int32_t row, int32_t h8,
                                                 int64_t col) {
  const bool take = row >= 0;
  const u32x4* base = g2 + (int64_t)(take ? row : 0) * h8;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4*>(base), 0, take ? h8 * 16 : 0, kBufferWord3);
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)col * 16, 0, kBufferNonTemporal);
}

// The 16-byte vectors of the token's rows at column vector col, every load
// issued before any is used; zeros for a skipped slot.
template <int KMAX, bool EXACT>
__device__ __forceinline__ void load_gathers(const GatherArgs& a, int64_t col,
                                             const int32_t row[KMAX], u32x4 v[KMAX]) {
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    v[j] = load_row_vector(a.g2, (EXACT || j < a.k) ? row[j] : -1, a.h8, col);
}

// w' = fp32(w * rsf) per slot, from fp32 weights or the bf16 half of packed
// words, kept in registers. Wave-uniform scalar loads.
template <int KMAX, bool EXACT>
__device__ __forceinline__ void load_weights(const GatherArgs& a, int t, float w[KMAX]) {
  const int64_t base = (int64_t)t * a.k;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    uint32_t word = 0u;
    if (EXACT || j < a.k) word = a.w[base + j];
    w[j] = __uint_as_float(a.packed ? (word << 16) : word) * a.rsf;
  }
}

// Sets the caller's error flag if any slot of the wave's token was out of
// range (after the wave's stores, off the call's critical path).
__device__ __forceinline__ void report_out_of_range(const GatherArgs& a, bool oob) {
  if (oob && a.err != nullptr && (threadIdx.x & 63) == 0)
    atomicOr(a.err, MOEF_DEVERR_INDEX_OUT_OF_RANGE);
}

// The operands of one column vector that do not depend on the routing: the
// shared-expert and residual vectors. They are issued before the token's
// indices arrive, so their latency overlaps the index fetch.
struct Side {
  u32x4 s;
  u32x4 r;
};

__device__ __forceinline__ Side load_side(const GatherArgs& a, int t, int64_t col,
                                          const u32x4* residual_row) {
  Side d;
  d.s = u32x4{0u, 0u, 0u, 0u};
  d.r = u32x4{0u, 0u, 0u, 0u};
  if (a.shared != nullptr) d.s = __builtin_nontemporal_load(a.shared + (int64_t)t * a.h8 + col);
  if (residual_row != nullptr) d.r = __builtin_nontemporal_load(residual_row + col);
  return d;
}

// acc[0..7] for columns [8*col, 8*col + 8): the weighted sum of the gathered
// rows in slot order, then + shared, then + residual (when given), each step
// in fp32. A skipped slot's vector is zeros (load_gathers) and its weight is
// taken as -0, so its product is -0 and acc + (-0) == acc for every acc,
// +0 and -0 included: the sum over the taken slots, with no branch.
template <int KMAX, bool EXACT>
__device__ __forceinline__ void reduce_rows(const GatherArgs& a, const int32_t row[KMAX],
                                            const u32x4 v[KMAX], const float w[KMAX],
                                            const Side& d, bool has_residual, float acc[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const float wj = ((EXACT || j < a.k) && row[j] >= 0) ? w[j] : -0.0f;
    float x[8];
    unpack8(v[j], x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + wj * x[e];
  }
  if (a.shared != nullptr) {
    float x[8];
    unpack8(d.s, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
  }
  if (has_residual) {
    float x[8];
    unpack8(d.r, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
  }
}

// One column vector's gather in flight: the token's rows, their loaded
// vectors, the weights, and whether a slot was out of range.
template <int KMAX>
struct Gathered {
  int32_t row[KMAX];
  u32x4 v[KMAX];
  float w[KMAX];
  bool oob;
};

// Issues the loads of one column vector of token t: row indices, then the
// row loads, then the weights (the order above).
template <int KMAX, bool EXACT>
__device__ __forceinline__ void issue_gather(const GatherArgs& a, int t, int64_t col,
                                             Gathered<KMAX>& g) {
  g.oob = load_rows<KMAX, EXACT>(a, t, g.row);
  load_gathers<KMAX, EXACT>(a, col, g.row, g.v);
  load_weights<KMAX, EXACT>(a, t, g.w);
}

// The finalize of one column vector of token t. Returns whether a slot was
// out of range.
template <int KMAX, bool EXACT>
__device__ __forceinline__ bool finalize_vector(const GatherArgs& a, int t, int64_t col,
                                                const Side& d, bool has_residual, float acc[8]) {
  Gathered<KMAX> g;
  issue_gather<KMAX, EXACT>(a, t, col, g);
  reduce_rows<KMAX, EXACT>(a, g.row, g.v, g.w, d, has_residual, acc);
  return g.oob;
}

// ------------------------------------------------------------------ plain

template <int KMAX, bool EXACT>
__global__ void __launch_bounds__(kWavesPerBlock * kWaveLanes)
finalize_kernel(MOEF_ROUTED_PARAMS, u32x4* __restrict__ out) {
  const GatherArgs a = MOEF_ROUTED_GATHER_ARGS;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  // Waves past the last unit (the grid's last workgroup) redo the last unit
  // and store nothing, instead of returning early: no branch then stands
  // between the kernel's first argument loads and the rest of them.
  const int units = a.tokens * a.nchunks;
  const bool live = (int)blockIdx.x * kWavesPerBlock + wave < units;
  const int unit = live ? (int)blockIdx.x * kWavesPerBlock + wave : units - 1;
  const int t = unit / a.nchunks;
  const int colv = (unit - t * a.nchunks) * kWaveLanes + lane;
  const bool active = colv < a.h8;
  const int64_t col = active ? colv : a.h8 - 1;   // keep every lane's loads in bounds

  const Side d = load_side(a, t, col, nullptr);
  Gathered<KMAX> g;
  issue_gather<KMAX, EXACT>(a, t, col, g);
  load_now(out);           // after every load: the asm counts as a memory access
  load_now(a.err);
  float acc[8];
  reduce_rows<KMAX, EXACT>(a, g.row, g.v, g.w, d, false, acc);
  const bool oob = g.oob;

  if (live && active) __builtin_nontemporal_store(pack8_rne(acc), out + (int64_t)t * a.h8 + colv);
  report_out_of_range(a, oob);
}

// ------------------------------------------------------- residual + RMSNorm

template <int KMAX, bool EXACT, int CPT>
__global__ void __launch_bounds__(kNormMaxThreads)
finalize_rmsnorm_kernel(MOEF_ROUTED_PARAMS, const u32x4* residual,
                        const u32x4* __restrict__ gamma, float eps, float inv_hidden,
                        u32x4* residual_out, u32x4* __restrict__ normed) {
  const GatherArgs a = MOEF_ROUTED_GATHER_ARGS;
  __shared__ float partial[kNormMaxChunks];
  const int t = blockIdx.x;
  const int nthreads = blockDim.x;

  const u32x4* res_row = residual + (int64_t)t * a.h8;
  // row-independent operands first: shared, residual and gamma vectors
  Side d[CPT];
  u32x4 gv[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int colv = threadIdx.x + i * nthreads;
    const int64_t col = colv < a.h8 ? colv : a.h8 - 1;
    d[i] = load_side(a, t, col, res_row);
    gv[i] = gamma[col];
  }
  int32_t row[KMAX];
  const bool oob = load_rows<KMAX, EXACT>(a, t, row);
  float w[KMAX];

  float ro[CPT][8];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int colv = threadIdx.x + i * nthreads;
    const bool active = colv < a.h8;
    const int64_t col = active ? colv : a.h8 - 1;
    u32x4 v[KMAX];
    load_gathers<KMAX, EXACT>(a, col, row, v);
    if (i == 0) {
      load_weights<KMAX, EXACT>(a, t, w);
      load_now(residual_out);  // after the loads: the asm counts as a memory access
      load_now(normed);
      load_now(eps);
      load_now(inv_hidden);
      load_now(a.err);
      load_now((int)blockDim.x);
    }
    float acc[8];
    reduce_rows<KMAX, EXACT>(a, row, v, w, d[i], true, acc);
    const u32x4 rb = pack8_rne(acc);
    unpack8(rb, ro[i]);                     // the stored bf16 residual_out
    float ss = 0.0f;
    if (active) {
      __builtin_nontemporal_store(rb, residual_out + (int64_t)t * a.h8 + colv);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = ss + ro[i][e] * ro[i][e];
    }
    put_chunk_sum(ss, i, partial);
  }
  const float inv = row_inv_rms<CPT>(partial, inv_hidden, eps);
  store_normed<CPT>(ro, gv, inv, a.h8, normed + (int64_t)t * a.h8);
  report_out_of_range(a, oob);
}

// ------------------------------------- residual + RMSNorm, staged output

// finalize_rmsnorm_kernel's result for large grids, with every write after
// the workgroup's gathers (the scheme of finalize_quant_staged_kernel below).
// One workgroup per CU owns whole tokens t0 + b + i * gridDim.x, i < ntok,
// and its waves take the (token, chunk) units j = i * nchunks + c from the
// LDS counter. Unit j leaves its residual_out vector (1 KiB of bf16) in LDS
// slot j and its sum of squares, reduced over the wave exactly as the
// one-workgroup-per-token kernel reduces a chunk, in sumsq[j]. After the
// last gather each token's 1 / rms is formed from its chunk sums added in
// chunk order, as row_inv_rms does, so the two kernels give bit-identical
// results; then the workgroup writes residual_out and normed. A token's
// residual is read only by the workgroup that writes its residual_out, and
// before it does, so residual_out may alias residual. The host sizes
// launches so that ntok * nchunks <= kStageRmsUnits.
template <int KMAX, bool EXACT>
__global__ void __launch_bounds__(kStageThreads)
finalize_rmsnorm_staged_kernel(GatherArgs a, const u32x4* residual,
                               const u32x4* __restrict__ gamma, float eps, float inv_hidden,
                               u32x4* residual_out, u32x4* __restrict__ normed, int t0, int t1) {
  __shared__ u32x4 stage_r[kStageRmsUnits * kWaveLanes];
  __shared__ float sumsq[kStageRmsUnits];
  __shared__ float inv_rms[kStageRmsUnits];     // per token
  __shared__ int next_j;
  const int nb = (int)gridDim.x;
  const int b = (int)blockIdx.x;
  const int nch = a.nchunks;
  int ntok = t1 - t0 > b ? (t1 - t0 - b + nb - 1) / nb : 0;
  if (ntok > kStageRmsUnits / nch) ntok = kStageRmsUnits / nch;   // launches are sized below it
  const int n = ntok * nch;
  const int lane = threadIdx.x & 63;
  bool oob = false;
  if (threadIdx.x == 0) next_j = 0;
  __syncthreads();

  for (int it = 0; it < n; ++it) {
    const int j = next_unit(&next_j);
    if ((unsigned)j >= (unsigned)n) break;
    const int i = j / nch;
    const int t = t0 + b + i * nb;
    const int colv = (j - i * nch) * kWaveLanes + lane;
    const bool active = colv < a.h8;
    const int64_t col = active ? colv : a.h8 - 1;

    const Side d = load_side(a, t, col, residual + (int64_t)t * a.h8);
    float acc[8];
    oob = finalize_vector<KMAX, EXACT>(a, t, col, d, true, acc) || oob;
    const u32x4 rb = pack8_rne(acc);
    float ro[8];
    unpack8(rb, ro);
    float ss = 0.0f;
    if (active) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = ss + ro[e] * ro[e];
    }
    const float chunk_sum = wave_sum(ss);
    stage_r[j * kWaveLanes + lane] = rb;
    sumsq[j] = chunk_sum;                   // every lane stores the same value
  }
  __syncthreads();         // every unit of the workgroup is staged

  for (int i = threadIdx.x; i < ntok; i += kStageThreads) {
    float tot = 0.0f;
    for (int c = 0; c < nch; ++c) tot = tot + sumsq[i * nch + c];
    inv_rms[i] = rsqrtf(tot * inv_hidden + eps);
  }
  __syncthreads();

  for (int x = threadIdx.x; x < n * kWaveLanes; x += kStageThreads) {
    const int j = x / kWaveLanes;
    const int i = j / nch;
    const int colv = (j - i * nch) * kWaveLanes + (x - j * kWaveLanes);
    if (colv < a.h8) {
      const int64_t o = (int64_t)(t0 + b + i * nb) * a.h8 + colv;
      const u32x4 rb = stage_r[x];
      __builtin_nontemporal_store(rb, residual_out + o);
      float xv[8], g[8], nv[8];
      unpack8(rb, xv);
      unpack8(gamma[colv], g);
      const float inv = inv_rms[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) nv[e] = (xv[e] * inv) * g[e];
      __builtin_nontemporal_store(pack8_rne(nv), normed + o);
    }
  }
  report_out_of_range(a, oob);
}

// ------------------------------------------------------- UE8M0 / E4M3 quant

template <int KMAX, bool EXACT>
__global__ void __launch_bounds__(kWavesPerBlock * kWaveLanes)
finalize_quant_kernel(MOEF_ROUTED_PARAMS, u32x2* __restrict__ out_q,
                      uint8_t* __restrict__ scale) {
  const GatherArgs a = MOEF_ROUTED_GATHER_ARGS;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  // as finalize_kernel: waves past the last unit redo it and store nothing
  const int units = a.tokens * a.nchunks;
  const bool live = (int)blockIdx.x * kWavesPerBlock + wave < units;
  const int unit = live ? (int)blockIdx.x * kWavesPerBlock + wave : units - 1;
  const int t = unit / a.nchunks;
  const int colv = (unit - t * a.nchunks) * kWaveLanes + lane;
  const bool active = live && colv < a.h8;   // h8 % 16 == 0: whole DPP rows agree
  const int64_t col = colv < a.h8 ? colv : a.h8 - 1;

  const Side d = load_side(a, t, col, nullptr);
  Gathered<KMAX> g;
  issue_gather<KMAX, EXACT>(a, t, col, g);
  load_now(out_q);         // after every load: the asm counts as a memory access
  load_now(scale);
  load_now(a.err);
  float acc[8];
  reduce_rows<KMAX, EXACT>(a, g.row, g.v, g.w, d, false, acc);
  const bool oob = g.oob;

  const u32x4 y = pack8_rne(acc);                    // the bf16 finalize result
  const uint32_t amax = row16_max(active ? absmax8_bits(y) : 0u);
  const int ex = ue8m0_exponent(amax);
  const u32x2 q = e4m3x8_scaled(y, ue8m0_scale(ex));
  if (active) {
    __builtin_nontemporal_store(q, out_q + (int64_t)t * a.h8 + colv);
    if ((lane & 15) == 0) scale[(int64_t)t * (a.h8 >> 4) + (colv >> 4)] = (uint8_t)(ex + 127);
  }
  report_out_of_range(a, oob);
}

// ------------------------------------- UE8M0 / E4M3 quant, staged output

// Where the staged quant kernel's units go. A launch covers the tokens
// [t0, t1); its workgroups form g groups of wpx = gridDim.x / g, group x
// being the workgroups b with b % g == x, which the dispatcher places on one
// XCD (workgroups go to the XCDs round-robin). Tokens are dealt to the
// groups in blocks of kXcdTokenBlock (block m to group m % g) for as many
// full rounds of g blocks as the launch holds, and the remaining tokens one
// by one (token r of the rest to group r % g), so no group holds more than
// ceil((t1 - t0) / g) tokens. Within its group, workgroup w = b / g takes the
// group's units lu = w + j * wpx, j = 0, 1, ..., unit lu being chunk
// lu % nchunks of the group's token lu / nchunks. All chunks of a token, and
// so all the scale bytes of a block of 16 tokens (at H = 7168, 896 bytes:
// seven whole 128-byte lines), are written through one XCD's L2, which
// merges them into whole lines.
struct TokenGroups {
  int t0;      // first token of the launch
  int g;       // groups
  int x;       // this workgroup's group
  int full;    // full rounds of g blocks
};

// Token of the group-local token index lt.
__device__ __forceinline__ int group_token(const TokenGroups& p, int lt) {
  const int in_full = p.full * kXcdTokenBlock;
  return lt < in_full
             ? p.t0 + ((lt / kXcdTokenBlock) * p.g + p.x) * kXcdTokenBlock + lt % kXcdTokenBlock
             : p.t0 + in_full * p.g + p.x + (lt - in_full) * p.g;
}

// The quantized output of one unit: the bf16 finalize result y of the
// lane's 8 columns, its 1 x 128 block's UE8M0 exponent (one DPP row holds a
// block) and the E4M3 codes of y / 2^e.
__device__ __forceinline__ u32x2 quant_unit(const float acc[8], bool active, int& ex) {
  const u32x4 y = pack8_rne(acc);
  const uint32_t amax = row16_max(active ? absmax8_bits(y) : 0u);
  ex = ue8m0_exponent(amax);
  return e4m3x8_scaled(y, ue8m0_scale(ex));
}

// The same result as finalize_quant_kernel, for large grids. The quant
// output is 5% of the launch's bytes, but written in the middle of the
// gathers it costs about 15% of the time: the DRAM turns between reads and
// writes all through the launch. Here every write waits until the reads are
// done. The first `staged` workgroups (one per CU, kStageThreads lanes each)
// own a CU's whole LDS and process their units (placed as TokenGroups says,
// over staged / groups workgroups per group) in order j = 0, 1, ...: their
// waves take the next j from an LDS counter (so a workgroup's waves finish
// together), keep the E4M3 codes and scale bytes of unit j in LDS slot j
// (j < kStageUnits) or, beyond that, in one of R register slots of the wave,
// and only after the workgroup's last gather write them all (the workgroup
// barrier also keeps the compiler from moving any store up into the gather
// loop). The launch start aligns the read phases of all CUs, so the chip's
// writes come in the last stretch of the launch, while the slowest CUs
// finish reading, instead of all through it. (No grid-wide barrier: each
// workgroup only writes its own units.)
// The last tail_percent of each group's units go to the workgroups after
// the staged ones, kStageWaves units each (one per wave, written at
// once). Each needs a whole CU's LDS too, so the dispatcher starts them on
// the CUs whose staged workgroup finished first, which evens out the ends of
// the CUs' read phases; tail workgroup b goes to the XCD of group
// (b - staged) % groups, as its group's staged workgroups do.
// The host sizes a launch so that every staged workgroup's units fit,
// n <= kStageUnits + kStageWaves * R; a unit that still found no slot would
// be written at once, so no sizing can drop one.
template <int KMAX, bool EXACT, int R>
__global__ void __launch_bounds__(kStageThreads)
finalize_quant_staged_kernel(GatherArgs a, u32x2* __restrict__ out_q,
                             uint8_t* __restrict__ scale, int t0, int t1, int groups,
                             int staged, int tail_percent) {
  __shared__ u32x2 stage_q[kStageUnits * kWaveLanes];
  __shared__ uint32_t stage_e[kStageUnits];     // four scale bytes per unit
  __shared__ int next_j;
  constexpr int RS = R > 0 ? R : 1;
  const int b = (int)blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wpx = staged / groups;
  const bool tail_wg = b >= staged;
  TokenGroups p;
  p.t0 = t0;
  p.g = groups;
  p.x = (tail_wg ? b - staged : b) % groups;
  p.full = (t1 - t0) / (groups * kXcdTokenBlock);
  const int rest = (t1 - t0) - p.full * groups * kXcdTokenBlock;
  const int group_tokens = p.full * kXcdTokenBlock + (rest > p.x ? (rest - p.x + groups - 1) / groups : 0);
  const int group_units = group_tokens * a.nchunks;
  const int static_units = group_units - group_units * tail_percent / 100;

  if (tail_wg) {                         // one unit per wave, written at once
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lu = static_units + ((b - staged) / groups) * kStageWaves + wave;
    if (lu >= group_units) return;
    const int lt = lu / a.nchunks;
    const int t = group_token(p, lt);
    const int colv = (lu - lt * a.nchunks) * kWaveLanes + lane;
    const bool active = colv < a.h8;
    const int64_t col = active ? colv : a.h8 - 1;
    const Side d = load_side(a, t, col, nullptr);
    float acc[8];
    const bool oob = finalize_vector<KMAX, EXACT>(a, t, col, d, false, acc);
    int ex;
    const u32x2 q = quant_unit(acc, active, ex);
    if (active) {
      __builtin_nontemporal_store(q, out_q + (int64_t)t * a.h8 + colv);
      if ((lane & 15) == 0) scale[(int64_t)t * (a.h8 >> 4) + (colv >> 4)] = (uint8_t)(ex + 127);
    }
    report_out_of_range(a, oob);
    return;
  }

  const int w = b / groups;
  const int n = static_units > w ? (static_units - w + wpx - 1) / wpx : 0;   // this workgroup's units
  const int nl = n < kStageUnits ? n : kStageUnits;                         // of them staged in LDS
  if (threadIdx.x == 0) next_j = 0;
  __syncthreads();

  u32x2 rq[RS];            // register slots: codes, scale byte, group-local unit
  uint32_t re[RS];
  int ru[RS];
  int cnt = 0;             // register slots in use (wave-uniform)
  bool oob = false;        // a slot of one of the wave's tokens was out of range
  for (int it = 0; it < n; ++it) {
    const int j = next_unit(&next_j);
    if ((unsigned)j >= (unsigned)n) break;
    const int lu = w + j * wpx;
    const int lt = lu / a.nchunks;
    const int t = group_token(p, lt);
    const int colv = (lu - lt * a.nchunks) * kWaveLanes + lane;
    const bool active = colv < a.h8;
    const int64_t col = active ? colv : a.h8 - 1;

    const Side d = load_side(a, t, col, nullptr);
    float acc[8];
    oob = finalize_vector<KMAX, EXACT>(a, t, col, d, false, acc) || oob;
    int ex;
    const u32x2 q = quant_unit(acc, active, ex);
    if (j < nl) {
      stage_q[j * kWaveLanes + lane] = q;
      if ((lane & 15) == 0) reinterpret_cast<uint8_t*>(&stage_e[j])[lane >> 4] = (uint8_t)(ex + 127);
    } else if (R > 0 && cnt < R) {
#pragma unroll
      for (int s = 0; s < RS; ++s)
        if (cnt == s) {
          rq[s] = q;
          re[s] = (uint32_t)(ex + 127);
          ru[s] = lu;
        }
      ++cnt;
    } else if (active) {
      // No slot left (the host sizes launches so that this is not reached):
      // write now, as the one-wave-per-unit kernel does, so that no unit is
      // ever dropped whatever the sizing.
      __builtin_nontemporal_store(q, out_q + (int64_t)t * a.h8 + colv);
      if ((lane & 15) == 0) scale[(int64_t)t * (a.h8 >> 4) + (colv >> 4)] = (uint8_t)(ex + 127);
    }
  }
  __syncthreads();         // every unit of the workgroup is staged or written

#pragma unroll
  for (int s = 0; s < RS; ++s) {
    if (R > 0 && s < cnt) {
      const int lt = ru[s] / a.nchunks;
      const int t = group_token(p, lt);
      const int colv = (ru[s] - lt * a.nchunks) * kWaveLanes + lane;
      if (colv < a.h8) {
        __builtin_nontemporal_store(rq[s], out_q + (int64_t)t * a.h8 + colv);
        if ((lane & 15) == 0) scale[(int64_t)t * (a.h8 >> 4) + (colv >> 4)] = (uint8_t)re[s];
      }
    }
  }
  for (int x = threadIdx.x; x < nl * kWaveLanes; x += kStageThreads) {
    const int j = x / kWaveLanes;
    const int l = x - j * kWaveLanes;
    const int lu = w + j * wpx;
    const int lt = lu / a.nchunks;
    const int t = group_token(p, lt);
    const int colv = (lu - lt * a.nchunks) * kWaveLanes + l;
    if (colv < a.h8) {
      __builtin_nontemporal_store(stage_q[x], out_q + (int64_t)t * a.h8 + colv);
      if ((l & 15) == 0)
        scale[(int64_t)t * (a.h8 >> 4) + (colv >> 4)] =
            reinterpret_cast<const uint8_t*>(&stage_e[j])[l >> 4];
    }
  }
  report_out_of_range(a, oob);
}

// ---------------------------------------------- plain finalize, staged output

// finalize_kernel's result through the staging scheme of
// finalize_quant_staged_kernel above (one workgroup per CU, units
// u0 + b + j * gridDim.x taken from an LDS counter, writes after the
// workgroup's last gather). A unit's output is its 1 KiB of bf16: LDS holds
// kStagePlainUnits of them, each of the WAVES waves R more in registers. The
// output is 10% of the plain finalize's bytes (k = 8), so keeping it out of
// the read phase gains more than for the quant output. With 12 waves a wave
// may use up to 168 VGPRs (3 waves per SIMD), room for 25 register slots:
// 159 + 12 * 25 = 459 units per CU hold a 8192-token, H = 7168 call (448
// units per CU) in one launch.
template <int KMAX, bool EXACT, int R, int WAVES>
__global__ void __launch_bounds__(WAVES * kWaveLanes)
finalize_staged_kernel(GatherArgs a, u32x4* __restrict__ out, int u0, int u1) {
  __shared__ u32x4 stage_o[kStagePlainUnits * kWaveLanes];
  __shared__ int next_j;
  constexpr int RS = R > 0 ? R : 1;
  const int nb = (int)gridDim.x;
  const int b = (int)blockIdx.x;
  const int n = u1 - u0 > b ? (u1 - u0 - b + nb - 1) / nb : 0;       // this workgroup's units
  const int nl = n < kStagePlainUnits ? n : kStagePlainUnits;         // of them staged in LDS
  const int lane = threadIdx.x & 63;
  if (threadIdx.x == 0) next_j = 0;
  __syncthreads();

  u32x4 ro[RS];            // register slots: bf16 output vector, unit index
  int ru[RS];
  int cnt = 0;             // register slots in use (wave-uniform)
  bool oob = false;        // a slot of one of the wave's tokens was out of range
  for (int it = 0; it < n; ++it) {
    const int j = next_unit(&next_j);
    if ((unsigned)j >= (unsigned)n) break;
    const int unit = u0 + b + j * nb;
    const int t = unit / a.nchunks;
    const int colv = (unit - t * a.nchunks) * kWaveLanes + lane;
    const int64_t col = colv < a.h8 ? colv : a.h8 - 1;

    const Side d = load_side(a, t, col, nullptr);
    float acc[8];
    oob = finalize_vector<KMAX, EXACT>(a, t, col, d, false, acc) || oob;
    const u32x4 y = pack8_rne(acc);
    if (j < nl) stage_o[j * kWaveLanes + lane] = y;
    // Past the LDS slots, slot 0 of the registers takes the unit and the
    // others move down one; a branch-free select, top slot first, so the
    // update needs no second copy of the slots.
    const bool take = R > 0 && j >= nl && cnt < R;
#pragma unroll
    for (int s = RS - 1; s > 0; --s) {
      ro[s] = take ? ro[s - 1] : ro[s];
      ru[s] = take ? ru[s - 1] : ru[s];
    }
    ro[0] = take ? y : ro[0];
    ru[0] = take ? unit : ru[0];
    cnt += take ? 1 : 0;
    if (j >= nl && !take && colv < a.h8)
      __builtin_nontemporal_store(y, out + (int64_t)t * a.h8 + colv);   // no slot left
  }
  __syncthreads();         // every unit of the workgroup is staged or written

#pragma unroll
  for (int s = 0; s < RS; ++s) {
    if (R > 0 && s < cnt) {
      const int t = ru[s] / a.nchunks;
      const int colv = (ru[s] - t * a.nchunks) * kWaveLanes + lane;
      if (colv < a.h8) __builtin_nontemporal_store(ro[s], out + (int64_t)t * a.h8 + colv);
    }
  }
  for (int x = threadIdx.x; x < nl * kWaveLanes; x += WAVES * kWaveLanes) {
    const int j = x / kWaveLanes;
    const int l = x - j * kWaveLanes;
    const int unit = u0 + b + j * nb;
    const int t = unit / a.nchunks;
    const int colv = (unit - t * a.nchunks) * kWaveLanes + l;
    if (colv < a.h8) __builtin_nontemporal_store(stage_o[x], out + (int64_t)t * a.h8 + colv);
  }
  report_out_of_range(a, oob);
}

// ------------------------------------------------------------ packed decode

// (expert_id << 16) | bf16(weight) -> id (logical shift) and exact fp32 weight.
// ("[Deepseek V4] Keep fp32 routing weights in the mxfp4 trtllm MoE", PR
// description.)
__global__ void __launch_bounds__(256)
packed_decode_kernel(const uint32_t* __restrict__ packed, int64_t n,
                     int32_t* __restrict__ ids, float* __restrict__ w) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint32_t word = packed[i];
  if (ids != nullptr) ids[i] = (int32_t)(word >> 16);
  if (w != nullptr) w[i] = __uint_as_float(word << 16);
}

// ------------------------------------------------- expert-parallel combine

// out = bf16(sum_r partial_r + shared): with experts sharded over R ranks,
// each rank finalizes only its own slots (the others carry index -1) and no
// shared output; the shared expert is added once, here. fp32 adds in rank
// order, one rounding. Loads are issued four ranks at a time.
__global__ void __launch_bounds__(256)
ep_combine_kernel(const u32x4* __restrict__ partials, int R, int64_t stride,
                  const u32x4* __restrict__ shared, u32x4* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  int r = 0;
  for (; r + 4 <= R; r += 4) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(partials + (r + j) * stride + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x[8];
      unpack8(v[j], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
    }
  }
  for (; r < R; ++r) {
    float x[8];
    unpack8(__builtin_nontemporal_load(partials + r * stride + i), x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
  }
  if (shared != nullptr) {
    float x[8];
    unpack8(__builtin_nontemporal_load(shared + i), x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
  }
  __builtin_nontemporal_store(pack8_rne(acc), out + i);
}

// ---------------------------------------------------------------- dispatch

template <int V>
using IC = std::integral_constant<int, V>;

// Exact instantiations for the common top_k, guarded ones otherwise.
template <typename F>
hipError_t dispatch_top_k(int k, F&& f) {
  switch (k) {
    case 1: return f(IC<1>{}, std::true_type{});
    case 2: return f(IC<2>{}, std::true_type{});
    case 4: return f(IC<4>{}, std::true_type{});
    case 6: return f(IC<6>{}, std::true_type{});
    case 8: return f(IC<8>{}, std::true_type{});
    default:
      if (k <= 4) return f(IC<4>{}, std::false_type{});
      if (k <= 8) return f(IC<8>{}, std::false_type{});
      return f(IC<16>{}, std::false_type{});
  }
}

GatherArgs make_args(const Routed& r) {
  GatherArgs a;
  a.g2 = reinterpret_cast<const u32x4*>(r.gemm2_out);
  a.num_rows = (int32_t)r.num_rows;       // validated <= INT32_MAX
  a.idx = r.idx;
  a.w = r.weights;
  a.shared = reinterpret_cast<const u32x4*>(r.shared);
  a.rsf = r.rsf;
  a.packed = r.packed ? 1 : 0;
  a.tokens = (int32_t)r.tokens;
  a.h8 = (int32_t)(r.hidden / kVecElems);
  a.k = r.top_k;
  a.nchunks = (a.h8 + kWaveLanes - 1) / kWaveLanes;
  a.err = r.err_flag;
  return a;
}

unsigned int plain_blocks(const GatherArgs& a) {
  const int64_t units = (int64_t)a.tokens * a.nchunks;
  return (unsigned int)((units + kWavesPerBlock - 1) / kWavesPerBlock);
}

}  // namespace

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_cus[kMaxDevices];

// Splits the grid's units into as few launches as hold every unit (a
// workgroup holds at most lds_units + reg_capacity of them; see plan_staged)
// and calls launch(u0, u1, registers) for each; `registers` says whether a
// workgroup's units can exceed lds_units (it then needs the kernel with
// register slots).
template <typename F>
hipError_t staged_launches(const GatherArgs& a, int ncu, int lds_units, int reg_capacity,
                           F&& launch) {
  const int64_t units = (int64_t)a.tokens * a.nchunks;
  const StagedPlan plan = plan_staged(units, ncu, lds_units + reg_capacity);
  const int64_t per_launch = plan.per_launch;
  for (int64_t u0 = 0; u0 < units; u0 += per_launch) {
    const int64_t u1 = u0 + per_launch < units ? u0 + per_launch : units;
    const int64_t per_wg = (u1 - u0 + ncu - 1) / ncu;
    launch((int)u0, (int)u1, per_wg > lds_units);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int KM, bool EX>
hipError_t launch_quant_staged(const GatherArgs& a, u32x2* q, uint8_t* scale, int ncu,
                               const StagedPlan& plan, int groups, hipStream_t stream) {
  for (int64_t t0 = 0; t0 < a.tokens; t0 += plan.per_launch) {
    const int64_t t1 = t0 + plan.per_launch < a.tokens ? t0 + plan.per_launch : a.tokens;
    const bool regs = quant_launch_regs(t1 - t0, a.nchunks, ncu, groups);
    const int pct = quant_launch_tail_percent(t1 - t0, a.nchunks, ncu);
    const dim3 grid((unsigned)(ncu + quant_launch_tail_workgroups(t1 - t0, a.nchunks, groups, pct)));
    if (regs)
      hipLaunchKernelGGL((finalize_quant_staged_kernel<KM, EX, kStageRegUnits>), grid,
                         dim3(kStageThreads), 0, stream, a, q, scale, (int)t0, (int)t1, groups,
                         ncu, pct);
    else
      hipLaunchKernelGGL((finalize_quant_staged_kernel<KM, EX, 0>), grid, dim3(kStageThreads), 0,
                         stream, a, q, scale, (int)t0, (int)t1, groups, ncu, pct);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int KM, bool EX>
hipError_t launch_plain_staged(const GatherArgs& a, u32x4* o, int ncu, const PlainChoice& c,
                               hipStream_t stream) {
  if (!c.wide)
    return staged_launches(a, ncu, kStagePlainUnits, kStagePlainWaves * kStagePlainRegUnits,
                           [&](int u0, int u1, bool regs) {
      if (regs)
        hipLaunchKernelGGL((finalize_staged_kernel<KM, EX, kStagePlainRegUnits, kStagePlainWaves>),
                           dim3(ncu), dim3(kStagePlainWaves * kWaveLanes), 0, stream, a, o, u0,
                           u1);
      else
        hipLaunchKernelGGL((finalize_staged_kernel<KM, EX, 0, kStagePlainWaves>), dim3(ncu),
                           dim3(kStagePlainWaves * kWaveLanes), 0, stream, a, o, u0, u1);
    });
  constexpr int W = kStagePlainWideWaves;
  constexpr int R = kStagePlainWideRegUnits;
  return staged_launches(a, ncu, kStagePlainUnits, W * R, [&](int u0, int u1, bool regs) {
    if (regs)
      hipLaunchKernelGGL((finalize_staged_kernel<KM, EX, R, W>), dim3(ncu), dim3(W * kWaveLanes),
                         0, stream, a, o, u0, u1);
    else
      hipLaunchKernelGGL((finalize_staged_kernel<KM, EX, 0, W>), dim3(ncu), dim3(W * kWaveLanes),
                         0, stream, a, o, u0, u1);
  });
}

}  // namespace

// The count of each device is queried once and kept: it sizes the staged
// kernels' grids. A failed query leaves no error behind for the launch
// checks that follow (they read hipGetLastError).
int device_cus(hipStream_t stream) {
  int dev = -1;
  if (stream == nullptr || hipStreamGetDevice(stream, &dev) != hipSuccess) {
    if (stream != nullptr) (void)hipGetLastError();
    if (hipGetDevice(&dev) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
  }
  if (dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int known = g_device_cus[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
  }
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev < kMaxDevices && ncu > 0) g_device_cus[dev].store(ncu, std::memory_order_relaxed);
  return ncu;
}

hipError_t launch_finalize(const Routed& r, uint16_t* out, hipStream_t stream) {
  const GatherArgs a = make_args(r);
  u32x4* o = reinterpret_cast<u32x4*>(out);
  const int ncu = a.k <= kStagedMaxTopK ? device_cus(stream) : 0;
  const PlainChoice c = plain_choice(a.tokens, r.hidden, a.k, ncu);
  if (c.staged) {
    return dispatch_top_k(a.k, [&](auto km, auto ex) {
      constexpr int KM = decltype(km)::value;
      constexpr bool EX = decltype(ex)::value;
      if constexpr (KM <= kStagedMaxTopK)
        return launch_plain_staged<KM, EX>(a, o, ncu, c, stream);
      else
        return hipErrorInvalidValue;   // not reached: top_k <= 8 dispatches KM <= 8
    });
  }
  const size_t lds = stream_cap_lds((int64_t)a.tokens * a.nchunks);
  return dispatch_top_k(a.k, [&](auto km, auto ex) {
    constexpr int KM = decltype(km)::value;
    constexpr bool EX = decltype(ex)::value;
    hipLaunchKernelGGL((finalize_kernel<KM, EX>), dim3(plain_blocks(a)),
                       dim3(kWavesPerBlock * kWaveLanes), lds, stream, MOEF_ROUTED_ARGS(a), o);
    return hipGetLastError();
  });
}

hipError_t launch_finalize_rmsnorm(const Routed& r, const uint16_t* residual,
                                   const uint16_t* gamma, float eps,
                                   uint16_t* residual_out, uint16_t* normed,
                                   hipStream_t stream) {
  const GatherArgs a = make_args(r);
  const float inv_hidden = 1.0f / (float)r.hidden;
  const u32x4* res = reinterpret_cast<const u32x4*>(residual);
  const u32x4* gam = reinterpret_cast<const u32x4*>(gamma);
  u32x4* ro = reinterpret_cast<u32x4*>(residual_out);
  u32x4* nm = reinterpret_cast<u32x4*>(normed);
  const int ncu = a.k <= kStagedMaxTopK ? device_cus(stream) : 0;
  const RmsChoice c = rmsnorm_choice(a.tokens, r.hidden, a.k, ncu);
  if (c.staged) {
    return dispatch_top_k(a.k, [&](auto km, auto ex) {
      constexpr int KM = decltype(km)::value;
      constexpr bool EX = decltype(ex)::value;
      if constexpr (KM <= kStagedMaxTopK) {
        for (int64_t t0 = 0; t0 < a.tokens; t0 += c.plan.per_launch) {
          const int64_t t1 = t0 + c.plan.per_launch < a.tokens ? t0 + c.plan.per_launch : a.tokens;
          hipLaunchKernelGGL((finalize_rmsnorm_staged_kernel<KM, EX>), dim3(ncu),
                             dim3(kStageThreads), 0, stream, a, res, gam, eps, inv_hidden, ro,
                             nm, (int)t0, (int)t1);
          const hipError_t e = hipGetLastError();
          if (e != hipSuccess) return e;
        }
        return hipSuccess;
      } else {
        return hipErrorInvalidValue;   // not reached: top_k <= 8 dispatches KM <= 8
      }
    });
  }
  // Two vectors per lane: reserve LDS (unused by the kernel) so that at most
  // kNorm2MaxWavesPerCu waves are resident per CU; a workgroup too large for
  // two to fit needs no reservation.
  const int norm2_blocks = kNorm2MaxWavesPerCu / (c.threads / kWaveLanes);
  const size_t lds2 = norm2_blocks >= 2 ? lds_for_blocks_per_cu(norm2_blocks) : 0;
  return dispatch_top_k(a.k, [&](auto km, auto ex) {
    constexpr int KM = decltype(km)::value;
    constexpr bool EX = decltype(ex)::value;
    if (c.cpt == 1)
      hipLaunchKernelGGL((finalize_rmsnorm_kernel<KM, EX, 1>), dim3(a.tokens), dim3(c.threads),
                         0, stream, MOEF_ROUTED_ARGS(a), res, gam, eps, inv_hidden, ro, nm);
    else
      hipLaunchKernelGGL((finalize_rmsnorm_kernel<KM, EX, 2>), dim3(a.tokens), dim3(c.threads),
                         lds2, stream, MOEF_ROUTED_ARGS(a), res, gam, eps, inv_hidden, ro, nm);
    return hipGetLastError();
  });
}


hipError_t launch_finalize_quant(const Routed& r, uint8_t* out_e4m3, uint8_t* scale_e8m0,
                                 hipStream_t stream) {
  const GatherArgs a = make_args(r);
  u32x2* q = reinterpret_cast<u32x2*>(out_e4m3);
  const int ncu = a.k <= kStagedMaxTopK ? device_cus(stream) : 0;
  const QuantChoice c = quant_choice(a.tokens, r.hidden, a.k, ncu);
  if (c.staged) {
    return dispatch_top_k(a.k, [&](auto km, auto ex) {
      constexpr int KM = decltype(km)::value;
      constexpr bool EX = decltype(ex)::value;
      if constexpr (KM <= kStagedMaxTopK)
        return launch_quant_staged<KM, EX>(a, q, scale_e8m0, ncu, c.plan, c.groups, stream);
      else
        return hipErrorInvalidValue;   // not reached: top_k <= 8 dispatches KM <= 8
    });
  }
  // Large launches reserve LDS (unused by the kernel) to hold 4 workgroups
  // per CU instead of 8: measured 1-2% faster from about a thousand tokens
  // at H = 7168 (T = 8192: 181.9-182.5 against 185.3-185.7 us), slower for a
  // grid that would otherwise fit on the chip in one round.
  const size_t lds = stream_cap_lds((int64_t)a.tokens * a.nchunks);
  return dispatch_top_k(a.k, [&](auto km, auto ex) {
    constexpr int KM = decltype(km)::value;
    constexpr bool EX = decltype(ex)::value;
    hipLaunchKernelGGL((finalize_quant_kernel<KM, EX>), dim3(plain_blocks(a)),
                       dim3(kWavesPerBlock * kWaveLanes), lds, stream, MOEF_ROUTED_ARGS(a), q,
                       scale_e8m0);
    return hipGetLastError();
  });
}

hipError_t launch_ep_combine(const uint16_t* partials, int32_t num_partials,
                             const uint16_t* shared, uint16_t* out, int64_t tokens,
                             int64_t hidden, hipStream_t stream) {
  const int64_t n = tokens * (hidden / kVecElems);
  const unsigned int blocks = (unsigned int)((n + 255) / 256);
  const size_t lds = ep_cap_lds(((int64_t)blocks * 256) / kWaveLanes, num_partials);
  hipLaunchKernelGGL(ep_combine_kernel, dim3(blocks), dim3(256), lds, stream,
                     reinterpret_cast<const u32x4*>(partials), (int)num_partials, n,
                     reinterpret_cast<const u32x4*>(shared), reinterpret_cast<u32x4*>(out), n);
  return hipGetLastError();
}

hipError_t launch_packed_decode(const int32_t* packed, int64_t n, int32_t* expert_ids,
                                float* weights, hipStream_t stream) {
  const unsigned int blocks = (unsigned int)((n + 255) / 256);
  hipLaunchKernelGGL(packed_decode_kernel, dim3(blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(packed), n, expert_ids, weights);
  return hipGetLastError();
}

}  // namespace moef
