// gfx950 all-reduce + residual + RMSNorm after the deferred finalize: the part
// one GPU runs of the step that follows the finalize when the MoE layer is
// split over R ranks.
//
// "[Kimi K2.5] Fuse deferred MoE finalize into next-layer AR + residual +
// RMSNorm", Numerics & speed vs the separate-finalize fallback: under
// graph-captured decode the faster and more accurate path is the deferred
// finalize followed by a separate all-reduce + residual + RMSNorm kernel that
// also emits residual_out and accumulates in fp32. Every rank's finalize
// output is one input here. residual_out = bf16(+0 + o_0 + ... + o_{R-1} +
// residual), fp32 adds in that order with one rounding; normed is the RMSNorm
// of the stored residual_out.
//
// The R inputs come as device pointers passed by value in the kernel
// arguments. On a multi-GPU node they are the peers' buffers mapped into this
// process, read over xGMI: a one-shot all-reduce hands each rank every token,
// and a two-shot one hands it its token slice, followed by an all-gather of
// the results. On one GPU they are local buffers.
//
// One workgroup per token, as in the fused finalize + RMSNorm epilogue. Each
// thread holds CPT vectors of 8 columns and issues all of its loads (R rank
// vectors, the residual, gamma) before the first add; large grids stage
// whole tokens per CU and write after their reads, as the epilogue does.
// HBM-bound: 2H(R + 3) bytes per token, plus 2H for gamma per launch.

#include "device_common.h"
#include "moef_internal.h"

namespace moef {
namespace {

using namespace dev;

struct RankPtrs {
  const u32x4* p[MOEF_MAX_AR_RANKS];
};

template <int RMAX, bool EXACT, int CPT>
__global__ void __launch_bounds__(kNormMaxThreads)
allreduce_rmsnorm_kernel(RankPtrs ranks, int R, int h8, const u32x4* residual,
                         const u32x4* __restrict__ gamma, float eps, float inv_hidden,
                         u32x4* residual_out, u32x4* __restrict__ normed) {
  __shared__ float partial[kNormMaxChunks];
  const int t = blockIdx.x;
  const int nthreads = blockDim.x;
  const int64_t row = (int64_t)t * h8;

  float ro[CPT][8];
  u32x4 gv[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int colv = threadIdx.x + i * nthreads;
    const bool active = colv < h8;
    const int64_t col = active ? colv : h8 - 1;      // in bounds; not stored
    u32x4 v[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r)
      if (EXACT || r < R) v[r] = __builtin_nontemporal_load(ranks.p[r] + row + col);
    const u32x4 rv = __builtin_nontemporal_load(residual + row + col);
    gv[i] = gamma[col];
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (EXACT || r < R) {
        float x[8];
        unpack8(v[r], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
      }
    }
    float x[8];
    unpack8(rv, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
    const u32x4 rb = pack8_rne(acc);
    unpack8(rb, ro[i]);                               // the stored bf16 residual_out
    float ss = 0.0f;
    if (active) {
      __builtin_nontemporal_store(rb, residual_out + row + colv);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = ss + ro[i][e] * ro[i][e];
    }
    put_chunk_sum(ss, i, partial);
  }
  const float inv = row_inv_rms<CPT>(partial, inv_hidden, eps);
  store_normed<CPT>(ro, gv, inv, h8, normed + row);
}

// allreduce_rmsnorm_kernel's result for large grids, with every write after
// the workgroup's reads (the scheme of the finalize's staged RMSNorm
// epilogue). One workgroup of kStageWaves waves per CU owns whole tokens
// t0 + b + i * gridDim.x, i < ntok; its waves take the (token, chunk) units
// j = i * nch + c from an LDS counter. Unit j leaves its residual_out vector
// in LDS slot j and its chunk's sum of squares, reduced over the wave as the
// one-workgroup-per-token kernel reduces a chunk, in sumsq[j]. After the
// last read each token's 1 / rms is formed from its chunk sums added in
// chunk order, as row_inv_rms does, so both kernels give the same bits; then
// the workgroup writes residual_out and normed. A token's residual is read
// only by the workgroup that writes its residual_out (in place is allowed).
template <int RMAX, bool EXACT>
__global__ void __launch_bounds__(kStageThreads)
allreduce_rmsnorm_staged_kernel(RankPtrs ranks, int R, int h8, int nch, const u32x4* residual,
                                const u32x4* __restrict__ gamma, float eps, float inv_hidden,
                                u32x4* residual_out, u32x4* __restrict__ normed, int t0,
                                int t1) {
  __shared__ u32x4 stage_r[kStageRmsUnits * kWaveLanes];
  __shared__ float sumsq[kStageRmsUnits];
  __shared__ float inv_rms[kStageRmsUnits];     // per token
  __shared__ int next_j;
  const int nb = (int)gridDim.x;
  const int b = (int)blockIdx.x;
  int ntok = t1 - t0 > b ? (t1 - t0 - b + nb - 1) / nb : 0;
  if (ntok > kStageRmsUnits / nch) ntok = kStageRmsUnits / nch;   // launches are sized below it
  const int n = ntok * nch;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x == 0) next_j = 0;
  __syncthreads();

  for (int it = 0; it < n; ++it) {
    const int j = next_unit(&next_j);
    if ((unsigned)j >= (unsigned)n) break;
    const int i = j / nch;
    const int64_t row = (int64_t)(t0 + b + i * nb) * h8;
    const int colv = (j - i * nch) * kWaveLanes + lane;
    const bool active = colv < h8;
    const int64_t col = active ? colv : h8 - 1;      // in bounds; not stored
    u32x4 v[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r)
      if (EXACT || r < R) v[r] = __builtin_nontemporal_load(ranks.p[r] + row + col);
    const u32x4 rv = __builtin_nontemporal_load(residual + row + col);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (EXACT || r < R) {
        float x[8];
        unpack8(v[r], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
      }
    }
    float x[8];
    unpack8(rv, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + x[e];
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
    if (colv < h8) {
      const int64_t o = (int64_t)(t0 + b + i * nb) * h8 + colv;
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
}

template <int V>
using IC = std::integral_constant<int, V>;

// Exact instantiations for the usual rank counts, guarded ones otherwise.
template <typename F>
hipError_t dispatch_ranks(int R, F&& f) {
  switch (R) {
    case 1: return f(IC<1>{}, std::true_type{});
    case 2: return f(IC<2>{}, std::true_type{});
    case 4: return f(IC<4>{}, std::true_type{});
    case 8: return f(IC<8>{}, std::true_type{});
    default:
      if (R <= 4) return f(IC<4>{}, std::false_type{});
      if (R <= 8) return f(IC<8>{}, std::false_type{});
      return f(IC<16>{}, std::false_type{});
  }
}

}  // namespace

hipError_t launch_allreduce_rmsnorm(const uint16_t* const* rank_outputs, int32_t num_ranks,
                                    const uint16_t* residual, const uint16_t* gamma, float eps,
                                    uint16_t* residual_out, uint16_t* normed, int64_t tokens,
                                    int64_t hidden, hipStream_t stream) {
  RankPtrs ranks{};
  for (int r = 0; r < num_ranks; ++r) ranks.p[r] = reinterpret_cast<const u32x4*>(rank_outputs[r]);
  const int h8 = (int)(hidden / kVecElems);
  int threads = ((h8 + kWaveLanes - 1) / kWaveLanes) * kWaveLanes;
  if (threads > kNormMaxThreads) threads = kNormMaxThreads;
  const int cpt = (h8 + threads - 1) / threads;     // 1 or 2 (hidden <= 16384)
  const float inv_hidden = 1.0f / (float)hidden;
  const u32x4* res = reinterpret_cast<const u32x4*>(residual);
  const u32x4* gam = reinterpret_cast<const u32x4*>(gamma);
  u32x4* ro = reinterpret_cast<u32x4*>(residual_out);
  u32x4* nm = reinterpret_cast<u32x4*>(normed);
  const int nch = (h8 + kWaveLanes - 1) / kWaveLanes;
  const int ncu = device_cus(stream);
  if (ncu > 0 && tokens * nch >= kStagedArFromUnitsPerCu * ncu) {
    const StagedPlan plan = plan_staged(tokens, ncu, kStageRmsUnits / nch);
    return dispatch_ranks(num_ranks, [&](auto rm, auto ex) {
      constexpr int RM = decltype(rm)::value;
      constexpr bool EX = decltype(ex)::value;
      for (int64_t t0 = 0; t0 < tokens; t0 += plan.per_launch) {
        const int64_t t1 = t0 + plan.per_launch < tokens ? t0 + plan.per_launch : tokens;
        hipLaunchKernelGGL((allreduce_rmsnorm_staged_kernel<RM, EX>), dim3(ncu),
                           dim3(kStageThreads), 0, stream, ranks, (int)num_ranks, h8, nch, res,
                           gam, eps, inv_hidden, ro, nm, (int)t0, (int)t1);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    });
  }
  const dim3 grid((unsigned int)tokens), block(threads);
  return dispatch_ranks(num_ranks, [&](auto rm, auto ex) {
    constexpr int RM = decltype(rm)::value;
    constexpr bool EX = decltype(ex)::value;
    if (cpt == 1)
      hipLaunchKernelGGL((allreduce_rmsnorm_kernel<RM, EX, 1>), grid, block, 0, stream, ranks,
                         (int)num_ranks, h8, res, gam, eps, inv_hidden, ro, nm);
    else
      hipLaunchKernelGGL((allreduce_rmsnorm_kernel<RM, EX, 2>), grid, block, 0, stream, ranks,
                         (int)num_ranks, h8, res, gam, eps, inv_hidden, ro, nm);
    return hipGetLastError();
  });
}

}  // namespace moef
