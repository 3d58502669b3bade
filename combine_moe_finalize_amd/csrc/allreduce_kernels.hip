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
// vectors, the residual, gamma) before the first add. HBM-bound:
// 2H(R + 3) bytes per token, plus 2H for gamma per launch.

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
