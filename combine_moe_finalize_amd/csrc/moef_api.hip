// C-ABI entry points of the deferred MoE finalize library.
//
// Each entry point validates every argument before it makes any HIP runtime
// call (so a rejected call enqueues nothing and the checks run on a machine
// without a GPU), then launches on the caller's stream and returns without
// synchronizing. The library allocates nothing and keeps no state beyond a
// per-device cache of the CU count, so a call can be captured into a HIP graph (the pages size their workspaces before
// graph capture and never grow them inside: "[Kimi K2.5] Fuse deferred MoE
// finalize into next-layer AR + residual + RMSNorm", Key modifications).

#include <cstdio>
#include <type_traits>

#include "moef_internal.h"

namespace {

using moef::Routed;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte ranges [p, p + n) overlap?
bool overlap(const void* p, int64_t np, const void* q, int64_t nq) {
  if (p == nullptr || q == nullptr || np <= 0 || nq <= 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uintptr_t b = reinterpret_cast<uintptr_t>(q);
  return a < b + (uintptr_t)nq && b < a + (uintptr_t)np;
}

struct Span {
  const void* p;
  int64_t bytes;
};

// Shape rules shared by the finalize entry points. Sets *noop for T == 0.
int check_shape(int64_t num_rows, int64_t tokens, int64_t hidden, int32_t top_k, bool* noop) {
  *noop = false;
  if (tokens < 0 || num_rows < 0) return MOEF_ERR_BAD_SHAPE;
  if (top_k < 1 || top_k > MOEF_MAX_TOP_K) return MOEF_ERR_BAD_SHAPE;
  if (hidden < 1) return MOEF_ERR_BAD_SHAPE;
  if (hidden % moef::kVecElems != 0 || hidden > MOEF_MAX_HIDDEN) return MOEF_ERR_UNSUPPORTED;
  if (num_rows > INT32_MAX) return MOEF_ERR_UNSUPPORTED;   // rows are named by int32
  if (tokens > INT32_MAX) return MOEF_ERR_UNSUPPORTED;
  const int64_t nchunks = (hidden / moef::kVecElems + moef::kWaveLanes - 1) / moef::kWaveLanes;
  if (tokens * nchunks > moef::kMaxUnits) return MOEF_ERR_UNSUPPORTED;
  if (tokens == 0) *noop = true;
  return MOEF_OK;
}

// Pointer, format and alignment rules of the routed inputs.
int check_routed_inputs(const Routed& r) {
  if (r.idx == nullptr || r.weights == nullptr) {
    return r.idx == nullptr ? MOEF_ERR_NULL_POINTER : MOEF_ERR_BAD_FORMAT;
  }
  if (r.num_rows > 0 && r.gemm2_out == nullptr) return MOEF_ERR_NULL_POINTER;
  if (!aligned(r.gemm2_out, 16) || !aligned(r.shared, 16)) return MOEF_ERR_MISALIGNED;
  if (!aligned(r.idx, 4) || !aligned(r.weights, 4) || !aligned(r.err_flag, 4))
    return MOEF_ERR_MISALIGNED;
  return MOEF_OK;
}

// Fills the routed block; exactly one weight format must be given.
int make_routed(Routed* r, const uint16_t* gemm2_out, int64_t num_rows, const int32_t* idx,
                const float* w32, const int32_t* packed, const uint16_t* shared, float rsf,
                int64_t tokens, int64_t hidden, int32_t top_k, int32_t* err_flag) {
  if ((w32 == nullptr) == (packed == nullptr)) return MOEF_ERR_BAD_FORMAT;
  r->gemm2_out = gemm2_out;
  r->num_rows = num_rows;
  r->idx = idx;
  r->weights = w32 != nullptr ? reinterpret_cast<const uint32_t*>(w32)
                              : reinterpret_cast<const uint32_t*>(packed);
  r->packed = packed != nullptr;
  r->shared = shared;
  r->rsf = rsf;
  r->tokens = tokens;
  r->hidden = hidden;
  r->top_k = top_k;
  r->err_flag = err_flag;
  return MOEF_OK;
}

// Index of err_flag's own range in the list routed_spans() builds.
constexpr int kErrSpan = 4;

// The input byte ranges of a routed call (for alias checks).
int routed_spans(const Routed& r, Span* s) {
  const int64_t row_bytes = r.hidden * 2;
  const int64_t slot_bytes = r.tokens * r.top_k * 4;
  s[0] = {r.gemm2_out, r.num_rows * row_bytes};
  s[1] = {r.idx, slot_bytes};
  s[2] = {r.weights, slot_bytes};
  s[3] = {r.shared, r.shared ? r.tokens * row_bytes : 0};
  s[kErrSpan] = {r.err_flag, r.err_flag ? 4 : 0};
  return kErrSpan + 1;
}

bool overlaps_any(const void* p, int64_t n, const Span* s, int ns) {
  for (int i = 0; i < ns; ++i)
    if (overlap(p, n, s[i].p, s[i].bytes)) return true;
  return false;
}

// err_flag is written by the kernels, so it may not overlap anything they
// read: every span of s (routed_spans() first, then any others) but its own.
bool err_flag_clear(const Routed& r, const Span* s, int ns) {
  if (r.err_flag == nullptr) return true;
  for (int i = 0; i < ns; ++i)
    if (i != kErrSpan && overlap(r.err_flag, 4, s[i].p, s[i].bytes)) return false;
  return true;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOEF_OK : MOEF_ERR_HIP; }

// Shared checks and launch of the two activation-quant entry points.
int act_quant(const uint16_t* x, int64_t num_tokens, int64_t hidden, uint8_t* out_e4m3,
              uint8_t* scale_e8m0, float* scale_f32, void* stream) {
  if (num_tokens < 0 || hidden < 1) return MOEF_ERR_BAD_SHAPE;
  if (hidden % MOEF_QUANT_BLOCK != 0 || hidden > MOEF_MAX_HIDDEN || num_tokens > INT32_MAX)
    return MOEF_ERR_UNSUPPORTED;
  const int64_t nchunks = (hidden / moef::kVecElems + moef::kWaveLanes - 1) / moef::kWaveLanes;
  if (num_tokens * nchunks > moef::kMaxUnits) return MOEF_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOEF_OK;
  if (x == nullptr || out_e4m3 == nullptr || (scale_e8m0 == nullptr && scale_f32 == nullptr))
    return MOEF_ERR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(out_e4m3, 8) || !aligned(scale_f32, 4))
    return MOEF_ERR_MISALIGNED;
  const int64_t xb = num_tokens * hidden * 2;
  const int64_t qb = num_tokens * hidden;
  const int64_t sb = num_tokens * (hidden / MOEF_QUANT_BLOCK) * (scale_f32 != nullptr ? 4 : 1);
  const void* sp = scale_f32 != nullptr ? (const void*)scale_f32 : (const void*)scale_e8m0;
  if (overlap(out_e4m3, qb, x, xb) || overlap(sp, sb, x, xb) || overlap(out_e4m3, qb, sp, sb))
    return MOEF_ERR_BAD_ALIAS;
  return hip_status(moef::launch_act_quant(x, num_tokens, hidden, out_e4m3, scale_e8m0,
                                           scale_f32, static_cast<hipStream_t>(stream)));
}


}  // namespace

namespace moef {

// The kernel names below follow the form profilers print template instances
// in ("name<8, true, 12>"), so a benchmark can find them in a trace.
void describe_finalize(int op, int64_t tokens, int64_t hidden, int top_k, int ncu, char* buf,
                       int64_t len) {
  const TopKChoice k = top_k_choice(top_k);
  const char* ex = k.exact ? "true" : "false";
  const int64_t nch = nchunks_of(hidden);
  const int64_t one_wave_blocks = (tokens * nch + kWavesPerBlock - 1) / kWavesPerBlock;
  if (op == 0) {
    const PlainChoice c = plain_choice(tokens, hidden, top_k, ncu);
    if (c.staged) {
      const int waves = c.wide ? kStagePlainWideWaves : kStagePlainWaves;
      const int reg = c.wide ? kStagePlainWideRegUnits : kStagePlainRegUnits;
      const bool regs = (c.plan.per_launch + ncu - 1) / ncu > kStagePlainUnits;
      snprintf(buf, (size_t)len, "finalize_staged_kernel<%d, %s, %d, %d> launches=%lld grid=%dx%d",
               k.kmax, ex, regs ? reg : 0, waves, (long long)c.plan.launches, ncu,
               waves * kWaveLanes);
    } else {
      snprintf(buf, (size_t)len, "finalize_kernel<%d, %s> launches=1 grid=%lldx%d", k.kmax, ex,
               (long long)one_wave_blocks, kWavesPerBlock * kWaveLanes);
    }
  } else if (op == 1) {
    const RmsChoice c = rmsnorm_choice(tokens, hidden, top_k, ncu);
    if (c.staged)
      snprintf(buf, (size_t)len, "finalize_rmsnorm_staged_kernel<%d, %s> launches=%lld grid=%dx%d",
               k.kmax, ex, (long long)c.plan.launches, ncu, kStageThreads);
    else
      snprintf(buf, (size_t)len, "finalize_rmsnorm_kernel<%d, %s, %d> launches=1 grid=%lldx%d",
               k.kmax, ex, c.cpt, (long long)tokens, c.threads);
  } else {
    const QuantChoice c = quant_choice(tokens, hidden, top_k, ncu);
    if (c.staged) {
      const int64_t tl = c.plan.per_launch < tokens ? c.plan.per_launch : tokens;
      const bool regs = quant_launch_regs(tl, nch, ncu, c.groups);
      const int pct = quant_launch_tail_percent(tl, nch, ncu);
      const int64_t tail = quant_launch_tail_workgroups(tl, nch, c.groups, pct);
      snprintf(buf, (size_t)len,
               "finalize_quant_staged_kernel<%d, %s, %d> launches=%lld grid=%lldx%d groups=%d "
               "tail=%d%%",
               k.kmax, ex, regs ? kStageRegUnits : 0, (long long)c.plan.launches,
               (long long)(ncu + tail), kStageThreads, c.groups, pct);
    } else {
      snprintf(buf, (size_t)len, "finalize_quant_kernel<%d, %s> launches=1 grid=%lldx%d", k.kmax,
               ex, (long long)one_wave_blocks, kWavesPerBlock * kWaveLanes);
    }
  }
}

}  // namespace moef

extern "C" {

int moe_finalize_abi_version(void) { return MOEF_ABI_VERSION; }

int moe_finalize_describe_launch(int32_t op, int64_t num_tokens, int64_t hidden, int32_t top_k,
                                 void* stream, char* buf, int64_t buf_len) {
  if (buf == nullptr || buf_len < 1) return MOEF_ERR_NULL_POINTER;
  buf[0] = '\0';
  if (op < MOEF_OP_FINALIZE || op > MOEF_OP_QUANT_UE8M0) return MOEF_ERR_BAD_SHAPE;
  bool noop = false;
  const int st = check_shape(0, num_tokens, hidden, top_k, &noop);
  if (st != MOEF_OK) return st;
  if (op == MOEF_OP_RESIDUAL_RMSNORM && hidden > MOEF_MAX_HIDDEN_RMSNORM) return MOEF_ERR_UNSUPPORTED;
  if (op == MOEF_OP_QUANT_UE8M0 && hidden % MOEF_QUANT_BLOCK != 0) return MOEF_ERR_UNSUPPORTED;
  if (noop) {
    snprintf(buf, (size_t)buf_len, "none (num_tokens == 0)");
    return MOEF_OK;
  }
  const int ncu = top_k <= moef::kStagedMaxTopK ? moef::device_cus(static_cast<hipStream_t>(stream)) : 0;
  moef::describe_finalize(op, num_tokens, hidden, top_k, ncu, buf, buf_len);
  return MOEF_OK;
}

const char* moe_finalize_status_string(int status) {
  switch (status) {
    case MOEF_OK: return "ok";
    case MOEF_ERR_NULL_POINTER: return "a required pointer is NULL";
    case MOEF_ERR_BAD_SHAPE: return "bad shape (negative count, hidden or top_k out of range)";
    case MOEF_ERR_UNSUPPORTED: return "unsupported size (hidden alignment or limits)";
    case MOEF_ERR_MISALIGNED: return "pointer misaligned";
    case MOEF_ERR_BAD_FORMAT: return "give exactly one routing-weight format (fp32 or packed)";
    case MOEF_ERR_BAD_ALIAS: return "an output overlaps an input or another output";
    case MOEF_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int moe_finalize(const uint16_t* gemm2_out, int64_t num_rows,
                 const int32_t* expanded_idx_to_permuted_idx, const float* topk_weights,
                 const int32_t* topk_packed, const uint16_t* shared_out,
                 float routed_scaling_factor, uint16_t* out, int64_t num_tokens,
                 int64_t hidden, int32_t top_k, int32_t* err_flag, void* stream) {
  bool noop;
  int st = check_shape(num_rows, num_tokens, hidden, top_k, &noop);
  if (st != MOEF_OK || noop) return st;
  Routed r;
  st = make_routed(&r, gemm2_out, num_rows, expanded_idx_to_permuted_idx, topk_weights,
                   topk_packed, shared_out, routed_scaling_factor, num_tokens, hidden,
                   top_k, err_flag);
  if (st != MOEF_OK) return st;
  if ((st = check_routed_inputs(r)) != MOEF_OK) return st;
  if (out == nullptr) return MOEF_ERR_NULL_POINTER;
  if (!aligned(out, 16)) return MOEF_ERR_MISALIGNED;
  Span s[8];
  const int ns = routed_spans(r, s);
  if (!err_flag_clear(r, s, ns)) return MOEF_ERR_BAD_ALIAS;
  if (overlaps_any(out, num_tokens * hidden * 2, s, ns)) return MOEF_ERR_BAD_ALIAS;
  return hip_status(moef::launch_finalize(r, out, static_cast<hipStream_t>(stream)));
}

int moe_finalize_residual_rmsnorm(const uint16_t* gemm2_out, int64_t num_rows,
                                  const int32_t* expanded_idx_to_permuted_idx,
                                  const float* topk_weights, const int32_t* topk_packed,
                                  const uint16_t* shared_out, float routed_scaling_factor,
                                  const uint16_t* residual, const uint16_t* gamma, float eps,
                                  uint16_t* residual_out, uint16_t* normed,
                                  int64_t num_tokens, int64_t hidden, int32_t top_k,
                                  int32_t* err_flag, void* stream) {
  bool noop;
  int st = check_shape(num_rows, num_tokens, hidden, top_k, &noop);
  if (st != MOEF_OK) return st;
  if (hidden > MOEF_MAX_HIDDEN_RMSNORM) return MOEF_ERR_UNSUPPORTED;
  if (noop) return MOEF_OK;
  Routed r;
  st = make_routed(&r, gemm2_out, num_rows, expanded_idx_to_permuted_idx, topk_weights,
                   topk_packed, shared_out, routed_scaling_factor, num_tokens, hidden,
                   top_k, err_flag);
  if (st != MOEF_OK) return st;
  if ((st = check_routed_inputs(r)) != MOEF_OK) return st;
  if (residual == nullptr || gamma == nullptr || residual_out == nullptr || normed == nullptr)
    return MOEF_ERR_NULL_POINTER;
  if (!aligned(residual, 16) || !aligned(gamma, 16) || !aligned(residual_out, 16) ||
      !aligned(normed, 16))
    return MOEF_ERR_MISALIGNED;
  const int64_t tb = num_tokens * hidden * 2;
  Span s[8];
  int ns = routed_spans(r, s);
  s[ns++] = {gamma, hidden * 2};
  // residual_out may be residual itself, but no other overlap is allowed
  if (overlaps_any(residual_out, tb, s, ns)) return MOEF_ERR_BAD_ALIAS;
  if (residual_out != residual && overlap(residual_out, tb, residual, tb)) return MOEF_ERR_BAD_ALIAS;
  s[ns++] = {residual, tb};
  if (!err_flag_clear(r, s, ns)) return MOEF_ERR_BAD_ALIAS;
  if (overlaps_any(normed, tb, s, ns) || overlap(normed, tb, residual_out, tb))
    return MOEF_ERR_BAD_ALIAS;
  return hip_status(moef::launch_finalize_rmsnorm(r, residual, gamma, eps, residual_out, normed,
                                                  static_cast<hipStream_t>(stream)));
}

int moe_finalize_quant_ue8m0(const uint16_t* gemm2_out, int64_t num_rows,
                             const int32_t* expanded_idx_to_permuted_idx,
                             const float* topk_weights, const int32_t* topk_packed,
                             const uint16_t* shared_out, float routed_scaling_factor,
                             uint8_t* out_e4m3, uint8_t* scale_e8m0, int64_t num_tokens,
                             int64_t hidden, int32_t top_k, int32_t* err_flag, void* stream) {
  bool noop;
  int st = check_shape(num_rows, num_tokens, hidden, top_k, &noop);
  if (st != MOEF_OK) return st;
  if (hidden % MOEF_QUANT_BLOCK != 0) return MOEF_ERR_UNSUPPORTED;
  if (noop) return MOEF_OK;
  Routed r;
  st = make_routed(&r, gemm2_out, num_rows, expanded_idx_to_permuted_idx, topk_weights,
                   topk_packed, shared_out, routed_scaling_factor, num_tokens, hidden,
                   top_k, err_flag);
  if (st != MOEF_OK) return st;
  if ((st = check_routed_inputs(r)) != MOEF_OK) return st;
  if (out_e4m3 == nullptr || scale_e8m0 == nullptr) return MOEF_ERR_NULL_POINTER;
  if (!aligned(out_e4m3, 8)) return MOEF_ERR_MISALIGNED;
  const int64_t qb = num_tokens * hidden;
  const int64_t sb = num_tokens * (hidden / MOEF_QUANT_BLOCK);
  Span s[8];
  const int ns = routed_spans(r, s);
  if (!err_flag_clear(r, s, ns)) return MOEF_ERR_BAD_ALIAS;
  if (overlaps_any(out_e4m3, qb, s, ns) || overlaps_any(scale_e8m0, sb, s, ns) ||
      overlap(out_e4m3, qb, scale_e8m0, sb))
    return MOEF_ERR_BAD_ALIAS;
  return hip_status(moef::launch_finalize_quant(r, out_e4m3, scale_e8m0,
                                                static_cast<hipStream_t>(stream)));
}

int moe_finalize_ep_combine(const uint16_t* partials, int32_t num_partials,
                            const uint16_t* shared_out, uint16_t* out, int64_t num_tokens,
                            int64_t hidden, void* stream) {
  if (num_tokens < 0 || hidden < 1 || num_partials < 1 || num_partials > MOEF_MAX_EP_PARTIALS)
    return MOEF_ERR_BAD_SHAPE;
  if (hidden % moef::kVecElems != 0 || hidden > MOEF_MAX_HIDDEN) return MOEF_ERR_UNSUPPORTED;
  if (num_tokens > moef::kMaxGridItems ||
      num_tokens * (hidden / moef::kVecElems) > moef::kMaxGridItems)
    return MOEF_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOEF_OK;
  if (partials == nullptr || out == nullptr) return MOEF_ERR_NULL_POINTER;
  if (!aligned(partials, 16) || !aligned(shared_out, 16) || !aligned(out, 16))
    return MOEF_ERR_MISALIGNED;
  const int64_t tb = num_tokens * hidden * 2;
  if (overlap(out, tb, partials, tb * num_partials) || overlap(out, tb, shared_out, tb))
    return MOEF_ERR_BAD_ALIAS;
  return hip_status(moef::launch_ep_combine(partials, num_partials, shared_out, out, num_tokens,
                                            hidden, static_cast<hipStream_t>(stream)));
}

int moe_allreduce_residual_rmsnorm(const uint16_t* const* rank_outputs, int32_t num_ranks,
                                   const uint16_t* residual, const uint16_t* gamma, float eps,
                                   uint16_t* residual_out, uint16_t* normed, int64_t num_tokens,
                                   int64_t hidden, void* stream) {
  if (num_tokens < 0 || hidden < 1 || num_ranks < 1 || num_ranks > MOEF_MAX_AR_RANKS)
    return MOEF_ERR_BAD_SHAPE;
  if (hidden % moef::kVecElems != 0 || hidden > MOEF_MAX_HIDDEN_RMSNORM ||
      num_tokens > moef::kMaxUnits ||
      num_tokens * ((hidden / moef::kVecElems + moef::kWaveLanes - 1) / moef::kWaveLanes) >
          moef::kMaxUnits)
    return MOEF_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOEF_OK;
  if (rank_outputs == nullptr || residual == nullptr || gamma == nullptr ||
      residual_out == nullptr || normed == nullptr)
    return MOEF_ERR_NULL_POINTER;
  for (int r = 0; r < num_ranks; ++r)
    if (rank_outputs[r] == nullptr) return MOEF_ERR_NULL_POINTER;
  for (int r = 0; r < num_ranks; ++r)
    if (!aligned(rank_outputs[r], 16)) return MOEF_ERR_MISALIGNED;
  if (!aligned(residual, 16) || !aligned(gamma, 16) || !aligned(residual_out, 16) ||
      !aligned(normed, 16))
    return MOEF_ERR_MISALIGNED;
  const int64_t tb = num_tokens * hidden * 2;
  Span s[MOEF_MAX_AR_RANKS + 3];
  int ns = 0;
  for (int r = 0; r < num_ranks; ++r) s[ns++] = {rank_outputs[r], tb};
  s[ns++] = {gamma, hidden * 2};
  // residual_out may be residual itself, but no other overlap is allowed
  if (overlaps_any(residual_out, tb, s, ns)) return MOEF_ERR_BAD_ALIAS;
  if (residual_out != residual && overlap(residual_out, tb, residual, tb)) return MOEF_ERR_BAD_ALIAS;
  s[ns++] = {residual, tb};
  if (overlaps_any(normed, tb, s, ns) || overlap(normed, tb, residual_out, tb))
    return MOEF_ERR_BAD_ALIAS;
  return hip_status(moef::launch_allreduce_rmsnorm(rank_outputs, num_ranks, residual, gamma, eps,
                                                   residual_out, normed, num_tokens, hidden,
                                                   static_cast<hipStream_t>(stream)));
}

int moe_topk_packed_decode(const int32_t* packed, int64_t n, int32_t* expert_ids,
                           float* weights, void* stream) {
  if (n < 0) return MOEF_ERR_BAD_SHAPE;
  if (n > moef::kMaxGridItems) return MOEF_ERR_UNSUPPORTED;
  if (n == 0) return MOEF_OK;
  if (packed == nullptr || (expert_ids == nullptr && weights == nullptr))
    return MOEF_ERR_NULL_POINTER;
  if (!aligned(packed, 4) || !aligned(expert_ids, 4) || !aligned(weights, 4))
    return MOEF_ERR_MISALIGNED;
  const int64_t nb = n * 4;
  if (overlap(expert_ids, nb, packed, nb) || overlap(weights, nb, packed, nb) ||
      overlap(expert_ids, nb, weights, nb))
    return MOEF_ERR_BAD_ALIAS;
  return hip_status(moef::launch_packed_decode(packed, n, expert_ids, weights,
                                               static_cast<hipStream_t>(stream)));
}

int moe_topk_sigmoid_gate(const float* router_logits, int64_t num_tokens, int32_t num_experts,
                          int32_t top_k, int32_t* topk_ids, float* topk_weights,
                          int32_t* topk_packed, void* stream) {
  if (num_tokens < 0 || num_experts < 1 || top_k < 1 || top_k > MOEF_MAX_TOP_K ||
      top_k > num_experts)
    return MOEF_ERR_BAD_SHAPE;
  if (num_experts > MOEF_MAX_GATE_EXPERTS) return MOEF_ERR_UNSUPPORTED;
  if (num_tokens > moef::kMaxUnits) return MOEF_ERR_UNSUPPORTED;   // one wave per token
  if (num_tokens == 0) return MOEF_OK;
  if (router_logits == nullptr || topk_ids == nullptr) return MOEF_ERR_NULL_POINTER;
  if (!aligned(router_logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) ||
      !aligned(topk_packed, 4))
    return MOEF_ERR_MISALIGNED;
  const int64_t lb = num_tokens * num_experts * 4;
  const int64_t ob = num_tokens * top_k * 4;
  const Span in[1] = {{router_logits, lb}};
  if (overlaps_any(topk_ids, ob, in, 1) || overlaps_any(topk_weights, ob, in, 1) ||
      overlaps_any(topk_packed, ob, in, 1) || overlap(topk_ids, ob, topk_weights, ob) ||
      overlap(topk_ids, ob, topk_packed, ob) || overlap(topk_weights, ob, topk_packed, ob))
    return MOEF_ERR_BAD_ALIAS;
  return hip_status(moef::launch_topk_sigmoid_gate(router_logits, num_tokens, num_experts,
                                                   top_k, topk_ids, topk_weights, topk_packed,
                                                   static_cast<hipStream_t>(stream)));
}

int moe_act_quant_fp8_ue8m0(const uint16_t* x, int64_t num_tokens, int64_t hidden,
                            uint8_t* out_e4m3, uint8_t* scale_e8m0, void* stream) {
  if (scale_e8m0 == nullptr && num_tokens > 0) return MOEF_ERR_NULL_POINTER;
  return act_quant(x, num_tokens, hidden, out_e4m3, scale_e8m0, nullptr, stream);
}

int moe_act_quant_fp8_amax(const uint16_t* x, int64_t num_tokens, int64_t hidden,
                           uint8_t* out_e4m3, float* scale_f32, void* stream) {
  if (scale_f32 == nullptr && num_tokens > 0) return MOEF_ERR_NULL_POINTER;
  return act_quant(x, num_tokens, hidden, out_e4m3, nullptr, scale_f32, stream);
}

}  // extern "C"
