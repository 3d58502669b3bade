/*
 * moe_finalize.h - C ABI of the MI355X (gfx950) deferred MoE finalize library.
 *
 * The deferred finalize is the step after a grouped expert GEMM that was told
 * not to combine its outputs: for every token it gathers that token's top_k
 * un-weighted, expert-sorted rows of gemm2_out, weights each by its routing
 * weight times the routed scaling factor, sums them in fp32, adds the
 * shared-expert output and writes bf16. Optional fused epilogues add the
 * residual and apply RMSNorm (emitting residual_out too), or quantize the
 * result to FP8 E4M3 with one power-of-two (UE8M0) scale per 1 x 128 block.
 * Around it: the sigmoid top-k gate that produces the routing, a standalone
 * FP8 activation quant, the expert-parallel combine, and the all-reduce +
 * residual + RMSNorm that follows the finalize when the layer is split over
 * ranks (the part one GPU runs).
 *
 * Sources (sglang pull-request pages):
 *  - "Support deferred MoE finalize for MXFP4 and FP8 block-scale":
 *    Motivation (the deferred top-k weighted combine, fused with the
 *    shared-expert add) and Modifications item 2 (the routed scaling factor
 *    is folded into the register-held expert weight; 1.0 is neutral), item 1
 *    (the routing format is an explicit per-configuration choice).
 *  - "[Kimi K2.5] Fuse deferred MoE finalize into next-layer AR + residual +
 *    RMSNorm": Key modifications (the index map and weights are
 *    [token, top_k]; a flat index caused out-of-bounds reads; workspaces are
 *    sized before graph capture and never grow inside it) and "Numerics &
 *    speed" (gathering from the padded permuted buffer; residual + RMSNorm
 *    with residual_out; fp32 accumulation; the separate finalize followed by
 *    an all-reduce + residual + RMSNorm kernel as the preferred path).
 *  - "[FP8][MoE] Honor UE8M0 activation scales in Triton MoE": Motivation and
 *    "More context" (power-of-two FP32 activation scales, FP8 range 448).
 *  - "[Deepseek V4] Keep fp32 routing weights in the mxfp4 trtllm MoE":
 *    PR description (packed word (expert_id << 16) | bf16(weight) versus
 *    genuine fp32 weights; the finalize weight type is bf16 or float) and the
 *    follow-up commit (reading fp32 weights as bf16 broke decoding).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller, row-major
 *    and contiguous. bf16 values travel as raw bits in uint16_t, FP8 E4M3
 *    codes and UE8M0 scale bytes as uint8_t. The library never allocates,
 *    frees or keeps a pointer after the call returns, never synchronizes and
 *    never reads device memory from the host, so every call may be captured
 *    into a HIP graph. Its only global state is a per-device cache of the
 *    CU count (queried on first use, then read); calls on any streams and
 *    threads may run at once.
 *  - `stream` is a hipStream_t passed as void* (NULL: the null stream). Work
 *    is enqueued on it; the call returns without waiting.
 *  - Return value: MOEF_OK (0) or a MOEF_ERR_* status. Every argument check
 *    runs before any HIP runtime call; a failed check enqueues nothing.
 *    MOEF_ERR_HIP reports a launch failure (hipGetLastError after the launch);
 *    faults inside a kernel surface at the caller's next synchronization, as
 *    in any HIP API.
 *  - num_tokens == 0 is a successful no-op (pointers may then be NULL).
 *  - Device error flag: `err_flag` is an optional device int32 that the
 *    caller zeroes. The kernels OR MOEF_DEVERR_INDEX_OUT_OF_RANGE into it
 *    when an index is >= num_rows; that slot is skipped. A negative index
 *    marks a slot whose expert is not held here: it is skipped silently.
 *  - Routing weights: exactly one of `topk_weights` (float32 [T, top_k]) and
 *    `topk_packed` (int32 [T, top_k], (expert_id << 16) | bf16_bits(weight),
 *    the id read with a logical shift and not used by the finalize) is
 *    non-NULL, else MOEF_ERR_BAD_FORMAT. The two formats have distinct C
 *    types so fp32 weights cannot be read as packed words by mistake.
 *  - Arithmetic: w' = fp32(weight * routed_scaling_factor); acc = +0; for each
 *    slot k in ascending order acc = acc + w'_k * x_k (separate fp32 multiply
 *    and add, no fused multiply-add); acc = acc + shared; [acc = acc +
 *    residual]; one round-to-nearest-even to bf16. The routed scaling factor
 *    never scales the shared-expert output. Non-finite values propagate
 *    through that arithmetic (an fp32 overflow of the sum gives inf); the
 *    sign of a NaN the arithmetic creates (inf - inf) is not specified.
 *  - Alignment: bf16 row tensors (gemm2_out, shared_out, out, residual,
 *    residual_out, normed, gamma) 16-byte aligned; FP8 output 8-byte aligned;
 *    index and weight tensors 4-byte aligned. Else MOEF_ERR_MISALIGNED.
 *  - Aliasing: outputs may not overlap inputs or each other
 *    (MOEF_ERR_BAD_ALIAS), except that residual_out may be exactly residual
 *    (in-place residual update). err_flag counts as an output.
 */
#ifndef MOE_FINALIZE_H
#define MOE_FINALIZE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEF_ABI_VERSION 1
#define MOEF_MAX_TOP_K 16            /* top_k must lie in [1, 16] */
#define MOEF_MAX_HIDDEN 1048576      /* hidden must lie in [8, 2^20], multiple of 8 */
#define MOEF_MAX_HIDDEN_RMSNORM 16384 /* the RMSNorm epilogue keeps a row on chip */
#define MOEF_QUANT_BLOCK 128         /* the UE8M0 epilogue needs hidden % 128 == 0 */
#define MOEF_MAX_GATE_EXPERTS 512    /* the gate keeps a token's logits in registers */
#define MOEF_MAX_EP_PARTIALS 64      /* partials one combine call may sum */
#define MOEF_MAX_AR_RANKS 16         /* rank outputs one all-reduce call may sum */
/* Launch-size limits. A kernel dispatch packet counts a grid's work-items in
 * 32 bits, so one launch covers at most 2^32 - 1 of them. A call may therefore
 * hold at most MOEF_MAX_UNITS one-wave units (a token's 512-column chunk, or
 * one token of the gate) or MOEF_MAX_ITEMS one-lane items (16-byte vectors of
 * the combine, words of the decoder); beyond them it returns
 * MOEF_ERR_UNSUPPORTED. */
#define MOEF_MAX_UNITS 67108860LL    /* 2^26 - 4 */
#define MOEF_MAX_ITEMS 4294967040LL  /* 2^32 - 256 */

#define MOEF_DEVERR_INDEX_OUT_OF_RANGE 1

enum moef_status {
  MOEF_OK = 0,
  MOEF_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  MOEF_ERR_BAD_SHAPE = 2,    /* negative count, hidden/top_k out of range */
  MOEF_ERR_UNSUPPORTED = 3,  /* hidden not a multiple of 8 (or 128 for quant), too large */
  MOEF_ERR_MISALIGNED = 4,   /* a pointer breaks the alignment rule */
  MOEF_ERR_BAD_FORMAT = 5,   /* not exactly one routing-weight format given */
  MOEF_ERR_BAD_ALIAS = 6,    /* an output overlaps an input or another output */
  MOEF_ERR_HIP = 7           /* the HIP runtime rejected a launch */
};

/*
 * moe_finalize - deferred finalize, bf16 out.
 * ("Support deferred MoE finalize for MXFP4 and FP8 block-scale", Motivation
 *  and Modifications item 2.)
 *
 *  gemm2_out   bf16 [num_rows, hidden]: expert-sorted, padded, un-weighted
 *              expert outputs. Only rows named by the index map are read, so
 *              padding may hold anything (NaN) and cost does not grow with
 *              num_rows. May be NULL only if num_rows == 0.
 *  num_rows    P >= 0, rows in gemm2_out; at most 2^31 - 1 (rows are named
 *              by int32 indices), else MOEF_ERR_UNSUPPORTED.
 *  expanded_idx_to_permuted_idx  int32 [num_tokens, top_k]: the gemm2_out
 *              row of slot (t, k), at element t * top_k + k.
 *  topk_weights / topk_packed    routing weights, exactly one non-NULL.
 *  shared_out  bf16 [num_tokens, hidden] or NULL (no shared expert).
 *  routed_scaling_factor         folded into every routed weight (1.0: none).
 *  out         bf16 [num_tokens, hidden], written.
 *  err_flag    optional device int32 (see conventions).
 *  num_tokens, hidden, top_k  shape rules of the conventions, and
 *              num_tokens * ceil(hidden / 512) <= MOEF_MAX_UNITS (one wave
 *              per 512-column chunk of a token), else MOEF_ERR_UNSUPPORTED.
 */
int moe_finalize(const uint16_t* gemm2_out, int64_t num_rows,
                 const int32_t* expanded_idx_to_permuted_idx,
                 const float* topk_weights, const int32_t* topk_packed,
                 const uint16_t* shared_out, float routed_scaling_factor,
                 uint16_t* out,
                 int64_t num_tokens, int64_t hidden, int32_t top_k,
                 int32_t* err_flag, void* stream);

/*
 * moe_finalize_residual_rmsnorm - finalize + residual add + RMSNorm.
 * ("[Kimi K2.5] Fuse deferred MoE finalize into next-layer AR + residual +
 *  RMSNorm", Summary and "Numerics & speed"; on one GPU the all-reduce is the
 *  identity.)
 *
 *  Routed arguments as moe_finalize, plus
 *  residual      bf16 [num_tokens, hidden].
 *  gamma         bf16 [hidden], the RMSNorm weight.
 *  eps           added to the mean square inside the square root.
 *  residual_out  bf16 [num_tokens, hidden] = bf16(acc + residual) with one
 *                rounding; may be exactly `residual` (in place).
 *  normed        bf16 [num_tokens, hidden] =
 *                bf16(ro / sqrt(mean_h(ro^2) + eps) * gamma), ro being the
 *                stored bf16 residual_out, computed in fp32; not
 *                specified for a token whose residual_out holds inf or NaN.
 *  hidden        at most MOEF_MAX_HIDDEN_RMSNORM.
 */
int moe_finalize_residual_rmsnorm(const uint16_t* gemm2_out, int64_t num_rows,
                                  const int32_t* expanded_idx_to_permuted_idx,
                                  const float* topk_weights, const int32_t* topk_packed,
                                  const uint16_t* shared_out, float routed_scaling_factor,
                                  const uint16_t* residual, const uint16_t* gamma, float eps,
                                  uint16_t* residual_out, uint16_t* normed,
                                  int64_t num_tokens, int64_t hidden, int32_t top_k,
                                  int32_t* err_flag, void* stream);

/*
 * moe_finalize_quant_ue8m0 - finalize + FP8 E4M3 quantization with one
 * power-of-two scale per 1 x 128 block along hidden.
 * ("[FP8][MoE] Honor UE8M0 activation scales in Triton MoE", Motivation and
 *  "More context".)
 *
 *  Routed arguments as moe_finalize, plus
 *  out_e4m3    uint8 [num_tokens, hidden], OCP E4M3 ("e4m3fn", max 448) codes
 *              of y * 2^-e, y being the bf16-rounded finalize result; nearest
 *              even, subnormals kept, sign of zero kept.
 *  scale_e8m0  uint8 [num_tokens, hidden / 128], the byte e + 127 where e is
 *              the least integer with max|y over the block| <= 448 * 2^e,
 *              clamped to [-127, 127] (an all-zero block gives e = -127).
 *              A block where y holds inf or NaN gets e = 127; its finite
 *              values encode as above and each non-finite one gets an E4M3
 *              NaN code (0x7F or 0xFF, the sign not specified).
 *  hidden      a multiple of 128.
 */
int moe_finalize_quant_ue8m0(const uint16_t* gemm2_out, int64_t num_rows,
                             const int32_t* expanded_idx_to_permuted_idx,
                             const float* topk_weights, const int32_t* topk_packed,
                             const uint16_t* shared_out, float routed_scaling_factor,
                             uint8_t* out_e4m3, uint8_t* scale_e8m0,
                             int64_t num_tokens, int64_t hidden, int32_t top_k,
                             int32_t* err_flag, void* stream);

/*
 * moe_finalize_ep_combine - sum of expert-parallel finalize partials.
 * The finalize is linear, so with the experts sharded over R ranks each rank
 * can run moe_finalize on its own slots only (every other slot's index set to
 * -1, which the finalize skips) and without the shared-expert output; this
 * call adds the R partials and the shared output, once. ("[Deepseek V4] Keep
 * fp32 routing weights in the mxfp4 trtllm MoE", follow-up commit: a TP4 /
 * EP4 deployment; "[Kimi K2.5] Fuse deferred MoE finalize into next-layer AR
 * + residual + RMSNorm", "Numerics & speed": the cross-rank reduction runs
 * over the finalized rows.) On one GPU the partials arrive in one buffer.
 *
 *  partials     bf16 [num_partials, num_tokens, hidden], rank-major.
 *  num_partials R in [1, MOEF_MAX_EP_PARTIALS].
 *  shared_out   bf16 [num_tokens, hidden] or NULL.
 *  out          bf16 [num_tokens, hidden] = bf16(+0 + p_0 + ... + p_{R-1}
 *               [+ shared]), fp32 adds in rank order, one rounding.
 *  hidden       a multiple of 8. num_tokens == 0 is a no-op.
 *  Errors: num_tokens < 0, hidden < 1 or num_partials outside
 *  [1, MOEF_MAX_EP_PARTIALS] give BAD_SHAPE; hidden not a multiple of 8 or
 *  above MOEF_MAX_HIDDEN, or num_tokens * hidden / 8 above MOEF_MAX_ITEMS,
 *  give UNSUPPORTED; a NULL partials or out gives NULL_POINTER; a pointer
 *  that is not 16-byte aligned gives MISALIGNED; out overlapping the partials
 *  or shared_out gives BAD_ALIAS.
 */
int moe_finalize_ep_combine(const uint16_t* partials, int32_t num_partials,
                            const uint16_t* shared_out, uint16_t* out,
                            int64_t num_tokens, int64_t hidden, void* stream);

/*
 * moe_allreduce_residual_rmsnorm - the part one GPU runs of the all-reduce +
 * residual + RMSNorm that follows the deferred finalize when the MoE layer is
 * split over R ranks. ("[Kimi K2.5] Fuse deferred MoE finalize into
 * next-layer AR + residual + RMSNorm", Numerics & speed vs the
 * separate-finalize fallback: the preferred path is the deferred finalize
 * followed by an all-reduce + residual + RMSNorm kernel that emits
 * residual_out and accumulates in fp32.) Each input is one rank's
 * moe_finalize output: its tensor-parallel partial sum, or its
 * expert-parallel slots. The shared-expert output is inside those outputs
 * (each rank adds its share, or one rank adds all of it). On a multi-GPU node
 * the pointers are the peers' buffers mapped into this process; on one GPU
 * they are local buffers.
 *
 *  rank_outputs  host array of num_ranks device pointers, each bf16
 *                [num_tokens, hidden]. The array is read during the call only;
 *                the pointers go to the kernel by value.
 *  num_ranks     R in [1, MOEF_MAX_AR_RANKS].
 *  residual      bf16 [num_tokens, hidden].
 *  gamma         bf16 [hidden].
 *  residual_out  bf16 [num_tokens, hidden] = bf16(+0 + o_0 + ... + o_{R-1}
 *                + residual): fp32 adds in that order, one rounding. May be
 *                residual itself (in-place update), but no other overlap.
 *  normed        bf16 [num_tokens, hidden] = bf16(residual_out *
 *                rsqrt(mean(residual_out^2) + eps) * gamma), fp32 math; must
 *                not overlap any input or residual_out.
 *  hidden        a multiple of 8, at most MOEF_MAX_HIDDEN_RMSNORM.
 *  num_tokens == 0 is a no-op.
 *  Errors: R outside [1, MOEF_MAX_AR_RANKS], num_tokens < 0 or hidden < 1
 *  give BAD_SHAPE; hidden not a multiple of 8, hidden above the limit or
 *  num_tokens * ceil(hidden / 512) above MOEF_MAX_UNITS give UNSUPPORTED; a NULL array, rank pointer or
 *  buffer gives NULL_POINTER; a pointer that is not 16-byte aligned gives
 *  MISALIGNED; the overlaps above give BAD_ALIAS.
 */
int moe_allreduce_residual_rmsnorm(const uint16_t* const* rank_outputs, int32_t num_ranks,
                                   const uint16_t* residual, const uint16_t* gamma, float eps,
                                   uint16_t* residual_out, uint16_t* normed,
                                   int64_t num_tokens, int64_t hidden, void* stream);

/*
 * moe_topk_packed_decode - split packed routing words.
 * ("[Deepseek V4] Keep fp32 routing weights in the mxfp4 trtllm MoE",
 *  PR description.)
 *
 *  packed      int32 [n], (expert_id << 16) | bf16_bits(weight).
 *  expert_ids  int32 [n] = (uint32)packed >> 16, or NULL to skip.
 *  weights     float32 [n] = the bf16 weight widened exactly, or NULL.
 *  At least one output must be non-NULL. n == 0 is a no-op.
 *  Errors: n < 0 gives BAD_SHAPE; n above MOEF_MAX_ITEMS gives UNSUPPORTED;
 *  a NULL packed, or both outputs NULL, gives NULL_POINTER; a pointer that is
 *  not 4-byte aligned gives MISALIGNED; an output that overlaps packed or the
 *  other output gives BAD_ALIAS.
 */
int moe_topk_packed_decode(const int32_t* packed, int64_t n,
                           int32_t* expert_ids, float* weights, void* stream);

/*
 * moe_topk_sigmoid_gate - the routing front-end that feeds the finalize:
 * top_k experts per token from router logits, with fp32 weights and/or the
 * packed words. ("[Deepseek V4] Keep fp32 routing weights in the mxfp4
 * trtllm MoE", PR description: the gate produces fp32 routing weights, and
 * packing them into (expert_id << 16) | bf16(weight) truncates them.)
 *
 *  router_logits  float32 [num_tokens, num_experts].
 *  num_experts    E in [1, MOEF_MAX_GATE_EXPERTS].
 *  top_k          in [1, min(E, MOEF_MAX_TOP_K)].
 *  topk_ids       int32 [num_tokens, top_k], written: the top_k largest logits
 *                 (= the top_k sigmoid scores), in descending order; ties go to
 *                 the lower expert id; NaN logits rank below every number.
 *  topk_weights   float32 [num_tokens, top_k] or NULL: sigmoid(logit) of each
 *                 chosen expert divided by their sum (fp32; the routed scaling
 *                 factor is not applied here).
 *  topk_packed    int32 [num_tokens, top_k] or NULL: (id << 16) | bf16 bits of
 *                 the weight, rounded to nearest even.
 *  num_tokens == 0 is a no-op.
 *  Errors: num_tokens < 0, num_experts < 1 or top_k outside [1, min(E, 16)]
 *  give BAD_SHAPE; num_experts above MOEF_MAX_GATE_EXPERTS or num_tokens
 *  above MOEF_MAX_UNITS give UNSUPPORTED; a NULL router_logits or topk_ids gives
 *  NULL_POINTER; a pointer that is not 4-byte aligned gives MISALIGNED; an
 *  output that overlaps the logits or another output gives BAD_ALIAS.
 */
int moe_topk_sigmoid_gate(const float* router_logits, int64_t num_tokens,
                          int32_t num_experts, int32_t top_k,
                          int32_t* topk_ids, float* topk_weights, int32_t* topk_packed,
                          void* stream);

/*
 * moe_act_quant_fp8_ue8m0 / moe_act_quant_fp8_amax - standalone FP8 E4M3
 * activation quantization with one FP32 scale per 1 x 128 block along hidden,
 * for the activations entering the expert linear layers ("[FP8][MoE] Honor
 * UE8M0 activation scales in Triton MoE", Motivation and "More context").
 *
 *  x           bf16 [num_tokens, hidden], finite values (a NaN or inf makes
 *              its block's codes unspecified).
 *  hidden      a multiple of 128.
 *  out_e4m3    uint8 [num_tokens, hidden], OCP E4M3 codes.
 *  _ue8m0:     power-of-two scales, the finalize epilogue's rule:
 *              scale_e8m0 uint8 [num_tokens, hidden / 128] = e + 127, e the
 *              least integer with max|x| <= 448 * 2^e (clamped to [-127, 127]),
 *              codes = e4m3(x / 2^e).
 *  _amax:      the continuous policy the pages replace, for comparison:
 *              scale_f32 float32 [num_tokens, hidden / 128] = max|x| / 448
 *              (correctly rounded fp32; 1 for an all-zero block),
 *              codes = e4m3(fp32(x / scale)), nearest even.
 *  num_tokens == 0 is a no-op.
 *  Errors: num_tokens < 0 or hidden < 1 give BAD_SHAPE; hidden not a
 *  multiple of 128 or above MOEF_MAX_HIDDEN, or num_tokens * ceil(hidden /
 *  512) above MOEF_MAX_UNITS give UNSUPPORTED; a NULL x,
 *  out_e4m3 or scale gives NULL_POINTER (a NULL scale is reported before the
 *  shape checks when num_tokens > 0); x not 16-, out_e4m3 not 8- or
 *  scale_f32 not 4-byte aligned gives MISALIGNED; an output that overlaps x
 *  or the other output gives BAD_ALIAS.
 */
int moe_act_quant_fp8_ue8m0(const uint16_t* x, int64_t num_tokens, int64_t hidden,
                            uint8_t* out_e4m3, uint8_t* scale_e8m0, void* stream);
int moe_act_quant_fp8_amax(const uint16_t* x, int64_t num_tokens, int64_t hidden,
                           uint8_t* out_e4m3, float* scale_f32, void* stream);

/* Operations moe_finalize_describe_launch describes. */
enum moef_op {
  MOEF_OP_FINALIZE = 0,           /* moe_finalize */
  MOEF_OP_RESIDUAL_RMSNORM = 1,   /* moe_finalize_residual_rmsnorm */
  MOEF_OP_QUANT_UE8M0 = 2         /* moe_finalize_quant_ue8m0 */
};

/*
 * moe_finalize_describe_launch - which kernel a finalize call of this shape
 * launches on the device of `stream`, and how many launches of what grid.
 * It computes nothing and launches nothing: benchmarks and profiles use it
 * to name the kernel they time. (No page defines it; the kernels it names
 * implement the operations above.)
 *
 *  op          a MOEF_OP_* value.
 *  num_tokens, hidden, top_k  as the call's, under the same shape rules.
 *  stream      its device's CU count sizes the staged (one workgroup per CU)
 *              kernels; the count of each device is queried once and kept.
 *  buf         receives one NUL-terminated line, cut to buf_len - 1 bytes:
 *              the kernel as profilers print it, e.g.
 *              "finalize_quant_staged_kernel<8, true, 12> launches=1
 *              grid=616x1024 groups=8 tail=5%" (workgroups x lanes).
 *  Errors: a NULL buf or buf_len < 1 gives NULL_POINTER; an unknown op gives
 *  BAD_SHAPE; the call's shape rules give BAD_SHAPE or UNSUPPORTED.
 */
int moe_finalize_describe_launch(int32_t op, int64_t num_tokens, int64_t hidden, int32_t top_k,
                                 void* stream, char* buf, int64_t buf_len);

/* Human-readable text of a status code (static storage, never NULL). */
const char* moe_finalize_status_string(int status);

/* MOEF_ABI_VERSION of the built library. */
int moe_finalize_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FINALIZE_H */
