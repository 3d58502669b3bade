"""CPU oracle for the deferred MoE finalize and its fused epilogues.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module; the HIP library and
its Python binding never do, and this module imports nothing from them.

What is computed (plain definition, written from the pages):

* Deferred finalize ("Support deferred MoE finalize for MXFP4 and FP8
  block-scale", Motivation): the MoE GEMM leaves *unweighted* per-expert
  output rows; a later kernel does the top-k weighted combine and merges the
  shared-expert addition into the same kernel.
* Routed scaling factor (same page, Modifications item 2): the factor is
  multiplied into the expert weight held in a register; 1.0 leaves results
  unchanged.
* Gather map (page "[Kimi K2.5] Fuse deferred MoE finalize into next-layer
  AR + residual + RMSNorm", Key modifications): expanded_idx_to_permuted_idx
  and expert_scale_factor are [token, top_k] tensors; the rows are gathered
  from the padded permuted gemm2_out buffer (same page, "Numerics & speed").
* Residual + RMSNorm epilogue emitting residual_out (same page, Summary and
  "Numerics & speed"), with fp32 accumulation preferred over a bf16 pipeline.
* Routing-weight formats ("[Deepseek V4] Keep fp32 routing weights in the
  mxfp4 trtllm MoE", PR description): fp32 weights, or the packed int32
  word (expert_id << 16) | bf16(weight).
* Power-of-two (UE8M0) FP8 activation scales ("[FP8][MoE] Honor UE8M0
  activation scales in Triton MoE", Motivation and "More context").

Readings taken where the pages are silent (R1, the fp32 operation order, is
the mirror mode below):
  R2, R3   out[t,h] = bf16( sum_k w'[t,k] * x[perm[t,k], h] + shared[t,h] ),
           w' = fp32(w * rsf); rsf scales routed experts only, never shared;
           shared is added into the accumulator before the rounding.
  R4       one rounding to bf16 (nearest even) at the very end.
  R5, R6   perm is token-major [T, top_k]; perm < 0 skips the slot (expert
           not local); perm >= P skips the slot and sets bit 0 of the error
           flag; P = 0 (no rows here) is allowed.
  R7       shared_out may be absent (zeros).
  R11, R12 residual_out = bf16(finalize_acc + residual) (one rounding);
           normed = bf16(ro / sqrt(mean(ro^2) + eps) * gamma) on the stored
           bf16 residual_out.
  R13-R18  OCP E4M3 (max 448); the quant input is the bf16-rounded finalize
           result y; per 1x128 block e = least integer with
           amax <= 448 * 2^e (clamp [-127, 127], amax 0 gives -127),
           q = e4m3(y * 2^-e) with ties to even and the sign of zero kept,
           scale byte e + 127, row-major [T, H/128].

Two modes:
  * ``*_truth``: fp64 gather, products and sums (each product w' * x is
    exact in fp64: 24 x 8 significand bits), one final rounding. This is
    the contract the GPU is checked against, within tolerance.
  * ``*_mirror``: the fp32 operation sequence the kernels are asked to
    follow, each op rounded to fp32 with no fused multiply-add:
    acc = +0; for k ascending: acc = acc + (w'_k * x_k); acc = acc + shared;
    [acc = acc + residual]; round to bf16. A GPU that follows the same
    sequence is bit-identical on out, residual_out, y, the UE8M0 exponents
    and the e4m3 codes; it decides the integer outputs (exponents, codes) in
    the kernel's precision.
"""
from __future__ import annotations

import numpy as np

from . import formats as F

ERR_INDEX_OUT_OF_RANGE = 1   # bit 0 of the device error flag
QUANT_BLOCK = 128            # 1 x 128 blocks along H


# ---------------------------------------------------------------- routing

def decode_packed(words):
    """Split packed routing words (expert_id << 16) | bf16_bits(weight).

    Returns (expert_ids as int32, weights as float32). The id is the upper
    16 bits read as unsigned (logical shift); the weight is the lower 16
    bits widened exactly from bfloat16.
    ("[Deepseek V4] Keep fp32 routing weights in the mxfp4 trtllm MoE",
    PR description.)"""
    u = np.asarray(words).astype(np.int32).view(np.uint32)
    ids = (u >> 16).astype(np.int32)
    w = F.bf16_to_f32((u & 0xFFFF).astype(np.uint16))
    return ids, w


def effective_weights(weights_f32, packed, rsf):
    """w' = fp32(w * rsf), the weight as held in a register after the routed
    scaling factor is folded in ("Support deferred MoE finalize for MXFP4 and
    FP8 block-scale", Modifications item 2). Exactly one of ``weights_f32``
    (float32 [T, k]) and ``packed`` (int32 [T, k]) is given."""
    if (weights_f32 is None) == (packed is None):
        raise ValueError("give exactly one of weights_f32 / packed")
    if packed is not None:
        _, w = decode_packed(packed)
    else:
        w = np.asarray(weights_f32, dtype=np.float32)
    return (w * np.float32(rsf)).astype(np.float32)   # one fp32 rounding


def slot_validity(idx, num_rows):
    """Readings R5, R6: which (t, k) slots are gathered, and the error flag."""
    idx = np.asarray(idx, dtype=np.int64)
    valid = (idx >= 0) & (idx < num_rows)
    flag = ERR_INDEX_OUT_OF_RANGE if np.any(idx >= num_rows) else 0
    return valid, flag


def _rows_or_zero(gemm2_out):
    """gemm2_out itself, or one zero row when it has none (a rank holding no
    expert of the batch): every slot is then skipped, and the row stands in
    only so that the skipped slots have something to index."""
    if gemm2_out.shape[0] > 0:
        return gemm2_out
    return np.zeros((1, gemm2_out.shape[1]), dtype=gemm2_out.dtype)


def _gather(gemm2_out, idx, valid):
    """float64 rows x[perm[t,k], :] for valid slots, 0 for skipped ones."""
    safe = np.where(valid, idx, 0)
    x = F.bf16_to_f64(_rows_or_zero(gemm2_out)[safe])   # [T, k, H]
    x[~valid] = 0.0
    return x


# ---------------------------------------------------------------- finalize

def finalize_truth_f64(gemm2_out, idx, weights_f32=None, packed=None,
                       shared=None, rsf=1.0):
    """fp64 finalize accumulator [T, H] before rounding (readings R2-R7),
    and the error flag. ``gemm2_out`` is uint16 bf16 bits [P, H]."""
    gemm2_out = np.asarray(gemm2_out, dtype=np.uint16)
    idx = np.asarray(idx)
    P = gemm2_out.shape[0]
    w = effective_weights(weights_f32, packed, rsf).astype(np.float64)
    valid, flag = slot_validity(idx, P)
    x = _gather(gemm2_out, idx, valid)
    acc = np.einsum("tk,tkh->th", np.where(valid, w, 0.0), x)
    if shared is not None:
        acc = acc + F.bf16_to_f64(shared)
    return acc, flag


def finalize_truth(gemm2_out, idx, weights_f32=None, packed=None,
                   shared=None, rsf=1.0):
    """bf16 bits [T, H] of the finalize result (fp64 math, one rounding)."""
    acc, flag = finalize_truth_f64(gemm2_out, idx, weights_f32, packed,
                                   shared, rsf)
    return F.bf16_bits(acc), flag


def finalize_mirror_f32(gemm2_out, idx, weights_f32=None, packed=None,
                        shared=None, rsf=1.0, residual=None):
    """The fp32 accumulator [T, H] in the kernels' operation order (see the
    module docstring), before the bf16 rounding; and the error flag."""
    gemm2_out = np.asarray(gemm2_out, dtype=np.uint16)
    idx = np.asarray(idx)
    P = gemm2_out.shape[0]
    T, K = idx.shape
    H = gemm2_out.shape[1]
    w = effective_weights(weights_f32, packed, rsf)
    valid, flag = slot_validity(idx, P)
    acc = np.zeros((T, H), dtype=np.float32)
    for k in range(K):
        rows = np.where(valid[:, k], idx[:, k], 0)
        x = F.bf16_to_f32(_rows_or_zero(gemm2_out)[rows])  # [T, H]
        prod = w[:, k, None] * x                            # fp32 multiply
        acc = np.where(valid[:, k, None], acc + prod, acc)  # fp32 add
    if shared is not None:
        acc = acc + F.bf16_to_f32(shared)
    if residual is not None:
        acc = acc + F.bf16_to_f32(residual)
    return acc, flag


def finalize_mirror(gemm2_out, idx, weights_f32=None, packed=None,
                    shared=None, rsf=1.0):
    """bf16 bits [T, H] of the finalize result in the kernels' fp32 order."""
    acc, flag = finalize_mirror_f32(gemm2_out, idx, weights_f32, packed,
                                    shared, rsf)
    return F.bf16_bits(acc), flag


# ------------------------------------------------------- residual + RMSNorm

def rmsnorm_f64(x_bits, gamma_bits, eps):
    """RMSNorm of bf16 rows in fp64, rounded once to bf16:
    y = x / sqrt(mean(x^2) + eps) * gamma (reading R11)."""
    x = F.bf16_to_f64(x_bits)
    g = F.bf16_to_f64(gamma_bits)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    inv = 1.0 / np.sqrt(ms + np.float64(np.float32(eps)))
    return F.bf16_bits(x * inv * g)


def finalize_residual_rmsnorm_truth(gemm2_out, idx, weights_f32=None,
                                    packed=None, shared=None, rsf=1.0,
                                    residual=None, gamma=None, eps=1e-6):
    """(residual_out bits, normed bits, flag) with fp64 math (readings R11, R12).
    ("[Kimi K2.5] Fuse deferred MoE finalize into next-layer AR + residual +
    RMSNorm", Summary: combine + shared add + residual + RMSNorm, keeping
    residual_out.)"""
    acc, flag = finalize_truth_f64(gemm2_out, idx, weights_f32, packed,
                                   shared, rsf)
    ro = F.bf16_bits(acc + F.bf16_to_f64(residual))
    return ro, rmsnorm_f64(ro, gamma, eps), flag


def finalize_residual_rmsnorm_mirror(gemm2_out, idx, weights_f32=None,
                                     packed=None, shared=None, rsf=1.0,
                                     residual=None, gamma=None, eps=1e-6):
    """Same outputs with residual_out in the kernels' fp32 order; normed is
    the fp64 RMSNorm of that residual_out (its reduction order is free)."""
    acc, flag = finalize_mirror_f32(gemm2_out, idx, weights_f32, packed,
                                    shared, rsf, residual=residual)
    ro = F.bf16_bits(acc)
    return ro, rmsnorm_f64(ro, gamma, eps), flag


# ------------------------------------------------------ UE8M0 FP8 quant

def quant_ue8m0(y_bits, block=QUANT_BLOCK):
    """Quantize bf16 rows [T, H] to OCP E4M3 codes [T, H] with one
    power-of-two scale per 1 x ``block`` block along H (readings R13-R18).
    Returns (codes uint8 [T, H], scale bytes uint8 [T, H/block],
    exponents int64 [T, H/block])."""
    y = F.bf16_to_f64(y_bits)
    T, H = y.shape
    if H % block:
        raise ValueError("H must be a multiple of the quant block")
    yb = y.reshape(T, H // block, block)
    amax = np.max(np.abs(yb), axis=-1)
    e = F.ue8m0_exponent(amax)
    scaled = yb * np.ldexp(1.0, -e)[..., None]     # exact power-of-two scale
    codes = F.e4m3_encode(scaled).reshape(T, H)
    return codes, F.ue8m0_code(e), e


def finalize_quant_truth(gemm2_out, idx, weights_f32=None, packed=None,
                         shared=None, rsf=1.0):
    """(codes, scale bytes, flag): quant of the fp64-truth finalize."""
    y, flag = finalize_truth(gemm2_out, idx, weights_f32, packed, shared, rsf)
    codes, scales, _ = quant_ue8m0(y)
    return codes, scales, flag


def finalize_quant_mirror(gemm2_out, idx, weights_f32=None, packed=None,
                          shared=None, rsf=1.0):
    """(codes, scale bytes, flag): quant of the fp32-mirror finalize, so the
    exponent and code decisions are taken in the kernels' precision."""
    y, flag = finalize_mirror(gemm2_out, idx, weights_f32, packed, shared, rsf)
    codes, scales, _ = quant_ue8m0(y)
    return codes, scales, flag


# ------------------------------------------------- expert-parallel partials

def ep_rank_slots(expert_ids, num_experts, num_ranks, rank):
    """Which slots a rank holds when experts are split into num_ranks
    contiguous, equal ranges (reading: EP shards the expert dimension)."""
    per = -(-num_experts // num_ranks)
    e = np.asarray(expert_ids)
    return (e >= rank * per) & (e < (rank + 1) * per)


def ep_partial_index(idx, expert_ids, num_experts, num_ranks, rank, row_offset=0):
    """The rank-local index map: a held slot's row minus the rank's first row
    (its local gemm2_out starts there), -1 for every other slot (skipped)."""
    held = ep_rank_slots(expert_ids, num_experts, num_ranks, rank)
    return np.where(held, np.asarray(idx, np.int64) - row_offset, -1).astype(np.int32)


def ep_combine_mirror(partials, shared=None):
    """Combine of bf16 partials [R, T, H] (readings: the finalize is linear, so
    each rank finalizes its own slots; the shared-expert output is added once,
    here): acc = +0; acc = acc + partial_r for r ascending; acc = acc + shared;
    one rounding to bf16. fp32 steps, as the combine kernel does them."""
    p = np.asarray(partials, dtype=np.uint16)
    acc = np.zeros(p.shape[1:], dtype=np.float32)
    for r in range(p.shape[0]):
        acc = acc + F.bf16_to_f32(p[r])
    if shared is not None:
        acc = acc + F.bf16_to_f32(shared)
    return F.bf16_bits(acc)


def ep_combine_truth(partials, shared=None):
    """Same, with the sum in float64 (one rounding)."""
    p = np.asarray(partials, dtype=np.uint16)
    acc = F.bf16_to_f64(p).sum(axis=0)
    if shared is not None:
        acc = acc + F.bf16_to_f64(shared)
    return F.bf16_bits(acc)


# ------------------------------------------------------------------------
# All-reduce + residual + RMSNorm after the deferred finalize, one GPU's share.
#
# "[Kimi K2.5] Fuse deferred MoE finalize into next-layer AR + residual +
# RMSNorm", "Numerics & speed vs the separate-finalize fallback": the
# preferred path under graph-captured decode is the deferred finalize followed
# by a separate all-reduce + residual + RMSNorm kernel that also emits
# residual_out and accumulates in fp32 (the fused kernel's extra error comes
# from accumulating inside the bf16 all-reduce pipeline). Readings:
#   AR1  the R inputs are the ranks' bf16 finalize outputs for the same tokens
#        (under TP each holds a partial sum; under EP each holds its slots);
#        they are added in fp32 from +0 in rank order, then the residual, and
#        the sum is rounded once to bf16: that is residual_out;
#   AR2  the shared-expert output is already inside the ranks' outputs (each
#        rank's finalize adds its own share), so it is not a separate input;
#   AR3  normed is the RMSNorm of the stored bf16 residual_out (reading R11).
# ------------------------------------------------------------------------

def allreduce_residual_rmsnorm_mirror(partials, residual, gamma, eps=1e-6):
    """(residual_out bits, normed bits) for bf16 rank outputs [R, T, H]:
    acc = +0; acc = acc + partial_r for r ascending; acc = acc + residual;
    residual_out = bf16(acc), in fp32 steps (readings AR1, AR2); normed is the
    fp64 RMSNorm of residual_out (AR3; its reduction order is free)."""
    p = np.asarray(partials, dtype=np.uint16)
    acc = np.zeros(p.shape[1:], dtype=np.float32)
    for r in range(p.shape[0]):
        acc = acc + F.bf16_to_f32(p[r])
    acc = acc + F.bf16_to_f32(residual)
    ro = F.bf16_bits(acc)
    return ro, rmsnorm_f64(ro, gamma, eps)


def allreduce_residual_rmsnorm_truth(partials, residual, gamma, eps=1e-6):
    """Same outputs with the rank sum and the residual add in float64 (one
    rounding to bf16)."""
    p = np.asarray(partials, dtype=np.uint16)
    acc = F.bf16_to_f64(p).sum(axis=0) + F.bf16_to_f64(residual)
    ro = F.bf16_bits(acc)
    return ro, rmsnorm_f64(ro, gamma, eps)
