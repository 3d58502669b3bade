"""CPU oracle for the standalone FP8 activation quantization (1 x 128 blocks).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"[FP8][MoE] Honor UE8M0 activation scales in Triton MoE" (Motivation): the
activations entering each expert linear layer are quantized to FP8 with FP32
scales per block; the checkpoint's `scale_fmt: ue8m0` asks for power-of-two
scales, where the older path used the continuous `amax / 448`. Both policies
are given here so they can be compared:

  * power-of-two (UE8M0): exactly the finalize epilogue's rule
    (``finalize.quant_ue8m0``): e = least integer with amax <= 448 * 2^e,
    code byte e + 127, q = e4m3(x / 2^e);
  * continuous: s = fp32(amax / 448) (one correctly rounded fp32 division;
    an all-zero block takes s = 1), q = e4m3(fp32(x / s)) (a second correctly
    rounded fp32 division, then one nearest-even rounding to E4M3); the scale
    is returned as float32.

Readings: Q1 the block is 1 x 128 along the
hidden dimension (the workload's block); Q2, Q3 the continuous scale and
codes as above; Q4 inputs are finite bf16 (a NaN or inf input makes its
block's codes unspecified).
"""
from __future__ import annotations

import numpy as np

from . import finalize as FZ
from . import formats as F

QUANT_BLOCK = 128


def act_quant_ue8m0(x_bits, block=QUANT_BLOCK):
    """(codes uint8 [T, H], scale bytes uint8 [T, H/block])."""
    codes, scales, _ = FZ.quant_ue8m0(x_bits, block)
    return codes, scales


def act_quant_amax(x_bits, block=QUANT_BLOCK):
    """(codes uint8 [T, H], scales float32 [T, H/block]) for s = amax / 448."""
    x = F.bf16_to_f32(x_bits)
    T, H = x.shape
    if H % block:
        raise ValueError("H must be a multiple of the quant block")
    xb = x.reshape(T, H // block, block)
    amax = np.max(np.abs(xb), axis=-1)                          # exact
    s = np.where(amax > 0, amax / np.float32(F.E4M3_MAX), np.float32(1.0)).astype(np.float32)
    ratio = (xb / s[..., None]).astype(np.float32)              # fp32 division
    codes = F.e4m3_encode(ratio.astype(np.float64)).reshape(T, H)
    return codes, s
