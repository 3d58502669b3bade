"""Pins for the activation-quant oracle (CPU only)."""
import json
import os

import numpy as np

from oracle import act_quant as A
from oracle import formats as F
from combine_moe_finalize_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_amax_block():
    g = json.load(open(os.path.join(GOLDEN, "act_quant_amax.json")))
    head = g["block_values_head"]
    row = np.array(head + [0.0] * (128 - len(head)), dtype=np.float32)
    q, s = A.act_quant_amax(W.to_bf16_bits(row)[None, :])
    assert s[0, 0] == np.float32(g["scale"])
    assert [f"{c:02X}" for c in q[0, :len(head)]] == g["codes_head_hex"]
    assert np.all(q[0, len(head):] == 0)


def test_policies_agree_when_amax_over_448_is_a_power_of_two():
    """amax = 448 * 2^m makes the continuous scale exactly 2^m, the UE8M0
    exponent m: the two independently written policies must then agree."""
    rng = np.random.default_rng(1)
    T, H = 16, 1024
    x = rng.standard_normal((T, H)).astype(np.float32)
    xb = x.reshape(T, H // 128, 128)
    m = rng.integers(-20, 10, size=(T, H // 128))
    xb /= np.abs(xb).max(-1, keepdims=True)                    # |x| <= 1
    xb *= (448.0 * np.exp2(m))[..., None] * 0.999
    xb[:, :, 0] = 448.0 * np.exp2(m)                            # the block max
    bits = W.to_bf16_bits(xb.reshape(T, H))
    q1, s1 = A.act_quant_ue8m0(bits)
    q2, s2 = A.act_quant_amax(bits)
    assert np.array_equal(s1.astype(np.int64) - 127, m)
    assert np.array_equal(s2, np.exp2(m).astype(np.float32))
    assert np.array_equal(q1, q2)


def test_amax_policy_invariants():
    rng = np.random.default_rng(2)
    T, H = 64, 2048
    x = (rng.standard_normal((T, H)) * np.exp2(rng.uniform(-8, 8, (T, 1)))).astype(np.float32)
    x[3, 128:256] = 0.0                                          # a zero block
    bits = W.to_bf16_bits(x)
    q, s = A.act_quant_amax(bits)
    xv = F.bf16_to_f64(bits).reshape(T, H // 128, 128)
    qv = F.e4m3_decode(q).reshape(T, H // 128, 128)
    assert s[3, 1] == 1.0 and np.all(q[3, 128:256] == 0)
    nz = np.abs(xv).max(-1) > 0
    # the largest element of every nonzero block encodes to +-448
    top = np.abs(qv).max(-1)
    assert np.all(top[nz] == 448.0)
    # scale = amax / 448 within fp32 rounding
    amax = np.abs(xv).max(-1)
    assert np.all(np.abs(s[nz] - amax[nz] / 448) <= 2.0 ** -24 * amax[nz] / 448)
    # dequantized values within E4M3 rounding (plus the fp32 division)
    err = np.abs(qv * s[..., None] - xv)
    assert np.all(err <= 2.0 ** -4 * np.abs(xv) * (1 + 2.0 ** -20) + 2.0 ** -10 * s[..., None])


def test_ue8m0_policy_is_the_finalize_rule():
    rng = np.random.default_rng(3)
    bits = W.to_bf16_bits((rng.standard_normal((8, 512)) * 100).astype(np.float32))
    q, s = A.act_quant_ue8m0(bits)
    amax = np.abs(F.bf16_to_f64(bits)).reshape(8, 4, 128).max(-1)
    e = s.astype(np.int64) - 127
    assert np.all(amax <= 448 * np.exp2(e)) and np.all(amax > 448 * np.exp2(e - 1))
