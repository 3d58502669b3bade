"""Pins for the expert-parallel partial finalize and combine oracle (CPU)."""
from fractions import Fraction

import numpy as np

from oracle import finalize as O
from oracle import formats as F
from combine_moe_finalize_amd import workloads as W

from test_oracle_finalize import frac_bf16


def test_rank_slots_partition_every_slot_once():
    wl = W.make_workload(200, 64, 256, 8, seed=1)
    for R in (1, 2, 4, 8, 3):
        held = np.stack([O.ep_rank_slots(wl.expert_ids, 256, R, r) for r in range(R)])
        assert np.all(held.sum(0) == 1)


def test_partials_sum_to_the_full_finalize_before_rounding():
    wl = W.make_workload(64, 256, 32, 4, rsf=2.5, seed=2, pad=16)
    full, _ = O.finalize_truth_f64(wl.gemm2_out, wl.idx, weights_f32=wl.weights, rsf=wl.rsf)
    parts = []
    for r in range(4):
        idx_r = O.ep_partial_index(wl.idx, wl.expert_ids, 32, 4, r)
        p, flag = O.finalize_truth_f64(wl.gemm2_out, idx_r, weights_f32=wl.weights, rsf=wl.rsf)
        assert flag == 0
        parts.append(p)
    assert np.allclose(np.sum(parts, axis=0), full, rtol=0, atol=1e-12 * np.abs(full).max())


def test_local_rows_with_offset_match_global_rows():
    """A rank whose local gemm2_out is a slice starting at its first row gives
    the same partial as the global buffer with the global index map."""
    wl = W.make_workload(48, 128, 16, 4, rsf=1.5, seed=3, pad=8)
    counts = np.bincount(wl.expert_ids.reshape(-1), minlength=16)
    starts = np.concatenate([[0], np.cumsum(((counts + 7) // 8) * 8)])
    R = 4
    per = 16 // R
    for r in range(R):
        lo, hi = starts[r * per], starts[(r + 1) * per]
        g_idx = O.ep_partial_index(wl.idx, wl.expert_ids, 16, R, r)
        l_idx = O.ep_partial_index(wl.idx, wl.expert_ids, 16, R, r, row_offset=lo)
        a, _ = O.finalize_mirror(wl.gemm2_out, g_idx, weights_f32=wl.weights, rsf=wl.rsf)
        b, _ = O.finalize_mirror(wl.gemm2_out[lo:hi], l_idx, weights_f32=wl.weights, rsf=wl.rsf)
        assert np.array_equal(a, b)


def test_combine_identity_and_single_partial():
    rng = np.random.default_rng(4)
    p = W.to_bf16_bits(rng.standard_normal((1, 8, 64)).astype(np.float32))
    assert np.array_equal(F.bf16_to_f64(O.ep_combine_mirror(p)), F.bf16_to_f64(p[0]))
    sh = W.to_bf16_bits(rng.standard_normal((8, 64)).astype(np.float32))
    z = np.zeros((3, 8, 64), np.uint16)
    z[1] = p[0]
    want = F.bf16_bits(F.bf16_to_f64(p[0]) + F.bf16_to_f64(sh))
    assert np.array_equal(O.ep_combine_mirror(z, sh), want)


def test_combine_exact_rational():
    """Values within a narrow binade range keep every fp32 partial sum exact,
    so the combine must equal the exactly rounded rational sum."""
    rng = np.random.default_rng(5)
    R, T, H = 4, 3, 32
    p = W.to_bf16_bits(rng.uniform(-4, 4, (R, T, H)).astype(np.float32))
    sh = W.to_bf16_bits(rng.uniform(-4, 4, (T, H)).astype(np.float32))
    got = F.bf16_to_f64(O.ep_combine_mirror(p, sh))
    for t in range(T):
        for h in range(H):
            q = sum(Fraction(float(F.bf16_to_f64(p[r, t, h]))) for r in range(R)) + \
                Fraction(float(F.bf16_to_f64(sh[t, h])))
            assert got[t, h] == frac_bf16(q)
    assert np.array_equal(O.ep_combine_truth(p, sh), O.ep_combine_mirror(p, sh))
