"""GPU parity of expert-parallel partial finalize + combine.

With the experts split into R contiguous ranges, rank r's local gemm2_out is
the slice of rows of its experts, its index map holds its slots (shifted to
local rows) and -1 elsewhere, and it passes no shared output; the combine adds
the partials and the shared output once. Everything is checked bit-exactly
against the oracle's same chain (fp32 mirror partials, fp32 combine), and the
final result against the single-GPU fp64 truth within the bound the extra
rounding of each bf16 partial allows."""
import numpy as np
import pytest
import torch

import combine_moe_finalize_amd as M
from combine_moe_finalize_amd import workloads as W
from oracle import finalize as O
from oracle import formats as F

from gpu_helpers import (DEV, abs_terms, announce, assert_bits_equal, d_bf16, d_f32, d_i32,
                         h_bits, ulp_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    M.load_library()


@pytest.mark.parametrize("R,with_shared", [(1, False), (2, True), (4, True), (5, False), (8, True)])
def test_combine_direct(R, with_shared):
    T, H = 37, 1000
    rng = np.random.default_rng(R)
    p = W.to_bf16_bits((rng.standard_normal((R, T, H)) * np.exp2(rng.uniform(-4, 4, (R, T, 1)))
                        ).astype(np.float32))
    sh = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)) if with_shared else None
    announce(f"ep combine R={R} shared={with_shared}")
    out = M.moe_finalize_ep_combine(d_bf16(p), shared_out=None if sh is None else d_bf16(sh))
    torch.cuda.synchronize()
    assert_bits_equal(h_bits(out), O.ep_combine_mirror(p, sh), "combine")


def expert_row_starts(wl):
    counts = np.bincount(wl.expert_ids.reshape(-1), minlength=wl.E)
    return np.concatenate([[0], np.cumsum(((counts + 127) // 128) * 128)])


@pytest.mark.parametrize("R", [2, 4, 8])
def test_ep_chain_on_one_gpu(R):
    wl = W.family_workload("packed_vs_unpacked")
    starts = expert_row_starts(wl)
    per = wl.E // R
    g2 = d_bf16(wl.gemm2_out)
    w = d_f32(wl.weights)
    announce(f"ep chain R={R} T={wl.T} H={wl.H}")
    parts = torch.empty((R, wl.T, wl.H), dtype=torch.bfloat16, device=DEV)
    o_parts = []
    for r in range(R):
        lo, hi = int(starts[r * per]), int(starts[(r + 1) * per])
        idx_r = O.ep_partial_index(wl.idx, wl.expert_ids, wl.E, R, r, row_offset=lo)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        M.moe_finalize(g2[lo:hi], d_i32(idx_r), topk_weights=w, routed_scaling_factor=wl.rsf,
                       out=parts[r], err_flag=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        p, _ = O.finalize_mirror(wl.gemm2_out[lo:hi], idx_r, weights_f32=wl.weights, rsf=wl.rsf)
        o_parts.append(p)
        assert_bits_equal(h_bits(parts[r]), p, f"partial {r}")
    out = h_bits(M.moe_finalize_ep_combine(parts, shared_out=d_bf16(wl.shared)))
    torch.cuda.synchronize()
    o_parts = np.stack(o_parts)
    assert_bits_equal(out, O.ep_combine_mirror(o_parts, wl.shared), "combined")
    # against the single-GPU fp64 truth: each bf16 partial adds up to half an ulp
    truth, _ = O.finalize_truth_f64(wl.gemm2_out, wl.idx, weights_f32=wl.weights,
                                    shared=wl.shared, rsf=wl.rsf)
    r_ = F.bf16_round(truth)
    terms = abs_terms(wl.gemm2_out, wl.idx, weights=wl.weights, shared=wl.shared, rsf=wl.rsf)
    u = 2.0 ** -24
    n = wl.top_k + R + 2
    bound = (2 * ulp_bf16(r_) + 0.5 * ulp_bf16(F.bf16_to_f64(o_parts)).sum(0)
             + n * u / (1 - n * u) * terms)
    assert np.all(np.abs(F.bf16_to_f64(out) - r_) <= bound)
