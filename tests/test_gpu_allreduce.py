"""GPU parity of the all-reduce + residual + RMSNorm step (one GPU's share)
against the CPU oracle. residual_out is bit-exact to the oracle's fp32 mirror
(rank order, then the residual, one rounding). normed is within one bf16 ulp
of the oracle's fp64 RMSNorm of the same residual_out: the kernel's fp32 norm
is within a few 2^-24 of it, so only a value that close to a bf16 rounding
tie can land one ulp away."""
import json
import os

import numpy as np
import pytest
import torch

import combine_moe_finalize_amd as M
from combine_moe_finalize_amd import workloads as W
from oracle import finalize as O
from oracle import formats as F

from gpu_helpers import (DEV, announce, assert_bits_equal, d_bf16, d_f32, d_i32, h_bits,
                         ulp_bf16)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "allreduce_residual_rmsnorm.json")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    M.load_library()


def check(parts, res, gam, eps, ro, nm, what):
    m_ro, m_nm = O.allreduce_residual_rmsnorm_mirror(parts, res, gam, eps)
    assert_bits_equal(ro, m_ro, f"{what}: residual_out")
    g, o = F.bf16_to_f64(nm), F.bf16_to_f64(m_nm)
    d = np.abs(g - o)
    assert np.all(d <= ulp_bf16(o)), f"{what}: normed off by {np.max(d / ulp_bf16(o))} ulp"
    assert np.mean(nm == m_nm) > 0.99, f"{what}: too many normed values one ulp away"


def test_golden_fixture():
    g = json.load(open(GOLDEN))

    def bits(rows):
        return W.to_bf16_bits(np.array([[float(v) for v in r] for r in rows], np.float32))

    parts = np.stack([bits(p) for p in g["partials"]])
    res, gam = bits(g["residual"]), bits([g["gamma"]])[0]
    announce("allreduce golden fixture R=3 T=3 H=8")
    ro, nm = M.moe_allreduce_residual_rmsnorm([d_bf16(p) for p in parts], residual=d_bf16(res),
                                              gamma=d_bf16(gam), eps=g["eps"])
    torch.cuda.synchronize()
    assert_bits_equal(h_bits(ro), bits(g["residual_out"]), "residual_out", zero_equal=False)
    assert_bits_equal(h_bits(nm), bits(g["normed"]), "normed", zero_equal=False)


@pytest.mark.parametrize("R,T,H", [(1, 5, 1000), (2, 1, 7168), (3, 7, 7168), (5, 33, 1024),
                                   (8, 1, 7168), (8, 16, 7168), (8, 256, 7168), (16, 3, 16384),
                                   (7, 9, 8), (4, 2, 8200)])
def test_random_rank_outputs(R, T, H):
    rng = np.random.default_rng(R * 1000 + T + H)
    mag = np.exp2(rng.uniform(-3, 3, (R, T, 1)))
    parts = W.to_bf16_bits((rng.standard_normal((R, T, H)) * mag).astype(np.float32))
    res = W.to_bf16_bits((rng.standard_normal((T, H)) * 4).astype(np.float32))
    gam = W.to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    announce(f"allreduce R={R} T={T} H={H}")
    ro, nm = M.moe_allreduce_residual_rmsnorm(d_bf16(parts), residual=d_bf16(res),
                                              gamma=d_bf16(gam), eps=1e-6)
    torch.cuda.synchronize()
    check(parts, res, gam, 1e-6, h_bits(ro), h_bits(nm), f"R={R} T={T} H={H}")


def test_separate_rank_buffers_and_in_place():
    """Rank outputs in separately allocated buffers (as peers' buffers would
    be), and residual_out written over residual."""
    R, T, H = 6, 20, 7168
    rng = np.random.default_rng(3)
    parts = W.to_bf16_bits(rng.standard_normal((R, T, H)).astype(np.float32))
    res = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    gam = W.to_bf16_bits(rng.standard_normal(H).astype(np.float32))
    bufs = []
    for r in range(R):
        torch.empty(4096 * (r + 1), dtype=torch.uint8, device=DEV)   # spread the allocations
        bufs.append(d_bf16(parts[r]))
    d_res = d_bf16(res)
    announce(f"allreduce separate buffers, in place R={R} T={T} H={H}")
    ro, nm = M.moe_allreduce_residual_rmsnorm(bufs, residual=d_res, gamma=d_bf16(gam), eps=1e-5,
                                              residual_out=d_res)
    torch.cuda.synchronize()
    assert ro.data_ptr() == d_res.data_ptr()
    check(parts, res, gam, 1e-5, h_bits(ro), h_bits(nm), "in place")


def test_expert_parallel_chain_on_one_gpu():
    """Each of R ranks finalizes its own slots on the GPU (rank 0 adds the
    shared output); the all-reduce + residual + RMSNorm sums them. Every step
    is compared with the oracle's same chain."""
    wl = W.family_workload("residual_rmsnorm", 64)
    R = 4
    g2, w = d_bf16(wl.gemm2_out), d_f32(wl.weights)
    announce(f"allreduce EP chain R={R} T={wl.T} H={wl.H}")
    outs, o_parts = [], []
    for r in range(R):
        idx_r = O.ep_partial_index(wl.idx, wl.expert_ids, wl.E, R, r)
        sh = wl.shared if r == 0 else None
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        outs.append(M.moe_finalize(g2, d_i32(idx_r), topk_weights=w,
                                   shared_out=None if sh is None else d_bf16(sh),
                                   routed_scaling_factor=wl.rsf, err_flag=err))
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        p, _ = O.finalize_mirror(wl.gemm2_out, idx_r, weights_f32=wl.weights, shared=sh,
                                 rsf=wl.rsf)
        assert_bits_equal(h_bits(outs[r]), p, f"rank {r} finalize")
        o_parts.append(p)
    ro, nm = M.moe_allreduce_residual_rmsnorm(outs, residual=d_bf16(wl.residual),
                                              gamma=d_bf16(wl.gamma), eps=wl.eps)
    torch.cuda.synchronize()
    check(np.stack(o_parts), wl.residual, wl.gamma, wl.eps, h_bits(ro), h_bits(nm), "EP chain")


def test_empty_batch_and_errors():
    z = torch.empty((0, 7168), dtype=torch.bfloat16, device=DEV)
    gam = torch.ones(7168, dtype=torch.bfloat16, device=DEV)
    ro, nm = M.moe_allreduce_residual_rmsnorm([z, z], residual=z, gamma=gam)
    assert ro.shape == (0, 7168) and nm.shape == (0, 7168)
    x = torch.zeros((2, 7168), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(M.MoeFinalizeError):
        M.moe_allreduce_residual_rmsnorm([x] * 17, residual=x.clone(), gamma=gam)
    with pytest.raises(M.MoeFinalizeError):                        # normed over a rank output
        M.moe_allreduce_residual_rmsnorm([x, x.clone()], residual=x.clone(), gamma=gam, normed=x)
