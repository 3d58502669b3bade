"""GPU parity of the staged path of the all-reduce + residual + RMSNorm step.

From 20 (token, 512-column chunk) units per CU the step runs one workgroup
per CU that owns whole tokens, takes their units from an LDS counter, keeps
each unit's residual_out vector and chunk sum of squares in LDS (158 units a
workgroup) and writes residual_out and normed after its last read; grids
larger than that take several launches. These tests size their grids from
the device's CU count so that each case lands on the staged path, and check
residual_out bit for bit against the oracle's fp32 mirror, normed within one
bf16 ulp of its fp64 RMSNorm, and that the staged path gives the same bits as
the one-workgroup-per-token kernel on the same tokens."""
import numpy as np
import pytest
import torch

import combine_moe_finalize_amd as M
from combine_moe_finalize_amd import workloads as W

from gpu_helpers import DEV, announce, d_bf16, h_bits
from test_gpu_allreduce import check

pytestmark = pytest.mark.gpu

STAGED_FROM_UNITS_PER_CU = 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    M.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def ncu():
    return torch.cuda.get_device_properties(0).multi_processor_count


def chunks(H):
    return (H // 8 + 63) // 64


def inputs(R, T, H, seed):
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.uniform(-3, 3, (R, T, 1)))
    parts = W.to_bf16_bits((rng.standard_normal((R, T, H)) * mag).astype(np.float32))
    res = W.to_bf16_bits((rng.standard_normal((T, H)) * 4).astype(np.float32))
    gam = W.to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    return parts, res, gam


@pytest.mark.parametrize("R,H,units_per_cu", [
    (8, 7168, 44),         # one launch, 3-4 tokens a workgroup
    (3, 7168, 200),        # guarded rank count, two launches
    (16, 7168, 60),        # the most ranks
    (1, 1000, 60),         # two chunks a token, the second one ragged
    (2, 16384, 140),       # 32 chunks a token: 4 tokens a workgroup, several launches
])
def test_staged_step(ncu, R, H, units_per_cu):
    T = -(-units_per_cu * ncu // chunks(H))
    parts, res, gam = inputs(R, T, H, seed=R * 100 + H)
    announce(f"staged allreduce R={R} T={T} H={H}")
    ro, nm = M.moe_allreduce_residual_rmsnorm(d_bf16(parts), residual=d_bf16(res),
                                              gamma=d_bf16(gam), eps=1e-6)
    torch.cuda.synchronize()
    check(parts, res, gam, 1e-6, h_bits(ro), h_bits(nm), f"staged R={R} T={T} H={H}")


def test_staged_equals_per_token_and_in_place(ncu):
    """The first 40 tokens alone (one workgroup per token) and inside a staged
    batch give the same bits; the staged call writes residual_out over
    residual, from separately allocated rank buffers."""
    R, H = 6, 7168
    T = -(-(STAGED_FROM_UNITS_PER_CU + 5) * ncu // chunks(H))
    parts, res, gam = inputs(R, T, H, seed=77)
    bufs = [d_bf16(parts[r]) for r in range(R)]
    d_res = d_bf16(res)
    g = d_bf16(gam)
    announce(f"staged allreduce in place R={R} T={T} H={H} against 40 tokens")
    small_ro, small_nm = M.moe_allreduce_residual_rmsnorm(
        [b[:40].contiguous() for b in bufs], residual=d_res[:40].clone(), gamma=g, eps=1e-6)
    ro, nm = M.moe_allreduce_residual_rmsnorm(bufs, residual=d_res, gamma=g, eps=1e-6,
                                              residual_out=d_res)
    torch.cuda.synchronize()
    assert ro.data_ptr() == d_res.data_ptr()
    assert torch.equal(ro[:40].view(torch.int16), small_ro.view(torch.int16))
    assert torch.equal(nm[:40].view(torch.int16), small_nm.view(torch.int16))
    check(parts, res, gam, 1e-6, h_bits(ro), h_bits(nm), "staged in place")


def test_threshold_boundary(ncu):
    """The last grid of the one-workgroup-per-token kernel and the first
    staged one."""
    R, H = 4, 7168
    units = STAGED_FROM_UNITS_PER_CU * ncu
    for T in (units // chunks(H) - (units % chunks(H) == 0), -(-units // chunks(H))):
        parts, res, gam = inputs(R, T, H, seed=T)
        announce(f"allreduce at the staged threshold R={R} T={T} H={H}")
        ro, nm = M.moe_allreduce_residual_rmsnorm(d_bf16(parts), residual=d_bf16(res),
                                                  gamma=d_bf16(gam), eps=1e-6)
        torch.cuda.synchronize()
        check(parts, res, gam, 1e-6, h_bits(ro), h_bits(nm), f"threshold T={T}")
