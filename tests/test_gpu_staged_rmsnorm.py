"""GPU parity of the residual + RMSNorm epilogue's staged-output path.

From 40 (token, chunk) units per CU the epilogue runs one workgroup per CU
that owns whole tokens, keeps each unit's residual_out vector and sum of
squares in LDS (158 units per workgroup and launch) and writes residual_out
and normed after its last gather; larger grids take several launches. Its
results must equal the one-workgroup-per-token kernel's bit for bit (the
chunk sums are added in the same order), which the tests check by running
the same tokens in batches small enough for that kernel, and residual_out
must equal the oracle's fp32 mirror bit for bit."""
import numpy as np
import pytest
import torch

import combine_moe_finalize_amd as M
from combine_moe_finalize_amd import workloads as W
from oracle import finalize as O
from oracle import formats as F

from gpu_helpers import DEV, announce, assert_bits_equal, d_bf16, d_i32, device_inputs, \
    h_bits, ulp_bf16

pytestmark = pytest.mark.gpu

STAGED_FROM_UNITS_PER_CU = 40
RMS_LDS_UNITS = 158


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


def run(kw, res, gam, eps, ro=None, nm=None):
    ro, nm = M.moe_finalize_residual_rmsnorm(**kw, residual=res, gamma=gam, eps=eps,
                                             residual_out=ro, normed=nm)
    return ro, nm


def run_in_small_batches(kw, res, gam, eps, T, H, ncu):
    """The same tokens in batches below the staged threshold (the
    one-workgroup-per-token kernel)."""
    n = max(1, (STAGED_FROM_UNITS_PER_CU * ncu - 1) // chunks(H))
    ro = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    nm = torch.empty_like(ro)
    for t0 in range(0, T, n):
        sl = slice(t0, min(T, t0 + n))
        part = dict(kw)
        for key in ("expanded_idx_to_permuted_idx", "topk_weights", "topk_packed", "shared_out"):
            if key in part:
                part[key] = kw[key][sl].contiguous()
        run(part, res[sl].contiguous(), gam, eps, ro[sl], nm[sl])
    return ro, nm


def check_vs_mirror(wl, ro, nm, packed=False, idx=None, with_shared=True):
    idx = wl.idx if idx is None else idx
    wkw = dict(packed=wl.packed) if packed else dict(weights_f32=wl.weights)
    m_ro, m_nm, _ = O.finalize_residual_rmsnorm_mirror(
        wl.gemm2_out, idx, shared=wl.shared if with_shared else None, rsf=wl.rsf,
        residual=wl.residual, gamma=wl.gamma, eps=wl.eps, **wkw)
    assert_bits_equal(h_bits(ro), m_ro, "residual_out vs mirror")
    g, o = F.bf16_to_f64(h_bits(nm)), F.bf16_to_f64(m_nm)
    assert np.all(np.abs(g - o) <= ulp_bf16(o)), "normed within one ulp of the mirror chain"


def test_two_launches_equal_per_token_kernel(ncu):
    """H = 7168: 11 tokens per workgroup and launch; T past one launch's
    11 * ncu tokens takes two. Bit-identical to the per-token kernel."""
    H, k = 7168, 8
    T = 11 * ncu + 5 * ncu // 4
    wl = W.make_workload(T, H, 256, k, rsf=2.5, seed=900, with_residual=True)
    kw = device_inputs(wl)
    res, gam = d_bf16(wl.residual), d_bf16(wl.gamma)
    announce(f"staged rmsnorm two launches T={T} H={H} k={k}")
    ro, nm = run(kw, res, gam, wl.eps)
    ro_s, nm_s = run_in_small_batches(kw, res, gam, wl.eps, T, H, ncu)
    torch.cuda.synchronize()
    assert torch.equal(ro.view(torch.int16), ro_s.view(torch.int16)), "residual_out"
    assert torch.equal(nm.view(torch.int16), nm_s.view(torch.int16)), "normed"
    check_vs_mirror(wl, ro, nm)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7, 8])
def test_every_top_k(ncu, k):
    """H = 512: one chunk per token, 158 tokens per workgroup; 60 units per
    CU. Exact and guarded top_k, packed words for even k."""
    H = 512
    T = 60 * ncu
    wl = W.make_workload(T, H, 16, k, rsf=2.5, seed=910 + k, pad=64, with_residual=True)
    packed = k % 2 == 0
    kw = device_inputs(wl, packed=packed)
    announce(f"staged rmsnorm T={T} H={H} k={k} packed={packed}")
    ro, nm = run(kw, d_bf16(wl.residual), d_bf16(wl.gamma), wl.eps)
    torch.cuda.synchronize()
    check_vs_mirror(wl, ro, nm, packed=packed)


def test_ragged_row_no_shared_with_skipped_slots(ncu):
    """H = 7176: 15 chunks per token, the last with one active lane; no
    shared output; 5% of the slots skipped (index -1) and a few out of
    range (flagged)."""
    H, k = 7176, 6
    T = (STAGED_FROM_UNITS_PER_CU * ncu) // chunks(H) + 123
    wl = W.make_workload(T, H, 64, k, rsf=1.5, seed=920, pad=64, with_residual=True,
                         with_shared=False)
    rng = np.random.default_rng(920)
    idx = wl.idx.copy()
    idx[rng.random(idx.shape) < 0.05] = -1
    idx[rng.integers(0, T, 5), rng.integers(0, k, 5)] = wl.P + 11
    kw = device_inputs(wl, with_shared=False)
    kw["expanded_idx_to_permuted_idx"] = d_i32(idx)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    announce(f"staged rmsnorm ragged T={T} H={H} k={k} skipped slots")
    ro, nm = M.moe_finalize_residual_rmsnorm(**kw, residual=d_bf16(wl.residual),
                                             gamma=d_bf16(wl.gamma), eps=wl.eps, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == M.DEVERR_INDEX_OUT_OF_RANGE
    check_vs_mirror(wl, ro, nm, idx=idx, with_shared=False)


def test_in_place_residual_several_launches(ncu):
    """residual_out aliasing residual, over three launches (H = 2048: 4
    chunks, 39 tokens per workgroup and launch)."""
    H, k = 2048, 4
    tpw = RMS_LDS_UNITS // chunks(H)
    T = 2 * tpw * ncu + 17
    wl = W.make_workload(T, H, 64, k, rsf=2.5, seed=930, pad=128, with_residual=True)
    kw = device_inputs(wl)
    res = d_bf16(wl.residual)
    announce(f"staged rmsnorm in place T={T} H={H} k={k}")
    ro, nm = M.moe_finalize_residual_rmsnorm(**kw, residual=res, gamma=d_bf16(wl.gamma),
                                             eps=wl.eps, residual_out=res)
    torch.cuda.synchronize()
    assert ro.data_ptr() == res.data_ptr()
    check_vs_mirror(wl, ro, nm)


def test_threshold_boundary(ncu):
    """The last token count below the staged threshold and the first one at
    it give the same bits for their common tokens."""
    H, k = 7168, 8
    T_hi = -(-STAGED_FROM_UNITS_PER_CU * ncu // chunks(H))
    T_lo = T_hi - 1
    wl = W.make_workload(T_hi, H, 256, k, rsf=2.5, seed=940, with_residual=True)
    kw = device_inputs(wl)
    res, gam = d_bf16(wl.residual), d_bf16(wl.gamma)
    lo = dict(kw)
    for key in ("expanded_idx_to_permuted_idx", "topk_weights", "shared_out"):
        lo[key] = kw[key][:T_lo].contiguous()
    announce(f"staged rmsnorm threshold T={T_lo} / {T_hi} H={H}")
    ro, nm = run(kw, res, gam, wl.eps)
    ro_l, nm_l = run(lo, res[:T_lo].contiguous(), gam, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(ro[:T_lo].view(torch.int16), ro_l.view(torch.int16))
    assert torch.equal(nm[:T_lo].view(torch.int16), nm_l.view(torch.int16))
    check_vs_mirror(wl, ro, nm)
