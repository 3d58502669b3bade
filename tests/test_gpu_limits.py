"""GPU parity at the size limits the C header states.

* The largest hidden size (MOEF_MAX_HIDDEN): the plain and UE8M0 finalize
  with fp32 and packed weights, and both activation-quant policies, checked
  on every output against the oracle.
* The largest grid (MOEF_MAX_UNITS one-wave (token, chunk) units, whose
  work-items fill the 32-bit grid field of a dispatch up to the last
  256-lane workgroup): the plain, RMSNorm and UE8M0 finalize at the smallest
  hidden size each allows, so that one token is one unit. The outputs of
  sampled tokens, the first and the last ones included, are compared bit for
  bit with the oracle's fp32 mirror (normed within 2e-2, relative).
* The most partials one expert-parallel combine may sum
  (MOEF_MAX_EP_PARTIALS).
* The staged-output plain and UE8M0 finalize at the largest hidden size.
"""
import os
import re

import numpy as np
import pytest
import torch

import combine_moe_finalize_amd as M
from combine_moe_finalize_amd import workloads as W
from oracle import act_quant as A
from oracle import finalize as O
from oracle import formats as F

from gpu_helpers import (DEV, abs_terms, announce, assert_bf16_within_tolerance,
                         assert_bits_equal, d_bf16, d_f32, d_i32, device_inputs, h_bits, h_u8)

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_limits():
    with open(os.path.join(ROOT, "include", "moe_finalize.h")) as f:
        txt = f.read()
    return {m.group(1): int(m.group(2))
            for m in re.finditer(r"#define (MOEF_MAX_\w+) (\d+)", txt)}


LIM = header_limits()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    M.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_header_limits_parsed():
    assert LIM["MOEF_MAX_HIDDEN"] == 1 << 20
    assert LIM["MOEF_MAX_UNITS"] == (1 << 26) - 4
    assert LIM["MOEF_MAX_UNITS"] * 64 == LIM["MOEF_MAX_ITEMS"]


# ------------------------------------------------------------ largest hidden
@pytest.mark.parametrize("packed", [False, True])
def test_finalize_at_maximum_hidden(packed):
    H = LIM["MOEF_MAX_HIDDEN"]
    wl = W.make_workload(3, H, 4, 2, rsf=2.5, seed=901, pad=8, log2_mag=(-8, 8))
    wkw = dict(packed=wl.packed) if packed else dict(weights_f32=wl.weights)
    announce(f"finalize + quant at H={H} T=3 k=2 packed={packed}")
    kw = device_inputs(wl, packed=packed)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = M.moe_finalize(**kw, err_flag=err)
    q, s = M.moe_finalize_quant_ue8m0(**kw, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got, q, s = h_bits(out), h_u8(q), h_u8(s)
    del kw, out
    mirror, _ = O.finalize_mirror(wl.gemm2_out, wl.idx, shared=wl.shared, rsf=wl.rsf, **wkw)
    assert_bits_equal(got, mirror, "finalize vs fp32 mirror")
    truth, _ = O.finalize_truth_f64(wl.gemm2_out, wl.idx, shared=wl.shared, rsf=wl.rsf, **wkw)
    terms = abs_terms(wl.gemm2_out, wl.idx, weights=None if packed else wl.weights,
                      packed=wl.packed if packed else None, shared=wl.shared, rsf=wl.rsf)
    assert_bf16_within_tolerance(got, truth, terms, wl.top_k + 2, "finalize vs truth")
    mq, ms, _ = O.finalize_quant_mirror(wl.gemm2_out, wl.idx, shared=wl.shared, rsf=wl.rsf,
                                        **wkw)
    assert_bits_equal(s, ms, "UE8M0 scales")
    assert_bits_equal(q, mq, "E4M3 codes")


def test_act_quant_at_maximum_hidden():
    H = LIM["MOEF_MAX_HIDDEN"]
    x = W.activations(2, H, seed=902)
    announce(f"act quant at H={H} T=2")
    xd = d_bf16(x)
    q1, s1 = M.moe_act_quant_fp8_ue8m0(xd)
    q2, s2 = M.moe_act_quant_fp8_amax(xd)
    torch.cuda.synchronize()
    oq, os_ = A.act_quant_ue8m0(x)
    assert_bits_equal(s1.cpu().numpy(), os_, "UE8M0 scales")
    assert_bits_equal(q1.cpu().numpy(), oq, "UE8M0 codes")
    oq, os_ = A.act_quant_amax(x)
    assert_bits_equal(s2.cpu().numpy().view(np.uint32), os_.view(np.uint32), "amax scales")
    assert_bits_equal(q2.cpu().numpy(), oq, "amax codes")


# -------------------------------------------------------------- largest grid
def sampled_tokens(T, seed, n=4096, ends=64):
    rng = np.random.default_rng(seed)
    mid = rng.choice(T, size=n, replace=False)
    return np.unique(np.concatenate([np.arange(ends), mid, np.arange(T - ends, T)]))


def routed_device(wl):
    return dict(gemm2_out=d_bf16(wl.gemm2_out), expanded_idx_to_permuted_idx=d_i32(wl.idx),
                topk_weights=d_f32(wl.weights), routed_scaling_factor=wl.rsf)


def rows_at(t, sample):
    return t[torch.from_numpy(sample).to(DEV)]


def test_plain_finalize_at_maximum_grid():
    T = LIM["MOEF_MAX_UNITS"]            # H = 8: one unit per token
    announce(f"drawing plain finalize inputs T={T} H=8 k=2")
    wl = W.random_gather(T, 4096, 8, 2, rsf=2.5, seed=903)
    announce(f"plain finalize at the largest grid: T={T} H=8 k=2")
    kw = routed_device(wl)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = M.moe_finalize(**kw, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    smp = sampled_tokens(T, 903)
    got = h_bits(rows_at(out, smp))
    del kw, out
    torch.cuda.empty_cache()
    mirror, _ = O.finalize_mirror(wl.gemm2_out, wl.idx[smp], weights_f32=wl.weights[smp],
                                  rsf=wl.rsf)
    assert_bits_equal(got, mirror, "sampled tokens vs fp32 mirror")


def test_quant_finalize_at_maximum_grid():
    T = LIM["MOEF_MAX_UNITS"]            # H = 128: one unit (one DPP row) per token
    announce(f"drawing quant finalize inputs T={T} H=128 k=2")
    wl = W.random_gather(T, 4096, 128, 2, rsf=2.5, seed=904, log2_mag=(-8, 8))
    announce(f"UE8M0 finalize at the largest grid: T={T} H=128 k=2")
    kw = routed_device(wl)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    q, s = M.moe_finalize_quant_ue8m0(**kw, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    smp = sampled_tokens(T, 904)
    gq, gs = h_u8(rows_at(q, smp)), h_u8(rows_at(s, smp))
    del kw, q, s
    torch.cuda.empty_cache()
    mq, ms, _ = O.finalize_quant_mirror(wl.gemm2_out, wl.idx[smp],
                                        weights_f32=wl.weights[smp], rsf=wl.rsf)
    assert_bits_equal(gs, ms, "sampled scale bytes vs mirror")
    assert_bits_equal(gq, mq, "sampled codes vs mirror")


def test_rmsnorm_finalize_at_maximum_grid():
    T = LIM["MOEF_MAX_UNITS"]            # H = 8: one one-wave workgroup per token
    announce(f"drawing residual + RMSNorm inputs T={T} H=8 k=2")
    wl = W.random_gather(T, 4096, 8, 2, rsf=2.5, seed=905, with_residual=True)
    announce(f"residual + RMSNorm finalize at the largest grid: T={T} H=8 k=2")
    kw = routed_device(wl)
    res, gam = d_bf16(wl.residual), d_bf16(wl.gamma)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ro, nm = M.moe_finalize_residual_rmsnorm(**kw, residual=res, gamma=gam, eps=wl.eps,
                                             err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    smp = sampled_tokens(T, 905)
    g_ro, g_nm = h_bits(rows_at(ro, smp)), h_bits(rows_at(nm, smp))
    del kw, res, ro, nm
    torch.cuda.empty_cache()
    m_ro, m_nm, _ = O.finalize_residual_rmsnorm_mirror(
        wl.gemm2_out, wl.idx[smp], weights_f32=wl.weights[smp], rsf=wl.rsf,
        residual=wl.residual[smp], gamma=wl.gamma, eps=wl.eps)
    assert_bits_equal(g_ro, m_ro, "sampled residual_out vs mirror")
    g, o = F.bf16_to_f64(g_nm), F.bf16_to_f64(m_nm)
    assert np.all(np.abs(g - o) <= 2e-2 * np.abs(o)), np.max(np.abs(g - o) / np.abs(o))


# -------------------------------------------------------- most EP partials
def test_ep_combine_at_maximum_partials():
    R, T, H = LIM["MOEF_MAX_EP_PARTIALS"], 5, 1000
    rng = np.random.default_rng(906)
    p = W.to_bf16_bits((rng.standard_normal((R, T, H)) * np.exp2(rng.uniform(-4, 4, (R, T, 1)))
                        ).astype(np.float32))
    sh = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    announce(f"ep combine R={R} T={T} H={H}")
    out = M.moe_finalize_ep_combine(d_bf16(p), shared_out=d_bf16(sh))
    torch.cuda.synchronize()
    assert_bits_equal(h_bits(out), O.ep_combine_mirror(p, sh), "combine of the most partials")


def test_staged_paths_at_maximum_hidden():
    """10 tokens of the largest hidden size: 20 480 units, so both the plain
    and the UE8M0 finalize take their staged-output kernels on 256 CUs."""
    H = LIM["MOEF_MAX_HIDDEN"]
    wl = W.make_workload(10, H, 4, 2, rsf=2.5, seed=907, pad=8, log2_mag=(-8, 8))
    announce(f"staged finalize + quant at H={H} T=10 k=2")
    kw = device_inputs(wl)
    out = M.moe_finalize(**kw)
    q, s = M.moe_finalize_quant_ue8m0(**kw)
    torch.cuda.synchronize()
    got, q, s = h_bits(out), h_u8(q), h_u8(s)
    del kw, out
    mirror, _ = O.finalize_mirror(wl.gemm2_out, wl.idx, weights_f32=wl.weights,
                                  shared=wl.shared, rsf=wl.rsf)
    assert_bits_equal(got, mirror, "finalize vs fp32 mirror")
    mq, ms, _ = O.quant_ue8m0(mirror)
    assert_bits_equal(s, ms, "UE8M0 scales")
    assert_bits_equal(q, mq, "E4M3 codes")
