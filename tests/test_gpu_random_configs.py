"""Seeded random configurations of every entry point against the CPU oracle.

Each case draws its own shape and options, so together they cross what the
structured tests cover one axis at a time:
  * top_k from 1 to 16, which reaches both the exact kernel instantiations
    (1, 2, 4, 6, 8) and the guarded ones;
  * hidden sizes that are not multiples of the 512-column wave chunk;
  * fp32 or packed weights, with or without the shared output;
  * random routed scaling factors and expert-segment padding;
  * slots skipped with -1 and slots pointing past the last row.
The finalize outputs, residual_out, the E4M3 codes and the UE8M0 bytes are
compared bit for bit with the oracle's fp32 mirror. normed is compared within
one bf16 ulp of the fp64 RMSNorm of the same residual_out. Gate ids are
compared bit for bit, and gate weights within 32 units of 2^-24, relative."""
import numpy as np
import pytest
import torch

import combine_moe_finalize_amd as M
from combine_moe_finalize_amd import workloads as W
from oracle import act_quant as A
from oracle import finalize as O
from oracle import formats as F
from oracle import routing as RT

from gpu_helpers import DEV, announce, assert_bits_equal, d_bf16, d_f32, d_i32, h_bits, ulp_bf16

pytestmark = pytest.mark.gpu

MAX_ELEMS = 400_000          # T * H per case keeps the oracle to well under a second


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    M.load_library()


def draw(rng, kind):
    k = int(rng.integers(1, 17))
    E = int(rng.choice([e for e in (16, 32, 64, 256) if e >= k]))
    if kind == "quant":
        H = 128 * int(rng.integers(1, 41))
    elif kind == "rmsnorm":
        H = 8 * int(rng.integers(1, 2049))
    else:
        H = 8 * int(rng.integers(1, 1601))
    T = int(rng.integers(1, max(2, min(300, MAX_ELEMS // H) + 1)))
    rsf = float(rng.choice([1.0, 2.5, float(np.float32(rng.uniform(0.1, 4.0)))]))
    wl = W.make_workload(T, H, E, k, rsf=rsf, seed=int(rng.integers(1 << 30)),
                         pad=int(rng.choice([8, 32, 128])),
                         with_shared=bool(rng.random() < 0.7),
                         with_residual=(kind == "rmsnorm"),
                         log2_mag=(-8.0, 8.0) if rng.random() < 0.5 else None)
    idx = wl.idx.copy()
    if rng.random() < 0.4:                               # experts held elsewhere
        idx[rng.random(idx.shape) < 0.1] = -1
    oob = rng.random() < 0.25
    if oob:                                              # past the last row
        for _ in range(int(rng.integers(1, 3))):
            idx[rng.integers(T), rng.integers(k)] = wl.P + int(rng.integers(0, 1000))
    packed = bool(rng.random() < 0.5)
    return wl, idx, packed, oob


def device_args(wl, idx, packed):
    kw = dict(topk_packed=d_i32(wl.packed)) if packed else dict(topk_weights=d_f32(wl.weights))
    return dict(gemm2_out=d_bf16(wl.gemm2_out), expanded_idx_to_permuted_idx=d_i32(idx),
                shared_out=None if wl.shared is None else d_bf16(wl.shared),
                routed_scaling_factor=wl.rsf, **kw)


def oracle_args(wl, idx, packed):
    kw = dict(packed=wl.packed) if packed else dict(weights_f32=wl.weights)
    return dict(shared=wl.shared, rsf=wl.rsf, **kw)


def describe(wl, packed, oob):
    return (f"T={wl.T} H={wl.H} E={wl.E} k={wl.top_k} rsf={wl.rsf:g} packed={packed} "
            f"shared={wl.shared is not None} oob={oob}")


@pytest.mark.parametrize("case", range(64))
def test_random_finalize(case):
    check_finalize(1000 + case)


def check_finalize(seed):
    rng = np.random.default_rng(seed)
    wl, idx, packed, oob = draw(rng, "plain")
    announce(f"random finalize seed {seed}: {describe(wl, packed, oob)}")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = M.moe_finalize(**device_args(wl, idx, packed), err_flag=err)
    torch.cuda.synchronize()
    ref, flag = O.finalize_mirror(wl.gemm2_out, idx, **oracle_args(wl, idx, packed))
    assert_bits_equal(h_bits(out), ref, f"seed {seed}")
    assert int(err.item()) == flag == (1 if oob else 0)


@pytest.mark.parametrize("case", range(48))
def test_random_residual_rmsnorm(case):
    check_residual_rmsnorm(2000 + case)


def check_residual_rmsnorm(seed):
    rng = np.random.default_rng(seed)
    wl, idx, packed, oob = draw(rng, "rmsnorm")
    announce(f"random residual+rmsnorm seed {seed}: {describe(wl, packed, oob)}")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ro, nm = M.moe_finalize_residual_rmsnorm(**device_args(wl, idx, packed),
                                             residual=d_bf16(wl.residual), gamma=d_bf16(wl.gamma),
                                             eps=wl.eps, err_flag=err)
    torch.cuda.synchronize()
    m_ro, m_nm, flag = O.finalize_residual_rmsnorm_mirror(
        wl.gemm2_out, idx, residual=wl.residual, gamma=wl.gamma, eps=wl.eps,
        **oracle_args(wl, idx, packed))
    assert_bits_equal(h_bits(ro), m_ro, f"seed {seed} residual_out")
    g, o = F.bf16_to_f64(h_bits(nm)), F.bf16_to_f64(m_nm)
    assert np.all(np.abs(g - o) <= ulp_bf16(o)), f"seed {seed} normed"
    assert int(err.item()) == flag == (1 if oob else 0)


@pytest.mark.parametrize("case", range(48))
def test_random_quant(case):
    check_quant(3000 + case)


def check_quant(seed):
    rng = np.random.default_rng(seed)
    wl, idx, packed, oob = draw(rng, "quant")
    announce(f"random quant seed {seed}: {describe(wl, packed, oob)}")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    q, s = M.moe_finalize_quant_ue8m0(**device_args(wl, idx, packed), err_flag=err)
    torch.cuda.synchronize()
    mq, ms, flag = O.finalize_quant_mirror(wl.gemm2_out, idx, **oracle_args(wl, idx, packed))
    assert_bits_equal(s.cpu().numpy(), ms, f"seed {seed} scales")
    assert_bits_equal(q.cpu().numpy(), mq, f"seed {seed} codes")
    assert int(err.item()) == flag == (1 if oob else 0)


@pytest.mark.parametrize("case", range(48))
def test_random_gate(case):
    check_gate(4000 + case)


def check_gate(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 513))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(1, 400))
    if rng.random() < 0.5:
        lg = rng.integers(-4, 5, size=(T, E)).astype(np.float32)        # many exact ties
        lg[rng.random((T, E)) < 0.02] = np.nan
    else:
        lg = W.router_logits(T, E, seed=seed, scale=float(rng.uniform(0.5, 4.0)))
    announce(f"random gate seed {seed}: T={T} E={E} k={k}")
    ids, w, pk = M.moe_topk_sigmoid_gate(torch.from_numpy(lg).to(DEV), k)
    torch.cuda.synchronize()
    oid, ow, _ = RT.topk_sigmoid_gate(lg, k)
    assert np.array_equal(ids.cpu().numpy(), oid), f"seed {seed} ids"
    w = w.cpu().numpy()
    fin = np.isfinite(ow)
    assert np.all(np.abs(w[fin] - ow[fin]) <= 32 * 2.0 ** -24 * np.abs(ow[fin]) + 1e-38)
    assert np.array_equal(np.isnan(w), np.isnan(ow))
    assert np.array_equal(pk.cpu().numpy().view(np.uint32) >> 16, oid.astype(np.uint32))


@pytest.mark.parametrize("case", range(24))
def test_random_act_quant(case):
    check_act_quant(5000 + case)


def check_act_quant(seed):
    rng = np.random.default_rng(seed)
    H = 128 * int(rng.integers(1, 129))
    T = int(rng.integers(1, max(2, MAX_ELEMS // H)))
    x = W.activations(T, H, seed=seed)
    announce(f"random act quant seed {seed}: T={T} H={H}")
    xd = d_bf16(x)
    q1, s1 = M.moe_act_quant_fp8_ue8m0(xd)
    q2, s2 = M.moe_act_quant_fp8_amax(xd)
    torch.cuda.synchronize()
    oq1, os1 = A.act_quant_ue8m0(x)
    oq2, os2 = A.act_quant_amax(x)
    assert_bits_equal(s1.cpu().numpy(), os1, f"seed {seed} ue8m0 scales")
    assert_bits_equal(q1.cpu().numpy(), oq1, f"seed {seed} ue8m0 codes")
    assert_bits_equal(s2.cpu().numpy().view(np.uint32), os2.view(np.uint32),
                      f"seed {seed} amax scales")
    assert_bits_equal(q2.cpu().numpy(), oq2, f"seed {seed} amax codes")


@pytest.mark.parametrize("case", range(24))
def test_random_combine_and_allreduce(case):
    check_combine_and_allreduce(6000 + case)


def check_combine_and_allreduce(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 17))
    H = 8 * int(rng.integers(1, 2049))
    T = int(rng.integers(1, max(2, MAX_ELEMS // (H * R) + 1)))
    mag = np.exp2(rng.uniform(-4, 4, (R, T, 1)))
    parts = W.to_bf16_bits((rng.standard_normal((R, T, H)) * mag).astype(np.float32))
    sh = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    res = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    gam = W.to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    announce(f"random combine/all-reduce seed {seed}: R={R} T={T} H={H}")
    eo = M.moe_finalize_ep_combine(d_bf16(parts), shared_out=d_bf16(sh))
    ro, nm = M.moe_allreduce_residual_rmsnorm([d_bf16(p) for p in parts], residual=d_bf16(res),
                                              gamma=d_bf16(gam))
    torch.cuda.synchronize()
    assert_bits_equal(h_bits(eo), O.ep_combine_mirror(parts, sh), f"seed {seed} combine")
    m_ro, m_nm = O.allreduce_residual_rmsnorm_mirror(parts, res, gam)
    assert_bits_equal(h_bits(ro), m_ro, f"seed {seed} residual_out")
    g, o = F.bf16_to_f64(h_bits(nm)), F.bf16_to_f64(m_nm)
    assert np.all(np.abs(g - o) <= ulp_bf16(o)), f"seed {seed} normed"
