"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

The contract: index / gather work bit-exact; bf16 outputs within 2 bf16 ulp
of the fp64 truth rounded to bf16 (plus the fp32 forward-error term under
cancellation); UE8M0 exponents exact; E4M3 codes within 1 code; RMSNorm
within relative 2e-2. The kernels follow the oracle's fp32 mirror order, so
the tests also require bit-identity with the mirror for every output except
the RMSNorm one (its reduction order is free)."""
import numpy as np
import pytest
import torch

import combine_moe_finalize_amd as M
from combine_moe_finalize_amd import workloads as W
from oracle import finalize as O
from oracle import formats as F

from gpu_helpers import (DEV, abs_terms, announce, assert_bf16_within_tolerance,
                         assert_bits_equal, d_bf16, d_f32, d_i32, device_inputs, h_bits, h_u8,
                         ulp_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on CPU-only machines)")
    M.load_library()
    yield
    torch.cuda.synchronize()


def run_finalize(wl, packed=False, with_shared=True, err=None):
    kw = device_inputs(wl, packed=packed, with_shared=with_shared)
    out = M.moe_finalize(**kw, err_flag=err)
    torch.cuda.synchronize()
    return h_bits(out)


def check_finalize(wl, got, packed=False, with_shared=True, what=""):
    wkw = dict(packed=wl.packed) if packed else dict(weights_f32=wl.weights)
    sh = wl.shared if with_shared else None
    mirror, flag = O.finalize_mirror(wl.gemm2_out, wl.idx, shared=sh, rsf=wl.rsf, **wkw)
    assert flag == 0
    assert_bits_equal(got, mirror, f"{what} vs fp32 mirror")
    truth, _ = O.finalize_truth_f64(wl.gemm2_out, wl.idx, shared=sh, rsf=wl.rsf, **wkw)
    terms = abs_terms(wl.gemm2_out, wl.idx, weights=None if packed else wl.weights,
                      packed=wl.packed if packed else None, shared=sh, rsf=wl.rsf)
    return assert_bf16_within_tolerance(got, truth, terms, wl.top_k + 2, what)


# ------------------------------------------------------- workload families
@pytest.mark.parametrize("packed", [False, True])
def test_tiny_workload(packed):
    wl = W.family_workload("tiny")
    announce(f"tiny T=1 H=1024 k=2 packed={packed}")
    got = run_finalize(wl, packed=packed)
    check_finalize(wl, got, packed=packed, what="tiny")


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("T", [1, 4, 8, 16, 64, 256])
def test_decode_sweep(T, packed):
    wl = W.family_workload("decode_sweep", T)
    announce(f"decode sweep T={T} H=4096 k=8 packed={packed}")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_finalize(wl, packed=packed, err=err)
    assert int(err.item()) == 0
    assert np.isfinite(F.bf16_to_f64(got)).all()          # NaN padding never read
    check_finalize(wl, got, packed=packed, what=f"decode T={T}")


def test_packed_vs_unpacked_full_size():
    wl = W.family_workload("packed_vs_unpacked")
    announce("packed vs unpacked T=256 H=7168 k=8")
    up = run_finalize(wl, packed=False)
    pk = run_finalize(wl, packed=True)
    check_finalize(wl, up, packed=False, what="unpacked")
    check_finalize(wl, pk, packed=True, what="packed")
    # the packed path equals the fp32 path with weights pre-rounded to bf16
    wr = F.bf16_to_f32(W.to_bf16_bits(wl.weights))
    kw = device_inputs(wl)
    kw["topk_weights"] = d_f32(wr)
    pre = h_bits(M.moe_finalize(**kw))
    torch.cuda.synchronize()
    assert_bits_equal(pk, pre, "packed == bf16-rounded fp32")
    assert not np.array_equal(pk, up)        # genuine fp32 weights differ


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("T", [16, 256, 1024])
def test_residual_rmsnorm(T, packed):
    wl = W.family_workload("residual_rmsnorm", T)
    announce(f"residual+rmsnorm T={T} H=7168 k=8 packed={packed}")
    kw = device_inputs(wl, packed=packed)
    ro, nm = M.moe_finalize_residual_rmsnorm(**kw, residual=d_bf16(wl.residual),
                                             gamma=d_bf16(wl.gamma), eps=wl.eps)
    torch.cuda.synchronize()
    ro, nm = h_bits(ro), h_bits(nm)
    check_rmsnorm(wl, ro, nm, packed=packed)


def check_rmsnorm(wl, ro, nm, packed=False):
    wkw = dict(packed=wl.packed) if packed else dict(weights_f32=wl.weights)
    m_ro, m_nm, _ = O.finalize_residual_rmsnorm_mirror(
        wl.gemm2_out, wl.idx, shared=wl.shared, rsf=wl.rsf, residual=wl.residual,
        gamma=wl.gamma, eps=wl.eps, **wkw)
    assert_bits_equal(ro, m_ro, "residual_out vs mirror")
    acc, _ = O.finalize_truth_f64(wl.gemm2_out, wl.idx, shared=wl.shared, rsf=wl.rsf, **wkw)
    truth = acc + F.bf16_to_f64(wl.residual)
    terms = abs_terms(wl.gemm2_out, wl.idx, weights=None if packed else wl.weights,
                      packed=wl.packed if packed else None, shared=wl.shared, rsf=wl.rsf,
                      residual=wl.residual)
    assert_bf16_within_tolerance(ro, truth, terms, wl.top_k + 3, "residual_out vs truth")
    # RMSNorm within relative 2e-2 of the oracle's (mirror chain: the same
    # residual_out the kernel is required to produce)
    g = F.bf16_to_f64(nm)
    o = F.bf16_to_f64(m_nm)
    assert np.all(np.abs(g - o) <= 2e-2 * np.abs(o)), np.max(np.abs(g - o) / np.abs(o))
    # and against the fp64 truth chain, allowing for its own bf16 residual_out
    t_ro, t_nm, _ = O.finalize_residual_rmsnorm_truth(
        wl.gemm2_out, wl.idx, shared=wl.shared, rsf=wl.rsf, residual=wl.residual,
        gamma=wl.gamma, eps=wl.eps, **wkw)
    o = F.bf16_to_f64(t_nm)
    slack = 2 * np.abs(F.bf16_to_f64(t_ro) - F.bf16_to_f64(ro)) * np.abs(o) / np.maximum(
        np.abs(F.bf16_to_f64(t_ro)), 1e-30)
    assert np.all(np.abs(g - o) <= 2e-2 * np.abs(o) + slack)


@pytest.fixture(scope="module")
def prefill_workload():
    return W.family_workload("prefill_fp8_ue8m0")


@pytest.mark.parametrize("packed", [False, True])
def test_prefill_quant_full_size(prefill_workload, packed):
    wl = prefill_workload
    announce(f"prefill quant T=8192 H=7168 k=8 packed={packed}")
    kw = device_inputs(wl, packed=packed)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    q, s = M.moe_finalize_quant_ue8m0(**kw, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    q, s = h_u8(q), h_u8(s)
    del kw
    torch.cuda.empty_cache()
    check_quant(wl, q, s, packed=packed)


def check_quant(wl, q, s, packed=False, with_shared=True, chunk=512):
    wkw = dict(packed=wl.packed) if packed else dict(weights_f32=wl.weights)
    sh_all = wl.shared if with_shared else None
    for t0 in range(0, wl.T, chunk):
        sl = slice(t0, min(wl.T, t0 + chunk))
        wk = {k: v[sl] for k, v in wkw.items()}
        sh = None if sh_all is None else sh_all[sl]
        mq, ms, _ = O.finalize_quant_mirror(wl.gemm2_out, wl.idx[sl], shared=sh, rsf=wl.rsf, **wk)
        assert_bits_equal(s[sl], ms, f"UE8M0 scales tokens {sl}")
        assert_bits_equal(q[sl], mq, f"E4M3 codes tokens {sl}")
        # against the fp64 truth: exponents exact unless y itself differs,
        # codes within one code
        tq, ts, _ = O.finalize_quant_truth(wl.gemm2_out, wl.idx[sl], shared=sh, rsf=wl.rsf, **wk)
        assert np.mean(ts != ms) < 1e-3
        same_scale = np.repeat(ts == ms, 128, axis=1)
        dq = np.abs(q[sl].astype(np.int64) - tq.astype(np.int64))
        sign_flip = ((q[sl] ^ tq) & 0x80) != 0
        mag = np.abs((q[sl] & 0x7F).astype(np.int64) - (tq & 0x7F).astype(np.int64))
        ok = np.where(sign_flip, ((q[sl] & 0x7F) <= 1) & ((tq & 0x7F) <= 1), mag <= 1)
        assert np.all(ok | ~same_scale), dq.max()


# --------------------------------------------------------- exhaustive quant
def test_quant_exhaustive_codes_and_exponents():
    """Pure gather (top_k 1, weight 1, rsf 1, no shared): y is the gathered
    bf16 row itself. Part A: every finite bf16 value in [-448, 448] inside a
    block whose max is 448 (e = 0) -> all E4M3 code decisions. Part B: every
    positive finite bf16 as a block amax -> every exponent decision, with
    subnormal and zero blocks, and the block's other values scaled by it."""
    allv = F.bf16_to_f64(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16))
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    inr = np.isfinite(allv) & (np.abs(allv) <= 448)
    a_vals = pats[inr]
    per = 127
    nblk_a = -(-a_vals.size // per)
    blocks_a = np.full((nblk_a, 128), 0, dtype=np.uint16)
    flat = np.zeros(nblk_a * per, dtype=np.uint16)
    flat[:a_vals.size] = a_vals
    blocks_a[:, 1:] = flat.reshape(nblk_a, per)
    blocks_a[:, 0] = 0x43E0                          # 448
    pos = pats[np.isfinite(allv) & (allv > 0)]
    blocks_b = np.zeros((pos.size + 1, 128), dtype=np.uint16)
    blocks_b[:-1, 0] = pos                            # the block amax
    blocks_b[:-1, 1] = pos | 0x8000                   # -amax
    rng = np.random.default_rng(21)
    # other entries: the amax times random factors in (0, 1), rounded to bf16
    fac = rng.uniform(0, 1, size=(pos.size, 126)).astype(np.float64)
    blocks_b[:-1, 2:] = F.bf16_bits(F.bf16_to_f64(pos)[:, None] * fac *
                                    np.where(rng.random((pos.size, 126)) < 0.5, -1, 1))
    # (the last block stays all zero)
    blocks = np.concatenate([blocks_a, blocks_b])
    H = 7168
    nb = H // 128
    T = -(-blocks.shape[0] // nb)
    rows = np.zeros((T * nb, 128), dtype=np.uint16)
    rows[:blocks.shape[0]] = blocks
    g2 = rows.reshape(T, H)
    P = T + 128
    g2p = np.full((P, H), W.NAN_BF16, dtype=np.uint16)
    perm = np.random.default_rng(22).permutation(P)[:T]
    g2p[perm] = g2
    idx = perm.reshape(T, 1).astype(np.int32)
    w = np.ones((T, 1), dtype=np.float32)
    announce(f"exhaustive quant T={T} H={H} k=1")
    q, s = M.moe_finalize_quant_ue8m0(d_bf16(g2p), d_i32(idx), topk_weights=d_f32(w),
                                      routed_scaling_factor=1.0)
    torch.cuda.synchronize()
    q, s = h_u8(q), h_u8(s)
    y, _ = O.finalize_mirror(g2p, idx, weights_f32=w, rsf=1.0)
    # the pure gather reproduces each row, except that the +0 start of the
    # fp32 sum turns a gathered -0 into +0
    assert np.array_equal(y, np.where(g2 == 0x8000, np.uint16(0), g2))
    oq, osc, _ = O.quant_ue8m0(y)
    assert_bits_equal(s, osc, "exhaustive exponents")
    assert_bits_equal(q, oq, "exhaustive codes")


def test_bf16_rounding_of_arbitrary_fp32():
    """top_k 1, every gathered row 1.0, rsf 1, no shared output: out = bf16(w)
    for the fp32 weight w, so every fp32 -> bf16 rounding decision (ties both
    ways, subnormals, overflow to inf) is checked against the oracle."""
    rng = np.random.default_rng(81)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    bits = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi,
                           rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)])
    w = bits.view(np.float32)
    w = w[~np.isnan(w)].reshape(-1, 1)
    T, H = w.shape[0], 8
    g2 = np.full((128, H), W.NAN_BF16, dtype=np.uint16)
    g2[5] = 0x3F80                                     # 1.0
    idx = np.full((T, 1), 5, dtype=np.int32)
    announce(f"bf16 rounding of {T} fp32 values")
    out = M.moe_finalize(d_bf16(g2), d_i32(idx), topk_weights=d_f32(w), routed_scaling_factor=1.0)
    torch.cuda.synchronize()
    got = h_bits(out)
    want, _ = O.finalize_mirror(g2, idx, weights_f32=w, rsf=1.0)
    assert_bits_equal(got, want, "bf16 rounding")


# ------------------------------------------------------------- edge cases
@pytest.mark.parametrize("k", [1, 2, 3, 5, 6, 7, 9, 16])
def test_every_top_k_path(k):
    wl = W.make_workload(37, 1000, 32, k, rsf=1.75, seed=100 + k, pad=16)   # ragged H
    announce(f"top_k={k} T=37 H=1000")
    for packed in (False, True):
        got = run_finalize(wl, packed=packed)
        check_finalize(wl, got, packed=packed, what=f"k={k} packed={packed}")


@pytest.mark.parametrize("H", [8, 64, 520, 4104, 16384])
def test_ragged_hidden(H):
    wl = W.make_workload(5, H, 16, 4, rsf=2.5, seed=200 + H, pad=8)
    announce(f"ragged H={H}")
    got = run_finalize(wl)
    check_finalize(wl, got, what=f"H={H}")


def test_empty_batch_is_noop():
    g2 = torch.zeros((128, 256), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    w = torch.zeros((0, 4), dtype=torch.float32, device=DEV)
    announce("empty batch")
    out = M.moe_finalize(g2, idx, topk_weights=w)
    q, s = M.moe_finalize_quant_ue8m0(g2, idx, topk_weights=w)
    torch.cuda.synchronize()
    assert out.shape == (0, 256) and q.shape == (0, 256) and s.shape == (0, 2)


def test_negative_index_skips_and_out_of_range_flags():
    wl = W.make_workload(24, 512, 16, 4, rsf=2.5, seed=31, pad=16)
    idx = wl.idx.copy()
    idx[2, 1] = -1
    idx[7, 3] = -5
    idx[11, 0] = wl.P          # out of range
    idx[12, 2] = 2 ** 31 - 1
    wl.idx = idx
    announce("negative and out-of-range indices")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_finalize(wl, err=err)
    assert int(err.item()) == M.DEVERR_INDEX_OUT_OF_RANGE
    mirror, flag = O.finalize_mirror(wl.gemm2_out, idx, weights_f32=wl.weights,
                                     shared=wl.shared, rsf=wl.rsf)
    assert flag == O.ERR_INDEX_OUT_OF_RANGE
    assert_bits_equal(got, mirror, "skipped slots")
    # only negative indices: no flag
    idx2 = wl.idx.copy()
    idx2[11, 0] = 3
    idx2[12, 2] = 4
    wl.idx = idx2
    err.zero_()
    run_finalize(wl, err=err)
    assert int(err.item()) == 0


def test_padding_row_reference_is_visible():
    """An index that points at a NaN padding row gives NaN in that token's
    output: proof that the NaN sentinel would expose a wrong gather."""
    wl = W.make_workload(4, 256, 8, 2, rsf=1.0, seed=41, pad=128)
    pad_rows = np.where(np.all(wl.gemm2_out == W.NAN_BF16, axis=1))[0]
    idx = wl.idx.copy()
    idx[1, 0] = pad_rows[0]
    wl.idx = idx
    announce("padding-row reference")
    got = run_finalize(wl)
    v = F.bf16_to_f64(got)
    assert np.isnan(v[1]).all() and np.isfinite(v[[0, 2, 3]]).all()


def test_no_shared_and_rsf_one():
    wl = W.family_workload("decode_sweep", 16)
    wl.rsf = 1.0
    announce("no shared, rsf 1")
    got = run_finalize(wl, with_shared=False)
    check_finalize(wl, got, with_shared=False, what="no shared")
    q_wl = W.make_workload(16, 1024, 16, 8, rsf=1.0, seed=51, log2_mag=(-8, 8))
    kw = device_inputs(q_wl, with_shared=False)
    q, s = M.moe_finalize_quant_ue8m0(**kw)
    torch.cuda.synchronize()
    check_quant(q_wl, h_u8(q), h_u8(s), with_shared=False)


def test_quant_packed_and_ragged_blocks():
    wl = W.make_workload(33, 128 * 13, 64, 6, rsf=2.5, seed=61, log2_mag=(-8, 8))
    announce("quant packed H=1664 k=6")
    kw = device_inputs(wl, packed=True)
    q, s = M.moe_finalize_quant_ue8m0(**kw)
    torch.cuda.synchronize()
    check_quant(wl, h_u8(q), h_u8(s), packed=True)


@pytest.mark.parametrize("H,k", [(16384, 8), (4096, 16), (1000, 3), (8, 1)])
def test_rmsnorm_shapes(H, k):
    wl = W.make_workload(9, H, 32, k, rsf=2.5, seed=300 + H + k, with_residual=True, pad=16)
    announce(f"rmsnorm H={H} k={k}")
    for packed in (False, True):
        kw = device_inputs(wl, packed=packed)
        ro, nm = M.moe_finalize_residual_rmsnorm(**kw, residual=d_bf16(wl.residual),
                                                 gamma=d_bf16(wl.gamma), eps=wl.eps)
        torch.cuda.synchronize()
        check_rmsnorm(wl, h_bits(ro), h_bits(nm), packed=packed)


def test_rmsnorm_in_place_residual():
    wl = W.family_workload("residual_rmsnorm", 16)
    announce("rmsnorm in place")
    kw = device_inputs(wl)
    res = d_bf16(wl.residual)
    ro, nm = M.moe_finalize_residual_rmsnorm(**kw, residual=res, gamma=d_bf16(wl.gamma),
                                             eps=wl.eps, residual_out=res)
    torch.cuda.synchronize()
    assert ro.data_ptr() == res.data_ptr()
    check_rmsnorm(wl, h_bits(ro), h_bits(nm))


def test_packed_decode():
    rng = np.random.default_rng(71)
    words = rng.integers(-2 ** 31, 2 ** 31, size=100_003, dtype=np.int64).astype(np.int32)
    g = np.array([0x00033F80, 0x00FF3E80, 0x3F40, 0x00113DCD, 0xFFFF4000], dtype=np.uint32)
    words[:5] = g.view(np.int32)
    announce("packed decode n=100003")
    ids, w = M.moe_topk_packed_decode(d_i32(words).view(1, -1))
    torch.cuda.synchronize()
    oid, ow = O.decode_packed(words)
    assert np.array_equal(ids.cpu().numpy().reshape(-1), oid)
    assert np.array_equal(w.cpu().numpy().reshape(-1).view(np.uint32), ow.view(np.uint32))


def test_layout_invariance_on_gpu():
    """The same rows in another order (token-ordered instead of expert-sorted,
    no padding), with the map updated, give bitwise the same output."""
    wl = W.family_workload("packed_vs_unpacked")
    announce("layout invariance T=256 H=7168")
    a = run_finalize(wl)
    wl.gemm2_out = wl.gemm2_out[wl.idx.reshape(-1)]
    wl.idx = np.arange(wl.T * wl.top_k, dtype=np.int32).reshape(wl.T, wl.top_k)
    b = run_finalize(wl)
    assert_bits_equal(a, b, "token-ordered layout", zero_equal=False)
    check_finalize(wl, b, what="token-ordered layout")


# -------------------------------------------------------------- robustness
def test_deterministic_and_canaries():
    wl = W.family_workload("decode_sweep", 64)
    announce("determinism and canaries")
    kw = device_inputs(wl)
    T, H = wl.T, wl.H
    G = 4096
    buf = torch.full((T * H + 2 * G,), 0x5A5A, dtype=torch.int16, device=DEV)
    out = buf[G:G + T * H].view(T, H).view(torch.bfloat16)
    M.moe_finalize(**kw, out=out)
    a = h_bits(out).copy()
    M.moe_finalize(**kw, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(a, h_bits(out))
    guard = buf.cpu().numpy()
    assert np.all(guard[:G] == 0x5A5A) and np.all(guard[G + T * H:] == 0x5A5A)
    check_finalize(wl, a, what="canary run")


def test_graph_capture_replay():
    wl = W.family_workload("decode_sweep", 16)
    announce("graph capture")
    kw = device_inputs(wl)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=DEV)
    eager = h_bits(M.moe_finalize(**kw, out=torch.empty_like(out)))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        M.moe_finalize(**kw, out=out)          # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.moe_finalize(**kw, out=out)
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(h_bits(out), eager, f"graph replay {i}")
        _ = (torch.ones(1000, device=DEV) * i).sum().item()   # eager work between replays


def test_float8_output_tensors():
    """A float8_e4m3fn output is written through a byte view and returned as
    the caller's own tensor; torch's decoding of the codes matches the
    oracle's E4M3 decoding."""
    wl = W.make_workload(8, 1024, 16, 4, rsf=2.5, seed=41)
    announce("float8_e4m3fn outputs")
    kw = device_inputs(wl)
    q8 = torch.empty((wl.T, wl.H), dtype=torch.float8_e4m3fn, device=DEV)
    got, s = M.moe_finalize_quant_ue8m0(**kw, out_e4m3=q8)
    ref_q, ref_s = M.moe_finalize_quant_ue8m0(**kw)
    xa = d_bf16(W.activations(8, 1024, seed=42))
    a8 = torch.empty((8, 1024), dtype=torch.float8_e4m3fn, device=DEV)
    got_a, _ = M.moe_act_quant_fp8_ue8m0(xa, out_e4m3=a8)
    ref_a, _ = M.moe_act_quant_fp8_ue8m0(xa)
    torch.cuda.synchronize()
    assert got is q8 and got_a is a8
    assert torch.equal(q8.view(torch.uint8), ref_q) and torch.equal(a8.view(torch.uint8), ref_a)
    dec = q8.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(dec, F.e4m3_decode(ref_q.cpu().numpy()), equal_nan=True)


def test_rank_with_no_rows():
    """An expert-parallel rank that holds none of the batch's experts: no
    gemm2_out rows (num_rows 0) and every slot -1. Each routed entry point
    returns what the oracle gives for the shared output alone, and an index
    >= 0 is skipped and flagged. The C call also takes a NULL gemm2_out."""
    T, H, K = 5, 1024, 4
    rng = np.random.default_rng(17)
    g2 = np.zeros((0, H), np.uint16)
    sh = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    res = W.to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    gam = W.to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    w = rng.random((T, K)).astype(np.float32)
    for stray in (False, True):
        idx = np.full((T, K), -1, np.int32)
        if stray:
            idx[2, 1] = 0                                  # row 0 does not exist here
        announce(f"rank with no rows, stray index {stray}")
        kw = dict(topk_weights=d_f32(w), shared_out=d_bf16(sh), routed_scaling_factor=2.5)
        errs = [torch.zeros(1, dtype=torch.int32, device=DEV) for _ in range(3)]
        d_g2, d_idx = d_bf16(g2), d_i32(idx)
        out = M.moe_finalize(d_g2, d_idx, err_flag=errs[0], **kw)
        ro, nm = M.moe_finalize_residual_rmsnorm(d_g2, d_idx, residual=d_bf16(res),
                                                 gamma=d_bf16(gam), eps=1e-6, err_flag=errs[1],
                                                 **kw)
        q, sc = M.moe_finalize_quant_ue8m0(d_g2, d_idx, err_flag=errs[2], **kw)
        torch.cuda.synchronize()
        okw = dict(weights_f32=w, shared=sh, rsf=2.5)
        m_out, flag = O.finalize_mirror(g2, idx, **okw)
        assert_bits_equal(h_bits(out), m_out, "finalize")
        m_ro, m_nm, _ = O.finalize_residual_rmsnorm_mirror(g2, idx, residual=res, gamma=gam,
                                                           eps=1e-6, **okw)
        assert_bits_equal(h_bits(ro), m_ro, "residual_out")
        g, o = F.bf16_to_f64(h_bits(nm)), F.bf16_to_f64(m_nm)
        assert np.all(np.abs(g - o) <= ulp_bf16(o)), "normed"
        m_q, m_s, _ = O.finalize_quant_mirror(g2, idx, **okw)
        assert_bits_equal(sc.cpu().numpy(), m_s, "scales")
        assert_bits_equal(q.cpu().numpy(), m_q, "codes")
        assert flag == (M.DEVERR_INDEX_OUT_OF_RANGE if stray else 0)
        assert [int(e.item()) for e in errs] == [flag] * 3
    L = M.load_library()
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    d_idx = d_i32(np.full((T, K), -1, np.int32))
    d_w, err = d_f32(w), torch.zeros(1, dtype=torch.int32, device=DEV)
    announce("rank with no rows, NULL gemm2_out and no shared output")
    assert L.moe_finalize(None, 0, d_idx.data_ptr(), d_w.data_ptr(), None, None, 2.5,
                          out.data_ptr(), T, H, K, err.data_ptr(),
                          torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert not h_bits(out).any() and int(err.item()) == 0     # +0 everywhere


def test_non_finite_values():
    """Non-finite results follow the fp32 arithmetic of the definition:
    +inf and -inf rows in one token give NaN, one +inf gives +inf, bf16-max
    rows whose weighted sum passes the fp32 range give +inf, a NaN row gives
    NaN. A generated NaN's sign is the platform's (x86 and gfx950 differ), so
    NaNs are compared as NaN and every other element bit for bit. In the
    quant epilogue a block holding a non-finite value takes e = 127 (the
    clamp), its finite values encode exactly, and each non-finite value gets
    an E4M3 NaN code. residual_out follows the same rule; normed is checked
    on the tokens whose residual_out is finite."""
    wl = W.make_workload(4, 256, 8, 4, rsf=2.5, seed=5, pad=8, with_residual=True)
    g2, r = wl.gemm2_out.copy(), wl.idx
    g2[r[0, 0], 3], g2[r[0, 1], 3] = 0x7F80, 0xFF80      # +inf, -inf -> NaN
    g2[r[0, 2], 4] = 0x7F80                              # +inf
    for k in range(4):
        g2[r[1, k], 5] = 0x7F7F                          # bf16 max: fp32 overflow
    g2[r[2, 3], 6] = 0x7FC0                              # NaN
    w = wl.weights.copy()
    w[1, :] = 0.25
    wl.gemm2_out, wl.weights = g2, w
    kw = device_inputs(wl)
    announce("non-finite values")
    out = M.moe_finalize(**kw)
    q, s = M.moe_finalize_quant_ue8m0(**kw)
    ro, nm = M.moe_finalize_residual_rmsnorm(**kw, residual=d_bf16(wl.residual),
                                             gamma=d_bf16(wl.gamma), eps=wl.eps)
    torch.cuda.synchronize()
    okw = dict(weights_f32=w, shared=wl.shared, rsf=wl.rsf)
    with np.errstate(over="ignore", invalid="ignore"):
        m_out, _ = O.finalize_mirror(g2, r, **okw)
        m_q, m_s, _ = O.finalize_quant_mirror(g2, r, **okw)
        m_ro, m_nm, _ = O.finalize_residual_rmsnorm_mirror(
            g2, r, residual=wl.residual, gamma=wl.gamma, eps=wl.eps, **okw)

    def nan_aware(got, want, what):
        gn = np.isnan(F.bf16_to_f64(got))
        wn = np.isnan(F.bf16_to_f64(want))
        assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
        assert_bits_equal(got[~wn], want[~wn], what)

    got = h_bits(out)
    nan_aware(got, m_out, "finalize")
    assert got[0, 4] == 0x7F80 and got[1, 5] == 0x7F80
    assert np.isnan(F.bf16_to_f64(got[[0, 2], [3, 6]])).all()
    y = F.bf16_to_f64(m_out)
    bad = ~np.isfinite(y)
    assert_bits_equal(h_u8(s), m_s, "scales")
    assert (h_u8(s)[[0, 1, 2], 0] == 254).all()
    gq = h_u8(q)
    assert_bits_equal(gq[~bad], m_q[~bad], "codes of finite values")
    assert np.isin(gq[bad], [0x7F, 0xFF]).all(), "non-finite values need a NaN code"
    nan_aware(h_bits(ro), m_ro, "residual_out")
    fin = np.isfinite(F.bf16_to_f64(m_ro)).all(axis=1)
    assert fin.tolist() == [False, False, False, True]
    g, o = F.bf16_to_f64(h_bits(nm)[fin]), F.bf16_to_f64(m_nm[fin])
    assert np.all(np.abs(g - o) <= ulp_bf16(o)), "normed of the finite token"


def test_results_do_not_depend_on_batch_size():
    """The same tokens give the same bits whether they come in a batch of
    1100 tokens or of 40: at 1100 tokens the RMSNorm epilogue stages whole
    tokens per CU, at 40 it runs one workgroup per token, and both sum the
    per-chunk partials in the same order. Plain and quant outputs are checked
    too (staged at 1100 tokens, one wave per unit at 40)."""
    T, n = 1100, 40
    wl = W.make_workload(T, 7168, 256, 8, rsf=2.5, seed=77, with_residual=True)
    kw = device_inputs(wl)
    res, gam = d_bf16(wl.residual), d_bf16(wl.gamma)
    small = dict(kw, expanded_idx_to_permuted_idx=kw["expanded_idx_to_permuted_idx"][:n].contiguous(),
                 topk_weights=kw["topk_weights"][:n].contiguous(),
                 shared_out=kw["shared_out"][:n].contiguous())
    announce(f"batch invariance T={T} vs {n}")
    ro, nm = M.moe_finalize_residual_rmsnorm(**kw, residual=res, gamma=gam, eps=wl.eps)
    ro_s, nm_s = M.moe_finalize_residual_rmsnorm(**small, residual=res[:n].contiguous(),
                                                 gamma=gam, eps=wl.eps)
    out, out_s = M.moe_finalize(**kw), M.moe_finalize(**small)
    (q, s), (q_s, s_s) = M.moe_finalize_quant_ue8m0(**kw), M.moe_finalize_quant_ue8m0(**small)
    torch.cuda.synchronize()
    for big, sm, what in ((ro, ro_s, "residual_out"), (nm, nm_s, "normed"), (out, out_s, "out"),
                          (q, q_s, "codes"), (s, s_s, "scales")):
        assert torch.equal(big[:n].view(torch.uint8), sm.view(torch.uint8)), what
    m_ro, m_nm, _ = O.finalize_residual_rmsnorm_mirror(
        wl.gemm2_out, wl.idx, residual=wl.residual, gamma=wl.gamma, eps=wl.eps,
        weights_f32=wl.weights, shared=wl.shared, rsf=wl.rsf)
    assert_bits_equal(h_bits(ro), m_ro, "residual_out")
    g, o = F.bf16_to_f64(h_bits(nm)), F.bf16_to_f64(m_nm)
    assert np.all(np.abs(g - o) <= ulp_bf16(o)), "normed"


@pytest.mark.parametrize("H", [1000, 4104, 5000, 16384])
def test_rmsnorm_half_width_ragged(H):
    """From 288 tokens on (below the staged path's 40 units per CU), a row
    with an even number of 512-column chunks takes half-width workgroups with
    two vectors per lane. Ragged hidden sizes there: H=1000 (2 chunks, the
    second vector of most lanes past the row end), 4104 (9 chunks: odd, stays
    full width), 5000 (10 chunks, partly filled), 16384 (32 chunks, the
    widest workgroup either way). residual_out is bit-exact to the mirror,
    normed within one ulp of the fp64 RMSNorm, and the first tokens match a
    16-token (full-width) call bit for bit."""
    T, k = 300, 4
    wl = W.make_workload(T, H, 32, k, rsf=2.5, seed=H, with_residual=True, log2_mag=(-4.0, 4.0))
    kw = device_inputs(wl)
    res, gam = d_bf16(wl.residual), d_bf16(wl.gamma)
    announce(f"half-width rmsnorm T={T} H={H}")
    ro, nm = M.moe_finalize_residual_rmsnorm(**kw, residual=res, gamma=gam, eps=wl.eps)
    n = 16
    small = dict(kw, expanded_idx_to_permuted_idx=kw["expanded_idx_to_permuted_idx"][:n],
                 topk_weights=kw["topk_weights"][:n], shared_out=kw["shared_out"][:n])
    ro_s, nm_s = M.moe_finalize_residual_rmsnorm(**small, residual=res[:n], gamma=gam, eps=wl.eps)
    torch.cuda.synchronize()
    m_ro, m_nm, _ = O.finalize_residual_rmsnorm_mirror(
        wl.gemm2_out, wl.idx, residual=wl.residual, gamma=wl.gamma, eps=wl.eps,
        weights_f32=wl.weights, shared=wl.shared, rsf=wl.rsf)
    assert_bits_equal(h_bits(ro), m_ro, f"H={H} residual_out")
    g, o = F.bf16_to_f64(h_bits(nm)), F.bf16_to_f64(m_nm)
    assert np.all(np.abs(g - o) <= ulp_bf16(o)), f"H={H} normed"
    assert torch.equal(ro[:n].view(torch.int16), ro_s.view(torch.int16))
    assert torch.equal(nm[:n].view(torch.int16), nm_s.view(torch.int16))


@pytest.mark.parametrize("T_per_cu,H,k,packed", [
    (None, 1024, 3, False),      # one wave per unit, top_k below its template's width
    (None, 1024, 8, True),
    (100, 1024, 4, False),       # the staged plain, RMSNorm and quant kernels
])
def test_skipped_slots_ignore_their_weights(T_per_cu, H, k, packed):
    """A slot whose index is negative or out of range is skipped whatever its
    weight holds. NaN, +-inf and huge fp32 weights, or packed words whose bf16
    half is NaN or inf, on skipped slots leave every output equal to the
    oracle's, which never reads them: the gather takes such a slot's weight
    as -0 instead of multiplying by it. Plain, residual + RMSNorm and quant
    entry points, one-wave-per-unit and staged sizes."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    T = 40 if T_per_cu is None else T_per_cu * ncu
    wl = W.make_workload(T, H, 16, k, rsf=2.5, seed=900 + k, pad=32, with_residual=True,
                         log2_mag=(-4.0, 4.0))
    rng = np.random.default_rng(900 + k)
    idx = wl.idx.copy()
    skip = rng.random(idx.shape) < 0.3
    oob = (rng.random(idx.shape) < 0.05) & ~skip
    idx[skip] = -1
    idx[oob] = wl.P + 7
    dead = skip | oob
    w = wl.weights.copy()
    w[dead] = np.array([np.nan, np.inf, -np.inf, 3.0e38], np.float32)[rng.integers(0, 4, dead.sum())]
    pk = wl.packed.view(np.uint32).copy()
    halves = np.array([0x7FC0, 0x7F80, 0xFF80, 0xFFC1], np.uint32)[rng.integers(0, 4, dead.sum())]
    pk[dead] = (pk[dead] & np.uint32(0xFFFF0000)) | halves
    wl.idx, wl.weights, wl.packed = idx, w, pk.view(np.int32)
    wkw = dict(packed=wl.packed) if packed else dict(weights_f32=w)
    np.seterr(over="ignore")       # the oracle scales the dead slots' huge weights too
    announce(f"skipped slots with non-finite weights T={T} H={H} k={k} packed={packed}")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_finalize(wl, packed=packed, err=err)
    assert int(err.item()) == M.DEVERR_INDEX_OUT_OF_RANGE
    mirror, _ = O.finalize_mirror(wl.gemm2_out, idx, shared=wl.shared, rsf=wl.rsf, **wkw)
    assert_bits_equal(got, mirror, "finalize")
    assert np.isfinite(F.bf16_to_f64(got)).all()
    kw = device_inputs(wl, packed=packed)
    ro, nm = M.moe_finalize_residual_rmsnorm(**kw, residual=d_bf16(wl.residual),
                                             gamma=d_bf16(wl.gamma), eps=wl.eps)
    q, s = M.moe_finalize_quant_ue8m0(**kw)
    torch.cuda.synchronize()
    m_ro, m_nm, _ = O.finalize_residual_rmsnorm_mirror(
        wl.gemm2_out, idx, shared=wl.shared, rsf=wl.rsf, residual=wl.residual, gamma=wl.gamma,
        eps=wl.eps, **wkw)
    assert_bits_equal(h_bits(ro), m_ro, "residual_out")
    g, o = F.bf16_to_f64(h_bits(nm)), F.bf16_to_f64(m_nm)
    assert np.all(np.abs(g - o) <= ulp_bf16(o)), "normed"
    mq, ms, _ = O.finalize_quant_mirror(wl.gemm2_out, idx, shared=wl.shared, rsf=wl.rsf, **wkw)
    assert_bits_equal(h_u8(s), ms, "scale bytes")
    assert_bits_equal(h_u8(q), mq, "codes")
