"""Robustness of every entry point on the GPU: HIP-graph capture and replay,
launch on the caller's stream, run-to-run determinism, guard canaries around every output, the maximum
hidden size and an odd large token count. Expected values come from the
oracle or from the same call run eagerly (replay and determinism checks)."""
import numpy as np
import pytest
import torch

import combine_moe_finalize_amd as M
from combine_moe_finalize_amd import workloads as W
from oracle import act_quant as A
from oracle import finalize as O
from oracle import routing as R

from gpu_helpers import (DEV, announce, assert_bits_equal, d_bf16, d_f32, d_i32, device_inputs,
                         h_bits)

pytestmark = pytest.mark.gpu

GUARD = 4096   # bytes of canary on each side of every output


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    M.load_library()


def guarded(shape, dtype):
    """A tensor of `shape` inside a byte buffer with canaries on both sides."""
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((n + 2 * GUARD,), 0xA5, dtype=torch.uint8, device=DEV)
    t = buf[GUARD:GUARD + n].view(dtype).view(*shape)
    return buf, t


def canaries_intact(buf):
    b = buf.cpu().numpy()
    return bool(np.all(b[:GUARD] == 0xA5) and np.all(b[-GUARD:] == 0xA5))


def snapshot(ts):
    return [t.detach().clone() for t in ts]


def same(a, b):
    return all(torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                           y.view(torch.uint8) if y.dtype != torch.uint8 else y)
               for x, y in zip(a, b))


def entry_points():
    """(name, fn writing into its outputs, outputs, buffers) per entry point."""
    wl = W.family_workload("decode_sweep", 16)
    wr = W.make_workload(8, 7168, 64, 8, rsf=2.5, seed=3, with_residual=True)
    cases = []

    kw = device_inputs(wl)
    b, out = guarded((wl.T, wl.H), torch.bfloat16)
    cases.append(("finalize", lambda: M.moe_finalize(**kw, out=out), [out], [b]))

    kwp = device_inputs(wl, packed=True)
    b2, outp = guarded((wl.T, wl.H), torch.bfloat16)
    cases.append(("finalize_packed", lambda: M.moe_finalize(**kwp, out=outp), [outp], [b2]))

    kr = device_inputs(wr)
    res, gam = d_bf16(wr.residual), d_bf16(wr.gamma)
    b3, ro = guarded((wr.T, wr.H), torch.bfloat16)
    b4, nm = guarded((wr.T, wr.H), torch.bfloat16)
    cases.append(("rmsnorm", lambda: M.moe_finalize_residual_rmsnorm(
        **kr, residual=res, gamma=gam, eps=wr.eps, residual_out=ro, normed=nm), [ro, nm], [b3, b4]))

    b5, q = guarded((wr.T, wr.H), torch.uint8)
    b6, s = guarded((wr.T, wr.H // 128), torch.uint8)
    cases.append(("quant", lambda: M.moe_finalize_quant_ue8m0(**kr, out_e4m3=q, scale_e8m0=s),
                  [q, s], [b5, b6]))

    pk = d_i32(wl.packed)
    b7, ids = guarded(tuple(wl.packed.shape), torch.int32)
    b8, dw = guarded(tuple(wl.packed.shape), torch.float32)
    cases.append(("decode", lambda: M.moe_topk_packed_decode(pk, expert_ids=ids, weights=dw),
                  [ids, dw], [b7, b8]))

    lg = torch.from_numpy(W.router_logits(33, 256, seed=2)).to(DEV)
    b9, gi = guarded((33, 8), torch.int32)
    b10, gw = guarded((33, 8), torch.float32)
    b11, gp = guarded((33, 8), torch.int32)
    cases.append(("gate", lambda: M.moe_topk_sigmoid_gate(lg, 8, topk_ids=gi, topk_weights=gw,
                                                          topk_packed=gp), [gi, gw, gp],
                  [b9, b10, b11]))

    xa = d_bf16(W.activations(9, 1152, seed=4))
    b12, aq = guarded((9, 1152), torch.uint8)
    b13, a8 = guarded((9, 9), torch.uint8)
    b14, aq2 = guarded((9, 1152), torch.uint8)
    b15, af = guarded((9, 9), torch.float32)
    cases.append(("act_quant", lambda: (M.moe_act_quant_fp8_ue8m0(xa, out_e4m3=aq, scale_e8m0=a8),
                                        M.moe_act_quant_fp8_amax(xa, out_e4m3=aq2, scale_f32=af)),
                  [aq, a8, aq2, af], [b12, b13, b14, b15]))

    parts = d_bf16(W.activations(3 * 5, 1000, seed=6, log2_mag=None)).view(3, 5, 1000)
    shp = d_bf16(W.activations(5, 1000, seed=7, log2_mag=None))
    b16, eo = guarded((5, 1000), torch.bfloat16)
    cases.append(("ep_combine", lambda: M.moe_finalize_ep_combine(parts, shared_out=shp, out=eo),
                  [eo], [b16]))

    ranks = [d_bf16(W.activations(6, 7168, seed=20 + r, log2_mag=None)) for r in range(3)]
    ares = d_bf16(W.activations(6, 7168, seed=24, log2_mag=None))
    agam = d_bf16(W.activations(1, 7168, seed=25, log2_mag=None)[0])
    b17, aro = guarded((6, 7168), torch.bfloat16)
    b18, anm = guarded((6, 7168), torch.bfloat16)
    cases.append(("allreduce", lambda: M.moe_allreduce_residual_rmsnorm(
        ranks, residual=ares, gamma=agam, residual_out=aro, normed=anm), [aro, anm], [b17, b18]))
    return cases


def test_determinism_and_canaries():
    for name, fn, outs, bufs in entry_points():
        announce(f"determinism + canaries: {name}")
        fn()
        torch.cuda.synchronize()
        first = snapshot(outs)
        fn()
        torch.cuda.synchronize()
        assert same(first, outs), f"{name}: two runs differ"
        assert all(canaries_intact(b) for b in bufs), f"{name}: wrote outside its outputs"


def test_graph_capture_replay_every_entry_point():
    for name, fn, outs, bufs in entry_points():
        announce(f"graph replay: {name}")
        fn()
        torch.cuda.synchronize()
        eager = snapshot(outs)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for i in range(4):
            for t in outs:
                t.view(torch.uint8).fill_(0x3C) if t.dtype != torch.uint8 else t.fill_(0x3C)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert same(eager, outs), f"{name}: replay {i} differs from the eager run"
            _ = (torch.arange(4096, device=DEV) * i).sum().item()   # eager work between replays
        assert all(canaries_intact(b) for b in bufs), name
        del g


def test_calls_run_on_the_callers_stream():
    """Every entry point launches on the stream current at the call. A side
    stream runs a few milliseconds of fills, then overwrites the outputs with
    a pattern, then makes the call: only a launch queued on that stream,
    behind the pattern, leaves the eager result in the outputs."""
    busy = torch.empty(1 << 28, dtype=torch.int32, device=DEV)          # 1 GiB
    for name, fn, outs, bufs in entry_points():
        announce(f"caller's stream: {name}")
        fn()
        torch.cuda.synchronize()
        eager = snapshot(outs)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(8):
                busy.fill_(i)
            for t in outs:
                t.view(torch.uint8).fill_(0x3C) if t.dtype != torch.uint8 else t.fill_(0x3C)
            fn()
        torch.cuda.synchronize()
        assert same(eager, outs), f"{name}: the call did not run behind its stream's work"
        assert all(canaries_intact(b) for b in bufs), name
    del busy


def test_maximum_hidden_size():
    H = 1 << 20
    wl = W.make_workload(2, H, 2, 2, rsf=2.5, seed=8, pad=2)
    announce(f"finalize and quant at H={H}")
    kw = device_inputs(wl)
    out = h_bits(M.moe_finalize(**kw))
    q, s = M.moe_finalize_quant_ue8m0(**kw)
    torch.cuda.synchronize()
    ref, _ = O.finalize_mirror(wl.gemm2_out, wl.idx, weights_f32=wl.weights, shared=wl.shared,
                               rsf=wl.rsf)
    assert_bits_equal(out, ref, "H=2^20 finalize")
    mq, ms, _ = O.quant_ue8m0(ref)
    assert_bits_equal(s.cpu().numpy(), ms, "H=2^20 scales")
    assert_bits_equal(q.cpu().numpy(), mq, "H=2^20 codes")


def test_odd_large_token_count():
    wl = W.make_workload(12345, 1000, 64, 3, rsf=0.75, seed=9, pad=32)
    announce("finalize T=12345 H=1000 k=3")
    out = h_bits(M.moe_finalize(**device_inputs(wl, packed=True)))
    torch.cuda.synchronize()
    ref, _ = O.finalize_mirror(wl.gemm2_out, wl.idx, packed=wl.packed, shared=wl.shared,
                               rsf=wl.rsf)
    assert_bits_equal(out, ref, "T=12345")
    lg = W.router_logits(12345, 100, seed=10)
    ids, _, _ = M.moe_topk_sigmoid_gate(torch.from_numpy(lg).to(DEV), 5)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), R.topk_order(lg, 5))
    xa = W.activations(12345, 256, seed=11)
    q, s = M.moe_act_quant_fp8_amax(d_bf16(xa))
    torch.cuda.synchronize()
    oq, os_ = A.act_quant_amax(xa)
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_)


def test_largest_row_indices():
    """num_rows = 2^31 - 1 rows of H = 8 (32 GiB): rows near the top of the
    int32 index range sit more than 2^34 bytes into gemm2_out, so any 32-bit
    offset arithmetic would fail. Only the gathered rows are written; the
    expected values come from the same rows in a compact buffer (layout
    invariance) through the oracle."""
    H, T, K = 8, 64, 4
    P = 2 ** 31 - 1
    wl = W.make_workload(T, H, 16, K, rsf=2.5, seed=12, pad=8)
    rng = np.random.default_rng(13)
    top = P - 1 - rng.choice(2 ** 20, size=T * K, replace=False)   # distinct rows near the top
    idx_big = top.reshape(T, K).astype(np.int32)
    compact = wl.gemm2_out[wl.idx.reshape(-1)]                       # the rows, in slot order
    announce(f"largest row indices: P={P} H={H}")
    g2 = torch.empty((P, H), dtype=torch.bfloat16, device=DEV)     # 32 GiB, not initialised
    g2[torch.from_numpy(top).to(DEV)] = d_bf16(compact)
    out = M.moe_finalize(g2, d_i32(idx_big), topk_weights=d_f32(wl.weights),
                         shared_out=d_bf16(wl.shared), routed_scaling_factor=wl.rsf)
    torch.cuda.synchronize()
    got = h_bits(out)
    del g2
    torch.cuda.empty_cache()
    idx_c = np.arange(T * K, dtype=np.int32).reshape(T, K)
    ref, flag = O.finalize_mirror(compact, idx_c, weights_f32=wl.weights, shared=wl.shared,
                                  rsf=wl.rsf)
    assert flag == 0
    assert_bits_equal(got, ref, "largest row indices")
