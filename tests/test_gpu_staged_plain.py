"""GPU parity of the plain finalize's staged-output path.

From 48 (token, chunk) units per CU the bf16 finalize runs one workgroup per
CU that takes units from an LDS counter, keeps each unit's 1 KiB of output in
LDS (159 units per CU) and, past that, in register slots, and writes it all
after its last gather. Workgroups of 16 waves with 8 slots a wave hold 287
units per CU; larger grids take workgroups of 12 waves with 25 slots a wave
(459 units per CU) and, past that, several launches. The grids here are
sized from the device's CU count so that each case lands on one of those
paths; every output is compared bit for bit with the oracle's fp32 mirror."""
import numpy as np
import pytest
import torch

import combine_moe_finalize_amd as M
from combine_moe_finalize_amd import workloads as W
from oracle import finalize as O

from gpu_helpers import DEV, announce, assert_bits_equal, device_inputs, h_bits

pytestmark = pytest.mark.gpu

STAGED_FROM_UNITS_PER_CU = 48
LDS_UNITS = 159
REG_UNITS_PER_CU = 16 * 8


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


def run_plain(wl, packed=False, with_shared=True, idx=None, err=None):
    kw = device_inputs(wl, packed=packed, with_shared=with_shared)
    if idx is not None:
        kw["expanded_idx_to_permuted_idx"] = torch.from_numpy(idx).to(DEV)
    out = M.moe_finalize(**kw, err_flag=err)
    torch.cuda.synchronize()
    return h_bits(out)


def check_mirror(wl, got, packed=False, with_shared=True, idx=None, chunk=8192):
    idx = wl.idx if idx is None else idx
    for t0 in range(0, wl.T, chunk):
        sl = slice(t0, min(wl.T, t0 + chunk))
        wk = dict(packed=wl.packed[sl]) if packed else dict(weights_f32=wl.weights[sl])
        sh = wl.shared[sl] if with_shared else None
        m, _ = O.finalize_mirror(wl.gemm2_out, idx[sl], shared=sh, rsf=wl.rsf, **wk)
        assert_bits_equal(got[sl], m, f"tokens {sl}")


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7, 8])
def test_lds_staged_every_top_k(ncu, k):
    """64 units per CU: every unit staged in LDS; exact and guarded top_k."""
    H = 128
    T = 64 * ncu
    wl = W.make_workload(T, H, 16, k, rsf=2.5, seed=800 + k, pad=32)
    announce(f"staged finalize (LDS) T={T} H={H} k={k}")
    got = run_plain(wl, packed=(k % 2 == 0))
    check_mirror(wl, got, packed=(k % 2 == 0))


def test_register_slots(ncu):
    """250 units per CU: 91 of each CU's units wait in register slots."""
    H, k = 128, 8
    T = 250 * ncu
    assert LDS_UNITS * ncu < T * chunks(H) <= (LDS_UNITS + REG_UNITS_PER_CU) * ncu
    wl = W.make_workload(T, H, 16, k, rsf=2.5, seed=811, pad=128)
    announce(f"staged finalize (LDS + registers) T={T} H={H} k={k}")
    got = run_plain(wl)
    check_mirror(wl, got)


def test_several_launches(ncu):
    """More units than one launch holds: the grid is split over launches."""
    H, k = 128, 2
    T = 700 * ncu
    assert T * chunks(H) > (LDS_UNITS + REG_UNITS_PER_CU) * ncu * 2
    wl = W.make_workload(T, H, 16, k, rsf=1.5, seed=812, pad=128)
    announce(f"staged finalize, several launches T={T} H={H} k={k}")
    got = run_plain(wl, packed=True)
    check_mirror(wl, got, packed=True)


def test_ragged_chunks_no_shared(ncu):
    """H = 1160: three chunks per token, the last one 17 of 64 lanes."""
    H, k = 1160, 6
    T = (STAGED_FROM_UNITS_PER_CU * ncu) // chunks(H) + 37
    wl = W.make_workload(T, H, 32, k, rsf=2.5, seed=813, pad=64)
    announce(f"staged finalize ragged T={T} H={H} k={k} no shared")
    got = run_plain(wl, with_shared=False)
    check_mirror(wl, got, with_shared=False)


def test_skipped_and_out_of_range_slots(ncu):
    H, k = 256, 8
    T = 100 * ncu
    wl = W.make_workload(T, H, 64, k, rsf=2.5, seed=814, pad=128)
    rng = np.random.default_rng(814)
    idx = wl.idx.copy()
    idx[rng.random(idx.shape) < 0.05] = -1
    idx[rng.integers(0, T, 7), rng.integers(0, k, 7)] = wl.P + 3
    announce(f"staged finalize with skipped / out-of-range slots T={T} H={H}")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run_plain(wl, idx=idx, err=err)
    assert int(err.item()) == M.DEVERR_INDEX_OUT_OF_RANGE
    check_mirror(wl, got, idx=idx)


def test_batch_split_gives_the_same_bits(ncu):
    """A batch on the staged path against the same tokens in slices small
    enough for the one-wave-per-unit kernel: identical bits."""
    H, k = 7168, 8
    T = 2 * STAGED_FROM_UNITS_PER_CU * ncu // chunks(H) + 5
    wl = W.make_workload(T, H, 256, k, rsf=2.5, seed=815)
    kw = device_inputs(wl)
    announce(f"staged finalize vs sliced batches T={T} H={H}")
    out = M.moe_finalize(**kw)
    out2 = torch.empty_like(out)
    step = max(1, (STAGED_FROM_UNITS_PER_CU * ncu) // chunks(H) // 4)
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        M.moe_finalize(kw["gemm2_out"], kw["expanded_idx_to_permuted_idx"][t0:t1],
                       topk_weights=kw["topk_weights"][t0:t1], shared_out=kw["shared_out"][t0:t1],
                       routed_scaling_factor=wl.rsf, out=out2[t0:t1])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    check_mirror(wl, h_bits(out), chunk=512)


def test_graph_capture_of_several_launches(ncu):
    H, k = 128, 4
    T = 400 * ncu
    wl = W.make_workload(T, H, 16, k, rsf=2.5, seed=816, pad=128)
    kw = device_inputs(wl)
    announce(f"staged finalize under graph capture T={T} H={H}")
    o0 = M.moe_finalize(**kw)
    o = torch.zeros_like(o0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.moe_finalize(**kw, out=o)                      # warm-up off the graph
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            M.moe_finalize(**kw, out=o)
    torch.cuda.synchronize()
    for _ in range(3):
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16))
    check_mirror(wl, h_bits(o0))


def test_concurrent_calls_on_two_streams(ncu):
    H, k = 7168, 8
    T = 2 * STAGED_FROM_UNITS_PER_CU * ncu // chunks(H)
    wa = W.make_workload(T, H, 256, k, rsf=2.5, seed=817)
    wb = W.make_workload(T, H, 256, k, rsf=1.25, seed=818)
    ka, kb = device_inputs(wa), device_inputs(wb, packed=True)
    announce(f"staged finalize, two streams T={T} H={H}")
    a0, b0 = M.moe_finalize(**ka), M.moe_finalize(**kb)
    torch.cuda.synchronize()
    a, b = torch.zeros_like(a0), torch.zeros_like(b0)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            M.moe_finalize(**ka, out=a)
        with torch.cuda.stream(s2):
            M.moe_finalize(**kb, out=b)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), a0.view(torch.int16))
    assert torch.equal(b.view(torch.int16), b0.view(torch.int16))


@pytest.mark.parametrize("case", range(4))
def test_random_staged_configs(ncu, case):
    rng = np.random.default_rng(5200 + case)
    k = int(rng.integers(1, 9))
    H = 8 * int(rng.integers(1, 513))
    per_cu = int(rng.integers(48, 301))
    T = -(-per_cu * ncu // chunks(H))
    packed = bool(rng.random() < 0.5)
    with_shared = bool(rng.random() < 0.7)
    rsf = float(np.float32(rng.uniform(0.25, 4.0)))
    wl = W.make_workload(T, H, 64, k, rsf=rsf, seed=int(rng.integers(1 << 30)),
                         pad=int(rng.choice([8, 64, 128])), with_shared=with_shared)
    idx = wl.idx.copy()
    idx[rng.random(idx.shape) < 0.03] = -1
    announce(f"staged finalize random case {case}: T={T} H={H} k={k} per_cu={per_cu} "
             f"packed={packed} shared={with_shared}")
    got = run_plain(wl, packed=packed, with_shared=with_shared, idx=idx)
    check_mirror(wl, got, packed=packed, with_shared=with_shared, idx=idx)


def test_exactly_one_launch_capacity(ncu):
    """H = 128 at the largest grid one launch holds: every workgroup gets
    287 units, 159 in LDS and 16 x 8 in register slots, so a wave that takes
    more than its share of the units past the LDS slots writes its extra
    units at once."""
    H, k = 128, 4
    T = (LDS_UNITS + REG_UNITS_PER_CU) * ncu
    wl = W.make_workload(T, H, 16, k, rsf=2.5, seed=815, pad=64)
    announce(f"staged finalize at one launch's capacity T={T} H={H} k={k}")
    got = run_plain(wl)
    check_mirror(wl, got)


WIDE_UNITS_PER_CU = 159 + 12 * 25


def test_wide_layout_at_capacity(ncu):
    """Past what one 16-wave launch holds, the plain finalize takes 12-wave
    workgroups with 25 register slots a wave: H = 128 at exactly one such
    launch's capacity (459 units per CU, 300 of them in register slots)."""
    H, k = 128, 4
    T = WIDE_UNITS_PER_CU * ncu
    wl = W.make_workload(T, H, 16, k, rsf=2.5, seed=816, pad=64)
    announce(f"staged finalize, wide layout at capacity T={T} H={H} k={k}")
    got = run_plain(wl, packed=True)
    check_mirror(wl, got, packed=True)


def test_wide_layout_prefill_shape(ncu):
    """The prefill shape the wide layout exists for (T = 8192, H = 7168,
    top_k = 8: 448 units per CU on 256 CUs, one launch), against the mirror."""
    wl = W.family_workload("prefill_fp8_ue8m0")
    announce(f"staged finalize, prefill T={wl.T} H={wl.H} (wide layout from "
             f"{(LDS_UNITS + REG_UNITS_PER_CU) * ncu} units)")
    got = run_plain(wl)
    check_mirror(wl, got, chunk=2048)
