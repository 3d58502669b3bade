"""GPU parity of the UE8M0 finalize's staged-output path.

From 80 (token, chunk) units per CU the quant finalize runs one workgroup per
CU (tokens dealt to one group of workgroups per XCD in blocks of 16) that
takes units from an LDS counter, keeps their codes and scale bytes in
LDS (317 units per CU) and, past that, in 12 register slots per wave, and
writes them after its last gather; grids larger than that take several
launches. From 160 units per CU the last 5% of each group's units go to
extra workgroups that write at once (the register-slot, out-of-range and
several-launch cases below run with them). These tests size their grids from the device's CU count so that
each case lands on one of those paths, and compare every code and scale byte
with the oracle's fp32 mirror (bit for bit)."""
import numpy as np
import pytest
import torch

import combine_moe_finalize_amd as M
from combine_moe_finalize_amd import workloads as W
from oracle import finalize as O

from gpu_helpers import DEV, announce, assert_bits_equal, device_inputs, h_u8

pytestmark = pytest.mark.gpu

STAGED_FROM_UNITS_PER_CU = 80
LDS_UNITS = 317
REG_UNITS_PER_CU = 16 * 12


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


def run_quant(wl, packed=False, with_shared=True, idx=None, err=None):
    kw = device_inputs(wl, packed=packed, with_shared=with_shared)
    if idx is not None:
        kw["expanded_idx_to_permuted_idx"] = torch.from_numpy(idx).to(DEV)
    q, s = M.moe_finalize_quant_ue8m0(**kw, err_flag=err)
    torch.cuda.synchronize()
    return h_u8(q), h_u8(s)


def check_mirror(wl, q, s, packed=False, with_shared=True, idx=None, chunk=8192):
    idx = wl.idx if idx is None else idx
    for t0 in range(0, wl.T, chunk):
        sl = slice(t0, min(wl.T, t0 + chunk))
        wk = dict(packed=wl.packed[sl]) if packed else dict(weights_f32=wl.weights[sl])
        sh = wl.shared[sl] if with_shared else None
        mq, ms, _ = O.finalize_quant_mirror(wl.gemm2_out, idx[sl], shared=sh, rsf=wl.rsf, **wk)
        assert_bits_equal(s[sl], ms, f"scale bytes, tokens {sl}")
        assert_bits_equal(q[sl], mq, f"codes, tokens {sl}")


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7, 8])
def test_lds_staged_every_top_k(ncu, k):
    """150 units per CU: every unit staged in LDS (no tail workgroups below
    160 units per CU); exact and guarded top_k."""
    H = 128
    T = 150 * ncu
    wl = W.make_workload(T, H, 16, k, rsf=2.5, seed=700 + k, pad=32, log2_mag=(-8, 8))
    announce(f"staged quant (LDS) T={T} H={H} k={k}")
    q, s = run_quant(wl, packed=(k % 2 == 1))
    check_mirror(wl, q, s, packed=(k % 2 == 1))


def test_register_slots(ncu):
    """400 units per CU: 83 of each CU's units wait in register slots."""
    H, k = 128, 8
    T = 400 * ncu
    assert T * chunks(H) > LDS_UNITS * ncu
    wl = W.make_workload(T, H, 16, k, rsf=2.5, seed=711, pad=128, log2_mag=(-8, 8))
    announce(f"staged quant (LDS + registers) T={T} H={H} k={k}")
    q, s = run_quant(wl)
    check_mirror(wl, q, s)


def test_several_launches(ncu):
    """More units than one launch holds: the grid is split over launches."""
    H, k = 128, 2
    T = 1100 * ncu
    assert T * chunks(H) > (LDS_UNITS + REG_UNITS_PER_CU) * ncu * 2
    wl = W.make_workload(T, H, 16, k, rsf=1.5, seed=712, pad=128, log2_mag=(-8, 8))
    announce(f"staged quant, several launches T={T} H={H} k={k}")
    q, s = run_quant(wl, packed=True)
    check_mirror(wl, q, s, packed=True)


def test_ragged_chunks_no_shared(ncu):
    """H = 1152: three chunks per token, the last one a quarter full."""
    H, k = 1152, 6
    T = (STAGED_FROM_UNITS_PER_CU * ncu) // chunks(H) + 37
    wl = W.make_workload(T, H, 32, k, rsf=2.5, seed=713, pad=64, log2_mag=(-8, 8))
    announce(f"staged quant ragged T={T} H={H} k={k} no shared")
    q, s = run_quant(wl, with_shared=False)
    check_mirror(wl, q, s, with_shared=False)


def test_skipped_and_out_of_range_slots(ncu):
    H, k = 256, 8
    T = 200 * ncu
    wl = W.make_workload(T, H, 64, k, rsf=2.5, seed=714, pad=128, log2_mag=(-8, 8))
    rng = np.random.default_rng(714)
    idx = wl.idx.copy()
    idx[rng.random(idx.shape) < 0.05] = -1
    idx[rng.integers(0, T, 7), rng.integers(0, k, 7)] = wl.P + 3
    announce(f"staged quant with skipped / out-of-range slots T={T} H={H}")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    q, s = run_quant(wl, idx=idx, err=err)
    assert int(err.item()) == M.DEVERR_INDEX_OUT_OF_RANGE
    check_mirror(wl, q, s, idx=idx)


def test_batch_split_gives_the_same_bytes(ncu):
    """A batch large enough for the staged path against the same tokens in
    slices small enough for the one-wave-per-unit kernel: identical bytes."""
    H, k = 7168, 8
    T = 2 * STAGED_FROM_UNITS_PER_CU * ncu // chunks(H)
    wl = W.make_workload(T, H, 256, k, rsf=2.5, seed=715, log2_mag=(-8, 8))
    kw = device_inputs(wl)
    announce(f"staged quant vs sliced batches T={T} H={H}")
    q, s = M.moe_finalize_quant_ue8m0(**kw)
    q2 = torch.empty_like(q)
    s2 = torch.empty_like(s)
    step = max(1, (STAGED_FROM_UNITS_PER_CU * ncu) // chunks(H) // 4)
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        M.moe_finalize_quant_ue8m0(kw["gemm2_out"], kw["expanded_idx_to_permuted_idx"][t0:t1],
                                   topk_weights=kw["topk_weights"][t0:t1],
                                   shared_out=kw["shared_out"][t0:t1],
                                   routed_scaling_factor=wl.rsf,
                                   out_e4m3=q2[t0:t1], scale_e8m0=s2[t0:t1])
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2)
    check_mirror(wl, h_u8(q), h_u8(s), chunk=1024)


def test_graph_capture_of_several_launches(ncu):
    """The staged path (two launches here) captured in a HIP graph: every
    replay gives the eager call's bytes."""
    H, k = 128, 4
    T = 600 * ncu
    wl = W.make_workload(T, H, 16, k, rsf=2.5, seed=716, pad=128, log2_mag=(-8, 8))
    kw = device_inputs(wl)
    announce(f"staged quant under graph capture T={T} H={H}")
    q0, s0 = M.moe_finalize_quant_ue8m0(**kw)
    q = torch.zeros_like(q0)
    s = torch.zeros_like(s0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.moe_finalize_quant_ue8m0(**kw, out_e4m3=q, scale_e8m0=s)      # warm-up off the graph
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            M.moe_finalize_quant_ue8m0(**kw, out_e4m3=q, scale_e8m0=s)
    torch.cuda.synchronize()
    for _ in range(3):
        q.zero_()
        s.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q, q0) and torch.equal(s, s0)
    check_mirror(wl, h_u8(q0), h_u8(s0))


def test_concurrent_calls_on_two_streams(ncu):
    """Two staged launches in flight at once on two streams (default
    priority): each workgroup waits on nothing outside itself, so the calls
    share the CUs in any order and both give the single-stream bytes."""
    H, k = 7168, 8
    T = 2 * STAGED_FROM_UNITS_PER_CU * ncu // chunks(H)
    wa = W.make_workload(T, H, 256, k, rsf=2.5, seed=717, log2_mag=(-8, 8))
    wb = W.make_workload(T, H, 256, k, rsf=1.25, seed=718, log2_mag=(-8, 8))
    ka, kb = device_inputs(wa), device_inputs(wb, packed=True)
    announce(f"staged quant, two streams T={T} H={H}")
    qa0, sa0 = M.moe_finalize_quant_ue8m0(**ka)
    qb0, sb0 = M.moe_finalize_quant_ue8m0(**kb)
    torch.cuda.synchronize()
    qa, sa = torch.zeros_like(qa0), torch.zeros_like(sa0)
    qb, sb = torch.zeros_like(qb0), torch.zeros_like(sb0)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            M.moe_finalize_quant_ue8m0(**ka, out_e4m3=qa, scale_e8m0=sa)
        with torch.cuda.stream(s2):
            M.moe_finalize_quant_ue8m0(**kb, out_e4m3=qb, scale_e8m0=sb)
    torch.cuda.synchronize()
    assert torch.equal(qa, qa0) and torch.equal(sa, sa0)
    assert torch.equal(qb, qb0) and torch.equal(sb, sb0)


@pytest.mark.parametrize("case", range(6))
def test_random_staged_configs(ncu, case):
    """Seeded random shapes and options on the staged path: top_k 1..8,
    hidden a multiple of 128 up to 4096, 80..400 units per CU (LDS slots
    only, or LDS and register slots), fp32 or packed weights, with or without the shared output, random
    routed scaling factor and skipped slots."""
    rng = np.random.default_rng(4200 + case)
    k = int(rng.integers(1, 9))
    H = 128 * int(rng.integers(1, 33))
    per_cu = int(rng.integers(80, 401))
    T = -(-per_cu * ncu // chunks(H))
    packed = bool(rng.random() < 0.5)
    with_shared = bool(rng.random() < 0.7)
    rsf = float(np.float32(rng.uniform(0.25, 4.0)))
    wl = W.make_workload(T, H, 64, k, rsf=rsf, seed=int(rng.integers(1 << 30)),
                         pad=int(rng.choice([8, 64, 128])), with_shared=with_shared,
                         log2_mag=(-8.0, 8.0))
    idx = wl.idx.copy()
    idx[rng.random(idx.shape) < 0.03] = -1
    announce(f"staged quant random case {case}: T={T} H={H} k={k} per_cu={per_cu} "
             f"packed={packed} shared={with_shared}")
    q, s = run_quant(wl, packed=packed, with_shared=with_shared, idx=idx)
    check_mirror(wl, q, s, packed=packed, with_shared=with_shared, idx=idx)


def test_exactly_one_launch_capacity(ncu):
    """H = 128 (one chunk per token) at the largest grid one launch holds:
    every workgroup gets 509 units, 317 in LDS and 16 x 12 in register
    slots, so a wave that takes more than its share of the units past the
    LDS slots writes its extra units at once. The placement deals the tokens
    to groups of workgroups (one group per XCD) in blocks of 16."""
    H, k = 128, 2
    T = (LDS_UNITS + REG_UNITS_PER_CU) * ncu
    wl = W.make_workload(T, H, 16, k, rsf=2.5, seed=719, pad=64, log2_mag=(-8, 8))
    announce(f"staged quant at one launch's capacity T={T} H={H} k={k}")
    q, s = run_quant(wl)
    check_mirror(wl, q, s)

