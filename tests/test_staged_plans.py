"""CPU checks of the staged kernels' launch sizing and index arithmetic.

The launch plan is the library's own host code (plan_staged in
moef_internal.h, exported by the host-stub build). The kernels' unit and
slot arithmetic is modelled here from finalize_kernels.hip and checked for
every workgroup: each unit is computed and written exactly once, every LDS
slot index stays below the capacity the launch was sized for, and every
global offset stays inside its tensor. No GPU is used.
"""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STUB = os.path.join(ROOT, "tests", "c", "libmoef_host_stub.so")

WAVE = 64
CHUNK_COLS = 512


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(STUB):
        pytest.skip("host stub library not built (python combine_moe_finalize_amd/build.py)")
    L = ctypes.CDLL(STUB)
    L.moef_test_plan_staged.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                        ctypes.POINTER(ctypes.c_int64)]
    L.moef_test_stage_caps.argtypes = [ctypes.POINTER(ctypes.c_int64)]
    L.moef_test_plan_staged_tokens.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                               ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
    return L


def plan(L, items, ncu, per_wg_max):
    out = (ctypes.c_int64 * 2)()
    L.moef_test_plan_staged(items, ncu, per_wg_max, out)
    return out[0], out[1]


def plan_tokens(L, tokens, nchunks, ncu, per_wg_max):
    out = (ctypes.c_int64 * 3)()
    L.moef_test_plan_staged_tokens(tokens, nchunks, ncu, per_wg_max, out)
    return out[0], out[1], out[2]


def caps(L):
    out = (ctypes.c_int64 * 15)()
    L.moef_test_stage_caps(out)
    keys = ["quant_lds", "quant_reg", "plain_lds", "plain_reg", "rms_lds", "waves",
            "quant_from", "plain_from", "rms_from", "max_top_k", "tail_pct", "plain_waves",
            "tail_from", "plain_wide_waves", "plain_wide_reg"]
    return dict(zip(keys, list(out)))


def ranges(items, per_launch):
    return [(u0, min(items, u0 + per_launch)) for u0 in range(0, items, per_launch)]


def per_wg_counts(u0, u1, nb):
    """Items of workgroup b in a launch over [u0, u1): u0 + b + j * nb."""
    b = np.arange(nb)
    return np.where(u1 - u0 > b, (u1 - u0 - b + nb - 1) // nb, 0)


def test_capacities_fit_the_lds(lib):
    c = caps(lib)
    lds = 160 * 1024
    assert c["quant_lds"] * (CHUNK_COLS + 4) + 4 <= lds
    assert c["plain_lds"] * (CHUNK_COLS * 2) + 4 <= lds
    # the plain kernel's wide layout holds a 8192-token, H = 7168 call in one
    # launch on 256 CUs, and holds more than the 16-wave layout
    wide = c["plain_lds"] + c["plain_wide_waves"] * c["plain_wide_reg"]
    assert wide >= 8192 * 14 // 256
    assert wide > c["plain_lds"] + c["plain_waves"] * c["plain_reg"]
    assert c["plain_wide_waves"] * WAVE <= 1024
    assert c["rms_lds"] * (CHUNK_COLS * 2 + 8) + 4 <= lds
    assert c["waves"] * WAVE == 1024
    # the largest RMSNorm hidden size still fits one token per workgroup
    assert c["rms_lds"] // (16384 // CHUNK_COLS) >= 1


@pytest.mark.parametrize("ncu", [1, 32, 80, 256, 304])
def test_plan_covers_every_item_within_capacity(lib, ncu):
    rng = np.random.default_rng(ncu)
    sizes = [0, 1, 2, ncu - 1, ncu, ncu + 1] + list(rng.integers(1, 3_000_000, 40))
    for per_wg_max in (1, 4, 11, 158, 287, 509):
        cap = ncu * per_wg_max
        for items in sizes + [cap - 1, cap, cap + 1, 2 * cap, 2 * cap + 1, 7 * cap - 3]:
            items = int(items)
            if items < 0:
                continue
            launches, per_launch = plan(lib, items, ncu, per_wg_max)
            if items == 0:
                assert launches == 0
                continue
            # as few launches as hold every item
            assert launches == -(-items // cap)
            # launch r covers [r * per_launch, min(items, (r + 1) * per_launch)):
            # contiguous, all items, and only two range lengths occur
            assert (launches - 1) * per_launch < items <= launches * per_launch
            for length in {per_launch, items - (launches - 1) * per_launch}:
                assert per_wg_counts(0, length, ncu).max() <= per_wg_max


def staged_unit_model(u0, u1, nb, nchunks, h8, lds_units, per_wg_max):
    """The unit, slot and offset arithmetic of the staged plain finalize for one launch over [u0, u1): workgroup b computes units
    u0 + b + j * nb for j < its count n; unit j takes LDS slot j while
    j < lds_units, otherwise a register slot or (none free) a store at once.
    Returns how often each unit of the range is computed, and the largest
    global vector offset any unit writes."""
    counts = per_wg_counts(u0, u1, nb)
    assert counts.max() <= per_wg_max
    b = np.repeat(np.arange(nb), counts)
    j = np.concatenate([np.arange(n) for n in counts]) if counts.sum() else np.zeros(0, int)
    unit = u0 + b + j * nb
    assert ((unit >= u0) & (unit < u1)).all()
    slot = j[j < lds_units]
    assert (slot < lds_units).all()
    t = unit // nchunks
    first_col = (unit - t * nchunks) * WAVE
    assert (first_col < h8).all()                 # every unit has an active lane
    last = t * h8 + np.minimum(first_col + WAVE, h8) - 1
    return np.bincount(unit - u0, minlength=u1 - u0), (last.max() if last.size else -1)


BLOCK = 16          # tokens per block dealt to one workgroup group


def group_token(t0, g, x, full, lt):
    """Token of group x's local token index lt (finalize_quant_staged_kernel)."""
    in_full = full * BLOCK
    return np.where(lt < in_full, t0 + ((lt // BLOCK) * g + x) * BLOCK + lt % BLOCK,
                    t0 + in_full * g + x + (lt - in_full) * g)


@pytest.mark.parametrize("T,H,ncu", [(1463, 7168, 256), (8192, 7168, 256), (9305, 7168, 256),
                                     (30000, 7168, 256), (8192, 7168, 80), (1000, 7176, 64),
                                     (5000, 128, 32), (130304, 128, 256), (700, 131072, 256),
                                     (33, 1 << 20, 256)])
def test_staged_quant_token_groups(lib, T, H, ncu):
    """Every unit computed once, by a staged workgroup (within the launch's
    staging capacity) or by a tail workgroup (one unit per wave); groups
    within one token of each other; and each 16-token block of a full round
    (its scale bytes: whole lines when H is a multiple of 1024) computed by
    one group, i.e. through one XCD's L2."""
    c = caps(lib)
    per_wg_max = c["quant_lds"] + c["waves"] * c["quant_reg"]
    h8 = H // 8
    nch = -(-h8 // WAVE)
    launches, per_launch, g = plan_tokens(lib, T, nch, ncu, per_wg_max)
    assert g == (8 if ncu % 8 == 0 else 1)
    assert launches >= 1 and (launches - 1) * per_launch < T <= launches * per_launch
    wpx = ncu // g
    seen = np.zeros((T, nch), np.int64)
    owner = np.full(T, -1, np.int64)
    for t0 in range(0, T, per_launch):
        t1 = min(T, t0 + per_launch)
        full = (t1 - t0) // (g * BLOCK)
        rest = (t1 - t0) - full * g * BLOCK
        # the launcher's grid: the staged workgroups plus the tail workgroups
        pct = c["tail_pct"] if (t1 - t0) * nch >= c["tail_from"] * ncu else 0
        max_units = -(-(t1 - t0) // g) * nch
        tail_wgs = g * (-(-(max_units * pct // 100) // c["waves"]))
        for b in range(ncu + tail_wgs):
            x = (b - ncu if b >= ncu else b) % g
            group_tokens = full * BLOCK + ((rest - x + g - 1) // g if rest > x else 0)
            assert group_tokens <= -(-(t1 - t0) // g)
            units = group_tokens * nch
            static = units - units * pct // 100
            if b >= ncu:
                lu = static + ((b - ncu) // g) * c["waves"] + np.arange(c["waves"])
                lu = lu[lu < units]
            else:
                w = b // g
                n = (static - w + wpx - 1) // wpx if static > w else 0
                assert n <= per_wg_max
                lu = w + np.arange(n) * wpx
            if lu.size == 0:
                continue
            lt = lu // nch
            t = group_token(t0, g, x, full, lt)
            assert ((t >= t0) & (t < t1)).all()
            np.add.at(seen, (t, lu - lt * nch), 1)
            assert ((owner[t] == -1) | (owner[t] == x)).all()
            owner[t] = x
    assert (seen == 1).all()
    # blocks of a launch's full rounds belong to one group each
    for t0 in range(0, T, per_launch):
        t1 = min(T, t0 + per_launch)
        full = (t1 - t0) // (g * BLOCK)
        for m in range(full * g):
            blk = owner[t0 + m * BLOCK:t0 + (m + 1) * BLOCK]
            assert (blk == blk[0]).all()


@pytest.mark.parametrize("kind", ["plain"])
@pytest.mark.parametrize("T,H,ncu", [(1463, 7168, 256), (8192, 7168, 256), (8192, 7168, 80),
                                     (1000, 7176, 64), (5000, 128, 32)])
def test_staged_unit_arithmetic(lib, kind, T, H, ncu):
    """The plain staged kernel: the 16-wave layout while one launch of it
    holds the grid, else the wide (12-wave) layout, in as few launches as
    hold every unit."""
    c = caps(lib)
    lds_units = c["plain_lds"]
    h8 = H // 8
    nchunks = -(-h8 // WAVE)
    units = T * nchunks
    if units <= ncu * (lds_units + c["plain_waves"] * c["plain_reg"]):
        per_wg_max = lds_units + c["plain_waves"] * c["plain_reg"]
    else:
        per_wg_max = lds_units + c["plain_wide_waves"] * c["plain_wide_reg"]
    launches, per_launch = plan(lib, units, ncu, per_wg_max)
    seen = np.zeros(units, np.int64)
    for u0, u1 in ranges(units, per_launch):
        cnt, last = staged_unit_model(u0, u1, ncu, nchunks, h8, lds_units, per_wg_max)
        seen[u0:u1] += cnt
        assert last < T * h8
    assert (seen == 1).all()
    assert launches >= 1
    if units <= ncu * (lds_units + c["plain_wide_waves"] * c["plain_wide_reg"]):
        assert launches == 1


@pytest.mark.parametrize("T,H,ncu", [(1, 7168, 256), (256, 7168, 256), (1024, 7168, 256),
                                     (2816, 7168, 256), (2817, 7168, 256), (4096, 7168, 256),
                                     (1500, 7176, 80), (300, 16384, 64), (777, 512, 32),
                                     (5000, 136, 304)])
def test_rmsnorm_staged_index_arithmetic(lib, T, H, ncu):
    """The RMSNorm staged kernel's token plan and both index phases (the
    gather loop over units j, the write loop over elements x), for every
    workgroup of every launch."""
    c = caps(lib)
    cap = c["rms_lds"]
    h8 = H // 8
    nch = -(-h8 // WAVE)
    tpw = cap // nch
    launches, per_launch = plan(lib, T, ncu, tpw)
    written = np.zeros(T * h8, np.int64)
    res_reader = np.full(T, -1, np.int64)
    for li, (t0, t1) in enumerate(ranges(T, per_launch)):
        for b, ntok in enumerate(per_wg_counts(t0, t1, ncu)):
            assert ntok <= cap // nch                   # the kernel's guard never clamps
            n = ntok * nch
            assert n <= cap
            if n == 0:
                continue
            wg = li * ncu + b
            # gather phase: unit j -> token i = j / nch, chunk j % nch; slots j < n <= cap
            j = np.arange(n)
            i = j // nch
            t = t0 + b + i * ncu
            assert ((t >= t0) & (t < t1)).all()
            assert (res_reader[t] == -1).all() or (res_reader[t] == wg).all()
            res_reader[t] = wg
            # write phase: element x -> unit x / 64, lane x % 64; inverse-rms slot i < ntok
            x = np.arange(n * WAVE)
            jx = x // WAVE
            ix = jx // nch
            assert ix.max() < ntok
            colv = (jx - ix * nch) * WAVE + (x - jx * WAVE)
            keep = colv < h8
            tx = t0 + b + ix[keep] * ncu
            assert ((tx >= t0) & (tx < t1)).all()
            # a token's residual_out comes from the workgroup that read its residual
            assert (res_reader[tx] == wg).all()
            np.add.at(written, tx * h8 + colv[keep], 1)
    assert (written == 1).all()
    assert (res_reader >= 0).all()


def describe(L, op, T, H, k, ncu):
    L.moef_test_set_cus.argtypes = [ctypes.c_int]
    L.moef_test_set_cus(ncu)
    L.moe_finalize_describe_launch.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int32, ctypes.c_void_p, ctypes.c_char_p,
                                               ctypes.c_int64]
    buf = ctypes.create_string_buffer(256)
    st = L.moe_finalize_describe_launch(op, T, H, k, None, buf, 256)
    return st, buf.value.decode()


DESCRIBE_CASES = [
    # the prefill quant call: one staged launch, 8 XCD groups, 360 tail workgroups
    (2, 8192, 7168, 8, 256,
     "finalize_quant_staged_kernel<8, true, 12> launches=1 grid=616x1024 groups=8 tail=5%"),
    (2, 2048, 7168, 8, 256,
     "finalize_quant_staged_kernel<8, true, 0> launches=1 grid=256x1024 groups=8 tail=0%"),
    # tail workgroups from 160 units per CU: T = 3072 is 168 per CU, T = 2560 is 140
    (2, 3072, 7168, 8, 256,
     "finalize_quant_staged_kernel<8, true, 0> launches=1 grid=392x1024 groups=8 tail=5%"),
    (2, 2560, 7168, 8, 256,
     "finalize_quant_staged_kernel<8, true, 0> launches=1 grid=256x1024 groups=8 tail=0%"),
    (2, 1024, 7168, 8, 256, "finalize_quant_kernel<8, true> launches=1 grid=3584x256"),
    (2, 8192, 7168, 16, 256, "finalize_quant_kernel<16, false> launches=1 grid=28672x256"),
    (0, 1, 4096, 8, 256, "finalize_kernel<8, true> launches=1 grid=2x256"),
    (0, 8192, 7168, 8, 256, "finalize_staged_kernel<8, true, 25, 12> launches=1 grid=256x768"),
    (0, 4096, 7168, 8, 256, "finalize_staged_kernel<8, true, 8, 16> launches=1 grid=256x1024"),
    (0, 1024, 7168, 3, 256, "finalize_staged_kernel<4, false, 0, 16> launches=1 grid=256x1024"),
    (1, 16, 7168, 8, 256, "finalize_rmsnorm_kernel<8, true, 1> launches=1 grid=16x896"),
    (1, 1024, 7168, 8, 256, "finalize_rmsnorm_staged_kernel<8, true> launches=1 grid=256x1024"),
    (1, 4096, 7168, 8, 256, "finalize_rmsnorm_staged_kernel<8, true> launches=2 grid=256x1024"),
    (1, 700, 7168, 8, 256, "finalize_rmsnorm_kernel<8, true, 2> launches=1 grid=700x448"),
    (1, 287, 7168, 8, 256, "finalize_rmsnorm_kernel<8, true, 1> launches=1 grid=287x896"),
    (1, 288, 4104, 8, 256, "finalize_rmsnorm_kernel<8, true, 1> launches=1 grid=288x576"),
    (0, 0, 7168, 8, 256, "none (num_tokens == 0)"),
]


@pytest.mark.parametrize("op,T,H,k,ncu,want", DESCRIBE_CASES)
def test_describe_launch(lib, op, T, H, k, ncu, want):
    """The library's own description of a call's launch, planned for 256
    CUs, for the shapes the benchmark times."""
    st, text = describe(lib, op, T, H, k, ncu)
    assert st == 0 and text == want


def test_describe_launch_rules(lib):
    L = lib
    assert describe(L, 3, 16, 7168, 8, 256)[0] == 2                 # unknown op: BAD_SHAPE
    assert describe(L, 2, 16, 7000, 8, 256)[0] == 3                 # quant needs H % 128 == 0
    assert describe(L, 1, 16, 16392, 8, 256)[0] == 3                # RMSNorm hidden limit
    assert describe(L, 0, -1, 7168, 8, 256)[0] == 2
    L.moe_finalize_describe_launch.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int32, ctypes.c_void_p, ctypes.c_char_p,
                                               ctypes.c_int64]
    assert L.moe_finalize_describe_launch(0, 16, 7168, 8, None, None, 256) == 1
    buf = ctypes.create_string_buffer(8)
    assert L.moe_finalize_describe_launch(2, 8192, 7168, 8, None, buf, 8) == 0
    assert buf.value.decode() == "finaliz"                         # cut to buf_len - 1
    # a CU count that 8 does not divide: one group
    st, text = describe(L, 2, 8192, 7168, 8, 76)
    assert st == 0 and "groups=1" in text and text.startswith("finalize_quant_staged_kernel")
