"""The seeded input generators (CPU only)."""
import numpy as np

from combine_moe_finalize_amd import workloads as W


def test_deterministic_per_seed_and_seed_sensitive():
    a = W.make_workload(33, 256, 16, 4, seed=3, with_residual=True)
    b = W.make_workload(33, 256, 16, 4, seed=3, with_residual=True)
    c = W.make_workload(33, 256, 16, 4, seed=4, with_residual=True)
    for f in ("gemm2_out", "idx", "weights", "packed", "shared", "residual", "gamma"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert not np.array_equal(a.weights, c.weights)


def test_layout_is_a_padded_bijection():
    wl = W.make_workload(300, 64, 32, 8, seed=8, pad=128)
    T, K = wl.idx.shape
    flat = wl.idx.reshape(-1)
    assert len(np.unique(flat)) == T * K              # one row per slot
    assert flat.min() >= 0 and flat.max() < wl.P
    used = np.zeros(wl.P, bool)
    used[flat] = True
    nan_rows = np.all(wl.gemm2_out == W.NAN_BF16, axis=1)
    assert np.array_equal(~used, nan_rows)            # padding rows are NaN
    # segments: rows of one expert are contiguous, ascending expert id,
    # each segment a multiple of 128 rows
    eid_of_row = np.full(wl.P, -1)
    eid_of_row[flat] = wl.expert_ids.reshape(-1)
    counts = np.bincount(wl.expert_ids.reshape(-1), minlength=wl.E)
    padded = ((counts + 127) // 128) * 128
    assert wl.P == padded.sum()
    start = np.concatenate([[0], np.cumsum(padded)[:-1]])
    for e in range(wl.E):
        seg = eid_of_row[start[e]:start[e] + padded[e]]
        assert np.all(seg[:counts[e]] == e) and np.all(seg[counts[e]:] == -1)
    # within a segment the order is ascending (token, slot)
    for e in range(wl.E):
        rows = np.sort(flat[wl.expert_ids.reshape(-1) == e])
        tk = [divmod(int(np.where(flat == r)[0][0]), K) for r in rows]
        assert tk == sorted(tk)


def test_routing_distinct_and_normalised():
    wl = W.make_workload(500, 16, 256, 8, seed=9)
    for row in wl.expert_ids:
        assert len(set(row.tolist())) == 8
    s = wl.weights.astype(np.float64).sum(1)
    assert np.all(np.abs(s - 1) < 1e-6)
    assert np.all(wl.weights > 0)


def test_family_shapes_and_magnitudes():
    wl = W.family_workload("tiny")
    assert (wl.T, wl.H, wl.E, wl.top_k, wl.rsf) == (1, 1024, 16, 2, 2.5)
    assert wl.shared.shape == (1, 1024) and wl.idx.dtype == np.int32
    assert wl.P % 128 == 0
    w4 = W.make_workload(64, 1024, 256, 8, seed=1, log2_mag=(-8, 8))
    rows = w4.gemm2_out[w4.idx.reshape(-1)]
    v = (rows.astype(np.uint32) << 16).view(np.float32)
    rms = np.sqrt(np.mean(v.astype(np.float64) ** 2, axis=1))
    assert rms.min() < 2.0 ** -5 and rms.max() > 2.0 ** 5   # spans the range
    assert rms.min() > 2.0 ** -9 and rms.max() < 2.0 ** 9


def test_empty_token_batch():
    wl = W.make_workload(0, 128, 8, 2, seed=1)
    assert wl.idx.shape == (0, 2) and wl.P == 0 and wl.shared.shape == (0, 128)


def test_random_gather_inputs():
    a = W.random_gather(5000, 300, 64, 3, rsf=1.5, seed=11, with_residual=True)
    b = W.random_gather(5000, 300, 64, 3, rsf=1.5, seed=11, with_residual=True)
    assert np.array_equal(a.idx, b.idx) and np.array_equal(a.gemm2_out, b.gemm2_out)
    assert a.idx.shape == (5000, 3) and a.idx.dtype == np.int32
    assert a.idx.min() >= 0 and a.idx.max() < 300 and len(np.unique(a.idx)) == 300
    assert a.gemm2_out.shape == (300, 64) and a.P == 300
    assert np.all(np.abs(a.weights.astype(np.float64).sum(1) - 1) < 1e-6)
    assert np.all(a.weights > 0) and a.weights.dtype == np.float32
    assert a.shared is None and a.residual.shape == (5000, 64) and a.gamma.shape == (64,)
    g = (a.gamma.astype(np.uint32) << 16).view(np.float32)
    assert np.all((g >= 0.5) & (g <= 1.5))
    # packed words carry the bf16 of each weight (expert id 0)
    assert np.array_equal(a.packed.view(np.uint32) >> 16, np.zeros_like(a.idx, dtype=np.uint32))
