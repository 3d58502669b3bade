"""GPU parity of the routing gate against the CPU oracle.

Expert ids must match exactly (the choice is taken on the logits, which both
sides read bit-identically). Weights are fp32 sigmoid ratios; expf differs
between the two sides, so they are compared within a derived bound:
|w - w_oracle| <= 32 * 2^-24 * |w_oracle| (the GPU's sigmoid, sum and
division together stay below about 15 units of 2^-24 for top_k <= 16). The
packed words carry the exact id and a bf16 weight within one bf16 ulp of the
oracle's (and equal to the nearest-even bf16 of the GPU's own fp32 weight)."""
import numpy as np
import pytest
import torch

import combine_moe_finalize_amd as M
from combine_moe_finalize_amd import workloads as W
from oracle import formats as F
from oracle import routing as R

from gpu_helpers import DEV, announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    M.load_library()


def run_gate(l, k):
    ids, w, pk = M.moe_topk_sigmoid_gate(torch.from_numpy(l).to(DEV), k)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), pk.cpu().numpy()


def check_gate(l, k, ids, w, pk):
    oid, ow, opk = R.topk_sigmoid_gate(l, k)
    bad = np.argwhere(ids != oid)
    assert bad.size == 0, f"ids differ at {bad[:3].tolist()}: got {ids[tuple(bad[0])]} want {oid[tuple(bad[0])]}"
    fin = np.isfinite(ow)
    err = np.abs(w.astype(np.float64) - ow.astype(np.float64))
    assert np.all(err[fin] <= 32 * 2.0 ** -24 * np.abs(ow[fin].astype(np.float64)) + 1e-38)
    assert np.array_equal(np.isnan(w), np.isnan(ow))
    pu, ou = pk.view(np.uint32), opk.view(np.uint32)
    assert np.array_equal(pu >> 16, ou >> 16)
    gb = (pu & 0xFFFF).astype(np.uint16)
    assert np.array_equal(gb, W.to_bf16_bits(w)) or np.isnan(w).any()
    d = np.abs(F.bf16_to_f64(gb) - F.bf16_to_f64((ou & 0xFFFF).astype(np.uint16)))
    ulp = np.ldexp(1.0, np.frexp(np.abs(F.bf16_to_f64((ou & 0xFFFF).astype(np.uint16))))[1] - 8)
    assert np.all(d[fin] <= ulp[fin])


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (37, 16, 2), (300, 64, 6), (513, 100, 16),
                                   (256, 256, 8), (64, 512, 8), (8192, 256, 8), (5, 8, 8)])
def test_gate_random(T, E, k):
    l = W.router_logits(T, E, seed=900 + T + E + k, scale=3.0)
    announce(f"gate T={T} E={E} k={k}")
    check_gate(l, k, *run_gate(l, k))


@pytest.mark.parametrize("E", [64, 100, 256, 512])
def test_gate_ties_specials_and_equal_logits(E):
    """Exact ties inside and across a lane's register slots (E > 64 puts
    experts e and e + 64 in one lane), NaN, +-inf, -0, all-equal and all-NaN
    rows."""
    rng = np.random.default_rng(31 + E)
    l = rng.integers(-3, 4, size=(400, E)).astype(np.float32)    # many exact ties
    l[::9, 7] = np.nan
    l[::5, 11] = -np.inf
    l[::6, 12] = np.inf
    l[::4, 13] = -0.0
    l[1] = 0.5                                                     # all equal
    l[2] = np.nan                                                  # all NaN
    announce(f"gate ties and specials E={E}")
    ids, w, pk = run_gate(l, 8)
    oid, ow, _ = R.topk_sigmoid_gate(l, 8)
    assert np.array_equal(ids, oid)
    assert np.array_equal(ids[1], np.arange(8)) and np.array_equal(ids[2], np.arange(8))
    ok = np.isfinite(ow)
    assert np.all(np.abs(w[ok] - ow[ok]) <= 32 * 2.0 ** -24 * np.abs(ow[ok]) + 1e-38)


def test_gate_feeds_the_packed_decoder():
    l = W.router_logits(128, 256, seed=77)
    announce("gate -> packed decode")
    ids, w, pk = M.moe_topk_sigmoid_gate(torch.from_numpy(l).to(DEV), 8)
    dids, dw = M.moe_topk_packed_decode(pk)
    torch.cuda.synchronize()
    assert torch.equal(dids, ids)
    assert torch.equal(dw, w.to(torch.bfloat16).to(torch.float32))
