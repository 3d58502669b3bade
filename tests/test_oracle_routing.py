"""Pins for the routing front-end oracle (CPU only)."""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import finalize as O
from oracle import routing as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def logits_from(rows):
    return np.array([[float(v) for v in r] for r in rows], dtype=np.float32)


def test_golden_gate():
    g = json.load(open(os.path.join(GOLDEN, "routing_gate.json")))
    l = logits_from(g["logits"])
    ids, w, packed = R.topk_sigmoid_gate(l, g["top_k"])
    assert ids.tolist() == g["expert_ids"]
    want = np.array([[n / d for n, d in row] for row in g["weights_num_den"]])
    assert np.allclose(w, want, rtol=1e-6, atol=0)
    assert [f"{x:08X}" for x in packed[1].view(np.uint32)] == g["packed_hex_token1"]


def test_selection_invariants():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((500, 64)).astype(np.float32)
    l[::7, 5] = l[::7, 9]                      # planted ties
    l[::11, 3] = np.nan
    l[::13, 4] = -np.inf
    k = 8
    ids = R.topk_order(l, k)
    for t in range(l.shape[0]):
        chosen = set(ids[t].tolist())
        row = l[t]
        key = lambda e: (np.isnan(row[e]), -row[e] if not np.isnan(row[e]) else 0.0, e)
        ref = sorted(range(64), key=key)[:k]      # a Python sort with tuple keys
        assert ids[t].tolist() == ref
        for e in range(64):
            if e in chosen or np.isnan(row[e]):
                continue
            assert all(not np.isnan(row[c]) and (row[c] > row[e] or (row[c] == row[e] and c < e))
                       for c in chosen), (t, e)


def test_sigmoid_matches_library():
    x = np.linspace(-40, 40, 10001)
    assert np.allclose(R.sigmoid_f64(x), scipy.special.expit(x), rtol=1e-14, atol=0)


def test_weights_normalised_and_equal_logits():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((300, 256)).astype(np.float32) * 3
    ids, w, _ = R.topk_sigmoid_gate(l, 8)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) < 1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)         # descending logits -> descending weights
    ids, w, _ = R.topk_sigmoid_gate(np.zeros((3, 16), np.float32), 4)
    assert np.all(ids == np.arange(4)) and np.all(w == np.float32(0.25))


def test_packed_words_decode_to_ids_and_bf16_weights():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((200, 256)).astype(np.float32)
    ids, w, packed = R.topk_sigmoid_gate(l, 8)
    dids, dw = O.decode_packed(packed)
    assert np.array_equal(dids, ids)
    assert np.array_equal(dw, torch.from_numpy(w).to(torch.bfloat16).float().numpy())
