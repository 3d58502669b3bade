"""CPU oracle for the routing front-end that feeds the deferred finalize.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests,
the smoke check and the benchmark's CPU leg, never by the library.

The pages name the step before the finalize: a gate ("moe_fused_gate")
that produces fp32 routing weights, optionally packed by "PackTopkIds" into
(expert_id << 16) | bf16(weight) ("[Deepseek V4] Keep fp32 routing weights
in the mxfp4 trtllm MoE", PR description). They give no formula. Readings
taken:
  G1  scores are sigmoid(logit); the top_k experts are the top_k scores,
      which, sigmoid being increasing, are the top_k logits: the integer
      decision never depends on how sigmoid is evaluated;
  G2  ties go to the lower expert id; NaN logits rank below every number
      (and below -inf); outputs are ordered by descending logit;
  G3  weight = sigmoid(l) / sum of the chosen sigmoids (fp64 here, one
      rounding to fp32); the routed scaling factor is not applied here (the
      finalize applies it);
  G4  packed word = (uint32(id) << 16) | bf16_rne_bits(weight).
"""
from __future__ import annotations

import numpy as np

from . import formats as F


def topk_order(logits, top_k):
    """Expert ids [T, top_k], descending logit, ties to the lower id, NaN last."""
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    # key: NaN -> +inf after negation is wrong (it would sort first), so sort
    # on (isnan, -l) lexicographically with a stable sort on the index order
    nan = np.isnan(l)
    neg = np.where(nan, 0.0, -l)
    order = np.lexsort((neg, nan.astype(np.int8)), axis=-1)   # last key primary
    return order[:, :top_k].astype(np.int32)


def sigmoid_f64(x):
    """1 / (1 + exp(-x)) in float64 (NaN stays NaN)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def topk_sigmoid_gate(logits, top_k):
    """(ids int32 [T,k], weights float32 [T,k], packed int32 [T,k])."""
    l = np.asarray(logits, dtype=np.float32)
    ids = topk_order(l, top_k)
    chosen = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    s = sigmoid_f64(chosen)
    w = (s / s.sum(axis=1, keepdims=True)).astype(np.float32)
    packed = ((ids.astype(np.uint32) << 16) | F.bf16_bits(w).astype(np.uint32)).view(np.int32)
    return ids, w, packed
