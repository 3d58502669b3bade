"""Seeded synthetic inputs for the deferred MoE finalize.

This module only *draws* inputs; it holds none of the finalize arithmetic
(no gather, weighting, reduction, normalisation or quantisation). Both the
HIP path (tests, benchmark) and the CPU oracle take their inputs from here.
Casting the drawn float32 values to bfloat16 goes through torch's CPU cast.

The inputs stand in for the decode / prefill MoE layers the pages profile
(DeepSeek-V4-Flash decode at batch 1..256 in "Support deferred MoE finalize
for MXFP4 and FP8 block-scale", Speed; Kimi K2.5 decode in "[Kimi K2.5] Fuse
deferred MoE finalize into next-layer AR + residual + RMSNorm", "Numerics &
speed"). Real routing is skewed; uniform routing is the stand-in.

Recipe (every array is a deterministic function of the seed):
  * routing: per token, top_k distinct experts uniformly without
    replacement (the first top_k of a random permutation of E); top_k
    logits N(0,1), weight = sigmoid(logit) / sum over the token, stored fp32;
  * permuted layout: rows grouped by expert in ascending expert id, within
    an expert by ascending (token, slot); each expert's segment padded to a
    multiple of ``pad`` rows (an expert with no tokens has no rows); padding
    rows hold the bf16 quiet NaN 0x7FC0;
  * expanded_idx_to_permuted_idx[t, k]: the permuted row of slot (t, k);
  * real rows: bf16(N(0,1)), or bf16(m * N(0,1)) with a per-row magnitude
    m = 2^U(lo, hi) when ``log2_mag`` is given;
  * shared expert output, residual: bf16(N(0,1)) [T, H]; gamma:
    bf16(U(0.5, 1.5)) [H];
  * packed routing: (expert_id << 16) | bf16_bits(weight), the bf16 cast
    being torch's round-to-nearest-even.
Seeds default to 20261202 + 1000 * (the family's seed offset) + T.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

NAN_BF16 = np.uint16(0x7FC0)
_ROW_BLOCK = 512            # rows per independently seeded generator block


@dataclass
class Workload:
    """One batch of finalize inputs (host numpy arrays)."""
    name: str
    T: int
    H: int
    E: int
    top_k: int
    rsf: float
    seed: int
    gemm2_out: np.ndarray          # uint16 bf16 bits [P, H]
    idx: np.ndarray                # int32 [T, top_k]
    weights: np.ndarray            # float32 [T, top_k]
    expert_ids: np.ndarray         # int32 [T, top_k]
    packed: np.ndarray             # int32 [T, top_k]
    shared: Optional[np.ndarray]   # uint16 [T, H] or None
    residual: Optional[np.ndarray] = None   # uint16 [T, H]
    gamma: Optional[np.ndarray] = None      # uint16 [H]
    eps: float = 1e-6
    meta: dict = field(default_factory=dict)

    @property
    def P(self) -> int:
        return int(self.gemm2_out.shape[0])


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal_block(seed: int, stream: int, block: int, shape) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, block])))
    return g.standard_normal(shape, dtype=np.float32)


def _bf16_normal_matrix(seed: int, stream: int, rows: int, H: int,
                        scale: Optional[np.ndarray] = None) -> np.ndarray:
    """bf16(scale[r] * N(0,1)) [rows, H], drawn in seeded 512-row blocks."""
    out = np.empty((rows, H), dtype=np.uint16)

    def fill(b):
        r0 = b * _ROW_BLOCK
        r1 = min(rows, r0 + _ROW_BLOCK)
        x = _normal_block(seed, stream, b, (r1 - r0, H))
        if scale is not None:
            x *= scale[r0:r1, None]
        out[r0:r1] = to_bf16_bits(x)

    nblk = (rows + _ROW_BLOCK - 1) // _ROW_BLOCK
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(nblk)))
    return out


def draw_routing(rng: np.random.Generator, T: int, E: int, top_k: int):
    """(expert_ids int32 [T,k], weights float32 [T,k]) per the recipe."""
    if top_k > E:
        raise ValueError("top_k > E")
    if T == 0:
        return np.zeros((0, top_k), np.int32), np.zeros((0, top_k), np.float32)
    keys = rng.random((T, E))
    experts = np.argsort(keys, axis=1, kind="stable")[:, :top_k].astype(np.int32)
    logits = rng.standard_normal((T, top_k))
    s = 1.0 / (1.0 + np.exp(-logits))
    w = (s / s.sum(axis=1, keepdims=True)).astype(np.float32)
    return experts, w


def permuted_layout(expert_ids: np.ndarray, E: int, pad: int = 128):
    """Expert-sorted, padded row layout. Returns (idx int32 [T,k], P,
    real_rows int64 [T*k] listing the real permuted rows in layout order)."""
    T, K = expert_ids.shape
    flat = expert_ids.reshape(-1).astype(np.int64)
    order = np.lexsort((np.arange(T * K), flat))   # by expert, then (t, slot)
    counts = np.bincount(flat, minlength=E)
    padded = ((counts + pad - 1) // pad) * pad
    start = np.zeros(E, dtype=np.int64)
    start[1:] = np.cumsum(padded)[:-1]
    P = int(padded.sum())
    # rank of each slot inside its expert segment
    seg_first = np.zeros(E, dtype=np.int64)
    seg_first[1:] = np.cumsum(counts)[:-1]
    pos_sorted = np.arange(T * K) - seg_first[flat[order]]
    perm_row = np.empty(T * K, dtype=np.int64)
    perm_row[order] = start[flat[order]] + pos_sorted
    idx = perm_row.reshape(T, K).astype(np.int32)
    real_rows = start[flat[order]] + pos_sorted
    return idx, P, real_rows


def pack_routing(expert_ids: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """(expert_id << 16) | bf16_bits(weight) as int32 (bf16 by torch RNE)."""
    hi = expert_ids.astype(np.uint32) << 16
    lo = to_bf16_bits(weights).astype(np.uint32)
    return (hi | lo).view(np.int32)


def make_workload(T: int, H: int, E: int, top_k: int, *, rsf: float = 2.5,
                  seed: int = 0, pad: int = 128, with_shared: bool = True,
                  with_residual: bool = False,
                  log2_mag: Optional[tuple] = None, name: str = "custom",
                  eps: float = 1e-6) -> Workload:
    """Draw one workload per the module recipe."""
    rng = np.random.Generator(np.random.PCG64(seed))
    experts, w = draw_routing(rng, T, E, top_k)
    idx, P, real_rows = permuted_layout(experts, E, pad)
    n_real = real_rows.shape[0]
    scale = None
    if log2_mag is not None:
        lo, hi = log2_mag
        scale = np.exp2(rng.uniform(lo, hi, size=n_real)).astype(np.float32)
    real = _bf16_normal_matrix(seed, 1, n_real, H, scale)
    g2 = np.full((P, H), NAN_BF16, dtype=np.uint16)
    g2[real_rows] = real
    del real
    shared = _bf16_normal_matrix(seed, 2, T, H) if with_shared else None
    residual = gamma = None
    if with_residual:
        residual = _bf16_normal_matrix(seed, 3, T, H)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 4])))
        gamma = to_bf16_bits(g.uniform(0.5, 1.5, size=H).astype(np.float32))
    return Workload(name=name, T=T, H=H, E=E, top_k=top_k, rsf=rsf, seed=seed,
                    gemm2_out=g2, idx=idx, weights=w, expert_ids=experts,
                    packed=pack_routing(experts, w), shared=shared,
                    residual=residual, gamma=gamma, eps=eps)


def random_gather(T: int, P: int, H: int, top_k: int, *, rsf: float = 2.5, seed: int = 0,
                  log2_mag: Optional[tuple] = None, with_residual: bool = False,
                  name: str = "random_gather", eps: float = 1e-6) -> Workload:
    """Inputs for grids far larger than any routed batch, drawn cheaply: P
    real rows (no padding) and an index map of independent uniform draws
    from [0, P), so a row may be named by many slots. Weights follow the
    routing recipe (sigmoid of N(0,1) logits, normalised per token, fp32);
    the residual, when asked for, is bf16(N(0,1)) and gamma bf16(U(0.5,1.5)).
    There is no shared output."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 8])))
    idx = rng.integers(0, P, size=(T, top_k), dtype=np.int32)
    s = rng.standard_normal((T, top_k), dtype=np.float32)
    np.negative(s, out=s)
    np.exp(s, out=s)
    s += np.float32(1.0)
    np.reciprocal(s, out=s)                       # sigmoid
    s /= s.sum(axis=1, keepdims=True)
    scale = None
    if log2_mag is not None:
        scale = np.exp2(rng.uniform(log2_mag[0], log2_mag[1], size=P)).astype(np.float32)
    g2 = _bf16_normal_matrix(seed, 1, P, H, scale)
    residual = gamma = None
    if with_residual:
        residual = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
        gamma = to_bf16_bits(rng.uniform(0.5, 1.5, size=H).astype(np.float32))
    experts = np.zeros((T, top_k), np.int32)     # one expert: ids carry no layout here
    return Workload(name=name, T=T, H=H, E=1, top_k=top_k, rsf=rsf, seed=seed,
                    gemm2_out=g2, idx=idx, weights=s, expert_ids=experts,
                    packed=pack_routing(experts, s), shared=None,
                    residual=residual, gamma=gamma, eps=eps,
                    meta={"index_map": "uniform draws from [0, P)"})


def router_logits(T: int, E: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """float32 router logits [T, E], scale * N(0,1), for the gate."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 5])))
    return (g.standard_normal((T, E), dtype=np.float32) * np.float32(scale))


def activations(T: int, H: int, seed: int, log2_mag: Optional[tuple] = (-8.0, 8.0)) -> np.ndarray:
    """bf16 activations [T, H]: bf16(m_t * N(0,1)) with a per-token magnitude
    m_t = 2^U(lo, hi) (or 1 when log2_mag is None)."""
    scale = None
    if log2_mag is not None:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 6])))
        scale = np.exp2(g.uniform(log2_mag[0], log2_mag[1], size=T)).astype(np.float32)
    return _bf16_normal_matrix(seed, 7, T, H, scale)


# The synthetic workload families (sizes as in the published setup), each
# with the offset of its default seed.
FAMILIES = {
    "tiny": dict(Ts=(1,), H=1024, E=16, top_k=2, seed_offset=0),
    "decode_sweep": dict(Ts=(1, 4, 8, 16, 64, 256), H=4096, E=256, top_k=8, seed_offset=1),
    "packed_vs_unpacked": dict(Ts=(256,), H=7168, E=256, top_k=8, seed_offset=2),
    "residual_rmsnorm": dict(Ts=(16, 256, 1024), H=7168, E=256, top_k=8, seed_offset=3,
                             with_residual=True),
    "prefill_fp8_ue8m0": dict(Ts=(8192,), H=7168, E=256, top_k=8, seed_offset=4,
                              log2_mag=(-8.0, 8.0)),
}


def default_seed(seed_offset: int, T: int) -> int:
    return 20261202 + 1000 * seed_offset + T


def family_workload(family: str, T: Optional[int] = None,
                    seed: Optional[int] = None) -> Workload:
    """Workload of a named family at token count T (default: its first)."""
    c = FAMILIES[family]
    T = c["Ts"][0] if T is None else T
    seed = default_seed(c["seed_offset"], T) if seed is None else seed
    kw = dict(rsf=2.5, seed=seed, name=f"{family}_T{T}")
    if c.get("with_residual"):
        kw["with_residual"] = True
    if "log2_mag" in c:
        kw["log2_mag"] = c["log2_mag"]
    return make_workload(T, c["H"], c["E"], c["top_k"], **kw)
