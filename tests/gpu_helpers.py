"""Shared helpers of the GPU parity tests: host <-> device marshalling and
the tolerance rules. Expected values always come from ``oracle``."""
import sys

import numpy as np
import torch

from oracle import finalize as O
from oracle import formats as F

DEV = "cuda:0"


def announce(msg: str) -> None:
    """Name the case before a GPU step (survives a crash of the process)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def d_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).to(DEV)


def d_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def d_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def h_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def h_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.uint8)


def device_inputs(wl, packed=False, with_shared=True):
    """Upload a workload; returns kwargs for the binding's routed arguments."""
    kw = dict(gemm2_out=d_bf16(wl.gemm2_out), expanded_idx_to_permuted_idx=d_i32(wl.idx),
              routed_scaling_factor=wl.rsf)
    if packed:
        kw["topk_packed"] = d_i32(wl.packed)
    else:
        kw["topk_weights"] = d_f32(wl.weights)
    if with_shared and wl.shared is not None:
        kw["shared_out"] = d_bf16(wl.shared)
    return kw


def ulp_bf16(r: np.ndarray) -> np.ndarray:
    """Spacing of bf16 at |r| (subnormal spacing at and near zero)."""
    r = np.abs(np.asarray(r, dtype=np.float64))
    e = np.full(r.shape, -126, dtype=np.int64)
    nz = r > 0
    e[nz] = np.maximum(np.frexp(r[nz])[1] - 1, -126)
    return np.ldexp(1.0, e - 7)


def abs_terms(g2, idx, weights=None, packed=None, shared=None, rsf=1.0, residual=None):
    """sum_k |w'_k x_k| + |shared| (+ |residual|): the magnitude that bounds
    fp32 rounding error under cancellation. Uses the oracle on |inputs|."""
    g2a = np.asarray(g2, np.uint16) & np.uint16(0x7FFF)
    w = None if weights is None else np.abs(weights)
    pk = None
    if packed is not None:
        pk = (np.asarray(packed).view(np.uint32) & np.uint32(0xFFFF7FFF)).view(np.int32)
    sh = None if shared is None else (np.asarray(shared, np.uint16) & np.uint16(0x7FFF))
    acc, _ = O.finalize_truth_f64(g2a, idx, w, pk, sh, abs(rsf))
    if residual is not None:
        acc = acc + F.bf16_to_f64(np.asarray(residual, np.uint16) & np.uint16(0x7FFF))
    return acc


def assert_bf16_within_tolerance(got_bits, truth_f64, terms, n_ops, what=""):
    """|g - bf16(truth)| <= 2 ulp(bf16(truth)) + gamma_n * terms, with
    gamma_n = n u / (1 - n u), u = 2^-24 (fp32 forward error bound)."""
    g = F.bf16_to_f64(got_bits)
    r = F.bf16_round(truth_f64)
    u = 2.0 ** -24
    gam = n_ops * u / (1 - n_ops * u)
    bound = 2 * ulp_bf16(r) + gam * terms
    err = np.abs(g - r)
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements beyond tolerance, first at {tuple(i)}: "
                             f"got {g[tuple(i)]} truth {truth_f64[tuple(i)]}")
    return float(np.max(err / ulp_bf16(r))) if err.size else 0.0


def assert_bits_equal(got, want, what="", zero_equal=True):
    """Bitwise equality (optionally treating +0 and -0 as equal)."""
    got = np.asarray(got)
    want = np.asarray(want)
    neq = got != want
    if zero_equal and got.dtype == np.uint16:
        neq &= ~(((got & 0x7FFF) == 0) & ((want & 0x7FFF) == 0))
    if neq.any():
        i = np.argwhere(neq)[0]
        raise AssertionError(f"{what}: {neq.sum()} of {neq.size} differ, first at {tuple(i)}: "
                             f"got {got[tuple(i)]:#x} want {want[tuple(i)]:#x}")
