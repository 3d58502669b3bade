"""ctypes binding of libmoe_finalize.so: argument marshalling only.

Each function checks tensor dtypes, shapes, devices and contiguity, passes
raw device pointers and the current HIP stream to the C entry point of the
same name, and raises MoeFinalizeError on a nonzero status. Every step of
the computation runs in the library's HIP kernels; torch supplies device
memory and streams. Outputs not supplied are allocated with torch (outside
graph capture only). There is no fallback: if the library is missing the
call fails.

Shape rules worth calling out (both are failure modes the pages report):
  * the index map and weights must be 2-D [T, top_k]; top_k is their last
    dimension, and a flat tensor is rejected ("[Kimi K2.5] Fuse deferred
    MoE finalize into next-layer AR + residual + RMSNorm", Key
    modifications: a flat index caused out-of-bounds reads);
  * fp32 weights must be float32 and packed words int32; one is never
    accepted in place of the other ("[Deepseek V4] Keep fp32 routing weights
    in the mxfp4 trtllm MoE", follow-up commit: fp32 buffers read as bf16
    broke decoding).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from ._paths import LIB_PATH

c_void_p = ctypes.c_void_p
c_i64 = ctypes.c_int64
c_i32 = ctypes.c_int32
c_f32 = ctypes.c_float

MOEF_OK = 0
QUANT_BLOCK = 128
OP_FINALIZE, OP_RESIDUAL_RMSNORM, OP_QUANT_UE8M0 = 0, 1, 2
DEVERR_INDEX_OUT_OF_RANGE = 1

_ROUTED = [c_void_p, c_i64, c_void_p, c_void_p, c_void_p, c_void_p, c_f32]
_SIGNATURES = {
    "moe_finalize": _ROUTED + [c_void_p, c_i64, c_i64, c_i32, c_void_p, c_void_p],
    "moe_finalize_residual_rmsnorm": _ROUTED + [c_void_p, c_void_p, c_f32, c_void_p, c_void_p,
                                                c_i64, c_i64, c_i32, c_void_p, c_void_p],
    "moe_finalize_quant_ue8m0": _ROUTED + [c_void_p, c_void_p, c_i64, c_i64, c_i32,
                                           c_void_p, c_void_p],
    "moe_topk_packed_decode": [c_void_p, c_i64, c_void_p, c_void_p, c_void_p],
    "moe_topk_sigmoid_gate": [c_void_p, c_i64, c_i32, c_i32, c_void_p, c_void_p, c_void_p,
                              c_void_p],
    "moe_act_quant_fp8_ue8m0": [c_void_p, c_i64, c_i64, c_void_p, c_void_p, c_void_p],
    "moe_finalize_ep_combine": [c_void_p, c_i32, c_void_p, c_void_p, c_i64, c_i64, c_void_p],
    "moe_act_quant_fp8_amax": [c_void_p, c_i64, c_i64, c_void_p, c_void_p, c_void_p],
    "moe_allreduce_residual_rmsnorm": [ctypes.POINTER(c_void_p), c_i32, c_void_p, c_void_p, c_f32,
                                       c_void_p, c_void_p, c_i64, c_i64, c_void_p],
    "moe_finalize_describe_launch": [c_i32, c_i64, c_i64, c_i32, c_void_p, ctypes.c_char_p,
                                     c_i64],
    "moe_finalize_status_string": [ctypes.c_int],
    "moe_finalize_abi_version": [],
}

_lib = None


class MoeFinalizeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status}: {status_string(status)}")


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load (once) the built library; raise if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python combine_moe_finalize_amd/build.py`")
    lib = ctypes.CDLL(p)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "moe_finalize_status_string" else ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().moe_finalize_status_string(int(status)).decode()


def abi_version() -> int:
    return load_library().moe_finalize_abi_version()


def moe_finalize_describe_launch(op: int, num_tokens: int, hidden: int, top_k: int,
                                 device=None) -> str:
    """The kernel (as profilers print it), launch count and grid that a call
    of this shape runs on `device` (default: the current one)."""
    if device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    buf = ctypes.create_string_buffer(256)
    st = load_library().moe_finalize_describe_launch(int(op), int(num_tokens), int(hidden),
                                                     int(top_k), _stream(torch.device(device)),
                                                     buf, len(buf))
    if st != MOEF_OK:
        raise MoeFinalizeError("moe_finalize_describe_launch", st)
    return buf.value.decode()


# ------------------------------------------------------------- marshalling

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _code_bytes(t):
    """E4M3 output as its bytes: a float8_e4m3fn tensor is written through a
    uint8 view of the same memory (the caller gets its own tensor back)."""
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    return t


def _tensor(t, name, dtype, shape):
    """dtype / shape / layout rule of one argument. The accepted case is one
    test; the messages are built only for a rejected argument."""
    if isinstance(t, torch.Tensor) and t.dtype == dtype and t.shape == shape and \
            t.is_contiguous():
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    raise ValueError(f"{name} must be contiguous")


def _on_device(device, **tensors):
    """Every given tensor lives on the one GPU device."""
    if device.type != "cuda":
        raise ValueError("tensors must be GPU tensors")
    index = device.index
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.get_device() != index):
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _dev_tensor(t, name, dtype, shape, device):
    _tensor(t, name, dtype, shape)
    _on_device(device, **{name: t})
    return t


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> int:
    """Handle of the device's current stream. torch's raw accessor returns it
    without building a Stream object (a few hundred ns against about 2 us)."""
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _routed(gemm2_out, idx, topk_weights, topk_packed, shared_out, err_flag):
    if not isinstance(gemm2_out, torch.Tensor) or gemm2_out.dim() != 2:
        raise ValueError("gemm2_out must be a 2-D [num_rows, hidden] tensor")
    if not isinstance(idx, torch.Tensor) or idx.dim() != 2:
        raise ValueError("expanded_idx_to_permuted_idx must be 2-D [tokens, top_k] "
                         "(a flat index tensor is rejected)")
    device = gemm2_out.device
    P, H = gemm2_out.shape
    T, K = idx.shape
    _tensor(gemm2_out, "gemm2_out", torch.bfloat16, (P, H))
    _tensor(idx, "expanded_idx_to_permuted_idx", torch.int32, (T, K))
    if (topk_weights is None) == (topk_packed is None):
        raise ValueError("give exactly one of topk_weights (float32) / topk_packed (int32)")
    if topk_weights is not None:
        _tensor(topk_weights, "topk_weights", torch.float32, (T, K))
    else:
        _tensor(topk_packed, "topk_packed", torch.int32, (T, K))
    if shared_out is not None:
        _tensor(shared_out, "shared_out", torch.bfloat16, (T, H))
    if err_flag is not None:
        _tensor(err_flag, "err_flag", torch.int32, (1,))
    _on_device(device, gemm2_out=gemm2_out, expanded_idx_to_permuted_idx=idx,
               topk_weights=topk_weights, topk_packed=topk_packed, shared_out=shared_out,
               err_flag=err_flag)
    args = [_ptr(gemm2_out), P, _ptr(idx), _ptr(topk_weights), _ptr(topk_packed),
            _ptr(shared_out)]
    return device, T, H, K, args


def _check(fn, status):
    if status != MOEF_OK:
        raise MoeFinalizeError(fn, status)


def _call(name, device, *args):
    """Call the C entry point with the tensors' device current (kernels launch
    on the current device; the stream passed is that device's current one).
    The device is switched only when it is not already the current one."""
    fn = getattr(_lib if _lib is not None else load_library(), name)
    if device.index == torch.cuda.current_device():
        st = fn(*args, _stream(device))
    else:
        with torch.cuda.device(device):
            st = fn(*args, _stream(device))
    _check(name, st)


# ------------------------------------------------------------- entry points

def moe_finalize(gemm2_out: torch.Tensor, expanded_idx_to_permuted_idx: torch.Tensor, *,
                 topk_weights: Optional[torch.Tensor] = None,
                 topk_packed: Optional[torch.Tensor] = None,
                 shared_out: Optional[torch.Tensor] = None,
                 routed_scaling_factor: float = 1.0,
                 out: Optional[torch.Tensor] = None,
                 err_flag: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [T, H] deferred finalize (see moe_finalize in moe_finalize.h)."""
    device, T, H, K, args = _routed(gemm2_out, expanded_idx_to_permuted_idx, topk_weights,
                                    topk_packed, shared_out, err_flag)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    _dev_tensor(out, "out", torch.bfloat16, (T, H), device)
    _call("moe_finalize", device, *args, float(routed_scaling_factor), _ptr(out), T, H, K,
          _ptr(err_flag))
    return out


def moe_finalize_residual_rmsnorm(gemm2_out: torch.Tensor,
                                  expanded_idx_to_permuted_idx: torch.Tensor, *,
                                  residual: torch.Tensor, gamma: torch.Tensor,
                                  eps: float = 1e-6,
                                  topk_weights: Optional[torch.Tensor] = None,
                                  topk_packed: Optional[torch.Tensor] = None,
                                  shared_out: Optional[torch.Tensor] = None,
                                  routed_scaling_factor: float = 1.0,
                                  residual_out: Optional[torch.Tensor] = None,
                                  normed: Optional[torch.Tensor] = None,
                                  err_flag: Optional[torch.Tensor] = None):
    """(residual_out, normed), both bf16 [T, H]. residual_out may be residual
    (in-place update)."""
    device, T, H, K, args = _routed(gemm2_out, expanded_idx_to_permuted_idx, topk_weights,
                                    topk_packed, shared_out, err_flag)
    _dev_tensor(residual, "residual", torch.bfloat16, (T, H), device)
    _dev_tensor(gamma, "gamma", torch.bfloat16, (H,), device)
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    if normed is None:
        normed = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    _dev_tensor(residual_out, "residual_out", torch.bfloat16, (T, H), device)
    _dev_tensor(normed, "normed", torch.bfloat16, (T, H), device)
    _call("moe_finalize_residual_rmsnorm", device, *args, float(routed_scaling_factor),
          _ptr(residual), _ptr(gamma), float(eps), _ptr(residual_out), _ptr(normed), T, H, K,
          _ptr(err_flag))
    return residual_out, normed


def moe_finalize_quant_ue8m0(gemm2_out: torch.Tensor,
                             expanded_idx_to_permuted_idx: torch.Tensor, *,
                             topk_weights: Optional[torch.Tensor] = None,
                             topk_packed: Optional[torch.Tensor] = None,
                             shared_out: Optional[torch.Tensor] = None,
                             routed_scaling_factor: float = 1.0,
                             out_e4m3: Optional[torch.Tensor] = None,
                             scale_e8m0: Optional[torch.Tensor] = None,
                             err_flag: Optional[torch.Tensor] = None):
    """(codes uint8 [T, H] as OCP E4M3 bits, scale bytes uint8 [T, H/128])."""
    device, T, H, K, args = _routed(gemm2_out, expanded_idx_to_permuted_idx, topk_weights,
                                    topk_packed, shared_out, err_flag)
    if H % QUANT_BLOCK:
        raise ValueError("hidden must be a multiple of 128 for the UE8M0 epilogue")
    if out_e4m3 is None:
        out_e4m3 = torch.empty((T, H), dtype=torch.uint8, device=device)
    if scale_e8m0 is None:
        scale_e8m0 = torch.empty((T, H // QUANT_BLOCK), dtype=torch.uint8, device=device)
    codes = _code_bytes(out_e4m3)
    _dev_tensor(codes, "out_e4m3", torch.uint8, (T, H), device)
    _dev_tensor(scale_e8m0, "scale_e8m0", torch.uint8, (T, H // QUANT_BLOCK), device)
    _call("moe_finalize_quant_ue8m0", device, *args, float(routed_scaling_factor),
          _ptr(codes), _ptr(scale_e8m0), T, H, K, _ptr(err_flag))
    return out_e4m3, scale_e8m0


def moe_topk_packed_decode(topk_packed: torch.Tensor, *,
                           expert_ids: Optional[torch.Tensor] = None,
                           weights: Optional[torch.Tensor] = None):
    """(expert_ids int32, weights float32), both shaped like topk_packed."""
    if not isinstance(topk_packed, torch.Tensor):
        raise TypeError("topk_packed must be a torch.Tensor")
    device = topk_packed.device
    shape = tuple(topk_packed.shape)
    _dev_tensor(topk_packed, "topk_packed", torch.int32, shape, device)
    if expert_ids is None:
        expert_ids = torch.empty(shape, dtype=torch.int32, device=device)
    if weights is None:
        weights = torch.empty(shape, dtype=torch.float32, device=device)
    _dev_tensor(expert_ids, "expert_ids", torch.int32, shape, device)
    _dev_tensor(weights, "weights", torch.float32, shape, device)
    _call("moe_topk_packed_decode", device, _ptr(topk_packed), topk_packed.numel(),
          _ptr(expert_ids), _ptr(weights))
    return expert_ids, weights


def moe_topk_sigmoid_gate(router_logits: torch.Tensor, top_k: int, *,
                          topk_ids: Optional[torch.Tensor] = None,
                          topk_weights: Optional[torch.Tensor] = None,
                          topk_packed: Optional[torch.Tensor] = None,
                          want_weights: bool = True, want_packed: bool = True):
    """(topk_ids int32, topk_weights float32 or None, topk_packed int32 or
    None), each [T, top_k], from float32 router logits [T, E]."""
    if not isinstance(router_logits, torch.Tensor) or router_logits.dim() != 2:
        raise ValueError("router_logits must be a 2-D [tokens, experts] tensor")
    T, E = router_logits.shape
    device = router_logits.device
    _tensor(router_logits, "router_logits", torch.float32, (T, E))
    shape = (T, int(top_k))
    if topk_ids is None:
        topk_ids = torch.empty(shape, dtype=torch.int32, device=device)
    if topk_weights is None and want_weights:
        topk_weights = torch.empty(shape, dtype=torch.float32, device=device)
    if topk_packed is None and want_packed:
        topk_packed = torch.empty(shape, dtype=torch.int32, device=device)
    _tensor(topk_ids, "topk_ids", torch.int32, shape)
    if topk_weights is not None:
        _tensor(topk_weights, "topk_weights", torch.float32, shape)
    if topk_packed is not None:
        _tensor(topk_packed, "topk_packed", torch.int32, shape)
    _on_device(device, router_logits=router_logits, topk_ids=topk_ids,
               topk_weights=topk_weights, topk_packed=topk_packed)
    _call("moe_topk_sigmoid_gate", device, _ptr(router_logits), T, E, int(top_k),
          _ptr(topk_ids), _ptr(topk_weights), _ptr(topk_packed))
    return topk_ids, topk_weights, topk_packed


def _act_quant(fn_name, x, out_e4m3, scale, scale_dtype):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D [tokens, hidden] tensor")
    T, H = x.shape
    if H % QUANT_BLOCK:
        raise ValueError("hidden must be a multiple of 128")
    device = x.device
    _tensor(x, "x", torch.bfloat16, (T, H))
    if out_e4m3 is None:
        out_e4m3 = torch.empty((T, H), dtype=torch.uint8, device=device)
    if scale is None:
        scale = torch.empty((T, H // QUANT_BLOCK), dtype=scale_dtype, device=device)
    codes = _code_bytes(out_e4m3)
    _tensor(codes, "out_e4m3", torch.uint8, (T, H))
    _tensor(scale, "scale", scale_dtype, (T, H // QUANT_BLOCK))
    _on_device(device, x=x, out_e4m3=codes, scale=scale)
    _call(fn_name, device, _ptr(x), T, H, _ptr(codes), _ptr(scale))
    return out_e4m3, scale


def moe_act_quant_fp8_ue8m0(x: torch.Tensor, *, out_e4m3: Optional[torch.Tensor] = None,
                            scale_e8m0: Optional[torch.Tensor] = None):
    """(codes uint8 [T, H], scale bytes uint8 [T, H/128]): power-of-two scales."""
    return _act_quant("moe_act_quant_fp8_ue8m0", x, out_e4m3, scale_e8m0, torch.uint8)


def moe_act_quant_fp8_amax(x: torch.Tensor, *, out_e4m3: Optional[torch.Tensor] = None,
                           scale_f32: Optional[torch.Tensor] = None):
    """(codes uint8 [T, H], scales float32 [T, H/128]): s = amax / 448."""
    return _act_quant("moe_act_quant_fp8_amax", x, out_e4m3, scale_f32, torch.float32)


def moe_finalize_ep_combine(partials: torch.Tensor, *,
                            shared_out: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [T, H] = sum of the R expert-parallel partials [R, T, H] (+ shared)."""
    if not isinstance(partials, torch.Tensor) or partials.dim() != 3:
        raise ValueError("partials must be a 3-D [ranks, tokens, hidden] tensor")
    R, T, H = partials.shape
    device = partials.device
    _tensor(partials, "partials", torch.bfloat16, (R, T, H))
    if shared_out is not None:
        _tensor(shared_out, "shared_out", torch.bfloat16, (T, H))
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    _tensor(out, "out", torch.bfloat16, (T, H))
    _on_device(device, partials=partials, shared_out=shared_out, out=out)
    _call("moe_finalize_ep_combine", device, _ptr(partials), R, _ptr(shared_out), _ptr(out),
          T, H)
    return out


def moe_allreduce_residual_rmsnorm(rank_outputs, *, residual: torch.Tensor, gamma: torch.Tensor,
                                   eps: float = 1e-6,
                                   residual_out: Optional[torch.Tensor] = None,
                                   normed: Optional[torch.Tensor] = None):
    """(residual_out, normed), both bf16 [T, H]: the R ranks' finalize outputs
    summed in fp32 in rank order, plus the residual, rounded once; then the
    RMSNorm of that residual_out. rank_outputs is a sequence of bf16 [T, H]
    tensors (separate buffers, as peers' buffers would be) or one [R, T, H]
    tensor. residual_out may be residual (in-place update)."""
    if isinstance(rank_outputs, torch.Tensor):
        if rank_outputs.dim() != 3:
            raise ValueError("rank_outputs must be [ranks, tokens, hidden] or a sequence of "
                             "[tokens, hidden] tensors")
        ranks = list(rank_outputs.unbind(0))
    else:
        ranks = list(rank_outputs)
    if not ranks or not isinstance(ranks[0], torch.Tensor) or ranks[0].dim() != 2:
        raise ValueError("rank_outputs must hold at least one [tokens, hidden] tensor")
    T, H = ranks[0].shape
    device = ranks[0].device
    named = {}
    for i, t in enumerate(ranks):
        named[f"rank_outputs[{i}]"] = _tensor(t, f"rank_outputs[{i}]", torch.bfloat16, (T, H))
    _tensor(residual, "residual", torch.bfloat16, (T, H))
    _tensor(gamma, "gamma", torch.bfloat16, (H,))
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    if normed is None:
        normed = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    _tensor(residual_out, "residual_out", torch.bfloat16, (T, H))
    _tensor(normed, "normed", torch.bfloat16, (T, H))
    _on_device(device, residual=residual, gamma=gamma, residual_out=residual_out, normed=normed,
               **named)
    ptrs = (c_void_p * len(ranks))(*[t.data_ptr() for t in ranks])
    _call("moe_allreduce_residual_rmsnorm", device, ptrs, len(ranks), _ptr(residual), _ptr(gamma),
          float(eps), _ptr(residual_out), _ptr(normed), T, H)
    return residual_out, normed
