#!/usr/bin/env python3
"""Benchmark of the MI355X deferred MoE finalize (one GPU).

One step = one call of the timed entry point over one batch of synthetic
input already resident in HBM. The default workload is the prefill-size
finalize with the FP8 / UE8M0 epilogue (T=8192 tokens, hidden 7168, 256
experts, top_k 8, routed scaling factor 2.5, per-row magnitudes 2^U(-8,8)):
the largest batch, where the path must run at HBM speed. Its call carries
every step of the path: routing-weight load and scaling, index load, row
gather, fp32 weighted reduce, shared-expert add, bf16 rounding and the 1x128
UE8M0 / E4M3 quantization.

Printed: one JSON line with
  value      algorithmic GB/s of the whole step (bytes the method must move /
             wall time per step, inputs resident),
  kernel_source_sha256  the finalize kernel sources the run used
             (all_sources_sha256: every kernel source and header and the
             build script),
  ceilings   same-session streaming read and copy rates (the bandwidth probe
             kernels) and torch's device copy, with the headline kernel's rate
             as a fraction of the read and copy rates (the kernel moves 95%
             reads, a copy half),
  roofline   the kernel's algorithmic bytes per launch / its average duration
             (HIP events recorded on the launch stream around the K timed
             launches, divided by K), against the 8 TB/s HBM peak; `kernel`
             is the launch as the library plans it on this device
             (moe_finalize_describe_launch); `traffic` is the
             counter-measured HBM bytes per launch from the committed
             rocprofv3 counter summary when it matches the current kernel
             source, else null,
  steady_state  the same kernel's time per launch and rate over the last 100
             of 300 back-to-back launches right after the timed ones (after
             an idle gap the first ~100 launches run 2-5% slower while the
             device's clocks ramp up; the timed region follows the short
             warm-up directly),
  cpu_baseline  the CPU oracle's fp32 mirror timed on a bounded sample of the
             same workload, on one thread and on a pool of
             min(usable CPUs, 16) threads,
  parity     the timed launches' outputs against the mirror (every token) and
             the fp64 truth (a sample),
  sweep      per workload shape and NEXT-row entry point (decode T=1..256,
             packed vs fp32 routing, residual + RMSNorm, the routing gate,
             standalone FP8 activation quant in both scale policies, the
             expert-parallel combine, the all-reduce + RMSNorm share, the
             packed decoder; for the gate the "H" field holds the expert
             count E; the first row is an empty kernel): the per-call time
             of 20 calls captured in a HIP graph and replayed, and
             host-inclusive event times (warm, cold after a 1 GiB read-only
             stream through the caches, and 100 back-to-back calls). A marker
             launch opens each case, so a kernel trace of the run splits
             into cases; kernel-only durations come from rocprofv3,
  us_per_call  the timed operation on its first T = 1, 2, 4, ..., 8192
             tokens, the plain bf16 finalize of the same tokens at
             T = 256..8192, the decode finalize at T = 1..256, and an empty kernel
             (one wave, no memory access), all per call under HIP-graph
             replay: the empty kernel is the floor under any call's time.

CPU-only modes (--summarize-trace, --summarize-counters,
--summarize-sweep-counters) turn rocprofv3 output of a run of this script
into the summaries kept under profiles/.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = [os.path.join(ROOT, "combine_moe_finalize_amd", "csrc", f)
                  for f in ("finalize_kernels.hip", "device_common.h", "moef_internal.h")]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "prefill_quant_T8192_H7168_counters.json")


# ------------------------------------------------------------ byte models
def bytes_plain(T, H, k, shared=True):
    return T * (2 * H * (k + (2 if shared else 1)) + 8 * k)


def bytes_rmsnorm(T, H, k, shared=True):
    return T * (2 * H * (k + (4 if shared else 3)) + 8 * k) + 2 * H


def bytes_quant(T, H, k, shared=True):
    return T * (2 * H * (k + (1 if shared else 0)) + H + H // 128 + 8 * k)


def kernel_source_hash() -> str:
    """SHA-256 over the sources the timed kernel is built from."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def all_sources_hash() -> str:
    """SHA-256 over every kernel source file of the library and its build
    script (sorted by name): what the sweep's kernels are built from."""
    csrc = os.path.join(ROOT, "combine_moe_finalize_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(ROOT, "combine_moe_finalize_amd", "build.py"), "rb") as f:
        h.update(b"build.py\0" + f.read())
    return h.hexdigest()


def counters_traffic():
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


# ------------------------------------------------------------- utilities
def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def upload(wl, torch, packed=False):
    dev = "cuda:0"

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    kw = dict(gemm2_out=bf16(wl.gemm2_out),
              expanded_idx_to_permuted_idx=torch.from_numpy(wl.idx).to(dev),
              routed_scaling_factor=wl.rsf)
    if packed:
        kw["topk_packed"] = torch.from_numpy(wl.packed).to(dev)
    else:
        kw["topk_weights"] = torch.from_numpy(wl.weights).to(dev)
    if wl.shared is not None:
        kw["shared_out"] = bf16(wl.shared)
    extra = {}
    if wl.residual is not None:
        extra = dict(residual=bf16(wl.residual), gamma=bf16(wl.gamma), eps=wl.eps)
    return kw, extra


# Steady state of the headline launch: after any idle gap of 20 ms or more
# the first ~100 back-to-back launches run 2-5% slower while the device's
# clocks ramp back up, so a short timed region right after the warm-up
# reads above the rate a busy device sustains.
STEADY_LAUNCHES, STEADY_TIMED = 300, 100


def steady_state_us(torch, step):
    """HIP-event time per launch of the last STEADY_TIMED of STEADY_LAUNCHES
    back-to-back launches."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    for _ in range(STEADY_LAUNCHES - STEADY_TIMED):
        step()
    a.record()
    for _ in range(STEADY_TIMED):
        step()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / STEADY_TIMED


def event_times_us(torch, fn, iters, flush=None):
    """Per-call GPU time (HIP events on the current stream) of fn()."""
    s = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    for i in range(iters):
        if flush is not None:
            flush()
        starts[i].record(s)
        fn()
        ends[i].record(s)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) * 1e3 for a, b in zip(starts, ends)])


def batched_us(torch, fn, n):
    """Per-call time of n back-to-back calls between two events (launches
    overlap, so this is the sustained rate of repeated calls)."""
    s = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    a.record(s)
    for _ in range(n):
        fn()
    b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def graph_us(torch, fn, n, reps=10):
    """Per-call time of n calls captured in one HIP graph, replayed."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(reps):
        g.replay()
    b.record(s)
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) * 1e3 / (n * reps)


# --------------------------------------------------------------- CPU leg
def e4m3_steps(a, b):
    """Distance in E4M3 code steps between code arrays (sign-magnitude codes
    mapped onto one ordered line; +0 and -0 coincide)."""
    def line(c):
        c = c.astype(np.int64)
        m = c & 0x7F
        return np.where(c & 0x80, -m, m)
    return np.abs(line(a) - line(b))


def host_threads():
    """Threads for the CPU leg: the host CPUs this process may run on, at most
    16 (one GPU's share of its host: the 8-GPU hosts these numbers come from
    give each GPU's jobs 16 CPUs, and the affinity mask can show more)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def oracle_chunk(O, wl, sl, mode="mirror"):
    fn = O.finalize_quant_mirror if mode == "mirror" else O.finalize_quant_truth
    return fn(wl.gemm2_out, wl.idx[sl], weights_f32=wl.weights[sl], shared=wl.shared[sl],
              rsf=wl.rsf)


def cpu_baseline(wl, q_gpu=None, s_gpu=None, min_s=10.0, max_s=30.0, chunk=256,
                 truth_tokens=512, threads=None, min_s_threads=5.0):
    """The oracle's fp32 mirror of the kernels' operation order (finalize +
    UE8M0 quant, numpy), as it stands, in token chunks over the same
    workload: the CPU counterpart of the timed launch.

    One thread first, repeating passes until at least min_s seconds of CPU
    work (stopping early at max_s); then, with threads > 1 (default: the host
    CPUs available, at most 16), the same chunks on a thread pool for at
    least min_s_threads seconds. The reported value is the thread-pool rate
    (cores = its thread count), the one-thread rate beside it.

    With the GPU's codes and scale bytes given, they are then compared with
    the first one-thread pass's outputs (bit for bit, every token it
    covered), and, untimed, with the oracle's fp64 truth on the first
    truth_tokens tokens (scale bytes equal, codes within one E4M3 step)."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import finalize as O
    keep = q_gpu is not None
    m_codes = np.empty((wl.T, wl.H), np.uint8) if keep else None
    m_scales = np.empty((wl.T, wl.H // 128), np.uint8) if keep else None
    done = 0
    t0 = time.perf_counter()
    while True:
        start = done % wl.T
        sl = slice(start, min(wl.T, start + chunk))
        qc, sc, _ = oracle_chunk(O, wl, sl)
        if keep and done < wl.T:
            m_codes[sl], m_scales[sl] = qc, sc
        done += sl.stop - sl.start
        el = time.perf_counter() - t0
        if (el >= min_s and done % wl.T == 0) or el >= max_s:
            break
    dt = time.perf_counter() - t0
    gbs1 = bytes_quant(done, wl.H, wl.top_k) / dt / 1e9
    one = {"value": round(gbs1, 4), "cores": 1,
           "sample": f"{done} tokens ({done / wl.T:.2f} passes over the T={wl.T} workload), "
                     f"{dt:.1f} s"}
    n_thr = host_threads() if threads is None else threads
    what = "the oracle's fp32 mirror of the finalize + UE8M0/E4M3 quant, numpy"
    base = {"value": round(gbs1, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{one['sample']} through {what}, one thread"}
    if n_thr > 1:
        slices = [slice(a, min(wl.T, a + chunk)) for a in range(0, wl.T, chunk)]
        mt_done, passes = 0, 0
        t1 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=n_thr) as pool:
            while True:
                for _ in pool.map(lambda sl: oracle_chunk(O, wl, sl), slices):
                    pass
                mt_done += wl.T
                passes += 1
                if time.perf_counter() - t1 >= min_s_threads:
                    break
        dt_mt = time.perf_counter() - t1
        base = {"value": round(bytes_quant(mt_done, wl.H, wl.top_k) / dt_mt / 1e9, 4),
                "unit": "GB/s", "cores": n_thr, "kind": "oracle",
                "sample": f"{mt_done} tokens ({passes} passes over the T={wl.T} workload) "
                          f"through {what}, {n_thr} threads over {chunk}-token chunks, "
                          f"{dt_mt:.1f} s",
                "single_thread": one}
    if not keep:
        return base, None
    n = min(done, wl.T)
    m = min(truth_tokens, wl.T)
    tq, ts, _ = O.finalize_quant_truth(wl.gemm2_out, wl.idx[:m], weights_f32=wl.weights[:m],
                                       shared=wl.shared[:m], rsf=wl.rsf)
    steps = e4m3_steps(q_gpu[:m], tq)
    parity = {"tokens_vs_fp32_mirror": int(n),
              "code_mismatches_vs_mirror": int(np.count_nonzero(q_gpu[:n] != m_codes[:n])),
              "scale_mismatches_vs_mirror": int(np.count_nonzero(s_gpu[:n] != m_scales[:n])),
              "tokens_vs_fp64_truth": int(m),
              "scale_bytes_differing_vs_truth": int(np.count_nonzero(s_gpu[:m] != ts)),
              "max_code_steps_vs_truth": int(steps.max()) if steps.size else 0,
              "codes_differing_vs_truth": int(np.count_nonzero(steps))}
    return base, parity


# ----------------------------------------------------------------- sweep
def probe_lib():
    """The bandwidth probe library (csrc/bandwidth_probes.h); fails loudly
    when it is not built."""
    import ctypes
    from combine_moe_finalize_amd._paths import PROBE_LIB_PATH
    P = ctypes.CDLL(PROBE_LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    P.moef_probe_read.argtypes = [vp, i64, vp, vp]
    P.moef_probe_copy.argtypes = [vp, vp, i64, vp]
    P.moef_probe_empty.argtypes = [vp]
    P.moef_probe_mark.argtypes = [vp]
    return P


def sweep(torch, M, W, iters_small=700, iters_big=100):
    """Every workload shape and NEXT-row entry point. Before each case the
    probe library's marker kernel (the empty kernel on two workgroups) is
    launched, so a kernel trace of this run splits into one block per case,
    in the order of the returned rows. A case's dispatches: 10 warm-up calls,
    `iters` back-to-back event-timed calls (warm; 700 for the decode-size
    cases, 100 for the prefill-size ones), iters / 10 calls each
    after a 1 GiB read-only stream through the caches (cold), 100
    back-to-back calls, and 20 calls captured in a HIP graph and replayed.
    The read-only flush leaves no dirty lines behind, so a cold call is not
    charged for writing back someone else's data."""
    P = probe_lib()
    flush_src = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda:0")
    flush_sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")

    def stream():
        return torch.cuda.current_stream().cuda_stream

    def flush():
        if P.moef_probe_read(flush_src.data_ptr(), 1 << 30, flush_sink.data_ptr(), stream()) != 0:
            raise RuntimeError("read probe: launch failed")

    rows = []

    def measure(name, T, H, k, nbytes, fn, iters, kernel=None, write_bytes=None):
        torch.cuda.synchronize()
        if P.moef_probe_mark(stream()) != 0:
            raise RuntimeError("marker launch failed")
        torch.cuda.synchronize()
        for _ in range(10):
            fn()
        warm = event_times_us(torch, fn, iters)
        cold = event_times_us(torch, fn, max(10, iters // 10), flush=flush)
        batched = batched_us(torch, fn, 100)
        graph = graph_us(torch, fn, 20)
        rows.append({"case": name, "T": T, "H": H, "top_k": k, "kernel": kernel,
                     "us_graph_replay": round(graph, 3),
                     "gbs_graph_replay": round(nbytes / (graph * 1e-6) / 1e9, 1),
                     "algorithmic_bytes": int(nbytes),
                     "algorithmic_write_bytes": None if write_bytes is None else int(write_bytes),
                     # per-call times seen from the host: each includes the launch and
                     # event overhead (several us at decode sizes); kernel-only times,
                     # warm and cold, come from the kernel trace of this run
                     "host_inclusive": {
                         "us_event_median": round(float(np.median(warm)), 3),
                         "us_event_p10": round(float(np.percentile(warm, 10)), 3),
                         "us_event_p90": round(float(np.percentile(warm, 90)), 3),
                         "us_event_cold_median": round(float(np.median(cold)), 3),
                         "us_batched": round(batched, 3)}})
        log(f"sweep {rows[-1]}")

    def describe(op, T, H, k):
        return M.moe_finalize_describe_launch(op, T, H, k)

    measure("empty kernel (launch floor)", 0, 0, 0, 0, lambda: P.moef_probe_empty(stream()),
            iters_small, kernel="empty_probe_kernel", write_bytes=0)
    wl = W.family_workload("tiny")
    kw, _ = upload(wl, torch)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda:0")
    measure("tiny", wl.T, wl.H, wl.top_k, bytes_plain(wl.T, wl.H, wl.top_k),
            lambda: M.moe_finalize(**kw, out=out), iters_small,
            kernel=describe(M.OP_FINALIZE, wl.T, wl.H, wl.top_k), write_bytes=wl.T * wl.H * 2)
    for T in W.FAMILIES["decode_sweep"]["Ts"]:
        wl = W.family_workload("decode_sweep", T)
        kw, _ = upload(wl, torch)
        out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda:0")
        measure("decode", T, wl.H, wl.top_k, bytes_plain(T, wl.H, wl.top_k),
                lambda: M.moe_finalize(**kw, out=out), iters_small,
                kernel=describe(M.OP_FINALIZE, T, wl.H, wl.top_k), write_bytes=T * wl.H * 2)
    for T in (1, 16):                      # the Kimi K2.5 decode shape (H 7168, 384 experts)
        wl = W.make_workload(T, 7168, 384, 8, rsf=2.5, seed=W.default_seed(9, T))
        kw, _ = upload(wl, torch)
        out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda:0")
        measure("decode_H7168_E384", T, wl.H, wl.top_k, bytes_plain(T, wl.H, wl.top_k),
                lambda: M.moe_finalize(**kw, out=out), iters_small,
                kernel=describe(M.OP_FINALIZE, T, wl.H, wl.top_k), write_bytes=T * wl.H * 2)
    wl = W.family_workload("packed_vs_unpacked")
    for packed in (False, True):
        kw, _ = upload(wl, torch, packed=packed)
        out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda:0")
        measure("packed" if packed else "fp32_weights", wl.T, wl.H, wl.top_k,
                bytes_plain(wl.T, wl.H, wl.top_k), lambda: M.moe_finalize(**kw, out=out),
                iters_small, kernel=describe(M.OP_FINALIZE, wl.T, wl.H, wl.top_k),
                write_bytes=wl.T * wl.H * 2)
    for T in W.FAMILIES["residual_rmsnorm"]["Ts"]:
        wl = W.family_workload("residual_rmsnorm", T)
        kw, ex = upload(wl, torch)
        ro = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda:0")
        nm = torch.empty_like(ro)
        measure("residual_rmsnorm", T, wl.H, wl.top_k, bytes_rmsnorm(T, wl.H, wl.top_k),
                lambda: M.moe_finalize_residual_rmsnorm(**kw, **ex, residual_out=ro, normed=nm),
                iters_big if T >= 1024 else iters_small,
                kernel=describe(M.OP_RESIDUAL_RMSNORM, T, wl.H, wl.top_k),
                write_bytes=2 * T * wl.H * 2)
    for T in (1, 256, 8192):
        E, k = 256, 8
        lg = torch.from_numpy(W.router_logits(T, E, seed=T)).to("cuda:0")
        gi = torch.empty((T, k), dtype=torch.int32, device="cuda:0")
        gw = torch.empty((T, k), dtype=torch.float32, device="cuda:0")
        gp = torch.empty((T, k), dtype=torch.int32, device="cuda:0")
        measure("topk_sigmoid_gate", T, E, k, T * (4 * E + 12 * k),
                lambda: M.moe_topk_sigmoid_gate(lg, k, topk_ids=gi, topk_weights=gw,
                                                topk_packed=gp), iters_small,
                write_bytes=T * 12 * k)
    for T in (16, 8192):
        H = 7168
        xa = torch.from_numpy(W.activations(T, H, seed=T).view(np.int16)).view(
            torch.bfloat16).to("cuda:0")
        aq = torch.empty((T, H), dtype=torch.uint8, device="cuda:0")
        a8 = torch.empty((T, H // 128), dtype=torch.uint8, device="cuda:0")
        af = torch.empty((T, H // 128), dtype=torch.float32, device="cuda:0")
        measure("act_quant_ue8m0", T, H, 0, T * (3 * H + H // 128),
                lambda: M.moe_act_quant_fp8_ue8m0(xa, out_e4m3=aq, scale_e8m0=a8), iters_small,
                write_bytes=T * (H + H // 128))
        measure("act_quant_amax", T, H, 0, T * (3 * H + 4 * (H // 128)),
                lambda: M.moe_act_quant_fp8_amax(xa, out_e4m3=aq, scale_f32=af), iters_small,
                write_bytes=T * (H + 4 * (H // 128)))
    T, H, R = 8192, 7168, 4
    parts = torch.from_numpy(W.activations(R * T, H, seed=R, log2_mag=None).view(np.int16)).view(
        torch.bfloat16).to("cuda:0").view(R, T, H)
    shp = torch.from_numpy(W.activations(T, H, seed=5, log2_mag=None).view(np.int16)).view(
        torch.bfloat16).to("cuda:0")
    ep_out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda:0")
    measure("ep_combine_R4", T, H, 0, T * H * 2 * (R + 2),
            lambda: M.moe_finalize_ep_combine(parts, shared_out=shp, out=ep_out), iters_big,
            write_bytes=T * H * 2)
    del parts, shp, ep_out
    R, H = 8, 7168
    for T in (1, 16, 256, 2048):
        ranks = [torch.from_numpy(W.activations(T, H, seed=30 + r, log2_mag=None).view(np.int16))
                 .view(torch.bfloat16).to("cuda:0") for r in range(R)]
        ares = torch.from_numpy(W.activations(T, H, seed=40, log2_mag=None).view(np.int16)).view(
            torch.bfloat16).to("cuda:0")
        agam = torch.ones(H, dtype=torch.bfloat16, device="cuda:0")
        aro = torch.empty_like(ares)
        anm = torch.empty_like(ares)
        measure("allreduce_residual_rmsnorm_R8", T, H, 0, T * 2 * H * (R + 3) + 2 * H,
                lambda: M.moe_allreduce_residual_rmsnorm(ranks, residual=ares, gamma=agam,
                                                         residual_out=aro, normed=anm),
                iters_big if T >= 2048 else iters_small, write_bytes=2 * T * H * 2)
        del ranks, ares, aro, anm
    n = 8192 * 8
    pk = torch.from_numpy(W.family_workload("tiny").packed.reshape(-1).repeat(n // 2)).to("cuda:0")
    ids = torch.empty_like(pk)
    wts = torch.empty(pk.shape, dtype=torch.float32, device="cuda:0")
    measure("packed_decode", 8192, 0, 8, 12 * n,
            lambda: M.moe_topk_packed_decode(pk, expert_ids=ids, weights=wts), iters_small,
            write_bytes=8 * n)
    del flush_src, flush_sink
    torch.cuda.empty_cache()
    return rows


def launch_floor_us(torch):
    """Per-call time of the probe library's empty kernel (one wave, no memory
    access) under the same HIP-graph replay as the small calls: the floor
    under any kernel's time per call."""
    P = probe_lib()

    def launch():
        if P.moef_probe_empty(torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("empty probe: launch failed")

    return graph_us(torch, launch, 20, reps=5)


def ceilings(torch, nbytes=1 << 30):
    """Same-session HBM rates in GB/s: the streaming read and copy probes
    (csrc/bandwidth_probes.h) over `nbytes`, 10 back-to-back launches between
    two events, median of 5; and torch's own device-to-device copy, median
    of 20 event-timed copies. A copy moves 2 x nbytes."""
    P = probe_lib()
    src = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream

    def per_launch_s(fn, n=10, reps=5):
        for _ in range(2):
            assert fn() == 0
        times = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                fn()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3 / n)
        return float(np.median(times))

    read = nbytes / per_launch_s(lambda: P.moef_probe_read(src.data_ptr(), nbytes,
                                                           sink.data_ptr(), stream)) / 1e9
    copy = 2 * nbytes / per_launch_s(lambda: P.moef_probe_copy(src.data_ptr(), dst.data_ptr(),
                                                               nbytes, stream)) / 1e9
    torch.cuda.synchronize()
    if int(sink.item()) != 0 or not torch.equal(dst[:1 << 20], src[:1 << 20]):
        raise RuntimeError("bandwidth probes: unexpected output")
    times = []
    for _ in range(20):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    torch_copy = 2 * nbytes / float(np.median(times)) / 1e9
    del src, dst, sink
    torch.cuda.empty_cache()
    return read, copy, torch_copy


# ------------------------------------------------------- profile summaries
# CPU-only: these read what rocprofv3 wrote during a run of this script and
# write the summaries kept under profiles/.

def _short_kernel(name):
    """A trace's kernel name without namespaces and arguments:
    "finalize_quant_staged_kernel<8, true, 12>"."""
    import re
    core = name.replace("(anonymous namespace)::", "").split("(", 1)[0]
    core = core.replace("void ", "", 1).strip() if core.startswith("void ") else core.strip()
    depth, cut = 0, 0
    for i, ch in enumerate(core):       # the last "::" outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == ":" and depth == 0 and i > 0 and core[i - 1] == ":":
            cut = i + 1
    out = core[cut:]
    return re.sub(r"\s+", " ", out)


def _read_trace(path):
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({"name": _short_kernel(r["Kernel_Name"]), "grid": int(r["Grid_Size_X"]),
                         "wg": int(r["Workgroup_Size_X"]), "id": int(r["Dispatch_Id"]),
                         "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
    rows.sort(key=lambda r: r["id"])
    return rows


def _last_json_line(path):
    with open(path) as f:
        lines = [l for l in f.read().splitlines() if l.startswith("{")]
    return json.loads(lines[-1])


def _stats(us):
    us = np.asarray(us, dtype=float)
    if us.size == 0:
        return None
    return {"n": int(us.size), "median": float(np.median(us)), "p10": float(np.percentile(us, 10)),
            "p90": float(np.percentile(us, 90))}


def _case_blocks(rows):
    """A run's dispatches split at the sweep's marker launches (the empty
    kernel on two 64-lane workgroups): one list per sweep case, in order."""
    blocks, cur = [], None
    for r in rows:
        if r["name"] == "empty_probe_kernel" and r["grid"] == 128:
            cur = []
            blocks.append(cur)
        elif cur is not None:
            cur.append(r)
    return blocks


def _launches_per_call(kernel):
    """Launches per call from the library's launch description
    ("name<...> launches=2 grid=..."); one for kernels it does not plan."""
    if kernel and " launches=" in kernel:
        return max(1, int(kernel.split(" launches=")[1].split()[0]))
    return 1


def summarize_trace(trace_csv, bench_json, out_dir, command):
    """The kernel trace of one `bench.py` run: the timed launches of the
    headline call, and per sweep case the kernel's durations split into warm
    dispatches and cold ones (those right after the 1 GiB read-only flush)."""
    rows = _read_trace(trace_csv)
    line = _last_json_line(bench_json)
    srcs = line.get("kernel_source_sha256") or kernel_source_hash()
    # headline: the first warmup + steps dispatches of the timed kernel
    kname = line["roofline"]["kernel"].split(" launches=")[0]
    grid = line["roofline"]["kernel"].split(" grid=")[1].split()[0]
    nwg, wg = (int(x) for x in grid.split("x"))
    nhead = line["warmup"] + line["steps"]
    allhead = [r for r in rows if r["name"] == kname and r["grid"] == nwg * wg]
    head = allhead[:nhead]
    timed = [r["us"] for r in head[line["warmup"]:]]
    steady = []
    if "steady_state" in line:   # the launches that follow the timed ones
        run = allhead[nhead:nhead + STEADY_LAUNCHES]
        steady = [r["us"] for r in run[STEADY_LAUNCHES - STEADY_TIMED:]]
    nbytes = line["roofline"]["algorithmic_bytes_per_launch"]
    hl = [f"# {kname}: prefill FP8/UE8M0 finalize, T={line['config']['tokens']}, "
          f"H={line['config']['hidden']}, top_k={line['config']['top_k']}", "",
          "Command (from `/tmp` with `TMPDIR=/tmp` on the MI355X box; `$R` is the repository root):",
          "", f"    {command}", "",
          "Summary written by `python bench.py --summarize-trace` from that run's kernel trace "
          "and JSON line.", "",
          f"Kernel source SHA-256 (`finalize_kernels.hip` + `device_common.h` + "
          f"`moef_internal.h`): `{srcs}`", "",
          f"Launch, as `moe_finalize_describe_launch` reports it: `{line['roofline']['kernel']}`.",
          "", "| dispatches | avg µs | median µs | min µs | max µs |", "|---|---|---|---|---|"]
    avg = float(np.mean(timed)) if timed else float("nan")
    hl.append(f"| {len(timed)} timed (after {line['warmup']} warm-up) | {avg:.3f} | "
              f"{np.median(timed):.3f} | {min(timed):.3f} | {max(timed):.3f} |")
    if len(steady) == STEADY_TIMED:
        hl.append(f"| {len(steady)} steady state (the last of {STEADY_LAUNCHES} launches "
                  f"right after the timed ones) | {np.mean(steady):.3f} | "
                  f"{np.median(steady):.3f} | {min(steady):.3f} | {max(steady):.3f} |")
    hl += ["", f"Algorithmic bytes per launch: {nbytes:,} → **{nbytes / avg / 1e3:,.0f} GB/s** at "
           f"the timed average ({nbytes / avg / 1e3 / HBM_PEAK_GBS * 100:.1f}% of 8 TB/s).", "",
           f"The same run's bench line (HIP events on the launch stream around the {line['steps']} "
           f"timed launches): **{line['roofline']['kernel_us_avg']:.3f} µs** per launch "
           f"({(line['roofline']['kernel_us_avg'] / avg - 1) * 100:+.1f}% against the trace).", ""]
    if len(steady) == STEADY_TIMED and "steady_state" in line:
        sa = float(np.mean(steady))
        hl += [f"Steady state: {nbytes / sa / 1e3:,.0f} GB/s at the trace average "
               f"({nbytes / sa / 1e3 / HBM_PEAK_GBS * 100:.1f}% of 8 TB/s); the bench line's "
               f"events: {line['steady_state']['kernel_us_avg']:.3f} µs per launch. After an "
               f"idle gap the first ~100 launches run 2-5% slower while the device's clocks "
               f"ramp up, and the timed launches follow the warm-up directly.", ""]
    with open(os.path.join(out_dir, "prefill_quant_T8192_H7168_kernel_trace.md"), "w") as f:
        f.write("\n".join(hl))
    blocks = _case_blocks(rows)
    sw = line.get("sweep", [])
    out = ["# Kernel durations of every bench sweep case (rocprofv3 kernel trace)", "",
           "Same run and command as `prefill_quant_T8192_H7168_kernel_trace.md`:", "",
           f"    {command}", "",
           "Written by `python bench.py --summarize-trace`. Each sweep case starts with a marker "
           "launch; its dispatches are 10 warm-up calls, back-to-back calls, calls each after a "
           "1 GiB read-only stream through the caches (**cold**: the dispatch right after the "
           "flush kernel), 100 back-to-back calls and 20-call HIP-graph replays. **Warm** is "
           "every dispatch of the case's kernel that does not follow a flush; **graph** is the "
           "last 10 replays of the 20-call graph (200 calls back to back, the way a captured "
           "model runs them), per call (launches per call × the median dispatch). The first "
           "row, the empty kernel (one wave, no memory access), is the floor under every other "
           "row, in the same states.", "",
           f"Kernel source SHA-256 (`finalize_kernels.hip` + `device_common.h` + "
           f"`moef_internal.h`): `{srcs}`; every kernel source and the build script: "
           f"`{line.get('all_sources_sha256', 'not recorded')}`", "",
           "| case | kernel | grid | warm n | warm median µs | p10 | p90 | cold n | cold median µs "
           "| graph µs/call | algorithmic bytes | GB/s warm | GB/s cold | GB/s graph |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    summary = []
    for case, blk in zip(sw, blocks):
        by = {}
        for r in blk:
            if r["name"] in ("read_probe_kernel",):
                continue
            by.setdefault((r["name"], r["grid"]), []).append(r)
        if not by:
            continue
        key = max(by, key=lambda kk: sum(x["us"] for x in by[kk]))
        ids = {r["id"] for r in by[key]}
        warm, cold = [], []
        prev = None
        for r in blk:
            if r["id"] in ids:
                (cold if prev is not None and prev["name"] == "read_probe_kernel" else warm).append(r["us"])
            prev = r
        w, c = _stats(warm), _stats(cold)
        lpc = _launches_per_call(case.get("kernel"))
        tail = [r["us"] for r in blk if r["id"] in ids][-200 * lpc:]
        g = float(np.median(tail)) * lpc if len(tail) == 200 * lpc else None
        nb = case["algorithmic_bytes"]
        label = f"{case['case']} T={case['T']} H={case['H']} k={case['top_k']}"
        gw = f"{nb / w['median'] / 1e3:,.1f}" if nb and w else "—"
        gc = f"{nb / c['median'] / 1e3:,.1f}" if nb and c else "—"
        gg = f"{nb / g / 1e3:,.1f}" if nb and g else "—"
        out.append(f"| {label} | `{key[0]}` | {key[1]} | {w['n']} | {w['median']:.3f} | "
                   f"{w['p10']:.3f} | {w['p90']:.3f} | {c['n'] if c else 0} | "
                   f"{c['median'] if c else float('nan'):.3f} | "
                   f"{g if g else float('nan'):.3f} | {nb:,} | {gw} | {gc} | {gg} |")
        summary.append({"case": label, "kernel": key[0], "grid": key[1], "warm": w, "cold": c,
                        "graph_us_per_call": g, "algorithmic_bytes": nb})
    with open(os.path.join(out_dir, "finalize_sweep_kernel_trace.md"), "w") as f:
        f.write("\n".join(out) + "\n")
    return summary


def summarize_counters(fetch_csv, write_csv, out_dir, commands, bench_json=None):
    """The two counter passes of `bench.py --copy-calibration --no-sweep`:
    FETCH_SIZE and WRITE_SIZE of the three 1 GiB device copies (the factor
    that turns each counter into bytes) and of the headline launches. The
    kernel source hash is the one a pass's JSON line records, when given."""
    import csv
    srcs = kernel_source_hash()
    if bench_json is not None:
        srcs = _last_json_line(bench_json).get("kernel_source_sha256") or srcs

    def read(path, counter):
        d = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                k = int(r["Dispatch_Id"])
                e = d.setdefault(k, {"name": _short_kernel(r["Kernel_Name"]), "v": 0.0})
                if r["Counter_Name"] == counter:
                    e["v"] += float(r["Counter_Value"])
        return [d[k] for k in sorted(d)]

    fe, wr = read(fetch_csv, "FETCH_SIZE"), read(write_csv, "WRITE_SIZE")
    cf = [r["v"] for r in fe if r["name"] == "__amd_rocclr_copyBuffer"][:3]
    cw = [r["v"] for r in wr if r["name"] == "__amd_rocclr_copyBuffer"][:3]
    qf = [r["v"] for r in fe if r["name"].startswith("finalize_quant")]
    qw = [r["v"] for r in wr if r["name"].startswith("finalize_quant")]
    qname = next(r["name"] for r in fe if r["name"].startswith("finalize_quant"))
    ff, fw = (1 << 30) / (np.median(cf) * 1024), (1 << 30) / (np.median(cw) * 1024)
    fk, wk = float(np.median(qf[1:])), float(np.median(qw[1:]))     # the first is the warm-up
    fb, wb = fk * 1024 * ff, wk * 1024 * fw
    nbytes = bytes_quant(8192, 7168, 8)
    reads = 8192 * (2 * 7168 * 9 + 64)
    j = {"kernel": qname,
         "workload": "prefill finalize + UE8M0/E4M3, T=8192, H=7168, E=256, top_k=8, fp32 "
                     "weights, shared expert",
         "kernel_source_sha256": srcs,
         "fetch_size_kib_per_launch": fk, "write_size_kib_per_launch": wk,
         "copy_calibration": {"bytes_read": 1 << 30, "bytes_written": 1 << 30,
                              "fetch_size_kib": float(np.median(cf)),
                              "write_size_kib": float(np.median(cw)),
                              "fetch_factor": round(float(ff), 6), "write_factor": round(float(fw), 6)},
         "fetch_bytes_per_launch": int(round(fb)), "write_bytes_per_launch": int(round(wb)),
         "hbm_bytes_per_launch": int(round(fb + wb)), "algorithmic_bytes_per_launch": nbytes,
         "traffic_over_algorithmic": round((fb + wb) / nbytes, 5)}
    with open(os.path.join(out_dir, "prefill_quant_T8192_H7168_counters.json"), "w") as f:
        json.dump(j, f, indent=1)
    md = [f"# HBM traffic counters: {qname}, prefill T=8192, H=7168, top_k=8", "",
          "Two counter passes, each in its own run (from `/tmp` with `TMPDIR=/tmp` on the MI355X "
          "box; `$R` is the repository root there):", ""]
    md += [f"    {c}" for c in commands]
    md += ["", "`--copy-calibration` adds three 1 GiB device-to-device copies "
           "(`__amd_rocclr_copyBuffer`) that read and write exactly 1 073 741 824 bytes each. "
           "Written by `python bench.py --summarize-counters`.", "",
           f"Kernel source SHA-256: `{j['kernel_source_sha256']}`", "",
           "| dispatch | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---|---|",
           "| copy 1 GiB (×3) | " + " / ".join(f"{v:,.1f}" for v in cf) + " | "
           + " / ".join(f"{v:,.1f}" for v in cw) + " |",
           f"| {qname} (×{len(qf)}: 1 warm-up + {len(qf) - 1}) | "
           + " / ".join(f"{v:,.1f}" for v in qf) + " | " + " / ".join(f"{v:,.1f}" for v in qw) + " |",
           "", f"Calibration (known bytes / counter reading): fetch {ff:.6f}, write {fw:.6f}.", "",
           f"Per launch (median of the timed launches): fetch {fk:,.1f} KiB × {ff:.6f} = "
           f"{int(round(fb)):,} B; write {wk:,.1f} KiB × {fw:.6f} = {int(round(wb)):,} B; "
           f"**total {int(round(fb + wb)):,} B** against {nbytes:,} algorithmic bytes "
           f"(**{(fb + wb) / nbytes:.4f}×**). Reads: {fb / reads:.4f}× the algorithmic "
           f"{reads:,} B; writes: {wb / (nbytes - reads):.4f}× the algorithmic "
           f"{nbytes - reads:,} B.", ""]
    with open(os.path.join(out_dir, "prefill_quant_T8192_H7168_counters.md"), "w") as f:
        f.write("\n".join(md))
    return j


def _read_counters(path):
    """Per dispatch of a rocprofv3 counter pass: kernel, grid and the summed
    value of each counter collected."""
    import csv
    d = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            k = int(r["Dispatch_Id"])
            e = d.setdefault(k, {"name": _short_kernel(r["Kernel_Name"]), "grid": int(r["Grid_Size"]),
                                 "id": k, "c": {}})
            e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [d[k] for k in sorted(d)]


def _sweep_case_counters(rows, sweep):
    """Per sweep case: the case's kernel (the name with the most dispatches in
    its block, flush kernels aside) and each counter's mean per call (the sum
    over the kernel's dispatches divided by the calls, a call being as many
    dispatches as the library's plan launches)."""
    out = []
    for case, blk in zip(sweep, _case_blocks(rows)):
        by = {}
        for r in blk:
            if r["name"] != "read_probe_kernel":
                by.setdefault(r["name"], []).append(r)
        if not by:
            continue
        name = max(by, key=lambda n: len(by[n]))
        calls = len(by[name]) / _launches_per_call(case.get("kernel"))
        tot = {}
        for r in by[name]:
            for c, v in r["c"].items():
                tot[c] = tot.get(c, 0.0) + v
        out.append({"case": case, "kernel": name, "dispatches": len(by[name]),
                    "per_call": {c: v / calls for c, v in tot.items()}})
    return out


def summarize_sweep_counters(bench_json, counter_csvs, out_dir, commands, trace_csv=None):
    """Counter passes over a whole `bench.py --copy-calibration` run (sweep
    included). With FETCH_SIZE and WRITE_SIZE passes: HBM bytes per call of
    every sweep case against its algorithmic bytes, each counter scaled by
    what it reads for the run's three 1 GiB copies. With an SQ pass
    (SQ_WAVES, SQ_INSTS_VALU, SQ_INSTS_SALU): instructions per wave and the
    time vector issue alone needs, beside the warm median of the kernel
    trace `trace_csv` when given."""
    line = _last_json_line(bench_json)
    sweep = line.get("sweep", [])
    passes = [_read_counters(p) for p in counter_csvs]
    names = set()
    for rows in passes:
        for r in rows:
            names.update(r["c"])
    srcs = line.get("kernel_source_sha256") or kernel_source_hash()
    head = ["Commands (from `/tmp` with `TMPDIR=/tmp` on the MI355X box; `$R` is the repository "
            "root there), each in its own run:", ""] + [f"    {c}" for c in commands] + [
            "", "Written by `python bench.py --summarize-sweep-counters`. A sweep case's calls are "
            "its warm-up, back-to-back, cold (after a 1 GiB read-only flush), batched and "
            "graph-replayed calls; each figure is the mean per call over all of them.", "",
            f"Kernel source SHA-256 (`finalize_kernels.hip` + `device_common.h` + "
            f"`moef_internal.h`): `{srcs}`; every kernel source and the build script: "
            f"`{line.get('all_sources_sha256', 'not recorded')}`", ""]
    written = {}
    if "FETCH_SIZE" in names and "WRITE_SIZE" in names:
        per = {}
        factor = {}
        for rows in passes:
            for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
                cal = [r["c"][ctr] for r in rows
                       if r["name"] == "__amd_rocclr_copyBuffer" and ctr in r["c"]][:3]
                if cal:
                    factor[ctr] = (1 << 30) / (float(np.median(cal)) * 1024)
                    for e in _sweep_case_counters(rows, sweep):
                        per.setdefault(e["case"]["case"] + f" T={e['case']['T']}", {}).update(
                            {"case": e["case"], "kernel": e["kernel"],
                             "dispatches": e["dispatches"],
                             ctr: e["per_call"][ctr] * 1024 * factor[ctr]})
        if set(factor) != {"FETCH_SIZE", "WRITE_SIZE"}:
            raise ValueError("FETCH_SIZE and WRITE_SIZE passes need the --copy-calibration copies")
        md = ["# HBM traffic of every bench sweep case (rocprofv3 FETCH_SIZE / WRITE_SIZE)", ""]
        md += head
        md += [f"Calibration (1 GiB / counter reading of the three copies): fetch "
               f"{factor['FETCH_SIZE']:.6f}, write {factor['WRITE_SIZE']:.6f}.", "",
               "| case | kernel | dispatches | algorithmic read MB | counter read MB | read ratio "
               "| algorithmic write MB | counter write MB | write ratio |",
               "|---|---|---|---|---|---|---|---|---|"]
        rows_out = []
        for key, e in per.items():
            c = e["case"]
            if "FETCH_SIZE" not in e or "WRITE_SIZE" not in e or not c["algorithmic_bytes"]:
                continue
            wb = c.get("algorithmic_write_bytes")
            rb = c["algorithmic_bytes"] - wb if wb is not None else None
            label = f"{c['case']} T={c['T']} H={c['H']} k={c['top_k']}"
            fr, fw = e["FETCH_SIZE"], e["WRITE_SIZE"]
            md.append(f"| {label} | `{e['kernel']}` | {e['dispatches']} | "
                      f"{rb / 1e6 if rb is not None else float('nan'):,.3f} | {fr / 1e6:,.3f} | "
                      f"{fr / rb if rb else float('nan'):.4f} | "
                      f"{wb / 1e6 if wb is not None else float('nan'):,.3f} | {fw / 1e6:,.3f} | "
                      f"{fw / wb if wb else float('nan'):.4f} |")
            rows_out.append({"case": label, "kernel": e["kernel"], "read_bytes": fr,
                             "write_bytes": fw, "algorithmic_read_bytes": rb,
                             "algorithmic_write_bytes": wb})
        with open(os.path.join(out_dir, "finalize_sweep_counters.md"), "w") as f:
            f.write("\n".join(md) + "\n")
        written["hbm"] = rows_out
    if {"SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU"} <= names:
        warm = {}
        if trace_csv:
            for case, blk in zip(sweep, _case_blocks(_read_trace(trace_csv))):
                by = {}
                prev = None
                for r in blk:
                    if r["name"] != "read_probe_kernel" and not (
                            prev is not None and prev["name"] == "read_probe_kernel"):
                        by.setdefault(r["name"], []).append(r["us"])
                    prev = r
                if by:
                    n = max(by, key=lambda k: sum(by[k]))
                    warm[case["case"] + f" T={case['T']}"] = (
                        float(np.median(by[n])) * _launches_per_call(case.get("kernel")))
        md = ["# Instructions per wave and the vector-issue bound of every sweep case "
              "(rocprofv3 SQ counters)", ""]
        md += head
        md += ["A wave64 vector instruction occupies a 16-lane SIMD for 4 cycles, and the chip "
               "has 1024 SIMDs at 2.4 GHz, so the vector instructions of one call alone need "
               "VALU × 4 / (1024 × 2.4e9) s (the **VALU issue bound**). The time column is the "
               "warm median per call of the kernel trace named above (launches per call × the "
               "median dispatch).", "",
               "| case | kernel | waves | VALU / wave | SALU / wave | VALU issue bound µs | "
               "trace median µs | bound / time |", "|---|---|---|---|---|---|---|---|"]
        rows_out = []
        kd = line.get("roofline", {}).get("kernel", "")
        hname, hgrid = kd.split(" launches=")[0], None
        if " grid=" in kd:
            nwg, wg = (int(x) for x in kd.split(" grid=")[1].split()[0].split("x"))
            hgrid = nwg * wg
        for rows in passes:
            if not any("SQ_WAVES" in r["c"] for r in rows):
                continue
            # the headline launches: before the sweep's first marker
            head = []
            for r in rows:
                if r["name"] == "empty_probe_kernel" and r["grid"] == 128:
                    break
                if r["name"] == hname and r["grid"] == hgrid:
                    head.append(r)
            if head:
                tot = {c: sum(r["c"].get(c, 0.0) for r in head) / len(head)
                       for c in ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU")}
                t = None
                if trace_csv:
                    tr = [r["us"] for r in _read_trace(trace_csv)
                          if r["name"] == hname and r["grid"] == hgrid]
                    t = float(np.median(tr)) if tr else None
                cfg = line.get("config", {})
                label = (f"headline T={cfg.get('tokens')} H={cfg.get('hidden')} "
                         f"k={cfg.get('top_k')} (one launch)")
                waves = tot["SQ_WAVES"]
                bound = tot["SQ_INSTS_VALU"] * 4 / (1024 * 2.4e9) * 1e6
                md.append(f"| {label} | `{hname}` | {waves:,.0f} | "
                          f"{tot['SQ_INSTS_VALU'] / waves:,.0f} | {tot['SQ_INSTS_SALU'] / waves:,.0f} "
                          f"| {bound:.2f} | {t if t else float('nan'):.3f} | "
                          f"{bound / t * 100 if t else float('nan'):.0f}% |")
                rows_out.append({"case": label, "kernel": hname, "waves": waves,
                                 "valu_per_wave": tot["SQ_INSTS_VALU"] / waves,
                                 "salu_per_wave": tot["SQ_INSTS_SALU"] / waves,
                                 "valu_bound_us": bound, "trace_median_us": t})
            for e in _sweep_case_counters(rows, sweep):
                c, pc = e["case"], e["per_call"]
                if not pc.get("SQ_WAVES"):
                    continue
                waves = pc["SQ_WAVES"]
                valu, salu = pc["SQ_INSTS_VALU"] / waves, pc["SQ_INSTS_SALU"] / waves
                bound = pc["SQ_INSTS_VALU"] * 4 / (1024 * 2.4e9) * 1e6
                t = warm.get(c["case"] + f" T={c['T']}")
                label = f"{c['case']} T={c['T']} H={c['H']} k={c['top_k']}"
                md.append(f"| {label} | `{e['kernel']}` | {waves:,.0f} | {valu:,.0f} | {salu:,.0f} "
                          f"| {bound:.2f} | {t if t else float('nan'):.3f} | "
                          f"{bound / t * 100 if t else float('nan'):.0f}% |")
                rows_out.append({"case": label, "kernel": e["kernel"], "waves": waves,
                                 "valu_per_wave": valu, "salu_per_wave": salu,
                                 "valu_bound_us": bound, "trace_median_us": t})
        with open(os.path.join(out_dir, "finalize_sweep_instruction_counters.md"), "w") as f:
            f.write("\n".join(md) + "\n")
        written["sq"] = rows_out
    return written


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the shape sweep, the T curve and the same-session ceilings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "BENCH_JSON"),
                    help="CPU only: write the kernel-trace summaries under profiles/ from a "
                         "rocprofv3 kernel trace of this script and its JSON line")
    ap.add_argument("--summarize-counters", nargs="+", metavar="FILE",
                    help="CPU only: FETCH_CSV WRITE_CSV [BENCH_JSON]: write the counter summary "
                         "under profiles/ from the FETCH_SIZE and WRITE_SIZE passes (the kernel "
                         "source hash from a pass's JSON line when given)")
    ap.add_argument("--summarize-sweep-counters", nargs="+", metavar="FILE",
                    help="CPU only: BENCH_JSON COUNTER_CSV... [--trace TRACE_CSV]: write the "
                         "per-case counter summaries of a run with the sweep under profiles/")
    ap.add_argument("--trace", help="with --summarize-sweep-counters: a kernel trace of the "
                                    "same command, for the time column")
    ap.add_argument("--command", action="append", default=[],
                    help="the command that made the summarized data (recorded verbatim)")
    args = ap.parse_args()
    out_dir = os.path.join(ROOT, "profiles")
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, out_dir, " ".join(args.command) or "(not given)")
        return
    if args.summarize_counters:
        f, w, *bj = args.summarize_counters
        summarize_counters(f, w, out_dir, args.command or ["(not given)"], bj[0] if bj else None)
        return
    if args.summarize_sweep_counters:
        bj, *csvs = args.summarize_sweep_counters
        summarize_sweep_counters(bj, csvs, out_dir, args.command or ["(not given)"], args.trace)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the finalize "
              f"shards by token with no exchange, so N GPUs would each run this same "
              f"single-GPU step on T/N tokens)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import combine_moe_finalize_amd as M
    from combine_moe_finalize_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    M.load_library()   # fails loudly when the HIP library is missing

    t0 = time.perf_counter()
    wl = W.family_workload("prefill_fp8_ue8m0")
    log(f"generated workload T={wl.T} H={wl.H} k={wl.top_k} P={wl.P} in "
        f"{time.perf_counter() - t0:.1f} s")
    kw, _ = upload(wl, torch)
    T, H, k = wl.T, wl.H, wl.top_k
    q = torch.empty((T, H), dtype=torch.uint8, device="cuda:0")
    s = torch.empty((T, H // 128), dtype=torch.uint8, device="cuda:0")
    nbytes = bytes_quant(T, H, k)

    def step():
        M.moe_finalize_quant_ue8m0(**kw, out_e4m3=q, scale_e8m0=s)

    # the kernel this call launches on this device, as the library plans it
    kernel = M.moe_finalize_describe_launch(M.OP_QUANT_UE8M0, T, H, k)
    log(f"timed call: {kernel}")

    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda:0").fill_(3)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device-to-device copies")
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    avg_us = ev0.elapsed_time(ev1) * 1e3 / args.steps   # GPU time per launch
    ms_per_step = wall / args.steps * 1e3
    value = nbytes / (wall / args.steps) / 1e9
    achieved = nbytes / (avg_us * 1e-6) / 1e9
    log(f"kernel avg {avg_us:.2f} us (HIP events around the {args.steps} launches), "
        f"wall/step {ms_per_step * 1e3:.2f} us, {achieved:.0f} GB/s")

    result = {
        "metric": "finalize achieved HBM GB/s (% of peak) and us/call at T=1..8192 tokens",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "kernel_source_sha256": kernel_source_hash(),
        "all_sources_sha256": all_sources_hash(),
        "config": {"workload": "prefill_finalize_fp8_ue8m0", "tokens": T, "hidden": H,
                   "experts": wl.E, "top_k": k, "padded_rows": wl.P,
                   "routed_scaling_factor": wl.rsf, "shared_expert": True,
                   "routing": "fp32 weights",
                   "io": "bf16 in, fp32 accumulation, e4m3 + ue8m0 out",
                   "algorithmic_bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counters_traffic(),
                     "kernel": kernel,
                     "kernel_us_avg": round(avg_us, 3),
                     "kernel_us_method": f"HIP events on the launch stream around the {args.steps} "
                                         f"timed launches, divided by {args.steps}",
                     "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_sweep:
        st_us = steady_state_us(torch, step)
        log(f"steady state: {st_us:.2f} us per launch")
        result["steady_state"] = {
            "kernel_us_avg": round(st_us, 3),
            "achieved": round(nbytes / (st_us * 1e-6) / 1e9, 1),
            "frac": round(nbytes / (st_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "method": f"HIP events around launches {STEADY_LAUNCHES - STEADY_TIMED + 1}-"
                      f"{STEADY_LAUNCHES} of {STEADY_LAUNCHES} back-to-back launches right "
                      f"after the timed ones (not the timed region: after an idle gap the "
                      f"first ~100 launches run 2-5% slower while the clocks ramp up)"}
        read_gbs, copy_gbs, torch_copy_gbs = ceilings(torch)
        log(f"same-session ceilings: read {read_gbs:.0f}, copy {copy_gbs:.0f}, torch copy "
            f"{torch_copy_gbs:.0f} GB/s")
        result["ceilings"] = {
            "read_gbs": round(read_gbs, 1), "copy_gbs": round(copy_gbs, 1),
            "torch_copy_gbs": round(torch_copy_gbs, 1),
            "method": "1 GiB streams after the timed launches: the read and copy probes "
                      "(csrc/bandwidth_probes.h), 10 launches per event pair, median of 5; "
                      "torch's device copy, median of 20",
            "headline_frac_of_read": round(achieved / read_gbs, 4),
            "headline_frac_of_copy": round(achieved / copy_gbs, 4)}
    # us/call of the same operation on the first T tokens of the same workload,
    # T = 1, 2, 4, ..., 8192, per call under HIP-graph replay
    curve, curve_plain = {}, {}
    if not args.no_sweep:
        idx_all, w_all, sh_all = (kw["expanded_idx_to_permuted_idx"], kw["topk_weights"],
                                  kw["shared_out"])
        Tc = 1
        while Tc <= T:
            kc = dict(kw, expanded_idx_to_permuted_idx=idx_all[:Tc], topk_weights=w_all[:Tc],
                      shared_out=sh_all[:Tc])
            qc, sc = q[:Tc], s[:Tc]
            us = graph_us(torch, lambda: M.moe_finalize_quant_ue8m0(**kc, out_e4m3=qc,
                                                                     scale_e8m0=sc),
                          n=20 if Tc <= 256 else 5, reps=5 if Tc <= 1024 else 2)
            gbs = bytes_quant(Tc, H, k) / us / 1e3
            curve[str(Tc)] = {"us": round(us, 3), "gbs": round(gbs, 1),
                              "frac": round(gbs / HBM_PEAK_GBS, 4)}
            log(f"prefill op T={Tc}: {us:.3f} us/call, {gbs:.0f} GB/s")
            Tc *= 2
        # the plain bf16 finalize of the same tokens (no quant epilogue)
        out_bf16 = torch.empty((T, H), dtype=torch.bfloat16, device="cuda:0")
        for Tc in (256, 1024, 2048, 4096, 8192):
            if Tc > T:
                break
            kc = dict(kw, expanded_idx_to_permuted_idx=idx_all[:Tc], topk_weights=w_all[:Tc],
                      shared_out=sh_all[:Tc])
            oc = out_bf16[:Tc]
            us = graph_us(torch, lambda: M.moe_finalize(**kc, out=oc),
                          n=20 if Tc <= 256 else 5, reps=5 if Tc <= 1024 else 2)
            gbs = bytes_plain(Tc, H, k) / us / 1e3
            curve_plain[str(Tc)] = {"us": round(us, 3), "gbs": round(gbs, 1),
                                    "frac": round(gbs / HBM_PEAK_GBS, 4)}
            log(f"plain finalize T={Tc}: {us:.3f} us/call, {gbs:.0f} GB/s")
        del out_bf16
        step()                                   # the timed launches' outputs again
        torch.cuda.synchronize()
    # the timed launches' outputs, kept on the host for the CPU leg's parity report
    q_host = q.cpu().numpy() if not args.no_cpu_baseline else None
    s_host = s.cpu().numpy() if not args.no_cpu_baseline else None
    del kw, q, s
    torch.cuda.empty_cache()
    if not args.no_sweep:
        result["sweep"] = sweep(torch, M, W)
        # us/call over T = 1..8192: decode finalize (H=4096, top_k=8) per call
        # under HIP-graph replay, and the timed prefill launch (T=8192)
        per_call = {str(r["T"]): r["us_graph_replay"] for r in result["sweep"]
                    if r["case"] == "decode"}
        result["us_per_call"] = {
            "finalize_quant_ue8m0_H7168_k8_graph_replay": curve,
            "finalize_bf16_H7168_k8_graph_replay": curve_plain,
            "finalize_H4096_k8_graph_replay": per_call,
            "empty_kernel_graph_replay": round(launch_floor_us(torch), 3)}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"], result["parity"] = cpu_baseline(wl, q_host, s_host)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
