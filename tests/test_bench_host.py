"""Host-side parts of bench.py (no GPU): the one-GPU rule, the loud failure
without a GPU, the algorithmic byte models against a count taken from the
workload's own arrays, and the rule that HBM traffic is reported only for the
kernel source the counters were taken on."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from combine_moe_finalize_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "--gpus 2" in r.stderr and "one GPU" in r.stderr
    assert r.stdout == ""


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = run_bench("--steps", "1", "--warmup", "0", "--no-sweep", "--no-cpu-baseline")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""


def counted_bytes(wl, with_shared, outputs):
    """Bytes the method must move, counted from the arrays themselves: the
    gathered rows (one per live slot), the shared rows, the index and weight
    rows, and the outputs."""
    live = int(np.count_nonzero(wl.idx >= 0))
    row = wl.gemm2_out.shape[1] * wl.gemm2_out.itemsize
    n = live * row + wl.idx.nbytes + wl.weights.nbytes
    if with_shared:
        n += wl.shared.nbytes
    return n + outputs


@pytest.mark.parametrize("with_shared", [True, False])
def test_byte_models_match_a_direct_count(with_shared):
    wl = W.make_workload(64, 1024, 16, 8, rsf=1.0, seed=1, with_residual=True)
    T, H, k = wl.T, wl.H, wl.top_k
    plain = counted_bytes(wl, with_shared, T * H * 2)
    assert bench.bytes_plain(T, H, k, shared=with_shared) == plain
    rms = counted_bytes(wl, with_shared, 2 * T * H * 2) + wl.residual.nbytes + wl.gamma.nbytes
    assert bench.bytes_rmsnorm(T, H, k, shared=with_shared) == rms
    quant = counted_bytes(wl, with_shared, T * H + T * (H // 128))
    assert bench.bytes_quant(T, H, k, shared=with_shared) == quant


def test_headline_bytes_per_launch():
    """The prefill figure quoted with the roofline: 136 312 B per token."""
    assert bench.bytes_quant(8192, 7168, 8) == 1_116_667_904
    assert bench.bytes_quant(1, 7168, 8) == 136_312


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    good = {"kernel_source_sha256": bench.kernel_source_hash(), "hbm_bytes_per_launch": 123}
    p = tmp_path / "c.json"
    p.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(p))
    assert bench.counters_traffic() == 123
    p.write_text(json.dumps(dict(good, kernel_source_sha256="0" * 64)))
    assert bench.counters_traffic() is None
    p.write_text("not json")
    assert bench.counters_traffic() is None
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "missing.json"))
    assert bench.counters_traffic() is None


def test_committed_counters_match_the_committed_source():
    """The counter summary in the repository was taken on the kernel sources
    in the repository, so the bench line carries traffic."""
    with open(bench.COUNTERS_FILE) as f:
        c = json.load(f)
    assert c["kernel_source_sha256"] == bench.kernel_source_hash()
    assert c["algorithmic_bytes_per_launch"] == bench.bytes_quant(8192, 7168, 8)
    assert 1.0 <= c["traffic_over_algorithmic"] < 1.05


def test_parity_statistics_of_the_cpu_leg():
    """The CPU leg times the oracle's fp32 mirror and reports parity: outputs
    equal to the mirror show no mismatch against it (every token of the
    timed pass) and at most one step against the fp64 truth (its sample);
    one flipped code is counted against both references."""
    from oracle import finalize as O
    wl = W.make_workload(40, 1024, 16, 8, rsf=2.5, seed=3, log2_mag=(-8.0, 8.0))
    q, s, _ = O.finalize_quant_mirror(wl.gemm2_out, wl.idx, weights_f32=wl.weights,
                                      shared=wl.shared, rsf=wl.rsf)
    base, par = bench.cpu_baseline(wl, q, s, min_s=0.0, max_s=60.0, chunk=16, truth_tokens=24,
                                   threads=1)
    assert base["kind"] == "oracle" and base["cores"] == 1 and "fp32 mirror" in base["sample"]
    assert par["tokens_vs_fp32_mirror"] == 40 and par["tokens_vs_fp64_truth"] == 24
    assert par["code_mismatches_vs_mirror"] == 0 and par["scale_mismatches_vs_mirror"] == 0
    assert par["max_code_steps_vs_truth"] <= 1
    q2 = q.copy()
    q2[3, 5] = q2[3, 5] ^ 0x04                     # four steps away
    _, par2 = bench.cpu_baseline(wl, q2, s, min_s=0.0, max_s=60.0, chunk=16, truth_tokens=24,
                                 threads=1)
    assert par2["code_mismatches_vs_mirror"] == 1
    assert par2["max_code_steps_vs_truth"] >= 3


def test_e4m3_step_distance():
    a = np.array([0x00, 0x80, 0x01, 0x81, 0x7E, 0x38], np.uint8)
    b = np.array([0x80, 0x00, 0x81, 0x01, 0x7D, 0x3A], np.uint8)
    assert bench.e4m3_steps(a, b).tolist() == [0, 0, 2, 2, 1, 2]


def test_cpu_leg_on_a_thread_pool():
    """With threads > 1 the value is the thread pool's rate, cores its thread
    count, and the one-thread rate is kept beside it."""
    wl = W.make_workload(32, 1024, 16, 8, rsf=2.5, seed=4)
    base, par = bench.cpu_baseline(wl, min_s=0.0, max_s=60.0, chunk=8, threads=3,
                                   min_s_threads=0.0)
    assert par is None
    assert base["cores"] == 3 and base["kind"] == "oracle" and base["unit"] == "GB/s"
    assert base["value"] > 0 and base["single_thread"]["cores"] == 1
    assert base["single_thread"]["value"] > 0
    assert "3 threads" in base["sample"]
    assert 1 <= bench.host_threads() <= 16
