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


def _counter_csv(path, dispatches, counter):
    """A rocprofv3 counter-collection CSV: (kernel name, grid, value) per
    dispatch, each value split over two rows as the per-instance rows are."""
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
            "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
            "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
            "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    lines = [",".join(f'"{c}"' for c in cols)]
    for i, (name, grid, vals) in enumerate(dispatches, 1):
        for ctr, v in vals.items():
            if counter is not None and ctr != counter:
                continue
            for half in (0.25 * v, 0.75 * v):
                lines.append(f'{i},{i},"Agent 1",1,1,1,{grid},1,"{name}",256,0,0,8,0,16,'
                             f'"{ctr}",{half},{1000 * i},{1000 * i + 500}')
    path.write_text("\n".join(lines) + "\n")


def test_sweep_counter_summary(tmp_path, monkeypatch):
    """Cases split at the marker launches; the copies calibrate each counter
    (here FETCH_SIZE reads half the bytes, as it does for 128-byte requests);
    a call of a two-launch kernel counts both dispatches; flush kernels and
    the markers are left out."""
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h" * 64)
    copy = ("__amd_rocclr_copyBuffer", 1 << 20, {"FETCH_SIZE": 524288.0, "WRITE_SIZE": 1048576.0})
    mark = ("void (anonymous namespace)::empty_probe_kernel()", 128, {"FETCH_SIZE": 0.0,
                                                                        "WRITE_SIZE": 0.0})
    flush = ("void (anonymous namespace)::read_probe_kernel(uint4 const*, unsigned int*)", 1 << 26,
             {"FETCH_SIZE": 1e6, "WRITE_SIZE": 0.0})
    one = ("void moef::finalize_kernel<8, true>(moef::GatherArgs, uint4*)", 4096,
           {"FETCH_SIZE": 50.0, "WRITE_SIZE": 10.0})
    two = ("void moef::finalize_rmsnorm_staged_kernel<8, true>(moef::GatherArgs)", 65536,
           {"FETCH_SIZE": 500.0, "WRITE_SIZE": 300.0})
    d = [copy, copy, copy, mark, one, one, flush, one, mark, two, two, flush, two, two]
    _counter_csv(tmp_path / "f.csv", d, "FETCH_SIZE")
    _counter_csv(tmp_path / "w.csv", d, "WRITE_SIZE")
    sweep = [{"case": "decode", "T": 1, "H": 4096, "top_k": 8, "algorithmic_bytes": 110 * 1024,
              "algorithmic_write_bytes": 10 * 1024, "kernel": "finalize_kernel<8, true> launches=1 grid=1"},
             {"case": "residual_rmsnorm", "T": 4096, "H": 7168, "top_k": 8,
              "algorithmic_bytes": 2600 * 1024, "algorithmic_write_bytes": 600 * 1024,
              "kernel": "finalize_rmsnorm_staged_kernel<8, true> launches=2 grid=256x1024"}]
    (tmp_path / "b.json").write_text("log line\n" + json.dumps({"sweep": sweep}) + "\n")
    out = bench.summarize_sweep_counters(str(tmp_path / "b.json"),
                                         [str(tmp_path / "f.csv"), str(tmp_path / "w.csv")],
                                         str(tmp_path), ["cmd one", "cmd two"])
    hbm = {r["case"].split()[0]: r for r in out["hbm"]}
    assert hbm["decode"]["kernel"] == "finalize_kernel<8, true>"
    assert hbm["decode"]["read_bytes"] == pytest.approx(100 * 1024)
    assert hbm["decode"]["write_bytes"] == pytest.approx(10 * 1024)
    assert hbm["residual_rmsnorm"]["read_bytes"] == pytest.approx(2000 * 1024)
    assert hbm["residual_rmsnorm"]["write_bytes"] == pytest.approx(600 * 1024)
    text = (tmp_path / "finalize_sweep_counters.md").read_text()
    assert "cmd one" in text and "cmd two" in text and "1.0000" in text
    sq = ("void moef::finalize_kernel<8, true>(moef::GatherArgs, uint4*)", 4096,
          {"SQ_WAVES": 64.0, "SQ_INSTS_VALU": 64.0 * 300, "SQ_INSTS_SALU": 64.0 * 100})
    sq_mark = (mark[0], 128, {"SQ_WAVES": 1.0, "SQ_INSTS_VALU": 0.0, "SQ_INSTS_SALU": 2.0})
    _counter_csv(tmp_path / "sq.csv", [sq_mark, sq, sq, sq_mark], None)
    out = bench.summarize_sweep_counters(str(tmp_path / "b.json"), [str(tmp_path / "sq.csv")],
                                         str(tmp_path), ["cmd"])
    r = out["sq"][0]
    assert r["waves"] == 64 and r["valu_per_wave"] == 300 and r["salu_per_wave"] == 100
    assert r["valu_bound_us"] == pytest.approx(64 * 300 * 4 / (1024 * 2.4e9) * 1e6)


def test_trace_summary(tmp_path, monkeypatch):
    """The headline's timed launches follow its warm-up ones, and the steady
    state is the last 100 of the 300 launches after them; a sweep case is
    split at its marker into warm dispatches, cold ones (right after the
    flush kernel) and the last 200 (the graph replays)."""
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h" * 64)
    head = "void moef::finalize_quant_staged_kernel<8, true, 12>(moef::GatherArgs, uint2*)"
    dec = "void moef::finalize_kernel<8, true>(moef::GatherArgs, uint4*)"
    mark = "void (anonymous namespace)::empty_probe_kernel()"
    flush = "void (anonymous namespace)::read_probe_kernel(uint4 const*, unsigned int*)"
    d = [(head, 616 * 1024, 180.0)] + [(head, 616 * 1024, us) for us in (170.0, 172.0)]
    d += [(head, 616 * 1024, 175.0)] * 200 + [(head, 616 * 1024, 168.0)] * 100   # steady state
    d += [(mark, 128, 1.0)] + [(dec, 512, 3.0)] * 30
    d += [(flush, 1 << 26, 150.0), (dec, 512, 5.0)] * 3 + [(dec, 512, 2.0)] * 200
    lines = ["Kernel_Name,Grid_Size_X,Workgroup_Size_X,Dispatch_Id,Start_Timestamp,End_Timestamp"]
    t = 0
    for i, (n, g, us) in enumerate(d, 1):
        lines.append(f'"{n}",{g},256,{i},{t},{t + int(us * 1000)}')
        t += int(us * 1000) + 500
    (tmp_path / "t.csv").write_text("\n".join(lines) + "\n")
    line = {"warmup": 1, "steps": 2, "config": {"tokens": 8192, "hidden": 7168, "top_k": 8},
            "roofline": {"kernel": "finalize_quant_staged_kernel<8, true, 12> launches=1 "
                                   "grid=616x1024 groups=8 tail=5%",
                         "algorithmic_bytes_per_launch": 1_116_667_904, "kernel_us_avg": 171.5},
            "steady_state": {"kernel_us_avg": 168.5},
            "sweep": [{"case": "decode", "T": 1, "H": 4096, "top_k": 8,
                       "algorithmic_bytes": 81_984,
                       "kernel": "finalize_kernel<8, true> launches=1 grid=2x256"}]}
    (tmp_path / "b.json").write_text(json.dumps(line) + "\n")
    out = bench.summarize_trace(str(tmp_path / "t.csv"), str(tmp_path / "b.json"), str(tmp_path),
                                "cmd")
    assert len(out) == 1 and out[0]["kernel"] == "finalize_kernel<8, true>"
    assert out[0]["cold"]["n"] == 3 and out[0]["cold"]["median"] == pytest.approx(5.0)
    assert out[0]["warm"]["n"] == 230 and out[0]["graph_us_per_call"] == pytest.approx(2.0)
    text = (tmp_path / "prefill_quant_T8192_H7168_kernel_trace.md").read_text()
    assert "| 2 timed (after 1 warm-up) | 171.000 |" in text and "cmd" in text
    assert "| 100 steady state (the last of 300 launches right after the timed ones) | 168.000 |" in text
