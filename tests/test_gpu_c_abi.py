"""The C ABI from plain C: a gcc-built driver (tests/c/abi_driver.c) links the
library and the HIP runtime, with no Python or torch, runs the finalize (fp32
and packed weights), the UE8M0 quant, and the all-reduce + residual + RMSNorm
over the two finalize outputs (a host array of device pointers) on a stream it
creates, and checks rejected calls; its outputs are compared here with the CPU
oracle."""
import os
import subprocess

import numpy as np
import pytest

from combine_moe_finalize_amd import workloads as W
from oracle import finalize as O
from oracle import formats as F

from gpu_helpers import announce, assert_bits_equal, ulp_bf16

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c", "abi_driver")


# (20608, 128, ...): 20 608 one-chunk units, 80 per CU on 256 CUs, so the UE8M0
# call takes the staged-output kernel there
@pytest.mark.parametrize("T,H,E,k", [(7, 1024, 16, 2), (64, 7168, 256, 8), (5, 1000, 32, 3),
                                     (20608, 128, 16, 2)])
def test_c_driver_matches_oracle(tmp_path, T, H, E, k):
    if not os.path.exists(DRIVER):
        pytest.fail(f"{DRIVER} is not built (run __graft_entry__.build())")
    wl = W.make_workload(T, H, E, k, rsf=2.5, seed=T + H)
    d = str(tmp_path)
    with open(os.path.join(d, "meta.txt"), "w") as f:
        f.write(f"{wl.T} {wl.H} {wl.top_k} {wl.P} {wl.rsf}\n")
    wl.gemm2_out.tofile(os.path.join(d, "g2.bin"))
    wl.idx.tofile(os.path.join(d, "idx.bin"))
    wl.weights.tofile(os.path.join(d, "w.bin"))
    wl.packed.tofile(os.path.join(d, "packed.bin"))
    wl.shared.tofile(os.path.join(d, "shared.bin"))
    gamma = W.to_bf16_bits(np.random.default_rng(H).uniform(0.5, 1.5, H).astype(np.float32))
    gamma.tofile(os.path.join(d, "gamma.bin"))
    announce(f"C driver T={T} H={H} k={k}")
    res = subprocess.run([DRIVER, d], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    out = np.fromfile(os.path.join(d, "out.bin"), dtype=np.uint16).reshape(T, H)
    outp = np.fromfile(os.path.join(d, "out_packed.bin"), dtype=np.uint16).reshape(T, H)
    ref, _ = O.finalize_mirror(wl.gemm2_out, wl.idx, weights_f32=wl.weights, shared=wl.shared,
                               rsf=wl.rsf)
    refp, _ = O.finalize_mirror(wl.gemm2_out, wl.idx, packed=wl.packed, shared=wl.shared,
                                rsf=wl.rsf)
    assert_bits_equal(out, ref, "C driver fp32")
    assert_bits_equal(outp, refp, "C driver packed")
    assert np.fromfile(os.path.join(d, "err.bin"), dtype=np.int32)[0] == 0
    ro = np.fromfile(os.path.join(d, "ro.bin"), dtype=np.uint16).reshape(T, H)
    nm = np.fromfile(os.path.join(d, "nm.bin"), dtype=np.uint16).reshape(T, H)
    m_ro, m_nm = O.allreduce_residual_rmsnorm_mirror(np.stack([ref, refp]), wl.shared, gamma)
    assert_bits_equal(ro, m_ro, "C driver all-reduce residual_out")
    g, o = F.bf16_to_f64(nm), F.bf16_to_f64(m_nm)
    assert np.all(np.abs(g - o) <= ulp_bf16(o)), "C driver all-reduce normed"
    if H % 128 == 0:
        q = np.fromfile(os.path.join(d, "q.bin"), dtype=np.uint8).reshape(T, H)
        s = np.fromfile(os.path.join(d, "s.bin"), dtype=np.uint8).reshape(T, H // 128)
        mq, ms, _ = O.quant_ue8m0(ref)
        assert_bits_equal(s, ms, "C driver scales")
        assert_bits_equal(q, mq, "C driver codes")
