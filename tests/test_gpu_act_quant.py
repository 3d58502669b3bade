"""GPU parity of the standalone FP8 activation quant against the CPU oracle.
Both policies are bit-exact by contract: the power-of-two one shares the
finalize epilogue's rule, and the continuous one is two correctly rounded
fp32 divisions followed by one nearest-even E4M3 rounding."""
import numpy as np
import pytest
import torch

import combine_moe_finalize_amd as M
from combine_moe_finalize_amd import workloads as W
from oracle import act_quant as A
from oracle import formats as F

from gpu_helpers import announce, assert_bits_equal, d_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    M.load_library()


def run_both(x_bits):
    x = d_bf16(x_bits)
    q1, s1 = M.moe_act_quant_fp8_ue8m0(x)
    q2, s2 = M.moe_act_quant_fp8_amax(x)
    torch.cuda.synchronize()
    return (q1.cpu().numpy(), s1.cpu().numpy()), (q2.cpu().numpy(), s2.cpu().numpy())


def check_both(x_bits, got, chunk=1024):
    (q1, s1), (q2, s2) = got
    for t0 in range(0, x_bits.shape[0], chunk):
        sl = slice(t0, t0 + chunk)
        oq, os_ = A.act_quant_ue8m0(x_bits[sl])
        assert_bits_equal(s1[sl], os_, f"UE8M0 scales {sl}")
        assert_bits_equal(q1[sl], oq, f"UE8M0 codes {sl}")
        oq, os_ = A.act_quant_amax(x_bits[sl])
        assert_bits_equal(s2[sl].view(np.uint32), os_.view(np.uint32), f"amax scales {sl}")
        assert_bits_equal(q2[sl], oq, f"amax codes {sl}")


def test_prefill_size():
    x = W.activations(8192, 7168, seed=11)
    announce("act quant T=8192 H=7168, both policies")
    check_both(x, run_both(x))


@pytest.mark.parametrize("T,H", [(1, 128), (3, 384), (17, 1152), (64, 7168), (5, 16384)])
def test_shapes(T, H):
    x = W.activations(T, H, seed=T * 7 + H)
    announce(f"act quant T={T} H={H}")
    check_both(x, run_both(x))


@pytest.mark.parametrize("T,H", [(131077, 128), (2340, 7168), (2341, 7168)])
def test_two_vectors_per_lane_threshold_and_tail(T, H):
    """Inputs of at least 2^21 16-byte vectors take two vectors per lane.
    T=131077, H=128 is just above that with a last wave half-filled in its
    first vector (64 lanes) and partly in its second (16 lanes); T=2340 and
    2341 at H=7168 sit on either side of the threshold."""
    x = W.activations(T, H, seed=T + H)
    announce(f"act quant threshold/tail T={T} H={H} vectors={T * H // 8}")
    check_both(x, run_both(x), chunk=max(1, (1 << 20) // H))


def test_exhaustive_values_and_scales():
    """Every finite bf16 value in [-448, 448] inside blocks whose max is 448;
    then every positive finite bf16 as a block max with random others, and an
    all-zero block."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f64(pats)
    a_vals = pats[np.isfinite(v) & (np.abs(v) <= 448)]
    nblk = -(-a_vals.size // 127)
    A_ = np.zeros((nblk, 128), np.uint16)
    flat = np.zeros(nblk * 127, np.uint16)
    flat[:a_vals.size] = a_vals
    A_[:, 1:] = flat.reshape(nblk, 127)
    A_[:, 0] = 0x43E0
    pos = pats[np.isfinite(v) & (v > 0)]
    B_ = np.zeros((pos.size + 1, 128), np.uint16)
    B_[:-1, 0] = pos
    B_[:-1, 1] = pos | 0x8000
    rng = np.random.default_rng(5)
    fac = rng.uniform(-1, 1, size=(pos.size, 126))
    B_[:-1, 2:] = F.bf16_bits(F.bf16_to_f64(pos)[:, None] * fac)
    blocks = np.concatenate([A_, B_])
    H = 7168
    T = -(-blocks.shape[0] // (H // 128))
    rows = np.zeros((T * (H // 128), 128), np.uint16)
    rows[:blocks.shape[0]] = blocks
    x = rows.reshape(T, H)
    announce(f"act quant exhaustive T={T}")
    check_both(x, run_both(x))


def test_policies_agree_on_power_of_two_blocks():
    rng = np.random.default_rng(9)
    T, H = 32, 2048
    xb = rng.uniform(-0.99, 0.99, size=(T, H // 128, 128))
    m = rng.integers(-30, 20, size=(T, H // 128))
    xb *= (448.0 * np.exp2(m))[..., None]
    xb[:, :, 7] = -448.0 * np.exp2(m)
    x = F.bf16_bits(xb.reshape(T, H))
    announce("act quant policies agree")
    (q1, s1), (q2, s2) = run_both(x)
    assert np.array_equal(q1, q2)
    assert np.array_equal(s1.astype(np.int64) - 127, m)
    assert np.array_equal(s2, np.exp2(m).astype(np.float32))


def blocks_under_maxima(maxima):
    """Blocks of 128: the maximum A first, then every finite bf16 x with |x| <= A
    (127 per block, the last block padded with zeros)."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f64(pats)
    out = []
    for a in maxima:
        A = F.bf16_to_f64(np.array([a], np.uint16))[0]
        xs = pats[np.isfinite(v) & (np.abs(v) <= A)]
        nblk = -(-xs.size // 127)
        b = np.zeros((nblk, 128), np.uint16)
        flat = np.zeros(nblk * 127, np.uint16)
        flat[:xs.size] = xs
        b[:, 1:] = flat.reshape(nblk, 127)
        b[:, 0] = a
        out.append(b)
    return np.concatenate(out)


def test_continuous_scale_every_value_under_sampled_maxima():
    """The continuous policy's quotient x / s against the oracle's IEEE fp32
    division, bit for bit through the codes, for every bf16 x under sampled
    block maxima A:
      * A whose mantissa has a factor 7 (1.75, 1.3125, 1.09375 times 2^k),
        so s = A/448 is short and many quotients sit exactly on E4M3 midpoints;
      * random A;
      * A whose scale sits on either side of 2^-60 and 2^60, where the
        kernel switches between its two division paths;
      * the smallest and largest A (subnormal and huge scales)."""
    rng = np.random.default_rng(21)
    sevens = []
    for m in (1.75, 1.3125, 1.09375):
        for k in rng.integers(-120, 120, size=20):
            sevens.append(m * 2.0 ** int(k))
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f64(pats)
    pos = pats[np.isfinite(v) & (v > 0)]
    edges = []
    for e in (-60, 60):
        b = int(F.bf16_bits(np.array([448.0 * 2.0 ** e]))[0])
        edges += [b - 2, b - 1, b, b + 1, b + 2]
    maxima = np.concatenate([F.bf16_bits(np.array(sevens)), rng.choice(pos, 200, replace=False),
                             np.array(edges, np.uint16),
                             np.array([0x0001, 0x0080, 0x7F7F], np.uint16)])
    blocks = blocks_under_maxima(maxima)
    H = 7168
    T = -(-blocks.shape[0] // (H // 128))
    rows = np.zeros((T * (H // 128), 128), np.uint16)
    rows[:blocks.shape[0]] = blocks
    x = rows.reshape(T, H)
    announce(f"act quant continuous scale, {maxima.size} maxima, T={T}")
    check_both(x, run_both(x))
