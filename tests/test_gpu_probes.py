"""The bandwidth probes on the GPU: the copy is byte-exact, the read probe
really reads (its sink is written when, and only when, a lane's bytes XOR to
the sentinel), and the empty kernel launches."""
import ctypes

import pytest
import torch

from combine_moe_finalize_amd._paths import PROBE_LIB_PATH

from gpu_helpers import DEV, announce

pytestmark = pytest.mark.gpu
GRAIN = 16384
SENTINEL = 0x9E3779B9


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    L = ctypes.CDLL(PROBE_LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.moef_probe_read.argtypes = [vp, i64, vp, vp]
    L.moef_probe_copy.argtypes = [vp, vp, i64, vp]
    L.moef_probe_empty.argtypes = [vp]
    return L


def test_empty_probe_launches(lib):
    announce("probe empty, 100 launches")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(100):
        assert lib.moef_probe_empty(stream) == 0
    torch.cuda.synchronize()


def test_copy_is_exact(lib):
    n = 67 * GRAIN
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros_like(src)
    announce(f"probe copy {n} bytes")
    assert lib.moef_probe_copy(src.data_ptr(), dst.data_ptr(), n,
                               torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_read_probe_reads(lib):
    n = 5 * GRAIN
    src = torch.zeros(n // 4, dtype=torch.int32, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    announce("probe read, all zero")
    assert lib.moef_probe_read(src.data_ptr(), n, sink.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    # block 3, lane 7: its vectors are 3*1024 + 7 + {0, 256, 512, 768}; plant
    # the sentinel in the first word of the third one
    vec = 3 * 1024 + 7 + 512
    src[vec * 4] = SENTINEL - (1 << 32)                  # the same 32 bits, as int32
    announce("probe read, one planted sentinel")
    assert lib.moef_probe_read(src.data_ptr(), n, sink.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == SENTINEL
