"""moe_finalize_describe_launch on the device: the launch plan it names is
the CPU model's for this device's CU count (the host-stub cases, computed
for 256 CUs, are compared exactly when the device has 256), it is the same
on a non-default stream, and the kernel it names for the bench's headline
call is the staged quant kernel."""
import pytest
import torch

import combine_moe_finalize_amd as M

from test_staged_plans import DESCRIBE_CASES

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    M.load_library()


@pytest.fixture(scope="module")
def ncu():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("op,T,H,k,cus,want", [c for c in DESCRIBE_CASES if c[4] == 256])
def test_description_on_the_device(ncu, op, T, H, k, cus, want):
    if ncu != cus:
        pytest.skip(f"the expected strings are for {cus} CUs; this device has {ncu}")
    assert M.moe_finalize_describe_launch(op, T, H, k) == want


def test_same_on_another_stream():
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        on_side = M.moe_finalize_describe_launch(M.OP_QUANT_UE8M0, 8192, 7168, 8)
    assert on_side == M.moe_finalize_describe_launch(M.OP_QUANT_UE8M0, 8192, 7168, 8)


def test_headline_call_is_staged(ncu):
    d = M.moe_finalize_describe_launch(M.OP_QUANT_UE8M0, 8192, 7168, 8)
    assert d.startswith("finalize_quant_staged_kernel<8, true, ")
    nwg = int(d.split(" grid=")[1].split("x")[0])
    assert nwg >= ncu
