"""Host logic of the Python binding (no GPU): which stream handle and which
current device an entry point is called with. A stub stands in for the
library and records its arguments; torch's device queries are patched."""
import contextlib

import pytest
import torch

from combine_moe_finalize_amd import _binding as B


class Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append((name, args, entered[-1] if entered else None))
            return 0
        return fn


entered = []


@pytest.fixture
def stub(monkeypatch):
    rec = Recorder()
    monkeypatch.setattr(B, "_lib", rec)
    monkeypatch.setattr(B, "_raw_stream", lambda index: 0x1000 + index)

    @contextlib.contextmanager
    def device_ctx(device):
        entered.append(device.index)
        try:
            yield
        finally:
            entered.pop()

    monkeypatch.setattr(torch.cuda, "device", device_ctx)
    return rec


def test_current_device_calls_directly_with_its_stream(stub, monkeypatch):
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    B._call("moe_topk_packed_decode", torch.device("cuda:0"), 1, 2)
    name, args, ctx = stub.calls[-1]
    assert name == "moe_topk_packed_decode"
    assert args == (1, 2, 0x1000)            # the stream of device 0 comes last
    assert ctx is None                       # no device switch


def test_other_device_is_made_current_for_the_call(stub, monkeypatch):
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    B._call("moe_topk_packed_decode", torch.device("cuda:1"), 7)
    name, args, ctx = stub.calls[-1]
    assert args == (7, 0x1001)               # device 1's stream
    assert ctx == 1                          # called inside device 1's context


def test_failed_status_raises(monkeypatch):
    class Failing:
        def __getattr__(self, name):
            return lambda *a: 3
    monkeypatch.setattr(B, "_lib", Failing())
    monkeypatch.setattr(B, "_raw_stream", lambda index: 0)
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    monkeypatch.setattr(B, "status_string", lambda s: "unsupported")
    with pytest.raises(B.MoeFinalizeError) as e:
        B._call("moe_finalize", torch.device("cuda:0"))
    assert e.value.status == 3


def test_tensor_rules_report_the_first_broken_rule():
    t = torch.zeros((2, 8), dtype=torch.bfloat16)
    assert B._tensor(t, "x", torch.bfloat16, (2, 8)) is t
    assert B._tensor(t, "x", torch.bfloat16, t.shape) is t
    with pytest.raises(TypeError, match="torch.Tensor"):
        B._tensor([1, 2], "x", torch.bfloat16, (2,))
    with pytest.raises(TypeError, match="torch.float32"):
        B._tensor(t, "x", torch.float32, (2, 8))
    with pytest.raises(ValueError, match="shape"):
        B._tensor(t, "x", torch.bfloat16, (8, 2))
    with pytest.raises(ValueError, match="contiguous"):
        B._tensor(t.t(), "x", torch.bfloat16, (8, 2))


def test_cpu_tensors_are_rejected():
    t = torch.zeros(4)
    with pytest.raises(ValueError, match="GPU"):
        B._on_device(t.device, x=t)
    with pytest.raises(ValueError, match="expected cuda:0"):
        B._on_device(torch.device("cuda:0"), x=t)


def test_fp8_outputs_are_written_through_a_byte_view_and_returned_as_given():
    f8 = torch.zeros((2, 128), dtype=torch.float8_e4m3fn)
    codes = B._code_bytes(f8)
    assert codes.dtype == torch.uint8 and codes.data_ptr() == f8.data_ptr()
    u8 = torch.zeros((2, 128), dtype=torch.uint8)
    assert B._code_bytes(u8) is u8
