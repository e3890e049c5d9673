"""The Python binding checks every tensor a caller hands to Matmul before any pointer
reaches the library (CPU only, no GPU and no library call): a wrong device, element
type, layout or size would otherwise become an out-of-bounds or host-pointer access in
the kernel. Device tensors are stood in for by a small fake with the attributes the
checks read."""
import pytest
import torch

import gemm_epilogues_epilog_amd as ge
from gemm_epilogues_epilog_amd import _require


class FakeDev:
    """What the checks read of a device tensor."""

    def __init__(self, shape, dtype, device="cuda:0", contiguous=True):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = self.device.type == "cuda"
        self._contig = contiguous

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def is_contiguous(self):
        return self._contig


DEV = torch.device("cuda:0")


def test_require_accepts_a_matching_tensor():
    _require(FakeDev((64,), torch.float16), "bias", "f16", 64, DEV)
    _require(FakeDev((2, 48), torch.int32), "relu_aux", "i32", 96, DEV)


@pytest.mark.parametrize("t,why", [
    (torch.zeros(64, dtype=torch.float16), "device tensor"),                 # host memory
    (FakeDev((64,), torch.float16, device="cuda:1"), "is on"),               # another GPU
    (FakeDev((64,), torch.float32), "f16 elements"),                          # fp32 read as 16-bit
    (FakeDev((64,), torch.float16, contiguous=False), "contiguous"),
    (FakeDev((48,), torch.float16), "64 elements"),                           # length n, not m
])
def test_require_rejects(t, why):
    with pytest.raises(ValueError, match=why):
        _require(t, "bias", "f16", 64, DEV)


def mm(epilog="RELU_AUX_BIAS", dtype="f16", vec=None):
    return ge.Matmul(64, 48, 32, dtype, epilog, vec_dtype=vec)


def ops(dtype=torch.float16):
    return FakeDev((64, 32), dtype), FakeDev((32, 48), dtype)


def test_outputs_rejects_host_operands():
    with pytest.raises(ValueError, match="device tensor"):
        mm()._outputs(torch.zeros(64, 32, dtype=torch.float16), torch.zeros(32, 48, dtype=torch.float16),
                      None, None, None, None)


def test_outputs_rejects_bad_tensors_before_planning():
    A, B = ops()
    bias = FakeDev((64,), torch.float16)
    cases = [
        dict(bias=None),                                                     # RELU_AUX_BIAS needs a bias
        dict(bias=torch.zeros(64, dtype=torch.float16)),                     # host bias
        dict(bias=FakeDev((48,), torch.float16)),                            # length n
        dict(bias=FakeDev((64,), torch.float32)),                            # fp32 bias for an f16 plan
        dict(bias=bias, out=FakeDev((64, 40), torch.float16)),               # out of another shape
        dict(bias=bias, out=FakeDev((64, 48), torch.bfloat16)),              # out of another type
        dict(bias=bias, relu_aux=FakeDev((1, 48), torch.int32)),             # mask for m <= 32
        dict(bias=bias, relu_aux=FakeDev((2, 48), torch.float32)),           # mask not int32
        dict(bias=bias, relu_aux=FakeDev((2, 48), torch.int32, device="cuda:1")),
    ]
    for kw in cases:
        m = mm()
        with pytest.raises(ValueError):
            m._outputs(A, B, kw.get("bias"), kw.get("relu_aux"), kw.get("out"), kw.get("bgrad"))
        assert m.handle is None, kw   # rejected before any plan was made


def test_outputs_backward_checks():
    A, B = ops(torch.bfloat16)
    m = mm("DRELU_BGRAD", "bf16")
    with pytest.raises(ValueError, match="relu_aux"):
        m._outputs(A, B, None, None, None, None)
    with pytest.raises(ValueError, match="bgrad"):
        m._outputs(A, B, None, FakeDev((2, 48), torch.int32), None, FakeDev((64,), torch.float16))
    with pytest.raises(ValueError, match="bgrad"):
        mm("DRELU_BGRAD", "bf16", vec="f32")._outputs(A, B, None, FakeDev((2, 48), torch.int32), None,
                                                      FakeDev((64,), torch.bfloat16))
    assert m.handle is None


def test_outputs_operand_shapes_and_devices():
    A, B = ops()
    with pytest.raises(ValueError, match="shapes"):
        mm()._outputs(FakeDev((32, 64), torch.float16), B, None, None, None, None)
    with pytest.raises(ValueError, match="same device"):
        mm()._outputs(A, FakeDev((32, 48), torch.float16, device="cuda:1"), None, None, None, None)


def test_outputs_unfused_backward_checks():
    # DRELU_BGRAD_UNFUSED reads the forward activation (m, n) in the plan's type
    A, B = ops(torch.bfloat16)
    m = mm("DRELU_BGRAD_UNFUSED", "bf16")
    with pytest.raises(ValueError, match="act"):
        m._outputs(A, B, None, None, None, None)                                   # no activation
    with pytest.raises(ValueError, match="act"):
        m._outputs(A, B, None, None, None, None, FakeDev((2, 48), torch.int32))    # a mask is not it
    with pytest.raises(ValueError, match="act"):
        m._outputs(A, B, None, None, None, None, FakeDev((64, 40), torch.bfloat16))
    with pytest.raises(ValueError, match="act"):
        m._outputs(A, B, None, None, None, None, FakeDev((64, 48), torch.float16))
    with pytest.raises(ValueError, match="bgrad"):
        m._outputs(A, B, None, None, None, FakeDev((48,), torch.bfloat16), FakeDev((64, 48), torch.bfloat16))
    assert m.handle is None
