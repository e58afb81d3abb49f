"""The Python binding rejects mismatched buffers before any C call: the C ABI takes
plain pointers and cannot see a tensor's length, dtype or layout, so a wrong one would
otherwise read or write device memory out of bounds.  CPU only: every library entry
point is replaced by a function that fails the test if it is reached."""
import types

import pytest
import torch

import moe_expert_ffn_softmax_amd as pkg
from moe_expert_ffn_softmax_amd import MoeExpertFFN, RouteBuffers

C_CALLS = [n for n in dir(pkg) if n.startswith("afd_ffn_")] + ["load"]


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def reached(*a, **k):
        raise AssertionError("a library call was reached")
    for n in C_CALLS:
        monkeypatch.setattr(pkg, n, reached)


def stub_layer(dtype="bf16", H=256, M=128, E=4, k=2, T=8):
    """A layer object with the fields the checks read (no handle, CPU 'device')."""
    layer = MoeExpertFFN.__new__(MoeExpertFFN)
    layer.cfg = types.SimpleNamespace(hidden=H, inter=M, num_experts=E, top_k=k, max_tokens=T, shared_inter=0)
    layer.dtype = dtype
    layer.device = torch.device("cpu")
    layer.handle = None
    rb = RouteBuffers.__new__(RouteBuffers)
    rb.max_tokens, rb.num_experts, rb.top_k = T, E, k
    return layer, rb


def test_forward_rejects_wrong_dtype_size_layout_and_T():
    layer, rb = stub_layer()
    T, H = 8, 256
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    y = torch.zeros(T, H, dtype=torch.bfloat16)
    bad = {
        "fp32 x on a bf16 layer": dict(x=x.float()),
        "fp16 y": dict(y=y.half()),
        "x shorter than T rows": dict(x=x[:5]),
        "non-contiguous x": dict(x=torch.zeros(H, T, dtype=torch.bfloat16).t()),
        "y not a tensor": dict(y=[0.0]),
        "T above max_tokens": dict(T=9),
        "negative T": dict(T=-1),
    }
    for what, over in bad.items():
        args = dict(x=x, T=T, y=y)
        args.update(over)
        with pytest.raises((ValueError, TypeError)):
            layer.forward(args["x"], args["T"], rb, args["y"])
        assert what


def test_forward_rejects_route_buffers_of_another_layer():
    layer, rb = stub_layer()
    _, rb_other = stub_layer(E=8)
    x = torch.zeros(8, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        layer.forward(x, 8, rb_other, x.clone())
    with pytest.raises(ValueError):
        layer.forward(x, 8, object(), x.clone())


def test_route_and_capacity_reject_wrong_id_and_logit_types():
    layer, rb = stub_layer()
    T, E, k = 8, 4, 2
    with pytest.raises(ValueError):
        layer.route(torch.zeros(T, E, dtype=torch.float64), T, rb)
    with pytest.raises(ValueError):
        layer.route(torch.zeros(T - 1, E), T, rb)
    ids64 = torch.zeros(T, k, dtype=torch.int64)   # torch.topk's index type
    gates = torch.zeros(T, k)
    limits = torch.zeros(E, dtype=torch.int32)
    with pytest.raises(ValueError):
        layer.route_capacity(ids64, gates, T, limits, 1)
    with pytest.raises(ValueError):
        layer.route_capacity(ids64.int(), gates, T, limits.long(), 1)
    out = (torch.zeros(T, dtype=torch.int32), torch.zeros(T), torch.zeros(E, dtype=torch.int32),
           torch.zeros(T, dtype=torch.int32))     # offsets one short
    with pytest.raises(ValueError):
        layer.route_capacity(ids64.int(), gates, T, limits, 1, out=out)
    with pytest.raises(ValueError):
        layer.route_select_bias(torch.zeros(T, E), torch.zeros(E - 1), T, rb)


def test_fp8_input_and_route_hidden_checks():
    layer, rb = stub_layer(dtype="fp8")
    T, H, E = 8, 256, 4
    xq = torch.zeros(T, H, dtype=torch.uint8)
    xs = torch.zeros(T, H // 128)
    y = torch.zeros(T, H, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        layer.forward_fp8_input(xq, xs[:, :1], T, rb, y)
    with pytest.raises(ValueError):
        layer.forward_fp8_input(xq.float(), xs, T, rb, y)
    bf_layer, bf_rb = stub_layer()
    with pytest.raises(ValueError):
        bf_layer.forward_fp8_input(xq, xs, T, bf_rb, y)
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bf_layer.route_hidden(x, torch.zeros(E, H), torch.zeros(T, E), T, bf_rb)
    with pytest.raises(ValueError):
        bf_layer.route_hidden(x, torch.zeros(E, H, dtype=torch.bfloat16), torch.zeros(T, E - 1), T, bf_rb)


def test_constructor_checks_weight_shapes_dtypes_and_device():
    H, M, E = 256, 128, 4
    kw = dict(hidden=H, inter=M, num_experts=E, top_k=2, max_tokens=8, dtype="bf16")
    wgu = torch.zeros(E, H, 2 * M, dtype=torch.bfloat16)
    wd = torch.zeros(E, M, H, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        MoeExpertFFN(w_gate_up=torch.zeros(E, H, M, dtype=torch.bfloat16), w_down=wd, **kw)
    with pytest.raises(ValueError, match="dtype"):
        MoeExpertFFN(w_gate_up=wgu.float(), w_down=wd, **kw)
    with pytest.raises(ValueError, match="GPU"):
        MoeExpertFFN(w_gate_up=wgu, w_down=wd, **kw)    # right shapes, but host tensors
    fp8 = dict(kw, dtype="fp8")
    with pytest.raises(TypeError, match="s_gate_up"):
        MoeExpertFFN(w_gate_up=torch.zeros(E, H, 2 * M, dtype=torch.uint8),
                     w_down=torch.zeros(E, M, H, dtype=torch.uint8), s_gate_up=None, s_down=None, **fp8)
    with pytest.raises(ValueError, match="inter"):
        MoeExpertFFN(**dict(kw, inter=100), w_gate_up=wgu, w_down=wd)


def test_quantize_rejects_fp16_and_ragged_columns():
    with pytest.raises(ValueError):
        pkg.quantize_fp8(torch.zeros(4, 128, dtype=torch.float16))
    with pytest.raises(ValueError):
        pkg.quantize_fp8(torch.zeros(4, 100))
    with pytest.raises(ValueError):
        pkg.quantize_fp8(torch.zeros(4, 128))   # a host tensor
