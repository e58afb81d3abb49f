"""afd_ffn_forward_fp8_input: the fp8 layer on activations that arrive as e4m3 codes
plus per-token, per-128-channel fp32 scales (the FP8/BF16 mixed precision of the
omica.com.cn AFD article, §3.3).

* Codes and scales from the library's own quantiser: the output equals
  afd_ffn_forward on the bf16 activations bit-for-bit (same kernels, same codes).
* Codes and scales from another quantiser (torch's e4m3 cast with scale amax/224):
  the output matches the oracle run on the dequantised activations code * scale,
  within the fp8 bar 6e-2 * max|ref|, so the GEMMs honour the scales they are given.
* Other layer types reject the call.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_expert_ffn_softmax_amd import AfdError, MoeExpertFFN, afd_ffn_forward_fp8_input, quantize_fp8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _case(name, **kw):
    base = dict(name=name, index=400, T=37, H=256, M=384, E=16, k=4, Ms=0, dtype="fp8")
    base.update(kw)
    return workloads.Workload(**base)


CASES = [
    _case("fp8_input_ragged", T=37, H=256, M=384, E=16, k=4),
    _case("fp8_input_shared", T=50, H=384, M=256, E=6, k=2, Ms=256),
    _case("fp8_input_one_token", T=1, H=128, M=128, E=8, k=2, Ms=128),
    _case("fp8_input_many_rows", T=600, H=512, M=256, E=4, k=2, Ms=128),
]


def _layer(w, weights):
    return MoeExpertFFN(hidden=w.H, inter=w.M, num_experts=w.E, top_k=w.k, max_tokens=w.T, dtype="fp8",
                        w_gate_up=weights["w_gu"], w_down=weights["w_d"], s_gate_up=weights["s_gu"],
                        s_down=weights["s_d"], shared_inter=w.Ms, ws_gate_up=weights["ws_gu"],
                        ws_down=weights["ws_d"], ss_gate_up=weights["ss_gu"], ss_down=weights["ss_d"])


@pytest.mark.parametrize("kernel", ["stream", "tiled"])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_fp8_input_equals_bf16_forward(w, kernel):
    print(f"case {w.name} gemm={kernel}: own quantiser, bit-exact", flush=True)
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = _layer(w, weights)
    layer.set_gemm_kernel(kernel)
    rb = layer.new_route()
    layer.route(logits, w.T, rb)
    y_ref = torch.full((w.T, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    layer.forward(x, w.T, rb, y_ref)
    xq, xs = quantize_fp8(x)
    y = torch.full((w.T, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    layer.forward_fp8_input(xq, xs, w.T, rb, y)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    layer.close()


@pytest.mark.parametrize("kernel", ["stream", "tiled"])
@pytest.mark.parametrize("w", CASES[:2] + CASES[3:], ids=lambda w: w.name)
def test_fp8_input_other_quantiser_vs_oracle(w, kernel):
    print(f"case {w.name} gemm={kernel}: foreign quantiser vs oracle", flush=True)
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    # scale = amax / 224 per token and 128 channels, codes = torch's e4m3 cast of x / scale
    xg = x.float().view(w.T, w.H // 128, 128)
    amax = xg.abs().amax(dim=2, keepdim=True)
    xs = torch.where(amax > 0, amax / 224.0, torch.ones_like(amax))
    codes = (xg / xs).to(torch.float8_e4m3fn)
    xq = codes.view(torch.uint8).view(w.T, w.H).contiguous()
    xs = xs.view(w.T, w.H // 128).contiguous()
    x_deq = (codes.float() * xs.view(w.T, w.H // 128, 1)).view(w.T, w.H)
    layer = _layer(w, weights)
    layer.set_gemm_kernel(kernel)
    rb = layer.new_route()
    layer.route(logits, w.T, rb)
    y = torch.full((w.T, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    layer.forward_fp8_input(xq, xs, w.T, rb, y)
    torch.cuda.synchronize()
    _, _, yref, _ = oracle.layer_from_weights(x_deq.cpu().numpy(), logits.cpu().numpy(), w, weights)
    yg = y.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(yg).all()
    err = np.abs(yg - yref).max()
    scale = np.abs(yref).max()
    print(f"  max|err|/max|ref| = {err / scale:.3e}", flush=True)
    assert err <= 6e-2 * scale
    layer.close()


def test_fp8_input_rejects_other_layers_and_overlap():
    w = workloads.Workload("fp8_input_bf16_layer", 401, T=8, H=128, M=128, E=4, k=2, Ms=0, dtype="bf16")
    weights = workloads.make_weights(w, device="cuda")
    layer = MoeExpertFFN(hidden=w.H, inter=w.M, num_experts=w.E, top_k=w.k, max_tokens=w.T, dtype="bf16",
                         w_gate_up=weights["w_gu"], w_down=weights["w_d"])
    rb = layer.new_route()
    xq = torch.zeros((8, 128), dtype=torch.uint8, device="cuda")
    xs = torch.ones((8, 1), dtype=torch.float32, device="cuda")
    y = torch.empty((8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # the binding refuses first
        layer.forward_fp8_input(xq, xs, 8, rb, y)
    with pytest.raises(AfdError):    # and so does the C ABI
        afd_ffn_forward_fp8_input(layer.handle, xq, xs, 8, rb.c, y)
    layer.close()
    w8 = CASES[0]
    weights = workloads.make_weights(w8, device="cuda")
    layer = _layer(w8, weights)
    rb = layer.new_route()
    buf = torch.zeros(w8.T * w8.H * 2, dtype=torch.uint8, device="cuda")
    xs = torch.ones((w8.T, w8.H // 128), dtype=torch.float32, device="cuda")
    with pytest.raises(AfdError):  # y on top of xq (the C ABI's own overlap check)
        afd_ffn_forward_fp8_input(layer.handle, buf, xs, w8.T, rb.c, buf)
    afd_ffn_forward_fp8_input(layer.handle, buf, xs, 0, rb.c, buf)  # T = 0: no-op, nothing checked past the route
    torch.cuda.synchronize()
    layer.close()


def test_select_bias_route_and_fp8_input_forward_in_a_hip_graph():
    """The selection-only-bias route and the pre-quantised fp8 forward captured in one
    HIP graph: every replay, with eager work and synchronisations in between, equals
    the eager calls bit for bit."""
    w = _case("fp8_input_graph", T=70, H=256, M=256, E=16, k=4, Ms=128)
    print(f"case {w.name}: graph of route_select_bias + forward_fp8_input", flush=True)
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    bias = torch.linspace(-1.0, 1.0, w.E, device="cuda")
    xq, xs = quantize_fp8(x)
    layer = _layer(w, weights)
    rb_e = layer.new_route()
    y_e = torch.zeros((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    layer.route_select_bias(logits, bias, w.T, rb_e)
    layer.forward_fp8_input(xq, xs, w.T, rb_e, y_e)
    torch.cuda.synchronize()
    rb = layer.new_route()
    y = torch.zeros_like(y_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        layer.route_select_bias(logits, bias, w.T, rb, stream=s)  # warm-up on the capture stream
        layer.forward_fp8_input(xq, xs, w.T, rb, y, stream=s)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            layer.route_select_bias(logits, bias, w.T, rb, stream=s)
            layer.forward_fp8_input(xq, xs, w.T, rb, y, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    other = torch.zeros_like(y_e)
    for rep in range(3):
        y.zero_()
        rb.sorted_pair.fill_(-1)
        rb2 = layer.new_route()
        layer.route_select_bias(logits.flip(0), bias.flip(0), w.T, rb2)  # unrelated eager work
        layer.forward_fp8_input(xq.flip(0).contiguous(), xs.flip(0).contiguous(), w.T, rb2, other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_e.view(torch.int16)), f"replay {rep}: output differs"
        assert torch.equal(rb.sorted_pair, rb_e.sorted_pair), f"replay {rep}: permutation differs"
        assert torch.equal(rb.topk_gates, rb_e.topk_gates), f"replay {rep}: gates differ"
    layer.close()
