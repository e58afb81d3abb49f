"""afd_ffn_forward_noalloc (the forward for callers that cannot allocate: its
intermediate buffers live in the library's static device scratch) gives the same
output as afd_ffn_forward, bit for bit, on two calls in a row, the second with a
smaller batch; a batch too large for the scratch is refused before anything runs."""
import numpy as np
import pytest
import torch

import workloads
from moe_expert_ffn_softmax_amd import AfdError, MoeExpertFFN, afd_ffn_forward, afd_ffn_forward_noalloc
from moe_expert_ffn_softmax_amd._ffi import AFD_EINVAL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def layer_of(w, max_tokens):
    weights = workloads.make_weights(w, device="cuda")
    return MoeExpertFFN(hidden=w.H, inter=w.M, num_experts=w.E, top_k=w.k, max_tokens=max_tokens, dtype=w.dtype,
                        w_gate_up=weights["w_gu"], w_down=weights["w_d"], s_gate_up=weights["s_gu"],
                        s_down=weights["s_d"], shared_inter=w.Ms, ws_gate_up=weights["ws_gu"],
                        ws_down=weights["ws_d"], ss_gate_up=weights["ss_gu"], ss_down=weights["ss_d"])


CASES = [
    workloads.Workload("noalloc_bf16", 501, T=200, H=1024, M=512, E=16, k=4, Ms=0, dtype="bf16"),
    workloads.Workload("noalloc_bf16_decode_shared", 502, T=6, H=1024, M=512, E=32, k=8, Ms=256, dtype="bf16"),
    workloads.Workload("noalloc_fp8_shared", 503, T=160, H=1024, M=512, E=16, k=4, Ms=256, dtype="fp8"),
    workloads.Workload("noalloc_f32", 504, T=50, H=256, M=256, E=8, k=2, Ms=128, dtype="f32"),
]


@pytest.mark.parametrize("w,kernel", [(w, "auto") for w in CASES] +
                         [(workloads.Workload("noalloc_fused", 506, T=6, H=512, M=512, E=16, k=4, Ms=256,
                                              dtype="bf16"), "fused")], ids=lambda v: v if isinstance(v, str) else v.name)
def test_noalloc_forward_equals_forward_twice(w, kernel):
    print(f"no-alloc case {w.name} gemm={kernel}", flush=True)
    layer = layer_of(w, w.T)
    layer.set_gemm_kernel(kernel)
    x, logits = workloads.make_activations(w, device="cuda")
    ydt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    for T in (w.T, max(1, w.T // 3)):     # the second call with a smaller batch
        rb = layer.new_route()
        layer.route(logits[:T].contiguous(), T, rb)
        y_ref = torch.full((T, w.H), float("nan"), dtype=ydt, device="cuda")
        y = torch.full((T, w.H), float("nan"), dtype=ydt, device="cuda")
        afd_ffn_forward(layer.handle, x, T, rb.c, y_ref)
        torch.cuda.synchronize()
        afd_ffn_forward_noalloc(layer.handle, x, T, rb.c, y)
        torch.cuda.synchronize()
        assert torch.isfinite(y.float()).all()
        assert torch.equal(y, y_ref), f"{w.name} T={T}: max diff {(y.float() - y_ref.float()).abs().max().item()}"
    layer.close()


def test_noalloc_refuses_a_layer_beyond_the_scratch():
    """The scratch is laid out for the handle's max_tokens.  bf16 buffers: h and O take
    (max_tokens * k) * (M + H) * 2 bytes: 54.1 MB at 1200 tokens (fits the 64 MiB =
    67.1 MB scratch), 67.6 MB at 1500 (refused, whatever T the call passes)."""
    w = workloads.Workload("noalloc_big", 505, T=1200, H=4096, M=1536, E=4, k=4, Ms=0, dtype="bf16")
    x = torch.zeros((1500, w.H), dtype=torch.bfloat16, device="cuda")
    logits = torch.zeros((1500, w.E), dtype=torch.float32, device="cuda")
    y = torch.zeros((1500, w.H), dtype=torch.bfloat16, device="cuda")
    big = layer_of(w, 1500)
    rb = big.new_route()
    big.route(logits, 16, rb)
    with pytest.raises(AfdError) as e:
        afd_ffn_forward_noalloc(big.handle, x, 16, rb.c, y)
    assert e.value.code == AFD_EINVAL
    big.close()
    fits = layer_of(w, 1200)
    rb = fits.new_route()
    fits.route(logits, 1200, rb)
    afd_ffn_forward_noalloc(fits.handle, x, 1200, rb.c, y)
    torch.cuda.synchronize()
    assert torch.isfinite(y[:1200].float()).all()
    fits.close()
