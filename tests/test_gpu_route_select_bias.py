"""Parity of afd_ffn_route_select_bias with the oracle's selection-only-bias router.

The experts are chosen on the fp32 sum score + bias and the gates are the softmax of the
chosen experts' unbiased scores (the dynamic bias of "MoE 大规模分布式推理工程实战：从
All-to-All 通信到动态专家放置", §4.1, steering only the choice).  ids, counts, offsets,
sorted pairs and pair positions are compared bit-exactly, gates to 2e-6 (the two sides
use different exp implementations).  Both paths of the route call are covered: the
one-launch route of batches of at most 64 tokens, and router + permute above that
(with the permute's multi-block form above 8192 pairs).
"""
import numpy as np
import pytest
import torch

import oracle
from moe_expert_ffn_softmax_amd import MoeExpertFFN

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _layer(E, k, T, H=128, M=128, dtype="bf16", w_gu=None, w_d=None):
    """A layer used only for routing unless weights are given (zeros otherwise)."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    if w_gu is None:
        w_gu = torch.zeros((E, H, 2 * M), dtype=tdt, device="cuda")
        w_d = torch.zeros((E, M, H), dtype=tdt, device="cuda")
    return MoeExpertFFN(hidden=H, inter=M, num_experts=E, top_k=k, max_tokens=max(T, 1), dtype=dtype,
                        w_gate_up=w_gu, w_down=w_d)


def _compare(layer, rb, scores, bias, T, E, k):
    P = T * k
    ids_o, gates_o = oracle.route_select_bias(scores, bias, k)
    counts_o, offsets_o, sp_o, pp_o = oracle.permute(ids_o, E)
    np.testing.assert_array_equal(rb.topk_ids[:P].cpu().numpy(), ids_o.ravel())
    np.testing.assert_allclose(rb.topk_gates[:P].cpu().numpy(), gates_o.ravel(), rtol=0, atol=2e-6)
    np.testing.assert_array_equal(rb.expert_counts.cpu().numpy(), counts_o)
    np.testing.assert_array_equal(rb.expert_offsets.cpu().numpy(), offsets_o)
    np.testing.assert_array_equal(rb.sorted_pair[:P].cpu().numpy(), sp_o)
    np.testing.assert_array_equal(rb.pair_pos[:P].cpu().numpy(), pp_o)


def _run(scores, bias, k, T_max=None):
    T, E = scores.shape
    layer = _layer(E, k, T_max or T)
    rb = layer.new_route()
    layer.route_select_bias(torch.from_numpy(scores).cuda(), torch.from_numpy(bias).cuda(), T, rb)
    torch.cuda.synchronize()
    return layer, rb


@pytest.mark.parametrize("T,E,k", [
    (1, 8, 2),         # one token
    (6, 128, 8),       # the starved-decode router shape (one-launch route)
    (64, 256, 8),      # largest one-launch batch
    (65, 128, 8),      # smallest router + permute batch
    (37, 20, 4),       # ragged expert count (not a multiple of the wave)
    (1580, 128, 8),    # the aggregated batch's router shape
    (4096, 256, 8),    # the fp8 layer's router shape: 32768 pairs, multi-block permute
    (200, 1024, 32),   # the largest expert count and slot count the library takes
    (50, 48, 3),       # the coarse layer's router shape
])
def test_select_bias_random(T, E, k):
    """scores ~ N(0, 1), bias ~ N(0, 0.5) (variance), as in the decode layer's logits."""
    print(f"case select_bias random T={T} E={E} k={k}", flush=True)
    rng = np.random.default_rng(T * 131 + E)
    scores = rng.standard_normal((T, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * np.sqrt(0.5)).astype(np.float32)
    layer, rb = _run(scores, bias, k)
    _compare(layer, rb, scores, bias, T, E, k)
    layer.close()


@pytest.mark.parametrize("T,E,k", [(40, 16, 4), (300, 64, 6), (9000, 32, 2)])
def test_select_bias_integer_ties(T, E, k):
    """Integer scores and biases in [-2, 2]: equal keys are common, so the order of
    equal keys (lower expert first) decides most slots."""
    print(f"case select_bias ties T={T} E={E} k={k}", flush=True)
    rng = np.random.default_rng(7 + T)
    scores = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    bias = rng.integers(-2, 3, size=E).astype(np.float32)
    layer, rb = _run(scores, bias, k)
    _compare(layer, rb, scores, bias, T, E, k)
    layer.close()


@pytest.mark.parametrize("T", [20, 700])
def test_select_bias_rounding_ties(T):
    """Scores in [1, 2) with a fine mantissa and biases of 0, 2 or 6: score + bias lands
    in [3, 4) or [7, 8), where the ulp is 2 or 4 times that of the score, so keys of
    distinct scores round together (and halfway cases round to even).  The selection
    must follow the rounded fp32 keys, the gates the unrounded scores."""
    print(f"case select_bias rounding ties T={T}", flush=True)
    E, k = 32, 4
    rng = np.random.default_rng(T)
    scores = (1.0 + rng.integers(0, 16, size=(T, E)) * 2.0 ** -23).astype(np.float32)
    bias = rng.choice(np.array([0.0, 2.0, 6.0], np.float32), size=E).astype(np.float32)
    keys = (scores + bias).astype(np.float32)
    same_key = keys[:, :, None] == keys[:, None, :]
    diff_score = scores[:, :, None] != scores[:, None, :]
    assert np.any(same_key & diff_score)  # ties that exist only after rounding
    layer, rb = _run(scores, bias, k)
    _compare(layer, rb, scores, bias, T, E, k)
    layer.close()


@pytest.mark.parametrize("T,E,k", [(6, 128, 8), (500, 64, 4)])
def test_zero_bias_equals_plain_route(T, E, k):
    """With an all-zero bias the call is the plain router: every route field is equal,
    gates bit-for-bit."""
    rng = np.random.default_rng(11)
    scores = rng.standard_normal((T, E)).astype(np.float32)
    layer = _layer(E, k, T)
    a, b = layer.new_route(), layer.new_route()
    s = torch.from_numpy(scores).cuda()
    layer.route_select_bias(s, torch.zeros(E, dtype=torch.float32, device="cuda"), T, a)
    layer.route(s, T, b)
    torch.cuda.synchronize()
    for name in ("topk_ids", "topk_gates", "expert_counts", "expert_offsets", "sorted_pair", "pair_pos"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    layer.close()


def test_select_bias_rejects_null_bias_and_handles_empty():
    from moe_expert_ffn_softmax_amd import AfdError, afd_ffn_route_select_bias
    layer = _layer(8, 2, 4)
    rb = layer.new_route()
    s = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):  # the binding
        layer.route_select_bias(s, None, 4, rb)
    with pytest.raises(AfdError):   # the C ABI
        afd_ffn_route_select_bias(layer.handle, s, None, 4, rb.c)
    layer.route_select_bias(s, torch.zeros(8, device="cuda"), 0, rb)  # T = 0: no-op
    torch.cuda.synchronize()
    layer.close()


@pytest.mark.parametrize("T", [6, 150])
def test_forward_after_select_bias_route(T):
    """Whole layer: a bias of +64 on a set S of k experts forces every token onto S, so
    each token's output is sum over S of softmax(scores restricted to S) times the expert
    FFNs.  The oracle layer computes the same from logits that keep the scores on S and
    lower every other expert by 1e4 (its plain router then picks S with the same gates)."""
    import workloads
    print(f"case select_bias forward T={T}", flush=True)
    E, k, H, M = 16, 4, 256, 256
    w = workloads.Workload(f"select_bias_fwd_T{T}", 300 + T, T=T, H=H, M=M, E=E, k=k, Ms=0, dtype="bf16")
    weights = workloads.make_weights(w, device="cuda")
    x, _ = workloads.make_activations(w, device="cuda")
    rng = np.random.default_rng(T)
    scores = rng.standard_normal((T, E)).astype(np.float32)
    S = np.array([2, 5, 11, 14])
    bias = np.zeros(E, np.float32)
    bias[S] = 64.0
    layer = _layer(E, k, T, H=H, M=M, w_gu=weights["w_gu"], w_d=weights["w_d"])
    rb = layer.new_route()
    layer.route_select_bias(torch.from_numpy(scores).cuda(), torch.from_numpy(bias).cuda(), T, rb)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    layer.forward(x, T, rb, y)
    torch.cuda.synchronize()
    ids = rb.topk_ids[:T * k].cpu().numpy().reshape(T, k)
    assert np.array_equal(np.sort(ids, axis=1), np.broadcast_to(S, (T, k)))
    forced = scores.copy()
    off = np.ones(E, bool)
    off[S] = False
    forced[:, off] -= 1e4
    _, gates_o, yref, _ = oracle.layer_from_weights(x.float().cpu().numpy(), forced, w, weights,
                                                    experts_needed=S)
    # slot orders may differ (keys score + 64 can round together), so compare gates by expert
    gates = rb.topk_gates[:T * k].cpu().numpy().reshape(T, k)
    g_gpu = np.zeros((T, E))
    np.put_along_axis(g_gpu, ids.astype(np.int64), gates, axis=1)
    ids_o = np.argsort(-forced, axis=1, kind="stable")[:, :k]
    g_o = np.zeros((T, E))
    np.put_along_axis(g_o, ids_o, gates_o, axis=1)
    np.testing.assert_allclose(g_gpu, g_o, rtol=0, atol=2e-6)
    err = np.abs(y.float().cpu().numpy() - yref).max()
    scale = np.abs(yref).max()
    print(f"  max|err|/max|ref| = {err / scale:.2e}", flush=True)
    assert err <= 2e-2 * scale
    layer.close()
