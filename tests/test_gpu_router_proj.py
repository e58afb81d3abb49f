"""Parity of afd_ffn_route_hidden (router projection, then routing) with the oracle.

On inputs from a grid where every fp32 partial sum is exact (test_route_hidden_exact_*)
the scores and the whole routing result are compared bit-exactly (gates to 2e-6).
On random inputs the scores are floating point and decide integers (the selection), so
the comparison is split:
  * scores: |gpu - oracle| within the fp32 summation bound for any order of the H
    products (each bf16 x bf16 product is exact in fp32): 2 (H + 2) 2^-24 sum_h
    |x_h w_h| + 2^-23 |score|, a factor 2 above the textbook bound;
  * tokens whose top-(k+1) oracle scores are separated by more than twice that bound
    are unambiguous: their ids equal the oracle's routing of its own scores (rounded to
    fp32) and their gates agree to 1e-4;
  * for the other tokens the selection is checked to be a valid top-k of the GPU's own
    scores (stable order: ties to the lower expert index);
  * counts, offsets, sorted pairs and pair positions are those of the GPU's ids.
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


def _layer(H, E, k, T, dtype):
    """A layer whose FFN weights are zero: only its routing is used here."""
    M = 128
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    w_gu = torch.zeros((E, H, 2 * M), dtype=tdt, device="cuda")
    w_d = torch.zeros((E, M, H), dtype=tdt, device="cuda")
    return MoeExpertFFN(hidden=H, inter=M, num_experts=E, top_k=k, max_tokens=max(T, 1), dtype=dtype,
                        w_gate_up=w_gu, w_down=w_d)


def _inputs(T, H, E, seed, dtype, bias_scale):
    """Seeded x ~ N(0, 1), gate vectors ~ N(0, 1/H), bias ~ N(0, bias_scale^2), rounded
    to the layer's activation type (bf16 values are exact in fp32)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((T, H), generator=g)
    w = torch.randn((E, H), generator=g) / np.sqrt(H)
    b = torch.randn(E, generator=g) * bias_scale
    if dtype != "f32":
        x, w = x.to(torch.bfloat16), w.to(torch.bfloat16)
    return x, w, b


def _check(T, H, E, k, dtype="bf16", seed=0, bias_scale=0.1, use_bias=True):
    print(f"case route_hidden T={T} H={H} E={E} k={k} {dtype} bias={use_bias}", flush=True)
    layer = _layer(H, E, k, T, dtype)
    x, w, b = _inputs(T, H, E, seed, dtype, bias_scale)
    rb = layer.new_route()
    logits = torch.full((max(T, 1), E), float("nan"), dtype=torch.float32, device="cuda")
    layer.route_hidden(x.cuda(), w.cuda(), logits, T, rb, bias=b.cuda() if use_bias else None)
    torch.cuda.synchronize()
    xf, wf, bf = x.float().numpy(), w.float().numpy(), b.numpy()
    ref = oracle.router_scores(xf, wf, bf if use_bias else None)
    got = logits[:T].cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    absum = np.abs(xf.astype(np.float64)) @ np.abs(wf.astype(np.float64)).T
    bound = 2 * (H + 2) * 2.0 ** -24 * absum + 2.0 ** -23 * np.abs(ref)
    err = np.abs(got - ref)
    print(f"  scores: max err {err.max():.3e}, max err/bound {(err / bound).max():.3f}", flush=True)
    assert np.all(err <= bound)

    P = T * k
    ids = rb.topk_ids[:P].cpu().numpy().reshape(T, k)
    gates = rb.topk_gates[:P].cpu().numpy().reshape(T, k)
    ids_o, gates_o = oracle.route(ref.astype(np.float32), k)
    # unambiguous tokens: adjacent gaps among the k+1 largest oracle scores exceed 2 bounds
    kk = min(k + 1, E)
    order = np.argsort(-ref, axis=1, kind="stable")[:, :kk]
    top = np.take_along_axis(ref, order, axis=1)
    tb = np.take_along_axis(bound, order, axis=1).max(axis=1, keepdims=True)
    clear = np.all(-np.diff(top, axis=1) > 2 * tb, axis=1) if kk > 1 else np.ones(T, bool)
    print(f"  {int(clear.sum())} of {T} tokens unambiguous", flush=True)
    np.testing.assert_array_equal(ids[clear], ids_o[clear])
    np.testing.assert_allclose(gates[clear], gates_o[clear], rtol=0, atol=1e-4)
    # every token: a valid stable top-k of the GPU's own scores, gates their softmax
    np.testing.assert_array_equal(ids, np.argsort(-logits[:T].cpu().numpy(), axis=1, kind="stable")[:, :k])
    sel = np.take_along_axis(got, ids.astype(np.int64), axis=1)
    p = np.exp(sel - sel.max(axis=1, keepdims=True))
    np.testing.assert_allclose(gates, p / p.sum(axis=1, keepdims=True), rtol=0, atol=2e-6)
    # the permutation of the GPU's ids: stable counting sort (numpy's stable argsort)
    flat = ids.ravel()
    counts = np.bincount(flat, minlength=E)
    sp = np.argsort(flat, kind="stable")
    np.testing.assert_array_equal(rb.expert_counts.cpu().numpy(), counts)
    np.testing.assert_array_equal(rb.expert_offsets.cpu().numpy(), np.concatenate([[0], np.cumsum(counts)]))
    np.testing.assert_array_equal(rb.sorted_pair[:P].cpu().numpy(), sp)
    pp = np.empty(P, np.int64)
    pp[sp] = np.arange(P)
    np.testing.assert_array_equal(rb.pair_pos[:P].cpu().numpy(), pp)
    layer.close()


def _check_exact(T, H, E, k, dtype="bf16", seed=0):
    """Inputs on a grid where every partial sum is exact in fp32 whatever the order
    (x, w in {-1, -7/8, ..., 1}, bias in quarters): the GPU's scores must equal the
    oracle's rounded to fp32, and with them the whole routing result (ties included:
    the grid makes equal scores common)."""
    print(f"case route_hidden exact T={T} H={H} E={E} k={k} {dtype}", flush=True)
    layer = _layer(H, E, k, T, dtype)
    rng = np.random.default_rng(seed)
    xf = (rng.integers(-8, 9, size=(T, H)) / 8.0).astype(np.float32)
    wf = (rng.integers(-8, 9, size=(E, H)) / 8.0).astype(np.float32)
    bf = (rng.integers(-16, 17, size=E) / 4.0).astype(np.float32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    x = torch.from_numpy(xf).to(tdt).cuda()
    w = torch.from_numpy(wf).to(tdt).cuda()
    rb = layer.new_route()
    logits = torch.full((max(T, 1), E), float("nan"), dtype=torch.float32, device="cuda")
    layer.route_hidden(x, w, logits, T, rb, bias=torch.from_numpy(bf).cuda())
    torch.cuda.synchronize()
    ref = oracle.router_scores(xf, wf, bf).astype(np.float32)
    np.testing.assert_array_equal(logits[:T].cpu().numpy(), ref)
    P = T * k
    ids_o, gates_o = oracle.route(ref, k)
    counts_o, offsets_o, sp_o, pp_o = oracle.permute(ids_o, E)
    np.testing.assert_array_equal(rb.topk_ids[:P].cpu().numpy(), ids_o.ravel())
    np.testing.assert_allclose(rb.topk_gates[:P].cpu().numpy(), gates_o.ravel(), rtol=0, atol=2e-6)
    np.testing.assert_array_equal(rb.expert_counts.cpu().numpy(), counts_o)
    np.testing.assert_array_equal(rb.expert_offsets.cpu().numpy(), offsets_o)
    np.testing.assert_array_equal(rb.sorted_pair[:P].cpu().numpy(), sp_o)
    np.testing.assert_array_equal(rb.pair_pos[:P].cpu().numpy(), pp_o)
    layer.close()


@pytest.mark.parametrize("T,H,E,k,dtype", [
    (3, 128, 8, 2, "bf16"),
    (45, 384, 20, 4, "bf16"),
    (130, 1024, 128, 8, "bf16"),
    (100, 128, 16, 2, "bf16"),      # one 128-deep stage: the second reduction half is empty
    (200, 384, 40, 4, "bf16"),      # three stages: halves of 2 and 1
    (4096, 7168, 256, 8, "bf16"),   # the fp8 layer's router shape
    (64, 256, 8, 2, "f32"),
])
def test_route_hidden_exact_grid(T, H, E, k, dtype):
    _check_exact(T, H, E, k, dtype, seed=T * 7 + E)


@pytest.mark.parametrize("T,H,E,k", [
    (1, 128, 8, 2),        # one token, fused small route
    (37, 384, 20, 4),      # ragged tokens and experts (not multiples of 16); H/32 % 8 != 0
    (100, 1024, 128, 8),   # multi-launch route path (T > 64)
    (300, 256, 256, 8),
])
def test_route_hidden_bf16(T, H, E, k):
    _check(T, H, E, k, seed=T + E)


def test_route_hidden_without_bias():
    _check(50, 512, 64, 6, seed=3, use_bias=False)


def test_route_hidden_f32():
    _check(64, 256, 8, 2, dtype="f32", seed=4)


def test_route_hidden_dominant_bias():
    """A bias of 1e4 on one expert puts it in slot 0 of every token with gate 1."""
    T, H, E, k = 80, 256, 32, 4
    layer = _layer(H, E, k, T, "bf16")
    x, w, b = _inputs(T, H, E, 9, "bf16", 0.1)
    b[7] = 1e4
    rb = layer.new_route()
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    layer.route_hidden(x.cuda(), w.cuda(), logits, T, rb, bias=b.cuda())
    torch.cuda.synchronize()
    ids = rb.topk_ids[:T * k].cpu().numpy().reshape(T, k)
    gates = rb.topk_gates[:T * k].cpu().numpy().reshape(T, k)
    assert np.all(ids[:, 0] == 7)
    np.testing.assert_allclose(gates[:, 0], 1.0, rtol=0, atol=1e-6)
    layer.close()


def test_route_hidden_deepseek_v3_shape():
    """The fp8 layer's router shape: 4096 tokens, H = 7168, 256 experts, top-8."""
    _check(4096, 7168, 256, 8, seed=5, bias_scale=0.01)
