"""Parity of afd_ffn_route_capacity with the oracle's adaptive token dropper.

The dropper ("MoE 大规模分布式推理工程实战：从 All-to-All 通信到动态专家放置", §4.2) is
integer work on fp32 gates that are copied or halved, so every output is compared
bit-exactly: assign, weight, offsets, the kept tokens grouped by expert, and the adapted
limits.  Preference lists come from the oracle's router on seeded logits (uniform, and
skewed towards a few hot experts), or are seeded random permutations, at capacities from
none at all to room for every token; the cases cover several staging passes (T * k above
4096), chunk tails, k = 32, E = 1024, and a sequence of batches carrying the limits.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_expert_ffn_softmax_amd import AfdError, MoeExpertFFN, afd_ffn_route_capacity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _layer(E, k, T):
    w_gu = torch.zeros((E, 128, 256), dtype=torch.bfloat16, device="cuda")
    w_d = torch.zeros((E, 128, 128), dtype=torch.bfloat16, device="cuda")
    return MoeExpertFFN(hidden=128, inter=128, num_experts=E, top_k=k, max_tokens=max(T, 1), dtype="bf16",
                        w_gate_up=w_gu, w_down=w_d)


def _prefs(T, E, k, seed, kind="router"):
    rng = np.random.default_rng(seed)
    if kind == "perm":
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32).reshape(T, k)
        gates = rng.random((T, k)).astype(np.float32)
        return ids, gates
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if kind == "skewed":
        logits[:, : max(1, E // 16)] += 3.0
    ids, gates = oracle.route(logits, k)
    return ids, gates.astype(np.float32)


def _gpu_call(layer, ids, gates, limits, base, adaptive):
    T = ids.shape[0]
    lim = torch.from_numpy(np.asarray(limits, np.int32).copy()).cuda()
    out = layer.route_capacity(torch.from_numpy(ids).cuda(), torch.from_numpy(gates).cuda(), T, lim, base, adaptive)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out], lim.cpu().numpy()


def _check(got, lim_got, ref, T, E):
    assign, weight, offsets, sorted_token = got
    np.testing.assert_array_equal(assign[:T], ref["assign"])
    np.testing.assert_array_equal(weight[:T].view(np.uint32), ref["weight"].view(np.uint32))
    np.testing.assert_array_equal(offsets, ref["offsets"])
    np.testing.assert_array_equal(sorted_token[: int(offsets[E])], ref["sorted_token"])
    np.testing.assert_array_equal(lim_got, ref["limits"])


@pytest.mark.parametrize("T,E,k,L,kind,seed", [
    (64, 8, 2, 4, "router", 0),          # heavy pressure: fallbacks and drops
    (1000, 16, 4, 50, "router", 1),      # experts fill part-way through
    (4096, 256, 8, 20, "router", 2),     # capacity factor 1.25 over T*1/E
    (4096, 256, 8, 4096, "router", 3),   # room everywhere: top-1, whole chunks commit
    (5000, 128, 8, 1, "router", 4),      # almost everything falls back or drops
    (777, 48, 3, 12, "skewed", 5),       # hot experts fill first
    (3000, 1024, 32, 3, "router", 6),    # k = 32, E = 1024, 24 staging passes
    (300, 1, 1, 100, "perm", 7),         # one expert
    (2049, 64, 8, 40, "perm", 8),        # T*k spans 5 staging passes with a tail
    (130, 5, 5, 0, "perm", 9),           # no capacity: everything dropped
])
@pytest.mark.parametrize("adaptive", [True, False])
def test_capacity_parity(T, E, k, L, kind, seed, adaptive):
    ids, gates = _prefs(T, E, k, seed, kind)
    limits = np.full(E, L, np.int32)
    base = max(1, L // 2)
    ref = oracle.route_capacity(ids, gates, E, limits, base, adaptive)
    got, lim_got = _gpu_call(_layer(E, k, T), ids, gates, limits, base, adaptive)
    _check(got, lim_got, ref, T, E)


def test_capacity_uneven_limits_and_batches():
    """Four batches carrying the adaptive limits on the device, from uneven start
    limits, against the oracle carrying them on the host."""
    E, k, base = 32, 4, 6
    layer = _layer(E, k, 1500)
    rng = np.random.default_rng(11)
    lim_o = rng.integers(0, 60, E).astype(np.int32)
    lim_d = torch.from_numpy(lim_o.copy()).cuda()
    for b, T in enumerate((1500, 200, 0, 900)):
        ids, gates = _prefs(T, E, k, 100 + b, "skewed" if b % 2 else "router")
        ref = oracle.route_capacity(ids, gates, E, lim_o, base, True)
        out = layer.route_capacity(torch.from_numpy(ids).cuda(), torch.from_numpy(gates).cuda(), T, lim_d, base,
                                   True)
        torch.cuda.synchronize()
        _check([o.cpu().numpy() for o in out], lim_d.cpu().numpy(), ref, T, E)
        lim_o = ref["limits"]


def test_capacity_rejects_bad_arguments():
    E, k, T = 8, 2, 16
    layer = _layer(E, k, T)
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    gates = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    lim = torch.zeros(E, dtype=torch.int32, device="cuda")
    a = torch.zeros(T, dtype=torch.int32, device="cuda")
    w = torch.zeros(T, dtype=torch.float32, device="cuda")
    off = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    st = torch.zeros(T, dtype=torch.int32, device="cuda")
    h = layer.handle
    bad = [
        (ids, gates, T + 1, 1, lim, a, w, off, st),              # T above max_tokens
        (ids, gates, T, -1, lim, a, w, off, st),                 # negative base
        (None, gates, T, 1, lim, a, w, off, st),                 # NULL input
        (ids, gates, T, 1, None, a, w, off, st),                 # NULL limits
        (ids, gates, T, 1, lim, a, a, off, st),                  # weight overlaps assign
        (ids, gates, T, 1, lim, a, w, off, ids),                 # output overlaps an input
        (ids, gates, T, 1, lim, a, w, off, st.data_ptr() + 2),   # misaligned
    ]
    for args in bad:
        with pytest.raises(AfdError):
            afd_ffn_route_capacity(h, *args[:4], True, *args[4:])
    afd_ffn_route_capacity(h, ids, gates, T, 1, True, lim, a, w, off, st)   # the good call still works
    torch.cuda.synchronize()


FFN_TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


@pytest.mark.parametrize("dtype,T,H,M,E,k,Ms,L,kernel", [
    ("bf16", 200, 256, 256, 16, 4, 0, 9, "stream"),     # some fallbacks at half gate
    ("bf16", 700, 384, 256, 8, 2, 128, 60, "tiled"),    # drops, shared expert for every token
    ("fp8", 300, 256, 256, 12, 3, 128, 20, "auto"),
    ("f32", 150, 128, 128, 6, 2, 0, 12, "auto"),
    ("bf16", 64, 128, 128, 4, 2, 128, 0, "auto"),       # every token dropped: shared expert only
])
def test_forward_on_capacity_route(dtype, T, H, M, E, k, Ms, L, kernel):
    """Capacity routing, then the expert FFN on its result, against the oracle layer on
    the oracle dropper's assignment: y[t] = weight[t] FFN_assign[t](x[t]) (+ shared)."""
    import workloads
    w = workloads.Workload(f"cap_{dtype}_T{T}", 700 + T, T=T, H=H, M=M, E=E, k=k, Ms=Ms, dtype=dtype)
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = MoeExpertFFN(hidden=H, inter=M, num_experts=E, top_k=k, max_tokens=T, dtype=dtype,
                         w_gate_up=weights["w_gu"], w_down=weights["w_d"], s_gate_up=weights["s_gu"],
                         s_down=weights["s_d"], shared_inter=Ms, ws_gate_up=weights["ws_gu"],
                         ws_down=weights["ws_d"], ss_gate_up=weights["ss_gu"], ss_down=weights["ss_d"])
    layer.set_gemm_kernel(kernel)
    ids, gates = oracle.route(logits.cpu().numpy(), k)
    gates = gates.astype(np.float32)
    limits = np.full(E, L, np.int32)
    ref = oracle.route_capacity(ids, gates, E, limits, 1, False)
    cap = layer.route_capacity(torch.from_numpy(ids).cuda(), torch.from_numpy(gates).cuda(), T,
                               torch.from_numpy(limits).cuda(), 1, False)
    rb = layer.new_route()
    layer.route_from_capacity(cap, T, rb)
    ydt = torch.float32 if dtype == "f32" else torch.bfloat16
    y = torch.full((T, H), float("nan"), dtype=ydt, device="cuda")
    layer.forward(x, T, rb, y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cap[0].cpu().numpy()[:T], ref["assign"])
    kept = int(ref["offsets"][E])
    np.testing.assert_array_equal(rb.expert_offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(rb.sorted_pair[:kept].cpu().numpy(), ref["sorted_token"] * k)
    yref, _ = oracle.layer_assigned(x.float().cpu().numpy(), ref["assign"], ref["weight"], H=H, M=M, E=E,
                                    dtype=dtype, w_gu=weights["w_gu"], w_d=weights["w_d"], s_gu=weights["s_gu"],
                                    s_d=weights["s_d"], Ms=Ms, ws_gu=weights["ws_gu"], ws_d=weights["ws_d"],
                                    ss_gu=weights["ss_gu"], ss_d=weights["ss_d"])
    yg = y.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(yg).all()
    dropped = ref["assign"] < 0
    if Ms == 0:
        assert (yg[dropped] == 0).all()
    scale = max(np.abs(yref).max(), 1e-30)
    err = np.abs(yg - yref).max()
    print(f"  kept {kept}/{T}, max|err|/max|ref| = {err / scale:.3e}", flush=True)
    assert err <= FFN_TOL[dtype] * scale
    layer.close()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_capacity_route_and_forward_in_a_graph(dtype):
    """route -> capacity routing -> route from capacity -> forward captured in one HIP
    graph: every replay, with eager work and synchronisations in between, reproduces the
    eager result bit for bit (the capacity calls allocate and clear nothing)."""
    import workloads
    T, H, M, E, k, Ms, L = 240, 256, 256, 16, 4, 128 if dtype == "fp8" else 0, 8
    w = workloads.Workload(f"capgraph_{dtype}", 760, T=T, H=H, M=M, E=E, k=k, Ms=Ms, dtype=dtype)
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = MoeExpertFFN(hidden=H, inter=M, num_experts=E, top_k=k, max_tokens=T, dtype=dtype,
                         w_gate_up=weights["w_gu"], w_down=weights["w_d"], s_gate_up=weights["s_gu"],
                         s_down=weights["s_d"], shared_inter=Ms, ws_gate_up=weights["ws_gu"],
                         ws_down=weights["ws_d"], ss_gate_up=weights["ss_gu"], ss_down=weights["ss_d"])
    limits = torch.full((E,), L, dtype=torch.int32, device="cuda")
    rb_top, rb = layer.new_route(), layer.new_route()
    cap = (torch.empty(T, dtype=torch.int32, device="cuda"), torch.empty(T, device="cuda"),
           torch.empty(E + 1, dtype=torch.int32, device="cuda"), torch.empty(T, dtype=torch.int32, device="cuda"))
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def step(s=None):
        layer.route(logits, T, rb_top, stream=s)
        layer.route_capacity(rb_top.topk_ids[: T * k], rb_top.topk_gates[: T * k], T, limits, 1, False, out=cap,
                             stream=s)
        layer.route_from_capacity(cap, T, rb, stream=s)
        layer.forward(x, T, rb, y, stream=s)

    step()
    torch.cuda.synchronize()
    y_e, a_e, st_e = y.clone(), cap[0].clone(), cap[3].clone()
    assert int(cap[2][E]) < T    # 16 experts x at most 12 tokens (1.5 x 8) < 240: some tokens are dropped
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step(s)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            step(s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        y.zero_()
        cap[0].fill_(-7)
        cap[3].fill_(-7)
        layer.route(logits.flip(0), T, rb_top)      # unrelated eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_e), f"replay {rep}: output differs from the eager run"
        assert torch.equal(cap[0], a_e) and torch.equal(cap[3][: int(cap[2][E])], st_e[: int(cap[2][E])])
    layer.close()
