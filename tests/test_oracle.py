"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks one oracle function against something other than its own formula:
a library routine (numpy's stable argsort, numpy float64 matmuls, torch's e4m3 cast),
a closed form derived by hand (tests/golden/*.txt), a brute-force enumeration, or an
invariant of the method (bijection, gate sums, k = E mixture, token-order
equivariance, the 6*H*M FLOPs per token-expert pair of the AFD article's §2.1).
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [c.strip() for c in line.split("|")]


# ----------------------------------------------------------------------------- routing
@pytest.mark.parametrize("T,E,k,seed", [(50, 8, 2, 0), (40, 128, 8, 1), (30, 256, 8, 2), (20, 48, 3, 3),
                                        (10, 5, 5, 4), (16, 1, 1, 5)])
def test_route_ids_match_stable_argsort(T, E, k, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.route(logits, k)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(ids, ref)


def test_route_ids_bruteforce_with_ties():
    """Integer logits in [-2, 2] force many ties.  Brute force: the selected set is the
    lexicographically first among the k-subsets with the largest logit sum, and the
    slots order it by (logit desc, index asc)."""
    rng = np.random.default_rng(7)
    for E in (2, 3, 5, 8):
        for k in range(1, E + 1):
            logits = rng.integers(-2, 3, size=(40, E)).astype(np.float32)
            ids, gates = oracle.route(logits, k)
            for t in range(logits.shape[0]):
                l = logits[t].astype(np.int64)
                best = max(itertools.combinations(range(E), k), key=lambda s: (sum(l[list(s)]), [-i for i in s]))
                slots = sorted(best, key=lambda i: (-l[i], i))
                assert list(ids[t]) == slots
                # equal logits -> equal gates
                for a in range(k):
                    for b in range(k):
                        if l[slots[a]] == l[slots[b]]:
                            assert gates[t, a] == gates[t, b]


def test_route_golden_cases():
    for name, k, logits, ids, gates, tol in _rows("route_cases.txt"):
        lg = np.array([float(v) for v in logits.split(",")], np.float32)[None, :]
        got_ids, got_g = oracle.route(lg, int(k))
        assert list(got_ids[0]) == [int(v) for v in ids.split(",")], name
        np.testing.assert_allclose(got_g[0], [float(v) for v in gates.split(",")], rtol=0, atol=float(tol),
                                   err_msg=name)


@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (256, 8), (48, 3)])
def test_gates_renormalised_and_equal_to_softmax_of_selected(E, k):
    """The page's router takes the top-k logits and then a softmax over those k; the
    workload definition takes a softmax over all E, then top-k, then renormalises.
    Both are exp(l_j) / sum_selected exp(l_i) in exact arithmetic."""
    rng = np.random.default_rng(E * 31 + k)
    logits = (rng.standard_normal((64, E)) * 3).astype(np.float32)
    ids, gates = oracle.route(logits, k)
    np.testing.assert_allclose(gates.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(gates, axis=1) <= 0)
    sel = np.take_along_axis(logits.astype(np.float64), ids, axis=1)
    p = np.exp(sel - sel.max(axis=1, keepdims=True))
    np.testing.assert_allclose(gates, p / p.sum(axis=1, keepdims=True), rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------- router projection
def _mat(text):
    return np.array([[float(v) for v in row.split(",")] for row in text.split(";")], np.float32)


def test_router_scores_golden_cases():
    for name, k, x, w, bias, scores, ids, gates, tol in _rows("router_proj_cases.txt"):
        b = None if bias == "-" else _mat(bias)[0]
        got = oracle.router_scores(_mat(x), _mat(w), b)
        np.testing.assert_array_equal(got, _mat(scores).astype(np.float64), err_msg=name)
        got_ids, got_g = oracle.route(got.astype(np.float32), int(k))
        np.testing.assert_array_equal(got_ids, _mat(ids).astype(np.int32), err_msg=name)
        np.testing.assert_allclose(got_g, _mat(gates).astype(np.float64), rtol=0, atol=float(tol), err_msg=name)


def test_router_scores_one_hot_gate_vectors_pick_columns():
    """Gate vector of expert e = unit vector of channel perm[e]: the score is that
    channel of x plus the bias, exactly."""
    rng = np.random.default_rng(11)
    T, H, E = 9, 40, 24
    x = rng.standard_normal((T, H)).astype(np.float32)
    perm = rng.permutation(H)[:E]
    w = np.zeros((E, H), np.float32)
    w[np.arange(E), perm] = 1.0
    bias = rng.standard_normal(E).astype(np.float32)
    got = oracle.router_scores(x, w, bias)
    np.testing.assert_array_equal(got, x[:, perm].astype(np.float64) + bias.astype(np.float64))


def test_router_scores_integer_inputs_exact():
    """Small integers: every sum is exact in double, so the scores equal numpy's int64
    matrix product (a library routine) plus the bias."""
    rng = np.random.default_rng(12)
    for T, H, E in ((1, 128, 8), (7, 384, 20), (33, 1024, 256)):
        x = rng.integers(-8, 9, size=(T, H))
        w = rng.integers(-8, 9, size=(E, H))
        bias = rng.integers(-50, 51, size=E)
        got = oracle.router_scores(x.astype(np.float32), w.astype(np.float32), bias.astype(np.float32))
        np.testing.assert_array_equal(got, (x @ w.T + bias[None, :]).astype(np.float64))


def test_router_bias_shift_invariance_and_dominant_bias():
    """Adding one constant to every expert's bias changes neither the selection nor the
    gates (softmax over the selected scores); a dominant bias puts its expert in slot 0
    of every token with a gate of 1 to double precision."""
    rng = np.random.default_rng(13)
    T, H, E, k = 20, 64, 16, 4
    x = rng.integers(-4, 5, size=(T, H)).astype(np.float32)
    w = rng.integers(-4, 5, size=(E, H)).astype(np.float32)
    bias = rng.integers(-3, 4, size=E).astype(np.float32)
    ids0, g0 = oracle.route(oracle.router_scores(x, w, bias).astype(np.float32), k)
    ids1, g1 = oracle.route(oracle.router_scores(x, w, bias + 64.0).astype(np.float32), k)
    np.testing.assert_array_equal(ids0, ids1)
    np.testing.assert_allclose(g0, g1, rtol=0, atol=1e-12)
    forced = bias.copy()
    forced[5] = 1e4
    ids2, g2 = oracle.route(oracle.router_scores(x, w, forced).astype(np.float32), k)
    assert np.all(ids2[:, 0] == 5)
    np.testing.assert_allclose(g2[:, 0], 1.0, rtol=0, atol=1e-12)


def test_route_select_bias_closed_form_cases():
    """Selection on score + bias, gates from the unbiased scores, against values worked
    out by hand: the bias of expert 0 lifts it into the chosen pair, but its gate is
    that of its own score 0 against expert 3's score 3."""
    s = np.array([[0.0, 1.0, 2.0, 3.0]], np.float32)
    b = np.array([5.0, 0.0, 0.0, 0.0], np.float32)
    ids, g = oracle.route_select_bias(s, b, 2)
    np.testing.assert_array_equal(ids, [[0, 3]])
    e3 = math.exp(3.0)
    np.testing.assert_allclose(g, [[1.0 / (1.0 + e3), e3 / (1.0 + e3)]], rtol=0, atol=1e-15)
    # the same choice with the bias inside the gates gives other weights: softmax(5, 3)
    ids_in, g_in = oracle.route((s + b).astype(np.float32), 2)
    np.testing.assert_array_equal(ids_in, ids)
    e2 = math.exp(2.0)
    np.testing.assert_allclose(g_in, [[e2 / (1.0 + e2), 1.0 / (1.0 + e2)]], rtol=0, atol=1e-15)
    # equal keys (1.0 + 0.0 and 0.5 + 0.5): the lower expert takes slot 0; gates from 1.0 and 0.5
    ids, g = oracle.route_select_bias(np.array([[1.0, 0.5]], np.float32), np.array([0.0, 0.5], np.float32), 2)
    np.testing.assert_array_equal(ids, [[0, 1]])
    q = math.exp(0.5)
    np.testing.assert_allclose(g, [[q / (q + 1.0), 1.0 / (q + 1.0)]], rtol=0, atol=1e-15)
    # k = 1: the gate is exactly 1 whatever the scores
    ids, g = oracle.route_select_bias(s, b, 1)
    assert ids[0, 0] == 0 and g[0, 0] == 1.0


def test_route_select_bias_key_is_decided_in_fp32():
    """1 + 2^-25 is 1 in fp32: the two keys tie after rounding and the lower expert
    wins, although the exact sums would put expert 1 first."""
    s = np.array([[1.0, 1.0, -1.0]], np.float32)
    b = np.array([0.0, 2.0 ** -25, 0.0], np.float32)
    assert np.float32(s[0, 1]) + np.float32(b[1]) == np.float32(1.0)
    ids, _ = oracle.route_select_bias(s, b, 2)
    np.testing.assert_array_equal(ids, [[0, 1]])
    b[1] = 2.0 ** -22  # now representable above 1: expert 1 first
    ids, _ = oracle.route_select_bias(s, b, 2)
    np.testing.assert_array_equal(ids, [[1, 0]])


@pytest.mark.parametrize("E,k,seed", [(8, 2, 0), (128, 8, 1), (256, 8, 2)])
def test_route_select_bias_reductions_and_forced_set(E, k, seed):
    """Zero bias reproduces the plain router; a bias of +16 on k chosen experts (scores
    are N(0, 1)) forces exactly that set, with the gates the plain router gives when
    only those k experts exist; gates are positive and sum to one.  Rounding is
    monotone, so with no two chosen keys equal the key order is the score order."""
    rng = np.random.default_rng(seed)
    T = 40
    s = rng.standard_normal((T, E)).astype(np.float32)
    ids0, g0 = oracle.route(s, k)
    ids1, g1 = oracle.route_select_bias(s, np.zeros(E, np.float32), k)
    np.testing.assert_array_equal(ids0, ids1)
    np.testing.assert_allclose(g0, g1, rtol=0, atol=1e-15)
    chosen = rng.choice(E, size=k, replace=False)
    b = np.zeros(E, np.float32)
    b[chosen] = 16.0
    keys = (s[:, chosen] + np.float32(16.0)).astype(np.float32)
    assert all(len(set(r.tolist())) == k for r in keys)
    assert keys.min() > (s + b).max(initial=-np.inf, where=(b == 0)[None, :])
    ids, g = oracle.route_select_bias(s, b, k)
    sub_ids, sub_g = oracle.route(np.ascontiguousarray(s[:, chosen]), k)
    np.testing.assert_array_equal(ids, chosen[sub_ids])
    np.testing.assert_allclose(g, sub_g, rtol=0, atol=1e-12)
    assert np.all(g > 0)
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- permute
@pytest.mark.parametrize("T,E,k,seed", [(64, 8, 2, 0), (6, 128, 8, 1), (300, 256, 8, 2), (1, 4, 4, 3), (0, 8, 2, 4)])
def test_permute_is_stable_counting_sort(T, E, k, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.route(logits, k) if T else (np.zeros((0, k), np.int32), None)
    counts, offsets, sp, pp = oracle.permute(ids, E)
    np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    assert counts.sum() == T * k and offsets[-1] == T * k and offsets[0] == 0
    np.testing.assert_array_equal(np.diff(offsets), counts)
    np.testing.assert_array_equal(sp, np.argsort(ids.ravel(), kind="stable"))
    np.testing.assert_array_equal(np.sort(sp), np.arange(T * k))          # bijection
    np.testing.assert_array_equal(pp[sp], np.arange(T * k))                # inverse
    flat = ids.ravel()
    for e in range(E):                                                      # segments
        seg = sp[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


# ----------------------------------------------------------------------------- expert FFN
def _silu(z):
    return z / (1.0 + np.exp(-z))


def _dense_swiglu(x, wgu, wd):
    M = wd.shape[0]
    a = x @ wgu
    return (_silu(a[:, :M]) * a[:, M:]) @ wd


def _to_np64(t):
    return t.detach().to(torch.float64).cpu().numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_expert_equals_dense_swiglu(dtype):
    """E = 1, k = 1: every token goes to the one expert with gate 1, so the layer is a
    dense SwiGLU FFN; numpy float64 matmuls are the reference."""
    H, M, T = 64, 96, 12
    g = torch.Generator().manual_seed(11)
    wgu = torch.randn(1, H, 2 * M, generator=g) / math.sqrt(H)
    wd = torch.randn(1, M, H, generator=g) / math.sqrt(M)
    x = torch.randn(T, H, generator=g)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    wgu, wd, x = wgu.to(tdt), wd.to(tdt), x.to(tdt)
    logits = np.zeros((T, 1), np.float32)
    ids, gates, y, macs = oracle.layer(x.float().numpy(), logits, H=H, M=M, E=1, k=1, dtype=dtype,
                                       w_gu=[wgu[0]], w_d=[wd[0]])
    ref = _dense_swiglu(_to_np64(x), _to_np64(wgu[0]), _to_np64(wd[0]))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    assert np.all(gates == 1.0) and np.all(ids == 0)
    assert 2 * macs == 6 * T * 1 * H * M


def test_gate_up_split_and_down_orientation():
    """Gate columns [0, M) go through SiLU, up columns [M, 2M) do not; W_down is
    [M, H].  Swapping the halves or transposing W_down changes y, so the dense
    reference above fails on either mistake; this checks it does on this data."""
    H, M, T = 32, 48, 5
    rng = np.random.default_rng(3)
    wgu = rng.standard_normal((H, 2 * M)).astype(np.float32) / math.sqrt(H)
    wd = rng.standard_normal((M, H)).astype(np.float32) / math.sqrt(M)
    x = rng.standard_normal((T, H)).astype(np.float32)
    _, _, y, _ = oracle.layer(x, np.zeros((T, 1), np.float32), H=H, M=M, E=1, k=1, dtype="f32",
                              w_gu=[wgu], w_d=[wd])
    swapped = np.concatenate([wgu[:, M:], wgu[:, :M]], axis=1).astype(np.float64)
    assert np.abs(y - _dense_swiglu(x.astype(np.float64), swapped, wd.astype(np.float64))).max() > 1e-3
    np.testing.assert_allclose(y, _dense_swiglu(x.astype(np.float64), wgu.astype(np.float64), wd.astype(np.float64)),
                               rtol=1e-12, atol=1e-12)


def test_diagonal_weights_closed_form():
    """H = M with W_gate = a_e I, W_up = b_e I, W_down = c_e I gives, per channel,
    y_i = sum_j g_j c_e SiLU(a_e x_i) b_e x_i (e = expert of slot j)."""
    H = M = 16
    E, k, T = 4, 2, 9
    a = [0.5, -1.25, 2.0, 0.75]
    b = [1.5, 0.25, -0.5, 1.0]
    c = [2.0, -1.0, 0.5, 3.0]
    wgu = [np.concatenate([a[e] * np.eye(H), b[e] * np.eye(H)], axis=1).astype(np.float32) for e in range(E)]
    wd = [(c[e] * np.eye(M)).astype(np.float32) for e in range(E)]
    rng = np.random.default_rng(5)
    x = rng.standard_normal((T, H)).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, gates, y, _ = oracle.layer(x, logits, H=H, M=M, E=E, k=k, dtype="f32", w_gu=wgu, w_d=wd)
    for t in range(T):
        for i in range(H):
            xi = float(x[t, i])
            ref = 0.0
            for j in range(k):
                e = ids[t, j]
                z = a[e] * xi
                ref += gates[t, j] * c[e] * (z / (1.0 + math.exp(-z))) * b[e] * xi
            assert abs(y[t, i] - ref) <= 1e-13 * max(1.0, abs(ref))


def test_k_equals_E_is_dense_softmax_mixture():
    """With k = E renormalisation is the identity: y = sum_e softmax(l)_e FFN_e(x)."""
    H, M, E, T = 32, 32, 4, 6
    rng = np.random.default_rng(9)
    wgu = [rng.standard_normal((H, 2 * M)).astype(np.float32) / math.sqrt(H) for _ in range(E)]
    wd = [rng.standard_normal((M, H)).astype(np.float32) / math.sqrt(M) for _ in range(E)]
    x = rng.standard_normal((T, H)).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    _, _, y, _ = oracle.layer(x, logits, H=H, M=M, E=E, k=E, dtype="f32", w_gu=wgu, w_d=wd)
    l64 = logits.astype(np.float64)
    p = np.exp(l64 - l64.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = sum(p[:, e:e + 1] * _dense_swiglu(x.astype(np.float64), wgu[e].astype(np.float64),
                                            wd[e].astype(np.float64)) for e in range(E))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_token_order_equivariance_and_shared_expert():
    """Permuting the token order of (x, logits) permutes y; the shared expert adds a
    dense SwiGLU FFN with gate 1."""
    H, M, Ms, E, k, T = 32, 64, 48, 6, 2, 10
    rng = np.random.default_rng(13)
    wgu = [rng.standard_normal((H, 2 * M)).astype(np.float32) / math.sqrt(H) for _ in range(E)]
    wd = [rng.standard_normal((M, H)).astype(np.float32) / math.sqrt(M) for _ in range(E)]
    sgu = rng.standard_normal((H, 2 * Ms)).astype(np.float32) / math.sqrt(H)
    sd = rng.standard_normal((Ms, H)).astype(np.float32) / math.sqrt(Ms)
    x = rng.standard_normal((T, H)).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    kw = dict(H=H, M=M, E=E, k=k, dtype="f32", w_gu=wgu, w_d=wd)
    _, _, y0, m0 = oracle.layer(x, logits, **kw)
    _, _, y1, m1 = oracle.layer(x, logits, Ms=Ms, ws_gu=sgu, ws_d=sd, **kw)
    shared = _dense_swiglu(x.astype(np.float64), sgu.astype(np.float64), sd.astype(np.float64))
    np.testing.assert_allclose(y1, y0 + shared, rtol=1e-12, atol=1e-12)
    assert 2 * m1 == 6 * T * k * H * M + 6 * T * H * Ms
    perm = rng.permutation(T)
    _, _, yp, _ = oracle.layer(x[perm], logits[perm], Ms=Ms, ws_gu=sgu, ws_d=sd, **kw)
    np.testing.assert_array_equal(yp, y1[perm])


def test_mac_count_matches_work_model():
    """The oracle's loop-counted multiply-adds times 2 equal the 6*T*k*H*M (+6*T*H*Ms)
    FLOPs of the work model; the fixture also holds the model's values for the five
    workloads and the 3M/dtype_size intensity."""
    rows = list(_rows("work_model.txt"))
    for name, T, H, M, k, Ms, flops in [r for r in rows if r[0] != "ai"]:
        T, H, M, k, Ms, flops = map(int, (T, H, M, k, Ms, flops))
        assert 6 * T * k * H * M + 6 * T * H * Ms == flops, name
    for _, M, dsz, ai in [r for r in rows if r[0] == "ai"]:
        B, H = 7, 64
        assert (6 * B * H * int(M)) / (2 * B * H * int(dsz)) == int(ai)
    H, M, E, k, T, Ms = 64, 128, 5, 3, 7, 128
    rng = np.random.default_rng(1)
    wgu = [rng.standard_normal((H, 2 * M)).astype(np.float32) for _ in range(E)]
    wd = [rng.standard_normal((M, H)).astype(np.float32) for _ in range(E)]
    sgu = rng.standard_normal((H, 2 * Ms)).astype(np.float32)
    sd = rng.standard_normal((Ms, H)).astype(np.float32)
    _, _, _, macs = oracle.layer(rng.standard_normal((T, H)).astype(np.float32),
                                 rng.standard_normal((T, E)).astype(np.float32), H=H, M=M, E=E, k=k, dtype="f32",
                                 w_gu=wgu, w_d=wd, Ms=Ms, ws_gu=sgu, ws_d=sd)
    assert 2 * macs == 6 * T * k * H * M + 6 * T * H * Ms


# ----------------------------------------------------------------------------- fp8
def test_fp8_decode_every_code_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.fp8_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert oracle.fp8_decode(0x7E) == 448.0 and oracle.fp8_decode(0x38) == 1.0
    assert oracle.fp8_decode(0x08) == 2.0 ** -6 and oracle.fp8_decode(0x01) == 2.0 ** -9


def test_fp8_encode_matches_torch_cast_including_ties():
    rng = np.random.default_rng(2)
    vals = list((rng.standard_normal(3000) * rng.choice([1e-3, 0.1, 1, 30, 200], 3000)).astype(np.float32))
    finite = [oracle.fp8_decode(c) for c in range(127)]
    vals += [np.float32(0.5 * (finite[i] + finite[i + 1])) for i in range(126)]   # exact midpoints
    vals += [np.float32(-v) for v in vals[-126:]] + [np.float32(448.0), np.float32(-0.0)]
    v = np.array(vals, np.float32)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.fp8_encode(float(a)) for a in v], np.uint8)
    np.testing.assert_array_equal(got, ref)
    for c in range(127):                                                         # round trip
        assert oracle.fp8_encode(oracle.fp8_decode(c)) == c
    assert oracle.fp8_encode(1000.0) == 0x7E and oracle.fp8_encode(-1000.0) == 0xFE


def test_fp8_row_quant_against_torch():
    """Per-128 quantisation: scale = amax/448 (fp32), codes = RNE(v/scale) (fp32);
    torch's fp32 ops and e4m3 cast are the reference.  Dequantisation error is at most
    half an e4m3 step times the scale."""
    rng = np.random.default_rng(4)
    v = (rng.standard_normal(512) * np.repeat([0.01, 1.0, 50.0, 0.0], 128)).astype(np.float32)
    codes, scales, deq = oracle.quant_row_fp8(v)
    tv = torch.from_numpy(v).view(4, 128)
    amax = tv.abs().amax(dim=1)
    ts = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    tq = (tv / ts[:, None]).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(scales, ts.numpy())
    np.testing.assert_array_equal(codes, tq.view(torch.uint8).numpy().ravel())
    np.testing.assert_array_equal(deq, (tq.to(torch.float64) * ts[:, None].double()).numpy().ravel())
    for g in range(4):
        seg = v[g * 128:(g + 1) * 128].astype(np.float64)
        err = np.abs(deq[g * 128:(g + 1) * 128] - seg)
        step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(seg) / scales[g], 2.0 ** -6))) - 3), 2.0 ** -9)
        assert np.all(err <= 0.5 * step * scales[g] * (1 + 1e-12))


def test_fp8_layer_equals_dequantised_reference():
    """fp8 weights: W = code * block scale; activations x and h are quantised per 128
    channels before each product.  Reference: torch's e4m3 decode and cast with numpy
    float64 matmuls."""
    H, M, T = 256, 128, 4
    g = torch.Generator().manual_seed(21)
    w = [torch.randn(H, 2 * M, generator=g) / math.sqrt(H), torch.randn(M, H, generator=g) / math.sqrt(M)]
    qs = []
    for m in w:
        R, C = m.shape
        blk = m.view(R // 128, 128, C // 128, 128)
        s = blk.abs().amax(dim=(1, 3)) / 448.0
        q = (blk / s[:, None, :, None]).to(torch.float8_e4m3fn).view(R, C)
        qs.append((q, s))
    x = torch.randn(T, H, generator=g).to(torch.bfloat16).float()
    _, _, y, _ = oracle.layer(x.numpy(), np.zeros((T, 1), np.float32), H=H, M=M, E=1, k=1, dtype="fp8",
                              w_gu=[qs[0][0]], w_d=[qs[1][0]], s_gu=[qs[0][1]], s_d=[qs[1][1]])

    def deq_w(q, s):
        R, C = q.shape
        return (q.to(torch.float64).view(R // 128, 128, C // 128, 128) * s.double()[:, None, :, None]).view(R, C)

    def quant_act(a32):
        n = a32.shape[1]
        blk = a32.view(a32.shape[0], n // 128, 128)
        amax = blk.abs().amax(dim=2)
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (blk / s[..., None]).to(torch.float8_e4m3fn)
        return (q.to(torch.float64) * s.double()[..., None]).view(a32.shape[0], n)

    a = quant_act(x) @ deq_w(*qs[0])
    h = torch.nn.functional.silu(a[:, :M]) * a[:, M:]
    ref = quant_act(h.float()) @ deq_w(*qs[1])
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-9, atol=1e-9)


def _fp8_blocks(m):
    """e4m3 codes and fp32 128x128 block scales (amax / 448) of a float32 matrix."""
    R, C = m.shape
    blk = m.view(R // 128, 128, C // 128, 128)
    s = (blk.abs().amax(dim=(1, 3)) / 448.0).float()
    q = (blk / s[:, None, :, None]).to(torch.float8_e4m3fn).view(R, C)
    return q, s


def _fp8_deq(q, s):
    R, C = q.shape
    return (q.to(torch.float64).view(R // 128, 128, C // 128, 128) * s.double()[:, None, :, None]).view(R, C)


def _fp8_quant_act(a32):
    """Activations quantised per row and per 128 channels (scale amax / 448, 1 for an
    all-zero group; code = e4m3 of the fp32 quotient), returned dequantised in float64."""
    n = a32.shape[1]
    blk = a32.view(a32.shape[0], n // 128, 128)
    amax = blk.abs().amax(dim=2)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (blk / s[..., None]).to(torch.float8_e4m3fn)
    return (q.to(torch.float64) * s.double()[..., None]).view(a32.shape[0], n)


def _fp8_ffn(xf32, wgu, wd, M):
    a = _fp8_quant_act(xf32) @ wgu
    h = torch.nn.functional.silu(a[:, :M]) * a[:, M:]
    return _fp8_quant_act(h.float()) @ wd


def test_fp8_layer_several_experts_and_shared_equals_dequantised_reference():
    """The fp8 layer as the DeepSeek-V3-like workload runs it: several experts with
    block scales of their own, k = 2 with non-trivial gates, an intermediate size of two
    scale blocks (gate blocks 0-1, up blocks 2-3 of [H, 2M]) and a block-scaled shared
    expert.  Reference: per-expert dequantisation with torch's e4m3 decode, numpy
    argsort routing, softmax gates over the chosen logits and float64 matmuls.

    The experts' weight magnitudes differ by factors of 2.5-6, so their block scales do:
    reading expert 0's scales for every expert, giving the shared expert a routed
    expert's scales, splitting gate and up at the wrong block or dropping the shared
    term each move the result far outside the bar (checked below on the reference
    itself, so that an oracle making any of these mistakes would fail this pin)."""
    H, M, E, k, Ms, T = 256, 256, 3, 2, 128, 9
    g = torch.Generator().manual_seed(33)
    mags = [1.0, 2.5, 0.4]
    wgu = [_fp8_blocks(torch.randn(H, 2 * M, generator=g) * mags[e] / math.sqrt(H)) for e in range(E)]
    wd = [_fp8_blocks(torch.randn(M, H, generator=g) * mags[e] / math.sqrt(M)) for e in range(E)]
    sgu = _fp8_blocks(torch.randn(H, 2 * Ms, generator=g) * 1.6 / math.sqrt(H))
    sd = _fp8_blocks(torch.randn(Ms, H, generator=g) * 1.6 / math.sqrt(Ms))
    for e in range(E):  # the block scales of one matrix differ between its blocks too
        assert not torch.equal(wgu[e][1][0], wgu[e][1][1])
    x = torch.randn(T, H, generator=g).to(torch.bfloat16).float()
    logits = torch.randn(T, E, generator=g).float().numpy()
    ids, gates, y, _ = oracle.layer(x.numpy(), logits, H=H, M=M, E=E, k=k, dtype="fp8",
                                    w_gu=[q for q, _ in wgu], w_d=[q for q, _ in wd],
                                    s_gu=[s for _, s in wgu], s_d=[s for _, s in wd], Ms=Ms,
                                    ws_gu=sgu[0], ws_d=sd[0], ss_gu=sgu[1], ss_d=sd[1])

    ref_ids = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(ids, ref_ids)
    sel = np.take_along_axis(logits.astype(np.float64), ref_ids, axis=1)
    ref_g = np.exp(sel - sel.max(axis=1, keepdims=True))
    ref_g /= ref_g.sum(axis=1, keepdims=True)
    assert len(set(ref_ids[:, 0])) == E, "every expert is some token's first choice"

    def reference(scale_of, shared_scales, interleave=False, shared=True):
        deq_gu = [_fp8_deq(wgu[e][0], scale_of(e, "gu")) for e in range(E)]
        if interleave:  # gate = column blocks 0 and 2, up = blocks 1 and 3
            order = torch.cat([torch.arange(0, 128), torch.arange(256, 384), torch.arange(128, 256),
                               torch.arange(384, 512)])
            deq_gu = [d[:, order] for d in deq_gu]
        deq_d = [_fp8_deq(wd[e][0], scale_of(e, "d")) for e in range(E)]
        out = np.zeros((T, H))
        for t in range(T):
            for j in range(k):
                e = int(ref_ids[t, j])
                o = _fp8_ffn(x[t:t + 1], deq_gu[e], deq_d[e], M)[0].numpy()
                out[t] += ref_g[t, j] * o
        if shared:
            out += _fp8_ffn(x, _fp8_deq(sgu[0], shared_scales[0]), _fp8_deq(sd[0], shared_scales[1]),
                            Ms).numpy()
        return out

    own = {"gu": lambda e: wgu[e][1], "d": lambda e: wd[e][1]}
    ref = reference(lambda e, m: own[m](e), (sgu[1], sd[1]))
    np.testing.assert_allclose(y, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())

    bar = 6e-2 * np.abs(ref).max()   # the fp8 layer's parity bar
    wrong = {
        "expert 0's scales for every expert": reference(lambda e, m: own[m](0), (sgu[1], sd[1])),
        "routed scales for the shared expert": reference(lambda e, m: own[m](e), (wgu[0][1][:, :2], wd[0][1][:1])),
        "gate and up split per 128-column block": reference(lambda e, m: own[m](e), (sgu[1], sd[1]),
                                                            interleave=True),
        "no shared expert": reference(lambda e, m: own[m](e), (sgu[1], sd[1]), shared=False),
    }
    for what, bad in wrong.items():
        assert np.abs(bad - ref).max() > 3 * bar, (what, np.abs(bad - ref).max() / bar)


# ----------------------------------------------------------------------------- capacity-aware routing
def _capacity_check_lists(r, E):
    """counts/offsets/sorted_token are a stable counting sort of the routed tokens."""
    a = r["assign"]
    routed = np.nonzero(a >= 0)[0]
    assert np.array_equal(r["counts"], np.bincount(a[routed], minlength=E).astype(np.int32))
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(r["counts"])]).astype(np.int32))
    order = routed[np.argsort(a[routed], kind="stable")]
    assert np.array_equal(r["sorted_token"], order.astype(np.int32))


def test_capacity_golden_cases():
    n = 0
    for name, E, k, base, adaptive, limits, ids, gates, assign, weight, after in _rows("capacity_cases.txt"):
        E, k = int(E), int(k)
        ids = np.array([[int(v) for v in tok.split(",")] for tok in ids.split(";")], np.int32)
        gates = np.array([[float(v) for v in tok.split(",")] for tok in gates.split(";")], np.float32)
        assert ids.shape == gates.shape and ids.shape[1] == k, name
        lim = np.array([int(v) for v in limits.split(",")], np.int32)
        r = oracle.route_capacity(ids, gates, E, lim, int(base), adaptive=bool(int(adaptive)))
        assert r["assign"].tolist() == [int(v) for v in assign.split(",")], name
        assert r["weight"].tolist() == [float(v) for v in weight.split(",")], name
        assert r["limits"].tolist() == [int(v) for v in after.split(",")], name
        assert lim.tolist() == [int(v) for v in limits.split(",")], name      # input left alone
        _capacity_check_lists(r, E)
        n += 1
    assert n == 7


def _prefs(rng, T, E, k):
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    gates = rng.random((T, k)).astype(np.float32)
    return ids, gates


@pytest.mark.parametrize("T,E,k,seed", [(200, 16, 4, 0), (64, 8, 8, 1), (300, 1, 1, 2)])
def test_capacity_unlimited_is_top1(T, E, k, seed):
    """With room for every token, each takes its first preference at its first gate."""
    ids, gates = _prefs(np.random.default_rng(seed), T, E, k)
    r = oracle.route_capacity(ids, gates, E, np.full(E, T, np.int32), 1)
    assert np.array_equal(r["assign"], ids[:, 0])
    assert np.array_equal(r["weight"], gates[:, 0])
    _capacity_check_lists(r, E)


def test_capacity_zero_drops_every_token():
    ids, gates = _prefs(np.random.default_rng(7), 50, 6, 3)
    r = oracle.route_capacity(ids, gates, 6, np.zeros(6, np.int32), 0)
    assert (r["assign"] == -1).all() and (r["weight"] == 0).all() and (r["counts"] == 0).all()
    assert (r["limits"] == 0).all()


@pytest.mark.parametrize("T,E,k,L,seed", [(400, 16, 4, 10, 0), (500, 8, 2, 30, 1), (100, 32, 8, 1, 2),
                                          (257, 5, 5, 3, 3), (1000, 64, 8, 12, 4)])
def test_capacity_bounds_and_weights(T, E, k, L, seed):
    """Preference routing stops at the limit and the fallback at 1.5x it, so no count
    passes ceil(1.5 L); a token is dropped only when the least-loaded expert, hence every
    expert, already holds that many; a routed token's weight is the gate of the slot that
    names its expert, or half its first gate (the fallback)."""
    ids, gates = _prefs(np.random.default_rng(seed), T, E, k)
    r = oracle.route_capacity(ids, gates, E, np.full(E, L, np.int32), 1)
    cap = -(-3 * L // 2)
    assert r["counts"].max() <= cap
    dropped = r["assign"] < 0
    if dropped.any():
        assert (r["counts"] == cap).all()
    for t in np.nonzero(~dropped)[0]:
        e = r["assign"][t]
        ok = {float(gates[t, 0]) * 0.5}
        ok |= {float(gates[t, j]) for j in range(k) if ids[t, j] == e}
        assert float(r["weight"][t]) in ok
    _capacity_check_lists(r, E)
    # a tight limit makes both rules fire on these seeds
    assert (r["weight"] == gates[:, 0] * 0.5).any() or L >= T


def test_capacity_integer_limit_forms():
    """The GPU kernel updates limits with 64-bit integer forms; they equal the page's
    truncated float products (taken in double, as the oracle takes them).  An exhaustive
    run over all 0 <= L < 2^31 found no difference; this re-checks the first 2^22, the
    last 2^20 and 2^22 random values."""
    rng = np.random.default_rng(5)
    L = np.concatenate([np.arange(1 << 22), np.arange((1 << 31) - (1 << 20), 1 << 31),
                        rng.integers(0, 1 << 31, 1 << 22)]).astype(np.int64)
    f = L.astype(np.float64)
    assert np.array_equal(np.trunc(f * 1.2).astype(np.int64), 6 * L // 5)
    assert np.array_equal(np.trunc(f * 0.9).astype(np.int64), 9 * L // 10)
    c = rng.integers(0, 1 << 31, L.size).astype(np.int64)
    assert np.array_equal(c.astype(np.float64) < f * 1.5, 2 * c < 3 * L)
    assert np.array_equal(c.astype(np.float64) < f * 0.5, 2 * c < L)


def _small_f32_layer(rng, H=32, M=16, E=4, Ms=0):
    w_gu = [rng.standard_normal((H, 2 * M)).astype(np.float32) / 4 for _ in range(E)]
    w_d = [rng.standard_normal((M, H)).astype(np.float32) / 4 for _ in range(E)]
    ws = (rng.standard_normal((H, 2 * Ms)).astype(np.float32) / 4,
          rng.standard_normal((Ms, H)).astype(np.float32) / 4) if Ms else (None, None)
    return w_gu, w_d, ws


def test_layer_assigned_reduces_to_top1_layer():
    """An assignment equal to the k = 1 router's choice at weight 1 is that layer."""
    rng = np.random.default_rng(21)
    H, M, E, n = 32, 16, 4, 12
    w_gu, w_d, _ = _small_f32_layer(rng, H, M, E)
    x = rng.standard_normal((n, H)).astype(np.float32)
    logits = rng.standard_normal((n, E)).astype(np.float32)
    ids, gates, y1, _ = oracle.layer(x, logits, H=H, M=M, E=E, k=1, dtype="f32", w_gu=w_gu, w_d=w_d)
    assert (gates == 1.0).all()
    y, macs = oracle.layer_assigned(x, ids[:, 0], np.ones(n, np.float32), H=H, M=M, E=E, dtype="f32",
                                    w_gu=w_gu, w_d=w_d)
    assert np.array_equal(y, y1)
    assert macs == n * 3 * H * M
    yh, _ = oracle.layer_assigned(x, ids[:, 0], np.full(n, 0.5, np.float32), H=H, M=M, E=E, dtype="f32",
                                  w_gu=w_gu, w_d=w_d)
    assert np.array_equal(yh, 0.5 * y1)


def test_layer_assigned_dropped_tokens():
    """A dropped token gets nothing from the routed experts and still gets the shared
    expert, which alone is a one-expert layer with the shared weights at gate 1."""
    rng = np.random.default_rng(22)
    H, M, E, Ms, n = 32, 16, 4, 24, 9
    w_gu, w_d, (ws_gu, ws_d) = _small_f32_layer(rng, H, M, E, Ms)
    x = rng.standard_normal((n, H)).astype(np.float32)
    assign = np.array([2, -1, 0, -1, 3, 1, -1, 2, 0], np.int32)
    w = rng.random(n).astype(np.float32)
    y, macs = oracle.layer_assigned(x, assign, w, H=H, M=M, E=E, dtype="f32", w_gu=w_gu, w_d=w_d,
                                    Ms=Ms, ws_gu=ws_gu, ws_d=ws_d)
    _, _, ys, _ = oracle.layer(x, np.zeros((n, 1), np.float32), H=H, M=Ms, E=1, k=1, dtype="f32",
                               w_gu=[ws_gu], w_d=[ws_d])
    drop = assign < 0
    assert np.array_equal(y[drop], ys[drop])
    assert macs == int((~drop).sum()) * 3 * H * M + n * 3 * H * Ms
    y0, _ = oracle.layer_assigned(x, np.full(n, -1, np.int32), w, H=H, M=M, E=E, dtype="f32", w_gu=w_gu, w_d=w_d)
    assert (y0 == 0).all()
