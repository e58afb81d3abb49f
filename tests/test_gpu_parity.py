"""Parity of the HIP path (through the C ABI) with the CPU oracle on the same seeded
inputs.

Bars: expert ids, counts, offsets, sorted pairs and pair positions bit-exact; gates
within 2e-6 absolute (both are fp32-exp based; the oracle works in double); layer
output max|y - ref| <= tol * max|ref| with tol = 1e-4 (fp32 layer), 2e-2 (bf16) and
6e-2 (fp8), fp32 accumulation on the GPU.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_expert_ffn_softmax_amd import MoeExpertFFN

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
GATE_ATOL = 2e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def say(msg):
    print(msg, flush=True)


def make_layer(w, weights, max_tokens=None):
    return MoeExpertFFN(hidden=w.H, inter=w.M, num_experts=w.E, top_k=w.k, max_tokens=max_tokens or max(w.T, 1),
                        dtype=w.dtype, w_gate_up=weights["w_gu"], w_down=weights["w_d"], s_gate_up=weights["s_gu"],
                        s_down=weights["s_d"], shared_inter=w.Ms, ws_gate_up=weights["ws_gu"],
                        ws_down=weights["ws_d"], ss_gate_up=weights["ss_gu"], ss_down=weights["ss_d"])


def run_layer(layer, x, logits, T=None):
    T = x.shape[0] if T is None else T
    rb = layer.new_route()
    y = torch.full((max(T, 1), layer.cfg.hidden), float("nan"), device=x.device,
                   dtype=torch.float32 if layer.dtype == "f32" else torch.bfloat16)
    layer.route(logits, T, rb)
    layer.forward(x, T, rb, y)
    torch.cuda.synchronize()
    return rb, y


def check_route(rb, logits_np, E, k):
    T = logits_np.shape[0]
    P = T * k
    ids_o, gates_o = oracle.route(logits_np, k)
    counts_o, offsets_o, sp_o, pp_o = oracle.permute(ids_o, E)
    np.testing.assert_array_equal(rb.topk_ids[:P].cpu().numpy(), ids_o.ravel())
    np.testing.assert_array_equal(rb.expert_counts.cpu().numpy(), counts_o)
    np.testing.assert_array_equal(rb.expert_offsets.cpu().numpy(), offsets_o)
    np.testing.assert_array_equal(rb.sorted_pair[:P].cpu().numpy(), sp_o)
    np.testing.assert_array_equal(rb.pair_pos[:P].cpu().numpy(), pp_o)
    g = rb.topk_gates[:P].cpu().numpy().astype(np.float64)
    assert np.abs(g - gates_o.ravel()).max() <= GATE_ATOL
    return ids_o, counts_o


def check_y(y_rows, ref, tol, what=""):
    y = y_rows.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = np.abs(y - ref).max()
    scale = np.abs(ref).max()
    say(f"{what}: max|err| = {err:.3e}, max|ref| = {scale:.3e}, ratio = {err / scale:.3e} (tol {tol})")
    assert err <= tol * scale, f"{what}: {err} > {tol} * {scale}"


def oracle_rows(w, weights, x, logits_np, rows):
    """Oracle output for token rows `rows`, copying only the experts they use."""
    rows = np.asarray(sorted(set(int(r) for r in rows)))
    xs = x[torch.as_tensor(rows, device=x.device)].float().cpu().numpy()
    ls = logits_np[rows]
    ids, _ = oracle.route(ls, w.k)
    need = np.unique(ids)
    # host copies of the experts the rows use, once; then the oracle in chunks, with a
    # progress line per chunk
    host = {k: v for k, v in weights.items() if k not in ("w_gu", "w_d", "s_gu", "s_d")}
    for k in ("w_gu", "w_d", "s_gu", "s_d"):
        host[k] = None if weights.get(k) is None else {int(e): weights[k][int(e)].cpu() for e in need}
    host = {k: (v.cpu() if hasattr(v, "cpu") else v) for k, v in host.items()}
    yref = np.zeros((len(rows), w.H))
    chunk = 256
    for c0 in range(0, len(rows), chunk):
        sl = slice(c0, c0 + chunk)
        _, _, yref[sl], _ = oracle.layer_from_weights(xs[sl], ls[sl], w, host, experts_needed=np.unique(ids[sl]))
        if len(rows) > chunk:
            say(f"  oracle: {min(c0 + chunk, len(rows))} of {len(rows)} tokens")
    return rows, yref


def tile_boundary_rows(counts, offsets, sorted_pair, k, T, Ms, tile_rows, even):
    """Tokens holding the first and the last row of every row tile of every expert (and
    of the shared expert's T rows), with the tiling of the kernel that runs: 128-row
    tiles with an expert's rows split evenly over them (the tiled kernels), or 16-row
    tiles cut in order (the streaming kernels).  Returns (tokens, experts, tiles)."""
    def bounds(n):
        if n == 0:
            return []
        nt = -(-n // tile_rows)
        if not even:
            return [(t * tile_rows, min(n, (t + 1) * tile_rows) - 1) for t in range(nt)]
        base, extra = divmod(n, nt)
        out, r0 = [], 0
        for t in range(nt):
            r1 = r0 + base + (1 if t < extra else 0)
            out.append((r0, r1 - 1))
            r0 = r1
        return out

    tokens, tiles, experts = set(), 0, 0
    for e in range(len(counts)):
        b = bounds(int(counts[e]))
        experts += bool(b)
        tiles += len(b)
        for r0, r1 in b:
            tokens.add(int(sorted_pair[offsets[e] + r0]) // k)
            tokens.add(int(sorted_pair[offsets[e] + r1]) // k)
    if Ms:
        b = bounds(T)
        tiles += len(b)
        for r0, r1 in b:
            tokens.update((r0, r1))
    return sorted(tokens), experts, tiles


def full_case(w, sample=None, kernel="auto", tiles=False):
    say(f"case {w.name}: T={w.T} H={w.H} M={w.M} E={w.E} k={w.k} Ms={w.Ms} {w.dtype} gemm={kernel}")
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    logits_np = logits.cpu().numpy()
    layer = make_layer(w, weights)
    layer.set_gemm_kernel(kernel)
    rb, y = run_layer(layer, x, logits)
    _, counts = check_route(rb, logits_np, w.E, w.k)
    if sample is None:
        rows = np.arange(w.T)
    else:
        rng = np.random.default_rng(w.index)
        # first and last tokens, random ones, and the tokens at the tail of the
        # hottest expert's segment (its last, possibly ragged, row tile)
        hot = int(np.argmax(counts))
        off = rb.expert_offsets.cpu().numpy()
        sp = rb.sorted_pair.cpu().numpy()
        tail = sp[max(off[hot], off[hot + 1] - 3):off[hot + 1]] // w.k
        rows = np.concatenate([[0, 1, w.T - 1], rng.integers(0, w.T, sample), tail])
        if tiles:
            # every row tile of every expert: first and last row, in the tiling of the
            # kernel the automatic choice (or `kernel`) runs
            P = w.T * w.k
            tiled = kernel == "tiled" or (kernel == "auto" and P > (12 if w.dtype == "fp8" else 8) * w.E)
            bt, ne, nt = tile_boundary_rows(counts, off, sp, w.k, w.T, w.Ms, 128 if tiled else 16, tiled)
            rows = np.concatenate([rows, bt])
            say(f"{w.name}: {len(set(rows.tolist()))} tokens cover the first and last row of all {nt} row tiles "
                f"({'128-row even split' if tiled else '16-row'}) of {ne} experts" + (" and the shared expert"
                                                                                        if w.Ms else ""))
    rows, yref = oracle_rows(w, weights, x, logits_np, rows)
    check_y(y[torch.as_tensor(rows, device="cuda")], yref, TOL[w.dtype], w.name)
    return layer, x, logits, y


def small(name, **kw):
    base = dict(name=name, index=100, T=37, H=256, M=384, E=16, k=4, Ms=0, dtype="bf16")
    base.update(kw)
    return workloads.Workload(**base)


# ----------------------------------------------------------------------------- workloads
def test_tiny_f32_full():
    full_case(workloads.TINY)


def test_starved_decode_full():
    full_case(workloads.STARVED_DECODE)


@pytest.mark.parametrize("kernel", ["auto", "stream"])
def test_afd_aggregated_every_tile(kernel):
    full_case(workloads.AGGREGATED, sample=6, kernel=kernel, tiles=True)


def test_coarse_experts_with_shared_every_tile():
    full_case(workloads.COARSE, sample=3, tiles=True)


def test_fp8_decode_full():
    """The fp8 layer at a decode batch of 6 tokens (streaming GEMMs), every token."""
    full_case(workloads.FP8_DECODE)


def test_starved_decode_tiled_kernel():
    """The 128-row kernel on a decode batch: one partial tile per touched expert."""
    full_case(workloads.STARVED_DECODE, kernel="tiled")


def test_fp8_blockscaled_every_tile():
    full_case(workloads.FP8_DSV3, sample=3, tiles=True)


def test_tp4_share_of_the_decode_layer_full():
    """One GPU's share of the starved-decode layer under 4-way tensor parallelism in the
    experts (M = 384 of 1536), every token."""
    full_case(workloads.TP4_SHARE)


def test_ep8_share_of_the_fp8_layer_every_tile():
    """One GPU's share of the DeepSeek-V3-like fp8 layer under 8-way expert parallelism
    (32 local experts, 4096 received rows, each to one local expert), on the tokens at
    both ends of every row tile."""
    full_case(workloads.EP8_SHARE, sample=3, tiles=True)


@pytest.mark.parametrize("w", [workloads.mfma_sweep("bf16")[0], workloads.mfma_sweep("bf16")[-1],
                               workloads.mfma_sweep("fp8")[-1]], ids=lambda w: w.name)
def test_mfma_sweep_every_tile(w):
    """The 256 / 1024 tokens-per-expert batches on which the matrix-core rate is
    measured, at full size and in the launch configuration timed there (automatic
    kernel choice: the 128-row tiled GEMMs), on the tokens at both ends of every row
    tile of every expert."""
    full_case(w, sample=3, tiles=True)


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_fp8_quantisation_bit_exact(src):
    """Step a0 alone: codes and scales equal the oracle's per-128 quantisation
    bit for bit (both decide in fp32)."""
    from moe_expert_ffn_softmax_amd import quantize_fp8
    rng = np.random.default_rng(17)
    rows, cols = 37, 640
    v = rng.standard_normal((rows, cols)).astype(np.float32)
    v *= rng.choice([1e-6, 1e-2, 1.0, 300.0], size=(rows, 1)).astype(np.float32)
    v[3, :128] = 0.0                      # an all-zero group: scale 1
    v[4, 128:256] = -0.0                  # negative zeros keep their sign bit
    v[5, 5] = 1e-30                       # far below the group's amax: rounds to +-0
    v[6, 256:384] = 7.0                   # constant group: every code 448
    t = torch.from_numpy(v)
    if src == "bf16":
        t = t.to(torch.bfloat16)
        v = t.float().numpy()
    codes, scales = quantize_fp8(t.cuda())
    torch.cuda.synchronize()
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    for r in range(rows):
        c_ref, s_ref, _ = oracle.quant_row_fp8(v[r])
        np.testing.assert_array_equal(scales[r], s_ref, err_msg=f"row {r}")
        np.testing.assert_array_equal(codes[r], c_ref, err_msg=f"row {r}")


def test_fp8_quantisation_more_rows_than_waves():
    """Step a0 on more rows than the launch has waves (32768): the rows past the grid are
    taken in a second pass.  Sampled rows at both ends and across that boundary are
    bit-exact against the oracle, for a row length that is not a multiple of a wave's
    step (640 bf16 channels: 512 + 128)."""
    from moe_expert_ffn_softmax_amd import quantize_fp8
    rng = np.random.default_rng(23)
    rows, cols = 32768 + 300, 640
    v = rng.standard_normal((rows, cols)).astype(np.float32)
    v *= rng.choice([1e-3, 1.0, 50.0], size=(rows, 1)).astype(np.float32)
    t = torch.from_numpy(v).to(torch.bfloat16)
    v = t.float().numpy()
    codes, scales = quantize_fp8(t.cuda())
    torch.cuda.synchronize()
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    sample = list(range(40)) + list(range(32768 - 40, 32768 + 40)) + list(range(rows - 40, rows))
    for r in sample:
        c_ref, s_ref, _ = oracle.quant_row_fp8(v[r])
        np.testing.assert_array_equal(scales[r], s_ref, err_msg=f"row {r}")
        np.testing.assert_array_equal(codes[r], c_ref, err_msg=f"row {r}")


@pytest.mark.parametrize("w", workloads.ORDERED, ids=lambda w: w.name)
def test_route_full_size_every_workload(w):
    """Routing alone at every workload's full T, E, k (small H, M: routing does not
    depend on them)."""
    say(f"route case {w.name}")
    tiny = dataclasses.replace(w, H=128, M=128, Ms=0, dtype="bf16", name=w.name + "_route")
    weights = workloads.make_weights(dataclasses.replace(tiny, E=w.E), device="cuda")
    layer = make_layer(tiny, weights, max_tokens=w.T)
    logits = torch.from_numpy(workloads.router_logits(w)).cuda()
    rb = layer.new_route()
    layer.route(logits, w.T, rb)
    torch.cuda.synchronize()
    check_route(rb, logits.cpu().numpy(), w.E, w.k)


@pytest.mark.parametrize("T,E,k,ties", [
    (16384 + 37, 128, 8, False),   # 32 full blocks of pairs and a ragged last one
    (16384, 256, 8, True),         # integer logits: many ties, decided by expert index
    (300, 1024, 32, False),        # E = 1024 and k = 32: 9600 pairs, three blocks
    (1025, 8, 8, False),           # k = E: every expert gets every token
], ids=["ragged_last_block", "ties_large", "many_experts_k32", "k_equals_E"])
def test_route_large_batches(T, E, k, ties):
    """The multi-block permute (used above 8192 pairs) is bit-identical to the
    stable counting sort of the oracle."""
    say(f"route case T={T} E={E} k={k} ties={ties}")
    w = workloads.Workload(name="route_large", index=200, T=T, H=128, M=128, E=E, k=k, Ms=0, dtype="bf16")
    weights = workloads.make_weights(w, device="cuda")
    layer = make_layer(w, weights, max_tokens=T)
    rng = np.random.default_rng(T + E)
    lg = (rng.integers(-2, 3, size=(T, E)) if ties else rng.standard_normal((T, E))).astype(np.float32)
    logits = torch.from_numpy(lg).cuda()
    rb = layer.new_route()
    layer.route(logits, T, rb)
    torch.cuda.synchronize()
    check_route(rb, lg, E, k)


# ----------------------------------------------------------------------------- shapes and edges
@pytest.mark.parametrize("w", [
    small("ragged_bf16"),
    small("ragged_bf16_shared", Ms=256),
    small("ragged_f32_shared", dtype="f32", T=50, H=128, M=256, E=4, k=2, Ms=128),
    small("one_token", T=1, E=8, k=2),
    small("k1", T=40, E=8, k=1),
    small("k_equals_E", T=21, E=4, k=4),
    small("single_expert", T=33, E=1, k=1, Ms=128),
    small("many_experts", T=9, E=1024, k=32, H=128, M=128),
    small("wide_f32", dtype="f32", T=17, H=384, M=128, E=6, k=3),
], ids=lambda w: w.name)
@pytest.mark.parametrize("kernel", ["stream", "tiled"])
def test_small_shapes(w, kernel):
    full_case(w, kernel=kernel)


@pytest.mark.parametrize("w", [
    small("fp8_ragged", dtype="fp8", T=37, H=256, M=384, E=16, k=4),
    small("fp8_shared", dtype="fp8", T=50, H=384, M=256, E=6, k=2, Ms=256),
    small("fp8_one_token", dtype="fp8", T=1, H=128, M=128, E=8, k=2, Ms=128),
    small("fp8_skewed_long_k", dtype="fp8", T=90, H=1024, M=512, E=3, k=2),
    # more down items (64 experts x 8 column tiles + the shared expert's) than resident
    # workgroups, row counts of 2 and 4 blocks: the tiled down GEMM chains items within
    # runs of equal block count and restarts between runs
    small("fp8_chained_runs", dtype="fp8", T=256, H=2048, M=384, E=64, k=8, Ms=384),
    # the same with a shared expert of another width: a chained routed item hands over to a
    # shared one with another reduction length (chunk count) and back
    small("fp8_chained_runs_unequal_k", dtype="fp8", T=256, H=2048, M=384, E=64, k=8, Ms=640),
], ids=lambda w: w.name)
@pytest.mark.parametrize("kernel", ["stream", "tiled"])
def test_fp8_shapes(w, kernel):
    full_case(w, kernel=kernel)


@pytest.mark.parametrize("w", [
    small("tiled_multi_tile", T=300, E=4, k=2, H=256, M=256, Ms=384),
    small("tiled_odd_groups", T=200, E=3, k=2, H=384, M=128),
    small("tiled_long_k", T=140, E=2, k=1, H=1024, M=640, Ms=128),
], ids=lambda w: w.name)
def test_tiled_shapes(w):
    """Experts with several 128-row tiles (ragged last tile), a column count that
    leaves half of the last column tile empty, and long reductions."""
    full_case(w, kernel="tiled")


def test_skewed_routing_multi_tile_expert():
    """Every token prefers experts 3 and 5, so those two get 100 rows each (seven
    16-row tiles, the last ragged)."""
    w = small("skewed", T=100, E=8, k=3)
    say(f"case {w.name}")
    weights = workloads.make_weights(w, device="cuda")
    x, _ = workloads.make_activations(w, device="cuda")
    lg = np.random.default_rng(1).standard_normal((w.T, w.E)).astype(np.float32)
    lg[:, 3] += 20
    lg[:, 5] += 19
    logits = torch.from_numpy(lg).cuda()
    layer = make_layer(w, weights)
    rb, y = run_layer(layer, x, logits)
    _, counts = check_route(rb, lg, w.E, w.k)
    assert counts[3] == 100 and counts[5] == 100
    rows, yref = oracle_rows(w, weights, x, lg, np.arange(w.T))
    check_y(y, yref, TOL[w.dtype], w.name)


def test_integer_logits_ties():
    w = small("ties", T=64, E=8, k=3)
    say(f"case {w.name}")
    weights = workloads.make_weights(w, device="cuda")
    x, _ = workloads.make_activations(w, device="cuda")
    lg = np.random.default_rng(3).integers(-2, 3, size=(w.T, w.E)).astype(np.float32)
    lg[0, :] = 0.0
    lg[1, ::2] = -0.0
    logits = torch.from_numpy(lg).cuda()
    layer = make_layer(w, weights)
    rb, y = run_layer(layer, x, logits)
    check_route(rb, lg, w.E, w.k)
    rows, yref = oracle_rows(w, weights, x, lg, np.arange(w.T))
    check_y(y, yref, TOL[w.dtype], w.name)


@pytest.mark.parametrize("w,kernel", [
    (small("graph_decode", T=6, E=16, k=4, Ms=128), "auto"),        # one-launch route, streaming GEMMs
    (small("graph_tiled", T=200, E=4, k=2, H=256, M=256), "tiled"),  # two-kernel route, 128-row tiles
    (small("graph_fp8", dtype="fp8", T=50, H=384, M=256, E=6, k=2, Ms=256), "tiled"),
    (small("graph_fused", T=6, H=512, M=512, E=16, k=4, Ms=256), "fused"),  # one persistent GEMM launch
], ids=lambda v: v if isinstance(v, str) else v.name)
def test_hip_graph_replays_match_eager(w, kernel):
    """route + forward captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, reproduces the eager result bit for bit."""
    say(f"case {w.name} graph gemm={kernel}")
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = make_layer(w, weights)
    layer.set_gemm_kernel(kernel)
    rb_e, y_e = run_layer(layer, x, logits)
    rb = layer.new_route()
    y = torch.zeros_like(y_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        layer.route(logits, w.T, rb, stream=s)       # warm-up on the capture stream
        layer.forward(x, w.T, rb, y, stream=s)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            layer.route(logits, w.T, rb, stream=s)
            layer.forward(x, w.T, rb, y, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        y.zero_()
        rb.sorted_pair.fill_(-1)
        run_layer(layer, x.flip(0), logits.flip(0))  # unrelated eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_e), f"replay {rep}: output differs from the eager run"
        assert torch.equal(rb.sorted_pair, rb_e.sorted_pair), f"replay {rep}: permutation differs"


@pytest.mark.parametrize("w", [
    small("ubatch_bf16", T=100, H=256, M=384, E=16, k=4),
    small("ubatch_decode", T=6, H=512, M=256, E=32, k=4),
    small("ubatch_fp8_shared", dtype="fp8", T=90, H=384, M=256, E=6, k=2, Ms=256),
], ids=lambda w: w.name)
def test_two_micro_batches_on_two_streams(w):
    """Two micro-batches in flight on one handle (the AFD blog's two-micro-batch
    overlap, FFN side): micro-batch 2 is routed on a second stream while micro-batch
    1's forward runs; both forwards run on the first stream.  Each micro-batch's
    output equals that micro-batch run alone, bit for bit, over several rounds."""
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = make_layer(w, weights)
    T1 = (w.T + 1) // 2
    T2 = w.T - T1
    ydt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    # each micro-batch alone, on the default stream
    ref = torch.empty((w.T, w.H), dtype=ydt, device="cuda")
    ra, rb_ = layer.new_route(), layer.new_route()
    layer.route(logits, T1, ra)
    layer.forward(x, T1, ra, ref)
    layer.route(logits[T1:], T2, rb_)
    layer.forward(x[T1:], T2, rb_, ref[T1:])
    torch.cuda.synchronize()
    # overlapped, three rounds reusing the route buffers
    sa = torch.cuda.current_stream()
    sb = torch.cuda.Stream()
    r1, r2 = layer.new_route(), layer.new_route()
    ev_route, ev_free = torch.cuda.Event(), torch.cuda.Event()
    ev_free.record(sa)
    for rnd in range(3):
        y = torch.full((w.T, w.H), float("nan"), dtype=ydt, device="cuda")
        sb.wait_event(ev_free)
        layer.route(logits[T1:], T2, r2, stream=sb)
        ev_route.record(sb)
        layer.route(logits, T1, r1)
        layer.forward(x, T1, r1, y)
        sa.wait_event(ev_route)
        layer.forward(x[T1:], T2, r2, y[T1:])
        ev_free.record(sa)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"round {rnd}: overlapped micro-batches differ from the runs alone"
    # and the whole output against the oracle
    rows, yref = oracle_rows(w, weights, x, logits.cpu().numpy(), np.arange(w.T))
    check_y(y, yref, TOL[w.dtype], w.name)
    layer.close()


def test_overlapping_buffers_are_rejected():
    """forward's x and y, and route_hidden's logits and inputs, must not overlap: the
    host checks return AFD_EINVAL and enqueue nothing."""
    from moe_expert_ffn_softmax_amd._ffi import AFD_EINVAL, AfdError, afd_ffn_forward
    w = small("overlap", T=8, H=128, M=128, E=4, k=2)
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = make_layer(w, weights)
    rb = layer.new_route()
    layer.route(logits, w.T, rb)
    with pytest.raises(ValueError):  # the binding refuses a y one row short
        layer.forward(x, w.T, rb, x[1:])
    with pytest.raises(AfdError) as e:  # the C ABI refuses the overlap
        afd_ffn_forward(layer.handle, x, w.T, rb.c, x[1:])
    assert e.value.code == AFD_EINVAL
    wr = torch.zeros((w.E, w.H), dtype=torch.bfloat16, device="cuda")
    buf = torch.zeros(w.T * w.H, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(AfdError) as e:
        layer.route_hidden(buf.view(w.T, w.H), wr, buf.view(torch.float32), w.T, rb)
    assert e.value.code == AFD_EINVAL
    torch.cuda.synchronize()
    layer.close()


def test_route_bytes_matches_the_route_buffers():
    from moe_expert_ffn_softmax_amd import afd_ffn_route_bytes
    w = small("route_bytes", T=37, E=20, k=3)
    weights = workloads.make_weights(w, device="cuda")
    layer = make_layer(w, weights)
    rb = layer.new_route()
    arrays = [rb.topk_ids, rb.topk_gates, rb.expert_counts, rb.expert_offsets, rb.sorted_pair, rb.pair_pos]
    assert afd_ffn_route_bytes(layer.handle) == sum(a.numel() * a.element_size() for a in arrays)
    layer.close()


def test_misaligned_buffers_are_rejected():
    """Views off their required boundary fail with AFD_EINVAL before any work is queued."""
    from moe_expert_ffn_softmax_amd import AfdError, afd_ffn_forward, afd_ffn_route
    w = small("aligned", T=8, E=8, k=2)
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = make_layer(w, weights)
    rb = layer.new_route()
    layer.route(logits, w.T, rb)
    buf = torch.zeros(w.T * w.H + 8, dtype=torch.bfloat16, device="cuda")
    x_off = buf[1:1 + w.T * w.H]            # 2 bytes off a 16-byte boundary
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(AfdError):
        afd_ffn_forward(layer.handle, x_off, w.T, rb.c, y)
    lg = torch.zeros(w.T * w.E + 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(AfdError):
        afd_ffn_route(layer.handle, lg[1:], w.T, rb.c)  # logits 1 byte off
    # the aligned call still works after the rejected ones
    layer.forward(x, w.T, rb, y)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    layer.close()


def test_route_buffer_overlaps_are_rejected():
    """Inputs or outputs aliasing the route buffers, or route buffers aliasing each
    other, fail with AFD_EINVAL before any work is queued."""
    from moe_expert_ffn_softmax_amd import AfdError, afd_ffn_forward, afd_ffn_route, afd_route
    w = small("route_alias", T=8, E=8, k=2)
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = make_layer(w, weights)
    rb = layer.new_route()
    P = w.T * w.k
    # logits whose storage holds the route's expert ids
    big = torch.zeros(w.T * w.E + 4 * P + 64, dtype=torch.int32, device="cuda")
    alias = afd_route(big.data_ptr(), rb.topk_gates.data_ptr(), rb.expert_counts.data_ptr(),
                      rb.expert_offsets.data_ptr(), rb.sorted_pair.data_ptr(), rb.pair_pos.data_ptr())
    with pytest.raises(AfdError):
        afd_ffn_route(layer.handle, big, w.T, alias)
    # two route buffers at one address
    twin = afd_route(rb.topk_ids.data_ptr(), rb.topk_ids.data_ptr(), rb.expert_counts.data_ptr(),
                     rb.expert_offsets.data_ptr(), rb.sorted_pair.data_ptr(), rb.pair_pos.data_ptr())
    with pytest.raises(AfdError):
        afd_ffn_route(layer.handle, logits, w.T, twin)
    # y on top of the permutation the combine reads
    layer.route(logits, w.T, rb)
    yb = torch.zeros(w.T * w.H * 2 + 4 * P, dtype=torch.uint8, device="cuda")
    yalias = afd_route(rb.topk_ids.data_ptr(), rb.topk_gates.data_ptr(), rb.expert_counts.data_ptr(),
                       rb.expert_offsets.data_ptr(), yb.data_ptr() + 64, rb.pair_pos.data_ptr())
    with pytest.raises(AfdError):
        afd_ffn_forward(layer.handle, x, w.T, yalias, yb)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    layer.forward(x, w.T, rb, y)  # separate buffers still work
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    layer.close()


def test_zero_tokens_is_a_no_op():
    w = small("empty", T=8)
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = make_layer(w, weights)
    rb = layer.new_route()
    rb.expert_counts.fill_(-7)
    y = torch.full((8, w.H), 3.0, dtype=torch.bfloat16, device="cuda")
    layer.route(logits, 0, rb)
    layer.forward(x, 0, rb, y)
    torch.cuda.synchronize()
    assert torch.all(rb.expert_counts == -7) and torch.all(y == 3.0)


def test_smaller_batch_after_larger_and_determinism():
    """A handle sized for 64 tokens serves 64, then 5, then 64 again; repeated calls
    give bitwise identical results."""
    w = small("reuse", T=64, E=16, k=4, Ms=128)
    say(f"case {w.name}")
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = make_layer(w, weights)
    _, y1 = run_layer(layer, x, logits)
    _, y5 = run_layer(layer, x[:5].contiguous(), logits[:5].contiguous())
    _, y2 = run_layer(layer, x, logits)
    assert torch.equal(y1, y2)
    rows, yref = oracle_rows(w, weights, x, logits.cpu().numpy(), np.arange(5))
    check_y(y5[:5], yref, TOL[w.dtype], "reuse T=5")
    # the first five tokens route the same alone as in the full batch
    assert torch.equal(y5[:5], y1[:5])


@pytest.mark.parametrize("T", [100, 32])
def test_profiling_counts_launches(T):
    """Every stage is timed once per call; batches of at most 64 tokens route and
    permute in one launch, timed as the router stage."""
    w = small("profiled", T=T)
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = make_layer(w, weights)
    from moe_expert_ffn_softmax_amd import afd_ffn_profile_read, afd_ffn_set_profiling
    afd_ffn_set_profiling(layer.handle, True)
    for _ in range(3):
        run_layer(layer, x, logits)
    prof = afd_ffn_profile_read(layer.handle)
    afd_ffn_set_profiling(layer.handle, False)
    fused = T <= 64
    for st in ("router", "permute", "gate_up", "down", "combine"):
        if st == "permute" and fused:
            assert prof[st][1] == 0
        else:
            assert prof[st][1] == 3 and prof[st][0] > 0
    assert afd_ffn_profile_read(layer.handle)["gate_up"][1] == 0


# ----------------------------------------------------------------------------- fused decode launch
def test_fused_decode_layer_every_token():
    """AFD_GEMM_FUSED on the starved-decode layer: both GEMMs in one persistent launch
    with a grid barrier, the gates applied in the down epilogue; every token against
    the oracle, and two calls in a row bitwise equal (the barrier counters return to
    zero)."""
    layer, x, logits, y = full_case(workloads.STARVED_DECODE, kernel="fused")
    _, y2 = run_layer(layer, x, logits)
    assert torch.equal(y, y2)
    layer.set_gemm_kernel("stream")
    _, y3 = run_layer(layer, x, logits)
    d = (y3.float() - y.float()).abs().max().item()
    say(f"fused vs separate launches: max |diff| = {d:.3e}")  # the gate is applied before O's rounding
    assert d <= 2e-2 * y3.float().abs().max().item()
    layer.close()


@pytest.mark.parametrize("w", [
    small("fused_shared", T=37, H=512, M=256, E=16, k=4, Ms=256),
    small("fused_k1", T=40, H=256, M=512, E=8, k=1),
    small("fused_k_equals_E", T=9, H=256, M=256, E=4, k=4, Ms=512),
    small("fused_one_token", T=1, H=768, M=512, E=8, k=2),
    small("fused_many_items", T=60, H=1024, M=768, E=32, k=8, Ms=256),
], ids=lambda w: w.name)
def test_fused_decode_shapes(w):
    full_case(w, kernel="fused")


def test_fused_decode_barrier_give_up_writes_nan(monkeypatch):
    """A workgroup that gives up waiting at the fused launch's barrier writes NaN into the
    down rows it owns instead of leaving them stale.  The poll limit is forced to 0 from
    the host (AFD_FUSED_SPIN_LIMIT, read at handle creation): every workgroup but the
    last to arrive gives up at once, and every wave still exits.  Some outputs are then
    NaN, every other output equals a normal fused call's bitwise, and a later call on the
    same handle does not hang (the barrier counters were returned to zero)."""
    w = workloads.STARVED_DECODE
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    ref = make_layer(w, weights)
    ref.set_gemm_kernel("fused")
    _, y_ref = run_layer(ref, x, logits)
    assert not torch.isnan(y_ref.float()).any()
    monkeypatch.setenv("AFD_FUSED_SPIN_LIMIT", "0")
    bad = make_layer(w, weights)
    monkeypatch.delenv("AFD_FUSED_SPIN_LIMIT")
    bad.set_gemm_kernel("fused")
    for call in range(2):
        _, y = run_layer(bad, x, logits)
        nan = torch.isnan(y.float())
        say(f"call {call}: {int(nan.sum())} of {nan.numel()} outputs NaN")
        assert nan.any()
        assert torch.equal(y[~nan], y_ref[~nan])
    bad.close()
    ref.close()


def test_fused_decode_on_a_capacity_route():
    """Empty slots of a capacity route carry gate 0: the fused launch computes no row for
    them and the combine skips them."""
    w = small("fused_capacity", T=48, H=512, M=256, E=8, k=4, Ms=256)
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = make_layer(w, weights)
    layer.set_gemm_kernel("fused")
    rb = layer.new_route()
    layer.route(logits, w.T, rb)
    limits = torch.full((w.E,), 2, dtype=torch.int32, device="cuda")  # at most 3 per expert: drops
    cap = layer.route_capacity(rb.topk_ids[:w.T * w.k].contiguous(), rb.topk_gates[:w.T * w.k].contiguous(), w.T,
                               limits, 2, False)
    rc = layer.new_route()
    layer.route_from_capacity(cap, w.T, rc)
    y = torch.full((w.T, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    layer.forward(x, w.T, rc, y)
    torch.cuda.synchronize()
    assign, weight = cap[0].cpu().numpy(), cap[1].cpu().numpy()
    assert (assign < 0).any(), "the case drops some tokens"
    yref, _ = oracle.layer_assigned(x.float().cpu().numpy(), assign, weight, H=w.H, M=w.M, E=w.E, dtype=w.dtype,
                                    w_gu=weights["w_gu"], w_d=weights["w_d"], Ms=w.Ms, ws_gu=weights["ws_gu"],
                                    ws_d=weights["ws_d"])
    check_y(y, yref, TOL[w.dtype], w.name)
    layer.close()
