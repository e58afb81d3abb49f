"""Parity on seeded random layer shapes within the documented limits: dtype, H, M, E,
k, T, the shared expert and the GEMM kernel all drawn from a fixed seed (the same 24
cases on every run), and 6 larger fp8 cases on the tiled GEMMs whose down items chain.  Bars as in the other parity tests: ids, counts and the
permutation bit-exact; gates within 2e-6; outputs within 1e-4 / 2e-2 / 6e-2 of
max|ref| (fp32 / bf16 / fp8)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_expert_ffn_softmax_amd import MoeExpertFFN

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


def _cases(n=24, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ["bf16", "fp8", "f32"][int(rng.integers(0, 3))]
        H = 128 * int(rng.integers(1, 7))
        M = 128 * int(rng.integers(1, 5))
        E = int(rng.integers(1, 97))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 300))
        Ms = 128 * int(rng.integers(0, 3)) if dtype != "f32" or rng.random() < 0.5 else 0
        kernel = ["auto", "stream", "tiled"][int(rng.integers(0, 3))]
        w = workloads.Workload(f"random{i}_{dtype}_T{T}_H{H}_M{M}_E{E}_k{k}_Ms{Ms}", 500 + i,
                               T=T, H=H, M=M, E=E, k=k, Ms=Ms, dtype=dtype)
        out.append((w, kernel))
    return out


def _chain_cases(n=6, seed=2027):
    """fp8 layers on the 128-row tiled GEMMs with more down items than resident
    workgroups (E >= 40 row tiles x 6-8 column tiles of 256), reductions above 256 and
    mixed row counts per expert: the down GEMM chains items within runs of equal 16-row
    block count and restarts between runs, also across the hand-over to a shared expert
    of another width."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = 256 * int(rng.integers(6, 9))
        M = 128 * int(rng.integers(3, 6))
        E = int(rng.integers(40, 129))
        k = int(rng.integers(2, 9))
        T = int(rng.integers(64, 301))
        Ms = 128 * [0, 3, 5][int(rng.integers(0, 3))]
        w = workloads.Workload(f"chain{i}_fp8_T{T}_H{H}_M{M}_E{E}_k{k}_Ms{Ms}", 600 + i,
                               T=T, H=H, M=M, E=E, k=k, Ms=Ms, dtype="fp8")
        out.append((w, "tiled"))
    return out


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


@pytest.mark.parametrize("w,kernel", _cases() + _chain_cases(), ids=lambda v: v.name if hasattr(v, "name") else v)
def test_random_shape(w, kernel):
    print(f"case {w.name} gemm={kernel}", flush=True)
    weights = workloads.make_weights(w, device="cuda")
    x, logits = workloads.make_activations(w, device="cuda")
    layer = MoeExpertFFN(hidden=w.H, inter=w.M, num_experts=w.E, top_k=w.k, max_tokens=w.T, dtype=w.dtype,
                         w_gate_up=weights["w_gu"], w_down=weights["w_d"], s_gate_up=weights["s_gu"],
                         s_down=weights["s_d"], shared_inter=w.Ms, ws_gate_up=weights["ws_gu"],
                         ws_down=weights["ws_d"], ss_gate_up=weights["ss_gu"], ss_down=weights["ss_d"])
    layer.set_gemm_kernel(kernel)
    rb = layer.new_route()
    ydt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    y = torch.full((w.T, w.H), float("nan"), dtype=ydt, device="cuda")
    layer.route(logits, w.T, rb)
    layer.forward(x, w.T, rb, y)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    P = w.T * w.k
    ids_o, gates_o = oracle.route(lg, w.k)
    counts_o, offsets_o, sp_o, pp_o = oracle.permute(ids_o, w.E)
    np.testing.assert_array_equal(rb.topk_ids[:P].cpu().numpy(), ids_o.ravel())
    np.testing.assert_array_equal(rb.expert_counts.cpu().numpy(), counts_o)
    np.testing.assert_array_equal(rb.expert_offsets.cpu().numpy(), offsets_o)
    np.testing.assert_array_equal(rb.sorted_pair[:P].cpu().numpy(), sp_o)
    np.testing.assert_array_equal(rb.pair_pos[:P].cpu().numpy(), pp_o)
    assert np.abs(rb.topk_gates[:P].cpu().numpy() - gates_o.ravel()).max() <= 2e-6
    _, _, yref, _ = oracle.layer_from_weights(x.float().cpu().numpy(), lg, w, weights)
    yg = y.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(yg).all()
    err = np.abs(yg - yref).max()
    scale = np.abs(yref).max()
    print(f"  max|err|/max|ref| = {err / scale:.3e}", flush=True)
    assert err <= TOL[w.dtype] * scale
    layer.close()
