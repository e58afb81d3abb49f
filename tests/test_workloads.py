"""The seeded input generator: determinism, distributions, calibration."""
import numpy as np
import pytest
import torch

import oracle
import workloads


def test_small_tensors_are_deterministic():
    w = workloads.STARVED_DECODE
    a = workloads.router_logits(w)
    b = workloads.router_logits(w)
    np.testing.assert_array_equal(a, b)
    assert a.dtype == np.float32 and a.shape == (w.T, w.E)
    x1, l1 = workloads.make_activations(w)
    assert x1.dtype == torch.bfloat16 and x1.shape == (w.T, w.H)
    x2, _ = workloads.make_activations(w)
    assert torch.equal(x1, x2)
    # a shorter batch is a prefix of the longer one
    np.testing.assert_array_equal(workloads.router_logits(w, T=3), a[:3])


def test_bias_distributions():
    w = workloads.STARVED_DECODE
    b = workloads.expert_bias(w).astype(np.float64)
    assert abs(b.var() - 0.5) < 0.2 and abs(b.mean()) < 0.25
    z = workloads.expert_bias(workloads.AGGREGATED)
    assert sorted(np.round(np.exp(-z / (workloads.ZIPF_ALPHA_AGGREGATED * 1.1)))) == list(range(1, 129))


@pytest.mark.parametrize("w", [workloads.AGGREGATED, workloads.FP8_DSV3], ids=lambda w: w.name)
def test_zipf_calibration_gives_about_4x_hottest_load(w):
    ids, _ = oracle.route(workloads.router_logits(w), w.k)
    counts = np.bincount(ids.ravel(), minlength=w.E)
    ratio = counts.max() / (w.T * w.k / w.E)
    assert 3.8 <= ratio <= 4.2


def test_weights_deterministic_and_scaled():
    w = workloads.TINY
    a = workloads.make_weights(w)
    b = workloads.make_weights(w)
    assert torch.equal(a["w_gu"], b["w_gu"]) and torch.equal(a["w_d"], b["w_d"])
    assert a["w_gu"].shape == (w.E, w.H, 2 * w.M) and a["w_d"].shape == (w.E, w.M, w.H)
    assert abs(a["w_gu"].float().var().item() * w.H - 1) < 0.05
    assert abs(a["w_d"].float().var().item() * w.M - 1) < 0.05


def test_fp8_weight_encoding():
    import dataclasses
    w = dataclasses.replace(workloads.FP8_DSV3, E=2, H=256, M=256, Ms=128, T=4)
    d = workloads.make_weights(w)
    assert d["w_gu"].dtype == torch.float8_e4m3fn and d["s_gu"].shape == (2, 2, 4)
    assert d["ws_gu"].shape == (256, 256) and d["ss_d"].shape == (1, 2)
    # every block uses the full e4m3 range: its largest code is +-448
    q = d["w_gu"][0].float().view(2, 128, 4, 128).abs().amax(dim=(1, 3))
    assert torch.all(q == 448.0)
