"""The work model bench.py reports against (CPU): algorithmic bytes, FLOPs and peaks.

Pinned to the figures of the measurement plan, which come from the layer shapes and
the FLOP formula 6 * B * H * M of the omica.com.cn AFD article (section 2.1):
the fp8 DeepSeek-V3-like layer moves ~11.44 GB when all 256 experts are touched and
does ~3.25e12 FLOPs; the starved-decode layer ~1.41 GB at ~37 touched experts; the
ridge points are ~312 FLOP/B (bf16) and ~625 (fp8) at 8 TB/s.
"""
import numpy as np

import bench
import workloads


def test_peaks_are_the_published_mi355x_figures():
    assert bench.HBM_PEAK_GBS == 8000.0
    assert bench.MFMA_PEAK_TFLOPS == {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
    ridge_bf16 = bench.MFMA_PEAK_TFLOPS["bf16"] * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    ridge_fp8 = bench.MFMA_PEAK_TFLOPS["fp8"] * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    assert round(ridge_bf16) == 312 and round(ridge_fp8) == 625


def test_fp8_layer_bytes_and_flops():
    w = workloads.FP8_DSV3
    counts = np.full(w.E, 1, np.int64)  # every expert touched
    nbytes, touched = bench.algorithmic_bytes(w, counts)
    assert touched == 256
    # weights: 3*H*M bytes per expert plus one fp32 scale per 128x128 block; shared
    # expert 3*H*Ms; bf16 x in and y out; fp32 logits
    per_expert = 3 * 7168 * 2048 + (3 * 7168 * 2048 // 16384) * 4
    assert nbytes == 256 * per_expert + 3 * 7168 * 2048 + 4096 * 7168 * 4 + 4 * 4096 * 256
    assert abs(nbytes / 11.44e9 - 1) < 0.01
    assert abs(w.flops() / 3.25e12 - 1) < 0.01
    assert w.flops() == 6 * 4096 * 8 * 7168 * 2048 + 6 * 4096 * 7168 * 2048


def test_decode_layer_bytes_count_only_touched_experts():
    w = workloads.STARVED_DECODE
    counts = np.zeros(w.E, np.int64)
    counts[:37] = 1
    nbytes, touched = bench.algorithmic_bytes(w, counts)
    assert touched == 37
    assert nbytes == 37 * 3 * 4096 * 1536 * 2 + 6 * 4096 * 2 * 2 + 4 * 6 * 128
    assert abs(nbytes / 1.41e9 - 1) < 0.02
    # gate/up launch: 2*H*M weights per touched expert, x in, h out
    assert bench.gate_up_bytes(w, counts) == 37 * 2 * 4096 * 1536 * 2 + 6 * 4096 * 2 + 48 * 1536 * 2
    # an untouched expert costs nothing
    counts[0] = 0
    assert bench.algorithmic_bytes(w, counts)[0] == nbytes - 3 * 4096 * 1536 * 2


def test_flops_are_six_hm_per_pair_plus_shared():
    for w in workloads.ORDERED + workloads.CONTEXT + workloads.SHARES:
        assert w.flops() == 6 * w.T * w.k * w.H * w.M + 6 * w.T * w.H * w.Ms


def test_fp8_gate_up_launch_bytes_count_codes_and_scales():
    """The fp8 gate/up launch reads e4m3 x codes with one fp32 scale per 128 channels and
    writes h the same way; weights are codes plus one fp32 scale per 128x128 block."""
    w = workloads.FP8_DSV3
    counts = np.ones(w.E, np.int64)
    T, H, M, Ms, P = 4096, 7168, 2048, 2048, 4096 * 8
    want = (256 * (2 * H * M + 56 * 32 * 4) + 2 * H * Ms + 56 * 32 * 4 + T * H + T * 56 * 4
            + (P * M + T * Ms) + (P * 16 + T * 16) * 4)
    assert bench.gate_up_bytes(w, counts) == want
    assert abs(want / 7.70e9 - 1) < 0.01


def test_gate_up_kernel_names_match_the_kernels_the_library_defines():
    """The names bench.py matches against rocprofv3's kernel names (for the committed
    traffic counters) are instances of kernels defined in the listed sources, with one
    template argument per template parameter: a renamed or re-templated kernel would
    leave the counters unmatched."""
    import os
    import re
    csrc = os.path.join(os.path.dirname(bench.__file__), "moe_expert_ffn_softmax_amd", "csrc")
    for name, files in bench.KERNEL_SOURCES.items():
        base, args = re.fullmatch(r"(\w+)<(.*)>", name).groups()
        src = open(os.path.join(csrc, files[0])).read()
        m = re.search(r"template <([^>]*)>\s*__global__ void (?:__launch_bounds__\([^)]*\) )?" + base + r"\(", src)
        assert m, name
        assert len(args.split(",")) == len(m.group(1).split(",")), name
    seen = {bench.gate_up_kernel(w) for w in workloads.ORDERED + workloads.CONTEXT}
    assert seen <= set(bench.KERNEL_SOURCES)
