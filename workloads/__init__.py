"""Seeded synthetic workloads for one MoE layer's expert FFN (the FFN side of
Attention-FFN disaggregation).

This module only *generates inputs*: shapes, value distributions and dtype
encodings of the tensors that both the HIP library and the CPU oracle consume.
It holds none of the layer's arithmetic (no routing, no top-k, no FFN, no
activation quantisation), and neither the oracle nor the library imports it.

Shapes and distributions follow the pages' workloads:
  * "大模型推理的内存与计算解耦：AFD 架构解析与性能验证", §1 (decode batch B=395 at
    2K context falling to B=6 at 128K on a Qwen3-235B-A22B-FP8 model) and §3 (several
    attention instances feed one FFN instance, so the FFN sees their summed batch);
  * the omica.com.cn AFD article, §2.1 and §3.2 (DeepSeek-V3 M=2048, 256 experts,
    top-8; Step3 M=5120, 48 experts, top-3).
No page gives weights or routing traces; every tensor here is synthetic.

Conventions (the pages leave them open):
  * N(0, v): the second parameter is the variance, so W ~ N(0, 1/fan_in) with
    fan_in = H for the gate/up projection and M for the down projection.
  * W_gate_up[e] is [H, 2M]; columns [0, M) are the gate projection, [M, 2M) the up
    projection.
  * Router logits are fp32; a per-expert bias is added to the logits once.
  * fp8 weights: OCP e4m3 ("e4m3fn") with one fp32 scale per 128x128 block,
    scale = amax/448 (1 for an all-zero block); the cast rounds to nearest even.
  * Seeds: numpy SeedSequence(0xAFD, spawn_key=(workload index, tensor id, expert)).
    Small tensors (logits, bias, x) come from numpy's PCG64 and are identical on
    every machine; weights come from torch's generator on the target device (fast
    on a GPU) seeded from the same SeedSequence, one generator per expert.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

ROOT_SEED = 0xAFD
FP8_MAX = 448.0
FP8_BLOCK = 128

# tensor ids inside the spawn key
_T_X, _T_LOGITS, _T_BIAS, _T_ZIPF_PERM, _T_WGU, _T_WD, _T_WSGU, _T_WSD = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed stream of this workload
    T: int              # tokens in the batch
    H: int              # hidden size
    M: int              # expert intermediate size
    E: int              # routed experts
    k: int              # experts per token
    Ms: int             # shared-expert intermediate size (0 = none)
    dtype: str          # "f32" | "bf16" | "fp8"
    bias: Optional[str] = None      # None | "normal" | "zipf"
    bias_param: float = 0.0         # variance for "normal", exponent s for "zipf"
    zipf_alpha: float = 1.0         # calibration factor on the Zipf log-bias
    note: str = ""

    @property
    def pairs(self) -> int:
        return self.T * self.k

    @property
    def tokens_per_expert(self) -> float:
        return self.T * self.k / self.E

    def flops(self) -> int:
        """6 FLOPs per hidden x intermediate element per routed token-expert pair
        (2 for each of the gate, up and down products), plus the shared expert."""
        return 6 * self.T * self.k * self.H * self.M + 6 * self.T * self.H * self.Ms

    def with_tokens(self, T: int, suffix: str = "") -> "Workload":
        return dataclasses.replace(self, T=T, name=self.name + (suffix or f"@T{T}"))


# Calibrated Zipf factors: with the fixed seeds below, the hottest expert receives
# 3.8x-4.2x the mean load (T*k/E).  They were found by bisection with
# tests/golden/zipf_alpha.py, which routes with the oracle only; the test
# tests/test_workloads.py re-checks the load ratio with the oracle.
ZIPF_ALPHA_AGGREGATED = 0.1887
ZIPF_ALPHA_FP8 = 0.1495

WORKLOADS: Dict[str, Workload] = {}


def _add(w: Workload) -> Workload:
    WORKLOADS[w.name] = w
    return w


TINY = _add(Workload(
    "tiny_f32_T64_H256_M512_E8_k2", 0, T=64, H=256, M=512, E=8, k=2, Ms=0, dtype="f32",
    note="small all-fp32 case the oracle finishes in well under a second"))
STARVED_DECODE = _add(Workload(
    "starved_decode_bf16_T6_H4096_M1536_E128_k8", 1, T=6, H=4096, M=1536, E=128, k=8, Ms=0,
    dtype="bf16", bias="normal", bias_param=0.5,
    note="Qwen3-235B-A22B-like layer at 128K context: decode batch of 6, weight streaming"))
AGGREGATED = _add(Workload(
    "afd_aggregated_bf16_T1580_H4096_M1536_E128_k8", 2, T=1580, H=4096, M=1536, E=128, k=8,
    Ms=0, dtype="bf16", bias="zipf", bias_param=1.1, zipf_alpha=ZIPF_ALPHA_AGGREGATED,
    note="4 attention instances x 395 decode tokens gathered on one FFN instance"))
COARSE = _add(Workload(
    "coarse_experts_bf16_T2048_H7168_M5120_E48_k3_shared5120", 3, T=2048, H=7168, M=5120, E=48,
    k=3, Ms=5120, dtype="bf16",
    note="Step-3-like coarse experts with one always-on shared expert"))
FP8_DSV3 = _add(Workload(
    "fp8_blockscaled_T4096_H7168_M2048_E256_k8_shared2048", 4, T=4096, H=7168, M=2048, E=256,
    k=8, Ms=2048, dtype="fp8", bias="zipf", bias_param=1.1, zipf_alpha=ZIPF_ALPHA_FP8,
    note="DeepSeek-V3-like layer, fp8 e4m3 weights with 128x128 block scales"))

ORDERED = [TINY, STARVED_DECODE, AGGREGATED, COARSE, FP8_DSV3]

# The fp8 DeepSeek-V3-like layer at a starved decode batch (the fp8 end of the MFU
# collapse the AFD lecture notes describe in their first section), with the decode
# layer's per-expert logit bias N(0, 0.5).  A measured context case, not one of the
# five layer configurations above.
FP8_DECODE = _add(Workload(
    "fp8_decode_T6_H7168_M2048_E256_k8_shared2048", 5, T=6, H=7168, M=2048, E=256, k=8, Ms=2048,
    dtype="fp8", bias="normal", bias_param=0.5,
    note="DeepSeek-V3-like fp8 layer at a decode batch of 6: weight streaming"))
CONTEXT = [FP8_DECODE]

# One GPU's share of a layer sharded over 8 GPUs of a node (measured here on one GPU,
# at its real shape):
#  * expert parallelism over 8 GPUs for the DeepSeek-V3-like fp8 layer: a GPU owns 32
#    of the 256 experts and, after the dispatch exchange, runs the grouped GEMMs on
#    the ~T*k/8 = 4096 token rows routed to them, each row to one local expert
#    (top-1 over the local experts; the weighted sum over a token's k rows happens on
#    the token's owner after the return exchange).  The local routing is uniform.
#  * tensor parallelism over 4 GPUs inside the experts of the starved-decode layer: a
#    GPU holds M/4 = 384 of the 1536 intermediate columns of every expert and runs the
#    whole routing (the same logits as the full layer: same seed stream) on the same 6
#    tokens; a reduce-scatter of y ends the layer.  (Over 8 GPUs the share would be
#    M = 192, which the kernels' 128-column blocking does not divide.)
EP8_SHARE = _add(Workload(
    "fp8_ep8_share_T4096_H7168_M2048_E32_k1", 6, T=4096, H=7168, M=2048, E=32, k=1, Ms=0, dtype="fp8",
    note="one GPU's share of the DeepSeek-V3-like fp8 layer under 8-way expert parallelism"))
TP4_SHARE = _add(Workload(
    "starved_decode_tp4_share_bf16_T6_H4096_M384_E128_k8", 1, T=6, H=4096, M=384, E=128, k=8, Ms=0,
    dtype="bf16", bias="normal", bias_param=0.5,
    note="one GPU's share of the starved-decode layer under 4-way tensor parallelism in the experts"))
SHARES = [EP8_SHARE, TP4_SHARE]


def mfma_sweep(dtype: str = "bf16"):
    """Token-count sweep at 256/512/1024 routed tokens per expert (the regime where the
    expert GEMMs become compute-bound), on the aggregated-batch shapes for bf16 and on
    the fp8 shapes without the shared expert for fp8."""
    out = []
    if dtype == "bf16":
        base = dataclasses.replace(AGGREGATED, bias=None, zipf_alpha=1.0, index=10)
        for T in (4096, 8192, 16384):
            out.append(dataclasses.replace(base, T=T, name=f"sweep_bf16_T{T}_H4096_M1536_E128_k8"))
    else:
        base = dataclasses.replace(FP8_DSV3, bias=None, zipf_alpha=1.0, Ms=0, index=11)
        for T in (8192, 16384, 32768):
            out.append(dataclasses.replace(base, T=T, name=f"sweep_fp8_T{T}_H7168_M2048_E256_k8"))
    return out


def get(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    for w in mfma_sweep("bf16") + mfma_sweep("fp8"):
        if w.name == name:
            return w
    raise KeyError(name)


# ----------------------------------------------------------------------------- seeds
def _seq(w: Workload, tensor: int, expert: int = 0) -> np.random.SeedSequence:
    return np.random.SeedSequence(ROOT_SEED, spawn_key=(w.index, tensor, expert))


def _np_rng(w: Workload, tensor: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_seq(w, tensor, expert)))


def _torch_seed(w: Workload, tensor: int, expert: int) -> int:
    return int(_seq(w, tensor, expert).generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)


# ----------------------------------------------------------------------------- small tensors
def expert_bias(w: Workload, T: Optional[int] = None) -> np.ndarray:
    """Per-expert logit bias [E] (float32) or zeros."""
    if w.bias is None:
        return np.zeros(w.E, np.float32)
    if w.bias == "normal":
        return (_np_rng(w, _T_BIAS).standard_normal(w.E) * math.sqrt(w.bias_param)).astype(np.float32)
    if w.bias == "zipf":
        # Zipf(s) popularity over a seeded ranking of the experts: the expert with rank r
        # gets prior weight r^-s, i.e. a log-bias of -s*ln(r), scaled by the calibration
        # factor alpha.
        ranks = _np_rng(w, _T_ZIPF_PERM).permutation(w.E) + 1
        return (w.zipf_alpha * (-w.bias_param) * np.log(ranks.astype(np.float64))).astype(np.float32)
    raise ValueError(w.bias)


def router_logits(w: Workload, T: Optional[int] = None, alpha: Optional[float] = None, batch: int = 0) -> np.ndarray:
    """fp32 logits [T, E] = N(0,1) + per-expert bias (added in fp32).  `batch` selects
    an independent draw of the N(0,1) part (the bias is a property of the layer)."""
    T = w.T if T is None else T
    base = _np_rng(w, _T_LOGITS, batch).standard_normal((T, w.E), dtype=np.float32)
    if alpha is not None:
        w = dataclasses.replace(w, zipf_alpha=alpha)
    return (base + expert_bias(w)[None, :]).astype(np.float32)


def tokens_f32(w: Workload, T: Optional[int] = None, batch: int = 0) -> np.ndarray:
    """Token activations x ~ N(0,1) as float32 [T, H] (before the dtype cast)."""
    T = w.T if T is None else T
    return _np_rng(w, _T_X, batch).standard_normal((T, w.H), dtype=np.float32)


# ----------------------------------------------------------------------------- tensors on a device
def _fp8_blockwise(wf32, torch):
    """Encode a [R, C] fp32 matrix as OCP e4m3 with one fp32 scale per 128x128 block."""
    R, C = wf32.shape
    blocks = wf32.reshape(R // FP8_BLOCK, FP8_BLOCK, C // FP8_BLOCK, FP8_BLOCK)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (blocks / scale[:, None, :, None]).to(torch.float8_e4m3fn)
    return q.reshape(R, C), scale.to(torch.float32).contiguous()


def _gen_matrix(w: Workload, tensor: int, expert: int, rows: int, cols: int, fan_in: int, device, torch):
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(w, tensor, expert))
    m = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    return m.mul_(1.0 / math.sqrt(fan_in))


def make_weights(w: Workload, device="cpu"):
    """Expert (and shared-expert) weights on `device`.

    Returns a dict with w_gu [E,H,2M], w_d [E,M,H] in the workload dtype
    (float32 / bfloat16 / float8_e4m3fn), s_gu [E,H/128,2M/128] and s_d [E,M/128,H/128]
    fp32 block scales (fp8 only, else None), and ws_gu [H,2Ms], ws_d [Ms,H], ss_gu, ss_d
    for the shared expert (None when Ms == 0)."""
    import torch
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[w.dtype]
    E, H, M, Ms = w.E, w.H, w.M, w.Ms
    out = {"w_gu": torch.empty((E, H, 2 * M), dtype=dt, device=device),
           "w_d": torch.empty((E, M, H), dtype=dt, device=device),
           "s_gu": None, "s_d": None, "ws_gu": None, "ws_d": None, "ss_gu": None, "ss_d": None}
    if w.dtype == "fp8":
        out["s_gu"] = torch.empty((E, H // FP8_BLOCK, 2 * M // FP8_BLOCK), dtype=torch.float32, device=device)
        out["s_d"] = torch.empty((E, M // FP8_BLOCK, H // FP8_BLOCK), dtype=torch.float32, device=device)

    def store(dst, sdst, idx, m):
        if w.dtype == "fp8":
            q, s = _fp8_blockwise(m, torch)
            dst[idx].copy_(q)
            sdst[idx].copy_(s)
        else:
            dst[idx].copy_(m.to(dt))

    for e in range(E):
        store(out["w_gu"], out["s_gu"], e, _gen_matrix(w, _T_WGU, e, H, 2 * M, H, device, torch))
        store(out["w_d"], out["s_d"], e, _gen_matrix(w, _T_WD, e, M, H, M, device, torch))
    if Ms:
        gu = _gen_matrix(w, _T_WSGU, 0, H, 2 * Ms, H, device, torch)
        dn = _gen_matrix(w, _T_WSD, 0, Ms, H, Ms, device, torch)
        if w.dtype == "fp8":
            out["ws_gu"], out["ss_gu"] = _fp8_blockwise(gu, torch)
            out["ws_d"], out["ss_d"] = _fp8_blockwise(dn, torch)
        else:
            out["ws_gu"], out["ws_d"] = gu.to(dt).contiguous(), dn.to(dt).contiguous()
    return out


def make_activations(w: Workload, device="cpu", T: Optional[int] = None, batch: int = 0):
    """x [T,H] (float32 for f32 workloads, bfloat16 otherwise) and fp32 logits [T,E]
    of batch number `batch` (batch 0 is the workload's reference batch)."""
    import torch
    T = w.T if T is None else T
    x = torch.from_numpy(tokens_f32(w, T, batch))
    x = x if w.dtype == "f32" else x.to(torch.bfloat16)
    logits = torch.from_numpy(router_logits(w, T, batch=batch))
    return x.to(device), logits.to(device)


def fp8_bytes(t):
    """Raw e4m3 codes of a float8 tensor as uint8 (a view, no conversion)."""
    import torch
    return t.view(torch.uint8)
