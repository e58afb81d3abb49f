"""Benchmark of one MoE layer's expert FFN (route + forward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--launch graph|eager]
                    [--no-cpu] [--no-context]

A step is one pass of the whole layer -- router, permute, fp8 quantisation of x,
gate/up GEMM + SwiGLU, down GEMM (+ shared expert), combine -- over one batch already
resident in HBM.  The default workload is the DeepSeek-V3-like layer, the largest
configuration that fits one GPU: T=4096 tokens, H=7168, M=2048, 256 experts, top-8,
a shared expert of 2048, e4m3 weights with 128x128 fp32 block scales, activations
quantised per token per 128 channels.  Steps cycle over a ring of independently
drawn batches, replayed from captured HIP graphs (the production launch form).

Prints one JSON line: tokens/s of the whole job, TFLOPS, the roofline of the
dominant kernel (the gate/up GEMM; HIP events around each launch on the launch
stream; HBM traffic from committed rocprofv3 counters when they were taken on the
current kernel sources), the CPU oracle timed on a bounded token sample of the same
workload, and under "context" the starved-decode layer (T=6, the HBM-bound regime)
and the 1024-tokens-per-expert bf16 and fp8 batches (the matrix-core regime).

--copy-calibration runs only a 1 GiB device-to-device copy (a kernel of known
traffic, used to scale rocprofv3's FETCH_SIZE / WRITE_SIZE counters).
--pmc-summary turns the rocprofv3 counter CSVs of a workload's runs into its entry of
profiles/traffic_counters.json.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "MoE-layer tokens/sec and TFLOPS at 1 GPU; % of HBM or MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
PMC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=workloads.FP8_DSV3.name)
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's batch size T (same layer, same input distributions)")
    ap.add_argument("--batches", type=int, default=0,
                    help="distinct resident batches cycled over the steps (default 16 up to 64 tokens, else 4)")
    ap.add_argument("--launch", default="graph", choices=["graph", "eager"],
                    help="timed steps replayed from captured HIP graphs (default) or launched eagerly")
    ap.add_argument("--graph", action="store_true", help="same as --launch graph (kept for old command lines)")
    ap.add_argument("--no-context", action="store_true",
                    help="only the headline workload: skip the decode and matrix-core records")
    ap.add_argument("--gemm", default="auto", choices=["auto", "stream", "tiled", "fused"],
                    help="grouped-GEMM kernel: automatic choice, 16-row streaming tiles or 128-row tiles")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--attainable", action="store_true",
                    help="measured HBM read rates (the streaming GEMM's pattern, a device copy) and matrix-core rates "
                         "on random operands, from the in-tree probes; not the benchmark line")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write the gate/up launch's HBM bytes of --workload into profiles/traffic_counters.json "
                         "from rocprofv3 counter_collection CSVs")
    ap.add_argument("--sweep", action="store_true",
                    help="one JSON line per workload: every layer shape plus the 256/512/1024 tokens-per-expert "
                         "bf16 and fp8 sweeps (HBM and MFMA fractions); not the benchmark line")
    ap.add_argument("--only", default="", help="with --sweep: run the workloads whose name contains this text")
    ap.add_argument("--ubatches", action="store_true",
                    help="one JSON line per workload: the batch as one call vs split in two micro-batches, "
                         "serial or with the second's routing on a second stream under the first's forward; "
                         "not the benchmark line")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="the starved-decode layer shape (Qwen3-235B-A22B-like) in bf16 and fp8 at batch sizes "
                         "6..1580: tokens/s, matrix-core utilisation (MFU) and HBM fraction per batch size")
    ap.add_argument("--router-proj", action="store_true",
                    help="one JSON line per workload shape: the router projection of afd_ffn_route_hidden "
                         "(logits = x W_r^T + bias) timed alone, with its roofline; not the benchmark line")
    ap.add_argument("--capacity", action="store_true",
                    help="one JSON line per workload shape: capacity-aware routing (afd_ffn_route_capacity) of the "
                         "routed batch at capacity factors 1.25 and unlimited, timed alone; not the benchmark line")
    return ap.parse_args()


def weight_bytes(w):
    return {"f32": 4, "bf16": 2, "fp8": 1}[w.dtype]


def algorithmic_bytes(w, counts):
    """Bytes the layer must move: each touched expert's weights once (+ fp8 scales),
    the shared expert, x in, y out and the fp32 logits."""
    wb = weight_bytes(w)
    touched = int((counts > 0).sum())
    per_expert = 3 * w.H * w.M * wb + (3 * w.H * w.M // (128 * 128) * 4 if w.dtype == "fp8" else 0)
    shared = 3 * w.H * w.Ms * wb
    act = 4 if w.dtype == "f32" else 2
    return touched * per_expert + shared + w.T * w.H * 2 * act + 4 * w.T * w.E, touched


def gate_up_bytes(w, counts):
    """Algorithmic bytes of one gate/up launch: 2*H*M weights per touched expert (+ the
    shared expert's 2*H*Ms), x in and h out, in the forms the launch reads and writes:
    bf16 (fp32 in the fp32 layer), or for the fp8 layer e4m3 codes plus one fp32 scale
    per 128 (weights: per 128x128 block; x and h: per row and 128 channels)."""
    touched = int((counts > 0).sum())
    T, H, M, Ms, P = w.T, w.H, w.M, w.Ms, w.T * w.k
    if w.dtype == "fp8":
        wts = touched * (2 * H * M + (H // 128) * (2 * M // 128) * 4) + \
            (2 * H * Ms + (H // 128) * (2 * Ms // 128) * 4 if Ms else 0)
        return wts + T * H * (1 + 4 / 128) + (P * M + T * Ms) * (1 + 4 / 128)
    wb = weight_bytes(w)
    act = 4 if w.dtype == "f32" else 2
    return touched * 2 * H * M * wb + 2 * H * Ms * wb + T * H * act + (P * M + T * Ms) * act


def down_bytes(w, counts):
    """Algorithmic bytes of one down launch (bf16/fp32 layers): H*M weights per touched
    expert (+ the shared expert's H*Ms), h in, the expert output rows out."""
    touched = int((counts > 0).sum())
    T, H, M, Ms, P = w.T, w.H, w.M, w.Ms, w.T * w.k
    wb = weight_bytes(w)
    act = 4 if w.dtype == "f32" else 2
    return touched * H * M * wb + H * Ms * wb + (P * M + T * Ms) * act + (P * H + (T * H if Ms else 0)) * act


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}))


# Device sources each gate/up kernel is built from: committed counters of a kernel
# stay valid while these files are unchanged.
KERNEL_SOURCES = {
    "gemm_bf16_stream_kernel<true>": ("gemm_bf16.hip", "grouped.h", "afd_device.h", "afd_internal.h"),
    "gemm_bf16_tiled_kernel<true>": ("gemm_bf16_tiled.hip", "grouped.h", "afd_device.h", "afd_internal.h"),
    "gemm_fp8_stream_kernel<true>": ("gemm_fp8.hip", "grouped.h", "afd_device.h", "afd_internal.h"),
    "gemm_fp8_tiled_kernel<true, false>": ("gemm_fp8_tiled.hip", "grouped.h", "afd_device.h", "afd_internal.h"),
    "gemm_f32_kernel<true>": ("gemm_f32.hip", "grouped.h", "afd_device.h", "afd_internal.h"),
}


def gate_up_kernel(w, gemm="auto"):
    """Name of the gate/up kernel the layer launches for workload w (the automatic
    choice: 16-row streaming tiles up to 8 rows per expert in bf16, 12 in fp8)."""
    if w.dtype == "f32":
        return "gemm_f32_kernel<true>"
    tiled = gemm == "tiled" or (gemm == "auto" and w.T * w.k > (12 if w.dtype == "fp8" else 8) * w.E)
    if w.dtype == "fp8" and tiled:
        return "gemm_fp8_tiled_kernel<true, false>"  # <SWIGLU, CHAIN>: gate/up items are not chained
    return f"gemm_{w.dtype}_{'tiled' if tiled else 'stream'}_kernel<true>"


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_expert_ffn_softmax_amd", "csrc")
    for f in sorted(files):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_counters(w, gemm="auto"):
    """HBM bytes per gate/up launch from committed rocprofv3 counter runs, if they were
    taken on this workload with the kernel that runs now, built from the current
    sources; else None."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(w.name, {}).get("gate_up")
    kern = gate_up_kernel(w, gemm)
    if not e or e.get("kernel") != kern or e.get("source_digest") != source_digest(KERNEL_SOURCES[kern]):
        return None
    return e.get("bytes_per_launch")


def _counter_means(path, name_filter=None):
    """{kernel name: (dispatches, mean Counter_Value)} of a rocprofv3 counter_collection CSV."""
    import collections
    import csv
    acc = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            n = r["Kernel_Name"]
            if name_filter and name_filter not in n:
                continue
            acc[n].append(float(r["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v)) for k, v in acc.items()}


def pmc_summary(args):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the workload's gate/up launch
    by what the same counters read for a 1 GiB copy, and record the bytes per launch
    with the digest of the kernel's sources."""
    w = workloads.get(args.workload)
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.pmc_summary
    kern = gate_up_kernel(w, args.gemm)
    n = 1 << 30
    cf, cw = _counter_means(cfetch_csv), _counter_means(cwrite_csv)
    copy = max(cf, key=lambda k: cf[k][1])   # the copy is the largest fetch of that run
    fetch_scale = round(n / 1024 / cf[copy][1], 4)
    write_scale = round(n / 1024 / cw[copy][1], 4)
    f, wr = _counter_means(fetch_csv, "afd::"), _counter_means(write_csv, "afd::")
    key = next(k for k in f if kern in k)
    nbytes = int(f[key][1] * 1024 * fetch_scale + wr[key][1] * 1024 * write_scale)
    try:
        with open(PMC_FILE) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        d = {}
    d.setdefault(w.name, {})["gate_up"] = {
        "kernel": kern, "sources": sorted(KERNEL_SOURCES[kern]), "source_digest": source_digest(KERNEL_SOURCES[kern]),
        "bytes_per_launch": nbytes, "fetch_kib": round(f[key][1], 1), "write_kib": round(wr[key][1], 1),
        "dispatches": f[key][0], "fetch_scale": fetch_scale, "write_scale": write_scale}
    with open(PMC_FILE, "w") as fh:
        json.dump(d, fh, indent=1)
        fh.write("\n")
    rows = [f"| {k} | {f[k][0]} | {f[k][1]:.1f} | {wr.get(k, (0, 0.0))[1]:.1f} | "
            f"{(f[k][1] * 1024 * fetch_scale + wr.get(k, (0, 0.0))[1] * 1024 * write_scale) / 1e6:.2f} |"
            for k in sorted(f, key=lambda k: -f[k][1])]
    print(json.dumps(d[w.name]["gate_up"]))
    print("| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | scaled HBM bytes per dispatch (MB) |")
    print("|---|---|---|---|---|")
    print("\n".join(rows))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class HostExperts:
    """Host copies of a workload's per-expert weights, made on first use (not timed)."""

    def __init__(self, weights):
        self.weights = weights
        self.host = {k: (v.cpu() if v is not None else None) for k, v in weights.items()
                     if k not in ("w_gu", "w_d", "s_gu", "s_d")}
        for k in ("w_gu", "w_d", "s_gu", "s_d"):
            self.host[k] = {} if weights[k] is not None else None

    def need(self, experts):
        for k in ("w_gu", "w_d", "s_gu", "s_d"):
            if self.host[k] is not None:
                for e in experts:
                    if int(e) not in self.host[k]:
                        self.host[k][int(e)] = self.weights[k][int(e)].cpu()
        return self.host


def oracle_rate(w, hx, tokens, seconds, nthreads, chunk):
    """Oracle tokens/s on the rows of `tokens` = (x, logits) [bf16-exact fp32, fp32],
    `chunk` tokens per call, cycling until about `seconds` of oracle time; the host
    copies of the experts each chunk needs are made before its timer starts."""
    import oracle
    x, logits = tokens
    n = x.shape[0]
    spent, done, calls = 0.0, 0, 0
    while spent < seconds:
        r0 = (calls * chunk) % n
        xs, ls = x[r0:r0 + chunk], logits[r0:r0 + chunk]
        need = np.unique(oracle.route(ls, w.k)[0])
        host = hx.need(need)
        t0 = time.perf_counter()
        oracle.layer_from_weights(xs, ls, w, host, experts_needed=need, nthreads=nthreads)
        spent += time.perf_counter() - t0
        done += xs.shape[0]
        calls += 1
    return done, spent, calls


def host_tokens(w, batch=0):
    import torch
    x = workloads.tokens_f32(w, batch=batch)
    if w.dtype != "f32":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    return x, workloads.router_logits(w, batch=batch)


def cpu_baseline(w, weights, seconds, single_seconds=3.0, single_workloads=()):
    """The oracle (as it stands) on a bounded token sample of the timed workload: its
    first batch's tokens in calls of up to 64 tokens (whole batches when smaller),
    cycling until about `seconds` of oracle time, on every host core; then about
    `single_seconds` on one thread.  `single_workloads`: (workload, weights) pairs also
    timed on one thread."""
    import oracle
    chunk = min(w.T, 64)
    toks = host_tokens(w)
    hx = HostExperts(weights)
    done, spent, calls = oracle_rate(w, hx, toks, seconds, 0, chunk)
    out = {"value": round(done / spent, 3), "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{done} tokens of the workload's first batch ({calls} oracle calls of {chunk} tokens, the "
                     f"first {min(done, w.T)} tokens cycled), {spent:.1f} s of oracle time on the host, "
                     f"double precision"}
    if single_seconds > 0:
        d1, s1, c1 = oracle_rate(w, hx, toks, single_seconds, 1, min(chunk, 8))
        out["single_thread"] = {"value": round(d1 / s1, 3), "unit": "tokens/s", "cores": 1,
                                "sample": f"{d1} tokens in {c1} calls, {s1:.1f} s on one thread"}
    by = {}
    for sw, sweights in single_workloads:
        sc = min(sw.T, 16)
        d1, s1, c1 = oracle_rate(sw, HostExperts(sweights), host_tokens(sw), single_seconds, 1, sc)
        by[sw.name] = {"value": round(d1 / s1, 3), "unit": "tokens/s", "cores": 1,
                       "sample": f"{d1} tokens in {c1} calls of {sc}, {s1:.1f} s on one thread"}
    if by:
        out["single_thread_by_workload"] = by
    return out


def cold_steps(run, n, torch):
    """Per-step times (ms) of `n` steps, each preceded by a 1 GiB write that evicts the
    L2 caches and the 256 MB MALL; HIP events on the launch stream bracket the step
    alone.  Returns median, p10 and p90."""
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream()
    evs = []
    for i in range(n):
        flush.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        run(i)
        b.record(st)
        evs.append((a, b))
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    del flush
    return {"steps": n, "median_ms": round(float(np.median(t)), 4), "p10_ms": round(float(np.percentile(t, 10)), 4),
            "p90_ms": round(float(np.percentile(t, 90)), 4)}


def run_workload(w, steps, warmup, batches, gemm, torch):
    """Time `steps` route+forward steps of workload `w`; returns a dict of figures."""
    from moe_expert_ffn_softmax_amd import MoeExpertFFN, afd_ffn_profile_read, afd_ffn_set_profiling
    weights = workloads.make_weights(w, device="cuda")
    layer = MoeExpertFFN(hidden=w.H, inter=w.M, num_experts=w.E, top_k=w.k, max_tokens=w.T, dtype=w.dtype,
                         w_gate_up=weights["w_gu"], w_down=weights["w_d"], s_gate_up=weights["s_gu"],
                         s_down=weights["s_d"], shared_inter=w.Ms, ws_gate_up=weights["ws_gu"],
                         ws_down=weights["ws_d"], ss_gate_up=weights["ss_gu"], ss_down=weights["ss_d"])
    layer.set_gemm_kernel(gemm)
    del weights
    ydt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    xs, lgs, ys, rbs = [], [], [], []
    for b in range(batches):
        x, lg = workloads.make_activations(w, device="cuda", batch=b)
        xs.append(x)
        lgs.append(lg)
        ys.append(torch.empty((w.T, w.H), dtype=ydt, device="cuda"))
        rbs.append(layer.new_route())

    def step(i):
        b = i % batches
        layer.route(lgs[b], w.T, rbs[b])
        layer.forward(xs[b], w.T, rbs[b], ys[b])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    afd_ffn_set_profiling(layer.handle, True)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    prof = afd_ffn_profile_read(layer.handle)
    counts = [rb.expert_counts.cpu().numpy() for rb in rbs]
    layer.close()
    step_bytes = float(np.mean([algorithmic_bytes(w, c)[0] for c in counts]))
    tflops = w.flops() / (ms / 1e3) / 1e12
    gbs = step_bytes / (ms / 1e3) / 1e9
    return {"workload": w.name, "dtype": w.dtype, "tokens_per_expert": round(w.tokens_per_expert, 2),
            "ms_per_step": round(ms, 4), "tokens_per_s": round(w.T / (ms / 1e3), 1), "tflops": round(tflops, 2),
            "hbm_GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "mfma_frac": round(tflops / MFMA_PEAK_TFLOPS[w.dtype], 4),
            "kernels_us": {k: round(v[0] / max(v[1], 1) * 1e3, 2) for k, v in prof.items() if v[1]}}


def sweep(args, torch):
    wls = (list(workloads.ORDERED) + list(workloads.CONTEXT) + workloads.mfma_sweep("bf16") +
           workloads.mfma_sweep("fp8") + list(workloads.SHARES))
    for w in wls:
        if args.only and not any(o in w.name for o in args.only.split(",")):
            continue
        steps = args.steps if w.T <= 64 else max(3, min(args.steps, 20))
        r = run_workload(w, steps, min(args.warmup, 3), args.batches or (4 if w.T <= 64 else 2), args.gemm, torch)
        print(json.dumps(r), flush=True)
        torch.cuda.empty_cache()


BATCH_SWEEP_T = (6, 25, 100, 197, 395, 788, 1580)


def batch_sweep(args, torch):
    """One JSON line per (dtype, T): the starved-decode layer's shape at decode batch sizes
    from 6 to 1580 tokens (one attention instance's batch up to four aggregated), with its
    utilisation of the dense matrix-core peak and of HBM."""
    base = workloads.STARVED_DECODE
    for dt in ("bf16", "fp8"):
        for T in BATCH_SWEEP_T:
            w = dataclasses.replace(base, T=T, dtype=dt, name=f"decode_layer_{dt}_T{T}_H4096_M1536_E128_k8")
            steps = args.steps if T <= 64 else max(3, min(args.steps, 50))
            r = run_workload(w, steps, min(args.warmup, 5), args.batches or 8, args.gemm, torch)
            print(json.dumps(r), flush=True)
            torch.cuda.empty_cache()


def router_proj(args, torch):
    """Time the router projection (the first kernel of afd_ffn_route_hidden) on each
    workload's (T, H, E) with seeded synthetic x, gate vectors ~ N(0, 1/H) and bias.
    Algorithmic bytes: W_r and x read once, logits written once; FLOPs 2 T H E."""
    from moe_expert_ffn_softmax_amd import MoeExpertFFN, afd_ffn_profile_read, afd_ffn_set_profiling
    wls = list(workloads.ORDERED) + workloads.mfma_sweep("bf16") + workloads.mfma_sweep("fp8")
    for w in wls:
        if args.only and not any(o in w.name for o in args.only.split(",")):
            continue
        dt = "f32" if w.dtype == "f32" else "bf16"
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        a = 4 if dt == "f32" else 2
        M = 128
        layer = MoeExpertFFN(hidden=w.H, inter=M, num_experts=w.E, top_k=w.k, max_tokens=w.T, dtype=dt,
                             w_gate_up=torch.zeros((w.E, w.H, 2 * M), dtype=tdt, device="cuda"),
                             w_down=torch.zeros((w.E, M, w.H), dtype=tdt, device="cuda"))
        g = torch.Generator(device="cuda").manual_seed(1000 + w.index)
        x = torch.randn((w.T, w.H), generator=g, device="cuda").to(tdt)
        wr = (torch.randn((w.E, w.H), generator=g, device="cuda") / float(np.sqrt(w.H))).to(tdt)
        bias = torch.randn(w.E, generator=g, device="cuda") * 0.01
        logits = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
        rb = layer.new_route()
        steps = args.steps if w.T <= 64 else max(5, min(args.steps, 50))
        for _ in range(min(args.warmup, 5)):
            layer.route_hidden(x, wr, logits, w.T, rb, bias=bias)
        torch.cuda.synchronize()
        afd_ffn_set_profiling(layer.handle, True)
        for _ in range(steps):
            layer.route_hidden(x, wr, logits, w.T, rb, bias=bias)
        torch.cuda.synchronize()
        prof = afd_ffn_profile_read(layer.handle)
        layer.close()
        us = prof["router_proj"][0] / max(prof["router_proj"][1], 1) * 1e3
        nbytes = (w.E * w.H + w.T * w.H) * a + w.T * w.E * 4 + w.E * 4
        flops = 2.0 * w.T * w.H * w.E
        peak_tf = MFMA_PEAK_TFLOPS[dt]
        mfma_bound = flops / (peak_tf * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9)
        if mfma_bound:
            ach, peak, unit = flops / (us * 1e-6) / 1e12, peak_tf, "TFLOP/s"
        else:
            ach, peak, unit = nbytes / (us * 1e-6) / 1e9, HBM_PEAK_GBS, "GB/s"
        route_us = {k: round(v[0] / max(v[1], 1) * 1e3, 2) for k, v in prof.items() if v[1] and k != "router_proj"}
        print(json.dumps({"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "dtype": dt,
                          "router_proj_us": round(us, 2), "bytes": nbytes, "flops": flops,
                          "roofline": {"bound": "mfma" if mfma_bound else "hbm", "achieved": round(ach, 1),
                                       "peak": peak, "unit": unit, "frac": round(ach / peak, 4)},
                          "route_us": route_us}), flush=True)
        del x, wr, logits, rb
        torch.cuda.empty_cache()


def capacity(args, torch):
    """Time capacity-aware routing on each workload's (T, E, k): the preference lists are
    that batch's routing of seeded logits, every expert's limit is ceil(f T / E) for
    capacity factor f = 1.25 (the top-1 share with 25% headroom) or T (room everywhere),
    limits held fixed so every call does the same work.  The walk is sequential by
    definition (one workgroup); its bytes (lists read, outputs written) are reported with
    the time, not a roofline."""
    from moe_expert_ffn_softmax_amd import MoeExpertFFN
    wls = list(workloads.ORDERED) + workloads.mfma_sweep("bf16") + workloads.mfma_sweep("fp8")
    for w in wls:
        if args.only and not any(o in w.name for o in args.only.split(",")):
            continue
        M = 128
        layer = MoeExpertFFN(hidden=128, inter=M, num_experts=w.E, top_k=w.k, max_tokens=w.T, dtype="bf16",
                             w_gate_up=torch.zeros((w.E, 128, 2 * M), dtype=torch.bfloat16, device="cuda"),
                             w_down=torch.zeros((w.E, M, 128), dtype=torch.bfloat16, device="cuda"))
        g = torch.Generator(device="cuda").manual_seed(2000 + w.index)
        logits = torch.randn((w.T, w.E), generator=g, device="cuda")
        rb = layer.new_route()
        layer.route(logits, w.T, rb)
        ids = rb.topk_ids[: w.T * w.k]
        gates = rb.topk_gates[: w.T * w.k]
        out = (torch.empty(w.T, dtype=torch.int32, device="cuda"), torch.empty(w.T, device="cuda"),
               torch.empty(w.E + 1, dtype=torch.int32, device="cuda"),
               torch.empty(w.T, dtype=torch.int32, device="cuda"))
        res = {}
        for name, f in (("cf1.25", 1.25), ("unlimited", None)):
            L = w.T if f is None else -(-int(f * w.T * 4) // (4 * w.E))
            limits = torch.full((w.E,), L, dtype=torch.int32, device="cuda")
            for _ in range(3):
                layer.route_capacity(ids, gates, w.T, limits, 1, False, out=out)
            steps = max(5, min(args.steps, 50))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                layer.route_capacity(ids, gates, w.T, limits, 1, False, out=out)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            kept = int(out[2][w.E].item())
            res[name] = {"limit": L, "us": round(us, 2), "kept": kept, "dropped": w.T - kept,
                         "tokens_per_us": round(w.T / us, 2)}
        layer.close()
        nbytes = w.T * w.k * 8 + w.T * 16 + (w.E + 1) * 4
        print(json.dumps({"workload": w.name, "T": w.T, "E": w.E, "k": w.k, "bytes": nbytes, **res}), flush=True)


def ubatches(args, torch):
    """Two micro-batches in flight on one handle (the two-micro-batch overlap of the
    AFD blog's section 4, on the FFN side): micro-batch 2's route runs on a second stream
    while micro-batch 1's forward runs; both forwards stay on the first stream, which
    owns the handle's workspace.  Compared with the whole batch as one call and with
    the two micro-batches run back to back on one stream."""
    from moe_expert_ffn_softmax_amd import MoeExpertFFN
    wls = list(workloads.ORDERED) + workloads.mfma_sweep("bf16") + workloads.mfma_sweep("fp8")
    for w in wls:
        if args.only and not any(o in w.name for o in args.only.split(",")):
            continue
        weights = workloads.make_weights(w, device="cuda")
        layer = MoeExpertFFN(hidden=w.H, inter=w.M, num_experts=w.E, top_k=w.k, max_tokens=w.T, dtype=w.dtype,
                             w_gate_up=weights["w_gu"], w_down=weights["w_d"], s_gate_up=weights["s_gu"],
                             s_down=weights["s_d"], shared_inter=w.Ms, ws_gate_up=weights["ws_gu"],
                             ws_down=weights["ws_d"], ss_gate_up=weights["ss_gu"], ss_down=weights["ss_d"])
        del weights
        nb = 2
        T1 = (w.T + 1) // 2
        T2 = w.T - T1
        ydt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        xs, lgs, ys = [], [], []
        for b in range(nb):
            x, lg = workloads.make_activations(w, device="cuda", batch=b)
            xs.append(x)
            lgs.append(lg)
            ys.append(torch.empty((w.T, w.H), dtype=ydt, device="cuda"))
        rb0 = [layer.new_route() for _ in range(nb)]
        rb1 = [layer.new_route() for _ in range(nb)]
        rb2 = [layer.new_route() for _ in range(nb)]
        sa = torch.cuda.current_stream()
        sb = torch.cuda.Stream()
        ev_route = [torch.cuda.Event() for _ in range(nb)]
        ev_free = [torch.cuda.Event() for _ in range(nb)]
        for e in ev_free:
            e.record(sa)

        def whole(i):
            b = i % nb
            layer.route(lgs[b], w.T, rb0[b])
            layer.forward(xs[b], w.T, rb0[b], ys[b])

        def serial(i):
            b = i % nb
            layer.route(lgs[b], T1, rb1[b])
            layer.forward(xs[b], T1, rb1[b], ys[b])
            layer.route(lgs[b][T1:], T2, rb2[b])
            layer.forward(xs[b][T1:], T2, rb2[b], ys[b][T1:])

        def overlapped(i):
            b = i % nb
            sb.wait_event(ev_free[b])  # the last forward that read rb2[b] is done
            layer.route(lgs[b][T1:], T2, rb2[b], stream=sb)
            ev_route[b].record(sb)
            layer.route(lgs[b], T1, rb1[b])
            layer.forward(xs[b], T1, rb1[b], ys[b])
            sa.wait_event(ev_route[b])
            layer.forward(xs[b][T1:], T2, rb2[b], ys[b][T1:])
            ev_free[b].record(sa)

        steps = args.steps if w.T <= 64 else max(5, min(args.steps, 20))
        out = {"workload": w.name, "T": w.T, "micro_batches": [T1, T2]}
        for name, fn in (("whole_ms", whole), ("serial_ms", serial), ("overlapped_ms", overlapped),
                         ("whole_ms_again", whole)):
            for i in range(min(args.warmup, 5)):
                fn(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                fn(i)
            torch.cuda.synchronize()
            out[name] = round((time.perf_counter() - t0) * 1e3 / steps, 4)
        layer.close()
        print(json.dumps(out), flush=True)
        del xs, lgs, ys, rb0, rb1, rb2
        torch.cuda.empty_cache()


def attainable(args, torch):
    """What the part attains, measured with the in-tree probes (libafd_probe.so): HBM
    reads in the weight-streaming GEMM's pattern (private runs per wave, 16-byte
    nontemporal loads, a ring of steps in flight), a plain 1 GiB device copy, and
    matrix-core loops on random bf16 and e4m3 operands.  One JSON line per probe; the
    read probes' sums are checked against the buffer's."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "moe_expert_ffn_softmax_amd", "libafd_probe.so"))
    V = ctypes.c_void_p
    lib.afd_probe_stream.argtypes = [V, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, V, V]
    lib.afd_probe_mfma.argtypes = [ctypes.c_int, V, ctypes.c_int, ctypes.c_int, V, V]
    lib.afd_probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, V, V]
    lib.afd_probe_fp8_block.argtypes = [ctypes.c_int, V, ctypes.c_int, ctypes.c_int, V, V, V]
    lib.afd_probe_bf16_block.argtypes = [ctypes.c_int, V, ctypes.c_int, ctypes.c_int, V, V, V]
    st = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3

    KiB = 1024
    cases = [("decode gate/up pattern", 3360, 256 * KiB, 8), ("same runs, 16 steps in flight", 3360, 256 * KiB, 16),
             ("twice the runs, half as long, 16 in flight", 6720, 128 * KiB, 16),
             ("one 4 MiB run per resident wave", 2048, 4096 * KiB, 8)]
    nbytes = max(r * b for _, r, b, _ in cases)
    g = torch.Generator(device="cuda").manual_seed(7)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=g)
    for name, runs, rb, depth in cases:
        out = torch.empty(runs * 256, dtype=torch.int32, device="cuda")

        def run():
            rc = lib.afd_probe_stream(buf.data_ptr(), rb, runs, depth, out.data_ptr(), st.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"afd_probe_stream returned {rc}")
        t = timed(run, args.steps if args.steps <= 50 else 20)
        want = int(buf[: runs * rb // 4].to(torch.int64).sum().item()) % (1 << 32)
        got = int(out.to(torch.int64).sum().item()) % (1 << 32)
        if got != want:
            raise RuntimeError(f"stream probe read the wrong bytes ({got} vs {want})")
        print(json.dumps({"probe": "hbm_read", "pattern": name, "runs": runs, "run_bytes": rb,
                          "steps_in_flight": depth, "bytes": runs * rb, "us": round(t * 1e6, 1),
                          "GBps": round(runs * rb / t / 1e9, 1),
                          "frac_of_8TBps": round(runs * rb / t / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)
    del buf
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    t = timed(lambda: b.copy_(a), 10)
    print(json.dumps({"probe": "device_copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30,
                      "us": round(t * 1e6, 1), "GBps_read_plus_write": round(2 * (1 << 30) / t / 1e9, 1)}),
          flush=True)
    del a, b
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    waves = cus * 8  # two waves per SIMD
    chains = 8       # independent accumulators per wave (the probe's kChains)
    for kind, dt, per, peak, opbytes in ((0, "bf16", 32768, MFMA_PEAK_TFLOPS["bf16"], 16),
                                         (1, "fp8", 65536, MFMA_PEAK_TFLOPS["fp8"], 32)):
        n = waves * 2 * chains * 64 * opbytes
        for operands in ("random", "constant"):
            if kind == 0:
                ops = (torch.randn(n // 2, generator=g, device="cuda") if operands == "random"
                       else torch.full((n // 2,), 0.5, device="cuda")).to(torch.bfloat16)
            else:
                ops = (torch.randn(n, generator=g, device="cuda") if operands == "random"
                       else torch.full((n,), 0.5, device="cuda")).to(torch.float8_e4m3fn).view(torch.uint8)
            out = torch.empty(waves * 64, dtype=torch.float32, device="cuda")
            iters = 2048

            def run():
                rc = lib.afd_probe_mfma(kind, ops.data_ptr(), waves, iters, out.data_ptr(), st.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"afd_probe_mfma returned {rc}")
            t = timed(run, 10)
            flops = waves * iters * chains * per
            print(json.dumps({"probe": "mfma", "instruction": "v_mfma_f32_32x32x16_bf16" if kind == 0 else
                              "v_mfma_f32_16x16x128_f8f6f4", "operands": f"{operands} {dt}", "waves": waves,
                              "chains_per_wave": chains, "flops": flops, "us": round(t * 1e6, 1),
                              "TFLOPs": round(flops / t / 1e12, 1),
                              "frac_of_peak": round(flops / t / 1e12 / peak, 4)}), flush=True)
    # LDS reads in the tiled GEMMs' operand pattern, one 8-wave workgroup per compute unit
    iters = 20000
    cyc = torch.zeros(cus * 8, dtype=torch.int64, device="cuda")

    def run_lds():
        rc = lib.afd_probe_lds(cus, iters, cyc.data_ptr(), st.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"afd_probe_lds returned {rc}")
    t = timed(run_lds, 5)
    per_wg = 8 * 16 * 1024 * iters
    cmax = int(cyc.max().item())
    print(json.dumps({"probe": "lds_read", "pattern": "16-byte reads, one 256-byte slot per 16-lane quarter",
                      "workgroups": cus, "waves_per_cu": 8, "bytes": per_wg * cus, "us": round(t * 1e6, 1),
                      "bytes_per_clk_per_cu": round(per_wg / cmax, 1), "clock_GHz": round(cmax / t / 1e9, 3),
                      "TBps": round(per_wg * cus / t / 1e12, 1)}), flush=True)
    # the fp8 tiled GEMM's inner loop without global memory, piece by piece
    ops = (torch.randn(cus * 8 * 12 * 64 * 32, generator=g, device="cuda")
           .to(torch.float8_e4m3fn).view(torch.uint8))
    out = torch.empty(cus * 8 * 64, dtype=torch.float32, device="cuda")
    cyc = torch.zeros(cus * 8, dtype=torch.int64, device="cuda")
    iters = 512
    names = ("MFMAs accumulating directly, operands in registers", "+ block rescale of the products",
             "+ token operands read from LDS", "+ a chunk's staging writes and barrier every two blocks",
             "the same writes spread over the second block's steps, the barrier at its end",
             "the barrier alone every two blocks, no writes",
             "4 waves of 64 columns: rescale, token operands from LDS",
             "4 waves of 64 columns: + a chunk's staging writes and barrier every two blocks")
    for mode in range(8):
        waves = cus * (4 if mode >= 6 else 8)  # one workgroup per compute unit
        per_wave = 32 if mode >= 6 else 16    # instructions per wave per iteration

        def run_blk():
            rc = lib.afd_probe_fp8_block(mode, ops.data_ptr(), waves, iters, out.data_ptr(), cyc.data_ptr(),
                                         st.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"afd_probe_fp8_block returned {rc}")
        t = timed(run_blk, 10)
        flops = waves * iters * per_wave * 65536
        cmax = int(cyc[:waves].max().item())
        # a SIMD's matrix core gets 32 instructions of 32 cycles per iteration (two waves
        # of 16, or one of 32)
        print(json.dumps({"probe": "fp8_block", "mode": mode, "what": names[mode], "waves": waves,
                          "flops": flops, "us": round(t * 1e6, 1), "TFLOPs": round(flops / t / 1e12, 1),
                          "frac_of_peak": round(flops / t / 1e12 / MFMA_PEAK_TFLOPS["fp8"], 4),
                          "cycles_per_iteration": round(cmax / iters, 1),
                          "matrix_core_busy": round(1024 * iters / cmax, 4),
                          "clock_GHz": round(cmax / t / 1e9, 3)}), flush=True)
    # the bf16 tiled GEMM's inner loop without global memory: one 4-wave workgroup per
    # compute unit (one wave per SIMD), 64 MFMAs of 32 cycles per wave per chunk
    waves = cus * 4
    ops = (torch.randn(waves * 6 * 64 * 8, generator=g, device="cuda").to(torch.bfloat16))
    out = torch.empty(waves * 64, dtype=torch.float32, device="cuda")
    cyc = torch.zeros(waves, dtype=torch.int64, device="cuda")
    iters = 256
    names = ("MFMAs, operands in registers", "+ row blocks' operands read from LDS",
             "+ a chunk's staging writes and barrier")
    for mode in range(3):
        def run_bf():
            rc = lib.afd_probe_bf16_block(mode, ops.data_ptr(), waves, iters, out.data_ptr(), cyc.data_ptr(),
                                          st.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"afd_probe_bf16_block returned {rc}")
        t = timed(run_bf, 10)
        flops = waves * iters * 64 * 32768
        cmax = int(cyc.max().item())
        print(json.dumps({"probe": "bf16_block", "mode": mode, "what": names[mode], "waves": waves,
                          "flops": flops, "us": round(t * 1e6, 1), "TFLOPs": round(flops / t / 1e12, 1),
                          "frac_of_peak": round(flops / t / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4),
                          "cycles_per_chunk": round(cmax / iters, 1),
                          "matrix_core_busy": round(2048 * iters / cmax, 4),
                          "clock_GHz": round(cmax / t / 1e9, 3)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only: this layer is built and measured on a single MI355X "
              f"(got --gpus {args.gpus}); sharding across GPUs is a design note, not a run mode.", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.attainable:
        torch.cuda.set_device(0)
        attainable(args, torch)
        return
    if args.sweep:
        torch.cuda.set_device(0)
        sweep(args, torch)
        return
    if args.router_proj:
        torch.cuda.set_device(0)
        router_proj(args, torch)
        return
    if args.capacity:
        torch.cuda.set_device(0)
        capacity(args, torch)
        return
    if args.batch_sweep:
        torch.cuda.set_device(0)
        batch_sweep(args, torch)
        return
    if args.ubatches:
        torch.cuda.set_device(0)
        ubatches(args, torch)
        return
    w = workloads.get(args.workload)
    if args.tokens > 0 and args.tokens != w.T:
        w = dataclasses.replace(w, T=args.tokens, name=f"{w.name}_at_T{args.tokens}")
    torch.cuda.set_device(0)
    launch = "graph" if args.graph else args.launch
    nb = args.batches or (16 if w.T <= 64 else 4)
    rec, weights = measure(w, torch, args.steps, args.warmup, nb, launch, args.gemm, min(args.steps, 100),
                           keep_weights=not args.no_cpu)
    out = {
        "metric": METRIC,
        "value": rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": rec["config"],
    }
    out.update({k: v for k, v in rec.items() if k not in ("tokens_per_s", "ms_per_step", "config", "workload")})
    if not args.no_context:
        ctx = {}
        for cw in (workloads.STARVED_DECODE, workloads.mfma_sweep("bf16")[-1], workloads.mfma_sweep("fp8")[-1]):
            if cw.name == w.name:
                continue
            small = cw.T <= 64
            r, _ = measure(cw, torch, 200 if small else 10, 20 if small else 3, 16 if small else 2, launch, "auto",
                           0, keep_weights=False)
            ctx[r["config"]["workload"]] = {k: r[k] for k in ("ms_per_step", "tokens_per_s", "tflops", "mfma_frac",
                                                               "step_hbm", "roofline", "kernels_us")}
            torch.cuda.empty_cache()
        out["context"] = ctx
    if not args.no_cpu:
        singles = []
        for sw in (workloads.TINY, workloads.STARVED_DECODE, workloads.AGGREGATED):
            if sw.name != w.name:
                singles.append((sw, workloads.make_weights(sw, device="cuda")))
        out["cpu_baseline"] = cpu_baseline(w, weights, args.cpu_seconds, single_workloads=singles)
        del singles
    print(json.dumps(out), flush=True)


def measure(w, torch, steps, warmup, nb, launch, gemm, cold_n, keep_weights):
    """Time `steps` route+forward steps of workload w over a ring of nb resident batches
    (wall clock between synchronisations), then cold_n steps after a cache flush each,
    then per-kernel HIP-event times; returns (record, weights or None)."""
    from moe_expert_ffn_softmax_amd import MoeExpertFFN, afd_ffn_profile_read, afd_ffn_set_profiling
    dev = "cuda"
    weights = workloads.make_weights(w, device=dev)
    layer = MoeExpertFFN(hidden=w.H, inter=w.M, num_experts=w.E, top_k=w.k, max_tokens=w.T, dtype=w.dtype,
                         w_gate_up=weights["w_gu"], w_down=weights["w_d"], s_gate_up=weights["s_gu"],
                         s_down=weights["s_d"], shared_inter=w.Ms, ws_gate_up=weights["ws_gu"],
                         ws_down=weights["ws_d"], ss_gate_up=weights["ss_gu"], ss_down=weights["ss_d"])
    layer.set_gemm_kernel(gemm)
    if not keep_weights:
        weights = None
    xs, lgs = [], []
    for b in range(nb):
        x, lg = workloads.make_activations(w, device=dev, batch=b)
        xs.append(x)
        lgs.append(lg)
    ydt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    ys = [torch.empty((w.T, w.H), dtype=ydt, device=dev) for _ in range(nb)]
    rbs = [layer.new_route() for _ in range(nb)]

    def step(i):
        b = i % nb
        layer.route(lgs[b], w.T, rbs[b])
        layer.forward(xs[b], w.T, rbs[b], ys[b])

    graphs = None
    if launch == "graph":
        # capture one graph per batch; every replay is checked bit for bit against the
        # eager result, three times, with eager work in between
        for b in range(nb):
            step(b)
        torch.cuda.synchronize()
        ref = [y.clone() for y in ys]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graphs = []
        with torch.cuda.stream(s):
            for b in range(nb):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    step(b)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(s)
        for rep in range(3):
            for b in range(nb):
                ys[b].zero_()
                graphs[b].replay()
            torch.cuda.synchronize()
            for b in range(nb):
                if not torch.equal(ys[b], ref[b]):
                    raise RuntimeError(f"graph replay {rep} of batch {b} differs from the eager result")
            step(rep)
            torch.cuda.synchronize()

    def run(i):
        if graphs is not None:
            graphs[i % nb].replay()
        else:
            step(i)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps
    t0 = time.perf_counter()
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps

    # the same steps with caches flushed before each one (reported beside the value)
    cold = cold_steps(run, cold_n, torch) if cold_n else None

    # per-kernel durations: the same steps again, eager, with HIP events around every
    # launch on the launch stream (the events add small gaps between kernels, so this
    # pass only feeds the per-kernel figures)
    afd_ffn_set_profiling(layer.handle, True)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    prof = afd_ffn_profile_read(layer.handle)
    afd_ffn_set_profiling(layer.handle, False)

    counts = [rbs[b].expert_counts.cpu().numpy() for b in range(nb)]
    layer.close()
    del graphs, xs, lgs, ys, rbs
    step_bytes = np.mean([algorithmic_bytes(w, c)[0] for c in counts])
    touched = np.mean([algorithmic_bytes(w, c)[1] for c in counts])
    gu_bytes = np.mean([gate_up_bytes(w, c) for c in counts])
    gu_ms, gu_n = prof["gate_up"]
    kern = gate_up_kernel(w, gemm)
    traffic = traffic_from_counters(w, gemm)
    kname = "gate_up"
    gu_flops = 4.0 * w.T * w.k * w.H * w.M + 4.0 * w.T * w.H * w.Ms
    if gu_n == 0 and prof.get("fused", (0, 0))[1]:
        # both GEMMs in one launch: its roofline covers both
        gu_ms, gu_n = prof["fused"]
        kern, kname, traffic = "gemm_bf16_fused_kernel", "fused_gate_up_down", None
        gu_bytes = np.mean([gate_up_bytes(w, c) + down_bytes(w, c) for c in counts])
        gu_flops = 6.0 * w.T * w.k * w.H * w.M + 6.0 * w.T * w.H * w.Ms
    gu_avg_s = gu_ms / max(gu_n, 1) / 1e3

    # the gate/up launch is bound by HBM below the ridge point (peak FLOP/s / peak B/s)
    # and by the matrix cores above it
    ridge = MFMA_PEAK_TFLOPS[w.dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    gu_tf = gu_flops / gu_avg_s / 1e12
    if gu_flops / gu_bytes <= ridge:
        achieved = gu_bytes / gu_avg_s / 1e9
        roofline = {"kernel": kname, "name": kern, "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "algorithmic_bytes": int(gu_bytes), "avg_launch_us": round(gu_avg_s * 1e6, 2),
                    "mfma_frac": round(gu_tf / MFMA_PEAK_TFLOPS[w.dtype], 4)}
    else:
        roofline = {"kernel": kname, "name": kern, "bound": "mfma", "achieved": round(gu_tf, 1),
                    "peak": MFMA_PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s",
                    "frac": round(gu_tf / MFMA_PEAK_TFLOPS[w.dtype], 4), "traffic": traffic,
                    "algorithmic_flops": gu_flops, "algorithmic_bytes": int(gu_bytes),
                    "avg_launch_us": round(gu_avg_s * 1e6, 2),
                    "hbm_frac": round(gu_bytes / gu_avg_s / 1e9 / HBM_PEAK_GBS, 4)}
    tflops = w.flops() / (ms_per_step / 1e3) / 1e12
    rec = {
        "workload": w.name,
        "ms_per_step": round(ms_per_step, 5),
        "tokens_per_s": round(w.T / (ms_per_step / 1e3), 2),
        "config": {"workload": w.name, "T": w.T, "H": w.H, "M": w.M, "E": w.E, "top_k": w.k, "shared_inter": w.Ms,
                   "tokens_per_expert": round(w.tokens_per_expert, 2), "batches": nb, "launch": launch, "gemm": gemm},
        "tflops": round(tflops, 3),
        "mfma_frac": round(tflops / MFMA_PEAK_TFLOPS[w.dtype], 4),
        "step_hbm": {"algorithmic_bytes": int(step_bytes), "touched_experts": round(float(touched), 2),
                     "achieved_GBps": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
                     "frac": round(step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "kernels_us": {k: round(v[0] / max(v[1], 1) * 1e3, 2) for k, v in prof.items() if v[1]},
    }
    if cold is not None:
        rec["cold"] = cold
    return rec, weights


if __name__ == "__main__":
    main()
