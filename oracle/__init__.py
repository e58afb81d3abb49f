"""CPU oracle for one MoE layer's expert FFN -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and the CPU-baseline leg of bench.py
may import this package.  The HIP library does not depend on it, and it shares no
code with the library: the arithmetic lives in afd_oracle.c (plain C, double
precision, OpenMP over independent token-expert pairs), and this module only
marshals numpy arrays into it.

Function-by-function pins (tests/test_oracle.py):
  route      -- numpy stable argsort; rank-count brute force; closed-form gates;
                the top-k-then-softmax form of the router on the MoE engineering page.
  route_select_bias -- closed-form gates of hand-made cases; a key tie that exists only
                after fp32 rounding of score + bias; zero bias reproduces route; a
                dominant bias forces the chosen set while the gates stay those of
                the unbiased scores.
  router_scores -- a hand-computed integer example; one-hot gate vectors pick x's
                columns; exact integer sums against brute force; bias shift invariance
                of the routing and a dominant bias forcing an expert.
  route_capacity -- hand-traced fixtures (tests/golden/capacity_cases.txt); unlimited
                capacity reduces to top-1 routing; zero capacity drops every token;
                count bounds of the preference and fallback rules; a drop only once
                every expert holds 1.5x its limit; numpy stable argsort of assign.
  permute    -- numpy stable argsort of the flattened ids; bijection; count sums.
  layer      -- numpy float64 matmuls for one expert; a diagonal-weight closed form;
                the k = E dense mixture; token-order equivariance; MAC count 3*H*M per
                token-expert pair (the 6*B*H*M FLOPs of the AFD article's §2.1).
  fp8 codec  -- every code's value from the OCP E4M3 definition; round trips;
                torch's float8_e4m3fn cast (a library routine) on random values.
  fp8 layer  -- x and h quantised per row and per 128 channels (fp32 decisions),
                weights dequantised per 128x128 block: torch's e4m3 decode and float64
                matmuls for one expert, and for three experts with scales of their own,
                k = 2, two scale blocks in M and a block-scaled shared expert.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "afd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, FP8 = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "fp8": FP8}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, no fused multiply-add contraction."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int), ("M", ctypes.c_int), ("E", ctypes.c_int), ("k", ctypes.c_int),
                ("Ms", ctypes.c_int), ("dtype", ctypes.c_int),
                ("w_gu", ctypes.POINTER(ctypes.c_void_p)), ("w_d", ctypes.POINTER(ctypes.c_void_p)),
                ("s_gu", ctypes.POINTER(ctypes.c_void_p)), ("s_d", ctypes.POINTER(ctypes.c_void_p)),
                ("ws_gu", ctypes.c_void_p), ("ws_d", ctypes.c_void_p),
                ("ss_gu", ctypes.c_void_p), ("ss_d", ctypes.c_void_p)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.afdo_route.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P]
        lib.afdo_route.restype = None
        lib.afdo_route_select_bias.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P]
        lib.afdo_route_select_bias.restype = None
        lib.afdo_router_scores.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P]
        lib.afdo_router_scores.restype = None
        lib.afdo_route_capacity.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int32,
                                            ctypes.c_int, P, P, P, P, P, P]
        lib.afdo_route_capacity.restype = None
        lib.afdo_permute.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P, P]
        lib.afdo_permute.restype = None
        lib.afdo_layer.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int, P, P, P, P, P,
                                   ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
        lib.afdo_layer.restype = ctypes.c_int
        lib.afdo_fp8_decode.argtypes = [ctypes.c_uint8]
        lib.afdo_fp8_decode.restype = ctypes.c_double
        lib.afdo_fp8_encode.argtypes = [ctypes.c_float]
        lib.afdo_fp8_encode.restype = ctypes.c_uint8
        lib.afdo_quant_row_fp8.argtypes = [ctypes.c_int, P, P, P, P]
        lib.afdo_quant_row_fp8.restype = None
        lib.afdo_max_threads.argtypes = []
        lib.afdo_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().afdo_max_threads())


def route(logits: np.ndarray, k: int):
    """ids [T,k] int32 and gates [T,k] float64 for fp32 logits [T,E]."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.zeros((T, k), np.int32)
    gates = np.zeros((T, k), np.float64)
    _load().afdo_route(T, E, k, _p(logits), _p(ids), _p(gates))
    return ids, gates


def route_select_bias(scores: np.ndarray, bias: np.ndarray, k: int):
    """ids [T,k] int32 and gates [T,k] float64: experts chosen on fp32(scores + bias),
    gates from the unbiased fp32 scores [T,E] (the selection-only bias router)."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    T, E = scores.shape
    bias = np.ascontiguousarray(bias, dtype=np.float32)
    if bias.shape != (E,):
        raise ValueError("bias must have shape [E]")
    ids = np.zeros((T, k), np.int32)
    gates = np.zeros((T, k), np.float64)
    _load().afdo_route_select_bias(T, E, k, _p(scores), _p(bias), _p(ids), _p(gates))
    return ids, gates


def router_scores(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """scores [T,E] float64 = x [T,H] w [E,H]^T + bias [E] (the router projection)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, H = x.shape
    E = w.shape[0]
    if w.shape[1] != H:
        raise ValueError("x and w disagree on H")
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.zeros((T, E), np.float64)
    _load().afdo_router_scores(T, E, H, _p(x), _p(w), None if b is None else _p(b), _p(out))
    return out


def route_capacity(ids: np.ndarray, gates: np.ndarray, E: int, limits: np.ndarray, base: int,
                   adaptive: bool = True):
    """The adaptive token dropper for one batch of preference lists ids [T,k] int32 with
    fp32 gates [T,k].  Returns assign [T] (expert or -1), weight [T] fp32, counts [E],
    offsets [E+1], sorted_token [n routed] and the updated limits [E] (all int32 but
    weight); the input limits are not modified."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    gates = np.ascontiguousarray(gates, dtype=np.float32)
    T, k = ids.shape
    if gates.shape != (T, k):
        raise ValueError("gates must match ids")
    if ids.size and (ids.min() < 0 or ids.max() >= E):
        raise ValueError("expert id out of range")
    lim = np.array(limits, dtype=np.int32, copy=True)
    if lim.shape != (E,):
        raise ValueError("limits must have shape [E]")
    assign = np.zeros(T, np.int32)
    weight = np.zeros(T, np.float32)
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    st = np.zeros(max(T, 1), np.int32)
    _load().afdo_route_capacity(T, E, k, _p(ids), _p(gates), int(base), int(bool(adaptive)), _p(lim), _p(assign),
                                _p(weight), _p(counts), _p(offsets), _p(st))
    return dict(assign=assign, weight=weight, counts=counts, offsets=offsets,
                sorted_token=st[:int(offsets[E])].copy(), limits=lim)


def permute(ids: np.ndarray, E: int):
    """counts [E], offsets [E+1], sorted_pair [T*k], pair_pos [T*k] (all int32)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    if ids.size and (ids.min() < 0 or ids.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    sp = np.zeros(T * k, np.int32)
    pp = np.zeros(T * k, np.int32)
    _load().afdo_permute(T, E, k, _p(ids), _p(counts), _p(offsets), _p(sp), _p(pp))
    return counts, offsets, sp, pp


def fp8_decode(code: int) -> float:
    return float(_load().afdo_fp8_decode(int(code) & 0xFF))


def fp8_encode(v: float) -> int:
    return int(_load().afdo_fp8_encode(float(v)))


def quant_row_fp8(v: np.ndarray):
    """Per-128-group e4m3 quantisation of one fp32 row: (codes uint8, scales fp32, dequant f64)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    n = v.shape[0]
    codes = np.zeros(n, np.uint8)
    scales = np.zeros(n // 128, np.float32)
    deq = np.zeros(n, np.float64)
    _load().afdo_quant_row_fp8(n, _p(v), _p(codes), _p(scales), _p(deq))
    return codes, scales, deq


def _raw(a) -> np.ndarray:
    """Contiguous numpy view of a weight in its storage encoding: float32 stays float32,
    bfloat16 becomes its uint16 bit pattern and float8_e4m3fn its uint8 codes."""
    if isinstance(a, np.ndarray):
        return np.ascontiguousarray(a)
    import torch
    t = a.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def layer(x: np.ndarray, logits: np.ndarray, *, H: int, M: int, E: int, k: int, dtype: str,
          w_gu: Sequence, w_d: Sequence, s_gu: Optional[Sequence] = None, s_d: Optional[Sequence] = None,
          Ms: int = 0, ws_gu=None, ws_d=None, ss_gu=None, ss_d=None, nthreads: int = 0):
    """Whole layer for n tokens.

    x: [n,H] float32 (bf16 activations widened exactly); logits: [n,E] float32.
    w_gu / w_d: length-E sequences of per-expert matrices ([H,2M] / [M,H]) in their
    storage dtype, or None for experts that none of the n tokens selects.
    Returns (ids [n,k] int32, gates [n,k] f64, y [n,H] f64, macs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    n = x.shape[0]
    assert x.shape == (n, H) and logits.shape == (n, E)
    keep = []

    def arr(seq):
        ptrs = (ctypes.c_void_p * E)()
        for e in range(E):
            a = None if seq is None else seq[e]
            if a is None:
                ptrs[e] = None
            else:
                r = _raw(a)
                keep.append(r)
                ptrs[e] = r.ctypes.data
        return ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), ptrs

    def one(a):
        if a is None:
            return None
        r = _raw(a)
        keep.append(r)
        return r.ctypes.data

    pgu, kgu = arr(w_gu)
    pd, kd = arr(w_d)
    psgu, ksgu = arr(s_gu)
    psd, ksd = arr(s_d)
    pb = _Problem(H, M, E, k, Ms, _DT[dtype], pgu, pd, psgu, psd, one(ws_gu), one(ws_d), one(ss_gu), one(ss_d))
    ids = np.zeros((n, k), np.int32)
    gates = np.zeros((n, k), np.float64)
    y = np.zeros((n, H), np.float64)
    macs = ctypes.c_int64(0)
    rc = _load().afdo_layer(ctypes.byref(pb), n, _p(x), _p(logits), _p(ids), _p(gates), _p(y),
                            ctypes.byref(macs), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle layer failed with code {rc}")
    return ids, gates, y, int(macs.value)


def layer_assigned(x: np.ndarray, assign: np.ndarray, weight: np.ndarray, *, H: int, M: int, E: int, dtype: str,
                   w_gu: Sequence, w_d: Sequence, s_gu: Optional[Sequence] = None,
                   s_d: Optional[Sequence] = None, Ms: int = 0, ws_gu=None, ws_d=None, ss_gu=None, ss_d=None,
                   nthreads: int = 0):
    """Whole layer on a given one-expert-per-token assignment (the capacity-aware
    dropper's): y[t] = weight[t] * FFN_assign[t](x[t]) (+ the shared expert), with
    assign -1 for a dropped token.  Returns (y [n,H] f64, macs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.shape[0]
    ids = np.ascontiguousarray(assign, dtype=np.int32).reshape(n, 1).copy()
    gates = np.ascontiguousarray(weight, dtype=np.float32).astype(np.float64).reshape(n, 1)
    keep = []

    def arr(seq):
        ptrs = (ctypes.c_void_p * E)()
        for e in range(E):
            a = None if seq is None else seq[e]
            if a is not None:
                r = _raw(a)
                keep.append(r)
                ptrs[e] = r.ctypes.data
        return ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p))

    def one(a):
        if a is None:
            return None
        r = _raw(a)
        keep.append(r)
        return r.ctypes.data

    pb = _Problem(H, M, E, 1, Ms, _DT[dtype], arr(w_gu), arr(w_d), arr(s_gu), arr(s_d), one(ws_gu), one(ws_d),
                  one(ss_gu), one(ss_d))
    y = np.zeros((n, H), np.float64)
    macs = ctypes.c_int64(0)
    rc = _load().afdo_layer(ctypes.byref(pb), n, _p(x), None, _p(ids), _p(gates), _p(y), ctypes.byref(macs),
                            int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle layer failed with code {rc}")
    return y, int(macs.value)


def layer_from_weights(x, logits, wl, weights, nthreads: int = 0, experts_needed=None):
    """Convenience: run `layer` with a workload description `wl` (anything with
    H, M, E, k, Ms, dtype attributes) and a dict of weight tensors as produced by the
    input generator (numpy arrays or torch tensors, on any device).  Only the experts
    in `experts_needed` (default: all) are copied to host memory."""
    E = wl.E
    need = set(range(E)) if experts_needed is None else set(int(e) for e in experts_needed)

    def pick(t):
        if t is None:
            return None
        return [t[e] if e in need else None for e in range(E)]

    return layer(x, logits, H=wl.H, M=wl.M, E=E, k=wl.k, dtype=wl.dtype,
                 w_gu=pick(weights["w_gu"]), w_d=pick(weights["w_d"]),
                 s_gu=pick(weights.get("s_gu")), s_d=pick(weights.get("s_d")),
                 Ms=wl.Ms, ws_gu=weights.get("ws_gu"), ws_d=weights.get("ws_d"),
                 ss_gu=weights.get("ss_gu"), ss_d=weights.get("ss_d"), nthreads=nthreads)
