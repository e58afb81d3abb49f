"""MI355X (gfx950) MoE expert-FFN layer -- the FFN side of Attention-FFN
disaggregation -- as hand-written HIP kernels behind a C ABI (include/afd_ffn.h).

`_ffi` is the ctypes binding with the C function names.  `MoeExpertFFN` is a thin
convenience wrapper that allocates the caller-owned route buffers with torch (device
memory) and calls route/forward on torch's current stream.  There is no CPU or
PyTorch fallback: if libafd_ffn.so is missing, constructing a layer raises.
"""
from __future__ import annotations

from ._ffi import (AFD_BF16, AFD_F32, AFD_FP8_E4M3, AFD_GEMM_AUTO, AFD_GEMM_FUSED,  # noqa: F401
                   AFD_GEMM_STREAM, AFD_GEMM_TILED, STAGES, AfdError, afd_ffn_config, afd_ffn_create,
                   afd_ffn_destroy, afd_ffn_device_bytes, afd_ffn_forward, afd_ffn_forward_fp8_input,
                   afd_ffn_forward_noalloc, afd_ffn_last_error, afd_ffn_profile_read, afd_ffn_quantize_fp8,
                   afd_ffn_route, afd_ffn_route_bytes, afd_ffn_route_capacity, afd_ffn_route_from_capacity,
                   afd_ffn_route_hidden, afd_ffn_route_select_bias, afd_ffn_set_gemm_kernel, afd_ffn_set_profiling,
                   afd_ffn_strerror, afd_route, load)

GEMM_KERNELS = {"auto": AFD_GEMM_AUTO, "stream": AFD_GEMM_STREAM, "tiled": AFD_GEMM_TILED, "fused": AFD_GEMM_FUSED}

DTYPES = {"f32": AFD_F32, "bf16": AFD_BF16, "fp8": AFD_FP8_E4M3}


def _stream_handle(torch, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(t, name, dtypes, numel, device=None, shape=None):
    """Reject, before anything reaches the library, a buffer whose type, placement,
    layout or size does not match what the C call will read or write through its
    pointer (the C side cannot see lengths).  dtypes: one torch dtype or a tuple."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the layer on {device}")
    if device is None and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {numel}")


def _check_T(T, max_tokens):
    import numbers
    if not isinstance(T, numbers.Integral) or isinstance(T, bool) or T < 0 or T > max_tokens:
        raise ValueError(f"T={T!r} must be an int in [0, max_tokens={max_tokens}]")


def quantize_fp8(x, stream=None):
    """e4m3 codes (uint8 [rows, cols]) and fp32 scales ([rows, cols/128]) of a 2-D
    bf16 or fp32 CUDA tensor, computed by the library's quantisation kernel."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("quantize_fp8 takes a 2-D tensor")
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"quantize_fp8 takes bfloat16 or float32 activations, got {x.dtype}")
    rows, cols = x.shape
    if cols % 128:
        raise ValueError(f"cols={cols} must be a multiple of 128")
    x = x.contiguous()
    _check(x, "x", (torch.bfloat16, torch.float32), rows * cols)
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, cols // 128), dtype=torch.float32, device=x.device)
    dt = AFD_BF16 if x.dtype == torch.bfloat16 else AFD_F32
    afd_ffn_quantize_fp8(x, rows, cols, dt, codes, scales, _stream_handle(torch, stream))
    return codes, scales


class RouteBuffers:
    """Caller-owned device buffers of one routing result (one per batch in flight)."""

    def __init__(self, max_tokens: int, num_experts: int, top_k: int, device):
        import torch
        self.max_tokens, self.num_experts, self.top_k = max_tokens, num_experts, top_k
        P = max_tokens * top_k
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_ids = torch.zeros(P, **i32)
        self.topk_gates = torch.zeros(P, dtype=torch.float32, device=device)
        self.expert_counts = torch.zeros(num_experts, **i32)
        self.expert_offsets = torch.zeros(num_experts + 1, **i32)
        self.sorted_pair = torch.zeros(P, **i32)
        self.pair_pos = torch.zeros(P, **i32)
        self.c = afd_route(self.topk_ids.data_ptr(), self.topk_gates.data_ptr(), self.expert_counts.data_ptr(),
                           self.expert_offsets.data_ptr(), self.sorted_pair.data_ptr(), self.pair_pos.data_ptr())


class MoeExpertFFN:
    """One MoE layer's routed experts (+ optional shared expert) on the current device.

    w_gate_up [E,H,2M], w_down [E,M,H] (float32 / bfloat16 / float8_e4m3fn tensors on
    the GPU); for fp8 also s_gate_up, s_down fp32 block scales; ws_* / ss_* for the
    shared expert.  The library copies the weights at construction."""

    def __init__(self, *, hidden, inter, num_experts, top_k, max_tokens, dtype, w_gate_up, w_down,
                 s_gate_up=None, s_down=None, shared_inter=0, ws_gate_up=None, ws_down=None, ss_gate_up=None,
                 ss_down=None):
        import torch
        if dtype not in DTYPES:
            raise ValueError(f"dtype {dtype!r} not in {sorted(DTYPES)}")
        H, M, E, Ms = hidden, inter, num_experts, shared_inter
        for n, v in (("hidden", H), ("inter", M), ("shared_inter", Ms)):
            if not isinstance(v, int) or v < 0 or v % 128 or (v == 0 and n != "shared_inter"):
                raise ValueError(f"{n}={v!r} must be a positive multiple of 128" + (" or 0" if n == "shared_inter"
                                                                                       else ""))
        wdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": (torch.float8_e4m3fn, torch.uint8)}[dtype]
        self.device = getattr(w_gate_up, "device", None)
        dev = self.device
        _check(w_gate_up, "w_gate_up", wdt, 0, dev, (E, H, 2 * M))
        _check(w_down, "w_down", wdt, 0, dev, (E, M, H))
        f32 = torch.float32
        if dtype == "fp8":
            _check(s_gate_up, "s_gate_up", f32, 0, dev, (E, H // 128, 2 * M // 128))
            _check(s_down, "s_down", f32, 0, dev, (E, M // 128, H // 128))
        if Ms:
            _check(ws_gate_up, "ws_gate_up", wdt, 0, dev, (H, 2 * Ms))
            _check(ws_down, "ws_down", wdt, 0, dev, (Ms, H))
            if dtype == "fp8":
                _check(ss_gate_up, "ss_gate_up", f32, 0, dev, (H // 128, 2 * Ms // 128))
                _check(ss_down, "ss_down", f32, 0, dev, (Ms // 128, H // 128))
        if not w_gate_up.is_cuda:
            raise ValueError(f"the weights must be GPU tensors, got {w_gate_up.device}")
        load()
        self.cfg = afd_ffn_config(hidden, inter, num_experts, top_k, max_tokens, shared_inter, DTYPES[dtype])
        self.dtype = dtype
        self.handle = afd_ffn_create(self.cfg, w_gate_up, w_down, s_gate_up, s_down, ws_gate_up, ws_down,
                                     ss_gate_up, ss_down, _stream_handle(torch))

    # dtypes of the activations x / y of this layer
    def _act(self):
        import torch
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def _rb(self, rb, T):
        _check_T(T, self.cfg.max_tokens)
        if not isinstance(rb, RouteBuffers) or rb.num_experts != self.cfg.num_experts or \
                rb.top_k != self.cfg.top_k or rb.max_tokens < T:
            raise ValueError("route buffers must come from this layer's new_route()")

    def set_gemm_kernel(self, name: str) -> None:
        """'auto', 'stream' (16-row weight-streaming tiles), 'tiled' (128-row tiles) or 'fused'
        (bf16 decode layers: both streaming GEMMs in one persistent launch)."""
        afd_ffn_set_gemm_kernel(self.handle, GEMM_KERNELS[name])

    def new_route(self) -> RouteBuffers:
        return RouteBuffers(self.cfg.max_tokens, self.cfg.num_experts, self.cfg.top_k, self.device)

    def route(self, logits, T: int, rb: RouteBuffers, stream=None) -> None:
        import torch
        self._rb(rb, T)
        _check(logits, "logits", torch.float32, T * self.cfg.num_experts, self.device)
        afd_ffn_route(self.handle, logits, T, rb.c, _stream_handle(torch, stream))

    def route_select_bias(self, scores, bias, T: int, rb: RouteBuffers, stream=None) -> None:
        """Route with a bias that only steers the choice: experts ranked on scores + bias,
        gates = softmax of the chosen experts' unbiased scores."""
        import torch
        self._rb(rb, T)
        _check(scores, "scores", torch.float32, T * self.cfg.num_experts, self.device)
        _check(bias, "bias", torch.float32, self.cfg.num_experts, self.device)
        afd_ffn_route_select_bias(self.handle, scores, bias, T, rb.c, _stream_handle(torch, stream))

    def route_capacity(self, ids, gates, T: int, limits, base_capacity: int, adaptive: bool = True,
                       out=None, stream=None):
        """Capacity-aware routing (adaptive token dropper) of T preference lists ids/gates
        [T, top_k]; limits [E] int32 is updated in place when adaptive.  Returns (assign [T],
        weight [T], offsets [E+1], sorted_token [T]), allocated unless given in `out`."""
        import torch
        _check_T(T, self.cfg.max_tokens)
        E, k = self.cfg.num_experts, self.cfg.top_k
        _check(ids, "ids", torch.int32, T * k, self.device)
        _check(gates, "gates", torch.float32, T * k, self.device)
        _check(limits, "limits", torch.int32, E, self.device)
        dev = limits.device
        if out is None:
            n = max(T, 1)
            out = (torch.empty(n, dtype=torch.int32, device=dev), torch.empty(n, dtype=torch.float32, device=dev),
                   torch.empty(self.cfg.num_experts + 1, dtype=torch.int32, device=dev),
                   torch.empty(n, dtype=torch.int32, device=dev))
        self._check_capacity_result(out, T)
        assign, weight, offsets, sorted_token = out
        afd_ffn_route_capacity(self.handle, ids, gates, T, base_capacity, adaptive, limits, assign, weight, offsets,
                               sorted_token, _stream_handle(torch, stream))
        return assign, weight, offsets, sorted_token

    def route_from_capacity(self, cap, T: int, rb: RouteBuffers, stream=None) -> None:
        """Fill rb from a capacity result cap = (assign, weight, offsets, sorted_token), as
        returned by route_capacity, so that forward runs each kept token through its one
        expert with its weight."""
        import torch
        self._rb(rb, T)
        self._check_capacity_result(cap, T)
        assign, weight, offsets, sorted_token = cap
        afd_ffn_route_from_capacity(self.handle, assign, weight, offsets, sorted_token, T, rb.c,
                                    _stream_handle(torch, stream))

    def _check_capacity_result(self, cap, T):
        import torch
        if not isinstance(cap, (tuple, list)) or len(cap) != 4:
            raise ValueError("a capacity result is (assign, weight, offsets, sorted_token)")
        assign, weight, offsets, sorted_token = cap
        _check(assign, "assign", torch.int32, T, self.device)
        _check(weight, "weight", torch.float32, T, self.device)
        _check(offsets, "offsets", torch.int32, self.cfg.num_experts + 1, self.device)
        _check(sorted_token, "sorted_token", torch.int32, T, self.device)

    def route_hidden(self, x, w_router, logits, T: int, rb: RouteBuffers, bias=None, stream=None) -> None:
        """Route from hidden states: logits [T, E] (fp32, written) = x w_router^T + bias,
        then the routing of route()."""
        import torch
        self._rb(rb, T)
        H, E = self.cfg.hidden, self.cfg.num_experts
        _check(x, "x", self._act(), T * H, self.device)
        _check(w_router, "w_router", self._act(), E * H, self.device)
        if bias is not None:
            _check(bias, "bias", torch.float32, E, self.device)
        _check(logits, "logits", torch.float32, T * E, self.device)
        afd_ffn_route_hidden(self.handle, x, w_router, bias, logits, T, rb.c, _stream_handle(torch, stream))

    def forward(self, x, T: int, rb: RouteBuffers, y, stream=None) -> None:
        import torch
        self._rb(rb, T)
        H = self.cfg.hidden
        _check(x, "x", self._act(), T * H, self.device)
        _check(y, "y", self._act(), T * H, self.device)
        afd_ffn_forward(self.handle, x, T, rb.c, y, _stream_handle(torch, stream))

    def forward_fp8_input(self, xq, xs, T: int, rb: RouteBuffers, y, stream=None) -> None:
        """fp8 layers: forward on e4m3 codes xq [T, H] (uint8) and fp32 scales xs [T, H/128]."""
        import torch
        self._rb(rb, T)
        if self.dtype != "fp8":
            raise ValueError("forward_fp8_input needs an fp8 layer")
        H = self.cfg.hidden
        _check(xq, "xq", (torch.uint8, torch.float8_e4m3fn), T * H, self.device)
        _check(xs, "xs", torch.float32, T * (H // 128), self.device)
        _check(y, "y", torch.bfloat16, T * H, self.device)
        afd_ffn_forward_fp8_input(self.handle, xq, xs, T, rb.c, y, _stream_handle(torch, stream))

    def __call__(self, x, logits, rb: RouteBuffers = None, y=None):
        """route + forward of a whole batch; returns y (allocated if not given)."""
        import torch
        T = x.shape[0]
        rb = rb or self.new_route()
        if y is None:
            y = torch.empty((T, self.cfg.hidden), dtype=torch.float32 if self.dtype == "f32" else torch.bfloat16,
                            device=x.device)
        self.route(logits, T, rb)
        self.forward(x, T, rb, y)
        return y

    def close(self):
        if getattr(self, "handle", None):
            afd_ffn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
