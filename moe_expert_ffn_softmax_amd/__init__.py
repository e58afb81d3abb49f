"""MI355X (gfx950) MoE expert-FFN layer -- the FFN side of Attention-FFN
disaggregation -- as hand-written HIP kernels behind a C ABI (include/afd_ffn.h).

`_ffi` is the ctypes binding with the C function names.  `MoeExpertFFN` is a thin
convenience wrapper that allocates the caller-owned route buffers with torch (device
memory) and calls route/forward on torch's current stream.  There is no CPU or
PyTorch fallback: if libafd_ffn.so is missing, constructing a layer raises.
"""
from __future__ import annotations

from ._ffi import (AFD_BF16, AFD_F32, AFD_FP8_E4M3, AFD_GEMM_AUTO, AFD_GEMM_STREAM,  # noqa: F401
                   AFD_GEMM_TILED, AFD_GEMM_WIDE, STAGES, AfdError, afd_ffn_config, afd_ffn_create, afd_ffn_destroy,
                   afd_ffn_device_bytes, afd_ffn_forward, afd_ffn_forward_fp8_input, afd_ffn_last_error,
                   afd_ffn_profile_read, afd_ffn_quantize_fp8, afd_ffn_route, afd_ffn_route_capacity,
                   afd_ffn_route_from_capacity,
                   afd_ffn_route_hidden,
                   afd_ffn_route_bytes, afd_ffn_route_select_bias, afd_ffn_set_gemm_kernel, afd_ffn_set_profiling,
                   afd_ffn_strerror, afd_route, load)

GEMM_KERNELS = {"auto": AFD_GEMM_AUTO, "stream": AFD_GEMM_STREAM, "tiled": AFD_GEMM_TILED,
                "wide": AFD_GEMM_WIDE}

DTYPES = {"f32": AFD_F32, "bf16": AFD_BF16, "fp8": AFD_FP8_E4M3}


def _stream_handle(torch, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def quantize_fp8(x, stream=None):
    """e4m3 codes (uint8 [rows, cols]) and fp32 scales ([rows, cols/128]) of a 2-D
    bf16 or fp32 CUDA tensor, computed by the library's quantisation kernel."""
    import torch
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, cols // 128), dtype=torch.float32, device=x.device)
    dt = AFD_BF16 if x.dtype == torch.bfloat16 else AFD_F32
    afd_ffn_quantize_fp8(x.contiguous(), rows, cols, dt, codes, scales, _stream_handle(torch, stream))
    return codes, scales


class RouteBuffers:
    """Caller-owned device buffers of one routing result (one per batch in flight)."""

    def __init__(self, max_tokens: int, num_experts: int, top_k: int, device):
        import torch
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
        load()
        self.cfg = afd_ffn_config(hidden, inter, num_experts, top_k, max_tokens, shared_inter, DTYPES[dtype])
        self.dtype = dtype
        self.device = w_gate_up.device
        self.handle = afd_ffn_create(self.cfg, w_gate_up, w_down, s_gate_up, s_down, ws_gate_up, ws_down,
                                     ss_gate_up, ss_down, _stream_handle(torch))

    def set_gemm_kernel(self, name: str) -> None:
        """'auto', 'stream' (16-row weight-streaming tiles), 'tiled' (128-row tiles) or
        'wide' (256x256 tiles, bf16 layers)."""
        afd_ffn_set_gemm_kernel(self.handle, GEMM_KERNELS[name])

    def new_route(self) -> RouteBuffers:
        return RouteBuffers(self.cfg.max_tokens, self.cfg.num_experts, self.cfg.top_k, self.device)

    def route(self, logits, T: int, rb: RouteBuffers, stream=None) -> None:
        import torch
        afd_ffn_route(self.handle, logits, T, rb.c, _stream_handle(torch, stream))

    def route_select_bias(self, scores, bias, T: int, rb: RouteBuffers, stream=None) -> None:
        """Route with a bias that only steers the choice: experts ranked on scores + bias,
        gates = softmax of the chosen experts' unbiased scores."""
        import torch
        afd_ffn_route_select_bias(self.handle, scores, bias, T, rb.c, _stream_handle(torch, stream))

    def route_capacity(self, ids, gates, T: int, limits, base_capacity: int, adaptive: bool = True,
                       out=None, stream=None):
        """Capacity-aware routing (adaptive token dropper) of T preference lists ids/gates
        [T, top_k]; limits [E] int32 is updated in place when adaptive.  Returns (assign [T],
        weight [T], offsets [E+1], sorted_token [T]), allocated unless given in `out`."""
        import torch
        dev = limits.device
        if out is None:
            n = max(T, 1)
            out = (torch.empty(n, dtype=torch.int32, device=dev), torch.empty(n, dtype=torch.float32, device=dev),
                   torch.empty(self.cfg.num_experts + 1, dtype=torch.int32, device=dev),
                   torch.empty(n, dtype=torch.int32, device=dev))
        assign, weight, offsets, sorted_token = out
        afd_ffn_route_capacity(self.handle, ids, gates, T, base_capacity, adaptive, limits, assign, weight, offsets,
                               sorted_token, _stream_handle(torch, stream))
        return assign, weight, offsets, sorted_token

    def route_from_capacity(self, cap, T: int, rb: RouteBuffers, stream=None) -> None:
        """Fill rb from a capacity result cap = (assign, weight, offsets, sorted_token), as
        returned by route_capacity, so that forward runs each kept token through its one
        expert with its weight."""
        import torch
        assign, weight, offsets, sorted_token = cap
        afd_ffn_route_from_capacity(self.handle, assign, weight, offsets, sorted_token, T, rb.c,
                                    _stream_handle(torch, stream))

    def route_hidden(self, x, w_router, logits, T: int, rb: RouteBuffers, bias=None, stream=None) -> None:
        """Route from hidden states: logits [T, E] (fp32, written) = x w_router^T + bias,
        then the routing of route()."""
        import torch
        afd_ffn_route_hidden(self.handle, x, w_router, bias, logits, T, rb.c, _stream_handle(torch, stream))

    def forward(self, x, T: int, rb: RouteBuffers, y, stream=None) -> None:
        import torch
        afd_ffn_forward(self.handle, x, T, rb.c, y, _stream_handle(torch, stream))

    def forward_fp8_input(self, xq, xs, T: int, rb: RouteBuffers, y, stream=None) -> None:
        """fp8 layers: forward on e4m3 codes xq [T, H] (uint8) and fp32 scales xs [T, H/128]."""
        import torch
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
