"""ctypes binding of libafd_ffn.so: the C ABI declared in include/afd_ffn.h, with the
same function names.  Argument marshalling only -- every step of the layer runs in
the library's HIP kernels.  Pointer arguments accept torch tensors (their
data_ptr()), plain integers or None."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libafd_ffn.so")

AFD_OK, AFD_EINVAL, AFD_EUNSUPPORTED, AFD_ENOMEM, AFD_EHIP = 0, -1, -2, -3, -4
AFD_F32, AFD_BF16, AFD_FP8_E4M3 = 0, 1, 2
AFD_GEMM_AUTO, AFD_GEMM_STREAM, AFD_GEMM_TILED, AFD_GEMM_FUSED = 0, 1, 2, 3
STAGES = ("router", "permute", "quant", "gate_up", "down", "combine", "router_proj", "fused")
AFD_NUM_STAGES = len(STAGES)


class afd_ffn_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class afd_route(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_gates", ctypes.c_void_p), ("expert_counts", ctypes.c_void_p),
                ("expert_offsets", ctypes.c_void_p), ("sorted_pair", ctypes.c_void_p), ("pair_pos", ctypes.c_void_p)]


class AfdError(RuntimeError):
    def __init__(self, code: int, detail: str):
        super().__init__(f"{afd_ffn_strerror(code)} ({code}): {detail}")
        self.code = code


_lib = None


def load():
    """Load the library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m moe_expert_ffn_softmax_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    V, I32, P = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
    lib.afd_ffn_create.argtypes = [ctypes.POINTER(afd_ffn_config), V, V, V, V, V, V, V, V, V, ctypes.POINTER(V)]
    lib.afd_ffn_create.restype = ctypes.c_int
    lib.afd_ffn_route.argtypes = [V, P, I32, ctypes.POINTER(afd_route), V]
    lib.afd_ffn_route.restype = ctypes.c_int
    lib.afd_ffn_route_hidden.argtypes = [V, P, P, P, P, I32, ctypes.POINTER(afd_route), V]
    lib.afd_ffn_route_hidden.restype = ctypes.c_int
    lib.afd_ffn_route_select_bias.argtypes = [V, P, P, I32, ctypes.POINTER(afd_route), V]
    lib.afd_ffn_route_select_bias.restype = ctypes.c_int
    lib.afd_ffn_route_capacity.argtypes = [V, P, P, I32, I32, I32, P, P, P, P, P, V]
    lib.afd_ffn_route_capacity.restype = ctypes.c_int
    lib.afd_ffn_route_from_capacity.argtypes = [V, P, P, P, P, I32, ctypes.POINTER(afd_route), V]
    lib.afd_ffn_route_from_capacity.restype = ctypes.c_int
    lib.afd_ffn_forward.argtypes = [V, P, I32, ctypes.POINTER(afd_route), P, V]
    lib.afd_ffn_forward.restype = ctypes.c_int
    lib.afd_ffn_forward_fp8_input.argtypes = [V, P, P, I32, ctypes.POINTER(afd_route), P, V]
    lib.afd_ffn_forward_noalloc.argtypes = [V, P, I32, ctypes.POINTER(afd_route), P, V]
    lib.afd_ffn_forward_noalloc.restype = ctypes.c_int
    lib.afd_ffn_forward_fp8_input.restype = ctypes.c_int
    lib.afd_ffn_destroy.argtypes = [V]
    lib.afd_ffn_destroy.restype = ctypes.c_int
    lib.afd_ffn_strerror.argtypes = [ctypes.c_int]
    lib.afd_ffn_strerror.restype = ctypes.c_char_p
    lib.afd_ffn_last_error.argtypes = []
    lib.afd_ffn_last_error.restype = ctypes.c_char_p
    lib.afd_ffn_device_bytes.argtypes = [V]
    lib.afd_ffn_device_bytes.restype = ctypes.c_size_t
    lib.afd_ffn_route_bytes.argtypes = [V]
    lib.afd_ffn_route_bytes.restype = ctypes.c_size_t
    lib.afd_ffn_quantize_fp8.argtypes = [P, I32, I32, I32, P, P, V]
    lib.afd_ffn_quantize_fp8.restype = ctypes.c_int
    lib.afd_ffn_set_gemm_kernel.argtypes = [V, ctypes.c_int]
    lib.afd_ffn_set_gemm_kernel.restype = ctypes.c_int
    lib.afd_ffn_set_profiling.argtypes = [V, ctypes.c_int]
    lib.afd_ffn_set_profiling.restype = ctypes.c_int
    lib.afd_ffn_profile_read.argtypes = [V, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                         ctypes.c_int]
    lib.afd_ffn_profile_read.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _check(rc: int):
    if rc != AFD_OK:
        raise AfdError(rc, afd_ffn_last_error())


def afd_ffn_strerror(code: int) -> str:
    return load().afd_ffn_strerror(int(code)).decode()


def afd_ffn_last_error() -> str:
    return load().afd_ffn_last_error().decode()


def afd_ffn_create(cfg: afd_ffn_config, w_gate_up, w_down, s_gate_up=None, s_down=None, ws_gate_up=None,
                   ws_down=None, ss_gate_up=None, ss_down=None, stream=None) -> int:
    h = ctypes.c_void_p()
    _check(load().afd_ffn_create(ctypes.byref(cfg), _ptr(w_gate_up), _ptr(w_down), _ptr(s_gate_up), _ptr(s_down),
                                 _ptr(ws_gate_up), _ptr(ws_down), _ptr(ss_gate_up), _ptr(ss_down), stream,
                                 ctypes.byref(h)))
    return h.value


def afd_ffn_route(h: int, logits, T: int, route: afd_route, stream=None) -> None:
    _check(load().afd_ffn_route(h, _ptr(logits), int(T), ctypes.byref(route), stream))


def afd_ffn_route_select_bias(h: int, scores, bias, T: int, route: afd_route, stream=None) -> None:
    _check(load().afd_ffn_route_select_bias(h, _ptr(scores), _ptr(bias), int(T), ctypes.byref(route), stream))


def afd_ffn_route_capacity(h: int, ids, gates, T: int, base_capacity: int, adaptive: bool, limits, assign, weight,
                           offsets, sorted_token, stream=None) -> None:
    _check(load().afd_ffn_route_capacity(h, _ptr(ids), _ptr(gates), int(T), int(base_capacity), int(bool(adaptive)),
                                         _ptr(limits), _ptr(assign), _ptr(weight), _ptr(offsets),
                                         _ptr(sorted_token), stream))


def afd_ffn_route_from_capacity(h: int, assign, weight, offsets, sorted_token, T: int, route: afd_route,
                                stream=None) -> None:
    _check(load().afd_ffn_route_from_capacity(h, _ptr(assign), _ptr(weight), _ptr(offsets), _ptr(sorted_token),
                                              int(T), ctypes.byref(route), stream))


def afd_ffn_route_hidden(h: int, x, w_router, bias, logits, T: int, route: afd_route, stream=None) -> None:
    _check(load().afd_ffn_route_hidden(h, _ptr(x), _ptr(w_router), _ptr(bias), _ptr(logits), int(T),
                                       ctypes.byref(route), stream))


def afd_ffn_forward(h: int, x, T: int, route: afd_route, y, stream=None) -> None:
    _check(load().afd_ffn_forward(h, _ptr(x), int(T), ctypes.byref(route), _ptr(y), stream))


def afd_ffn_forward_noalloc(h: int, x, T: int, route: afd_route, y, stream=None) -> None:
    _check(load().afd_ffn_forward_noalloc(h, _ptr(x), int(T), ctypes.byref(route), _ptr(y), stream))


def afd_ffn_forward_fp8_input(h: int, xq, xs, T: int, route: afd_route, y, stream=None) -> None:
    _check(load().afd_ffn_forward_fp8_input(h, _ptr(xq), _ptr(xs), int(T), ctypes.byref(route), _ptr(y), stream))


def afd_ffn_destroy(h: int) -> None:
    _check(load().afd_ffn_destroy(h))


def afd_ffn_device_bytes(h: int) -> int:
    return int(load().afd_ffn_device_bytes(h))


def afd_ffn_route_bytes(h: int) -> int:
    return int(load().afd_ffn_route_bytes(h))


def afd_ffn_quantize_fp8(src, rows: int, cols: int, src_dtype: int, codes, scales, stream=None) -> None:
    _check(load().afd_ffn_quantize_fp8(_ptr(src), int(rows), int(cols), int(src_dtype), _ptr(codes), _ptr(scales),
                                       stream))


def afd_ffn_set_gemm_kernel(h: int, kernel: int) -> None:
    _check(load().afd_ffn_set_gemm_kernel(h, int(kernel)))


def afd_ffn_set_profiling(h: int, on: bool) -> None:
    _check(load().afd_ffn_set_profiling(h, 1 if on else 0))


def afd_ffn_profile_read(h: int):
    """{stage name: (milliseconds, launches)} summed since the last read."""
    ms = (ctypes.c_double * AFD_NUM_STAGES)()
    n = (ctypes.c_int64 * AFD_NUM_STAGES)()
    _check(load().afd_ffn_profile_read(h, ms, n, AFD_NUM_STAGES))
    return {STAGES[i]: (ms[i], int(n[i])) for i in range(AFD_NUM_STAGES)}
