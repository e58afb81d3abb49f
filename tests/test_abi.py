"""The C ABI without a GPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before touching the device."""
import ctypes
import os
import re

import pytest

from moe_expert_ffn_softmax_amd import _ffi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "afd_ffn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(afd_ffn_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("afd_ffn_create", "afd_ffn_route", "afd_ffn_forward", "afd_ffn_destroy", "afd_ffn_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _ffi.load()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_struct_layouts_match_header():
    assert ctypes.sizeof(_ffi.afd_ffn_config) == 7 * 4
    assert ctypes.sizeof(_ffi.afd_route) == 6 * 8


def _cfg(**kw):
    base = dict(hidden=256, inter=512, num_experts=8, top_k=2, max_tokens=64, shared_inter=0, dtype=_ffi.AFD_BF16)
    base.update(kw)
    return _ffi.afd_ffn_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=100), _ffi.AFD_EINVAL),
    (dict(hidden=0), _ffi.AFD_EINVAL),
    (dict(inter=96), _ffi.AFD_EINVAL),
    (dict(shared_inter=64), _ffi.AFD_EINVAL),
    (dict(num_experts=0), _ffi.AFD_EINVAL),
    (dict(num_experts=2048), _ffi.AFD_EINVAL),
    (dict(top_k=0), _ffi.AFD_EINVAL),
    (dict(top_k=9), _ffi.AFD_EINVAL),
    (dict(num_experts=64, top_k=33), _ffi.AFD_EINVAL),
    (dict(max_tokens=0), _ffi.AFD_EINVAL),
    (dict(max_tokens=1 << 28, top_k=8), _ffi.AFD_EINVAL),
    (dict(dtype=7), _ffi.AFD_EINVAL),
    # fp8 layers: each activation matrix of max_tokens rows must stay under 4 GiB (x, routed h, shared h)
    (dict(dtype=_ffi.AFD_FP8_E4M3, hidden=65536, inter=128, max_tokens=65536), _ffi.AFD_EINVAL),
    (dict(dtype=_ffi.AFD_FP8_E4M3, inter=256, top_k=8, max_tokens=1 << 21), _ffi.AFD_EINVAL),
    (dict(dtype=_ffi.AFD_FP8_E4M3, shared_inter=4096, max_tokens=1 << 20), _ffi.AFD_EINVAL),
])
def test_create_rejects_bad_config(kw, code):
    lib = _ffi.load()
    h = ctypes.c_void_p()
    rc = lib.afd_ffn_create(ctypes.byref(_cfg(**kw)), 1, 1, None, None, None, None, None, None, None, ctypes.byref(h))
    assert rc == code
    assert h.value is None
    assert _ffi.afd_ffn_last_error() != ""


@pytest.mark.parametrize("kw", [
    dict(hidden=65536, inter=128, max_tokens=65536),
    dict(inter=256, top_k=8, max_tokens=1 << 21),
    dict(shared_inter=4096, max_tokens=1 << 20),
])
def test_create_names_the_fp8_activation_limit(kw):
    # the fp8 128-row GEMMs address activation rows by 32-bit byte offsets
    lib = _ffi.load()
    h = ctypes.c_void_p()
    rc = lib.afd_ffn_create(ctypes.byref(_cfg(dtype=_ffi.AFD_FP8_E4M3, **kw)), 1, 1, None, None, None, None, None,
                            None, None, ctypes.byref(h))
    assert rc == _ffi.AFD_EINVAL and h.value is None
    assert "4 GiB" in _ffi.afd_ffn_last_error()


def test_create_rejects_bad_pointers():
    lib = _ffi.load()
    h = ctypes.c_void_p()
    cfg = _cfg()
    assert lib.afd_ffn_create(None, 1, 1, None, None, None, None, None, None, None, ctypes.byref(h)) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_create(ctypes.byref(cfg), None, 1, None, None, None, None, None, None, None,
                              ctypes.byref(h)) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_create(ctypes.byref(cfg), 1, 1, 1, None, None, None, None, None, None,
                              ctypes.byref(h)) == _ffi.AFD_EINVAL          # scales without fp8
    assert lib.afd_ffn_create(ctypes.byref(_cfg(shared_inter=128)), 1, 1, None, None, None, None, None, None, None,
                              ctypes.byref(h)) == _ffi.AFD_EINVAL          # missing shared weights
    assert lib.afd_ffn_create(ctypes.byref(cfg), 1, 1, None, None, 1, 1, None, None, None,
                              ctypes.byref(h)) == _ffi.AFD_EINVAL          # shared weights w/o shared_inter
    assert lib.afd_ffn_create(ctypes.byref(cfg), 1, 1, None, None, None, None, None, None, None,
                              None) == _ffi.AFD_EINVAL
    fp8 = _cfg(dtype=_ffi.AFD_FP8_E4M3)
    assert lib.afd_ffn_create(ctypes.byref(fp8), 1, 1, None, None, None, None, None, None, None,
                              ctypes.byref(h)) == _ffi.AFD_EINVAL          # fp8 without block scales
    fp8s = _cfg(dtype=_ffi.AFD_FP8_E4M3, shared_inter=128)
    assert lib.afd_ffn_create(ctypes.byref(fp8s), 1, 1, 1, 1, 1, 1, None, None, None,
                              ctypes.byref(h)) == _ffi.AFD_EINVAL          # fp8 shared without scales


def test_create_rejects_misaligned_weights():
    lib = _ffi.load()
    h = ctypes.c_void_p()
    cfg = _cfg()
    assert lib.afd_ffn_create(ctypes.byref(cfg), 0x10002, 0x20000, None, None, None, None, None, None, None,
                              ctypes.byref(h)) == _ffi.AFD_EINVAL
    assert "aligned" in _ffi.afd_ffn_last_error()
    assert h.value is None


def test_quantize_rejects_bad_arguments():
    lib = _ffi.load()
    assert lib.afd_ffn_quantize_fp8(1, 4, 100, _ffi.AFD_BF16, 1, 1, None) == _ffi.AFD_EINVAL   # cols % 128
    assert lib.afd_ffn_quantize_fp8(1, 4, 128, _ffi.AFD_FP8_E4M3, 1, 1, None) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_quantize_fp8(None, 4, 128, _ffi.AFD_BF16, 1, 1, None) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_quantize_fp8(None, 0, 128, _ffi.AFD_BF16, None, None, None) == _ffi.AFD_OK  # empty
    assert lib.afd_ffn_quantize_fp8(0x10008, 4, 128, _ffi.AFD_BF16, 0x20000, 0x30000, None) == _ffi.AFD_EINVAL
    assert "aligned" in _ffi.afd_ffn_last_error()


def test_route_and_forward_reject_null_handle():
    lib = _ffi.load()
    r = _ffi.afd_route(1, 1, 1, 1, 1, 1)
    assert lib.afd_ffn_route(None, 1, 4, ctypes.byref(r), None) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_forward(None, 1, 4, ctypes.byref(r), 1, None) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_forward_fp8_input(None, 1, 1, 4, ctypes.byref(r), 1, None) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_forward_noalloc(None, 1, 4, ctypes.byref(r), 1, None) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_route_hidden(None, 1, 1, None, 1, 4, ctypes.byref(r), None) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_route_select_bias(None, 1, 1, 4, ctypes.byref(r), None) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_route_capacity(None, 4, 4, 4, 1, 1, 4, 4, 4, 4, 4, None) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_route_from_capacity(None, 4, 4, 4, 4, 4, ctypes.byref(r), None) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_destroy(None) == _ffi.AFD_OK
    assert lib.afd_ffn_set_profiling(None, 1) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_set_gemm_kernel(None, 0) == _ffi.AFD_EINVAL
    assert lib.afd_ffn_device_bytes(None) == 0
    assert lib.afd_ffn_route_bytes(None) == 0


def test_strerror_names_every_code():
    seen = set()
    for c in (_ffi.AFD_OK, _ffi.AFD_EINVAL, _ffi.AFD_EUNSUPPORTED, _ffi.AFD_ENOMEM, _ffi.AFD_EHIP):
        s = _ffi.afd_ffn_strerror(c)
        assert s and s not in seen
        seen.add(s)
    assert "unknown" in _ffi.afd_ffn_strerror(12345)


def test_product_path_does_not_touch_the_oracle():
    """The HIP library and its binding never import, link or call the oracle."""
    pkg = os.path.join(ROOT, "moe_expert_ffn_softmax_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text and "afdo_" not in text, f


def test_probe_library_exports_its_entry_points():
    """The measurement probes of bench.py --attainable live in their own library."""
    import os
    path = os.path.join(os.path.dirname(_ffi.LIB_PATH), "libafd_probe.so")
    lib = ctypes.CDLL(path)
    for n in ("afd_probe_stream", "afd_probe_mfma"):
        assert hasattr(lib, n), n
    lib.afd_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    lib.afd_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
    # argument checks run on the host before any launch
    assert lib.afd_probe_stream(None, 8192, 4, 8, 64, None) == -1
    assert lib.afd_probe_stream(64, 1000, 4, 8, 64, None) == -1      # not a multiple of depth KiB
    assert lib.afd_probe_stream(64, 8192, 4, 5, 64, None) == -1      # unsupported depth
    assert lib.afd_probe_mfma(2, 64, 8, 1, 64, None) == -1           # unknown kind
    assert lib.afd_probe_mfma(0, 64, 6, 1, 64, None) == -1           # waves not a multiple of 4
