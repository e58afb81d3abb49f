"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU oracle and of the
C ABI's host code, each driven by a small program (tests/sanitize/): the oracle's
functions on small seeded inputs, and every entry point's argument checks on a
hand-built handle (no GPU).  Any sanitizer report, or a failed check, fails the test.

The sanitizers instrument host code only: on the hipcc line each -fsanitize= follows
-Xarch_host, so the gfx950 device code is built as usual.  Builds are cached under
_build/sanitize, keyed by a digest of their sources."""
import glob
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "moe_expert_ffn_softmax_amd", "csrc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _digest(files):
    h = hashlib.sha256()
    for f in sorted(files):
        with open(f, "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _cached(name, sources, build):
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, f"{name}-{_digest(sources)}")
    if not os.path.exists(exe):
        build(exe + ".tmp")
        os.replace(exe + ".tmp", exe)
    return exe


def _run(exe, expect):
    env = dict(os.environ, **SAN_ENV)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert expect in r.stdout, report[-4000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in report, report[-4000:]


def test_oracle_under_address_and_undefined_sanitizers():
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    srcs = [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "afd_oracle.c")]

    def build(exe):
        subprocess.check_call(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
                               "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe, *srcs, "-lm"])

    _run(_cached("oracle_driver", srcs, build), "oracle driver ok")


def test_abi_host_code_under_address_and_undefined_sanitizers():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    from moe_expert_ffn_softmax_amd import build as B
    lib_srcs = B.sources()
    driver = os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")
    headers = glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]

    def build(exe):
        objdir = exe + ".objs"
        os.makedirs(objdir, exist_ok=True)
        procs, objs = [], []
        for src in lib_srcs:
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            objs.append(obj)
            procs.append(subprocess.Popen([hipcc, *B.flags_for(src), *san, "-c", src, "-o", obj],
                                          stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
        for p in procs:
            out = p.communicate()[0]
            assert p.returncode == 0, out.decode()[-3000:]
        dobj = os.path.join(objdir, "abi_driver.o")
        subprocess.check_call([hipcc, *B.HIP_FLAGS, *san, "-x", "hip", "-c", driver, "-o", dobj],
                              stdout=subprocess.DEVNULL, stderr=subprocess.STDOUT)
        subprocess.check_call([hipcc, f"--offload-arch={B.ARCH}", *san, "-o", exe, *objs, dobj],
                              stdout=subprocess.DEVNULL, stderr=subprocess.STDOUT)
        shutil.rmtree(objdir, ignore_errors=True)

    _run(_cached("abi_driver", lib_srcs + [driver] + headers, build), "abi driver ok")
