"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
without a GPU: every library source is compiled with both sanitizers on its host
side only (device code is built as the library ships it) and linked with
tests/abi_sanitize_main.cpp, which calls every entry point with NULL,
misaligned, negative, extreme and empty arguments and checks the status and
message of each. A sanitizer report aborts the driver and fails the test."""
import concurrent.futures
import hashlib
import importlib.util
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_indexer_fp4_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "abi_sanitize_main.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OUT_DIR = os.path.join(ROOT, "_build", "sanitize")
# every sanitizer option goes to the host compile only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _lib_flags():
    """The library's own compile flags and target."""
    spec = importlib.util.spec_from_file_location(
        "_fp4kv_build", os.path.join(ROOT, "sparse_indexer_fp4_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.FLAGS, mod.ARCH


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip")) + [DRIVER]


def _build():
    flags, arch = _lib_flags()
    h = hashlib.sha256(" ".join(flags + SAN).encode())
    headers = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h"))
    for f in _sources() + headers + [os.path.join(ROOT, "include", "fp4kv.h")]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    exe = os.path.join(OUT_DIR, f"abi_sanitize_{h.hexdigest()[:12]}")
    if os.path.exists(exe):
        return exe
    os.makedirs(OUT_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [HIPCC, *lang, *flags, *SAN, "-g", "-I", CSRC, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, _sources()))
    tmp = exe + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={arch}", *SAN[:4], *objs, "-o", tmp],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    os.replace(tmp, exe)
    return exe


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_checks_under_asan_and_ubsan():
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "all ABI checks passed" in r.stdout, r.stdout[-4000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
