"""The boundary tests of test_abi.py once more, against a build of the
library whose host code carries AddressSanitizer and UndefinedBehavior-
Sanitizer (host code only: the GPU code is built as usual and never runs
here). An out-of-bounds access, use after free or undefined behaviour in the
validation, plan, layout or status code aborts the run and fails the test.
CPU only; the sanitizer runtime is clang's, preloaded into a child process."""
import glob
import importlib.util
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _build(outdir):
    spec = importlib.util.spec_from_file_location("oc_build", os.path.join(ROOT, "bit_fp8_attention_block_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    hipcc = b._hipcc()
    flags = [f for f in b.FLAGS if f != "-O3"] + ["-O1", "-g"] + SANITIZE

    def one(src):
        obj = os.path.join(outdir, src.replace(".hip", ".o"))
        r = subprocess.run([hipcc, *flags, "-c", os.path.join(b.CSRC, src), "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(len(b.SOURCES)) as ex:
        objs = list(ex.map(one, b.SOURCES))
    lib = os.path.join(outdir, "liboc_attn_sanitized.so")
    r = subprocess.run([hipcc, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-shared-libasan", *SANITIZE[:4],
                        "-o", lib, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return lib


def test_boundary_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    runtime = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not runtime:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    lib = _build(str(tmp_path))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the build is not instrumented"
    env = dict(os.environ, LD_PRELOAD=runtime[-1], OC_ATTN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "failed" not in r.stdout
    # the child really ran the sanitized build
    probe = subprocess.run([sys.executable, "-c", "import bit_fp8_attention_block_amd as oc; print(oc.LIB_PATH)"],
                           env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert probe.stdout.strip() == lib, probe.stderr[-2000:]
