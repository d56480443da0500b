"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Every call validates its arguments on the host before touching the device (null
pointers, sizes, alignments, overlaps, workspace sizes).  This builds the same
sources with the host side instrumented (device code is compiled as usual; the
sanitizers apply to host code only) and runs the host-validation tests
(tests/test_lib_cpu.py) against that build, with the sanitizer runtime preloaded
into the interpreter.  Any invalid access or undefined behaviour in a validator
aborts the run."""
import glob
import os
import shutil
import subprocess
import sys
import concurrent.futures as cf

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_attention_verification_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(not os.path.exists(HIPCC) or _asan_runtime() is None, reason="hipcc or the ASan runtime missing")
def test_host_validation_under_address_and_undefined_sanitizers(tmp_path):
    # host-only instrumentation: each sanitizer flag follows -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-Wno-unused-result"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, *san, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(min(len(sources), 4)) as ex:
        objs = list(ex.map(compile_one, sources))
    lib = str(tmp_path / "libtreeverify_san.so")
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-shared-libasan", *san[:4], *objs,
                        "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    nm = shutil.which("nm")
    if nm:
        syms = subprocess.run([nm, "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms, "the host code is not instrumented"
    env = dict(os.environ, TREEVERIFY_LIB=lib, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_lib_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
