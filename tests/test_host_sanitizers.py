"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt from the same sources with the sanitizers on its host
code only (device code is compiled as usual), then the host ABI tests run
against it in a child process with the sanitizer runtime preloaded: argument
validation, the closed-form planner (make_geo, tile_runs), the stride checks
(one_to_one, overlaps) and the useful-flop accounting, on every case those
tests hold.  The workgroup-map check (decode_block over many grids) is built
and run with the same sanitizers.  Any report aborts the child and fails the
test.  No GPU is used: the host tests launch nothing.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "partial_context_patch_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SOURCES = ["api.cpp", "attn_bf16.hip", "attn_f32.hip", "guidance.hip"]


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _env():
    return dict(os.environ, LD_PRELOAD=_runtime(), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) or _runtime() is None,
                                reason="hipcc or the clang sanitizer runtime is not available")


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")

    def compile_one(src):
        obj = str(d / (os.path.splitext(src)[0] + ".o"))
        subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN,
                        "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-c", os.path.join(CSRC, src),
                        "-o", obj], check=True, capture_output=True, timeout=600)
        return obj

    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = str(d / "libnpa_sanitized.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN[:4], "-shared-libsan", *objs,
                    "-o", lib], check=True, capture_output=True, timeout=300)
    return lib


def test_library_is_instrumented(sanitized_lib):
    syms = subprocess.run(["nm", sanitized_lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms


def test_host_abi_cases_under_sanitizers(sanitized_lib):
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from partial_context_patch_amd import npa\n"
            "npa.LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
            % (ROOT, sanitized_lib, os.path.join(ROOT, "tests", "test_abi_host.py")))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=_env(), timeout=600,
                       cwd=ROOT)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout and "error" not in r.stdout.lower()


def test_workgroup_map_under_sanitizers(tmp_path):
    exe = tmp_path / "block_order_check"
    subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(ROOT, "tests", "block_order_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
