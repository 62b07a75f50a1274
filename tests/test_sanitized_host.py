"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; device code is never built with a sanitizer).

The task-graph builder (graph.cpp) and the host side of api.hip are rebuilt
with -fsanitize=address,undefined on the host pass, and the CPU tests of the
C ABI (tests/test_abi_cpu.py: every exported symbol, config validation, the
graph builder, validator and protocol simulator, the megakernel's host-side
limits) run against that library in a child process with the clang ASan
runtime preloaded.  Any sanitizer report fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san():
    from decode_persistent_megakernel_02_amd import sanitize_build as build
    try:
        rt = build.asan_runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    lib = build.build_sanitized()
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = rt + (":" + pre if pre else "")
    env["MK_LIBRARY"] = lib
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return lib, rt, env


def test_sanitized_library_is_the_one_loaded(san):
    lib, rt, env = san
    lib, rt = os.path.realpath(lib), os.path.realpath(rt)  # /proc/self/maps lists resolved paths
    code = ("import os\nfrom decode_persistent_megakernel_02_amd import abi\n"
            "maps = open('/proc/self/maps').read()\n"
            f"assert os.path.realpath(abi.LIB_PATH) == {lib!r}, abi.LIB_PATH\n"
            f"assert {lib!r} in maps and {rt!r} in maps\n"
            "print('ok')\n")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-3000:]


def test_abi_cpu_tests_pass_under_asan_and_ubsan(san):
    _, _, env = san
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]


def test_the_sanitizer_build_reports_a_planted_overflow(san, tmp_path):
    """The same compiler flags on a throwaway program with a heap overflow:
    the report appears, so a clean run above means something."""
    src = tmp_path / "overflow.cpp"
    src.write_text("#include <cstdlib>\nint main(int c, char**) { int* p = (int*)std::malloc(8 * sizeof(int));\n"
                   "  int v = p[8 + c]; std::free(p); return v; }\n")
    exe = tmp_path / "overflow"
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang++")
    subprocess.run([clang, "-fsanitize=address", "-fsanitize=undefined", "-g", "-o", str(exe), str(src)],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60,
                       env={"ASAN_OPTIONS": "detect_leaks=0", "PATH": os.environ.get("PATH", "")})
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
