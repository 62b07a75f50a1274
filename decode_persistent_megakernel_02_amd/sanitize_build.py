"""The library with its host code under AddressSanitizer and
UndefinedBehaviorSanitizer, for CPU tests (tests/test_sanitized_host.py).

    python -m decode_persistent_megakernel_02_amd.sanitize_build

Device code is built as usual: the sanitizer flags go to the host pass only.
"""
import os

from decode_persistent_megakernel_02_amd.build import ARCH, CSRC, HIP_FLAGS, PKG, ROOT, _run, build_lib

SAN_LIB = os.path.join(PKG, "_build", "san", "libmk_san.so")


def asan_runtime():
    """The clang ASan runtime (which carries UBSan's handlers) that a process
    loading SAN_LIB must preload."""
    llvm = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(llvm), reverse=True):
        p = os.path.join(llvm, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under " + llvm)


def build_sanitized(verbose=False):
    """The library with its host code under AddressSanitizer and
    UndefinedBehaviorSanitizer: the task-graph builder (graph.cpp) and the host
    side of api.hip (argument checks, set-up, buffer bookkeeping).  Device
    code is built as usual (the sanitizer flags apply to the host pass only)
    and the kernel objects are those of build_lib, compiled first if absent.
    Load it with asan_runtime() preloaded and MK_LIBRARY=SAN_LIB."""
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang++")
    bdir = os.path.join(PKG, "_build")
    dev = [os.path.join(bdir, n) for n in ("kernels.hip.o", "mega.hip.MK_MEGA_PART0.o", "mega.hip.MK_MEGA_PART1.o",
                                            "mega.hip.MK_MEGA_PART2.o", "batched.hip.o", "prefill.hip.o")]
    if not all(os.path.exists(o) for o in dev):
        build_lib(verbose)
    sdir = os.path.dirname(SAN_LIB)
    os.makedirs(sdir, exist_ok=True)
    inc = ["-I", CSRC, "-I", os.path.join(ROOT, "include")]
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    api_o = os.path.join(sdir, "api.hip.o")
    host_san = [x for f in san for x in ("-Xarch_host", f)]
    _run([hipcc] + HIP_FLAGS + inc + host_san + ["-g", "-c", "-o", api_o, os.path.join(CSRC, "api.hip")], verbose)
    graph_o = os.path.join(sdir, "graph.o")
    _run([clang, "-O1", "-g", "-std=c++17", "-fPIC", "-Wall"] + san + inc +
         ["-c", "-o", graph_o, os.path.join(CSRC, "graph.cpp")], verbose)
    tmp = SAN_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-o", tmp] + dev + [api_o, graph_o, "-lrocblas"], verbose)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build_sanitized(verbose=True))
