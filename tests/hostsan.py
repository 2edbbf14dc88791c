"""Builds libwf with AddressSanitizer and UndefinedBehaviorSanitizer on the host
code (the C ABI glue, the planner and the launch wrappers; device code is
compiled as usual) and runs the host-side CPU tests against it.

The sanitizers apply to host code only: every -fsanitize flag reaches the
host compiler through -Xarch_host. The Python interpreter is not instrumented,
so the ASan runtime is preloaded into the child process that runs the tests.
"""
from __future__ import annotations

import glob
import os
import shlex
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

from chunk_causal_dit_amd import build as B  # noqa: E402

OUT_DIR = os.path.join(HERE, "_hostsan")
LIB = os.path.join(OUT_DIR, "libwf_hostsan.so")
HOST_SAN = shlex.split("-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-sanitize-recover=undefined "
                       "-Xarch_host -fno-omit-frame-pointer")
# host-side test files that drive the glue without a GPU
HOST_TESTS = ["tests/test_abi_cpu.py", "tests/test_rollout_cpu.py"]


def asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's ASan runtime (libclang_rt.asan-x86_64.so) was not found")
    return hits[-1]


def build_sanitized(jobs: int = 4) -> str:
    """Compile every source with host sanitizers into tests/_hostsan/libwf_hostsan.so."""
    cc = B.hipcc()
    os.makedirs(OUT_DIR, exist_ok=True)
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"-I{B.INCLUDE}", f"-I{B.CSRC}"] + HOST_SAN
    hip = [f"--offload-arch={B.ARCH}", "-x", "hip", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    procs, objs = [], []
    for src in B.SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        objs.append(obj)
        cmd = [cc, "-c"] + (hip if src.endswith(".hip") else ["-D__HIP_PLATFORM_AMD__"])
        cmd += [os.path.join(B.CSRC, src), "-o", obj] + common
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            B._drain(procs)
    B._drain(procs)
    link = [cc, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", "-o", LIB] + objs + HOST_SAN
    res = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout.decode(errors="replace"))
    return LIB


def run_host_tests(lib: str = LIB, leaks: bool = True, timeout: int = 600) -> subprocess.CompletedProcess:
    """Run the host-side CPU tests in a child process against the sanitized library.
    With leaks, LeakSanitizer reports every allocation still live at exit (the
    interpreter's included); the caller picks out those made by the library."""
    env = dict(os.environ)
    pre = asan_runtime()
    env["LD_PRELOAD"] = (env["LD_PRELOAD"] + ":" + pre) if env.get("LD_PRELOAD") else pre
    env["WF_LIBRARY"] = lib
    env["ASAN_OPTIONS"] = f"detect_leaks={int(leaks)}:abort_on_error=0:halt_on_error=1:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=24"
    llvm = pre
    for _ in range(6):  # <llvm>/lib/clang/<v>/lib/linux/<runtime> -> <llvm>
        llvm = os.path.dirname(llvm)
    sym = os.path.join(llvm, "bin", "llvm-symbolizer")
    if os.path.exists(sym):
        env["ASAN_SYMBOLIZER_PATH"] = sym
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + HOST_TESTS
    return subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                          timeout=timeout)


def instrumented(lib: str) -> bool:
    """True when the library's dynamic symbols reference the sanitizer runtimes."""
    res = subprocess.run(["nm", "-D", "--undefined-only", lib], stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    text = res.stdout.decode(errors="replace")
    return "__asan_report" in text and "__ubsan_handle" in text


if __name__ == "__main__":
    print(build_sanitized())
    r = run_host_tests()
    print(r.stdout.decode(errors="replace")[-4000:])
    sys.exit(r.returncode)
