"""Builds libwf.so (the HIP kernels and the C ABI host glue) for gfx950 with hipcc.

    python -m chunk_causal_dit_amd.build        # or build() from Python

The library is written next to this file so that it travels with the source
tree; nothing is installed.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libwf.so")

SOURCES = ["wf_api.cpp", "rollout.cpp", "kv_cache.hip", "rope3d.hip", "attn_fwd.hip", "attn_i8qk.hip", "w8a8.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False, jobs: int = 4, out: str = LIB) -> str:
    """Compile every source to an object, then link the library (libwf.so by
    default). Returns the library path."""
    cc = hipcc()
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    common = [
        "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"-I{INCLUDE}", f"-I{CSRC}",
        "-Wall", "-Wno-unused-function",
    ]
    hip_flags = [
        f"--offload-arch={ARCH}", "-x", "hip",
        # no packed-FP32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]
    procs = []
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(obj_dir, src + ".o")
        objs.append(obj)
        cmd = [cc, "-c"]
        if src.endswith(".hip"):
            cmd += hip_flags
        cmd += [path, "-o", obj] + common
        if src.endswith(".hip"):
            pass
        else:
            cmd += ["-D__HIP_PLATFORM_AMD__"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _drain(procs)
    _drain(procs)
    tmp = out + ".tmp"
    link = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout.decode(errors="replace"))
    os.replace(tmp, out)
    return out


C_CONSUMER_SRC = os.path.join(ROOT, "tests", "c_consumer", "wf_round.c")
C_CONSUMER = os.path.join(ROOT, "tests", "c_consumer", "wf_round")


def build_c_consumer(verbose: bool = False) -> str:
    """Compile the plain-C consumer of the ABI (tests/c_consumer/wf_round.c) with gcc as
    C11 against include/wf.h, linked to libwf.so next to this file and to the HIP runtime.
    Returns the program's path."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the C consumer")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    rpath = os.path.relpath(HERE, os.path.dirname(C_CONSUMER))
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-isystem", f"{rocm}/include", f"-I{INCLUDE}", C_CONSUMER_SRC, "-o", C_CONSUMER,
           f"-L{HERE}", "-l:libwf.so", f"-L{rocm}/lib", "-lamdhip64",
           f"-Wl,-rpath,$ORIGIN/{rpath}", f"-Wl,-rpath,{rocm}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if res.returncode != 0:
        raise RuntimeError("C consumer build failed:\n" + res.stdout.decode(errors="replace"))
    return C_CONSUMER


def _drain(procs):
    while procs:
        src, p = procs.pop(0)
        text, _ = p.communicate()
        msg = text.decode(errors="replace")
        # hipcc's host pass does not know the device-only feature flag; harmless.
        msg = "\n".join(l for l in msg.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            raise RuntimeError(f"compile of {src} failed:\n{msg}")
        if msg.strip():
            print(f"[{src}] {msg}", file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_c_consumer(verbose="-v" in sys.argv))
