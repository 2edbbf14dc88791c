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
