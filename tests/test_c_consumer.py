"""The C ABI from plain C: tests/c_consumer/wf_round.c includes include/wf.h, takes
device memory from the HIP runtime and runs one round through libwf with no Python,
torch or C++ in between.

  * CPU: the program and the header compile as C11 with gcc (-Wall -Wextra -Werror).
  * GPU: the program built by build() runs fp32 and bf16 rounds (bf16 with and without
    the key-split workspace); O and LSE match the fp64 oracle at the usual bounds.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import roundlib as RL
from workloads import CONFIGS, RoundConfig, make_round_inputs

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_consumer", "wf_round.c")
PROG = os.path.join(HERE, "c_consumer", "wf_round")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
WF_F32, WF_BF16 = 0, 1


def _gcc():
    cc = shutil.which("gcc")
    if cc is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("gcc or the HIP runtime headers are not available")
    return cc


def test_c_consumer_compiles_as_c11(tmp_path):
    cc = _gcc()
    res = subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic-errors", "-fsyntax-only",
                          "-D__HIP_PLATFORM_AMD__", "-isystem", f"{ROCM}/include", f"-I{ROOT}/include", SRC],
                         stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    assert res.returncode == 0, res.stdout.decode(errors="replace")


def test_header_alone_is_c89(tmp_path):
    """include/wf.h on its own compiles as strict C89 (no C99 or C++ constructs)."""
    cc = _gcc()
    tu = tmp_path / "tu.c"
    tu.write_text('#include "wf.h"\nint wf_header_probe(void) { return WF_OK + WF_MAX_TABLE; }\n')
    res = subprocess.run([cc, "-std=c89", "-Wall", "-Wextra", "-Werror", "-pedantic-errors", "-fsyntax-only",
                          f"-I{ROOT}/include", str(tu)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    assert res.returncode == 0, res.stdout.decode(errors="replace")


def _bits(a: np.ndarray, dtype: str) -> bytes:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a.tobytes()
    return (a.view(np.uint32) >> 16).astype(np.uint16).tobytes()  # values are bf16-representable


def _from_bits(raw: bytes, dtype: str, shape) -> np.ndarray:
    if dtype == "f32":
        return np.frombuffer(raw, dtype=np.float32).reshape(shape)
    u = np.frombuffer(raw, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).reshape(shape)


CASES = [
    CONFIGS["tiny_f32"],
    RoundConfig("c_bf16_ragged", 2, 128, 300, 3, 2, "bf16", seed=61),
]


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_c_consumer_round_matches_oracle(cfg, tmp_path):
    RL.require_gpu()
    assert os.path.exists(PROG), "tests/c_consumer/wf_round is missing: run build() first"
    print(f"[case] c consumer {cfg.name}", flush=True)
    inp = make_round_inputs(cfg)
    C, H, D, N, Hs = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, cfg.n_inflight, cfg.n_hist
    dt = WF_F32 if cfg.dtype == "f32" else WF_BF16
    hdr = np.array([C, H, D, Hs, N, dt], dtype=np.int32).tobytes() + np.float32(cfg.scale).tobytes()
    body = b"".join(_bits(a, cfg.dtype) for a in (inp.q, inp.k_hist, inp.v_hist, inp.k_in, inp.v_in))
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    fin.write_bytes(hdr + body)
    res = subprocess.run([PROG, str(fin), str(fout)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         timeout=120)
    print(res.stdout.decode(errors="replace").strip(), flush=True)
    assert res.returncode == 0
    raw = fout.read_bytes()
    esize = 4 if cfg.dtype == "f32" else 2
    o_bytes, l_bytes = N * C * H * D * esize, H * N * C * 4
    runs = 1 if cfg.dtype == "f32" else 2
    assert len(raw) == runs * (o_bytes + l_bytes)
    ref_o, ref_l = RL.oracle_round(inp)
    for run in range(runs):
        base = run * (o_bytes + l_bytes)
        out = _from_bits(raw[base:base + o_bytes], cfg.dtype, (N * C, H, D))
        lse = np.frombuffer(raw[base + o_bytes:base + o_bytes + l_bytes], dtype=np.float32).reshape(H, N * C)
        what = ("plain", "workspace split")[run]
        RL.assert_close(out, ref_o, cfg.dtype, f"C consumer {cfg.name} O ({what})")
        lse_err = np.abs(lse - ref_l).max()
        print(f"[parity] C consumer {cfg.name} LSE ({what}) max abs {lse_err:.3e}", flush=True)
        assert lse_err <= (1e-4 if cfg.dtype == "f32" else 2e-3)
