"""GPU parity of wf_chunk_causal_attn_fwd against the fp64 oracle (called through the C ABI)."""
import math

import numpy as np
import pytest
import torch

import roundlib as RL
from workloads import CONFIGS, RoundConfig, make_round_inputs

pytestmark = pytest.mark.gpu


def _small(name, H, D, C, N, Hs, dtype, seed):
    return RoundConfig(name, H, D, C, N, Hs, dtype, seed=seed)


SMALL = [
    CONFIGS["tiny_f32"],
    _small("ragged_bf16_d128", 2, 128, 300, 3, 2, "bf16", 11),   # 2 query tiles, ragged key/query tails
    _small("ragged_bf16_d64", 3, 64, 200, 2, 1, "bf16", 12),
    _small("ragged_f32_d128", 2, 128, 100, 3, 1, "f32", 13),
    _small("multi_tile_bf16", 2, 128, 520, 2, 0, "bf16", 14),    # 3 query tiles of 256 rows, 9 key tiles
    _small("one_chunk_bf16", 1, 128, 64, 1, 0, "bf16", 15),
    _small("tiny_chunks_bf16", 2, 128, 5, 4, 3, "bf16", 16),     # C < key tile
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_parity_full(cfg):
    wf = RL.require_gpu()
    print(f"[case] {cfg.name}", flush=True)
    inp = make_round_inputs(cfg)
    out, lse, _ = RL.gpu_round(wf, inp)
    ref_o, ref_l = RL.oracle_round(inp)
    RL.assert_close(out.float().cpu().numpy(), ref_o, cfg.dtype, "O")
    lse_err = np.abs(lse.cpu().numpy() - ref_l).max()
    print(f"[parity] LSE max abs {lse_err:.3e}", flush=True)
    assert lse_err <= (1e-4 if cfg.dtype == "f32" else 2e-3)


@pytest.mark.parametrize("split", [True, False], ids=["ws_split", "plain"])
def test_wan13b_4step_all_rows(split):
    """The 1.3B-shaped 4-step round at full size, every one of its 23,400 query rows
    and 12 heads against the oracle: the workspace call (chunk 0 split over its key
    range, the launch the bench times) and the plain call."""
    wf = RL.require_gpu()
    cfg = CONFIGS["wan13b_4step"]
    print(f"[case] {cfg.name} split={split}", flush=True)
    inp = make_round_inputs(cfg)
    out, lse, _ = RL.gpu_round(wf, inp, split=split)
    ref_o, ref_l = RL.oracle_round(inp)
    got = out.float().cpu().numpy()
    RL.assert_close(got, ref_o, "bf16", f"O (all {got.shape[0]} rows)")
    lse_err = np.abs(lse.cpu().numpy() - ref_l).max()
    print(f"[parity] LSE max abs {lse_err:.3e}", flush=True)
    assert lse_err <= 2e-3
