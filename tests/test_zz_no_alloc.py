"""wf_chunk_causal_attn_fwd_static (the allocation-free key-split call) through the C ABI,
against wf_chunk_causal_attn_fwd_ws (the same call with a caller's workspace): two calls
in a row on one GPU, the second on a smaller round, each bitwise equal to the workspace
call and within the bf16 bounds of the oracle."""
import numpy as np
import pytest
import torch

import roundlib as RL
from workloads import CONFIGS, RoundConfig, make_round_inputs

pytestmark = pytest.mark.gpu


def _static_vs_ws(wf, cfg, rows=None):
    print(f"[case] static scratch {cfg.name}", flush=True)
    inp = make_round_inputs(cfg)
    dt = RL.torch_dtype(cfg.dtype)
    C, H, D = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim
    dev = {k: RL.to_dev(getattr(inp, k), dt) for k in ("q", "k_hist", "v_hist", "k_in", "v_in")}
    cache = RL.build_cache(wf, C, H, D, dt, dev["k_hist"], dev["v_hist"], dev["k_in"], dev["v_in"])
    out_s, lse_s = wf.chunk_causal_attn_fwd_static(dev["q"], cache, cfg.n_inflight, cfg.scale)
    torch.cuda.synchronize()
    ws = RL.split_workspace(wf, cache)
    out_w, lse_w = wf.chunk_causal_attn_fwd(dev["q"], cache, cfg.n_inflight, cfg.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_w) and torch.equal(lse_s, lse_w), "static scratch differs from the workspace call"
    ref_o, ref_l = RL.oracle_round(inp, rows=rows)
    sel = slice(None) if rows is None else torch.from_numpy(rows).cuda()
    RL.assert_close(out_s[sel].float().cpu().numpy(), ref_o, cfg.dtype, f"static {cfg.name}")
    assert np.abs(lse_s[:, sel].cpu().numpy() - ref_l).max() <= 2e-3
    cache.close()


def test_static_scratch_two_calls_second_smaller():
    wf = RL.require_gpu()
    big = CONFIGS["wan13b_4step"]  # 58.4 MB of partials in the 64 MiB scratch
    _static_vs_ws(wf, big, rows=RL.boundary_rows(big.chunk_tokens, big.n_inflight, 4, seed=21))
    small = RoundConfig("static_small", 2, 128, 300, 3, 2, "bf16", seed=22)
    _static_vs_ws(wf, small)  # the scratch still holds the first call's partials
