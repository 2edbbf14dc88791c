"""Edge cases of the attention path through the C ABI, against the fp64 oracle:
chunk sizes on both sides of every tile boundary, the largest table
(WF_MAX_TABLE entries), a single chunk with no history, a long chunk, peaked
softmax rows (large logits, many moves of the reference max), the optional
LSE, and a launch on a side stream."""
import numpy as np
import pytest
import torch

import roundlib as RL
from workloads import RoundConfig, make_round_inputs

pytestmark = pytest.mark.gpu

# query tiles hold 256 rows (8 waves of 32), key tiles 64 keys, slots pad to 128
BOUNDARY_C = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


@pytest.mark.parametrize("C", BOUNDARY_C)
def test_chunk_sizes_around_tile_boundaries(C):
    wf = RL.require_gpu()
    cfg = RoundConfig(f"edge_c{C}", 2, 128, C, 3, 1, "bf16", seed=900 + C)
    print(f"[case] {cfg.name}", flush=True)
    inp = make_round_inputs(cfg)
    out, lse, _ = RL.gpu_round(wf, inp)
    ref_o, ref_l = RL.oracle_round(inp)
    RL.assert_close(out.float().cpu().numpy(), ref_o, "bf16", cfg.name)
    assert np.abs(lse.cpu().numpy() - ref_l).max() <= 2e-3


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_largest_table(dtype, D):
    """WF_MAX_TABLE = 64 entries: 60 history chunks and 4 in flight."""
    wf = RL.require_gpu()
    cfg = RoundConfig(f"maxtab_{dtype}", 2, D, 33, 4, 60, dtype, seed=950)
    print(f"[case] {cfg.name}", flush=True)
    inp = make_round_inputs(cfg)
    out, lse, cache = RL.gpu_round(wf, inp)
    assert len(cache.table()) == 64
    ref_o, ref_l = RL.oracle_round(inp)
    RL.assert_close(out.float().cpu().numpy(), ref_o, dtype, cfg.name)
    assert np.abs(lse.cpu().numpy() - ref_l).max() <= (1e-4 if dtype == "f32" else 2e-3)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_chunk_no_history(dtype):
    """n_inflight = 1, n_hist = 0: plain full attention over one chunk."""
    wf = RL.require_gpu()
    cfg = RoundConfig(f"single_{dtype}", 3, 128, 700, 1, 0, dtype, seed=951)
    inp = make_round_inputs(cfg)
    out, lse, _ = RL.gpu_round(wf, inp)
    ref_o, ref_l = RL.oracle_round(inp)
    RL.assert_close(out.float().cpu().numpy(), ref_o, dtype, cfg.name)


def test_long_chunk_sampled():
    """One head, two 32768-token chunks: 128 query tiles, 512 key tiles per chunk."""
    wf = RL.require_gpu()
    cfg = RoundConfig("long_chunk", 1, 128, 32768, 2, 0, "bf16", seed=952)
    inp = make_round_inputs(cfg)
    out, lse, _ = RL.gpu_round(wf, inp)
    rows = RL.boundary_rows(cfg.chunk_tokens, cfg.n_inflight, 16, seed=5)
    ref_o, ref_l = RL.oracle_round(inp, rows=rows)
    got = out[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    RL.assert_close(got, ref_o, "bf16", f"long chunk ({len(rows)} rows)")
    assert np.abs(lse.cpu().numpy()[:, rows] - ref_l).max() <= 2e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_peaked_rows_large_logits(dtype):
    """Q and K scaled by 6: logits up to ~±100 (scaled), so the reference max of
    a row moves many times; the result must still match."""
    wf = RL.require_gpu()
    cfg = RoundConfig(f"peaked_{dtype}", 2, 128, 300, 3, 2, dtype, seed=953)
    inp = make_round_inputs(cfg)
    rnd = RL.round_like(dtype)
    for name in ("q", "k_hist", "k_in"):
        setattr(inp, name, rnd(getattr(inp, name) * 6.0))
    out, lse, _ = RL.gpu_round(wf, inp)
    ref_o, ref_l = RL.oracle_round(inp)
    RL.assert_close(out.float().cpu().numpy(), ref_o, dtype, cfg.name)
    assert np.abs(lse.cpu().numpy() - ref_l).max() <= (1e-3 if dtype == "f32" else 2e-2)


def test_lse_is_optional_and_does_not_change_out():
    wf = RL.require_gpu()
    cfg = RoundConfig("nolse", 2, 128, 300, 3, 2, "bf16", seed=954)
    inp = make_round_inputs(cfg)
    a, la, cache = RL.gpu_round(wf, inp)
    q = RL.to_dev(inp.q, torch.bfloat16)
    b, lb = wf.chunk_causal_attn_fwd(q, cache, cfg.n_inflight, cfg.scale, with_lse=False)
    torch.cuda.synchronize()
    assert lb is None and torch.equal(a, b)


def test_side_stream_launch_is_ordered_on_that_stream():
    """Cache writes and attention enqueued on a side stream; the result equals the default-stream result."""
    wf = RL.require_gpu()
    cfg = RoundConfig("stream", 2, 128, 300, 3, 2, "bf16", seed=955)
    inp = make_round_inputs(cfg)
    ref, ref_l, _ = RL.gpu_round(wf, inp)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        dt = torch.bfloat16
        dev = {k: RL.to_dev(getattr(inp, k), dt) for k in ("q", "k_hist", "v_hist", "k_in", "v_in")}
        C, H, D = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim
        cache = wf.KVCache(cfg.n_hist + cfg.n_inflight, C, H, D, dt, stream=side)
        for k, v in zip(RL.chunks(torch.cat([dev["k_hist"], dev["k_in"]]), C),
                        RL.chunks(torch.cat([dev["v_hist"], dev["v_in"]]), C)):
            cache.append(k, v, stream=side)
        out, lse = wf.chunk_causal_attn_fwd(dev["q"], cache, cfg.n_inflight, cfg.scale, stream=side)
    side.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_l)
