"""The key split of in-flight chunk 0 (wf_chunk_causal_attn_fwd_ws) against the fp64
oracle and against the unsplit call: chunk 0's rows within the round tolerance of
the exact values, every other row bitwise that of wf_chunk_causal_attn_fwd; chunk
sizes around the key-tile boundaries (one key tile: no split), peaked rows, a long
chunk, permuted slots, causality and determinism, and rounds that do not split
(one chunk in flight, fp32). The workspace starts as NaN bytes, so a read of
anything the kernels did not write would show."""
import numpy as np
import pytest
import torch

import roundlib as RL
from workloads import CONFIGS, RoundConfig, make_round_inputs

pytestmark = pytest.mark.gpu


def _check_split(wf, inp, table=None, n_slots=None, lse_tol=2e-3):
    cfg = inp.cfg
    print(f"[case] split {cfg.name}", flush=True)
    out_s, lse_s, _ = RL.gpu_round(wf, inp, table=table, n_slots=n_slots, split=True)
    out_u, lse_u, _ = RL.gpu_round(wf, inp, table=table, n_slots=n_slots)
    ref_o, ref_l = RL.oracle_round(inp)
    RL.assert_close(out_s.float().cpu().numpy(), ref_o, cfg.dtype, f"{cfg.name} split")
    assert np.abs(lse_s.cpu().numpy() - ref_l).max() <= lse_tol
    C = cfg.chunk_tokens
    # chunks 1 .. N-1 take the unsplit kernel path: bitwise equal
    assert torch.equal(out_s[C:], out_u[C:])
    assert torch.equal(lse_s[:, C:].reshape(-1), lse_u[:, C:].reshape(-1))
    return out_s, out_u


# query tiles hold 256 rows, key tiles 64 keys: chunk 0 (with no history) has 1, 2 or 3 key tiles
@pytest.mark.parametrize("C", [33, 64, 65, 127, 128, 129, 255, 256, 257])
def test_split_chunk_sizes_no_history(C):
    wf = RL.require_gpu()
    cfg = RoundConfig(f"split_c{C}", 2, 128, C, 3, 0, "bf16", seed=1200 + C)
    out_s, out_u = _check_split(wf, make_round_inputs(cfg))
    if C <= 64:  # one key tile: nothing to halve, the call is the unsplit one
        assert torch.equal(out_s, out_u)


@pytest.mark.parametrize("cfg", [
    RoundConfig("split_hist_d128", 2, 128, 300, 3, 2, "bf16", seed=1301),   # 3 chunks x 5 tiles = 15: 7 + 8
    RoundConfig("split_hist_d64", 3, 64, 200, 2, 1, "bf16", seed=1302),
    RoundConfig("split_tiny_chunks", 2, 128, 5, 4, 3, "bf16", seed=1303),  # 4 one-tile chunks: 2 + 2
    RoundConfig("split_odd_tiles", 2, 128, 150, 2, 2, "bf16", seed=1304),  # 3 chunks x 3 tiles = 9: 4 + 5
    RoundConfig("split_multi_qtile", 2, 128, 520, 2, 0, "bf16", seed=1305),
], ids=lambda c: c.name)
def test_split_parity(cfg):
    wf = RL.require_gpu()
    _check_split(wf, make_round_inputs(cfg))


def test_split_peaked_rows():
    """Logits up to ~±100: the two halves see very different maxima, so the merge
    weights span many binades."""
    wf = RL.require_gpu()
    cfg = RoundConfig("split_peaked", 2, 128, 300, 3, 2, "bf16", seed=1306)
    inp = make_round_inputs(cfg)
    rnd = RL.round_like("bf16")
    for name in ("q", "k_hist", "k_in"):
        setattr(inp, name, rnd(getattr(inp, name) * 6.0))
    # a row whose weight sum is one bf16-rounded weight has an LSE error up to ln(1 + 2^-8):
    # the peaked rows' LSE bound of the unsplit call
    _check_split(wf, inp, lse_tol=2e-2)


def test_split_permuted_slots_bitwise():
    """Physical slot placement changes nothing, split or not."""
    wf = RL.require_gpu()
    cfg = RoundConfig("split_perm", 2, 128, 300, 3, 2, "bf16", seed=1307)
    inp = make_round_inputs(cfg)
    a, la, _ = RL.gpu_round(wf, inp, split=True)
    b, lb, _ = RL.gpu_round(wf, inp, table=[6, 2, 0, 5, 3], n_slots=7, split=True)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_split_causal_and_deterministic():
    """Chunk 0's split output ignores later chunks (bitwise) and repeats bitwise."""
    wf = RL.require_gpu()
    cfg = RoundConfig("split_causal", 2, 128, 300, 4, 2, "bf16", seed=1308)
    inp = make_round_inputs(cfg)
    a, la, _ = RL.gpu_round(wf, inp, split=True)
    a2, la2, _ = RL.gpu_round(wf, inp, split=True)
    assert torch.equal(a, a2) and torch.equal(la, la2)
    C = cfg.chunk_tokens
    rng = np.random.default_rng(5)
    rnd = RL.round_like("bf16")
    for name in ("q", "k_in", "v_in"):
        x = getattr(inp, name).copy()
        x[C:] = rnd(rng.standard_normal(x[C:].shape).astype(np.float32))
        setattr(inp, name, x)
    b, lb, _ = RL.gpu_round(wf, inp, split=True)
    assert torch.equal(a[:C], b[:C]) and torch.equal(la[:, :C], lb[:, :C])


@pytest.mark.parametrize("cfg", [
    RoundConfig("nosplit_one_inflight", 2, 128, 300, 1, 3, "bf16", seed=1309),
    RoundConfig("nosplit_f32", 2, 128, 300, 3, 2, "f32", seed=1310),
], ids=lambda c: c.name)
def test_rounds_that_do_not_split(cfg):
    """One chunk in flight (no longer class to balance), or an fp32 cache (no
    workspace): the workspace call returns the unsplit result bitwise."""
    wf = RL.require_gpu()
    inp = make_round_inputs(cfg)
    dt = RL.torch_dtype(cfg.dtype)
    dev = {k: RL.to_dev(getattr(inp, k), dt) for k in ("q", "k_hist", "v_hist", "k_in", "v_in")}
    cache = RL.build_cache(wf, cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, dt, dev["k_hist"], dev["v_hist"],
                           dev["k_in"], dev["v_in"])
    ws = torch.full((1 << 20,), 0xFF, dtype=torch.uint8, device="cuda")  # any buffer: it must go unused
    a, la = wf.chunk_causal_attn_fwd(dev["q"], cache, cfg.n_inflight, cfg.scale, workspace=ws)
    b, lb = wf.chunk_causal_attn_fwd(dev["q"], cache, cfg.n_inflight, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    assert bool((ws == 0xFF).all())
    if cfg.dtype == "f32":
        assert wf.attn_fwd_workspace_bytes(cache) == 0


def test_split_long_chunk_sampled():
    """One head, two 32768-token chunks: chunk 0's 512 key tiles halve to 256 + 256."""
    wf = RL.require_gpu()
    cfg = RoundConfig("split_long_chunk", 1, 128, 32768, 2, 0, "bf16", seed=1311)
    inp = make_round_inputs(cfg)
    out, lse, _ = RL.gpu_round(wf, inp, split=True)
    rows = RL.boundary_rows(cfg.chunk_tokens, 1, 24, seed=6)  # chunk 0 rows
    ref_o, ref_l = RL.oracle_round(inp, rows=rows)
    got = out[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    RL.assert_close(got, ref_o, "bf16", f"split long chunk ({len(rows)} rows)")
    assert np.abs(lse.cpu().numpy()[:, rows] - ref_l).max() <= 2e-3


def test_split_wan13b_4step_sampled_rows():
    """The 1.3B-shaped 4-step round at full size with the split: chunk 0 rows sampled
    densely, the rest bitwise against the unsplit call."""
    wf = RL.require_gpu()
    cfg = CONFIGS["wan13b_4step"]
    print(f"[case] split {cfg.name}", flush=True)
    inp = make_round_inputs(cfg)
    out_s, lse_s, _ = RL.gpu_round(wf, inp, split=True)
    out_u, lse_u, _ = RL.gpu_round(wf, inp)
    C = cfg.chunk_tokens
    assert torch.equal(out_s[C:], out_u[C:])
    rows = RL.boundary_rows(C, 1, 48, seed=7)
    ref_o, ref_l = RL.oracle_round(inp, rows=rows)
    got = out_s[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    RL.assert_close(got, ref_o, "bf16", f"split O chunk 0 ({len(rows)} rows)")
    assert np.abs(lse_s.cpu().numpy()[:, rows] - ref_l).max() <= 2e-3
    assert torch.isfinite(out_s.float()).all()


def test_short_workspace_is_refused_before_any_launch():
    """The binding checks a caller's workspace against the size the call needs (the C
    calls take no size): one byte short raises, and nothing is enqueued."""
    wf = RL.require_gpu()
    C, H, D = 64, 2, 64
    cache = wf.KVCache(3, C, H, D, torch.bfloat16)
    kv = torch.zeros(C, H, D, dtype=torch.bfloat16, device="cuda")
    cache.append(kv, kv)
    cache.append(kv, kv)
    q = torch.zeros(2 * C, H, D, dtype=torch.bfloat16, device="cuda")
    need = wf.attn_fwd_workspace_bytes(cache)
    short = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="workspace holds"):
        wf.chunk_causal_attn_fwd(q, cache, 2, D ** -0.5, workspace=short)
    plan = wf.plan_1f1c(1, 3, 1, 1)  # round 1 of a 1-step rollout: chunk 1 appended
    with pytest.raises(ValueError, match="workspace holds"):
        wf.run_round(cache, plan, q[:plan.n_inflight * C], [kv] * plan.n_inflight, [kv] * plan.n_inflight,
                     D ** -0.5, workspace=short)
    assert cache.table() == [0, 1]
