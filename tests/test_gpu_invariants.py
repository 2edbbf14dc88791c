"""Invariants of the round that hold exactly (or bitwise) on the GPU path,
checked through the C ABI: chunk causality, normalisation, a single visible
key, the Q = 0 closed form, determinism, and argument errors."""
import numpy as np
import pytest
import torch

import roundlib as RL
from workloads import CONFIGS, RoundConfig, make_round_inputs

pytestmark = pytest.mark.gpu


def _run(wf, cfg, q, kh, vh, ki, vi):
    dt = RL.torch_dtype(cfg.dtype)
    cache = RL.build_cache(wf, cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, dt, kh, vh, ki, vi)
    out, lse = wf.chunk_causal_attn_fwd(q, cache, cfg.n_inflight, cfg.scale)
    torch.cuda.synchronize()
    return out, lse


def _dev_inputs(cfg):
    inp = make_round_inputs(cfg)
    dt = RL.torch_dtype(cfg.dtype)
    return [RL.to_dev(a, dt) for a in (inp.q, inp.k_hist, inp.v_hist, inp.k_in, inp.v_in)]


@pytest.mark.parametrize("cfg", [RoundConfig("caus_bf16", 2, 128, 300, 4, 2, "bf16", seed=31),
                                 RoundConfig("caus_f32", 2, 64, 100, 3, 1, "f32", seed=32),
                                 CONFIGS["wan13b_4step"]], ids=lambda c: c.name)
def test_later_chunks_do_not_change_earlier_outputs(cfg):
    """Perturbing Q/K/V of chunks after j (finite values) leaves chunk j's O and LSE bitwise equal."""
    wf = RL.require_gpu()
    print(f"[case] {cfg.name}", flush=True)
    q, kh, vh, ki, vi = _dev_inputs(cfg)
    o0, l0 = _run(wf, cfg, q, kh, vh, ki, vi)
    C = cfg.chunk_tokens
    g = torch.Generator(device="cuda")
    for j in (0, cfg.n_inflight - 2):
        g.manual_seed(1000 + j)
        q2, ki2, vi2 = q.clone(), ki.clone(), vi.clone()
        lo = (j + 1) * C
        for t in (q2, ki2, vi2):
            t[lo:] = (torch.randn(t[lo:].shape, device="cuda", generator=g) * 3).to(t.dtype)
        o1, l1 = _run(wf, cfg, q2, kh, vh, ki2, vi2)
        assert torch.equal(o1[:lo], o0[:lo]), f"chunk <= {j} changed"
        assert torch.equal(l1[:, :lo], l0[:, :lo])
        assert not torch.equal(o1[lo:], o0[lo:])


def test_constant_values_give_constant_output():
    """V = 1 everywhere: every output is exactly 1 (weights are normalised by their own sum)."""
    wf = RL.require_gpu()
    for cfg in (RoundConfig("ones_bf16", 2, 128, 300, 3, 2, "bf16", seed=33),
                RoundConfig("ones_f32", 2, 64, 70, 3, 1, "f32", seed=34)):
        q, kh, vh, ki, vi = _dev_inputs(cfg)
        out, _ = _run(wf, cfg, q, kh, torch.ones_like(vh), ki, torch.ones_like(vi))
        err = (out.float() - 1).abs().max().item()
        print(f"[parity] {cfg.name}: max |O - 1| = {err:.3e}", flush=True)
        assert err <= (0.0 if cfg.dtype == "bf16" else 1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_visible_key_returns_its_value(dtype):
    """Chunks of one token, no history: the refresh chunk's only key is itself, so O[0] = V[0] exactly."""
    wf = RL.require_gpu()
    cfg = RoundConfig("single", 2, 128, 1, 3, 0, dtype, seed=35)
    q, kh, vh, ki, vi = _dev_inputs(cfg)
    out, lse = _run(wf, cfg, q, kh, vh, ki, vi)
    if dtype == "bf16":  # the weight is rounded to bf16 (exactly 1) before P.V
        assert torch.equal(out[0], vi[0])
    else:  # the fp32 weight is exp2 of a rounding error, 1 within an ulp
        assert torch.allclose(out[0], vi[0], rtol=1e-6, atol=0)
    ref = (q[0].float() * ki[0].float()).sum(-1) * cfg.scale
    assert torch.allclose(lse[:, 0], ref, atol=1e-5)


def test_zero_queries_average_the_visible_values():
    """Q = 0: every weight is equal, O = mean of the visible values, LSE = ln(#keys)."""
    wf = RL.require_gpu()
    cfg = RoundConfig("qzero", 2, 128, 200, 3, 2, "bf16", seed=36)
    inp = make_round_inputs(cfg)
    inp.q[:] = 0
    out, lse, _ = RL.gpu_round(wf, inp)
    C, Hs = cfg.chunk_tokens, cfg.n_hist
    v = np.concatenate([inp.v_hist, inp.v_in]).astype(np.float64)
    got = out.float().cpu().numpy()
    for j in range(cfg.n_inflight):
        L = (Hs + j + 1) * C
        mean = v[:L].mean(axis=0)
        np.testing.assert_allclose(got[j * C:(j + 1) * C], np.broadcast_to(mean, (C,) + mean.shape),
                                   atol=2e-3, rtol=0)
        np.testing.assert_allclose(lse.cpu().numpy()[:, j * C:(j + 1) * C], np.log(L), atol=1e-4)


def test_run_to_run_deterministic():
    wf = RL.require_gpu()
    cfg = CONFIGS["wan13b_4step"]
    q, kh, vh, ki, vi = _dev_inputs(cfg)
    dt = torch.bfloat16
    cache = RL.build_cache(wf, cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, dt, kh, vh, ki, vi)
    a, la = wf.chunk_causal_attn_fwd(q, cache, cfg.n_inflight, cfg.scale)
    b, lb = wf.chunk_causal_attn_fwd(q, cache, cfg.n_inflight, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_argument_errors_raise():
    wf = RL.require_gpu()
    cfg = RoundConfig("err", 1, 128, 64, 2, 1, "bf16", seed=37)
    q, kh, vh, ki, vi = _dev_inputs(cfg)
    cache = RL.build_cache(wf, 64, 1, 128, torch.bfloat16, kh, vh, ki, vi)
    with pytest.raises(wf.WFError):
        wf.chunk_causal_attn_fwd(q[:0].reshape(0, 1, 128), cache, 0, cfg.scale)
    with pytest.raises(ValueError):
        wf.chunk_causal_attn_fwd(q, cache, 4, cfg.scale)  # shape check in the binding
    with pytest.raises(wf.WFError):
        wf.chunk_causal_attn_fwd(q, cache, 2, 0.0)
    big = torch.zeros(4 * 64, 1, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(wf.WFError):
        wf.chunk_causal_attn_fwd(big, cache, 4, cfg.scale)  # more in-flight chunks than entries
