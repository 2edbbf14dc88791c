"""GPU parity of the int8-QK variant through the C ABI.

Three levels, each against the fp64 oracle on the same seeded inputs:
  * the quantization itself (key mean, block scales, int8 codes, read back from
    the documented workspace layout) is bit-exact against oracle.quant, whose
    integer decisions are taken in fp32 as the kernels take them;
  * O and LSE match the exact attention on the dequantized operands
    (oracle.quant.quantized_attention) to the bf16 bounds;
  * O stays close to the unquantized attention (mean rel <= 3e-2, cosine >= 0.999).
"""
import numpy as np
import pytest
import torch

import roundlib as RL
from oracle import quant as OQ
from workloads import CONFIGS, RoundConfig, make_round_inputs, round_to_bf16, slot_permutation

pytestmark = pytest.mark.gpu

I8_MEAN_REL_EXACT = 3e-2
I8_COSINE = 0.999
LSE_ATOL = 2e-3


def workspace_layout(n_tab, H, D, C, s_pad, N):
    """Byte offsets of the workspace arrays, in the order and alignment include/wf.h documents."""
    a = lambda x: (x + 255) // 256 * 256
    nb = -(-C // 128)
    n_mean = n_tab - N + 1  # the key mean covers the history and in-flight chunk 0
    L, off = {}, 0
    for name, size in (("partial", n_mean * 4 * H * D * 8), ("mean", H * D * 4), ("k_codes", n_tab * H * s_pad * D),
                       ("k_scales", n_tab * H * nb * 4), ("q_codes", N * C * H * D),
                       ("q_scales", H * N * nb * 4), ("qm", H * N * C * 4)):
        L[name] = (off, size)
        off = a(off + size)
    L["total"] = off
    return L, nb


def read_workspace(ws: torch.Tensor, cache, N):
    H, D, C, S = cache.n_heads, cache.head_dim, cache.chunk_tokens, cache.s_pad
    n_tab = len(cache.table())
    L, nb = workspace_layout(n_tab, H, D, C, S, N)
    raw = ws.cpu().numpy()
    get = lambda name, dt: raw[L[name][0]:L[name][0] + L[name][1]].view(dt)
    tiles = S // 64
    # K code tiles: [n_tab][H][tiles][D/16 pieces][64 keys][16 dims] -> [n_tab][H][S_pad][D]
    kc = get("k_codes", np.int8).reshape(n_tab, H, tiles, D // 16, 64, 16)
    kc = kc.transpose(0, 1, 2, 4, 3, 5).reshape(n_tab, H, S, D)
    return {
        "total": L["total"],
        "mean": get("mean", np.float32).reshape(H, D),
        "k_codes": np.ascontiguousarray(kc[:, :, :C].transpose(0, 2, 1, 3)).reshape(n_tab * C, H, D),
        "k_padded": kc,
        "k_scales": get("k_scales", np.float32).reshape(H, n_tab * nb),
        "q_codes": get("q_codes", np.int8).reshape(N * C, H, D),
        "q_scales": get("q_scales", np.float32).reshape(H, N * nb),
        "qm": get("qm", np.float32).reshape(H, N * C),
    }


def run_i8(wf, inp, table=None, n_slots=None):
    cfg = inp.cfg
    dt = torch.bfloat16
    C, H, D = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim
    dev = {k: RL.to_dev(getattr(inp, k), dt) for k in ("q", "k_hist", "v_hist", "k_in", "v_in")}
    cache = RL.build_cache(wf, C, H, D, dt, dev["k_hist"], dev["v_hist"], dev["k_in"], dev["v_in"],
                           n_slots=n_slots, table=table)
    nbytes = wf.attn_i8qk_workspace_bytes(cache, cfg.n_inflight)
    ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")  # garbage: every byte read is written first
    out, lse = wf.chunk_causal_attn_fwd_i8qk(dev["q"], cache, cfg.n_inflight, cfg.scale, workspace=ws)
    torch.cuda.synchronize()
    return out, lse, cache, ws


def visible_keys(inp):
    return np.concatenate([inp.k_hist, inp.k_in]), np.concatenate([inp.v_hist, inp.v_in])


def check_quantization(inp, cache, ws):
    cfg = inp.cfg
    k_vis, _ = visible_keys(inp)
    ref = OQ.quantize_round(inp.q, k_vis, cfg.n_hist, cfg.chunk_tokens)
    got = read_workspace(ws, cache, cfg.n_inflight)
    assert got["total"] == ws.numel(), "workspace layout differs from the documented one"
    assert np.array_equal(got["mean"], ref["mean"]), "key mean"
    assert np.array_equal(got["k_scales"], ref["k_scales"]), "K block scales"
    assert np.array_equal(got["q_scales"], ref["q_scales"]), "Q block scales"
    assert np.array_equal(got["k_codes"], ref["k_codes"]), "K codes"
    assert np.array_equal(got["q_codes"], ref["q_codes"]), "Q codes"
    # codes of the zero padding past each chunk end are 0
    C = cfg.chunk_tokens
    assert not got["k_padded"][:, :, C:].any()
    # <q^, mean> per query row, against the fp64 dot of the dequantized codes
    q_hat = OQ.dequantize(ref["q_codes"], ref["q_scales"], C)
    qm_ref = np.einsum("nhd,hd->hn", q_hat, ref["mean"].astype(np.float64))
    np.testing.assert_allclose(got["qm"], qm_ref, rtol=0, atol=1e-4 * max(1.0, np.abs(qm_ref).max()))
    print(f"[parity] {cfg.name}: mean, scales and codes bit-exact", flush=True)
    return ref


def check_outputs(inp, out, lse, ref_quant, rows=None):
    cfg = inp.cfg
    k_vis, v_vis = visible_keys(inp)
    o_q, l_q = OQ.quantized_attention(inp.q, k_vis, v_vis, cfg.n_hist, cfg.chunk_tokens, cfg.scale, rows=rows,
                                      workers=RL.oracle_workers(), quant=ref_quant)
    o_x, _ = RL.oracle_round(inp, rows=rows)
    sel = torch.arange(out.shape[0], device="cuda") if rows is None else torch.from_numpy(rows).cuda()
    got = out[sel].float().cpu().numpy()
    got_l = lse[:, sel].cpu().numpy()
    RL.assert_close(got, o_q, "bf16", f"{cfg.name} O vs quantized oracle")
    dl = np.abs(got_l - l_q).max()
    print(f"[parity] {cfg.name} LSE vs quantized oracle: max abs {dl:.3e}", flush=True)
    assert dl <= LSE_ATOL
    mx, rel = RL.error_stats(got, o_x)
    g64 = got.astype(np.float64)
    cos = float((g64 * o_x).sum() / np.linalg.norm(g64) / np.linalg.norm(o_x))
    print(f"[parity] {cfg.name} O vs exact oracle: max abs {mx:.3e}, mean rel {rel:.3e}, cosine {cos:.6f}",
          flush=True)
    assert rel <= I8_MEAN_REL_EXACT and cos >= I8_COSINE


SMALL = [
    RoundConfig("i8_ragged", 2, 128, 300, 3, 2, "bf16", seed=51, int8_qk=True),
    RoundConfig("i8_c64", 3, 128, 64, 4, 1, "bf16", seed=52, int8_qk=True),
    RoundConfig("i8_c200_nohist", 2, 128, 200, 2, 0, "bf16", seed=53, int8_qk=True),
    RoundConfig("i8_c1", 1, 128, 1, 3, 2, "bf16", seed=54, int8_qk=True),
    RoundConfig("i8_c4680_h1", 1, 128, 4680, 2, 1, "bf16", seed=55, int8_qk=True),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_i8_small_full_parity(cfg):
    wf = RL.require_gpu()
    print(f"[case] {cfg.name}", flush=True)
    inp = make_round_inputs(cfg)
    out, lse, cache, ws = run_i8(wf, inp)
    ref = check_quantization(inp, cache, ws)
    check_outputs(inp, out, lse, ref)


def test_i8_14b_round_all_rows():
    """The 14B-shaped round (40 heads, 4680-token chunks, 5 in flight, 2 history):
    quantization bit-exact in full, attention on every one of its 23,400 query rows
    and 40 heads."""
    wf = RL.require_gpu()
    cfg = CONFIGS["i8qk_14b"]
    print(f"[case] {cfg.name}", flush=True)
    inp = make_round_inputs(cfg)
    out, lse, cache, ws = run_i8(wf, inp)
    ref = check_quantization(inp, cache, ws)
    check_outputs(inp, out, lse, ref)


def test_i8_block_scales_spread():
    """K blocks scaled by factors from 1/1000 to 60 (Q blocks by 1/8 to 2), so the
    log2-domain factors of a row's tiles span about 2^11: the power-of-two grid the
    kernel keeps its reference max on coarsens several times inside a row, and the
    exact-max path runs often. Quantization bit-exact; O and LSE against the
    quantized oracle at the bf16 bounds (no comparison with unquantized attention:
    a key mean dominated by the large blocks leaves the small ones few levels)."""
    wf = RL.require_gpu()
    cfg = RoundConfig("i8_spread", 2, 128, 300, 3, 3, "bf16", seed=60, int8_qk=True)
    print(f"[case] {cfg.name}", flush=True)
    inp = make_round_inputs(cfg)
    C, nb = cfg.chunk_tokens, -(-cfg.chunk_tokens // 128)
    kf = [1.0, 1e-3, 20.0, 1.0 / 16, 60.0, 0.5, 7.0]
    qf = [1.0, 0.125, 2.0]

    def scale_blocks(x, factors, n_chunks, salt):
        for c in range(n_chunks):
            for b in range(nb):
                rows = slice(c * C + b * 128, min(c * C + (b + 1) * 128, (c + 1) * C))
                x[rows] = round_to_bf16(x[rows] * np.float32(factors[(c * nb + b + salt) % len(factors)]))

    scale_blocks(inp.k_hist, kf, cfg.n_hist, 0)
    scale_blocks(inp.k_in, kf, cfg.n_inflight, 3)
    scale_blocks(inp.q, qf, cfg.n_inflight, 0)
    out, lse, cache, ws = run_i8(wf, inp)
    ref = check_quantization(inp, cache, ws)
    k_vis, v_vis = visible_keys(inp)
    o_q, l_q = OQ.quantized_attention(inp.q, k_vis, v_vis, cfg.n_hist, C, cfg.scale,
                                      workers=RL.oracle_workers(), quant=ref)
    RL.assert_close(out.float().cpu().numpy(), o_q, "bf16", f"{cfg.name} O vs quantized oracle")
    dl = np.abs(lse.cpu().numpy() - l_q).max()
    print(f"[parity] {cfg.name} LSE vs quantized oracle: max abs {dl:.3e} (|LSE| up to {np.abs(l_q).max():.1f})",
          flush=True)
    assert dl <= LSE_ATOL


def test_i8_permuted_slots_bitwise():
    wf = RL.require_gpu()
    cfg = RoundConfig("i8_perm", 2, 128, 300, 3, 3, "bf16", seed=56, int8_qk=True)
    inp = make_round_inputs(cfg)
    o1, l1, _, _ = run_i8(wf, inp)
    perm = slot_permutation(9, seed=78)[:6]
    o2, l2, c2, _ = run_i8(wf, inp, table=perm, n_slots=9)
    assert c2.table() == perm
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_i8_constant_keys_average_values():
    """K constant per (head, channel): K - mean = 0 gives all-zero codes, every
    weight is equal, O is the mean of the visible values, and
    LSE = ln(#keys) + scale * <q^, k>."""
    wf = RL.require_gpu()
    cfg = RoundConfig("i8_constk", 2, 128, 200, 3, 2, "bf16", seed=57, int8_qk=True)
    inp = make_round_inputs(cfg)
    krow = inp.k_hist[:1].copy()
    inp.k_hist[:] = krow
    inp.k_in[:] = krow
    out, lse, cache, ws = run_i8(wf, inp)
    ref = check_quantization(inp, cache, ws)
    assert not ref["k_codes"].any()
    C, Hs = cfg.chunk_tokens, cfg.n_hist
    v = np.concatenate([inp.v_hist, inp.v_in]).astype(np.float64)
    got = out.float().cpu().numpy()
    q_hat = OQ.dequantize(ref["q_codes"], ref["q_scales"], C)
    for j in range(cfg.n_inflight):
        L = (Hs + j + 1) * C
        np.testing.assert_allclose(got[j * C:(j + 1) * C], np.broadcast_to(v[:L].mean(0), (C,) + v.shape[1:]),
                                   atol=2e-3, rtol=0)
        want = np.log(L) + cfg.scale * np.einsum("nhd,hd->hn", q_hat[j * C:(j + 1) * C],
                                                  krow[0].astype(np.float64))
        np.testing.assert_allclose(lse.cpu().numpy()[:, j * C:(j + 1) * C], want, atol=1e-3, rtol=0)


@pytest.mark.parametrize("j", [0, 1, 2])
def test_i8_later_chunks_do_not_change_earlier_outputs(j):
    """Q, K and V of every in-flight chunk after chunk j perturbed: the key mean
    covers only history and in-flight chunk 0, so chunks 0..j keep bitwise equal
    codes, O and LSE, while the perturbed chunks' outputs change."""
    wf = RL.require_gpu()
    cfg = RoundConfig("i8_caus", 2, 128, 300, 4, 2, "bf16", seed=58, int8_qk=True)
    inp = make_round_inputs(cfg)
    o0, l0, c0, w0 = run_i8(wf, inp)
    g0 = read_workspace(w0, c0, cfg.n_inflight)
    C = cfg.chunk_tokens
    lo = (j + 1) * C
    rng = np.random.default_rng(7 + j)
    draw = lambda a: round_to_bf16(rng.standard_normal(a.shape).astype(np.float32) * 3)
    inp.q[lo:] = draw(inp.q[lo:])
    inp.k_in[lo:] = draw(inp.k_in[lo:])
    inp.v_in[lo:] = draw(inp.v_in[lo:])
    o1, l1, c1, w1 = run_i8(wf, inp)
    g1 = read_workspace(w1, c1, cfg.n_inflight)
    assert np.array_equal(g1["mean"], g0["mean"])
    nk = (cfg.n_hist + j + 1) * C
    assert np.array_equal(g1["k_codes"][:nk], g0["k_codes"][:nk])
    assert torch.equal(o1[:lo], o0[:lo]) and torch.equal(l1[:, :lo], l0[:, :lo])
    assert not torch.equal(o1[lo:], o0[lo:])


def test_i8_run_to_run_deterministic():
    wf = RL.require_gpu()
    cfg = RoundConfig("i8_det", 4, 128, 1000, 3, 2, "bf16", seed=59, int8_qk=True)
    inp = make_round_inputs(cfg)
    a, la, cache, ws = run_i8(wf, inp)
    dev_q = RL.to_dev(inp.q, torch.bfloat16)
    b, lb = wf.chunk_causal_attn_fwd_i8qk(dev_q, cache, cfg.n_inflight, cfg.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_i8_argument_errors():
    wf = RL.require_gpu()
    C, H = 64, 1
    q = torch.zeros(2 * C, H, 128, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(C, H, 128, dtype=torch.bfloat16, device="cuda")
    cache = wf.KVCache(3, C, H, 128, torch.bfloat16)
    for _ in range(3):
        cache.append(kv, kv)
    with pytest.raises(wf.WFError):  # NULL workspace
        st = wf.lib().wf_chunk_causal_attn_fwd_i8qk(q.data_ptr(), cache.handle, 2, 0.1, None, q.data_ptr(), None,
                                                    None)
        wf._check(st, "wf_chunk_causal_attn_fwd_i8qk")
    ws = torch.empty(wf.attn_i8qk_workspace_bytes(cache, 2), dtype=torch.uint8, device="cuda")
    with pytest.raises(wf.WFError):
        wf.chunk_causal_attn_fwd_i8qk(q, cache, 2, -1.0, workspace=ws)
    f32 = wf.KVCache(3, C, H, 128, torch.float32)
    assert wf.attn_i8qk_workspace_bytes(f32, 1) == 0
    k32 = torch.zeros(C, H, 128, dtype=torch.float32, device="cuda")
    f32.append(k32, k32)
    with pytest.raises(wf.WFError):
        wf.chunk_causal_attn_fwd_i8qk(torch.zeros(C, H, 128, device="cuda"), f32, 1, 0.1, workspace=ws)
    d64 = wf.KVCache(2, C, H, 64, torch.bfloat16)
    k64 = torch.zeros(C, H, 64, dtype=torch.bfloat16, device="cuda")
    d64.append(k64, k64)
    with pytest.raises(wf.WFError):
        wf.chunk_causal_attn_fwd_i8qk(torch.zeros(C, H, 64, dtype=torch.bfloat16, device="cuda"), d64, 1, 0.1,
                                      workspace=ws)
