"""GPU tests of the history cache (append / refresh / evict / permuted tables)
through the C ABI: pool contents decoded with the documented tile-image layout
must equal the source chunks bit for bit, and attention must read the table."""
import numpy as np
import pytest
import torch

import roundlib as RL
from workloads import CONFIGS, RoundConfig, make_round_inputs, make_stale_refresh, slot_permutation

pytestmark = pytest.mark.gpu


def decode_slot(cache, pool: torch.Tensor, slot: int) -> np.ndarray:
    """[C][H][D] contents of one slot per the tile-image layout of include/wf.h."""
    H, D, C, S = cache.n_heads, cache.head_dim, cache.chunk_tokens, cache.s_pad
    E = 8 if cache.dtype == torch.bfloat16 else 4
    n_t = S // 64
    raw = pool.view(cache.dtype)[slot * H * S * D:(slot + 1) * H * S * D].float().cpu().numpy()
    return raw, H, D, C, S, E, n_t


def decode_k(cache, slot):
    raw, H, D, C, S, E, n_t = decode_slot(cache, cache.k_pool, slot)
    img = raw.reshape(H, n_t, D // E, 64, E).transpose(0, 1, 3, 2, 4).reshape(H, S, D)
    return img  # [H][S_pad][D]


def decode_v(cache, slot):
    raw, H, D, C, S, E, n_t = decode_slot(cache, cache.v_pool, slot)
    img = raw.reshape(H, n_t, 64 // E, D, E).transpose(0, 1, 2, 4, 3).reshape(H, S, D)
    return img  # [H][S_pad][D]


@pytest.mark.parametrize("dtype,C,D", [("bf16", 100, 128), ("bf16", 64, 64), ("f32", 130, 128), ("bf16", 4680, 128)])
def test_append_layout_bit_exact(dtype, C, D):
    wf = RL.require_gpu()
    H = 3
    dt = RL.torch_dtype(dtype)
    rng = np.random.default_rng(5)
    cache = wf.KVCache(4, C, H, D, dt)
    chunks = []
    for i in range(3):
        k = RL.to_dev(rng.standard_normal((C, H, D)).astype(np.float32), dt)
        v = RL.to_dev(rng.standard_normal((C, H, D)).astype(np.float32), dt)
        assert cache.append(k, v) == i
        chunks.append((k.float().cpu().numpy(), v.float().cpu().numpy()))
    torch.cuda.synchronize()
    assert cache.table() == [0, 1, 2]
    for i, (k, v) in enumerate(chunks):
        K, V = decode_k(cache, i), decode_v(cache, i)
        assert np.array_equal(K[:, :C, :], k.transpose(1, 0, 2))
        assert np.array_equal(V[:, :C, :], v.transpose(1, 0, 2))
        assert not K[:, C:, :].any() and not V[:, C:, :].any()  # padding stays zero
    # the unused slot is zero
    assert not decode_k(cache, 3).any() and not decode_v(cache, 3).any()


def test_refresh_evict_and_slot_reuse():
    wf = RL.require_gpu()
    C, H, D = 70, 2, 128
    dt = torch.bfloat16
    rng = np.random.default_rng(6)
    mk = lambda: RL.to_dev(rng.standard_normal((C, H, D)).astype(np.float32), dt)
    cache = wf.KVCache(3, C, H, D, dt)
    a = [mk() for _ in range(6)]
    assert [cache.append(a[0], a[1]), cache.append(a[2], a[3]), cache.append(a[4], a[5])] == [0, 1, 2]
    with pytest.raises(wf.WFError):
        cache.append(a[0], a[1])  # full
    knew, vnew = mk(), mk()
    cache.refresh(1, knew, vnew)
    torch.cuda.synchronize()
    assert np.array_equal(decode_k(cache, 1)[:, :C], knew.float().cpu().numpy().transpose(1, 0, 2))
    assert np.array_equal(decode_v(cache, 1)[:, :C], vnew.float().cpu().numpy().transpose(1, 0, 2))
    cache.evict(2)
    assert cache.table() == [2]
    assert cache.append(a[0], a[1]) == 0  # freed slots come back oldest first
    assert cache.append(a[2], a[3]) == 1
    assert cache.table() == [2, 0, 1]


def test_permuted_slots_bitwise_equal_to_contiguous():
    wf = RL.require_gpu()
    cfg = RoundConfig("perm", 2, 128, 300, 3, 3, "bf16", seed=21)
    inp = make_round_inputs(cfg)
    o1, l1, _ = RL.gpu_round(wf, inp)
    perm = slot_permutation(9, seed=77)[:6]
    o2, l2, c2 = RL.gpu_round(wf, inp, table=perm, n_slots=9)
    assert c2.table() == perm
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_step5_round_refresh_overwrites_stale_slot():
    """5-step round: the refresh chunk's slot first holds stale K/V (x8); the
    refresh writes this round's values before attention, which must use them."""
    wf = RL.require_gpu()
    cfg = CONFIGS["step5_refresh"]
    print(f"[case] {cfg.name}", flush=True)
    inp = make_round_inputs(cfg)
    stale_k, stale_v = make_stale_refresh(cfg)
    dt = torch.bfloat16
    C, H, D, N, Hs = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, cfg.n_inflight, cfg.n_hist
    dev = lambda a: RL.to_dev(a, dt)
    q, kh, vh, ki, vi = (dev(a) for a in (inp.q, inp.k_hist, inp.v_hist, inp.k_in, inp.v_in))
    cache = wf.KVCache(Hs + N, C, H, D, dt)
    for c in range(Hs):
        cache.append(kh[c * C:(c + 1) * C], vh[c * C:(c + 1) * C])
    cache.append(dev(stale_k), dev(stale_v))  # refresh chunk, stale
    for j in range(1, N):
        cache.append(ki[j * C:(j + 1) * C], vi[j * C:(j + 1) * C])
    cache.refresh(Hs, ki[:C], vi[:C])  # this round's K/V of the refresh chunk
    outs = {"whole": wf.chunk_causal_attn_fwd(q, cache, N, cfg.scale),
            "split": wf.chunk_causal_attn_fwd(q, cache, N, cfg.scale, workspace=RL.split_workspace(wf, cache))}
    torch.cuda.synchronize()
    ref_o, ref_l = RL.oracle_round(inp)  # every row of the round
    for name, (out, lse) in outs.items():
        got = out.float().cpu().numpy()
        RL.assert_close(got, ref_o, "bf16", f"O (all {got.shape[0]} rows, {name})")
        assert np.abs(lse.cpu().numpy() - ref_l).max() <= 2e-3, name
