"""GPU tests of the fused producer (RoPE applied to K inside the cache write):
its slot contents must equal, bit for bit, wf_rope3d on a copy of K followed by
the plain write, for append and refresh, bf16 and fp32, ragged chunks and both
head dims; and a few rollout rounds through the fused path must give bitwise
the attention output of the unfused path."""
import numpy as np
import pytest
import torch

import roundlib as RL
from workloads import slot_permutation

pytestmark = pytest.mark.gpu

GEOMS = [  # (frames_per_chunk, grid_h, grid_w, head_dim, split, heads)
    (3, 30, 52, 128, (44, 42, 42), 12),  # the 832x480 latent grid: 4680 tokens per chunk, 12 heads
    (3, 4, 5, 128, (44, 42, 42), 3),     # 60 tokens: ragged against every slice and tile size
    (2, 3, 7, 64, (22, 22, 20), 5),      # 42 tokens, head_dim 64; heads not a multiple of the head group
]


def _inputs(C, H, D, dt, seed):
    rng = np.random.default_rng(seed)
    k = RL.to_dev(rng.standard_normal((C, H, D)).astype(np.float32), dt)
    v = RL.to_dev(rng.standard_normal((C, H, D)).astype(np.float32), dt)
    return k, v


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: f"{g[0]}x{g[1]}x{g[2]}_d{g[3]}_h{g[5]}")
def test_append_and_refresh_rope_equal_rope_then_write(dtype, geom):
    wf = RL.require_gpu()
    fpc, gh, gw, D, split, H = geom
    C = fpc * gh * gw
    dt = RL.torch_dtype(dtype)
    print(f"[case] fused write {dtype} C={C} H={H} D={D}", flush=True)
    fused = wf.KVCache(4, C, H, D, dt)
    plain = wf.KVCache(4, C, H, D, dt)
    fused.set_rope(fpc, gh, gw, split)
    for i, g in enumerate((0, 7, 123)):
        k, v = _inputs(C, H, D, dt, seed=10 + i)
        k0 = k.clone()
        assert fused.append_rope(k, v, g) == i
        torch.cuda.synchronize()
        assert torch.equal(k, k0), "append_rope modified its source"
        kr = k.clone()
        wf.rope3d(kr, g, fpc, gh, gw, split)
        assert plain.append(kr, v) == i
    # refresh the middle entry at another chunk index
    k, v = _inputs(C, H, D, dt, seed=20)
    fused.refresh_rope(1, k, v, 41)
    kr = k.clone()
    wf.rope3d(kr, 41, fpc, gh, gw, split)
    plain.refresh(1, kr, v)
    torch.cuda.synchronize()
    assert torch.equal(fused.k_pool, plain.k_pool), "K slots differ"
    assert torch.equal(fused.v_pool, plain.v_pool), "V slots differ"
    # the rotated K really differs from the unrotated one (the rotation ran)
    raw = wf.KVCache(4, C, H, D, dt)
    raw.append(*_inputs(C, H, D, dt, seed=10))
    torch.cuda.synchronize()
    assert not torch.equal(raw.k_slot(0), fused.k_slot(0))
    assert torch.equal(raw.v_slot(0), fused.v_slot(0))


def test_rollout_rounds_fused_equal_unfused():
    """Three rollout rounds (permuted 8-slot ring, 2 history chunks, 3 in flight):
    attention after the fused producer equals attention after rope3d + write, bitwise."""
    wf = RL.require_gpu()
    fpc, gh, gw, D, split = 3, 10, 12, 128, (44, 42, 42)
    C, H, N, Hs = fpc * gh * gw, 2, 3, 2
    dt = torch.bfloat16
    scale = D ** -0.5
    rng = np.random.default_rng(71)
    dev = lambda shape: RL.to_dev(rng.standard_normal(shape).astype(np.float32), dt)
    caches = [wf.KVCache(8, C, H, D, dt) for _ in range(2)]
    perm = slot_permutation(8, seed=72)[:Hs + N - 1]
    caches[0].set_rope(fpc, gh, gw, split)
    k0, v0 = dev(((Hs + N - 1) * C, H, D)), dev(((Hs + N - 1) * C, H, D))
    for c in caches:
        c.set_table(perm)
    for i in range(Hs + N - 1):
        kc, vc = k0[i * C:(i + 1) * C], v0[i * C:(i + 1) * C]
        caches[0].refresh_rope(i, kc, vc, i)
        kr = kc.clone()
        wf.rope3d(kr, i, fpc, gh, gw, split)
        caches[1].refresh(i, kr, vc)
    for r in range(3):
        first = r + Hs
        q, k, v = dev((N * C, H, D)), dev((N * C, H, D)), dev((N * C, H, D))
        wf.rope3d(q, first, fpc, gh, gw, split)
        outs = []
        # fused: K rotated inside the writes
        c = caches[0]
        c.append_rope(k[(N - 1) * C:], v[(N - 1) * C:], first + N - 1)
        for j in range(N - 1):
            c.refresh_rope(Hs + j, k[j * C:(j + 1) * C], v[j * C:(j + 1) * C], first + j)
        outs.append(wf.chunk_causal_attn_fwd(q, c, N, scale))
        c.evict(1)
        # unfused: rope3d on K, then the plain writes
        c = caches[1]
        kr = k.clone()
        wf.rope3d(kr, first, fpc, gh, gw, split)
        c.append(kr[(N - 1) * C:], v[(N - 1) * C:])
        for j in range(N - 1):
            c.refresh(Hs + j, kr[j * C:(j + 1) * C], v[j * C:(j + 1) * C])
        outs.append(wf.chunk_causal_attn_fwd(q, c, N, scale))
        c.evict(1)
        torch.cuda.synchronize()
        print(f"[case] rollout round {r}: tables {caches[0].table()} {caches[1].table()}", flush=True)
        assert caches[0].table() == caches[1].table()
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
