"""Long rollout: 20 consecutive rounds over a 6-chunk history window kept in
12 ring slots placed by a seeded permutation, with 3D RoPE on the in-flight
queries and keys, append of the new chunk, refresh of the continuing chunks,
attention and eviction each round. Attention runs twice a round: with the
key-split workspace (chunk 0's key range in two halves, then the merge) and
without it. Both are compared with the plain-list ring model of the oracle:
sampled rows every round, every row at rounds 0 and 19."""
import os

import numpy as np
import pytest
import torch

import oracle.attention as OA
import oracle.rope as OR
import roundlib as RL
from oracle.ring import RingModel
from workloads import CONFIGS, make_rollout_init, make_rollout_round, slot_permutation

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
def test_long_rollout_20_rounds():
    wf = RL.require_gpu()
    cfg = CONFIGS["long_rollout"]
    C, H, D, N, Hs = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, cfg.n_inflight, cfg.n_hist
    fpc, gh, gw, split = cfg.frames_per_chunk, cfg.grid_h, cfg.grid_w, cfg.rope_split
    dt = torch.bfloat16
    workers = min(16, len(os.sched_getaffinity(0)))

    # initial state: chunks 0..9 (6 history + 4 continuing in-flight), keys rotated at their positions
    k0, v0 = make_rollout_init(cfg)
    n0 = Hs + N - 1
    cache = wf.KVCache(cfg.slots, C, H, D, dt)
    ws = RL.split_workspace(wf, cache)
    assert ws is not None
    cache.set_table(slot_permutation(cfg.slots, seed=cfg.seed)[:n0])
    ring = RingModel()
    kd, vd = RL.to_dev(k0, dt), RL.to_dev(v0, dt)
    wf.rope3d(kd, 0, fpc, gh, gw, split)
    k_rot_host = OR.rope3d(k0, 0, C, fpc, gh, gw, split)
    for g in range(n0):
        cache.refresh(g, kd[g * C:(g + 1) * C], vd[g * C:(g + 1) * C])
        ring.append(k_rot_host[g * C:(g + 1) * C], v0[g * C:(g + 1) * C])

    for r in range(cfg.rounds):
        first = r + Hs  # global index of the refresh chunk this round
        q, k, v = make_rollout_round(cfg, r)
        qd, kd, vd = (RL.to_dev(a, dt) for a in (q, k, v))
        wf.rope3d(qd, first, fpc, gh, gw, split)
        wf.rope3d(kd, first, fpc, gh, gw, split)
        cache.append(kd[(N - 1) * C:], vd[(N - 1) * C:])
        for j in range(N - 1):
            cache.refresh(Hs + j, kd[j * C:(j + 1) * C], vd[j * C:(j + 1) * C])
        outs = {"split": wf.chunk_causal_attn_fwd(qd, cache, N, cfg.scale, workspace=ws),
                "whole": wf.chunk_causal_attn_fwd(qd, cache, N, cfg.scale)}
        torch.cuda.synchronize()
        table = cache.table()
        assert len(table) == Hs + N and len(set(table)) == Hs + N
        cache.evict(1)

        full = r in (0, cfg.rounds - 1)
        rows = None if full else RL.boundary_rows(C, N, 4, seed=500 + r)
        qr = OR.rope3d(q, first, C, fpc, gh, gw, split) if full else \
            OR.rope3d(q[rows], first, C, fpc, gh, gw, split, tokens=rows)
        kr = OR.rope3d(k, first, C, fpc, gh, gw, split)
        ring.append(kr[(N - 1) * C:], v[(N - 1) * C:])
        for j in range(N - 1):
            ring.refresh(Hs + j, kr[j * C:(j + 1) * C], v[j * C:(j + 1) * C])
        kvis, vvis = ring.visible()
        if full:
            ref_o, ref_l = OA.chunk_causal_attention(qr, kvis, vvis, Hs, C, cfg.scale, workers=workers)
        else:  # qr holds only the sampled rows: place them at their indices
            qfull = np.zeros((N * C, H, D))
            qfull[rows] = qr
            ref_o, ref_l = OA.chunk_causal_attention(qfull, kvis, vvis, Hs, C, cfg.scale, rows=rows, workers=workers)
        print(f"[case] rollout round {r} ({'all' if full else len(rows)} rows), table {table}", flush=True)
        for name, (out, lse) in outs.items():
            got = out.float().cpu().numpy() if full else out[torch.from_numpy(rows).cuda()].float().cpu().numpy()
            RL.assert_close(got, ref_o, "bf16", f"round {r} O ({name})", row_rel=RL.BF16_ROW_REL_ROPE)
            got_l = lse.cpu().numpy() if full else lse.cpu().numpy()[:, rows]
            assert np.abs(got_l - ref_l).max() <= 5e-3, name
        ring.evict(1)
