"""Multi-round 1F1C rollouts through the native planner and round runner
(wf_1f1c_plan / wf_1f1c_run_round), every round against the schedule oracle
(oracle/schedule.py) with the same seeded null model: pipeline fill, steady
state, drain, 4-, 5- and 1-step layouts, a window wider than the history."""
import numpy as np
import pytest
import torch

import roundlib as RL
from oracle import schedule as SC
from workloads import NullModel

pytestmark = pytest.mark.gpu


class DeviceModel:
    """The null model's arrays on the device, one upload per (chunk, stage)."""

    def __init__(self, host: NullModel, n_steps: int, dtype):
        self.host, self.n_steps, self.dtype, self.dev = host, n_steps, dtype, {}

    def qkv(self, c, s):
        if (c, s) not in self.dev:
            self.dev[(c, s)] = tuple(RL.to_dev(a, self.dtype) for a in self.host(c, s))
        return self.dev[(c, s)]

    def __call__(self, plan):
        parts = [self.qkv(c, s) for c, s in plan.inflight]
        return torch.cat([p[0] for p in parts]), [p[1] for p in parts], [p[2] for p in parts]


def run_rollout(wf, S, F, W, C, H, D, dtype, seed, rows=None, check_rounds=None, rope=None):
    host = NullModel(seed, C, H, D, dtype)
    tdt = RL.torch_dtype(dtype)
    model = DeviceModel(host, S, tdt)
    scale = 1.0 / np.sqrt(D)
    ro = wf.Rollout1F1C(S, F, W, C, H, D, scale, tdt, rope=rope)
    got, outputs = {}, []
    for _ in range(ro.n_rounds):
        plan, out, lse = ro.step(model, with_lse=True)
        if plan.output is not None:
            outputs.append(plan.output)
        if check_rounds is None or plan.round in check_rounds:
            sel = None if rows is None else torch.from_numpy(rows(plan.round)).cuda()
            o = out if sel is None else out[sel]
            l = lse if sel is None else lse[:, sel]
            got[plan.round] = (o.float().cpu().numpy(), l.cpu().numpy(), plan.inflight, plan.hist)
    torch.cuda.synchronize()
    ref = SC.rollout_attention(S, F, W, host, scale, rounds=sorted(got), rows=rows, workers=RL.oracle_workers(),
                               rope=rope)
    for r, (o, l, inflight, hist) in got.items():
        ro_, rl_, plan = ref[r]
        assert inflight == plan["inflight"] and hist == plan["hist"]
        RL.assert_close(o, ro_, dtype, f"round {r} ({len(inflight)} in flight, {len(hist)} history)",
                        row_rel=RL.BF16_ROW_REL if rope is None else RL.BF16_ROW_REL_ROPE)
        assert np.abs(l - rl_).max() <= (1e-4 if dtype == "f32" else 2e-3)
    assert outputs == list(range(F))  # one output per round after the fill, in order
    return got


@pytest.mark.parametrize("S,F,W,C,dtype", [(4, 7, 2, 96, "bf16"), (5, 8, 3, 100, "bf16"),
                                           (1, 5, 1, 64, "f32"), (2, 5, 3, 33, "f32")])
def test_rollout_every_round_matches_oracle(S, F, W, C, dtype):
    wf = RL.require_gpu()
    print(f"[case] rollout S={S} F={F} W={W} C={C} {dtype}", flush=True)
    run_rollout(wf, S, F, W, C, 2, 128 if dtype == "bf16" else 64, dtype, seed=70 + S)


def test_rollout_is_deterministic():
    wf = RL.require_gpu()
    a = run_rollout(wf, 4, 6, 2, 80, 2, 128, "bf16", seed=77)
    b = run_rollout(wf, 4, 6, 2, 80, 2, 128, "bf16", seed=77)
    for r in a:
        assert np.array_equal(a[r][0], b[r][0]) and np.array_equal(a[r][1], b[r][1])


def test_wan13b_4step_rollout_sampled():
    """1.3B shapes (12 heads x 128, 4680-token chunks), 4 steps, 6 chunks, window 2:
    9 rounds; fill, steady and drain rounds checked on sampled rows."""
    wf = RL.require_gpu()
    C = 4680

    def rows(r):
        n = len(SC.round_plan(4, 6, 2, r)["inflight"])
        return RL.boundary_rows(C, n, 4, seed=r)

    run_rollout(wf, 4, 6, 2, C, 12, 128, "bf16", seed=91, rows=rows, check_rounds={0, 3, 4, 5, 8})


@pytest.mark.parametrize("S,F,W,dtype,D", [(4, 6, 2, "bf16", 128), (5, 7, 3, "f32", 64)])
def test_rollout_with_rope_every_round(S, F, W, dtype, D):
    """3D RoPE through the runner: the query block rotated in place, K inside the cache
    writes, at the chunks' global indices (3 frames of 4 x 8 latent tokens per chunk)."""
    wf = RL.require_gpu()
    print(f"[case] rope rollout S={S} F={F} W={W} {dtype} D={D}", flush=True)
    split = (44, 42, 42) if D == 128 else (22, 22, 20)
    rope = {"frames_per_chunk": 3, "grid_h": 4, "grid_w": 8, "split": split, "theta": 10000.0}
    run_rollout(wf, S, F, W, 96, 2, D, dtype, seed=80 + S, rope=rope)
