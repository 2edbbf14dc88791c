"""wf_rope3d on the GPU against the fp64 oracle rotation (long-rollout grid:
3 latent frames of 30x52, head_dim 128 split 44/42/42)."""
import numpy as np
import pytest
import torch

import oracle.rope as OR
import roundlib as RL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope3d_matches_oracle(dtype):
    wf = RL.require_gpu()
    C, H, D = 4680, 4, 128
    rng = np.random.default_rng(41)
    x = rng.standard_normal((2 * C, H, D)).astype(np.float32)
    dt = RL.torch_dtype(dtype)
    xd = RL.to_dev(x, dt)
    x_in = xd.float().cpu().numpy()  # exactly the values the kernel reads
    wf.rope3d(xd, first_global_chunk=5, frames_per_chunk=3, grid_h=30, grid_w=52, split=(44, 42, 42))
    torch.cuda.synchronize()
    ref = OR.rope3d(x_in, 5, C, 3, 30, 52, split=(44, 42, 42))
    got = xd.float().cpu().numpy()
    err = np.abs(got - ref)
    print(f"[parity] rope3d {dtype}: max abs {err.max():.3e}", flush=True)
    if dtype == "f32":
        assert err.max() <= 1e-4
    else:  # bf16 output: half an ulp of the result plus fp32 angle error
        assert (err <= np.abs(ref) * 2.0 ** -8 + 1e-4).all()


def test_rope3d_zero_position_is_identity_and_heads_share_angles():
    wf = RL.require_gpu()
    C, H, D = 60, 3, 64
    x = np.tile(np.random.default_rng(42).standard_normal((C, 1, D)).astype(np.float32), (1, H, 1))
    xd = RL.to_dev(x, torch.float32)
    wf.rope3d(xd, 0, 1, 6, 10, split=(20, 22, 22))
    torch.cuda.synchronize()
    got = xd.cpu().numpy()
    assert np.array_equal(got[0], x[0])  # frame 0, row 0, col 0
    assert np.array_equal(got[:, 0], got[:, 2])  # same token position in every head
