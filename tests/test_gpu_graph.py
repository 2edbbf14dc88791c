"""One round captured in a HIP graph (torch.cuda.CUDAGraph over the library's
stream-ordered calls) and replayed.

The captured work is the in-flight chunks' cache refreshes and the allocation-free
key-split attention (wf_chunk_causal_attn_fwd_static): no call allocates, fills with
hipMemsetAsync or synchronizes. Between replays the test writes new Q, K and V into
the captured input buffers and runs the same round eagerly (with synchronizations in
between); every replay must equal that eager round bitwise, and the first one the
fp64 oracle at the bf16 bounds.
"""
import numpy as np
import pytest
import torch

import roundlib as RL
from workloads import RoundConfig, make_round_inputs

pytestmark = pytest.mark.gpu


def test_round_replays_from_a_hip_graph():
    wf = RL.require_gpu()
    cfg = RoundConfig("graph_round", 2, 128, 300, 3, 2, "bf16", seed=62)
    print(f"[case] {cfg.name}", flush=True)
    C, H, D, N, Hs = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, cfg.n_inflight, cfg.n_hist
    inp = make_round_inputs(cfg)
    dt = torch.bfloat16
    k_hist, v_hist = RL.to_dev(inp.k_hist, dt), RL.to_dev(inp.v_hist, dt)
    q, k_in, v_in = RL.to_dev(inp.q, dt), RL.to_dev(inp.k_in, dt), RL.to_dev(inp.v_in, dt)
    cache = wf.KVCache(Hs + N, C, H, D, dt)
    for c in range(Hs):
        cache.append(k_hist[c * C:(c + 1) * C], v_hist[c * C:(c + 1) * C])
    for c in range(N):
        cache.append(k_in[c * C:(c + 1) * C], v_in[c * C:(c + 1) * C])

    def round_once(out, lse):
        for c in range(N):
            cache.refresh(Hs + c, k_in[c * C:(c + 1) * C], v_in[c * C:(c + 1) * C])
        wf.chunk_causal_attn_fwd_static(q, cache, N, cfg.scale, out=out, lse=lse)

    out_e, out_g = torch.empty_like(q), torch.empty_like(q)
    lse_e = torch.empty((H, N * C), dtype=torch.float32, device="cuda")
    lse_g = torch.empty_like(lse_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture (first static call looks up the scratch)
        round_once(out_g, lse_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        round_once(out_g, lse_g)
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda")
    gen.manual_seed(63)
    for rep in range(4):
        if rep:  # new contents in the captured input buffers
            for t in (q, k_in, v_in):
                t.copy_(torch.randn(t.shape, generator=gen, device="cuda").to(dt))
        torch.cuda.synchronize()
        round_once(out_e, lse_e)
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e)
        print(f"[parity] graph replay {rep}: bitwise equal to the eager round: {same}", flush=True)
        assert same
        if rep == 0:
            ref_o, ref_l = RL.oracle_round(inp)
            RL.assert_close(out_g.float().cpu().numpy(), ref_o, "bf16", "graph replay O")
            assert np.abs(lse_g.cpu().numpy() - ref_l).max() <= 2e-3
