"""Benchmark of one Wave Forcing round's hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config wan13b_4step]

One step = one 1F1C round of one layer on synthetic inputs already resident
in HBM: append the new noisiest chunk to the history cache, refresh the
continuing in-flight chunks (the refresh chunk included) with this round's
K/V, run chunk-wise causal attention over the whole in-flight block, evict the
oldest history chunk (host-only). The workload is the Wan2.1-1.3B-shaped
4-step round: 12 heads x 128, chunks of 3 latent frames x 1560 tokens,
5 in-flight chunks (4 denoising + 1 cache refresh) over 2 history chunks.

Prints ONE JSON line. value = effective attention FLOPs per round / step time
(TFLOP/s); effective FLOPs = 4 * head_dim per visible (query, key) pair and
head (padding, skipped tiles and softmax not counted). Also reported: the
attention kernel alone against the bf16 MFMA peak (roofline), chunk-rounds/s,
and the fp64 oracle timed on the host on a bounded sample of the same round.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import CONFIGS, RoundConfig, make_round_inputs  # noqa: E402

MI355X_BF16_DENSE_TFLOPS = 2500.0  # published dense bf16 MFMA peak
MI355X_HBM_GBS = 8000.0
METRIC = "effective attention TFLOP/s per 1F1C round (% bf16 MFMA peak); chunk-rounds/s"
PROFILES = os.path.join(ROOT, "profiles")
ATTN_SRC = os.path.join(ROOT, "chunk_causal_dit_amd", "csrc", "attn_fwd.hip")


def effective_pairs_per_head(cfg: RoundConfig) -> int:
    """Visible (query, key) pairs per head: chunk j's C queries see (n_hist + j + 1) * C keys."""
    C = cfg.chunk_tokens
    return sum(C * (cfg.n_hist + j + 1) * C for j in range(cfg.n_inflight))


def effective_flops(cfg: RoundConfig) -> float:
    return 4.0 * cfg.head_dim * cfg.n_heads * effective_pairs_per_head(cfg)


def kv_write_bytes(cfg: RoundConfig) -> float:
    """HBM bytes of the round's cache writes: n_inflight chunks of K and V, read once, written once."""
    es = 2 if cfg.dtype == "bf16" else 4
    return 2.0 * 2.0 * cfg.n_inflight * cfg.chunk_tokens * cfg.n_heads * cfg.head_dim * es


def source_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(cfg_name: str):
    """HBM traffic per attention launch from the committed rocprofv3 --pmc summary, or None
    when there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"attn_fwd_{cfg_name}_pmc.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != source_hash(ATTN_SRC):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg: RoundConfig, inp, rows_per_chunk: int):
    """The fp64 oracle on a bounded sample of the round (every head, the first
    rows_per_chunk query rows of every in-flight chunk), in effective TFLOP/s."""
    import oracle.attention as OA
    from threadpoolctl import threadpool_limits

    cores = len(os.sched_getaffinity(0))
    C = cfg.chunk_tokens
    r = min(rows_per_chunk, C)
    rows = np.concatenate([j * C + np.arange(r) for j in range(cfg.n_inflight)])
    k = np.concatenate([inp.k_hist, inp.k_in])
    v = np.concatenate([inp.v_hist, inp.v_in])
    with threadpool_limits(1):
        t0 = time.perf_counter()
        OA.chunk_causal_attention(inp.q, k, v, cfg.n_hist, C, cfg.scale, rows=rows, workers=cores)
        dt = time.perf_counter() - t0
    flops = 4.0 * cfg.head_dim * cfg.n_heads * sum(r * (cfg.n_hist + j + 1) * C for j in range(cfg.n_inflight))
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{r} query rows of each of the {cfg.n_inflight} in-flight chunks x {cfg.n_heads} heads "
                  f"({flops / effective_flops(cfg):.1%} of the round's effective FLOPs), numpy fp64, "
                  f"thread pool over (head, chunk) tasks, BLAS 1 thread per task",
        "seconds": dt,
        "round_seconds_extrapolated": dt * effective_flops(cfg) / flops,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="wan13b_4step", choices=sorted(CONFIGS))
    ap.add_argument("--cpu-rows", type=int, default=4680, help="query rows per chunk in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import chunk_causal_dit_amd as wf

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    cfg = CONFIGS[args.config]
    if cfg.int8_qk or cfg.rope or cfg.dtype != "bf16":
        print("bench.py times the bf16 round without RoPE; pick wan13b_4step or step5_refresh", file=sys.stderr)
        sys.exit(2)
    C, H, D, N, Hs = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, cfg.n_inflight, cfg.n_hist
    dt = torch.bfloat16
    inp = make_round_inputs(cfg)

    def dev(a):
        return torch.from_numpy(a).to("cuda").to(dt)

    q, k_in, v_in = dev(inp.q), dev(inp.k_in), dev(inp.v_in)
    k_hist, v_hist = dev(inp.k_hist), dev(inp.v_hist)
    kc = [k_in[j * C:(j + 1) * C] for j in range(N)]
    vc = [v_in[j * C:(j + 1) * C] for j in range(N)]

    # Steady state between rounds: n_hist history chunks + the N-1 continuing in-flight chunks.
    cache = wf.KVCache(Hs + N, C, H, D, dt)
    for c in range(Hs):
        cache.append(k_hist[c * C:(c + 1) * C], v_hist[c * C:(c + 1) * C])
    for j in range(N - 1):
        cache.append(kc[j], vc[j])
    out = torch.empty_like(q)
    lse = torch.empty((H, N * C), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        cache.append(kc[N - 1], vc[N - 1])              # new noisiest chunk
        for j in range(N - 1):                          # this round's K/V of the continuing chunks
            cache.refresh(Hs + j, kc[j], vc[j])
        if ev is not None:
            ev[0].record(stream)
        wf.chunk_causal_attn_fwd(q, cache, N, cfg.scale, out=out, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        cache.evict(1)                                  # refresh chunk is history from now on

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = np.array([a.elapsed_time(b) for a, b in events])
    ms_per_step = wall * 1e3 / args.steps

    eff = effective_flops(cfg)
    attn_avg_s = float(attn_ms.mean()) / 1e3
    achieved = eff / attn_avg_s / 1e12
    traffic = load_traffic(cfg.name)
    res = {
        "metric": METRIC,
        "value": eff / (ms_per_step / 1e3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "heads": H, "head_dim": D, "chunk_tokens": C, "n_inflight": N, "n_hist": Hs,
            "query_tokens": N * C, "visible_keys_max": (Hs + N) * C,
            "effective_flops_per_round": eff,
            "step": "kv append (1 chunk) + kv refresh (N-1 chunks) + attention + evict",
        },
        "chunk_rounds_per_s": 1e3 / ms_per_step,
        "attention": {
            "ms_mean": float(attn_ms.mean()), "ms_median": float(np.median(attn_ms)),
            "ms_p10": float(np.percentile(attn_ms, 10)), "ms_p90": float(np.percentile(attn_ms, 90)),
            "tflops": achieved, "frac_of_bf16_peak": achieved / MI355X_BF16_DENSE_TFLOPS,
            "rounds_per_s": 1.0 / attn_avg_s,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_bf16_kernel<128,8>",
            "achieved": achieved,
            "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / MI355X_BF16_DENSE_TFLOPS,
            "traffic": traffic,
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_rows)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
