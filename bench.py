"""Benchmark of one Wave Forcing round's hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu-baseline]

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
attention kernel alone against the bf16 MFMA peak (roofline, timed with
events on the stream it runs on), chunk-rounds/s, the cache writes against
HBM bandwidth and, unless --no-extras, the long-rollout round with 3D RoPE,
the 14B-shaped int8-QK round, the W8A8 linears around attention (QKV and
O projections of the round's tokens), library GEMMs in bf16 and int8 at the
board's power cap and a plain device copy (what a dense contraction and a
streaming kernel reach here, beside the fractions of the published peaks) and
whole 1F1C rollouts
(4 and 5 steps, 133 chunks = 399 latent frames: fill, steady state, drain);
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

from workloads import CONFIGS, RoundConfig, make_rollout_init, make_rollout_round, make_round_inputs  # noqa: E402

# Published MI355X peaks.
BF16_DENSE_TFLOPS = 2500.0
INT8_DENSE_TOPS = 5000.0
HBM_GBS = 8000.0
# int8-QK round: half of the effective operations run at the int8 rate (Q.K), half at the bf16
# rate (P.V), so the peak for the mix is 1 / (0.5 / 5000 + 0.5 / 2500) TOP/s.
I8QK_MIXED_PEAK = 1.0 / (0.5 / INT8_DENSE_TOPS + 0.5 / BF16_DENSE_TFLOPS)
METRIC = "effective attention TFLOP/s per 1F1C round (% bf16 MFMA peak); chunk-rounds/s"
PROFILES = os.path.join(ROOT, "profiles")
ATTN_SRC = os.path.join(ROOT, "chunk_causal_dit_amd", "csrc", "attn_fwd.hip")
ATTN_KERNEL = "attn_fwd_bf16_kernel<128, 8, false>"
MERGE_KERNEL = "attn_combine_kernel<128>"


def effective_pairs_per_head(cfg: RoundConfig) -> int:
    """Visible (query, key) pairs per head: chunk j's C queries see (n_hist + j + 1) * C keys."""
    C = cfg.chunk_tokens
    return sum(C * (cfg.n_hist + j + 1) * C for j in range(cfg.n_inflight))


def effective_flops(cfg: RoundConfig) -> float:
    return 4.0 * cfg.head_dim * cfg.n_heads * effective_pairs_per_head(cfg)


def executed_flops(cfg: RoundConfig, wave_rows: int = 32, key_tile: int = 64) -> float:
    """FLOPs the kernel issues: each wave holds 32 query rows (a wave past the chunk end
    issues nothing; the last one pads its rows) and covers whole 64-key tiles of every
    visible chunk (the tail tile padded)."""
    C = cfg.chunk_tokens
    qpad = -(-C // wave_rows) * wave_rows
    kpad = -(-C // key_tile) * key_tile
    return 4.0 * cfg.head_dim * cfg.n_heads * sum(qpad * (cfg.n_hist + j + 1) * kpad for j in range(cfg.n_inflight))


def chunk_bytes(cfg: RoundConfig) -> float:
    return float(cfg.chunk_tokens * cfg.n_heads * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4))


def attention_min_bytes(cfg: RoundConfig) -> float:
    """Least HBM traffic of one attention launch: Q read and O written once, every visible
    K and V chunk read once (LSE not counted)."""
    return chunk_bytes(cfg) * (2 * cfg.n_inflight + 2 * (cfg.n_hist + cfg.n_inflight))


def source_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(cfg_name: str):
    """HBM bytes per attention launch from the committed rocprofv3 --pmc summary, or None
    when there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"attn_fwd_{cfg_name}_pmc.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != source_hash(ATTN_SRC):
        return None
    return rec.get("hbm_bytes_per_launch")


def pct(a, q):
    return float(np.percentile(a, q))


def ms_summary(ms) -> dict:
    ms = np.asarray(ms)
    return {"ms_mean": float(ms.mean()), "ms_median": pct(ms, 50), "ms_p10": pct(ms, 10), "ms_p90": pct(ms, 90)}


def cpu_baseline(cfg: RoundConfig, inp, rows_per_chunk: int):
    """The fp64 oracle on a bounded sample of the round (every head, the first
    rows_per_chunk query rows of every in-flight chunk), in effective TFLOP/s."""
    import oracle.attention as OA
    from threadpoolctl import threadpool_info, threadpool_limits

    cores = len(os.sched_getaffinity(0))
    C = cfg.chunk_tokens
    r = min(rows_per_chunk, C)
    rows = np.concatenate([j * C + np.arange(r) for j in range(cfg.n_inflight)])
    k = np.concatenate([inp.k_hist, inp.k_in])
    v = np.concatenate([inp.v_hist, inp.v_in])
    blas = sorted({i.get("internal_api", "?") for i in threadpool_info() if i.get("user_api") == "blas"})
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
                  f"thread pool over (head, chunk) tasks, BLAS ({','.join(blas) or '?'}) 1 thread per task",
        "seconds": dt,
        "round_seconds_extrapolated": dt * effective_flops(cfg) / flops,
        "chunk_rounds_per_s": flops / dt / effective_flops(cfg),
    }


class Timer:
    """Events recorded on one stream; pairs give the GPU time between marks."""

    def __init__(self, torch, stream, n_marks):
        self.torch, self.stream = torch, stream
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_marks)]

    def mark(self, i):
        self.ev[i].record(self.stream)

    def ms(self, a, b):
        return self.ev[a].elapsed_time(self.ev[b])


def dev_bf16(torch, a):
    return torch.from_numpy(a).to("cuda").to(torch.bfloat16)


def bench_round(torch, wf, cfg, steps, warmup, stream, split=True):
    """The headline step; returns timings and the resident state. split: attention through
    the workspace call (key split of in-flight chunk 0)."""
    C, H, D, N, Hs = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, cfg.n_inflight, cfg.n_hist
    inp = make_round_inputs(cfg)
    q, k_in, v_in = (dev_bf16(torch, a) for a in (inp.q, inp.k_in, inp.v_in))
    k_hist, v_hist = dev_bf16(torch, inp.k_hist), dev_bf16(torch, inp.v_hist)
    kc = [k_in[j * C:(j + 1) * C] for j in range(N)]
    vc = [v_in[j * C:(j + 1) * C] for j in range(N)]
    # steady state between rounds: n_hist history chunks + the N-1 continuing in-flight chunks
    cache = wf.KVCache(Hs + N, C, H, D, torch.bfloat16)
    for c in range(Hs):
        cache.append(k_hist[c * C:(c + 1) * C], v_hist[c * C:(c + 1) * C])
    for j in range(N - 1):
        cache.append(kc[j], vc[j])
    out = torch.empty_like(q)
    lse = torch.empty((H, N * C), dtype=torch.float32, device="cuda")
    ws = wf.attn_fwd_workspace(cache) if split else None

    def step(t=None):
        if t:
            t.mark(0)
        cache.append(kc[N - 1], vc[N - 1])              # new noisiest chunk
        for j in range(N - 1):                          # this round's K/V of the continuing chunks
            cache.refresh(Hs + j, kc[j], vc[j])
        if t:
            t.mark(1)
        wf.chunk_causal_attn_fwd(q, cache, N, cfg.scale, out=out, lse=lse, workspace=ws)
        if t:
            t.mark(2)
        cache.evict(1)                                  # the refresh chunk is history from now on

    for _ in range(warmup):
        step()
    timers = [Timer(torch, stream, 3) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(timers[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kv_ms = [t.ms(0, 1) for t in timers]
    attn_ms = [t.ms(1, 2) for t in timers]
    return inp, wall * 1e3 / steps, kv_ms, attn_ms


def bench_rollout(torch, wf, cfg, rounds, warmup, stream, fused=False, split=True):
    """Long-rollout steady state on a permuted 12-slot ring: per round rope3d(Q), rope3d(K),
    append, refresh, attention, evict; with fused=True, K is rotated inside the cache writes
    (append_rope / refresh_rope) instead. Timing only (the values are those of round 0,
    rotated again every round)."""
    from workloads import slot_permutation
    C, H, D, N, Hs = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, cfg.n_inflight, cfg.n_hist
    fpc, gh, gw, rsplit = cfg.frames_per_chunk, cfg.grid_h, cfg.grid_w, cfg.rope_split
    k0, v0 = make_rollout_init(cfg)
    kd, vd = dev_bf16(torch, k0), dev_bf16(torch, v0)
    del k0, v0
    n0 = Hs + N - 1
    cache = wf.KVCache(cfg.slots, C, H, D, torch.bfloat16)
    cache.set_table(slot_permutation(cfg.slots, seed=cfg.seed)[:n0])
    if fused:
        cache.set_rope(fpc, gh, gw, rsplit)
    for g in range(n0):
        cache.refresh(g, kd[g * C:(g + 1) * C], vd[g * C:(g + 1) * C])
    q, k, v = (dev_bf16(torch, a) for a in make_rollout_round(cfg, 0))
    out = torch.empty_like(q)
    lse = torch.empty((H, N * C), dtype=torch.float32, device="cuda")
    ws = wf.attn_fwd_workspace(cache) if split else None

    def one(r, t=None):
        first = r + Hs
        if t:
            t.mark(0)
        wf.rope3d(q, first, fpc, gh, gw, rsplit)
        if not fused:
            wf.rope3d(k, first, fpc, gh, gw, rsplit)
        if t:
            t.mark(1)
        if fused:
            cache.append_rope(k[(N - 1) * C:], v[(N - 1) * C:], first + N - 1)
            for j in range(N - 1):
                cache.refresh_rope(Hs + j, k[j * C:(j + 1) * C], v[j * C:(j + 1) * C], first + j)
        else:
            cache.append(k[(N - 1) * C:], v[(N - 1) * C:])
            for j in range(N - 1):
                cache.refresh(Hs + j, k[j * C:(j + 1) * C], v[j * C:(j + 1) * C])
        if t:
            t.mark(2)
        wf.chunk_causal_attn_fwd(q, cache, N, cfg.scale, out=out, lse=lse, workspace=ws)
        if t:
            t.mark(3)
        cache.evict(1)

    for r in range(warmup):
        one(r)
    timers = [Timer(torch, stream, 4) for _ in range(rounds)]
    torch.cuda.synchronize()
    for r in range(rounds):
        one(warmup + r, timers[r])
    torch.cuda.synchronize()
    rope = np.array([t.ms(0, 1) for t in timers])
    kvw = np.array([t.ms(1, 2) for t in timers])
    attn = np.array([t.ms(2, 3) for t in timers])
    tot = rope + kvw + attn
    rope_bytes = (1 if fused else 2) * 2 * N * chunk_bytes(cfg)  # Q (and K unless fused), read + write
    kv_bytes = 4 * N * chunk_bytes(cfg)              # N chunks of K and V, read + write
    eff = effective_flops(cfg)
    return {
        "workload": f"{cfg.name}: {cfg.description}",
        "producer": "K rotated inside the cache writes" if fused else "rope3d on Q and K, then the cache writes",
        "rounds_timed": rounds,
        "round": ms_summary(tot),
        "hot_path_rounds_per_s": 1e3 / float(np.median(tot)),
        "attention": {**ms_summary(attn), "tflops_median": eff / (np.median(attn) / 1e3) / 1e12,
                      "frac_of_bf16_peak": eff / (np.median(attn) / 1e3) / 1e12 / BF16_DENSE_TFLOPS},
        ("rope3d_q" if fused else "rope3d_q_and_k"): {**ms_summary(rope), "gbs_median": rope_bytes / (np.median(rope) / 1e3) / 1e9,
                           "frac_of_hbm_peak": rope_bytes / (np.median(rope) / 1e3) / 1e9 / HBM_GBS,
                           "bytes": rope_bytes},
        "kv_writes": {**ms_summary(kvw), "gbs_median": kv_bytes / (np.median(kvw) / 1e3) / 1e9, "bytes": kv_bytes},
    }


def bench_i8qk(torch, wf, cfg, steps, warmup, stream, power_seconds=0.0):
    """14B-shaped int8-QK round: quantization kernels + int8 attention, one C call (with
    power_seconds > 0, also the board power, clock and energy per call back to back)."""
    C, H, D, N, Hs = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, cfg.n_inflight, cfg.n_hist
    inp = make_round_inputs(cfg)
    q = dev_bf16(torch, inp.q)
    cache = wf.KVCache(Hs + N, C, H, D, torch.bfloat16)
    for src_k, src_v, n in ((inp.k_hist, inp.v_hist, Hs), (inp.k_in, inp.v_in, N)):
        kk, vv = dev_bf16(torch, src_k), dev_bf16(torch, src_v)
        for c in range(n):
            cache.append(kk[c * C:(c + 1) * C], vv[c * C:(c + 1) * C])
        torch.cuda.synchronize()
        del kk, vv
    del inp
    ws = torch.empty(wf.attn_i8qk_workspace_bytes(cache, N), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((H, N * C), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        wf.chunk_causal_attn_fwd_i8qk(q, cache, N, cfg.scale, workspace=ws, out=out, lse=lse)
    timers = [Timer(torch, stream, 2) for _ in range(steps)]
    torch.cuda.synchronize()
    for t in timers:
        t.mark(0)
        wf.chunk_causal_attn_fwd_i8qk(q, cache, N, cfg.scale, workspace=ws, out=out, lse=lse)
        t.mark(1)
    torch.cuda.synchronize()
    ms = np.array([t.ms(0, 1) for t in timers])
    eff = effective_flops(cfg)
    tops = eff / (np.median(ms) / 1e3) / 1e12
    res = {
        "workload": f"{cfg.name}: {cfg.description}",
        "call": "key sums, key mean, quantize K - mean and Q (4 kernels) + int8-QK attention",
        **ms_summary(ms),
        "effective_tops_median": tops,
        "peak_mixed_tops": I8QK_MIXED_PEAK,
        "frac_of_mixed_peak": tops / I8QK_MIXED_PEAK,
        "frac_of_bf16_peak": tops / BF16_DENSE_TFLOPS,
        "chunk_rounds_per_s": 1e3 / float(np.median(ms)),
    }
    if power_seconds > 0:
        from chunk_causal_dit_amd.profiling import sample_power

        def run():
            for _ in range(5):
                wf.chunk_causal_attn_fwd_i8qk(q, cache, N, cfg.scale, workspace=ws, out=out, lse=lse)

        rec = sample_power(run, torch.cuda.synchronize, power_seconds)
        if rec is not None:
            s_per = rec["seconds"] / (rec["calls"] * 5)
            res["power"] = {"watts": rec["watts"], "cap_watts": rec["cap_watts"], "clock_mhz": rec["clock_mhz"],
                            "ms_per_call": s_per * 1e3, "joules_per_call": rec["watts"] * s_per}
    return res


def bench_gemm_ceiling(torch, stream, steps, power_seconds):
    """What a plain dense contraction reaches on this board: library GEMMs (torch.matmul
    on bf16, torch._int_mm with int32 out), 16384 x 16384 x 8192, timed with HIP events
    on the launch stream, with the board power and clock while they run back to back.
    Context for the attention kernels' fractions of the published peaks, which no kernel
    reaches at the board's power cap."""
    from chunk_causal_dit_amd.profiling import sample_power
    M = N = 16384
    K = 8192
    res = {"shape_mnk": [M, N, K], "library": "torch.matmul (hipBLASLt) / torch._int_mm"}
    # a plain device copy (1 GiB of bf16, read once and written once): the HBM rate a
    # streaming kernel reaches here, beside the published 8 TB/s
    src = torch.ones(512 * 1024 * 1024, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    timers = [Timer(torch, stream, 2) for _ in range(steps)]
    torch.cuda.synchronize()
    for t in timers:
        t.mark(0)
        dst.copy_(src)
        t.mark(1)
    torch.cuda.synchronize()
    ms = np.array([t.ms(0, 1) for t in timers])
    moved = 2.0 * src.numel() * src.element_size()
    res["copy"] = {**ms_summary(ms), "bytes_moved": moved, "gbs_median": moved / (np.median(ms) / 1e3) / 1e9,
                   "frac_of_hbm_peak": moved / (np.median(ms) / 1e3) / 1e9 / HBM_GBS}
    del src, dst
    torch.cuda.empty_cache()
    for name in ("bf16", "i8"):
        g = torch.Generator(device="cuda")
        g.manual_seed(15)
        if name == "bf16":
            a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=g)
            b = torch.randn(K, N, device="cuda", dtype=torch.bfloat16, generator=g)
            peak = BF16_DENSE_TFLOPS

            def f():
                return torch.matmul(a, b)
        else:
            a = torch.randint(-127, 128, (M, K), device="cuda", dtype=torch.int8, generator=g)
            b = torch.randint(-127, 128, (N, K), device="cuda", dtype=torch.int8, generator=g).t()
            peak = INT8_DENSE_TOPS

            def f():
                return torch._int_mm(a, b)
        for _ in range(3):
            f()
        timers = [Timer(torch, stream, 2) for _ in range(steps)]
        torch.cuda.synchronize()
        for t in timers:
            t.mark(0)
            f()
            t.mark(1)
        torch.cuda.synchronize()
        ms = np.array([t.ms(0, 1) for t in timers])
        rate = 2.0 * M * N * K / (np.median(ms) / 1e3) / 1e12
        leg = {**ms_summary(ms), "t_per_s_median": rate, "frac_of_peak": rate / peak, "peak": peak}
        if power_seconds > 0:
            def run():
                for _ in range(5):
                    f()

            rec = sample_power(run, torch.cuda.synchronize, power_seconds)
            if rec is not None:
                leg.update({"watts": rec["watts"], "cap_watts": rec["cap_watts"], "clock_mhz": rec["clock_mhz"]})
        res[name] = leg
        del a, b
        torch.cuda.empty_cache()
    return res


# Linear shapes of the DiT blocks around attention: (name, out features, in features).
W8A8_SHAPES = [
    ("wan13b_qkv", 4608, 1536), ("wan13b_o", 1536, 1536),
    ("wan14b_qkv", 15360, 5120), ("wan14b_o", 5120, 5120),
]


def bench_w8a8(torch, wf, tokens, steps, warmup, stream):
    """W8A8 linears on one round's in-flight tokens: per-token activation quantization and the
    int8 GEMM with the scale/bias epilogue, per shape; hipBLASLt's int8 GEMM (int32 output, no
    epilogue) timed beside it as context."""
    g = torch.Generator(device="cuda")
    g.manual_seed(8)
    out = {"tokens": tokens, "data": "X ~ N(0,1), W ~ N(0, 0.02^2), bias ~ N(0, 0.1^2), bf16, device RNG"}
    for name, N, K in W8A8_SHAPES:
        x = torch.randn(tokens, K, generator=g, device="cuda").to(torch.bfloat16)
        w = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        b = (torch.randn(N, generator=g, device="cuda") * 0.1).to(torch.bfloat16)
        wq, sw = wf.quant_rows_i8(w)
        xq, sx = wf.quant_rows_i8(x)
        y = wf.gemm_w8a8(xq, sx, wq, sw, b)
        for _ in range(warmup):
            wf.quant_rows_i8(x, xq, sx)
            wf.gemm_w8a8(xq, sx, wq, sw, b, out=y)
        timers = [Timer(torch, stream, 3) for _ in range(steps)]
        torch.cuda.synchronize()
        for t in timers:
            t.mark(0)
            wf.quant_rows_i8(x, xq, sx)
            t.mark(1)
            wf.gemm_w8a8(xq, sx, wq, sw, b, out=y)
            t.mark(2)
        torch.cuda.synchronize()
        q_ms = np.array([t.ms(0, 1) for t in timers])
        g_ms = np.array([t.ms(1, 2) for t in timers])
        ops = 2.0 * tokens * N * K
        tops = ops / (np.median(g_ms) / 1e3) / 1e12
        qbytes = tokens * K * 3 + tokens * 4  # bf16 in, int8 codes and fp32 scales out
        ref = {}
        try:
            wt = wq.t()
            for _ in range(3):
                torch._int_mm(xq, wt)
            tl = [Timer(torch, stream, 2) for _ in range(steps)]
            torch.cuda.synchronize()
            for t in tl:
                t.mark(0)
                torch._int_mm(xq, wt)
                t.mark(1)
            torch.cuda.synchronize()
            r_ms = np.array([t.ms(0, 1) for t in tl])
            ref = {"hipblaslt_int8_gemm_ms_median": pct(r_ms, 50),
                   "hipblaslt_tops_median": ops / (np.median(r_ms) / 1e3) / 1e12}
        except Exception as e:  # context only
            ref = {"hipblaslt_int8_gemm": f"unavailable: {type(e).__name__}"}
        out[name] = {
            "M_N_K": [tokens, N, K],
            "gemm": {**ms_summary(g_ms), "tops_median": tops, "frac_of_int8_peak": tops / INT8_DENSE_TOPS},
            "quant_activations": {**ms_summary(q_ms), "gbs_median": qbytes / (np.median(q_ms) / 1e3) / 1e9},
            **ref,
        }
        del x, w, b, wq, sw, xq, sx, y
        torch.cuda.empty_cache()
    return out


def bench_rollout_1f1c(torch, wf, n_steps, n_chunks, hist_window, chunk_tokens, n_heads, head_dim, stream,
                       rope=None, split=True):
    """A whole 1F1C rollout of one layer through wf_1f1c_plan / wf_1f1c_run_round: pipeline
    fill, steady state, drain. The null model's Q/K/V come from a device pool of seeded draws
    reused across chunks (timing only needs the shapes); each round is timed with events."""
    C, H, D = chunk_tokens, n_heads, head_dim
    g = torch.Generator(device="cuda")
    g.manual_seed(14)
    P = hist_window + n_steps + 2  # distinct chunk entries, reused modulo P

    def draw(rows):
        return torch.randn(rows, H, D, generator=g, device="cuda").to(torch.bfloat16)

    kpool = {(c, s): draw(C) for c in range(P) for s in range(n_steps + 1)}
    vpool = {(c, s): draw(C) for c in range(P) for s in range(n_steps + 1)}
    qblock = draw((n_steps + 1) * C)

    def model(plan):
        ks = [kpool[(c % P, s)] for c, s in plan.inflight]
        vs = [vpool[(c % P, s)] for c, s in plan.inflight]
        return qblock[:plan.n_inflight * C], ks, vs

    scale = 1.0 / float(np.sqrt(D))
    ro = wf.Rollout1F1C(n_steps, n_chunks, hist_window, C, H, D, scale, torch.bfloat16, stream=stream, rope=rope,
                        split=split)
    timers, plans = [], []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for _ in range(ro.n_rounds):
        t = Timer(torch, stream, 2)
        t.mark(0)
        plan, _, _ = ro.step(model)
        t.mark(1)
        timers.append(t)
        plans.append((plan.n_inflight, plan.n_hist, plan.output))
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = np.array([t.ms(0, 1) for t in timers])
    flops = np.array([4.0 * D * H * sum(C * (nh + j + 1) * C for j in range(n)) for n, nh, _ in plans])
    steady = [i for i, (n, nh, o) in enumerate(plans) if n == n_steps + 1 and nh == hist_window]
    fill = [i for i, (_, _, o) in enumerate(plans) if o is None]
    res = {
        "workload": f"{n_steps}-step rollout of {n_chunks} chunks ({3 * n_chunks} latent frames), history window "
                    f"{hist_window}, {H} heads x {D}, {C}-token chunks, one layer"
                    + (", 3D RoPE (query block rotated in place, K in the cache writes)" if rope else ""),
        "rounds": ro.n_rounds, "fill_rounds": len(fill), "steady_rounds": len(steady),
        "rollout_ms_gpu": float(ms.sum()), "rollout_s_wall": wall,
        "round_all": ms_summary(ms),
        "effective_tflops_whole_rollout": float(flops.sum() / (ms.sum() / 1e3) / 1e12),
        "outputs_per_s_whole_rollout": n_chunks / (ms.sum() / 1e3),
    }
    if steady:
        sm = ms[steady]
        res["round_steady"] = ms_summary(sm)
        res["steady_outputs_per_s"] = 1e3 / float(np.median(sm))
        res["steady_effective_tflops"] = float(flops[steady[0]] / (np.median(sm) / 1e3) / 1e12)
    return res


def bench_power(torch, wf, cfg, seconds, split=True):
    """Board power while the headline attention runs back to back, and energy per launch."""
    from chunk_causal_dit_amd.profiling import sample_power
    C, H, D, N, Hs = cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, cfg.n_inflight, cfg.n_hist
    inp = make_round_inputs(cfg)
    q = dev_bf16(torch, inp.q)
    cache = wf.KVCache(Hs + N, C, H, D, torch.bfloat16)
    for src_k, src_v, n in ((inp.k_hist, inp.v_hist, Hs), (inp.k_in, inp.v_in, N)):
        kk, vv = dev_bf16(torch, src_k), dev_bf16(torch, src_v)
        for c in range(n):
            cache.append(kk[c * C:(c + 1) * C], vv[c * C:(c + 1) * C])
    out = torch.empty_like(q)
    ws = wf.attn_fwd_workspace(cache) if split else None
    reps = 20

    def run():
        for _ in range(reps):
            wf.chunk_causal_attn_fwd(q, cache, N, cfg.scale, out=out, with_lse=False, workspace=ws)

    run()
    torch.cuda.synchronize()
    rec = sample_power(run, torch.cuda.synchronize, seconds)
    if rec is None:
        return {"available": False}
    launches = rec["calls"] * reps
    s_per = rec["seconds"] / launches
    return {"available": True, "watts": rec["watts"], "launches": launches, "ms_per_launch": s_per * 1e3,
            "joules_per_launch": rec["watts"] * s_per,
            "effective_gflop_per_joule": effective_flops(cfg) / (rec["watts"] * s_per) / 1e9,
            "clock_mhz": rec["clock_mhz"], "cap_watts": rec["cap_watts"], "sensor": rec["sensor"],
            "clock_sensor": rec["clock_sensor"]}


def copy_probe(torch, mib: int):
    """A plain device-to-device copy of known size, for calibrating HBM byte counters."""
    n = mib * 1024 * 1024 // 2
    a = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"[bench] copy probe: {n * 2} bytes x 3", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-rows", type=int, default=4680, help="query rows per chunk in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the rollout, int8-QK, W8A8, library-GEMM and 1F1C rollout measurements")
    ap.add_argument("--copy-probe-mib", type=int, default=0, help="run a plain copy of this size first")
    ap.add_argument("--no-split", action="store_true",
                    help="time wf_chunk_causal_attn_fwd (no key split of chunk 0) instead of the workspace call")
    ap.add_argument("--w8a8-only", action="store_true",
                    help="run only the W8A8 linear measurement and print its JSON (for profiling)")
    ap.add_argument("--rollout-only", action="store_true",
                    help="run only the 1F1C rollout measurement and print its JSON (for profiling)")
    ap.add_argument("--i8qk-only", action="store_true",
                    help="run only the 14B-shaped int8-QK round (--steps timed calls) and print its JSON (for profiling)")
    ap.add_argument("--power-seconds", type=float, default=3.0,
                    help="seconds of back-to-back attention launches with the board power sensor read (0: off)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunk_causal_dit_amd as wf

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wf.lib()  # fails loudly when the HIP library is missing
    stream = torch.cuda.current_stream()
    if args.copy_probe_mib:
        copy_probe(torch, args.copy_probe_mib)

    cfg = CONFIGS["wan13b_4step"]
    split = not args.no_split
    if args.w8a8_only:
        print(json.dumps({"w8a8": bench_w8a8(torch, wf, cfg.nq, args.steps, args.warmup, stream)}), flush=True)
        return
    if args.i8qk_only:
        print(json.dumps({"i8qk": bench_i8qk(torch, wf, CONFIGS["i8qk_14b"], args.steps, args.warmup, stream,
                                             power_seconds=args.power_seconds)}),
              flush=True)
        return
    if args.rollout_only:
        print(json.dumps({"rollout_1f1c": {
            "4step": bench_rollout_1f1c(torch, wf, 4, 133, 2, cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, stream,
                                        split=split)}}),
            flush=True)
        return
    inp, ms_per_step, kv_ms, attn_ms = bench_round(torch, wf, cfg, args.steps, args.warmup, stream, split=split)
    print(f"[bench] {cfg.name}: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    eff = effective_flops(cfg)
    attn_s = float(np.mean(attn_ms)) / 1e3
    # the published dense peak, and the same figure from this device's CU count and peak clock
    n_cu, clk_khz = wf.device_peak_info(torch.cuda.current_device())
    peak_note = {"published_bf16_dense_tflops": BF16_DENSE_TFLOPS, "device_cus": n_cu,
                 "device_peak_clock_mhz": clk_khz / 1e3,
                 "derived_bf16_dense_tflops": n_cu * 4096 * clk_khz * 1e3 / 1e12,
                 "used": "published"}
    achieved = eff / attn_s / 1e12
    kv_bytes = 4 * cfg.n_inflight * chunk_bytes(cfg)
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
            "heads": cfg.n_heads, "head_dim": cfg.head_dim, "chunk_tokens": cfg.chunk_tokens,
            "n_inflight": cfg.n_inflight, "n_hist": cfg.n_hist,
            "query_tokens": cfg.nq, "visible_keys_max": cfg.nkv,
            "effective_flops_per_round": eff,
            "executed_flops_per_round": executed_flops(cfg),
            "step": "kv append (1 chunk) + kv refresh (N-1 chunks) + attention + evict",
        },
        "chunk_rounds_per_s": 1e3 / ms_per_step,
        "attention": {
            **ms_summary(attn_ms),
            "tflops": achieved, "frac_of_bf16_peak": achieved / BF16_DENSE_TFLOPS,
            "executed_tflops": executed_flops(cfg) / attn_s / 1e12,
            "rounds_per_s": 1.0 / attn_s,
        },
        "kv_writes": {**ms_summary(kv_ms), "bytes": kv_bytes,
                      "gbs_median": kv_bytes / (np.median(kv_ms) / 1e3) / 1e9,
                      "frac_of_hbm_peak": kv_bytes / (np.median(kv_ms) / 1e3) / 1e9 / HBM_GBS},
        "peak_note": peak_note,
        "roofline": {
            "bound": "mfma",
            "kernel": ATTN_KERNEL + (" + " + MERGE_KERNEL if split else ""),
            "call": "wf_chunk_causal_attn_fwd_ws (key split of in-flight chunk 0)" if split
                    else "wf_chunk_causal_attn_fwd",
            "achieved": achieved,
            "peak": BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / BF16_DENSE_TFLOPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": attention_min_bytes(cfg),
            "timing": "hip events on the launch stream around each attention call (the attention kernel, plus the "
                      "merge kernel of the split), mean over the timed steps",
            "call_avg_us": attn_s * 1e6,
        },
    }
    if args.power_seconds > 0:
        res["power"] = bench_power(torch, wf, cfg, args.power_seconds, split=split)
        clk = res["power"].get("clock_mhz")
        if clk:
            # the clock level the driver reported while the call ran back to back (sampled
            # during the power loop; the counters' GRBM_GUI_ACTIVE / duration gives the lower
            # effective clock, see profiles/), and the dense bf16 peak at that level:
            # CUs x 4096 flop/clk x clock
            clk_peak = n_cu * 4096 * clk * 1e6 / 1e12
            res["roofline"].update({"dpm_clock_mhz": clk, "dpm_clock_peak_tflops": clk_peak,
                                    "frac_of_dpm_clock_peak": achieved / clk_peak})
    if not args.no_extras:
        res["rollout"] = bench_rollout(torch, wf, CONFIGS["long_rollout"], 20, 5, stream, split=split)
        res["rollout_fused"] = bench_rollout(torch, wf, CONFIGS["long_rollout"], 20, 5, stream, fused=True,
                                             split=split)
        print("[bench] rollout done", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        res["i8qk"] = bench_i8qk(torch, wf, CONFIGS["i8qk_14b"], 20, 3, stream, power_seconds=args.power_seconds)
        print("[bench] int8-QK done", file=sys.stderr, flush=True)
        res["w8a8"] = bench_w8a8(torch, wf, cfg.nq, 20, 3, stream)
        print("[bench] W8A8 linears done", file=sys.stderr, flush=True)
        ceil = bench_gemm_ceiling(torch, stream, 10, min(args.power_seconds, 2.0))
        res["gemm_ceiling"] = ceil
        res["roofline"]["frac_of_library_gemm"] = achieved / ceil["bf16"]["t_per_s_median"]
        res["kv_writes"]["frac_of_plain_copy"] = res["kv_writes"]["gbs_median"] / ceil["copy"]["gbs_median"]
        res["i8qk"]["frac_of_library_gemms_mixed"] = res["i8qk"]["effective_tops_median"] / (
            1.0 / (0.5 / ceil["i8"]["t_per_s_median"] + 0.5 / ceil["bf16"]["t_per_s_median"]))
        print("[bench] library GEMM ceiling done", file=sys.stderr, flush=True)
        res["rollout_1f1c"] = {
            "4step": bench_rollout_1f1c(torch, wf, 4, 133, 2, cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, stream,
                                        split=split),
            "5step": bench_rollout_1f1c(torch, wf, 5, 133, 3, cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, stream,
                                        split=split),
            "4step_rope": bench_rollout_1f1c(torch, wf, 4, 133, 2, cfg.chunk_tokens, cfg.n_heads, cfg.head_dim, stream,
                                             split=split,
                                             rope={"frames_per_chunk": 3, "grid_h": 30, "grid_w": 52}),
        }
        print("[bench] 1F1C rollouts done", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_rows)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
