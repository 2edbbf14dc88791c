"""Pins of the 1F1C schedule oracle (oracle/schedule.py) to values fixed outside it:
hand-worked round tables, the pages' step lists and wp-size, counting invariants of
the staggered pipeline, and a scalar assembly of each round's visible keys."""
import math
import os

import numpy as np
import pytest

from oracle import schedule as SC

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "schedule_hand_tables.txt")


def read_tables():
    tables, cur = {}, None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("table"):
            S, F, W = map(int, line.split()[1:])
            cur = tables.setdefault((S, F, W), [])
            continue
        r, inf, hist, out = (x.strip() for x in line.split("|"))
        cur.append((int(r), [tuple(map(int, t.split(":"))) for t in inf.split()],
                    [] if hist == "-" else list(map(int, hist.split())), None if out == "-" else int(out)))
    return tables


def plan_as_row(S, plan):
    ts = SC.timesteps(S) + [0]
    return (plan["round"], [(c, ts[s]) for c, s in plan["inflight"]], plan["hist"], plan["output"])


def check_tables(round_plan):
    for (S, F, W), rows in read_tables().items():
        assert SC.n_rounds(S, F) == len(rows)
        for row in rows:
            assert plan_as_row(S, round_plan(S, F, W, row[0])) == row


def test_hand_tables():
    check_tables(SC.round_plan)


def test_step_lists_of_the_pages():
    assert SC.timesteps(4) == [1000, 750, 500, 250]
    assert SC.timesteps(5) == [1000, 800, 600, 400, 200]


@pytest.mark.parametrize("S,F,W", [(1, 1, 0), (1, 5, 1), (4, 1, 2), (4, 3, 2), (4, 8, 2), (4, 20, 6),
                                   (5, 8, 3), (5, 133, 6), (2, 7, 0)])
def test_pipeline_invariants(S, F, W):
    R = SC.n_rounds(S, F)
    seen = {c: [] for c in range(F)}
    outputs = []
    for r in range(R):
        p = SC.round_plan(S, F, W, r)
        chunks = [c for c, _ in p["inflight"]]
        assert chunks == sorted(chunks) and len(chunks) <= S + 1  # cleanest first, at most wp-size stages
        assert [s for _, s in p["inflight"]] == sorted((s for _, s in p["inflight"]), reverse=True)
        if S <= r < F:
            assert len(chunks) == S + 1  # steady state: every stage busy
        for c, s in p["inflight"]:
            seen[c].append((r, s))
        assert len(p["hist"]) <= W and all(h < min(chunks) for h in p["hist"])
        assert p["new"] == (r if r < F else None)
        if r >= S - 1:
            outputs.append(p["output"])
        else:
            assert p["output"] is None  # pipeline fill
    assert outputs == list(range(F))  # one output per round after the fill, in order
    for c, visits in seen.items():
        last = S - 1 if c == F - 1 else S
        assert visits == [(c + s, s) for s in range(last + 1)]  # stages in consecutive rounds


def _qkv_model(S, C, H, D):
    def qkv(c, s):
        rng = np.random.default_rng(1000 * c + s)
        return tuple(rng.standard_normal((C, H, D)) for _ in range(3))
    return qkv


def test_rollout_attention_matches_scalar_assembly():
    """Each round's output from the definition: a query of chunk c sees the clean K/V of the
    history chunks, then this round's K/V of the in-flight chunks up to and including c."""
    S, F, W, C, H, D = 3, 5, 2, 2, 2, 3
    qkv = _qkv_model(S, C, H, D)
    scale = 0.4
    res = SC.rollout_attention(S, F, W, qkv, scale)
    for r, (o, lse, plan) in res.items():
        for qi, (c, s) in enumerate(plan["inflight"]):
            keys, vals = [], []
            for hc in plan["hist"]:
                _, k, v = qkv(hc, S)
                keys += list(k)
                vals += list(v)
            for c2, s2 in plan["inflight"]:
                if c2 <= c:
                    _, k, v = qkv(c2, s2)
                    keys += list(k)
                    vals += list(v)
            q = qkv(c, s)[0]
            for t in range(C):
                for h in range(H):
                    logits = [scale * sum(q[t, h, d] * kk[h, d] for d in range(D)) for kk in keys]
                    m = max(logits)
                    w = [math.exp(x - m) for x in logits]
                    z = sum(w)
                    ref = [sum(w[i] * vals[i][h, d] for i in range(len(w))) / z for d in range(D)]
                    assert np.allclose(o[qi * C + t, h], ref, atol=1e-12)
                    assert abs(lse[h, qi * C + t] - (m + math.log(z))) < 1e-12


def test_rollout_attention_with_rope_matches_scalar_rotation():
    """With rope, chunk c's Q and K are rotated at global chunk c: here each pair is rotated
    by explicit cos/sin of the pages-independent angle list (rotation_angles), then the
    round's attention is built from the definition as above."""
    from oracle.rope import rotation_angles
    S, F, W, fpc, gh, gw, H, D = 2, 4, 1, 1, 2, 2, 1, 8
    C = fpc * gh * gw
    split = (4, 2, 2)
    qkv = _qkv_model(S, C, H, D)
    scale = 0.5
    rope = {"frames_per_chunk": fpc, "grid_h": gh, "grid_w": gw, "split": split, "theta": 100.0}
    res = SC.rollout_attention(S, F, W, qkv, scale, rope=rope)

    def rot(x, c):
        y = np.array(x, dtype=np.float64)
        for t in range(C):
            pos = (fpc * c + t // (gh * gw), (t // gw) % gh, t % gw)
            ang = rotation_angles(pos, split, 100.0)
            for h in range(H):
                for i, a in enumerate(ang):
                    x0, x1 = x[t, h, 2 * i], x[t, h, 2 * i + 1]
                    y[t, h, 2 * i] = x0 * math.cos(a) - x1 * math.sin(a)
                    y[t, h, 2 * i + 1] = x0 * math.sin(a) + x1 * math.cos(a)
        return y

    for r, (o, lse, plan) in res.items():
        for qi, (c, s) in enumerate(plan["inflight"]):
            keys, vals = [], []
            for hc in plan["hist"]:
                _, k, v = qkv(hc, S)
                keys += list(rot(k, hc))
                vals += list(v)
            for c2, s2 in plan["inflight"]:
                if c2 <= c:
                    _, k, v = qkv(c2, s2)
                    keys += list(rot(k, c2))
                    vals += list(v)
            q = rot(qkv(c, s)[0], c)
            for t in range(C):
                logits = [scale * float(np.dot(q[t, 0], kk[0])) for kk in keys]
                m = max(logits)
                w = [math.exp(x - m) for x in logits]
                ref = sum(wi * vv[0] for wi, vv in zip(w, vals)) / sum(w)
                assert np.allclose(o[qi * C + t, 0], ref, atol=1e-12)


@pytest.mark.parametrize("kind", ["noisiest_first", "refresh_late", "window_plus_one", "refresh_chunk_in_history",
                                  "window_slice_wraps"])
def test_planted_mistakes_are_caught(kind):
    def bad_plan(S, F, W, r):
        p = SC.round_plan(S, F, W, r)
        if kind == "noisiest_first":
            p["inflight"] = p["inflight"][::-1]
        elif kind == "refresh_late":  # refresh pass one round after the last denoising step
            p["inflight"] = [(c, s) for c, s in p["inflight"] if s != S]
        elif kind == "window_plus_one":
            done = [c for c in range(F) if c + S < r and c != F - 1]
            p["hist"] = done[-(W + 1):]
        elif kind == "window_slice_wraps":  # slice start len - W goes negative while fewer than W are done
            done = [c for c in range(F) if c + S < r and c != F - 1]
            p["hist"] = done[len(done) - W:] if W > 0 else []
        elif kind == "refresh_chunk_in_history":  # history already holds the chunk refreshed this round
            done = [c for c in range(F) if c + S <= r and c != F - 1]
            p["hist"] = done[-W:]
        return p
    with pytest.raises(AssertionError):
        check_tables(bad_plan)
