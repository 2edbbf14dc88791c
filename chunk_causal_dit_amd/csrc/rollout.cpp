// The 1F1C round planner and the round runner: host code that turns a
// rollout (steps, chunks, history window) into the cache operations and the
// attention launch of each round, on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "wf_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// History chunks visible in round r: chunks refreshed in rounds before r (chunk c is
// refreshed in round c + S, and the last chunk never), at most W of them.
int refreshed_before(int S, int F, int r) { return std::max(0, std::min(r - S, F - 1)); }

}  // namespace

using wf::fail;

WF_EXPORT int wf_1f1c_rounds(int n_steps, int n_chunks) {
  if (n_steps < 1 || n_chunks < 1 || n_steps + 1 > WF_MAX_TABLE)
    return fail(WF_E_SHAPE, "wf_1f1c_rounds: need n_steps in [1, %d] and n_chunks >= 1 (got %d, %d)",
                WF_MAX_TABLE - 1, n_steps, n_chunks);
  if (n_chunks > (1 << 30) - n_steps) return fail(WF_E_SHAPE, "wf_1f1c_rounds: too many chunks");
  return n_chunks + n_steps - 1;
}

WF_EXPORT int wf_1f1c_plan(int n_steps, int n_chunks, int hist_window, int round, wf_round_plan* plan) {
  const char* who = "wf_1f1c_plan";
  if (!plan) return fail(WF_E_NULL, "%s: NULL plan", who);
  const int rounds = wf_1f1c_rounds(n_steps, n_chunks);
  if (rounds < 0) return rounds;
  if (hist_window < 0 || hist_window + n_steps + 1 > WF_MAX_TABLE)
    return fail(WF_E_SHAPE, "%s: need 0 <= hist_window <= %d - n_steps - 1 (got %d)", who, WF_MAX_TABLE, hist_window);
  if (round < 0 || round >= rounds) return fail(WF_E_SHAPE, "%s: round %d outside [0, %d)", who, round, rounds);
  const int S = n_steps, F = n_chunks, r = round;
  wf_round_plan p;
  std::memset(&p, 0, sizeof p);
  p.round = r;
  // chunks lo .. hi are in flight, chunk c at stage r - c; the last chunk's refresh
  // (round F - 1 + S) lies past the final round, so the range needs no exclusion
  const int lo = std::max(0, r - S), hi = std::min(F - 1, r);
  p.n_inflight = hi - lo + 1;
  for (int i = 0; i < p.n_inflight; ++i) {
    p.inflight_chunk[i] = lo + i;
    p.inflight_stage[i] = r - (lo + i);
  }
  const int done = refreshed_before(S, F, r);
  p.n_hist = std::min(hist_window, done);
  for (int i = 0; i < p.n_hist; ++i) p.hist_chunk[i] = done - p.n_hist + i;
  p.new_chunk = r < F ? r : -1;
  const int out = r - (S - 1);
  p.output_chunk = (out >= 0 && out < F) ? out : -1;
  if (r + 1 < rounds) {
    // after attention the refresh chunk (if any) turns into history; drop what the
    // next round's window no longer holds
    const bool has_refresh = (r - lo) == S;
    p.evict_after = p.n_hist + (has_refresh ? 1 : 0) - std::min(hist_window, refreshed_before(S, F, r + 1));
  }
  *plan = p;
  return WF_OK;
}

WF_EXPORT int wf_1f1c_run_round(wf_kv_cache* kv, const wf_round_plan* plan, void* q, const void* const* k,
                                const void* const* v, float scale, void* workspace, void* out, float* lse,
                                void* stream) {
  const char* who = "wf_1f1c_run_round";
  if (!kv || !plan || !q || !k || !v || !out) return fail(WF_E_NULL, "%s: NULL argument", who);
  const int N = plan->n_inflight, Hs = plan->n_hist;
  if (N < 1 || Hs < 0 || Hs + N > WF_MAX_TABLE)
    return fail(WF_E_SHAPE, "%s: plan has n_inflight %d, n_hist %d", who, N, Hs);
  const bool append = plan->new_chunk >= 0;
  const int before = Hs + N - (append ? 1 : 0);
  if ((int)kv->table.size() != before)
    return fail(WF_E_SHAPE, "%s: table holds %zu entries, the plan expects %d before round %d", who,
                kv->table.size(), before, plan->round);
  if (plan->evict_after < 0 || plan->evict_after > Hs + N)
    return fail(WF_E_SHAPE, "%s: evict_after %d outside [0, %d]", who, plan->evict_after, Hs + N);
  for (int i = 0; i < N; ++i) {
    if (!k[i] || !v[i]) return fail(WF_E_NULL, "%s: NULL K/V of in-flight entry %d", who, i);
    if (!aligned16(k[i]) || !aligned16(v[i]))
      return fail(WF_E_SHAPE, "%s: K/V of in-flight entry %d must be 16-byte aligned", who, i);
  }
  if (!aligned16(q) || !aligned16(out) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return fail(WF_E_SHAPE, "%s: q and out must be 16-byte aligned, lse 4-byte aligned", who);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(WF_E_SHAPE, "%s: scale must be positive and finite", who);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(WF_E_SHAPE, "%s: workspace must be 256-byte aligned", who);
  if (append && kv->free_slots.empty()) return fail(WF_E_FULL, "%s: no free slot for the new chunk", who);
  if (const int st = wf::check_attn_size(*kv, N, who); st != WF_OK) return st;
  if (const int st = wf::check_workspace_disjoint(*kv, N, workspace, wf::attn_split_bytes(*kv), q, out, lse, who);
      st != WF_OK)
    return st;
  const bool rope = kv->rope.on;
  const int first = plan->inflight_chunk[0];
  if (rope) {
    // the query block is rotated as one run of whole chunks: its chunk ids must be consecutive
    for (int i = 0; i < N; ++i)
      if (plan->inflight_chunk[i] != first + i)
        return fail(WF_E_SHAPE, "%s: with RoPE the in-flight chunk ids must be consecutive", who);
    if (first < 0 || (double)kv->rope.fpc * ((double)first + N + 1) > 16777216.0)
      return fail(WF_E_SHAPE, "%s: frame positions of chunks %d .. %d exceed the exact fp32 integer range", who,
                  first, first + N - 1);
  }

  // every check passed: the calls below can fail only at launch (WF_E_HIP)
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int st = WF_OK;
  if (rope) {
    const wf::RopeConfig& rc = kv->rope;
    hipError_t e = wf::launch_rope3d(q, N * kv->chunk_tokens, kv->n_heads, kv->head_dim, kv->dtype, first, rc.fpc,
                                     rc.gh, rc.gw, rc.table, hs);
    if (e != hipSuccess) return fail(WF_E_HIP, "%s: rope launch failed: %s", who, hipGetErrorString(e));
    if (append && (st = wf_kv_append_rope(kv, k[N - 1], v[N - 1], first + N - 1, stream, nullptr)) != WF_OK)
      return st;
    for (int i = 0; i < N - (append ? 1 : 0); ++i)
      if ((st = wf_kv_refresh_rope(kv, Hs + i, k[i], v[i], first + i, stream)) != WF_OK) return st;
  } else {
    if (append && (st = wf_kv_append(kv, k[N - 1], v[N - 1], stream, nullptr)) != WF_OK) return st;
    for (int i = 0; i < N - (append ? 1 : 0); ++i)
      if ((st = wf_kv_refresh(kv, Hs + i, k[i], v[i], stream)) != WF_OK) return st;
  }
  if ((st = wf_chunk_causal_attn_fwd_ws(q, kv, N, scale, workspace, out, lse, stream)) != WF_OK) return st;
  return wf_kv_evict(kv, plan->evict_after);
}
