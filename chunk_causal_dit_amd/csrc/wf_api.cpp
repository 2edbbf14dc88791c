// Host side of the C ABI: argument validation, the history-cache table and
// the launch glue. Every check runs before any device work, so an error
// return leaves the stream and the cache untouched.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "wf_internal.h"

namespace wf {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

static int ok() { return WF_OK; }

static int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(WF_E_HIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
}

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static int check_shape(int n_slots, int chunk_tokens, int n_heads, int head_dim, int dtype) {
  if (dtype_size(dtype) == 0) return fail(WF_E_DTYPE, "unknown dtype %d", dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(WF_E_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (n_slots < 1 || n_slots > WF_MAX_TABLE)
    return fail(WF_E_SHAPE, "n_slots %d outside [1, %d]", n_slots, WF_MAX_TABLE);
  if (chunk_tokens < 1 || chunk_tokens > (1 << 20))
    return fail(WF_E_SHAPE, "chunk_tokens %d outside [1, 2^20]", chunk_tokens);
  if (n_heads < 1 || n_heads > 1024) return fail(WF_E_SHAPE, "n_heads %d outside [1, 1024]", n_heads);
  return ok();
}

int check_attn_size(const wf_kv_cache& kv, int n_inflight, const char* who) {
  const long long H = kv.n_heads, C = kv.chunk_tokens;
  if (n_inflight * C * H * kv.head_dim >= (1LL << 40)) return fail(WF_E_SHAPE, "%s: query block too large", who);
  // Work-items per launch must fit in 32 bits: the attention kernels run about two
  // threads per query row and head, padded to their query tiles, over at most
  // n_inflight + 1 chunks (the key split adds chunk 0 once more), and the merge one
  // wave per row and head of a chunk.
  if ((n_inflight + 1LL) * H * (C + 255) * 2 >= (1LL << 32) || C * H * 64 >= (1LL << 32))
    return fail(WF_E_SHAPE, "%s: %d chunks of %lld tokens x %lld heads exceed one launch", who, n_inflight, C, H);
  return WF_OK;
}

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_workspace_disjoint(const wf_kv_cache& kv, int n_inflight, const void* ws, size_t ws_bytes, const void* q,
                             const void* out, const float* lse, const char* who) {
  const size_t rows = (size_t)n_inflight * kv.chunk_tokens * kv.n_heads;
  const size_t qb = rows * kv.head_dim * kv.esize, lb = rows * sizeof(float);
  const size_t pool = (size_t)kv.n_slots * kv.slot_elems * kv.esize;
  if (overlaps(ws, ws_bytes, q, qb) || overlaps(ws, ws_bytes, out, qb) || overlaps(ws, ws_bytes, lse, lb) ||
      overlaps(ws, ws_bytes, kv.k_pool, pool) || overlaps(ws, ws_bytes, kv.v_pool, pool))
    return fail(WF_E_SHAPE, "%s: workspace overlaps q, out, lse or a cache pool", who);
  return WF_OK;
}

}  // namespace wf

using namespace wf;

WF_EXPORT size_t wf_kv_pool_bytes(int n_slots, int chunk_tokens, int n_heads, int head_dim, int dtype) {
  if (check_shape(n_slots, chunk_tokens, n_heads, head_dim, dtype) != WF_OK) return 0;
  return (size_t)n_slots * n_heads * pad_tokens(chunk_tokens) * head_dim * dtype_size(dtype);
}

WF_EXPORT int wf_kv_cache_create(wf_kv_cache** out, void* k_pool, void* v_pool, int n_slots,
                                 int chunk_tokens, int n_heads, int head_dim, int dtype, int flags,
                                 void* stream) {
  if (!out || !k_pool || !v_pool) return fail(WF_E_NULL, "wf_kv_cache_create: NULL argument");
  int st = check_shape(n_slots, chunk_tokens, n_heads, head_dim, dtype);
  if (st != WF_OK) return st;
  if (!aligned(k_pool, 256) || !aligned(v_pool, 256))
    return fail(WF_E_SHAPE, "wf_kv_cache_create: pools must be 256-byte aligned");
  if (flags != WF_KV_ADOPT && flags != WF_KV_ZERO_FILL)
    return fail(WF_E_SHAPE, "wf_kv_cache_create: unknown flags %d", flags);
  auto* kv = new wf_kv_cache;
  kv->k_pool = k_pool;
  kv->v_pool = v_pool;
  kv->n_slots = n_slots;
  kv->chunk_tokens = chunk_tokens;
  kv->n_heads = n_heads;
  kv->head_dim = head_dim;
  kv->dtype = dtype;
  kv->s_pad = pad_tokens(chunk_tokens);
  kv->esize = dtype_size(dtype);
  kv->slot_elems = (size_t)n_heads * kv->s_pad * head_dim;
  for (int s = 0; s < n_slots; ++s) kv->free_slots.push_back(s);
  const size_t bytes = (size_t)n_slots * kv->slot_elems * kv->esize;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (flags == WF_KV_ZERO_FILL) {
    e = launch_fill_zero(k_pool, bytes, s);
    if (e == hipSuccess) e = launch_fill_zero(v_pool, bytes, s);
  }
  if (e != hipSuccess) {
    delete kv;
    return hip_status(e, "wf_kv_cache_create");
  }
  *out = kv;
  return ok();
}

WF_EXPORT int wf_kv_cache_destroy(wf_kv_cache* kv) {
  delete kv;
  return WF_OK;
}

WF_EXPORT int wf_kv_append(wf_kv_cache* kv, const void* k, const void* v, void* stream, int* out_slot) {
  if (!kv || !k || !v) return fail(WF_E_NULL, "wf_kv_append: NULL argument");
  if (!aligned(k, 16) || !aligned(v, 16)) return fail(WF_E_SHAPE, "wf_kv_append: k and v must be 16-byte aligned");
  if (kv->free_slots.empty()) return fail(WF_E_FULL, "wf_kv_append: no free slot (%d slots)", kv->n_slots);
  if ((int)kv->table.size() >= WF_MAX_TABLE)
    return fail(WF_E_FULL, "wf_kv_append: table holds WF_MAX_TABLE entries");
  const int slot = kv->free_slots.front();
  hipError_t e = launch_kv_write(*kv, slot, k, v, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "wf_kv_append");
  kv->free_slots.pop_front();
  kv->table.push_back(slot);
  if (out_slot) *out_slot = slot;
  return ok();
}

WF_EXPORT int wf_kv_refresh(wf_kv_cache* kv, int logical_idx, const void* k, const void* v, void* stream) {
  if (!kv || !k || !v) return fail(WF_E_NULL, "wf_kv_refresh: NULL argument");
  if (!aligned(k, 16) || !aligned(v, 16)) return fail(WF_E_SHAPE, "wf_kv_refresh: k and v must be 16-byte aligned");
  if (logical_idx < 0 || logical_idx >= (int)kv->table.size())
    return fail(WF_E_SLOT, "wf_kv_refresh: logical index %d outside table of %zu", logical_idx,
                kv->table.size());
  hipError_t e = launch_kv_write(*kv, kv->table[logical_idx], k, v, static_cast<hipStream_t>(stream));
  return hip_status(e, "wf_kv_refresh");
}

WF_EXPORT int wf_kv_evict(wf_kv_cache* kv, int n_oldest) {
  if (!kv) return fail(WF_E_NULL, "wf_kv_evict: NULL cache");
  if (n_oldest < 0) return fail(WF_E_SHAPE, "wf_kv_evict: negative count %d", n_oldest);
  if (n_oldest > (int)kv->table.size())
    return fail(WF_E_EMPTY, "wf_kv_evict: %d entries requested, table holds %zu", n_oldest,
                kv->table.size());
  for (int i = 0; i < n_oldest; ++i) kv->free_slots.push_back(kv->table[i]);
  kv->table.erase(kv->table.begin(), kv->table.begin() + n_oldest);
  return ok();
}

WF_EXPORT int wf_kv_set_table(wf_kv_cache* kv, const int* slots, int n) {
  if (!kv) return fail(WF_E_NULL, "wf_kv_set_table: NULL cache");
  if (n < 0 || n > kv->n_slots) return fail(WF_E_SHAPE, "wf_kv_set_table: length %d outside [0, %d]", n, kv->n_slots);
  if (n > 0 && !slots) return fail(WF_E_NULL, "wf_kv_set_table: NULL slots");
  std::vector<char> used(kv->n_slots, 0);
  for (int i = 0; i < n; ++i) {
    if (slots[i] < 0 || slots[i] >= kv->n_slots)
      return fail(WF_E_SLOT, "wf_kv_set_table: slot %d outside [0, %d)", slots[i], kv->n_slots);
    if (used[slots[i]]) return fail(WF_E_SLOT, "wf_kv_set_table: slot %d listed twice", slots[i]);
    used[slots[i]] = 1;
  }
  kv->table.assign(slots, slots + n);
  kv->free_slots.clear();
  for (int s = 0; s < kv->n_slots; ++s)
    if (!used[s]) kv->free_slots.push_back(s);
  return ok();
}

WF_EXPORT int wf_kv_get_table(const wf_kv_cache* kv, int* slots, int cap, int* n) {
  if (!kv || !n) return fail(WF_E_NULL, "wf_kv_get_table: NULL argument");
  if (cap < 0) return fail(WF_E_SHAPE, "wf_kv_get_table: negative capacity");
  if (cap > 0 && !slots) return fail(WF_E_NULL, "wf_kv_get_table: NULL slots");
  const int m = std::min<int>(cap, (int)kv->table.size());
  for (int i = 0; i < m; ++i) slots[i] = kv->table[i];
  *n = (int)kv->table.size();
  return ok();
}

// Checks the RoPE geometry and builds its per-pair table (inverse frequency
// rounded once to fp32, axis of the pair).
static int rope_table(int head_dim, int frames_per_chunk, int grid_h, int grid_w, int d_t, int d_h, int d_w,
                      float theta, RopeTable& t, const char* who) {
  if (head_dim != 64 && head_dim != 128) return fail(WF_E_UNSUPPORTED, "%s: head_dim %d not supported", who, head_dim);
  if (frames_per_chunk < 1 || grid_h < 1 || grid_w < 1) return fail(WF_E_SHAPE, "%s: non-positive grid", who);
  if (d_t < 0 || d_h < 0 || d_w < 0 || (d_t | d_h | d_w) & 1 || d_t + d_h + d_w != head_dim)
    return fail(WF_E_SHAPE, "%s: split %d/%d/%d must be even and sum to %d", who, d_t, d_h, d_w, head_dim);
  if (!(theta > 0.f) || !std::isfinite(theta)) return fail(WF_E_SHAPE, "%s: theta must be positive", who);
  if ((long long)frames_per_chunk * grid_h * grid_w > (1 << 20))
    return fail(WF_E_SHAPE, "%s: chunk larger than 2^20 tokens", who);
  t = RopeTable{};
  const int seg[3] = {d_t, d_h, d_w};
  int p = 0;
  for (int a = 0; a < 3; ++a)
    for (int i = 0; i < seg[a] / 2; ++i, ++p) {
      t.inv_freq[p] = (float)std::pow((double)theta, -2.0 * i / seg[a]);
      t.axis[p] = a;
    }
  return WF_OK;
}

// Frame positions of chunks first .. first + n_chunks - 1 must be exact fp32 integers.
static int rope_positions_ok(int frames_per_chunk, long long first, long long n_chunks, const char* who) {
  if (first < 0) return fail(WF_E_SHAPE, "%s: negative chunk index", who);
  if ((double)frames_per_chunk * (first + n_chunks + 1) > 16777216.0)
    return fail(WF_E_SHAPE, "%s: frame positions exceed the exact fp32 integer range", who);
  return WF_OK;
}

WF_EXPORT int wf_rope3d(void* x, int n_tokens, int n_heads, int head_dim, int dtype, int first_global_chunk,
                        int frames_per_chunk, int grid_h, int grid_w, int d_t, int d_h, int d_w,
                        float theta, void* stream) {
  const char* who = "wf_rope3d";
  if (!x) return fail(WF_E_NULL, "wf_rope3d: NULL x");
  if (!aligned(x, 16)) return fail(WF_E_SHAPE, "wf_rope3d: x must be 16-byte aligned");
  if (dtype_size(dtype) == 0) return fail(WF_E_DTYPE, "wf_rope3d: unknown dtype %d", dtype);
  if (n_heads < 1 || n_tokens < 0) return fail(WF_E_SHAPE, "wf_rope3d: non-positive size");
  // one thread per token and 8-element group: the launch stays below 2^32 work-items
  if (n_tokens > (1 << 27)) return fail(WF_E_SHAPE, "wf_rope3d: n_tokens %d above 2^27", n_tokens);
  RopeTable t;
  int st = rope_table(head_dim, frames_per_chunk, grid_h, grid_w, d_t, d_h, d_w, theta, t, who);
  if (st != WF_OK) return st;
  const long long chunk = (long long)frames_per_chunk * grid_h * grid_w;
  if (n_tokens % chunk)
    return fail(WF_E_SHAPE, "wf_rope3d: n_tokens %d is not a multiple of the chunk (%lld)", n_tokens, chunk);
  st = rope_positions_ok(frames_per_chunk, first_global_chunk, n_tokens / chunk, who);
  if (st != WF_OK) return st;
  if (n_tokens == 0) return ok();
  hipError_t e = launch_rope3d(x, n_tokens, n_heads, head_dim, dtype, first_global_chunk, frames_per_chunk,
                               grid_h, grid_w, t, static_cast<hipStream_t>(stream));
  return hip_status(e, "wf_rope3d");
}

WF_EXPORT int wf_kv_set_rope(wf_kv_cache* kv, int frames_per_chunk, int grid_h, int grid_w, int d_t, int d_h,
                             int d_w, float theta) {
  const char* who = "wf_kv_set_rope";
  if (!kv) return fail(WF_E_NULL, "wf_kv_set_rope: NULL cache");
  RopeTable t;
  const int st = rope_table(kv->head_dim, frames_per_chunk, grid_h, grid_w, d_t, d_h, d_w, theta, t, who);
  if (st != WF_OK) return st;
  if ((long long)frames_per_chunk * grid_h * grid_w != kv->chunk_tokens)
    return fail(WF_E_SHAPE, "wf_kv_set_rope: frames_per_chunk * grid_h * grid_w = %lld, chunk_tokens %d",
                (long long)frames_per_chunk * grid_h * grid_w, kv->chunk_tokens);
  kv->rope.on = true;
  kv->rope.fpc = frames_per_chunk;
  kv->rope.gh = grid_h;
  kv->rope.gw = grid_w;
  kv->rope.table = t;
  return ok();
}

static int rope_write_checks(const wf_kv_cache* kv, const void* k, const void* v, int global_chunk, const char* who) {
  if (!kv || !k || !v) return fail(WF_E_NULL, "%s: NULL argument", who);
  if (!aligned(k, 16) || !aligned(v, 16)) return fail(WF_E_SHAPE, "%s: k and v must be 16-byte aligned", who);
  if (!kv->rope.on) return fail(WF_E_UNSUPPORTED, "%s: no RoPE configured (wf_kv_set_rope)", who);
  return rope_positions_ok(kv->rope.fpc, global_chunk, 1, who);
}

WF_EXPORT int wf_kv_append_rope(wf_kv_cache* kv, const void* k, const void* v, int global_chunk, void* stream,
                                int* out_slot) {
  const char* who = "wf_kv_append_rope";
  int st = rope_write_checks(kv, k, v, global_chunk, who);
  if (st != WF_OK) return st;
  if (kv->free_slots.empty()) return fail(WF_E_FULL, "wf_kv_append_rope: no free slot (%d slots)", kv->n_slots);
  if ((int)kv->table.size() >= WF_MAX_TABLE)
    return fail(WF_E_FULL, "wf_kv_append_rope: table holds WF_MAX_TABLE entries");
  const int slot = kv->free_slots.front();
  hipError_t e = launch_kv_write_rope(*kv, slot, k, v, global_chunk, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, who);
  kv->free_slots.pop_front();
  kv->table.push_back(slot);
  if (out_slot) *out_slot = slot;
  return ok();
}

WF_EXPORT int wf_kv_refresh_rope(wf_kv_cache* kv, int logical_idx, const void* k, const void* v, int global_chunk,
                                 void* stream) {
  const char* who = "wf_kv_refresh_rope";
  int st = rope_write_checks(kv, k, v, global_chunk, who);
  if (st != WF_OK) return st;
  if (logical_idx < 0 || logical_idx >= (int)kv->table.size())
    return fail(WF_E_SLOT, "wf_kv_refresh_rope: logical index %d outside table of %zu", logical_idx,
                kv->table.size());
  hipError_t e =
      launch_kv_write_rope(*kv, kv->table[logical_idx], k, v, global_chunk, static_cast<hipStream_t>(stream));
  return hip_status(e, who);
}

static int fill_attn_params(const void* q, const wf_kv_cache* kv, int n_inflight, float scale, void* out,
                            float* lse, AttnParams& p, const char* who) {
  if (!q || !kv || !out) return fail(WF_E_NULL, "%s: NULL argument", who);
  if (n_inflight < 1) return fail(WF_E_SHAPE, "%s: n_inflight %d < 1", who, n_inflight);
  if ((int)kv->table.size() < n_inflight)
    return fail(WF_E_EMPTY, "%s: n_inflight %d exceeds table length %zu", who, n_inflight, kv->table.size());
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(WF_E_SHAPE, "%s: scale must be positive and finite", who);
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(WF_E_SHAPE, "%s: q and out must be 16-byte aligned", who);
  if (lse && !aligned(lse, 4)) return fail(WF_E_SHAPE, "%s: lse must be 4-byte aligned", who);
  const int st = check_attn_size(*kv, n_inflight, who);
  if (st != WF_OK) return st;
  std::memset(&p, 0, sizeof p);
  p.q = q;
  p.o = out;
  p.lse = lse;
  p.k_pool = kv->k_pool;
  p.v_pool = kv->v_pool;
  p.slot_elems = (long long)kv->slot_elems;
  p.n_heads = kv->n_heads;
  p.chunk_tokens = kv->chunk_tokens;
  p.s_pad = kv->s_pad;
  p.n_inflight = n_inflight;
  p.n_hist = (int)kv->table.size() - n_inflight;
  p.scale_log2e = scale * 1.4426950408889634f;
  p.scale = scale;
  for (size_t i = 0; i < kv->table.size(); ++i) p.slots[i] = kv->table[i];
  return ok();
}

WF_EXPORT int wf_chunk_causal_attn_fwd(const void* q, const wf_kv_cache* kv, int n_inflight, float scale,
                                       void* out, float* lse, void* stream) {
  AttnParams p;
  int st = fill_attn_params(q, kv, n_inflight, scale, out, lse, p, "wf_chunk_causal_attn_fwd");
  if (st != WF_OK) return st;
  return hip_status(launch_attn_fwd(*kv, p, nullptr, static_cast<hipStream_t>(stream)), "wf_chunk_causal_attn_fwd");
}

WF_EXPORT size_t wf_attn_fwd_workspace_bytes(const wf_kv_cache* kv) { return kv ? attn_split_bytes(*kv) : 0; }

WF_EXPORT int wf_chunk_causal_attn_fwd_ws(const void* q, const wf_kv_cache* kv, int n_inflight, float scale,
                                          void* workspace, void* out, float* lse, void* stream) {
  const char* who = "wf_chunk_causal_attn_fwd_ws";
  if (workspace && !aligned(workspace, 256)) return fail(WF_E_SHAPE, "%s: workspace must be 256-byte aligned", who);
  AttnParams p;
  int st = fill_attn_params(q, kv, n_inflight, scale, out, lse, p, who);
  if (st != WF_OK) return st;
  st = check_workspace_disjoint(*kv, n_inflight, workspace, attn_split_bytes(*kv), q, out, lse, who);
  if (st != WF_OK) return st;
  return hip_status(launch_attn_fwd(*kv, p, workspace, static_cast<hipStream_t>(stream)), who);
}

WF_EXPORT int wf_chunk_causal_attn_fwd_static(const void* q, const wf_kv_cache* kv, int n_inflight, float scale,
                                              void* out, float* lse, void* stream) {
  const char* who = "wf_chunk_causal_attn_fwd_static";
  AttnParams p;
  int st = fill_attn_params(q, kv, n_inflight, scale, out, lse, p, who);
  if (st != WF_OK) return st;
  const size_t need = attn_split_bytes(*kv);
  if (need > (size_t)WF_STATIC_SCRATCH_BYTES)
    return fail(WF_E_SHAPE, "%s: the key-split partials of this cache need %zu bytes, more than the %zu-byte static "
                "scratch (use wf_chunk_causal_attn_fwd_ws with a workspace)", who, need,
                (size_t)WF_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need) {
    const hipError_t e = static_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, who);
  }
  return hip_status(launch_attn_fwd(*kv, p, ws, static_cast<hipStream_t>(stream)), who);
}

WF_EXPORT size_t wf_attn_i8qk_workspace_bytes(const wf_kv_cache* kv, int n_inflight) {
  if (!kv || n_inflight < 1 || n_inflight > (int)kv->table.size()) return 0;
  if (kv->dtype != WF_BF16 || kv->head_dim != 128) return 0;
  return i8_layout(*kv, n_inflight).total;
}

WF_EXPORT int wf_chunk_causal_attn_fwd_i8qk(const void* q, const wf_kv_cache* kv, int n_inflight, float scale,
                                            void* workspace, void* out, float* lse, void* stream) {
  const char* who = "wf_chunk_causal_attn_fwd_i8qk";
  if (!workspace) return fail(WF_E_NULL, "%s: NULL workspace", who);
  if (kv && kv->dtype != WF_BF16) return fail(WF_E_DTYPE, "%s: needs a bf16 cache", who);
  if (kv && kv->head_dim != 128) return fail(WF_E_UNSUPPORTED, "%s: needs head_dim 128", who);
  if (!aligned(workspace, 256)) return fail(WF_E_SHAPE, "%s: workspace must be 256-byte aligned", who);
  if (kv && kv->table.size() * (size_t)((kv->chunk_tokens + 127) / 128) > 16384)
    return fail(WF_E_SHAPE, "%s: table length x 128-token blocks per chunk exceeds 16384", who);
  AttnParams p;
  int st = fill_attn_params(q, kv, n_inflight, scale, out, lse, p, who);
  if (st != WF_OK) return st;
  st = check_workspace_disjoint(*kv, n_inflight, workspace, i8_layout(*kv, n_inflight).total, q, out, lse, who);
  if (st != WF_OK) return st;
  return hip_status(launch_attn_fwd_i8qk(*kv, p, workspace, static_cast<hipStream_t>(stream)), who);
}

WF_EXPORT int wf_quant_rows_i8(const void* x, int rows, int cols, int dtype, void* codes, float* scales,
                               void* stream) {
  const char* who = "wf_quant_rows_i8";
  if (!x || !codes || !scales) return fail(WF_E_NULL, "%s: NULL argument", who);
  if (dtype != WF_BF16) return fail(WF_E_DTYPE, "%s: input must be WF_BF16", who);
  if (rows < 0 || rows > (1 << 24) || cols < 8 || cols % 8)
    return fail(WF_E_SHAPE, "%s: need rows in [0, 2^24] and cols a positive multiple of 8 (rows %d cols %d)", who, rows,
                cols);
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(scales, 4))
    return fail(WF_E_SHAPE, "%s: x must be 16-byte, codes 8-byte, scales 4-byte aligned", who);
  if (rows == 0) return ok();
  return hip_status(launch_quant_rows_i8(x, rows, cols, codes, scales, static_cast<hipStream_t>(stream)), who);
}

WF_EXPORT int wf_gemm_w8a8(const void* xq, const float* sx, const void* wq, const float* sw, const void* bias, int M,
                           int N, int K, int out_dtype, void* y, void* stream) {
  const char* who = "wf_gemm_w8a8";
  if (!xq || !wq || !y) return fail(WF_E_NULL, "%s: NULL argument", who);
  if (out_dtype != WF_BF16 && out_dtype != WF_I32) return fail(WF_E_DTYPE, "%s: out_dtype must be WF_BF16 or WF_I32", who);
  if (out_dtype == WF_BF16 && (!sx || !sw)) return fail(WF_E_NULL, "%s: NULL scales", who);
  if (M < 0 || N < 8 || N % 8 || K < 64 || K % 64 || K > 131072)
    return fail(WF_E_SHAPE, "%s: need N a positive multiple of 8, K a multiple of 64 in [64, 131072] (M %d N %d K %d)",
                who, M, N, K);
  // one workgroup per 256 x 256 output tile; the grid stays below 2^22 workgroups
  if ((size_t)((M + 255) / 256) * (size_t)((N + 255) / 256) > ((size_t)1 << 22))
    return fail(WF_E_SHAPE, "%s: M x N too large (more than 2^22 tiles of 256 x 256)", who);
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(y, 16) || (sx && !aligned(sx, 4)) || (sw && !aligned(sw, 4)) ||
      (bias && !aligned(bias, 2)))
    return fail(WF_E_SHAPE, "%s: xq, wq, y must be 16-byte aligned", who);
  if (M == 0) return ok();
  return hip_status(launch_gemm_w8a8(xq, sx, wq, sw, bias, M, N, K, out_dtype == WF_I32, y,
                                     static_cast<hipStream_t>(stream)), who);
}

WF_EXPORT const char* wf_status_str(int status) {
  switch (status) {
    case WF_OK: return "WF_OK";
    case WF_E_NULL: return "WF_E_NULL: NULL pointer argument";
    case WF_E_SHAPE: return "WF_E_SHAPE: size out of range or inconsistent";
    case WF_E_DTYPE: return "WF_E_DTYPE: unsupported element type";
    case WF_E_SLOT: return "WF_E_SLOT: bad slot or logical index";
    case WF_E_FULL: return "WF_E_FULL: no free slot";
    case WF_E_EMPTY: return "WF_E_EMPTY: too few table entries";
    case WF_E_UNSUPPORTED: return "WF_E_UNSUPPORTED: unsupported configuration";
    case WF_E_HIP: return "WF_E_HIP: HIP launch failure";
    default: return "unknown status";
  }
}

WF_EXPORT const char* wf_last_error(void) { return g_last_error.c_str(); }

WF_EXPORT int wf_version(void) { return 100; }  // 0.1.0

WF_EXPORT int wf_device_peak_info(int device, int* n_cu, int* peak_clock_khz) {
  const char* who = "wf_device_peak_info";
  if (!n_cu || !peak_clock_khz) return fail(WF_E_NULL, "%s: NULL argument", who);
  hipError_t e = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(peak_clock_khz, hipDeviceAttributeClockRate, device);
  return hip_status(e, who);
}
