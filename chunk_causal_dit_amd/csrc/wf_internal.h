// Internal declarations shared by the host glue (wf_api.cpp) and the kernel
// translation units (*.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <deque>
#include <vector>

#include "wf.h"

#define WF_EXPORT extern "C" __attribute__((visibility("default")))

namespace wf {
struct RopeTable {
  float inv_freq[64];  // per pair, rounded once to fp32
  int axis[64];        // 0 frame, 1 row, 2 column
};
// 3D RoPE applied to K by the fused cache writes (wf_kv_set_rope).
struct RopeConfig {
  bool on = false;
  int fpc = 0, gh = 0, gw = 0;
  RopeTable table{};
};
}  // namespace wf

struct wf_kv_cache {
  void* k_pool = nullptr;
  void* v_pool = nullptr;
  int n_slots = 0;
  int chunk_tokens = 0;
  int n_heads = 0;
  int head_dim = 0;
  int dtype = 0;
  int s_pad = 0;            // chunk_tokens rounded up to a multiple of 128
  size_t esize = 0;         // bytes per element
  size_t slot_elems = 0;    // n_heads * s_pad * head_dim elements per slot (each pool)
  std::vector<int> table;   // logical order, oldest first: physical slot ids
  std::deque<int> free_slots;
  wf::RopeConfig rope;      // set by wf_kv_set_rope
};

namespace wf {

constexpr int kSlotPadTokens = 128;

inline int pad_tokens(int c) { return (c + kSlotPadTokens - 1) / kSlotPadTokens * kSlotPadTokens; }
inline size_t dtype_size(int dtype) { return dtype == WF_F32 ? 4 : dtype == WF_BF16 ? 2 : 0; }

// Records the message in the thread-local error slot and returns code.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// WF_E_SHAPE (with the message) when an attention round of n_inflight chunks of
// this cache would not fit one launch; checked before any device work.
int check_attn_size(const wf_kv_cache& kv, int n_inflight, const char* who);
// WF_E_SHAPE when a workspace of ws_bytes (NULL: none) overlaps q, out, lse or a
// cache pool of an attention round of n_inflight chunks.
int check_workspace_disjoint(const wf_kv_cache& kv, int n_inflight, const void* ws, size_t ws_bytes, const void* q,
                             const void* out, const float* lse, const char* who);

// ---- kernel launchers (defined in the .hip files); each returns the launch status ----
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

hipError_t launch_kv_write(const wf_kv_cache& kv, int slot, const void* k, const void* v,
                           hipStream_t s);

hipError_t launch_kv_write_rope(const wf_kv_cache& kv, int slot, const void* k, const void* v, int global_chunk,
                                hipStream_t s);

hipError_t launch_rope3d(void* x, int n_tokens, int n_heads, int head_dim, int dtype,
                         int first_global_chunk, int frames_per_chunk, int grid_h, int grid_w,
                         const RopeTable& table, hipStream_t s);

// Arguments of the attention kernels, passed by value (the slot table of the
// visible chunks travels inside the launch, so later host edits never race).
struct AttnParams {
  const void* q;
  void* o;
  float* lse;
  const void* k_pool;
  const void* v_pool;
  long long slot_elems;
  int n_heads;
  int chunk_tokens;
  int s_pad;
  int n_inflight;
  int n_hist;
  int q_tiles;     // query tiles per chunk
  int key_tiles;   // key tiles per chunk
  float scale_log2e;
  float scale;
  // int8-QK path only (workspace arrays, see attn_i8qk.hip)
  const signed char* q_codes;  // [N*C][H][D]
  const float* q_scales;       // [H][N][q_blocks]
  const signed char* k_codes;  // [n_tab][H][key_tiles][64*D] tile images, logical order
  const float* k_scales;       // [H][n_tab][q_blocks]
  const float* qm;             // [H][N*C]
  int q_blocks;                // 128-token blocks per chunk
  // Key-range split of in-flight chunk 0 (bf16 path): with split set, each of its query
  // tiles runs as two workgroups over the two halves of its key tiles, which write
  // unnormalized partials to part_o [2][H][C][D] and their log2-domain row max and
  // weight sum to part_ml [2][H][C][2]; attn_combine_kernel merges them.
  int split;
  float* part_o;
  float* part_ml;
  int slots[WF_MAX_TABLE];  // physical slot of logical chunk c = 0..n_hist+n_inflight-1
};

// Device address of the current device's WF_STATIC_SCRATCH_BYTES-byte static scratch
// (looked up on the first call on each device, with that device current).
hipError_t static_scratch(void** ptr);
// workspace: NULL, or attn_split_bytes(kv) bytes (256-byte aligned) that enable the key split
hipError_t launch_attn_fwd(const wf_kv_cache& kv, AttnParams& prm, void* workspace, hipStream_t s);
// Bytes of the key-split partials of a bf16 cache (0 for fp32 caches, which never split).
size_t attn_split_bytes(const wf_kv_cache& kv);

// ---- W8A8 linear ----
hipError_t launch_quant_rows_i8(const void* x, int rows, int cols, void* q, float* scales, hipStream_t s);
hipError_t launch_gemm_w8a8(const void* xq, const float* sx, const void* wq, const float* sw, const void* bias, int M,
                            int N, int K, bool out_i32, void* y, hipStream_t s);
// Whether a W8A8 GEMM of this shape (K % 128 == 0) runs on 256 x 192 tiles instead of 256 x 256.
bool use_narrow_tiles(int M, int N);

// ---- int8-QK path ----
struct I8Layout {
  size_t q_codes, q_scales, k_codes, k_scales, mean, qm, partial, total;
  int blocks_per_chunk;
};
I8Layout i8_layout(const wf_kv_cache& kv, int n_inflight);
// Quantizes K - mean and Q into the workspace and fills prm's int8 fields.
hipError_t launch_quant_i8(const wf_kv_cache& kv, AttnParams& prm, void* workspace, hipStream_t s);
hipError_t launch_attn_fwd_i8qk(const wf_kv_cache& kv, AttnParams& prm, void* workspace, hipStream_t s);

}  // namespace wf
