// 3D rotary embedding over (frame, row, column), in place on [tokens][H][D].
// The pages do not describe positional encoding; the convention (segment
// split, interleaved pairs, theta, token order inside a chunk of 3 latent
// frames of the 30x52 latent grid) is the one documented in include/wf.h.
//
// One thread owns 4 consecutive pairs (8 elements) of one token and applies
// the same 4 rotations to that token's row in every head, so each sin/cos is
// evaluated once per token rather than once per head. HBM-bound.
#include "rope_common.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec8 {
  T v[8];
};

template <typename T>
__device__ __forceinline__ Vec8<T> load8(const T* p) {
  Vec8<T> r;
  constexpr int N16 = 8 * sizeof(T) / 16;  // 1 for bf16, 2 for fp32
  u32x4 raw[N16];
#pragma unroll
  for (int i = 0; i < N16; ++i) raw[i] = reinterpret_cast<const u32x4*>(p)[i];
  __builtin_memcpy(r.v, raw, sizeof r.v);
  return r;
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const Vec8<T>& r) {
  constexpr int N16 = 8 * sizeof(T) / 16;
  u32x4 raw[N16];
  __builtin_memcpy(raw, r.v, sizeof r.v);
#pragma unroll
  for (int i = 0; i < N16; ++i) reinterpret_cast<u32x4*>(p)[i] = raw[i];
}

template <typename T, int D>
__global__ __launch_bounds__(256) void rope3d_kernel(T* __restrict__ x, int n_tokens, int H, int first_chunk,
                                                     int fpc, int gh, int gw, wf::RopeTable tab) {
  constexpr int GROUPS = D / 8;  // 8-element groups per head row
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)n_tokens * GROUPS) return;
  const int t = (int)(gid / GROUPS);
  const int grp = (int)(gid - (long long)t * GROUPS);
  const int chunk = fpc * gh * gw;
  float pos[3];
  wf::rope_token_pos(first_chunk + t / chunk, t % chunk, fpc, gh, gw, pos);
  float cs[4], sn[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) wf::rope_sincos(pos, tab, grp * 4 + k, sn[k], cs[k]);
  T* row = x + (size_t)t * H * D + grp * 8;
  for (int h = 0; h < H; ++h, row += D) {
    Vec8<T> a = load8(row);
#pragma unroll
    for (int k = 0; k < 4; ++k) wf::rope_rotate_pair(a.v[2 * k], a.v[2 * k + 1], cs[k], sn[k]);
    store8(row, a);
  }
}

template <typename T>
hipError_t launch_typed(void* x, int n_tokens, int H, int D, int first_chunk, int fpc, int gh, int gw,
                        const wf::RopeTable& tab, hipStream_t s) {
  const long long threads = (long long)n_tokens * (D / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (D == 128)
    rope3d_kernel<T, 128><<<blocks, 256, 0, s>>>(static_cast<T*>(x), n_tokens, H, first_chunk, fpc, gh, gw, tab);
  else
    rope3d_kernel<T, 64><<<blocks, 256, 0, s>>>(static_cast<T*>(x), n_tokens, H, first_chunk, fpc, gh, gw, tab);
  return hipGetLastError();
}

}  // namespace

namespace wf {

hipError_t launch_rope3d(void* x, int n_tokens, int n_heads, int head_dim, int dtype, int first_global_chunk,
                         int frames_per_chunk, int grid_h, int grid_w, const RopeTable& table, hipStream_t s) {
  if (dtype == WF_BF16)
    return launch_typed<__bf16>(x, n_tokens, n_heads, head_dim, first_global_chunk, frames_per_chunk, grid_h,
                                grid_w, table, s);
  return launch_typed<float>(x, n_tokens, n_heads, head_dim, first_global_chunk, frames_per_chunk, grid_h,
                             grid_w, table, s);
}

}  // namespace wf
