// History-cache writes: zero fill of the pools, and the copy of one chunk's
// K/V into a ring slot (append and cache refresh write the same way; the
// cache-refresh stage is described in the Wave Forcing paper pages, Abstract).
//
// Slot layout. Each slot stores, per head, the chunk as a sequence of 64-key
// tiles, and each tile as the exact image the attention kernel copies into
// LDS, split into 16-byte pieces (E = elements per piece, 8 for bf16, 4 for fp32):
//   K tile image: [D/E pieces][64 keys][16 B]   piece p of key k = K[k][p*E .. p*E+E)
//   V tile image: [64/E pieces][D dims][16 B]   piece p of dim d = V[p*E .. p*E+E)[d]
// so slot bytes = H * S_pad * D * sizeof(T) for each pool, tiles in key order.
// A 64-key tile image is one contiguous block, which the attention kernel
// moves with direct global->LDS loads; inside LDS this piece-major order lets
// 16 lanes reading one piece of 16 different rows hit 16 different bank groups.
// Keys past C inside the last tile are zero.
//
// One workgroup handles one (64-token tile, head): it stages the tile's K and
// V rows in LDS (coalesced reads of the token-major source) and writes both
// images with fully coalesced 16-byte stores. HBM-bound.
//
// The fused write (append/refresh with RoPE) rotates K on its way into the
// slot, so rotated K never makes a round trip through HBM. One workgroup
// handles a slice of 256 / (pieces per row) tokens (16 for bf16 at head_dim
// 128) of a group of kRopeHeads heads: each thread owns one 16-byte piece
// position of a token row, starts the loads of that piece of K and V for
// every head of the group, computes the sin/cos of its pairs once (the angle
// depends on the token and the pair, not on the head), rotates each head's K
// pairs with them, and the slice is written through LDS as that key range of
// the tile images of each head.
#include "rope_common.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void fill_zero_kernel(u32x4* p, size_t n16) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = z;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void kv_tile_kernel(const T* __restrict__ ksrc, const T* __restrict__ vsrc,
                                                      char* __restrict__ kdst, char* __restrict__ vdst, int C, int H,
                                                      int s_pad) {
  constexpr int TT = 64;               // keys per tile
  constexpr int E = 16 / sizeof(T);    // elements per 16-byte piece
  constexpr int RB = D * sizeof(T);    // bytes per source row
  constexpr int KROW = RB + 16;        // LDS row pitch of the K tile (16-byte aligned, conflict-free)
  constexpr int VROW = D + 2;          // LDS row pitch (elements) of the V tile for column gathers
  __shared__ __attribute__((aligned(16))) char kt[TT * KROW];
  __shared__ T vt[TT][VROW];
  const int h = blockIdx.y;
  const int tile = blockIdx.x;
  const int t0 = tile * TT;

  constexpr int PIECES = TT * D / E;  // 16-byte pieces per tile and tensor
  for (int i = threadIdx.x; i < PIECES; i += blockDim.x) {
    const int r = i / (D / E), c = i % (D / E);
    const int t = t0 + r;
    u32x4 kr = {0u, 0u, 0u, 0u}, vr = {0u, 0u, 0u, 0u};
    if (t < C) {
      const size_t off = ((size_t)t * H + h) * D + c * E;
      kr = *reinterpret_cast<const u32x4*>(ksrc + off);
      vr = *reinterpret_cast<const u32x4*>(vsrc + off);
    }
    *reinterpret_cast<u32x4*>(kt + r * KROW + c * 16) = kr;
    T vals[E];
    __builtin_memcpy(vals, &vr, 16);
#pragma unroll
    for (int e = 0; e < E; ++e) vt[r][c * E + e] = vals[e];
  }
  __syncthreads();

  const size_t tile_off = (size_t)h * s_pad * RB + (size_t)tile * TT * RB;
  u32x4* kimg = reinterpret_cast<u32x4*>(kdst + tile_off);
  u32x4* vimg = reinterpret_cast<u32x4*>(vdst + tile_off);
  for (int i = threadIdx.x; i < PIECES; i += blockDim.x) {
    {  // K image position i = piece * 64 + key
      const int p = i / TT, r = i % TT;
      kimg[i] = *reinterpret_cast<const u32x4*>(kt + r * KROW + p * 16);
    }
    {  // V image position i = piece * D + dim
      const int p = i / D, d = i % D;
      T vals[E];
#pragma unroll
      for (int e = 0; e < E; ++e) vals[e] = vt[p * E + e][d];
      u32x4 raw;
      __builtin_memcpy(&raw, vals, 16);
      vimg[i] = raw;
    }
  }
}

// Heads per workgroup of the fused write: the sin/cos of a (token, pair) is
// computed once and used for this many heads (3-4 measured fastest).
constexpr int kRopeHeads = 4;

template <typename T, int D>
__global__ __launch_bounds__(256) void kv_rope_tile_kernel(const T* __restrict__ ksrc, const T* __restrict__ vsrc,
                                                           char* __restrict__ kdst, char* __restrict__ vdst, int C,
                                                           int H, int s_pad, int g, int fpc, int gh, int gw,
                                                           wf::RopeTable tab) {
  constexpr int E = 16 / sizeof(T);    // elements per 16-byte piece
  constexpr int PPR = D / E;           // pieces per token row
  constexpr int TG = 256 / PPR;        // tokens per workgroup: one piece per thread
  constexpr int PAIRS = E / 2;         // rotated pairs per piece
  constexpr int HG = kRopeHeads;
  constexpr int KROW = PPR * 16 + 16;  // LDS row pitch (bytes) of the K slice
  constexpr int VROW = D + 2;          // LDS row pitch (elements) of the V slice
  constexpr int TILE = 64 * D * (int)sizeof(T);
  static_assert(TG * PPR == 256 && 64 % TG == 0 && TG % E == 0, "tile slices must split evenly");
  __shared__ __attribute__((aligned(16))) char kt[HG][TG * KROW];
  __shared__ T vt[HG][TG][VROW];
  const int t0 = blockIdx.x * TG, h0 = blockIdx.y * HG;
  const int tile = t0 / 64, key0 = t0 % 64;
  const int tid = threadIdx.x;
  {  // load, rotate, stage: thread (row r, piece c) of every head of the group
    const int r = tid / PPR, c = tid % PPR;
    const int t = t0 + r;
    u32x4 kr[HG], vr[HG];
#pragma unroll
    for (int i = 0; i < HG; ++i) {
      kr[i] = u32x4{0u, 0u, 0u, 0u};
      vr[i] = u32x4{0u, 0u, 0u, 0u};
      if (t < C && h0 + i < H) {
        const size_t off = ((size_t)t * H + h0 + i) * D + c * E;
        kr[i] = *reinterpret_cast<const u32x4*>(ksrc + off);
        vr[i] = *reinterpret_cast<const u32x4*>(vsrc + off);
      }
    }
    if (t < C) {
      float pos[3], sn[PAIRS], cs[PAIRS];
      wf::rope_token_pos(g, t, fpc, gh, gw, pos);
#pragma unroll
      for (int k = 0; k < PAIRS; ++k) wf::rope_sincos(pos, tab, c * PAIRS + k, sn[k], cs[k]);
#pragma unroll
      for (int i = 0; i < HG; ++i) {
        T x[E];
        __builtin_memcpy(x, &kr[i], 16);
#pragma unroll
        for (int k = 0; k < PAIRS; ++k) wf::rope_rotate_pair(x[2 * k], x[2 * k + 1], cs[k], sn[k]);
        __builtin_memcpy(&kr[i], x, 16);
      }
    }
#pragma unroll
    for (int i = 0; i < HG; ++i) {
      *reinterpret_cast<u32x4*>(kt[i] + r * KROW + c * 16) = kr[i];
      T vals[E];
      __builtin_memcpy(vals, &vr[i], 16);
#pragma unroll
      for (int e = 0; e < E; ++e) vt[i][r][c * E + e] = vals[e];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < HG; ++i) {
    if (h0 + i >= H) break;
    const size_t tile_off = ((size_t)(h0 + i) * (s_pad / 64) + tile) * TILE;
    {  // K image: piece p, keys key0 .. key0+TG-1 (TG contiguous 16-byte rows)
      const int p = tid / TG, r = tid % TG;
      *reinterpret_cast<u32x4*>(kdst + tile_off + p * (64 * 16) + (key0 + r) * 16) =
          *reinterpret_cast<const u32x4*>(kt[i] + r * KROW + p * 16);
    }
    {  // V image: group of E keys (key0/E + grp), dim d
      const int grp = tid / D, d = tid % D;
      T vals[E];
#pragma unroll
      for (int e = 0; e < E; ++e) vals[e] = vt[i][grp * E + e][d];
      u32x4 raw;
      __builtin_memcpy(&raw, vals, 16);
      *reinterpret_cast<u32x4*>(vdst + tile_off + (key0 / E + grp) * (D * 16) + d * 16) = raw;
    }
  }
}

template <typename T>
hipError_t launch_rope_tiles(const wf_kv_cache& kv, const void* k, const void* v, char* kdst, char* vdst, int g,
                             hipStream_t s) {
  const int tg = 256 * 16 / (int)sizeof(T) / kv.head_dim;      // tokens per workgroup (as in the kernel)
  // slices up to the end of the last tile, by groups of kRopeHeads heads
  const dim3 grid((kv.chunk_tokens + 63) / 64 * (64 / tg), (kv.n_heads + kRopeHeads - 1) / kRopeHeads);
  const T* kp = static_cast<const T*>(k);
  const T* vp = static_cast<const T*>(v);
  const wf::RopeConfig& rc = kv.rope;
  if (kv.head_dim == 128)
    kv_rope_tile_kernel<T, 128><<<grid, 256, 0, s>>>(kp, vp, kdst, vdst, kv.chunk_tokens, kv.n_heads, kv.s_pad, g,
                                                        rc.fpc, rc.gh, rc.gw, rc.table);
  else
    kv_rope_tile_kernel<T, 64><<<grid, 256, 0, s>>>(kp, vp, kdst, vdst, kv.chunk_tokens, kv.n_heads, kv.s_pad, g,
                                                       rc.fpc, rc.gh, rc.gw, rc.table);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_tiles(const wf_kv_cache& kv, const void* k, const void* v, char* kdst, char* vdst, hipStream_t s) {
  dim3 grid((kv.chunk_tokens + 63) / 64, kv.n_heads);
  const T* kp = static_cast<const T*>(k);
  const T* vp = static_cast<const T*>(v);
  if (kv.head_dim == 128)
    kv_tile_kernel<T, 128><<<grid, 256, 0, s>>>(kp, vp, kdst, vdst, kv.chunk_tokens, kv.n_heads, kv.s_pad);
  else
    kv_tile_kernel<T, 64><<<grid, 256, 0, s>>>(kp, vp, kdst, vdst, kv.chunk_tokens, kv.n_heads, kv.s_pad);
  return hipGetLastError();
}

}  // namespace

namespace wf {

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n16 + 255) / 256, 8192);
  fill_zero_kernel<<<blocks, 256, 0, s>>>(static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_kv_write(const wf_kv_cache& kv, int slot, const void* k, const void* v, hipStream_t s) {
  const size_t slot_bytes = kv.slot_elems * kv.esize;
  char* kdst = static_cast<char*>(kv.k_pool) + (size_t)slot * slot_bytes;
  char* vdst = static_cast<char*>(kv.v_pool) + (size_t)slot * slot_bytes;
  if (kv.dtype == WF_BF16) return launch_tiles<__bf16>(kv, k, v, kdst, vdst, s);
  return launch_tiles<float>(kv, k, v, kdst, vdst, s);
}

hipError_t launch_kv_write_rope(const wf_kv_cache& kv, int slot, const void* k, const void* v, int global_chunk,
                                hipStream_t s) {
  const size_t slot_bytes = kv.slot_elems * kv.esize;
  char* kdst = static_cast<char*>(kv.k_pool) + (size_t)slot * slot_bytes;
  char* vdst = static_cast<char*>(kv.v_pool) + (size_t)slot * slot_bytes;
  if (kv.dtype == WF_BF16) return launch_rope_tiles<__bf16>(kv, k, v, kdst, vdst, global_chunk, s);
  return launch_rope_tiles<float>(kv, k, v, kdst, vdst, global_chunk, s);
}

}  // namespace wf
