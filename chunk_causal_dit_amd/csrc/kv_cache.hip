// History-cache writes: zero fill of the pools, and the copy of one chunk's
// K/V into a ring slot (append and cache refresh write the same way; the
// cache-refresh stage is described in the Wave Forcing paper pages, Abstract).
//
// Slot layout (per pool, per slot):  K [H][S_pad][D]   V [H][D][S_pad]
// Sources are token-major [C][H][D]. Both kernels are HBM-bound copies.
#include "wf_internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void fill_zero_kernel(u32x4* p, size_t n16) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = z;
}

// K: every (token, head) row of D elements is one contiguous run on both sides.
// One thread per 16-byte piece; consecutive threads read consecutive bytes.
__global__ void k_rows_kernel(const u32x4* __restrict__ src, char* __restrict__ dst_slot, int C, int H,
                              int row_bytes, int s_pad) {
  const int per_row = row_bytes / 16;
  const size_t total = (size_t)C * H * per_row;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t row = i / per_row;  // = t*H + h
    const int piece = (int)(i - row * per_row);
    const int t = (int)(row / H), h = (int)(row - (size_t)t * H);
    u32x4* d = reinterpret_cast<u32x4*>(dst_slot + ((size_t)h * s_pad + t) * row_bytes) + piece;
    *d = src[i];
  }
}

// V: transpose a [64 tokens][D] tile of one head into D rows of 64 tokens.
// Tokens past C inside the last tile are written as zero (the padding).
template <typename T, int D>
__global__ __launch_bounds__(256) void v_transpose_kernel(const T* __restrict__ src, T* __restrict__ dst_slot,
                                                          int C, int H, int s_pad) {
  constexpr int TT = 64;               // tokens per tile
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte piece
  __shared__ T tile[TT][D + 2];        // +2 elements: column reads hit distinct banks
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * TT;
  // load: rows of D elements, 16 bytes per thread
  constexpr int PIECES = TT * D / EPC;
  for (int i = threadIdx.x; i < PIECES; i += blockDim.x) {
    const int r = i / (D / EPC), c = (i % (D / EPC)) * EPC;
    const int t = t0 + r;
    if (t < C) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(src + ((size_t)t * H + h) * D + c);
      T vals[EPC];
      __builtin_memcpy(vals, &raw, 16);
#pragma unroll
      for (int e = 0; e < EPC; ++e) tile[r][c + e] = vals[e];
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) tile[r][c + e] = T(0);
    }
  }
  __syncthreads();
  // store: D rows, TT tokens each, 16 bytes per thread
  constexpr int OUT_PIECES = D * TT / EPC;
  for (int i = threadIdx.x; i < OUT_PIECES; i += blockDim.x) {
    const int d = i / (TT / EPC), tc = (i % (TT / EPC)) * EPC;
    T vals[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) vals[e] = tile[tc + e][d];
    u32x4 raw;
    __builtin_memcpy(&raw, vals, 16);
    *reinterpret_cast<u32x4*>(dst_slot + ((size_t)h * D + d) * s_pad + t0 + tc) = raw;
  }
}

template <typename T>
hipError_t launch_v(const wf_kv_cache& kv, const void* v, void* vdst, hipStream_t s) {
  dim3 grid((kv.chunk_tokens + 63) / 64, kv.n_heads);
  if (kv.head_dim == 128)
    v_transpose_kernel<T, 128><<<grid, 256, 0, s>>>(static_cast<const T*>(v), static_cast<T*>(vdst),
                                                    kv.chunk_tokens, kv.n_heads, kv.s_pad);
  else
    v_transpose_kernel<T, 64><<<grid, 256, 0, s>>>(static_cast<const T*>(v), static_cast<T*>(vdst),
                                                   kv.chunk_tokens, kv.n_heads, kv.s_pad);
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
  const int row_bytes = kv.head_dim * (int)kv.esize;
  const size_t pieces = (size_t)kv.chunk_tokens * kv.n_heads * row_bytes / 16;
  const unsigned blocks = (unsigned)std::min<size_t>((pieces + 255) / 256, 16384);
  k_rows_kernel<<<blocks, 256, 0, s>>>(static_cast<const u32x4*>(k), kdst, kv.chunk_tokens, kv.n_heads,
                                       row_bytes, kv.s_pad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (kv.dtype == WF_BF16) return launch_v<__bf16>(kv, v, vdst, s);
  return launch_v<float>(kv, v, vdst, s);
}

}  // namespace wf
