// int8-QK variant of the round's attention: quantization of K and Q into the
// caller's workspace. The scheme (include/wf.h): one per-(head, channel) key
// mean over the keys every query chunk sees, the history chunks and in-flight
// chunk 0 (float64 sum, rounded once to fp32), so that no chunk's codes depend
// on a later chunk (chunk-wise causal attention, Abstract);
// Q and K - mean cut per head into 128-token blocks that start at every chunk
// start; per block s = amax / 127 (1 when amax = 0) and code =
// clamp(round_half_even(x / s), -127, 127), every decision in fp32 with a
// correctly rounded division. The pages name a quantized-QK backend
// (SageAttention) for their DiT-only tests (Wave Forcing paper pages,
// Abstract) without its internals; this is one concrete scheme.
//
// Workspace layout (all offsets 256-byte aligned), n_tab = table length,
// n_mean = n_hist + 1 (the chunks the key mean is taken over):
//   partial  f64  [n_mean][KQ][H][D]   key sums of each quarter of a chunk's key tiles
//   mean     f32  [H][D]
//   k_codes  i8   [n_tab][H][tiles][D/16][64][16]   LDS images of 64-key tiles, logical order
//   k_scales f32  [H][n_tab][nb]       nb = ceil(C / 128)
//   q_codes  i8   [N*C][H][D]
//   q_scales f32  [H][N][nb]
//   qm       f32  [H][N*C]             <q^_i, mean_h> for the LSE of the unshifted keys
#include <cmath>

#include "wf_internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int QB = 128;  // quantization block (tokens)
constexpr int KQ = 4;    // parts of a chunk's key tiles summed by separate workgroups

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float block_max(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = x;
  __syncthreads();
  float m = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  return m;
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4& raw, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(raw[e] << 16);
    x[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
  }
}

__device__ __forceinline__ int quant_code(float x, float s) {
  const float c = rintf(x / s);  // correctly rounded division, ties to even
  return (int)fminf(fmaxf(c, -127.f), 127.f);
}

// Key sums (float64) of one quarter g of the key tiles of one (table position
// c, head h): grid (n_mean, H, KQ), c < n_mean = n_hist + 1. 256 threads = 4
// waves; wave w owns 16-byte pieces w, w+4, w+8, w+12 of every tile image (8
// dims each), lane r its key row r. Reduction order is fixed.
__global__ __launch_bounds__(256) void k_partial_kernel(wf::AttnParams p, double* partial) {
  constexpr int D = 128;
  const int c = blockIdx.x, h = blockIdx.y, g = blockIdx.z, H = p.n_heads, C = p.chunk_tokens;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t tile_bytes = 64 * D * 2;
  const char* img = static_cast<const char*>(p.k_pool) + (size_t)p.slots[c] * p.slot_elems * 2 +
                    (size_t)h * p.s_pad * D * 2;
  const int t0 = g * p.key_tiles / KQ, t1 = (g + 1) * p.key_tiles / KQ;
  double acc[4][8];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[m][e] = 0.0;
#pragma unroll 4
  for (int t = t0; t < t1; ++t) {  // unrolled: the loads of four tiles in flight, adds in tile order
    const bool ok = t * 64 + lane < C;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int piece = wave + 4 * m;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(img + t * tile_bytes + piece * 1024 + lane * 16);
      float x[8];
      bf16x8_to_f32(raw, x);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ok) acc[m][e] += (double)x[e];
    }
  }
  double* out = partial + (((size_t)c * KQ + g) * H + h) * D;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double sm = wave_sum(acc[m][e]);
      if (lane == 0) out[(wave + 4 * m) * 8 + e] = sm;
    }
}

// Mean of the keys of the first n_mean table entries: fp64 sum of the key sums
// in table order, quarter by quarter, one rounding to fp32. Grid H, 128
// threads (one per dim).
__global__ __launch_bounds__(128) void key_mean_kernel(const double* partial, int n_mean, int H, long long nkeys,
                                                       float* mean) {
  const int h = blockIdx.x, d = threadIdx.x;
  double s = 0.0;
  for (int c = 0; c < n_mean; ++c)
    for (int g = 0; g < KQ; ++g) s += partial[(((size_t)c * KQ + g) * H + h) * 128 + d];
  mean[(size_t)h * 128 + d] = (float)(s / (double)nkeys);
}

__device__ __forceinline__ void load_mean(const float* mean, int h, float* mean_s) {
  for (int d = threadIdx.x; d < 128; d += blockDim.x) mean_s[d] = mean[(size_t)h * 128 + d];
  __syncthreads();
}

// K - mean quantized per 128-token block of one chunk: grid (nb, n_tab, H).
// The block's keys span two 64-key tile images; 256 threads each take 4
// (key row, 16 dims) pieces: two 16-byte bf16 pieces in, one 16-byte piece of
// codes out, so every load and store instruction of a wave covers 1 KB
// contiguously. Keys past C get code 0.
__global__ __launch_bounds__(256) void quant_k_kernel(wf::AttnParams p, const float* mean, signed char* kcodes,
                                                      float* kscales, int n_tab) {
  constexpr int D = 128;
  __shared__ float mean_s[D];
  __shared__ float red[4];
  const int b = blockIdx.x, c = blockIdx.y, h = blockIdx.z, H = p.n_heads, C = p.chunk_tokens;
  const int nb = (C + QB - 1) / QB;
  load_mean(mean, h, mean_s);
  const size_t tile_bytes = 64 * D * 2;
  const char* img = static_cast<const char*>(p.k_pool) + (size_t)p.slots[c] * p.slot_elems * 2 +
                    (size_t)h * p.s_pad * D * 2;
  // piece m of this thread: pos = tid + 256 m (m = 0..3) over 2 tiles x 8 code pieces x 64 rows;
  // code piece q of a row = dims 16q .. 16q+15 = bf16 pieces 2q and 2q+1
  float xs[4][16];
  float amax = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int pos = threadIdx.x + 256 * m;  // 0..1023
    const int tl = pos >> 9, q = (pos >> 6) & 7, row = pos & 63;
    const int t = b * 2 + tl;  // tile inside the chunk
    const int key = t * 64 + row;
    const bool ok = key < C && key < (b + 1) * QB;
#pragma unroll
    for (int e = 0; e < 16; ++e) xs[m][e] = 0.f;
    if (ok) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x4 raw =
            *reinterpret_cast<const u32x4*>(img + (size_t)t * tile_bytes + (2 * q + hf) * 1024 + row * 16);
        float x[8];
        bf16x8_to_f32(raw, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xs[m][8 * hf + e] = x[e] - mean_s[16 * q + 8 * hf + e];
          amax = fmaxf(amax, fabsf(xs[m][8 * hf + e]));
        }
      }
    }
  }
  amax = block_max(amax, red);
  const float s = amax > 0.f ? amax / 127.0f : 1.0f;
  if (threadIdx.x == 0) kscales[((size_t)h * n_tab + c) * nb + b] = s;
  // int8 image of tile t: [8 pieces of 16 dims][64 rows][16 B]
  const int tiles = p.s_pad / 64;
  signed char* out = kcodes + (((size_t)c * H + h) * tiles) * (64 * D);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int pos = threadIdx.x + 256 * m;
    const int tl = pos >> 9, q = (pos >> 6) & 7, row = pos & 63;
    const int t = b * 2 + tl;
    if (t >= tiles) continue;
    const int key = t * 64 + row;
    const bool ok = key < C && key < (b + 1) * QB;
    unsigned w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const unsigned code = ok ? (unsigned)(quant_code(xs[m][e], s) & 0xff) : 0u;
      w[e >> 2] |= code << (8 * (e & 3));
    }
    *reinterpret_cast<u32x4*>(out + (size_t)t * (64 * D) + q * 1024 + row * 16) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Q quantized per 128-token block of one in-flight chunk: grid (nb, N, H).
// Thread i takes query row i/2 of the block and half (i%2) of head_dim.
__global__ __launch_bounds__(256) void quant_q_kernel(wf::AttnParams p, const float* mean, signed char* qcodes,
                                                      float* qscales, float* qm) {
  constexpr int D = 128;
  __shared__ float mean_s[D];
  __shared__ float red[4];
  const int b = blockIdx.x, j = blockIdx.y, h = blockIdx.z, H = p.n_heads, C = p.chunk_tokens;
  const int nb = (C + QB - 1) / QB;
  load_mean(mean, h, mean_s);
  const int r = b * QB + (threadIdx.x >> 1), half = threadIdx.x & 1;
  const bool ok = r < C;
  const size_t row = (size_t)j * C + r;
  float x[64];
  float amax = 0.f;
  if (ok) {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(p.q) + (row * H + h) * D + half * 64);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float v[8];
      bf16x8_to_f32(src[k], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[8 * k + e] = v[e];
        amax = fmaxf(amax, fabsf(v[e]));
      }
    }
  }
  amax = block_max(amax, red);
  const float s = amax > 0.f ? amax / 127.0f : 1.0f;
  if (threadIdx.x == 0) qscales[((size_t)h * p.n_inflight + j) * nb + b] = s;
  if (!ok) return;
  float dotm = 0.f;
  unsigned words[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    unsigned w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int code = quant_code(x[4 * k + e], s);
      w |= (unsigned)(code & 0xff) << (8 * e);
      dotm = fmaf(s * (float)code, mean_s[half * 64 + 4 * k + e], dotm);
    }
    words[k] = w;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(qcodes + (row * H + h) * D + half * 64);
#pragma unroll
  for (int k = 0; k < 4; ++k) dst[k] = u32x4{words[4 * k], words[4 * k + 1], words[4 * k + 2], words[4 * k + 3]};
  const float other = __shfl_xor(dotm, 1);
  if (half == 0) qm[(size_t)h * p.n_inflight * C + row] = dotm + other;
}

}  // namespace

namespace wf {

I8Layout i8_layout(const wf_kv_cache& kv, int n_inflight) {
  I8Layout L{};
  const int n_tab = (int)kv.table.size();
  const size_t H = kv.n_heads, D = kv.head_dim, C = kv.chunk_tokens;
  L.blocks_per_chunk = (int)((C + QB - 1) / QB);
  size_t off = 0;
  const int n_mean = n_tab - n_inflight + 1;  // history + in-flight chunk 0
  L.partial = off;
  off = align256(off + (size_t)n_mean * KQ * H * D * sizeof(double));
  L.mean = off;
  off = align256(off + H * D * sizeof(float));
  L.k_codes = off;
  off = align256(off + (size_t)n_tab * H * kv.s_pad * D);
  L.k_scales = off;
  off = align256(off + (size_t)n_tab * H * L.blocks_per_chunk * sizeof(float));
  L.q_codes = off;
  off = align256(off + (size_t)n_inflight * C * H * D);
  L.q_scales = off;
  off = align256(off + H * n_inflight * L.blocks_per_chunk * sizeof(float));
  L.qm = off;
  off = align256(off + H * n_inflight * C * sizeof(float));
  L.total = off;
  return L;
}

hipError_t launch_quant_i8(const wf_kv_cache& kv, AttnParams& p, void* workspace, hipStream_t s) {
  const I8Layout L = i8_layout(kv, p.n_inflight);
  char* ws = static_cast<char*>(workspace);
  const int n_tab = (int)kv.table.size();
  p.key_tiles = (kv.chunk_tokens + 63) / 64;
  p.q_blocks = L.blocks_per_chunk;
  p.q_codes = reinterpret_cast<const signed char*>(ws + L.q_codes);
  p.q_scales = reinterpret_cast<const float*>(ws + L.q_scales);
  p.k_codes = reinterpret_cast<const signed char*>(ws + L.k_codes);
  p.k_scales = reinterpret_cast<const float*>(ws + L.k_scales);
  p.qm = reinterpret_cast<const float*>(ws + L.qm);
  double* partial = reinterpret_cast<double*>(ws + L.partial);
  const int n_mean = p.n_hist + 1;  // the key mean covers history + in-flight chunk 0
  k_partial_kernel<<<dim3(n_mean, kv.n_heads, KQ), 256, 0, s>>>(p, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* mean = reinterpret_cast<float*>(ws + L.mean);
  key_mean_kernel<<<kv.n_heads, 128, 0, s>>>(partial, n_mean, kv.n_heads, (long long)n_mean * kv.chunk_tokens,
                                             mean);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  quant_k_kernel<<<dim3(L.blocks_per_chunk, n_tab, kv.n_heads), 256, 0, s>>>(
      p, mean, reinterpret_cast<signed char*>(ws + L.k_codes), reinterpret_cast<float*>(ws + L.k_scales), n_tab);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  quant_q_kernel<<<dim3(L.blocks_per_chunk, p.n_inflight, kv.n_heads), 256, 0, s>>>(
      p, mean, reinterpret_cast<signed char*>(ws + L.q_codes), reinterpret_cast<float*>(ws + L.q_scales),
      reinterpret_cast<float*>(ws + L.qm));
  return hipGetLastError();
}

}  // namespace wf
