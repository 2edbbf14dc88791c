// W8A8 linear: per-row int8 quantization of activations / weights, and the
// int8 x int8 -> int32 GEMM with a per-row x per-column scale epilogue. The
// pages name a W8A8 backend for the DiT linears around attention (Wave
// Forcing paper pages, Abstract) without its internals; the scheme is the
// one documented in include/wf.h.
//
// GEMM: Y[M][N] = s_x[m] s_w[n] sum_k Xq[m][k] Wq[n][k] (+ bias[n]),
// X and W both row-major with K contiguous.
//   * workgroup tile 256 x 256, 8 waves of 64 x 128 (2 x 4 MFMA tiles of
//     32 x 32), v_mfma_i32_32x32x32_i8;
//   * K advances 64 bytes per stage; three LDS stages of A and B (32 KB
//     each) filled by direct HBM -> LDS copies (global_load_lds_dwordx4)
//     two stages ahead;
//   * LDS tile rows are 64 bytes (four 16-byte pieces); piece p of row r sits
//     in slot p ^ ((r >> 2) & 3), so the 16 lanes of an MFMA operand read hit
//     16 different bank groups while each copy instruction still reads whole
//     64-byte row segments from HBM;
//   * epilogue in fp32: (float)acc * (s_x[m] * s_w[n]) + bias[n], rounded to
//     bf16, staged through LDS and stored as full 16-byte row pieces;
//   * XCD-contiguous tile order: each XCD gets one contiguous run of the
//     column-major tile order, i.e. a few weight tiles that stay in its L2.
#include <algorithm>

#include "wf_internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
#define LDS_AS __attribute__((address_space(3)))

// ---------------------------------------------------------------- row quantization
// One wave per row: s = amax / 127 (1 when amax = 0), code = clamp(rint(x / s), +-127),
// fp32 decisions with a correctly rounded division. cols % 8 == 0.
__global__ __launch_bounds__(256) void quant_rows_kernel(const __bf16* __restrict__ x, int rows, int cols,
                                                         signed char* __restrict__ q, float* __restrict__ scales) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const __bf16* xr = x + (size_t)row * cols;
  float amax = 0.f;
  for (int c = lane * 8; c < cols; c += 512) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(xr + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      amax = fmaxf(amax, fabsf(__uint_as_float(raw[e] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(raw[e] & 0xffff0000u)));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float s = amax > 0.f ? amax / 127.0f : 1.0f;
  if (lane == 0) scales[row] = s;
  signed char* qr = q + (size_t)row * cols;
  for (int c = lane * 8; c < cols; c += 512) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(xr + c);
    unsigned w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned bits = (e & 1) ? (raw[e >> 1] & 0xffff0000u) : (raw[e >> 1] << 16);
      const float v = rintf(__uint_as_float(bits) / s);
      const int code = (int)fminf(fmaxf(v, -127.f), 127.f);
      w[e >> 2] |= (unsigned)(code & 0xff) << (8 * (e & 3));
    }
    *reinterpret_cast<uint2*>(qr + c) = uint2{w[0], w[1]};
  }
}

// ---------------------------------------------------------------- GEMM
constexpr int BM = 256, BN = 256, BK = 64;  // BK in bytes (= int8 elements)
constexpr int NWV = 8;                      // waves: 4 along M x 2 along N
constexpr int NST = 3;                      // LDS stages
constexpr int TILE_A = BM * BK, TILE_B = BN * BK;
constexpr int STAGE = TILE_A + TILE_B;
constexpr int LDS_MAIN = NST * STAGE;                 // 96 KB
constexpr int LDS_OUT = BM * BN * 2;                  // bf16 output staging, 128 KB
constexpr int LDS_BYTES = LDS_OUT > LDS_MAIN ? LDS_OUT : LDS_MAIN;

extern __shared__ __attribute__((aligned(1024))) char g_lds[];

__device__ __forceinline__ int slot_of(int r, int p) { return p ^ ((r >> 2) & 3); }

// Copies the 64-byte K slice [k0, k0+64) of 256 consecutive rows (row0 ..) of a
// row-major int8 matrix into an LDS tile image: wave w issues instructions w
// and w + 8 of 16; instruction j covers rows 16j .. 16j+15, lane i the piece
// (i % 4) ^ ((row >> 2) & 3) of row 16j + i / 4. Rows past `rows` repeat the last row.
__device__ __forceinline__ void copy_rows(const signed char* src, int rows, int row0, int K, int k0, char* lds,
                                          int wave, int lane) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = wave + u * NWV;
    const int r = 16 * j + (lane >> 2);
    const int p = slot_of(r, lane & 3);
    const int gr = min(row0 + r, rows - 1);
    __builtin_amdgcn_global_load_lds(src + (size_t)gr * K + k0 + p * 16, (LDS_AS void*)(lds + j * 1024), 16, 0, 0);
  }
}

#define WF_W8_WAIT_VM_BARRIER(n) asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)\n\ts_barrier" ::: "memory")

// XCD-contiguous order: workgroup b runs on XCD b % 8; XCD x takes the x-th
// contiguous run of the column-major tile order (tile row fastest).
__device__ __forceinline__ void tile_of(int b, int tm_count, int total, int& tm, int& tn) {
  const int q = total / 8, rem = total % 8;
  const int x = b % 8, i = b / 8;
  const int item = x * q + min(x, rem) + i;
  tm = item % tm_count;
  tn = item / tm_count;
}

template <bool OUT_I32>
__global__ __launch_bounds__(NWV * 64) void gemm_w8a8_kernel(const signed char* __restrict__ xq,
                                                             const float* __restrict__ sx,
                                                             const signed char* __restrict__ wq,
                                                             const float* __restrict__ sw,
                                                             const __bf16* __restrict__ bias, int M, int N, int K,
                                                             void* __restrict__ y) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_m * tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;  // wave tile: rows wm*64 .. +64, cols wn*128 .. +128
  const int rr = lane & 31, hh = lane >> 5;
  char* lds = g_lds;
  auto stA = [&](int s) { return lds + s * STAGE; };
  auto stB = [&](int s) { return lds + s * STAGE + TILE_A; };
  const int KT = K / BK;

  auto copy_stage = [&](int kt, int s) {
    copy_rows(xq, M, m0, K, kt * BK, stA(s), wave, lane);
    copy_rows(wq, N, n0, K, kt * BK, stB(s), wave, lane);
  };
  copy_stage(0, 0);
  if (KT > 1) copy_stage(1, 1);
  WF_W8_WAIT_VM_BARRIER(0);

  i32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // per-lane LDS offsets of the operand rows (row index fixed per lane; the piece varies)
  int aoff[2][4], boff[4][4];  // [block][piece]
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wm * 64 + 32 * i + rr;
#pragma unroll
    for (int p = 0; p < 4; ++p) aoff[i][p] = r * 64 + 16 * slot_of(r, p);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wn * 128 + 32 * j + rr;
#pragma unroll
    for (int p = 0; p < 4; ++p) boff[j][p] = r * 64 + 16 * slot_of(r, p);
  }

  for (int kt = 0, s = 0; kt < KT; ++kt, s = s == NST - 1 ? 0 : s + 1) {
    const char* a = stA(s);
    const char* b = stB(s);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {  // two k32 steps per stage
      const int p = 2 * ks + hh;
      i32x4 av[2], bv[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) av[i] = *reinterpret_cast<const i32x4*>(a + aoff[i][p]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = *reinterpret_cast<const i32x4*>(b + boff[j][p]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    // copies of stage kt+2 into the stage read in step kt-1, then wait for stage kt+1
    if (kt + 2 < KT) {
      const int s2 = s == 0 ? 2 : s - 1;
      copy_stage(kt + 2, s2);
      WF_W8_WAIT_VM_BARRIER(4);
    } else {
      WF_W8_WAIT_VM_BARRIER(0);
    }
  }

  // accumulator element e of lane l in tile (i, j): row 8*(e/4) + 4*hh + e%4, column rr
  if constexpr (OUT_I32) {
    int* yo = static_cast<int*>(y);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 128 + 32 * j + rr;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (m < M && n < N) yo[(size_t)m * N + n] = acc[i][j][e];
        }
      }
    return;
  }
  // fp32 epilogue into the bf16 LDS staging tile [BM][BN] (the stages are no longer read)
  __bf16* out_lds = reinterpret_cast<__bf16*>(lds);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int cl = wn * 128 + 32 * j + rr;
    const int n = min(n0 + cl, N - 1);
    const float swn = sw[n];
    const float bn = bias ? (float)bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rl = wm * 64 + 32 * i + 8 * (e >> 2) + 4 * hh + (e & 3);
        const float sxm = sx[min(m0 + rl, M - 1)];
        out_lds[rl * BN + cl] = (__bf16)fmaf((float)acc[i][j][e], sxm * swn, bn);
      }
  }
  __syncthreads();
  // coalesced stores: 16-byte pieces (8 columns) of each row
  __bf16* yo = static_cast<__bf16*>(y);
  constexpr int PIECES = BM * BN / 8;
  for (int idx = tid; idx < PIECES; idx += NWV * 64) {
    const int rl = idx / (BN / 8), cp = idx % (BN / 8);
    const int m = m0 + rl, n = n0 + cp * 8;
    if (m < M && n < N)
      *reinterpret_cast<u32x4*>(yo + (size_t)m * N + n) = *reinterpret_cast<const u32x4*>(out_lds + rl * BN + cp * 8);
  }
}

}  // namespace

namespace wf {

hipError_t launch_quant_rows_i8(const void* x, int rows, int cols, void* q, float* scales, hipStream_t s) {
  quant_rows_kernel<<<(rows + 3) / 4, 256, 0, s>>>(static_cast<const __bf16*>(x), rows, cols,
                                                    static_cast<signed char*>(q), scales);
  return hipGetLastError();
}

hipError_t launch_gemm_w8a8(const void* xq, const float* sx, const void* wq, const float* sw, const void* bias, int M,
                            int N, int K, bool out_i32, void* y, hipStream_t s) {
  const int blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  auto run = [&](auto kern) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       LDS_BYTES);
    if (e != hipSuccess) return e;
    kern<<<blocks, NWV * 64, LDS_BYTES, s>>>(static_cast<const signed char*>(xq), sx,
                                              static_cast<const signed char*>(wq), sw,
                                              static_cast<const __bf16*>(bias), M, N, K, y);
    return hipGetLastError();
  };
  return out_i32 ? run(gemm_w8a8_kernel<true>) : run(gemm_w8a8_kernel<false>);
}

}  // namespace wf
