// W8A8 linear: per-row int8 quantization of activations / weights, and the
// int8 x int8 -> int32 GEMM with a per-row x per-column scale epilogue. The
// pages name a W8A8 backend for the DiT linears around attention (Wave
// Forcing paper pages, Abstract) without its internals; the scheme is the
// one documented in include/wf.h.
//
// GEMM: Y[M][N] = s_x[m] s_w[n] sum_k Xq[m][k] Wq[n][k] (+ bias[n]),
// X and W both row-major with K contiguous.
//   * workgroup tile 256 x 256, 4 waves of 128 x 128 (4 x 4 MFMA tiles of
//     32 x 32), v_mfma_i32_32x32x32_i8, one wave per SIMD: the large wave
//     tile keeps LDS reads at 64 B/clk per CU at full MFMA rate (LDS serves
//     about 128 B/clk, and the HBM -> LDS copies take another 32);
//   * K advances 128 bytes per stage (K % 128 == 0; gemm_w8a8_k128_kernel)
//     through two 64 KB LDS stages of A and B, or 64 bytes per stage through
//     three 32 KB stages otherwise (gemm_w8a8_kernel), filled by direct
//     HBM -> LDS copies (global_load_lds_dwordx4); the operands of the next
//     k32 step are read into a second register set while the MFMAs of the
//     current one run, and the one barrier per stage sits before its last k32
//     step, where the stage's buffer is free to refill;
//   * LDS tile rows are 128 (64) bytes; piece p of row r sits in slot
//     p ^ ((r >> 1) & 7) (p ^ ((r >> 2) & 3)), so the 16 lanes of an MFMA
//     operand read hit 16 different bank groups while each copy instruction
//     still reads whole row segments from HBM;
//   * epilogue in fp32: (float)acc * (s_x[m] * s_w[n]) + bias[n], rounded to
//     bf16, staged through LDS (rows padded to 520 bytes: conflict-free 8-byte
//     writes) and stored as full 16-byte row pieces;
//   * XCD-aware tile order: each XCD gets one contiguous run of a banded
//     order (4 tile rows at a time), so the tiles it runs together share
//     operands in its L2.
#include <algorithm>
#include <type_traits>

#include "wf_internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
#define LDS_AS __attribute__((address_space(3)))

// ---------------------------------------------------------------- row quantization
// One wave per row: s = amax / 127 (1 when amax = 0), code = clamp(rint(x / s), +-127),
// fp32 decisions with a correctly rounded division. cols % 8 == 0. Rows of up to
// NP * 512 columns are read from HBM once and kept in registers (16-byte pieces,
// piece p of lane l at column 512 p + 8 l); NP is picked per launch from cols, so a
// short row holds few registers (and more waves fit); longer rows are read twice.
constexpr int RPIECES_MAX = 16;

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint2 quant_piece(const u32x4& raw, float s) {
  unsigned w[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = (e & 1) ? bf16_hi(raw[e >> 1]) : bf16_lo(raw[e >> 1]);
    const int code = (int)fminf(fmaxf(rintf(x / s), -127.f), 127.f);
    w[e >> 2] |= (unsigned)(code & 0xff) << (8 * (e & 3));
  }
  return uint2{w[0], w[1]};
}

__device__ __forceinline__ float piece_amax(const u32x4& raw, float amax) {
#pragma unroll
  for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(raw[e])), fabsf(bf16_hi(raw[e]))));
  return amax;
}

template <int RPIECES>
__global__ __launch_bounds__(256) void quant_rows_kernel(const __bf16* __restrict__ x, int rows, int cols,
                                                         signed char* __restrict__ q, float* __restrict__ scales) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const __bf16* xr = x + (size_t)row * cols;
  signed char* qr = q + (size_t)row * cols;
  u32x4 held[RPIECES];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < RPIECES; ++p) {
    const int c = p * 512 + lane * 8;
    held[p] = c < cols ? *reinterpret_cast<const u32x4*>(xr + c) : u32x4{0u, 0u, 0u, 0u};
    amax = piece_amax(held[p], amax);
  }
  for (int c = RPIECES * 512 + lane * 8; c < cols; c += 512)  // rows longer than the register set
    amax = piece_amax(*reinterpret_cast<const u32x4*>(xr + c), amax);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float s = amax > 0.f ? amax / 127.0f : 1.0f;
  if (lane == 0) scales[row] = s;
#pragma unroll
  for (int p = 0; p < RPIECES; ++p) {
    const int c = p * 512 + lane * 8;
    if (c < cols) *reinterpret_cast<uint2*>(qr + c) = quant_piece(held[p], s);
  }
  for (int c = RPIECES * 512 + lane * 8; c < cols; c += 512)
    *reinterpret_cast<uint2*>(qr + c) = quant_piece(*reinterpret_cast<const u32x4*>(xr + c), s);
}

// ---------------------------------------------------------------- GEMM
constexpr int BM = 256, BN = 256, BK = 64;  // BK in bytes (= int8 elements)
constexpr int NWV = 4;                      // waves: 2 along M x 2 along N, 128 x 128 each
constexpr int NST = 3;                      // LDS stages
constexpr int TILE_A = BM * BK, TILE_B = BN * BK;
constexpr int STAGE = TILE_A + TILE_B;      // 32 KB
constexpr int LDS_MAIN = NST * STAGE;
constexpr int LDS_OUT = BM * (BN + 4) * 2;  // bf16 staging of a 256 x 256 tile (see gemm_epilogue)
constexpr int LDS_BYTES = LDS_OUT > LDS_MAIN ? LDS_OUT : LDS_MAIN;
constexpr int COPIES = 2 * (BM / 16) / NWV;  // copy instructions per wave per stage (A and B)
static_assert(BM == BN, "copy_rows serves both operands");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");

extern __shared__ __attribute__((aligned(1024))) char g_lds[];

__device__ __forceinline__ int slot_of(int r, int p) { return p ^ ((r >> 2) & 3); }

// Copies the 64-byte K slice [k0, k0+64) of 256 consecutive rows (row0 ..) of a
// row-major int8 matrix into an LDS tile image: instruction j (0..15) covers
// rows 16j .. 16j+15, lane i the piece (i % 4) ^ ((row >> 2) & 3) of row
// 16j + i / 4; wave w issues instructions w, w+4, w+8, w+12. Rows past `rows`
// repeat the last row.
__device__ __forceinline__ void copy_row_piece(const signed char* src, int rows, int row0, int K, int k0, char* lds,
                                               int wave, int lane, int u) {
  const int j = wave + u * NWV;
  const int r = 16 * j + (lane >> 2);
  const int p = slot_of(r, lane & 3);
  const int gr = min(row0 + r, rows - 1);
  __builtin_amdgcn_global_load_lds(src + (size_t)gr * K + k0 + p * 16, (LDS_AS void*)(lds + j * 1024), 16, 0, 0);
}
__device__ __forceinline__ void copy_rows(const signed char* src, int rows, int row0, int K, int k0, char* lds,
                                          int wave, int lane) {
#pragma unroll
  for (int u = 0; u < BM / 16 / NWV; ++u) copy_row_piece(src, rows, row0, K, k0, lds, wave, lane, u);
}

// Waits until at most N copy instructions of this wave are in flight and all
// its LDS reads are done, then joins the workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 14) asm volatile("s_waitcnt vmcnt(14) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 24) asm volatile("s_waitcnt vmcnt(24) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else static_assert(N == 0, "unsupported wait count");
}

// Tile order: workgroup b runs on XCD b % 8, and XCD x takes the x-th contiguous
// run of the order. The order walks bands of 4 tile rows, column by column inside
// a band, so the 32 workgroups an XCD runs at once share 4 X tiles and about 8 W
// tiles in its L2, and a band's X rows stay there while its columns pass.
__device__ __forceinline__ void tile_of(int b, int tm_count, int tn_count, int& tm, int& tn) {
  constexpr int G = 4;
  const int total = tm_count * tn_count;
  const int q = total / 8, rem = total % 8;
  const int x = b % 8, i = b / 8;
  const int item = x * q + min(x, rem) + i;
  const int band = item / (G * tn_count), in = item % (G * tn_count);
  const int rows = min(G, tm_count - band * G);
  tm = band * G + in % rows;
  tn = in / rows;
}

// Epilogue of a 256 x TN tile held as acc[i][j] by 4 waves (2 x 2, each 128 x TN/2; layout
// as in the kernels below): the raw int32 accumulators, or the fp32 scale/bias step
// rounded to bf16, staged through LDS and stored as 16-byte row pieces. The tile's LDS
// stages must no longer be read when it starts.
template <bool OUT_I32, int TN>
__device__ __forceinline__ void gemm_epilogue(const i32x16 (&acc)[4][TN / 64], char* lds,
                                              const float* __restrict__ sx, const float* __restrict__ sw,
                                              const __bf16* __restrict__ bias, int M, int N, int m0, int n0, int wm,
                                              int wn, int rr, int hh, int tid, void* __restrict__ y) {
  constexpr int JB = TN / 64;     // 32-column blocks per wave
  constexpr int LD = TN + 4;      // staging row stride (elements): LD / 2 dwords is 2 mod 4, so the
                                  // 32 rows of one 8-byte write land on 32 different bank pairs
  static_assert((LD / 2) % 4 == 2, "staging stride");
  if constexpr (OUT_I32) {
    int* yo = static_cast<int*>(y);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 128 + 32 * i + rr;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * (TN / 2) + 32 * j + 8 * g + 4 * hh;
          if (n < N)
            *reinterpret_cast<i32x4*>(yo + (size_t)m * N + n) =
                i32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        }
    }
    return;
  }
  // fp32 epilogue into the bf16 staging tile [BM][LD] (the stages are no longer read)
  __bf16* out_lds = reinterpret_cast<__bf16*>(lds);
  float sxm[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sxm[i] = sx[min(m0 + wm * 128 + 32 * i + rr, M - 1)];
#pragma unroll
  for (int j = 0; j < JB; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int nl = wn * (TN / 2) + 32 * j + 8 * g + 4 * hh;
      float swn[4], bn[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int n = min(n0 + nl + c, N - 1);
        swn[c] = sw[n];
        bn[c] = bias ? (float)bias[n] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ml = wm * 128 + 32 * i + rr;
        __bf16 v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (__bf16)fmaf((float)acc[i][j][4 * g + c], sxm[i] * swn[c], bn[c]);
        *reinterpret_cast<uint2*>(out_lds + ml * LD + nl) = *reinterpret_cast<const uint2*>(v);
      }
    }
  __syncthreads();
  // coalesced stores: 16-byte pieces (8 columns) of each row
  __bf16* yo = static_cast<__bf16*>(y);
  constexpr int PIECES = BM * TN / 8;
#pragma unroll 4
  for (int idx = tid; idx < PIECES; idx += NWV * 64) {
    const int rl = idx / (TN / 8), cp = idx % (TN / 8);
    const int m = m0 + rl, n = n0 + cp * 8;
    if (m < M && n < N) {
      const uint2* src = reinterpret_cast<const uint2*>(out_lds + rl * LD + cp * 8);  // 8-byte aligned
      const uint2 lo = src[0], hi = src[1];
      *reinterpret_cast<u32x4*>(yo + (size_t)m * N + n) = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  }
}

template <bool OUT_I32>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w8a8_kernel(
    const signed char* __restrict__ xq, const float* __restrict__ sx, const signed char* __restrict__ wq,
    const float* __restrict__ sw, const __bf16* __restrict__ bias, int M, int N, int K, void* __restrict__ y) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // wave tile: rows wm*128 .. +128, cols wn*128 .. +128
  const int rr = lane & 31, hh = lane >> 5;
  char* lds = g_lds;
  const int KT = K / BK;

  auto copy_stage = [&](int kt, int s) {
    copy_rows(xq, M, m0, K, kt * BK, lds + s * STAGE, wave, lane);
    copy_rows(wq, N, n0, K, kt * BK, lds + s * STAGE + TILE_A, wave, lane);
  };

  // Operand rows of this lane: A row wm*128 + 32i + rr, B row wn*128 + 32j + rr. In k32 step
  // ks of a stage the lane takes piece 2ks + hh, stored in slot (2ks + hh) ^ ((rr >> 2) & 3);
  // block i (j) adds 32 rows = 2048 bytes.
  const int x = (rr >> 2) & 3;
  int aoff[2], boff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    aoff[ks] = (wm * 128 + rr) * 64 + 16 * ((2 * ks + hh) ^ x);
    boff[ks] = TILE_A + (wn * 128 + rr) * 64 + 16 * ((2 * ks + hh) ^ x);
  }
  i32x4 a0[4], b0[4], a1[4], b1[4];
  auto load_ops = [&](const char* st, int ks, i32x4(&av)[4], i32x4(&bv)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = *reinterpret_cast<const i32x4*>(st + aoff[ks] + 2048 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = *reinterpret_cast<const i32x4*>(st + boff[ks] + 2048 * j);
  };
  // acc[i][j]: D = Bblock_j x Ablock_i^T, so lane l holds m = 32i + (l % 32) and four runs of
  // four consecutive n: n = 32j + 8g + 4hh + (0..3) in elements 4g .. 4g+3
  i32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;
  auto mma = [&](const i32x4(&av)[4], const i32x4(&bv)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bv[j], av[i], acc[i][j], 0, 0, 0);
  };

  // prologue: every stage buffer in flight; wait for stage 0
#pragma unroll
  for (int st = 0; st < NST; ++st)
    if (st < KT) copy_stage(st, st);
  if (KT >= NST) wait_vm_barrier<COPIES * (NST - 1)>();
  else wait_vm_barrier<0>();
  load_ops(lds, 0, a0, b0);

  // One stage: reads of its second k32 step under the MFMAs of the first; then the barrier
  // (stage kt+1 has landed, every wave's reads of stage kt are done), the refill of the
  // buffer just read, and the reads of the next stage's first step under the second MFMAs.
  // The steady-state body has no branches, so the compiler's own waits before the MFMAs
  // count only the reads each MFMA needs.
  // Instruction order inside each half is pinned: MFMAs alternate with the reads (and
  // copies), so the matrix pipe never waits behind a run of memory instructions.
  auto body = [&](auto full, int kt, int s) {
    const int s1 = s == NST - 1 ? 0 : s + 1;
    __builtin_amdgcn_sched_barrier(0);
    load_ops(lds + s * STAGE, 1, a1, b1);
    mma(a0, b0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(full)::value) {
      wait_vm_barrier<COPIES * (NST - 2)>();
      __builtin_amdgcn_sched_barrier(0);
      // one MFMA per slot; after it the next stage's operand reads (needed first), then
      // the copies that refill this stage's buffer with stage kt + NST
      const char* nst = lds + s1 * STAGE;
      char* cst = lds + s * STAGE;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int i = t >> 2, j = t & 3;
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b1[j], a1[i], acc[i][j], 0, 0, 0);
        if (t < 4) a0[t] = *reinterpret_cast<const i32x4*>(nst + aoff[0] + 2048 * t);
        else if (t < 8) b0[t - 4] = *reinterpret_cast<const i32x4*>(nst + boff[0] + 2048 * (t - 4));
        else if (t < 12) copy_row_piece(xq, M, m0, K, (kt + NST) * BK, cst, wave, lane, t - 8);
        else copy_row_piece(wq, N, n0, K, (kt + NST) * BK, cst + TILE_A, wave, lane, t - 12);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      wait_vm_barrier<0>();
      if (kt + 1 < KT) load_ops(lds + s1 * STAGE, 0, a0, b0);
      mma(a1, b1);
    }
  };
  int kt = 0, s = 0;
  for (; kt + NST < KT; ++kt, s = s == NST - 1 ? 0 : s + 1) body(std::true_type{}, kt, s);
  for (; kt < KT; ++kt, s = s == NST - 1 ? 0 : s + 1) body(std::false_type{}, kt, s);
  __syncthreads();

  gemm_epilogue<OUT_I32, BN>(acc, lds, sx, sw, bias, M, N, m0, n0, wm, wn, rr, hh, tid, y);
}

// ---------------------------------------------------------------- GEMM, 128-byte K stages
// Same waves and epilogue as above, tiles 256 x TN (TN = 256 or 192: 4 waves of 128 x TN/2),
// with K advancing 128 bytes per stage through two LDS stages: one barrier per 16 TN/64
// MFMAs of a wave instead of per 32. LDS rows are 128 bytes (eight 16-byte pieces); piece p
// of row r sits in slot p ^ ((r >> 1) & 7), which keeps the 16 lanes of each operand read
// on 16 different bank groups. The 192-column tile is for shapes whose 256-column tiles
// leave the last wave of workgroups mostly empty (it is picked per launch).
constexpr int BK2 = 128;
constexpr int TILE_A2 = BM * BK2;
template <int TN>
struct K128 {
  static constexpr int JB = TN / 64;                  // 32-column MFMA blocks per wave
  static constexpr int TILE_B = TN * BK2;
  static constexpr int STAGE = TILE_A2 + TILE_B;      // 64 KB (256) or 56 KB (192)
  static constexpr int OUT = BM * (TN + 4) * 2;
  static constexpr int LDS = OUT > 2 * STAGE ? OUT : 2 * STAGE;
  static constexpr int BCOPY = TN / 8 / NWV;          // B copy instructions per wave per stage
  static_assert(LDS <= 160 * 1024, "LDS");
};

__device__ __forceinline__ int slot2_of(int r, int p) { return p ^ ((r >> 1) & 7); }

// Copy instruction j (0..31) of one operand covers rows 8j .. 8j+7 of the 128-byte K
// slice [k0, k0+128); lane i takes slot i % 8 of row 8j + i / 8, i.e. the piece
// slot2_of(row, i % 8). Wave w issues instructions w + 4u, u = 0..7.
__device__ __forceinline__ void copy2_piece(const signed char* src, int rows, int row0, int K, int k0, char* lds,
                                            int wave, int lane, int u) {
  const int j = wave + u * NWV;
  const int r = 8 * j + (lane >> 3);
  const int p = slot2_of(r, lane & 7);
  const int gr = min(row0 + r, rows - 1);
  __builtin_amdgcn_global_load_lds(src + (size_t)gr * K + k0 + p * 16, (LDS_AS void*)(lds + j * 1024), 16, 0, 0);
}

template <bool OUT_I32, int TN>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w8a8_k128_kernel(
    const signed char* __restrict__ xq, const float* __restrict__ sx, const signed char* __restrict__ wq,
    const float* __restrict__ sw, const __bf16* __restrict__ bias, int M, int N, int K, void* __restrict__ y) {
  using T = K128<TN>;
  constexpr int JB = T::JB, STAGE2 = T::STAGE;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + TN - 1) / TN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * TN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int rr = lane & 31, hh = lane >> 5;
  char* lds = g_lds;
  const int KT = K / BK2;

  auto copy_stage = [&](int kt, char* st) {
#pragma unroll
    for (int u = 0; u < 8; ++u) copy2_piece(xq, M, m0, K, kt * BK2, st, wave, lane, u);
#pragma unroll
    for (int u = 0; u < T::BCOPY; ++u) copy2_piece(wq, N, n0, K, kt * BK2, st + TILE_A2, wave, lane, u);
  };
  // operand rows: A row wm*128 + 32i + rr, B row wn*TN/2 + 32j + rr; k32 step ks takes piece
  // 2ks + hh; block i (j) adds 32 rows = 4096 bytes
  const int x = (rr >> 1) & 7;
  int aoff[4], boff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    aoff[ks] = (wm * 128 + rr) * BK2 + 16 * ((2 * ks + hh) ^ x);
    boff[ks] = TILE_A2 + (wn * (TN / 2) + rr) * BK2 + 16 * ((2 * ks + hh) ^ x);
  }
  constexpr int NOPS = 4 + JB;  // operand reads per k32 step
  i32x4 a0[4], b0[JB], a1[4], b1[JB];
  // one read of operand q (0..NOPS-1, in the order the MFMAs use them: a[0], b[0..JB-1], a[1..3])
  auto read_op = [&](const char* st, int ks, int q, i32x4(&av)[4], i32x4(&bv)[JB]) {
    if (q == 0) av[0] = *reinterpret_cast<const i32x4*>(st + aoff[ks]);
    else if (q <= JB) bv[q - 1] = *reinterpret_cast<const i32x4*>(st + boff[ks] + 4096 * (q - 1));
    else av[q - JB] = *reinterpret_cast<const i32x4*>(st + aoff[ks] + 4096 * (q - JB));
  };
  i32x16 acc[4][JB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;
  auto mfma_t = [&](int t, const i32x4(&av)[4], const i32x4(&bv)[JB]) {
    acc[t / JB][t % JB] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bv[t % JB], av[t / JB], acc[t / JB][t % JB], 0, 0, 0);
  };
  // a k32 step: 4 JB MFMAs on (av, bv), the first NOPS each followed by one read of the
  // next step's operands into (nav, nbv)
  auto step = [&](const i32x4(&av)[4], const i32x4(&bv)[JB], const char* nst, int nks, i32x4(&nav)[4],
                  i32x4(&nbv)[JB]) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4 * JB; ++t) {
      mfma_t(t, av, bv);
      if (t < NOPS) read_op(nst, nks, t, nav, nbv);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  copy_stage(0, lds);
  if (KT > 1) copy_stage(1, lds + STAGE2);
  if (KT > 1) wait_vm_barrier<8 + T::BCOPY>();
  else wait_vm_barrier<0>();
#pragma unroll
  for (int q = 0; q < NOPS; ++q) read_op(lds, 0, q, a0, b0);

  // Stage kt in buffer s: steps 0-2 each read the next step's operands; the barrier
  // (stage kt+1 has landed, every wave's reads of stage kt are done) comes before step 3,
  // whose MFMAs carry the reads of stage kt+1's first step and the copies that refill
  // buffer s with stage kt+2.
  auto body = [&](auto full, int kt, int s) {
    const char* st = lds + s * STAGE2;
    const char* nst = lds + (1 - s) * STAGE2;
    step(a0, b0, st, 1, a1, b1);
    step(a1, b1, st, 2, a0, b0);
    step(a0, b0, st, 3, a1, b1);
    wait_vm_barrier<0>();
    // the asm above already drained lgkmcnt; saying so keeps the compiler from placing its
    // own lgkmcnt(0) after the first new read of step 3
    __builtin_amdgcn_s_waitcnt(0xC07F);
    if constexpr (decltype(full)::value) {
      char* cst = lds + s * STAGE2;
      __builtin_amdgcn_sched_barrier(0);
      // slot t: MFMA t, then the next stage's read t (t < NOPS), the refill copies of A
      // (t < 8) and of B (the last BCOPY slots)
      constexpr int B0 = 4 * JB - T::BCOPY;
#pragma unroll
      for (int t = 0; t < 4 * JB; ++t) {
        mfma_t(t, a1, b1);
        if (t < NOPS) read_op(nst, 0, t, a0, b0);
        if (t < 8) copy2_piece(xq, M, m0, K, (kt + 2) * BK2, cst, wave, lane, t);
        if (t >= B0) copy2_piece(wq, N, n0, K, (kt + 2) * BK2, cst + TILE_A2, wave, lane, t - B0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      if (kt + 1 < KT) {
#pragma unroll
        for (int q = 0; q < NOPS; ++q) read_op(nst, 0, q, a0, b0);
      }
#pragma unroll
      for (int t = 0; t < 4 * JB; ++t) mfma_t(t, a1, b1);
    }
  };
  int kt = 0, s = 0;
  for (; kt + 2 < KT; ++kt, s ^= 1) body(std::true_type{}, kt, s);
  for (; kt < KT; ++kt, s ^= 1) body(std::false_type{}, kt, s);
  __syncthreads();
  gemm_epilogue<OUT_I32, TN>(acc, lds, sx, sw, bias, M, N, m0, n0, wm, wn, rr, hh, tid, y);
}

}  // namespace

namespace wf {

bool use_narrow_tiles(int M, int N) {
  // Modelled time in units of one 256 x 256 tile: waves of workgroups (one per CU) times
  // the tile's width share, with the narrow tile's measured 10 % lower efficiency per unit
  // of work (shorter MFMA runs per operand read, fixed per-tile prologue and epilogue).
  // Measured on the Wan2.1 projections (23,400 tokens): the 1.3B O projection (552 wide
  // tiles = 2.2 waves) gains 96 -> 82 us; the 14B O projection (7.2 waves) would lose 4 %.
  constexpr int kCUs = 256;
  const long long tm = (M + BM - 1) / BM;
  const long long w256 = (tm * ((N + 255) / 256) + kCUs - 1) / kCUs;
  const long long w192 = (tm * ((N + 191) / 192) + kCUs - 1) / kCUs;
  return (double)w192 * 0.75 * 1.10 <= (double)w256;
}

hipError_t launch_quant_rows_i8(const void* x, int rows, int cols, void* q, float* scales, hipStream_t s) {
  const int pieces = (cols + 511) / 512;
  auto run = [&](auto kern) {
    kern<<<(rows + 3) / 4, 256, 0, s>>>(static_cast<const __bf16*>(x), rows, cols, static_cast<signed char*>(q),
                                        scales);
    return hipGetLastError();
  };
  if (pieces <= 1) return run(quant_rows_kernel<1>);
  if (pieces <= 2) return run(quant_rows_kernel<2>);
  if (pieces <= 3) return run(quant_rows_kernel<3>);
  if (pieces <= 4) return run(quant_rows_kernel<4>);
  if (pieces <= 6) return run(quant_rows_kernel<6>);
  if (pieces <= 8) return run(quant_rows_kernel<8>);
  if (pieces <= 10) return run(quant_rows_kernel<10>);
  if (pieces <= 12) return run(quant_rows_kernel<12>);
  return run(quant_rows_kernel<RPIECES_MAX>);
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
  if (K % BK2 == 0) {  // 128-byte stages: half the barriers per MFMA
    const bool narrow = use_narrow_tiles(M, N);
    auto run2 = [&](auto kern, int tn, int lds) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
      const int nb = ((M + BM - 1) / BM) * ((N + tn - 1) / tn);
      kern<<<nb, NWV * 64, lds, s>>>(static_cast<const signed char*>(xq), sx, static_cast<const signed char*>(wq),
                                     sw, static_cast<const __bf16*>(bias), M, N, K, y);
      return hipGetLastError();
    };
    if (narrow)
      return out_i32 ? run2(gemm_w8a8_k128_kernel<true, 192>, 192, K128<192>::LDS)
                     : run2(gemm_w8a8_k128_kernel<false, 192>, 192, K128<192>::LDS);
    return out_i32 ? run2(gemm_w8a8_k128_kernel<true, 256>, 256, K128<256>::LDS)
                   : run2(gemm_w8a8_k128_kernel<false, 256>, 256, K128<256>::LDS);
  }
  return out_i32 ? run(gemm_w8a8_kernel<true>) : run(gemm_w8a8_kernel<false>);
}

}  // namespace wf
