// Chunk-wise causal attention of one Wave Forcing round on gfx950.
//
// What is computed (Wave Forcing paper pages, Abstract; airadar.tv summaries,
// first paragraph): query chunk j of the in-flight block (0 = cache-refresh
// chunk) attends to every history chunk, to in-flight chunks 0..j and to
// itself; later chunks are invisible. With keys in logical order that is the
// prefix of the first (n_hist + j + 1) chunks, so visibility is decided per
// (query tile, key tile) pair: query tiles never straddle chunks, key tiles are
// aligned to chunk starts, and the tiles of later chunks are never visited.
// Only the zero padding past the end of a chunk is masked inside a tile.
//
// Kernel structure (one workgroup = NW waves = NW*32 query rows of one chunk
// and one head; grid ordered longest-first):
//   * Each wave keeps its 32 query rows in registers as the stationary MFMA B
//     operand.
//   * Key tiles (64 keys) are stored in the cache as LDS images (see
//     kv_cache.hip) and copied HBM -> LDS with global_load_lds_dwordx4: no
//     staging registers, no LDS write instructions. Three K stages and three V
//     stages; the copies of K(t+2) and V(t+1) are in flight while tile t is
//     consumed.
//   * S^T = K Q^T on MFMA: lane (q, half) of the 32x32 output holds one query
//     and 16 keys, so the softmax row statistics need one cross-half exchange.
//     The K rows are read in a permuted order (key_of_arow) so that the 16 keys
//     of a lane come out as two runs of 8 consecutive keys, which is exactly
//     the B-operand layout of the next contraction.
//   * O^T += V^T P^T on MFMA, P taken straight from registers (bf16 for the
//     bf16 path).
//   * Online softmax in the exp2 domain with a lazily moved reference max:
//     the accumulators are rescaled only when a row's max grows by more than
//     2^8, which keeps weights <= 256 and the result exact up to rounding.
#include <cmath>
#include <mutex>
#include <type_traits>

#include "wf_internal.h"

// Scratch of the allocation-free call (wf_chunk_causal_attn_fwd_static): the
// key-split partials live in this file-scope device array, one copy per GPU
// the library runs on, held until the process ends. Host code never uses the
// name itself (in host code it is a stand-in, not a device address): the
// address comes from hipGetSymbolAddress, per device (wf::static_scratch).
static __device__ __align__(256) char scratch[WF_STATIC_SCRATCH_BYTES];

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int KT = 64;  // keys per tile
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kRescaleLog2 = 8.0f;
constexpr float kTileSumMax = 256.0f;  // 2^kRescaleLog2
// The int8 scores accumulate on top of kMagicI, the bits of the float kMagicF =
// 1.5 * 2^23: for |score| < 2^22 (127 * 127 * 128 < 2^21) the int32 sum read as
// a float is exactly kMagicF + score, so no int -> float conversion is needed.
constexpr int kMagicI = 0x4B400000;
constexpr float kMagicF = 12582912.0f;

// A-operand row i of a 32-key block reads key key_of_arow(i). With the 32x32
// output layout (lane half hh, element r <-> row 8*(r/4) + 4*hh + r%4) this
// makes element r of half hh the key 16*(r/8) + 8*hh + r%8.
__device__ __forceinline__ int key_of_arow(int i) {
  const int a = i >> 3, b = (i >> 2) & 1, c = i & 3;
  return ((a >> 1) << 4) + (b << 3) + ((a & 1) << 2) + c;
}
__device__ __forceinline__ int key_of_elem(int hh, int r) { return ((r >> 3) << 4) + (hh << 3) + (r & 7); }

// max / sum over the two halves of a row with one v_permlane32_swap: for lane
// l < 32 it returns (x[l], x[l+32]), for l >= 32 (x[l-32], x[l]).
__device__ __forceinline__ float halves_max(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Wait until at most N of this wave's vector-memory operations are still in
// flight (the LDS copies of the newest step), finish this wave's LDS reads,
// then meet the other waves. Unlike __syncthreads() this does not drain the
// copies that are meant to stay in flight across the barrier.
#define WF_WAIT_VM_BARRIER(n) asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)\n\ts_barrier" ::: "memory")
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N <= 8, "unsupported wait count");
  if constexpr (N == 0) WF_WAIT_VM_BARRIER(0);
  if constexpr (N == 1) WF_WAIT_VM_BARRIER(1);
  if constexpr (N == 2) WF_WAIT_VM_BARRIER(2);
  if constexpr (N == 3) WF_WAIT_VM_BARRIER(3);
  if constexpr (N == 4) WF_WAIT_VM_BARRIER(4);
  if constexpr (N == 6) WF_WAIT_VM_BARRIER(6);
  if constexpr (N == 8) WF_WAIT_VM_BARRIER(8);
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Keep a block's results on its side of the next barrier: the compiler may
// not sink the instructions producing these registers past this point (volatile
// asm statements keep their order, and the barrier is one).
__device__ __forceinline__ void pin_scores(f32x16& a, f32x16& b) { asm volatile("" : "+v"(a), "+v"(b)); }
__device__ __forceinline__ void pin_scores(i32x16& a, i32x16& b) { asm volatile("" : "+v"(a), "+v"(b)); }
__device__ __forceinline__ void pin_weights(bf16x8 (&p)[4]) {
  asm volatile("" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]));
}

struct Work {
  int j, h, qt;
  int part;  // -1, or the half (0, 1) of the key tiles of a split query tile
};

constexpr int kXcds = 8;  // workgroup i of a launch runs on XCD i % 8; each XCD has its own L2

// Work item of workgroup b. Items are numbered longest-first (query chunk
// N-1 sees the most keys), then by head, then by query tile. The T query
// tiles of one (chunk, head) read the same K/V tiles in the same order, so
// they are placed on one XCD, where they share its L2: in every run of
// 8*T consecutive workgroups, XCD x takes the T tiles of one (chunk, head),
// alternating direction from run to run (which evens out the work per XCD
// across the longest-first order). The last partial run keeps the plain order.
__device__ __forceinline__ Work decode_block(int b, int N, int H, int T) {
  int item = b;
  const int run = kXcds * T;
  const int full = (N * H * T) / run * run;
  if (b < full) {
    const int s = b / run, in = b - s * run;
    int x = in % kXcds;
    if (s & 1) x = kXcds - 1 - x;
    item = s * run + x * T + in / kXcds;
  }
  const int per = H * T;
  const int cls = item / per;
  const int rem = item - cls * per;
  Work w;
  w.j = N - 1 - cls;
  w.h = rem / T;
  w.qt = rem - w.h * T;
  w.part = -1;
  return w;
}

// Work item of workgroup b when in-flight chunk 0 is split into two halves of its
// key tiles (p.split set): chunks N-1 .. 1 first, in the order above; then the query tiles of
// chunk 0 as 2H "heads" (head h, half p -> 2h + p) in the same XCD-run order, so the
// short halves fill the end of the grid.
__device__ __forceinline__ Work decode_work(int b, const wf::AttnParams& p) {
  const int N = p.n_inflight, H = p.n_heads, T = p.q_tiles;
  if (!p.split) return decode_block(b, N, H, T);
  const int n_main = (N - 1) * H * T;
  if (b < n_main) {
    Work w = decode_block(b, N - 1, H, T);
    w.j += 1;
    return w;
  }
  Work w = decode_block(b - n_main, 1, 2 * H, T);
  w.part = w.h & 1;
  w.h >>= 1;
  return w;
}

// Tile images: K [D/E pieces][64 keys][16 B], V [64/E pieces][D dims][16 B].
template <typename E, int D, int NW>
struct Geo {
  static constexpr int ES = sizeof(E);
  static constexpr int TILE = KT * D * ES;      // bytes of one K (or V) tile image
  static constexpr int KPS = KT * 16;           // K image: bytes per piece (64 keys)
  static constexpr int VPS = D * 16;            // V image: bytes per piece (D dims)
  static constexpr int NSTAGE = 3;
  static constexpr int LDS = 2 * NSTAGE * TILE; // three K stages, then three V stages
  static constexpr int NT = NW * 64;
  static constexpr int COPIES = TILE / 1024;    // 1 KB copy instructions per tile image
  static constexpr int CPW = COPIES / NW;       // per wave, per tensor
  static_assert(CPW * NW == COPIES, "tile copies must split evenly over the waves");
};

// Direct HBM -> LDS copy of one image of BYTES bytes: wave w issues the 1 KB
// copies w, w+NW, ...
template <int BYTES, int NW>
__device__ __forceinline__ void copy_image(const char* src, char* lds_dst, int wave, int lane) {
  static_assert(BYTES % (1024 * NW) == 0, "image copies must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < BYTES / (1024 * NW); ++i) {
    const int c = wave + i * NW;
    __builtin_amdgcn_global_load_lds(src + c * 1024 + lane * 16, (LDS_AS void*)(lds_dst + c * 1024), 16, 0, 0);
  }
}
template <typename G>
__device__ __forceinline__ void copy_tile(const char* src, char* lds_dst, int wave, int lane) {
  copy_image<G::TILE, G::NT / 64>(src, lds_dst, wave, lane);
}

// Addresses of key tile t (logical chunk t / ktc, tile t % ktc) for head h.
struct TileSrc {
  const char* kpool;
  const char* vpool;
  size_t slot_bytes, head_off;
  int tile_bytes, ktc;
  const int* slots;
  __device__ __forceinline__ size_t off(int t) const {
    const int cl = t / ktc;
    return (size_t)slots[cl] * slot_bytes + head_off + (size_t)(t - cl * ktc) * tile_bytes;
  }
};

extern __shared__ __attribute__((aligned(1024))) char g_smem[];

// ---------------------------------------------------------------- bf16
// Work of one wave on key tile t is split into an MFMA block and a VALU block:
//   M_t = { O^T += V(t-1)^T P(t-1)^T ;  S^T = K(t) Q^T }   (two independent contractions)
//   V_t = { online softmax of S -> P(t) }
// Step t: start the copies of K(t+2) and V(t+1), run M_t and V_t, wait for the
// copies of the previous step (K(t+1), V(t)), barrier. K(t) lives in K stage
// t%3 from step t-2 to step t, V(t) in V stage t%3 from step t-1 to step t+1,
// so no stage is overwritten while a wave can still read it.
//
// Ping-pong: waves 4-7 lead waves 0-3 (one of each per SIMD) by half a step,
// each half-step ending with a barrier, so that on every SIMD one wave feeds
// the matrix cores while the other runs the softmax.

// I8 = true: the int8-QK variant. S^T = K'^T Q^T runs on int8 MFMA over the
// codes that attn_i8qk.hip wrote (K - mean and Q, 128-token blocks); the wave's
// 32 query rows share one Q scale and a 64-key tile one K scale, so the
// dequantization is one factor per (wave, tile) folded into the exp2 argument.
// K code tiles come from the workspace in logical order, V from the cache.
// P.V stays bf16.
template <int D, bool I8>
struct TileBytes {
  static constexpr int K = KT * D * (I8 ? 1 : 2);
  static constexpr int V = KT * D * 2;
  static constexpr int LDS = 3 * K + 3 * V;
};

// int8-QK MFMA block of one step, written out with exact LDS waits: the 8
// Q.K MFMAs of tile t (int8, scores start from kMagicI), then the 16 P.V MFMAs
// of tile t-1 (bf16). Each MFMA's A operand is read from LDS four reads ahead,
// and the wait before it lets the three later reads stay in flight (the
// compiler's own waits drained all reads every fourth MFMA). The Q.K MFMAs go
// first, so the scores are ready long before the block ends; the caller waits
// out the MFMA-result hazard (mfma_to_valu) before the VALU touches o. The
// leading s_nop covers VALU writes of P and O just before the block. Every
// read is waited for inside the block.
//   kaddr: LDS address of this lane's first K-code piece (stage + k_lane);
//   vaddr: LDS address of this lane's first V piece (stage + v_lane).
__device__ __forceinline__ void mblock_i8(f32x16 (&o)[4], i32x16 (&si)[2], const i32x4 (&qop8)[4],
                                          const bf16x8 (&pk)[4], const i32x16& magic16, unsigned kaddr,
                                          unsigned vaddr) {
  bf16x8 abuf[4];
  asm volatile(
      "s_nop 3\n\t"
      "ds_read_b128 %6, %18 offset:0\n\t"
      "ds_read_b128 %7, %18 offset:512\n\t"
      "ds_read_b128 %8, %18 offset:1024\n\t"
      "ds_read_b128 %9, %18 offset:1536\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_i32_32x32x32_i8 %4, %6, %10, %20\n\t"
      "ds_read_b128 %6, %18 offset:2048\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_i32_32x32x32_i8 %5, %7, %10, %20\n\t"
      "ds_read_b128 %7, %18 offset:2560\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_i32_32x32x32_i8 %4, %8, %11, %4\n\t"
      "ds_read_b128 %8, %18 offset:3072\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_i32_32x32x32_i8 %5, %9, %11, %5\n\t"
      "ds_read_b128 %9, %18 offset:3584\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_i32_32x32x32_i8 %4, %6, %12, %4\n\t"
      "ds_read_b128 %6, %19 offset:0\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_i32_32x32x32_i8 %5, %7, %12, %5\n\t"
      "ds_read_b128 %7, %19 offset:512\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_i32_32x32x32_i8 %4, %8, %13, %4\n\t"
      "ds_read_b128 %8, %19 offset:1024\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_i32_32x32x32_i8 %5, %9, %13, %5\n\t"
      "ds_read_b128 %9, %19 offset:1536\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %6, %14, %0\n\t"
      "ds_read_b128 %6, %19 offset:4096\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %7, %14, %1\n\t"
      "ds_read_b128 %7, %19 offset:4608\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %8, %14, %2\n\t"
      "ds_read_b128 %8, %19 offset:5120\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %9, %14, %3\n\t"
      "ds_read_b128 %9, %19 offset:5632\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %6, %15, %0\n\t"
      "ds_read_b128 %6, %19 offset:8192\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %7, %15, %1\n\t"
      "ds_read_b128 %7, %19 offset:8704\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %8, %15, %2\n\t"
      "ds_read_b128 %8, %19 offset:9216\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %9, %15, %3\n\t"
      "ds_read_b128 %9, %19 offset:9728\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %6, %16, %0\n\t"
      "ds_read_b128 %6, %19 offset:12288\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %7, %16, %1\n\t"
      "ds_read_b128 %7, %19 offset:12800\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %8, %16, %2\n\t"
      "ds_read_b128 %8, %19 offset:13312\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %9, %16, %3\n\t"
      "ds_read_b128 %9, %19 offset:13824\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %6, %17, %0\n\t"
      "s_waitcnt lgkmcnt(2)\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %7, %17, %1\n\t"
      "s_waitcnt lgkmcnt(1)\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %8, %17, %2\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %9, %17, %3\n\t"
      : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]), "=&v"(si[0]), "=&v"(si[1]), "=&v"(abuf[0]), "=&v"(abuf[1]), "=&v"(abuf[2]), "=&v"(abuf[3])
      : "v"(qop8[0]), "v"(qop8[1]), "v"(qop8[2]), "v"(qop8[3]), "v"(pk[0]), "v"(pk[1]), "v"(pk[2]), "v"(pk[3]), "v"(kaddr), "v"(vaddr), "v"(magic16));
}

// The int8 MFMA block is inline asm, so the compiler does not know that its
// last MFMAs write o: wait out the MFMA-result hazard before the VALU reads o.
__device__ __forceinline__ void mfma_to_valu(f32x16 (&o)[4]) {
  asm volatile("s_nop 15\n\ts_nop 7" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
}

template <int D, int NW, bool I8 = false>
__global__ __launch_bounds__(NW * 64) void attn_fwd_bf16_kernel(wf::AttnParams p) {
  static_assert(NW == 8, "8 waves: two per SIMD");
  static_assert(!I8 || D == 128, "the int8 block is written for head_dim 128");
  using G = Geo<__bf16, D, NW>;
  using TB = TileBytes<D, I8>;
  constexpr int KS = D / 16;               // bf16 MFMA steps over head_dim (16 per step)
  constexpr int KSQ = I8 ? D / 32 : KS;    // Q.K MFMA steps (int8: 32 per step)
  constexpr int DB = D / 32;               // 32-row blocks of O^T
  char* smem = g_smem;

  const Work w = decode_work(blockIdx.x, p);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = (wave >> 2) ^ 1;  // group 0 (waves 4-7) leads by half a step
  const int qi = lane & 31, hh = lane >> 5;
  const int C = p.chunk_tokens, H = p.n_heads;
  const int wrow = w.qt * (NW * 32) + wave * 32;
  const bool wave_on = wrow < C;
  const int row = wrow + qi;
  const bool row_ok = row < C;
  const size_t qoff = (((size_t)w.j * C + row) * H + w.h) * D;

  const int ktc = p.key_tiles;
  const int n_vis = p.n_hist + w.j + 1;  // visible logical chunks
  // key tiles t_base .. t_base + n_iter - 1 of the visible ones (all of them, or one half)
  const int n_all = n_vis * ktc;
  const int t_base = w.part == 1 ? n_all / 2 : 0;
  const int n_iter = w.part < 0 ? n_all : (w.part == 0 ? n_all / 2 : n_all - n_all / 2);
  const char* kpool = I8 ? reinterpret_cast<const char*>(p.k_codes) : static_cast<const char*>(p.k_pool);
  const char* vpool = static_cast<const char*>(p.v_pool);
  const size_t slot_bytes = (size_t)p.slot_elems * G::ES;
  const size_t head_off = (size_t)w.h * p.s_pad * D * G::ES;
  // int8 K codes: [table position][head][s_pad / 64 tiles][TB::K bytes]
  const size_t kchunk_bytes = (size_t)(p.s_pad / KT) * TB::K;
  // Wave-uniform cursor over the tiles in visiting order (chunk by chunk), so
  // the loop needs no divisions: byte offsets of the tile's K and V images.
  struct Cursor {
    int cl, kt;
    size_t koff, voff;
  };
  auto chunk_start = [&](Cursor& c) {
    c.voff = (size_t)p.slots[c.cl] * slot_bytes + head_off;
    c.koff = I8 ? ((size_t)c.cl * H + w.h) * kchunk_bytes : c.voff;
  };
  auto cursor_at = [&](int t) {  // t counts from the first tile of this workgroup's range
    Cursor c;
    c.cl = (t_base + t) / ktc;
    c.kt = (t_base + t) - c.cl * ktc;
    chunk_start(c);
    c.voff += (size_t)c.kt * TB::V;
    c.koff += (size_t)c.kt * TB::K;
    return c;
  };
  auto advance = [&](Cursor& c) {
    c.voff += TB::V;
    c.koff += TB::K;
    if (++c.kt == ktc) {
      c.kt = 0;
      if (++c.cl < n_vis) chunk_start(c);
    }
  };
  auto kst = [&](int r) { return smem + r * TB::K; };                   // K stage r
  auto vst = [&](int r) { return smem + 3 * TB::K + r * TB::V; };      // V stage r
  auto copy_k = [&](size_t off, char* dst) { copy_image<TB::K, NW>(kpool + off, dst, wave, lane); };
  auto copy_v = [&](size_t off, char* dst) { copy_image<TB::V, NW>(vpool + off, dst, wave, lane); };

  // prologue copies: K(0) -> K stage 0, K(1) -> K stage 1, V(0) -> V stage 0
  copy_k(cursor_at(0).koff, kst(0));
  if (n_iter > 1) copy_k(cursor_at(1).koff, kst(1));
  copy_v(cursor_at(0).voff, vst(0));

  // Stationary B operand: this lane's query row, half hh of head_dim (bf16
  // values, or int8 codes for I8).
  bf16x8 qop[I8 ? 1 : KS];
  i32x4 qop8[I8 ? KSQ : 1];
  float sl2e = p.scale_log2e;
  float* ksc = reinterpret_cast<float*>(smem + TB::LDS);  // I8: K scales of the visible chunks
  if constexpr (I8) {
    const u32x4* qp = reinterpret_cast<const u32x4*>(p.q_codes + qoff + hh * (D / 2));
#pragma unroll
    for (int k = 0; k < KSQ; ++k) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (row_ok) raw = qp[k];
      __builtin_memcpy(&qop8[k], &raw, 16);
    }
    const int nb = p.q_blocks;
    if (wave_on) sl2e *= p.q_scales[((size_t)w.h * p.n_inflight + w.j) * nb + wrow / 128];
    const float* ks_src = p.k_scales + (size_t)w.h * (p.n_hist + p.n_inflight) * nb;
    for (int i = tid; i < n_vis * nb; i += NW * 64) ksc[i] = ks_src[i];
  } else {
    const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(p.q) + qoff + hh * (D / 2));
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (row_ok) raw = qp[k];
      __builtin_memcpy(&qop[k], &raw, 16);
    }
  }
  {  // V stage of "tile -1" (read once, multiplied by P = 0) must hold finite values
    u32x4* z = reinterpret_cast<u32x4*>(vst(G::NSTAGE - 1));
    for (int i = tid; i < TB::V / 16; i += G::NT) z[i] = u32x4{0u, 0u, 0u, 0u};
  }
  wait_vm_barrier<0>();

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  f32x16 s[2];
  i32x16 si[2];  // I8: integer scores, biased by kMagicI
  i32x16 magic16;
#pragma unroll
  for (int e = 0; e < 16; ++e) magic16[e] = kMagicI;
  bf16x8 pk[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int e = 0; e < 8; ++e) pk[kk][e] = (__bf16)0.f;
  float m_ref = -INFINITY;                  // reference max (log2 domain) of this lane's query row
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};     // this half's share of the row sum of weights
  int gexp = 0;  // I8: every m_ref is a multiple of 2^(gexp - 127) (wave-uniform; 0: no grid yet)
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  // per-lane operand offsets inside a stage; every op adds a compile-time constant
  const int k_lane = key_of_arow(qi) * 16 + hh * KSQ * G::KPS;
  const int v_lane = qi * 16 + hh * G::VPS;

  // MFMA block with an explicit operand pipeline: LDS reads run DEPTH
  // operands ahead of the MFMAs in one straight-line region. Op i < NPV is a
  // P.V step (kk = i / DB, d = i % DB); op i >= NPV a Q.K step (k, b).
  constexpr int DEPTH = 4;
  constexpr int NPV = 4 * DB, NQK = 2 * KSQ;
  auto mrun = [&](const char* vs, const char* ks, auto has_pv, auto has_qk) {
    constexpr bool PV = decltype(has_pv)::value, QK = decltype(has_qk)::value;
    constexpr int I0 = PV ? 0 : NPV, I1 = QK ? NPV + NQK : NPV;
    auto rd = [&](auto ic) -> bf16x8 {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < NPV)
        return *reinterpret_cast<const bf16x8*>(vs + (i / DB) * 2 * G::VPS + (i % DB) * 32 * 16);
      else
        return *reinterpret_cast<const bf16x8*>(ks + ((i - NPV) / 2) * G::KPS + ((i - NPV) % 2) * 32 * 16);
    };
    auto mm = [&](auto ic, const bf16x8& a) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < NPV) {
        o[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[i / DB], o[i % DB], 0, 0, 0);
      } else if constexpr (I8) {
        constexpr int j = i - NPV;
        const i32x4 a8 = __builtin_bit_cast(i32x4, a);
        if constexpr (j < 2)
          si[j % 2] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a8, qop8[j / 2], i32x16{}, 0, 0, 0);
        else
          si[j % 2] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a8, qop8[j / 2], si[j % 2], 0, 0, 0);
      } else {
        constexpr int j = i - NPV;
        if constexpr (j < 2)
          s[j % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[j / 2], f32x16{}, 0, 0, 0);
        else
          s[j % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[j / 2], s[j % 2], 0, 0, 0);
      }
    };
    bf16x8 buf[DEPTH];
    static_for<0, DEPTH>([&](auto q) {
      constexpr int i = I0 + decltype(q)::value;
      if constexpr (i < I1) buf[decltype(q)::value] = rd(std::integral_constant<int, i>{});
    });
    static_for<I0, I1>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const bf16x8 a = buf[(i - I0) % DEPTH];
      if constexpr (i + DEPTH < I1) buf[(i - I0) % DEPTH] = rd(std::integral_constant<int, i + DEPTH>{});
      mm(ic, a);
    });
    // keep the pattern: DEPTH reads, then {MFMA, read} pairs, then the tail MFMAs
    constexpr int N = I1 - I0;
    __builtin_amdgcn_sched_group_barrier(0x100, DEPTH < N ? DEPTH : N, 0);
    static_for<0, N>([&](auto ic) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (decltype(ic)::value + DEPTH < N) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    });
  };
  // One fused MFMA block every step: at step 0 the P.V half multiplies P = 0
  // with the zero-filled V stage of "tile -1"; at step n_iter the Q.K half
  // computes scores that are never used. r = t % 3 is the K stage of tile t.
  auto mblock = [&](int r) {
    const int rv = r == 0 ? G::NSTAGE - 1 : r - 1;  // V stage of tile t-1
    if constexpr (I8) {
      mblock_i8(o, si, qop8, pk, magic16, (unsigned)(size_t)(LDS_AS char*)(kst(r) + k_lane),
                (unsigned)(size_t)(LDS_AS char*)(vst(rv) + v_lane));
    } else {
      mrun(vst(rv) + v_lane, kst(r) + k_lane, std::true_type{}, std::true_type{});
    }
  };

  // online softmax of a tile; kt = its index inside its chunk, cl its chunk
  auto vblock = [&](int kt, int cl) {
    float ct = sl2e;   // log2-domain factor of the raw scores
    float bias = 0.f;  // I8: the float bias kMagicF of the integer scores
    bool regrid = false;
    if constexpr (I8) {
      // ct is rounded to 21 significant bits, so kMagicF * ct = 3 * 2^22 * ct is exact and
      // a multiple of 2^(E - 22), E its binary exponent. With m_ref on that grid and
      // |m_ref| <= 2^(E + 1) (scores are below 2^22, so a row's max in log2 units is far
      // below kMagicF * ct unless another tile's factor is much larger), the per-row
      // constant -(kMagicF * ct + m_ref) of the weights below is exact: the float bias
      // of the scores cancels exactly and every tile's weights share one reference.
      // Otherwise the constant rounds at the fp32 precision of m_ref itself.
      const unsigned cb = __builtin_amdgcn_readfirstlane(__float_as_uint(ct * ksc[cl * p.q_blocks + (kt >> 1)]));
      ct = __uint_as_float((cb + 4u) & ~7u);  // nearest (ties up); a carry gives a power of two
      const int gt = (int)((__float_as_uint(kMagicF * ct) >> 23) & 0xffu) - 22;
      if (gt > gexp) {  // a coarser grid: m_ref moves onto it below
        gexp = gt;
        regrid = true;
      }
      bias = kMagicF;
#pragma unroll
      for (int b = 0; b < 2; ++b) s[b] = __builtin_bit_cast(f32x16, si[b]);  // kMagicF + score, exactly
    }
    const int valid = min(KT, C - kt * KT);
    if (valid < KT) {  // zero padding past the chunk end takes no weight
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * b + key_of_elem(hh, e) >= valid) s[b][e] = -INFINITY;
    }
    // Exact row max of the tile (four independent chains, then the other half of
    // the row) and the move of the reference max, with the running output and
    // sums rescaled. The fast path below calls it only when a weight against the
    // current m_ref could exceed 2^kRescaleLog2, so m_ref moves lazily.
    auto move_max = [&]() {
      float m4[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        m4[c] = fmaxf(s[c >> 1][(c & 1) * 8], s[c >> 1][(c & 1) * 8 + 1]);
#pragma unroll
        for (int e = 2; e < 8; ++e) m4[c] = fmaxf(m4[c], s[c >> 1][(c & 1) * 8 + e]);
      }
      float mx = halves_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
      const float tmax = (mx - bias) * ct;  // I8: exact subtraction (both in [2^23, 2^24))
      float mn = fmaxf(m_ref, tmax);
      if (I8 && gexp > 0)  // up to the next multiple of the grid 2^(gexp - 127), exactly
        mn = ceilf(mn * __uint_as_float((unsigned)(254 - gexp) << 23)) * __uint_as_float((unsigned)gexp << 23);
      const float alpha = fast_exp2(m_ref - mn);
      m_ref = mn;
#pragma unroll
      for (int c = 0; c < 4; ++c) lsum[c] *= alpha;
      if constexpr (I8) mfma_to_valu(o);
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
    };
    // weights 2^(s ct - m_ref) rounded to bf16, and this lane's share of their sum
    // in four accumulators: bf16 sums the rounded weights actually used (v_dot2);
    // I8 sums the fp32 weights with plain adds, which overlap the other wave's
    // MFMAs where the dot instructions do not.
    auto weights = [&](float (&ts)[4]) {
      const float nm = I8 ? fmaf(-bias, ct, -m_ref) : -m_ref;  // I8: exact (see above)
      if constexpr (I8) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          float w8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            w8[e] = fast_exp2(fmaf(s[kk >> 1][(kk & 1) * 8 + e], ct, nm));
            pk[kk][e] = (__bf16)w8[e];
          }
          ts[kk] = ((w8[0] + w8[1]) + (w8[2] + w8[3])) + ((w8[4] + w8[5]) + (w8[6] + w8[7]));
        }
      } else {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) pk[2 * b + (e >> 3)][e & 7] = (__bf16)fast_exp2(fmaf(s[b][e], ct, nm));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          ts[kk] = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 pr = {pk[kk][2 * e], pk[kk][2 * e + 1]};
            ts[kk] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ts[kk], false);
          }
        }
      }
    };
    // Max-free fast path: weights against the current reference max. A lane's
    // 32 weights summing to at most 2^kRescaleLog2 bound every weight by it, as
    // the lazy move above would; a larger, infinite or NaN sum (the first tile,
    // where m_ref = -inf, or a tile whose max moved up) takes the exact path, as
    // does an I8 tile whose scale needs a coarser grid for m_ref.
    float ts[4];
    weights(ts);
    const float tl = (ts[0] + ts[1]) + (ts[2] + ts[3]);
    if (regrid || __builtin_amdgcn_ballot_w64(!(tl <= kTileSumMax))) {
      move_max();
      weights(ts);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) lsum[kk] += ts[kk];
  };

  // Copies started in step t: K(t+2) into K stage (t+2)%3, V(t+1) into V stage
  // (t+1)%3; then wait for the copies of step t-1 and meet the other waves.
  Cursor ck = cursor_at(n_iter > 2 ? 2 : 0), cv = cursor_at(n_iter > 1 ? 1 : 0);
  auto copies_and_wait = [&](int t, int r) {
    const bool dk = t + 2 < n_iter, dv = t + 1 < n_iter;
    const int r1 = r == G::NSTAGE - 1 ? 0 : r + 1, r2 = r1 == G::NSTAGE - 1 ? 0 : r1 + 1;
    if (dk) {
      copy_k(ck.koff, kst(r2));
      advance(ck);
    }
    if (dv) {
      copy_v(cv.voff, vst(r1));
      advance(cv);
    }
    constexpr int nk = TB::K / (1024 * NW), nv = TB::V / (1024 * NW);  // copy instructions per wave
    if (dk && dv)
      wait_vm_barrier<nk + nv>();
    else if (dv)
      wait_vm_barrier<nv>();
    else
      wait_vm_barrier<0>();
  };

  // The mid-step barrier only phases the two groups (no LDS stage changes hands
  // there: the copies of step t write stages that no wave reads in step t). The
  // bf16 kernel keeps it, which holds the ping-pong and measured less energy per
  // call; the int8 kernel, whose MFMA block is shorter than its softmax, runs
  // faster with the waves left to interleave between the step barriers.
  auto mid_barrier = [&]() {
    if constexpr (!I8) lds_barrier();
  };
  if (!wave_on) {  // a wave past the chunk end still copies and meets every barrier
    for (int t = 0, r = 0; t <= n_iter; ++t, r = r == G::NSTAGE - 1 ? 0 : r + 1) {
      mid_barrier();
      copies_and_wait(t, r);
    }
  } else if (grp == 0) {
    // ping-pong group 0: M_t, (mid barrier), V_t, copies + barrier
    int vkt = t_base % ktc, vcl = t_base / ktc;
    for (int t = 0, r = 0; t <= n_iter; ++t, r = r == G::NSTAGE - 1 ? 0 : r + 1) {
      mblock(r);
      if constexpr (I8)
        pin_scores(si[0], si[1]);
      else
        pin_scores(s[0], s[1]);
      mid_barrier();
      if (t < n_iter) {
        vblock(vkt, vcl);
        if (++vkt == ktc) vkt = 0, ++vcl;
      }
      pin_weights(pk);
      copies_and_wait(t, r);
    }
  } else {
    // ping-pong group 1, half a step behind: V_{t-1}, (mid barrier), M_t, copies + barrier
    int vkt = t_base % ktc, vcl = t_base / ktc;
    for (int t = 0, r = 0; t <= n_iter; ++t, r = r == G::NSTAGE - 1 ? 0 : r + 1) {
      if (t >= 1) {
        vblock(vkt, vcl);
        if (++vkt == ktc) vkt = 0, ++vcl;
      }
      pin_weights(pk);
      mid_barrier();
      mblock(r);
      if constexpr (I8)
        pin_scores(si[0], si[1]);
      else
        pin_scores(s[0], s[1]);
      copies_and_wait(t, r);
    }
  }

  if constexpr (I8) mfma_to_valu(o);
  if (wave_on && w.part >= 0) {  // one half of a split query tile: unnormalized partials
    const float lt = halves_sum((lsum[0] + lsum[1]) + (lsum[2] + lsum[3]));
    if (row_ok) {
      const size_t pr = ((size_t)w.part * H + w.h) * C + row;  // chunk 0: row is the chunk row
      float* orow = p.part_o + pr * D;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<f32x4*>(orow + 32 * d + 8 * a + 4 * hh) =
              f32x4{o[d][4 * a], o[d][4 * a + 1], o[d][4 * a + 2], o[d][4 * a + 3]};
      if (hh == 0) *reinterpret_cast<float2*>(p.part_ml + 2 * pr) = float2{m_ref, lt};
    }
  } else if (wave_on) {
    const float lt = halves_sum((lsum[0] + lsum[1]) + (lsum[2] + lsum[3]));
    const float inv = 1.0f / lt;
    if (row_ok) {
      __bf16* orow = static_cast<__bf16*>(p.o) + qoff;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          __bf16 v4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[d][4 * a + e] * inv);
          uint2 raw;
          __builtin_memcpy(&raw, v4, 8);
          *reinterpret_cast<uint2*>(orow + 32 * d + 8 * a + 4 * hh) = raw;
        }
      if (p.lse && hh == 0) {
        const size_t li = (size_t)w.h * p.n_inflight * C + (size_t)w.j * C + row;
        float lse = (m_ref + log2f(lt)) * kLn2;
        if constexpr (I8) lse += p.scale * p.qm[li];  // the keys' shared mean shift, added back
        p.lse[li] = lse;
      }
    }
  }
}


// ---------------------------------------------------------------- fp32
// fp32 operands on v_mfma_f32_32x32x2_f32 (two head_dim or key values per
// instruction), weights stay fp32. Plain schedule: copy tile t+1 while tile t
// is consumed (two stages), QK, softmax, PV, barrier.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_f32_kernel(wf::AttnParams p) {
  using G = Geo<float, D, NW>;
  constexpr int DB = D / 32;
  constexpr int QP = D / 8;  // 4-float pieces in this lane's half of head_dim
  char* smem = g_smem;

  const Work w = decode_block(blockIdx.x, p.n_inflight, p.n_heads, p.q_tiles);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = lane & 31, hh = lane >> 5;
  const int C = p.chunk_tokens, H = p.n_heads;
  const int wrow = w.qt * (NW * 32) + wave * 32;
  const bool wave_on = wrow < C;
  const int row = wrow + qi;
  const bool row_ok = row < C;
  const size_t qoff = (((size_t)w.j * C + row) * H + w.h) * D;

  const TileSrc src{static_cast<const char*>(p.k_pool), static_cast<const char*>(p.v_pool),
                    (size_t)p.slot_elems * G::ES, (size_t)w.h * p.s_pad * D * G::ES, G::TILE, p.key_tiles,
                    p.slots};
  const int n_iter = (p.n_hist + w.j + 1) * p.key_tiles;
  // two stages: stage b = K image at b*2*TILE, V image right after it
  auto copy_kv = [&](int t) {
    char* st = smem + (t & 1) * 2 * G::TILE;
    copy_tile<G>(src.kpool + src.off(t), st, wave, lane);
    copy_tile<G>(src.vpool + src.off(t), st + G::TILE, wave, lane);
  };

  copy_kv(0);
  f32x4 qop[QP];
  {
    const f32x4* qp = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.q) + qoff + hh * (D / 2));
#pragma unroll
    for (int k = 0; k < QP; ++k) qop[k] = row_ok ? qp[k] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  wait_vm_barrier<0>();

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  float m_ref = -INFINITY, lsum = 0.f;
  const float sl2e = p.scale_log2e;
  const int k_lane = key_of_arow(qi) * 16 + hh * QP * G::KPS;
  const int v_lane = qi * 16;

  for (int it = 0; it < n_iter; ++it) {
    if (it + 1 < n_iter) copy_kv(it + 1);
    const char* ks = smem + (it & 1) * 2 * G::TILE + k_lane;
    const char* vs = smem + (it & 1) * 2 * G::TILE + G::TILE + v_lane;
    if (wave_on) {
      f32x16 s[2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[b][e] = 0.f;
#pragma unroll
      for (int k = 0; k < QP; ++k) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(ks + k * G::KPS + b * 32 * 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qop[k][e], s[b], 0, 0, 0);
        }
      }
      const int kt = it % p.key_tiles;
      const int valid = min(KT, C - kt * KT);
      if (valid < KT) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * b + key_of_elem(hh, e) >= valid) s[b][e] = -INFINITY;
      }
      float mx = s[0][0];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[b][e]);
      mx = halves_max(mx);
      const float tmax = mx * sl2e;
      if (__builtin_amdgcn_ballot_w64(tmax > m_ref + kRescaleLog2)) {
        const float mn = fmaxf(m_ref, tmax);
        const float alpha = fast_exp2(m_ref - mn);
        m_ref = mn;
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
      }
      const float nm = -m_ref;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s[b][e] = fast_exp2(fmaf(s[b][e], sl2e, nm));
          lsum += s[b][e];
        }
      // element r of block b is key 32b + 16(r/8) + 8hh + r%8; V piece
      // 8b + 4(g/2) + 2hh + (g%2) (4 keys each) holds the keys of elements 4g..4g+3
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int d = 0; d < DB; ++d) {
            const int c = 8 * b + 4 * (g >> 1) + (g & 1);
            const f32x4 a = *reinterpret_cast<const f32x4*>(vs + (c + 2 * hh) * G::VPS + d * 32 * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              o[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], s[b][4 * g + e], o[d], 0, 0, 0);
          }
    }
    wait_vm_barrier<0>();
  }

  if (wave_on) {
    const float lt = halves_sum(lsum);
    const float inv = 1.0f / lt;
    if (row_ok) {
      float* orow = static_cast<float*>(p.o) + qoff;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = o[d][4 * a + e] * inv;
          *reinterpret_cast<f32x4*>(orow + 32 * d + 8 * a + 4 * hh) = v4;
        }
      if (p.lse && hh == 0)
        p.lse[(size_t)w.h * p.n_inflight * C + (size_t)w.j * C + row] = (m_ref + log2f(lt)) * kLn2;
    }
  }
}

// Merges the two halves of the split query tiles of chunk 0: one wave per (row, head).
// With the halves' log2-domain maxima m0, m1 and weight sums l0, l1 (weights taken
// against their own maxima): M = max, w_p = 2^(m_p - M), L = l0 w0 + l1 w1,
// O = (O0 w0 + O1 w1) / L, LSE = (M + log2 L) ln 2.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(wf::AttnParams p) {
  constexpr int PER = D / 64;  // dims per lane
  const int C = p.chunk_tokens, H = p.n_heads;
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wv >= C * H) return;
  const int row = wv / H, h = wv - row * H;
  const size_t r0 = (size_t)h * C + row, r1 = ((size_t)H + h) * C + row;
  const float2 ml0 = *reinterpret_cast<const float2*>(p.part_ml + 2 * r0);
  const float2 ml1 = *reinterpret_cast<const float2*>(p.part_ml + 2 * r1);
  const float m = fmaxf(ml0.x, ml1.x);
  const float w0 = fast_exp2(ml0.x - m), w1 = fast_exp2(ml1.x - m);
  const float l = ml0.y * w0 + ml1.y * w1;
  const float inv = 1.0f / l;
  const float* o0 = p.part_o + r0 * D + lane * PER;
  const float* o1 = p.part_o + r1 * D + lane * PER;
  __bf16* out = static_cast<__bf16*>(p.o) + ((size_t)row * H + h) * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = (__bf16)((o0[e] * w0 + o1[e] * w1) * inv);
  if (p.lse && lane == 0) p.lse[(size_t)h * p.n_inflight * C + row] = (m + log2f(l)) * kLn2;
}

template <typename Kern>
hipError_t launch(Kern k, int lds, int grid, int block, const wf::AttnParams& p, hipStream_t s) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  k<<<grid, block, lds, s>>>(p);
  return hipGetLastError();
}

}  // namespace

namespace wf {

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {  // first call on this device, which is current: look its copy up once
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t attn_split_bytes(const wf_kv_cache& kv) {
  if (kv.dtype != WF_BF16) return 0;
  const size_t rows = (size_t)2 * kv.n_heads * kv.chunk_tokens;
  return (rows * kv.head_dim * 4 + 255) / 256 * 256 + (rows * 8 + 255) / 256 * 256;
}

hipError_t launch_attn_fwd(const wf_kv_cache& kv, AttnParams& p, void* workspace, hipStream_t s) {
  const int C = kv.chunk_tokens;
  p.key_tiles = (C + KT - 1) / KT;
  if (kv.dtype == WF_BF16) {
    constexpr int NW = 8;
    p.q_tiles = (C + NW * 32 - 1) / (NW * 32);
    // Split chunk 0 (the shortest items) over its key tiles when there is a longer
    // chunk class for its halves to fill in behind and at least two key tiles to halve.
    p.split = workspace && p.n_inflight >= 2 && (long long)(p.n_hist + 1) * p.key_tiles >= 2;
    if (p.split) {
      const size_t rows = (size_t)2 * kv.n_heads * C;
      p.part_o = static_cast<float*>(workspace);
      p.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + (rows * kv.head_dim * 4 + 255) / 256 * 256);
    }
    // a split chunk 0 runs as two workgroups per query tile
    const int grid = (p.n_inflight + (p.split ? 1 : 0)) * kv.n_heads * p.q_tiles;
    hipError_t e = kv.head_dim == 128
                       ? launch(attn_fwd_bf16_kernel<128, NW>, TileBytes<128, false>::LDS, grid,
                                NW * 64, p, s)
                       : launch(attn_fwd_bf16_kernel<64, NW>, TileBytes<64, false>::LDS, grid,
                                NW * 64, p, s);
    if (e != hipSuccess || !p.split) return e;
    const int blocks = (C * kv.n_heads + 3) / 4;  // one wave per (row, head) of chunk 0
    if (kv.head_dim == 128)
      attn_combine_kernel<128><<<blocks, 256, 0, s>>>(p);
    else
      attn_combine_kernel<64><<<blocks, 256, 0, s>>>(p);
    return hipGetLastError();
  }
  constexpr int NW = 4;
  p.q_tiles = (C + NW * 32 - 1) / (NW * 32);
  const int grid = p.n_inflight * kv.n_heads * p.q_tiles;
  // the fp32 kernel uses two stages of K + V
  if (kv.head_dim == 128)
    return launch(attn_fwd_f32_kernel<128, NW>, 4 * Geo<float, 128, NW>::TILE, grid, NW * 64, p, s);
  return launch(attn_fwd_f32_kernel<64, NW>, 4 * Geo<float, 64, NW>::TILE, grid, NW * 64, p, s);
}

hipError_t launch_attn_fwd_i8qk(const wf_kv_cache& kv, AttnParams& p, void* workspace, hipStream_t s) {
  if (kv.dtype != WF_BF16 || kv.head_dim != 128) return hipErrorInvalidValue;
  const int n_tab = p.n_hist + p.n_inflight;
  const int nb = (kv.chunk_tokens + 127) / 128;
  // the K scales of every visible chunk sit in LDS after the tile stages
  const int lds = TileBytes<128, true>::LDS + (n_tab * nb * 4 + 15) / 16 * 16;
  if (n_tab * nb > 16384 || lds > 160 * 1024) return hipErrorInvalidValue;
  hipError_t e = launch_quant_i8(kv, p, workspace, s);
  if (e != hipSuccess) return e;
  constexpr int NW = 8;
  p.key_tiles = (kv.chunk_tokens + KT - 1) / KT;
  p.q_tiles = (kv.chunk_tokens + NW * 32 - 1) / (NW * 32);
  const int grid = p.n_inflight * kv.n_heads * p.q_tiles;
  return launch(attn_fwd_bf16_kernel<128, NW, true>, lds, grid, NW * 64, p, s);
}

}  // namespace wf
