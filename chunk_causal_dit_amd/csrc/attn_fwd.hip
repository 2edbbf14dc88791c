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
//   * Each wave keeps its 32 query rows as the stationary MFMA B operand.
//   * K and V^T tiles of 64 keys are staged global -> registers -> LDS with a
//     double buffer, one barrier per tile; the next tile's global loads are in
//     flight while the current tile is consumed.
//   * S^T = K Q^T on MFMA: lane (q, half) of the 32x32 output holds one query
//     and 16 keys, so the softmax row statistics need one cross-half exchange.
//     The K rows are read in a permuted order (key_of_arow) so that the 16 keys
//     of a lane come out as two runs of 8 consecutive keys, which is exactly
//     the B-operand layout of the next contraction.
//   * O^T += V^T P^T on MFMA, P taken straight from registers (bf16 for the
//     bf16 path). V is stored transposed (key-contiguous) in the cache, so the
//     A operand is one 16-byte LDS read.
//   * Online softmax in the exp2 domain with a lazily moved reference max:
//     the accumulators are rescaled only when a row's max grows by more than
//     2^8, which keeps weights <= 256 and the result exact up to rounding.
#include <cmath>

#include "wf_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int KT = 64;  // keys per tile
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kRescaleLog2 = 8.0f;

// A-operand row i of a 32-key block reads key key_of_arow(i). With the 32x32
// output layout (lane half hh, element r <-> row 8*(r/4) + 4*hh + r%4) this
// makes element r of half hh the key 16*(r/8) + 8*hh + r%8.
__device__ __forceinline__ int key_of_arow(int i) {
  const int a = i >> 3, b = (i >> 2) & 1, c = i & 3;
  return ((a >> 1) << 4) + (b << 3) + ((a & 1) << 2) + c;
}
__device__ __forceinline__ int key_of_elem(int hh, int r) { return ((r >> 3) << 4) + (hh << 3) + (r & 7); }

// XOR swizzles of 16-byte pieces inside an LDS row (low 3 bits only). The
// K swizzle gives the 8 rows read together by a lane group (rows key_of_arow)
// 8 distinct pieces; the V^T swizzle does the same for 8 consecutive rows.
__device__ __forceinline__ int swz_k(int row) { return (row & 7) ^ ((row >> 1) & 4); }
__device__ __forceinline__ int swz_v(int row) { return row & 7; }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct Work {
  int j, h, qt;
};

// Longest-first order: query chunk N-1 sees the most keys, so its tiles go first.
__device__ __forceinline__ Work decode_block(int b, int N, int H, int T) {
  const int per = H * T;
  const int cls = b / per;
  const int rem = b - cls * per;
  Work w;
  w.j = N - 1 - cls;
  w.h = rem / T;
  w.qt = rem - w.h * T;
  return w;
}

template <typename E, int D, int NW>
struct Geo {
  static constexpr int ES = sizeof(E);
  static constexpr int CK = D * ES / 16;   // 16-byte pieces per K row
  static constexpr int CV = KT * ES / 16;  // 16-byte pieces per V^T row
  static constexpr int K_BYTES = KT * D * ES;
  static constexpr int STAGE = 2 * K_BYTES;  // K tile + V^T tile
  static constexpr int LDS = 2 * STAGE;      // double buffer
  static constexpr int NT = NW * 64;
  static constexpr int NK = KT * CK / NT;
  static constexpr int NV = D * CV / NT;
  static_assert(NK * NT == KT * CK && NV * NT == D * CV, "tile must split evenly over the threads");
  static_assert(CK % 8 == 0 && CV % 8 == 0, "swizzles need >= 8 pieces per row");
};

// Global -> register -> LDS staging of one K tile and one V^T tile.
template <typename G>
struct Stager {
  u32x4 k[G::NK];
  u32x4 v[G::NV];
  __device__ __forceinline__ void load(const char* kb, const char* vb, size_t v_row_bytes, int tid) {
#pragma unroll
    for (int i = 0; i < G::NK; ++i) {
      const int id = tid + i * G::NT, row = id / G::CK, c = id % G::CK;
      k[i] = *reinterpret_cast<const u32x4*>(kb + (size_t)row * (G::CK * 16) + c * 16);
    }
#pragma unroll
    for (int i = 0; i < G::NV; ++i) {
      const int id = tid + i * G::NT, d = id / G::CV, c = id % G::CV;
      v[i] = *reinterpret_cast<const u32x4*>(vb + (size_t)d * v_row_bytes + c * 16);
    }
  }
  __device__ __forceinline__ void store(char* stage, int tid) const {
#pragma unroll
    for (int i = 0; i < G::NK; ++i) {
      const int id = tid + i * G::NT, row = id / G::CK, c = id % G::CK;
      *reinterpret_cast<u32x4*>(stage + row * (G::CK * 16) + ((c ^ swz_k(row)) << 4)) = k[i];
    }
    char* vs = stage + G::K_BYTES;
#pragma unroll
    for (int i = 0; i < G::NV; ++i) {
      const int id = tid + i * G::NT, d = id / G::CV, c = id % G::CV;
      *reinterpret_cast<u32x4*>(vs + d * (G::CV * 16) + ((c ^ swz_v(d)) << 4)) = v[i];
    }
  }
};

// Addresses of key tile kt of logical chunk cl for head h.
template <typename G, int D>
struct TileSrc {
  const char* kpool;
  const char* vpool;
  size_t slot_bytes, khead, vhead;
  const int* slots;
  __device__ __forceinline__ void at(int cl, int kt, const char*& kb, const char*& vb) const {
    const size_t base = (size_t)slots[cl] * slot_bytes;
    kb = kpool + base + khead + (size_t)kt * (KT * D * G::ES);
    vb = vpool + base + vhead + (size_t)kt * (KT * G::ES);
  }
};

extern __shared__ __attribute__((aligned(16))) char g_smem[];

// ---------------------------------------------------------------- bf16
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_bf16_kernel(wf::AttnParams p) {
  using G = Geo<__bf16, D, NW>;
  constexpr int KS = D / 16;  // MFMA steps over head_dim (16 per step)
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  char* smem = g_smem;

  const Work w = decode_block(blockIdx.x, p.n_inflight, p.n_heads, p.q_tiles);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = lane & 31, hh = lane >> 5;
  const int C = p.chunk_tokens, H = p.n_heads, s_pad = p.s_pad;
  const int wrow = w.qt * (NW * 32) + wave * 32;
  const bool wave_on = wrow < C;
  const int row = wrow + qi;
  const bool row_ok = row < C;
  const size_t qoff = (((size_t)w.j * C + row) * H + w.h) * D;

  // Stationary B operand: this lane's query row, half hh of head_dim.
  bf16x8 qop[KS];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(p.q) + qoff + hh * (D / 2));
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (row_ok) raw = qp[k];
      __builtin_memcpy(&qop[k], &raw, 16);
    }
  }

  TileSrc<G, D> src{static_cast<const char*>(p.k_pool), static_cast<const char*>(p.v_pool),
                    (size_t)p.slot_elems * G::ES, (size_t)w.h * s_pad * D * G::ES,
                    (size_t)w.h * D * s_pad * G::ES, p.slots};
  const size_t v_row_bytes = (size_t)s_pad * G::ES;
  const int ktc = p.key_tiles;
  const int n_iter = (p.n_hist + w.j + 1) * ktc;

  Stager<G> st;
  {
    const char *kb, *vb;
    src.at(0, 0, kb, vb);
    st.load(kb, vb, v_row_bytes, tid);
    st.store(smem, tid);
  }
  __syncthreads();

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  float m_ref = -INFINITY;  // reference max (log2 domain) of this lane's query row
  float lsum = 0.f;         // this half's share of the row sum of weights
  const float sl2e = p.scale_log2e;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  int cl = 0, kt = 0;
  for (int it = 0; it < n_iter; ++it) {
    const int valid = min(KT, C - kt * KT);
    int ncl = cl, nkt = kt + 1;
    if (nkt == ktc) {
      nkt = 0;
      ++ncl;
    }
    const bool more = it + 1 < n_iter;
    if (more) {
      const char *kb, *vb;
      src.at(ncl, nkt, kb, vb);
      st.load(kb, vb, v_row_bytes, tid);
    }
    const char* ks = smem + (it & 1) * G::STAGE;
    if (wave_on) {
      // S^T = K Q^T for 64 keys x 32 queries
      f32x16 s[2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[b][e] = 0.f;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int r = 32 * b + key_of_arow(qi);
          const int c = hh * KS + k;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + r * (G::CK * 16) + ((c ^ swz_k(r)) << 4));
          s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[k], s[b], 0, 0, 0);
        }
      }
      if (valid < KT) {  // zero padding past the chunk end takes no weight
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
      mx = fmaxf(mx, xor32(mx));
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
      bf16x8 pk[4];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) pk[2 * b + (e >> 3)][e & 7] = (__bf16)fast_exp2(fmaf(s[b][e], sl2e, nm));
      // row sum of the weights actually used (bf16-rounded)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e)
        {
          const bf16x2 pr = {pk[kk][2 * e], pk[kk][2 * e + 1]};
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
        }
      // O^T += V^T P^T
      const char* vs = ks + G::K_BYTES;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const int r = 32 * d + qi;
          const int c = 2 * kk + hh;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vs + r * (G::CV * 16) + ((c ^ swz_v(r)) << 4));
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kk], o[d], 0, 0, 0);
        }
      }
    }
    if (more) st.store(smem + ((it + 1) & 1) * G::STAGE, tid);
    __syncthreads();
    cl = ncl;
    kt = nkt;
  }

  if (wave_on) {
    const float lt = lsum + xor32(lsum);
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
      if (p.lse && hh == 0)
        p.lse[(size_t)w.h * p.n_inflight * C + (size_t)w.j * C + row] = (m_ref + log2f(lt)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------- fp32
// Same schedule with fp32 operands on v_mfma_f32_32x32x2_f32 (two head_dim
// or key values per instruction); weights stay fp32.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_f32_kernel(wf::AttnParams p) {
  using G = Geo<float, D, NW>;
  constexpr int DB = D / 32;
  constexpr int QP = D / 8;  // 4-float pieces in this lane's half of head_dim
  char* smem = g_smem;

  const Work w = decode_block(blockIdx.x, p.n_inflight, p.n_heads, p.q_tiles);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = lane & 31, hh = lane >> 5;
  const int C = p.chunk_tokens, H = p.n_heads, s_pad = p.s_pad;
  const int wrow = w.qt * (NW * 32) + wave * 32;
  const bool wave_on = wrow < C;
  const int row = wrow + qi;
  const bool row_ok = row < C;
  const size_t qoff = (((size_t)w.j * C + row) * H + w.h) * D;

  f32x4 qop[QP];
  {
    const f32x4* qp = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.q) + qoff + hh * (D / 2));
#pragma unroll
    for (int k = 0; k < QP; ++k) qop[k] = row_ok ? qp[k] : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  TileSrc<G, D> src{static_cast<const char*>(p.k_pool), static_cast<const char*>(p.v_pool),
                    (size_t)p.slot_elems * G::ES, (size_t)w.h * s_pad * D * G::ES,
                    (size_t)w.h * D * s_pad * G::ES, p.slots};
  const size_t v_row_bytes = (size_t)s_pad * G::ES;
  const int ktc = p.key_tiles;
  const int n_iter = (p.n_hist + w.j + 1) * ktc;

  Stager<G> st;
  {
    const char *kb, *vb;
    src.at(0, 0, kb, vb);
    st.load(kb, vb, v_row_bytes, tid);
    st.store(smem, tid);
  }
  __syncthreads();

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  float m_ref = -INFINITY, lsum = 0.f;
  const float sl2e = p.scale_log2e;

  int cl = 0, kt = 0;
  for (int it = 0; it < n_iter; ++it) {
    const int valid = min(KT, C - kt * KT);
    int ncl = cl, nkt = kt + 1;
    if (nkt == ktc) {
      nkt = 0;
      ++ncl;
    }
    const bool more = it + 1 < n_iter;
    if (more) {
      const char *kb, *vb;
      src.at(ncl, nkt, kb, vb);
      st.load(kb, vb, v_row_bytes, tid);
    }
    const char* ks = smem + (it & 1) * G::STAGE;
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
          const int r = 32 * b + key_of_arow(qi);
          const int c = hh * QP + k;
          const f32x4 a = *reinterpret_cast<const f32x4*>(ks + r * (G::CK * 16) + ((c ^ swz_k(r)) << 4));
#pragma unroll
          for (int e = 0; e < 4; ++e) s[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qop[k][e], s[b], 0, 0, 0);
        }
      }
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
      mx = fmaxf(mx, xor32(mx));
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
      const char* vs = ks + G::K_BYTES;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int d = 0; d < DB; ++d) {
            const int r = 32 * d + qi;
            const int c = 8 * b + 4 * (g >> 1) + 2 * hh + (g & 1);
            const f32x4 a = *reinterpret_cast<const f32x4*>(vs + r * (G::CV * 16) + ((c ^ swz_v(r)) << 4));
#pragma unroll
            for (int e = 0; e < 4; ++e)
              o[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], s[b][4 * g + e], o[d], 0, 0, 0);
          }
    }
    if (more) st.store(smem + ((it + 1) & 1) * G::STAGE, tid);
    __syncthreads();
    cl = ncl;
    kt = nkt;
  }

  if (wave_on) {
    const float lt = lsum + xor32(lsum);
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

template <typename Kern>
hipError_t launch(Kern k, int lds, int grid, int block, const wf::AttnParams& p, hipStream_t s) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  k<<<grid, block, lds, s>>>(p);
  return hipGetLastError();
}

}  // namespace

namespace wf {

hipError_t launch_attn_fwd(const wf_kv_cache& kv, AttnParams& p, hipStream_t s) {
  const int C = kv.chunk_tokens;
  p.key_tiles = (C + KT - 1) / KT;
  if (kv.dtype == WF_BF16) {
    constexpr int NW = 8;
    p.q_tiles = (C + NW * 32 - 1) / (NW * 32);
    const int grid = p.n_inflight * kv.n_heads * p.q_tiles;
    if (kv.head_dim == 128)
      return launch(attn_fwd_bf16_kernel<128, NW>, Geo<__bf16, 128, NW>::LDS, grid, NW * 64, p, s);
    return launch(attn_fwd_bf16_kernel<64, NW>, Geo<__bf16, 64, NW>::LDS, grid, NW * 64, p, s);
  }
  constexpr int NW = 4;
  p.q_tiles = (C + NW * 32 - 1) / (NW * 32);
  const int grid = p.n_inflight * kv.n_heads * p.q_tiles;
  if (kv.head_dim == 128) return launch(attn_fwd_f32_kernel<128, NW>, Geo<float, 128, NW>::LDS, grid, NW * 64, p, s);
  return launch(attn_fwd_f32_kernel<64, NW>, Geo<float, 64, NW>::LDS, grid, NW * 64, p, s);
}

}  // namespace wf
