// MLA prolog for MI355X (gfx950 / CDNA4): kernels and the C ABI.
//
// The operation is the Multi-Head Latent Attention prolog of the Ascend
// operator page aclnnMlaPrologV2WeightNz ("Function", formula block); the
// rotate-half RoPE is the mode the aclnnMlaPreprocess page fixes
// (constraints, rope mode).  Four stream-ordered kernels:
//
//   K1 down_proj        y = x [W^DQ | W^DKV | W^KR], split-K partials (fp32,
//                       or exact int32 in int8 mode) into the workspace
//   K2 norm_rope_cache  fixed-order split-K sum, both RmsNorms, k^R RoPE,
//                       kv/kr rows scattered at cacheIndex, c^Q emitted as
//                       bf16 (or per-token int8 + scale)
//   K3 up_proj          u = c^Q [W^UQ | W^QR] per head; nope columns -> q^C
//                       (bf16, workspace), rope columns -> RoPE -> queryRopeOut
//   K4 uk               q^N = q^C W^UK[h] per head; bf16 store, or per-(token,
//                       head) dynamic int8 with its dequantisation scale
//
// All matrix products run on MFMA (v_mfma_f32_16x16x32_bf16,
// v_mfma_i32_16x16x64_i8).  Weights are (k, n) row-major, so a weight tile is
// staged through LDS with an odd dword row stride and read back column-wise
// (one k-run of 8 or 16 elements per lane) without bank conflicts; activation
// fragments are k-contiguous and come straight from global memory.
// There are no float atomics: every reduction has a fixed order, so a run is
// deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <type_traits>

#include "../../include/mla_prolog.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves of 64

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16, round to nearest even (finite inputs; NaN stays NaN)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// symmetric int8 code of v for scale s > 0: nearest integer (ties to even)
// of v / s, kept within [-127, 127]
__device__ __forceinline__ int8_t quant_code(float v, float s) {
  float r = rintf(v / s);
  r = fminf(127.0f, fmaxf(-127.0f, r));
  return static_cast<int8_t>(r);
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum (or max) of one value per thread over the 256-thread block, in a fixed
// order; red must hold 4 floats.  Every thread gets the result.
template <bool MAX>
__device__ float block_reduce(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = MAX ? wave_max(v) : wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < 4; ++w) r = MAX ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

// ---------------------------------------------------------------------------
// MFMA tile of C[BM x BN] = A[BM x K] B[K x BN] over a k range.
//
// A: row-major, k-contiguous (activations), element size EB; each lane reads
//    its 16-byte fragment directly from global memory.
// B: row-major (k, n) weights; BK x BN stages go global -> registers -> LDS
//    (next stage prefetched into registers while the current one is used),
//    LDS rows padded to an odd number of dwords so the column-wise fragment
//    reads of the four lane groups land in distinct banks.
// Wave w owns column tiles [w*NTW, (w+1)*NTW) of 16 columns; each wave covers
// all BM = 16*MT rows.  MFMA lane layout (16x16 output): lane l holds
// column l%16 and rows 4*(l/16) + i, i < 4.
// ---------------------------------------------------------------------------
template <bool I8, int MT, int NTW, int BKS>
struct Tile {
  static constexpr int EB = I8 ? 1 : 2;          // bytes per element
  static constexpr int KM = I8 ? 64 : 32;        // k per MFMA
  static constexpr int KL = 16 / EB;             // k per lane per MFMA
  static constexpr int BM = 16 * MT;
  static constexpr int BN = 64 * NTW;
  static constexpr int BK = KM * BKS;            // B rows per stage
  static constexpr int ROW_DW = BN * EB / 4 + 1; // odd LDS row stride (dwords)
  static constexpr int CPR = BN * EB / 16;       // 16-byte chunks per B row
  static constexpr int PT = BK * CPR / kThreads; // chunks per thread per stage
  static constexpr int LDS_DW = BK * ROW_DW;
  static_assert(PT * kThreads == BK * CPR, "stage must split evenly over the block");
  using Acc = typename std::conditional<I8, i32x4, f32x4>::type;
};

template <bool I8, int MT, int NTW, int BKS>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ A, int64_t lda, int m0, int M,
                                          const uint8_t* __restrict__ B, int64_t ldb, int width,
                                          int k_begin, int k_end,
                                          typename Tile<I8, MT, NTW, BKS>::Acc (&acc)[MT][NTW],
                                          uint32_t* lds) {
  using C = Tile<I8, MT, NTW, BKS>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wbytes = width * C::EB;

  for (int mt = 0; mt < MT; ++mt)
    for (int j = 0; j < NTW; ++j)
      for (int i = 0; i < 4; ++i) acc[mt][j][i] = 0;

  uint4 pre[C::PT];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::PT; ++i) {
      const int q = tid + kThreads * i;
      const int r = q / C::CPR, ch = q % C::CPR;
      const int k = k0 + r;
      if (k < k_end && ch * 16 < wbytes)
        pre[i] = *reinterpret_cast<const uint4*>(B + static_cast<int64_t>(k) * ldb + ch * 16);
      else
        pre[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int i = 0; i < C::PT; ++i) {
      const int q = tid + kThreads * i;
      const int r = q / C::CPR, ch = q % C::CPR;
      uint32_t* d = lds + r * C::ROW_DW + ch * 4;
      d[0] = pre[i].x; d[1] = pre[i].y; d[2] = pre[i].z; d[3] = pre[i].w;
    }
  };

  load_stage(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += C::BK) {
    __syncthreads();
    store_stage();
    __syncthreads();
    if (k0 + C::BK < k_end) load_stage(k0 + C::BK);
#pragma unroll
    for (int s = 0; s < BKS; ++s) {
      const int kb = k0 + s * C::KM;
      if (kb >= k_end) break;
      // B fragments: k-run (s*KM + KL*g + i), column 16*(wave*NTW+j) + c
      typename std::conditional<I8, i32x4, bf16x8>::type bfr[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int col = 16 * (wave * NTW + j) + c;
        const int row0 = s * C::KM + C::KL * g;
        if constexpr (I8) {
          const uint8_t* l8 = reinterpret_cast<const uint8_t*>(lds);
          union { i32x4 v; uint8_t b[16]; } u;
#pragma unroll
          for (int i = 0; i < 16; ++i) u.b[i] = l8[(row0 + i) * (4 * C::ROW_DW) + col];
          bfr[j] = u.v;
        } else {
          const uint16_t* l16 = reinterpret_cast<const uint16_t*>(lds);
          union { bf16x8 v; uint16_t h[8]; } u;
#pragma unroll
          for (int i = 0; i < 8; ++i) u.h[i] = l16[(row0 + i) * (2 * C::ROW_DW) + col];
          bfr[j] = u.v;
        }
      }
      const int ka = kb + C::KL * g;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + 16 * mt + c;
        uint4 a = make_uint4(0, 0, 0, 0);
        if (m < M && ka < k_end)
          a = *reinterpret_cast<const uint4*>(A + static_cast<int64_t>(m) * lda +
                                              static_cast<int64_t>(ka) * C::EB);
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          if constexpr (I8) {
            union { uint4 u; i32x4 v; } av; av.u = a;
            acc[mt][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av.v, bfr[j], acc[mt][j], 0, 0, 0);
          } else {
            union { uint4 u; bf16x8 v; } av; av.u = a;
            acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av.v, bfr[j], acc[mt][j], 0, 0, 0);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// kernel parameters (plain values and device pointers)
// ---------------------------------------------------------------------------
struct Dims {
  int T, He, Hcq, Hckv, N, D, Dr;
  int64_t slots;  // block_num * block_size
  float eps_cq, eps_ckv;
};

struct Ptrs {
  const uint8_t* x;
  const uint8_t* w_dq;
  const uint8_t* w_uq_qr;
  const uint16_t* w_uk;
  const uint8_t* w_dkv_kr;
  const uint16_t* gamma_cq;
  const uint16_t* gamma_ckv;
  const uint16_t* sin;
  const uint16_t* cos;
  const int64_t* cache_index;
  uint16_t* kv_cache;
  uint16_t* kr_cache;
  const float* sx;
  const float* sw_dq;
  const float* sw_uq_qr;
  const float* sw_dkv_kr;
  void* q_out;
  uint16_t* qr_out;
  float* q_scale;
  // workspace
  void* part;        // [S][T][Hcq+Hckv+Dr] fp32 (int32 in int8 mode)
  uint8_t* cq;       // [T][Hcq] bf16 (int8 in int8 mode)
  float* cq_scale;   // [T]
  uint16_t* qc;      // [T][N][D] bf16
  // streaming (small-T) path
  float* y;          // [T][Hcq+Hckv+Dr] fp32: x [W^DQ | W^DkvKr], split-K reduced
  float* ssq;        // [column tile][T]: sum of squares of the tile's q or kv columns
  float* amax;       // [q column tile][T]: max |gamma_cq * y| over the tile's columns
  unsigned* ticket;  // [column tile]: split-K arrival counters, zero between runs
};

// K1 ------------------------------------------------------------------------
// grid (column tiles of [W^DQ | W^DkvKr], split, token tile)
template <bool I8, int MT>
__global__ __launch_bounds__(kThreads) void k_down_proj(Dims d, Ptrs p, int tiles_q, int kps) {
  using C = Tile<I8, MT, 1, 2>;
  __shared__ uint32_t lds[C::LDS_DW];
  const int jt = blockIdx.x, split = blockIdx.y, m0 = blockIdx.z * C::BM;
  const int Nkr = d.Hckv + d.Dr, Ntot = d.Hcq + Nkr;
  const uint8_t* B;
  int64_t ldb;
  int n0, width, outc;
  if (jt < tiles_q) {
    n0 = 64 * jt; width = min(64, d.Hcq - n0); B = p.w_dq; ldb = int64_t(d.Hcq) * C::EB; outc = n0;
  } else {
    n0 = 64 * (jt - tiles_q); width = min(64, Nkr - n0); B = p.w_dkv_kr;
    ldb = int64_t(Nkr) * C::EB; outc = d.Hcq + n0;
  }
  const int kb = split * kps, ke = min(d.He, kb + kps);
  typename C::Acc acc[MT][1];
  gemm_tile<I8, MT, 1, 2>(p.x, int64_t(d.He) * C::EB, m0, d.T, B + int64_t(n0) * C::EB, ldb, width,
                          kb, ke, acc, lds);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int col = 16 * wave + c;
  if (col >= width) return;
  for (int mt = 0; mt < MT; ++mt)
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * mt + 4 * g + i;
      if (m >= d.T) continue;
      const int64_t o = (int64_t(split) * d.T + m) * Ntot + outc + col;
      if constexpr (I8) static_cast<int32_t*>(p.part)[o] = acc[mt][0][i];
      else static_cast<float*>(p.part)[o] = acc[mt][0][i];
    }
}

// K2 ------------------------------------------------------------------------
// one block per token
template <bool I8>
__global__ __launch_bounds__(kThreads) void k_norm_rope_cache(Dims d, Ptrs p, int S) {
  extern __shared__ float y[];  // Hcq + Hckv + Dr
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int Nkr = d.Hckv + d.Dr, Ntot = d.Hcq + Nkr;
  for (int n = tid; n < Ntot; n += kThreads) {
    float v;
    if constexpr (I8) {
      const int32_t* part = static_cast<const int32_t*>(p.part);
      int32_t a = 0;
      for (int s = 0; s < S; ++s) a += part[(int64_t(s) * d.T + t) * Ntot + n];
      const float sw = n < d.Hcq ? p.sw_dq[n] : p.sw_dkv_kr[n - d.Hcq];
      v = static_cast<float>(a) * p.sx[t] * sw;
    } else {
      const float* part = static_cast<const float*>(p.part);
      v = 0.0f;
      for (int s = 0; s < S; ++s) v += part[(int64_t(s) * d.T + t) * Ntot + n];
    }
    y[n] = v;
  }
  __syncthreads();
  float sq = 0.0f, skv = 0.0f;
  for (int n = tid; n < d.Hcq; n += kThreads) sq += y[n] * y[n];
  for (int n = tid; n < d.Hckv; n += kThreads) skv += y[d.Hcq + n] * y[d.Hcq + n];
  sq = block_reduce<false>(sq, red);
  skv = block_reduce<false>(skv, red);
  const float inv_q = 1.0f / sqrtf(sq / float(d.Hcq) + d.eps_cq);
  const float inv_kv = 1.0f / sqrtf(skv / float(d.Hckv) + d.eps_ckv);

  // c^Q
  if constexpr (I8) {
    float amax = 0.0f;
    for (int n = tid; n < d.Hcq; n += kThreads) {
      const float v = bf2f(p.gamma_cq[n]) * (y[n] * inv_q);
      y[n] = v;
      amax = fmaxf(amax, fabsf(v));
    }
    amax = block_reduce<true>(amax, red);
    const float s = amax / 127.0f;
    int8_t* cq = reinterpret_cast<int8_t*>(p.cq) + int64_t(t) * d.Hcq;
    for (int n = tid; n < d.Hcq; n += kThreads) cq[n] = s > 0.0f ? quant_code(y[n], s) : 0;
    if (tid == 0) p.cq_scale[t] = s;
  } else {
    uint16_t* cq = reinterpret_cast<uint16_t*>(p.cq) + int64_t(t) * d.Hcq;
    for (int n = tid; n < d.Hcq; n += kThreads) cq[n] = f2bf(bf2f(p.gamma_cq[n]) * (y[n] * inv_q));
  }

  // c^KV and k^R into the caches
  const int64_t slot = p.cache_index[t];
  if (slot < 0 || slot >= d.slots) return;
  uint16_t* kv = p.kv_cache + slot * d.Hckv;
  for (int n = tid; n < d.Hckv; n += kThreads)
    kv[n] = f2bf(bf2f(p.gamma_ckv[n]) * (y[d.Hcq + n] * inv_kv));
  const int h = d.Dr / 2;
  const float* yr = y + d.Hcq + d.Hckv;
  const uint16_t* cs = p.cos + int64_t(t) * d.Dr;
  const uint16_t* sn = p.sin + int64_t(t) * d.Dr;
  uint16_t* kr = p.kr_cache + slot * d.Dr;
  for (int i = tid; i < h; i += kThreads) {
    const float a = yr[i], b = yr[i + h];
    kr[i] = f2bf(a * bf2f(cs[i]) - b * bf2f(sn[i]));
    kr[i + h] = f2bf(b * bf2f(cs[i + h]) + a * bf2f(sn[i + h]));
  }
}

// K3 ------------------------------------------------------------------------
// grid (head * tiles_per_head, 1, token tile); per head the tiles are the
// nope columns in chunks of 64, then the Dr rope columns
template <bool I8, int MT>
__global__ __launch_bounds__(kThreads) void k_up_proj(Dims d, Ptrs p, int nope_tiles) {
  using C = Tile<I8, MT, 1, 2>;
  __shared__ uint32_t lds[C::LDS_DW];
  __shared__ float E[C::BM][65];
  const int hp = nope_tiles + 1;
  const int h = blockIdx.x / hp, part = blockIdx.x % hp, m0 = blockIdx.z * C::BM;
  const bool rope = part == nope_tiles;
  const int W = d.N * (d.D + d.Dr);
  const int col0 = h * (d.D + d.Dr) + (rope ? d.D : 64 * part);
  const int width = rope ? d.Dr : min(64, d.D - 64 * part);
  typename C::Acc acc[MT][1];
  gemm_tile<I8, MT, 1, 2>(p.cq, int64_t(d.Hcq) * C::EB, m0, d.T, p.w_uq_qr + int64_t(col0) * C::EB,
                          int64_t(W) * C::EB, width, 0, d.Hcq, acc, lds);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c = lane & 15;
  const int col = 16 * wave + c;
  if (col < width) {
    for (int mt = 0; mt < MT; ++mt)
      for (int i = 0; i < 4; ++i) {
        const int ml = 16 * mt + 4 * g + i, m = m0 + ml;
        float v;
        if constexpr (I8) {
          v = (m < d.T) ? static_cast<float>(acc[mt][0][i]) * p.cq_scale[m] * p.sw_uq_qr[col0 + col]
                        : 0.0f;
        } else {
          v = acc[mt][0][i];
        }
        E[ml][col] = v;
      }
  }
  __syncthreads();
  if (!rope) {
    for (int idx = tid; idx < C::BM * width; idx += kThreads) {
      const int ml = idx / width, cc = idx % width, m = m0 + ml;
      if (m < d.T) p.qc[(int64_t(m) * d.N + h) * d.D + 64 * part + cc] = f2bf(E[ml][cc]);
    }
  } else {
    const int hf = d.Dr / 2;
    for (int idx = tid; idx < C::BM * hf; idx += kThreads) {
      const int ml = idx / hf, i = idx % hf, m = m0 + ml;
      if (m >= d.T) continue;
      const float a = E[ml][i], b = E[ml][i + hf];
      const uint16_t* cs = p.cos + int64_t(m) * d.Dr;
      const uint16_t* sn = p.sin + int64_t(m) * d.Dr;
      uint16_t* o = p.qr_out + (int64_t(m) * d.N + h) * d.Dr;
      o[i] = f2bf(a * bf2f(cs[i]) - b * bf2f(sn[i]));
      o[i + hf] = f2bf(b * bf2f(cs[i + hf]) + a * bf2f(sn[i + hf]));
    }
  }
}

// K4 ------------------------------------------------------------------------
// grid (head, column split, token tile)
template <int MT, int NTW, bool Q8>
__global__ __launch_bounds__(kThreads) void k_uk(Dims d, Ptrs p) {
  using C = Tile<false, MT, NTW, 1>;
  __shared__ uint32_t lds[C::LDS_DW];
  __shared__ float rmax[4][C::BM];
  const int h = blockIdx.x, cs = blockIdx.y, m0 = blockIdx.z * C::BM;
  const int c0 = cs * C::BN, width = min(C::BN, d.Hckv - c0);
  typename C::Acc acc[MT][NTW];
  gemm_tile<false, MT, NTW, 1>(reinterpret_cast<const uint8_t*>(p.qc + int64_t(h) * d.D),
                               int64_t(d.N) * d.D * 2, m0, d.T,
                               reinterpret_cast<const uint8_t*>(p.w_uk + (int64_t(h) * d.D) * d.Hckv + c0),
                               int64_t(d.Hckv) * 2, width, 0, d.D, acc, lds);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c = lane & 15;
  if constexpr (!Q8) {
    uint16_t* qo = static_cast<uint16_t*>(p.q_out);
    for (int mt = 0; mt < MT; ++mt)
      for (int j = 0; j < NTW; ++j) {
        const int col = 16 * (wave * NTW + j) + c;
        if (col >= width) continue;
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 16 * mt + 4 * g + i;
          if (m < d.T) qo[(int64_t(m) * d.N + h) * d.Hckv + c0 + col] = f2bf(acc[mt][j][i]);
        }
      }
  } else {
    // the whole Hckv row of (token, head) is in this block (c0 == 0)
    for (int mt = 0; mt < MT; ++mt)
      for (int i = 0; i < 4; ++i) {
        float mx = 0.0f;
        for (int j = 0; j < NTW; ++j) {
          const int col = 16 * (wave * NTW + j) + c;
          if (col < width) mx = fmaxf(mx, fabsf(acc[mt][j][i]));
        }
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        if (c == 0) rmax[wave][16 * mt + 4 * g + i] = mx;
      }
    __syncthreads();
    int8_t* qo = static_cast<int8_t*>(p.q_out);
    for (int mt = 0; mt < MT; ++mt)
      for (int i = 0; i < 4; ++i) {
        const int ml = 16 * mt + 4 * g + i, m = m0 + ml;
        if (m >= d.T) continue;
        const float amax = fmaxf(fmaxf(rmax[0][ml], rmax[1][ml]), fmaxf(rmax[2][ml], rmax[3][ml]));
        const float s = amax / 127.0f;
        for (int j = 0; j < NTW; ++j) {
          const int col = 16 * (wave * NTW + j) + c;
          if (col < width)
            qo[(int64_t(m) * d.N + h) * d.Hckv + col] = s > 0.0f ? quant_code(acc[mt][j][i], s) : 0;
        }
        if (wave == 0 && c == 0) p.q_scale[int64_t(m) * d.N + h] = s;
      }
  }
}

// ---------------------------------------------------------------------------
// Streaming path for small token counts (T <= 32): weight-bandwidth bound.
//
// Every wave streams its own k-stages of a 64-column weight window: a stage
// is one MFMA k-step (32 bf16 rows or 64 int8 rows, 4 KB), loaded with
// 16-byte coalesced loads into a register ring D stages deep (the activation
// fragments of the same stage travel in the same ring, so the in-order
// vector-memory counter never makes a stage wait for a later one), written
// to the wave's own 4 KB LDS buffer with an XOR swizzle, and read back as
// MFMA B fragments with the gfx950 transpose reads (ds_read_b64_tr_b16 /
// ds_read_b64_tr_b8), two per fragment.  No block barrier is needed while
// streaming; the waves of a block cover interleaved stages of one k range
// and are summed through LDS in a fixed order at the end.
//
// Transpose-read lane layout (gfx950): within each 16-lane group, lane l
// receives element l%4 (b16) or l%8 (b8) of the 8 bytes addressed by source
// lanes l/4 + 4j (b16, j < 4) or l/8 + 2j (b8, j < 8).  With source lane s
// of group g addressing row 8g + s/4 (b16) or 16g + s/2 (b8) and column
// 16*ct + 4*(s%4) (b16) or 16*ct + 8*(s%2) (b8), lane l gets column 16*ct + l
// for consecutive rows: exactly the k-run an MFMA B operand holds.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ s16x4 lds_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}
__device__ __forceinline__ i32x2 lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(p));
}

template <bool I8>
struct Stage {
  static constexpr int EB = I8 ? 1 : 2;
  static constexpr int KS = I8 ? 64 : 32;    // k rows per stage (one MFMA k-step)
  static constexpr int KL = 16 / EB;         // k per lane per MFMA
  static constexpr int RB = 64 * EB;         // bytes per stage row (64 columns)
  static constexpr int CPR = RB / 16;        // 16-byte chunks per row
  static constexpr int BYTES = KS * RB;      // 4096
  using Acc = typename std::conditional<I8, i32x4, f32x4>::type;
  using Frag = typename std::conditional<I8, i32x4, bf16x8>::type;
  // 16-byte chunk index XOR of row r: makes the transpose reads of the four
  // lane groups (and both halves of a wave) hit distinct banks
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (I8) return ((r >> 1) & 3) ^ ((r >> 4) & 1);
    else return 2 * ((r & 3) ^ ((r >> 3) & 1));
  }
  __device__ static __forceinline__ int off(int r, int chunk) { return r * RB + 16 * (chunk ^ swz(r)); }
  // B fragment of column tile ct from a stage buffer
  __device__ static __forceinline__ Frag frag(const uint8_t* buf, int lane, int ct) {
    const int g = lane >> 4, s = lane & 15;
    if constexpr (I8) {
      const int r1 = 16 * g + (s >> 1), r2 = r1 + 8, o = 8 * (s & 1);
      const i32x2 v1 = lds_tr8(buf + off(r1, ct) + o);
      const i32x2 v2 = lds_tr8(buf + off(r2, ct) + o);
      i32x4 f = {v1[0], v1[1], v2[0], v2[1]};
      return f;
    } else {
      const int r1 = 8 * g + (s >> 2), r2 = r1 + 4, ch = 2 * ct + ((s & 3) >> 1), o = 8 * (s & 1);
      const s16x4 v1 = lds_tr16(buf + off(r1, ch) + o);
      const s16x4 v2 = lds_tr16(buf + off(r2, ch) + o);
      union { s16x4 h[2]; bf16x8 v; } u;
      u.h[0] = v1; u.h[1] = v2;
      return u.v;
    }
  }
};

// Buffer loads: an offset at or past num_records returns zeros without a
// memory request, so predicated loads need no branch.  Every buffer here is
// addressed with 32-bit offsets below 2 GiB.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = static_cast<int>(bytes < int64_t(kOOB) ? bytes : int64_t(kOOB) - 1);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return __builtin_bit_cast(uint4, v);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ i32x4 mfma(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Activation operands.  A policy loads the raw 16-byte registers of the MT
// fragments of one stage (load) and turns them into MFMA A fragments (frag).

// Fragments read as stored (bf16 or int8, k-contiguous rows); rows are
// relative to the buffer base (the block's first row).
template <bool I8, int MT>
struct APlain {
  static constexpr int NR = MT;  // 16-byte registers per stage
  rsrc_t A;
  uint32_t lda;  // bytes per row
  int M;         // valid rows from the base
  __device__ __forceinline__ void load(uint4 (&r)[NR], int m0, int ka, int ke) const {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + 16 * mt;
      const bool ok = m < M && ka < ke;
      r[mt] = bload16(A, ok ? uint32_t(m) * lda + uint32_t(ka) * Stage<I8>::EB : kOOB);
    }
  }
  __device__ __forceinline__ typename Stage<I8>::Frag frag(const uint4 (&r)[NR], int mt, int) const {
    union { uint4 u; typename Stage<I8>::Frag f; } c;
    c.u = r[mt];
    return c.f;
  }
};

// c^Q fragments computed from the reduced down-projection y (fp32):
// c = (gamma * y) * inv_rms, then bf16 (nearest even), or the per-token
// int8 code nearest to c / s_cq.  gamma is loaded once per stage.
template <bool I8, int MT>
struct ACq {
  static constexpr int NY = I8 ? 4 : 2;   // 16-byte y registers per fragment
  static constexpr int NG = I8 ? 2 : 1;   // 16-byte gamma registers per stage
  static constexpr int NR = MT * NY + NG;
  rsrc_t y;        // [M][ldy] fp32
  uint32_t ldy;    // bytes per y row
  rsrc_t gamma;    // [Hcq] bf16
  int M;
  const float* inv;    // LDS, per row of the block
  const float* scale;  // LDS, per row (int8)
  __device__ __forceinline__ void load(uint4 (&r)[NR], int m0, int ka, int ke) const {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + 16 * mt;
      const bool ok = m < M && ka < ke;
#pragma unroll
      for (int i = 0; i < NY; ++i)
        r[mt * NY + i] = bload16(y, ok ? uint32_t(m) * ldy + uint32_t(ka + 4 * i) * 4 : kOOB);
    }
#pragma unroll
    for (int i = 0; i < NG; ++i)
      r[MT * NY + i] = bload16(gamma, ka < ke ? uint32_t(ka + 8 * i) * 2 : kOOB);
  }
  __device__ __forceinline__ typename Stage<I8>::Frag frag(const uint4 (&r)[NR], int mt, int ml) const {
    constexpr int NV = I8 ? 16 : 8;
    const float* yv = reinterpret_cast<const float*>(&r[mt * NY]);
    const uint16_t* gv = reinterpret_cast<const uint16_t*>(&r[MT * NY]);
    const float iv = inv[ml];
    if constexpr (I8) {
      const float sc = scale[ml];
      union { int8_t b[16]; i32x4 v; } u;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const float c = (bf2f(gv[i]) * yv[i]) * iv;
        u.b[i] = sc > 0.0f ? quant_code(c, sc) : 0;
      }
      return u.v;
    } else {
      union { uint16_t h[8]; bf16x8 v; } u;
#pragma unroll
      for (int i = 0; i < NV; ++i) u.h[i] = f2bf((bf2f(gv[i]) * yv[i]) * iv);
      return u.v;
    }
  }
};

// One wave streams stages j = 0..ns-1 (rows kfirst + j*kstep .. +KS, clipped
// to ke) of the 64-column weight window starting at byte n0b of each row of
// the weight buffer Bw (row stride ldb bytes, wbytes valid bytes per row)
// against MT activation fragments of rows m0 + 16*mt + lane%16.  The ring
// loop is straight-line: stages past the end load zeros (no memory traffic)
// and add nothing.
template <bool I8, int MT, int D, class AP>
__device__ __forceinline__ void stream_wave(const AP& ap, int m0, rsrc_t Bw, uint32_t ldb,
                                            uint32_t n0b, int wbytes, int kfirst, int kstep,
                                            int ns, int ke, typename Stage<I8>::Acc (&acc)[MT][4],
                                            uint8_t* buf) {
  using S = Stage<I8>;
  const int lane = threadIdx.x & 63;
  const int ml = lane & 15, g = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[mt][ct] = typename S::Acc{0, 0, 0, 0};

  uint4 bq[D][4];
  uint4 aq[D][AP::NR];
  auto issue = [&](uint4 (&b)[4], uint4 (&a)[AP::NR], int j) {
    const int k0 = kfirst + j * kstep;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = lane + 64 * i, r = q / S::CPR, c = q % S::CPR;
      const bool ok = j < ns && k0 + r < ke && 16 * c < wbytes;
      b[i] = bload16(Bw, ok ? uint32_t(k0 + r) * ldb + n0b + 16 * c : kOOB);
    }
    ap.load(a, m0 + ml, j < ns ? k0 + S::KL * g : ke, ke);
  };
#pragma unroll
  for (int p = 0; p < D; ++p) issue(bq[p], aq[p], p);

  const int nsr = (ns + D - 1) / D * D;
  for (int j0 = 0; j0 < nsr; j0 += D) {
#pragma unroll
    for (int p = 0; p < D; ++p) {
      const int j = j0 + p;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = lane + 64 * i, r = q / S::CPR, c = q % S::CPR;
        *reinterpret_cast<uint4*>(buf + S::off(r, c)) = bq[p][i];
      }
      typename S::Frag af[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) af[mt] = ap.frag(aq[p], mt, 16 * mt + ml);
      issue(bq[p], aq[p], j + D);
      typename S::Frag bf[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) bf[ct] = S::frag(buf, lane, ct);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[mt][ct] = mfma(af[mt], bf[ct], acc[mt][ct]);
    }
  }
}

// Sum of the NW waves' accumulators into wave 0, in a fixed pairing order.
// red: (NW/2) * MT * 16 * 64 words of LDS.  Ends with a block barrier.
template <int NW, int MT, class Acc>
__device__ __forceinline__ void reduce_waves(Acc (&acc)[MT][4], uint32_t* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int half = NW / 2; half >= 1; half /= 2) {
    __syncthreads();
    if (w >= half && w < 2 * half) {
      uint32_t* r = red + (w - half) * (MT * 16 * 64);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // copy the vector element to a scalar first: bit-casting the
            // element expression itself reads element 0
            const auto e = acc[mt][ct][i];
            r[((mt * 4 + ct) * 4 + i) * 64 + lane] = __builtin_bit_cast(uint32_t, e);
          }
    }
    __syncthreads();
    if (w < half) {
      const uint32_t* r = red + w * (MT * 16 * 64);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            using E = decltype(acc[mt][ct][i] + 0);
            const E add = __builtin_bit_cast(E, r[((mt * 4 + ct) * 4 + i) * 64 + lane]);
            acc[mt][ct][i] += add;
          }
    }
  }
  __syncthreads();
}

template <bool I8, int MT, int NW>
struct StreamLds {
  static constexpr int STAGE = NW * Stage<I8>::BYTES;
  static constexpr int RED = (NW / 2) * MT * 16 * 64 * 4;
  static constexpr int BYTES = STAGE > RED ? STAGE : RED;
};

// K1s: grid (column tiles x splits).  The block streams its k range of one
// 64-column window of [W^DQ | W^DkvKr] and writes a partial tile; the last
// block of a column tile to arrive sums the S partials in split order into y
// and writes the tile's per-token statistics.
template <bool I8, int MT, int NW, int D>
__global__ __launch_bounds__(64 * NW) void k1_stream(Dims d, Ptrs p, int tiles_q, int tiles, int S,
                                                     int kps) {
  using St = Stage<I8>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[StreamLds<I8, MT, NW>::BYTES];
  __shared__ int last;
  const int jt = blockIdx.x % tiles, split = blockIdx.x / tiles;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Nkr = d.Hckv + d.Dr, Ntot = d.Hcq + Nkr;
  const uint8_t* B;
  int64_t ldb;
  int n0, width, outc;
  if (jt < tiles_q) {
    n0 = 64 * jt; width = min(64, d.Hcq - n0); B = p.w_dq; ldb = int64_t(d.Hcq) * St::EB; outc = n0;
  } else {
    n0 = 64 * (jt - tiles_q); width = min(64, Nkr - n0); B = p.w_dkv_kr;
    ldb = int64_t(Nkr) * St::EB; outc = d.Hcq + n0;
  }
  const int kb = split * kps, ke = min(d.He, kb + kps);
  const int nst = (ke - kb + St::KS - 1) / St::KS;
  const int ns = w < nst ? (nst - w + NW - 1) / NW : 0;
  typename St::Acc acc[MT][4];
  const APlain<I8, MT> ap{make_rsrc(p.x, int64_t(d.T) * d.He * St::EB), uint32_t(d.He * St::EB), d.T};
  const rsrc_t Bw = make_rsrc(B, int64_t(d.He) * ldb);
  stream_wave<I8, MT, D>(ap, 0, Bw, uint32_t(ldb), uint32_t(n0 * St::EB), width * St::EB,
                         kb + w * St::KS, NW * St::KS, ns, ke, acc, lds + w * St::BYTES);
  reduce_waves<NW, MT>(acc, reinterpret_cast<uint32_t*>(lds));

  // partial tile, written by wave 0
  if (w == 0) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int col = 16 * ct + c;
        if (col >= width) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 16 * mt + 4 * g + i;
          if (m >= d.T) continue;
          const int64_t o = (int64_t(split) * d.T + m) * Ntot + outc + col;
          if constexpr (I8) static_cast<int32_t*>(p.part)[o] = acc[mt][ct][i];
          else static_cast<float*>(p.part)[o] = acc[mt][ct][i];
        }
      }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) last = atomicAdd(&p.ticket[jt], 1u) == unsigned(S - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();

  // the last arrival: y = sum of the partials (split order), and statistics.
  // 16 threads per row, 4 columns each, 4*NW rows per pass; the partials of
  // 8 splits are loaded before they are added (splits past S read as zeros).
  const rsrc_t P = make_rsrc(p.part, int64_t(S) * d.T * Ntot * 4);
  const int cq = 4 * (tid & 15);
  const bool col_ok = cq < width;
  for (int m = tid >> 4; m < 16 * MT; m += 4 * NW) {
    const bool row_ok = m < d.T;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int32_t iv[4] = {0, 0, 0, 0};
    for (int s0 = 0; s0 < S; s0 += 8) {
      uint4 r[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sp = s0 + e;
        const bool ok = row_ok && col_ok && sp < S;
        r[e] = bload16(P, ok ? uint32_t(((int64_t(sp) * d.T + m) * Ntot + outc + cq) * 4) : kOOB);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (I8) {
          const int4 q = __builtin_bit_cast(int4, r[e]);
          iv[0] += q.x; iv[1] += q.y; iv[2] += q.z; iv[3] += q.w;
        } else {
          const float4 q = __builtin_bit_cast(float4, r[e]);
          v[0] += q.x; v[1] += q.y; v[2] += q.z; v[3] += q.w;
        }
      }
    }
    float ss = 0.0f, am = 0.0f;
    if (row_ok && col_ok) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gc = outc + cq + e;   // column of y
        if constexpr (I8) {
          const float sw = gc < d.Hcq ? p.sw_dq[gc] : p.sw_dkv_kr[gc - d.Hcq];
          v[e] = static_cast<float>(iv[e]) * p.sx[m] * sw;
        }
        if (gc < d.Hcq + d.Hckv) ss += v[e] * v[e];
        if (gc < d.Hcq) am = fmaxf(am, fabsf(bf2f(p.gamma_cq[gc]) * v[e]));
      }
      *reinterpret_cast<float4*>(p.y + int64_t(m) * Ntot + outc + cq) = make_float4(v[0], v[1], v[2], v[3]);
    }
    for (int o = 1; o < 16; o <<= 1) {
      ss += __shfl_xor(ss, o, 64);
      am = fmaxf(am, __shfl_xor(am, o, 64));
    }
    if ((tid & 15) == 0 && row_ok) {
      p.ssq[int64_t(jt) * d.T + m] = ss;
      if (jt < tiles_q) p.amax[int64_t(jt) * d.T + m] = am;
    }
  }
  if (tid == 0) p.ticket[jt] = 0u;
}

// Per-token RmsNorm factors of the query rows: inv = 1/sqrt(sum ssq / Hcq + eps)
// (tiles summed in order), and in int8 mode the c^Q scale max|c| / 127.
template <bool I8>
__device__ __forceinline__ void cq_factors(const Dims& d, const Ptrs& p, int tiles_q, int m,
                                           float& inv, float& scale) {
  float ss = 0.0f, am = 0.0f;
  for (int jt = 0; jt < tiles_q; ++jt) {
    ss += p.ssq[int64_t(jt) * d.T + m];
    if constexpr (I8) am = fmaxf(am, p.amax[int64_t(jt) * d.T + m]);
  }
  inv = 1.0f / sqrtf(ss / float(d.Hcq) + d.eps_cq);
  scale = I8 ? (am * inv) / 127.0f : 0.0f;
}

// K3s: grid (head tiles + kv blocks).  Head tiles: per head the nope columns
// in windows of 64, then the Dr rope columns; the block's waves split the
// whole Hcq reduction.  kv blocks: RmsNorm of c^KV and RoPE of k^R for
// kv_tpb tokens each, written at their cacheIndex slots.
template <bool I8, int MT, int NW, int D>
__global__ __launch_bounds__(64 * NW) void k3_stream(Dims d, Ptrs p, int nope_tiles, int tiles_q,
                                                     int tiles_kr, int head_blocks, int kv_tpb) {
  using St = Stage<I8>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[StreamLds<I8, MT, NW>::BYTES];
  __shared__ float inv_s[16 * MT], scale_s[16 * MT];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Nkr = d.Hckv + d.Dr, Ntot = d.Hcq + Nkr;

  if (int(blockIdx.x) >= head_blocks) {
    // c^KV and k^R for tokens [t0, t0 + kv_tpb)
    const int t0 = (blockIdx.x - head_blocks) * kv_tpb;
    for (int t = t0; t < min(d.T, t0 + kv_tpb); ++t) {
      const int64_t slot = p.cache_index[t];
      if (slot < 0 || slot >= d.slots) continue;
      float ss = 0.0f;
      for (int jt = tiles_q; jt < tiles_q + tiles_kr; ++jt) ss += p.ssq[int64_t(jt) * d.T + t];
      const float inv = 1.0f / sqrtf(ss / float(d.Hckv) + d.eps_ckv);
      const float* yk = p.y + int64_t(t) * Ntot + d.Hcq;
      uint16_t* kv = p.kv_cache + slot * d.Hckv;
      for (int n = tid; n < d.Hckv; n += 64 * NW) kv[n] = f2bf((bf2f(p.gamma_ckv[n]) * yk[n]) * inv);
      const int h = d.Dr / 2;
      const float* yr = yk + d.Hckv;
      const uint16_t* cs = p.cos + int64_t(t) * d.Dr;
      const uint16_t* sn = p.sin + int64_t(t) * d.Dr;
      uint16_t* kr = p.kr_cache + slot * d.Dr;
      for (int i = tid; i < h; i += 64 * NW) {
        const float a = yr[i], b = yr[i + h];
        kr[i] = f2bf(a * bf2f(cs[i]) - b * bf2f(sn[i]));
        kr[i + h] = f2bf(b * bf2f(cs[i + h]) + a * bf2f(sn[i + h]));
      }
    }
    return;
  }

  const int hp = nope_tiles + 1;
  const int h = blockIdx.x / hp, part = blockIdx.x % hp;
  const bool rope = part == nope_tiles;
  const int W = d.N * (d.D + d.Dr);
  const int col0 = h * (d.D + d.Dr) + (rope ? d.D : 64 * part);
  const int width = rope ? d.Dr : min(64, d.D - 64 * part);
  for (int m = tid; m < 16 * MT; m += 64 * NW) {
    float iv = 0.0f, sc = 0.0f;
    if (m < d.T) cq_factors<I8>(d, p, tiles_q, m, iv, sc);
    inv_s[m] = iv;
    scale_s[m] = sc;
  }
  __syncthreads();
  const int nst = (d.Hcq + St::KS - 1) / St::KS;
  const int ns = w < nst ? (nst - w + NW - 1) / NW : 0;
  typename St::Acc acc[MT][4];
  const ACq<I8, MT> ap{make_rsrc(p.y, int64_t(d.T) * Ntot * 4), uint32_t(Ntot * 4),
                       make_rsrc(p.gamma_cq, int64_t(d.Hcq) * 2), d.T, inv_s, scale_s};
  const rsrc_t Bw = make_rsrc(p.w_uq_qr, int64_t(d.Hcq) * W * St::EB);
  stream_wave<I8, MT, D>(ap, 0, Bw, uint32_t(W * St::EB), uint32_t(col0 * St::EB), width * St::EB,
                         w * St::KS, NW * St::KS, ns, d.Hcq, acc, lds + w * St::BYTES);
  reduce_waves<NW, MT>(acc, reinterpret_cast<uint32_t*>(lds));

  // epilogue: the reduced tile goes to LDS (fp32), then out
  float* E = reinterpret_cast<float*>(lds);   // [16*MT][65]
  if (w == 0) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ml = 16 * mt + 4 * g + i, col = 16 * ct + c;
          float v;
          if constexpr (I8)
            v = (ml < d.T && col < width)
                    ? static_cast<float>(acc[mt][ct][i]) * scale_s[ml] * p.sw_uq_qr[col0 + col]
                    : 0.0f;
          else
            v = acc[mt][ct][i];
          E[ml * 65 + col] = v;
        }
  }
  __syncthreads();
  const int BM = 16 * MT;
  if (!rope) {
    for (int idx = tid; idx < BM * width; idx += 64 * NW) {
      const int ml = idx / width, cc = idx % width;
      if (ml < d.T) p.qc[(int64_t(ml) * d.N + h) * d.D + 64 * part + cc] = f2bf(E[ml * 65 + cc]);
    }
  } else {
    const int hf = d.Dr / 2;
    for (int idx = tid; idx < BM * hf; idx += 64 * NW) {
      const int ml = idx / hf, i = idx % hf;
      if (ml >= d.T) continue;
      const float a = E[ml * 65 + i], b = E[ml * 65 + i + hf];
      const uint16_t* cs = p.cos + int64_t(ml) * d.Dr;
      const uint16_t* sn = p.sin + int64_t(ml) * d.Dr;
      uint16_t* o = p.qr_out + (int64_t(ml) * d.N + h) * d.Dr;
      o[i] = f2bf(a * bf2f(cs[i]) - b * bf2f(sn[i]));
      o[i + hf] = f2bf(b * bf2f(cs[i + hf]) + a * bf2f(sn[i + hf]));
    }
  }
}

// K4s, bf16 query: grid (head x 64-column window of Hckv); the block's waves
// split the D reduction.
template <int MT, int NW, int D>
__global__ __launch_bounds__(64 * NW) void k4_stream(Dims d, Ptrs p, int windows) {
  using St = Stage<false>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[StreamLds<false, MT, NW>::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x / windows, win = blockIdx.x % windows;
  const int c0 = 64 * win, width = min(64, d.Hckv - c0);
  const int nst = (d.D + St::KS - 1) / St::KS;
  const int ns = w < nst ? (nst - w + NW - 1) / NW : 0;
  typename St::Acc acc[MT][4];
  const APlain<false, MT> ap{make_rsrc(p.qc + int64_t(h) * d.D, (int64_t(d.T) * d.N - h) * d.D * 2),
                             uint32_t(d.N * d.D * 2), d.T};
  const rsrc_t Bw = make_rsrc(p.w_uk + int64_t(h) * d.D * d.Hckv, int64_t(d.D) * d.Hckv * 2);
  stream_wave<false, MT, D>(ap, 0, Bw, uint32_t(d.Hckv * 2), uint32_t(c0 * 2), width * 2,
                            w * St::KS, NW * St::KS, ns, d.D, acc, lds + w * St::BYTES);
  reduce_waves<NW, MT>(acc, reinterpret_cast<uint32_t*>(lds));
  // stage the tile through LDS as bf16, then 16-byte stores
  uint16_t* E = reinterpret_cast<uint16_t*>(lds);  // [16*MT][64]
  if (w == 0) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) E[(16 * mt + 4 * g + i) * 64 + 16 * ct + c] = f2bf(acc[mt][ct][i]);
  }
  __syncthreads();
  uint16_t* qo = static_cast<uint16_t*>(p.q_out);
  for (int idx = tid; idx < 16 * MT * 8; idx += 64 * NW) {
    const int ml = idx / 8, ch = idx % 8;
    if (ml < d.T && 8 * ch < width)
      *reinterpret_cast<uint4*>(qo + (int64_t(ml) * d.N + h) * d.Hckv + c0 + 8 * ch) =
          *reinterpret_cast<const uint4*>(E + ml * 64 + 8 * ch);
  }
}

// K4s, int8 query: grid (head); wave w owns the 64-column window w of Hckv
// (Hckv <= 512) over the whole D reduction; the row maximum is taken across
// the waves.
template <int MT, int D>
__global__ __launch_bounds__(512) void k4_stream_q8(Dims d, Ptrs p) {
  using St = Stage<false>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[8 * St::BYTES];
  __shared__ float rmax[8][16 * MT];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x;
  const int c0 = 64 * w, width = max(0, min(64, d.Hckv - c0));
  const int nst = (d.D + St::KS - 1) / St::KS;
  const int ns = width > 0 ? nst : 0;
  typename St::Acc acc[MT][4];
  const APlain<false, MT> ap{make_rsrc(p.qc + int64_t(h) * d.D, (int64_t(d.T) * d.N - h) * d.D * 2),
                             uint32_t(d.N * d.D * 2), d.T};
  const rsrc_t Bw = make_rsrc(p.w_uk + int64_t(h) * d.D * d.Hckv, int64_t(d.D) * d.Hckv * 2);
  stream_wave<false, MT, D>(ap, 0, Bw, uint32_t(d.Hckv * 2), uint32_t(max(0, c0) * 2), width * 2,
                            0, St::KS, ns, d.D, acc, lds + w * St::BYTES);
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = 0.0f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (16 * ct + c < width) mx = fmaxf(mx, fabsf(acc[mt][ct][i]));
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      if (c == 0) rmax[w][16 * mt + 4 * g + i] = mx;
    }
  __syncthreads();
  int8_t* qo = static_cast<int8_t*>(p.q_out);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ml = 16 * mt + 4 * g + i;
      if (ml >= d.T) continue;
      float amax = rmax[0][ml];
      for (int ww = 1; ww < 8; ++ww) amax = fmaxf(amax, rmax[ww][ml]);
      const float s = amax / 127.0f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int col = 16 * ct + c;
        if (col < width)
          qo[(int64_t(ml) * d.N + h) * d.Hckv + c0 + col] = s > 0.0f ? quant_code(acc[mt][ct][i], s) : 0;
      }
      if (w == 0 && c == 0) p.q_scale[int64_t(ml) * d.N + h] = s;
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Token counts up to this run on the streaming kernels.
constexpr int kStreamMaxT = 32;
constexpr int kStreamWaves = 4;

struct Plan {
  bool stream;       // small-T streaming path
  int mt1, S, kps;   // K1 rows per tile (16*mt1), split count, k per split
  int mt3;           // K3
  int ntw4, cs4;     // K4 column tiles per wave, column splits
};

int ceil_div(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

int mt_for(int64_t T, int cap) {
  int mt = 1;
  while (mt < cap && 16 * mt < T) mt *= 2;
  return mt;
}

int column_tiles(const mla_prolog_desc& d) { return ceil_div(d.Hcq, 64) + ceil_div(d.Hckv + d.Dr, 64); }

Plan make_plan(const mla_prolog_desc& d, int64_t T) {
  Plan pl;
  const bool i8 = d.in_dtype == MLA_INT8;
  pl.stream = T <= kStreamMaxT;
  if (pl.stream) {
    // about two blocks of 8 waves per CU over the column tiles x splits
    const int ks = i8 ? 64 : 32;
    const int tiles = column_tiles(d);
    const int nst = ceil_div(d.He, ks);
    int S = std::max(1, std::min(nst, (512 + tiles / 2) / tiles));
    pl.kps = ceil_div(nst, S) * ks;
    pl.S = ceil_div(d.He, pl.kps);
    pl.mt1 = T <= 16 ? 1 : 2;
    pl.mt3 = pl.mt1;
    pl.ntw4 = pl.cs4 = 0;
    return pl;
  }
  const int bk = i8 ? 128 : 64;
  pl.mt1 = mt_for(T, 16);
  const int col_tiles = ceil_div(d.Hcq, 64) + ceil_div(d.Hckv + d.Dr, 64);
  const int m_tiles = ceil_div(T, 16 * pl.mt1);
  const int kchunks = ceil_div(d.He, bk);
  int S = 1;
  if (T < 512) {
    S = std::max(1, 512 / std::max(1, col_tiles * m_tiles));
    S = std::min(S, std::min(16, kchunks));
  }
  pl.kps = ceil_div(kchunks, S) * bk;
  pl.S = ceil_div(d.He, pl.kps);
  pl.mt3 = mt_for(T, 8);
  int need = ceil_div(d.Hckv, 64), ntw = 1;
  while (ntw < need && ntw < 8) ntw *= 2;
  if (d.query_dtype == MLA_BF16 && d.Hckv > 256) ntw = 4;
  pl.ntw4 = ntw;
  pl.cs4 = ceil_div(d.Hckv, 64 * ntw);
  return pl;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct Layout {
  size_t part, cq, cq_scale, qc, y, ssq, amax, ticket, total;
};

Layout layout(const mla_prolog_desc& d) {
  Layout L;
  const int64_t Ntot = d.Hcq + d.Hckv + d.Dr;
  int64_t part_rows = 0;
  // the largest S*T over all T <= max_tokens
  for (int64_t T = 1; T <= d.max_tokens; ++T) {
    const Plan pl = make_plan(d, T);
    part_rows = std::max<int64_t>(part_rows, int64_t(pl.S) * T);
    if (T >= 512) { part_rows = std::max<int64_t>(part_rows, d.max_tokens); break; }
  }
  L.part = 0;
  L.cq = align256(L.part + size_t(part_rows) * Ntot * 4);
  L.cq_scale = align256(L.cq + size_t(d.max_tokens) * d.Hcq * 2);
  L.qc = align256(L.cq_scale + size_t(d.max_tokens) * 4);
  const int64_t Ts = std::min<int64_t>(d.max_tokens, kStreamMaxT);
  const int tiles = column_tiles(d);
  L.y = align256(L.qc + size_t(d.max_tokens) * d.N * d.D * 2);
  L.ssq = align256(L.y + size_t(Ts) * Ntot * 4);
  L.amax = align256(L.ssq + size_t(tiles) * Ts * 4);
  L.ticket = align256(L.amax + size_t(tiles) * Ts * 4);
  L.total = align256(L.ticket + size_t(tiles) * 4);
  return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

mla_status check_desc(const mla_prolog_desc* d) {
  if (!d) return MLA_ERR_NULLPTR;
  const int64_t dims[6] = {d->He, d->Hcq, d->Hckv, d->N, d->D, d->Dr};
  for (int64_t v : dims)
    if (v <= 0 || v > (1 << 20)) return MLA_ERR_PARAM_INVALID;
  // the page's dtype table has an int8 queryOut only in the int8
  // full-quantisation scenario
  if ((d->in_dtype != MLA_BF16 && d->in_dtype != MLA_INT8) ||
      (d->query_dtype != MLA_BF16 && d->query_dtype != MLA_INT8))
    return MLA_ERR_PARAM_INVALID;
  if (d->query_dtype == MLA_INT8 && d->in_dtype != MLA_INT8) return MLA_ERR_PARAM_INVALID;
  if (d->block_num < 0 || d->max_tokens < 0 || d->max_tokens > (1 << 20))
    return MLA_ERR_PARAM_INVALID;
  if (d->block_num > 0 && (d->block_size < 16 || d->block_size > 1024 || d->block_size % 16))
    return MLA_ERR_PARAM_INVALID;
  if (!(d->eps_cq >= 0.0) || !(d->eps_ckv >= 0.0) || !std::isfinite(d->eps_cq) ||
      !std::isfinite(d->eps_ckv))
    return MLA_ERR_PARAM_INVALID;
  const int64_t vec_dims[5] = {d->He, d->Hcq, d->Hckv, d->D, d->Dr};
  for (int64_t v : vec_dims)
    if (v % 8) return MLA_ERR_UNSUPPORTED;
  if (d->Dr > 64 || d->Hckv > 512 || d->D > 512 || d->Hcq > 8192 || d->He > 65536)
    return MLA_ERR_UNSUPPORTED;
  // int8 operands move in 16-byte (16-element) chunks that must not cross a
  // row or column-block end
  if (d->in_dtype == MLA_INT8 &&
      (d->He % 16 || d->Hcq % 16 || (d->Hckv + d->Dr) % 16 || d->D % 16 || d->Dr % 16))
    return MLA_ERR_UNSUPPORTED;
  if (d->N * (d->D + d->Dr) > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

mla_status check_tensors(const mla_prolog_desc* d, const mla_prolog_tensors* t, int64_t T) {
  if (T < 0 || T > d->max_tokens) return MLA_ERR_PARAM_INVALID;
  if (!t) return MLA_ERR_NULLPTR;
  if (T == 0) return MLA_OK;
  const void* req[] = {t->token_x, t->weight_dq, t->weight_uq_qr, t->weight_uk, t->weight_dkv_kr,
                       t->gamma_cq, t->gamma_ckv, t->rope_sin, t->rope_cos, t->cache_index,
                       t->query_out, t->query_rope_out};
  for (const void* q : req)
    if (!q) return MLA_ERR_NULLPTR;
  for (const void* q : req)
    if (!aligned16(q)) return MLA_ERR_PARAM_INVALID;
  if (d->block_num > 0) {
    if (!t->kv_cache || !t->kr_cache) return MLA_ERR_NULLPTR;
    if (!aligned16(t->kv_cache) || !aligned16(t->kr_cache)) return MLA_ERR_PARAM_INVALID;
  }
  const float* sc[] = {t->scale_x, t->scale_w_dq, t->scale_w_uq_qr, t->scale_w_dkv_kr};
  for (const float* q : sc) {
    if (d->in_dtype == MLA_INT8 && !q) return MLA_ERR_NULLPTR;
    if (d->in_dtype == MLA_BF16 && q) return MLA_ERR_PARAM_INVALID;
    if (q && !aligned4(q)) return MLA_ERR_PARAM_INVALID;
  }
  if (d->query_dtype == MLA_INT8 && !t->dequant_scale_q_nope) return MLA_ERR_NULLPTR;
  if (d->query_dtype == MLA_BF16 && t->dequant_scale_q_nope) return MLA_ERR_PARAM_INVALID;
  if (t->dequant_scale_q_nope && !aligned4(t->dequant_scale_q_nope)) return MLA_ERR_PARAM_INVALID;
  return MLA_OK;
}

}  // namespace

constexpr int kProfileRing = 2048;
constexpr int kProfileEvents = 5;

struct mla_prolog {
  mla_prolog_desc desc;
  Layout lay;
  uint8_t* ws;
  hipEvent_t* events;  // kProfileRing x kProfileEvents when profiling, else NULL
  int64_t recorded;    // runs recorded since the last read
};

namespace {

template <bool I8>
void launch_k1(int mt, dim3 grid, hipStream_t s, const Dims& d, const Ptrs& p, int tq, int kps) {
  switch (mt) {
    case 1: k_down_proj<I8, 1><<<grid, kThreads, 0, s>>>(d, p, tq, kps); break;
    case 2: k_down_proj<I8, 2><<<grid, kThreads, 0, s>>>(d, p, tq, kps); break;
    case 4: k_down_proj<I8, 4><<<grid, kThreads, 0, s>>>(d, p, tq, kps); break;
    case 8: k_down_proj<I8, 8><<<grid, kThreads, 0, s>>>(d, p, tq, kps); break;
    default: k_down_proj<I8, 16><<<grid, kThreads, 0, s>>>(d, p, tq, kps); break;
  }
}

template <bool I8>
void launch_k3(int mt, dim3 grid, hipStream_t s, const Dims& d, const Ptrs& p, int nt) {
  switch (mt) {
    case 1: k_up_proj<I8, 1><<<grid, kThreads, 0, s>>>(d, p, nt); break;
    case 2: k_up_proj<I8, 2><<<grid, kThreads, 0, s>>>(d, p, nt); break;
    case 4: k_up_proj<I8, 4><<<grid, kThreads, 0, s>>>(d, p, nt); break;
    default: k_up_proj<I8, 8><<<grid, kThreads, 0, s>>>(d, p, nt); break;
  }
}

template <bool Q8>
void launch_k4(int ntw, dim3 grid, hipStream_t s, const Dims& d, const Ptrs& p) {
  switch (ntw) {
    case 1: k_uk<2, 1, Q8><<<grid, kThreads, 0, s>>>(d, p); break;
    case 2: k_uk<2, 2, Q8><<<grid, kThreads, 0, s>>>(d, p); break;
    case 4: k_uk<2, 4, Q8><<<grid, kThreads, 0, s>>>(d, p); break;
    default: k_uk<2, 8, Q8><<<grid, kThreads, 0, s>>>(d, p); break;
  }
}

template <bool I8, int MT>
void stream_k1k3(const Plan& pl, hipStream_t s, const Dims& d, const Ptrs& p) {
  constexpr int D = I8 ? 2 : 4;
  const int tiles_q = ceil_div(d.Hcq, 64), tiles_kr = ceil_div(d.Hckv + d.Dr, 64);
  const int tiles = tiles_q + tiles_kr;
  k1_stream<I8, MT, kStreamWaves, D><<<dim3(tiles * pl.S), 64 * kStreamWaves, 0, s>>>(
      d, p, tiles_q, tiles, pl.S, pl.kps);
}

template <bool I8, int MT>
void stream_k3(hipStream_t s, const Dims& d, const Ptrs& p) {
  constexpr int D = I8 ? 2 : 3;
  const int tiles_q = ceil_div(d.Hcq, 64), tiles_kr = ceil_div(d.Hckv + d.Dr, 64);
  const int nope_tiles = ceil_div(d.D, 64);
  const int head_blocks = d.N * (nope_tiles + 1);
  const int kv_tpb = 4;
  const int kv_blocks = ceil_div(d.T, kv_tpb);
  k3_stream<I8, MT, kStreamWaves, D><<<dim3(head_blocks + kv_blocks), 64 * kStreamWaves, 0, s>>>(
      d, p, nope_tiles, tiles_q, tiles_kr, head_blocks, kv_tpb);
}

template <int MT>
void stream_k4(hipStream_t s, const Dims& d, const Ptrs& p, bool q8) {
  if (q8) {
    k4_stream_q8<MT, 2><<<dim3(d.N), 512, 0, s>>>(d, p);
  } else {
    const int windows = ceil_div(d.Hckv, 64);
    k4_stream<MT, 4, 1><<<dim3(d.N * windows), 256, 0, s>>>(d, p, windows);
  }
}

template <class Mark>
void launch_stream(const Plan& pl, hipStream_t s, const Dims& d, const Ptrs& p, bool i8, bool q8,
                   Mark& mark) {
  if (pl.mt1 == 1) {
    if (i8) stream_k1k3<true, 1>(pl, s, d, p); else stream_k1k3<false, 1>(pl, s, d, p);
  } else {
    if (i8) stream_k1k3<true, 2>(pl, s, d, p); else stream_k1k3<false, 2>(pl, s, d, p);
  }
  mark(1);
  mark(2);
  if (pl.mt1 == 1) {
    if (i8) stream_k3<true, 1>(s, d, p); else stream_k3<false, 1>(s, d, p);
  } else {
    if (i8) stream_k3<true, 2>(s, d, p); else stream_k3<false, 2>(s, d, p);
  }
  mark(3);
  if (pl.mt1 == 1) stream_k4<1>(s, d, p, q8); else stream_k4<2>(s, d, p, q8);
  mark(4);
}

}  // namespace

extern "C" {

mla_status mla_prolog_validate(const mla_prolog_desc* desc, const mla_prolog_tensors* tensors,
                               int64_t T) {
  mla_status st = check_desc(desc);
  if (st != MLA_OK || !tensors) return st;
  return check_tensors(desc, tensors, T);
}

size_t mla_prolog_workspace_bytes(const mla_prolog_desc* desc) {
  if (check_desc(desc) != MLA_OK) return 0;
  return layout(*desc).total;
}

mla_status mla_prolog_create(const mla_prolog_desc* desc, mla_prolog_t* out) {
  if (!out) return MLA_ERR_NULLPTR;
  *out = nullptr;
  mla_status st = check_desc(desc);
  if (st != MLA_OK) return st;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_RUNTIME;
  if (hipSetDevice(desc->device) != hipSuccess) return MLA_ERR_PARAM_INVALID;
  mla_prolog* h = new (std::nothrow) mla_prolog;
  if (!h) { (void)hipSetDevice(prev); return MLA_ERR_RUNTIME; }
  h->desc = *desc;
  h->lay = layout(*desc);
  h->ws = nullptr;
  h->events = nullptr;
  h->recorded = 0;
  if (hipMalloc(&h->ws, h->lay.total) != hipSuccess) {
    delete h;
    (void)hipSetDevice(prev);
    return MLA_ERR_RUNTIME;
  }
  // split-K arrival counters start at zero; every run leaves them at zero
  if (hipMemset(h->ws + h->lay.ticket, 0, h->lay.total - h->lay.ticket) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(h->ws);
    delete h;
    (void)hipSetDevice(prev);
    return MLA_ERR_RUNTIME;
  }
  (void)hipSetDevice(prev);
  *out = h;
  return MLA_OK;
}

mla_status mla_prolog_run(mla_prolog_t h, const mla_prolog_tensors* t, int64_t T, void* stream) {
  if (!h) return MLA_ERR_NULLPTR;
  const mla_prolog_desc& dd = h->desc;
  mla_status st = check_tensors(&dd, t, T);
  if (st != MLA_OK) return st;
  if (T == 0) return MLA_OK;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_RUNTIME;
  if (prev != dd.device && hipSetDevice(dd.device) != hipSuccess) return MLA_ERR_RUNTIME;
  (void)hipGetLastError();

  const bool i8 = dd.in_dtype == MLA_INT8, q8 = dd.query_dtype == MLA_INT8;
  const Plan pl = make_plan(dd, T);
  Dims d;
  d.T = int(T); d.He = int(dd.He); d.Hcq = int(dd.Hcq); d.Hckv = int(dd.Hckv); d.N = int(dd.N);
  d.D = int(dd.D); d.Dr = int(dd.Dr);
  d.slots = dd.block_num * dd.block_size;
  d.eps_cq = float(dd.eps_cq); d.eps_ckv = float(dd.eps_ckv);
  Ptrs p;
  p.x = static_cast<const uint8_t*>(t->token_x);
  p.w_dq = static_cast<const uint8_t*>(t->weight_dq);
  p.w_uq_qr = static_cast<const uint8_t*>(t->weight_uq_qr);
  p.w_uk = static_cast<const uint16_t*>(t->weight_uk);
  p.w_dkv_kr = static_cast<const uint8_t*>(t->weight_dkv_kr);
  p.gamma_cq = static_cast<const uint16_t*>(t->gamma_cq);
  p.gamma_ckv = static_cast<const uint16_t*>(t->gamma_ckv);
  p.sin = static_cast<const uint16_t*>(t->rope_sin);
  p.cos = static_cast<const uint16_t*>(t->rope_cos);
  p.cache_index = t->cache_index;
  p.kv_cache = static_cast<uint16_t*>(t->kv_cache);
  p.kr_cache = static_cast<uint16_t*>(t->kr_cache);
  p.sx = t->scale_x; p.sw_dq = t->scale_w_dq; p.sw_uq_qr = t->scale_w_uq_qr;
  p.sw_dkv_kr = t->scale_w_dkv_kr;
  p.q_out = t->query_out;
  p.qr_out = static_cast<uint16_t*>(t->query_rope_out);
  p.q_scale = t->dequant_scale_q_nope;
  p.part = h->ws + h->lay.part;
  p.cq = h->ws + h->lay.cq;
  p.cq_scale = reinterpret_cast<float*>(h->ws + h->lay.cq_scale);
  p.qc = reinterpret_cast<uint16_t*>(h->ws + h->lay.qc);
  p.y = reinterpret_cast<float*>(h->ws + h->lay.y);
  p.ssq = reinterpret_cast<float*>(h->ws + h->lay.ssq);
  p.amax = reinterpret_cast<float*>(h->ws + h->lay.amax);
  p.ticket = reinterpret_cast<unsigned*>(h->ws + h->lay.ticket);
  hipStream_t s = static_cast<hipStream_t>(stream);

  hipEvent_t* ev = nullptr;
  if (h->events) {
    ev = h->events + (h->recorded % kProfileRing) * kProfileEvents;
    ++h->recorded;
  }
  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(ev[i], s);
  };
  mark(0);
  if (pl.stream) {
    launch_stream(pl, s, d, p, i8, q8, mark);
    const hipError_t e = hipGetLastError();
    if (prev != dd.device) (void)hipSetDevice(prev);
    return e == hipSuccess ? MLA_OK : MLA_ERR_RUNTIME;
  }
  const int tiles_q = ceil_div(d.Hcq, 64);
  const int tiles_kr = ceil_div(d.Hckv + d.Dr, 64);
  dim3 g1(tiles_q + tiles_kr, pl.S, ceil_div(T, 16 * pl.mt1));
  if (i8) launch_k1<true>(pl.mt1, g1, s, d, p, tiles_q, pl.kps);
  else launch_k1<false>(pl.mt1, g1, s, d, p, tiles_q, pl.kps);
  mark(1);

  const size_t y_bytes = size_t(d.Hcq + d.Hckv + d.Dr) * sizeof(float);
  if (i8) k_norm_rope_cache<true><<<dim3(d.T), kThreads, y_bytes, s>>>(d, p, pl.S);
  else k_norm_rope_cache<false><<<dim3(d.T), kThreads, y_bytes, s>>>(d, p, pl.S);
  mark(2);

  const int nope_tiles = ceil_div(d.D, 64);
  dim3 g3(d.N * (nope_tiles + 1), 1, ceil_div(T, 16 * pl.mt3));
  if (i8) launch_k3<true>(pl.mt3, g3, s, d, p, nope_tiles);
  else launch_k3<false>(pl.mt3, g3, s, d, p, nope_tiles);
  mark(3);

  dim3 g4(d.N, pl.cs4, ceil_div(T, 32));
  if (q8) launch_k4<true>(pl.ntw4, g4, s, d, p);
  else launch_k4<false>(pl.ntw4, g4, s, d, p);
  mark(4);

  const hipError_t e = hipGetLastError();
  if (prev != dd.device) (void)hipSetDevice(prev);
  return e == hipSuccess ? MLA_OK : MLA_ERR_RUNTIME;
}

static void destroy_events(mla_prolog* h) {
  if (!h->events) return;
  for (int i = 0; i < kProfileRing * kProfileEvents; ++i)
    if (h->events[i]) (void)hipEventDestroy(h->events[i]);
  delete[] h->events;
  h->events = nullptr;
  h->recorded = 0;
}

mla_status mla_prolog_profile_enable(mla_prolog_t h, int enable) {
  if (!h) return MLA_ERR_NULLPTR;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(h->desc.device) != hipSuccess)
    return MLA_ERR_RUNTIME;
  mla_status st = MLA_OK;
  if (hipDeviceSynchronize() != hipSuccess) st = MLA_ERR_RUNTIME;
  destroy_events(h);
  if (st == MLA_OK && enable) {
    h->events = new (std::nothrow) hipEvent_t[kProfileRing * kProfileEvents]();
    if (!h->events) st = MLA_ERR_RUNTIME;
    for (int i = 0; st == MLA_OK && i < kProfileRing * kProfileEvents; ++i)
      if (hipEventCreate(&h->events[i]) != hipSuccess) st = MLA_ERR_RUNTIME;
    if (st != MLA_OK) destroy_events(h);
  }
  (void)hipSetDevice(prev);
  return st;
}

mla_status mla_prolog_profile_read(mla_prolog_t h, double* kernel_ms, int64_t* runs) {
  if (!h || !kernel_ms || !runs) return MLA_ERR_NULLPTR;
  if (!h->events) return MLA_ERR_PARAM_INVALID;
  const int64_t n = h->recorded;
  h->recorded = 0;
  if (n > kProfileRing) return MLA_ERR_PARAM_INVALID;
  for (int k = 0; k < kProfileEvents - 1; ++k) kernel_ms[k] = 0.0;
  for (int64_t r = 0; r < n; ++r) {
    hipEvent_t* ev = h->events + r * kProfileEvents;
    if (hipEventSynchronize(ev[kProfileEvents - 1]) != hipSuccess) return MLA_ERR_RUNTIME;
    for (int k = 0; k < kProfileEvents - 1; ++k) {
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, ev[k], ev[k + 1]) != hipSuccess) return MLA_ERR_RUNTIME;
      kernel_ms[k] += ms;
    }
  }
  *runs = n;
  return MLA_OK;
}

mla_status mla_prolog_destroy(mla_prolog_t h) {
  if (!h) return MLA_ERR_NULLPTR;
  int prev = 0;
  mla_status st = MLA_OK;
  if (hipGetDevice(&prev) != hipSuccess) st = MLA_ERR_RUNTIME;
  if (st == MLA_OK && hipSetDevice(h->desc.device) == hipSuccess) {
    if (hipDeviceSynchronize() != hipSuccess) st = MLA_ERR_RUNTIME;
    destroy_events(h);
    if (hipFree(h->ws) != hipSuccess) st = MLA_ERR_RUNTIME;
    (void)hipSetDevice(prev);
  }
  delete h;
  return st;
}

const char* mla_prolog_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULLPTR: return "a required pointer is null";
    case MLA_ERR_PARAM_INVALID: return "a shape, dtype, alignment or size is invalid";
    case MLA_ERR_RUNTIME: return "HIP runtime error";
    case MLA_ERR_UNSUPPORTED: return "no kernel tiling for these sizes";
  }
  return "unknown status";
}

}  // extern "C"
