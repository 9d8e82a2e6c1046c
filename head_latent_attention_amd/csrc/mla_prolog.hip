// MLA prolog for MI355X (gfx950 / CDNA4): kernels and the C ABI.
//
// The operation is the Multi-Head Latent Attention prolog of the Ascend
// operator page aclnnMlaPrologV2WeightNz ("Function", formula block); the
// rotate-half RoPE is the mode the aclnnMlaPreprocess page fixes
// (constraints, rope mode).  Its steps:
//
//   down-projection   y = x [W^DQ | W^DKV | W^KR] (fp32 accumulation, or
//                     exact int32 with int8 inputs)
//   norms             both RmsNorms (in double), c^Q as bf16 or per-token
//                     int8 (+ smoothScalesCq), c^KV and RoPE(k^R) scattered
//                     to the cacheIndex slots (bf16, or static int8 codes)
//   up-projection     u = c^Q [W^UQ | W^QR] per head; nope columns -> q^C
//                     (bf16), rope columns -> RoPE -> queryRopeOut
//   W^UK product      q^N = q^C W^UK[h] per head; bf16, or per-(token, head)
//                     dynamic int8 with its dequantisation scale
//
// The static int8 scenario of the aclnnMlaPreprocess page ("Function",
// parameter table, quantMode 0) puts k0_xquant in front: x is quantised by
// RmsNormQuant (static, per tensor, asymmetric); the int8 products add a
// per-channel int32 bias before their deScale; c^Q takes the same static
// codes.  Every path writes the separate outputs and caches, or the same
// rows concatenated (that page's cacheMode 0), through per-output row
// strides; the packer also takes (n, k) transposed weights.
//
// Execution paths, by token count and weight layout:
//   - packed weights (mla_prolog_pack_weights: 64-column windows stored as
//     4 KB k-stages in MFMA operand order), T <= 32, bf16 tensors (bf16,
//     partial quantisation, or the static scenario after k0_xquant): one
//     launch
//     (k_fused) whose blocks hand partial results to one another through
//     agent-scope tagged words and flags;
//   - packed weights, T <= 32 otherwise: k1_tiled, k2_norm, then the
//     up-projection and W^UK product (k34_pair, k34_stream, or k3_packed
//     and k4_packed);
//   - packed weights, T > 32: k1_tiled, k2_norm, k3_tiled, k4_tiled
//     (direct or LDS-staged tiles, by shape class);
//   - row-major weights only: k_down_proj, k2_norm, k_up_proj, k_uk.
//
// All matrix products run on MFMA (v_mfma_f32_16x16x32_bf16,
// v_mfma_i32_16x16x64_i8).  There are no float atomics: every reduction has
// a fixed order, so a run is deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <type_traits>

#include "../../include/mla_prolog.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// four floats -> four bf16 (RNE) in 8 bytes, first value lowest
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float e) {
  return make_uint2(uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16),
                    uint32_t(f2bf(c)) | (uint32_t(f2bf(e)) << 16));
}

// fp16 (IEEE binary16) <-> float; the conversion rounds to nearest even
__device__ __forceinline__ float h2f(uint16_t b) { return float(__builtin_bit_cast(_Float16, b)); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }

// A 16-bit float of the tensors whose format the caller chooses (the MLA
// preprocess page takes FLOAT16 or BFLOAT16 for them): fp16 when F16, else
// bf16.
template <bool F16>
__device__ __forceinline__ float ld16(uint16_t b) { return F16 ? h2f(b) : bf2f(b); }
template <bool F16>
__device__ __forceinline__ uint16_t st16(float f) { return F16 ? f2h(f) : f2bf(f); }
template <bool F16>
__device__ __forceinline__ uint2 pack16x4(float a, float b, float c, float e) {
  return make_uint2(uint32_t(st16<F16>(a)) | (uint32_t(st16<F16>(b)) << 16),
                    uint32_t(st16<F16>(c)) | (uint32_t(st16<F16>(e)) << 16));
}

// symmetric int8 code of v for scale s > 0: nearest integer (ties to even)
// of v / s, kept within [-127, 127]
__device__ __forceinline__ int8_t quant_code(float v, float s) {
  float r = rintf(v / s);
  r = fminf(127.0f, fmaxf(-127.0f, r));
  return static_cast<int8_t>(r);
}

// static int8 code of a cache value: v times its channel's scale, rounded
// half to even, saturated to [-128, 127] (quantScaleCkv / quantScaleCkr)
__device__ __forceinline__ uint32_t cache_code(float v, float s) {
  const float r = fminf(127.0f, fmaxf(-128.0f, rintf(v * s)));
  return uint32_t(uint8_t(int8_t(r)));
}

// static asymmetric int8 code of the MLA preprocess page's RmsNormQuant
// (quantMode 0): v times the scale, rounded half to even, plus the offset,
// saturated to [-128, 127]
__device__ __forceinline__ uint32_t static_code(float v, float s, float off) {
  const float r = fminf(127.0f, fmaxf(-128.0f, rintf(v * s) + off));
  return uint32_t(uint8_t(int8_t(r)));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_max_f64(double v) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
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
  double eps_cq, eps_ckv;
  // row strides, in elements, of queryOut (per token and head), of the q^R
  // rows, and of the kv and kr cache slots: Hckv, Dr, Hckv, Dr, or all
  // Hckv + Dr in the concatenated layout (q^R and k^R then start Hckv
  // elements into the queryOut row and the kv slot)
  int qs, qrs, kvs, krs;
  // the run's number (1, 2, ...; never 0, modulo 2^32), which the small-T
  // kernels' flags and tags hold, and the poll steps a bounded wait makes
  // before it gives up
  uint32_t run;
  int spin;
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
  uint16_t* kv_cache;        // bf16 rows, or int8 rows when qs_ckv is set
  uint16_t* kr_cache;        // bf16 rows, or int8 rows when qs_ckr is set
  const float* qs_ckv;       // quantScaleCkv (Hckv), or NULL
  const float* qs_ckr;       // quantScaleCkr (Dr), or NULL
  const float* sx;
  const float* sw_dq;
  const float* sw_uq_qr;
  const float* sw_dkv_kr;
  const float* smooth_cq;   // smoothScalesCq (Hcq), or NULL (int8 W^UqQr only)
  // the static int8 scenario (MLA preprocess page, quantMode 0)
  const int32_t* bias_dq;   // bias0 (Hcq + Hckv + Dr), or NULL (zeros)
  const int32_t* bias_uq;   // bias1 (N*(D+Dr)), or NULL (zeros)
  const uint16_t* beta_cq;  // beta1 (Hcq): set exactly when c^Q takes static codes
  const uint16_t* qsc_cq;   // quantScale1 (one bf16)
  const int8_t* qo_cq;      // quantOffset1
  void* q_out;
  uint16_t* qr_out;
  float* q_scale;
  // workspace
  void* part;        // [S][T][Hcq+Hckv+Dr] fp32 (int32 in int8 mode)
  uint8_t* cq;       // [T][Hcq] bf16 (int8 in int8 mode)
  float* cq_scale;   // [T]
  uint16_t* qc;      // [T][N][D] bf16
  uint8_t* xq;       // [N] q^C exchange of the paired small-T kernel, kPairXq bytes a head
  uint32_t* xflag;   // [N][4] its exchange flags (run numbers), then one spare word
  float* xmax;       // [N][2][32] its per-token row maxima
  float* xmax2;      // [N][2][kRingMaxT]: the medium-T fused kernel's per-token row maxima
  uint32_t* fpart;   // fused kernel: [phase-1 blocks][32][64] (fp32 split partial, run tag) words
  uint32_t* fss;     // fused kernel: [windows][32] (fp32 sum of squares, run tag) words, then (int8
                     // c^Q) [c^Q windows][32] (fp32 max |gamma m y|, run tag) words
  float* fykr;       // fused kernel: [32][Hckv + Dr] y of the c^KV and k^R columns
  uint32_t* fcnt;    // fused kernel: [2N] flags, 64 bytes apart
  uint32_t* herr;    // the handle's error word, in host-visible memory: set when a bounded wait gives up
  const uint8_t* packed;  // weights in the packed layout, or NULL
};

// int8 up-projection output of column n for token t: (acc + bias1[n]) *
// s_cq[t] * scaleW[n] in fp32 (bias1 only in the static scenario, whose
// s_cq is 1).  The biased sum is an int32, like the accumulator.
__device__ __forceinline__ float udq(const Ptrs& p, int32_t acc, int t, int n) {
  const int32_t b = p.bias_uq ? p.bias_uq[n] : 0;
  return static_cast<float>(acc + b) * p.cq_scale[t] * p.sw_uq_qr[n];
}

// K0 (static scenario) -------------------------------------------------------
// One 1024-thread block per token: x (bf16) to int8 codes with the MLA
// preprocess page's RmsNormQuant, v = gamma0 x / sqrt(mean(x^2) + eps) +
// beta0 (v = x without the norm), code = static_code(v, quantScale0,
// quantOffset0).  The sum of squares is taken in double (each square is
// exact), so the codes see v rounded once to fp32.  Each thread keeps its
// first 8-element chunk of x (and its gamma0 / beta0) in registers, loaded
// before the reduction; chunks beyond the first 1024 are read again.
struct XQuant {
  const uint16_t* x;      // (T, He) bf16 (or fp16)
  const uint16_t* gamma;  // (He) bf16 (or fp16), NULL without the norm
  const uint16_t* beta;   // (He) bf16 (or fp16)
  const uint16_t* scale;  // one bf16 (or fp16)
  const int8_t* offset;   // one int8
  uint8_t* out;           // (T, He) int8 codes
  int T, He;
  double eps;
};
constexpr int kXqThreads = 1024;

template <bool F16>
__device__ __forceinline__ void unpack16x8(const uint4& u, double (&v)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = ld16<F16>(uint16_t(w[e / 2] >> (16 * (e & 1))));
}

// F16: x, gamma0, beta0 and quantScale0 are fp16 (else bf16)
template <bool F16>
__global__ __launch_bounds__(kXqThreads) void k0_xquant(XQuant a) {
  __shared__ double red[kXqThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int chunks = a.He / 8;
  const uint4* row = reinterpret_cast<const uint4*>(a.x + int64_t(t) * a.He);
  const uint4* g4 = reinterpret_cast<const uint4*>(a.gamma);
  const uint4* b4 = reinterpret_cast<const uint4*>(a.beta);
  const bool mine = tid < chunks;
  const uint4 x0 = mine ? row[tid] : make_uint4(0, 0, 0, 0);
  uint4 g0 = make_uint4(0, 0, 0, 0), b0 = g0;
  double rms = 1.0;
  if (a.gamma) {
    if (mine) { g0 = g4[tid]; b0 = b4[tid]; }
    double v[8], ss = 0.0;
    unpack16x8<F16>(x0, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
    for (int j = tid + kXqThreads; j < chunks; j += kXqThreads) {
      unpack16x8<F16>(row[j], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
    }
    ss = wave_sum_f64(ss);
    if (lane == 0) red[w] = ss;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int k = 0; k < kXqThreads / 64; ++k) tot += red[k];
    rms = sqrt(tot / double(a.He) + a.eps);
  }
  const float qs = ld16<F16>(*a.scale), off = float(*a.offset);
  uint2* out = reinterpret_cast<uint2*>(a.out + int64_t(t) * a.He);
  auto emit = [&](int j, const uint4& xu, const uint4& gu, const uint4& bu) {
    double v[8];
    unpack16x8<F16>(xu, v);
    if (a.gamma) {
      double g[8], b[8];
      unpack16x8<F16>(gu, g);
      unpack16x8<F16>(bu, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = g[e] * v[e] / rms + b[e];
    }
    uint32_t code[2] = {0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) code[e / 4] |= static_code(float(v[e]), qs, off) << (8 * (e % 4));
    out[j] = make_uint2(code[0], code[1]);
  };
  if (mine) emit(tid, x0, g0, b0);
  for (int j = tid + kXqThreads; j < chunks; j += kXqThreads)
    emit(j, row[j], a.gamma ? g4[j] : x0, a.gamma ? b4[j] : x0);
}

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
          v = (m < d.T) ? udq(p, acc[mt][0][i], m, col0 + col)
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
      uint16_t* o = p.qr_out + (int64_t(m) * d.N + h) * d.qrs;
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
          if (m < d.T) qo[(int64_t(m) * d.N + h) * d.qs + c0 + col] = f2bf(acc[mt][j][i]);
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
            qo[(int64_t(m) * d.N + h) * d.qs + col] = s > 0.0f ? quant_code(acc[mt][j][i], s) : 0;
        }
        if (wave == 0 && c == 0) p.q_scale[int64_t(m) * d.N + h] = s;
      }
  }
}

// ---------------------------------------------------------------------------
// Small-T building blocks: MFMA operand geometry, buffer loads, activation
// operands and the fixed-order sum of several waves' accumulators.
// ---------------------------------------------------------------------------
template <bool I8>
struct Stage {
  static constexpr int EB = I8 ? 1 : 2;
  static constexpr int KS = I8 ? 64 : 32;    // k rows per stage (one MFMA k-step)
  static constexpr int KL = 16 / EB;         // k per lane per MFMA
  using Acc = typename std::conditional<I8, i32x4, f32x4>::type;
  using Frag = typename std::conditional<I8, i32x4, bf16x8>::type;
};

// Buffer loads: an offset at or past num_records returns zeros without a
// memory request, so predicated loads need no branch.  Every buffer here is
// addressed with 32-bit offsets below 2 GiB.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = static_cast<int>(bytes <= 0 ? 0 : bytes < int64_t(kOOB) ? bytes : int64_t(kOOB) - 1);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return __builtin_bit_cast(uint4, v);
}

// a 16-byte buffer load with the streaming hint, for data read once
__device__ __forceinline__ uint4 bload16s(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ i32x4 mfma(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// The 16-bit float products: bf16, or fp16 when F16 (the same 16x16x32
// shape); int8 fragments pass through to the int8 product
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <bool F16>
__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return mfma(a, b, c);
}
template <bool F16>
__device__ __forceinline__ i32x4 mma16(i32x4 a, i32x4 b, i32x4 c) {
  return mfma(a, b, c);
}

// Activation operands.  A policy loads the calling lane's 16-byte registers
// of the MT fragments (16 rows each) of one k-stage (load) and turns them
// into MFMA fragments (frag).
//
// APlain reads row-major rows (bf16 or int8, k-contiguous), counted from the
// buffer base: a wave's load touches 16 rows.
template <bool I8, int MT>
struct APlain {
  static constexpr int NR = MT;  // 16-byte registers per stage
  rsrc_t A;
  uint32_t lda;  // bytes per row
  int M;         // valid rows from the base
  int ke;        // valid k
  __device__ __forceinline__ void load(uint4 (&r)[NR], int st, bool ok) const {
    const int lane = threadIdx.x & 63, ml = lane & 15, g = lane >> 4;
    const int ka = st * Stage<I8>::KS + Stage<I8>::KL * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = ml + 16 * mt;
      r[mt] = bload16(A, ok && m < M && ka < ke ? uint32_t(m) * lda + uint32_t(ka) * Stage<I8>::EB
                                                : kOOB);
    }
  }
  __device__ __forceinline__ typename Stage<I8>::Frag frag(const uint4 (&r)[NR], int mt) const {
    return __builtin_bit_cast(typename Stage<I8>::Frag, r[mt]);
  }
  // the calling lane's 16 bytes of fragment tile c (rows 16c..) of stage st
  __device__ __forceinline__ uint4 load1(int c, int st, bool ok) const {
    const int lane = threadIdx.x & 63;
    const int m = 16 * c + (lane & 15), ka = st * Stage<I8>::KS + Stage<I8>::KL * (lane >> 4);
    return bload16(A, ok && m < M && ka < ke ? uint32_t(m) * lda + uint32_t(ka) * Stage<I8>::EB : kOOB);
  }
};

// APacked reads fragment-packed activations: every 16-row tile stores its
// k-stages one after the other, 1 KB each, in MFMA fragment order (lane l:
// row l%16, k-run KL*(l/16) of the stage), so a wave's load is one
// contiguous kilobyte.  Tiles are `tile` bytes apart from the base.
template <bool I8, int MT>
struct APacked {
  static constexpr int NR = MT;
  rsrc_t A;
  uint32_t tile;
  __device__ __forceinline__ void load(uint4 (&r)[NR], int st, bool ok) const {
    const uint32_t lane = threadIdx.x & 63;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      r[mt] = bload16(A, ok ? uint32_t(mt) * tile + uint32_t(st) * 1024u + lane * 16u : kOOB);
  }
  __device__ __forceinline__ typename Stage<I8>::Frag frag(const uint4 (&r)[NR], int mt) const {
    return __builtin_bit_cast(typename Stage<I8>::Frag, r[mt]);
  }
  __device__ __forceinline__ uint4 load1(int c, int st, bool ok) const {
    const uint32_t lane = threadIdx.x & 63;
    return bload16(A, ok ? uint32_t(c) * tile + uint32_t(st) * 1024u + lane * 16u : kOOB);
  }
};

// Byte offset of element (row t, k) in a fragment-packed activation buffer
// whose 16-row tiles are `tile` bytes apart.
__device__ __forceinline__ int64_t packed_offset(int64_t t, int k, int64_t tile, bool i8) {
  const int ks = i8 ? 64 : 32, kl = i8 ? 16 : 8, eb = i8 ? 1 : 2;
  const int st = k / ks, g = (k % ks) / kl, i = k % kl;
  return (t >> 4) * tile + int64_t(st) * 1024 + ((g * 16 + (t & 15)) * 16) + i * eb;
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

// ---------------------------------------------------------------------------
// Packed weights.  Each weight matrix is cut into windows of 64 columns; a
// window is stored as its k-stages one after the other (32 bf16 rows or 64
// int8 rows per stage, 4 KB), and inside a stage as 4 column tiles x 64
// lanes x 16 bytes in MFMA B-fragment order: lane l of column tile ct holds
// rows KL*(l/16) + i (i < KL) of column 16*ct + l%16.  A block streaming a
// window reads one contiguous region, and every 16-byte load lands directly
// in the register an MFMA reads; no LDS transposition is needed.
//
// Windows: W^DQ in 64-column steps; W^DkvKr likewise; W^UqQr per head, its
// nope columns in 64-column steps then its Dr rope columns; W^UK per head,
// Hckv in 64-column steps (k = the D rows).  Zero padding fills ragged
// windows and stages.
// ---------------------------------------------------------------------------
struct PackGeo {
  int64_t off_dq, off_kr, off_uq, off_uk, total;  // byte offsets in the packed buffer
  int win_dq, win_kr, win_uq, win_uk;             // windows per matrix
  int nst_he, nst_cq, nst_d;                      // stages along He, Hcq, D
  int nope_w, uk_w;                               // nope windows per head, W^UK windows per head
};

// i8d: W^DQ and W^DkvKr are int8 (k-stages of 64 rows, else 32); i8u:
// W^UqQr is int8.  W^UK is bf16 in every scenario.
PackGeo pack_geo(int64_t He, int64_t Hcq, int64_t Hckv, int64_t N, int64_t D, int64_t Dr, bool i8d,
                 bool i8u) {
  PackGeo g;
  const int ksd = i8d ? 64 : 32, ksu = i8u ? 64 : 32;
  g.nst_he = int((He + ksd - 1) / ksd);
  g.nst_cq = int((Hcq + ksu - 1) / ksu);
  g.nst_d = int((D + 31) / 32);
  g.nope_w = int((D + 63) / 64);
  g.uk_w = int((Hckv + 63) / 64);
  g.win_dq = int((Hcq + 63) / 64);
  g.win_kr = int((Hckv + Dr + 63) / 64);
  g.win_uq = int(N) * (g.nope_w + 1);
  g.win_uk = int(N) * g.uk_w;
  g.off_dq = 0;
  g.off_kr = g.off_dq + int64_t(g.win_dq) * g.nst_he * 4096;
  g.off_uq = g.off_kr + int64_t(g.win_kr) * g.nst_he * 4096;
  g.off_uk = g.off_uq + int64_t(g.win_uq) * g.nst_cq * 4096;
  g.total = g.off_uk + int64_t(g.win_uk) * g.nst_d * 4096;
  return g;
}

// One 16-byte chunk per thread: (window, stage, column tile, lane) of one
// matrix, gathered from the row-major source.
__global__ __launch_bounds__(256) void k_pack(Dims d, Ptrs p, PackGeo g, int i8d, int i8u, int nk,
                                              uint8_t* out) {
  const int64_t q = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t off = q * 16;
  if (off >= g.total) return;
  int64_t rel;
  int nst, win;
  const uint8_t* src;
  int64_t ld;          // source row stride, elements
  int K, col0, width, eb, kl;
  if (off < g.off_kr) {
    rel = off - g.off_dq; nst = g.nst_he; win = int(rel / (int64_t(nst) * 4096));
    src = p.w_dq; ld = d.Hcq; K = d.He; col0 = 64 * win; width = min(64, d.Hcq - col0);
    eb = i8d ? 1 : 2;
  } else if (off < g.off_uq) {
    rel = off - g.off_kr; nst = g.nst_he; win = int(rel / (int64_t(nst) * 4096));
    src = p.w_dkv_kr; ld = d.Hckv + d.Dr; K = d.He; col0 = 64 * win; width = min(64, d.Hckv + d.Dr - col0);
    eb = i8d ? 1 : 2;
  } else if (off < g.off_uk) {
    rel = off - g.off_uq; nst = g.nst_cq; win = int(rel / (int64_t(nst) * 4096));
    const int h = win / (g.nope_w + 1), part = win % (g.nope_w + 1);
    src = p.w_uq_qr; ld = int64_t(d.N) * (d.D + d.Dr); K = d.Hcq;
    col0 = h * (d.D + d.Dr) + (part < g.nope_w ? 64 * part : d.D);
    width = part < g.nope_w ? min(64, d.D - 64 * part) : d.Dr;
    eb = i8u ? 1 : 2;
  } else {
    rel = off - g.off_uk; nst = g.nst_d; win = int(rel / (int64_t(nst) * 4096));
    const int h = win / g.uk_w, part = win % g.uk_w;
    src = reinterpret_cast<const uint8_t*>(p.w_uk + int64_t(h) * d.D * d.Hckv);
    ld = d.Hckv; K = d.D; col0 = 64 * part; width = min(64, d.Hckv - col0);
    eb = 2;
    nk = 0;   // W^UK is always (N, D, Hckv)
  }
  const int in_win = int(rel % (int64_t(nst) * 4096));
  const int stage = in_win / 4096, ct = (in_win % 4096) / 1024, lane = (in_win % 1024) / 16;
  kl = 16 / eb;
  const int ks = 4 * kl;  // rows per stage: 32 bf16, 64 int8
  const int c = 16 * ct + (lane & 15);
  union { uint4 v; uint8_t b[16]; uint16_t h[8]; } u;
  u.v = make_uint4(0, 0, 0, 0);
  for (int i = 0; i < kl; ++i) {
    const int k = stage * ks + kl * (lane >> 4) + i;
    if (k >= K || c >= width) continue;
    // element (k, n): row k of a (k, n) weight, or row n of an (n, k) one
    const int64_t e = nk ? int64_t(col0 + c) * K + k : int64_t(k) * ld + col0 + c;
    if (eb == 1) u.b[i] = src[e];
    else u.h[i] = reinterpret_cast<const uint16_t*>(src)[e];
  }
  *reinterpret_cast<uint4*>(out + off) = u.v;
}

// One wave streams stages s = sfirst + j*sstep (j < ns) of the packed window
// at byte wbase against MT activation fragments; all loads go through one
// register ring D stages deep.
template <bool I8, int MT, int D, class AP>
__device__ __forceinline__ void stream_packed(const AP& ap, rsrc_t Wp, uint32_t wbase, int sfirst,
                                              int sstep, int ns, typename Stage<I8>::Acc (&acc)[MT][4]) {
  using S = Stage<I8>;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[mt][ct] = typename S::Acc{0, 0, 0, 0};
  uint4 bq[D][4];
  uint4 aq[D][AP::NR];
  auto issue = [&](uint4 (&b)[4], uint4 (&a)[AP::NR], int j) {
    const int st = sfirst + j * sstep;
    const bool ok = j < ns;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      b[ct] = bload16(Wp, ok ? wbase + uint32_t(st) * 4096u + uint32_t(ct * 1024 + lane * 16) : kOOB);
    ap.load(a, st, ok);
  };
#pragma unroll
  for (int q = 0; q < D; ++q) {
    issue(bq[q], aq[q], q);
    __builtin_amdgcn_sched_barrier(0);   // the loop expects the slots in this order
  }
  // each slot is refilled right after the MFMAs that read it; the
  // scheduling barriers keep the refills in slot order, so every wait is
  // for the oldest slot only
  const int nsr = (ns + D - 1) / D * D;
  for (int j0 = 0; j0 < nsr; j0 += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const typename S::Frag af = ap.frag(aq[q], mt);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          acc[mt][ct] = mfma(af, __builtin_bit_cast(typename S::Frag, bq[q][ct]), acc[mt][ct]);
      }
      issue(bq[q], aq[q], j0 + q + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// K2: NWT waves per token, TPB tokens per block.  y is the split-order sum
// of the token's S partials of x [W^DQ | W^DkvKr] (in double; with int8
// down-projection inputs, I8D, the exact int32 sum times the token and
// column scales; in the static scenario, ST, the sum plus bias0 times the
// column's deScale0, and c^Q + beta1 takes static codes with scale 1).  A first pass sums the squares of the c^Q and c^KV parts
// (and, for an int8 c^Q, I8U, finds the largest |gamma m y| of the c^Q part,
// m the optional smoothScalesCq), keeping each lane's first CPL 8-column
// chunks of y in registers (and, with one wave per token, the next four in
// the wave's LDS rows); a second pass writes c^Q (bf16, or the per-token
// int8 of c^Q * m + scale), the c^KV row at the token's cacheIndex slot and,
// through a small LDS row, the RoPE'd k^R row, reloading only the chunks
// held in neither.  The norms are computed in double, so the per-token
// int8 decision of c^Q sees c rounded once to fp32; c^Q * m is formed as
// (gamma m) y / rms, gamma m being exact in double.
// With cq_nst > 0, c^Q is stored fragment-packed (cq_nst k-stages per
// 16-token tile, the k padding as zeros); with 0, row-major.

template <bool I8D, bool I8U, bool ST, int NWT, int TPB, int CPL, bool F16 = false>
__global__ __launch_bounds__(64 * NWT * TPB) void k2_norm(Dims d, Ptrs p, int S, int cq_nst) {
  static_assert(!ST || (I8D && I8U), "the static scenario is int8 throughout");
  static_assert(!F16 || ST, "fp16 tensors belong to the static scenario");
  __shared__ double red[NWT * TPB][3];
  __shared__ double ry[TPB][64];   // the token's y of the k^R columns (Dr <= 64)
  // one wave per token: the lane's chunks CPL .. CPL+YX-1 of y wait for the
  // second pass in the wave's own LDS rows (element e of chunk k of lane l
  // at [k][e][l]), so only chunks past those are read twice
  constexpr int YX = NWT == 1 ? 4 : 0;
  __shared__ double ysl[YX ? TPB : 1][YX ? YX : 1][8][64];
  const int w = threadIdx.x >> 6;
  const int lane = (w % NWT) * 64 + (threadIdx.x & 63);   // lane among the token's waves
  constexpr int L = 64 * NWT;
  const int t = blockIdx.x * TPB + w / NWT;
  const bool active = t < d.T;
  const int Ntot = d.Hcq + d.Hckv + d.Dr;
  const int cq_c = d.Hcq / 8, kv_c = d.Hckv / 8, chunks = cq_c + kv_c + d.Dr / 8;
  const rsrc_t P = make_rsrc(p.part, int64_t(S) * d.T * Ntot * 4);
  const int tt = active ? t : 0;
  // the token's scalars, loaded first
  const double sx = (I8D && !ST) ? double(p.sx[tt]) : 1.0;
  const int64_t slot = p.cache_index[tt];
  const bool cache = active && slot >= 0 && slot < d.slots;
  const float st_s = ST ? ld16<F16>(*p.qsc_cq) : 0.0f, st_o = ST ? float(*p.qo_cq) : 0.0f;
  // a chunk's column parameters (dequantisation scales, bias, gamma,
  // smoothing, beta, cache scales); for the lane's first CPL chunks they are
  // loaded before the partials, so that every load of the kernel is in
  // flight at once.  Lanes without a chunk read chunk 0's.
  struct Side { uint4 sw0, sw1, b0, b1, g, sm0, sm1, be, qk0, qk1; };
  auto side = [&](int j) {
    Side r;
    const uint4 z = make_uint4(0, 0, 0, 0);
    const int jj = j < chunks ? j : 0;
    const bool isq = jj < cq_c, iskv = !isq && jj < cq_c + kv_c;
    const int n = 8 * jj, nq = isq ? n : 0, nk = iskv ? n - d.Hcq : 0;
    r.sw0 = r.sw1 = r.b0 = r.b1 = r.sm0 = r.sm1 = r.be = r.qk0 = r.qk1 = z;
    if constexpr (I8D) {
      const float* sw = isq ? p.sw_dq + n : p.sw_dkv_kr + (n - d.Hcq);
      r.sw0 = *reinterpret_cast<const uint4*>(sw);
      r.sw1 = *reinterpret_cast<const uint4*>(sw + 4);
    }
    if (ST && p.bias_dq) {
      r.b0 = *reinterpret_cast<const uint4*>(p.bias_dq + n);
      r.b1 = *reinterpret_cast<const uint4*>(p.bias_dq + n + 4);
    }
    r.g = *reinterpret_cast<const uint4*>(isq ? p.gamma_cq + nq : p.gamma_ckv + nk);
    if (I8U && p.smooth_cq) {
      r.sm0 = *reinterpret_cast<const uint4*>(p.smooth_cq + nq);
      r.sm1 = *reinterpret_cast<const uint4*>(p.smooth_cq + nq + 4);
    }
    if (ST) r.be = *reinterpret_cast<const uint4*>(p.beta_cq + nq);
    if (p.qs_ckv) {
      r.qk0 = *reinterpret_cast<const uint4*>(p.qs_ckv + nk);
      r.qk1 = *reinterpret_cast<const uint4*>(p.qs_ckv + nk + 4);
    }
    return r;
  };
  auto w32 = [](const uint4& a, const uint4& b, int e) {
    const uint4& v = e < 4 ? a : b;
    const int k = e & 3;
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
  };
  auto w16 = [](const uint4& a, int e) {
    const int k = e >> 1;
    const uint32_t v = k == 0 ? a.x : k == 1 ? a.y : k == 2 ? a.z : a.w;
    return uint16_t(v >> (16 * (e & 1)));
  };
  // y of the eight columns 8j .. 8j+7; the loads of eight splits at a time
  // are issued together (a missing split reads as zeros, an exact no-op)
  // with at most two splits, the loads (ld2, zeros unless ok) and the sum
  // (sum2) of a chunk are separate steps, so several chunks' loads can go
  // out together
  auto ld2 = [&](int j, bool ok, uint4 (&r)[4]) {
    const uint32_t o = uint32_t((int64_t(t) * Ntot + 8 * j) * 4);
    const uint32_t o2 = uint32_t(((int64_t(d.T) + t) * Ntot + 8 * j) * 4);
    r[0] = bload16(P, ok ? o : kOOB);
    r[1] = bload16(P, ok ? o + 16 : kOOB);
    r[2] = bload16(P, ok && S == 2 ? o2 : kOOB);
    r[3] = bload16(P, ok && S == 2 ? o2 + 16 : kOOB);
  };
  auto sum2 = [&](const uint4 (&r)[4], double (&f)[8], int32_t (&iv)[8]) {
    const uint32_t w8[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
    const uint32_t v8[8] = {r[2].x, r[2].y, r[2].z, r[2].w, r[3].x, r[3].y, r[3].z, r[3].w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if constexpr (I8D) iv[c] = int32_t(w8[c]) + int32_t(v8[c]);
      else f[c] = double(__uint_as_float(w8[c])) + double(__uint_as_float(v8[c]));
    }
  };
  // the column scaling of a chunk's sums into y
  auto scale8 = [&](const Side& sd, const double (&f)[8], const int32_t (&iv)[8], double (&v)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (I8D) {
        const double sw = double(__uint_as_float(w32(sd.sw0, sd.sw1, e)));
        const int32_t b = ST ? int32_t(w32(sd.b0, sd.b1, e)) : 0;
        v[e] = double(iv[e] + b) * sx * sw;
      } else {
        v[e] = f[e];
      }
    }
  };
  auto y8 = [&](int j, const Side& sd, double (&v)[8]) {
    double f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int32_t iv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (S <= 2) {
      uint4 r[4];
      ld2(j, true, r);
      sum2(r, f, iv);
    }
    for (int s0 = 0; S > 2 && s0 < S; s0 += 8) {
      uint4 r[16];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t o = uint32_t(((int64_t(s0 + e) * d.T + t) * Ntot + 8 * j) * 4);
        r[2 * e] = bload16(P, s0 + e < S ? o : kOOB);
        r[2 * e + 1] = bload16(P, s0 + e < S ? o + 16 : kOOB);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w8[8] = {r[2 * e].x, r[2 * e].y, r[2 * e].z, r[2 * e].w,
                                r[2 * e + 1].x, r[2 * e + 1].y, r[2 * e + 1].z, r[2 * e + 1].w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if constexpr (I8D) iv[c] += int32_t(w8[c]);
          else f[c] += double(__uint_as_float(w8[c]));
        }
      }
    }
    scale8(sd, f, iv, v);
  };

  // the c^Q weight: gamma, times smoothScalesCq for an int8 c^Q when given
  auto gq = [&](const Side& sd, int e) {
    const double g = double(ld16<F16>(w16(sd.g, e)));
    if constexpr (I8U) return p.smooth_cq ? g * double(__uint_as_float(w32(sd.sm0, sd.sm1, e))) : g;
    return g;
  };
  double sq = 0.0, skv = 0.0, gmax = 0.0;
  auto sums = [&](int j, const Side& sd, const double (&v)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (j < cq_c) {
        sq += v[e] * v[e];
        if constexpr (I8U) gmax = fmax(gmax, fabs(gq(sd, e) * v[e]));
      } else if (j < cq_c + kv_c) {
        skv += v[e] * v[e];
      }
    }
  };
  // the RoPE lanes' sin/cos (and kr cache scales), loaded up front too
  const int h = d.Dr / 2;
  const int ir = lane < h ? lane : 0;
  const uint16_t* cs = p.cos + int64_t(tt) * d.Dr;
  const uint16_t* sn = p.sin + int64_t(tt) * d.Dr;
  const float cs0 = ld16<F16>(cs[ir]), cs1 = ld16<F16>(cs[ir + h]);
  const float sn0 = ld16<F16>(sn[ir]), sn1 = ld16<F16>(sn[ir + h]);
  const float qr0 = p.qs_ckr ? p.qs_ckr[ir] : 0.0f, qr1 = p.qs_ckr ? p.qs_ckr[ir + h] : 0.0f;
  Side sdv[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) sdv[c] = side(lane + c * L);
  double yv[CPL][8];
  // pass 1 over the register-held chunks, then the LDS-held ones (YX); with
  // those and at most two splits every load of both goes out at once
  if (YX > 0 && S <= 2) {
    uint4 rc[CPL][4], raw[YX ? YX : 1][4];
    Side sdx[YX ? YX : 1];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = lane + c * L;
      ld2(j, active && j < chunks, rc[c]);
    }
#pragma unroll
    for (int k = 0; k < YX; ++k) {
      const int j = lane + (CPL + k) * L;
      ld2(j, active && j < chunks, raw[k]);
      sdx[k] = side(j);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = lane + c * L;
      if (active && j < chunks) {
        double f[8];
        int32_t iv[8];
        sum2(rc[c], f, iv);
        scale8(sdv[c], f, iv, yv[c]);
        sums(j, sdv[c], yv[c]);
      }
    }
#pragma unroll
    for (int k = 0; k < YX; ++k) {
      const int j = lane + (CPL + k) * L;
      if (active && j < chunks) {
        double f[8], v[8];
        int32_t iv[8];
        sum2(raw[k], f, iv);
        scale8(sdx[k], f, iv, v);
        sums(j, sdx[k], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) ysl[w / NWT][k][e][lane] = v[e];
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = lane + c * L;
      if (active && j < chunks) {
        y8(j, sdv[c], yv[c]);
        sums(j, sdv[c], yv[c]);
      }
    }
#pragma unroll
    for (int k = 0; k < YX; ++k) {
      const int j = lane + (CPL + k) * L;
      if (active && j < chunks) {
        double v[8];
        const Side sd = side(j);
        y8(j, sd, v);
        sums(j, sd, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) ysl[w / NWT][k][e][lane] = v[e];
      }
    }
  }
  for (int j = lane + (CPL + YX) * L; active && j < chunks; j += L) {
    double v[8];
    const Side sd = side(j);
    y8(j, sd, v);
    sums(j, sd, v);
  }
  sq = wave_sum_f64(sq);
  skv = wave_sum_f64(skv);
  gmax = wave_max_f64(gmax);
  if constexpr (NWT > 1) {
    if ((threadIdx.x & 63) == 0) { red[w][0] = sq; red[w][1] = skv; red[w][2] = gmax; }
    __syncthreads();
    const int w0 = w - w % NWT;
    sq = red[w0][0]; skv = red[w0][1]; gmax = red[w0][2];
#pragma unroll
    for (int k = 1; k < NWT; ++k) {
      sq += red[w0 + k][0]; skv += red[w0 + k][1]; gmax = fmax(gmax, red[w0 + k][2]);
    }
  }
  if (!active) return;
  const double rms_q = sqrt(sq / double(d.Hcq) + d.eps_cq);
  const double rms_kv = sqrt(skv / double(d.Hckv) + d.eps_ckv);
  // the static scenario quantises c^Q + beta1 with quantScale1 and
  // quantOffset1 and its dequantisation scale is 1 (the per-channel deScale1
  // does the rest)
  constexpr bool stq = ST;
  float sc = 0.0f;
  if constexpr (I8U) sc = stq ? 1.0f : float(gmax / rms_q) / 127.0f;
  const int64_t tile = int64_t(cq_nst) * 1024;

  auto store_cq = [&](int j, const float (&c)[8], bool pad) {
    if constexpr (I8U) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t code = pad   ? 0u
                              : stq ? static_code(c[e], st_s, st_o)
                                    : uint8_t(sc > 0.0f ? quant_code(c[e], sc) : int8_t(0));
        if (e < 4) lo |= code << (8 * e);
        else hi |= code << (8 * (e - 4));
      }
      const int64_t o = cq_nst ? packed_offset(t, 8 * j, tile, true) : int64_t(t) * d.Hcq + 8 * j;
      *reinterpret_cast<uint2*>(p.cq + o) = make_uint2(lo, hi);
    } else {
      const uint2 a = pack16x4<F16>(c[0], c[1], c[2], c[3]), b = pack16x4<F16>(c[4], c[5], c[6], c[7]);
      const int64_t o = cq_nst ? packed_offset(t, 8 * j, tile, false) : (int64_t(t) * d.Hcq + 8 * j) * 2;
      *reinterpret_cast<uint4*>(p.cq + o) = make_uint4(a.x, a.y, b.x, b.y);
    }
  };
  auto emit = [&](int j, const Side& sd, const double (&v)[8]) {
    float c[8];
    if (j < cq_c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        double w = gq(sd, e) * v[e] / rms_q;
        if (stq) w += double(ld16<F16>(w16(sd.be, e)));
        c[e] = float(w);
      }
      store_cq(j, c, false);
    } else if (j >= cq_c + kv_c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ry[w / NWT][8 * (j - cq_c - kv_c) + e] = v[e];
    } else if (cache) {
      const int jk = j - cq_c;
#pragma unroll
      for (int e = 0; e < 8; ++e) c[e] = float(double(ld16<F16>(w16(sd.g, e))) * v[e] / rms_kv);
      if (p.qs_ckv) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo |= cache_code(c[e], __uint_as_float(w32(sd.qk0, sd.qk1, e))) << (8 * e);
          hi |= cache_code(c[e + 4], __uint_as_float(w32(sd.qk0, sd.qk1, e + 4))) << (8 * e);
        }
        *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(p.kv_cache) + slot * d.kvs + 8 * jk) =
            make_uint2(lo, hi);
      } else {
        const uint2 a = pack16x4<F16>(c[0], c[1], c[2], c[3]), b = pack16x4<F16>(c[4], c[5], c[6], c[7]);
        *reinterpret_cast<uint4*>(p.kv_cache + slot * d.kvs + 8 * jk) = make_uint4(a.x, a.y, b.x, b.y);
      }
    }
  };
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int j = lane + c * L;
    if (j < chunks) emit(j, sdv[c], yv[c]);
  }
#pragma unroll
  for (int k = 0; k < YX; ++k) {
    const int j = lane + (CPL + k) * L;
    if (j < chunks && (j < cq_c || cache)) {
      double v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = ysl[w / NWT][k][e][lane];
      emit(j, side(j), v);
    }
  }
  for (int j = lane + (CPL + YX) * L; j < chunks; j += L) {
    if (j >= cq_c && !cache) break;
    double v[8];
    const Side sd = side(j);
    y8(j, sd, v);
    emit(j, sd, v);
  }
  // the zero k padding of packed c^Q
  const int cq_chunks = cq_nst ? cq_nst * (I8U ? 8 : 4) : cq_c;
  for (int j = cq_c + lane; j < cq_chunks; j += L) {
    const float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    store_cq(j, z, true);
  }
  if (I8U && lane == 0) p.cq_scale[t] = sc;
  if (!cache) return;   // the same for every wave of the token
  if constexpr (NWT > 1) {
    __syncthreads();
  } else {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  const double* yr = ry[w / NWT];
  uint16_t* kr = p.kr_cache + slot * d.krs;
  uint8_t* kr8 = reinterpret_cast<uint8_t*>(p.kr_cache) + slot * d.krs;
  // Dr <= 64, so each RoPE pair has a lane of its own (L >= 64)
  if (lane < h) {
    const int i = lane;
    const double a = yr[i], b = yr[i + h];
    const float r0 = float(a * cs0 - b * sn0);
    const float r1 = float(b * cs1 + a * sn1);
    if (p.qs_ckr) {
      kr8[i] = uint8_t(cache_code(r0, qr0));
      kr8[i + h] = uint8_t(cache_code(r1, qr1));
    } else {
      kr[i] = st16<F16>(r0);
      kr[i + h] = st16<F16>(r1);
    }
  }
}

// K3p: grid (head windows of W^UqQr: per head the nope windows, then the rope
// window), NW waves splitting the Hcq stages of one window; the waves are
// summed in LDS, then the nope columns are rounded to bf16 q^C (workspace)
// and the rope columns go through RoPE to queryRopeOut.
template <bool I8, int MT, int NW, int D>
__global__ __launch_bounds__(64 * NW) void k3_packed(Dims d, Ptrs p, PackGeo pg) {
  using St = Stage<I8>;
  constexpr int RED = (NW / 2) * MT * 16 * 64 * 4, EPI = 16 * MT * 65 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[RED > EPI ? RED : EPI];
  const int P = pg.nope_w + 1;
  const int h = blockIdx.x / P, part = blockIdx.x % P;
  const bool rope = part == pg.nope_w;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col0 = h * (d.D + d.Dr) + (rope ? d.D : 64 * part);
  const int width = rope ? d.Dr : min(64, d.D - 64 * part);
  const int ns = w < pg.nst_cq ? (pg.nst_cq - w + NW - 1) / NW : 0;
  typename St::Acc acc[MT][4];
  const int64_t ctile = int64_t(pg.nst_cq) * 1024;
  const APacked<I8, MT> ap{make_rsrc(p.cq, int64_t((d.T + 15) / 16) * ctile), uint32_t(ctile)};
  const int64_t wbase = pg.off_uq + int64_t(blockIdx.x) * pg.nst_cq * 4096;
  stream_packed<I8, MT, D>(ap, make_rsrc(p.packed, pg.total), uint32_t(wbase), w, NW, ns, acc);
  reduce_waves<NW, MT>(acc, reinterpret_cast<uint32_t*>(lds));
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
                    ? udq(p, acc[mt][ct][i], ml, col0 + col)
                    : 0.0f;
          else
            v = acc[mt][ct][i];
          E[ml * 65 + col] = v;
        }
  }
  __syncthreads();
  const int BM = 16 * MT;
  if (!rope) {
    // q^C goes out fragment-packed for the W^UK product, its k padding as zeros
    const int wq = min(64, 32 * pg.nst_d - 64 * part);
    const int64_t qtile = int64_t(d.N) * pg.nst_d * 1024;
    uint8_t* qcb = reinterpret_cast<uint8_t*>(p.qc) + int64_t(h) * pg.nst_d * 1024;
    for (int idx = tid; idx < BM * wq; idx += 64 * NW) {
      const int ml = idx / wq, cc = idx % wq;
      if (ml < d.T)
        *reinterpret_cast<uint16_t*>(qcb + packed_offset(ml, 64 * part + cc, qtile, false)) =
            f2bf(E[ml * 65 + cc]);
    }
  } else {
    const int hf = d.Dr / 2;
    for (int idx = tid; idx < BM * hf; idx += 64 * NW) {
      const int ml = idx / hf, i = idx % hf;
      if (ml >= d.T) continue;
      const float a = E[ml * 65 + i], b = E[ml * 65 + i + hf];
      const uint16_t* cs = p.cos + int64_t(ml) * d.Dr;
      const uint16_t* sn = p.sin + int64_t(ml) * d.Dr;
      uint16_t* o = p.qr_out + (int64_t(ml) * d.N + h) * d.qrs;
      o[i] = f2bf(a * bf2f(cs[i]) - b * bf2f(sn[i]));
      o[i + hf] = f2bf(b * bf2f(cs[i + hf]) + a * bf2f(sn[i + hf]));
    }
  }
}

// K4p, bf16 query: grid (head x 64-column window of Hckv); NW waves split
// the D stages; the tile is staged through LDS for 16-byte stores.
template <int MT, int NW, int D>
__global__ __launch_bounds__(64 * NW) void k4_packed(Dims d, Ptrs p, PackGeo pg) {
  using St = Stage<false>;
  constexpr int RED = (NW / 2) * MT * 16 * 64 * 4, EPI = 16 * MT * 64 * 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[RED > EPI ? RED : EPI];
  const int h = blockIdx.x / pg.uk_w, win = blockIdx.x % pg.uk_w;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = 64 * win, width = min(64, d.Hckv - c0);
  const int ns = w < pg.nst_d ? (pg.nst_d - w + NW - 1) / NW : 0;
  typename St::Acc acc[MT][4];
  const int64_t qtile = int64_t(d.N) * pg.nst_d * 1024, qh = int64_t(h) * pg.nst_d * 1024;
  const APacked<false, MT> ap{make_rsrc(reinterpret_cast<const uint8_t*>(p.qc) + qh,
                                        int64_t((d.T + 15) / 16) * qtile - qh),
                              uint32_t(qtile)};
  const int64_t wbase = pg.off_uk + int64_t(blockIdx.x) * pg.nst_d * 4096;
  stream_packed<false, MT, D>(ap, make_rsrc(p.packed, pg.total), uint32_t(wbase), w, NW, ns, acc);
  reduce_waves<NW, MT>(acc, reinterpret_cast<uint32_t*>(lds));
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
      *reinterpret_cast<uint4*>(qo + (int64_t(ml) * d.N + h) * d.qs + c0 + 8 * ch) =
          *reinterpret_cast<const uint4*>(E + ml * 64 + 8 * ch);
  }
}

// K4p, int8 query: grid (head); wave w owns the 64-column window w of Hckv
// over the whole D reduction; the row maximum is taken across the waves.
template <int MT, int D>
__global__ __launch_bounds__(512) void k4_packed_q8(Dims d, Ptrs p, PackGeo pg) {
  __shared__ float rmax[8][16 * MT];
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const bool active = w < pg.uk_w;
  const int c0 = 64 * w, width = active ? min(64, d.Hckv - c0) : 0;
  typename Stage<false>::Acc acc[MT][4];
  const int64_t qtile = int64_t(d.N) * pg.nst_d * 1024, qh = int64_t(h) * pg.nst_d * 1024;
  const APacked<false, MT> ap{make_rsrc(reinterpret_cast<const uint8_t*>(p.qc) + qh,
                                        int64_t((d.T + 15) / 16) * qtile - qh),
                              uint32_t(qtile)};
  const int64_t wbase = pg.off_uk + int64_t(h * pg.uk_w + (active ? w : 0)) * pg.nst_d * 4096;
  stream_packed<false, MT, D>(ap, make_rsrc(p.packed, pg.total), uint32_t(wbase), 0, 1,
                              active ? pg.nst_d : 0, acc);
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
  if (!active) return;
  int8_t* qo = static_cast<int8_t*>(p.q_out);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ml = 16 * mt + 4 * g + i;
      if (ml >= d.T) continue;
      float amax = rmax[0][ml];
      for (int ww = 1; ww < pg.uk_w; ++ww) amax = fmaxf(amax, rmax[ww][ml]);
      const float sc = amax / 127.0f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int col = 16 * ct + c;
        if (col < width)
          qo[(int64_t(ml) * d.N + h) * d.qs + c0 + col] = sc > 0.0f ? quant_code(acc[mt][ct][i], sc) : 0;
      }
      if (w == 0 && c == 0) p.q_scale[int64_t(ml) * d.N + h] = sc;
    }
}

// Sum of the accumulators of each group of G consecutive waves into the
// group's first wave, in wave order, for the first `groups` groups.
// red: groups * (G - 1) * MT * 16 * 64 words of LDS.  Starts and ends with a
// block barrier.
template <int MT, class Acc>
__device__ __forceinline__ void reduce_groups(Acc (&acc)[MT][4], uint32_t* red, int G, int groups) {
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = w / G, r = w % G;
  constexpr int W = MT * 16 * 64;
  __syncthreads();
  if (grp < groups && r > 0) {
    uint32_t* o = red + (grp * (G - 1) + r - 1) * W;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const auto e = acc[mt][ct][i];
          o[((mt * 4 + ct) * 4 + i) * 64 + lane] = __builtin_bit_cast(uint32_t, e);
        }
  }
  __syncthreads();
  if (grp < groups && r == 0) {
    for (int k = 1; k < G; ++k) {
      const uint32_t* o = red + (grp * (G - 1) + k - 1) * W;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            using E = decltype(acc[mt][ct][i] + 0);
            acc[mt][ct][i] += __builtin_bit_cast(E, o[((mt * 4 + ct) * 4 + i) * 64 + lane]);
          }
    }
  }
  __syncthreads();
}

// Fragment-packed activations held in LDS (tiles `tile` bytes apart).
template <int MT>
struct ALds {
  static constexpr int NR = MT;
  const uint8_t* base;
  uint32_t tile;
  __device__ __forceinline__ void load(uint4 (&r)[NR], int st, bool ok) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      r[mt] = ok ? *reinterpret_cast<const uint4*>(base + mt * tile + st * 1024 + lane * 16)
                 : make_uint4(0, 0, 0, 0);
  }
};

// K34s: the up-projection and the W^UK product of one head in one block, for
// small token counts (T <= 16 * MT).  Blocks [0, N): head h.  Its W^UK
// fragments are loaded first (one wave group per 64-column window of Hckv,
// the groups splitting the D stages), so their latency hides under the first
// phase; then one wave group per nope window of W^UqQr splits the Hcq stages,
// the groups are summed, and q^C is rounded to bf16 straight into LDS,
// fragment-packed (it never goes to HBM); then q^C W^UK[h] gives q^N (bf16,
// or the per-(token, head) int8 quantisation with the row maximum taken over
// the window groups).  Blocks [N, 2N): head h's rope window through RoPE to
// queryRopeOut.  512 threads.
constexpr int kK34Waves = 8, kK34Stages = 4;

template <bool I8, int MT, int D, bool Q8, int NW = kK34Waves, int NS2 = kK34Stages>
__global__ __launch_bounds__(64 * NW) void k34_stream(Dims d, Ptrs p, PackGeo pg) {
  using St = Stage<I8>;
  constexpr int W = MT * 16 * 64;
  constexpr int RED = (NW - 1) * W * 4, QCL = 16 * MT * 4 * 32 * 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[RED + QCL + NW * 16 * MT * 4];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const bool rope_blk = int(blockIdx.x) >= d.N;
  const int h = rope_blk ? blockIdx.x - d.N : blockIdx.x;
  const int P = pg.nope_w;
  const rsrc_t Wp = make_rsrc(p.packed, pg.total);
  const int64_t ctile = int64_t(pg.nst_cq) * 1024;
  const APacked<I8, MT> ap{make_rsrc(p.cq, int64_t((d.T + 15) / 16) * ctile), uint32_t(ctile)};
  uint32_t* red = reinterpret_cast<uint32_t*>(lds);
  typename St::Acc acc[MT][4];

  if (rope_blk) {
    const int col0 = h * (d.D + d.Dr) + d.D;
    const int ns = w < pg.nst_cq ? (pg.nst_cq - w + NW - 1) / NW : 0;
    const int64_t wbase = pg.off_uq + int64_t(h * (P + 1) + P) * pg.nst_cq * 4096;
    stream_packed<I8, MT, D>(ap, Wp, uint32_t(wbase), w, NW, ns, acc);
    reduce_groups<MT>(acc, red, NW, 1);
    float* E = reinterpret_cast<float*>(lds);  // [16*MT][65], over the reduction area
    if (w == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ml = 16 * mt + 4 * g + i, col = 16 * ct + c;
            float v;
            if constexpr (I8)
              v = (ml < d.T && col < d.Dr)
                      ? udq(p, acc[mt][ct][i], ml, col0 + col)
                      : 0.0f;
            else
              v = acc[mt][ct][i];
            E[ml * 65 + col] = v;
          }
    }
    __syncthreads();
    const int hf = d.Dr / 2;
    for (int idx = threadIdx.x; idx < 16 * MT * hf; idx += 64 * NW) {
      const int ml = idx / hf, i = idx % hf;
      if (ml >= d.T) continue;
      const float a = E[ml * 65 + i], b = E[ml * 65 + i + hf];
      const uint16_t* cs = p.cos + int64_t(ml) * d.Dr;
      const uint16_t* sn = p.sin + int64_t(ml) * d.Dr;
      uint16_t* o = p.qr_out + (int64_t(ml) * d.N + h) * d.qrs;
      o[i] = f2bf(a * bf2f(cs[i]) - b * bf2f(sn[i]));
      o[i + hf] = f2bf(b * bf2f(cs[i + hf]) + a * bf2f(sn[i + hf]));
    }
    return;
  }

  // W^UK[h] fragments of this wave's stages
  const int uk_w = pg.uk_w, nst_d = pg.nst_d;
  const int G2 = NW / uk_w, jw = w / G2, r2 = w % G2;
  const bool act2 = jw < uk_w && r2 < nst_d;
  const int ns2 = act2 ? (nst_d - r2 + G2 - 1) / G2 : 0;
  const uint32_t wb2 = uint32_t(pg.off_uk + int64_t(h * uk_w + (jw < uk_w ? jw : 0)) * nst_d * 4096);
  uint4 bk[NS2][4];
#pragma unroll
  for (int j = 0; j < NS2; ++j)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      bk[j][ct] = bload16(Wp, j < ns2 ? wb2 + uint32_t(r2 + j * G2) * 4096u + uint32_t(ct * 1024 + lane * 16)
                                      : kOOB);

  // phase 1: the nope windows
  const int G1 = NW / P, p1 = w / G1, r1 = w % G1;
  const bool act1 = p1 < P && r1 < pg.nst_cq;
  const int ns1 = act1 ? (pg.nst_cq - r1 + G1 - 1) / G1 : 0;
  const uint32_t wb1 = uint32_t(pg.off_uq + int64_t(h * (P + 1) + (p1 < P ? p1 : 0)) * pg.nst_cq * 4096);
  stream_packed<I8, MT, D>(ap, Wp, wb1, r1, G1, ns1, acc);
  reduce_groups<MT>(acc, red, G1, P);
  uint8_t* qcl = lds + RED;
  const int64_t qt = int64_t(nst_d) * 1024;
  if (p1 < P && r1 == 0) {
    const int col0 = h * (d.D + d.Dr) + 64 * p1;
    const int width = min(64, d.D - 64 * p1), wq = min(64, 32 * nst_d - 64 * p1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * mt + 4 * g + i, col = 16 * ct + c;
          if (col >= wq) continue;
          float v;
          if constexpr (I8)
            v = (row < d.T && col < width)
                    ? udq(p, acc[mt][ct][i], row, col0 + col)
                    : 0.0f;
          else
            v = acc[mt][ct][i];
          *reinterpret_cast<uint16_t*>(qcl + packed_offset(row, 64 * p1 + col, qt, false)) = f2bf(v);
        }
  }
  __syncthreads();

  // phase 2: q^N = q^C W^UK[h]
  const ALds<MT> al{qcl, uint32_t(qt)};
  typename Stage<false>::Acc acc2[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc2[mt][ct] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < NS2; ++j) {
    if (j >= ns2) break;
    uint4 a[MT];
    al.load(a, r2 + j * G2, true);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 af = __builtin_bit_cast(bf16x8, a[mt]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc2[mt][ct] = mfma(af, __builtin_bit_cast(bf16x8, bk[j][ct]), acc2[mt][ct]);
    }
  }
  reduce_groups<MT>(acc2, red, G2, uk_w);
  const bool lead = jw < uk_w && r2 == 0;
  const int width2 = lead ? min(64, d.Hckv - 64 * jw) : 0;
  if constexpr (!Q8) {
    if (!lead) return;
    uint16_t* qo = static_cast<uint16_t*>(p.q_out);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * g + i;
        if (row >= d.T) continue;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int col = 16 * ct + c;
          if (col < width2) qo[(int64_t(row) * d.N + h) * d.qs + 64 * jw + col] = f2bf(acc2[mt][ct][i]);
        }
      }
  } else {
    float* rmax = reinterpret_cast<float*>(lds + RED + QCL);   // [NW][16*MT]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = 0.0f;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          if (16 * ct + c < width2) mx = fmaxf(mx, fabsf(acc2[mt][ct][i]));
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        if (lead && c == 0) rmax[jw * 16 * MT + 16 * mt + 4 * g + i] = mx;
      }
    __syncthreads();
    if (!lead) return;
    int8_t* qo = static_cast<int8_t*>(p.q_out);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * g + i;
        if (row >= d.T) continue;
        float amax = rmax[16 * mt + 4 * g + i];
        for (int k = 1; k < uk_w; ++k) amax = fmaxf(amax, rmax[k * 16 * MT + 16 * mt + 4 * g + i]);
        const float sc = amax / 127.0f;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int col = 16 * ct + c;
          if (col < width2)
            qo[(int64_t(row) * d.N + h) * d.qs + 64 * jw + col] =
                sc > 0.0f ? quant_code(acc2[mt][ct][i], sc) : int8_t(0);
        }
        if (jw == 0 && c == 0) p.q_scale[int64_t(row) * d.N + h] = sc;
      }
  }
}

// K34p: the up-projection and the W^UK product for small token counts
// (T <= 16 * MT) with two blocks per head, for heads of two nope windows and
// Dr = 64.  Half p of head h streams nope window p (q^C columns 64p ..),
// the rope column tiles p and p + 2 (the RoPE pairs i, i + 32 stay in one
// lane) and the W^UK windows of its half of Hckv, so every block moves the
// same bytes.  The halves trade their q^C columns (bf16, 4 KB) through a
// per-head exchange buffer: each block publishes its half with a release
// flag and waits for its partner's, which is already running (a head's two
// blocks are on the same XCD when N % 8 == 0); the wait is bounded and a
// block that gives up marks an error word.  A flag holds the number of the
// run that raised it, so a flag left by an earlier run (also one whose wait
// gave up) never passes for this run's, and nothing is reset between runs.
// Products use swapped MFMA operands
// (weights as the A operand), so a lane's accumulator holds four adjacent
// columns of one token: q^C goes to the exchange buffer in 8-byte pieces,
// q^N and q^R leave in 8-byte stores.  With the int8 query the two halves
// also trade their per-token row maxima.  The wave partial sums are added in
// wave order, so the result is deterministic.  512 threads.

// The exchanged words are written and read with agent-scope relaxed atomics,
// which bypass the caches that are not coherent across XCDs, so no L2
// writeback or invalidation (an agent-scope fence) is needed: a wave waits
// for its own exchange stores to complete, the block meets at a barrier, and
// one lane raises the flag.
__device__ __forceinline__ void xstore64(void* p, uint2 v) {
  __hip_atomic_store(static_cast<uint64_t*>(p), (uint64_t(v.y) << 32) | v.x, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint4 xload128(const void* p) {
  const uint64_t a = __hip_atomic_load(static_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b =
      __hip_atomic_load(static_cast<const uint64_t*>(p) + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_uint4(uint32_t(a), uint32_t(a >> 32), uint32_t(b), uint32_t(b >> 32));
}

__device__ __forceinline__ void pair_publish(uint32_t* flag, uint32_t run) {
  __builtin_amdgcn_s_waitcnt(0);   // this wave's exchange stores have completed
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// waits (at most `spin` poll steps) until the partner's flag holds this run's
// number; the flag is left as it is
__device__ __forceinline__ void pair_wait(const uint32_t* flag, uint32_t* err, uint32_t run, int spin) {
  if (threadIdx.x == 0) {
    int n = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != run) {
      if (++n > spin) {
        __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

constexpr int kPairXq = 8192;   // exchange bytes per head: 2 token tiles x 4 D stages x 1 KB

template <bool I8, int MT, bool Q8, int D = 2, bool F16 = false>
__global__ __launch_bounds__(512) void k34_pair(Dims d, Ptrs p, PackGeo pg) {
  static_assert(!F16 || (I8 && !Q8), "fp16 tensors: the static scenario, 16-bit q^N");
  using St = Stage<I8>;
  using Acc = typename St::Acc;
  using Frag = typename St::Frag;
  constexpr int NW = 8, NT = 6 * MT;   // parked tiles per wave: nope MT x 4, rope MT x 2
  __shared__ uint4 red[NW * NT * 64];
  __shared__ float rmw[NW][32];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int b = blockIdx.x;
  const int h = d.N % 8 == 0 ? (b / 16) * 8 + b % 8 : b / 2;
  const int half = d.N % 8 == 0 ? (b / 8) % 2 : b % 2;
  const int P = pg.nope_w, DDr = d.D + d.Dr;
  const rsrc_t Wp = make_rsrc(p.packed, pg.total);
  const int64_t ctile = int64_t(pg.nst_cq) * 1024;
  const APacked<I8, MT> ap{make_rsrc(p.cq, int64_t((d.T + 15) / 16) * ctile), uint32_t(ctile)};
  uint8_t* xq = p.xq + int64_t(h) * kPairXq;

  // W^UK fragments first: window j of this half, column tiles 2 (w % 2) + k,
  // every D stage; their latency hides under the stream
  const int ja = (pg.uk_w + 1) / 2, jlo = half ? ja : 0, jhi = half ? pg.uk_w : ja;
  const int j = jlo + w / 2, ctu = 2 * (w % 2);
  const bool ukact = j < jhi;
  const uint32_t ukb = uint32_t(pg.off_uk + int64_t(h * pg.uk_w + (ukact ? j : 0)) * pg.nst_d * 4096);
  uint4 bu[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int k = 0; k < 2; ++k)
      bu[s][k] = bload16(Wp, ukact && s < pg.nst_d ? ukb + uint32_t(s * 4096 + (ctu + k) * 1024 + lane * 16)
                                                   : kOOB);

  // the stream: stages w, w + 8, ... of nope window `half` (4 column tiles)
  // and of the rope window (column tiles half, half + 2), one activation load
  // for both
  const uint32_t nb = uint32_t(pg.off_uq + int64_t(h * (P + 1) + half) * pg.nst_cq * 4096);
  const uint32_t rb = uint32_t(pg.off_uq + int64_t(h * (P + 1) + P) * pg.nst_cq * 4096);
  const int ns = w < pg.nst_cq ? (pg.nst_cq - w + NW - 1) / NW : 0;
  Acc an[MT][4], ar[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) an[mt][ct] = Acc{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 2; ++k) ar[mt][k] = Acc{0, 0, 0, 0};
  }
  uint4 qb[D][6], qa[D][MT];
  auto issue = [&](int q, int jj) {
    const int st = w + jj * NW;
    const bool ok = jj < ns;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      qb[q][ct] = bload16(Wp, ok ? nb + uint32_t(st) * 4096u + uint32_t(ct * 1024 + lane * 16) : kOOB);
#pragma unroll
    for (int k = 0; k < 2; ++k)
      qb[q][4 + k] = bload16(Wp, ok ? rb + uint32_t(st) * 4096u + uint32_t((half + 2 * k) * 1024 + lane * 16)
                                    : kOOB);
    ap.load(qa[q], st, ok);
  };
  auto consume = [&](int q) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const Frag af = ap.frag(qa[q], mt);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) an[mt][ct] = mfma(__builtin_bit_cast(Frag, qb[q][ct]), af, an[mt][ct]);
#pragma unroll
      for (int k = 0; k < 2; ++k) ar[mt][k] = mfma(__builtin_bit_cast(Frag, qb[q][4 + k]), af, ar[mt][k]);
    }
  };
#pragma unroll
  for (int q = 0; q < D; ++q) {
    issue(q, q);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the last round issues no refills, so no load is left in flight
  const int nsr = (ns + D - 1) / D * D;
  for (int j0 = 0; j0 < nsr - D; j0 += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
      consume(q);
      issue(q, j0 + q + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int q = 0; q < D; ++q) {
    consume(q);
    __builtin_amdgcn_sched_barrier(0);
  }

  // every wave parks its tiles; tile q is summed in wave order by its owner
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) red[(w * NT + mt * 4 + ct) * 64 + lane] = __builtin_bit_cast(uint4, an[mt][ct]);
#pragma unroll
    for (int k = 0; k < 2; ++k)
      red[(w * NT + 4 * MT + mt * 2 + k) * 64 + lane] = __builtin_bit_cast(uint4, ar[mt][k]);
  }
  __syncthreads();
  auto sum_tile = [&](int q) {
    Acc s = __builtin_bit_cast(Acc, red[q * 64 + lane]);
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) s += __builtin_bit_cast(Acc, red[(w2 * NT + q) * 64 + lane]);
    return s;
  };

  // q^C tile (mt, ct) of this half -> bf16 -> exchange buffer, in the
  // fragment order of the W^UK product's activation operand
  if (w < 4 * MT) {
    const int mt = w / 4, ct = w % 4, t = 16 * mt + c;
    const Acc s = sum_tile(w);
    const int col = 64 * half + 16 * ct + 4 * g;   // q^C column of element 0
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (I8)
        v[r] = (t < d.T && col + r < d.D)
                   ? udq(p, s[r], t, h * DDr + col + r)
                   : 0.0f;
      else
        v[r] = s[r];
    }
    const int st = 2 * half + ct / 2;
    if (st < pg.nst_d)
      xstore64(xq + (mt * 4 + st) * 1024 + (16 * (2 * (ct % 2) + g / 2) + c) * 16 + 8 * (g % 2),
               pack16x4<F16>(v[0], v[1], v[2], v[3]));
  }
  pair_publish(p.xflag + 4 * h + half, d.run);

  // q^R: the owner of token tile mt holds both tiles of every RoPE pair
  if (w >= NW - MT) {
    const int mt = NW - 1 - w, t = 16 * mt + c;
    const Acc a0 = sum_tile(4 * MT + 2 * mt), a1 = sum_tile(4 * MT + 2 * mt + 1);
    if (t < d.T) {
      const int i0 = 16 * half + 4 * g, hf = d.Dr / 2;
      const uint2 c0 = *reinterpret_cast<const uint2*>(p.cos + int64_t(t) * d.Dr + i0);
      const uint2 c1 = *reinterpret_cast<const uint2*>(p.cos + int64_t(t) * d.Dr + i0 + hf);
      const uint2 s0 = *reinterpret_cast<const uint2*>(p.sin + int64_t(t) * d.Dr + i0);
      const uint2 s1 = *reinterpret_cast<const uint2*>(p.sin + int64_t(t) * d.Dr + i0 + hf);
      const uint16_t* cs0 = reinterpret_cast<const uint16_t*>(&c0);
      const uint16_t* cs1 = reinterpret_cast<const uint16_t*>(&c1);
      const uint16_t* sn0 = reinterpret_cast<const uint16_t*>(&s0);
      const uint16_t* sn1 = reinterpret_cast<const uint16_t*>(&s1);
      float o0[4], o1[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float a, bb;
        if constexpr (I8) {
          a = udq(p, a0[r], t, h * DDr + d.D + i0 + r);
          bb = udq(p, a1[r], t, h * DDr + d.D + i0 + hf + r);
        } else {
          a = a0[r];
          bb = a1[r];
        }
        o0[r] = a * ld16<F16>(cs0[r]) - bb * ld16<F16>(sn0[r]);
        o1[r] = bb * ld16<F16>(cs1[r]) + a * ld16<F16>(sn1[r]);
      }
      uint16_t* o = p.qr_out + (int64_t(t) * d.N + h) * d.qrs + i0;
      *reinterpret_cast<uint2*>(o) = pack16x4<F16>(o0[0], o0[1], o0[2], o0[3]);
      *reinterpret_cast<uint2*>(o + hf) = pack16x4<F16>(o1[0], o1[1], o1[2], o1[3]);
    }
  }

  // q^N = q^C W^UK[h] over this half's columns, all of D
  pair_wait(p.xflag + 4 * h + (1 - half), p.herr, d.run, d.spin);
  uint4 aq[4][MT];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      aq[s][mt] = s < pg.nst_d ? xload128(xq + (mt * 4 + s) * 1024 + lane * 16) : make_uint4(0, 0, 0, 0);
  f32x4 au[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      au[mt][k] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        au[mt][k] = mma16<F16>(__builtin_bit_cast(bf16x8, bu[s][k]), __builtin_bit_cast(bf16x8, aq[s][mt]), au[mt][k]);
    }
  const int col0 = 64 * j + 16 * ctu + 4 * g;   // q^N column of element 0 of tile k = 0
  if constexpr (!Q8) {
    if (!ukact) return;
    uint16_t* qo = static_cast<uint16_t*>(p.q_out);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int t = 16 * mt + c;
      if (t >= d.T) continue;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int col = col0 + 16 * k;
        if (col < d.Hckv)
          *reinterpret_cast<uint2*>(qo + (int64_t(t) * d.N + h) * d.qs + col) =
              pack16x4<F16>(au[mt][k][0], au[mt][k][1], au[mt][k][2], au[mt][k][3]);
      }
    }
  } else {
    // per-token max |q^N| of this block, then of the head
    float* xm = p.xmax + int64_t(h) * 64;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float m = 0.0f;
      if (ukact)
#pragma unroll
        for (int k = 0; k < 2; ++k)
          if (col0 + 16 * k < d.Hckv)
#pragma unroll
            for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(au[mt][k][r]));
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (g == 0) rmw[w][16 * mt + c] = m;
    }
    __syncthreads();
    if (w == 0 && lane < 16 * MT) {
      float m = rmw[0][lane];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) m = fmaxf(m, rmw[w2][lane]);
      __hip_atomic_store(xm + 32 * half + lane, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    pair_publish(p.xflag + 4 * h + 2 + half, d.run);
    pair_wait(p.xflag + 4 * h + 2 + (1 - half), p.herr, d.run, d.spin);
    if (!ukact) return;
    int8_t* qo = static_cast<int8_t*>(p.q_out);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int t = 16 * mt + c;
      if (t >= d.T) continue;
      const float amax = fmaxf(__hip_atomic_load(xm + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                               __hip_atomic_load(xm + 32 + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      const float sc = amax / 127.0f;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int col = col0 + 16 * k;
        if (col >= d.Hckv) continue;
        uint32_t u = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          u |= uint32_t(uint8_t(sc > 0.0f ? quant_code(au[mt][k][r], sc) : 0)) << (8 * r);
        *reinterpret_cast<uint32_t*>(qo + (int64_t(t) * d.N + h) * d.qs + col) = u;
      }
      if (half == 0 && w == 0 && g == 0) p.q_scale[int64_t(t) * d.N + h] = sc;
    }
  }
}

// ---------------------------------------------------------------------------
// Fused small-T kernel: the whole prolog (bf16; with I8U the partial
// quantisation scenario: bf16 down-projection, int8 c^Q and W^UqQr; with ST
// as well the static scenario: int8 x codes and weights, bias0/deScale0,
// static c^Q codes, bias1/deScale1) in one launch of 2N blocks, two per
// head, 512 threads, all resident on the device at once (the host checks
// the occupancy before it picks this kernel).
//
// Phase 1.  Blocks 0 .. P1-1 each take a split of the He k-stages of one
// 64-column window of [W^DQ | W^DkvKr] (at most eight splits a window, the
// blocks spread over the windows).  Every wave streams its stages straight
// into MFMA, the waves are summed in LDS, and wave 0 publishes the block's
// [16 MT][64] fp32 partial.
//
// Window sum.  Each 8-byte word of a partial carries the run number next
// to its value, so the split blocks of a window need no counter: each polls
// the window's partials for its own rows until every word holds this run's
// tag, then sums them in split order (the bits do not depend on which block
// finishes first).  It publishes each row's sum of y^2 over the window (over
// the c^KV columns in the c^KV / k^R windows), tagged the same way; the
// c^KV / k^R blocks also publish y as fp32 rows.  A c^Q block then polls the
// tagged window sums of its rows, adds them in a fixed order (the same bits
// in every block) and writes c^Q = bf16(gamma_cq y / rms), fragment-packed
// like c^Q on the packed path: the rounding point of the row-by-row
// RmsNorm.  With I8U each c^Q window's split blocks also publish the row's
// max |gamma m y| over the window (m: smoothScalesCq), tagged next to the
// sum of squares, so the c^Q blocks take the row's int8 scale
// s = max |c^Q m| / 127 from the same poll and write int8 codes (and window
// 0's blocks the scale) instead; with ST the window sums are exact int32
// sums made y = (acc + bias0) deScale0 in double, and c^Q takes the static
// codes of gamma y / rms + beta1.  Every split block raises its own flag once
// its stores are complete, and every block waits for all flags of the run.
//
// Phase 3 is the paired up-projection and W^UK product of k34_pair.  One
// wave per block also writes one 64-column chunk of a c^KV row (and, for
// chunk 0, the RoPE'd k^R row) to the token's cache slot.
//
// Data that crosses blocks moves through agent-scope atomic loads and stores
// (coherent across the XCDs' L2 caches; aligned 8-byte words are
// single-copy atomic), and a wave waits for its stores before it raises a
// flag; no cache writeback or invalidation is needed.  Tags and flags hold
// the run number the host passes (1, 2, ...), so nothing is reset between
// runs.  Polling the data itself instead of counting arrivals keeps atomics
// off the critical path: many same-address atomics arriving together
// serialise.  Every wait is bounded and marks the error word when it gives
// up.
//
// The memory counter of a wave completes in order, so a wave that waits on
// another block must not have loads of its own in flight: wave 0 does all the
// waiting and takes no phase-3 k-stages, while waves 1..7 share the Hcq
// stages, issue their W^UK loads right behind phase 1's and the first
// kFusedPE k-stages of phase 3 once wave 0 has summed its window rows, and
// hold them in registers through the rest of the wait.  Wave 0 issues no load that spans
// that point (the compiler merges outstanding-load counts where the waves'
// paths join, so a load older than the prefetch would make wave 0 wait for
// loads it never issued).
// ---------------------------------------------------------------------------
constexpr int kFusedP1 = 4;       // phase-1 k-stages a wave may have
constexpr int kFusedPF = 4;       // phase-3 register ring: k-stages a wave has in flight
constexpr int kFusedPE = 3;       // of those, the ones issued before the wait
constexpr int kFusedStages = 7;   // phase-3 k-stages a wave may have (waves 1..7)
constexpr int kFusedMaxSplits = 8;
constexpr int kFusedRowSets = 2;  // rows per lane polled together in the handoffs (two per pass)
constexpr int kFusedFlagStride = 16;   // uint32 words between the fused kernel's flags
constexpr int kFusedSpin = 1 << 20;   // poll steps before a wait gives up (about a second)

struct FusedGeo {
  int nwin;            // windows of [W^DQ | W^DkvKr]
  int hi_win, hi_s;    // windows below hi_win take hi_s splits, the others hi_s - 1
  int p1;              // blocks with phase-1 work (the sum of the splits)
};

// a 16-byte buffer load coherent at agent scope (the sc1 cache policy of an
// agent-scope atomic load)
__device__ __forceinline__ uint4 bload16c(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}
__device__ __forceinline__ float bload4c(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 16));
}
__device__ __forceinline__ uint2 bload8u(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 16));
}
// one step of a bounded wave-wide poll: true once every lane's `ok` holds;
// after `spin` steps it marks the error word and gives up
__device__ __forceinline__ bool fused_poll_done(bool ok, int& n, int spin, uint32_t* err) {
  if (__builtin_amdgcn_ballot_w64(!ok) == 0) return true;
  if (++n > spin) {
    if ((threadIdx.x & 63) == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    return true;
  }
  __builtin_amdgcn_s_sleep(2);
  return false;
}

template <int MT, bool I8U = false, bool ST = false>
__global__ __launch_bounds__(512) void k_fused(Dims d, Ptrs p, PackGeo pg, FusedGeo fg) {
  static_assert(!ST || I8U, "the static scenario is int8 throughout");
  using Acc = f32x4;
  // the down-projection's operands: bf16, or (ST, the static scenario) the
  // int8 codes of x and int8 [W^DQ | W^DkvKr], exact int32 partials
  using S1 = Stage<ST>;
  using Acc1 = typename S1::Acc;
  using Frag1 = typename S1::Frag;
  // the up-projection's operands: bf16, or int8 c^Q codes and W^UqQr (the
  // partial-quantisation and static scenarios)
  using S3 = Stage<I8U>;
  using Acc3 = typename S3::Acc;
  using Frag3 = typename S3::Frag;
  constexpr int NW = 8, NT = 6 * MT, R = 16 * MT;
  __shared__ __attribute__((aligned(16))) uint4 red[NW * NT * 64];
  // int8: the dequantisation scales of the block's 96 up-projection columns
  // (nope window `half`, then rope column tiles half and half + 2)
  __shared__ float swl[I8U ? 96 : 1];
  __shared__ int32_t bsl[ST ? 96 : 1];   // ST: their bias1
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int b = blockIdx.x, G = gridDim.x;
  const rsrc_t Wp = make_rsrc(p.packed, pg.total);
  // flags of the split blocks, one per 64-byte line
  uint32_t* const flag = p.fcnt;
  uint32_t* const err = p.herr;
  // int8 c^Q: the row maxima's tagged words follow the sums of squares
  uint32_t* const fgm = p.fss + (pg.win_dq + pg.win_kr) * 64;

  // ---- the block's head and half in phase 3 (as in k34_pair)
  const int h = d.N % 8 == 0 ? (b / 16) * 8 + b % 8 : b / 2;
  const int half = d.N % 8 == 0 ? (b / 8) % 2 : b % 2;
  const int P = pg.nope_w, DDr = d.D + d.Dr;
  const int ja = (pg.uk_w + 1) / 2, jlo = half ? ja : 0, jhi = half ? pg.uk_w : ja;
  const int jw = jlo + w / 2, ctu = 2 * (w % 2);
  const bool ukact = jw < jhi;
  const uint32_t ukb = uint32_t(pg.off_uk + int64_t(h * pg.uk_w + (ukact ? jw : 0)) * pg.nst_d * 4096);
  const uint32_t nb = uint32_t(pg.off_uq + int64_t(h * (P + 1) + half) * pg.nst_cq * 4096);
  const uint32_t rb = uint32_t(pg.off_uq + int64_t(h * (P + 1) + P) * pg.nst_cq * 4096);
  // phase-3 k-stages: wave w >= 1 takes stages w - 1, w + 6, ...
  const int ns3 = w >= 1 && w - 1 < pg.nst_cq ? (pg.nst_cq - (w - 1) + NW - 2) / (NW - 1) : 0;
  uint4 bu[4][2];
  uint4 pre[kFusedPF][6];
#pragma unroll
  for (int q = 0; q < kFusedPF; ++q)
#pragma unroll
    for (int i = 0; i < 6; ++i) pre[q][i] = make_uint4(0, 0, 0, 0);
  auto issue_uk = [&](bool ok) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int k = 0; k < 2; ++k)
        bu[s][k] = bload16s(Wp, ok && ukact && s < pg.nst_d
                                   ? ukb + uint32_t(s * 4096 + (ctu + k) * 1024 + lane * 16)
                                   : kOOB);
  };
  // weights of the wave's q-th phase-3 k-stage: the four column tiles of
  // nope window `half`, rope column tiles half and half + 2
  auto issue_w3 = [&](uint4 (&r)[6], int q) {
    const int st = w - 1 + q * (NW - 1);
    const bool ok = q < ns3;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      r[ct] = bload16s(Wp, ok ? nb + uint32_t(st) * 4096u + uint32_t(ct * 1024 + lane * 16) : kOOB);
#pragma unroll
    for (int k = 0; k < 2; ++k)
      r[4 + k] = bload16s(Wp, ok ? rb + uint32_t(st) * 4096u + uint32_t((half + 2 * k) * 1024 + lane * 16) : kOOB);
  };

  // ---- phase 1: block -> split s of S of window j
  int j = 0, s = 0, S = 0, jfirst = 0;
  if (b < fg.p1) {
    const int nhi = fg.hi_win * fg.hi_s;
    if (b < nhi) {
      j = b / fg.hi_s; s = b % fg.hi_s; S = fg.hi_s; jfirst = j * fg.hi_s;
    } else {
      S = fg.hi_s - 1;
      j = fg.hi_win + (b - nhi) / S; s = (b - nhi) % S; jfirst = nhi + (j - fg.hi_win) * S;
    }
  }
  const int st0 = S ? s * pg.nst_he / S : 0, st1 = S ? (s + 1) * pg.nst_he / S : 0;
  const int ns1 = st0 + w < st1 ? (st1 - st0 - w + NW - 1) / NW : 0;
  const uint32_t w1b = uint32_t(j < pg.win_dq ? pg.off_dq + int64_t(j) * pg.nst_he * 4096
                                              : pg.off_kr + int64_t(j - pg.win_dq) * pg.nst_he * 4096);
  const APlain<ST, MT> ax{make_rsrc(p.x, int64_t(d.T) * d.He * S1::EB), uint32_t(d.He * S1::EB), d.T, d.He};
  uint4 b1[kFusedP1][4], a1[kFusedP1][MT];
#pragma unroll
  for (int q = 0; q < kFusedP1; ++q) {
    const int st = st0 + w + q * NW;
    const bool ok = q < ns1;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      b1[q][ct] = bload16s(Wp, ok ? w1b + uint32_t(st) * 4096u + uint32_t(ct * 1024 + lane * 16) : kOOB);
    ax.load(a1[q], st, ok);
  }
  __builtin_amdgcn_sched_barrier(0);
  // waves 1..7 fetch their W^UK fragments behind phase 1's loads: phase 1
  // leaves HBM short of its rate, and phase 1's waits are for the loads
  // issued before these (wave 0's are out of range and return at once)
  issue_uk(w != 0);
  // int8: the 96 column scales, behind phase 1's loads; they go to LDS once
  // phase 1's waves have been summed
  float swv = 0.0f;
  int32_t bsv = 0;
  if constexpr (I8U) {
    const int k = threadIdx.x;
    const int col = k < 64 ? 64 * half + k : d.D + 16 * (half + 2 * ((k - 64) >> 4)) + (k & 15);
    if (k < 96 && (k >= 64 || col < d.D)) {
      swv = p.sw_uq_qr[h * DDr + col];
      if (ST && p.bias_uq) bsv = p.bias_uq[h * DDr + col];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  Acc1 acc1[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc1[mt][ct] = Acc1{0, 0, 0, 0};
#pragma unroll
  for (int q = 0; q < kFusedP1; ++q)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const Frag1 af = __builtin_bit_cast(Frag1, a1[q][mt]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        acc1[mt][ct] = mma16<false>(af, __builtin_bit_cast(Frag1, b1[q][ct]), acc1[mt][ct]);
    }
  reduce_waves<NW, MT>(acc1, reinterpret_cast<uint32_t*>(red));
  if constexpr (I8U) {
    if (threadIdx.x < 96) {
      swl[threadIdx.x] = swv;
      if constexpr (ST) bsl[threadIdx.x] = bsv;
    }
  }

  // wave 0 of a split block publishes the block's partial before any
  // prefetch is issued (its memory pipeline is then free of other loads).
  // Its rows of the window are summed below: lane -> row 2 pass + lane / 32,
  // columns 2 (lane % 32) and + 1.
  const int r0 = S ? s * R / S : 0, r1 = S ? (s + 1) * R / S : 0, q2 = lane & 31;
  const bool qwin = j < pg.win_dq;
  const int col0 = (qwin ? 64 * j : 64 * (j - pg.win_dq)) + 2 * q2;   // column in W^DQ or W^DkvKr
  const uint32_t run = d.run;
  // int8 c^Q: gamma times the smoothing factor of the lane's two columns
  double gq2[2] = {0.0, 0.0};
  // ST: the lane's columns' bias0 and deScale0 (y = (acc + bias) deScale,
  // in double), and beta1 of its c^Q columns
  int32_t bq2[2] = {0, 0};
  double sw2[2] = {0.0, 0.0}, be2[2] = {0.0, 0.0};
  if constexpr (I8U) {
    if (w == 0 && S && qwin) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
        if (col0 + e < d.Hcq) {
          gq2[e] = double(bf2f(p.gamma_cq[col0 + e])) * (p.smooth_cq ? double(p.smooth_cq[col0 + e]) : 1.0);
          if constexpr (ST) be2[e] = double(bf2f(p.beta_cq[col0 + e]));
        }
    }
  }
  if constexpr (ST) {
    if (w == 0 && S) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int cc = col0 + e;
        if (cc < (qwin ? d.Hcq : d.Hckv + d.Dr)) {
          if (p.bias_dq) bq2[e] = p.bias_dq[(qwin ? 0 : d.Hcq) + cc];
          sw2[e] = double(qwin ? p.sw_dq[cc] : p.sw_dkv_kr[cc]);
        }
      }
    }
  }
  if (w == 0 && S) {
    // the block's partial, rows 16 mt + 4 g + i, columns 16 ct + c, each
    // value next to this run's tag
    uint32_t* mine = p.fpart + int64_t(b) * R * 64 * 2;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const auto v = acc1[mt][ct][i];
          xstore64(mine + ((16 * mt + 4 * g + i) * 64 + 16 * ct + c) * 2,
                   make_uint2(__builtin_bit_cast(uint32_t, v), run));
        }
  }
  float* const ylds = reinterpret_cast<float*>(red);   // [R][64] y of the c^Q window rows
  double* const ylds_d = reinterpret_cast<double*>(red);   // ST: in double
  if (w == 0 && S) {
    {
      const rsrc_t Fp = make_rsrc(p.fpart, int64_t(fg.p1) * R * 64 * 8);
      // kFusedRowSets row pairs per poll: the rows of a block are published
      // together, so one round trip serves them all
      for (int rb = r0; rb < r1; rb += 2 * kFusedRowSets) {
        int rr[kFusedRowSets];
        bool act[kFusedRowSets];
#pragma unroll
        for (int u = 0; u < kFusedRowSets; ++u) {
          rr[u] = rb + 2 * u + (lane >> 5);
          act[u] = rr[u] < r1;
        }
        // S <= kFusedMaxSplits; the words past S are not waited for
        uint2 v[kFusedRowSets][kFusedMaxSplits][2];
        int n = 0;
        for (;;) {
#pragma unroll
          for (int u = 0; u < kFusedRowSets; ++u)
#pragma unroll
            for (int k = 0; k < kFusedMaxSplits; ++k)
#pragma unroll
              for (int e = 0; e < 2; ++e)
                v[u][k][e] = bload8u(Fp, act[u] && k < S ? uint32_t(((jfirst + k) * R + rr[u]) * 64 + 2 * q2 + e) * 8u
                                                       : kOOB);
          bool ok = true;
#pragma unroll
          for (int u = 0; u < kFusedRowSets; ++u)
#pragma unroll
            for (int k = 0; k < kFusedMaxSplits; ++k)
#pragma unroll
              for (int e = 0; e < 2; ++e) ok &= !(act[u] && k < S) || v[u][k][e].y == run;
          if (fused_poll_done(ok, n, d.spin, err)) break;
        }
#pragma unroll
        for (int u = 0; u < kFusedRowSets; ++u) {
          const int r = rr[u];
          float y[2] = {0, 0};
          double yd[2];   // ST: y in double
          if constexpr (ST) {
            // exact int32 sums, then (acc + bias0) deScale0
            int32_t iy[2] = {0, 0};
#pragma unroll
            for (int k = 0; k < kFusedMaxSplits; ++k)
#pragma unroll
              for (int e = 0; e < 2; ++e) iy[e] += int32_t(v[u][k][e].x);   // words past S read zeros
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              yd[e] = double(iy[e] + bq2[e]) * sw2[e];
              y[e] = float(yd[e]);
            }
          } else {
#pragma unroll
            for (int k = 0; k < kFusedMaxSplits; ++k)
#pragma unroll
              for (int e = 0; e < 2; ++e) y[e] += __uint_as_float(v[u][k][e].x);   // words past S read zeros
#pragma unroll
            for (int e = 0; e < 2; ++e) yd[e] = double(y[e]);
          }
          // the row's sum of squares over the window (c^KV columns only in
          // the c^KV / k^R windows), tagged
          double ss = 0.0;
#pragma unroll
          for (int e = 0; e < 2; ++e)
            if (qwin || col0 + e < d.Hckv) ss += yd[e] * yd[e];
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) ss += __shfl_xor(ss, o, 64);
          if (act[u] && q2 == 0) xstore64(p.fss + (j * 32 + r) * 2, make_uint2(__float_as_uint(float(ss)), run));
          if constexpr (I8U && !ST) {
            // and the row's max |gamma m y| over the window, for c^Q's int8 scale
            if (qwin) {
              double gm = fmax(fabs(gq2[0] * double(y[0])), fabs(gq2[1] * double(y[1])));
#pragma unroll
              for (int o = 1; o < 32; o <<= 1) gm = fmax(gm, __shfl_xor(gm, o, 64));
              if (act[u] && q2 == 0) xstore64(fgm + (j * 32 + r) * 2, make_uint2(__float_as_uint(float(gm)), run));
            }
          }
          if (!act[u]) continue;
          if (qwin && ST) {
            ylds_d[r * 64 + 2 * q2] = yd[0];
            ylds_d[r * 64 + 2 * q2 + 1] = yd[1];
          } else if (qwin) {
            ylds[r * 64 + 2 * q2] = y[0];
            ylds[r * 64 + 2 * q2 + 1] = y[1];
          } else if (col0 < d.Hckv + d.Dr) {
            // Hckv + Dr is even: the lane's 2 columns are both in the row
            xstore64(p.fykr + r * (d.Hckv + d.Dr) + col0, make_uint2(__float_as_uint(y[0]), __float_as_uint(y[1])));
          }
        }
      }
    }
  }
  // the phase-3 ring prefetch goes out once phase 1's loads are in (so that
  // it does not delay them) and wave 0 has summed its window rows (the
  // partials land far faster while HBM is quiet); the barrier orders LDS only
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  if (w != 0) {
#pragma unroll
    for (int q = 0; q < kFusedPE; ++q) issue_w3(pre[q], q);
  }
  __builtin_amdgcn_sched_barrier(0);

  if (w == 0) {
    if (S) {
      if (qwin) {
        // c^Q = bf16(gamma y / rms) once every window sum of the rows is out
        const uint32_t gq = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.gamma_cq, int64_t(d.Hcq) * 2),
                                                                 col0 < d.Hcq ? col0 * 2u : kOOB, 0, 0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const rsrc_t Sp = make_rsrc(p.fss, int64_t(pg.win_dq) * 32 * 8);
        const rsrc_t Gp = make_rsrc(fgm, I8U ? int64_t(pg.win_dq) * 32 * 8 : 0);
        for (int rb = r0; rb < r1; rb += 2 * kFusedRowSets) {
          int rr[kFusedRowSets];
          bool act[kFusedRowSets];
          double ss[kFusedRowSets];
          float gmx[kFusedRowSets];   // int8: the row's max |gamma m y| so far
#pragma unroll
          for (int u = 0; u < kFusedRowSets; ++u) {
            rr[u] = rb + 2 * u + (lane >> 5);
            act[u] = rr[u] < r1;
            ss[u] = 0.0;
            gmx[u] = 0.0f;
          }
          // lane q2 adds windows q2, q2 + 32, ..., then the row's 32 lanes
          // are added: a fixed order, the same in every block; the row sets
          // are polled together
          for (int j0 = q2; j0 < pg.win_dq; j0 += 128) {
            uint2 v[kFusedRowSets][4], vg[kFusedRowSets][I8U ? 4 : 1];
            int n = 0;
            for (;;) {
#pragma unroll
              for (int u = 0; u < kFusedRowSets; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                  const int jj = j0 + 32 * k;
                  v[u][k] = bload8u(Sp, act[u] && jj < pg.win_dq ? uint32_t(jj * 32 + rr[u]) * 8u : kOOB);
                  if constexpr (I8U && !ST)
                    vg[u][k] = bload8u(Gp, act[u] && jj < pg.win_dq ? uint32_t(jj * 32 + rr[u]) * 8u : kOOB);
                }
              bool ok = true;
#pragma unroll
              for (int u = 0; u < kFusedRowSets; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                  ok &= !(act[u] && j0 + 32 * k < pg.win_dq) || v[u][k].y == run;
                  if constexpr (I8U && !ST) ok &= !(act[u] && j0 + 32 * k < pg.win_dq) || vg[u][k].y == run;
                }
              if (fused_poll_done(ok, n, d.spin, err)) break;
            }
#pragma unroll
            for (int u = 0; u < kFusedRowSets; ++u)
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                ss[u] += double(__uint_as_float(v[u][k].x));   // zeros past win_dq
                if constexpr (I8U && !ST) gmx[u] = fmaxf(gmx[u], __uint_as_float(vg[u][k].x));
              }
          }
#pragma unroll
          for (int u = 0; u < kFusedRowSets; ++u) {
            const int r = rr[u];
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) ss[u] += __shfl_xor(ss[u], o, 64);
            if constexpr (ST) {
              // static codes of c^Q + beta1 (quantScale1, quantOffset1); the
              // even lane of each pair stores the pair's four codes
              const double rms = sqrt(ss[u] / double(d.Hcq) + d.eps_cq);
              const float st_s = bf2f(*p.qsc_cq), st_o = float(*p.qo_cq);
              uint32_t mine = 0;
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const float cv = float(gq2[e] * ylds_d[r * 64 + 2 * q2 + e] / rms + be2[e]);
                mine |= static_code(cv, st_s, st_o) << (8 * e);
              }
              const uint32_t other = __shfl_xor(mine, 1, 64);
              if (act[u] && (q2 & 1) == 0) {
                uint32_t* dst = reinterpret_cast<uint32_t*>(
                    p.cq + packed_offset(r, col0, int64_t(pg.nst_cq) * 1024, true));
                __hip_atomic_store(dst, mine | (other << 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              }
              continue;
            } else if constexpr (I8U) {
              // int8 c^Q: the row's scale s = max |c^Q m| / 127 and the
              // codes of the lane's two columns; the even lane of each pair
              // stores the pair's four codes, and window 0's blocks the scale
#pragma unroll
              for (int o = 1; o < 32; o <<= 1) gmx[u] = fmaxf(gmx[u], __shfl_xor(gmx[u], o, 64));
              const double rms = sqrt(ss[u] / double(d.Hcq) + d.eps_cq);
              const float sc = float(double(gmx[u]) / rms) / 127.0f;
              uint32_t mine = 0;
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const float cv = float(gq2[e] * double(ylds[r * 64 + 2 * q2 + e]) / rms);
                mine |= uint32_t(uint8_t(sc > 0.0f ? quant_code(cv, sc) : int8_t(0))) << (8 * e);
              }
              const uint32_t other = __shfl_xor(mine, 1, 64);
              if (act[u] && (q2 & 1) == 0) {
                uint32_t* dst = reinterpret_cast<uint32_t*>(
                    p.cq + packed_offset(r, col0, int64_t(pg.nst_cq) * 1024, true));
                __hip_atomic_store(dst, mine | (other << 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              }
              if (act[u] && j == 0 && q2 == 0 && r < d.T)
                __hip_atomic_store(p.cq_scale + r, sc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              continue;
            }
            const int stg = col0 / 32;
            if (act[u] && stg < pg.nst_cq) {
              const double rms = sqrt(ss[u] / double(d.Hcq) + d.eps_cq);
              const float c0 = float(double(bf2f(uint16_t(gq))) * double(ylds[r * 64 + 2 * q2]) / rms);
              const float c1 = float(double(bf2f(uint16_t(gq >> 16))) * double(ylds[r * 64 + 2 * q2 + 1]) / rms);
              uint32_t* dst = reinterpret_cast<uint32_t*>(p.cq + int64_t(r >> 4) * pg.nst_cq * 1024 + stg * 1024 +
                                                          ((((col0 % 32) / 8) * 16 + (r & 15)) * 16) + (col0 % 8) * 2);
              __hip_atomic_store(dst, uint32_t(f2bf(c0)) | (uint32_t(f2bf(c1)) << 16), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
      // the block's outputs are complete: raise its flag.  The stores above
      // and the flag are relaxed atomics to different addresses; the wait
      // for every outstanding memory operation orders them on the device,
      // and the signal fence keeps the compiler from moving the flag store
      // above that wait
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (lane == 0) __hip_atomic_store(flag + b * kFusedFlagStride, run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // wait for the flags of every split block of this run
    int n = 0;
    for (;;) {
      bool ok = true;
      for (int i0 = 0; i0 < fg.p1; i0 += 256) {
        uint32_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = i0 + lane + 64 * k;
          v[k] = i < fg.p1 ? __hip_atomic_load(flag + i * kFusedFlagStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : run;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) ok &= v[k] == run;
      }
      if (fused_poll_done(ok, n, d.spin, err)) break;
    }
  }
  __syncthreads();

  // ---- phase 3 (wave 0's W^UK fragments are only read at the very end)
  if (w == 0) issue_uk(true);
  // int8: c^Q's scale for the lane's tokens c and 16 + c (written this run
  // by window 0's blocks, before their flags)
  float scq[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    scq[mt] = ST ? 1.0f : 0.0f;   // static codes: the per-channel deScale1 does all the scaling
    if constexpr (I8U && !ST)
      if (16 * mt + c < d.T)
        scq[mt] = __hip_atomic_load(p.cq_scale + 16 * mt + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // cache jobs: job jb = (token jb / cj, 64-column chunk jb % cj of c^KV;
  // chunk 0 also writes k^R).  Wave 7 takes jobs b, b + G, ...; the loads of
  // the first are issued now and used after the stream.
  const int cj = (d.Hckv + 63) / 64, W2 = d.Hckv + d.Dr;
  // the loads are predicated buffer loads (no branches), so that their
  // waits come only where the values are used
  struct CacheJob {
    int t, ch;
    float y, a, b2;
    uint32_t gam;
    double ss;
  };
  const rsrc_t Yp = make_rsrc(p.fykr, int64_t(d.T) * W2 * 4);
  const rsrc_t Sk = make_rsrc(p.fss, int64_t(pg.win_dq + pg.win_kr) * 32 * 8);
  const rsrc_t Gk = make_rsrc(p.gamma_ckv, int64_t(d.Hckv) * 2);
  auto job_load = [&](int jb, bool on) {
    CacheJob cjb;
    cjb.t = on ? jb / cj : 0; cjb.ch = on ? jb % cj : 1;
    const int col = 64 * cjb.ch + lane;
    const bool kv = on && col < d.Hckv, kr = on && cjb.ch == 0 && lane < d.Dr / 2;
    cjb.y = bload4c(Yp, kv ? uint32_t(cjb.t * W2 + col) * 4u : kOOB);
    cjb.gam = __builtin_amdgcn_raw_buffer_load_b16(Gk, kv ? uint32_t(col) * 2u : kOOB, 0, 0);
    cjb.a = bload4c(Yp, kr ? uint32_t(cjb.t * W2 + d.Hckv + lane) * 4u : kOOB);
    cjb.b2 = bload4c(Yp, kr ? uint32_t(cjb.t * W2 + d.Hckv + lane + d.Dr / 2) * 4u : kOOB);
    cjb.ss = double(__uint_as_float(
        bload8u(Sk, on && lane < pg.win_kr ? uint32_t((pg.win_dq + lane) * 32 + cjb.t) * 8u : kOOB).x));   // (float, tag)
    return cjb;
  };
  // c^KV = gamma y / rms, k^R = RoPE(y_kr), bf16, at the token's slot
  auto job_store = [&](const CacheJob& cjb) {
    double ssk = cjb.ss;
    for (int o = 32; o > 0; o >>= 1) ssk += __shfl_xor(ssk, o, 64);
    const int64_t slot = p.cache_index[cjb.t];
    if (slot < 0 || slot >= d.slots) return;
    const double rms = sqrt(ssk / double(d.Hckv) + d.eps_ckv);
    const int col = 64 * cjb.ch + lane;
    if (col < d.Hckv)
      p.kv_cache[slot * d.kvs + col] = f2bf(float(double(bf2f(uint16_t(cjb.gam))) * double(cjb.y) / rms));
    if (cjb.ch == 0 && lane < d.Dr / 2) {
      const int hf = d.Dr / 2;
      const uint16_t* cs = p.cos + int64_t(cjb.t) * d.Dr;
      const uint16_t* sn = p.sin + int64_t(cjb.t) * d.Dr;
      uint16_t* kr = p.kr_cache + slot * d.krs;
      kr[lane] = f2bf(float(double(cjb.a) * bf2f(cs[lane]) - double(cjb.b2) * bf2f(sn[lane])));
      kr[lane + hf] = f2bf(float(double(cjb.b2) * bf2f(cs[lane + hf]) + double(cjb.a) * bf2f(sn[lane + hf])));
    }
  };
  // predicated loads rather than a branch: a select between loaded and
  // default values would wait for the loads right here
  const bool cjob = w == NW - 1 && b < d.T * cj;
  const CacheJob job0 = job_load(b, cjob);

  const int64_t ctile = int64_t(pg.nst_cq) * 1024;
  const rsrc_t Cq = make_rsrc(p.cq, int64_t((d.T + 15) / 16) * ctile);
  uint4 aq[kFusedPF][MT];
  auto issue_a = [&](uint4 (&r)[MT], int q) {
    const int st = w - 1 + q * (NW - 1);
    const bool ok = q < ns3;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      r[mt] = bload16c(Cq, ok ? uint32_t(mt * ctile + st * 1024 + lane * 16) : kOOB);
  };
  // the ring's stages that were not prefetched, then the activation operand
#pragma unroll
  for (int q = kFusedPE; q < kFusedPF; ++q) issue_w3(pre[q], q);
#pragma unroll
  for (int q = 0; q < kFusedPF; ++q) issue_a(aq[q], q);
  __builtin_amdgcn_sched_barrier(0);
  Acc3 an[MT][4], ar[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) an[mt][ct] = Acc3{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 2; ++k) ar[mt][k] = Acc3{0, 0, 0, 0};
  }
  auto consume = [&](const uint4 (&wq)[6], const uint4 (&a)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const Frag3 af = __builtin_bit_cast(Frag3, a[mt]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) an[mt][ct] = mma16<false>(__builtin_bit_cast(Frag3, wq[ct]), af, an[mt][ct]);
#pragma unroll
      for (int k = 0; k < 2; ++k) ar[mt][k] = mma16<false>(__builtin_bit_cast(Frag3, wq[4 + k]), af, ar[mt][k]);
    }
  };
  // a register ring of kFusedPF stages: stage q + kFusedPF refills the slot
  // of stage q once that is consumed
#pragma unroll
  for (int q = 0; q < kFusedStages; ++q) {
    consume(pre[q % kFusedPF], aq[q % kFusedPF]);
    __builtin_amdgcn_sched_barrier(0);
    if (q + kFusedPF < kFusedStages) {
      issue_w3(pre[q % kFusedPF], q + kFusedPF);
      issue_a(aq[q % kFusedPF], q + kFusedPF);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // every wave parks its tiles; tile q is summed in wave order by its owner
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) red[(w * NT + mt * 4 + ct) * 64 + lane] = __builtin_bit_cast(uint4, an[mt][ct]);
#pragma unroll
    for (int k = 0; k < 2; ++k)
      red[(w * NT + 4 * MT + mt * 2 + k) * 64 + lane] = __builtin_bit_cast(uint4, ar[mt][k]);
  }
  __syncthreads();
  auto sum_tile = [&](int q) {
    Acc3 sm = __builtin_bit_cast(Acc3, red[q * 64 + lane]);
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) sm += __builtin_bit_cast(Acc3, red[(w2 * NT + q) * 64 + lane]);
    return sm;
  };
  // a summed tile as floats: int8 products dequantised (s_cq of the lane's
  // token, the column's scale), in fp32 as the other int8 paths do
  auto to_f = [&](const Acc3& v, int mt, int k0) {
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (ST) o[i] = static_cast<float>(v[i] + bsl[k0 + i]) * scq[mt] * swl[k0 + i];
      else if constexpr (I8U) o[i] = static_cast<float>(v[i]) * scq[mt] * swl[k0 + i];
      else o[i] = v[i];
    }
    return o;
  };
  uint8_t* xq = p.xq + int64_t(h) * kPairXq;

  // q^C tile (mt, ct) of this half -> bf16 -> exchange buffer, in the
  // fragment order of the W^UK product's activation operand
  if (w < 4 * MT) {
    const int mt = w / 4, ct = w % 4;
    const Acc sm = to_f(sum_tile(w), mt, 16 * ct + 4 * g);
    const int st = 2 * half + ct / 2;
    if (st < pg.nst_d)
      xstore64(xq + (mt * 4 + st) * 1024 + (16 * (2 * (ct % 2) + g / 2) + c) * 16 + 8 * (g % 2),
               pack_bf16x4(sm[0], sm[1], sm[2], sm[3]));
  }
  pair_publish(p.xflag + 4 * h + half, d.run);

  // the cache rows and q^R leave after the exchange is published (its wait
  // for the exchange stores then does not wait for these)
  if (cjob) {
    job_store(job0);
    for (int jb = b + G; jb < d.T * cj; jb += G) job_store(job_load(jb, true));
  }

  // q^R: the owner of token tile mt holds both tiles of every RoPE pair
  if (w >= NW - MT) {
    const int mt = NW - 1 - w, t = 16 * mt + c;
    const Acc a0 = to_f(sum_tile(4 * MT + 2 * mt), mt, 64 + 4 * g),
              a1v = to_f(sum_tile(4 * MT + 2 * mt + 1), mt, 80 + 4 * g);
    if (t < d.T) {
      const int i0 = 16 * half + 4 * g, hf = d.Dr / 2;
      const uint2 c0 = *reinterpret_cast<const uint2*>(p.cos + int64_t(t) * d.Dr + i0);
      const uint2 c1 = *reinterpret_cast<const uint2*>(p.cos + int64_t(t) * d.Dr + i0 + hf);
      const uint2 s0 = *reinterpret_cast<const uint2*>(p.sin + int64_t(t) * d.Dr + i0);
      const uint2 s1 = *reinterpret_cast<const uint2*>(p.sin + int64_t(t) * d.Dr + i0 + hf);
      const uint16_t* cs0 = reinterpret_cast<const uint16_t*>(&c0);
      const uint16_t* cs1 = reinterpret_cast<const uint16_t*>(&c1);
      const uint16_t* sn0 = reinterpret_cast<const uint16_t*>(&s0);
      const uint16_t* sn1 = reinterpret_cast<const uint16_t*>(&s1);
      float o0[4], o1[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = a0[r], bb = a1v[r];
        o0[r] = a * bf2f(cs0[r]) - bb * bf2f(sn0[r]);
        o1[r] = bb * bf2f(cs1[r]) + a * bf2f(sn1[r]);
      }
      uint16_t* o = p.qr_out + (int64_t(t) * d.N + h) * d.qrs + i0;
      *reinterpret_cast<uint2*>(o) = pack_bf16x4(o0[0], o0[1], o0[2], o0[3]);
      *reinterpret_cast<uint2*>(o + hf) = pack_bf16x4(o1[0], o1[1], o1[2], o1[3]);
    }
  }

  // q^N = q^C W^UK[h] over this half's columns, all of D
  pair_wait(p.xflag + 4 * h + (1 - half), p.herr, d.run, d.spin);
  uint4 aqc[4][MT];
#pragma unroll
  for (int st = 0; st < 4; ++st)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      aqc[st][mt] = st < pg.nst_d ? xload128(xq + (mt * 4 + st) * 1024 + lane * 16) : make_uint4(0, 0, 0, 0);
  f32x4 au[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      au[mt][k] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        au[mt][k] = mfma(__builtin_bit_cast(bf16x8, bu[st][k]), __builtin_bit_cast(bf16x8, aqc[st][mt]), au[mt][k]);
    }
  if (!ukact) return;
  const int qcol0 = 64 * jw + 16 * ctu + 4 * g;   // q^N column of element 0 of tile k = 0
  uint16_t* qo = static_cast<uint16_t*>(p.q_out);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int t = 16 * mt + c;
    if (t >= d.T) continue;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int col = qcol0 + 16 * k;
      if (col < d.Hckv)
        *reinterpret_cast<uint2*>(qo + (int64_t(t) * d.N + h) * d.qs + col) =
            pack_bf16x4(au[mt][k][0], au[mt][k][1], au[mt][k][2], au[mt][k][3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Tiled path for larger token counts.  Every wave owns a 16*MT-token x
// 64*NWW-column output tile and streams the packed k-stages of its NWW
// windows against MT activation fragments per stage; 16-byte loads land in
// the registers the MFMAs read, and the waves of a block that share a
// window or a token range share those loads through L1.  The MFMA takes the
// weight fragment as its first operand, so the 16x16 result is the
// transposed tile: lane l holds token l%16 and columns 4*(l/16) + r, r < 4 --
// four consecutive output columns of one token, stored as one 8- or 16-byte
// vector.
// ---------------------------------------------------------------------------
template <bool I8, int MT, int NWW, int D, class AP, bool F16 = false>
__device__ __forceinline__ void tile_mma(const AP& ap, rsrc_t Wp, const uint32_t (&wb)[NWW], int s0,
                                         int ns, typename Stage<I8>::Acc (&acc)[MT][NWW * 4]) {
  using S = Stage<I8>;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NWW * 4; ++j) acc[mt][j] = typename S::Acc{0, 0, 0, 0};
  uint4 bq[D][NWW * 4];
  uint4 aq[D][AP::NR];
  auto issue = [&](uint4 (&b)[NWW * 4], uint4 (&a)[AP::NR], int j) {
    const bool ok = j < ns;
    const uint32_t st = uint32_t(s0 + j);
#pragma unroll
    for (int w = 0; w < NWW; ++w)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        b[w * 4 + ct] = bload16(Wp, ok && wb[w] != kOOB
                                        ? wb[w] + st * 4096u + uint32_t(ct * 1024 + lane * 16)
                                        : kOOB);
    ap.load(a, int(st), ok);
  };
#pragma unroll
  for (int q = 0; q < D; ++q) {
    issue(bq[q], aq[q], q);
    __builtin_amdgcn_sched_barrier(0);   // the loop expects the slots in this order
  }
  // a slot is refilled right after the MFMAs that read it, so the ring
  // needs no spare registers and no copies on the loop's back edge
  const int nsr = (ns + D - 1) / D * D;
  for (int j0 = 0; j0 < nsr; j0 += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const typename S::Frag af = ap.frag(aq[q], mt);
#pragma unroll
        for (int j = 0; j < NWW * 4; ++j)
          acc[mt][j] = mma16<F16>(__builtin_bit_cast(typename S::Frag, bq[q][j]), af, acc[mt][j]);
      }
      issue(bq[q], aq[q], j0 + q + D);
      // keep each slot's MFMAs after its own wait and before the next
      // slot's: the scheduler would otherwise gather every refill at the end
      // of the iteration and wait for all of them at its top
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Activation operand of a wave whose first token is m0: rows m0.. of a
// row-major [T][ld] matrix (element size EB) starting at column col.
template <bool I8, int MT>
__device__ __forceinline__ APlain<I8, MT> rows_from(const void* base, int64_t ld, int m0, int T) {
  constexpr int EB = Stage<I8>::EB;
  const int rows = m0 < T ? T - m0 : 0;
  const uint8_t* b = static_cast<const uint8_t*>(base) + int64_t(m0 < T ? m0 : 0) * ld * EB;
  return APlain<I8, MT>{make_rsrc(b, int64_t(rows) * ld * EB), uint32_t(ld * EB), rows, int(ld)};
}

// Fragment-packed activations from the 16-row tile holding row m0 (a
// multiple of 16) on; `tile` bytes per tile, `tiles` tiles in the buffer.
template <bool I8, int MT>
__device__ __forceinline__ APacked<I8, MT> tiles_from(const void* base, int64_t tile, int64_t tiles,
                                                      int m0) {
  const int64_t t0 = m0 / 16;
  return APacked<I8, MT>{make_rsrc(static_cast<const uint8_t*>(base) + (t0 < tiles ? t0 : 0) * tile,
                                   (tiles - t0) * tile),
                         uint32_t(tile)};
}

// Block-cooperative tile product for large token counts.  The block's WM*MT
// activation tiles and its WN*NWW weight windows (consecutive in the packed
// buffer, `wstride` bytes apart, the first at wbase, nwin of them valid) of
// each k-stage are copied, 1 KB per wave load, into a two-buffer LDS ring;
// every wave then reads its fragments with conflict-free 16-byte LDS reads.
// The global loads run two groups of KPB stages ahead of the MFMAs through
// two register sets.  ns must be the same for the whole block.
// SH: weight loads carry the streaming hint; set where each weight byte is
// read once per step (few token tiles), left off where token tiles re-read
// the weights and want them kept in the caches
template <bool I8, int MT, int NWW, int WM, int WN, class AP, int KPB = 1, bool SH = false, bool F16 = false>
__device__ __forceinline__ void tile_mma_lds(const AP& ap, rsrc_t Wp, uint32_t wbase, uint32_t wstride,
                                             int nwin, int s0, int ns, uint8_t* lds,
                                             typename Stage<I8>::Acc (&acc)[MT][NWW * 4]) {
  using S = Stage<I8>;
  // chunks of a stage: AT activation tiles, then BC weight chunks; wave w
  // takes activation tiles w, w + NW, ... and weight chunks w, w + NW, ...
  constexpr int NW = WM * WN, AT = MT * WM, BC = NWW * WN * 4;
  constexpr int CA = (AT + NW - 1) / NW, CB = (BC + NW - 1) / NW, CH = CA + CB;
  constexpr int BUF = (AT + BC) * 1024;   // one k-stage; a ring slot holds KPB of them
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % WM, wn = w / WM;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NWW * 4; ++j) acc[mt][j] = typename S::Acc{0, 0, 0, 0};
  using Regs = uint4[KPB][CH];
  // group g = stages s0 + g*KPB .. s0 + g*KPB + KPB - 1
  auto gload = [&](Regs& r, int g) {
#pragma unroll
    for (int kk = 0; kk < KPB; ++kk) {
      const int j = g * KPB + kk;
      const bool ok = j < ns;
      const int st = s0 + j;
#pragma unroll
      for (int q = 0; q < CA; ++q) {
        const int c = w + q * NW;
        r[kk][q] = ap.load1(c < AT ? c : 0, st, ok && c < AT);
      }
#pragma unroll
      for (int q = 0; q < CB; ++q) {
        const int b = w + q * NW, v = b >> 2;
        const uint32_t off = ok && b < BC && v < nwin ? wbase + uint32_t(v) * wstride + uint32_t(st) * 4096u +
                                                            uint32_t((b & 3) * 1024 + lane * 16)
                                                      : kOOB;
        r[kk][CA + q] = SH ? bload16s(Wp, off) : bload16(Wp, off);
      }
    }
  };
  auto lwrite = [&](const Regs& r, int slot) {
#pragma unroll
    for (int kk = 0; kk < KPB; ++kk) {
      uint8_t* L = lds + (slot * KPB + kk) * BUF;
#pragma unroll
      for (int q = 0; q < CA; ++q)
        if (w + q * NW < AT) *reinterpret_cast<uint4*>(L + (w + q * NW) * 1024 + lane * 16) = r[kk][q];
#pragma unroll
      for (int q = 0; q < CB; ++q)
        if (w + q * NW < BC)
          *reinterpret_cast<uint4*>(L + (AT + w + q * NW) * 1024 + lane * 16) = r[kk][CA + q];
    }
  };
  // all of a stage's fragment reads are issued before its MFMAs, so the
  // LDS latency is paid once per stage rather than once per token tile
  auto compute = [&](int slot) {
#pragma unroll
    for (int kk = 0; kk < KPB; ++kk) {
      const uint8_t* L = lds + (slot * KPB + kk) * BUF;
      typename S::Frag bf[NWW * 4], af[MT];
#pragma unroll
      for (int j = 0; j < NWW * 4; ++j)
        bf[j] = *reinterpret_cast<const typename S::Frag*>(L + (AT + wn * NWW * 4 + j) * 1024 + lane * 16);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        af[mt] = *reinterpret_cast<const typename S::Frag*>(L + (wm * MT + mt) * 1024 + lane * 16);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NWW * 4; ++j) acc[mt][j] = mma16<F16>(bf[j], af[mt], acc[mt][j]);
    }
  };
  const int ngr = (ns + KPB - 1) / KPB;
  // groups past ngr load as zeros, so an odd count costs one zero group but
  // keeps the loop free of an exit between its two halves
  Regs R0, R1;   // group k waits in R(k % 2)
  gload(R0, 0);
  __builtin_amdgcn_sched_barrier(0);
  gload(R1, 1);
  __builtin_amdgcn_sched_barrier(0);
  lwrite(R0, 0);
  gload(R0, 2);
  __syncthreads();
  for (int j = 0; j < ngr; j += 2) {
    compute(0);                      // group j
    __builtin_amdgcn_sched_barrier(0);
    lwrite(R1, 1);                   // group j + 1
    gload(R1, j + 3);
    __syncthreads();
    compute(1);                      // group j + 1
    __builtin_amdgcn_sched_barrier(0);
    lwrite(R0, 0);                   // group j + 2
    gload(R0, j + 4);
    __syncthreads();
  }
}

// K1t: grid (token tiles fastest, then window groups, then k splits).  Wave
// (wm, wn) takes tokens 16*MT*wm.. of the block's token tile and windows
// NWW*wn.. of its group of [W^DQ | W^DkvKr] windows; the split's stages go
// into fp32 (int32) partials, one 16-byte store per 4 columns.
// With nreal > 0 the grid is padded to a multiple of 8 and taken in XCD
// order: blocks go to the XCDs in turn (block b to XCD b % 8), so block b
// takes work item (b % 8) * (grid / 8) + b / 8, and the token tiles that
// read the same weights run on one XCD and share its L2.
template <bool I8, int MT, int NWW, int WM, int WN, int D, bool LC = false, int KPB = 1, bool SH = false>
__global__ __launch_bounds__(64 * WM * WN) void k1_tiled(Dims d, Ptrs p, PackGeo pg, int sps, int mtiles,
                                                      int ngrp, int nreal = 0) {
  using St = Stage<I8>;
  constexpr int BM = 16 * MT * WM, GW = NWW * WN;
  int bid = blockIdx.x;
  if (nreal > 0) {
    bid = int(blockIdx.x % 8) * int(gridDim.x / 8) + int(blockIdx.x / 8);
    if (bid >= nreal) return;
  }
  const int mtile = bid % mtiles, rest = bid / mtiles;
  const int grp = rest % ngrp, split = rest / ngrp;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % WM, wn = w / WM;
  const int m0 = mtile * BM + 16 * MT * wm;
  const int tiles = pg.win_dq + pg.win_kr;
  const int Nkr = d.Hckv + d.Dr, Ntot = d.Hcq + Nkr;
  uint32_t wb[NWW];
#pragma unroll
  for (int i = 0; i < NWW; ++i) {
    const int j = grp * GW + wn * NWW + i;
    wb[i] = j < tiles ? uint32_t(pg.off_dq + int64_t(j) * pg.nst_he * 4096) : kOOB;
  }
  const int s0 = split * sps;
  typename St::Acc acc[MT][NWW * 4];
  if constexpr (LC) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[2 * KPB * (MT * WM + NWW * WN * 4) * 1024];
    const int mb = mtile * BM, j0 = grp * GW;
    const int nsb = mb < d.T ? max(0, min(pg.nst_he, s0 + sps) - s0) : 0;
    tile_mma_lds<I8, MT, NWW, WM, WN, APlain<I8, MT * WM>, KPB, SH>(rows_from<I8, MT * WM>(p.x, d.He, mb, d.T),
                                      make_rsrc(p.packed, pg.total),
                                      uint32_t(pg.off_dq + int64_t(j0) * pg.nst_he * 4096),
                                      uint32_t(pg.nst_he * 4096), tiles - j0, s0, nsb, ring, acc);
  } else {
    const int ns = m0 < d.T ? max(0, min(pg.nst_he, s0 + sps) - s0) : 0;
    const auto ap = rows_from<I8, MT>(p.x, d.He, m0, d.T);
    tile_mma<I8, MT, NWW, D>(ap, make_rsrc(p.packed, pg.total), wb, s0, ns, acc);
  }
  if (m0 >= d.T) return;
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int i = 0; i < NWW; ++i) {
    const int j = grp * GW + wn * NWW + i;
    if (j >= tiles) break;
    const int width = j < pg.win_dq ? min(64, d.Hcq - 64 * j) : min(64, Nkr - 64 * (j - pg.win_dq));
    const int outc = j < pg.win_dq ? 64 * j : d.Hcq + 64 * (j - pg.win_dq);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + 16 * mt + c;
      if (m >= d.T) continue;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int col = 16 * ct + 4 * g;
        if (col >= width) continue;
        const auto& a = acc[mt][i * 4 + ct];
        const uint4 v = make_uint4(__builtin_bit_cast(uint32_t, a[0] + 0), __builtin_bit_cast(uint32_t, a[1] + 0),
                                   __builtin_bit_cast(uint32_t, a[2] + 0), __builtin_bit_cast(uint32_t, a[3] + 0));
        *reinterpret_cast<uint4*>(static_cast<uint32_t*>(p.part) + (int64_t(split) * d.T + m) * Ntot +
                                  outc + col) = v;
      }
    }
  }
}

// K3t: grid (token tiles fastest, then groups of W^UqQr windows).  Nope
// windows go to q^C (bf16, workspace); a rope window goes through a per-wave
// LDS tile of 16 tokens x 64 columns to RoPE and queryRopeOut.
template <bool I8, int MT, int NWW, int WM, int WN, int D, bool LC = false, int KPB = 1, bool SH = false,
          bool F16 = false>
__global__ __launch_bounds__(64 * WM * WN) void k3_tiled(Dims d, Ptrs p, PackGeo pg, int mtiles) {
  using St = Stage<I8>;
  constexpr int BM = 16 * MT * WM, GW = NWW * WN;
  // per-wave RoPE tiles; with the LDS-staged core they reuse its ring,
  // which is idle once the main loop has ended with a barrier
  constexpr int ERING = 2 * KPB * (MT * WM + NWW * WN * 4) * 1024;
  constexpr int EBYTES = WM * WN * 16 * 65 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds_k3[LC && ERING > EBYTES ? ERING : EBYTES];
  const int mtile = blockIdx.x % mtiles, grp = blockIdx.x / mtiles;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % WM, wn = w / WM;
  const int m0 = mtile * BM + 16 * MT * wm;
  uint32_t wb[NWW];
#pragma unroll
  for (int i = 0; i < NWW; ++i) {
    const int j = grp * GW + wn * NWW + i;
    wb[i] = j < pg.win_uq ? uint32_t(pg.off_uq + int64_t(j) * pg.nst_cq * 4096) : kOOB;
  }
  typename St::Acc acc[MT][NWW * 4];
  if constexpr (LC) {
    uint8_t* ring = lds_k3;
    const int mb = mtile * BM, j0 = grp * GW;
    tile_mma_lds<I8, MT, NWW, WM, WN, APacked<I8, MT * WM>, KPB, SH>(
        tiles_from<I8, MT * WM>(p.cq, int64_t(pg.nst_cq) * 1024, (d.T + 15) / 16, mb),
        make_rsrc(p.packed, pg.total), uint32_t(pg.off_uq + int64_t(j0) * pg.nst_cq * 4096),
        uint32_t(pg.nst_cq * 4096), pg.win_uq - j0, 0, mb < d.T ? pg.nst_cq : 0, ring, acc);
  } else {
    const int ns = m0 < d.T ? pg.nst_cq : 0;
    const auto ap = tiles_from<I8, MT>(p.cq, int64_t(pg.nst_cq) * 1024, (d.T + 15) / 16, m0);
    tile_mma<I8, MT, NWW, D>(ap, make_rsrc(p.packed, pg.total), wb, 0, ns, acc);
  }
  if (m0 >= d.T) return;
  const int g = lane >> 4, c = lane & 15;
  const int P = pg.nope_w + 1, hf = d.Dr / 2;
  float* e = reinterpret_cast<float*>(lds_k3) + w * 16 * 65;
#pragma unroll
  for (int i = 0; i < NWW; ++i) {
    const int j = grp * GW + wn * NWW + i;
    if (j >= pg.win_uq) break;
    const int h = j / P, part = j % P;
    const bool rope = part == pg.nope_w;
    const int col0 = h * (d.D + d.Dr) + (rope ? d.D : 64 * part);
    const int width = rope ? d.Dr : min(64, d.D - 64 * part);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + 16 * mt + c;
      float v[4][4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int col = 16 * ct + 4 * g + r;
          if constexpr (I8)
            v[ct][r] = (m < d.T && col < width)
                           ? udq(p, acc[mt][i * 4 + ct][r], m, col0 + col)
                           : 0.0f;
          else
            v[ct][r] = acc[mt][i * 4 + ct][r];
        }
      if (!rope) {
        // q^C goes out fragment-packed for the W^UK product, its k padding
        // as zeros (the padded weight columns give exact zeros)
        if (m < d.T) {
          const int wq = min(64, 32 * pg.nst_d - 64 * part);
          const int64_t qtile = int64_t(d.N) * pg.nst_d * 1024;
          uint8_t* qcb = reinterpret_cast<uint8_t*>(p.qc) + int64_t(h) * pg.nst_d * 1024;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const int col = 16 * ct + 4 * g;
            if (col < wq)
              *reinterpret_cast<uint2*>(qcb + packed_offset(m, 64 * part + col, qtile, false)) =
                  pack16x4<F16>(v[ct][0], v[ct][1], v[ct][2], v[ct][3]);
          }
        }
      } else {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) e[c * 65 + 16 * ct + 4 * g + r] = v[ct][r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // lane: token c, pair groups of 4 starting at 4*g, stepping by 16
        const int64_t mrow = int64_t(m0 + 16 * mt + c);
        if (mrow < d.T) {
          const uint16_t* cs = p.cos + mrow * d.Dr;
          const uint16_t* sn = p.sin + mrow * d.Dr;
          uint16_t* o = p.qr_out + (mrow * d.N + h) * d.qrs;
          for (int i0 = 4 * g; i0 < hf; i0 += 16) {
            float lo[4], hi[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int ii = i0 + r;
              const float a = e[c * 65 + ii], b = e[c * 65 + ii + hf];
              lo[r] = a * ld16<F16>(cs[ii]) - b * ld16<F16>(sn[ii]);
              hi[r] = b * ld16<F16>(cs[ii + hf]) + a * ld16<F16>(sn[ii + hf]);
            }
            *reinterpret_cast<uint2*>(o + i0) = pack16x4<F16>(lo[0], lo[1], lo[2], lo[3]);
            *reinterpret_cast<uint2*>(o + i0 + hf) = pack16x4<F16>(hi[0], hi[1], hi[2], hi[3]);
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  }
}

// K4w: the W^UK product of long runs, q^N = q^C[., h, .] W^UK[h] in bf16 (or
// fp16).  ph blocks per head, heads fastest, so that the blocks running
// together write neighbouring heads of the same token rows; block (h, j)
// takes the 512-token tiles j, j + ph, ...  The head's whole W^UK (at most
// 8 windows x 4 D stages x 4 KB = 128 KB) is loaded into LDS once.  Wave w
// holds the q^C fragments of its 64 tokens of a tile (every D stage,
// D <= 128) in registers, the next tile's loading while the current one is
// multiplied, and walks the windows with no block barrier; each 16-token x
// 64-column result goes out through the wave's LDS tile as 16-byte
// non-temporal stores of whole 128-byte row pieces.  q^C is read once, and
// the stores of one tile overlap the loads of the next.
constexpr int kRowsTile = 512;   // K4w: tokens of a tile (8 waves x 64)

template <bool F16>
__global__ __launch_bounds__(512) void k4_rows(Dims d, Ptrs p, PackGeo pg, int ph) {
  constexpr int MT = 4, NW = 8, NSD = 4, UKMAX = 8 * NSD * 4 * 1024;
  __shared__ __attribute__((aligned(16))) uint8_t wl[UKMAX];
  __shared__ __attribute__((aligned(16))) uint8_t stage[NW * 16 * 144];
  const int h = blockIdx.x % d.N, j0 = blockIdx.x / d.N;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int nst = pg.nst_d, nt = (d.T + 15) / 16, mtiles = (d.T + kRowsTile - 1) / kRowsTile;
  const int64_t qtile = int64_t(d.N) * nst * 1024;
  const rsrc_t Q = make_rsrc(p.qc, int64_t(nt) * qtile);
  const rsrc_t Wp = make_rsrc(p.packed, pg.total);
  const uint32_t wbytes = uint32_t(nst) * 4096u, ubytes = uint32_t(pg.uk_w) * wbytes;
  const uint32_t ukh = uint32_t(pg.off_uk + int64_t(h) * ubytes);
  // the wave's q^C fragments of tile j (zeros past the run)
  using AF = uint4[MT][NSD];
  auto aload = [&](AF& a, int j) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int st = 0; st < NSD; ++st) {
        const int tt = (j * NW + w) * MT + mt;
        a[mt][st] = bload16(Q, j < mtiles && tt < nt && st < nst
                                   ? uint32_t(tt * qtile + int64_t(h) * nst * 1024) + uint32_t(st) * 1024u +
                                         uint32_t(lane * 16)
                                   : kOOB);
      }
  };
  // the head's W^UK: 16 bytes at thread offsets 0, 8192, ... of its ubytes
  {
    uint4 r[UKMAX / 8192];
#pragma unroll
    for (int i = 0; i < UKMAX / 8192; ++i) {
      const uint32_t o = uint32_t(threadIdx.x) * 16u + 8192u * i;
      r[i] = bload16(Wp, o < ubytes ? ukh + o : kOOB);
    }
#pragma unroll
    for (int i = 0; i < UKMAX / 8192; ++i) {
      const uint32_t o = uint32_t(threadIdx.x) * 16u + 8192u * i;
      if (o < ubytes) *reinterpret_cast<uint4*>(wl + o) = r[i];
    }
  }
  AF a0, a1;
  aload(a0, j0);
  // orders LDS only (the q^C loads may still be in flight)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  using Frag = bf16x8;
  const int64_t qbytes = int64_t(d.T) * d.N * d.qs * 2;
  const int64_t rows_n = int64_t(d.N) * d.qs * 2;   // bytes from one token row to the next
  uint8_t* tile = stage + w * 16 * 144;
  auto work = [&](const AF& a, int j) {
    const int tt0 = (j * NW + w) * MT;
    for (int jw = 0; jw < pg.uk_w; ++jw) {
      const uint8_t* L = wl + jw * wbytes;
      f32x4 acc[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[mt][ct] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < NSD; ++st) {
        if (st >= nst) break;
        Frag bf[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) bf[ct] = *reinterpret_cast<const Frag*>(L + (st * 4 + ct) * 1024 + lane * 16);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            acc[mt][ct] = mma16<F16>(bf[ct], __builtin_bit_cast(Frag, a[mt][st]), acc[mt][ct]);
      }
      // each 16-token x 64-column piece through the wave's LDS tile, out as
      // 16-byte non-temporal buffer stores (rows past T and columns past
      // Hckv at an out-of-range offset, which the hardware drops)
      const int width = min(64, d.Hckv - 64 * jw);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          *reinterpret_cast<uint2*>(tile + c * 144 + (16 * ct + 4 * g) * 2) =
              pack16x4<F16>(acc[mt][ct][0], acc[mt][ct][1], acc[mt][ct][2], acc[mt][ct][3]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int m0 = 16 * (tt0 + mt);
        const int64_t base = m0 < d.T ? (int64_t(m0) * d.N + h) * d.qs * 2 : qbytes;
        const rsrc_t O = make_rsrc(reinterpret_cast<uint8_t*>(p.q_out) + base, qbytes - base);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int k = lane + 64 * hh, row = k >> 3, col = 8 * (k & 7);
          const uint32_t off = m0 + row < d.T && col < width ? uint32_t(row * rows_n + (64 * jw + col) * 2) : kOOB;
          __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const i32x4*>(tile + row * 144 + col * 2), O,
                                                 off, 0, 2);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  };
  // two tiles a round, each loading while the other is multiplied
  for (int j = j0; j < mtiles; j += 2 * ph) {
    aload(a1, j + ph);
    work(a0, j);
    aload(a0, j + 2 * ph);
    if (j + ph < mtiles) work(a1, j + ph);
  }
}

// K4w with the int8 query: q^N = q^C[., h, .] W^UK[h] quantised per
// (token, head) with scale RowMax(|q^N|)/127 (the same fp32 accumulation
// order per element as K4t's int8 epilogue).  ph blocks per head, heads
// fastest; block (h, j) takes the 128-token tiles j, j + ph, ...  The head's
// whole W^UK is loaded into LDS once.  Wave w takes 16 tokens of a tile and
// every window, so the whole 512-column row of its tokens is in its
// registers (32 accumulators) and the row maximum needs no other wave; the
// next tile's q^C fragments load while the current tile is multiplied.
constexpr int kRowsQ8Tile = 128;   // tokens of a tile (8 waves x 16)

__global__ __launch_bounds__(512) void k4_rows_q8(Dims d, Ptrs p, PackGeo pg, int ph) {
  constexpr int NW = 8, NSD = 4, NWIN = 8, UKMAX = NWIN * NSD * 4 * 1024;
  constexpr int TP = 80;   // the code tile's row pitch (bytes): 16 tokens x 64 codes
  __shared__ __attribute__((aligned(16))) uint8_t wl[UKMAX];
  __shared__ __attribute__((aligned(16))) uint8_t ctile[NW * 16 * TP];
  const int h = blockIdx.x % d.N, j0 = blockIdx.x / d.N;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int nst = pg.nst_d, nt = (d.T + 15) / 16, mtiles = (d.T + kRowsQ8Tile - 1) / kRowsQ8Tile;
  const int64_t qtile = int64_t(d.N) * nst * 1024;
  const rsrc_t Q = make_rsrc(p.qc, int64_t(nt) * qtile);
  const rsrc_t Wp = make_rsrc(p.packed, pg.total);
  const uint32_t wbytes = uint32_t(nst) * 4096u, ubytes = uint32_t(pg.uk_w) * wbytes;
  const uint32_t ukh = uint32_t(pg.off_uk + int64_t(h) * ubytes);
  // the wave's q^C fragments of tile j (zeros past the run)
  using AF = uint4[NSD];
  auto aload = [&](AF& a, int j) {
    const int tt = j * NW + w;
#pragma unroll
    for (int st = 0; st < NSD; ++st)
      a[st] = bload16(Q, j < mtiles && tt < nt && st < nst
                             ? uint32_t(tt * qtile + int64_t(h) * nst * 1024) + uint32_t(st) * 1024u +
                                   uint32_t(lane * 16)
                             : kOOB);
  };
  // the head's W^UK in LDS at 16 KB per window (4 D stages of 4 KB), the
  // stages past nst and the windows past uk_w as zeros, so that the product
  // below runs over 8 windows x 4 D stages with no branch
  {
    uint4 r[UKMAX / 8192];
#pragma unroll
    for (int i = 0; i < UKMAX / 8192; ++i) {
      const uint32_t o = uint32_t(threadIdx.x) * 16u + 8192u * i;   // LDS byte
      const uint32_t jw = o / (NSD * 4096u), rem = o % (NSD * 4096u);
      r[i] = bload16(Wp, int(jw) < pg.uk_w && rem < wbytes ? ukh + jw * wbytes + rem : kOOB);
    }
#pragma unroll
    for (int i = 0; i < UKMAX / 8192; ++i)
      *reinterpret_cast<uint4*>(wl + uint32_t(threadIdx.x) * 16u + 8192u * i) = r[i];
  }
  AF a0, a1;
  aload(a0, j0);
  // orders LDS only (the q^C loads may still be in flight)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  int8_t* const qo = static_cast<int8_t*>(p.q_out);
  auto work = [&](const AF& a, int j) {
    f32x4 acc[NWIN * 4];
#pragma unroll
    for (int i = 0; i < NWIN * 4; ++i) acc[i] = f32x4{0, 0, 0, 0};
    // step k = (window, D stage, column tile); its W^UK fragment is read RA
    // steps ahead into a ring
    constexpr int NSTEP = NWIN * NSD * 4, RA = 8;
    auto frag = [&](int k) {
      const int jw = k / 16, st = (k / 4) % 4, ct = k % 4;
      return *reinterpret_cast<const bf16x8*>(wl + jw * NSD * 4096 + (st * 4 + ct) * 1024 + lane * 16);
    };
    bf16x8 ring[RA];
#pragma unroll
    for (int k = 0; k < RA; ++k) ring[k] = frag(k);
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
      const int jw = k / 16, st = (k / 4) % 4, ct = k % 4;
      acc[jw * 4 + ct] = mfma(ring[k % RA], __builtin_bit_cast(bf16x8, a[st]), acc[jw * 4 + ct]);
      if (k + RA < NSTEP) ring[k % RA] = frag(k + RA);
    }
    // the row maximum of |q^N| over the valid columns: lane (c, g) holds
    // token c, columns 16 ct + 4 g + r of each window
    float mx = 0.0f;
#pragma unroll
    for (int jw = 0; jw < NWIN; ++jw)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (jw < pg.uk_w && 64 * jw + 16 * ct + 4 * g < d.Hckv)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(acc[jw * 4 + ct][r]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const int m = 16 * (j * NW + w) + c;
    const float sc = mx / 127.0f;
    // each window's 16 x 64 codes through the wave's LDS tile, out as
    // 16-byte stores of whole 64-byte row pieces (lane: token l/4, piece l%4)
    uint8_t* const tl = ctile + w * 16 * TP;
    const int mr = 16 * (j * NW + w) + (lane >> 2), pc = 16 * (lane & 3);
#pragma unroll
    for (int jw = 0; jw < NWIN; ++jw) {
      if (jw >= pg.uk_w) break;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        uint32_t q = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          q |= uint32_t(uint8_t(sc > 0.0f ? quant_code(acc[jw * 4 + ct][r], sc) : int8_t(0))) << (8 * r);
        *reinterpret_cast<uint32_t*>(tl + c * TP + 16 * ct + 4 * g) = q;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint4 v = *reinterpret_cast<const uint4*>(tl + (lane >> 2) * TP + pc);
      if (j < mtiles && mr < d.T && 64 * jw + pc < d.Hckv)
        *reinterpret_cast<uint4*>(qo + (int64_t(mr) * d.N + h) * d.qs + 64 * jw + pc) = v;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (g == 0 && j < mtiles && m < d.T) p.q_scale[int64_t(m) * d.N + h] = sc;
  };
  // two tiles a round, each loading while the other is multiplied
  for (int j = j0; j < mtiles; j += 2 * ph) {
    aload(a1, j + ph);
    work(a0, j);
    aload(a0, j + 2 * ph);
    if (j + ph < mtiles) work(a1, j + ph);
  }
}

// K4t: grid (token tiles fastest, then column groups, then heads).  q^N =
// q^C[., h, .] W^UK[h]; bf16 stores, or (one column group holding the whole
// Hckv row) the per-(token, head) int8 quantisation with the row maximum
// taken across the WN waves of a token range.
// HF: heads vary fastest along the grid, so blocks running together write
// neighbouring heads of the same tokens (one contiguous q^N row per token).
// K3r: the medium-T up-projection (up to 16*8*MT tokens) for heads of two
// nope windows and Dr = 64, one block per (head, half) as in k34_pair: the
// block's 96 weight columns are nope window `half` and rope column tiles
// half and half + 2, whose RoPE pairs (i, i + Dr/2) are then all in the
// block.  Every weight byte is read from HBM once.  Wave w owns the token
// tiles w, w + 8, ... and all 96 columns.
//
// The k-stages stream through a register ring R entries deep; entry i holds
// an eighth of the weights of stage i + 2 (each wave loads 768 bytes) and
// the wave's own activation tiles of stage i (fragment-packed c^Q, 1 KB per
// 16 tokens), so every load of an entry is issued together and used at the
// same step, and a wave's in-order load completion never holds a later
// stage behind an earlier one.  The weights pass through three LDS slots:
// at step i a wave writes its piece of stage i + 2, reads the six weight
// fragments of stage i + 1 ahead, runs the MFMAs of stage i (weights read at
// the previous step, activations from the ring), refills the entry with
// stage i + R, and meets the block at one barrier.  The fragment reads of
// one stage so overlap the MFMAs of the one before.
//
// Epilogue: rope columns -> RoPE -> queryRopeOut; nope columns -> q^C (bf16;
// with int8 operands each value is first dequantised, udq).  Without UK, q^C
// goes to the workspace, fragment-packed for the W^UK kernel.  With UK (the
// W^UK product in the same launch, as in k34_pair): the block's half of the
// W^UK columns (the windows of its half of Hckv, at most 64 KB) is loaded
// into registers during the stream and parked in LDS; each block writes its
// q^C half to the workspace with agent-scope stores and to LDS, raises its
// flag (the run's number), waits for the partner's, and multiplies both
// halves with the parked W^UK fragments: q^N for its tokens and columns, in
// bf16, or in int8 with the per-(token, head) row maxima traded through the
// workspace and a second flag.
constexpr int kRingMaxT = 256;   // K3r: tokens a block holds at most (8 waves x 2 tiles of 16)

template <bool I8, int MT, int R, int NSTMAX, bool UK, bool Q8>
__global__ __launch_bounds__(512) void k3_ring(Dims d, Ptrs p, PackGeo pg) {
  using St = Stage<I8>;
  using Acc = typename St::Acc;
  using Frag = typename St::Frag;
  constexpr int NW = 8, NTM = NW * MT;
  constexpr int WB = 6 * 1024;                    // weight bytes of a stage
  constexpr int UKB = UK ? 64 * 1024 : 0;         // parked W^UK: 4 windows x 4 stages x 4 KB
  constexpr int QCB = UK ? NTM * 2048 : 0;        // own q^C half: 2 D-stages per token tile
  __shared__ __attribute__((aligned(16))) uint8_t lds[3 * WB + UKB + QCB];
  // int8 operands: the dequantisation scale (and static bias) of each of the
  // block's 96 columns, loaded once at the start
  __shared__ float swl[I8 ? 96 : 1];
  __shared__ int32_t bsl[I8 ? 96 : 1];
  uint8_t* const ukl = lds + 3 * WB;
  uint8_t* const qcl = lds + 3 * WB + UKB;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int b = blockIdx.x;
  // a head's two blocks are 8 apart, so they run on the same XCD
  const int h = d.N % 8 == 0 ? (b / 16) * 8 + b % 8 : b / 2;
  const int half = d.N % 8 == 0 ? (b / 8) % 2 : b % 2;
  const int P = pg.nope_w, DDr = d.D + d.Dr, nst = pg.nst_cq;
  const int nt = (d.T + 15) / 16;
  const rsrc_t Wp = make_rsrc(p.packed, pg.total);
  const int64_t ctile = int64_t(nst) * 1024;
  const rsrc_t Cq = make_rsrc(p.cq, int64_t(nt) * ctile);
  const uint32_t nb = uint32_t(pg.off_uq + int64_t(h * (P + 1) + half) * nst * 4096);
  const uint32_t rb = uint32_t(pg.off_uq + int64_t(h * (P + 1) + P) * nst * 4096);
  // A stage's 6 KB of weights, in LDS order: the nope window's 4 KB, then
  // rope tiles half and half + 2.  Wave w loads bytes 768 w .. 768 w + 767
  // (lanes 0..47), one 16-byte piece per lane, each within one tile.
  const int wbyte = 768 * w + 16 * lane;
  const bool wl = lane < 48;
  const uint32_t wseg = wbyte < 4096   ? nb + uint32_t(wbyte)
                        : wbyte < 5120 ? rb + uint32_t(half * 1024 + wbyte - 4096)
                                       : rb + uint32_t((half + 2) * 1024 + wbyte - 5120);
  auto wload = [&](int st) { return bload16s(Wp, st < nst && wl ? wseg + uint32_t(st) * 4096u : kOOB); };
  auto aload = [&](int st, int m) {
    return bload16(Cq, st < nst && w + NW * m < nt
                           ? uint32_t((w + NW * m) * ctile) + uint32_t(st) * 1024u + uint32_t(lane * 16)
                           : kOOB);
  };
  auto lwrite = [&](int st, const uint4& v) {
    if (wl) *reinterpret_cast<uint4*>(lds + (st % 3) * WB + wbyte) = v;
  };
  auto lread = [&](int st, Frag (&f)[6]) {
#pragma unroll
    for (int j = 0; j < 6; ++j) f[j] = *reinterpret_cast<const Frag*>(lds + (st % 3) * WB + j * 1024 + lane * 16);
  };
  auto barrier = [] {
    // orders LDS only: the loads in flight are not waited for
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  // this half's W^UK windows jlo .. jhi-1 (at most four), in LDS as chunk
  // (window - jlo) * 16 + stage * 4 + column tile, 1 KB each; wave w loads
  // chunks w, w + 8, ..
  const int ja = (pg.uk_w + 1) / 2, jlo = half ? ja : 0, jhi = half ? pg.uk_w : ja;
  uint4 ukr[UK ? 8 : 1];
  auto ukload = [&] {
#pragma unroll
    for (int i = 0; i < (UK ? 8 : 0); ++i) {
      const int ch = w + NW * i, jj = ch >> 4, s = (ch >> 2) & 3, ct = ch & 3;
      const bool ok = jlo + jj < jhi && s < pg.nst_d;
      ukr[i] = bload16s(Wp, ok ? uint32_t(pg.off_uk + int64_t(h * pg.uk_w + jlo + jj) * pg.nst_d * 4096) +
                                     uint32_t(s * 4096 + ct * 1024 + lane * 16)
                               : kOOB);
    }
  };
  // block column k: k < 64 nope column 64 half + k; 64..79 rope column
  // 16 half + k - 64; 80..95 rope column Dr/2 + 16 half + k - 80
  auto wcol = [&](int k) {
    return h * DDr + (k < 64 ? 64 * half + k : d.D + (k < 80 ? 16 * half + k - 64 : d.Dr / 2 + 16 * half + k - 80));
  };
  // (loaded before the stream starts, stored to LDS once the first loads
  // of the stream are out)
  float swv = 0.0f;
  int32_t bsv = 0;
  if constexpr (I8) {
    const int k = threadIdx.x < 96 ? threadIdx.x : 0, n = wcol(k);
    const bool ok = threadIdx.x < 96 && (k >= 64 || 64 * half + k < d.D);
    const rsrc_t Sw = make_rsrc(p.sw_uq_qr, int64_t(d.N) * DDr * 4);
    const rsrc_t Bs = make_rsrc(p.bias_uq, p.bias_uq ? int64_t(d.N) * DDr * 4 : 0);
    swv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(Sw, ok ? uint32_t(n) * 4u : kOOB, 0, 0));
    bsv = __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(Bs, ok ? uint32_t(n) * 4u : kOOB, 0, 0));
  }
  // stages 0 and 1 of the weights go to LDS first; then entries 0 .. R-1,
  // then the W^UK fragments (used only after the stream)
  uint4 rw[R], ra[R][MT];
  {
    const uint4 w0 = wload(0), w1 = wload(1);
    lwrite(0, w0);
    lwrite(1, w1);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < R; ++q) {
    rw[q] = wload(q + 2);
#pragma unroll
    for (int m = 0; m < MT; ++m) ra[q][m] = aload(q, m);
  }
  ukload();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (I8) {
    if (threadIdx.x < 96) {
      swl[threadIdx.x] = swv;
      bsl[threadIdx.x] = bsv;
    }
  }
  barrier();
  // the epilogue's per-token values (the lane's cos/sin pieces and c^Q's
  // scale), loaded R stages before the stream ends: every later wait of the
  // ring is for a load issued before them, so they cost the stream nothing,
  // and they are in before q^C is traded
  const int hf = d.Dr / 2, i0 = 16 * half + 4 * g;
  uint2 cs[MT][4];
  float csc[MT];
  auto epi_load = [&] {
    const rsrc_t Cs = make_rsrc(p.cos, int64_t(d.T) * d.Dr * 2), Sn = make_rsrc(p.sin, int64_t(d.T) * d.Dr * 2);
    const rsrc_t Sc = make_rsrc(p.cq_scale, I8 ? int64_t(d.T) * 4 : 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int t = 16 * (w + NW * mt) + c;
      const uint32_t ro = t < d.T ? uint32_t(t * d.Dr + i0) * 2u : kOOB;
      cs[mt][0] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(Cs, ro, 0, 0));
      cs[mt][1] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(Cs, ro == kOOB ? kOOB : ro + hf * 2, 0, 0));
      cs[mt][2] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(Sn, ro, 0, 0));
      cs[mt][3] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(Sn, ro == kOOB ? kOOB : ro + hf * 2, 0, 0));
      csc[mt] = I8 ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(Sc, t < d.T ? uint32_t(t) * 4u : kOOB, 0, 0))
                   : 1.0f;
    }
  };
  Frag bf[6], bfn[6];
  lread(0, bf);
  Acc acc[MT][6];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 6; ++j) acc[mt][j] = Acc{0, 0, 0, 0};
  // all NSTMAX stages, unrolled, with no exit: stages past nst load zeros
  // (an exact no-op).  At a loop head the wait counts of the ring's
  // registers would merge and the ring drain once a round; an early exit
  // lets the compiler sink each load to its use, which drains it at every
  // stage.
#pragma unroll
  for (int st = 0; st < NSTMAX; ++st) {
    const int q = st % R;
    lwrite(st + 2, rw[q]);
    if (st + 1 < NSTMAX) lread(st + 1, bfn);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const Frag af = __builtin_bit_cast(Frag, ra[q][mt]);
#pragma unroll
      for (int j = 0; j < 6; ++j) acc[mt][j] = mfma(bf[j], af, acc[mt][j]);
    }
    __builtin_amdgcn_sched_barrier(0);
    rw[q] = wload(st + 2 + R);
#pragma unroll
    for (int m = 0; m < MT; ++m) ra[q][m] = aload(st + R, m);
    if (st == (NSTMAX > R ? NSTMAX - R : 0)) epi_load();
    barrier();
#pragma unroll
    for (int j = 0; j < 6; ++j) bf[j] = bfn[j];
  }
  if constexpr (UK) {
    // park the W^UK fragments
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(ukl + (w + NW * i) * 1024 + lane * 16) = ukr[i];
  }
  // u of block column k from its accumulator: (acc + bias) s_cq s_w in fp32,
  // as udq
  auto dq = [&](auto a, int mt, int k) -> float {
    if constexpr (I8) return static_cast<float>(a + bsl[k]) * csc[mt] * swl[k];
    else return a;
  };

  // lane: token 16 (w + 8 mt) + c, columns 16 j + 4 g + r of the block's
  // tiles (j < 4: nope window `half`; j = 4, 5: rope tiles half, half + 2)
  const int64_t qtile = int64_t(d.N) * pg.nst_d * 1024;
  uint8_t* const qcb = reinterpret_cast<uint8_t*>(p.qc) + int64_t(h) * pg.nst_d * 1024;
  const int wq = min(64, 32 * pg.nst_d - 64 * half);   // q^C columns of this window, with the k padding
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int tt = w + NW * mt, t = 16 * tt + c;
    // q^C (for a token past T: zeros into the LDS copy only)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = 16 * j + 4 * g;   // in the window
      if (col >= wq) continue;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = t < d.T ? dq(acc[mt][j][r], mt, col + r) : 0.0f;
      const uint2 pk = pack_bf16x4(v[0], v[1], v[2], v[3]);
      if constexpr (UK) {
        // fragment order of the W^UK product's activation operand: stage
        // 2 half + j / 2, lane group 2 (j % 2) + g / 2, token c
        const int fo = (16 * (2 * (j % 2) + g / 2) + c) * 16 + 8 * (g % 2);
        *reinterpret_cast<uint2*>(qcl + (tt * 2 + j / 2) * 1024 + fo) = pk;
        if (t < d.T) xstore64(qcb + int64_t(tt) * qtile + (2 * half + j / 2) * 1024 + fo, pk);
      } else {
        if (t < d.T) *reinterpret_cast<uint2*>(qcb + packed_offset(t, 64 * half + col, qtile, false)) = pk;
      }
    }
  }
  if constexpr (UK) pair_publish(p.xflag + 4 * h + half, d.run);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int t = 16 * (w + NW * mt) + c;
    if (t >= d.T) continue;
    // q^R: pairs (i0 + r, i0 + r + Dr/2)
    const uint16_t* cs0 = reinterpret_cast<const uint16_t*>(&cs[mt][0]);
    const uint16_t* cs1 = reinterpret_cast<const uint16_t*>(&cs[mt][1]);
    const uint16_t* sn0 = reinterpret_cast<const uint16_t*>(&cs[mt][2]);
    const uint16_t* sn1 = reinterpret_cast<const uint16_t*>(&cs[mt][3]);
    float o0[4], o1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a = dq(acc[mt][4][r], mt, 64 + 4 * g + r), bb = dq(acc[mt][5][r], mt, 80 + 4 * g + r);
      o0[r] = a * bf2f(cs0[r]) - bb * bf2f(sn0[r]);
      o1[r] = bb * bf2f(cs1[r]) + a * bf2f(sn1[r]);
    }
    uint16_t* o = p.qr_out + (int64_t(t) * d.N + h) * d.qrs + i0;
    *reinterpret_cast<uint2*>(o) = pack_bf16x4(o0[0], o0[1], o0[2], o0[3]);
    *reinterpret_cast<uint2*>(o + hf) = pack_bf16x4(o1[0], o1[1], o1[2], o1[3]);
  }
  if constexpr (UK) {
    // q^N = q^C W^UK[h] over this half's windows, all of D; the operand's
    // stages 2 half, 2 half + 1 are this block's (LDS), the others the
    // partner's (workspace)
    pair_wait(p.xflag + 4 * h + (1 - half), p.herr, d.run, d.spin);
    uint4 aq[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int tt = w + NW * mt;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s >= pg.nst_d) {
          aq[mt][s] = make_uint4(0, 0, 0, 0);
        } else if (s / 2 == half) {
          aq[mt][s] = *reinterpret_cast<const uint4*>(qcl + (tt * 2 + s % 2) * 1024 + lane * 16);
        } else {
          aq[mt][s] = tt < nt ? xload128(qcb + int64_t(tt) * qtile + s * 1024 + lane * 16) : make_uint4(0, 0, 0, 0);
        }
      }
    }
    constexpr int NCT = 16;   // column tiles of the half: 4 windows x 4 tiles
    f32x4 au[MT][Q8 ? NCT : 1];
    auto tile_mma = [&](int j, f32x4 (&o)[MT]) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 wf = *reinterpret_cast<const bf16x8*>(ukl + ((j >> 2) * 16 + s * 4 + (j & 3)) * 1024 + lane * 16);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[mt] = mfma(wf, __builtin_bit_cast(bf16x8, aq[mt][s]), o[mt]);
      }
    };
    if constexpr (!Q8) {
      // each 16-token x 64-column piece goes through the wave's tile in the
      // (idle) ring slots, rows 144 bytes apart, and leaves as 16-byte
      // non-temporal stores of whole 128-byte row pieces
      uint16_t* qo = static_cast<uint16_t*>(p.q_out);
      uint8_t* const tile = lds + w * 16 * 144;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (jlo + jj >= jhi) break;
        f32x4 o[4][MT];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) tile_mma(4 * jj + ct, o[ct]);
        const int width = min(64, d.Hckv - 64 * (jlo + jj));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            *reinterpret_cast<uint2*>(tile + c * 144 + (16 * ct + 4 * g) * 2) =
                pack_bf16x4(o[ct][mt][0], o[ct][mt][1], o[ct][mt][2], o[ct][mt][3]);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int k = lane + 64 * hh, row = k >> 3, col = 8 * (k & 7);
            const int t = 16 * (w + NW * mt) + row;
            if (t < d.T && col < width)
              __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(tile + row * 144 + col * 2),
                                          reinterpret_cast<u32x4*>(qo + (int64_t(t) * d.N + h) * d.qs +
                                                                   64 * (jlo + jj) + col));
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
      }
    } else {
      // per-token max |q^N| over this half's columns (a wave holds whole
      // token rows), traded with the partner
      float mx[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) mx[mt] = 0.0f;
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        f32x4 o[MT];
        tile_mma(j, o);
        const bool on = jlo + j / 4 < jhi && 64 * jlo + 16 * j + 4 * g < d.Hckv;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          au[mt][j] = o[mt];
          if (on)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx[mt] = fmaxf(mx[mt], fabsf(o[mt][r]));
        }
      }
      float* const xm = p.xmax2 + int64_t(h) * 2 * kRingMaxT;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        mx[mt] = fmaxf(mx[mt], __shfl_xor(mx[mt], 16, 64));
        mx[mt] = fmaxf(mx[mt], __shfl_xor(mx[mt], 32, 64));
        const int t = 16 * (w + NW * mt) + c;
        if (g == 0 && t < d.T)
          __hip_atomic_store(xm + half * kRingMaxT + t, mx[mt], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      pair_publish(p.xflag + 4 * h + 2 + half, d.run);
      pair_wait(p.xflag + 4 * h + 2 + (1 - half), p.herr, d.run, d.spin);
      int8_t* qo = static_cast<int8_t*>(p.q_out);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int t = 16 * (w + NW * mt) + c;
        if (t >= d.T) continue;
        const float amax =
            fmaxf(mx[mt], __hip_atomic_load(xm + (1 - half) * kRingMaxT + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        const float sc = amax / 127.0f;
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
          const int col = 64 * jlo + 16 * j + 4 * g;
          if (jlo + j / 4 >= jhi || col >= d.Hckv) continue;
          uint32_t u = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            u |= uint32_t(uint8_t(sc > 0.0f ? quant_code(au[mt][j][r], sc) : 0)) << (8 * r);
          *reinterpret_cast<uint32_t*>(qo + (int64_t(t) * d.N + h) * d.qs + col) = u;
        }
        if (half == 0 && g == 0) p.q_scale[int64_t(t) * d.N + h] = sc;
      }
    }
  }
}

template <int MT, int NWW, int WM, int WN, int D, bool Q8, bool LC = false, bool HF = false, bool F16 = false>
__global__ __launch_bounds__(64 * WM * WN) void k4_tiled(Dims d, Ptrs p, PackGeo pg, int mtiles,
                                                      int cgroups) {
  constexpr int BM = 16 * MT * WM, GW = NWW * WN;
  __shared__ float rmax[Q8 ? WN : 1][Q8 ? BM : 1];
  __shared__ __attribute__((aligned(16))) uint8_t stage[Q8 ? 16 : WM * WN * 16 * 144];
  int mtile, cg, h;
  if constexpr (HF) {
    h = blockIdx.x % d.N;
    const int rest = blockIdx.x / d.N;
    cg = rest % cgroups; mtile = rest / cgroups;
  } else {
    mtile = blockIdx.x % mtiles;
    const int rest = blockIdx.x / mtiles;
    cg = rest % cgroups; h = rest / cgroups;
  }
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % WM, wn = w / WM;
  const int m0 = mtile * BM + 16 * MT * wm;
  uint32_t wb[NWW];
#pragma unroll
  for (int i = 0; i < NWW; ++i) {
    const int jw = cg * GW + wn * NWW + i;
    wb[i] = jw < pg.uk_w ? uint32_t(pg.off_uk + int64_t(h * pg.uk_w + jw) * pg.nst_d * 4096) : kOOB;
  }
  const int64_t qtile = int64_t(d.N) * pg.nst_d * 1024, qh = int64_t(h) * pg.nst_d * 1024;
  typename Stage<false>::Acc acc[MT][NWW * 4];
  if constexpr (LC) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[2 * (MT * WM + NWW * WN * 4) * 1024];
    const int mb = mtile * BM, j0 = cg * GW;
    tile_mma_lds<false, MT, NWW, WM, WN, APacked<false, MT * WM>, 1, false, F16>(
        tiles_from<false, MT * WM>(reinterpret_cast<const uint8_t*>(p.qc) + qh, qtile, (d.T + 15) / 16, mb),
        make_rsrc(p.packed, pg.total), uint32_t(pg.off_uk + int64_t(h * pg.uk_w + j0) * pg.nst_d * 4096),
        uint32_t(pg.nst_d * 4096), pg.uk_w - j0, 0, mb < d.T ? pg.nst_d : 0, ring, acc);
  } else {
    const int ns = m0 < d.T ? pg.nst_d : 0;
    const auto ap = tiles_from<false, MT>(reinterpret_cast<const uint8_t*>(p.qc) + qh, qtile,
                                          (d.T + 15) / 16, m0);
    tile_mma<false, MT, NWW, D, decltype(ap), F16>(ap, make_rsrc(p.packed, pg.total), wb, 0, ns, acc);
  }
  const int g = lane >> 4, c = lane & 15;
  if constexpr (!Q8) {
    // each 16-token x 64-column piece goes through the wave's LDS tile
    // (rows 144 bytes apart, which spreads the 8-byte writes over the banks)
    // and out as 16-byte stores, eight whole 128-byte row pieces per store;
    // the stores are non-temporal (queryOut is written once and not read
    // back here, and the streaming hint keeps it from displacing the
    // operands in the caches)
    if (m0 >= d.T) return;
    uint16_t* qo = static_cast<uint16_t*>(p.q_out);
    uint8_t* tile = stage + w * 16 * 144;
#pragma unroll
    for (int i = 0; i < NWW; ++i) {
      const int jw = cg * GW + wn * NWW + i;
      if (jw >= pg.uk_w) break;
      const int width = min(64, d.Hckv - 64 * jw);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const auto& a = acc[mt][i * 4 + ct];
          *reinterpret_cast<uint2*>(tile + c * 144 + (16 * ct + 4 * g) * 2) = pack16x4<F16>(a[0], a[1], a[2], a[3]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int k = lane + 64 * half, row = k >> 3, col = 8 * (k & 7);
          const int m = m0 + 16 * mt + row;
          if (m < d.T && col < width)
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(tile + row * 144 + col * 2),
                                        reinterpret_cast<u32x4*>(qo + (int64_t(m) * d.N + h) * d.qs + 64 * jw + col));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < NWW; ++i) {
        const int width = min(64, d.Hckv - 64 * (wn * NWW + i));
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          if (16 * ct + 4 * g < width)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(acc[mt][i * 4 + ct][r]));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (g == 0) rmax[wn][16 * MT * wm + 16 * mt + c] = mx;
    }
    __syncthreads();
    if (m0 >= d.T) return;
    int8_t* qo = static_cast<int8_t*>(p.q_out);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + 16 * mt + c;
      if (m >= d.T) continue;
      float amax = rmax[0][16 * MT * wm + 16 * mt + c];
#pragma unroll
      for (int k = 1; k < WN; ++k) amax = fmaxf(amax, rmax[k][16 * MT * wm + 16 * mt + c]);
      const float sc = amax / 127.0f;
#pragma unroll
      for (int i = 0; i < NWW; ++i) {
        const int jw = wn * NWW + i;
        if (jw >= pg.uk_w) break;
        const int width = min(64, d.Hckv - 64 * jw);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int col = 16 * ct + 4 * g;
          if (col >= width) continue;
          const auto& a = acc[mt][i * 4 + ct];
          uint32_t q = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = a[r];
            const int8_t code = sc > 0.0f ? quant_code(x, sc) : int8_t(0);
            q |= uint32_t(uint8_t(code)) << (8 * r);
          }
          *reinterpret_cast<uint32_t*>(qo + (int64_t(m) * d.N + h) * d.qs + 64 * jw + col) = q;
        }
      }
      if (wn == 0 && g == 0) p.q_scale[int64_t(m) * d.N + h] = sc;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Token counts up to this run on the streaming kernels.
constexpr int kStreamMaxT = 32;

struct Plan {
  bool stream;       // T small enough for the packed kernels
  int mt1, S, kps;   // K1 rows per tile (16*mt1), split count, k per split
  int mt3;           // K3
  int ntw4, cs4;     // K4 column tiles per wave, column splits
};

int ceil_div(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

// int8 down-projection operands (x, W^DQ, W^DkvKr): full quantisation only;
// int8 W^UqQr (and an int8 c^Q): full and partial quantisation
bool is_static(const mla_prolog_desc& d) { return d.in_dtype == MLA_INT8_STATIC; }
bool down_i8(const mla_prolog_desc& d) { return d.in_dtype == MLA_INT8 || is_static(d); }
bool up_i8(const mla_prolog_desc& d) { return down_i8(d) || d.in_dtype == MLA_INT8_PARTIAL; }
PackGeo geo_of(const mla_prolog_desc& d) {
  return pack_geo(d.He, d.Hcq, d.Hckv, d.N, d.D, d.Dr, down_i8(d), up_i8(d));
}

int mt_for(int64_t T, int cap) {
  int mt = 1;
  while (mt < cap && 16 * mt < T) mt *= 2;
  return mt;
}

Plan make_plan(const mla_prolog_desc& d, int64_t T) {
  Plan pl;
  const bool i8 = down_i8(d);
  pl.stream = T <= kStreamMaxT;
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

// Tiled path (token counts above the streaming range, packed weights).
// Shape classes.  Large (T >= kTiledLargeT): K1 and K3 in LDS-staged
// 256-token x 256-column blocks of sixteen 64x64 waves (four per SIMD, which
// hides the LDS and barrier latency better than eight 128x64 waves), K1
// split in two along He; K4 likewise (bf16 query), heads fastest.  Medium: K1 with one 16*mt-token
// wave per 64-column window, He split so that about kTiledK1Blocks blocks
// run (above 128 tokens: LDS-staged 256 x 128 blocks, about one per CU);
// K3 with one 64-token wave per window up to 128 tokens, LDS-staged
// 256 x 128 blocks above; an int8 K1 or K3 switches to LDS-staged
// 128 x 128 blocks from 65 tokens on.  K4 with eight 64-column waves per
// 16*mt tokens.  The int8-query K4 always takes 64 tokens x the whole Hckv
// row per block.
constexpr int kTiledLargeT = 2048;
constexpr bool kRingK3 = true;
// K3r instances unroll 8, 24 or 48 k-stages of Hcq (the smallest that holds
// the shape's; 48 is Hcq 1536 in bf16, 24 Hcq 1536 in int8)
constexpr int kRingStages = 48;
constexpr int kTiledK1Blocks = 512;   // medium: one-wave blocks

// Medium token counts also take some of the large shapes' kernels, each
// from where it measured faster at the model shapes (bf16 and int8): the
// 256 x 256 up-projection above 256 tokens (past the ring kernel), the
// long-run W^UK kernels from kMixK4RowsT (bf16 query) or kMixK4RowsQ8T
// (int8 query) and the 256 x 256 down-projection from kMixK1LargeT tokens.
constexpr int kMixK4RowsT = 768;
constexpr int kMixK4RowsQ8T = 448;
constexpr int kMixK1LargeT = 1792;

struct TiledPlan {
  bool large;
  bool k1L, k3L, k4R;      // the large shapes' down-projection, up-projection, W^UK kernel (k4_rows)
  bool ring;               // medium up-projection on K3r (heads of two nope windows, Dr = 64, T <= 256)
  int mt;                  // medium: 16-token tiles per K4 wave (and per direct K1 wave)
  int k1v, k3v;            // medium kernel shapes: 0 direct, 1 LDS-staged 256-token, 2 128-token, 3 64-token
  int m1, ngrp1, S, sps;   // K1: token tiles, window groups, splits, stages per split
  int m3, ngrp3;           // K3
  int m4, cg4;             // K4 bf16
  int m4q;                 // K4 int8 query: token tiles of 64
};

TiledPlan tiled_plan(const mla_prolog_desc& d, int64_t T) {
  TiledPlan tp;
  const PackGeo g = geo_of(d);
  const int tiles = g.win_dq + g.win_kr;
  tp.large = T >= kTiledLargeT;
  tp.ring = !tp.large && T <= 256 && g.nope_w == 2 && d.Dr == 64 && g.nst_cq <= kRingStages &&
            d.float_dtype != MLA_FP16 && kRingK3;
  tp.mt = T <= 64 ? 4 : 8;
  // medium shapes: LDS-staged blocks above 128 tokens; for an int8 product
  // also from 65 tokens on, in 128-token blocks (the int8 k-stages are twice
  // as deep)
  // (224-256 tokens: two full 128-token tiles halve the splits, and so
  // the partials the norm kernel reads, for one more read of the weights
  // from the caches; int8 x at 65-128 tokens likewise in 64-token tiles)
  tp.k1v = (T >= 224 && T <= 256) ? 2 : T > 128 ? 1 : (down_i8(d) && T > 64) ? 3 : 0;
  tp.k3v = T > 128 ? 1 : (up_i8(d) && T > 64) ? 2 : 0;
  tp.k1L = tp.large || T >= kMixK1LargeT;
  tp.k3L = tp.large || (!tp.ring && T > 256);
  tp.k4R = g.nst_d <= 4 && g.uk_w <= 8 && (tp.large || T >= (d.query_dtype == MLA_INT8 ? kMixK4RowsQ8T : kMixK4RowsT));
  if (tp.large) {
    tp.m1 = ceil_div(T, 256); tp.ngrp1 = ceil_div(tiles, 4);      // LDS-staged 256 x 256
    tp.m3 = ceil_div(T, 256); tp.ngrp3 = ceil_div(g.win_uq, 4);
    tp.m4 = ceil_div(T, 256); tp.cg4 = ceil_div(g.uk_w, 4);      // LDS-staged 256 x 256
  } else {
    // LDS-staged block rows
    const int bm1 = tp.k1v == 1 ? 256 : tp.k1v == 3 ? 64 : 128, bm3 = tp.k3v == 1 ? 256 : 128;
    if (tp.k1L) { tp.m1 = ceil_div(T, 256); tp.ngrp1 = ceil_div(tiles, 4); }
    else if (tp.k1v) { tp.m1 = ceil_div(T, bm1); tp.ngrp1 = ceil_div(tiles, 2); }
    else { tp.m1 = ceil_div(T, 16 * tp.mt); tp.ngrp1 = tiles; }
    if (tp.k3L) { tp.m3 = ceil_div(T, 256); tp.ngrp3 = ceil_div(g.win_uq, 4); }
    else if (tp.k3v) { tp.m3 = ceil_div(T, bm3); tp.ngrp3 = ceil_div(g.win_uq, 2); }
    else { tp.m3 = ceil_div(T, 64); tp.ngrp3 = g.win_uq; }                            // 64-token waves
    tp.m4 = ceil_div(T, 16 * tp.mt); tp.cg4 = ceil_div(g.uk_w, 8);
  }
  // large: two k splits, so that the 1-block-per-CU grid fills whole rounds;
  // medium LDS-staged: about one block per CU
  const int target = tp.k1L ? 2 * tp.m1 * tp.ngrp1 : tp.k1v ? 256 : kTiledK1Blocks;
  int S = std::max(1, std::min(g.nst_he, target / std::max(1, tp.m1 * tp.ngrp1)));
  tp.sps = ceil_div(g.nst_he, S);
  tp.S = ceil_div(g.nst_he, tp.sps);
  tp.m4q = ceil_div(T, 64);
  return tp;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct Layout {
  size_t part, cq, cq_scale, qc, xq, xflag, xmax, xmax2, x8, fpart, fss, fykr, fcnt, total;
};

// split-partial rows (S * T) a run of T tokens writes, on any of its paths
int64_t part_rows_at(const mla_prolog_desc& d, int64_t T) {
  // every down-projection a run of T tokens may take (row-major, packed
  // small-T, tiled: fp16 runs take the tiled one at any T)
  const Plan pl = make_plan(d, T);
  const int S = std::max(pl.S, tiled_plan(d, T).S);
  return int64_t(S) * T;
}

// The workspace regions for runs of up to d.max_tokens tokens whose split
// partials take part_rows rows.  small_t: also the regions of the small-T
// kernels that hand data across blocks (exchange buffers, flags, tagged
// partials); without them those kernels must not run.
Layout layout(const mla_prolog_desc& d, int64_t part_rows, bool small_t) {
  Layout L;
  const int64_t Ntot = d.Hcq + d.Hckv + d.Dr;
  // c^Q and q^C are row-major on the row-major-weight path and
  // fragment-packed (16-token tiles of 1 KB k-stages) on the packed path
  const PackGeo g = geo_of(d);
  const size_t tiles = size_t((d.max_tokens + 15) / 16);
  const size_t cq_bytes = std::max(size_t(d.max_tokens) * d.Hcq * 2, tiles * g.nst_cq * 1024);
  const size_t qc_bytes = std::max(size_t(d.max_tokens) * d.N * d.D * 2, tiles * d.N * g.nst_d * 1024);
  L.part = 0;
  L.cq = align256(L.part + size_t(part_rows) * Ntot * 4);
  L.cq_scale = align256(L.cq + cq_bytes);
  L.qc = align256(L.cq_scale + size_t(d.max_tokens) * 4);
  L.xq = align256(L.qc + qc_bytes);
  const size_t st = small_t ? 1 : 0;
  L.xflag = align256(L.xq + st * size_t(d.N) * kPairXq);
  L.xmax = align256(L.xflag + st * size_t(4 * d.N + 1) * 4);
  // the fused small-T kernel: 2N blocks' partials, per-window sums of
  // squares, the c^KV / k^R rows, counters
  const size_t nwin = size_t(g.win_dq + g.win_kr);
  // the static scenario's int8 codes of x
  L.xmax2 = align256(L.xmax + st * size_t(d.N) * 64 * 4);
  L.x8 = align256(L.xmax2 + st * size_t(d.N) * 2 * kRingMaxT * 4);
  const size_t x8_bytes = d.in_dtype == MLA_INT8_STATIC ? size_t(d.max_tokens) * d.He : 0;
  L.fpart = align256(L.x8 + x8_bytes);
  L.fss = align256(L.fpart + st * size_t(2 * d.N) * 32 * 64 * 8);
  L.fykr = align256(L.fss + st * (nwin + g.win_dq) * 32 * 8);
  L.fcnt = align256(L.fykr + st * size_t(32) * (d.Hckv + d.Dr) * 4);
  L.total = align256(L.fcnt + st * (size_t(2 * d.N) * kFusedFlagStride + 1) * 4);
  return L;
}

// A handle's workspace: every T <= max_tokens, every path
Layout layout(const mla_prolog_desc& d) {
  int64_t part_rows = 0;
  // the largest S*T over all T <= max_tokens (plans are cheap host arithmetic)
  for (int64_t T = 1; T <= d.max_tokens; ++T) part_rows = std::max(part_rows, part_rows_at(d, T));
  return layout(d, part_rows, true);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// every rule of a description but the workspace's size
mla_status check_desc_core(const mla_prolog_desc* d) {
  if (!d) return MLA_ERR_NULLPTR;
  const int64_t dims[6] = {d->He, d->Hcq, d->Hckv, d->N, d->D, d->Dr};
  for (int64_t v : dims)
    if (v <= 0 || v > (1 << 20)) return MLA_ERR_PARAM_INVALID;
  // the page's dtype table has an int8 queryOut only in the int8
  // full-quantisation scenario
  if ((d->in_dtype != MLA_BF16 && d->in_dtype != MLA_INT8 && d->in_dtype != MLA_INT8_PARTIAL &&
       d->in_dtype != MLA_INT8_STATIC) ||
      (d->query_dtype != MLA_BF16 && d->query_dtype != MLA_INT8))
    return MLA_ERR_PARAM_INVALID;
  if (d->query_dtype == MLA_INT8 && d->in_dtype != MLA_INT8) return MLA_ERR_PARAM_INVALID;
  // quantised caches: only in the two int8 scenarios (the tables' "kv_cache
  // quantized" columns)
  if (d->cache_dtype != MLA_BF16 && d->cache_dtype != MLA_INT8) return MLA_ERR_PARAM_INVALID;
  if (d->cache_dtype == MLA_INT8 && d->in_dtype != MLA_INT8 && d->in_dtype != MLA_INT8_PARTIAL)
    return MLA_ERR_PARAM_INVALID;
  // the preprocess page's layout and weight options; its concatenated
  // layout holds bf16 rows only
  if ((d->concat != 0 && d->concat != 1) || (d->weights_nk != 0 && d->weights_nk != 1) ||
      (d->x_quant_only != 0 && d->x_quant_only != 1) || (d->check_index != 0 && d->check_index != 1))
    return MLA_ERR_PARAM_INVALID;
  if (d->concat && (d->query_dtype != MLA_BF16 || d->cache_dtype != MLA_BF16)) return MLA_ERR_PARAM_INVALID;
  if (d->x_quant_only && d->in_dtype != MLA_INT8_STATIC) return MLA_ERR_PARAM_INVALID;
  // fp16 tensors: the preprocess page's FLOAT16 input, its static scenario
  if ((d->float_dtype != MLA_BF16 && d->float_dtype != MLA_FP16) || d->reserved != 0)
    return MLA_ERR_PARAM_INVALID;
  if (d->float_dtype == MLA_FP16 && d->in_dtype != MLA_INT8_STATIC) return MLA_ERR_PARAM_INVALID;
  if (d->in_dtype == MLA_INT8_STATIC && (!(d->eps_x >= 0.0) || !std::isfinite(d->eps_x)))
    return MLA_ERR_PARAM_INVALID;
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
  if (d->Dr > 64 || d->Hckv > 512 || d->D > 512 || d->He > 65536) return MLA_ERR_UNSUPPORTED;
  // int8 operands move in 16-byte (16-element) chunks that must not cross a
  // row or column-block end
  if (down_i8(*d) &&
      (d->He % 16 || d->Hcq % 16 || (d->Hckv + d->Dr) % 16 || d->D % 16 || d->Dr % 16))
    return MLA_ERR_UNSUPPORTED;
  if (d->in_dtype == MLA_INT8_PARTIAL && (d->Hcq % 16 || d->D % 16 || d->Dr % 16))
    return MLA_ERR_UNSUPPORTED;
  if (d->N * (d->D + d->Dr) > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

mla_status check_desc(const mla_prolog_desc* d) {
  const mla_status st = check_desc_core(d);
  if (st != MLA_OK) return st;
  // the norm kernel addresses the split partials with 32-bit offsets
  const Layout L = layout(*d);
  if (L.cq - L.part >= size_t(kOOB)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

mla_status check_tensors(const mla_prolog_desc* d, const mla_prolog_tensors* t, int64_t T) {
  if (T < 0 || T > d->max_tokens) return MLA_ERR_PARAM_INVALID;
  if (!t) return MLA_ERR_NULLPTR;
  if (T == 0) return MLA_OK;
  // the concatenated layout has no separate q^R output or k^R cache
  const void* qr_or_q = d->concat ? t->query_out : t->query_rope_out;
  const void* req[] = {t->token_x, t->gamma_cq, t->gamma_ckv, t->rope_sin, t->rope_cos, t->cache_index,
                       t->query_out, qr_or_q};
  for (const void* q : req)
    if (!q) return MLA_ERR_NULLPTR;
  for (const void* q : req)
    if (!aligned16(q)) return MLA_ERR_PARAM_INVALID;
  // the unpacked weights: read only by the kernels of runs without the
  // packed copy
  const void* wts[] = {t->weight_dq, t->weight_uq_qr, t->weight_uk, t->weight_dkv_kr};
  for (const void* q : wts) {
    if (!q && !t->packed_weights) return MLA_ERR_NULLPTR;
    if (q && !aligned16(q)) return MLA_ERR_PARAM_INVALID;
  }
  if (d->concat && (t->query_rope_out || t->kr_cache)) return MLA_ERR_PARAM_INVALID;
  if (d->block_num > 0) {
    const void* kr = d->concat ? t->kv_cache : t->kr_cache;
    if (!t->kv_cache || !kr) return MLA_ERR_NULLPTR;
    if (!aligned16(t->kv_cache) || !aligned16(kr)) return MLA_ERR_PARAM_INVALID;
  }
  // the static scenario's norm and quantisation parameters, absent elsewhere
  const bool st = is_static(*d), xn = st && !d->x_quant_only;
  const void* st_req[] = {t->quant_scale_x, t->quant_offset_x, t->beta_cq, t->quant_scale_cq,
                          t->quant_offset_cq};
  for (const void* q : st_req) {
    if (st && !q) return MLA_ERR_NULLPTR;
    if (!st && q) return MLA_ERR_PARAM_INVALID;
  }
  if (xn && (!t->gamma_x || !t->beta_x)) return MLA_ERR_NULLPTR;
  if (!xn && (t->gamma_x || t->beta_x)) return MLA_ERR_PARAM_INVALID;
  if (!st && (t->bias_dqkv || t->bias_uq_qr)) return MLA_ERR_PARAM_INVALID;
  // every tensor is 16-byte aligned (the per-channel vectors are read in
  // 16-byte chunks)
  const void* opt[] = {t->gamma_x, t->beta_x, t->quant_scale_x, t->quant_offset_x, t->beta_cq,
                       t->quant_scale_cq, t->quant_offset_cq, t->bias_dqkv, t->bias_uq_qr,
                       t->scale_x, t->scale_w_dq, t->scale_w_uq_qr, t->scale_w_dkv_kr,
                       t->smooth_scales_cq, t->quant_scale_ckv, t->quant_scale_ckr,
                       t->dequant_scale_q_nope};
  for (const void* q : opt)
    if (q && !aligned16(q)) return MLA_ERR_PARAM_INVALID;
  // the unpacked kernels read (k, n) bf16 weights only
  if ((d->weights_nk || d->float_dtype == MLA_FP16) && !t->packed_weights) return MLA_ERR_UNSUPPORTED;
  // the scales each scenario takes: all four in full quantisation, that of
  // weightUqQr alone in partial quantisation, none without quantisation
  const float* sc[] = {t->scale_x, t->scale_w_dq, t->scale_w_uq_qr, t->scale_w_dkv_kr};
  const bool need[] = {down_i8(*d) && !st, down_i8(*d), up_i8(*d), down_i8(*d)};
  for (int i = 0; i < 4; ++i) {
    if (need[i] && !sc[i]) return MLA_ERR_NULLPTR;
    if (!need[i] && sc[i]) return MLA_ERR_PARAM_INVALID;
  }
  // smoothScalesCq: optional with an int8 weightUqQr, absent otherwise
  if (t->smooth_scales_cq && (!up_i8(*d) || st))
    return MLA_ERR_PARAM_INVALID;
  // quantScaleCkv with an int8 kv cache; quantScaleCkr with an int8 kr
  // cache, which partial quantisation has and full quantisation does not
  const bool kv8 = d->cache_dtype == MLA_INT8, kr8 = kv8 && d->in_dtype == MLA_INT8_PARTIAL;
  if (kv8 && !t->quant_scale_ckv) return MLA_ERR_NULLPTR;
  if (kr8 && !t->quant_scale_ckr) return MLA_ERR_NULLPTR;
  if ((!kv8 && t->quant_scale_ckv) || (!kr8 && t->quant_scale_ckr)) return MLA_ERR_PARAM_INVALID;
  if (t->packed_weights && (reinterpret_cast<uintptr_t>(t->packed_weights) & 255u))
    return MLA_ERR_PARAM_INVALID;
  if (d->query_dtype == MLA_INT8 && !t->dequant_scale_q_nope) return MLA_ERR_NULLPTR;
  if (d->query_dtype == MLA_BF16 && t->dequant_scale_q_nope) return MLA_ERR_PARAM_INVALID;
  return MLA_OK;
}

// cacheIndex copied to the host (after the stream's earlier work) and
// checked: MLA_ERR_PARAM_INVALID if an entry lies outside [0, slots)
mla_status check_cache_index(const int64_t* idx, int64_t T, int64_t slots, hipStream_t s) {
  int64_t* host = nullptr;
  if (hipHostMalloc(reinterpret_cast<void**>(&host), size_t(T) * sizeof(int64_t), hipHostMallocDefault) !=
      hipSuccess)
    return MLA_ERR_RUNTIME;
  mla_status st = MLA_OK;
  if (hipMemcpyAsync(host, idx, size_t(T) * sizeof(int64_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    st = MLA_ERR_RUNTIME;
  for (int64_t i = 0; st == MLA_OK && i < T; ++i)
    if (host[i] < 0 || host[i] >= slots) st = MLA_ERR_PARAM_INVALID;
  (void)hipHostFree(host);
  return st;
}

}  // namespace

constexpr int kProfileRing = 2048;
constexpr int kProfileEvents = 5;

// The workspace of mla_prolog_run_noalloc: one array per device, allocated
// with the library's code object when it is loaded on that device and held
// until the process ends.  In host code `scratch` is only a stand-in for the
// symbol; its device address comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct mla_prolog {
  mla_prolog_desc desc;
  int spin;            // poll steps of the small-T kernels' bounded waits
  Layout lay;
  uint8_t* ws;
  hipEvent_t* events;  // kProfileRing x kProfileEvents when profiling, else NULL
  uint8_t* fused;      // per recorded run: 0 four kernels, 1 up_proj and uk as one, 2 one kernel
  int64_t recorded;    // runs recorded since the last read
  bool fused_fit[2];   // the fused kernel (16 or 32 tokens) has all 2N blocks resident at once
  uint32_t run_no;     // number of the last run (1, 2, ...; 0 is skipped on a wrap)
  uint32_t* herr;      // error word in mapped, coherent host memory (host address)
  uint32_t* herr_dev;  // the same word's device address
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

// K2 with eight waves per token when there are few tokens, one otherwise.
template <bool I8D, bool I8U, bool F16 = false>
void launch_norm(hipStream_t s, const Dims& d, const Ptrs& p, int S, int cq_nst) {
  if constexpr (I8D && I8U) {
    if (p.beta_cq) {   // the static scenario (fp16 tensors when F16)
      if (d.T <= 512) k2_norm<true, true, true, 8, 1, 1, F16><<<dim3(d.T), 512, 0, s>>>(d, p, S, cq_nst);
      else k2_norm<true, true, true, 1, 4, 1, F16><<<dim3((d.T + 3) / 4), 256, 0, s>>>(d, p, S, cq_nst);
      return;
    }
  }
  if (d.T <= 512) k2_norm<I8D, I8U, false, 8, 1, 1><<<dim3(d.T), 512, 0, s>>>(d, p, S, cq_nst);
  else k2_norm<I8D, I8U, false, 1, 4, 1><<<dim3((d.T + 3) / 4), 256, 0, s>>>(d, p, S, cq_nst);
}

// The int8-query W^UK kernel gives one wave to each 64-column window of Hckv.
// Small-T run on packed weights: K1p (down-projection, split partials), K2
// (norms, c^Q, caches), K3p (up-projection, q-RoPE, q^C), K4p (W^UK).
// Profiling marks follow the kernels.  I8D: int8 down-projection operands;
// I8U: int8 c^Q and W^UqQr.
// The down-projection of a small-T packed run, as on the tiled path at these
// token counts: one 64-token wave per 64-column window, He split to about
// kTiledK1Blocks blocks (9.5 -> 6.7 us int8 and 12.4 -> 9.7 us bf16 at 32
// tokens, the model shapes, against a four-wave split-window kernel), then
// the norm kernel.
template <bool I8D, bool I8U, class Mark, bool F16 = false>
void small_down_norm(hipStream_t s, const Dims& d, const Ptrs& p, const PackGeo& g, Mark& mark) {
  const int tiles = g.win_dq + g.win_kr, m1 = ceil_div(d.T, 64);
  int S1 = std::max(1, std::min(g.nst_he, kTiledK1Blocks / std::max(1, m1 * tiles)));
  const int sps1 = ceil_div(g.nst_he, S1);
  S1 = ceil_div(g.nst_he, sps1);
  k1_tiled<I8D, 4, 1, 1, 1, 2><<<dim3(m1 * tiles * S1), 64, 0, s>>>(d, p, g, sps1, m1, tiles);
  mark(1);
  launch_norm<I8D, I8U, F16>(s, d, p, S1, g.nst_cq);
  mark(2);
}

// fp16 tensors (the static scenario), small T, the paired kernel's shapes
template <int MT, class Mark>
void packed_launch_f16(hipStream_t s, const Dims& d, const Ptrs& p, const PackGeo& g, Mark& mark) {
  small_down_norm<true, true, Mark, true>(s, d, p, g, mark);
  k34_pair<true, MT, false, 2, true><<<dim3(2 * d.N), 512, 0, s>>>(d, p, g);
  mark(3);
  mark(-1);
}

template <bool I8D, bool I8U, int MT, class Mark>
void packed_launch(hipStream_t s, const Dims& d, const Ptrs& p, const PackGeo& g, bool q8, bool pair_ok,
                   Mark& mark) {
  constexpr bool I8 = I8U;   // the up-projection kernels below
  small_down_norm<I8D, I8U>(s, d, p, g, mark);
  if (pair_ok && g.nope_w == 2 && d.Dr == 64 && g.uk_w <= 8) {
    // two balanced blocks per head; the profile books both products to the first
    if (q8) k34_pair<I8, MT, true><<<dim3(2 * d.N), 512, 0, s>>>(d, p, g);
    else k34_pair<I8, MT, false><<<dim3(2 * d.N), 512, 0, s>>>(d, p, g);
    mark(3);
    mark(-1);
    return;
  }
  if (g.nope_w <= kK34Waves && g.uk_w <= kK34Waves && g.nst_d <= kK34Stages) {
    // up-projection and W^UK fused; the profile books both to the first
    if (q8) k34_stream<I8, MT, 2, true><<<dim3(2 * d.N), 512, 0, s>>>(d, p, g);
    else k34_stream<I8, MT, 2, false><<<dim3(2 * d.N), 512, 0, s>>>(d, p, g);
    mark(3);
    mark(-1);
    return;
  }
  k3_packed<I8, MT, 8, 2><<<dim3(d.N * (g.nope_w + 1)), 512, 0, s>>>(d, p, g);
  mark(3);
  if (q8) k4_packed_q8<MT, 4><<<dim3(d.N), 512, 0, s>>>(d, p, g);
  else k4_packed<MT, 4, 1><<<dim3(d.N * g.uk_w), 256, 0, s>>>(d, p, g);
  mark(4);
}

// The fused small-T kernel (bf16, two nope windows, Dr = 64): the split of
// the phase-1 windows over the 2N blocks, or false when the shapes are
// outside what the kernel holds in registers.
bool fused_geo(const mla_prolog_desc& dd, FusedGeo* fg) {
  if ((dd.in_dtype != MLA_BF16 && dd.in_dtype != MLA_INT8_PARTIAL && dd.in_dtype != MLA_INT8_STATIC) ||
      dd.query_dtype != MLA_BF16 || dd.cache_dtype != MLA_BF16 || dd.float_dtype != MLA_BF16)
    return false;
  const PackGeo g = geo_of(dd);
  if (g.nope_w != 2 || dd.Dr != 64 || g.uk_w > 8 || g.nst_d > 4) return false;
  const int G = int(2 * dd.N), W = g.win_dq + g.win_kr;
  if (G < W || (g.nst_cq + 6) / 7 > kFusedStages) return false;
  const int base = G / W;
  if (base >= kFusedMaxSplits) {
    fg->hi_win = W; fg->hi_s = kFusedMaxSplits;
  } else if (G % W == 0) {
    fg->hi_win = W; fg->hi_s = base;
  } else {
    fg->hi_win = G % W; fg->hi_s = base + 1;
  }
  fg->nwin = W;
  fg->p1 = fg->hi_win * fg->hi_s + (W - fg->hi_win) * (fg->hi_s - 1);
  const int smin = fg->hi_win < W ? fg->hi_s - 1 : fg->hi_s;
  if ((ceil_div(g.nst_he, smin) + 7) / 8 > kFusedP1) return false;
  return true;
}

// the fused kernel's instance for a description's scenario, MT 1 or 2
const void* fused_kernel(const mla_prolog_desc& dd, int mt) {
  if (dd.in_dtype == MLA_INT8_STATIC)
    return mt == 1 ? reinterpret_cast<const void*>(k_fused<1, true, true>)
                   : reinterpret_cast<const void*>(k_fused<2, true, true>);
  if (dd.in_dtype == MLA_INT8_PARTIAL)
    return mt == 1 ? reinterpret_cast<const void*>(k_fused<1, true>) : reinterpret_cast<const void*>(k_fused<2, true>);
  return mt == 1 ? reinterpret_cast<const void*>(k_fused<1>) : reinterpret_cast<const void*>(k_fused<2>);
}

template <int MT, class Mark>
void packed_launch_mt(hipStream_t s, const Dims& d, const Ptrs& p, const PackGeo& g, bool i8d, bool i8u,
                      bool q8, bool pair_ok, Mark& mark) {
  if (i8d) packed_launch<true, true, MT>(s, d, p, g, q8, pair_ok, mark);
  else if (i8u) packed_launch<false, true, MT>(s, d, p, g, q8, pair_ok, mark);
  else packed_launch<false, false, MT>(s, d, p, g, q8, pair_ok, mark);
}

template <class Mark>
void launch_packed(const Plan& pl, hipStream_t s, const Dims& d, const Ptrs& p,
                   const mla_prolog_desc& dd, bool q8, bool pair_ok, Mark& mark) {
  const PackGeo g = geo_of(dd);
  if (pl.mt1 == 1) packed_launch_mt<1>(s, d, p, g, down_i8(dd), up_i8(dd), q8, pair_ok, mark);
  else packed_launch_mt<2>(s, d, p, g, down_i8(dd), up_i8(dd), q8, pair_ok, mark);
}

// K3r: 2N blocks; 16 or 32 tokens per wave; the instance unrolling the
// fewest stages that hold Hcq's
template <bool I8U, bool UK, bool Q8>
void launch_ring(hipStream_t s, const Dims& d, const Ptrs& p, const PackGeo& g) {
  const dim3 gr(2 * d.N);
  if (d.T <= 128) {
    if (g.nst_cq <= 8) k3_ring<I8U, 1, 4, 8, UK, Q8><<<gr, 512, 0, s>>>(d, p, g);
    else if (g.nst_cq <= 24) k3_ring<I8U, 1, 4, 24, UK, Q8><<<gr, 512, 0, s>>>(d, p, g);
    else k3_ring<I8U, 1, 4, 48, UK, Q8><<<gr, 512, 0, s>>>(d, p, g);
  } else {
    if (g.nst_cq <= 8) k3_ring<I8U, 2, 4, 8, UK, Q8><<<gr, 512, 0, s>>>(d, p, g);
    else if (g.nst_cq <= 24) k3_ring<I8U, 2, 4, 24, UK, Q8><<<gr, 512, 0, s>>>(d, p, g);
    else k3_ring<I8U, 2, 4, 48, UK, Q8><<<gr, 512, 0, s>>>(d, p, g);
  }
}

// The long-run W^UK kernel: about one block per CU, all of a head's blocks
// sharing its W^UK
template <bool F16>
void launch_k4_rows(hipStream_t s, const Dims& d, const Ptrs& p, const PackGeo& g) {
  const int mtiles = ceil_div(d.T, kRowsTile);
  const int ph = std::max(1, std::min(mtiles, 256 / d.N));
  k4_rows<F16><<<dim3(ph * d.N), 512, 0, s>>>(d, p, g, ph);
}

// The long-run W^UK kernel with the int8 query: about one block per CU
void launch_k4_rows_q8(hipStream_t s, const Dims& d, const Ptrs& p, const PackGeo& g) {
  const int mtiles = ceil_div(d.T, kRowsQ8Tile);
  const int ph = std::max(1, std::min(mtiles, 256 / d.N));
  k4_rows_q8<<<dim3(ph * d.N), 512, 0, s>>>(d, p, g, ph);
}

// Tiled run on packed weights (token counts above the streaming range).
template <bool I8D, bool I8U, int MT, class Mark, bool F16 = false>
void tiled_medium(const TiledPlan& tp, hipStream_t s, const Dims& d, const Ptrs& p, const PackGeo& g,
                  bool q8, bool pair_ok, Mark& mark) {
  const dim3 g1(tp.m1 * tp.ngrp1 * tp.S), g3(tp.m3 * tp.ngrp3);
  const int n1 = tp.m1 * tp.ngrp1 * tp.S;
  // the 128- and 256-token tiles run in XCD order (the token tiles of a
  // window group share an XCD's L2: at the model's shapes 24.1 -> 22.9 us
  // for 256 bf16 tokens, 94.8 -> 86 us for 1536); the int8 64-token tiles
  // keep the plain order (13.6 -> 14.0 us at 128 tokens with it)
  const dim3 g1x((n1 + 7) / 8 * 8);
  if (tp.k1L)
    k1_tiled<I8D, 4, 1, 4, 4, 2, true><<<g1, 1024, 0, s>>>(d, p, g, tp.sps, tp.m1, tp.ngrp1);
  else if (tp.k1v == 1)
    k1_tiled<I8D, 4, 1, 4, 2, 2, true, 1, true><<<g1x, 512, 0, s>>>(d, p, g, tp.sps, tp.m1, tp.ngrp1, n1);
  else if (tp.k1v == 3)
    k1_tiled<I8D, 1, 1, 4, 2, 2, true, 1, true><<<g1, 512, 0, s>>>(d, p, g, tp.sps, tp.m1, tp.ngrp1);
  else if (tp.k1v == 2)
    k1_tiled<I8D, 2, 1, 4, 2, 2, true, 1, true><<<g1x, 512, 0, s>>>(d, p, g, tp.sps, tp.m1, tp.ngrp1, n1);
  else k1_tiled<I8D, MT, 1, 1, 1, 2><<<g1, 64, 0, s>>>(d, p, g, tp.sps, tp.m1, tp.ngrp1);
  mark(1);
  launch_norm<I8D, I8U, F16>(s, d, p, tp.S, g.nst_cq);
  mark(2);
  // with paired blocks allowed (and at most eight W^UK windows of four D
  // stages), the W^UK product runs in the same launch
  const bool uk = tp.ring && pair_ok && g.uk_w <= 8 && g.nst_d <= 4;
  if (tp.ring) {
    if (uk) {
      if (q8) launch_ring<I8U, true, true>(s, d, p, g);
      else launch_ring<I8U, true, false>(s, d, p, g);
    } else {
      launch_ring<I8U, false, false>(s, d, p, g);
    }
  } else if (tp.k3L) {
    k3_tiled<I8U, 4, 1, 4, 4, 2, true, 1, false, F16><<<g3, 1024, 0, s>>>(d, p, g, tp.m3);
  } else if (tp.k3v == 1) {
    k3_tiled<I8U, 2, 1, 8, 2, 2, true, 1, true, F16><<<g3, 1024, 0, s>>>(d, p, g, tp.m3);
  } else if (I8U && tp.k3v == 2) {
    k3_tiled<I8U, 1, 1, 8, 2, 2, true, 1, true, F16><<<g3, 1024, 0, s>>>(d, p, g, tp.m3);
  } else {
    k3_tiled<I8U, 4, 1, 1, 1, 2, false, 1, false, F16><<<g3, 64, 0, s>>>(d, p, g, tp.m3);
  }
  if (uk) {
    // one kernel did both products; the profile books them to the first
    mark(3);
    mark(-1);
    return;
  }
  mark(3);
  if (q8 && tp.k4R) launch_k4_rows_q8(s, d, p, g);
  else if (q8) k4_tiled<4, 1, 1, 8, 2, true, false, true><<<dim3(tp.m4q * d.N), 512, 0, s>>>(d, p, g, tp.m4q, 1);
  else if (tp.k4R) launch_k4_rows<F16>(s, d, p, g);
  else k4_tiled<MT, 1, 1, 8, 2, false, false, true, F16><<<dim3(tp.m4 * tp.cg4 * d.N), 512, 0, s>>>(d, p, g, tp.m4,
                                                                                           tp.cg4);
  mark(4);
}

template <bool I8D, bool I8U, class Mark, bool F16 = false>
void tiled_large(const TiledPlan& tp, hipStream_t s, const Dims& d, const Ptrs& p, const PackGeo& g,
                 bool q8, Mark& mark) {
  k1_tiled<I8D, 4, 1, 4, 4, 2, true><<<dim3(tp.m1 * tp.ngrp1 * tp.S), 1024, 0, s>>>(d, p, g, tp.sps,
                                                                                   tp.m1, tp.ngrp1);
  mark(1);
  launch_norm<I8D, I8U, F16>(s, d, p, tp.S, g.nst_cq);
  mark(2);
  k3_tiled<I8U, 4, 1, 4, 4, 2, true, 1, false, F16><<<dim3(tp.m3 * tp.ngrp3), 1024, 0, s>>>(d, p, g, tp.m3);
  mark(3);
  if (q8 && tp.k4R) launch_k4_rows_q8(s, d, p, g);
  else if (q8) k4_tiled<4, 1, 1, 8, 2, true, false, true><<<dim3(tp.m4q * d.N), 512, 0, s>>>(d, p, g, tp.m4q, 1);
  else if (tp.k4R) launch_k4_rows<F16>(s, d, p, g);
  else k4_tiled<4, 1, 4, 4, 2, false, true, true, F16><<<dim3(tp.m4 * tp.cg4 * d.N), 1024, 0, s>>>(d, p, g, tp.m4,
                                                                                          tp.cg4);
  mark(4);
}

template <bool I8D, bool I8U, class Mark, bool F16 = false>
void tiled_run(const TiledPlan& tp, hipStream_t s, const Dims& d, const Ptrs& p, const PackGeo& g,
               bool q8, bool pair_ok, Mark& mark) {
  if (tp.large) tiled_large<I8D, I8U, Mark, F16>(tp, s, d, p, g, q8, mark);
  else if (tp.mt == 4) tiled_medium<I8D, I8U, 4, Mark, F16>(tp, s, d, p, g, q8, pair_ok, mark);
  else tiled_medium<I8D, I8U, 8, Mark, F16>(tp, s, d, p, g, q8, pair_ok, mark);
}

template <class Mark>
void launch_tiled(hipStream_t s, const Dims& d, const Ptrs& p, const mla_prolog_desc& dd, bool q8,
                  bool pair_ok, Mark& mark) {
  const PackGeo g = geo_of(dd);
  const TiledPlan tp = tiled_plan(dd, d.T);
  // fp16 tensors: the static scenario only, on these kernels at every T
  if (dd.float_dtype == MLA_FP16) tiled_run<true, true, Mark, true>(tp, s, d, p, g, q8, pair_ok, mark);
  else if (down_i8(dd)) tiled_run<true, true>(tp, s, d, p, g, q8, pair_ok, mark);
  else if (up_i8(dd)) tiled_run<false, true>(tp, s, d, p, g, q8, pair_ok, mark);
  else tiled_run<false, false>(tp, s, d, p, g, q8, pair_ok, mark);
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

size_t mla_prolog_packed_weights_bytes(const mla_prolog_desc* desc) {
  if (check_desc(desc) != MLA_OK) return 0;
  return size_t(geo_of(*desc).total);
}

mla_status mla_prolog_pack_weights(mla_prolog_t h, const mla_prolog_tensors* t, void* packed,
                                   void* stream) {
  if (!h || !t || !packed) return MLA_ERR_NULLPTR;
  const mla_prolog_desc& dd = h->desc;
  const void* w[4] = {t->weight_dq, t->weight_uq_qr, t->weight_uk, t->weight_dkv_kr};
  for (const void* q : w)
    if (!q) return MLA_ERR_NULLPTR;
  for (const void* q : w)
    if (!aligned16(q)) return MLA_ERR_PARAM_INVALID;
  if (reinterpret_cast<uintptr_t>(packed) & 255u) return MLA_ERR_PARAM_INVALID;
  const PackGeo g = geo_of(dd);
  if (g.total >= int64_t(kOOB)) return MLA_ERR_UNSUPPORTED;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_RUNTIME;
  if (prev != dd.device && hipSetDevice(dd.device) != hipSuccess) return MLA_ERR_RUNTIME;
  (void)hipGetLastError();
  Dims d;
  d.T = 0; d.He = int(dd.He); d.Hcq = int(dd.Hcq); d.Hckv = int(dd.Hckv); d.N = int(dd.N);
  d.D = int(dd.D); d.Dr = int(dd.Dr); d.slots = 0; d.eps_cq = d.eps_ckv = 0.0;
  d.run = 0; d.spin = 0;
  Ptrs p;
  std::memset(&p, 0, sizeof p);
  p.w_dq = static_cast<const uint8_t*>(t->weight_dq);
  p.w_uq_qr = static_cast<const uint8_t*>(t->weight_uq_qr);
  p.w_uk = static_cast<const uint16_t*>(t->weight_uk);
  p.w_dkv_kr = static_cast<const uint8_t*>(t->weight_dkv_kr);
  const int64_t chunks = g.total / 16;
  k_pack<<<dim3(unsigned((chunks + 255) / 256)), 256, 0, static_cast<hipStream_t>(stream)>>>(
      d, p, g, int(down_i8(dd)), int(up_i8(dd)), int(dd.weights_nk != 0), static_cast<uint8_t*>(packed));
  const hipError_t e = hipGetLastError();
  if (prev != dd.device) (void)hipSetDevice(prev);
  return e == hipSuccess ? MLA_OK : MLA_ERR_RUNTIME;
}

mla_status mla_prolog_create(const mla_prolog_desc* desc, mla_prolog_t* out) {
  if (!out) return MLA_ERR_NULLPTR;
  *out = nullptr;
  mla_status st = check_desc(desc);
  if (st != MLA_OK) return st;
  // MLA_PROLOG_FUSED_SPIN overrides the poll steps a bounded wait makes
  // before it gives up (a test of the failure report sets it to 1); a value
  // that is not a whole number in [1, kFusedSpin] is refused
  int spin = kFusedSpin;
  if (const char* sp = std::getenv("MLA_PROLOG_FUSED_SPIN")) {
    char* end = nullptr;
    const long v = std::strtol(sp, &end, 10);
    if (end == sp || *end != '\0' || v <= 0 || v > kFusedSpin) return MLA_ERR_PARAM_INVALID;
    spin = int(v);
  }
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_RUNTIME;
  if (hipSetDevice(desc->device) != hipSuccess) return MLA_ERR_PARAM_INVALID;
  mla_prolog* h = new (std::nothrow) mla_prolog;
  if (!h) { (void)hipSetDevice(prev); return MLA_ERR_RUNTIME; }
  h->desc = *desc;
  h->lay = layout(*desc);
  h->ws = nullptr;
  h->events = nullptr;
  h->fused = nullptr;
  h->recorded = 0;
  h->herr = h->herr_dev = nullptr;
  if (hipMalloc(&h->ws, h->lay.total) != hipSuccess) {
    delete h;
    (void)hipSetDevice(prev);
    return MLA_ERR_RUNTIME;
  }
  // the error word of the bounded waits, where the host can read it at any
  // time without a synchronisation
  if (hipHostMalloc(reinterpret_cast<void**>(&h->herr), 64, hipHostMallocMapped | hipHostMallocCoherent) !=
          hipSuccess ||
      hipHostGetDevicePointer(reinterpret_cast<void**>(&h->herr_dev), h->herr, 0) != hipSuccess) {
    if (h->herr) (void)hipHostFree(h->herr);
    (void)hipFree(h->ws);
    delete h;
    (void)hipSetDevice(prev);
    return MLA_ERR_RUNTIME;
  }
  __atomic_store_n(h->herr, 0u, __ATOMIC_RELEASE);
  // the flags and tags of the small-T kernels start at zero, which no run's
  // number is
  if (hipMemset(h->ws + h->lay.xflag, 0, size_t(4 * desc->N + 1) * 4) != hipSuccess ||
      hipMemset(h->ws + h->lay.fpart, 0, h->lay.total - h->lay.fpart) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipHostFree(h->herr);
    (void)hipFree(h->ws);
    delete h;
    (void)hipSetDevice(prev);
    return MLA_ERR_RUNTIME;
  }
  h->run_no = 0;
  h->spin = spin;
  // the fused kernel's blocks wait for one another, so all 2N of them must
  // be resident at once; MLA_PROLOG_FUSED=0 in the environment turns it off
  h->fused_fit[0] = h->fused_fit[1] = false;
  {
    FusedGeo fg;
    const char* env = std::getenv("MLA_PROLOG_FUSED");
    int cus = 0, nb1 = 0, nb2 = 0;
    if (!(env && env[0] == '0') && fused_geo(*desc, &fg) &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, desc->device) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb1, fused_kernel(*desc, 1), 512, 0) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb2, fused_kernel(*desc, 2), 512, 0) == hipSuccess) {
      h->fused_fit[0] = int64_t(nb1) * cus >= 2 * desc->N;
      h->fused_fit[1] = int64_t(nb2) * cus >= 2 * desc->N;
    }
    (void)hipGetLastError();
  }

  (void)hipSetDevice(prev);
  *out = h;
  return MLA_OK;
}

}  // extern "C"

namespace {

// One run's launches on stream s, with the workspace at ws (laid out as
// lay).  fused_ok / pair_ok allow the small-T kernels whose blocks hand data
// to one another through flags and tagged words that hold the run's number;
// without them every kernel of the run only reads what earlier kernels of
// the stream wrote.  ev / mark_kind are this run's profiling events (or
// NULL).  The caller has validated the run and made its device current.
struct RunCtx {
  const mla_prolog_desc* dd;
  const Layout* lay;
  uint8_t* ws;
  bool fused_ok, pair_ok;
  uint32_t run;
  int spin;
  hipEvent_t* ev;
  uint8_t* mark_kind;
  uint32_t* herr;   // device address of the error word of the bounded waits
};

mla_status enqueue(const RunCtx& c, const mla_prolog_tensors* t, int64_t T, hipStream_t s) {
  const mla_prolog_desc& dd = *c.dd;
  const Layout& lay = *c.lay;
  uint8_t* const ws = c.ws;
  const bool i8d = down_i8(dd), i8u = up_i8(dd), q8 = dd.query_dtype == MLA_INT8;
  const Plan pl = make_plan(dd, T);
  Dims d;
  d.T = int(T); d.He = int(dd.He); d.Hcq = int(dd.Hcq); d.Hckv = int(dd.Hckv); d.N = int(dd.N);
  d.D = int(dd.D); d.Dr = int(dd.Dr);
  d.slots = dd.block_num * dd.block_size;
  d.eps_cq = dd.eps_cq; d.eps_ckv = dd.eps_ckv;
  d.run = c.run;
  d.spin = c.spin;
  const int row = int(dd.Hckv + dd.Dr);
  d.qs = dd.concat ? row : d.Hckv;
  d.qrs = dd.concat ? row : d.Dr;
  d.kvs = dd.concat ? row : d.Hckv;
  d.krs = dd.concat ? row : d.Dr;
  Ptrs p;
  std::memset(&p, 0, sizeof p);
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
  if (dd.concat && p.kv_cache) p.kr_cache = p.kv_cache + dd.Hckv;   // k^R after c^KV in each slot
  p.qs_ckv = t->quant_scale_ckv;
  p.qs_ckr = t->quant_scale_ckr;
  p.sx = t->scale_x; p.sw_dq = t->scale_w_dq; p.sw_uq_qr = t->scale_w_uq_qr;
  p.sw_dkv_kr = t->scale_w_dkv_kr;
  p.smooth_cq = t->smooth_scales_cq;
  p.q_out = t->query_out;
  p.qr_out = dd.concat ? static_cast<uint16_t*>(t->query_out) + dd.Hckv   // q^R after q^N in each row
                       : static_cast<uint16_t*>(t->query_rope_out);
  p.bias_dq = t->bias_dqkv;
  p.bias_uq = t->bias_uq_qr;
  p.beta_cq = static_cast<const uint16_t*>(t->beta_cq);
  p.qsc_cq = static_cast<const uint16_t*>(t->quant_scale_cq);
  p.qo_cq = t->quant_offset_cq;
  p.q_scale = t->dequant_scale_q_nope;
  p.part = ws + lay.part;
  p.cq = ws + lay.cq;
  p.cq_scale = reinterpret_cast<float*>(ws + lay.cq_scale);
  p.qc = reinterpret_cast<uint16_t*>(ws + lay.qc);
  p.xq = ws + lay.xq;
  p.xflag = reinterpret_cast<uint32_t*>(ws + lay.xflag);
  p.xmax = reinterpret_cast<float*>(ws + lay.xmax);
  p.xmax2 = reinterpret_cast<float*>(ws + lay.xmax2);
  p.fpart = reinterpret_cast<uint32_t*>(ws + lay.fpart);
  p.fss = reinterpret_cast<uint32_t*>(ws + lay.fss);
  p.fykr = reinterpret_cast<float*>(ws + lay.fykr);
  p.fcnt = reinterpret_cast<uint32_t*>(ws + lay.fcnt);
  p.herr = c.herr;

  hipEvent_t* const ev = c.ev;
  uint8_t* const fused = c.mark_kind;
  if (fused) *fused = 0;
  // mark(i): event i (after kernel i); mark(-1): the last event of a run
  // whose up_proj and uk were one kernel; mark(-2): the last event of a run
  // that was one kernel
  auto mark = [&](int i) {
    if (!ev) return;
    if (i < 0) *fused = uint8_t(-i);
    (void)hipEventRecord(ev[i < 0 ? kProfileEvents - 1 : i], s);
  };
  mark(0);
  if (is_static(dd)) {
    // x to int8 codes first; the down-projection then reads the codes (the
    // profile books this to the down-projection)
    XQuant xq;
    xq.x = static_cast<const uint16_t*>(t->token_x);
    xq.gamma = static_cast<const uint16_t*>(t->gamma_x);
    xq.beta = static_cast<const uint16_t*>(t->beta_x);
    xq.scale = static_cast<const uint16_t*>(t->quant_scale_x);
    xq.offset = t->quant_offset_x;
    xq.out = ws + lay.x8;
    xq.T = d.T; xq.He = d.He; xq.eps = dd.eps_x;
    if (dd.float_dtype == MLA_FP16) k0_xquant<true><<<dim3(unsigned(T)), kXqThreads, 0, s>>>(xq);
    else k0_xquant<false><<<dim3(unsigned(T)), kXqThreads, 0, s>>>(xq);
    p.x = xq.out;
  }
  p.packed = static_cast<const uint8_t*>(t->packed_weights);
  FusedGeo fg;
  if (p.packed && pl.stream && c.fused_ok && dd.float_dtype != MLA_FP16 && fused_geo(dd, &fg)) {
    const PackGeo g = geo_of(dd);
    if (dd.in_dtype == MLA_INT8_STATIC) {
      if (pl.mt1 == 1) k_fused<1, true, true><<<dim3(2 * d.N), 512, 0, s>>>(d, p, g, fg);
      else k_fused<2, true, true><<<dim3(2 * d.N), 512, 0, s>>>(d, p, g, fg);
    } else if (dd.in_dtype == MLA_INT8_PARTIAL) {
      if (pl.mt1 == 1) k_fused<1, true><<<dim3(2 * d.N), 512, 0, s>>>(d, p, g, fg);
      else k_fused<2, true><<<dim3(2 * d.N), 512, 0, s>>>(d, p, g, fg);
    } else if (pl.mt1 == 1) {
      k_fused<1><<<dim3(2 * d.N), 512, 0, s>>>(d, p, g, fg);
    } else {
      k_fused<2><<<dim3(2 * d.N), 512, 0, s>>>(d, p, g, fg);
    }
    mark(-2);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MLA_OK : MLA_ERR_RUNTIME;
  }
  // with the packed copy, every run stays on kernels that read it (the
  // unpacked weights may be absent)
  if (p.packed) {
    const PackGeo g16 = geo_of(dd);
    const bool f16_pair = dd.float_dtype == MLA_FP16 && pl.stream && c.pair_ok && g16.nope_w == 2 && d.Dr == 64 &&
                          g16.uk_w <= 8;
    if (f16_pair && pl.mt1 == 1) packed_launch_f16<1>(s, d, p, g16, mark);
    else if (f16_pair) packed_launch_f16<2>(s, d, p, g16, mark);
    else if (pl.stream && dd.float_dtype != MLA_FP16) launch_packed(pl, s, d, p, dd, q8, c.pair_ok, mark);
    else launch_tiled(s, d, p, dd, q8, c.pair_ok, mark);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MLA_OK : MLA_ERR_RUNTIME;
  }
  const int tiles_q = ceil_div(d.Hcq, 64);
  const int tiles_kr = ceil_div(d.Hckv + d.Dr, 64);
  dim3 g1(tiles_q + tiles_kr, pl.S, ceil_div(T, 16 * pl.mt1));
  if (i8d) launch_k1<true>(pl.mt1, g1, s, d, p, tiles_q, pl.kps);
  else launch_k1<false>(pl.mt1, g1, s, d, p, tiles_q, pl.kps);
  mark(1);

  if (i8d) launch_norm<true, true>(s, d, p, pl.S, 0);
  else if (i8u) launch_norm<false, true>(s, d, p, pl.S, 0);
  else launch_norm<false, false>(s, d, p, pl.S, 0);
  mark(2);

  const int nope_tiles = ceil_div(d.D, 64);
  dim3 g3(d.N * (nope_tiles + 1), 1, ceil_div(T, 16 * pl.mt3));
  if (i8u) launch_k3<true>(pl.mt3, g3, s, d, p, nope_tiles);
  else launch_k3<false>(pl.mt3, g3, s, d, p, nope_tiles);
  mark(3);

  dim3 g4(d.N, pl.cs4, ceil_div(T, 32));
  if (q8) launch_k4<true>(pl.ntw4, g4, s, d, p);
  else launch_k4<false>(pl.ntw4, g4, s, d, p);
  mark(4);

  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MLA_OK : MLA_ERR_RUNTIME;
}


}  // namespace

extern "C" {

mla_status mla_prolog_run(mla_prolog_t h, const mla_prolog_tensors* t, int64_t T, void* stream) {
  if (!h) return MLA_ERR_NULLPTR;
  const mla_prolog_desc& dd = h->desc;
  mla_status st = check_tensors(&dd, t, T);
  if (st != MLA_OK) return st;
  if (T == 0) return MLA_OK;
  // an earlier run that gave up a bounded wait, once its mark is visible
  // here: nothing more runs until mla_prolog_check has reported it
  if (__atomic_load_n(h->herr, __ATOMIC_ACQUIRE) != 0) return MLA_ERR_RUNTIME;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_RUNTIME;
  if (prev != dd.device && hipSetDevice(dd.device) != hipSuccess) return MLA_ERR_RUNTIME;
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(stream);
  // under HIP graph capture a launch keeps the run number it was captured
  // with, so a replay could take the previous replay's tags and flags for
  // its own: a captured run takes only the kernels that hand no data across
  // blocks (as mla_prolog_run_noalloc), records no profiling events, and
  // cannot do the debugging check of cacheIndex, which waits for the device
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) {
    (void)hipGetLastError();
    cap = hipStreamCaptureStatusNone;
  }
  const bool captured = cap != hipStreamCaptureStatusNone;
  if (captured && dd.check_index) {
    if (prev != dd.device) (void)hipSetDevice(prev);
    return MLA_ERR_PARAM_INVALID;
  }
  if (dd.check_index && dd.block_num > 0) {
    // the debugging check of cacheIndex: every entry in [0, slots)
    st = check_cache_index(t->cache_index, T, dd.block_num * dd.block_size, s);
    if (st != MLA_OK) {
      if (prev != dd.device) (void)hipSetDevice(prev);
      return st;
    }
  }
  RunCtx c;
  c.dd = &dd;
  c.lay = &h->lay;
  c.ws = h->ws;
  c.fused_ok = !captured && h->fused_fit[T <= 16 ? 0 : 1];
  c.pair_ok = !captured;
  // run numbers 1, 2, ...: 0 is what the flags and tags of the workspace
  // start with, so a wrap of the counter skips it.  A run whose launch fails
  // still uses up its number: no flag can hold it.
  if (++h->run_no == 0) h->run_no = 1;
  c.run = h->run_no;
  c.spin = h->spin;
  c.ev = nullptr;
  c.mark_kind = nullptr;
  c.herr = h->herr_dev;
  if (h->events && !captured) {
    c.ev = h->events + (h->recorded % kProfileRing) * kProfileEvents;
    c.mark_kind = h->fused + (h->recorded % kProfileRing);
    ++h->recorded;
  }
  st = enqueue(c, t, T, s);
  if (prev != dd.device) (void)hipSetDevice(prev);
  return st;
}

}  // extern "C"

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
uint8_t* g_scratch[kScratchDevices];   // device address of scratch per device, once looked up

// The device address of `scratch` on the current device `dev` (looked up on
// the first call on that device), or NULL if the lookup fails.
uint8_t* scratch_on(int dev) {
  if (dev < 0 || dev >= kScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = static_cast<uint8_t*>(ptr);
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

mla_status mla_prolog_run_noalloc(const mla_prolog_desc* desc, const mla_prolog_tensors* t, int64_t T,
                                  void* stream) {
  mla_status st = check_desc_core(desc);
  if (st != MLA_OK) return st;
  st = check_tensors(desc, t, T);
  if (st != MLA_OK) return st;
  // the debugging check of cacheIndex needs a host buffer and a wait
  if (desc->check_index) return MLA_ERR_PARAM_INVALID;
  if (T == 0) return MLA_OK;
  // the workspace of this run alone (no regions of the kernels that hand
  // data across blocks) must fit the scratch array
  mla_prolog_desc dT = *desc;
  dT.max_tokens = T;
  const Layout L = layout(dT, part_rows_at(dT, T), false);
  if (L.total > kScratchBytes) return MLA_ERR_PARAM_INVALID;
  if (L.cq - L.part >= size_t(kOOB)) return MLA_ERR_UNSUPPORTED;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_RUNTIME;
  if (prev != desc->device && hipSetDevice(desc->device) != hipSuccess) return MLA_ERR_RUNTIME;
  (void)hipGetLastError();
  uint8_t* const ws = scratch_on(desc->device);
  if (!ws) {
    if (prev != desc->device) (void)hipSetDevice(prev);
    return MLA_ERR_RUNTIME;
  }
  // only kernels that read what earlier kernels of the stream wrote: nothing
  // in the array has to start at zero, and what an earlier call left there
  // is overwritten before it is read
  RunCtx c;
  c.dd = desc;
  c.lay = &L;
  c.ws = ws;
  c.fused_ok = c.pair_ok = false;
  c.run = 0;
  c.spin = 0;
  c.ev = nullptr;
  c.mark_kind = nullptr;
  // (no kernel of these runs waits on another block: the word is never written)
  c.herr = reinterpret_cast<uint32_t*>(ws + L.xflag) + 4 * desc->N;
  st = enqueue(c, t, T, static_cast<hipStream_t>(stream));
  if (prev != desc->device) (void)hipSetDevice(prev);
  return st;
}

static void destroy_events(mla_prolog* h) {
  if (h->events)
    for (int i = 0; i < kProfileRing * kProfileEvents; ++i)
      if (h->events[i]) (void)hipEventDestroy(h->events[i]);
  delete[] h->events;
  delete[] h->fused;
  h->events = nullptr;
  h->fused = nullptr;
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
    h->fused = new (std::nothrow) uint8_t[kProfileRing]();
    if (!h->events || !h->fused) st = MLA_ERR_RUNTIME;
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
    if (h->fused[r] == 2) {   // one kernel, booked to up_proj
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, ev[0], ev[kProfileEvents - 1]) != hipSuccess) return MLA_ERR_RUNTIME;
      kernel_ms[2] += ms;
      continue;
    }
    for (int k = 0; k < kProfileEvents - 1; ++k) {
      if (h->fused[r] && k == kProfileEvents - 2) continue;   // uk ran inside up_proj
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
    if (hipHostFree(h->herr) != hipSuccess) st = MLA_ERR_RUNTIME;
    (void)hipSetDevice(prev);
  }
  delete h;
  return st;
}

mla_status mla_prolog_set_poll_limit(mla_prolog_t h, int32_t steps) {
  if (!h) return MLA_ERR_NULLPTR;
  if (steps < 0 || steps > kFusedSpin) return MLA_ERR_PARAM_INVALID;
  h->spin = steps ? int(steps) : kFusedSpin;
  return MLA_OK;
}

mla_status mla_prolog_check(mla_prolog_t h) {
  if (!h) return MLA_ERR_NULLPTR;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(h->desc.device) != hipSuccess)
    return MLA_ERR_RUNTIME;
  const bool synced = hipDeviceSynchronize() == hipSuccess;
  (void)hipSetDevice(prev);
  // the word is read and cleared, also when the synchronisation failed
  const uint32_t v = __atomic_exchange_n(h->herr, 0u, __ATOMIC_ACQ_REL);
  return synced && v == 0 ? MLA_OK : MLA_ERR_RUNTIME;
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
