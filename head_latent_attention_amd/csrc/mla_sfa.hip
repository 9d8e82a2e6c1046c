// Sparse flash attention, MLA-absorb decode, for MI355X (gfx950): the
// consumer of the MLA prolog's paged caches (aclnnSparseFlashAttention,
// "Function" formula, parameter table, attentionMode 2).
//
// Per token t and head h, over the cache rows t's sparse indices select:
//   s_j = scale [q^N | q^R][t, h] . [c^KV_j | k^R_j],
//   out[t, h] = sum_j softmax(s)_j c^KV_j   (value = key = c^KV).
//
// k_sfa: one block per (token, split of the selected rows, group of 64
// heads); eight waves, two per 16 heads, each wave owning half of the
// output columns (so that a wave's registers hold its heads' queries and
// two waves share each SIMD).  32 selected cache rows at a time are
// gathered into an LDS tile (the next tile's loads in flight in
// registers); each wave takes S = Q K^T on MFMA (queries as A fragments in
// registers, B fragments 16-byte row reads of the tile), the online softmax
// of its heads (both waves of a head group compute the same), and its half
// of O += P V on MFMA, with P through a small per-wave LDS tile and the V
// fragments read from the same row-major tile by transposing LDS reads
// (ds_read_b64_tr_b16: lane i of each 16-lane group receives element i%4 of
// the 8-byte pieces read by lanes 4e + i/4).
// With more than one split, k_sfa_combine merges the splits' normalised
// partial outputs by their (max, sum) pairs in split order.  No atomics: a
// run is deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>

#include "../../include/mla_sfa.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWaves = 8;             // waves per block: 4 groups of 16 heads x 2 column halves
constexpr int kHeads = 64;            // heads per block
constexpr int kRows = 32;             // cache rows per tile
constexpr int kMaxW = 576;            // D + Dr at most
constexpr int kPitch = kMaxW + 8;     // LDS row pitch (bf16): rows 4 banks apart
constexpr int kMaxKS = kMaxW / 32;    // MFMA k-steps of S = Q K^T
constexpr int kMaxDT = 512 / 16 / 2;  // 16-column tiles of O per wave (half of the columns)
constexpr int kPer = 5;               // 16-byte loads per thread per tile: 32 rows in passes of >= 7 rows
constexpr int kMaxRows = 2048;        // selected rows of one block
constexpr int kPPitch = kRows + 8;    // per-wave P tile pitch (bf16)
constexpr float kLazy = 8.0f;         // how far a tile's maximum may pass the softmax reference

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// A barrier that orders LDS only: the tile loop keeps the next tiles'
// global loads in flight across it (a full __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Max and sum over each 16-lane row of the wave with DPP moves (quad
// permutations, then the half-row and row mirrors); every lane of the row
// ends with the result.  Cross-lane shuffles through the LDS crossbar would
// put four round trips per reduction on the tile loop's critical path.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kQuadSwap1>(v));
  v = fmaxf(v, dpp<kQuadSwap2>(v));
  v = fmaxf(v, dpp<kRowHalfMirror>(v));
  return fmaxf(v, dpp<kRowMirror>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kQuadSwap1>(v);
  v += dpp<kQuadSwap2>(v);
  v += dpp<kRowHalfMirror>(v);
  return v + dpp<kRowMirror>(v);
}

struct SfaArgs {
  const uint16_t* q;      // (T, N, D)
  const uint16_t* qr;     // (T, N, Dr)
  const uint16_t* kv;     // slots of kv_row elements
  const uint16_t* kr;     // slots of kr_row elements (kv + D with the concatenated cache)
  const int32_t* idx;     // (T, K)
  const int32_t* table;   // (T, max_blocks)
  const int32_t* lens;    // (T)
  uint16_t* out;          // (T, N, D)
  float* smax;            // (T, N) or NULL
  float* ssum;            // (T, N) or NULL
  float* part_o;          // [T][S][N][D] split outputs, each divided by its own sum
  float* part_ml;         // [T][S][N][2] their (max, sum)
  int T, N, D, Dr, bs, max_blocks, K, sbs, S, rows_per_split, block_num;
  int kv_row, kr_row;
  float scale;
};

__global__ __launch_bounds__(64 * kWaves) void k_sfa(SfaArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t kt[kRows * kPitch];
  // P of a head group (16 heads x the tile's 32 rows), its two halves
  // written by the group's two waves; their row maxima of the tile
  __shared__ __attribute__((aligned(16))) uint16_t pw[kWaves / 2][16 * kPPitch];
  __shared__ float xmax[kWaves][16];
  __shared__ int32_t slots[kMaxRows];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
  // head group of 16 and column half of this wave; the wave also takes the
  // tile's rows 16 dh .. 16 dh + 15 in S = Q K^T
  const int hg = w % 4, dh = w / 4;
  // block -> (token, split) and head group: the head groups of one (token,
  // split) are 8 blocks apart, so they run on the same XCD and share its L2
  const int HB = (a.N + kHeads - 1) / kHeads;
  const int b = blockIdx.x;
  const int flat = (b / (8 * HB)) * 8 + b % 8;
  const int hb = (b / 8) % HB;
  if (flat >= a.T * a.S) return;
  const int t = flat / a.S, s = flat % a.S;
  const int W = a.D + a.Dr, cpr = W / 8;

  // the selected slots of this split (-1: nothing)
  const int R = a.K * a.sbs;
  const int r0 = s * a.rows_per_split, nrows = max(0, min(R, r0 + a.rows_per_split) - r0);
  const int len = a.lens[t];
  for (int r = tid; r < nrows; r += 64 * kWaves) {
    const int rr = r0 + r, e = rr / a.sbs, off = rr % a.sbs;
    const int ix = a.idx[int64_t(t) * a.K + e];
    int slot = -1;
    if (ix >= 0) {
      const int64_t pos = int64_t(ix) * a.sbs + off;
      if (pos < len && pos / a.bs < a.max_blocks) {
        const int blk = a.table[int64_t(t) * a.max_blocks + pos / a.bs];
        if (blk >= 0 && blk < a.block_num) slot = blk * a.bs + int(pos % a.bs);
      }
    }
    slots[r] = slot;
  }
  // the tile's columns from D + Dr to the widest row stay zero (as do the
  // queries'), so the MFMA loops below run over the widest row with no
  // branches (a branch around each step keeps the LDS reads from overlapping)
  for (int q = tid; q < kRows * (kMaxW / 8 - cpr); q += 64 * kWaves) {
    const int n = kMaxW / 8 - cpr, r = q / n, cc = cpr + q % n;
    *reinterpret_cast<uint4*>(&kt[r * kPitch + 8 * cc]) = make_uint4(0, 0, 0, 0);
  }
  // this wave's A fragments of S: head 16hg + c, columns 32ks + 8g .. +7 of
  // [q^N | q^R] (zeros past N and past D + Dr)
  bf16x8 qa[kMaxKS];
  {
    const int h = hb * kHeads + 16 * hg + c;
#pragma unroll
    for (int ks = 0; ks < kMaxKS; ++ks) {
      const int k0 = 32 * ks + 8 * g;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (h < a.N && k0 < W)
        v = k0 < a.D ? *reinterpret_cast<const uint4*>(a.q + (int64_t(t) * a.N + h) * a.D + k0)
                     : *reinterpret_cast<const uint4*>(a.qr + (int64_t(t) * a.N + h) * a.Dr + k0 - a.D);
      __builtin_memcpy(&qa[ks], &v, 16);
    }
  }
  __syncthreads();

  const int ntiles = (nrows + kRows - 1) / kRows;
  uint4 pre[1][kPer];
  // thread -> (16-byte column cc of a row, first row rbase); rows rbase +
  // rstep*i, so the per-tile addressing has no division
  const int rstep = (64 * kWaves) / cpr, cc = tid % cpr, rbase = tid / cpr;
  const bool mover = rbase < rstep;
  const uint16_t* src = 8 * cc < a.D ? a.kv + 8 * cc : a.kr + (8 * cc - a.D);
  const int src_row = 8 * cc < a.D ? a.kv_row : a.kr_row;
  // loads of tile `tile`; rows without a slot read as zeros
  auto issue = [&](uint4 (&buf)[kPer], int tile) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int row = rbase + rstep * i, r = tile * kRows + row;
      buf[i] = make_uint4(0, 0, 0, 0);
      if (mover && row < kRows && tile < ntiles) {
        const int slot = r < nrows ? slots[r] : -1;
        if (slot >= 0) buf[i] = *reinterpret_cast<const uint4*>(src + int64_t(slot) * src_row);
      }
    }
  };
  auto commit = [&](const uint4 (&buf)[kPer]) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int row = rbase + rstep * i;
      if (mover && row < kRows) *reinterpret_cast<uint4*>(&kt[row * kPitch + 8 * cc]) = buf[i];
    }
  };

  f32x4 acc[kMaxDT];
#pragma unroll
  for (int dt = 0; dt < kMaxDT; ++dt) acc[dt] = f32x4{0, 0, 0, 0};
  // m: the reference the exponentials and l are taken against; mt: the
  // running maximum itself
  float m[4], mt[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m[i] = -INFINITY; mt[i] = -INFINITY; l[i] = 0.0f; }
  uint16_t* pwr = pw[hg];

  auto step = [&](int tile) {
    // S = Q K^T for this wave's 16-row half of the tile, in two accumulator
    // chains (even and odd k-steps) so that consecutive MFMAs do not wait
    // for each other, added at the end
    f32x4 s2[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
    for (int ks = 0; ks < kMaxKS; ++ks) {
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&kt[(16 * dh + c) * kPitch + 32 * ks + 8 * g]);
      s2[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb, s2[ks & 1], 0, 0, 0);
    }
    const f32x4 sacc = s2[0] + s2[1];
    // sacc[i]: head 4g+i of the wave, row 16 dh + c of the tile
    const int r = tile * kRows + 16 * dh + c;
    const bool ok = r < nrows && slots[r] >= 0;
    float sv[4], mh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = ok ? sacc[i] * a.scale : -INFINITY;
      mh[i] = row16_max(sv[i]);
      if (c == 0) xmax[w][4 * g + i] = mh[i];
    }
    // the tile's row maximum of each head takes both halves: the partner's
    // (the other column half of the head group) through LDS
    lds_barrier();
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mx = fmaxf(mh[i], xmax[w ^ 4][4 * g + i]);
      mt[i] = fmaxf(mt[i], mx);
      // the reference moves only when the tile's maximum passes it by more
      // than kLazy, so P stays below e^kLazy and O is rescaled about once per
      // row (softmax does not depend on the reference; the sum is referred
      // to the true maximum at the end)
      const float mn = mx > m[i] + kLazy ? mx : m[i];
      const bool none = mn == -INFINITY;
      alpha[i] = none ? 1.0f : __expf(m[i] - mn);
      const float pv = none ? 0.0f : __expf(sv[i] - mn);
      // this half's sum; both waves of the group scale theirs by the same
      // alpha, so the two sums add up at the end
      l[i] = l[i] * alpha[i] + row16_sum(pv);
      m[i] = mn;
      pwr[(4 * g + i) * kPPitch + 16 * dh + c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(pv));
    }
    // rescale O only when a running max of the wave moved (once the maxima
    // settle, most tiles leave them alone)
    if (__any(alpha[0] != 1.0f || alpha[1] != 1.0f || alpha[2] != 1.0f || alpha[3] != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < kMaxDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[dt][i] *= alpha[i];
    }
    // P (both halves) is read back by the lanes of both waves
    lds_barrier();
    const bf16x8 pa = *reinterpret_cast<const bf16x8*>(&pwr[c * kPPitch + 8 * g]);   // head c, rows 8g..
    // O += P V over this wave's column half: the B fragment (rows 8g..8g+7,
    // column 256dh + 16dt + c) from two transposing reads of 4 rows x 4
    // columns pieces of the row-major tile
    const int vr = 8 * g + c / 4, vc = 256 * dh + 4 * (c % 4);
    lds_char* kbase = (lds_char*)(kt);
    // (columns past D land in tiles that are never stored)
#pragma unroll
    for (int dt = 0; dt < kMaxDT; ++dt) {
      const int o0 = (vr * kPitch + 16 * dt + vc) * 2, o1 = o0 + 4 * kPitch * 2;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(kbase + o0));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(kbase + o1));
      const v4i16 vv[2] = {lo, hi};
      bf16x8 vb;
      __builtin_memcpy(&vb, vv, 16);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, acc[dt], 0, 0, 0);
    }
  };

  // the next tile's loads in flight while a tile is computed
  issue(pre[0], 0);
  for (int tile = 0; tile < ntiles; ++tile) {
    commit(pre[0]);
    lds_barrier();
    issue(pre[0], tile + 1);
    step(tile);
    lds_barrier();
  }

  // each wave holds the sum over its half of the rows: add the partner's
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (c == 0) xmax[w][4 * g + i] = l[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) l[i] += xmax[w ^ 4][4 * g + i];

  // this split's result, per head row 4g+i of the wave, its column half
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = hb * kHeads + 16 * hg + 4 * g + i;
    if (h >= a.N) continue;
    const float inv = l[i] > 0.0f ? 1.0f / l[i] : 0.0f;
    const float sum = mt[i] == -INFINITY ? 0.0f : l[i] * __expf(m[i] - mt[i]);
    if (a.S == 1) {
      uint16_t* o = a.out + (int64_t(t) * a.N + h) * a.D + 256 * dh;
#pragma unroll
      for (int dt = 0; dt < kMaxDT; ++dt)
        if (256 * dh + 16 * dt < a.D) o[16 * dt + c] = f2bf(acc[dt][i] * inv);
      if (c == 0 && dh == 0) {
        if (a.smax) a.smax[int64_t(t) * a.N + h] = mt[i];
        if (a.ssum) a.ssum[int64_t(t) * a.N + h] = sum;
      }
    } else {
      const int64_t row = (int64_t(t) * a.S + s) * a.N + h;
      float* o = a.part_o + row * a.D + 256 * dh;
#pragma unroll
      for (int dt = 0; dt < kMaxDT; ++dt)
        if (256 * dh + 16 * dt < a.D) o[16 * dt + c] = acc[dt][i] * inv;
      if (c == 0 && dh == 0) { a.part_ml[2 * row] = mt[i]; a.part_ml[2 * row + 1] = sum; }
    }
  }
}

// Merges the S splits of (token, head) rows: with M = max_s m_s and
// w_s = l_s exp(m_s - M), out = sum_s w_s o_s / sum_s w_s, softmax_max = M,
// softmax_sum = sum_s w_s, the splits taken in order.  One wave per row,
// eight columns per lane.
__global__ __launch_bounds__(256) void k_sfa_combine(SfaArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.T * a.N) return;
  const int t = row / a.N, h = row % a.N;
  float M = -INFINITY;
  for (int s = 0; s < a.S; ++s) M = fmaxf(M, a.part_ml[2 * ((int64_t(t) * a.S + s) * a.N + h)]);
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0}, W = 0.0f;
  const bool mine = 8 * lane < a.D;   // D is a multiple of 32: whole 8-column pieces
  if (M != -INFINITY) {
    for (int s = 0; s < a.S; ++s) {
      const int64_t pr = (int64_t(t) * a.S + s) * a.N + h;
      const float ms = a.part_ml[2 * pr], ls = a.part_ml[2 * pr + 1];
      if (ms == -INFINITY) continue;
      const float ws = ls * __expf(ms - M);
      W += ws;
      if (mine) {
        const float4* src = reinterpret_cast<const float4*>(a.part_o + pr * a.D + 8 * lane);
        const float4 u = src[0], v = src[1];
        o[0] += ws * u.x; o[1] += ws * u.y; o[2] += ws * u.z; o[3] += ws * u.w;
        o[4] += ws * v.x; o[5] += ws * v.y; o[6] += ws * v.z; o[7] += ws * v.w;
      }
    }
  }
  const float inv = W > 0.0f ? 1.0f / W : 0.0f;
  if (mine) {
    uint32_t pk[4];
    for (int e = 0; e < 4; ++e)
      pk[e] = uint32_t(f2bf(o[2 * e] * inv)) | (uint32_t(f2bf(o[2 * e + 1] * inv)) << 16);
    *reinterpret_cast<uint4*>(a.out + (int64_t(t) * a.N + h) * a.D + 8 * lane) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
  if (lane == 0) {
    if (a.smax) a.smax[int64_t(t) * a.N + h] = M;
    if (a.ssum) a.ssum[int64_t(t) * a.N + h] = W;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// splits of the selected rows: about one block per CU (a block's eight
// waves at up to 256 VGPRs fill a CU; at 32 tokens and 128 heads, 4 splits
// of 512 rows ran 80 us per step against 96 for 8 splits and 122 for 2), at
// most kMaxRows rows and at least one tile per split
int splits_for(const mla_sfa_desc& d, int64_t T) {
  const int64_t R = d.sparse_size * d.sparse_block_size;
  const int64_t HB = (d.N + kHeads - 1) / kHeads;
  int64_t S = std::max<int64_t>(1, 256 / std::max<int64_t>(1, T * HB));
  S = std::min<int64_t>(S, (R + kRows - 1) / kRows);
  S = std::max<int64_t>(S, (R + kMaxRows - 1) / kMaxRows);
  return int(S);
}

int64_t max_splits(const mla_sfa_desc& d) {
  int64_t best = 1;
  for (int64_t T = 1; T <= d.max_tokens; T = T < 16 ? T + 1 : T * 2) best = std::max<int64_t>(best, splits_for(d, T));
  return std::max<int64_t>(best, splits_for(d, d.max_tokens));
}

mla_status check_desc(const mla_sfa_desc* d) {
  if (!d) return MLA_ERR_NULLPTR;
  if (d->N <= 0 || d->D <= 0 || d->Dr <= 0 || d->block_num < 0 || d->block_size <= 0 || d->max_blocks <= 0 ||
      d->sparse_size <= 0 || d->sparse_block_size <= 0 || d->max_tokens < 0 || d->max_tokens > (1 << 20) ||
      (d->concat != 0 && d->concat != 1) || !std::isfinite(d->scale))
    return MLA_ERR_PARAM_INVALID;
  if (d->D % 32 || d->D > 512 || d->Dr % 32 || d->D + d->Dr > kMaxW || d->N > 128) return MLA_ERR_UNSUPPORTED;
  if (d->block_num * d->block_size >= (int64_t(1) << 31) || d->max_blocks > (1 << 24) ||
      d->sparse_size * d->sparse_block_size > (int64_t(1) << 24) || d->block_size > (1 << 20))
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

mla_status check_tensors(const mla_sfa_desc* d, const mla_sfa_tensors* t, int64_t T) {
  if (T < 0 || T > d->max_tokens) return MLA_ERR_PARAM_INVALID;
  if (!t) return MLA_ERR_NULLPTR;
  if (T == 0) return MLA_OK;
  const void* req[] = {t->query, t->query_rope, t->kv_cache, t->sparse_indices, t->block_table, t->seq_lens_kv,
                       t->attention_out};
  for (const void* q : req)
    if (!q) return MLA_ERR_NULLPTR;
  for (const void* q : req)
    if (!aligned16(q)) return MLA_ERR_PARAM_INVALID;
  if (d->concat ? t->kr_cache != nullptr : t->kr_cache == nullptr)
    return d->concat ? MLA_ERR_PARAM_INVALID : MLA_ERR_NULLPTR;
  if (t->kr_cache && !aligned16(t->kr_cache)) return MLA_ERR_PARAM_INVALID;
  if ((t->softmax_max && (reinterpret_cast<uintptr_t>(t->softmax_max) & 3u)) ||
      (t->softmax_sum && (reinterpret_cast<uintptr_t>(t->softmax_sum) & 3u)))
    return MLA_ERR_PARAM_INVALID;
  return MLA_OK;
}

}  // namespace

struct mla_sfa {
  mla_sfa_desc desc;
  int64_t max_s;
  float* part_o;
  float* part_ml;
};

extern "C" {

mla_status mla_sfa_validate(const mla_sfa_desc* desc, const mla_sfa_tensors* tensors, int64_t T) {
  mla_status st = check_desc(desc);
  if (st != MLA_OK || !tensors) return st;
  return check_tensors(desc, tensors, T);
}

mla_status mla_sfa_create(const mla_sfa_desc* desc, mla_sfa_t* out) {
  if (!out) return MLA_ERR_NULLPTR;
  *out = nullptr;
  mla_status st = check_desc(desc);
  if (st != MLA_OK) return st;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_RUNTIME;
  if (hipSetDevice(desc->device) != hipSuccess) return MLA_ERR_PARAM_INVALID;
  mla_sfa* h = new (std::nothrow) mla_sfa;
  if (!h) { (void)hipSetDevice(prev); return MLA_ERR_RUNTIME; }
  h->desc = *desc;
  h->max_s = max_splits(*desc);
  h->part_o = nullptr;
  h->part_ml = nullptr;
  const size_t rows = size_t(std::max<int64_t>(1, desc->max_tokens)) * size_t(h->max_s) * size_t(desc->N);
  if (h->max_s > 1 && (hipMalloc(&h->part_o, rows * desc->D * 4) != hipSuccess ||
                       hipMalloc(&h->part_ml, rows * 2 * 4) != hipSuccess)) {
    (void)hipFree(h->part_o);
    delete h;
    (void)hipSetDevice(prev);
    return MLA_ERR_RUNTIME;
  }
  (void)hipSetDevice(prev);
  *out = h;
  return MLA_OK;
}

mla_status mla_sfa_run(mla_sfa_t h, const mla_sfa_tensors* t, int64_t T, void* stream) {
  if (!h) return MLA_ERR_NULLPTR;
  const mla_sfa_desc& d = h->desc;
  mla_status st = check_tensors(&d, t, T);
  if (st != MLA_OK) return st;
  if (T == 0) return MLA_OK;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return MLA_ERR_RUNTIME;
  if (prev != d.device && hipSetDevice(d.device) != hipSuccess) return MLA_ERR_RUNTIME;
  (void)hipGetLastError();
  SfaArgs a;
  a.q = static_cast<const uint16_t*>(t->query);
  a.qr = static_cast<const uint16_t*>(t->query_rope);
  a.kv = static_cast<const uint16_t*>(t->kv_cache);
  a.kv_row = int(d.concat ? d.D + d.Dr : d.D);
  a.kr = d.concat ? a.kv + d.D : static_cast<const uint16_t*>(t->kr_cache);
  a.kr_row = int(d.concat ? d.D + d.Dr : d.Dr);
  a.idx = t->sparse_indices;
  a.table = t->block_table;
  a.lens = t->seq_lens_kv;
  a.out = static_cast<uint16_t*>(t->attention_out);
  a.smax = t->softmax_max;
  a.ssum = t->softmax_sum;
  a.part_o = h->part_o;
  a.part_ml = h->part_ml;
  a.T = int(T); a.N = int(d.N); a.D = int(d.D); a.Dr = int(d.Dr); a.bs = int(d.block_size);
  a.max_blocks = int(d.max_blocks); a.K = int(d.sparse_size); a.sbs = int(d.sparse_block_size);
  a.block_num = int(d.block_num);
  a.scale = float(d.scale);
  const int64_t R = d.sparse_size * d.sparse_block_size;
  a.S = splits_for(d, T);
  a.rows_per_split = int((R + a.S - 1) / a.S);
  const int HB = int((d.N + kHeads - 1) / kHeads);
  const int64_t flats = T * a.S;
  const dim3 grid(unsigned(((flats + 7) / 8) * 8 * HB));
  hipStream_t s = static_cast<hipStream_t>(stream);
  k_sfa<<<grid, 64 * kWaves, 0, s>>>(a);
  if (a.S > 1) k_sfa_combine<<<dim3(unsigned((T * d.N + 3) / 4)), 256, 0, s>>>(a);
  const hipError_t e = hipGetLastError();
  if (prev != d.device) (void)hipSetDevice(prev);
  return e == hipSuccess ? MLA_OK : MLA_ERR_RUNTIME;
}

mla_status mla_sfa_destroy(mla_sfa_t h) {
  if (!h) return MLA_ERR_NULLPTR;
  int prev = 0;
  mla_status st = MLA_OK;
  if (hipGetDevice(&prev) != hipSuccess) st = MLA_ERR_RUNTIME;
  if (st == MLA_OK && hipSetDevice(h->desc.device) == hipSuccess) {
    if (hipDeviceSynchronize() != hipSuccess) st = MLA_ERR_RUNTIME;
    if (h->part_o && hipFree(h->part_o) != hipSuccess) st = MLA_ERR_RUNTIME;
    if (h->part_ml && hipFree(h->part_ml) != hipSuccess) st = MLA_ERR_RUNTIME;
    (void)hipSetDevice(prev);
  }
  delete h;
  return st;
}

}  // extern "C"
