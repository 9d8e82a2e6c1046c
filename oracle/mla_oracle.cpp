// Plain, slow CPU oracle of the Multi-Head Latent Attention (MLA) prolog.
//
// TEST INFRASTRUCTURE ONLY.  The HIP library never links, loads or calls this
// file; only the tests, the smoke check and the benchmark's CPU-baseline leg
// do.  It shares no code, header, table or helper with the HIP path.
//
// What it computes is the formula block of the MLA prolog operator page
// (aclnnMlaPrologV2WeightNz, "Function", formulas), per token t:
//
//   c^Q  = RmsNorm(x W^DQ)                      (query down-projection + norm)
//   q^C  = c^Q W^UQ,   q^N = q^C W^UK  per head (the two up-projections)
//   q^R  = ROPE(c^Q W^QR)                       (query rotary part)
//   c^KV = RmsNorm(x W^DKV)  -> kvCache[cacheIndex[t]]
//   k^R  = ROPE(x W^KR)      -> krCache[cacheIndex[t]]
//   optional: dequantScaleQNope = RowMax(|q^N|)/127, q^N = round(q^N/scale)
//
// RmsNorm(v)_i = gamma_i v_i / sqrt((1/n) sum_j v_j^2 + eps), eps inside the
// root and n the vector length (same page, "RmsNorm formula").  RoPE is the
// rotate-half form, the only mode the MLA preprocess page (aclnnMlaPreprocess,
// constraints, rope mode) supports: pairs (i, i + Dr/2) with one cos/sin
// table entry per element.
//
// Arithmetic is double.  In the int8 full-quantisation scenario (same page,
// scenario and dtype tables) the integer products are summed exactly in
// int64 and dequantised as acc * scaleX[t] * scaleW[n].  A value is rounded
// exactly where the operator stores it as a tensor or feeds it to a bf16/int8
// matrix product (the readings R1..R7):
//   R1 kvCache row = bf16(c^KV)          R2 krCache row = bf16(k^R)
//   R3 bf16 operand bf16(c^Q)            R3' int8 operand: per-token dynamic
//                                            int8 of c^Q (times the optional
//                                            smoothScalesCq), decided in float32
//   R4 queryRopeOut = bf16(q^R)          R5 W^UK operand bf16(q^C)
//   R6 queryOut = bf16(q^N)              R7 int8 queryOut: per-(token, head)
//                                            dynamic int8, decided in float32
// round_intermediates = 0 skips R3 and R5 (used by the composition pin).
//
// KV-cache quantisation (same page: quantScaleCkv / quantScaleCkr and the
// "kv_cache quantized" columns of the scenario and dtype tables) replaces R1
// and R2 by static int8 codes (R1', R2'): the value times its channel's
// scale, rounded half to even and saturated to [-128, 127], decided in
// float32.  The page gives the scales' shapes and scenarios but no formula;
// multiplying is the reading taken (the preprocess page's quantising norm
// multiplies by its scale).  Full quantisation quantises the kv cache only;
// partial quantisation quantises both caches.
//
// The partial-quantisation scenario (same page, scenario table) takes tokenX,
// weightDq and weightDkvKr in bf16 and only weightUqQr in int8, with its
// per-channel dequantisation scale; the up-projection then runs on R3' as in
// full quantisation.  smoothScalesCq (1, Hcq), optional in both int8
// scenarios, multiplies c^Q element-wise before R3' decides the codes (the
// page's parameter table: a parameter of the dynamic quantisation of the
// RmsNorm output).  The product is not divided back: the caller's int8
// weightUqQr carries the inverse smoothing, as is usual for smoothing
// factors.  Here c^Q * m is formed as RmsNorm with gamma * m for its weight:
// gamma (bf16) times m (fp32) is exact in double, and the result is the
// same real number, so only the double-rounding order is a choice (the one
// the device uses, so that both take the same int8 decisions).
//
// The static scenario follows the MLA preprocess page (aclnnMlaPreprocess,
// "Function" formulas and parameter table, quantMode 0: per-tensor static
// asymmetric int8).  Its RmsNormQuant is read as
//   code = saturate[-128, 127](round-half-even(f32(v) * scale) + offset),
//   v = gamma * x / RMS(x) + beta,
// with the scale (quantScale, one value) multiplying as the page's formula
// writes it and the int8 offset (quantOffset) added to the rounded product;
// the code is decided in float32.  It is applied to the bf16 input x (gamma0,
// beta0, quantScale0, quantOffset0; without the norm when doRmsNorm is false:
// v = x) and to y_q (gamma1, beta1, quantScale1, quantOffset1).  The products
// with the int8 weights are exact integer sums, biased and dequantised per
// output channel: y = (acc + bias[n]) * deScale[n].  c^KV is the plain
// RmsNorm of y_kv with gamma2.  The page's cacheMode 0 concatenates the
// outputs: each queryOut row holds q^N then q^R (Hckv + Dr values) and each
// kvCache row c^KV then k^R; its weights come transposed, (n, k) row-major.
// Its FLOAT16 input (the parameter table gives x, gamma0/beta0/quantScale0,
// the other gammas and betas, sin/cos and wuk as FLOAT16 or BFLOAT16, and
// the caches and query outputs in the dtype of the input) makes every 16-bit
// float of the problem an IEEE binary16 value, and R1, R2, R4, R5 and R6 fp16
// roundings.
//
// The consumer of the caches, mla_oracle_sfa, is the sparse flash attention
// page (aclnnSparseFlashAttention, "Function" formula, parameter table,
// attentionMode 2 = MLA-absorb) for one query per batch (decode): per token
// t and head h, over the cache rows its sparse indices select (index i
// selects positions i*sparseBlockSize .. +sparseBlockSize-1, those below the
// batch's kv length, mapped to slots through its block table; negative
// indices select nothing),
//   s_j = scaleValue * ([q^N | q^R] . [c^KV_j | k^R_j]),
//   out = sum_j softmax(s)_j c^KV_j,
// softmaxMax = max_j s_j and softmaxSum = sum_j exp(s_j - max).  A token
// with no selected row gets out = 0, max = -inf, sum = 0.  Double
// arithmetic, out rounded to bf16 once.
//
// Every function here is pinned by the CPU tests (closed forms, invariants,
// special cases, brute force on tiny shapes, planted mistakes); none is
// unpinned.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// bf16 codec.  bf16 is the upper half of an IEEE-754 binary32 word: 1 sign
// bit, 8 exponent bits (bias 127), 7 stored fraction bits.
// ---------------------------------------------------------------------------
double bf16_value(uint16_t bits) {
  uint32_t w = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &w, sizeof f);
  return static_cast<double>(f);
}

// Nearest bf16 to v, ties to even, computed from v directly (no detour
// through binary32, which could round twice).  The spacing of bf16 values
// near |v| in [2^e, 2^(e+1)) is 2^(e-7), and 2^-133 below 2^-126.
uint16_t bf16_bits(double v) {
  if (std::isnan(v)) return 0x7FC0;
  const double kMax = (2.0 - std::ldexp(1.0, -7)) * std::ldexp(1.0, 127);
  uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  double a = std::fabs(v);
  if (std::isinf(a)) return sign | 0x7F80;
  if (a == 0.0) return sign;
  int e = std::ilogb(a);
  if (e < -126) e = -126;
  double r = std::ldexp(std::nearbyint(std::ldexp(a, 7 - e)), e - 7);  // RNE
  if (r > kMax) return sign | 0x7F80;
  float f = static_cast<float>(r);  // exact: r is a bf16 value
  uint32_t w;
  std::memcpy(&w, &f, sizeof w);
  return sign | static_cast<uint16_t>(w >> 16);
}

double bf16_round(double v) { return bf16_value(bf16_bits(v)); }

// ---------------------------------------------------------------------------
// fp16 codec (IEEE-754 binary16): 1 sign bit, 5 exponent bits (bias 15), 10
// stored fraction bits; exponent field 0 holds the subnormals f * 2^-24, 31
// the infinities and NaNs.
// ---------------------------------------------------------------------------
double f16_value(uint16_t bits) {
  const int sign = bits >> 15, ex = (bits >> 10) & 0x1F, fr = bits & 0x3FF;
  double v;
  if (ex == 0) v = std::ldexp(static_cast<double>(fr), -24);
  else if (ex == 31) v = fr ? NAN : INFINITY;
  else v = std::ldexp(static_cast<double>(1024 + fr), ex - 25);
  return sign ? -v : v;
}

// Nearest fp16 to v, ties to even, computed from v directly.  The spacing of
// fp16 values near |v| in [2^e, 2^(e+1)) is 2^(e-10), and 2^-24 below 2^-14;
// what rounds above the largest finite value, 65504, is infinite.
uint16_t f16_bits(double v) {
  if (std::isnan(v)) return 0x7E00;
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  const double a = std::fabs(v);
  if (std::isinf(a)) return sign | 0x7C00;
  if (a == 0.0) return sign;
  int e = std::ilogb(a);
  if (e < -14) e = -14;
  const double r = std::ldexp(std::nearbyint(std::ldexp(a, 10 - e)), e - 10);  // RNE
  if (r > 65504.0) return sign | 0x7C00;
  if (r < std::ldexp(1.0, -14))  // subnormal (or zero): the fraction counts 2^-24
    return sign | static_cast<uint16_t>(std::ldexp(r, 24));
  const int er = std::ilogb(r);   // the rounding may have carried into the next binade
  const int fr = static_cast<int>(std::ldexp(r, 10 - er)) - 1024;
  return sign | static_cast<uint16_t>(((er + 15) << 10) | fr);
}

double f16_round(double v) { return f16_value(f16_bits(v)); }

// RmsNorm over n values (aclnnMlaPrologV2WeightNz, "RmsNorm formula").
void rmsnorm(const double* v, const double* gamma, int64_t n, double eps, double* out,
             int mutation) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += v[i] * v[i];
  double ms = ss / static_cast<double>(n);
  double rms = std::sqrt(ms + eps);
  if (mutation == 2) rms = std::sqrt(ms) + eps;  // planted: eps outside the root
  for (int64_t i = 0; i < n; ++i) {
    double g = (mutation == 5) ? 1.0 : gamma[i];  // planted: gamma dropped
    out[i] = g * v[i] / rms;
  }
}

// Rotate-half RoPE of one vector of length Dr:
//   out_i     = v_i     cos_i     - v_{i+h} sin_i
//   out_{i+h} = v_{i+h} cos_{i+h} + v_i     sin_{i+h}        (h = Dr/2)
void rope(const double* v, const double* cos, const double* sin, int64_t Dr, double* out,
          int mutation) {
  int64_t h = Dr / 2;
  double s = (mutation == 1) ? -1.0 : 1.0;  // planted: rotation sign flipped
  for (int64_t i = 0; i < h; ++i) {
    out[i] = v[i] * cos[i] - s * v[i + h] * sin[i];
    out[i + h] = v[i + h] * cos[i + h] + s * v[i] * sin[i + h];
  }
}

// Symmetric dynamic int8 of one row, decided in float32:
//   scale = RowMax(|v|)/127,  q = round(v/scale) ties to even, within [-127, 127]
// (aclnnMlaPrologV2WeightNz, "Dequant Scale Query Nope calculation formula").
// A row of zeros gets scale 0 and q = 0.
void quant_int8(const double* v, int64_t n, int8_t* q, float* scale) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) amax = std::max(amax, std::fabs(static_cast<float>(v[i])));
  float s = amax / 127.0f;
  *scale = s;
  for (int64_t i = 0; i < n; ++i) {
    if (s == 0.0f) { q[i] = 0; continue; }
    float r = std::nearbyint(static_cast<float>(v[i]) / s);
    r = std::min(127.0f, std::max(-127.0f, r));
    q[i] = static_cast<int8_t>(r);
  }
}

// Static asymmetric int8 code of the preprocess page's RmsNormQuant:
// round-half-even(v * scale) + offset, saturated to [-128, 127], decided in
// float32.
int8_t quant_static_asym(double v, float scale, int offset, int mutation) {
  const float f = static_cast<float>(v);
  float r = std::nearbyint(f * scale);
  if (mutation != 9) r += static_cast<float>(offset);  // planted 9: offset ignored
  r = std::min(127.0f, std::max(-128.0f, r));
  return static_cast<int8_t>(r);
}

// Static int8 code of v with a given scale (R1', R2'): v times the scale,
// rounded half to even, saturated to [-128, 127], decided in float32.
int8_t quant_static(double v, float scale, int mutation) {
  const float f = static_cast<float>(v);
  float r = std::nearbyint(mutation == 8 ? f / scale : f * scale);  // planted 8: divided
  r = std::min(127.0f, std::max(-128.0f, r));
  return static_cast<int8_t>(r);
}

}  // namespace

extern "C" {

// One problem: dims, attributes, host tensors.  Layouts are those of the
// operator's parameter table: tokenX (T, He); weightDq (He, Hcq);
// weightUqQr (Hcq, N*(D+Dr)); weightUk (N, D, Hckv); weightDkvKr
// (He, Hckv+Dr); gammas (Hcq), (Hckv); ropeSin/ropeCos (T, Dr); cacheIndex
// (T) int64; caches (BlockNum, BlockSize, 1, Hckv|Dr).  All weights are
// (k, n) row-major.  weightUqQr columns are head-interleaved: column
// h*(D+Dr)+j is W^UQ column h*D+j for j < D and W^QR column h*Dr+j-D
// otherwise.  weightDkvKr holds W^DKV in columns [0, Hckv), W^KR after.
typedef struct {
  int64_t T, He, Hcq, Hckv, N, D, Dr;
  int64_t block_num, block_size;
  double eps_cq, eps_ckv;
  int32_t quant_in;             // 1: int8 x, W^DQ, W^UqQr, W^DkvKr + fp32 scales
  int32_t query_int8;           // 1: q^N as int8 + per-(token, head) scale
  int32_t round_intermediates;  // 0: skip R3 and R5
  int32_t mutation;             // planted mistake for the pin tests, 0 = none
  int32_t quant_uq;             // 1: int8 W^UqQr + fp32 scale and R3' (implied by quant_in)
  int32_t pad_;
  const void* x;                // uint16 bf16 bits, or int8
  const void* w_dq;
  const void* w_uq_qr;
  const uint16_t* w_uk;
  const void* w_dkv_kr;
  const uint16_t* gamma_cq;
  const uint16_t* gamma_ckv;
  const uint16_t* rope_sin;
  const uint16_t* rope_cos;
  const int64_t* cache_index;
  void* kv_cache;               // updated in place (bf16 bits, or int8); NULL = no cache writes
  void* kr_cache;
  const float* scale_x;         // (T)
  const float* scale_w_dq;      // (Hcq)
  const float* scale_w_uq_qr;   // (N*(D+Dr))
  const float* scale_w_dkv_kr;  // (Hckv+Dr)
  const float* smooth_cq;       // (Hcq) smoothScalesCq, int8 W^UqQr only; NULL = none
  const int64_t* tokens;        // rows to compute; NULL = 0..T-1
  int64_t n_tokens;
  // outputs, row r of each holds token tokens[r]
  void* query_out;              // (n, N, Hckv) bf16 bits or int8
  uint16_t* query_rope_out;     // (n, N, Dr)
  float* dequant_scale_q_nope;  // (n, N), int8 query only
  void* kv_rows;                // optional (n, Hckv): the row written to kvCache (bf16 bits or int8)
  void* kr_rows;                // optional (n, Dr)
  double* y_out;                // optional (n, Hcq+Hckv+Dr): x W^DQ | x W^DKV | x W^KR
  double* cq_out;               // optional (n, Hcq): c^Q before rounding
  double* u_out;                // optional (n, N*(D+Dr)): c^Q W^UqQr
  double* qn_out;               // optional (n, N, Hckv): q^N before rounding
  int32_t kv_int8;              // 1: kvCache rows are R1' codes with quant_scale_ckv
  int32_t kr_int8;              // 1: krCache rows are R2' codes with quant_scale_ckr
  const float* quant_scale_ckv; // (Hckv)
  const float* quant_scale_ckr; // (Dr)
  double* ckv_out;              // optional (n, Hckv): c^KV before rounding
  double* kr_out;               // optional (n, Dr): k^R before rounding
  // the preprocess page's static scenario (see the file header)
  int32_t static_quant;         // 1: bf16 x quantised here; int8 W^DQ, W^UqQr, W^DkvKr
  int32_t x_norm;               // static only: 1 = RmsNormQuant of x, 0 = quantise x as is
  int32_t concat;               // 1: queryOut (n, N, Hckv+Dr) and kvCache rows Hckv+Dr; kr unused
  int32_t weight_nk;            // 1: W^DQ (Hcq, He), W^DkvKr (Hckv+Dr, He), W^UqQr (N*(D+Dr), Hcq)
  double eps_x;                 // the RmsNorm of x
  const uint16_t* gamma_x;      // (He) gamma0
  const uint16_t* beta_x;       // (He) beta0
  const uint16_t* quant_scale_x;   // (1) quantScale0, bf16
  const int8_t* quant_offset_x;    // (1) quantOffset0
  const int32_t* bias_dqkv;        // (Hcq+Hckv+Dr) bias0, or NULL for zeros
  const uint16_t* beta_cq;         // (Hcq) beta1
  const uint16_t* quant_scale_cq;  // (1) quantScale1, bf16
  const int8_t* quant_offset_cq;   // (1) quantOffset1
  const int32_t* bias_uq_qr;       // (N*(D+Dr)) bias1, or NULL for zeros
  // static scenario only: every 16-bit float tensor (x, gamma0/beta0/
  // quantScale0, gamma1/beta1/quantScale1, gamma2, sin/cos, W^UK, the caches
  // and the query outputs) is fp16 instead of bf16, and so are the rounding
  // points R1, R2, R4, R5, R6 (the preprocess page's FLOAT16 input)
  int32_t fp16;
  int32_t pad2_;
} mla_oracle_problem;

double mla_oracle_bf16_value(uint16_t bits) { return bf16_value(bits); }
uint16_t mla_oracle_bf16_bits(double v) { return bf16_bits(v); }
double mla_oracle_f16_value(uint16_t bits) { return f16_value(bits); }
uint16_t mla_oracle_f16_bits(double v) { return f16_bits(v); }

void mla_oracle_rmsnorm(const double* v, const double* gamma, int64_t n, double eps,
                        double* out) {
  rmsnorm(v, gamma, n, eps, out, 0);
}

void mla_oracle_rope(const double* v, const double* cos, const double* sin, int64_t Dr,
                     double* out) {
  rope(v, cos, sin, Dr, out, 0);
}

void mla_oracle_quant_int8(const double* v, int64_t n, int8_t* q, float* scale) {
  quant_int8(v, n, q, scale);
}

void mla_oracle_quant_static_asym(const double* v, int64_t n, float scale, int offset, int8_t* q) {
  for (int64_t i = 0; i < n; ++i) q[i] = quant_static_asym(v[i], scale, offset, 0);
}

static double load(const void* base, int64_t i, int32_t is_int8) {
  if (is_int8) return static_cast<double>(static_cast<const int8_t*>(base)[i]);
  return bf16_value(static_cast<const uint16_t*>(base)[i]);
}

// Element (k, n) of a weight with K rows of reduction and Nc output columns:
// stored (k, n) row-major, or (n, k) with weight_nk.
static int64_t widx(const mla_oracle_problem* p, int64_t k, int64_t n, int64_t K, int64_t Nc) {
  return p->weight_nk ? n * K + k : k * Nc + n;
}

// The whole prolog for row r (token t) of the problem.
static void one_token(const mla_oracle_problem* p, int64_t r, int64_t t) {
  const int64_t He = p->He, Hcq = p->Hcq, Hckv = p->Hckv, N = p->N, D = p->D, Dr = p->Dr;
  const int64_t Wkr = Hckv + Dr, Wuq = N * (D + Dr);
  const int32_t q8in = p->quant_in;
  const int mut = p->mutation;
  // the 16-bit float format of the problem's float tensors and roundings
  const bool h16 = p->fp16 != 0;
  auto fval = [h16](uint16_t b) { return h16 ? f16_value(b) : bf16_value(b); };
  auto fbits = [h16](double v) { return h16 ? f16_bits(v) : bf16_bits(v); };
  auto fround = [h16](double v) { return h16 ? f16_round(v) : bf16_round(v); };

  // down-projections: y_q = x W^DQ (Hcq), y_kvr = x [W^DKV | W^KR] (Hckv+Dr)
  std::vector<double> y_q(Hcq, 0.0), y_kvr(Wkr, 0.0);
  if (p->static_quant) {
    // x to int8 codes: RmsNormQuant(x) = code(gamma0 x / RMS(x) + beta0)
    std::vector<double> xv(He), v(He), g0(He);
    for (int64_t k = 0; k < He; ++k) xv[k] = fval(static_cast<const uint16_t*>(p->x)[t * He + k]);
    if (p->x_norm) {
      for (int64_t k = 0; k < He; ++k) g0[k] = fval(p->gamma_x[k]);
      rmsnorm(xv.data(), g0.data(), He, p->eps_x, v.data(), mut);
      for (int64_t k = 0; k < He; ++k)
        if (mut != 10) v[k] += fval(p->beta_x[k]);  // planted 10: beta dropped
    } else {
      v = xv;
    }
    const float qs = static_cast<float>(fval(p->quant_scale_x[0]));
    std::vector<int64_t> x8(He);
    for (int64_t k = 0; k < He; ++k) x8[k] = quant_static_asym(v[k], qs, p->quant_offset_x[0], mut);
    const int8_t* wq = static_cast<const int8_t*>(p->w_dq);
    const int8_t* wk = static_cast<const int8_t*>(p->w_dkv_kr);
    std::vector<int64_t> aq(Hcq, 0), ak(Wkr, 0);
    for (int64_t k = 0; k < He; ++k) {
      for (int64_t n = 0; n < Hcq; ++n) aq[n] += x8[k] * wq[widx(p, k, n, He, Hcq)];
      for (int64_t n = 0; n < Wkr; ++n) ak[n] += x8[k] * wk[widx(p, k, n, He, Wkr)];
    }
    // y = (acc + bias0) * deScale0; planted 11 subtracts the bias
    auto bias = [&](int64_t n) -> int64_t {
      const int64_t b = p->bias_dqkv ? p->bias_dqkv[n] : 0;
      return mut == 11 ? -b : b;
    };
    for (int64_t n = 0; n < Hcq; ++n)
      y_q[n] = static_cast<double>(aq[n] + bias(n)) * p->scale_w_dq[n];
    for (int64_t n = 0; n < Wkr; ++n)
      y_kvr[n] = static_cast<double>(ak[n] + bias(Hcq + n)) * p->scale_w_dkv_kr[n];
  } else if (q8in) {
    const int8_t* x = static_cast<const int8_t*>(p->x) + t * He;
    const int8_t* wq = static_cast<const int8_t*>(p->w_dq);
    const int8_t* wk = static_cast<const int8_t*>(p->w_dkv_kr);
    std::vector<int64_t> aq(Hcq, 0), ak(Wkr, 0);
    for (int64_t k = 0; k < He; ++k) {
      int64_t xv = x[k];
      for (int64_t n = 0; n < Hcq; ++n) aq[n] += xv * wq[widx(p, k, n, He, Hcq)];
      for (int64_t n = 0; n < Wkr; ++n) ak[n] += xv * wk[widx(p, k, n, He, Wkr)];
    }
    double sx = p->scale_x[t];
    for (int64_t n = 0; n < Hcq; ++n) y_q[n] = static_cast<double>(aq[n]) * sx * p->scale_w_dq[n];
    for (int64_t n = 0; n < Wkr; ++n) y_kvr[n] = static_cast<double>(ak[n]) * sx * p->scale_w_dkv_kr[n];
  } else {
    for (int64_t k = 0; k < He; ++k) {
      double xv = load(p->x, t * He + k, 0);
      for (int64_t n = 0; n < Hcq; ++n) y_q[n] += xv * load(p->w_dq, widx(p, k, n, He, Hcq), 0);
      for (int64_t n = 0; n < Wkr; ++n) y_kvr[n] += xv * load(p->w_dkv_kr, widx(p, k, n, He, Wkr), 0);
    }
  }
  if (p->y_out) {
    double* yo = p->y_out + r * (Hcq + Wkr);
    for (int64_t n = 0; n < Hcq; ++n) yo[n] = y_q[n];
    for (int64_t n = 0; n < Wkr; ++n) yo[Hcq + n] = y_kvr[n];
  }

  std::vector<double> cosv(Dr), sinv(Dr);
  for (int64_t i = 0; i < Dr; ++i) {
    cosv[i] = fval(p->rope_cos[t * Dr + i]);
    sinv[i] = fval(p->rope_sin[t * Dr + i]);
  }

  // c^Q and c^KV
  std::vector<double> g(std::max(Hcq, Hckv));
  std::vector<double> c_q(Hcq), c_kv(Hckv), k_r(Dr);
  for (int64_t i = 0; i < Hcq; ++i) g[i] = fval(p->gamma_cq[i]);
  rmsnorm(y_q.data(), g.data(), Hcq, p->eps_cq, c_q.data(), mut);
  for (int64_t i = 0; i < Hckv; ++i) g[i] = fval(p->gamma_ckv[i]);
  rmsnorm(y_kvr.data(), g.data(), Hckv, p->eps_ckv, c_kv.data(), mut);
  rope(y_kvr.data() + Hckv, cosv.data(), sinv.data(), Dr, k_r.data(), mut);
  if (p->cq_out)
    for (int64_t i = 0; i < Hcq; ++i) p->cq_out[r * Hcq + i] = c_q[i];
  if (p->ckv_out)
    for (int64_t i = 0; i < Hckv; ++i) p->ckv_out[r * Hckv + i] = c_kv[i];
  if (p->kr_out)
    for (int64_t i = 0; i < Dr; ++i) p->kr_out[r * Dr + i] = k_r[i];
  if (p->kv_rows) {
    for (int64_t i = 0; i < Hckv; ++i) {
      if (p->kv_int8)   // R1'
        static_cast<int8_t*>(p->kv_rows)[r * Hckv + i] = quant_static(c_kv[i], p->quant_scale_ckv[i], mut);
      else              // R1
        static_cast<uint16_t*>(p->kv_rows)[r * Hckv + i] = fbits(c_kv[i]);
    }
  }
  if (p->kr_rows) {
    for (int64_t i = 0; i < Dr; ++i) {
      if (p->kr_int8)   // R2'
        static_cast<int8_t*>(p->kr_rows)[r * Dr + i] = quant_static(k_r[i], p->quant_scale_ckr[i], mut);
      else              // R2
        static_cast<uint16_t*>(p->kr_rows)[r * Dr + i] = fbits(k_r[i]);
    }
  }

  // up-projection u = c^Q [W^UQ | W^QR]
  std::vector<double> u(Wuq, 0.0);
  if (p->static_quant) {
    // c^Q to int8 codes: RmsNormQuant(y_q) = code(gamma1 y_q / RMS + beta1)
    std::vector<double> w(c_q);
    for (int64_t i = 0; i < Hcq; ++i)
      if (mut != 10) w[i] += fval(p->beta_cq[i]);
    const float qs = static_cast<float>(fval(p->quant_scale_cq[0]));
    std::vector<int64_t> c8(Hcq);
    for (int64_t i = 0; i < Hcq; ++i) c8[i] = quant_static_asym(w[i], qs, p->quant_offset_cq[0], mut);
    const int8_t* wu = static_cast<const int8_t*>(p->w_uq_qr);
    std::vector<int64_t> acc(Wuq, 0);
    for (int64_t k = 0; k < Hcq; ++k)
      for (int64_t n = 0; n < Wuq; ++n) acc[n] += c8[k] * wu[widx(p, k, n, Hcq, Wuq)];
    for (int64_t n = 0; n < Wuq; ++n) {
      int64_t b = p->bias_uq_qr ? p->bias_uq_qr[n] : 0;
      if (mut == 11) b = -b;
      u[n] = static_cast<double>(acc[n] + b) * p->scale_w_uq_qr[n];
    }
  } else if (q8in || p->quant_uq) {  // R3'
    std::vector<double> cm(c_q);
    if (p->smooth_cq) {
      // c^Q * m: the RmsNorm of y_q with weight gamma * m (exact products)
      for (int64_t i = 0; i < Hcq; ++i) {
        double m = p->smooth_cq[i];
        if (mut == 6) m = 1.0 / m;   // planted: smoothing divided out
        if (mut == 7) m = 1.0;       // planted: smoothing ignored
        g[i] = fval(p->gamma_cq[i]) * m;
      }
      rmsnorm(y_q.data(), g.data(), Hcq, p->eps_cq, cm.data(), mut);
    }
    std::vector<int8_t> c8(Hcq);
    float s_cq;
    quant_int8(cm.data(), Hcq, c8.data(), &s_cq);
    const int8_t* w = static_cast<const int8_t*>(p->w_uq_qr);
    std::vector<int64_t> acc(Wuq, 0);
    for (int64_t k = 0; k < Hcq; ++k) {
      int64_t cv = c8[k];
      for (int64_t n = 0; n < Wuq; ++n) acc[n] += cv * w[widx(p, k, n, Hcq, Wuq)];
    }
    for (int64_t n = 0; n < Wuq; ++n)
      u[n] = static_cast<double>(acc[n]) * static_cast<double>(s_cq) * p->scale_w_uq_qr[n];
  } else {
    for (int64_t k = 0; k < Hcq; ++k) {
      double cv = p->round_intermediates ? fround(c_q[k]) : c_q[k];  // R3
      for (int64_t n = 0; n < Wuq; ++n) u[n] += cv * load(p->w_uq_qr, widx(p, k, n, Hcq, Wuq), 0);
    }
  }
  if (p->u_out)
    for (int64_t n = 0; n < Wuq; ++n) p->u_out[r * Wuq + n] = u[n];

  // per head: split, q^R = RoPE(rope part), q^N = bf16(nope part) W^UK[h]
  std::vector<double> qc(D), qr(Dr), qn(Hckv);
  // queryOut row of (token, head): Hckv values, or Hckv + Dr with q^R after
  // q^N in the concatenated layout
  const int64_t qrow = p->concat ? Hckv + Dr : Hckv;
  for (int64_t h = 0; h < N; ++h) {
    // column offsets of head h inside weightUqQr
    int64_t nope0 = h * (D + Dr), rope0 = h * (D + Dr) + D;
    if (mut == 3) { nope0 = h * D; rope0 = N * D + h * Dr; }  // planted: blocked, not interleaved
    rope(u.data() + rope0, cosv.data(), sinv.data(), Dr, qr.data(), mut);
    for (int64_t i = 0; i < Dr; ++i) {  // R4
      if (p->concat)
        static_cast<uint16_t*>(p->query_out)[(r * N + h) * qrow + Hckv + i] = fbits(qr[i]);
      else
        p->query_rope_out[(r * N + h) * Dr + i] = fbits(qr[i]);
    }
    for (int64_t d = 0; d < D; ++d)
      qc[d] = p->round_intermediates ? fround(u[nope0 + d]) : u[nope0 + d];  // R5
    for (int64_t j = 0; j < Hckv; ++j) qn[j] = 0.0;
    for (int64_t d = 0; d < D; ++d) {
      for (int64_t j = 0; j < Hckv; ++j) {
        // W^UK[h][d][j]; planted mistake 4 reads it as if laid out (N, Hckv, D)
        int64_t idx = (mut == 4) ? (h * Hckv + j) * D + d : (h * D + d) * Hckv + j;
        qn[j] += qc[d] * fval(p->w_uk[idx]);
      }
    }
    if (p->qn_out)
      for (int64_t j = 0; j < Hckv; ++j) p->qn_out[(r * N + h) * Hckv + j] = qn[j];
    if (p->query_int8) {  // R7
      quant_int8(qn.data(), Hckv, static_cast<int8_t*>(p->query_out) + (r * N + h) * Hckv,
                 p->dequant_scale_q_nope + r * N + h);
    } else {              // R6
      uint16_t* qo = static_cast<uint16_t*>(p->query_out) + (r * N + h) * qrow;
      for (int64_t j = 0; j < Hckv; ++j) qo[j] = fbits(qn[j]);
    }
  }
}

// Runs the prolog on the selected rows with nthreads threads (0 = all cores),
// then writes the cache rows at cacheIndex, in row order, skipping indices
// outside [0, BlockNum*BlockSize).  Returns 0, or -1 on a bad argument.
int mla_oracle_run(mla_oracle_problem* p, int nthreads) {
  if (!p || !p->x || !p->w_dq || !p->w_uq_qr || !p->w_uk || !p->w_dkv_kr || !p->gamma_cq ||
      !p->gamma_ckv || !p->rope_sin || !p->rope_cos || !p->query_out ||
      (!p->concat && !p->query_rope_out))
    return -1;
  if (p->static_quant) {
    if (p->quant_in || p->quant_uq || p->smooth_cq || p->kv_int8 || p->kr_int8 || p->query_int8) return -1;
    if (!p->scale_w_dq || !p->scale_w_dkv_kr || !p->scale_w_uq_qr || !p->quant_scale_x ||
        !p->quant_offset_x || !p->beta_cq || !p->quant_scale_cq || !p->quant_offset_cq)
      return -1;
    if (p->x_norm && (!p->gamma_x || !p->beta_x)) return -1;
  }
  if (p->concat && (p->query_int8 || p->kv_int8 || p->kr_int8)) return -1;
  if (p->fp16 && !p->static_quant) return -1;
  if (p->Dr % 2 != 0 || p->Hcq <= 0 || p->Hckv <= 0 || p->N <= 0 || p->D <= 0 || p->Dr <= 0)
    return -1;
  if (p->quant_in && (!p->scale_x || !p->scale_w_dq || !p->scale_w_uq_qr || !p->scale_w_dkv_kr))
    return -1;
  if (p->quant_uq && !p->scale_w_uq_qr) return -1;
  if (p->smooth_cq && !p->quant_in && !p->quant_uq) return -1;
  if (p->query_int8 && !p->dequant_scale_q_nope) return -1;
  if ((p->kv_int8 && !p->quant_scale_ckv) || (p->kr_int8 && !p->quant_scale_ckr)) return -1;
  const int64_t n = p->tokens ? p->n_tokens : p->T;
  for (int64_t r = 0; r < n; ++r) {
    int64_t t = p->tokens ? p->tokens[r] : r;
    if (t < 0 || t >= p->T) return -1;
  }
  // cache rows are always produced (into caller buffers or scratch)
  const size_t kv_eb = p->kv_int8 ? 1 : 2, kr_eb = p->kr_int8 ? 1 : 2;
  std::vector<uint16_t> kv_tmp, kr_tmp;
  mla_oracle_problem q = *p;
  if (!q.kv_rows) { kv_tmp.resize(static_cast<size_t>(n * p->Hckv)); q.kv_rows = kv_tmp.data(); }
  if (!q.kr_rows) { kr_tmp.resize(static_cast<size_t>(n * p->Dr)); q.kr_rows = kr_tmp.data(); }

  unsigned hw = std::thread::hardware_concurrency();
  int nt = nthreads > 0 ? nthreads : static_cast<int>(hw ? hw : 1);
  nt = static_cast<int>(std::min<int64_t>(nt, std::max<int64_t>(n, 1)));
  std::vector<std::thread> pool;
  for (int w = 0; w < nt; ++w) {
    pool.emplace_back([&q, w, nt, n]() {
      for (int64_t r = w; r < n; r += nt) one_token(&q, r, q.tokens ? q.tokens[r] : r);
    });
  }
  for (auto& th : pool) th.join();

  // scatter (aclnnMlaPrologV2WeightNz, parameters cacheIndex / kvCacheRef /
  // krCacheRef): flat slot s is block s / BlockSize, offset s % BlockSize
  if (p->kv_cache && (p->kr_cache || p->concat) && p->cache_index) {
    const int64_t slots = p->block_num * p->block_size;
    for (int64_t r = 0; r < n; ++r) {
      int64_t t = p->tokens ? p->tokens[r] : r;
      int64_t s = p->cache_index[t];
      if (s < 0 || s >= slots) continue;
      int64_t blk = s / p->block_size, off = s % p->block_size;
      const int64_t slot = blk * p->block_size + off;
      if (p->concat) {  // one row: c^KV then k^R
        uint16_t* row = static_cast<uint16_t*>(p->kv_cache) + slot * (p->Hckv + p->Dr);
        std::memcpy(row, static_cast<const uint16_t*>(q.kv_rows) + r * p->Hckv, 2 * p->Hckv);
        std::memcpy(row + p->Hckv, static_cast<const uint16_t*>(q.kr_rows) + r * p->Dr, 2 * p->Dr);
        continue;
      }
      std::memcpy(static_cast<uint8_t*>(p->kv_cache) + slot * p->Hckv * kv_eb,
                  static_cast<const uint8_t*>(q.kv_rows) + r * p->Hckv * kv_eb, kv_eb * p->Hckv);
      std::memcpy(static_cast<uint8_t*>(p->kr_cache) + slot * p->Dr * kr_eb,
                  static_cast<const uint8_t*>(q.kr_rows) + r * p->Dr * kr_eb, kr_eb * p->Dr);
    }
  }
  return 0;
}


// ---------------------------------------------------------------------------
// sparse flash attention, MLA-absorb decode (see the file header)
// ---------------------------------------------------------------------------
typedef struct {
  int64_t T, N, D, Dr;            // D = the latent width (Hckv), Dr the rope width
  int64_t block_num, block_size, K, sparse_block_size, max_blocks;
  double scale;
  int32_t concat;                 // 1: kv rows hold D + Dr values, k^R after c^KV; kr unused
  int32_t mutation;               // planted mistake for the pin tests, 0 = none
  const uint16_t* query;          // (T, N, D) bf16
  const uint16_t* query_rope;     // (T, N, Dr) bf16
  const uint16_t* kv;             // (block_num, block_size, D or D + Dr) bf16
  const uint16_t* kr;             // (block_num, block_size, Dr) bf16
  const int32_t* indices;         // (T, K)
  const int32_t* block_table;     // (T, max_blocks)
  const int32_t* seq_lens;        // (T) kv length of each token's batch
  uint16_t* out;                  // (T, N, D) bf16
  float* softmax_max;             // (T, N) or NULL
  float* softmax_sum;             // (T, N) or NULL
  double* out_f64;                // (T, N, D) before rounding, or NULL
  const int64_t* tokens;          // rows to compute; NULL = 0..T-1 (row r holds token tokens[r])
  int64_t n_tokens;
} mla_oracle_sfa_problem;

static void sfa_token(const mla_oracle_sfa_problem* p, int64_t r, int64_t t) {
  const int64_t D = p->D, Dr = p->Dr, N = p->N, row = p->concat ? D + Dr : D;
  const int mut = p->mutation;
  // the selected slots, in index order
  std::vector<int64_t> slots;
  for (int64_t i = 0; i < p->K; ++i) {
    const int64_t idx = p->indices[t * p->K + i];
    if (idx < 0) continue;
    for (int64_t u = 0; u < p->sparse_block_size; ++u) {
      const int64_t pos = idx * p->sparse_block_size + u;
      if (pos >= p->seq_lens[t]) continue;
      const int64_t b = pos / p->block_size;
      if (b >= p->max_blocks) continue;
      const int64_t blk = mut == 23 ? b : p->block_table[t * p->max_blocks + b];  // planted 23: table ignored
      if (blk < 0 || blk >= p->block_num) continue;
      slots.push_back(blk * p->block_size + pos % p->block_size);
    }
  }
  std::vector<double> s(slots.size()), o(D);
  for (int64_t h = 0; h < N; ++h) {
    const uint16_t* q = p->query + (t * N + h) * D;
    const uint16_t* qr = p->query_rope + (t * N + h) * Dr;
    double mx = -INFINITY;
    for (size_t j = 0; j < slots.size(); ++j) {
      const uint16_t* kv = p->kv + slots[j] * row;
      const uint16_t* kr = p->concat ? kv + D : p->kr + slots[j] * Dr;
      double a = 0.0, b = 0.0;
      for (int64_t d = 0; d < D; ++d) a += bf16_value(q[d]) * bf16_value(kv[d]);
      for (int64_t d = 0; d < Dr; ++d) b += bf16_value(qr[d]) * bf16_value(kr[d]);
      if (mut == 21) b = 0.0;                                   // planted 21: rope part dropped
      s[j] = (mut == 22 ? p->scale * p->scale : p->scale) * (a + b);  // planted 22: scale squared
      mx = std::max(mx, s[j]);
    }
    double sum = 0.0;
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    for (size_t j = 0; j < slots.size(); ++j) {
      const double w = std::exp(s[j] - mx);
      sum += w;
      const uint16_t* kv = p->kv + slots[j] * row;
      for (int64_t d = 0; d < D; ++d) o[d] += w * bf16_value(kv[d]);
    }
    for (int64_t d = 0; d < D; ++d) {
      const double v = slots.empty() ? 0.0 : o[d] / sum;
      if (p->out_f64) p->out_f64[(r * N + h) * D + d] = v;
      p->out[(r * N + h) * D + d] = bf16_bits(v);
    }
    if (p->softmax_max) p->softmax_max[r * N + h] = static_cast<float>(mx);
    if (p->softmax_sum) p->softmax_sum[r * N + h] = static_cast<float>(sum);
  }
}

// Returns 0, or -1 on a bad argument.
int mla_oracle_sfa(mla_oracle_sfa_problem* p, int nthreads) {
  if (!p || !p->query || !p->query_rope || !p->kv || (!p->concat && !p->kr) || !p->indices ||
      !p->block_table || !p->seq_lens || !p->out)
    return -1;
  if (p->N <= 0 || p->D <= 0 || p->Dr <= 0 || p->block_size <= 0 || p->K <= 0 ||
      p->sparse_block_size <= 0 || p->max_blocks <= 0)
    return -1;
  const int64_t n = p->tokens ? p->n_tokens : p->T;
  for (int64_t r = 0; r < n; ++r) {
    const int64_t t = p->tokens ? p->tokens[r] : r;
    if (t < 0 || t >= p->T) return -1;
  }
  unsigned hw = std::thread::hardware_concurrency();
  int nt = nthreads > 0 ? nthreads : static_cast<int>(hw ? hw : 1);
  nt = static_cast<int>(std::min<int64_t>(nt, std::max<int64_t>(n, 1)));
  std::vector<std::thread> pool;
  for (int w = 0; w < nt; ++w)
    pool.emplace_back([p, w, nt, n]() {
      for (int64_t r = w; r < n; r += nt) sfa_token(p, r, p->tokens ? p->tokens[r] : r);
    });
  for (auto& th : pool) th.join();
  return 0;
}

}  // extern "C"
