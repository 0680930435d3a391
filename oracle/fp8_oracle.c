/*
 * fp8_oracle.c -- plain, slow CPU oracle for the FP8 scaled-GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may use it.  It shares no code, header, table or
 * constant with the HIP path.
 *
 * Sources (the pages this follows; cited by title and section):
 *   [guide]   "FP8 quantisation training practical guide" (scrxy.com news page):
 *             section "format choice: E4M3 and E5M2" (bit splits),
 *             section "three scaling algorithms" (tensor / delayed / just-in-time),
 *             section "blockwise scaling" (1x128 inputs and gradients,
 *             128x128 weights, E4M3 only, one scale per block),
 *             section "MXFP8 scaling" (1x32 blocks, E8M0 scale format),
 *             section "code changes" (the three GEMMs of a layer; inputs
 *             quantised, outputs kept in BF16).
 *   [colossal] QbitAI story on Colossal-AI FP8 mixed precision (liutaoaihuanlian.com):
 *             paragraph on the two scaling schemes (delayed scaling takes the
 *             scale from a window of past values; real-time scaling takes it
 *             from the current tensor).
 *   [snippets] search-result page "fp8+bf8" (cidian.kuaisou.com): the forward
 *             pass snippet (BF16 input, weights quantised to FP8, output cast
 *             back to BF16 after accumulation; dgrad cast to BF16).
 *
 * Readings where the pages are silent are listed next to each function; the
 * numeric format definitions are the OCP 8-bit float formats E4M3FN and E5M2,
 * whose largest finite values are 448 and 57344.
 *
 * Every floating-point decision that yields an integer code (the cast) is made
 * in FP32, the precision the kernels use: one FP32 multiply x*scale, then an
 * exact round-to-nearest-even of that FP32 value.  Everything else (decode,
 * GEMM sums, scale products) is computed in FP64, which holds every decoded
 * value and product exactly.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_E4M3 0
#define ORC_E5M2 1

/* Parameters of a binary float format with an implicit leading one.
 * mbits: stored mantissa bits; bias: exponent bias; emin: exponent of the
 * smallest normal binade; fmax: largest finite value.                       */
typedef struct {
  int ebits, mbits, bias, emin;
  double fmax;
} orc_fmt;

static orc_fmt orc_desc(int fmt) {
  orc_fmt d;
  if (fmt == ORC_E4M3) {
    /* [guide] format choice: 1 sign, 4 exponent, 3 mantissa bits.
     * E4M3FN: bias 7, no infinity, only S.1111.111 is NaN, so the top
     * binade keeps 1.000..1.110 and the largest value is 1.75*2^8 = 448. */
    d.ebits = 4; d.mbits = 3; d.bias = 7; d.emin = -6; d.fmax = 448.0;
  } else {
    /* [guide] format choice: 1 sign, 5 exponent, 2 mantissa bits.
     * E5M2: bias 15, IEEE-like (exponent 31 is inf/NaN); max 1.75*2^15. */
    d.ebits = 5; d.mbits = 2; d.bias = 15; d.emin = -14; d.fmax = 57344.0;
  }
  return d;
}

/* ---------------------------------------------------------------- decode */

/* Exact value of an FP8 code (NaN for NaN codes, +-inf for E5M2 inf). */
double oracle_fp8_decode(uint8_t c, int fmt) {
  orc_fmt d = orc_desc(fmt);
  int s = c >> 7;
  int e = (c >> d.mbits) & ((1 << d.ebits) - 1);
  int m = c & ((1 << d.mbits) - 1);
  double v;
  if (fmt == ORC_E4M3) {
    if (e == 15 && m == 7) return NAN;
  } else {
    if (e == 31) {
      if (m != 0) return NAN;
      return s ? -INFINITY : INFINITY;
    }
  }
  if (e == 0)
    v = ldexp((double)m, d.emin - d.mbits);           /* subnormal: m * 2^(emin-mbits) */
  else
    v = ldexp(1.0 + (double)m / (double)(1 << d.mbits), e - d.bias);
  return s ? -v : v;
}

/* ------------------------------------------------ generic nearest-even round */

/* Round |v| (finite, >= 0) to a format with `mbits` stored mantissa bits and
 * smallest normal exponent `emin`, with an unbounded top exponent:
 * quantum q = 2^(max(floor(log2 v), emin) - mbits), result = rint(v/q)*q.
 * v/q is exact (q is a power of two), and rint rounds ties to even under the
 * default rounding mode. */
static double orc_round_rne(double v, int mbits, int emin) {
  int ex;
  if (v == 0.0) return 0.0;
  frexp(v, &ex);                       /* v = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;                      /* floor(log2 v) */
  if (e < emin) e = emin;
  double q = ldexp(1.0, e - mbits);
  return rint(v / q) * q;
}

/* Pack an already-representable magnitude v (>= 0, <= fmax) with sign s. */
static uint32_t orc_pack(double v, int s, int ebits, int mbits, int bias, int emin) {
  uint32_t mag;
  if (v == 0.0) {
    mag = 0;
  } else if (v < ldexp(1.0, emin)) {   /* subnormal: exponent field 0 */
    mag = (uint32_t)(v / ldexp(1.0, emin - mbits));
  } else {
    int ex;
    frexp(v, &ex);
    int e = ex - 1;
    uint32_t mant = (uint32_t)((v / ldexp(1.0, e) - 1.0) * (double)(1 << mbits));
    mag = ((uint32_t)(e + bias) << mbits) | mant;
  }
  return ((uint32_t)s << (ebits + mbits)) | mag;
}

/* Saturating round-to-nearest-even FP32 -> FP8.
 * Readings (pages silent): any magnitude that rounds above the largest finite
 * value, and +-inf, saturates to +-fmax; the sign of zero is kept; a NaN input
 * gives one canonical NaN code whatever its sign or payload, 0xFF (S.1111.111)
 * for E4M3 and 0xFE (S.11111.10) for E5M2 -- the codes the gfx950 converter
 * produces (a NaN's sign carries no value, so the reading follows it). */
uint8_t oracle_fp8_encode(float f, int fmt) {
  orc_fmt d = orc_desc(fmt);
  double v = (double)f;
  int s = signbit(v) ? 1 : 0;
  if (isnan(v)) return fmt == ORC_E4M3 ? 0xFF : 0xFE;
  double a = fabs(v);
  double r = isinf(a) ? INFINITY : orc_round_rne(a, d.mbits, d.emin);
  if (r > d.fmax) r = d.fmax;
  return (uint8_t)orc_pack(r, s, d.ebits, d.mbits, d.bias, d.emin);
}

/* ------------------------------------------------------------------- BF16 */

float oracle_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* FP64 -> BF16 bits, one round-to-nearest-even step (8 significant bits,
 * FP32's exponent range incl. subnormals); NaN -> 0x7FC0|sign, overflow -> inf. */
uint16_t oracle_f64_to_bf16(double v) {
  int s = signbit(v) ? 1 : 0;
  if (isnan(v)) return (uint16_t)((s << 15) | 0x7FC0);
  double a = fabs(v);
  if (isinf(a)) return (uint16_t)((s << 15) | 0x7F80);
  double r = orc_round_rne(a, 7, -126);
  if (r >= ldexp(1.0, 128)) return (uint16_t)((s << 15) | 0x7F80);
  return (uint16_t)orc_pack(r, s, 8, 7, 127, -126);
}

/* ------------------------------------------------------------------- amax */

/* amax = max |x| over a BF16 tensor, as a total order on the magnitude bits
 * (bits & 0x7FFF as unsigned): NaN > inf > every finite value, so a NaN
 * anywhere makes amax NaN.  The result is exactly a BF16 value.
 * [colossal] real-time scaling; [guide] just-in-time scaling: the scale is
 * computed from the maximum of the current tensor. */
static uint16_t orc_absmax_bits(const uint16_t* x, int64_t n) {
  uint16_t m = 0;
  for (int64_t i = 0; i < n; ++i) {
    uint16_t a = x[i] & 0x7FFF;
    if (a > m) m = a;
  }
  return m;
}

float oracle_amax(const uint16_t* x, int64_t n) {
  return oracle_bf16_to_f32(orc_absmax_bits(x, n));
}

/* Scale rule (pages: "compute the scale from the maximum").  Reading:
 * scale = fmax / amax in FP32 (no margin); amax == 0 or non-finite -> 1;
 * a quotient that overflows FP32 is clamped to FLT_MAX.
 * scale_inv = 1 / scale in FP32; dequantisation multiplies by scale_inv. */
void oracle_scale_from_amax(float amax, int fmt, float* scale, float* scale_inv) {
  float fmax = (float)orc_desc(fmt).fmax;
  float s = 1.0f;
  if (amax > 0.0f && isfinite(amax)) {
    s = fmax / amax;
    if (isinf(s)) s = FLT_MAX;
  }
  *scale = s;
  *scale_inv = 1.0f / s;
}

/* ------------------------------------------------------- per-tensor cast */

/* q = sat_rne(fl32(x * scale)) for every element, with an optional transposed
 * copy qT[cols][rows] (the operand layout the weight-gradient GEMM reads) and
 * an optional amax of the input (delayed scaling records it for later steps).
 * [guide] code changes: the GEMM inputs are quantised. */
void oracle_quantize_tensor(const uint16_t* x, int64_t rows, int64_t cols, int fmt,
                            float scale, uint8_t* q, uint8_t* qT, float* amax_out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      float xv = oracle_bf16_to_f32(x[r * cols + c]);
      float p = xv * scale;
      uint8_t code = oracle_fp8_encode(p, fmt);
      if (q) q[r * cols + c] = code;
      if (qT) qT[c * rows + r] = code;
    }
  }
  if (amax_out) *amax_out = oracle_amax(x, rows * cols);
}

/* ---------------------------------------------- FP32 master-weight input */

/* The same amax and cast for an FP32 tensor ([snippets] forward-pass
 * snippet: the master weights are FP32 and are quantised to FP8).  amax is
 * the largest |x| under the same total order, now on the FP32 magnitude bits
 * (bits & 0x7FFFFFFF): NaN > inf > every finite value; the result is exactly
 * an FP32 value.  The cast is the BF16 one without the widening:
 * q = sat_rne(fl32(x * scale)). */
float oracle_amax_f32(const float* x, int64_t n) {
  uint32_t m = 0;
  for (int64_t i = 0; i < n; ++i) {
    uint32_t b;
    memcpy(&b, &x[i], 4);
    b &= 0x7FFFFFFFu;
    if (b > m) m = b;
  }
  float a;
  memcpy(&a, &m, 4);
  return a;
}

void oracle_quantize_tensor_f32(const float* x, int64_t rows, int64_t cols, int fmt,
                                float scale, uint8_t* q, uint8_t* qT, float* amax_out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      float p = x[r * cols + c] * scale;
      uint8_t code = oracle_fp8_encode(p, fmt);
      if (q) q[r * cols + c] = code;
      if (qT) qT[c * rows + r] = code;
    }
  }
  if (amax_out) *amax_out = oracle_amax_f32(x, rows * cols);
}

/* ------------------------------------------------------- delayed scaling */

/* One history step.  [colossal] delayed scaling computes the current scale
 * from the scales of a past window; [guide] delayed scaling keeps a buffer of
 * the maxima of past training steps.  Reading: the window holds the last
 * `hlen` amax values (ring, slot step % hlen, zeros before the first write),
 * its reduce is the maximum (NaN propagates: same total order as amax), and
 * the scale rule above turns that maximum into the scale used by step+1. */
void oracle_amax_history_update(float* hist, int32_t hlen, int64_t step, float amax,
                                int fmt, float* scale, float* scale_inv) {
  hist[step % hlen] = amax;
  uint32_t mbits = 0;
  for (int i = 0; i < hlen; ++i) {
    uint32_t b;
    memcpy(&b, &hist[i], 4);
    b &= 0x7FFFFFFFu;
    if (b > mbits) mbits = b;
  }
  float m;
  memcpy(&m, &mbits, 4);
  oracle_scale_from_amax(m, fmt, scale, scale_inv);
}

/* --------------------------------------------------------- blockwise cast */

/* [guide] blockwise scaling: inputs and gradients in 1x128 tiles, weights in
 * 128x128 blocks, each block with its own scale.  Reading: tiles run along
 * the contiguous (contraction) dimension; each tile applies the amax, scale
 * rule and cast above to its own elements; scale_inv is stored per tile in a
 * row-major grid [rows/br][cols/bc].  Requires cols % bc == 0, rows % br == 0. */
void oracle_quantize_block(const uint16_t* x, int64_t rows, int64_t cols, int fmt,
                           int32_t br, int32_t bc, uint8_t* q, float* scale_inv) {
  int64_t gr = rows / br, gc = cols / bc;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t tr = 0; tr < gr; ++tr) {
    for (int64_t tc = 0; tc < gc; ++tc) {
      uint16_t mb = 0;
      for (int64_t r = tr * br; r < (tr + 1) * br; ++r)
        for (int64_t c = tc * bc; c < (tc + 1) * bc; ++c) {
          uint16_t a = x[r * cols + c] & 0x7FFF;
          if (a > mb) mb = a;
        }
      float s, si;
      oracle_scale_from_amax(oracle_bf16_to_f32(mb), fmt, &s, &si);
      scale_inv[tr * gc + tc] = si;
      for (int64_t r = tr * br; r < (tr + 1) * br; ++r)
        for (int64_t c = tc * bc; c < (tc + 1) * bc; ++c)
          q[r * cols + c] = oracle_fp8_encode(oracle_bf16_to_f32(x[r * cols + c]) * s, fmt);
    }
  }
}

/* ---------------------------------------------------------------- MX cast */

/* Shared E8M0 exponent of one 1x32 block with magnitude maximum a (finite,
 * > 0): the smallest integer e with a <= fmax * 2^e, so that no element of the
 * block saturates.  Written with frexp: a = m*2^E, m in [0.5,1); fmax is
 * 0.875*2^F (F = 9 for E4M3, 16 for E5M2); a <= 0.875*2^(F+e) holds for
 * e = E-F exactly when m <= 0.875, otherwise e = E-F+1 is the smallest. */
int oracle_mx_exponent(float a, int fmt) {
  int E, F;
  double m = frexp((double)a, &E);
  double fm = frexp(orc_desc(fmt).fmax, &F);   /* fm = 0.875 */
  int e = (m <= fm) ? E - F : E - F + 1;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* [guide] MXFP8 scaling: uniform 1x32 blocks with E8M0 scale factors.
 * Reading: blocks run along the contiguous dimension; byte = e + 127 with e
 * from oracle_mx_exponent; an all-zero block gets e = 0 (byte 127); a block
 * whose amax is inf or NaN gets the E8M0 NaN byte 0xFF and its elements are
 * cast unscaled.  Elements: q = sat_rne(x * 2^-e), the multiply being exact
 * unless the product is far below the smallest FP8 subnormal (code 0 then).
 * Dequantisation multiplies by 2^e.  Requires cols % 32 == 0. */
void oracle_quantize_mx(const uint16_t* x, int64_t rows, int64_t cols, int fmt,
                        uint8_t* q, uint8_t* e8m0) {
  int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint16_t* xb = x + r * cols + b * 32;
      uint16_t mb = 0;
      for (int i = 0; i < 32; ++i) {
        uint16_t a = xb[i] & 0x7FFF;
        if (a > mb) mb = a;
      }
      float a = oracle_bf16_to_f32(mb);
      int e;
      uint8_t byte;
      if (!isfinite(a)) { e = 0; byte = 0xFF; }
      else if (a == 0.0f) { e = 0; byte = 127; }
      else { e = oracle_mx_exponent(a, fmt); byte = (uint8_t)(e + 127); }
      e8m0[r * nb + b] = byte;
      for (int i = 0; i < 32; ++i)
        q[r * cols + b * 32 + i] = oracle_fp8_encode(ldexpf(oracle_bf16_to_f32(xb[i]), -e), fmt);
    }
  }
}

/* ------------------------------------------------------------------ GEMMs */

#define ORC_SCALE_TENSOR 0
#define ORC_SCALE_BLOCK 1
#define ORC_SCALE_MX 2

/* Dequantisation multiplier of one operand element (row r, k), FP64. */
static double orc_operand_scale(int mode, const void* s, int64_t r, int64_t k,
                                int64_t K, int32_t block_rows) {
  if (mode == ORC_SCALE_TENSOR) return (double)((const float*)s)[0];
  if (mode == ORC_SCALE_BLOCK) {
    int64_t gc = K / 128;
    return (double)((const float*)s)[(r / block_rows) * gc + k / 128];
  }
  uint8_t byte = ((const uint8_t*)s)[r * (K / 32) + k / 32];
  if (byte == 0xFF) return NAN;
  return ldexp(1.0, (int)byte - 127);
}

/* Selected outputs of C[i,j] = sum_k deq(A[i,k]) * deq(B[j,k]), both operands
 * stored K-contiguous ("TN"): A[rows_a][K], B[rows_b][K].  This one routine
 * serves the three GEMMs of a linear layer ([guide] code changes; [snippets]
 * forward/backward flow):
 *   fprop  Y[M,N]  = X[M,K]   . W[N,K]^T    (contract K)
 *   dgrad  dX[M,K] = dY[M,N]  . WT[K,N]^T   (contract N)
 *   wgrad  dW[N,K] = dYT[N,M] . XT[K,M]^T   (contract M)
 * Each output is computed on its own, as the definition reads:
 *   tensor scaling: (sa * sb) * sum_k a_k b_k
 *   block scaling:  sum_b (sa[i,b] * sb[j,b]) * sum_{k in b} a_k b_k
 *   MX scaling:     sum_k (a_k 2^ea[i,k/32]) (b_k 2^eb[j,k/32])
 * in FP64 (every product of two decoded FP8 values is exact in FP64), then
 * one round to BF16.  absdot receives the matching sum of |terms|, used by
 * the tests' error bound for FP32 accumulation. */
void oracle_gemm_entries(const uint8_t* A, const uint8_t* B, int64_t K,
                         int fmt_a, int fmt_b, int mode,
                         const void* sa, int32_t block_rows_a,
                         const void* sb, int32_t block_rows_b,
                         int64_t n, const int64_t* ii, const int64_t* jj,
                         double* out, double* absdot, uint16_t* out_bf16) {
  double da[256], db[256];
  for (int c = 0; c < 256; ++c) {
    da[c] = oracle_fp8_decode((uint8_t)c, fmt_a);
    db[c] = oracle_fp8_decode((uint8_t)c, fmt_b);
  }
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n; ++t) {
    const uint8_t* a = A + ii[t] * K;
    const uint8_t* b = B + jj[t] * K;
    double acc = 0.0, aacc = 0.0;
    if (mode == ORC_SCALE_TENSOR) {
      for (int64_t k = 0; k < K; ++k) {
        double p = da[a[k]] * db[b[k]];
        acc += p;
        aacc += fabs(p);
      }
      double s = orc_operand_scale(mode, sa, ii[t], 0, K, 1) *
                 orc_operand_scale(mode, sb, jj[t], 0, K, 1);
      acc *= s;
      aacc *= fabs(s);
    } else if (mode == ORC_SCALE_BLOCK) {
      for (int64_t k0 = 0; k0 < K; k0 += 128) {
        double part = 0.0, apart = 0.0;
        for (int64_t k = k0; k < k0 + 128; ++k) {
          double p = da[a[k]] * db[b[k]];
          part += p;
          apart += fabs(p);
        }
        double s = orc_operand_scale(mode, sa, ii[t], k0, K, block_rows_a) *
                   orc_operand_scale(mode, sb, jj[t], k0, K, block_rows_b);
        acc += s * part;
        aacc += fabs(s) * apart;
      }
    } else {
      for (int64_t k = 0; k < K; ++k) {
        double p = da[a[k]] * orc_operand_scale(mode, sa, ii[t], k, K, 1) *
                   db[b[k]] * orc_operand_scale(mode, sb, jj[t], k, K, 1);
        acc += p;
        aacc += fabs(p);
      }
    }
    out[t] = acc;
    if (absdot) absdot[t] = aacc;
    if (out_bf16) out_bf16[t] = oracle_f64_to_bf16(acc);
  }
}

/* Elementwise FP64 -> BF16 over an array (used for whole-matrix results). */
void oracle_f64_to_bf16_array(const double* v, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(v[i]);
}

/* Encode an FP32 array (used by the codec pins). */
void oracle_fp8_encode_array(const float* f, int64_t n, int fmt, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_encode(f[i], fmt);
}

/* Encode every FP32 bit pattern in [lo, hi) (used by the exhaustive pin). */
void oracle_fp8_encode_bits_range(uint64_t lo, uint64_t hi, int fmt, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)(hi - lo); ++i) {
    uint32_t u = (uint32_t)(lo + (uint64_t)i);
    float f;
    memcpy(&f, &u, 4);
    out[i] = oracle_fp8_encode(f, fmt);
  }
}
