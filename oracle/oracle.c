/*
 * oracle.c -- plain, slow, scalar CPU oracle for the per-tensor-scaled
 * low-precision AdamW step of MS-AMP's O2 and O3 optimization levels.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The product path (the HIP library
 * and its binding) never calls, links or imports anything from here, and this
 * file includes nothing from the product.
 *
 * What the pages fix (MS-AMP "Optimization Level" page, section "O2" and the
 * optimization-level table; MS-AMP README, "Usage" and the O2 table):
 *   - O2: weight gradient in FP8, first moment (exp_avg) in FP8, second moment
 *     (exp_avg_sq) in FP16, weight in FP16, no master weight.
 *   - O3: as O2, plus an FP16 master weight and an FP8 regular weight.
 *   - the optimizer is torch.optim.Adam / AdamW.
 *   - the two FP8 encodings are E4M3 and E5M2 (TransformerEngine issue #131).
 * Everything else is a reading; each reading is named where it is used:
 *   R-ADAMW   AdamW is PyTorch's documented decoupled-weight-decay algorithm
 *             with bias correction and eps outside the square root.
 *   R-FP32    all arithmetic in IEEE binary32; FP8/FP16 are storage only; each
 *             stored value is rounded once; the update uses the unrounded
 *             FP32 new moments.
 *   R-ORDER   exact operation order, with exactly four fused multiply-adds:
 *               m1  = fma(B1, m0, OB1*g)
 *               v1  = fma(B2, v0, OB2*(g*g))
 *               den = fma(sqrt(v1), IBS, EPS)
 *               w1  = fma(-SS, m1/den, w0*DEC)
 *             where B1=b1, OB1=1-b1, B2=b2, OB2=1-b2, EPS=eps,
 *             SS=lr/(1-b1^t), IBS=1/sqrt(1-b2^t), DEC=1-lr*wd are computed
 *             in binary64 and rounded once to binary32.
 *   R-SCALE   per-tensor current scaling: s = fp8_max/amax; s = 1 when amax is
 *             0, NaN or Inf, or when the quotient is not finite and positive;
 *             s_inv = 1/s; dequantization is code*s_inv.
 *   R-AMAX    amax is the largest |x| compared as the unsigned integer
 *             (bits & 0x7FFFFFFF): order-free, -0 counts as +0, a NaN beats
 *             Inf beats every finite value, an empty tensor gives 0.
 *   R-TWOPASS the new first moment is scaled by its own amax (two passes:
 *             compute m1 and its amax, then encode with the new scale).
 *   R-CAST    FP8 casts are OCP E4M3 (max 448, no Inf, NaN = S.1111.111) and
 *             OCP E5M2 (max 57344, IEEE Inf/NaN), round to nearest, ties to
 *             even, subnormals kept, saturating: finite overflow and +-Inf go
 *             to +-max, NaN goes to 0x7F with the input's sign bit. FP16 is
 *             IEEE binary16, round to nearest even, subnormals kept, overflow
 *             to +-Inf.
 *   R-O3COPY  the FP8 regular weight of O3 is taken from the stored (rounded)
 *             FP16 master, E4M3, with the same scale rule.
 *   R-ADAM    torch.optim.Adam (the other optimizer the README recognizes)
 *             applies weight decay as an L2 term added to the gradient before
 *             the moments: gd = fma(WD, w0, g) with WD = (float)wd, then the
 *             AdamW formulas above with gd in place of g and DEC = 1 (no
 *             decoupled decay; w0*1 is exact).
 *
 * Build: a C11 compiler with -O2 -ffp-contract=off (no fast-math), so that
 * only the four fmaf calls above are fused and every other operation is a
 * separately rounded IEEE operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Bit views                                                                 */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return u;
}

static float f32_from_bits(uint32_t u) {
  float x;
  memcpy(&x, &u, sizeof x);
  return x;
}

/* ------------------------------------------------------------------------ */
/* Small floating-point formats (OCP FP8 E4M3 / E5M2, IEEE binary16)         */
/* ------------------------------------------------------------------------ */

typedef struct {
  int ebits;          /* exponent field width */
  int mbits;          /* stored mantissa (fraction) bits */
  int bias;           /* exponent bias */
  int ieee_specials;  /* 1: all-ones exponent is Inf (M = 0) / NaN (M != 0);
                         0: only the all-ones pattern S.1..1.1..1 is NaN */
  int saturate;       /* 1: finite overflow and +-Inf encode to +-max */
  uint32_t nan_code;  /* NaN produced by the encoder, sign bit clear */
} mf_format;

/* OCP 8-bit floating point, E4M3: bias 7, largest finite 1.110b * 2^8. */
static const mf_format FMT_E4M3 = {4, 3, 7, 0, 1, 0x7Fu};
/* OCP 8-bit floating point, E5M2: bias 15, IEEE-style Inf/NaN. */
static const mf_format FMT_E5M2 = {5, 2, 15, 1, 1, 0x7Fu};
/* IEEE 754 binary16. */
static const mf_format FMT_F16 = {5, 10, 15, 1, 0, 0x7E00u};

static int mf_total_bits(const mf_format* f) { return 1 + f->ebits + f->mbits; }

/* Largest finite magnitude of the format, exactly, as a double. */
static double mf_max(const mf_format* f) {
  int emax_field = (1 << f->ebits) - 1;
  int E, M;
  if (f->ieee_specials) {
    E = emax_field - 1;
    M = (1 << f->mbits) - 1;
  } else {
    E = emax_field;
    M = (1 << f->mbits) - 2;
  }
  return ldexp((double)((1 << f->mbits) + M), E - f->bias - f->mbits);
}

/* Bits of +max (sign clear). */
static uint32_t mf_max_code(const mf_format* f) {
  int emax_field = (1 << f->ebits) - 1;
  if (f->ieee_specials)
    return ((uint32_t)(emax_field - 1) << f->mbits) | ((1u << f->mbits) - 1u);
  return ((uint32_t)emax_field << f->mbits) | ((1u << f->mbits) - 2u);
}

/* Decode a code to its exact value (every value of these formats is exact in
 * binary64 and in binary32). */
static double mf_decode(const mf_format* f, uint32_t code) {
  int nb = mf_total_bits(f);
  int sign = (int)((code >> (nb - 1)) & 1u);
  int E = (int)((code >> f->mbits) & ((1u << f->ebits) - 1u));
  int M = (int)(code & ((1u << f->mbits) - 1u));
  int emax_field = (1 << f->ebits) - 1;
  double mag;
  if (f->ieee_specials && E == emax_field) {
    mag = (M == 0) ? INFINITY : NAN;
  } else if (!f->ieee_specials && E == emax_field && M == (1 << f->mbits) - 1) {
    mag = NAN;
  } else if (E == 0) {
    /* subnormal: 0.M * 2^(1-bias) */
    mag = ldexp((double)M, 1 - f->bias - f->mbits);
  } else {
    /* normal: 1.M * 2^(E-bias) */
    mag = ldexp((double)((1 << f->mbits) + M), E - f->bias - f->mbits);
  }
  return sign ? -mag : mag;
}

/* Round a non-negative finite double 'a' (which is a binary32 value) to the
 * format's precision, round to nearest with ties to the even integer
 * significand. Returns the code magnitude; handles overflow per the format. */
static uint32_t mf_encode_magnitude(const mf_format* f, double a) {
  const int emin = 1 - f->bias; /* exponent of the smallest normal binade */
  if (a == 0.0) return 0u;

  /* Binade of a: a = fr * 2^k with fr in [0.5, 1), so floor(log2 a) = k-1. */
  int k;
  (void)frexp(a, &k);
  int e = k - 1;
  if (e < emin) e = emin; /* subnormal range shares the smallest quantum */

  /* Quantum (unit in the last place) of the binade and the scaled value. The
   * division by a power of two is exact in binary64 for every binary32 a. */
  double q = ldexp(1.0, e - f->mbits);
  double r = a / q;
  double n = floor(r);
  double frac = r - n;
  if (frac > 0.5) {
    n += 1.0;
  } else if (frac == 0.5) {
    if (fmod(n, 2.0) != 0.0) n += 1.0; /* tie: go to the even significand */
  }
  double y = n * q; /* rounded magnitude, exact */

  if (y > mf_max(f)) {
    if (f->saturate) return mf_max_code(f);
    /* IEEE overflow: infinity */
    return (uint32_t)((1 << f->ebits) - 1) << f->mbits;
  }

  /* Compose the code of the exact value y. */
  long in = (long)n;
  if (in == (1L << (f->mbits + 1))) { /* rounding carried into the next binade */
    e += 1;
    in = 1L << f->mbits;
  }
  uint32_t E, M;
  if (in < (1L << f->mbits)) { /* only possible in the smallest binade */
    E = 0u;
    M = (uint32_t)in;
  } else {
    E = (uint32_t)(e + f->bias);
    M = (uint32_t)(in - (1L << f->mbits));
  }
  return (E << f->mbits) | M;
}

static uint32_t mf_encode(const mf_format* f, float x) {
  int nb = mf_total_bits(f);
  uint32_t sign = (f32_bits(x) >> 31) << (nb - 1);
  if (isnan(x)) return sign | f->nan_code;
  double a = fabs((double)x);
  if (isinf(x)) {
    if (f->saturate) return sign | mf_max_code(f);
    return sign | ((uint32_t)((1 << f->ebits) - 1) << f->mbits);
  }
  return sign | mf_encode_magnitude(f, a);
}

static const mf_format* fp8_format(int fmt) {
  return fmt == 0 ? &FMT_E4M3 : (fmt == 1 ? &FMT_E5M2 : NULL);
}

/* FP8 decode of one code to binary32 (exact). */
static float fp8_dec(const mf_format* f, uint8_t code) { return (float)mf_decode(f, code); }

static float f16_dec(uint16_t h) { return (float)mf_decode(&FMT_F16, h); }
static uint16_t f16_enc(float x) { return (uint16_t)mf_encode(&FMT_F16, x); }
static uint8_t fp8_enc(const mf_format* f, float x) { return (uint8_t)mf_encode(f, x); }

/* ------------------------------------------------------------------------ */
/* Exported codec entry points (array forms, for the tests)                   */
/* ------------------------------------------------------------------------ */

/* fmt: 0 = E4M3, 1 = E5M2. Returns 0 on success, -1 on a bad format. */
int oracle_fp8_encode_array(const float* x, int64_t n, int fmt, uint8_t* out) {
  const mf_format* f = fp8_format(fmt);
  if (!f) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = fp8_enc(f, x[i]);
  return 0;
}

int oracle_fp8_decode_array(const uint8_t* codes, int64_t n, int fmt, float* out) {
  const mf_format* f = fp8_format(fmt);
  if (!f) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = fp8_dec(f, codes[i]);
  return 0;
}

void oracle_f16_encode_array(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_enc(x[i]);
}

void oracle_f16_decode_array(const uint16_t* h, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_dec(h[i]);
}

/* Largest finite value of an FP8 format (448 or 57344). */
float oracle_fp8_max(int fmt) {
  const mf_format* f = fp8_format(fmt);
  return f ? (float)mf_max(f) : NAN;
}

/* ------------------------------------------------------------------------ */
/* amax and the scale rule                                                   */
/* ------------------------------------------------------------------------ */

/* R-AMAX: max over i of (bits(x[i]) & 0x7FFFFFFF), returned as a float. */
float oracle_amax(const float* x, int64_t n) {
  uint32_t m = 0u;
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = f32_bits(x[i]) & 0x7FFFFFFFu;
    if (u > m) m = u;
  }
  return f32_from_bits(m);
}

/* R-SCALE: s = fmax/amax, or 1 when that is undefined or degenerate. */
float oracle_scale(float amax, float fmax) {
  if (!(amax > 0.0f) || !isfinite(amax)) return 1.0f;
  float s = fmax / amax;
  if (!isfinite(s) || !(s > 0.0f)) return 1.0f;
  return s;
}

/* Per-tensor FP8 quantization of binary32 data with a given amax:
 * s = scale(amax), s_inv = 1/s, q[i] = enc(x[i]*s). meta_out receives
 * {amax, s, s_inv}. Returns -1 on a bad format. */
int oracle_quantize_fp8(const float* x, int64_t n, int fmt, float amax, float* meta_out,
                        uint8_t* q) {
  const mf_format* f = fp8_format(fmt);
  if (!f) return -1;
  float s = oracle_scale(amax, (float)mf_max(f));
  float s_inv = 1.0f / s;
  for (int64_t i = 0; i < n; ++i) q[i] = fp8_enc(f, x[i] * s);
  meta_out[0] = amax;
  meta_out[1] = s;
  meta_out[2] = s_inv;
  return 0;
}

/* Pre-scaled quantization for an FP8 gradient all-reduce over 'world' ranks
 * (the O1 level of the MS-AMP optimization-level page: FP8 weight gradients
 * and FP8 all-reduce). Reading: every rank uses the common amax of the
 * gradient over all ranks (an all-reduce MAX the caller performs) and the
 * scale s = scale(amax * world), with amax * world rounded to binary32, so
 * that the sum of the 'world' ranks' values stays within the FP8 range.
 * world = 1 is oracle_quantize_fp8. Returns -1 on a bad format or world < 1. */
int oracle_quantize_fp8_prescaled(const float* x, int64_t n, int fmt, float amax, int world,
                                  float* meta_out, uint8_t* q) {
  const mf_format* f = fp8_format(fmt);
  if (!f || world < 1) return -1;
  float s = oracle_scale(amax * (float)world, (float)mf_max(f));
  float s_inv = 1.0f / s;
  for (int64_t i = 0; i < n; ++i) q[i] = fp8_enc(f, x[i] * s);
  meta_out[0] = amax;
  meta_out[1] = s;
  meta_out[2] = s_inv;
  return 0;
}

/* Dequantization: out[i] = dec(q[i]) * s_inv. */
int oracle_dequantize_fp8(const uint8_t* q, int64_t n, int fmt, float s_inv, float* out) {
  const mf_format* f = fp8_format(fmt);
  if (!f) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = fp8_dec(f, q[i]) * s_inv;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* AdamW (R-ADAMW, R-FP32, R-ORDER)                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
  double lr, beta1, beta2, eps, weight_decay;
} oracle_hparams;

enum { K_B1 = 0, K_OB1, K_B2, K_OB2, K_EPS, K_SS, K_IBS, K_DEC, K_WD, K_COUNT };

/* Per-step constants, computed in binary64 and rounded once to binary32.
 * 'step' is the 1-based step count after increment. */
void oracle_adamw_constants(const oracle_hparams* hp, int64_t step, float* k) {
  double t = (double)step;
  double bc1 = 1.0 - pow(hp->beta1, t);
  double bc2 = 1.0 - pow(hp->beta2, t);
  k[K_B1] = (float)hp->beta1;
  k[K_OB1] = (float)(1.0 - hp->beta1);
  k[K_B2] = (float)hp->beta2;
  k[K_OB2] = (float)(1.0 - hp->beta2);
  k[K_EPS] = (float)hp->eps;
  k[K_SS] = (float)(hp->lr / bc1);
  k[K_IBS] = (float)(1.0 / sqrt(bc2));
  k[K_DEC] = (float)(1.0 - hp->lr * hp->weight_decay);
  k[K_WD] = (float)hp->weight_decay;
}

/* The gradient the moments see. AdamW: g. Adam (coupled L2, R-ADAM):
 * g + wd*w0 with one fused multiply-add. */
static float effective_grad(const float* k, int coupled, float g, float w0) {
  return coupled ? fmaf(k[K_WD], w0, g) : g;
}

/* Decay factor of the update: 1 - lr*wd for AdamW, 1 for Adam. */
static float decay_factor(const float* k, int coupled) { return coupled ? 1.0f : k[K_DEC]; }

/* First moment: m1 = beta1*m0 + (1-beta1)*g, one fused multiply-add. */
static float adamw_first_moment(const float* k, float g, float m0) {
  return fmaf(k[K_B1], m0, k[K_OB1] * g);
}

/* Second moment and weight. The weight update uses the unrounded m1 and v1:
 *   v1  = beta2*v0 + (1-beta2)*g^2
 *   den = sqrt(v1)/sqrt(1-beta2^t) + eps
 *   w1  = w0*(1-lr*wd) - (lr/(1-beta1^t)) * m1/den                          */
static void adamw_second_moment_and_weight(const float* k, float dec, float g, float m1, float v0,
                                           float w0, float* v1_out, float* w1_out) {
  float v1 = fmaf(k[K_B2], v0, k[K_OB2] * (g * g));
  float den = fmaf(sqrtf(v1), k[K_IBS], k[K_EPS]);
  float w1 = fmaf(-k[K_SS], m1 / den, w0 * dec);
  *v1_out = v1;
  *w1_out = w1;
}

/* AdamW (coupled = 0) or Adam (coupled = 1) with every state in binary32 (no
 * quantization). Used only to pin the arithmetic above against
 * torch.optim.AdamW / torch.optim.Adam. */
void oracle_adamw_f32_tensor(int64_t n, const float* g, float* m, float* v, float* w,
                             const oracle_hparams* hp, int64_t step, int coupled) {
  float k[K_COUNT];
  oracle_adamw_constants(hp, step, k);
  float dec = decay_factor(k, coupled);
  for (int64_t i = 0; i < n; ++i) {
    float gd = effective_grad(k, coupled, g[i], w[i]);
    float m1 = adamw_first_moment(k, gd, m[i]);
    float v1, w1;
    adamw_second_moment_and_weight(k, dec, gd, m1, v[i], w[i], &v1, &w1);
    m[i] = m1;
    v[i] = v1;
    w[i] = w1;
  }
}

/* One O2 step on one tensor, in place.
 *   qg, gfmt, g_scale_inv : FP8 gradient codes, their format and 1/scale
 *   qm, m_meta            : E4M3 first-moment codes and their {amax, scale,
 *                           scale_inv, reserved}; m_meta[2] is read as the old
 *                           1/scale, then m_meta[0..2] are overwritten
 *   v, w                  : FP16 second moment and FP16 weight (bits)
 * When 'amax_w_out' is not NULL the weight array is the O3 master and its new
 * amax (R-AMAX over the stored FP16 values) is returned there.
 * Returns 0, or -1 on a bad format or allocation failure. */
static int adamw_lowbit_tensor(int64_t n, const uint8_t* qg, int gfmt, float g_scale_inv,
                               uint8_t* qm, float* m_meta, uint16_t* v, uint16_t* w,
                               const oracle_hparams* hp, int64_t step, int coupled,
                               float* amax_w_out) {
  const mf_format* gf = fp8_format(gfmt);
  if (!gf) return -1;
  float k[K_COUNT];
  oracle_adamw_constants(hp, step, k);
  float dec = decay_factor(k, coupled);
  float m_scale_inv_old = m_meta[2];

  float* g = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  float* m1 = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  if (!g || !m1) {
    free(g);
    free(m1);
    return -1;
  }

  /* Pass 1: dequantize gradient and old first moment, new first moment, and
   * the amax of the new first moment (R-TWOPASS). g[] holds the gradient the
   * moments see (R-ADAM). */
  uint32_t amax_m_bits = 0u;
  for (int64_t i = 0; i < n; ++i) {
    g[i] = effective_grad(k, coupled, fp8_dec(gf, qg[i]) * g_scale_inv, f16_dec(w[i]));
    float m0 = fp8_dec(&FMT_E4M3, qm[i]) * m_scale_inv_old;
    m1[i] = adamw_first_moment(k, g[i], m0);
    uint32_t u = f32_bits(m1[i]) & 0x7FFFFFFFu;
    if (u > amax_m_bits) amax_m_bits = u;
  }
  float amax_m = f32_from_bits(amax_m_bits);
  float s_m = oracle_scale(amax_m, (float)mf_max(&FMT_E4M3));
  float s_m_inv = 1.0f / s_m;

  /* Pass 2: second moment, weight, and the stores (each rounded once). */
  uint32_t amax_w_bits = 0u;
  for (int64_t i = 0; i < n; ++i) {
    float v1, w1;
    adamw_second_moment_and_weight(k, dec, g[i], m1[i], f16_dec(v[i]), f16_dec(w[i]), &v1, &w1);
    v[i] = f16_enc(v1);
    w[i] = f16_enc(w1);
    qm[i] = fp8_enc(&FMT_E4M3, m1[i] * s_m);
    uint32_t u = f32_bits(f16_dec(w[i])) & 0x7FFFFFFFu;
    if (u > amax_w_bits) amax_w_bits = u;
  }
  m_meta[0] = amax_m;
  m_meta[1] = s_m;
  m_meta[2] = s_m_inv;
  if (amax_w_out) *amax_w_out = f32_from_bits(amax_w_bits);

  free(g);
  free(m1);
  return 0;
}

/* O2 step on one tensor (see adamw_lowbit_tensor for the arguments);
 * coupled = 1 selects Adam (R-ADAM). */
int oracle_adamw_o2_tensor(int64_t n, const uint8_t* qg, int gfmt, float g_scale_inv,
                           uint8_t* qm, float* m_meta, uint16_t* v, uint16_t* w,
                           const oracle_hparams* hp, int64_t step, int coupled) {
  return adamw_lowbit_tensor(n, qg, gfmt, g_scale_inv, qm, m_meta, v, w, hp, step, coupled, NULL);
}

/* Ablation (not the reading the step follows, see R-TWOPASS): the O2 step in
 * one pass with delayed scaling of the first moment. The new codes are
 * encoded with the scale of the previous step's amax, s = scale(m_meta[0]),
 * and m_meta becomes {amax(m1), s, 1/s}: the amax feeds the next step's
 * scale and 1/s decodes the codes stored now. Everything else as the O2 step
 * (coupled = 1: Adam). At step 1 the scale is 1, so |m1| below 2^-10 is
 * stored as 0; values above 448/s saturate. */
int oracle_adamw_o2_tensor_delayed(int64_t n, const uint8_t* qg, int gfmt, float g_scale_inv,
                                   uint8_t* qm, float* m_meta, uint16_t* v, uint16_t* w,
                                   const oracle_hparams* hp, int64_t step, int coupled) {
  const mf_format* gf = fp8_format(gfmt);
  if (!gf) return -1;
  float k[K_COUNT];
  oracle_adamw_constants(hp, step, k);
  float dec = decay_factor(k, coupled);
  float m_scale_inv_old = m_meta[2];
  float s_m = oracle_scale(m_meta[0], (float)mf_max(&FMT_E4M3));
  uint32_t amax_m_bits = 0u;
  for (int64_t i = 0; i < n; ++i) {
    float w0 = f16_dec(w[i]);
    float g = effective_grad(k, coupled, fp8_dec(gf, qg[i]) * g_scale_inv, w0);
    float m0 = fp8_dec(&FMT_E4M3, qm[i]) * m_scale_inv_old;
    float m1 = adamw_first_moment(k, g, m0);
    uint32_t u = f32_bits(m1) & 0x7FFFFFFFu;
    if (u > amax_m_bits) amax_m_bits = u;
    float v1, w1;
    adamw_second_moment_and_weight(k, dec, g, m1, f16_dec(v[i]), w0, &v1, &w1);
    v[i] = f16_enc(v1);
    w[i] = f16_enc(w1);
    qm[i] = fp8_enc(&FMT_E4M3, m1 * s_m);
  }
  m_meta[0] = f32_from_bits(amax_m_bits);
  m_meta[1] = s_m;
  m_meta[2] = 1.0f / s_m;
  return 0;
}

/* Ablation (not the reading the step follows, see R-FP32 / the flagged FP16
 * underflow of v): the O2 step with a per-tensor-scaled FP16 second moment.
 * v is stored as fp16(v1 * s_v) with s_v = scale(amax(v1), 65504) and its
 * own meta {amax_v, s_v, 1/s_v}; v0 = f32(code) * v_meta[2] (old 1/s_v).
 * Both amaxes come from the first pass (which therefore also reads v), the
 * second pass recomputes m1 and v1 identically and stores everything. */
int oracle_adamw_o2_tensor_scaled_v(int64_t n, const uint8_t* qg, int gfmt, float g_scale_inv,
                                    uint8_t* qm, float* m_meta, uint16_t* v, float* v_meta,
                                    uint16_t* w, const oracle_hparams* hp, int64_t step) {
  const mf_format* gf = fp8_format(gfmt);
  if (!gf) return -1;
  float k[K_COUNT];
  oracle_adamw_constants(hp, step, k);
  float m_si_old = m_meta[2], v_si_old = v_meta[2];
  float* g = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  float* m1 = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  float* v1 = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  if (!g || !m1 || !v1) {
    free(g);
    free(m1);
    free(v1);
    return -1;
  }
  uint32_t am = 0u, av = 0u;
  for (int64_t i = 0; i < n; ++i) {
    g[i] = fp8_dec(gf, qg[i]) * g_scale_inv;
    m1[i] = adamw_first_moment(k, g[i], fp8_dec(&FMT_E4M3, qm[i]) * m_si_old);
    v1[i] = fmaf(k[K_B2], f16_dec(v[i]) * v_si_old, k[K_OB2] * (g[i] * g[i]));
    uint32_t u = f32_bits(m1[i]) & 0x7FFFFFFFu;
    if (u > am) am = u;
    u = f32_bits(v1[i]) & 0x7FFFFFFFu;
    if (u > av) av = u;
  }
  float s_m = oracle_scale(f32_from_bits(am), (float)mf_max(&FMT_E4M3));
  float s_v = oracle_scale(f32_from_bits(av), (float)mf_max(&FMT_F16));
  for (int64_t i = 0; i < n; ++i) {
    float den = fmaf(sqrtf(v1[i]), k[K_IBS], k[K_EPS]);
    float w1 = fmaf(-k[K_SS], m1[i] / den, f16_dec(w[i]) * k[K_DEC]);
    w[i] = f16_enc(w1);
    v[i] = f16_enc(v1[i] * s_v);
    qm[i] = fp8_enc(&FMT_E4M3, m1[i] * s_m);
  }
  m_meta[0] = f32_from_bits(am);
  m_meta[1] = s_m;
  m_meta[2] = 1.0f / s_m;
  v_meta[0] = f32_from_bits(av);
  v_meta[1] = s_v;
  v_meta[2] = 1.0f / s_v;
  free(g);
  free(m1);
  free(v1);
  return 0;
}

/* O3 step on one tensor (coupled = 1: Adam): the O2 update applied to the
 * FP16 master weight,
 * then the FP8 E4M3 regular-weight copy from the stored master (R-O3COPY):
 * amax_w over the new master, s_w = scale(amax_w, 448), w8[i] =
 * enc(master[i]*s_w); w8_meta receives {amax_w, s_w, 1/s_w}. */
int oracle_adamw_o3_tensor(int64_t n, const uint8_t* qg, int gfmt, float g_scale_inv,
                           uint8_t* qm, float* m_meta, uint16_t* v, uint16_t* master,
                           uint8_t* w8, float* w8_meta, const oracle_hparams* hp, int64_t step,
                           int coupled) {
  float amax_w = 0.0f;
  int rc = adamw_lowbit_tensor(n, qg, gfmt, g_scale_inv, qm, m_meta, v, master, hp, step, coupled,
                               &amax_w);
  if (rc != 0) return rc;
  float s_w = oracle_scale(amax_w, (float)mf_max(&FMT_E4M3));
  for (int64_t i = 0; i < n; ++i) w8[i] = fp8_enc(&FMT_E4M3, f16_dec(master[i]) * s_w);
  w8_meta[0] = amax_w;
  w8_meta[1] = s_w;
  w8_meta[2] = 1.0f / s_w;
  return 0;
}
