/* Drives every function of oracle/oracle.c on a spread of inputs (binary32
 * bit patterns across all binades and specials, every FP8/FP16 code, empty
 * and one-element tensors, ragged sizes, all step variants over several
 * steps) so that the oracle can be run under AddressSanitizer and
 * UndefinedBehaviorSanitizer. Prints a checksum; any sanitizer report
 * aborts the run. Test infrastructure: built and run by
 * tests/test_sanitizers_cpu.py only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  double lr, beta1, beta2, eps, weight_decay;
} oracle_hparams;

int oracle_fp8_encode_array(const float* x, int64_t n, int fmt, uint8_t* out);
int oracle_fp8_decode_array(const uint8_t* codes, int64_t n, int fmt, float* out);
void oracle_f16_encode_array(const float* x, int64_t n, uint16_t* out);
void oracle_f16_decode_array(const uint16_t* h, int64_t n, float* out);
float oracle_fp8_max(int fmt);
float oracle_amax(const float* x, int64_t n);
float oracle_scale(float amax, float fmax);
int oracle_quantize_fp8(const float* x, int64_t n, int fmt, float amax, float* meta_out, uint8_t* q);
int oracle_quantize_fp8_prescaled(const float* x, int64_t n, int fmt, float amax, int world, float* meta_out,
                                  uint8_t* q);
int oracle_dequantize_fp8(const uint8_t* q, int64_t n, int fmt, float s_inv, float* out);
void oracle_adamw_constants(const oracle_hparams* hp, int64_t step, float* k);
void oracle_adamw_f32_tensor(int64_t n, const float* g, float* m, float* v, float* w, const oracle_hparams* hp,
                             int64_t step, int coupled);
int oracle_adamw_o2_tensor(int64_t n, const uint8_t* qg, int gfmt, float g_scale_inv, uint8_t* qm,
                           float* m_meta, uint16_t* v, uint16_t* w, const oracle_hparams* hp, int64_t step,
                           int coupled);
int oracle_adamw_o2_tensor_delayed(int64_t n, const uint8_t* qg, int gfmt, float g_scale_inv, uint8_t* qm,
                                   float* m_meta, uint16_t* v, uint16_t* w, const oracle_hparams* hp,
                                   int64_t step, int coupled);
int oracle_adamw_o2_tensor_scaled_v(int64_t n, const uint8_t* qg, int gfmt, float g_scale_inv, uint8_t* qm,
                                    float* m_meta, uint16_t* v, float* v_meta, uint16_t* w,
                                    const oracle_hparams* hp, int64_t step);
int oracle_adamw_o3_tensor(int64_t n, const uint8_t* qg, int gfmt, float g_scale_inv, uint8_t* qm,
                           float* m_meta, uint16_t* v, uint16_t* master, uint8_t* w8, float* w8_meta,
                           const oracle_hparams* hp, int64_t step, int coupled);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (uint32_t)(rng >> 16);
}
static float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static double uniform(void) { return (next_u32() + 0.5) / 4294967296.0; }
static float gauss(void) { return (float)(sqrt(-2.0 * log(uniform())) * cos(6.283185307179586 * uniform())); }

static uint64_t sum;
static void mix(const void* p, size_t bytes) {
  const unsigned char* b = (const unsigned char*)p;
  for (size_t i = 0; i < bytes; ++i) sum = sum * 1099511628211ull ^ b[i];
}

static int codec(void) {
  const int64_t n = 1 << 21;
  float* x = malloc(sizeof(float) * n);
  uint8_t* q = malloc(n);
  uint16_t* h = malloc(2 * n);
  float* y = malloc(sizeof(float) * n);
  if (!x || !q || !h || !y) return 1;
  for (int64_t i = 0; i < n; ++i) x[i] = from_bits(i < 65536 ? (uint32_t)i << 16 : next_u32());
  x[0] = INFINITY;
  x[1] = -INFINITY;
  x[2] = NAN;
  x[3] = -0.0f;
  for (int fmt = 0; fmt < 2; ++fmt) {
    if (oracle_fp8_encode_array(x, n, fmt, q) != 0) return 2;
    mix(q, n);
    uint8_t codes[256];
    for (int c = 0; c < 256; ++c) codes[c] = (uint8_t)c;
    if (oracle_fp8_decode_array(codes, 256, fmt, y) != 0) return 3;
    mix(y, 256 * sizeof(float));
    (void)oracle_fp8_max(fmt);
  }
  if (oracle_fp8_encode_array(x, 4, 7, q) != -1 || oracle_fp8_decode_array(q, 4, -1, y) != -1) return 4;
  oracle_f16_encode_array(x, n, h);
  mix(h, 2 * n);
  for (int64_t i = 0; i < 65536; ++i) h[i] = (uint16_t)i;
  oracle_f16_decode_array(h, 65536, y);
  mix(y, 65536 * sizeof(float));
  float specials[] = {0.0f, -0.0f, 1e-45f, 1.0f, 448.0f, 3.4e38f, INFINITY, NAN};
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 8; ++j) {
      float s = oracle_scale(specials[i], specials[j] == 0.0f ? 448.0f : specials[j]);
      mix(&s, 4);
    }
  float a = oracle_amax(x, n);
  float e = oracle_amax(x, 0);
  mix(&a, 4);
  mix(&e, 4);
  free(x);
  free(q);
  free(h);
  free(y);
  return 0;
}

static int steps(void) {
  const int64_t sizes[] = {0, 1, 2, 15, 16, 17, 1000, 4097, 65537};
  const oracle_hparams hps[] = {{1e-3, 0.9, 0.999, 1e-8, 0.01}, {5e-3, 0.8, 0.99, 1e-7, 0.05},
                                {0.0, 0.0, 0.0, 1.0, 0.0}};
  for (size_t si = 0; si < sizeof sizes / sizeof sizes[0]; ++si) {
    const int64_t n = sizes[si];
    const size_t cap = (size_t)(n > 0 ? n : 1);
    float* g = malloc(sizeof(float) * cap);
    float *m32 = calloc(cap, sizeof(float)), *v32 = calloc(cap, sizeof(float)), *w32 = malloc(sizeof(float) * cap);
    uint8_t *qg = malloc(cap), *qm = calloc(cap, 1), *w8 = calloc(cap, 1);
    uint16_t *v = calloc(cap, 2), *w = malloc(2 * cap), *vs = calloc(cap, 2);
    float* wf = malloc(sizeof(float) * cap);
    float* deq = malloc(sizeof(float) * cap);
    if (!g || !m32 || !v32 || !w32 || !qg || !qm || !w8 || !v || !w || !vs || !wf || !deq) return 10;
    for (int64_t i = 0; i < n; ++i) wf[i] = 0.02f * gauss();
    oracle_f16_encode_array(wf, n, w);
    memcpy(w32, wf, sizeof(float) * cap);
    for (size_t hi = 0; hi < sizeof hps / sizeof hps[0]; ++hi)
      for (int gfmt = 0; gfmt < 2; ++gfmt)
        for (int variant = 0; variant < 6; ++variant) {
          float m_meta[4] = {0.0f, 1.0f, 1.0f, 0.0f}, w8_meta[4] = {0}, v_meta[4] = {0.0f, 1.0f, 1.0f, 0.0f};
          memset(qm, 0, cap);
          memset(v, 0, 2 * cap);
          memset(vs, 0, 2 * cap);
          for (int64_t step = 1; step <= 3; ++step) {
            for (int64_t i = 0; i < n; ++i) g[i] = 1e-3f * gauss() * (step == 3 ? 1000.0f : 1.0f);
            float meta[4];
            const float amax = oracle_amax(g, n);
            if (oracle_quantize_fp8(g, n, gfmt, amax, meta, qg) != 0) return 11;
            if (oracle_quantize_fp8_prescaled(g, n, gfmt, amax, 4, meta + 1, qg) != 0) return 12;
            if (oracle_quantize_fp8(g, n, gfmt, amax, meta, qg) != 0) return 13;
            if (oracle_dequantize_fp8(qg, n, gfmt, meta[2], deq) != 0) return 14;
            int rc = 0;
            switch (variant) {
              case 0:
              case 1:
                rc = oracle_adamw_o2_tensor(n, qg, gfmt, meta[2], qm, m_meta, v, w, &hps[hi], step, variant);
                break;
              case 2:
              case 3:
                rc = oracle_adamw_o3_tensor(n, qg, gfmt, meta[2], qm, m_meta, v, w, w8, w8_meta, &hps[hi], step,
                                            variant - 2);
                break;
              case 4:
                rc = oracle_adamw_o2_tensor_delayed(n, qg, gfmt, meta[2], qm, m_meta, v, w, &hps[hi], step, 0);
                break;
              default:
                rc = oracle_adamw_o2_tensor_scaled_v(n, qg, gfmt, meta[2], qm, m_meta, vs, v_meta, w, &hps[hi],
                                                     step);
            }
            if (rc != 0) return 15;
            oracle_adamw_f32_tensor(n, g, m32, v32, w32, &hps[hi], step, variant & 1);
            mix(qm, (size_t)n);
            mix(v, 2 * (size_t)n);
            mix(w, 2 * (size_t)n);
            mix(m_meta, sizeof m_meta);
            mix(deq, sizeof(float) * (size_t)n);
          }
        }
    float k[9];
    oracle_adamw_constants(&hps[0], 1000000, k);
    mix(k, sizeof k);
    free(g);
    free(m32);
    free(v32);
    free(w32);
    free(qg);
    free(qm);
    free(w8);
    free(v);
    free(w);
    free(vs);
    free(wf);
    free(deq);
  }
  return 0;
}

int main(void) {
  int rc = codec();
  if (rc) {
    fprintf(stderr, "codec failed: %d\n", rc);
    return rc;
  }
  rc = steps();
  if (rc) {
    fprintf(stderr, "steps failed: %d\n", rc);
    return rc;
  }
  printf("oracle driver ok %016llx\n", (unsigned long long)sum);
  return 0;
}
