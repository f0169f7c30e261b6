/* A plain C11 client of include/msamp.h that runs on the GPU with no Python
 * or PyTorch: device memory and a stream from the HIP runtime API, then
 * msamp_amax, msamp_quantize_fp8 and one O2 and one O3 step on the
 * one-element worked example (w = fp16(0.02), g = 1e-3), and two O3 steps on
 * a three-element example. It prints every output bit pattern; the test that
 * runs it compares them with the oracle. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "msamp.h"

#define HIP_OK(x)                                                  \
  do {                                                             \
    hipError_t e_ = (x);                                           \
    if (e_ != hipSuccess) {                                        \
      fprintf(stderr, "%s failed: %d\n", #x, (int)e_);             \
      return 1;                                                    \
    }                                                              \
  } while (0)
#define MS_OK(x)                                                   \
  do {                                                             \
    msamp_status s_ = (x);                                         \
    if (s_ != MSAMP_OK) {                                          \
      fprintf(stderr, "%s: %s\n", #x, msamp_last_error());         \
      return 2;                                                    \
    }                                                              \
  } while (0)

static uint32_t bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* One tensor of k <= 16 elements through 'steps' steps of the O2 (o3 = 0)
 * or O3 layout; prints the state after the last step. */
static int run(const char* name, int o3, int k, const uint16_t* w0, const float* grads, int steps,
               hipStream_t s) {
  /* one 1 KiB device block per role: every base is 256-byte aligned */
  char* d = NULL;
  HIP_OK(hipMalloc((void**)&d, 8 * 1024));
  HIP_OK(hipMemset(d, 0, 8 * 1024));
  float* x = (float*)(d + 0 * 1024);
  uint8_t* q = (uint8_t*)(d + 1 * 1024);
  uint8_t* m = (uint8_t*)(d + 2 * 1024);
  uint16_t* v = (uint16_t*)(d + 3 * 1024);
  uint16_t* w = (uint16_t*)(d + 4 * 1024);
  uint8_t* w8 = (uint8_t*)(d + 5 * 1024);
  msamp_meta* gmeta = (msamp_meta*)(d + 6 * 1024);
  msamp_meta* mmeta = gmeta + 1;
  msamp_meta* w8meta = gmeta + 2;
  const msamp_meta init[3] = {{0, 1, 1, 0}, {0, 1, 1, 0}, {0, 1, 1, 0}};
  HIP_OK(hipMemcpy(gmeta, init, sizeof init, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(w, w0, (size_t)k * 2, hipMemcpyHostToDevice));
  const int64_t numel[1] = {k};
  const float* xs[1] = {x};
  uint8_t* qs[1] = {q};
  uint8_t* ms[1] = {m};
  uint16_t* vs[1] = {v};
  uint16_t* ws[1] = {w};
  uint8_t* w8s[1] = {w8};
  const msamp_adamw_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01};
  for (int t = 1; t <= steps; ++t) {
    HIP_OK(hipMemcpy(x, grads + (size_t)(t - 1) * k, (size_t)k * 4, hipMemcpyHostToDevice));
    MS_OK(msamp_amax(1, xs, numel, gmeta, s));
    MS_OK(msamp_quantize_fp8(1, xs, numel, MSAMP_FP8_E4M3, gmeta, qs, s));
    if (o3)
      MS_OK(msamp_adamw_o3_step(1, numel, (const uint8_t* const*)qs, MSAMP_FP8_E4M3, gmeta, ms, mmeta, vs,
                                ws, w8s, w8meta, &hp, t, s));
    else
      MS_OK(msamp_adamw_o2_step(1, numel, (const uint8_t* const*)qs, MSAMP_FP8_E4M3, gmeta, ms, mmeta, vs,
                                ws, &hp, t, s));
  }
  HIP_OK(hipStreamSynchronize(s));
  uint8_t hq[16], hm[16], hw8[16];
  uint16_t hv[16], hw[16];
  msamp_meta hmeta[3];
  HIP_OK(hipMemcpy(hq, q, (size_t)k, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hm, m, (size_t)k, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hw8, w8, (size_t)k, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hv, v, (size_t)k * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hw, w, (size_t)k * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hmeta, gmeta, sizeof hmeta, hipMemcpyDeviceToHost));
  printf("%s", name);
  for (int i = 0; i < 3; ++i)
    printf(" meta%d=%08x,%08x,%08x", i, bits(hmeta[i].amax), bits(hmeta[i].scale), bits(hmeta[i].scale_inv));
  printf(" q=");
  for (int i = 0; i < k; ++i) printf("%02x", hq[i]);
  printf(" m=");
  for (int i = 0; i < k; ++i) printf("%02x", hm[i]);
  printf(" v=");
  for (int i = 0; i < k; ++i) printf("%04x", hv[i]);
  printf(" w=");
  for (int i = 0; i < k; ++i) printf("%04x", hw[i]);
  printf(" w8=");
  for (int i = 0; i < k; ++i) printf("%02x", hw8[i]);
  printf("\n");
  HIP_OK(hipFree(d));
  return 0;
}

int main(void) {
  if (msamp_abi_version() != MSAMP_ABI_VERSION) return 3;
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  const uint16_t w1[1] = {0x251F};
  const float g1[1] = {1e-3f};
  const uint16_t w3[3] = {0x3800, 0xA51F, 0x0000};
  const float g3[6] = {0.5f, 1e-3f, 0.0f, -0.25f, 2e-3f, 0.0f};
  int rc = run("one_o2", 0, 1, w1, g1, 1, s);
  if (!rc) rc = run("one_o3", 1, 1, w1, g1, 1, s);
  if (!rc) rc = run("three_o3", 1, 3, w3, g3, 2, s);
  HIP_OK(hipStreamDestroy(s));
  if (!rc) printf("c abi gpu ok\n");
  return rc;
}
