/* A plain C11 client of include/msamp.h: the header compiles as C, the
 * program links against libmsamp.so, and calls that fail validation return
 * their status and message without touching a GPU (nothing is enqueued). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "msamp.h"

#define EXPECT(cond, code)                                            \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "failed: %s (%s)\n", #cond, msamp_last_error()); \
      return (code);                                                  \
    }                                                                 \
  } while (0)

int main(void) {
  EXPECT(msamp_abi_version() == MSAMP_ABI_VERSION, 1);
  EXPECT(sizeof(msamp_meta) == 16, 2);

  int64_t numel[2] = {32, 0};
  const float* x[2] = {NULL, NULL};
  msamp_meta* meta = (msamp_meta*)(uintptr_t)0x10000;
  EXPECT(msamp_amax(1, x, numel, meta, NULL) == MSAMP_E_INVALID_ARG, 3);
  EXPECT(strstr(msamp_last_error(), "NULL") != NULL, 4);
  EXPECT(msamp_amax(0, NULL, NULL, NULL, NULL) == MSAMP_OK, 5);
  EXPECT(msamp_last_error()[0] == '\0', 6);
  EXPECT(msamp_amax(-1, x, numel, meta, NULL) == MSAMP_E_INVALID_ARG, 7);

  const float* xm[1] = {(const float*)(uintptr_t)0x100004};
  EXPECT(msamp_amax(1, xm, numel, meta, NULL) == MSAMP_E_MISALIGNED, 8);

  uint8_t* q[1] = {(uint8_t*)(uintptr_t)0x200000};
  const float* xa[1] = {(const float*)(uintptr_t)0x100000};
  EXPECT(msamp_quantize_fp8(1, xa, numel, (msamp_fp8_format)7, meta, q, NULL) ==
             MSAMP_E_INVALID_ARG, 9);

  const uint8_t* g[1] = {(const uint8_t*)(uintptr_t)0x300000};
  uint8_t* m[1] = {(uint8_t*)(uintptr_t)0x400000};
  uint16_t* v[1] = {(uint16_t*)(uintptr_t)0x500000};
  uint16_t* w[1] = {(uint16_t*)(uintptr_t)0x600000};
  msamp_adamw_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01};
  EXPECT(msamp_adamw_o2_step(1, numel, g, MSAMP_FP8_E4M3, meta, m, meta, v, w, &hp, 0, NULL) ==
             MSAMP_E_INVALID_ARG, 10); /* step 0 */
  hp.beta2 = 1.0;
  EXPECT(msamp_adamw_o2_step(1, numel, g, MSAMP_FP8_E4M3, meta, m, meta, v, w, &hp, 1, NULL) ==
             MSAMP_E_INVALID_ARG, 11);
  EXPECT(strstr(msamp_last_error(), "beta2") != NULL, 12);
  EXPECT(strcmp(msamp_kernel_name(MSAMP_KERNEL_AMAX), "amax") == 0, 13);

  /* the quantizing steps validate the binary32 gradient list too */
  hp.beta2 = 0.999;
  const float* xf[1] = {(const float*)(uintptr_t)0x700008};
  uint8_t* gq[1] = {(uint8_t*)(uintptr_t)0x300000};
  EXPECT(msamp_quantize_adamw_o2_step(1, numel, xf, MSAMP_FP8_E4M3, meta, gq, m, meta, v, w, &hp, 1, NULL) ==
             MSAMP_E_MISALIGNED, 14);
  EXPECT(strstr(msamp_last_error(), "grad_f32[0]") != NULL, 15);
  xf[0] = (const float*)(uintptr_t)0x700000;
  uint8_t* w8[1] = {NULL};
  EXPECT(msamp_quantize_adamw_o3_step(1, numel, xf, MSAMP_FP8_E5M2, meta, gq, m, meta, v, w, w8, meta, &hp, 1,
                                      NULL) == MSAMP_E_INVALID_ARG, 16);
  EXPECT(strstr(msamp_last_error(), "weight_fp8[0]") != NULL, 17);

  /* the Adam and device-constant forms check the same lists, and the
   * device-constant forms refuse a NULL or misaligned constants record */
  xf[0] = (const float*)(uintptr_t)0x700008;
  EXPECT(msamp_quantize_adam_o2_step(1, numel, xf, MSAMP_FP8_E4M3, meta, gq, m, meta, v, w, &hp, 1, NULL) ==
             MSAMP_E_MISALIGNED, 26);
  xf[0] = (const float*)(uintptr_t)0x700000;
  EXPECT(msamp_quantize_adam_o3_step(1, numel, xf, MSAMP_FP8_E5M2, meta, gq, m, meta, v, w, w8, meta, &hp, 1,
                                     NULL) == MSAMP_E_INVALID_ARG, 27);
  EXPECT(msamp_quantize_adamw_o2_step_devconst(1, numel, xf, MSAMP_FP8_E4M3, meta, gq, m, meta, v, w, NULL, 0,
                                               NULL) == MSAMP_E_INVALID_ARG, 28);
  EXPECT(strstr(msamp_last_error(), "consts") != NULL, 29);
  const msamp_step_constants* kbad = (const msamp_step_constants*)(uintptr_t)0xA00002;
  EXPECT(msamp_quantize_adamw_o3_step_devconst(1, numel, xf, MSAMP_FP8_E4M3, meta, gq, m, meta, v, w, w8, meta,
                                               kbad, 1, NULL) == MSAMP_E_MISALIGNED, 30);

  /* measurement streams: size, alignment and overlap checks */
  void* src = (void*)(uintptr_t)0x800000;
  void* dst = (void*)(uintptr_t)0x800100;
  EXPECT(msamp_stream_probe(MSAMP_STREAM_READ, src, NULL, 24, NULL) == MSAMP_E_INVALID_ARG, 18);
  EXPECT(msamp_stream_probe(MSAMP_STREAM_COPY, src, dst, 4096, NULL) == MSAMP_E_INVALID_ARG, 19);
  EXPECT(strstr(msamp_last_error(), "overlap") != NULL, 20);
  EXPECT(msamp_stream_probe(MSAMP_STREAM_COPY, src, (void*)(uintptr_t)0x900008, 16, NULL) == MSAMP_E_MISALIGNED,
         21);
  EXPECT(msamp_stream_probe((msamp_stream_kind)5, src, dst, 16, NULL) == MSAMP_E_INVALID_ARG, 22);
  EXPECT(msamp_stream_probe(MSAMP_STREAM_READ, src, NULL, 0, NULL) == MSAMP_OK, 23);

  /* the allocation-free step refuses a list whose tables exceed its static
   * array, before any device work */
  int64_t huge[1] = {(int64_t)1 << 35};
  EXPECT(msamp_adamw_o2_step_noalloc(1, huge, g, MSAMP_FP8_E4M3, meta, m, meta, v, w, &hp, 1, NULL) ==
             MSAMP_E_INVALID_ARG, 24);
  EXPECT(strstr(msamp_last_error(), "at most") != NULL, 25);
  printf("c abi ok\n");
  return 0;
}
