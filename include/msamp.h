/*
 * msamp.h -- C ABI of the MI355X (gfx950) library for the per-tensor-scaled
 * low-precision AdamW step of MS-AMP's O2 and O3 optimization levels, with
 * the per-tensor amax reductions and saturating FP8 casts around it.
 *
 * Sources of the operations (web pages):
 *   [OL]  MS-AMP docs, "Optimization Level": sections O2 and O3 and the
 *         optimization-level table (weight gradient FP8; optimizer states
 *         FP8 + FP16; O2 weight FP16 with no master; O3 weight FP8 with an
 *         FP16 master weight).
 *   [RD]  MS-AMP README (giters.com mirror), "Usage": the recognized
 *         optimizers are torch.optim.Adam and torch.optim.AdamW; "Features":
 *         memory-limited operations read one byte per element.
 *   [TE]  TransformerEngine issue #131, "FP8 questions": the two FP8 formats
 *         E4M3 and E5M2; converting a tensor between precisions costs a
 *         full read and write of it.
 * The arithmetic the pages leave open is fixed as follows (identical in every
 * entry point):
 *   - FP8 formats are the OCP encodings: E4M3 (max 448, no Inf, NaN =
 *     S.1111.111) and E5M2 (max 57344, IEEE Inf/NaN).
 *   - Casts to FP8 round to nearest, ties to even, keep subnormals and
 *     saturate: finite overflow and +-Inf give +-max, NaN gives 0x7F with
 *     the input's sign bit. Casts to FP16 are IEEE round-to-nearest-even.
 *   - amax of a tensor is the largest |x| compared as the unsigned integer
 *     (bits & 0x7FFFFFFF): -0 counts as +0, NaN beats Inf beats finite, an
 *     empty tensor gives 0.
 *   - scale = fp8_max / amax, except scale = 1 when amax is 0, Inf or NaN or
 *     when that quotient is not a finite positive binary32; scale_inv = 1 /
 *     scale; a code c stands for decode(c) * scale_inv.
 *   - AdamW is PyTorch's decoupled-weight-decay AdamW in binary32 with the
 *     new first moment rescaled by its own amax (two passes):
 *       B1=b1 OB1=1-b1 B2=b2 OB2=1-b2 EPS=eps SS=lr/(1-b1^t)
 *       IBS=1/sqrt(1-b2^t) DEC=1-lr*wd      (binary64, rounded once)
 *       g   = decode(g_code) * g_scale_inv
 *       m0  = decode_e4m3(m_code) * m_scale_inv_old
 *       m1  = fma(B1, m0, OB1*g)
 *       v1  = fma(B2, v0, OB2*(g*g))
 *       den = fma(sqrt(v1), IBS, EPS)
 *       w1  = fma(-SS, m1/den, w0*DEC)
 *       m scale from amax(m1); m_code = enc_e4m3(m1*m_scale);
 *       v = fp16(v1); w = fp16(w1)
 *     Only the four fma above are fused; every other operation is a
 *     separately rounded IEEE binary32 operation (division and square root
 *     correctly rounded).
 *
 * Conventions for every entry point:
 *   - n is the number of tensors (n >= 0; n == 0 is a no-op returning OK).
 *   - Pointer arrays (x, q, grad, ...) and numel are HOST arrays of length n,
 *     read only during the call. The pointers they hold are DEVICE pointers
 *     to contiguous, flat 1-D arrays with a 16-byte aligned base. A base on
 *     a 64-byte boundary moves fewer bytes: with 16-byte aligned bases (FP8
 *     code arrays packed back to back) the stress list's 20,064 tensors
 *     moved 2-6% more bytes than with 256-byte aligned ones.
 *   - Meta arrays are DEVICE arrays of n msamp_meta records.
 *   - A tensor with numel == 0 may have NULL pointers.
 *   - stream is a hipStream_t (NULL = the null stream), passed as void* so
 *     that this header needs no HIP header and compiles as plain C (a C
 *     caller, or a binding that only holds the stream's address, includes
 *     nothing else). All work is enqueued on it; nothing synchronizes the
 *     host. Inputs must stay alive and
 *     unmodified until that work completes. The calling thread's current HIP
 *     device must be the device of the tensors and of the stream: the cached
 *     tables are built on, and looked up for, the current device.
 *   - The caller owns every tensor and meta array. The library owns cached
 *     device tables (tensor descriptors, chunk maps, amax scratch) keyed on
 *     the pointer lists; msamp_release_cache() frees them. The first call on
 *     a list builds its tables (device and pinned host allocations, one
 *     upload on the stream); at most 64 lists (512 MB of tables) are kept,
 *     and evicting the least recently used one first waits for its device.
 *   - Graph capture: a call whose stream is being captured uses the tables
 *     built by an earlier eager call on the same lists (building them
 *     allocates, which capture forbids) and PINS them: the captured kernels
 *     keep their addresses, so pinned tables are neither evicted nor freed
 *     by msamp_release_cache() (the cache may then exceed its bounds) until
 *     msamp_unpin_captured_tables() is called, after the graphs that use
 *     them have been destroyed or will not be replayed again.
 *   - Calls that use the same tensor lists must be ordered (same stream, or
 *     synchronized): they share that list's amax scratch.
 *   - Entry points may be called from several host threads at once; they
 *     take an internal lock while they look up the cached tables and enqueue
 *     their kernels, so a table is never freed under a call that uses it.
 *   - Errors: every argument is validated before anything is enqueued; on an
 *     error nothing is enqueued and a status other than MSAMP_OK is returned,
 *     with a description from msamp_last_error() (per thread). No C++
 *     exception crosses this interface. Faults inside kernels surface at the
 *     caller's next synchronization. A call whose size and pointer arrays are
 *     byte-equal to those of one of the last few lists of the same kind of
 *     call reuses that list's tables without re-checking each tensor (those
 *     arrays passed the checks when the tables were built); this changes the
 *     cost of a call, never its outcome.
 *   - Different roles must not alias (e.g. exp_avg and weight); this is not
 *     checked.
 */
#ifndef MSAMP_H_
#define MSAMP_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSAMP_ABI_VERSION 3

typedef enum {
  MSAMP_OK = 0,
  MSAMP_E_INVALID_ARG = 1, /* bad count, NULL pointer, bad format or hyperparameter */
  MSAMP_E_MISALIGNED = 2,  /* a tensor base is not 16-byte aligned */
  MSAMP_E_HIP = 3,         /* a HIP runtime call or kernel launch failed */
  MSAMP_E_NO_MEMORY = 4    /* the library could not allocate its tables */
} msamp_status;

typedef enum {
  MSAMP_FP8_E4M3 = 0, /* OCP E4M3, max 448 */
  MSAMP_FP8_E5M2 = 1  /* OCP E5M2, max 57344 */
} msamp_fp8_format;

/* Per-tensor scaling record (16 bytes). */
typedef struct {
  float amax;      /* largest |x| of the tensor it describes */
  float scale;     /* fp8_max / amax (see the scale rule above) */
  float scale_inv; /* 1 / scale: value = decode(code) * scale_inv */
  float reserved;  /* written as 0 by the library */
} msamp_meta;

/* AdamW hyperparameters (PyTorch's torch.optim.AdamW meaning, [RD] "Usage").
 * Valid: lr >= 0, 0 <= beta1 < 1, 0 <= beta2 < 1, eps > 0, weight_decay >= 0,
 * all finite. */
typedef struct {
  double lr;
  double beta1;
  double beta2;
  double eps;
  double weight_decay;
} msamp_adamw_hparams;

/* Version of this interface (MSAMP_ABI_VERSION). */
int msamp_abi_version(void);

/* Description of the last error of the calling thread ("" if none). */
const char* msamp_last_error(void);

/*
 * msamp_amax -- per-tensor amax of binary32 tensors ([OL] per-tensor scaled
 * FP8 gradients; [TE]: a format cast costs one full pass over the tensor).
 *   x[t]      device float[numel[t]]
 *   meta[t]   device; .amax is written, the other fields are left unchanged
 * Reads 4 bytes per element.
 */
msamp_status msamp_amax(int32_t n, const float* const* x, const int64_t* numel,
                        msamp_meta* meta, void* stream);

/*
 * msamp_quantize_fp8 -- saturating FP8 cast of binary32 tensors with their
 * per-tensor scale ([OL] FP8 weight gradient; [TE] E4M3/E5M2).
 *   x[t]      device float[numel[t]]
 *   meta[t]   device; .amax is READ (normally written by msamp_amax; a
 *             smaller caller value saturates the outliers), .scale and
 *             .scale_inv are written, .reserved is written as 0
 *   q[t]      device uint8[numel[t]]: enc(x * scale)
 * Reads 4 and writes 1 byte per element.
 */
msamp_status msamp_quantize_fp8(int32_t n, const float* const* x, const int64_t* numel,
                                msamp_fp8_format fmt, msamp_meta* meta, uint8_t* const* q,
                                void* stream);

/*
 * msamp_quantize_fp8_prescaled -- the quantize before an FP8 gradient
 * all-reduce over world_size ranks ([OL] O1: FP8 weight gradients and FP8
 * all-reduce). meta[t].amax must hold the common amax of tensor t over all
 * ranks (the caller's all-reduce MAX of the per-rank msamp_amax results);
 * the scale is scale(amax * world_size) with the product rounded to
 * binary32, so the sum of the ranks' values stays within the FP8 range.
 * world_size >= 1 (1 is msamp_quantize_fp8). Other arguments, outputs and
 * errors as msamp_quantize_fp8.
 */
msamp_status msamp_quantize_fp8_prescaled(int32_t n, const float* const* x, const int64_t* numel,
                                          msamp_fp8_format fmt, msamp_meta* meta,
                                          int32_t world_size, uint8_t* const* q, void* stream);

/*
 * msamp_dequantize_fp8 -- out = decode(q) * meta.scale_inv (binary32): the
 * value an FP8 tensor with per-tensor scaling stands for ([OL] table: the
 * weight gradient, the first moment and the O3 weight are FP8 with a
 * per-tensor scale; [TE]: the cast back costs a full pass over the tensor).
 *   q[t]      device uint8[numel[t]]
 *   meta[t]   device, read (.scale_inv)
 *   out[t]    device float[numel[t]]
 * Reads 1 and writes 4 bytes per element. Errors as msamp_quantize_fp8.
 */
msamp_status msamp_dequantize_fp8(int32_t n, const uint8_t* const* q, const int64_t* numel,
                                  msamp_fp8_format fmt, const msamp_meta* meta,
                                  float* const* out, void* stream);

/*
 * msamp_adamw_o2_step -- one AdamW step in the O2 layout ([OL] section O2
 * and table row "MS-AMP O2": weight FP16, no master, gradient FP8,
 * optimizer states FP8 + FP16), in place.
 *   numel[t]          host, elements of tensor t
 *   grad[t]           device uint8 FP8 codes in grad_fmt, read
 *   grad_meta[t]      device, read (.scale_inv)
 *   exp_avg[t]        device uint8 E4M3 codes of the first moment, in/out
 *   exp_avg_meta[t]   device, in (.scale_inv of the stored codes) / out
 *                     ({amax, scale, scale_inv} of the new codes)
 *   exp_avg_sq[t]     device binary16 bits of the second moment, in/out
 *   weight[t]         device binary16 bits of the weight, in/out
 *   hp                host hyperparameters
 *   step              1-based step count after increment (t >= 1); the
 *                     library keeps no step state
 * Initial state: exp_avg codes 0, exp_avg_meta {0, 1, 1, 0}, exp_avg_sq 0.
 * Two passes: 13 bytes per element (read g, m; then read g, m, v, w and
 * write m, v, w). Non-finite gradient codes are outside the contract (the
 * caller skips such steps, as GradScaler does in [RD] "Usage").
 */
msamp_status msamp_adamw_o2_step(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                 msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                 uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                 uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                 const msamp_adamw_hparams* hp, int64_t step, void* stream);

/*
 * msamp_adamw_o2_step_noalloc -- msamp_adamw_o2_step for callers that cannot
 * allocate device memory (tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, bit-identical results, and no allocation of
 * any kind in the call. Its tables (two u32 amax words per tensor, the
 * 64-byte descriptor of each tensor, 8 bytes per chunk of C elements) live
 * in a static device array of 4 MiB (MSAMP_NOALLOC_SCRATCH_BYTES) that each
 * device holds from its first call until the process ends. They are rebuilt
 * and copied into it on every call, synchronously: the call returns once
 * the earlier work on the stream has finished and the copy is done, then
 * the kernels run asynchronously as usual.
 * C = 4096 * clamp(floor(T / 1024), 1, 16) with T = sum_t ceil(numel[t] /
 * 4096): 65,536, or fewer for a list under 16,384 tiles (about 67M
 * elements), so that small lists still spread over every compute unit.
 * Large lists keep these chunks here, while msamp_adamw_o2_step runs their
 * passes over one-tile chunks (tables 8x larger than this array allows for
 * the 7B list) and splits the update pass of mid-size lists; the results
 * are the same, the update pass of such lists is slower here.
 * Limit: round256(8 n) + round256(64 n) + 8 * sum_t ceil(numel[t] / C)
 * <= MSAMP_NOALLOC_SCRATCH_BYTES (the Llama-2-13B list, 363 tensors and
 * 13.0e9 parameters, needs 1.6 MB); a larger list returns
 * MSAMP_E_INVALID_ARG before any device work.
 * Every call on a device uses that device's one array and leaves the amax
 * words at zero: calls that may overlap on one device (different streams or
 * threads with no ordering between them) race and give undefined results.
 * A stream being captured into a graph is rejected (MSAMP_E_INVALID_ARG).
 * Arguments, layouts and other errors as msamp_adamw_o2_step.
 */
#define MSAMP_NOALLOC_SCRATCH_BYTES (4u << 20)
msamp_status msamp_adamw_o2_step_noalloc(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                         msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                         uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                         uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                         const msamp_adamw_hparams* hp, int64_t step, void* stream);

/*
 * msamp_adamw_o3_step -- one AdamW step in the O3 layout ([OL] section O3
 * and table row "MS-AMP O3": FP16 master weight, FP8 regular weight), in
 * place. Arguments as msamp_adamw_o2_step, with the FP16 weight replaced by
 *   master[t]           device binary16 bits of the master weight, in/out
 *   weight_fp8[t]       device uint8 E4M3 codes, out: enc(master * s_w)
 *                       taken from the stored (rounded) new master
 *   weight_fp8_meta[t]  device, out: {amax_w, s_w, 1/s_w, 0}, amax_w over
 *                       the new master
 * Three passes: 16 bytes per element.
 */
msamp_status msamp_adamw_o3_step(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                 msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                 uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                 uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                 uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                 const msamp_adamw_hparams* hp, int64_t step, void* stream);

/*
 * msamp_quantize_adamw_o2_step / msamp_quantize_adamw_o3_step -- the
 * gradient quantize (msamp_quantize_fp8) and the AdamW step
 * (msamp_adamw_o2_step / msamp_adamw_o3_step) in one call, the quantize
 * done in the same pass as the step's pass 1: each FP8 gradient code is
 * computed once, stored to grad[t] and decoded from registers, so pass 1
 * does not read the codes back ([TE]: every cast between formats costs a
 * full pass over the tensor). Every output (codes, gradient scales, state,
 * meta) is bit-identical to msamp_quantize_fp8 followed by the step.
 *   grad_f32[t]  device binary32 gradient, read
 *   grad_meta[t] device, in (.amax, e.g. from msamp_amax) / out (.scale,
 *                .scale_inv, .reserved = 0), as msamp_quantize_fp8
 *   grad[t]      device uint8, out: the gradient's FP8 codes in grad_fmt
 *   other arguments, layouts and errors as msamp_adamw_o2_step /
 *   msamp_adamw_o3_step.
 * Passes: quantize + pass 1 (read g 4, m 1; write codes 1), pass 2 (11)
 * [, pass 3 (3)]: 17 bytes per element (O2) or 20 (O3), against 18 / 21 for
 * the two calls.
 */
msamp_status msamp_quantize_adamw_o2_step(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                          msamp_fp8_format grad_fmt, msamp_meta* grad_meta,
                                          uint8_t* const* grad, uint8_t* const* exp_avg,
                                          msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                                          uint16_t* const* weight, const msamp_adamw_hparams* hp,
                                          int64_t step, void* stream);
msamp_status msamp_quantize_adamw_o3_step(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                          msamp_fp8_format grad_fmt, msamp_meta* grad_meta,
                                          uint8_t* const* grad, uint8_t* const* exp_avg,
                                          msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                                          uint16_t* const* master, uint8_t* const* weight_fp8,
                                          msamp_meta* weight_fp8_meta, const msamp_adamw_hparams* hp,
                                          int64_t step, void* stream);

/* msamp_quantize_adam_o2_step / msamp_quantize_adam_o3_step -- the same for
 * torch.optim.Adam (coupled L2, see msamp_adam_o2_step): the fused pass also
 * reads the weight (O2) or master (O3), 8 bytes per element, 19 (O2) or 22
 * (O3) bytes per element in all against 20 / 23 for the two calls. */
msamp_status msamp_quantize_adam_o2_step(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                         msamp_fp8_format grad_fmt, msamp_meta* grad_meta, uint8_t* const* grad,
                                         uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                         uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                         const msamp_adamw_hparams* hp, int64_t step, void* stream);
msamp_status msamp_quantize_adam_o3_step(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                         msamp_fp8_format grad_fmt, msamp_meta* grad_meta, uint8_t* const* grad,
                                         uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                         uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                         uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                         const msamp_adamw_hparams* hp, int64_t step, void* stream);

/*
 * msamp_adam_o2_step / msamp_adam_o3_step -- the same steps for
 * torch.optim.Adam, the other optimizer the MS-AMP README recognizes ([RD]
 * "Usage"): weight decay is an L2 term added to the gradient before the
 * moments, gd = fma(WD, w0, g) with WD = (float)weight_decay and w0 the
 * weight (O2) or master (O3) before the step, and the update has no
 * decoupled decay (DEC = 1). Arguments, layouts and errors as for the AdamW
 * entry points. Pass 1 also reads the weight: 15 bytes per element (O2),
 * 18 (O3).
 */
msamp_status msamp_adam_o2_step(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                const msamp_adamw_hparams* hp, int64_t step, void* stream);
msamp_status msamp_adam_o3_step(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                const msamp_adamw_hparams* hp, int64_t step, void* stream);

/*
 * msamp_adamw_o2_step_delayed -- ABLATION, not the step defined above: the
 * O2 AdamW step in one pass (11 bytes per element) with delayed scaling of
 * the first moment. The new codes are encoded with s = scale(exp_avg_meta
 * .amax) taken from the previous step, and exp_avg_meta becomes {amax of the
 * new moment, s, 1/s}. At step 1 the scale is 1 and the moment (~1e-4 at
 * gradient scale 1e-3) is stored as +-0; a moment that grows past 448/s
 * saturates. It exists to measure what the second pass costs and what it
 * buys. Arguments, layouts and errors as msamp_adamw_o2_step.
 */
msamp_status msamp_adamw_o2_step_delayed(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                         msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                         uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                         uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                         const msamp_adamw_hparams* hp, int64_t step, void* stream);

/*
 * msamp_adamw_o2_step_scaled_v -- ABLATION, not the step defined above: the
 * O2 AdamW step with a per-tensor-scaled FP16 second moment, which keeps v
 * from underflowing binary16 at small gradient scales. exp_avg_sq holds
 * fp16(v * s_v) and exp_avg_sq_meta[t] = {amax_v, s_v, 1/s_v, 0} with
 * s_v = scale(amax(v), 65504) (initial meta {0, 1, 1, 0}); v0 is decoded as
 * f32(code) * exp_avg_sq_meta.scale_inv. Pass 1 also reads v and reduces
 * amax(v1): 15 bytes per element. Other arguments, layouts and errors as
 * msamp_adamw_o2_step.
 */
msamp_status msamp_adamw_o2_step_scaled_v(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                          msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                          uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                          uint16_t* const* exp_avg_sq, msamp_meta* exp_avg_sq_meta,
                                          uint16_t* const* weight, const msamp_adamw_hparams* hp,
                                          int64_t step, void* stream);

/*
 * Graph-capturable steps. The per-step constants of the AdamW definition
 * above (B1 OB1 B2 OB2 EPS SS IBS DEC, plus WD = (float)weight_decay for
 * Adam's L2 term; DEC is exactly 1 for Adam), in that order. The *_devconst
 * steps read them from DEVICE memory when their kernels run instead of
 * taking hparams and step by value, so a captured launch sequence (HIP
 * graph) can be replayed for later steps after the caller rewrites the
 * record. Everything else about them is the step of the same layout.
 */
typedef struct {
  float b1, ob1, b2, ob2, eps, ss, ibs, dec, wd;
} msamp_step_constants;

/* Host only: the constants of step 'step' (>= 1) for AdamW (coupled = 0) or
 * Adam (coupled = 1), bit-identical to what the by-value steps use. */
msamp_status msamp_step_constants_compute(const msamp_adamw_hparams* hp, int64_t step, int coupled,
                                          msamp_step_constants* out);

/* msamp_adamw_o2_step / msamp_adam_o2_step (coupled = 0 / 1) with the
 * constants read from consts (device, 4-byte aligned, one record), which
 * must hold the record for the step being taken when the kernels run. */
msamp_status msamp_adamw_o2_step_devconst(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                          msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                          uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                          uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                          const msamp_step_constants* consts, int coupled,
                                          void* stream);

/* msamp_adamw_o3_step / msamp_adam_o3_step (coupled = 0 / 1) with the
 * constants read from consts (device), as above. */
msamp_status msamp_adamw_o3_step_devconst(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                          msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                          uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                          uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                          uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                          const msamp_step_constants* consts, int coupled,
                                          void* stream);

/* The quantizing steps (msamp_quantize_adamw_o2_step / _o3_step, and the
 * Adam ones with coupled = 1) with the constants read from consts (device,
 * 4-byte aligned, one record) when the kernels run, as above: the gradient
 * amax, this call and the constants' copy can be captured and replayed. */
msamp_status msamp_quantize_adamw_o2_step_devconst(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                                   msamp_fp8_format grad_fmt, msamp_meta* grad_meta,
                                                   uint8_t* const* grad, uint8_t* const* exp_avg,
                                                   msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                                                   uint16_t* const* weight, const msamp_step_constants* consts,
                                                   int coupled, void* stream);
msamp_status msamp_quantize_adamw_o3_step_devconst(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                                   msamp_fp8_format grad_fmt, msamp_meta* grad_meta,
                                                   uint8_t* const* grad, uint8_t* const* exp_avg,
                                                   msamp_meta* exp_avg_meta, uint16_t* const* exp_avg_sq,
                                                   uint16_t* const* master, uint8_t* const* weight_fp8,
                                                   msamp_meta* weight_fp8_meta, const msamp_step_constants* consts,
                                                   int coupled, void* stream);

/*
 * Split-phase steps, for a flat intra-tensor partition of the parameters
 * over data-parallel ranks (each rank holds a contiguous slice of every
 * tensor, as a ZeRO-style sharded optimizer does; [OL] O3: ZeRO and the FP8
 * weight broadcast). The per-tensor amaxes couple the slices: the caller
 * combines the ranks' values (an all-reduce MAX over the ranks; binary32
 * amaxes are non-negative, so MAX on their bits is exact) between phases.
 * The arguments are those of msamp_adamw_o2_step / msamp_adamw_o3_step for
 * the rank's slices, with coupled = 0 (AdamW) or 1 (Adam), plus device
 * float[n] amax arrays (4-byte aligned):
 *   phase 1  amax_m[t] <- amax of the slice's new first moment; no state
 *            is written.
 *   phase 2  the update with s_m = scale(amax_m[t], 448) from the global
 *            amax_m; exp_avg_meta[t] <- {amax_m, s_m, 1/s_m, 0}. O3 also
 *            writes amax_w[t] <- amax of the slice's new master.
 *   phase 3  (O3) the FP8 copy with s_w = scale(amax_w[t], 448) from the
 *            global amax_w; weight_fp8_meta[t] <- {amax_w, s_w, 1/s_w, 0}.
 * With the global MAX between the phases, every slice's result is bit-
 * identical to the slice of the unpartitioned step. Phase 1 and phase 2 of
 * one step take the same hp and step.
 */
msamp_status msamp_adamw_o2_step_phase1(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                        msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                        uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                        uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                        const msamp_adamw_hparams* hp, int64_t step, int coupled,
                                        float* amax_m, void* stream);
msamp_status msamp_adamw_o2_step_phase2(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                        msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                        uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                        uint16_t* const* exp_avg_sq, uint16_t* const* weight,
                                        const msamp_adamw_hparams* hp, int64_t step, int coupled,
                                        const float* amax_m, void* stream);
msamp_status msamp_adamw_o3_step_phase1(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                        msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                        uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                        uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                        uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                        const msamp_adamw_hparams* hp, int64_t step, int coupled,
                                        float* amax_m, void* stream);
msamp_status msamp_adamw_o3_step_phase2(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                        msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                        uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                        uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                        uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                        const msamp_adamw_hparams* hp, int64_t step, int coupled,
                                        const float* amax_m, float* amax_w, void* stream);
msamp_status msamp_adamw_o3_step_phase3(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                                        msamp_fp8_format grad_fmt, const msamp_meta* grad_meta,
                                        uint8_t* const* exp_avg, msamp_meta* exp_avg_meta,
                                        uint16_t* const* exp_avg_sq, uint16_t* const* master,
                                        uint8_t* const* weight_fp8, msamp_meta* weight_fp8_meta,
                                        const float* amax_w, void* stream);

/* Frees every cached device table of the library (all devices) that is not
 * pinned by a graph capture, after waiting for the devices to finish. Safe to
 * call at any time from one thread while no other library call runs. */
msamp_status msamp_release_cache(void);

/* Unpins every table pinned by a graph capture (see "Graph capture" above);
 * call it once the graphs that use them are destroyed. The tables are then
 * evicted or released like any other. */
msamp_status msamp_unpin_captured_tables(void);

/* Cached tables: number of tensor lists, their device bytes, and how many of
 * them a graph capture pinned (each output may be NULL). */
msamp_status msamp_cache_stats(int64_t* lists, int64_t* bytes, int64_t* pinned);

/* ----------------------------------------------------------------------
 * Test- and measurement-facing entry points.
 * ---------------------------------------------------------------------- */

/* Element-wise device codec used by every kernel above, exposed so that it
 * can be compared with an independent codec on every input of interest:
 *   MSAMP_PROBE_F32_TO_E4M3 / _E5M2  in float[n]    -> out uint8[n] (unscaled
 *                                    saturating cast)
 *   MSAMP_PROBE_E4M3_TO_F32 / _E5M2  in uint8[n]    -> out float[n]
 *   MSAMP_PROBE_F32_TO_F16           in float[n]    -> out uint16[n]
 *   MSAMP_PROBE_F16_TO_F32           in uint16[n]   -> out float[n]
 * in/out are device pointers, 16-byte aligned; n >= 0. */
typedef enum {
  MSAMP_PROBE_F32_TO_E4M3 = 0,
  MSAMP_PROBE_F32_TO_E5M2 = 1,
  MSAMP_PROBE_E4M3_TO_F32 = 2,
  MSAMP_PROBE_E5M2_TO_F32 = 3,
  MSAMP_PROBE_F32_TO_F16 = 4,
  MSAMP_PROBE_F16_TO_F32 = 5
} msamp_probe_op;

msamp_status msamp_codec_probe(msamp_probe_op op, const void* in, void* out, int64_t n,
                               void* stream);

/*
 * msamp_rmw_probe -- MEASUREMENT AID, not part of the method: reads g, m, v
 * and w of an O2 step's tensor lists (or g, m, v and the master of an O3
 * list) and writes m, v and w back UNCHANGED, with the lanes, tiles and
 * launch shape of the update pass but none of its arithmetic: 6 bytes read
 * and 5 written per element. Its rate on the caller's own buffers is what
 * the memory system gives that traffic alone there: a reference for the
 * update pass, not a bound (the pass, whose arithmetic spaces out its
 * accesses, can run faster). Arguments
 * as msamp_adamw_o2_step; the same work must not run concurrently on these
 * tensors.
 */
msamp_status msamp_rmw_probe(int32_t n, const int64_t* numel, const uint8_t* const* grad,
                             uint8_t* const* exp_avg, uint16_t* const* exp_avg_sq,
                             uint16_t* const* weight, void* stream);

/*
 * msamp_quantize_pass1_probe -- MEASUREMENT AID, not part of the method:
 * the loads and stores of the fused gradient quantize + pass 1 of
 * msamp_quantize_adamw_o2_step without its arithmetic (same lanes, tiles and
 * launch): reads grad_f32 and exp_avg, and writes UNSPECIFIED values to the
 * gradient codes 'grad' (6 bytes per element). Its rate on the caller's own
 * buffers is what the memory system gives that traffic alone there (a
 * reference, not a bound). Arguments
 * and errors as msamp_quantize_adamw_o2_step (the lists must be the ones a
 * quantizing step uses, with exp_avg_sq and weight); no meta is touched.
 */
msamp_status msamp_quantize_pass1_probe(int32_t n, const int64_t* numel, const float* const* grad_f32,
                                        uint8_t* const* grad, uint8_t* const* exp_avg,
                                        uint16_t* const* exp_avg_sq, uint16_t* const* weight, void* stream);

/*
 * msamp_stream_probe -- MEASUREMENT AID, not part of the method: a plain
 * stream at the access shape of the library's kernels (16-byte accesses,
 * each wave instruction on 1 KB of consecutive memory, one 16 KB tile per
 * workgroup, non-temporal hints), giving the rates the memory system offers
 * a pure read and a copy, beside msamp_rmw_probe's read-modify-write:
 *   MSAMP_STREAM_READ  reads 'bytes' from src; dst is not used (may be NULL)
 *   MSAMP_STREAM_COPY  copies 'bytes' from src to dst (no overlap)
 * src, dst device, 16-byte aligned; bytes >= 0 and a multiple of 16. Invalid
 * arguments return MSAMP_E_INVALID_ARG / MSAMP_E_MISALIGNED before any launch.
 */
typedef enum { MSAMP_STREAM_READ = 0, MSAMP_STREAM_COPY = 1 } msamp_stream_kind;
msamp_status msamp_stream_probe(msamp_stream_kind kind, const void* src, void* dst, int64_t bytes,
                                void* stream);

/* Kernel timing with HIP events recorded on the launch stream around every
 * kernel the library enqueues (off by default). */
typedef enum {
  MSAMP_KERNEL_AMAX = 0,        /* msamp_amax reduction */
  MSAMP_KERNEL_QUANTIZE = 1,    /* msamp_quantize_fp8 */
  MSAMP_KERNEL_DEQUANTIZE = 2,  /* msamp_dequantize_fp8 */
  MSAMP_KERNEL_STEP_PASS1 = 3,  /* first-moment amax pass (O2 and O3) */
  MSAMP_KERNEL_O2_PASS2 = 4,    /* O2 update pass */
  MSAMP_KERNEL_O3_PASS2 = 5,    /* O3 update pass (+ master amax) */
  MSAMP_KERNEL_O3_PASS3 = 6,    /* O3 FP8 weight copy */
  MSAMP_KERNEL_FINALIZE = 7,    /* per-tensor meta write-back of a step */
  MSAMP_KERNEL_AMAX_FINALIZE = 8, /* amax write-back of msamp_amax */
  MSAMP_KERNEL_O2_DELAYED = 9,  /* one-pass delayed-scaling ablation */
  MSAMP_KERNEL_RMW_PROBE = 10,  /* msamp_rmw_probe (measurement aid) */
  MSAMP_KERNEL_QUANTIZE_PASS1 = 11, /* gradient quantize fused with pass 1 */
  MSAMP_KERNEL_READ_PROBE = 12, /* msamp_stream_probe, MSAMP_STREAM_READ */
  MSAMP_KERNEL_COPY_PROBE = 13, /* msamp_stream_probe, MSAMP_STREAM_COPY */
  MSAMP_KERNEL_QP1_PROBE = 14,  /* msamp_quantize_pass1_probe (measurement aid) */
  MSAMP_KERNEL_COUNT = 15
} msamp_kernel_kind;

/* on != 0 starts recording (and discards earlier records; the events for
 * the next 2048 launches are created here, outside the timed work); on == 0
 * stops. */
msamp_status msamp_profile_enable(int on);

/* Chooses the kernel kinds that get events (bit k = kind k; default: all).
 * Each pair of events costs the launch sequence some time, so a caller that
 * times a whole sequence selects only the kinds it needs. */
msamp_status msamp_profile_select(uint32_t kind_mask);

/* Waits for the recorded events and returns, for one kernel kind, the number
 * of launches and the summed duration in milliseconds since the last
 * msamp_profile_enable(1). */
msamp_status msamp_profile_read(msamp_kernel_kind kind, int64_t* launches, double* total_ms);

/* Name of a kernel kind (static string; "" for an unknown kind). */
const char* msamp_kernel_name(msamp_kernel_kind kind);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* MSAMP_H_ */
