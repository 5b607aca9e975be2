/*
 * fp4.h - C ABI of the MI355X (gfx950) online FP4 inference path.
 *
 * Three calls, matching the method's statement of the problem:
 *
 *   fp4_rotate_quantize   online: block-wise Hadamard rotation of bf16
 *                         activations fused with microscaled FP4 quantization.
 *   fp4_quantize_weights  offline: the same rotation and quantization applied
 *                         to a weight matrix, so the rotation is folded into W.
 *   fp4_linear            the W4A4 product Y = dq(Xq) dq(Wq)^T.
 *
 * Sources: "Bridging the Gap Between Promise and Performance for Microscaling
 * FP4 Quantization" (gist.science, German edition), Technische Zusammenfassung
 * §2 "Einführung von MR-GPTQ" (block-wise Hadamard rotations of weights and
 * activations) and §2 "GPU-Kernel-Unterstützung (QuTLASS)" (fused online
 * rotation + quantization kernel, 4-bit matmul); the same paper's English
 * abstract on chatpaper.ai (rotation fused into the weights, fast online
 * computation of the activations); §1 Problemstellung (MXFP4: 32 elements per
 * scale, NVFP4: 16).
 *
 * Conventions shared by every call:
 *  - Pointers named as device pointers must point to device memory of the
 *    current HIP device. The caller owns and allocates every buffer; the library
 *    allocates nothing. Its only state is a thread-local error string, per-device
 *    launch settings set up on first use, and the device array of the
 *    allocation-free decode call below.
 *  - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *    asynchronously; no call synchronises the host.
 *  - All arguments are validated before anything is launched. On a non-OK
 *    status nothing has been launched and no output has been written; the
 *    message is available from fp4_last_error().
 *  - bf16 X / W values must be finite, with |value| <= 2^100 (larger values may
 *    overflow inside the float32 rotation); NaN/Inf are outside the contract.
 */
#ifndef FP4_MI355X_H
#define FP4_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4_API __attribute__((visibility("default")))

/* Formats. MXFP4: groups of 32 E2M1 elements share one E8M0 (power-of-two)
 * scale. NVFP4: groups of 16 share one E4M3 scale, plus one float32 scale for
 * the whole tensor ("Unveiling the Potential of Quantization with MXFP4",
 * gist.science, Dutch edition, Technische samenvatting, Probleemstelling). */
enum { FP4_MXFP4 = 0, FP4_NVFP4 = 1 };

/* Scale rules of fp4_rotate_quantize_ex / fp4_quantize_weights_ex. */
enum {
  FP4_SCALE_STANDARD = 0,  /* the rules of fp4_rotate_quantize (both formats)                */
  FP4_SCALE_OCP_FLOOR = 1, /* MXFP4: e = floor(log2 alpha) - 2, maximum in [4, 8), saturated  */
  FP4_SCALE_OAS = 2,       /* MXFP4: overflow-aware scaling                                   */
  FP4_SCALE_FIT = 3,       /* both: least-squared-error neighbour of the standard scale       */
  FP4_TENSOR_SCALE_IN = 0x10 /* flag, NVFP4 only: *tensor_scale is an input (a given s_t)    */
};

/* Output dtypes of fp4_linear. */
enum { FP4_OUT_F32 = 0, FP4_OUT_BF16 = 1 };

/* Status codes (every call returns one). */
enum {
  FP4_OK = 0,
  FP4_E_NULLPTR = -1, /* a required pointer is NULL, or a forbidden one is not     */
  FP4_E_SHAPE = -2,   /* M, N or K out of range, K not a multiple of what is needed */
  FP4_E_BLOCK = -3,   /* Hadamard block not in {16, 32, 64, 128}                  */
  FP4_E_FORMAT = -4,  /* unknown format or output dtype                            */
  FP4_E_ALIGN = -5,   /* a pointer or leading dimension breaks the alignment rule  */
  FP4_E_HIP = -6      /* the HIP runtime reported an error at launch               */
};

/*
 * fp4_rotate_quantize - rotate every row of X by the block-diagonal Hadamard
 * matrix (blocks of `block` along K) and quantize it to MXFP4 or NVFP4.
 *
 * Per row, per aligned block of `block` elements: y = H_block x / sqrt(block),
 * computed in float32 as the fast Walsh-Hadamard transform with strides 1, 2,
 * 4, ... block/2 in that order (pairs (i, i+h) -> (x_i + x_{i+h}, x_i - x_{i+h}))
 * followed by one float32 multiply by fl32(1/sqrt(block)).
 * Then per group of g elements (g = 32 MXFP4, 16 NVFP4), with alpha = max |y|:
 *  MXFP4: e = smallest integer with alpha <= 6 * 2^e (the group maximum lands
 *         in (3, 6]), clamped to [-127, 127]; scale code = e + 127.
 *  NVFP4: T = max |y| over all of X; s_t = fl32(T / 2688) is written to
 *         *tensor_scale; scale code = nearest E4M3FN value to alpha / (6 s_t)
 *         (ties to even, saturating at 448); elements use u = fl32(y * R) with
 *         R = fl32(1 / fl32(d * s_t)), d the decoded group scale; a group with
 *         d * s_t < 2^-126 stores signed zeros; T == 0 stores all zeros, s_t = 0.
 * Element code: round-to-nearest-even of u = y / scale onto the E2M1 grid
 * {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at 6, bit 3 = sign of y.
 *
 *  X            device, bf16 [M, ldx] row-major; columns 0..K-1 are used.
 *               16-byte aligned; ldx >= K and ldx % 8 == 0.
 *  M            rows, M >= 1.   K: columns, K >= 1, K % block == 0, K % 32 == 0.
 *               M * (K / 32) <= 2^31 - 1 (32-element chunks are indexed in 32 bits)
 *               and ldx <= 2^40; larger shapes return FP4_E_SHAPE.
 *  block        16, 32, 64 or 128.
 *  fmt          FP4_MXFP4 or FP4_NVFP4.
 *  codes        device, uint8 [M, K/2]: byte j of a row holds element 2j in
 *               its low nibble, element 2j+1 in its high nibble. 16-byte aligned.
 *  scales       device, uint8 [M, K/g] row-major (E8M0 or E4M3FN codes).
 *               NVFP4: 2-byte aligned.
 *  tensor_scale NVFP4: device float[1]; receives s_t. MXFP4: must be NULL.
 *  stream       hipStream_t or NULL.
 * MXFP4 is one kernel launch; NVFP4 is three (the tensor-maximum pass, its
 * reduction to s_t, and the quantize pass), all on `stream`. Between the first
 * and the last of them the codes buffer holds intermediate per-workgroup maxima;
 * the quantize pass overwrites them. No atomics are used, so s_t is deterministic.
 */
FP4_API int fp4_rotate_quantize(const void *X, int64_t M, int64_t K, int64_t ldx, int block, int fmt,
                        uint8_t *codes, uint8_t *scales, float *tensor_scale, void *stream);

/*
 * fp4_quantize_weights - the same rotation and quantization on a weight matrix
 * W [N, K] (offline), so that the rotation cancels in the product:
 * (X R)(W R)^T = X W^T for the orthogonal block-diagonal R. Arguments as for
 * fp4_rotate_quantize with (W, N, ldw) in place of (X, M, ldx); the same
 * `block` and `fmt` must be used for X and W.
 */
FP4_API int fp4_quantize_weights(const void *W, int64_t N, int64_t K, int64_t ldw, int block, int fmt,
                         uint8_t *codes, uint8_t *scales, float *tensor_scale, void *stream);

/*
 * fp4_rotate_quantize_ex / fp4_quantize_weights_ex - the calls above with two
 * options of the quantizer; with scale_rule = FP4_SCALE_STANDARD and signs = NULL
 * they are identical to fp4_rotate_quantize / fp4_quantize_weights.
 *
 *  scale_rule  FP4_SCALE_STANDARD: as above.
 *              FP4_SCALE_OCP_FLOOR (MXFP4 only): e = floor(log2 alpha) - 2,
 *                clamped to [-127, 127]; the group maximum lands in [4, 8) and
 *                elements above 6 saturate.
 *              FP4_SCALE_OAS (MXFP4 only): overflow-aware scaling ("Unveiling the
 *                Potential of Quantization with MXFP4", gist.science, Dutch
 *                edition, Methodologie, 1. OAS): the standard e, lowered by one
 *                when alpha / 2^e lies in (3, 3.5], so the maximum lands in (6, 7]
 *                and saturates to 6 while smaller elements get twice the resolution.
 *              FP4_SCALE_FIT (both formats): data-free scale fitting ("Bridging the
 *                Gap Between Promise and Performance for Microscaling FP4
 *                Quantization", gist.science, German edition, Technische
 *                Zusammenfassung §2 "Einführung von MR-GPTQ", item 2: MXFP4 scales
 *                fitted to the data range, NVFP4 scales optimised for E4M3). Per
 *                group the standard scale and its two neighbours (MXFP4: e - 1,
 *                e + 1; NVFP4: the adjacent E4M3 codes, s_t unchanged) are tried in
 *                the order standard, smaller, larger; a candidate replaces the
 *                current one when its squared error is strictly smaller. The error
 *                is float32, summed in element order: d = fl32(y - q * s),
 *                acc = fl32(acc + fl32(d * d)), with q * s exact for MXFP4 and
 *                fl32(q * S), S = fl32(d_e4m3 * s_t), for NVFP4. Intended for
 *                weights: it costs about three quantizations.
 *              FP4_TENSOR_SCALE_IN may be OR-ed into FP4_SCALE_STANDARD or
 *                FP4_SCALE_FIT (NVFP4 only): the tensor scale s_t is read from
 *                *tensor_scale (a finite, non-negative float, e.g. a calibrated
 *                static activation scale) instead of being computed from this
 *                tensor; the word is left unchanged, the tensor-maximum pass is
 *                skipped (one launch, one pass over X), and group maxima above
 *                2688 s_t saturate at E4M3 448 and the elements at E2M1 6.
 *  signs       NULL, or device int8 [K], 16-byte aligned: the randomized block
 *              Hadamard R = D H with D = diag(signs). Channel k is negated before
 *              the rotation when signs[k] < 0 (entries are meant to be +1 or -1).
 *              X and W must be quantized with the same signs.
 * Other arguments, alignment rules and launches as for fp4_rotate_quantize.
 * Errors: FP4_E_FORMAT for an unknown rule or OCP_FLOOR / OAS with NVFP4;
 * FP4_E_ALIGN for misaligned signs.
 */
FP4_API int fp4_rotate_quantize_ex(const void *X, int64_t M, int64_t K, int64_t ldx, int block, int fmt,
                                   int scale_rule, const int8_t *signs, uint8_t *codes, uint8_t *scales,
                                   float *tensor_scale, void *stream);
FP4_API int fp4_quantize_weights_ex(const void *W, int64_t N, int64_t K, int64_t ldw, int block, int fmt,
                                    int scale_rule, const int8_t *signs, uint8_t *codes, uint8_t *scales,
                                    float *tensor_scale, void *stream);

/*
 * fp4_linear - Y[m, n] = sum_k dq(Xq)[m, k] * dq(Wq)[n, k], float32 accumulation.
 *  MXFP4: dq = e2m1(code) * 2^(scale - 127); runs on gfx950 scaled MFMA with
 *         the E8M0 scales consumed by the instruction.
 *  NVFP4: dq = e2m1(code) * e4m3(scale) * s_t; the E4M3 group scale is folded
 *         into an exact 16-bit operand before the products (fp16 in the 256-row-tile
 *         and decode kernels, bf16 in the general one; E4M3 scales have no native
 *         MFMA form on gfx950), x_ts * w_ts is applied to the sums. Scale codes are the finite non-negative E4M3FN codes
 *         0x00..0x7E that the quantizers write; other codes are outside the contract.
 *
 *  Xq  device uint8 [M, K/2], Xs device uint8 [M, K/g]  (fp4_rotate_quantize output)
 *  Wq  device uint8 [N, K/2], Ws device uint8 [N, K/g]  (fp4_quantize_weights output)
 *  x_ts, w_ts  NVFP4: device float[1] tensor scales (4-byte aligned); MXFP4: must be NULL.
 *  M, N >= 1; K >= 128 and K % 128 == 0. M, N, K <= 2^31 - 1 and M * K / 2,
 *  N * K / 2 <= 2^40 bytes; larger shapes return FP4_E_SHAPE.
 *  Xq, Wq 16-byte aligned; Xs, Ws 4-byte aligned. (With 16-byte-aligned Xs and Ws: MXFP4
 *  with K % 512 == 0 runs the weight-streaming decode kernel for M <= 16, and for M <= 64
 *  when K <= 8192, except 33 <= M <= 64 with N >= 8192, and the large-tile kernel for
 *  M, N >= 256 (K < 2^25), on 64-column tiles (one or two row tiles) for 64 < M < 256
 *  with N >= 1024 and for those 33-64 rows; NVFP4 runs the decode kernel for M <= 64 when
 *  K % 512 == 0 and K <= 8192, and the large-tile kernel for M, N >= 256, and for
 *  64 < M < 256 with N >= 1024, when K % 256 == 0. Other pointers or shapes run the general
 *  kernel, on 64 x 64 tiles when its 128 x 128 grid would be small.)
 *  Y   device [M, N] row-major, float32 (FP4_OUT_F32) or bf16 (FP4_OUT_BF16,
 *      round-to-nearest-even); 16-byte aligned.
 * No bias, no activation. One kernel launch on `stream`.
 */
FP4_API int fp4_linear(const uint8_t *Xq, const uint8_t *Xs, const float *x_ts,
               const uint8_t *Wq, const uint8_t *Ws, const float *w_ts,
               int64_t M, int64_t N, int64_t K, int fmt,
               void *Y, int y_dtype, void *stream);

/*
 * fp4_rotate_quantize_linear - the decode step of an MXFP4 linear layer:
 * Y = fp4_linear(fp4_rotate_quantize(X, block, MXFP4), Wq, Ws), bit for bit the same as
 * the two calls. "Bridging the Gap Between Promise and Performance for Microscaling FP4
 * Quantization" (gist.science, German edition), Technische Zusammenfassung §2
 * "GPU-Kernel-Unterstützung (QuTLASS)": the online rotation fused with quantization,
 * feeding the 4-bit matmul.
 * Normally one launch: every workgroup quantizes the whole of X into on-chip memory with
 * the quantizer's own device code, while its W streams in. That pays off for a few tokens
 * (MI355X, W from HBM: 1 token on N = 14336, K = 4096 in about 8 us against 10 us for the
 * two calls). With many rows of X per CU (M times the workgroups per CU, above about 14) the
 * repeated quantization costs more than a second launch; given a workspace, the call then
 * quantizes X once into it and runs the decode GEMM (two launches on `stream`; 16 tokens on
 * N = 14336: about 12 us instead of 21 us for one launch).
 *
 *  X       device bf16 [M, ldx], 16-byte aligned, ldx >= K, ldx % 8 == 0.
 *  M       1..16 tokens.   K: a multiple of 512 with M * (K/2 + 16 + K/32) <= 160 KiB.
 *  block   16, 32, 64 or 128 (the block W was quantized with).
 *  Wq, Ws  MXFP4 weights from fp4_quantize_weights: uint8 [N, K/2] and [N, K/32], both
 *          16-byte aligned (16 scale bytes of a row are read at once).
 *  Y       device [M, N], float32 or bf16 (y_dtype), 16-byte aligned.
 *  workspace, workspace_bytes  NULL (always one launch), or a 16-byte-aligned device buffer
 *          of at least FP4_LINEAR_WORKSPACE_BYTES(M, K) bytes, owned by the caller and
 *          free for the call's duration on `stream` (its contents afterwards: X's codes,
 *          then its scales at FP4_LINEAR_WORKSPACE_CODES(M, K), when two launches ran).
 * Errors: FP4_E_BLOCK, FP4_E_FORMAT (y_dtype), FP4_E_NULLPTR, FP4_E_SHAPE (M, K, ldx, the
 * on-chip size or a short workspace), FP4_E_ALIGN.
 */
#define FP4_LINEAR_WORKSPACE_CODES(M, K) ((((M) * (K) / 2 + 255) / 256) * 256)
#define FP4_LINEAR_WORKSPACE_BYTES(M, K) (FP4_LINEAR_WORKSPACE_CODES(M, K) + (M) * (K) / 32)
FP4_API int fp4_rotate_quantize_linear(const void *X, int64_t M, int64_t K, int64_t ldx, int block,
                                       const uint8_t *Wq, const uint8_t *Ws, int64_t N, void *Y, int y_dtype,
                                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * fp4_rotate_quantize_linear_noalloc - fp4_rotate_quantize_linear for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments without the workspace, the same results. Where the
 * workspace call would take two launches, this one uses an array of
 * FP4_DECODE_SCRATCH_BYTES (160 KiB + 256) bytes in the library's own device image, one per
 * GPU, held until the process ends; the call itself allocates nothing. That array is shared:
 * calls that overlap on one GPU (other streams, other threads) race on it and must be
 * serialized by the caller. Every size the decode step accepts fits it (FP4_E_SHAPE
 * otherwise). Errors as fp4_rotate_quantize_linear, and FP4_E_HIP if the array's address
 * cannot be obtained on the current device.
 */
#define FP4_DECODE_SCRATCH_BYTES (160 * 1024 + 256) /* >= every FP4_LINEAR_WORKSPACE_BYTES accepted */
FP4_API int fp4_rotate_quantize_linear_noalloc(const void *X, int64_t M, int64_t K, int64_t ldx, int block,
                                               const uint8_t *Wq, const uint8_t *Ws, int64_t N, void *Y,
                                               int y_dtype, void *stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
FP4_API const char *fp4_last_error(void);

/* ABI version of this header (major * 100 + minor). */
FP4_API int fp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4_MI355X_H */
