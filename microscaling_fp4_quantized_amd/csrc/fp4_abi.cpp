// C ABI of the gfx950 FP4 library: argument validation, then kernel launches.
// Declarations and the contract of every call are in include/fp4.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/fp4.h"
#include "common.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return FP4_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_quantize(const char* who, const void* X, int64_t M, int64_t K, int64_t ld, int block, int fmt,
                   const uint8_t* codes, const uint8_t* scales, const float* ts) {
  if (fmt != FP4_MXFP4 && fmt != FP4_NVFP4) return fail(FP4_E_FORMAT, "%s: unknown format %d", who, fmt);
  if (block != 16 && block != 32 && block != 64 && block != 128)
    return fail(FP4_E_BLOCK, "%s: Hadamard block %d not in {16, 32, 64, 128}", who, block);
  if (!X || !codes || !scales) return fail(FP4_E_NULLPTR, "%s: input, codes and scales must be non-NULL", who);
  if (fmt == FP4_NVFP4 && !ts) return fail(FP4_E_NULLPTR, "%s: NVFP4 needs a tensor_scale buffer", who);
  if (fmt == FP4_MXFP4 && ts) return fail(FP4_E_NULLPTR, "%s: tensor_scale must be NULL for MXFP4", who);
  if (M < 1 || K < 1) return fail(FP4_E_SHAPE, "%s: rows (%lld) and K (%lld) must be >= 1", who, (long long)M,
                                  (long long)K);
  if (K % 32 || K % block)
    return fail(FP4_E_SHAPE, "%s: K=%lld must be a multiple of 32 and of the block %d", who, (long long)K, block);
  if (ld < K) return fail(FP4_E_SHAPE, "%s: leading dimension %lld < K=%lld", who, (long long)ld, (long long)K);
  if (M > 0x7FFFFFFFLL / (K / 32) || ld > (int64_t)1 << 40)  // K >= 32 here; no product can overflow
    return fail(FP4_E_SHAPE, "%s: tensor too large (rows*K/32 must fit in 31 bits)", who);
  if (!aligned(X, 16) || ld % 8) return fail(FP4_E_ALIGN, "%s: input must be 16-byte aligned, ld %% 8 == 0", who);
  if (!aligned(codes, 16)) return fail(FP4_E_ALIGN, "%s: codes must be 16-byte aligned", who);
  if (fmt == FP4_NVFP4 && (!aligned(scales, 2) || !aligned(ts, 4)))
    return fail(FP4_E_ALIGN, "%s: NVFP4 scales must be 2-byte aligned, tensor_scale 4-byte aligned", who);
  return FP4_OK;
}

int launched(const char* who, hipError_t e) {
  if (e != hipSuccess) return fail(FP4_E_HIP, "%s: HIP error at launch: %s", who, hipGetErrorString(e));
  return ok();
}

int quantize(const char* who, const void* X, int64_t M, int64_t K, int64_t ld, int block, int fmt, int rule,
             const int8_t* signs, uint8_t* codes, uint8_t* scales, float* ts, void* stream) {
  int st = check_quantize(who, X, M, K, ld, block, fmt, codes, scales, ts);
  if (st != FP4_OK) return st;
  const bool given_ts = (rule & FP4_TENSOR_SCALE_IN) != 0;
  rule &= ~FP4_TENSOR_SCALE_IN;
  if (given_ts && fmt != FP4_NVFP4) return fail(FP4_E_FORMAT, "%s: a given tensor scale applies to NVFP4 only", who);
  if (rule != FP4_SCALE_STANDARD && rule != FP4_SCALE_OCP_FLOOR && rule != FP4_SCALE_OAS && rule != FP4_SCALE_FIT)
    return fail(FP4_E_FORMAT, "%s: unknown scale rule %d", who, rule);
  if (fmt == FP4_NVFP4 && (rule == FP4_SCALE_OCP_FLOOR || rule == FP4_SCALE_OAS))
    return fail(FP4_E_FORMAT, "%s: scale rule %d applies to MXFP4 only", who, rule);
  if (signs && !aligned(signs, 16)) return fail(FP4_E_ALIGN, "%s: signs must be 16-byte aligned", who);
  return launched(who, fp4_launch_rotate_quantize(static_cast<const uint16_t*>(X), M, K, ld, block, fmt, rule,
                                                  given_ts, signs, codes, scales, ts,
                                                  static_cast<hipStream_t>(stream)));
}

int check_decode_step(const char* who, const void* X, int64_t M, int64_t K, int64_t ldx, int block,
                      const uint8_t* Wq, const uint8_t* Ws, int64_t N, void* Y, int y_dtype) {
  if (block != 16 && block != 32 && block != 64 && block != 128)
    return fail(FP4_E_BLOCK, "%s: Hadamard block %d not in {16, 32, 64, 128}", who, block);
  if (y_dtype != FP4_OUT_F32 && y_dtype != FP4_OUT_BF16)
    return fail(FP4_E_FORMAT, "%s: unknown output dtype %d", who, y_dtype);
  if (!X || !Wq || !Ws || !Y) return fail(FP4_E_NULLPTR, "%s: X, Wq, Ws and Y must be non-NULL", who);
  if (M < 1 || M > 16 || N < 1 || K < 512 || K % 512 || N > 0x7FFFFFFF || K > 0x7FFFFFFF)
    return fail(FP4_E_SHAPE, "%s: need 1 <= M <= 16, N >= 1 and K a positive multiple of 512 (M=%lld N=%lld K=%lld)",
                who, (long long)M, (long long)N, (long long)K);
  if (!fp4_decode_fused_fits(M, N, K))
    return fail(FP4_E_SHAPE, "%s: M * K too large for the workgroup's LDS; use fp4_rotate_quantize + fp4_linear", who);
  if (ldx < K || ldx > (int64_t)1 << 40) return fail(FP4_E_SHAPE, "%s: leading dimension %lld < K", who, (long long)ldx);
  if (!aligned(X, 16) || ldx % 8) return fail(FP4_E_ALIGN, "%s: X must be 16-byte aligned, ldx %% 8 == 0", who);
  if (!aligned(Wq, 16) || !aligned(Ws, 16) || !aligned(Y, 16))
    return fail(FP4_E_ALIGN, "%s: Wq, Ws and Y must be 16-byte aligned", who);
  return FP4_OK;
}

// The validated decode step: one fused launch, or, with a workspace and more rows of X per CU
// than the fused kernel quantizes profitably, the quantizer into the workspace (codes, then the
// E8M0 scales at the next 256-byte boundary) followed by the decode GEMM. Both give the same bits.
int decode_step(const char* who, const void* X, int64_t M, int64_t K, int64_t ldx, int block, const uint8_t* Wq,
                const uint8_t* Ws, int64_t N, void* Y, int y_dtype, uint8_t* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = y_dtype == FP4_OUT_BF16;
  bool fused = true;
  if (ws) {
    const hipError_t e = fp4_decode_fused_preferred(M, N, K, &fused);
    if (e != hipSuccess) return launched(who, e);
  }
  if (fused)
    return launched(who, fp4_launch_decode_fused(static_cast<const uint16_t*>(X), ldx, block, Wq, Ws, M, N, K, Y, bf16,
                                                 st));
  uint8_t* xq = ws;
  uint8_t* xs = ws + FP4_LINEAR_WORKSPACE_CODES((size_t)M, (size_t)K);
  hipError_t e = fp4_launch_rotate_quantize(static_cast<const uint16_t*>(X), M, K, ldx, block, FP4_MXFP4,
                                            FP4_SCALE_STANDARD, false, nullptr, xq, xs, nullptr, st);
  if (e == hipSuccess) e = fp4_launch_gemm_mxfp4_decode(xq, xs, Wq, Ws, M, N, K, Y, bf16, st);
  return launched(who, e);
}

}  // namespace

extern "C" {

int fp4_rotate_quantize(const void* X, int64_t M, int64_t K, int64_t ldx, int block, int fmt, uint8_t* codes,
                        uint8_t* scales, float* tensor_scale, void* stream) {
  return quantize("fp4_rotate_quantize", X, M, K, ldx, block, fmt, FP4_SCALE_STANDARD, nullptr, codes, scales,
                  tensor_scale, stream);
}

int fp4_quantize_weights(const void* W, int64_t N, int64_t K, int64_t ldw, int block, int fmt, uint8_t* codes,
                         uint8_t* scales, float* tensor_scale, void* stream) {
  return quantize("fp4_quantize_weights", W, N, K, ldw, block, fmt, FP4_SCALE_STANDARD, nullptr, codes, scales,
                  tensor_scale, stream);
}

int fp4_rotate_quantize_ex(const void* X, int64_t M, int64_t K, int64_t ldx, int block, int fmt, int scale_rule,
                           const int8_t* signs, uint8_t* codes, uint8_t* scales, float* tensor_scale, void* stream) {
  return quantize("fp4_rotate_quantize_ex", X, M, K, ldx, block, fmt, scale_rule, signs, codes, scales, tensor_scale,
                  stream);
}

int fp4_quantize_weights_ex(const void* W, int64_t N, int64_t K, int64_t ldw, int block, int fmt, int scale_rule,
                            const int8_t* signs, uint8_t* codes, uint8_t* scales, float* tensor_scale, void* stream) {
  return quantize("fp4_quantize_weights_ex", W, N, K, ldw, block, fmt, scale_rule, signs, codes, scales,
                  tensor_scale, stream);
}

int fp4_linear(const uint8_t* Xq, const uint8_t* Xs, const float* x_ts, const uint8_t* Wq, const uint8_t* Ws,
               const float* w_ts, int64_t M, int64_t N, int64_t K, int fmt, void* Y, int y_dtype,
               void* stream) {
  const char* who = "fp4_linear";
  if (fmt != FP4_MXFP4 && fmt != FP4_NVFP4) return fail(FP4_E_FORMAT, "%s: unknown format %d", who, fmt);
  if (y_dtype != FP4_OUT_F32 && y_dtype != FP4_OUT_BF16)
    return fail(FP4_E_FORMAT, "%s: unknown output dtype %d", who, y_dtype);
  if (!Xq || !Xs || !Wq || !Ws || !Y) return fail(FP4_E_NULLPTR, "%s: operand pointers must be non-NULL", who);
  if (fmt == FP4_NVFP4 && (!x_ts || !w_ts))
    return fail(FP4_E_NULLPTR, "%s: NVFP4 needs both tensor scales", who);
  if (fmt == FP4_MXFP4 && (x_ts || w_ts))
    return fail(FP4_E_NULLPTR, "%s: tensor scales must be NULL for MXFP4", who);
  if (fmt == FP4_NVFP4 && (!aligned(x_ts, 4) || !aligned(w_ts, 4)))
    return fail(FP4_E_ALIGN, "%s: tensor scales must be 4-byte aligned", who);
  if (M < 1 || N < 1 || K < 128 || K % 128)
    return fail(FP4_E_SHAPE, "%s: need M, N >= 1 and K a positive multiple of 128 (M=%lld N=%lld K=%lld)", who,
                (long long)M, (long long)N, (long long)K);
  if (M > 0x7FFFFFFF || N > 0x7FFFFFFF || K > 0x7FFFFFFF || M * (K / 2) > ((int64_t)1 << 40) ||
      N * (K / 2) > ((int64_t)1 << 40))
    return fail(FP4_E_SHAPE, "%s: problem too large", who);
  if (((M + 127) / 128) * ((N + 127) / 128) > 0x7FFFFFFF)
    return fail(FP4_E_SHAPE, "%s: too many output tiles", who);
  if (!aligned(Xq, 16) || !aligned(Wq, 16) || !aligned(Xs, 4) || !aligned(Ws, 4) || !aligned(Y, 16))
    return fail(FP4_E_ALIGN, "%s: codes and Y must be 16-byte aligned, scales 4-byte aligned", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = fmt == FP4_MXFP4
                     ? fp4_launch_gemm_mxfp4(Xq, Xs, Wq, Ws, M, N, K, Y, y_dtype == FP4_OUT_BF16, st)
                     : fp4_launch_gemm_nvfp4(Xq, Xs, x_ts, Wq, Ws, w_ts, M, N, K, Y, y_dtype == FP4_OUT_BF16, st);
  return launched(who, e);
}

int fp4_rotate_quantize_linear(const void* X, int64_t M, int64_t K, int64_t ldx, int block, const uint8_t* Wq,
                               const uint8_t* Ws, int64_t N, void* Y, int y_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  const char* who = "fp4_rotate_quantize_linear";
  int st = check_decode_step(who, X, M, K, ldx, block, Wq, Ws, N, Y, y_dtype);
  if (st != FP4_OK) return st;
  const size_t need = FP4_LINEAR_WORKSPACE_BYTES((size_t)M, (size_t)K);
  if (workspace && !aligned(workspace, 16)) return fail(FP4_E_ALIGN, "%s: workspace must be 16-byte aligned", who);
  if (workspace && workspace_bytes < need)
    return fail(FP4_E_SHAPE, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes, need);
  return decode_step(who, X, M, K, ldx, block, Wq, Ws, N, Y, y_dtype, static_cast<uint8_t*>(workspace), stream);
}

int fp4_rotate_quantize_linear_noalloc(const void* X, int64_t M, int64_t K, int64_t ldx, int block,
                                       const uint8_t* Wq, const uint8_t* Ws, int64_t N, void* Y, int y_dtype,
                                       void* stream) {
  const char* who = "fp4_rotate_quantize_linear_noalloc";
  int st = check_decode_step(who, X, M, K, ldx, block, Wq, Ws, N, Y, y_dtype);
  if (st != FP4_OK) return st;
  const size_t need = FP4_LINEAR_WORKSPACE_BYTES((size_t)M, (size_t)K);
  if (need > (size_t)FP4_DECODE_SCRATCH_BYTES)
    return fail(FP4_E_SHAPE, "%s: needs %zu bytes of workspace, the library's array holds %zu", who, need,
                (size_t)FP4_DECODE_SCRATCH_BYTES);
  uint8_t* ws = nullptr;
  const hipError_t e = fp4_decode_scratch(&ws);
  if (e != hipSuccess) return launched(who, e);
  return decode_step(who, X, M, K, ldx, block, Wq, Ws, N, Y, y_dtype, ws, stream);
}

const char* fp4_last_error(void) { return g_err; }

int fp4_abi_version(void) { return 130; }

}  // extern "C"
