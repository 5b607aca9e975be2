// Shared device helpers and launcher declarations of the gfx950 FP4 library.
//
// Element format facts used throughout (E2M1 elements, E8M0 / E4M3 scales) are
// those of "Unveiling the Potential of Quantization with MXFP4" (gist.science,
// Dutch edition), Technische samenvatting, Probleemstelling, and of
// "Bridging the Gap Between Promise and Performance for Microscaling FP4
// Quantization" (gist.science, German edition), Technische Zusammenfassung §1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kMxGroup = 32;
constexpr int kNvGroup = 16;

// fl32(1/sqrt(b)) for the Hadamard block sizes, as bit patterns (correctly rounded).
__host__ __device__ constexpr unsigned hadamard_constant_bits(int b) {
  return b == 16 ? 0x3E800000u : b == 32 ? 0x3E3504F3u : b == 64 ? 0x3E000000u : 0x3DB504F3u;
}

// bf16 pair (one dword, element 2j in the low half) -> two exact float32.
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

// Cross-lane read within a quad: lane ^ 1 or lane ^ 2 (DPP quad_perm).
template <int XOR>
__device__ __forceinline__ float quad_xor(float v) {
  constexpr int ctrl = XOR == 1 ? 0xB1 : 0x4E;  // [1,0,3,2] / [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}

// Nearest non-negative E4M3FN code to q >= 0, ties to even, saturating at 448 (0x7E).
// Every step is exact in float64 (scaling by powers of two, round-to-integer).
__device__ __forceinline__ unsigned e4m3_rne_sat(double q) {
  if (q >= 448.0) return 0x7Eu;
  if (q < 0.015625) {  // below 2^-6: subnormal codes k * 2^-9 (k = 8 continues as 2^-6)
    return (unsigned)__builtin_rint(q * 512.0);
  }
  int E;
  double f = __builtin_frexp(q, &E);  // q = f 2^E, f in [0.5, 1), E in [-5, 9]
  (void)f;
  double k = __builtin_rint(__builtin_ldexp(q, 4 - E));  // 8..16 mantissa steps
  int code = ((E + 6) << 3) + ((int)k - 8);             // carry of k == 16 moves the exponent
  return (unsigned)(code > 0x7E ? 0x7E : code);
}

// Exact float32 value of a non-negative E4M3FN code 0..0x7E.
__device__ __forceinline__ float e4m3_value(unsigned c) {
  unsigned e = c >> 3, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

}  // namespace fp4

// ---------------------------------------------------------------------------
// Launchers (defined next to their kernels). Arguments are already validated.
// ---------------------------------------------------------------------------
hipError_t fp4_launch_rotate_quantize(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, int block,
                                      int fmt, int rule, bool given_tensor_scale, const int8_t* signs,
                                      uint8_t* codes, uint8_t* scales, float* tensor_scale, hipStream_t stream);
// Compute units of device `dev`, queried once per device.
hipError_t fp4_device_cus(int dev, int* cus);
hipError_t fp4_launch_gemm_mxfp4(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq,
                                 const uint8_t* Ws, int64_t M, int64_t N, int64_t K, void* Y,
                                 int out_bf16, hipStream_t stream);
bool fp4_gemm_mxfp4_ring_fits(int64_t M, int64_t N, int64_t K);
bool fp4_gemm_mxfp4_decode_fits(int64_t M, int64_t N, int64_t K);
bool fp4_decode_fused_fits(int64_t M, int64_t N, int64_t K);
hipError_t fp4_decode_fused_preferred(int64_t M, int64_t N, int64_t K, bool* fused);
hipError_t fp4_decode_scratch(uint8_t** ptr);
hipError_t fp4_launch_decode_fused(const uint16_t* X, int64_t ldx, int block, const uint8_t* Wq, const uint8_t* Ws,
                                   int64_t M, int64_t N, int64_t K, void* Y, int out_bf16, hipStream_t stream);
hipError_t fp4_launch_gemm_mxfp4_decode(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                                        int64_t M, int64_t N, int64_t K, void* Y, int out_bf16, hipStream_t stream);
hipError_t fp4_launch_gemm_mxfp4_ring(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                                      int64_t M, int64_t N, int64_t K, void* Y, int out_bf16, hipStream_t stream);
bool fp4_gemm_nvfp4_ring_fits(int64_t M, int64_t N, int64_t K);
bool fp4_gemm_nvfp4_decode_fits(int64_t M, int64_t N, int64_t K);
hipError_t fp4_launch_gemm_nvfp4_decode(const uint8_t* Xq, const uint8_t* Xs, const float* x_ts, const uint8_t* Wq,
                                        const uint8_t* Ws, const float* w_ts, int64_t M, int64_t N, int64_t K, void* Y,
                                        int out_bf16, hipStream_t stream);
hipError_t fp4_launch_gemm_nvfp4_ring(const uint8_t* Xq, const uint8_t* Xs, const float* x_ts, const uint8_t* Wq,
                                      const uint8_t* Ws, const float* w_ts, int64_t M, int64_t N, int64_t K, void* Y,
                                      int out_bf16, hipStream_t stream);
hipError_t fp4_launch_gemm_nvfp4(const uint8_t* Xq, const uint8_t* Xs, const float* x_ts,
                                 const uint8_t* Wq, const uint8_t* Ws, const float* w_ts, int64_t M,
                                 int64_t N, int64_t K, void* Y, int out_bf16, hipStream_t stream);

// Column plan of the large-tile GEMMs: tn1 panels of 256 columns, then tn2 panels of 192.
// The 256-wide tiles come first in dispatch order, so a split is only considered when they
// fill whole rounds of `cus` workgroups (the narrow tiles then start together); its makespan,
// in 256-wide tile times, is rounds(wide) + narrow_cost * rounds(narrow). The uniform 256-wide
// tiling is kept unless a split is shorter.
inline void fp4_plan_tile_columns(int tiles_m, int64_t N, int cus, float narrow_cost, int& tn1, int& tn2) {
  const int w_all = (int)((N + 255) / 256);
  tn1 = w_all;
  tn2 = 0;
  if (cus <= 0) return;
  const long long T = (long long)tiles_m * w_all;
  float best = (float)((T + cus - 1) / cus);
  // tiles_m * a is a multiple of cus exactly when a is a multiple of cus / gcd(tiles_m, cus)
  int g = cus, rem = tiles_m % cus;
  while (rem != 0) {
    const int r = g % rem;
    g = rem;
    rem = r;
  }
  const int step = cus / g;
  for (int a = 0; a < w_all; a += step) {
    const int b = (int)((N - 256LL * a + 191) / 192);
    const long long T2 = (long long)tiles_m * b;
    const float t = (float)((long long)tiles_m * a / cus) + narrow_cost * (float)((T2 + cus - 1) / cus);
    if (t < best - 1e-3f) {
      best = t;
      tn1 = a;
      tn2 = b;
    }
  }
}
