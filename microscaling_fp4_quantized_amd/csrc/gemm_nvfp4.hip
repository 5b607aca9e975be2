// W4A4 NVFP4 GEMM on gfx950: Y = s_tx s_tw sum_k (e2m1 d_x)(e2m1 d_w).
//
// "Bridging the Gap Between Promise and Performance for Microscaling FP4
// Quantization" (gist.science, Spanish edition), Resumen técnico §2.B item 2
// (NVFP4 carries group scales and a tensor scale) and §2.C (4-bit matmul).
//
// gfx950's scaled MFMA takes power-of-two (E8M0) scales per 32 K elements only;
// NVFP4 groups are 16 wide with E4M3 scales. The prologue therefore folds the
// group scale into the operand: e2m1 * d has at most 6 significant bits and lies
// in [2^-10, 2688], so it is exact in bf16. Tiles are dequantized once per
// workgroup into LDS and multiplied with v_mfma_f32_16x16x32_bf16 (float32
// accumulation); the two tensor scales are applied in the epilogue.
#include "common.hpp"

namespace fp4 {
namespace {

constexpr int BKE = 64;               // K elements per stage
constexpr int CB = BKE / 2;           // code bytes per row per stage (32)
constexpr int LP = BKE * 2 + 16;      // LDS pitch of a bf16 row (bytes, padded)

template <int BM, int BN, int WM, int WN>
struct NvCfg {
  static constexpr int WAVES = (BM / WM) * (BN / WN);
  static constexpr int NT = WAVES * 64;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int A_CHUNKS = BM * CB / 16;  // 16-byte code chunks (32 elements each)
  static constexpr int B_CHUNKS = BN * CB / 16;
  static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
  static constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
};

// 32 E2M1 codes (16 bytes) with two E4M3 group scales -> 32 exact bf16 (16 dwords).
__device__ __forceinline__ void dequant32(const v4u codes, unsigned sc2, v4u out[4]) {
  const float d0 = e4m3_value(sc2 & 0xFFu), d1 = e4m3_value((sc2 >> 8) & 0xFFu);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float d = w < 2 ? d0 : d1;
    v2f f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[w], 1.0f, 0);
    v2f f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[w], 1.0f, 1);
    v2f f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[w], 1.0f, 2);
    v2f f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[w], 1.0f, 3);
    // products are exact; the bf16 is the top half of the float32
    out[w][0] = __builtin_amdgcn_perm(__float_as_uint(f0[1] * d), __float_as_uint(f0[0] * d), 0x07060302u);
    out[w][1] = __builtin_amdgcn_perm(__float_as_uint(f1[1] * d), __float_as_uint(f1[0] * d), 0x07060302u);
    out[w][2] = __builtin_amdgcn_perm(__float_as_uint(f2[1] * d), __float_as_uint(f2[0] * d), 0x07060302u);
    out[w][3] = __builtin_amdgcn_perm(__float_as_uint(f3[1] * d), __float_as_uint(f3[0] * d), 0x07060302u);
  }
}

template <int BM, int BN, int WM, int WN, bool OUT_BF16>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_nvfp4_kernel(
    const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ Xs, const float* __restrict__ x_ts,
    const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Ws, const float* __restrict__ w_ts,
    void* __restrict__ Yv, int M, int N, int K, int tiles_n) {
  using C = NvCfg<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * LP];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * LP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm0 = (wave / (BN / WN)) * WM, wn0 = (wave % (BN / WN)) * WN;
  const int KB = K / 2, KS = K / 16;
  const int nstages = K / BKE;

  v4u ca[C::A_PER_T], cb[C::B_PER_T];
  unsigned sa[C::A_PER_T], sb[C::B_PER_T];

  auto gload = [&](int s) {
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int ch = tid + i * C::NT;
      const int r = ch >> 1, h = ch & 1;
      int row = m0 + r;
      row = row < M ? row : M - 1;
      if (ch < C::A_CHUNKS) {
        ca[i] = *reinterpret_cast<const v4u*>(Xq + (size_t)row * KB + s * CB + h * 16);
        sa[i] = *reinterpret_cast<const uint16_t*>(Xs + (size_t)row * KS + s * 4 + h * 2);
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int ch = tid + i * C::NT;
      const int r = ch >> 1, h = ch & 1;
      int row = n0 + r;
      row = row < N ? row : N - 1;
      if (ch < C::B_CHUNKS) {
        cb[i] = *reinterpret_cast<const v4u*>(Wq + (size_t)row * KB + s * CB + h * 16);
        sb[i] = *reinterpret_cast<const uint16_t*>(Ws + (size_t)row * KS + s * 4 + h * 2);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int ch = tid + i * C::NT;
      if (ch < C::A_CHUNKS) {
        const int r = ch >> 1, h = ch & 1;
        v4u o[4];
        dequant32(ca[i], sa[i], o);
        v4u* dst = reinterpret_cast<v4u*>(&sA[buf][r * LP + h * 64]);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = o[q];
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int ch = tid + i * C::NT;
      if (ch < C::B_CHUNKS) {
        const int r = ch >> 1, h = ch & 1;
        v4u o[4];
        dequant32(cb[i], sb[i], o);
        v4u* dst = reinterpret_cast<v4u*>(&sB[buf][r * LP + h * 64]);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = o[q];
      }
    }
  };

  v4f acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  const int fr = lane & 15, fg = lane >> 4;
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstages) gload(s + 1);
#pragma unroll
    for (int kk = 0; kk < BKE / 32; ++kk) {
      v8bf a[C::FM], b[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const v4u t = *reinterpret_cast<const v4u*>(&sA[buf][(wm0 + i * 16 + fr) * LP + kk * 64 + fg * 16]);
        a[i] = __builtin_bit_cast(v8bf, t);
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const v4u t = *reinterpret_cast<const v4u*>(&sB[buf][(wn0 + j * 16 + fr) * LP + kk * 64 + fg * 16]);
        b[j] = __builtin_bit_cast(v8bf, t);
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nstages) lstore(buf ^ 1);
    __syncthreads();
  }

  const float ts = x_ts[0] * w_ts[0];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int col = n0 + wn0 + j * 16 + fr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + wm0 + i * 16 + 4 * fg + q;
        if (row < M && col < N) {
          const float y = acc[i][j][q] * ts;
          if constexpr (OUT_BF16)
            reinterpret_cast<__bf16*>(Yv)[(size_t)row * N + col] = (__bf16)y;
          else
            reinterpret_cast<float*>(Yv)[(size_t)row * N + col] = y;
        }
      }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_general(const uint8_t* Xq, const uint8_t* Xs, const float* x_ts, const uint8_t* Wq,
                          const uint8_t* Ws, const float* w_ts, int64_t M, int64_t N, int64_t K, void* Y,
                          int out_bf16, hipStream_t st) {
  using C = NvCfg<BM, BN, WM, WN>;
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  const dim3 grid(tiles_m * tiles_n), block(C::NT);
  if (out_bf16)
    hipLaunchKernelGGL((gemm_nvfp4_kernel<BM, BN, WM, WN, true>), grid, block, 0, st, Xq, Xs, x_ts, Wq, Ws, w_ts, Y,
                       (int)M, (int)N, (int)K, tiles_n);
  else
    hipLaunchKernelGGL((gemm_nvfp4_kernel<BM, BN, WM, WN, false>), grid, block, 0, st, Xq, Xs, x_ts, Wq, Ws, w_ts, Y,
                       (int)M, (int)N, (int)K, tiles_n);
  return hipGetLastError();
}

}  // namespace
}  // namespace fp4

hipError_t fp4_launch_gemm_nvfp4(const uint8_t* Xq, const uint8_t* Xs, const float* x_ts,
                                 const uint8_t* Wq, const uint8_t* Ws, const float* w_ts, int64_t M,
                                 int64_t N, int64_t K, void* Y, int out_bf16, hipStream_t st) {
  // The large-tile kernel reads 16 scale bytes of a row at a time, which needs scale pointers
  // aligned to 16 bytes (K % 256 == 0 keeps every row aligned then); the general kernel below
  // reads 2-byte pieces.
  const bool scales16 = ((reinterpret_cast<uintptr_t>(Xs) | reinterpret_cast<uintptr_t>(Ws)) & 15) == 0;
  if (scales16 && fp4_gemm_nvfp4_decode_fits(M, N, K))
    return fp4_launch_gemm_nvfp4_decode(Xq, Xs, x_ts, Wq, Ws, w_ts, M, N, K, Y, out_bf16, st);
  if (scales16 && fp4_gemm_nvfp4_ring_fits(M, N, K))
    return fp4_launch_gemm_nvfp4_ring(Xq, Xs, x_ts, Wq, Ws, w_ts, M, N, K, Y, out_bf16, st);
  // 128x128 tiles on 4 waves; 64x64 tiles when those would give fewer than two workgroups per CU
  // and M <= 192 (at N = 14336: 1.4x faster for 1 to 16 rows, 1.1-1.2x for 65 to 192; slower at
  // 255 rows, where the 16-bit products outweigh the wider grid)
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = fp4_device_cus(dev, &cus);
  if (e != hipSuccess) return e;
  const bool small = ((M + 127) / 128) * ((N + 127) / 128) < 2 * (int64_t)cus && M <= 192;
  return small ? fp4::launch_general<64, 64, 32, 32>(Xq, Xs, x_ts, Wq, Ws, w_ts, M, N, K, Y, out_bf16, st)
               : fp4::launch_general<128, 128, 64, 64>(Xq, Xs, x_ts, Wq, Ws, w_ts, M, N, K, Y, out_bf16, st);
}
