// W4A4 MXFP4 GEMM on gfx950 scaled MFMA: Y = dq(Xq) dq(Wq)^T.
//
// "Bridging the Gap Between Promise and Performance for Microscaling FP4
// Quantization" (gist.science, German edition), Technische Zusammenfassung §2
// "GPU-Kernel-Unterstützung (QuTLASS)": the 4-bit matmul that consumes the
// quantized activations and the offline rotated, quantized weights.
//
// gfx950 v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in E2M1 takes one
// E8M0 scale byte per lane: lane l carries 32 consecutive K elements (16 bytes)
// of row (l % 16) and the scale of that 32-element group, which is exactly one
// MXFP4 group. So the E8M0 scales are consumed natively; no dequantization.
//
// This is the general kernel (any K % 128 == 0, any M, N); large shapes with K % 512 == 0
// go to the 256x256-tile kernel in gemm_mxfp4_ring.hip.
//
// Tiling: a workgroup computes a BM x BN tile of Y; its waves split it into
// WM x WN wave tiles of 16x16 MFMA fragments. Each K stage stages BK = 256 K
// elements (128 bytes per row) of A, B and their scales in LDS, double buffered:
// global loads of stage s+1 are issued before the MFMAs of stage s. LDS rows are
// padded by 16 bytes so the 16 lanes reading one fragment column hit distinct banks.
#include "common.hpp"

namespace fp4 {
namespace {

constexpr int BKB = 128;          // bytes of K per stage per row (256 elements)
constexpr int PITCH = BKB + 16;   // padded LDS row pitch (bytes)
constexpr int SPR = BKB / 16;     // scale bytes per row per stage (one per 32 elements)

template <int BM, int BN, int WM, int WN>
struct Cfg {
  static constexpr int WAVES = (BM / WM) * (BN / WN);
  static constexpr int NT = WAVES * 64;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int A_CHUNKS = BM * BKB / 16;  // 16-byte chunks per stage
  static constexpr int B_CHUNKS = BN * BKB / 16;
  static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
  static constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
};

template <int BM, int BN, int WM, int WN, bool OUT_BF16>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_mxfp4_kernel(
    const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ Xs, const uint8_t* __restrict__ Wq,
    const uint8_t* __restrict__ Ws, void* __restrict__ Yv, int M, int N, int K, int tiles_n) {
  using C = Cfg<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t sSA[2][BM * SPR];
  __shared__ __attribute__((aligned(16))) uint8_t sSB[2][BN * SPR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm0 = (wave / (BN / WN)) * WM, wn0 = (wave % (BN / WN)) * WN;
  const int KB = K / 2;       // bytes per packed row
  const int KS = K / 32;      // scale bytes per row
  const int nstages = (K + 255) / 256;

  v4u ra[C::A_PER_T], rb[C::B_PER_T];
  uint2 rsa = {0, 0}, rsb = {0, 0};

  auto gload = [&](int s) {
    const int kb0 = s * BKB;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int ch = tid + i * C::NT;
      const int r = ch / (BKB / 16), c = ch % (BKB / 16);
      int row = m0 + r;
      row = row < M ? row : M - 1;
      const int kb = kb0 + c * 16;
      if (ch < C::A_CHUNKS && kb < KB)
        ra[i] = *reinterpret_cast<const v4u*>(Xq + (size_t)row * KB + kb);
      else
        ra[i] = v4u{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int ch = tid + i * C::NT;
      const int r = ch / (BKB / 16), c = ch % (BKB / 16);
      int row = n0 + r;
      row = row < N ? row : N - 1;
      const int kb = kb0 + c * 16;
      if (ch < C::B_CHUNKS && kb < KB)
        rb[i] = *reinterpret_cast<const v4u*>(Wq + (size_t)row * KB + kb);
      else
        rb[i] = v4u{0, 0, 0, 0};
    }
    const int ks0 = s * SPR;
    if (tid < BM) {
      int row = m0 + tid;
      row = row < M ? row : M - 1;
      const uint8_t* p = Xs + (size_t)row * KS + ks0;
      rsa.x = ks0 < KS ? *reinterpret_cast<const unsigned*>(p) : 0u;
      rsa.y = ks0 + 4 < KS ? *reinterpret_cast<const unsigned*>(p + 4) : 0u;
    }
    if (tid < BN) {
      int row = n0 + tid;
      row = row < N ? row : N - 1;
      const uint8_t* p = Ws + (size_t)row * KS + ks0;
      rsb.x = ks0 < KS ? *reinterpret_cast<const unsigned*>(p) : 0u;
      rsb.y = ks0 + 4 < KS ? *reinterpret_cast<const unsigned*>(p + 4) : 0u;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int ch = tid + i * C::NT;
      if (ch < C::A_CHUNKS) {
        const int r = ch / (BKB / 16), c = ch % (BKB / 16);
        *reinterpret_cast<v4u*>(&sA[buf][r * PITCH + c * 16]) = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int ch = tid + i * C::NT;
      if (ch < C::B_CHUNKS) {
        const int r = ch / (BKB / 16), c = ch % (BKB / 16);
        *reinterpret_cast<v4u*>(&sB[buf][r * PITCH + c * 16]) = rb[i];
      }
    }
    if (tid < BM) *reinterpret_cast<uint2*>(&sSA[buf][tid * SPR]) = rsa;
    if (tid < BN) *reinterpret_cast<uint2*>(&sSB[buf][tid * SPR]) = rsb;
  };

  v4f acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();

  const int fr = lane & 15, fg = lane >> 4;  // fragment row, K sub-group (32 elements)
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstages) gload(s + 1);
    const int subs = (s * 256 + 256 <= K) ? 2 : 1;
    for (int ks = 0; ks < subs; ++ks) {
      v8i a[C::FM], b[C::FN];
      int sa[C::FM], sb[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int r = wm0 + i * 16 + fr;
        const v4u t = *reinterpret_cast<const v4u*>(&sA[buf][r * PITCH + ks * 64 + fg * 16]);
        a[i] = v8i{(int)t[0], (int)t[1], (int)t[2], (int)t[3], 0, 0, 0, 0};
        sa[i] = sSA[buf][r * SPR + ks * 4 + fg];
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int r = wn0 + j * 16 + fr;
        const v4u t = *reinterpret_cast<const v4u*>(&sB[buf][r * PITCH + ks * 64 + fg * 16]);
        b[j] = v8i{(int)t[0], (int)t[1], (int)t[2], (int)t[3], 0, 0, 0, 0};
        sb[j] = sSB[buf][r * SPR + ks * 4 + fg];
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0,
                                                                        sa[i], 0, sb[j]);
    }
    if (s + 1 < nstages) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane/16)+q, column lane%16 of each fragment
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int col = n0 + wn0 + j * 16 + fr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + wm0 + i * 16 + 4 * fg + q;
        if (row < M && col < N) {
          if constexpr (OUT_BF16) {
            reinterpret_cast<__bf16*>(Yv)[(size_t)row * N + col] = (__bf16)acc[i][j][q];
          } else {
            reinterpret_cast<float*>(Yv)[(size_t)row * N + col] = acc[i][j][q];
          }
        }
      }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_general(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws, int64_t M,
                          int64_t N, int64_t K, void* Y, int out_bf16, hipStream_t st) {
  using C = Cfg<BM, BN, WM, WN>;
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  const dim3 grid(tiles_m * tiles_n), block(C::NT);
  if (out_bf16)
    hipLaunchKernelGGL((gemm_mxfp4_kernel<BM, BN, WM, WN, true>), grid, block, 0, st, Xq, Xs, Wq, Ws, Y, (int)M,
                       (int)N, (int)K, tiles_n);
  else
    hipLaunchKernelGGL((gemm_mxfp4_kernel<BM, BN, WM, WN, false>), grid, block, 0, st, Xq, Xs, Wq, Ws, Y, (int)M,
                       (int)N, (int)K, tiles_n);
  return hipGetLastError();
}

}  // namespace
}  // namespace fp4

hipError_t fp4_launch_gemm_mxfp4(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq,
                                 const uint8_t* Ws, int64_t M, int64_t N, int64_t K, void* Y,
                                 int out_bf16, hipStream_t st) {
  // The decode and large-tile kernels read 16 scale bytes of a row at a time, which needs scale
  // pointers aligned to 16 bytes (K % 512 == 0 keeps every row aligned then); the general kernel
  // below reads 4-byte words and takes any 4-byte-aligned pair.
  const bool scales16 = ((reinterpret_cast<uintptr_t>(Xs) | reinterpret_cast<uintptr_t>(Ws)) & 15) == 0;
  const bool ring = scales16 && fp4_gemm_mxfp4_ring_fits(M, N, K);
  if (scales16 && !(ring && M > 32) && fp4_gemm_mxfp4_decode_fits(M, N, K))
    return fp4_launch_gemm_mxfp4_decode(Xq, Xs, Wq, Ws, M, N, K, Y, out_bf16, st);
  if (ring) return fp4_launch_gemm_mxfp4_ring(Xq, Xs, Wq, Ws, M, N, K, Y, out_bf16, st);
  // 128x128 tiles on 4 waves; when they would give fewer than two workgroups per CU (as for 65 to
  // 255 tokens against one layer), 64x64 tiles on 4 waves: four times the workgroups streaming W
  // (at N = 14336, K = 4096: 1.3-1.5x faster from 65 to 192 tokens, 1.06x at 255).
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = fp4_device_cus(dev, &cus);
  if (e != hipSuccess) return e;
  const bool small = ((M + 127) / 128) * ((N + 127) / 128) < 2 * (int64_t)cus;
  return small ? fp4::launch_general<64, 64, 32, 32>(Xq, Xs, Wq, Ws, M, N, K, Y, out_bf16, st)
               : fp4::launch_general<128, 128, 64, 64>(Xq, Xs, Wq, Ws, M, N, K, Y, out_bf16, st);
}
