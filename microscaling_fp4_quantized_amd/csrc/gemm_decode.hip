// Decode-shaped W4A4 MXFP4 GEMM for gfx950 (M <= 16 rows of activations).
//
// "Bridging the Gap Between Promise and Performance for Microscaling FP4
// Quantization" (gist.science, German edition), Technische Zusammenfassung §2
// "GPU-Kernel-Unterstützung (QuTLASS)": the 4-bit matmul of the online path,
// here in its token-generation shape, where W (N x K codes + scales) is the only
// large operand and the product is bound by HBM bandwidth on W.
//
// Design for CDNA4:
//  * One workgroup owns 16 output features (16 rows of W) and all of K; its 8 waves
//    take batches of 4 consecutive 128-wide K steps round-robin and are reduced through
//    LDS at the end, in a fixed order.
//  * Each step is one v_mfma_scale_f32_16x16x128_f8f6f4 with W as the row operand and
//    X as the column operand: lane l carries row l % 16 and the 32-element group l / 16
//    of the step (16 bytes of codes, one E8M0 byte), so the output fragment gives each
//    lane 4 consecutive features of one token.
//  * Every load of a wave's batch is issued before its first MFMA (4 steps, 4 KB of W per
//    wave, 32 KB per workgroup in flight), so the whole of W is requested at once for
//    K <= 4096 and the kernel runs at the HBM rate instead of the MFMA rate. A batch's
//    scales are 16 consecutive bytes of the row, read with one 16-byte load. X rows past M repeat row M-1
//    (their outputs are discarded); W rows past N repeat row N-1 likewise.
#include <atomic>

#include "quant_device.hpp"

namespace fp4 {
namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kDecBatch = 4;  // consecutive K steps per wave kept in flight

// Y[m][n .. n+3] = acc (four consecutive features of token m), bounds-checked.
template <bool OUT_BF16>
__device__ __forceinline__ void store_out(void* __restrict__ Yv, int M, int N, int m, int n, v4f acc) {
  if (m >= M) return;
  const bool vec = (N & 3) == 0 && n + 3 < N;
  if constexpr (OUT_BF16) {
    __bf16* dst = reinterpret_cast<__bf16*>(Yv) + (size_t)m * N + n;
    const __bf16 b[4] = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
    if (vec) {
      const uint2 pk = {(unsigned)__builtin_bit_cast(uint16_t, b[0]) | ((unsigned)__builtin_bit_cast(uint16_t, b[1]) << 16),
                        (unsigned)__builtin_bit_cast(uint16_t, b[2]) | ((unsigned)__builtin_bit_cast(uint16_t, b[3]) << 16)};
      *reinterpret_cast<uint2*>(dst) = pk;
    } else {
      for (int i = 0; i < 4; ++i)
        if (n + i < N) dst[i] = b[i];
    }
  } else {
    float* dst = reinterpret_cast<float*>(Yv) + (size_t)m * N + n;
    if (vec) {
      *reinterpret_cast<v4f*>(dst) = acc;
    } else {
      for (int i = 0; i < 4; ++i)
        if (n + i < N) dst[i] = acc[i];
    }
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kDecThreads) void gemm_mxfp4_decode(const uint8_t* __restrict__ Xq,
                                                                 const uint8_t* __restrict__ Xs,
                                                                 const uint8_t* __restrict__ Wq,
                                                                 const uint8_t* __restrict__ Ws,
                                                                 void* __restrict__ Yv, int M, int N, int K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int r = lane & 15, g = lane >> 4;
  const size_t KB = (size_t)K / 2, KS = (size_t)K / 32;
  const int steps = K / 128;  // 128-element steps; step t, lane group g: group 4t + g of the row
  const uint8_t* wp = Wq + (size_t)min(n0 + r, N - 1) * KB + 16 * g;
  const uint8_t* xp = Xq + (size_t)min(r, M - 1) * KB + 16 * g;
  const uint8_t* wsp = Ws + (size_t)min(n0 + r, N - 1) * KS;
  const uint8_t* xsp = Xs + (size_t)min(r, M - 1) * KS;
  const unsigned sh = 8u * (unsigned)g;

  // the waves take consecutive batches of kDecBatch steps, round-robin over K
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int t0 = wave * kDecBatch; t0 < steps; t0 += kDecWaves * kDecBatch) {
    v4u wa[kDecBatch], xb[kDecBatch];
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      const int t = min(t0 + u, steps - 1);  // in bounds; unused steps are skipped below
      wa[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wp + 64 * (size_t)t));
      xb[u] = *reinterpret_cast<const v4u*>(xp + 64 * (size_t)t);
    }
    // the batch's scale bytes 4 t0 .. 4 t0 + 15 of the row (steps % 4 == 0 keeps them in the row)
    const int tb = min(t0, steps - kDecBatch);
    const v4u wsv = *reinterpret_cast<const v4u*>(wsp + 4 * (size_t)tb);
    const v4u xsv = *reinterpret_cast<const v4u*>(xsp + 4 * (size_t)tb);
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      if (t0 + u < steps) {  // wave-uniform
        const v8i a = v8i{(int)wa[u][0], (int)wa[u][1], (int)wa[u][2], (int)wa[u][3], 0, 0, 0, 0};
        const v8i b = v8i{(int)xb[u][0], (int)xb[u][1], (int)xb[u][2], (int)xb[u][3], 0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 4, 0, (int)(wsv[u] >> sh), 0,
                                                                (int)(xsv[u] >> sh));
      }
    }
  }

  // fixed-order reduction over the waves' K slices
  __shared__ v4f red[kDecWaves][64];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) acc += red[w][lane];
  // lane holds D[n0 + 4g + i][m = r], i = 0..3: four consecutive features of token r
  store_out<OUT_BF16>(Yv, M, N, r, n0 + 4 * g, acc);
}

// ---------------------------------------------------------------------------
// Fused decode step: every workgroup first rotates and quantizes the (tiny) bf16 X into LDS
// with the same device code as fp4_rotate_quantize (so the codes are the same bits), then
// runs the decode product above with its X fragments read from LDS. One launch instead of
// two; X (M <= 16 rows) is read from L2 by every workgroup.
// ---------------------------------------------------------------------------
template <int B, bool OUT_BF16>
__global__ __launch_bounds__(kDecThreads) void decode_fused(const uint16_t* __restrict__ X, int64_t ldx,
                                                            const uint8_t* __restrict__ Wq,
                                                            const uint8_t* __restrict__ Ws, void* __restrict__ Yv,
                                                            int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int KB = K / 2, KS = K / 32, pitch = KB + 16;  // padded code rows: distinct banks per row
  uint8_t* xq = lds;                                   // [M][pitch]
  uint8_t* xs = lds + (size_t)M * pitch;               // [M][KS]
  const int total = M * KS;

  // phase 1: chunk c -> row c / KS, chunk c % KS. Quads of lanes hold the consecutive chunks of
  // one Hadamard block (KS % 16 == 0, and the loop base is a multiple of 512), and whole quads
  // are in or out of range together (total % 4 == 0).
  for (int c0 = 0; c0 < total; c0 += kDecThreads) {
    const int c = c0 + (int)threadIdx.x;
    if (c < total) {
      const int row = c / KS, cc = c - row * KS;
      const v4u* src = reinterpret_cast<const v4u*>(X + (size_t)row * (size_t)ldx + (size_t)cc * 32);
      float v[32];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4u w = src[q];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[8 * q + 2 * t] = bf16_lo(w[t]);
          v[8 * q + 2 * t + 1] = bf16_hi(w[t]);
        }
      }
      v4u out;
      const int code = mx_rotate_quantize_chunk<B, kRuleStandard>(v, out);
      *reinterpret_cast<v4u*>(xq + (size_t)row * pitch + (size_t)cc * 16) = out;
      xs[row * KS + cc] = (uint8_t)code;
    }
  }
  __syncthreads();

  // phase 2: the decode product (see gemm_mxfp4_decode) with X from LDS
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int r = lane & 15, g = lane >> 4;
  const int steps = K / 128;
  const uint8_t* wp = Wq + (size_t)min(n0 + r, N - 1) * KB + 16 * g;
  const uint8_t* wsp = Ws + (size_t)min(n0 + r, N - 1) * KS;
  const uint8_t* xp = xq + (size_t)min(r, M - 1) * pitch + 16 * g;
  const uint8_t* xsp = xs + (size_t)min(r, M - 1) * KS;
  const unsigned sh = 8u * (unsigned)g;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int t0 = wave * kDecBatch; t0 < steps; t0 += kDecWaves * kDecBatch) {
    v4u wa[kDecBatch], xb[kDecBatch];
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      const int t = min(t0 + u, steps - 1);
      wa[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wp + 64 * (size_t)t));
      xb[u] = *reinterpret_cast<const v4u*>(xp + 64 * t);
    }
    const int tb = min(t0, steps - kDecBatch);
    const v4u wsv = *reinterpret_cast<const v4u*>(wsp + 4 * (size_t)tb);
    const v4u xsv = *reinterpret_cast<const v4u*>(xsp + 4 * tb);
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      if (t0 + u < steps) {
        const v8i a = v8i{(int)wa[u][0], (int)wa[u][1], (int)wa[u][2], (int)wa[u][3], 0, 0, 0, 0};
        const v8i b = v8i{(int)xb[u][0], (int)xb[u][1], (int)xb[u][2], (int)xb[u][3], 0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 4, 0, (int)(wsv[u] >> sh), 0,
                                                                (int)(xsv[u] >> sh));
      }
    }
  }
  v4f* red = reinterpret_cast<v4f*>(lds);  // X in LDS is no longer read after this barrier
  __syncthreads();
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) acc += red[w * 64 + lane];
  store_out<OUT_BF16>(Yv, M, N, r, n0 + 4 * g, acc);
}

size_t fused_lds_bytes(int M, int K) { return (size_t)M * (K / 2 + 16) + (size_t)M * (K / 32); }

std::atomic<int> g_fused_attr[4][64];

template <int B>
hipError_t launch_fused(const uint16_t* X, int64_t ldx, const uint8_t* Wq, const uint8_t* Ws, int M, int N, int K,
                        void* Y, int out_bf16, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  auto kern = out_bf16 ? decode_fused<B, true> : decode_fused<B, false>;
  const int bi = B == 16 ? 0 : B == 32 ? 1 : B == 64 ? 2 : 3;
  const size_t lds = fused_lds_bytes(M, K) > (size_t)kDecWaves * 64 * 16 ? fused_lds_bytes(M, K)
                                                                         : (size_t)kDecWaves * 64 * 16;
  const bool cached = dev >= 0 && dev < 64;
  if (!cached || (g_fused_attr[bi][dev].load(std::memory_order_acquire) & (1 + out_bf16)) == 0) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    if (cached) g_fused_attr[bi][dev].fetch_or(1 + out_bf16, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)((N + 15) / 16)), dim3(kDecThreads), lds, st, X, ldx, Wq, Ws, Y, M, N, K);
  return hipGetLastError();
}

}  // namespace
}  // namespace fp4

bool fp4_gemm_mxfp4_decode_fits(int64_t M, int64_t N, int64_t K) { return M <= 16 && K % 512 == 0 && N >= 1; }

hipError_t fp4_launch_gemm_mxfp4_decode(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                                        int64_t M, int64_t N, int64_t K, void* Y, int out_bf16, hipStream_t st) {
  const dim3 grid((unsigned)((N + 15) / 16)), block(fp4::kDecThreads);
  if (out_bf16)
    hipLaunchKernelGGL(fp4::gemm_mxfp4_decode<true>, grid, block, 0, st, Xq, Xs, Wq, Ws, Y, (int)M, (int)N, (int)K);
  else
    hipLaunchKernelGGL(fp4::gemm_mxfp4_decode<false>, grid, block, 0, st, Xq, Xs, Wq, Ws, Y, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

bool fp4_decode_fused_fits(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 16 && N >= 1 && K % 512 == 0 && fp4::fused_lds_bytes((int)M, (int)K) <= 160 * 1024;
}

hipError_t fp4_launch_decode_fused(const uint16_t* X, int64_t ldx, int block, const uint8_t* Wq, const uint8_t* Ws,
                                   int64_t M, int64_t N, int64_t K, void* Y, int out_bf16, hipStream_t st) {
  switch (block) {
    case 16: return fp4::launch_fused<16>(X, ldx, Wq, Ws, (int)M, (int)N, (int)K, Y, out_bf16, st);
    case 32: return fp4::launch_fused<32>(X, ldx, Wq, Ws, (int)M, (int)N, (int)K, Y, out_bf16, st);
    case 64: return fp4::launch_fused<64>(X, ldx, Wq, Ws, (int)M, (int)N, (int)K, Y, out_bf16, st);
    default: return fp4::launch_fused<128>(X, ldx, Wq, Ws, (int)M, (int)N, (int)K, Y, out_bf16, st);
  }
}
