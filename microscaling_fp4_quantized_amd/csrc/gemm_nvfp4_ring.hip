// Large-tile W4A4 NVFP4 GEMM for gfx950: Y = s_tx s_tw sum_k (e2m1 d_x)(e2m1 d_w), 256-row tiles.
//
// "Bridging the Gap Between Promise and Performance for Microscaling FP4
// Quantization" (gist.science, Spanish edition), Resumen técnico §2.B item 2
// (NVFP4 carries E4M3 group scales and a tensor scale) and §2.C (4-bit matmul).
//
// The gfx950 scaled MFMA accepts power-of-two scales per 32 K elements only, so the
// NVFP4 group scale (E4M3, 16 elements) is folded into the operand instead: e2m1 * d
// has at most 6 significant bits and lies in [2^-10, 2688], so it is exact in fp16, and
// the product runs on v_mfma_f32_32x32x16_f16 with float32 accumulation. The two
// tensor scales multiply the result in the epilogue. fp16 rather than bf16 (the products
// are exact in both): one packed convert and one packed multiply make two operands.
//
// Design for CDNA4:
//  * 8 waves (2 x 4), 128 x 64 outputs per wave as 4 x 2 fragments of 32 x 32.
//  * K advances 64 per stage. The codes (16 bytes = 32 elements + their two scale bytes
//    per thread and chunk) are loaded into registers two stages ahead; after stage s is
//    multiplied, stage s+1 is dequantized once per workgroup into an fp16 tile in the
//    other LDS buffer (pitch 144 bytes: the fragment reads hit distinct banks).
//  * W is the row operand and X the column operand of every MFMA, so each lane ends with
//    four consecutive output features of one token: one 16-byte LDS write when the output
//    tile is staged for whole-row 16-byte stores of Y.
//  * Workgroup i runs on XCD i % 8; each XCD takes a contiguous range of tiles, walked
//    M-fastest within groups of 8 tile rows.
//  * Two tile widths in one launch, as in the MXFP4 kernel: when 256x256 tiles would leave
//    the last round part-filled, the columns after whole rounds of them are covered by
//    256x192 tiles (4 x 2 waves of 64 x 96).
#include <atomic>
#include <type_traits>

#include "common.hpp"

namespace fp4 {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 256;                       // tile rows (both widths)
constexpr int WAVES = 8, NT = WAVES * 64;
constexpr int BKE = 64;                       // K elements per stage
constexpr int KSTEPS = BKE / 16;              // 32x32x16 steps per stage
constexpr int PITCH = BKE * 2 + 16;           // bytes per fp16 row in LDS (padded)
constexpr int LDS_BYTES = 2 * (BM + 256) * PITCH;  // sized for the wide tile: 144 KB

// One tile shape: BN columns, WGM x WGN waves.
template <int BN_, int WGM_, int WGN_>
struct Tile {
  static constexpr int BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  static constexpr int STAGE = (BM + BN) * PITCH;
  static constexpr int EP = WN * 4 + 16;  // epilogue staging row pitch (bytes): 16 rows hit distinct banks
  static constexpr int CHUNKS = (BM + BN) * 2;         // 32-element chunks per stage
  static constexpr int CPT = (CHUNKS + NT - 1) / NT;   // chunks per thread (the last round may be partial)
  static_assert(WGM * WGN == WAVES, "wave layout");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "whole 32x32 fragments");
  static_assert(CHUNKS % 64 == 0, "whole waves per chunk round");
  static_assert(2 * STAGE <= LDS_BYTES, "two stages fit");
  static_assert(WAVES * 32 * EP <= LDS_BYTES, "epilogue staging fits");
};
using Wide = Tile<256, 2, 4>;
using Narrow = Tile<192, 4, 2>;
constexpr float kNvNarrowCost = 0.84f;  // measured time of a 256x192 tile over a 256x256 one

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// 32 E2M1 codes (16 bytes) with their two E4M3 group scales (low byte first) -> 32 exact fp16
// (64 bytes). The E4M3 code's seven magnitude bits, shifted left by 7, are the fp16 bit
// pattern of d * 2^-8 (the E4M3 exponent bias is 7, fp16's is 15; E4M3 subnormals land on
// fp16 subnormals, exactly), and the sign goes to bit 15. The packed convert's power-of-two
// scale 256 restores the factor: (e2m1 * 256) * (d * 2^-8) = e2m1 * d, exact in fp16.
__device__ __forceinline__ void dequant32(const v4u codes, unsigned sc2, v4u out[4]) {
  const unsigned lo = ((sc2 & 0x7Fu) << 7) | ((sc2 & 0x80u) << 8);
  const unsigned hi = ((sc2 & 0x7F00u) >> 1) | (sc2 & 0x8000u);
  const h2 dd0 = __builtin_bit_cast(h2, lo | (lo << 16)), dd1 = __builtin_bit_cast(h2, hi | (hi << 16));
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const h2 dd = w < 2 ? dd0 : dd1;  // words 0-1 are the first 16 elements (group 2c), 2-3 the second
    // byte q of the word holds elements 2q (low nibble) and 2q+1
    out[w][0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[w], 256.0f, 0) * dd);
    out[w][1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[w], 256.0f, 1) * dd);
    out[w][2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[w], 256.0f, 2) * dd);
    out[w][3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[w], 256.0f, 3) * dd);
  }
}

// One output tile [m0, m0 + 256) x [n0, n0 + C::BN) over all of K.
template <bool OUT_BF16, class C>
__device__ __forceinline__ void nv_tile(uint8_t* smem, const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ Xs,
                                        const float* __restrict__ x_ts, const uint8_t* __restrict__ Wq,
                                        const uint8_t* __restrict__ Ws, const float* __restrict__ w_ts,
                                        void* __restrict__ Yv, int M, int N, int K, int m0, int n0) {
  constexpr int WGN = C::WGN, WM = C::WM, WN = C::WN, FM = C::FM, FN = C::FN;
  constexpr int STAGE = C::STAGE, CHUNKS = C::CHUNKS, CPT = C::CPT;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;
  const size_t KB = (size_t)K / 2, KS = (size_t)K / 16;
  const int nst = K / BKE;

  // chunk c of a stage: tile row c / 2 (A rows first, then B rows), half c % 2 of the row's 64
  // elements. When CHUNKS is not a multiple of the thread count, the waves past the end of the
  // last round (a whole number of waves) skip it; their clamped chunk keeps every address valid.
  const uint8_t* csrc[CPT];
  const uint8_t* ssrc[CPT];
  int ldst[CPT];
  unsigned shs[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = min(tid + i * NT, CHUNKS - 1), r = c >> 1, h = c & 1;
    const bool isA = r < BM;
    const size_t row = isA ? (size_t)min(m0 + r, M - 1) : (size_t)min(n0 + r - BM, N - 1);
    csrc[i] = (isA ? Xq : Wq) + row * KB + h * 16;
    ssrc[i] = (isA ? Xs : Ws) + row * KS;  // the row's 4 scale bytes of a stage; this chunk's are 2h, 2h+1
    ldst[i] = r * PITCH + h * 64;
    shs[i] = 16 * h;
  }
  // two stages of codes in registers: stage s+2 is requested while stage s is multiplied
  v4u cr[2][CPT];
  unsigned sr[2][CPT];
  // register set P holds the stages with parity P (the stage count is even, so the loop below
  // is unrolled by two and every index into the register arrays is a constant)
  // The loads are unconditional (a skipped chunk loads its clamped, valid address) and the
  // scales come as whole dwords: a load under a branch, or a 16-bit load the compiler re-masks
  // where the two register sets meet, makes it wait for loads issued just before.
  auto gload = [&](auto P, int s) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      cr[P][i] = *reinterpret_cast<const v4u*>(csrc[i] + (size_t)s * (BKE / 2));
      sr[P][i] = *reinterpret_cast<const unsigned*>(ssrc[i] + (size_t)s * (BKE / 16));
    }
  };
  auto lstore = [&](auto P) {  // dequantize register set P into LDS buffer P
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      if ((i + 1) * NT > CHUNKS && wave * 64 + i * NT >= CHUNKS) continue;  // wave-uniform
      v4u o[4];
      dequant32(cr[P][i], sr[P][i] >> shs[i], o);
      v4u* dst = reinterpret_cast<v4u*>(smem + P * STAGE + ldst[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = o[q];
    }
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int fr = lane & 31, fh = lane >> 5;
  auto stage = [&](auto P, int s) {  // multiply stage s (LDS buffer P = s & 1)
    const uint8_t* buf = smem + P * STAGE;
    // Register set P was stored to LDS before the last barrier. The prefetch and the store below
    // run unconditionally (the stage index is clamped, and the last stage's extra store lands in
    // a buffer nobody reads again) so the whole stage is one block in which the compiler can
    // interleave the dequantization with the MFMAs.
    gload(P, min(s + 2, nst - 1));
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      // lane l: row l % 32 of the fragment, K elements 16 ks + 8 (l / 32) .. + 7
      const int off = ks * 32 + fh * 16;
      v8h a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = __builtin_bit_cast(v8h, *reinterpret_cast<const v4u*>(buf + (wm0 + i * 32 + fr) * PITCH + off));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[j] = __builtin_bit_cast(v8h, *reinterpret_cast<const v4u*>(buf + (BM + wn0 + j * 32 + fr) * PITCH + off));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[j], a[i], acc[i][j], 0, 0, 0);  // D[n][m]
    }
    lstore(std::integral_constant<int, 1 - P>{});
    __syncthreads();
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  gload(P0{}, 0);
  gload(P1{}, 1);
  lstore(P0{});
  __syncthreads();
  for (int s = 0; s < nst; s += 2) {
    stage(P0{}, s);
    stage(P1{}, s + 1);
  }

  // acc[i][j][4q + r] = Y[m][n + r] with m = wm0 + 32 i + l % 32, n = wn0 + 32 j + 8 q + 4 (l / 32).
  // Epilogue: each wave stages one 32 x WN slab of float32 at a time in its own region of the
  // (now idle) LDS ring, one 16-byte write per 4 values, then writes whole 16-byte pieces of its
  // rows: 4 float32 values, or 8 bf16 values (two 8-byte halves when N % 8 == 4). Every value is
  // scaled by s_tx * s_tw in float32 before the bf16 rounding (to nearest even).
  constexpr int EP = C::EP;
  constexpr int VPP = OUT_BF16 ? 8 : 4;  // values per 16-byte piece of Y
  constexpr int CPR = WN / VPP;          // pieces per row
  const float ts = x_ts[0] * w_ts[0];
  const bool vec = N % VPP == 0;  // every piece starts 16-byte aligned (Y itself is)
  const bool vec4 = N % 4 == 0;   // bf16: every piece starts 8-byte aligned
  __syncthreads();                // every wave is done with the ring
  float* ep = reinterpret_cast<float*>(smem + wave * 32 * EP);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<v4f*>(&ep[fr * (EP / 4) + j * 32 + 8 * q + 4 * fh]) =
            v4f{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's slab is in LDS (wave-private region)
#pragma unroll
    for (int k = 0; k < 32 * CPR / 64; ++k) {
      const int cix = k * 64 + lane;
      const int rr = cix / CPR, cc = cix % CPR;
      float y[VPP];
#pragma unroll
      for (int h = 0; h < VPP / 4; ++h) {
        const v4f t = *reinterpret_cast<const v4f*>(&ep[rr * (EP / 4) + cc * VPP + 4 * h]);
#pragma unroll
        for (int r = 0; r < 4; ++r) y[4 * h + r] = t[r] * ts;
      }
      const int m = m0 + wm0 + i * 32 + rr;
      const int n = n0 + wn0 + cc * VPP;
      if (m >= M) continue;
      if constexpr (OUT_BF16) {
        __bf16* dst = reinterpret_cast<__bf16*>(Yv) + (size_t)m * N + n;
        v4u pk;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          pk[r] = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)y[2 * r]) |
                  ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)y[2 * r + 1]) << 16);
        if (vec && n + VPP <= N) {
          __builtin_nontemporal_store(pk, reinterpret_cast<v4u*>(dst));
        } else if (vec4 && n + VPP <= N) {  // rows 8-byte aligned only: two 8-byte halves
          typedef unsigned v2u_ __attribute__((ext_vector_type(2)));
          __builtin_nontemporal_store(v2u_{pk[0], pk[1]}, reinterpret_cast<v2u_*>(dst));
          __builtin_nontemporal_store(v2u_{pk[2], pk[3]}, reinterpret_cast<v2u_*>(dst) + 1);
        } else {
          for (int r = 0; r < VPP; ++r)
            if (n + r < N) dst[r] = (__bf16)y[r];
        }
      } else {
        float* dst = reinterpret_cast<float*>(Yv) + (size_t)m * N + n;
        if (vec && n + VPP <= N) {
          __builtin_nontemporal_store(v4f{y[0], y[1], y[2], y[3]}, reinterpret_cast<v4f*>(dst));
        } else {
          for (int r = 0; r < VPP; ++r)
            if (n + r < N) dst[r] = y[r];
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // slab read back before the next one overwrites it
  }
}

// Tile index L of a tiles_m x cnt grid -> (tm, tn): groups of 8 tile rows, M fastest.
__device__ __forceinline__ void map_tile(int L, int tiles_m, int cnt, int& tm, int& tn) {
  constexpr int GM = 8;
  const int first_m = (L / (GM * cnt)) * GM;
  const int gsize = min(tiles_m - first_m, GM);
  tm = first_m + (L % gsize);
  tn = (L % (GM * cnt)) / gsize;
}

// Workgroups [0, tiles_m * tn1) take 256-wide tiles of columns [0, 256 tn1); the rest take
// 192-wide tiles of the columns from 256 tn1 on. Each range is spread over the XCDs when its
// size is a multiple of 8.
template <bool OUT_BF16>
__global__ __launch_bounds__(NT) void gemm_nvfp4_ring(const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ Xs,
                                                      const float* __restrict__ x_ts, const uint8_t* __restrict__ Wq,
                                                      const uint8_t* __restrict__ Ws, const float* __restrict__ w_ts,
                                                      void* __restrict__ Yv, int M, int N, int K, int tiles_m, int tn1,
                                                      int tn2) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int T1 = tiles_m * tn1, T2 = tiles_m * tn2;
  int b = blockIdx.x, tm, tn;
  if (b < T1) {
    const int L = (T1 % 8 == 0) ? (b & 7) * (T1 >> 3) + (b >> 3) : b;
    map_tile(L, tiles_m, tn1, tm, tn);
    nv_tile<OUT_BF16, Wide>(smem, Xq, Xs, x_ts, Wq, Ws, w_ts, Yv, M, N, K, tm * BM, tn * Wide::BN);
  } else {
    b -= T1;
    const int L = (T1 % 8 == 0 && T2 % 8 == 0) ? (b & 7) * (T2 >> 3) + (b >> 3) : b;
    map_tile(L, tiles_m, tn2, tm, tn);
    nv_tile<OUT_BF16, Narrow>(smem, Xq, Xs, x_ts, Wq, Ws, w_ts, Yv, M, N, K, tm * BM, tn1 * Wide::BN + tn * Narrow::BN);
  }
}

// per kernel instantiation and device: the dynamic-LDS limit has been raised
template <bool B>
std::atomic<int> g_attr_done[64];
std::atomic<int> g_cus[64];  // compute units per device, 0 until queried

template <bool B>
hipError_t launch(const uint8_t* Xq, const uint8_t* Xs, const float* x_ts, const uint8_t* Wq, const uint8_t* Ws,
                  const float* w_ts, int M, int N, int K, void* Y, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  auto kern = gemm_nvfp4_ring<B>;
  const bool cached = dev >= 0 && dev < 64;
  if (!cached || !g_attr_done<B>[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    if (cached) g_attr_done<B>[dev].store(1, std::memory_order_release);
  }
  int cus = cached ? g_cus[dev].load(std::memory_order_acquire) : 0;
  if (cus == 0) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (cached) g_cus[dev].store(cus, std::memory_order_release);
  }
  const int tiles_m = (M + BM - 1) / BM;
  int tn1, tn2;
  fp4_plan_tile_columns(tiles_m, N, cus, kNvNarrowCost, tn1, tn2);
  hipLaunchKernelGGL(kern, dim3(tiles_m * (tn1 + tn2)), dim3(NT), LDS_BYTES, st, Xq, Xs, x_ts, Wq, Ws, w_ts, Y, M, N,
                     K, tiles_m, tn1, tn2);
  return hipGetLastError();
}

}  // namespace
}  // namespace fp4

bool fp4_gemm_nvfp4_ring_fits(int64_t M, int64_t N, int64_t K) { return K % 64 == 0 && M >= 256 && N >= 256; }

hipError_t fp4_launch_gemm_nvfp4_ring(const uint8_t* Xq, const uint8_t* Xs, const float* x_ts, const uint8_t* Wq,
                                      const uint8_t* Ws, const float* w_ts, int64_t M, int64_t N, int64_t K, void* Y,
                                      int out_bf16, hipStream_t st) {
  return out_bf16 ? fp4::launch<true>(Xq, Xs, x_ts, Wq, Ws, w_ts, (int)M, (int)N, (int)K, Y, st)
                  : fp4::launch<false>(Xq, Xs, x_ts, Wq, Ws, w_ts, (int)M, (int)N, (int)K, Y, st);
}
