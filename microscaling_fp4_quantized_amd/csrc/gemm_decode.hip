// Decode-shaped W4A4 MXFP4 GEMM for gfx950 (M <= 16 rows of activations, and up to 64 rows
// for layers whose K fits the per-wave slices).
//
// "Bridging the Gap Between Promise and Performance for Microscaling FP4
// Quantization" (gist.science, German edition), Technische Zusammenfassung §2
// "GPU-Kernel-Unterstützung (QuTLASS)": the 4-bit matmul of the online path,
// here in its token-generation shape, where W (N x K codes + scales) is the only
// large operand and the product is bound by reading W from HBM.
//
// Design for CDNA4 (measured on MI355X with W streamed from HBM):
//  * One workgroup owns T tiles of 16 output features (16 rows of W each) and all of K; its 8
//    waves split K into slices of 512 elements (256 code bytes of a row), slice s going to wave
//    s % 8. Each wave fetches its own slices straight into its own LDS area with the LDS DMA
//    (buffer_load_dwordx4 ... lds): one instruction per 4 rows x 256 contiguous bytes, a pattern
//    that streams from HBM nearly as well as whole 1 KB rows (loading W in the MFMA operand
//    layout, 16 rows x 64 bytes per instruction, streamed about 20% slower). Lane l of an
//    instruction fetches chunk (l % 16) ^ row of its row, so the fragment reads hit distinct banks.
//  * As soon as its own slices have landed, the wave multiplies them with
//    v_mfma_scale_f32_16x16x128_f8f6f4, W as the row operand and X as the column operand: lane l
//    carries row l % 16 and the 32-element group l / 16 of a 128-wide K step (16 bytes of codes,
//    one E8M0 byte), so the output fragment gives each lane 4 consecutive features of one token.
//    X (a few rows, resident in L2) and the E8M0 bytes are read per lane in that layout. No
//    workgroup barrier stands between a wave's data and its products; the waves' partial sums
//    meet once, through LDS, in a fixed order.
//  * T = 2 when there are at least three tiles per CU: the two tiles share every X fragment the
//    wave loads, which halves the X traffic that dominates at 16 tokens, and the half-size grid is
//    resident at once (two workgroups per CU).
//  * Layers whose slices do not fit the LDS area (K above 8192 / T) take a chunked variant: the
//    workgroup stages W through LDS in chunks of at most 4096 elements as whole 1 KB row pieces,
//    the next chunk's loads in flight while the current one is multiplied.
//  * Up to 64 tokens (MF = ceil(M / 16) column fragments of X): every W fragment a wave reads
//    is multiplied with each of the MF X fragments, so W is still read once and only the MFMA
//    count and the L2 reads of X grow with M; the partial sums of all MF x T output fragments
//    meet in the same fixed order.
//  X rows past M repeat row M-1 and W rows past N repeat row N-1; their outputs are discarded.
#include <atomic>
#include <type_traits>

#include "../../include/fp4.h"
#include "quant_device.hpp"

namespace fp4 {
namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kDecBatch = 4;     // consecutive K steps of 128 per wave within a chunk
constexpr int kDecMaxKC = 4096;  // K elements of a W chunk staged in LDS

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

// Raw buffer resource over [base, base + bytes): stride 0, last word 0x00020000 (32-bit data
// format in the gfx9-family descriptor layout, which untyped loads need). Offsets at or past
// `bytes` read as zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const uint8_t* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, (int)bytes, 0x00020000);
}

// LDS bytes of one tile chunk of KC elements: 16 rows of KC/2 code bytes, then 16 rows of KC/32 scale bytes.
__host__ __device__ constexpr int dec_tile_bytes(int kc) { return 16 * (kc / 2) + 16 * (kc / 32); }

// Chunk size: the largest multiple of 512 that divides K and is at most kDecMaxKC.
inline int dec_chunk(int64_t K) {
  int d = kDecMaxKC / 512;
  while ((K / 512) % d) --d;
  return 512 * d;
}

// W of the workgroup's T tiles for one chunk of KC elements, on its way from HBM to LDS. Piece
// p = wave + 8 j (1 KB) of a tile chunk: lane -> 16-byte slot p * 64 + lane, which holds global
// chunk (slot-in-row) ^ (row & 15) of its row; the first KC/32 threads also carry 16 scale bytes
// each. Buffer loads over each tile's rows (32-bit offsets; rows past N read as zero, and their
// outputs are discarded).
template <int T>
struct DecodeW {
  v4u wr[T][4], sr[T];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Ws, int N, int K,
                                       int KC, int nb, int ch, int wave, int lane) {
    const unsigned KB = (unsigned)K / 2, KS = (unsigned)K / 32;
    const int cb = KC / 2, cs = KC / 32, pieces = KC / 128;
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      const int n0 = __builtin_amdgcn_readfirstlane(min(nb + 16 * tt, N - 1));
      const unsigned rows = (unsigned)__builtin_amdgcn_readfirstlane(min(16, N - n0));
      const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(Wq + (size_t)n0 * KB, rows * KB);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = wave + 8 * j;
        if (p < pieces) {  // wave-uniform
          const int slot = p * 64 + lane, row = slot / (cb / 16), sl = slot % (cb / 16);
          wr[tt][j] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
              rw, (int)((unsigned)row * KB + (unsigned)(ch * cb + 16 * (sl ^ (row & 15)))), 0, 0));
        }
      }
      if ((int)threadIdx.x < cs) {
        const int row = (int)threadIdx.x / (cs / 16), c16 = (int)threadIdx.x % (cs / 16);
        const int n = min(n0 + row, N - 1);
        sr[tt] = *reinterpret_cast<const v4u*>(Ws + (size_t)n * KS + (size_t)ch * cs + 16 * c16);
      }
    }
  }

  // tile tt's chunk at lds + tt * dec_tile_bytes(KC): 16 code rows of KC/2 bytes, then 16 scale rows
  __device__ __forceinline__ void store(uint8_t* lds, int KC, int wave, int lane) const {
    const int cb = KC / 2, cs = KC / 32, pieces = KC / 128, tile = dec_tile_bytes(KC);
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (wave + 8 * j < pieces) *reinterpret_cast<v4u*>(lds + tt * tile + (wave + 8 * j) * 1024 + lane * 16) = wr[tt][j];
      if ((int)threadIdx.x < cs) {
        const int row = (int)threadIdx.x / (cs / 16), c16 = (int)threadIdx.x % (cs / 16);
        *reinterpret_cast<v4u*>(lds + tt * tile + 16 * cb + row * cs + 16 * c16) = sr[tt];
      }
    }
  }
};

// This wave's 4 steps of one chunk for each tile: v_mfma_scale_f32_16x16x128_f8f6f4 with W (from LDS)
// as the row operand: lane l carries row r = l % 16 and the 32-element group g = l / 16 of the step
// (16 bytes of codes, one E8M0 byte); X fragments xb and scale dwords xsv as the column operand.
template <int T>
__device__ __forceinline__ void decode_chunk_mfma(const uint8_t* lds, int KC, int s0, int r, int g, const v4u (&xb)[kDecBatch],
                                                  v4u xsv, v4f (&acc)[T]) {
  const int cb = KC / 2, cs = KC / 32, tile = dec_tile_bytes(KC);
  const unsigned sh = 8u * (unsigned)g;
#pragma unroll
  for (int tt = 0; tt < T; ++tt) {
    const uint8_t* tl = lds + tt * tile;
    const v4u wsv = *reinterpret_cast<const v4u*>(tl + 16 * cb + r * cs + 4 * s0);
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      const int c = 4 * (s0 + u) + g;  // 16-byte chunk of the row = 32-element group
      const v4u w = *reinterpret_cast<const v4u*>(tl + r * cb + 16 * (c ^ r));
      const v8i a = v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
      const v8i b = v8i{(int)xb[u][0], (int)xb[u][1], (int)xb[u][2], (int)xb[u][3], 0, 0, 0, 0};
      acc[tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[tt], 4, 4, 0, (int)(wsv[u] >> sh), 0,
                                                                  (int)(xsv[u] >> sh));
    }
  }
}

// Fixed-order reduction of the waves' partial sums through LDS (8 KB per tile at lds), then store.
template <bool OUT_BF16, int T>
__device__ __forceinline__ void decode_reduce_store(uint8_t* lds, const v4f (&acc)[T], int wave, int lane, void* Yv,
                                                    int M, int N, int nb) {
  __syncthreads();
  v4f* red = reinterpret_cast<v4f*>(lds);
#pragma unroll
  for (int tt = 0; tt < T; ++tt) red[(tt * kDecWaves + wave) * 64 + lane] = acc[tt];
  __syncthreads();
  if (wave >= T) return;
  const int tt = wave;
  v4f sum = red[(tt * kDecWaves) * 64 + lane];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) sum += red[(tt * kDecWaves + w) * 64 + lane];
  // lane holds D[n + 4g + i][m = r], i = 0..3: four consecutive features of token r
  store_out<OUT_BF16>(Yv, M, N, lane & 15, nb + 16 * tt + 4 * (lane >> 4), sum);
}

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kDecSlice = 512;  // K elements of a wave's slice: 256 code bytes and 16 E8M0 bytes of a row
constexpr int kDecMaxSlices = 2;  // tile-slices (4 KB each) a wave holds in LDS at once

// At most 128 VGPRs (4 waves per SIMD), so that two workgroups share a CU. NPER (1 or 2): slices
// per wave; wave w takes slices w and w + 8. LDS: 8 waves x NPER x T x 4 KB. MF (1..4): 16-token
// column fragments of X; the MF x T partial sums of a wave fit its area (MF x T KB <= NPER x T x 4 KB).
template <bool OUT_BF16, int T, int MF>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void gemm_mxfp4_decode(
    const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ Xs, const uint8_t* __restrict__ Wq,
    const uint8_t* __restrict__ Ws, void* __restrict__ Yv, int M, int N, int K, int NPER) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const unsigned KB = (unsigned)K / 2, KS = (unsigned)K / 32;
  const int nsl = K / kDecSlice;
  const int nb = blockIdx.x * 16 * T;
  const int area_bytes = NPER * T * 4096;
  uint8_t* area = lds + wave * area_bytes;  // tile-slice (j, tt) at (j * T + tt) * 4 KB: 16 rows x 256 bytes
  static_assert(MF >= 1 && MF <= 4 && MF * T <= kDecWaves, "column fragments");
  constexpr int NJ = kDecMaxSlices / T;  // the launch takes this kernel only when NPER <= NJ

  // W of the wave's slices into its area: instruction i of a tile-slice carries rows 4i .. 4i+3;
  // lane l lands at byte 16 * (l % 16) of row 4i + l / 16 and fetches the row's 16-byte chunk
  // (l % 16) ^ row there. Buffer loads over each tile's rows (32-bit offsets; rows past N read as
  // zero, and their outputs are discarded). The rows' E8M0 bytes of a slice go to registers.
  v4u wsv[NJ][T];
#pragma unroll
  for (int tt = 0; tt < T; ++tt) {
    const int n0 = __builtin_amdgcn_readfirstlane(min(nb + 16 * tt, N - 1));
    const unsigned rows = (unsigned)__builtin_amdgcn_readfirstlane(min(16, N - n0));
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(Wq + (size_t)n0 * KB, rows * KB);
    const size_t wrow = (size_t)min(n0 + r, N - 1);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int sl = wave + 8 * j;
      if (j < NPER && sl < nsl) {  // wave-uniform
        uint8_t* dst = area + (j * T + tt) * 4096;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * i + (lane >> 4), q = lane & 15;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(dst + i * 1024), 16,
                                                   (unsigned)row * KB + (unsigned)sl * 256u + 16u * (unsigned)(q ^ row),
                                                   0, 0, 0);
        }
        wsv[j][tt] = *reinterpret_cast<const v4u*>(Ws + wrow * KS + (size_t)sl * 16);
      }
    }
  }
  v4f acc[MF][T];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int tt = 0; tt < T; ++tt) acc[f][tt] = v4f{0.f, 0.f, 0.f, 0.f};
  const unsigned sh = 8u * (unsigned)g;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int sl = wave + 8 * j;
    if (j < NPER && sl < nsl) {
      // X fragment f of the slice into buffer f % 2: token 16 f + r (clamped to M - 1), the lane's
      // 16 code bytes of each of the 4 steps and the 4 E8M0 bytes of its row. Two fragments are
      // requested before the wait for W; fragment f + 2 right after the products of fragment f
      // are issued, so its L2 latency overlaps those of fragment f + 1.
      v4u xb[2][kDecBatch], xsv[2];
      auto load_x = [&](int f) {
        const size_t xrow = (size_t)min(16 * f + r, M - 1);
#pragma unroll
        for (int u = 0; u < kDecBatch; ++u)
          xb[f & 1][u] = *reinterpret_cast<const v4u*>(Xq + xrow * KB + (size_t)sl * 256 + 64 * u + 16 * g);
        xsv[f & 1] = *reinterpret_cast<const v4u*>(Xs + xrow * KS + (size_t)sl * 16);
      };
      load_x(0);
      if (MF > 1) load_x(1);
      // this wave's DMA has landed (its area is read by no other wave until the reduction)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      asm volatile("" ::: "memory");
      v4u wf[T][kDecBatch];  // every fragment read first, then the products
#pragma unroll
      for (int tt = 0; tt < T; ++tt)
#pragma unroll
        for (int u = 0; u < kDecBatch; ++u)
          wf[tt][u] = *reinterpret_cast<const v4u*>(area + (j * T + tt) * 4096 + r * 256 + 16 * (((4 * u + g) ^ r) & 15));
#pragma unroll
      for (int f = 0; f < MF; ++f) {
#pragma unroll
        for (int tt = 0; tt < T; ++tt)
#pragma unroll
          for (int u = 0; u < kDecBatch; ++u) {
            const v4u& x = xb[f & 1][u];
            const v8i a = v8i{(int)wf[tt][u][0], (int)wf[tt][u][1], (int)wf[tt][u][2], (int)wf[tt][u][3], 0, 0, 0, 0};
            const v8i b = v8i{(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
            acc[f][tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[f][tt], 4, 4, 0,
                                                                         (int)(wsv[j][tt][u] >> sh), 0,
                                                                         (int)(xsv[f & 1][u] >> sh));
          }
        if (f + 2 < MF) load_x(f + 2);
      }
    }
  }
  // partial sums into the wave's own area (its fragment reads are done), then the fixed-order sum
  // of output fragment (f, tt) by wave f * T + tt
  v4f* red = reinterpret_cast<v4f*>(area);
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int tt = 0; tt < T; ++tt) red[(f * T + tt) * 64 + lane] = acc[f][tt];
  __syncthreads();
  if (wave >= MF * T) return;
  const int q = wave, f = q / T, tt = q % T;
  v4f sum = reinterpret_cast<const v4f*>(lds)[q * 64 + lane];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) sum += reinterpret_cast<const v4f*>(lds + w * area_bytes)[q * 64 + lane];
  // lane holds D[n + 4g + i][m = 16 f + r], i = 0..3: four consecutive features of one token
  store_out<OUT_BF16>(Yv, M, N, 16 * f + (lane & 15), nb + 16 * tt + 4 * (lane >> 4), sum);
}

// The chunked variant for long K. At most 128 VGPRs (4 waves per SIMD).
template <bool OUT_BF16, int T>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void gemm_mxfp4_decode_chunked(
    const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ Xs, const uint8_t* __restrict__ Wq,
    const uint8_t* __restrict__ Ws, void* __restrict__ Yv, int M, int N, int K, int KC) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const size_t KB = (size_t)K / 2, KS = (size_t)K / 32;
  const int cb = KC / 2, cs = KC / 32;
  const int nch = K / KC, steps = KC / 128;
  const int nb = blockIdx.x * 16 * T;
  const uint8_t* xp = Xq + (size_t)min(r, M - 1) * KB + 16 * g;
  const uint8_t* xsp = Xs + (size_t)min(r, M - 1) * KS;
  const int s0 = wave * kDecBatch;  // this wave's first K step within a chunk (steps % 4 == 0)

  DecodeW<T> w;
  v4f acc[T];
#pragma unroll
  for (int tt = 0; tt < T; ++tt) acc[tt] = v4f{0.f, 0.f, 0.f, 0.f};
  w.load(Wq, Ws, N, K, KC, nb, 0, wave, lane);
  for (int ch = 0; ch < nch; ++ch) {
    // this wave's X fragments of the chunk (a wave past the last step loads clamped ones it does not use)
    v4u xb[kDecBatch];
    const uint8_t* xc = xp + (size_t)ch * cb;
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) xb[u] = *reinterpret_cast<const v4u*>(xc + 64 * (size_t)min(s0 + u, steps - 1));
    const v4u xsv = *reinterpret_cast<const v4u*>(xsp + (size_t)ch * cs + 4 * (size_t)min(s0, steps - kDecBatch));
    if (ch > 0) __syncthreads();  // every wave is done reading the previous chunk
    w.store(lds, KC, wave, lane);
    __syncthreads();
    if (ch + 1 < nch) w.load(Wq, Ws, N, K, KC, nb, ch + 1, wave, lane);  // in flight during this chunk
    if (s0 < steps) decode_chunk_mfma<T>(lds, KC, s0, r, g, xb, xsv, acc);
  }
  decode_reduce_store<OUT_BF16, T>(lds, acc, wave, lane, Yv, M, N, nb);
}

// ---------------------------------------------------------------------------
// Fused decode step: every workgroup first rotates and quantizes the (tiny) bf16 X into LDS
// with the same device code as fp4_rotate_quantize (so the codes are the same bits), then
// multiplies 16 rows of W with its X fragments read from LDS. One launch instead of two; X
// (M <= 16 rows) is read from L2 by every workgroup. W is read straight into registers in the
// MFMA operand layout (lane l: row l % 16, 16 bytes of the 32-element group l / 16 of a 128-wide
// K step), each wave taking batches of 4 steps round-robin over K; the first batch and its scales
// are requested before X is quantized, so their HBM latency overlaps the quantization. (Staging W
// through LDS in coalesced pieces, as gemm_mxfp4_decode does, measured slower here at one token:
// the extra LDS pass and barrier fall after the quantization, on the critical path.)
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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int r = lane & 15, g = lane >> 4;
  const int steps = K / 128;
  const uint8_t* wp = Wq + (size_t)min(n0 + r, N - 1) * KB + 16 * g;
  const uint8_t* wsp = Ws + (size_t)min(n0 + r, N - 1) * KS;
  // a batch of W: steps t0 .. t0 + 3 (clamped into the row; the MFMA loop skips steps past the end)
  v4u wa[kDecBatch], wsv;
  auto load_w = [&](int t0) {
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u)
      wa[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wp + 64 * (size_t)min(t0 + u, steps - 1)));
    wsv = *reinterpret_cast<const v4u*>(wsp + 4 * (size_t)min(t0, steps - kDecBatch));
  };
  load_w(wave * kDecBatch);

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
        const v4u x4 = src[q];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[8 * q + 2 * t] = bf16_lo(x4[t]);
          v[8 * q + 2 * t + 1] = bf16_hi(x4[t]);
        }
      }
      v4u out;
      const int code = mx_rotate_quantize_chunk<B, kRuleStandard>(v, out);
      *reinterpret_cast<v4u*>(xq + (size_t)row * pitch + (size_t)cc * 16) = out;
      xs[row * KS + cc] = (uint8_t)code;
    }
  }
  __syncthreads();

  // phase 2: v_mfma_scale_f32_16x16x128_f8f6f4 with W as the row operand, X from LDS
  const uint8_t* xp = xq + (size_t)min(r, M - 1) * pitch + 16 * g;
  const uint8_t* xsp = xs + (size_t)min(r, M - 1) * KS;
  const unsigned sh = 8u * (unsigned)g;
  v4f acc[1] = {v4f{0.f, 0.f, 0.f, 0.f}};
  for (int t0 = wave * kDecBatch; t0 < steps; t0 += kDecWaves * kDecBatch) {
    if (t0 != wave * kDecBatch) load_w(t0);  // the first batch is already in flight
    v4u xb[kDecBatch];
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) xb[u] = *reinterpret_cast<const v4u*>(xp + 64 * min(t0 + u, steps - 1));
    const v4u xsv = *reinterpret_cast<const v4u*>(xsp + 4 * min(t0, steps - kDecBatch));
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      if (t0 + u < steps) {
        const v8i a = v8i{(int)wa[u][0], (int)wa[u][1], (int)wa[u][2], (int)wa[u][3], 0, 0, 0, 0};
        const v8i b = v8i{(int)xb[u][0], (int)xb[u][1], (int)xb[u][2], (int)xb[u][3], 0, 0, 0, 0};
        acc[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[0], 4, 4, 0, (int)(wsv[u] >> sh), 0,
                                                                   (int)(xsv[u] >> sh));
      }
    }
  }
  decode_reduce_store<OUT_BF16, 1>(lds, acc, wave, lane, Yv, M, N, n0);  // X in LDS is dead after its first barrier
}

// Fused decode step for K up to 8192 / T: each wave first sends its W slices (as in
// gemm_mxfp4_decode) to its LDS area with the LDS DMA, after requesting its first X chunks, so W
// streams in while X is quantized; then every wave multiplies its slices with X fragments read from
// LDS. With T = 2 a workgroup owns two 16-row tiles and quantizes X once for both.
constexpr int kFusedPre = 2;  // phase-1 iterations whose X loads are issued before the W DMA

template <int B, bool OUT_BF16, int T, int NPER>
__global__ __launch_bounds__(kDecThreads) void decode_fused_sliced(const uint16_t* __restrict__ X, int64_t ldx,
                                                                   const uint8_t* __restrict__ Wq,
                                                                   const uint8_t* __restrict__ Ws, void* __restrict__ Yv,
                                                                   int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const unsigned KB = (unsigned)K / 2, KS = (unsigned)K / 32;
  const int pitch = (int)KB + 16;  // padded X code rows: distinct banks per row
  const int nsl = K / kDecSlice;
  const int nb = blockIdx.x * 16 * T;
  constexpr int area_bytes = NPER * T * 4096;
  uint8_t* area = lds + wave * area_bytes;
  uint8_t* xq = lds + kDecWaves * area_bytes;  // [M][pitch]
  uint8_t* xs = xq + (size_t)M * pitch;        // [M][KS]
  const int total = M * (int)KS;

  // phase-1 chunk c -> row c / KS, chunk c % KS. Quads of lanes hold the consecutive chunks of
  // one Hadamard block (KS % 16 == 0, and the loop base is a multiple of 512), and whole quads
  // are in or out of range together (total % 4 == 0). The first iterations' X loads go out
  // before the W DMA, and every load below is issued unconditionally (lanes past the end load a
  // clamped chunk, waves past the last slice an out-of-range one, which reads zeros without
  // touching memory), so the wait for X counts exactly the later W loads and lets them fly.
  v4u xr[kFusedPre][4];
#pragma unroll
  for (int it = 0; it < kFusedPre; ++it) {
    const int c = min(it * kDecThreads + (int)threadIdx.x, total - 1);
    const int row = c / (int)KS, cc = c - row * (int)KS;
    const v4u* src = reinterpret_cast<const v4u*>(X + (size_t)row * (size_t)ldx + (size_t)cc * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) xr[it][q] = src[q];
  }
  v4u wsv[NPER][T];
#pragma unroll
  for (int tt = 0; tt < T; ++tt) {
    const int n0 = __builtin_amdgcn_readfirstlane(min(nb + 16 * tt, N - 1));
    const unsigned rows = (unsigned)__builtin_amdgcn_readfirstlane(min(16, N - n0));
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(Wq + (size_t)n0 * KB, rows * KB);
    const size_t wrow = (size_t)min(n0 + r, N - 1);
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const int sl = wave + 8 * j;
      uint8_t* dst = area + (j * T + tt) * 4096;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * i + (lane >> 4), q = lane & 15;
        const unsigned off = sl < nsl ? (unsigned)row * KB + (unsigned)sl * 256u + 16u * (unsigned)(q ^ row) : 0xFFFFFFF0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(dst + i * 1024), 16, off, 0, 0, 0);
      }
      wsv[j][tt] = *reinterpret_cast<const v4u*>(Ws + wrow * KS + (size_t)min(sl, nsl - 1) * 16);
    }
  }

  // phase 1: rotate and quantize X into LDS with the quantizer's own device code
  for (int c0 = 0; c0 < total; c0 += kDecThreads) {
    const int c = c0 + (int)threadIdx.x;
    const int it = c0 / kDecThreads;
    if (c < total) {
      const int row = c / (int)KS, cc = c - row * (int)KS;
      v4u x4[4];
      if (it < kFusedPre) {
#pragma unroll
        for (int q = 0; q < 4; ++q) x4[q] = it == 0 ? xr[0][q] : xr[kFusedPre - 1][q];
      } else {
        const v4u* src = reinterpret_cast<const v4u*>(X + (size_t)row * (size_t)ldx + (size_t)cc * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) x4[q] = src[q];
      }
      float v[32];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[8 * q + 2 * t] = bf16_lo(x4[q][t]);
          v[8 * q + 2 * t + 1] = bf16_hi(x4[q][t]);
        }
      v4u out;
      const int code = mx_rotate_quantize_chunk<B, kRuleStandard>(v, out);
      *reinterpret_cast<v4u*>(xq + (size_t)row * pitch + (size_t)cc * 16) = out;
      xs[(size_t)row * KS + cc] = (uint8_t)code;
    }
  }
  __syncthreads();  // X is in LDS

  // phase 2: this wave's slices once its DMA has landed
  const uint8_t* xp = xq + (size_t)min(r, M - 1) * pitch + 16 * g;
  const uint8_t* xsp = xs + (size_t)min(r, M - 1) * KS;
  const unsigned sh = 8u * (unsigned)g;
  v4f acc[T];
#pragma unroll
  for (int tt = 0; tt < T; ++tt) acc[tt] = v4f{0.f, 0.f, 0.f, 0.f};
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  asm volatile("" ::: "memory");
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const int sl = wave + 8 * j;
    if (sl < nsl) {
      v4u xb[kDecBatch], wf[T][kDecBatch];
#pragma unroll
      for (int u = 0; u < kDecBatch; ++u) xb[u] = *reinterpret_cast<const v4u*>(xp + (size_t)sl * 256 + 64 * u);
      const v4u xsv = *reinterpret_cast<const v4u*>(xsp + (size_t)sl * 16);
#pragma unroll
      for (int tt = 0; tt < T; ++tt)
#pragma unroll
        for (int u = 0; u < kDecBatch; ++u)
          wf[tt][u] = *reinterpret_cast<const v4u*>(area + (j * T + tt) * 4096 + r * 256 + 16 * (((4 * u + g) ^ r) & 15));
#pragma unroll
      for (int tt = 0; tt < T; ++tt)
#pragma unroll
        for (int u = 0; u < kDecBatch; ++u) {
          const v8i a = v8i{(int)wf[tt][u][0], (int)wf[tt][u][1], (int)wf[tt][u][2], (int)wf[tt][u][3], 0, 0, 0, 0};
          const v8i b = v8i{(int)xb[u][0], (int)xb[u][1], (int)xb[u][2], (int)xb[u][3], 0, 0, 0, 0};
          acc[tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[tt], 4, 4, 0, (int)(wsv[j][tt][u] >> sh), 0,
                                                                      (int)(xsv[u] >> sh));
        }
    }
  }
  v4f* red = reinterpret_cast<v4f*>(area);
#pragma unroll
  for (int tt = 0; tt < T; ++tt) red[tt * 64 + lane] = acc[tt];
  __syncthreads();
  if (wave >= T) return;
  const int tt = wave;
  v4f sum = reinterpret_cast<const v4f*>(lds)[tt * 64 + lane];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) sum += reinterpret_cast<const v4f*>(lds + w * area_bytes)[tt * 64 + lane];
  store_out<OUT_BF16>(Yv, M, N, lane & 15, nb + 16 * tt + 4 * (lane >> 4), sum);
}

// X codes and scales; at least the 8 KB the reduction reuses
size_t fused_lds_bytes(int M, int K) {
  const size_t x = (size_t)M * (K / 2 + 16) + (size_t)M * (K / 32);
  return x > (size_t)kDecWaves * 64 * 16 ? x : (size_t)kDecWaves * 64 * 16;
}

std::atomic<int> g_fused_attr[4][64];  // per block size and device: dynamic-LDS limits raised
std::atomic<int> g_cus[64];            // compute units per device, 0 until queried

hipError_t device_cus(int dev, int& cus) {
  const bool cached = dev >= 0 && dev < 64;
  cus = cached ? g_cus[dev].load(std::memory_order_acquire) : 0;
  if (cus != 0) return hipSuccess;
  const hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && cached) g_cus[dev].store(cus, std::memory_order_release);
  return e;
}

// Launch plan of the fused step: the sliced kernel when every wave's slices fit its LDS area
// beside X; two tiles per workgroup once there are at least three tiles per CU and two
// workgroups still fit a CU. Otherwise the register-streaming kernel, one tile per workgroup.
struct FusedPlan {
  bool sliced;
  int T, nper, grid;
  size_t lds;
};

FusedPlan fused_plan(int64_t M, int64_t N, int64_t K, int cus) {
  const size_t xb = (size_t)M * (K / 2 + 16) + (size_t)M * (K / 32);
  const int nper = (int)((K / kDecSlice + kDecWaves - 1) / kDecWaves);
  const int tiles = (int)((N + 15) / 16);
  FusedPlan p{false, 1, nper, tiles, fused_lds_bytes((int)M, (int)K)};
  if (nper <= kDecMaxSlices && (size_t)kDecWaves * nper * 4096 + xb <= 160 * 1024) {
    p.sliced = true;
    p.T = nper == 1 && tiles >= 3 * cus && (size_t)kDecWaves * 2 * 4096 + xb <= 80 * 1024 ? 2 : 1;
    p.grid = (tiles + p.T - 1) / p.T;
    p.lds = (size_t)kDecWaves * nper * p.T * 4096 + xb;
  }
  return p;
}

template <int B>
hipError_t launch_fused(const uint16_t* X, int64_t ldx, const uint8_t* Wq, const uint8_t* Ws, int M, int N, int K,
                        void* Y, int out_bf16, hipStream_t st) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = device_cus(dev, cus);
  if (e != hipSuccess) return e;
  const int bi = B == 16 ? 0 : B == 32 ? 1 : B == 64 ? 2 : 3;
  const bool cached = dev >= 0 && dev < 64;
  if (!cached || g_fused_attr[bi][dev].load(std::memory_order_acquire) == 0) {
    const void* kerns[8] = {(const void*)decode_fused<B, false>, (const void*)decode_fused<B, true>,
                            (const void*)decode_fused_sliced<B, false, 1, 1>, (const void*)decode_fused_sliced<B, true, 1, 1>,
                            (const void*)decode_fused_sliced<B, false, 2, 1>, (const void*)decode_fused_sliced<B, true, 2, 1>,
                            (const void*)decode_fused_sliced<B, false, 1, 2>, (const void*)decode_fused_sliced<B, true, 1, 2>};
    for (const void* k : kerns) {
      e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
    }
    if (cached) g_fused_attr[bi][dev].store(1, std::memory_order_release);
  }
  const FusedPlan pl = fused_plan(M, N, K, cus);
  const int tiles = (N + 15) / 16, nper = pl.nper;
  if (pl.sliced) {
    const bool two = pl.T == 2;
    const int T = pl.T;
    const size_t lds = pl.lds;
    auto kern = two         ? (out_bf16 ? decode_fused_sliced<B, true, 2, 1> : decode_fused_sliced<B, false, 2, 1>)
                : nper == 1 ? (out_bf16 ? decode_fused_sliced<B, true, 1, 1> : decode_fused_sliced<B, false, 1, 1>)
                            : (out_bf16 ? decode_fused_sliced<B, true, 1, 2> : decode_fused_sliced<B, false, 1, 2>);
    hipLaunchKernelGGL(kern, dim3((unsigned)((tiles + T - 1) / T)), dim3(kDecThreads), lds, st, X, ldx, Wq, Ws, Y, M, N, K);
    return hipGetLastError();
  }
  auto kern = out_bf16 ? decode_fused<B, true> : decode_fused<B, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kDecThreads), fused_lds_bytes(M, K), st, X, ldx, Wq, Ws, Y, M, N,
                     K);
  return hipGetLastError();
}

}  // namespace
}  // namespace fp4

// 16 rows of W and their 32-bit buffer offsets: 16 * K / 2 < 2^32
// M <= 16: any K (the chunked kernel takes long K). 16 < M <= 64: the sliced kernel only, whose
// per-wave slices hold K <= 8192 with one tile per workgroup.
bool fp4_gemm_mxfp4_decode_fits(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && N >= 1 && K % 512 == 0 && (M <= 16 ? K < ((int64_t)1 << 28) : (M <= 64 && K <= 8192));
}

namespace fp4 {
namespace {
std::atomic<int> g_dec_attr[2][2][4][64];  // per output dtype, T, MF and device: dynamic-LDS limit raised

template <bool OUT_BF16, int T, int MF>
hipError_t launch_decode(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws, int M, int N, int K,
                         void* Y, int dev, hipStream_t st) {
  const int nper = (K / kDecSlice + kDecWaves - 1) / kDecWaves;  // slices per wave
  const bool sliced = nper <= kDecMaxSlices / T;
  if (MF > 1 && !sliced) return hipErrorInvalidValue;  // excluded by fp4_gemm_mxfp4_decode_fits and the T choice
  const int KC = dec_chunk(K);
  auto kern = sliced ? gemm_mxfp4_decode<OUT_BF16, T, MF> : gemm_mxfp4_decode_chunked<OUT_BF16, T>;
  const int lds = sliced ? kDecWaves * nper * T * 4096
                         : T * (dec_tile_bytes(KC) > kDecWaves * 64 * 16 ? dec_tile_bytes(KC) : kDecWaves * 64 * 16);
  const bool cached = dev >= 0 && dev < 64;
  if (!cached || !g_dec_attr[OUT_BF16][T - 1][MF - 1][dev].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_mxfp4_decode<OUT_BF16, T, MF>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)gemm_mxfp4_decode_chunked<OUT_BF16, T>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    if (cached) g_dec_attr[OUT_BF16][T - 1][MF - 1][dev].store(1, std::memory_order_release);
  }
  const int tiles = (N + 15) / 16;
  hipLaunchKernelGGL(kern, dim3((unsigned)((tiles + T - 1) / T)), dim3(kDecThreads), lds, st, Xq, Xs, Wq, Ws, Y, M, N, K,
                     sliced ? nper : KC);
  return hipGetLastError();
}
}  // namespace
}  // namespace fp4

hipError_t fp4_launch_gemm_mxfp4_decode(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                                        int64_t M, int64_t N, int64_t K, void* Y, int out_bf16, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = 0;
  e = fp4::device_cus(dev, cus);
  if (e != hipSuccess) return e;
  // two tiles per workgroup once there are at least three tiles per CU: the tiles share the X
  // fragments, and every workgroup is resident at once (two per CU at up to 128 VGPRs). Above
  // 16 tokens only the sliced kernel runs, which holds two tiles' slices up to K = 4096.
  const int mf = (int)((M + 15) / 16);
  const bool two = (N + 15) / 16 >= 3 * (int64_t)cus && (mf == 1 || K <= 4096);
  const int m = (int)M, n = (int)N, k = (int)K;
  auto go = [&](auto bf16, auto t, auto f) {
    return fp4::launch_decode<decltype(bf16)::value, decltype(t)::value, decltype(f)::value>(Xq, Xs, Wq, Ws, m, n, k,
                                                                                             Y, dev, st);
  };
  auto with_mf = [&](auto bf16, auto t) {
    switch (mf) {
      case 1: return go(bf16, t, std::integral_constant<int, 1>{});
      case 2: return go(bf16, t, std::integral_constant<int, 2>{});
      case 3: return go(bf16, t, std::integral_constant<int, 3>{});
      default: return go(bf16, t, std::integral_constant<int, 4>{});
    }
  };
  auto with_t = [&](auto bf16) {
    return two ? with_mf(bf16, std::integral_constant<int, 2>{}) : with_mf(bf16, std::integral_constant<int, 1>{});
  };
  return out_bf16 ? with_t(std::true_type{}) : with_t(std::false_type{});
}

hipError_t fp4_device_cus(int dev, int* cus) { return fp4::device_cus(dev, *cus); }

bool fp4_decode_fused_fits(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 16 && N >= 1 && K % 512 == 0 && fp4::fused_lds_bytes((int)M, (int)K) <= 160 * 1024;
}

// Every workgroup of the fused step quantizes all M rows of X, so its cost grows with the rows
// quantized per CU, M times the workgroups per CU. Measured on MI355X with W from HBM, K = 4096
// (one launch against two): N = 4096, one workgroup per CU, 12 tokens 6.9 against 7.3 us, 16
// tokens 8.0 against 7.6 us; N = 14336, 1.75 workgroups per CU up to 7 tokens, 6 tokens 9.0
// against 10.8 us, then 3.5 per CU, 8 tokens 12.3 against 11.0 us. The crossover lies near 14
// rows per CU on both.
// The allocation-free decode step's workspace: one array per GPU, in the library's device
// image, held until the process ends. Host code uses the address hipGetSymbolAddress returns for
// the current device (the array's name on the host is only a stand-in), fetched on the first call
// on each device and kept.
static __device__ __align__(256) uint8_t scratch[FP4_DECODE_SCRATCH_BYTES];
static std::atomic<uint8_t*> g_scratch[64];

hipError_t fp4_decode_scratch(uint8_t** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  uint8_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(reinterpret_cast<void**>(&p), HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t fp4_decode_fused_preferred(int64_t M, int64_t N, int64_t K, bool* fused) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = fp4::device_cus(dev, cus);
  if (e != hipSuccess) return e;
  const fp4::FusedPlan p = fp4::fused_plan(M, N, K, cus);
  *fused = M * (int64_t)p.grid <= 14 * (int64_t)cus;
  return hipSuccess;
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

// ---------------------------------------------------------------------------
// NVFP4 decode (M <= 16, or up to 64 rows as MF = ceil(M / 16) column fragments of X that share
// every dequantized W fragment): the weight streaming of gemm_mxfp4_decode, with the E4M3 group scales
// applied by dequantizing both operands exactly to fp16 in registers (e2m1 * d has at most 6
// significant bits within [2^-10, 2688]) and multiplying with v_mfma_f32_16x16x32_f16: W (from
// the wave's LDS area) as the row operand, X (M rows, read from L2) as the column operand, so each
// lane again ends with 4 consecutive features of one token. Within each 128-element block q of a
// slice, k-step t of lane group g takes elements 32 (4 q + g) + 8 t .. + 7 of both operands: a
// lane reads one 16-byte chunk of codes per block, and every product still pairs x_k with w_k.
// The reduced sums are multiplied by x_ts * w_ts.
// "Bridging the Gap Between Promise and Performance for Microscaling FP4 Quantization"
// (gist.science, Spanish edition), Resumen técnico §2.B item 2 (NVFP4 group and tensor scales).
// ---------------------------------------------------------------------------
namespace fp4 {
namespace {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));

// E4M3 codes in the low two bytes of w -> the exact fp16 pair (every E4M3FN value is an fp16 number)
__device__ __forceinline__ h2v nv_scale_pair(unsigned w) { return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false); }

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times the fp16 scale d
__device__ __forceinline__ h8v nv_dequant8(unsigned codes, _Float16 d) {
  const h2v dd = {d, d};
  v4u o;
  o[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * dd);
  o[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * dd);
  o[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * dd);
  o[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * dd);
  return __builtin_bit_cast(h8v, o);
}

// The two scale bytes of chunk c = 4 q + g (bytes 2c, 2c + 1 of a row's 32 per slice): dword
// 2 q + g / 2 of the 8, half g % 2.
template <int Q>
__device__ __forceinline__ h2v nv_chunk_scales(const v4u (&s)[2], int g) {
  constexpr int d0 = 2 * Q, d1 = 2 * Q + 1;
  const unsigned w = (g >> 1) ? s[d1 >> 2][d1 & 3] : s[d0 >> 2][d0 & 3];
  return nv_scale_pair(w >> (16 * (g & 1)));
}

// At most 128 VGPRs (4 waves per SIMD). NPER slices per wave, as gemm_mxfp4_decode.
template <bool OUT_BF16, int T, int MF>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void gemm_nvfp4_decode(
    const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ Xs, const float* __restrict__ x_ts,
    const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Ws, const float* __restrict__ w_ts,
    void* __restrict__ Yv, int M, int N, int K, int NPER) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int NJ = kDecMaxSlices / T;  // the launch takes this kernel only when NPER <= NJ
  static_assert(MF >= 1 && MF <= 4 && MF * T <= kDecWaves, "column fragments");
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const unsigned KB = (unsigned)K / 2, KS = (unsigned)K / 16;
  const int nsl = K / kDecSlice;
  const int nb = blockIdx.x * 16 * T;
  const int area_bytes = NPER * T * 4096;
  uint8_t* area = lds + wave * area_bytes;  // tile-slice (j, tt) at (j * T + tt) * 4 KB: 16 rows x 256 bytes

  // W codes of the wave's slices into its area by the LDS DMA, as in gemm_mxfp4_decode (the code
  // layout is the same); the 32 E4M3 bytes of the lane's row and slice into registers.
  v4u wsv[NJ][T][2];
#pragma unroll
  for (int tt = 0; tt < T; ++tt) {
    const int n0 = __builtin_amdgcn_readfirstlane(min(nb + 16 * tt, N - 1));
    const unsigned rows = (unsigned)__builtin_amdgcn_readfirstlane(min(16, N - n0));
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(Wq + (size_t)n0 * KB, rows * KB);
    const size_t wrow = (size_t)min(n0 + r, N - 1);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int sl = wave + 8 * j;
      if (j < NPER && sl < nsl) {  // wave-uniform
        uint8_t* dst = area + (j * T + tt) * 4096;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * i + (lane >> 4), q = lane & 15;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(dst + i * 1024), 16,
                                                   (unsigned)row * KB + (unsigned)sl * 256u + 16u * (unsigned)(q ^ row),
                                                   0, 0, 0);
        }
        const uint8_t* ps = Ws + wrow * KS + (size_t)sl * 32;
        wsv[j][tt][0] = *reinterpret_cast<const v4u*>(ps);
        wsv[j][tt][1] = *reinterpret_cast<const v4u*>(ps + 16);
      }
    }
  }
  v4f acc[MF][T];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int tt = 0; tt < T; ++tt) acc[f][tt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int sl = wave + 8 * j;
    if (j < NPER && sl < nsl) {
      // X fragment f: token 16 f + r (clamped to M - 1); per block q, chunk 4 q + g of the slice
      // and the two E4M3 bytes of that chunk
      auto x_codes = [&](int f, int q) {
        const size_t xrow = (size_t)min(16 * f + r, M - 1);
        return *reinterpret_cast<const v4u*>(Xq + xrow * KB + (size_t)sl * 256 + 16 * (4 * q + g));
      };
      auto x_scales = [&](int f, int q) {  // the dword of the token's slice scales holding them
        const size_t xrow = (size_t)min(16 * f + r, M - 1);
        const unsigned w = *reinterpret_cast<const unsigned*>(Xs + xrow * KS + (size_t)sl * 32 + 4 * (2 * q + (g >> 1)));
        return nv_scale_pair(w >> (16 * (g & 1)));
      };
      auto w_chunk = [&](int tt, int q) {
        return *reinterpret_cast<const v4u*>(area + (j * T + tt) * 4096 + r * 256 + 16 * (((4 * q + g) ^ r) & 15));
      };
      if constexpr (MF == 1) {
        // one X fragment: all of its codes and scales of the slice requested before the wait for W,
        // and each W fragment dequantized right before its product
        v4u xc[4], xsv[2];
#pragma unroll
        for (int q = 0; q < 4; ++q) xc[q] = x_codes(0, q);
        const uint8_t* pxs = Xs + (size_t)min(r, M - 1) * KS + (size_t)sl * 32;
        xsv[0] = *reinterpret_cast<const v4u*>(pxs);
        xsv[1] = *reinterpret_cast<const v4u*>(pxs + 16);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA has landed
        asm volatile("" ::: "memory");
        auto block1 = [&](auto qc) {
          constexpr int q = decltype(qc)::value;
          const h2v dx = nv_chunk_scales<q>(xsv, g);
          v4u wc[T];
          h2v dw[T];
#pragma unroll
          for (int tt = 0; tt < T; ++tt) {
            wc[tt] = w_chunk(tt, q);
            dw[tt] = nv_chunk_scales<q>(wsv[j][tt], g);
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) {  // elements 32 (4 q + g) + 8 t .. + 7: group 2 (4 q + g) + t / 2
            const h8v b = nv_dequant8(xc[q][t], t < 2 ? dx[0] : dx[1]);
#pragma unroll
            for (int tt = 0; tt < T; ++tt) {
              const h8v a = nv_dequant8(wc[tt][t], t < 2 ? dw[tt][0] : dw[tt][1]);
              acc[0][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[0][tt], 0, 0, 0);
            }
          }
        };
        block1(std::integral_constant<int, 0>{});
        block1(std::integral_constant<int, 1>{});
        block1(std::integral_constant<int, 2>{});
        block1(std::integral_constant<int, 3>{});
        continue;
      }
      // several X fragments: the first block of each requested before the wait for W; per block, W
      // dequantized once and shared by the MF fragments
      v4u xc0[MF];
      h2v dx0[MF];
#pragma unroll
      for (int f = 0; f < MF; ++f) {
        xc0[f] = x_codes(f, 0);
        dx0[f] = x_scales(f, 0);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA has landed
      asm volatile("" ::: "memory");
      auto block = [&](auto qc) {
        constexpr int q = decltype(qc)::value;
        h8v wf[T][4];
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
          const v4u wc = w_chunk(tt, q);
          const h2v dw = nv_chunk_scales<q>(wsv[j][tt], g);
#pragma unroll
          for (int t = 0; t < 4; ++t) wf[tt][t] = nv_dequant8(wc[t], t < 2 ? dw[0] : dw[1]);
        }
#pragma unroll
        for (int f = 0; f < MF; ++f) {
          const v4u xc = q == 0 ? xc0[f] : x_codes(f, q);
          const h2v dx = q == 0 ? dx0[f] : x_scales(f, q);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const h8v b = nv_dequant8(xc[t], t < 2 ? dx[0] : dx[1]);
#pragma unroll
            for (int tt = 0; tt < T; ++tt)
              acc[f][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[tt][t], b, acc[f][tt], 0, 0, 0);
          }
        }
      };
      block(std::integral_constant<int, 0>{});
      block(std::integral_constant<int, 1>{});
      block(std::integral_constant<int, 2>{});
      block(std::integral_constant<int, 3>{});
    }
  }
  // partial sums into the wave's own area, then the fixed-order sum of output fragment (f, tt)
  // by wave f * T + tt, and the tensor scales
  v4f* red = reinterpret_cast<v4f*>(area);
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int tt = 0; tt < T; ++tt) red[(f * T + tt) * 64 + lane] = acc[f][tt];
  __syncthreads();
  if (wave >= MF * T) return;
  const int qo = wave, f = qo / T, tt = qo % T;
  v4f sum = reinterpret_cast<const v4f*>(lds)[qo * 64 + lane];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) sum += reinterpret_cast<const v4f*>(lds + w * area_bytes)[qo * 64 + lane];
  const float ts = x_ts[0] * w_ts[0];
  // lane holds D[n + 4g + i][m = 16 f + r], i = 0..3: four consecutive features of one token
  store_out<OUT_BF16>(Yv, M, N, 16 * f + (lane & 15), nb + 16 * tt + 4 * (lane >> 4), sum * ts);
}

std::atomic<int> g_nvdec_attr[2][2][4][64];  // per output dtype, T, MF and device: dynamic-LDS limit raised

template <bool OUT_BF16, int T, int MF>
hipError_t launch_nv_decode(const uint8_t* Xq, const uint8_t* Xs, const float* x_ts, const uint8_t* Wq,
                            const uint8_t* Ws, const float* w_ts, int M, int N, int K, void* Y, int dev, hipStream_t st) {
  const int nper = (K / kDecSlice + kDecWaves - 1) / kDecWaves;  // slices per wave
  if (nper > kDecMaxSlices / T) return hipErrorInvalidValue;    // excluded by the fits test and the T choice
  auto kern = gemm_nvfp4_decode<OUT_BF16, T, MF>;
  const bool cached = dev >= 0 && dev < 64;
  if (!cached || !g_nvdec_attr[OUT_BF16][T - 1][MF - 1][dev].load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    if (cached) g_nvdec_attr[OUT_BF16][T - 1][MF - 1][dev].store(1, std::memory_order_release);
  }
  const int tiles = (N + 15) / 16;
  hipLaunchKernelGGL(kern, dim3((unsigned)((tiles + T - 1) / T)), dim3(kDecThreads), kDecWaves * nper * T * 4096, st, Xq,
                     Xs, x_ts, Wq, Ws, w_ts, Y, M, N, K, nper);
  return hipGetLastError();
}

}  // namespace
}  // namespace fp4

// 1..64 tokens, K a multiple of 512 whose slices fit the waves' LDS areas with one tile (K <= 8192)
bool fp4_gemm_nvfp4_decode_fits(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 64 && N >= 1 && K % 512 == 0 && K <= 8192;
}

hipError_t fp4_launch_gemm_nvfp4_decode(const uint8_t* Xq, const uint8_t* Xs, const float* x_ts, const uint8_t* Wq,
                                        const uint8_t* Ws, const float* w_ts, int64_t M, int64_t N, int64_t K, void* Y,
                                        int out_bf16, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = 0;
  e = fp4::device_cus(dev, cus);
  if (e != hipSuccess) return e;
  // two tiles per workgroup (sharing the X fragments) once there are at least three tiles per CU
  // and two tiles' slices fit the waves' areas (K <= 4096)
  const bool two = (N + 15) / 16 >= 3 * (int64_t)cus && K <= 4096;
  const int m = (int)M, n = (int)N, k = (int)K, mf = (m + 15) / 16;
  auto go = [&](auto bf16, auto t, auto f) {
    return fp4::launch_nv_decode<decltype(bf16)::value, decltype(t)::value, decltype(f)::value>(
        Xq, Xs, x_ts, Wq, Ws, w_ts, m, n, k, Y, dev, st);
  };
  auto with_mf = [&](auto bf16, auto t) {
    switch (mf) {
      case 1: return go(bf16, t, std::integral_constant<int, 1>{});
      case 2: return go(bf16, t, std::integral_constant<int, 2>{});
      case 3: return go(bf16, t, std::integral_constant<int, 3>{});
      default: return go(bf16, t, std::integral_constant<int, 4>{});
    }
  };
  auto with_t = [&](auto bf16) {
    return two ? with_mf(bf16, std::integral_constant<int, 2>{}) : with_mf(bf16, std::integral_constant<int, 1>{});
  };
  return out_bf16 ? with_t(std::true_type{}) : with_t(std::false_type{});
}
