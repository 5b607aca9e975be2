// Online block-Hadamard rotation fused with MXFP4 / NVFP4 quantization (gfx950).
//
// Method: "Bridging the Gap Between Promise and Performance for Microscaling FP4
// Quantization" (gist.science, German edition), Technische Zusammenfassung §2
// "Einführung von MR-GPTQ" item 1 (block-wise Hadamard rotations of weights and
// activations) and §2 "GPU-Kernel-Unterstützung (QuTLASS)" (the activation
// rotation is fused into a lightweight quantization kernel computed online).
// Scale rule: "Unveiling the Potential of Quantization with MXFP4" (gist.science,
// Dutch edition), Methodologie, 1. Overflow-Aware Scaling: standard MXFP4 maps
// the block maximum into (3, 6].
//
// Work decomposition: one lane owns one 32-element chunk of a row (64 bytes of
// bf16 in, 16 bytes of packed codes out). A wave reads its 4 KB of X with fully
// coalesced 16-byte loads and redistributes them through LDS, so each lane owns a
// contiguous chunk (per-lane 64-byte strided loads reached only ~55% of HBM peak).
// A Hadamard block of b <= 32 lives in one lane's registers; b = 64 / 128 spans
// 2 / 4 adjacent lanes of a quad and its last stages exchange values with DPP quad
// permutes. The transform follows one fixed order (strides 1, 2, 4, ... then one
// multiply by fl32(1/sqrt(b))) so its float32 result is unique. The path is
// HBM-bound: MXFP4 reads X once, NVFP4 twice (the tensor maximum first), and every
// code and scale byte is written once.
#include "quant_device.hpp"

namespace fp4 {
namespace {

constexpr int kThreads = 256;

struct RowMap {
  // chunk -> (row, chunk-in-row) via multiply-high division by chunks_per_row
  uint32_t cpr;    // chunks (32 elements) per row
  uint32_t magic;  // see make_rowmap
  uint32_t shift;
  uint32_t pow2;   // cpr is a power of two: shift only
};

__device__ __forceinline__ uint32_t row_of(uint32_t gc, const RowMap& rm) {
  if (rm.pow2) return gc >> rm.shift;
  uint32_t t = __umulhi(gc, rm.magic);
  return (t + ((gc - t) >> 1)) >> (rm.shift - 1);
}

// Per-wave LDS staging area: 64 lanes x 64 bytes, padded so that both the coalesced
// writes and the per-lane reads below are free of bank conflicts.
constexpr int kStage = 4 * 68;  // 16-byte slots per wave

template <bool CONTIG>
__device__ __forceinline__ const uint16_t* chunk_ptr(const uint16_t* __restrict__ X, int64_t ldx, uint32_t gc,
                                                     const RowMap& rm) {
  if constexpr (CONTIG) return X + (size_t)gc * 32;
  const uint32_t row = row_of(gc, rm);
  return X + (size_t)row * (size_t)ldx + (size_t)(gc - row * rm.cpr) * 32;
}

// The wave's four coalesced 16-byte loads: instruction j covers 1 KB, part (lane % 4) of chunk
// wbase + 16 j + lane / 4. Past the end the chunk index is clamped to the last chunk, so every
// address stays inside X and all four loads are in flight before the first LDS write.
template <bool CONTIG, bool NT>
__device__ __forceinline__ void load_wave(const uint16_t* __restrict__ X, int64_t ldx, uint32_t wbase, uint32_t total,
                                          const RowMap& rm, v4u r[4]) {
  const uint32_t lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t owner = min(wbase + 16 * j + (lane >> 2), total - 1);
    const v4u* p = reinterpret_cast<const v4u*>(chunk_ptr<CONTIG>(X, ldx, owner, rm)) + (lane & 3);
    r[j] = NT ? __builtin_nontemporal_load(p) : *p;
  }
}

// Load the lane's 32 bf16 values and widen them to float32 (exact). The wave reads its 64
// chunks with fully coalesced loads and transposes them through LDS, so that each lane ends up
// with its own 64 contiguous bytes. Every lane of the wave must call this (lanes whose chunk
// is past the end still load for the others); stage is the wave's LDS area. `mode` bit 0: rows
// are contiguous (ldx == K); bit 1: streaming (nontemporal) loads, used for inputs too large to
// stay in the caches; smaller inputs (often just written by the previous kernel) load normally.
__device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ X, int64_t ldx, uint32_t gc, uint32_t total,
                                           const RowMap& rm, int mode, v4u* stage, float v[32]) {
  const uint32_t lane = threadIdx.x & 63, wbase = gc - lane;
  v4u r[4];
  switch (mode & 3) {
    case 0: load_wave<false, false>(X, ldx, wbase, total, rm, r); break;
    case 1: load_wave<true, false>(X, ldx, wbase, total, rm, r); break;
    case 2: load_wave<false, true>(X, ldx, wbase, total, rm, r); break;
    default: load_wave<true, true>(X, ldx, wbase, total, rm, r); break;
  }
  asm volatile("" ::: "memory");  // earlier reads of the area (a previous chunk) stay before these writes
#pragma unroll
  for (int j = 0; j < 4; ++j) stage[(16 * j + (lane >> 2)) + (lane & 3) * 68] = r[j];
  // The area is private to the wave: waiting for its own LDS writes (lgkmcnt(0)) is enough,
  // and the empty asm keeps the compiler from moving the reads above the writes.
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const v4u w = stage[lane + j * 68];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[8 * j + 2 * t] = bf16_lo(w[t]);
      v[8 * j + 2 * t + 1] = bf16_hi(w[t]);
    }
  }
}

// Randomized block Hadamard: flip channel k when signs[k] < 0, before the rotation. The
// lane's 32 channels start at 32 * (chunk index within its row).
__device__ __forceinline__ void apply_signs(float v[32], const int8_t* __restrict__ signs, uint32_t gc,
                                            const RowMap& rm) {
  const uint32_t cc = gc - row_of(gc, rm) * rm.cpr;
  const v4u* p = reinterpret_cast<const v4u*>(signs + (size_t)cc * 32);
  const v4u s0 = p[0], s1 = p[1];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const unsigned w = i < 16 ? s0[i >> 2] : s1[(i - 16) >> 2];
    const unsigned neg = (w >> (8 * (i & 3) + 7)) & 1u;
    v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (neg << 31));
  }
}

// ---------------------------------------------------------------------------
// MXFP4: one kernel. E8M0 code = max(0, biased_exp(alpha) - 2 + [mantissa > 0.5]),
// i.e. e = ceil(log2(alpha / 6)) clamped to [-127, 127] (alpha = 0 -> code 0).
// ---------------------------------------------------------------------------
template <int B, int RULE>
__global__ __launch_bounds__(kThreads) void rotate_quant_mx(const uint16_t* __restrict__ X, int64_t ldx,
                                                            RowMap rm, uint32_t total, int load_mode,
                                                            const int8_t* __restrict__ signs,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  __shared__ __attribute__((aligned(16))) v4u stage[kThreads / 64][kStage];
  const uint32_t gc = blockIdx.x * kThreads + threadIdx.x;
  float v[32];
  load_chunk(X, ldx, gc, total, rm, load_mode, stage[threadIdx.x >> 6], v);
  if (gc >= total) return;  // whole quads leave together (total % (B/32) == 0)
  if (signs) apply_signs(v, signs, gc, rm);
  v4u out;
  const int code = mx_rotate_quantize_chunk<B, RULE>(v, out);
  __builtin_nontemporal_store(out, reinterpret_cast<v4u*>(codes) + gc);
  scales[gc] = (uint8_t)code;
}

// ---------------------------------------------------------------------------
// NVFP4 pass 1: the tensor scale s_t = fl32(T / 2688), T = max |y| over the tensor.
// Each workgroup of the max pass writes the maximum of its chunks to its own float slot,
// then one workgroup reduces the slots and writes s_t. No atomics: when every workgroup
// finishes at once, same-address atomics serialise in L2. x -> fl32(x c) and
// x -> fl32(x / 2688) are monotone, so max fl32(|z| c) = fl32(max|z| c) (the multiply is
// applied once per chunk) and fl32(max / 2688) = fl32(T / 2688).
// ---------------------------------------------------------------------------
constexpr unsigned kMaxPassGrid = 1024;  // 4 workgroups per CU on the 256-CU gfx950, grid-stride

__global__ __launch_bounds__(kThreads) void amax_finish(const float* __restrict__ partial, int n,
                                                        float* __restrict__ ts) {
  static_assert(kMaxPassGrid % kThreads == 0, "whole loads per thread");
  // n <= kMaxPassGrid: every thread issues its (at most four) loads before using any of them
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < (int)(kMaxPassGrid / kThreads); ++j) {
    const int i = (int)threadIdx.x + j * kThreads;
    m = fmaxf(m, partial[i < n ? i : n - 1]);  // n >= 1; a repeated slot leaves the maximum unchanged
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float wmax[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = wmax[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) b = fmaxf(b, wmax[w]);
    ts[0] = (float)((double)b / 2688.0);  // fl32(T / 2688): 2688 = 2^7 * 21, so the fp64 step never
                                          // lands on a float32 rounding midpoint
  }
}

template <int B>
__global__ __launch_bounds__(kThreads) void rotate_amax(const uint16_t* __restrict__ X, int64_t ldx,
                                                        RowMap rm, uint32_t total, int load_mode,
                                                        const int8_t* __restrict__ signs,
                                                        float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) v4u stage[kThreads / 64][kStage];
  // Grid-stride over the chunks (the grid is capped at a few workgroups per CU), so each
  // workgroup pays the reduction and the atomic below once for many chunks.
  float m = 0.f;
  const float c = __uint_as_float(hadamard_constant_bits(B));
  for (uint32_t base = blockIdx.x * kThreads; base < total; base += gridDim.x * kThreads) {
    const uint32_t gc = base + threadIdx.x;
    float v[32];
    load_chunk(X, ldx, gc, total, rm, load_mode, stage[threadIdx.x >> 6], v);
    if (gc < total) {
      if (signs) apply_signs(v, signs, gc, rm);
      m = fmaxf(m, fwht_absmax<B>(v) * c);
    }
  }
  // wave reduction, then workgroup reduction through LDS; one float per workgroup
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float wmax[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = wmax[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) b = fmaxf(b, wmax[w]);
    partial[blockIdx.x] = b;
  }
}

// E4M3 group code of a group maximum a >= 0: the E4M3FN value nearest to a / den (ties to even,
// saturating at 448), den = 6 s_t. First from q = fl32(a * rD), rD within 1 ulp of
// 1 / fl32(6 s_t), so that q lies within 4 ulp of a / den: its rounding at the E4M3 mantissa
// point (or, below 2^-6, at multiples of 2^-9) is the exact decision unless q lies within 8 ulp
// of a rounding midpoint; those rare groups, and every group when rD is +inf (6 s_t < 2^-125),
// are decided exactly in float64.
__device__ __forceinline__ unsigned e4m3_code(float a, float rD, double den) {
  const float q = a * rD;
  const unsigned b = __float_as_uint(q);
  // normal E4M3 range (q >= 2^-6): round the float32 mantissa at bit 20, carry into the exponent
  const unsigned rn = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;
  const unsigned cn = min(rn - ((127u - 7u) << 3), 0x7Eu);
  const bool near_n = (b & 0xFFFFFu) - 0x7FFF8u < 16u;  // within 8 ulp of the midpoint
  // subnormal E4M3 range: k * 2^-9, k = 0..8
  const float k = fminf(q, 1.0f) * 512.0f;  // only read below 2^-6
  const float kr = __builtin_rintf(k);
  const bool near_s = fabsf(fabsf(k - kr) - 0.5f) < 1.52587890625e-05f;  // 2^-16
  const bool normal = q >= 0.015625f;
  unsigned code = normal ? cn : (unsigned)kr;
  const bool near = (normal ? near_n : near_s) || !(rD < __builtin_inff());
  if (near) code = e4m3_rne_sat((double)a / den);
  return code;
}

// NVFP4 pass 2: group scales and codes given T.
// One group of 16 under E4M3 code `code`: S = fl32(d * s_t), u = fl32(y * fl32(1/S)), codes
// rounded by the hardware convert (scale 1); S < 2^-126 stores signed zeros.
__device__ __forceinline__ void nv_group(const float* y, unsigned code, float s_t, unsigned* o, float* S_out) {
  const float S = e4m3_value(code) * s_t;
  *S_out = S;
  if (S < 1.17549435e-38f) {  // 2^-126: the group stores signed zeros
    o[0] = sign_codes8(y);
    o[1] = sign_codes8(y + 8);
    *S_out = 0.f;
    return;
  }
  const float R = 1.0f / S;  // correctly rounded float32 division: fl32(1 / S)
  float u[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] = y[i] * R;
  o[0] = cvt8(u, 1.0f);
  o[1] = cvt8(u + 8, 1.0f);
}

template <int B, int RULE>
__global__ __launch_bounds__(kThreads) void rotate_quant_nv(const uint16_t* __restrict__ X, int64_t ldx,
                                                            RowMap rm, uint32_t total, int load_mode,
                                                            const int8_t* __restrict__ signs,
                                                            const unsigned* __restrict__ amax_bits,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  __shared__ __attribute__((aligned(16))) v4u stage[kThreads / 64][kStage];
  // mode bit 2: workgroups take the chunks in reverse order (see launch_b)
  const uint32_t blk = (load_mode & 4) ? gridDim.x - 1 - blockIdx.x : blockIdx.x;
  const uint32_t gc = blk * kThreads + threadIdx.x;
  float v[32];
  load_chunk(X, ldx, gc, total, rm, load_mode, stage[threadIdx.x >> 6], v);
  if (gc >= total) return;
  if (signs) apply_signs(v, signs, gc, rm);
  fwht<B>(v);
  const float c = __uint_as_float(hadamard_constant_bits(B));
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] *= c;
  const float s_t = __uint_as_float(*amax_bits);  // = fl32(T / 2688) left by pass 1, or given by the caller
  v4u out;
  unsigned sc2 = 0;
  if (s_t == 0.f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = sign_codes8(v + 8 * j);
  } else {
    const double den = 6.0 * (double)s_t;  // exact
    // about 1 / den within 2 ulp; groups are decided exactly in float64 when 6 s_t is tiny
    const float d32 = 6.0f * s_t;
    const float rD = d32 >= 0x1p-125f ? __builtin_amdgcn_rcpf(d32) : __builtin_inff();
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float* y = v + 16 * g;
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(y[i]));
      unsigned code = e4m3_code(a, rD, den);
      unsigned o[2];
      float S;
      nv_group(y, code, s_t, o, &S);
      if constexpr (RULE == kRuleFit) {
        // data-free search over the neighbouring E4M3 codes (smaller first), tensor scale fixed
        float best = group_sse<16>(y, o, S);
        const int base = (int)code;
#pragma unroll
        for (int step = -1; step <= 1; step += 2) {
          const int cand = base + step;
          if (cand < 0 || cand > 0x7E) continue;
          unsigned oc[2];
          float Sc;
          nv_group(y, (unsigned)cand, s_t, oc, &Sc);
          const float e = group_sse<16>(y, oc, Sc);
          if (e < best) {
            best = e;
            code = (unsigned)cand;
            o[0] = oc[0];
            o[1] = oc[1];
          }
        }
      }
      sc2 |= code << (8 * g);
      out[2 * g] = o[0];
      out[2 * g + 1] = o[1];
    }
  }
  __builtin_nontemporal_store(out, reinterpret_cast<v4u*>(codes) + gc);
  reinterpret_cast<uint16_t*>(scales)[gc] = (uint16_t)sc2;
}

RowMap make_rowmap(uint32_t cpr) {
  RowMap rm{cpr, 0, 0, 0};
  if ((cpr & (cpr - 1)) == 0) {
    rm.pow2 = 1;
    while ((1u << rm.shift) < cpr) ++rm.shift;
    return rm;
  }
  uint32_t l = 0;
  while ((1ull << l) < cpr) ++l;  // l = ceil(log2 cpr) >= 2
  rm.magic = (uint32_t)((((1ull << l) - cpr) << 32) / cpr + 1);
  rm.shift = l;
  return rm;
}

template <int B, int RULE>
hipError_t launch_b(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, int fmt, bool given_ts,
                    const int8_t* signs, uint8_t* codes, uint8_t* scales, float* ts, hipStream_t st) {
  const uint32_t cpr = (uint32_t)(K / 32);
  const uint32_t total = (uint32_t)(M * (K / 32));
  const RowMap rm = make_rowmap(cpr);
  // load mode: bit 0 contiguous rows; bit 1 streaming loads for inputs beyond 64 MiB (they would
  // not stay in the 256 MB Infinity Cache next to their outputs anyway)
  const int64_t x_bytes = M * ldx * 2;
  const int load_mode = (ldx == K ? 1 : 0) | (x_bytes > (64ll << 20) ? 2 : 0);
  const dim3 grid((total + kThreads - 1) / kThreads), block(kThreads);
  if (fmt == 0) {
    hipLaunchKernelGGL((rotate_quant_mx<B, RULE>), grid, block, 0, st, X, ldx, rm, total, load_mode, signs, codes,
                       scales);
    return hipGetLastError();
  }
  constexpr int NV_RULE = RULE == kRuleFit ? kRuleFit : kRuleStandard;  // other rules are MXFP4 only
  unsigned* amax = reinterpret_cast<unsigned*>(ts);
  // With the tensor maximum computed here, X is read twice. Both passes then use cached loads and
  // the quantize pass walks X backwards: it starts on the chunks the max pass read last, which
  // are still in the 256 MB Infinity Cache when X is not much larger than that.
  const int nv_mode = given_ts ? load_mode : (load_mode & 1) | 4;
  if (!given_ts) {  // otherwise the caller's s_t is already in the word
    const dim3 grid_max(grid.x < kMaxPassGrid ? grid.x : kMaxPassGrid);
    // The per-workgroup maxima live in the codes buffer until the quantize pass overwrites it:
    // 4 bytes per workgroup against 16 bytes of codes per chunk, and grid_max <= chunks.
    float* partial = reinterpret_cast<float*>(codes);
    hipLaunchKernelGGL(rotate_amax<B>, grid_max, block, 0, st, X, ldx, rm, total, load_mode & 1, signs, partial);
    hipLaunchKernelGGL(amax_finish, dim3(1), block, 0, st, partial, (int)grid_max.x, ts);
  }
  hipLaunchKernelGGL((rotate_quant_nv<B, NV_RULE>), grid, block, 0, st, X, ldx, rm, total, nv_mode, signs, amax,
                     codes, scales);
  return hipGetLastError();
}

template <int RULE>
hipError_t launch_rule(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, int block, int fmt, bool given_ts,
                       const int8_t* signs, uint8_t* codes, uint8_t* scales, float* ts, hipStream_t st) {
  switch (block) {
    case 16: return launch_b<16, RULE>(X, M, K, ldx, fmt, given_ts, signs, codes, scales, ts, st);
    case 32: return launch_b<32, RULE>(X, M, K, ldx, fmt, given_ts, signs, codes, scales, ts, st);
    case 64: return launch_b<64, RULE>(X, M, K, ldx, fmt, given_ts, signs, codes, scales, ts, st);
    default: return launch_b<128, RULE>(X, M, K, ldx, fmt, given_ts, signs, codes, scales, ts, st);
  }
}

}  // namespace
}  // namespace fp4

hipError_t fp4_launch_rotate_quantize(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, int block,
                                      int fmt, int rule, bool given_ts, const int8_t* signs, uint8_t* codes,
                                      uint8_t* scales, float* ts, hipStream_t st) {
  switch (rule) {
    case fp4::kRuleOcpFloor:
      return fp4::launch_rule<fp4::kRuleOcpFloor>(X, M, K, ldx, block, fmt, given_ts, signs, codes, scales, ts, st);
    case fp4::kRuleOas:
      return fp4::launch_rule<fp4::kRuleOas>(X, M, K, ldx, block, fmt, given_ts, signs, codes, scales, ts, st);
    case fp4::kRuleFit:
      return fp4::launch_rule<fp4::kRuleFit>(X, M, K, ldx, block, fmt, given_ts, signs, codes, scales, ts, st);
    default:
      return fp4::launch_rule<fp4::kRuleStandard>(X, M, K, ldx, block, fmt, given_ts, signs, codes, scales, ts, st);
  }
}
