// Device helpers of the rotate+quantize step, shared by the stand-alone quantizer and the
// fused decode kernel so that both produce the same bits.
//
// "Bridging the Gap Between Promise and Performance for Microscaling FP4 Quantization"
// (gist.science, German edition), Technische Zusammenfassung §2 "Einführung von MR-GPTQ"
// item 1 (block-wise Hadamard rotation) and item 2 (scale fitting); scale rule: "Unveiling
// the Potential of Quantization with MXFP4" (gist.science, Dutch edition), Methodologie,
// 1. Overflow-Aware Scaling (standard MXFP4 maps the block maximum into (3, 6]).
#pragma once

#include "common.hpp"

namespace fp4 {

// Fast Walsh-Hadamard transform of the Hadamard block, unnormalised.
template <int B>
__device__ __forceinline__ void fwht(float v[32]) {
  constexpr int IN_LANE = B < 32 ? B : 32;
#pragma unroll
  for (int h = 1; h < IN_LANE; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & h)) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  // stride 32 (lane ^ 1) and 64 (lane ^ 2): the lower lane keeps x + partner,
  // the upper lane partner - x (its own value with the sign bit flipped).
  if constexpr (B >= 64) {
    const unsigned flip = (threadIdx.x & 1) ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = quad_xor<1>(v[i]) + __uint_as_float(__float_as_uint(v[i]) ^ flip);
  }
  if constexpr (B >= 128) {
    const unsigned flip = (threadIdx.x & 2) ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = quad_xor<2>(v[i]) + __uint_as_float(__float_as_uint(v[i]) ^ flip);
  }
}

// max_i |y_i| over this lane's 32 outputs of fwht<B> (before the 1/sqrt(B) factor), exactly,
// with the last butterfly stage folded into the maximum: for the two outputs of a pair,
// max(|fl(a + b)|, |fl(a - b)|) = fl(|a| + |b|), since {|a + b|, |a - b|} = {|a| + |b|,
// ||a| - |b||} and rounding to nearest is monotonic and symmetric in sign. Only the magnitudes
// are kept, so the cross-lane last stage (B >= 64) needs no per-lane sign flip. `v` is
// overwritten.
template <int B>
__device__ __forceinline__ float fwht_absmax(float v[32]) {
  constexpr int IN_LANE = B < 32 ? B : 32;
  // every in-lane stage but the last when B <= 32 (that one is folded below)
  constexpr int IN_LANE_FULL = B <= 32 ? IN_LANE / 2 : IN_LANE;
#pragma unroll
  for (int h = 1; h < IN_LANE_FULL; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & h)) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  float m = 0.f;
  if constexpr (B <= 32) {
    constexpr int h = IN_LANE / 2;  // the last stage, in lane
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (!(i & h)) m = fmaxf(m, fabsf(v[i]) + fabsf(v[i + h]));
  } else if constexpr (B == 64) {
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(quad_xor<1>(v[i])) + fabsf(v[i]));
  } else {
    const unsigned flip = (threadIdx.x & 1) ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = quad_xor<1>(v[i]) + __uint_as_float(__float_as_uint(v[i]) ^ flip);
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(quad_xor<2>(v[i])) + fabsf(v[i]));
  }
  return m;
}

// Eight float32 values -> one dword of eight E2M1 codes (element 2j in the low
// nibble of byte j), dividing by 2^(exponent field of `scale` - 127) exactly and
// rounding to nearest, ties to even, saturating at 6, keeping the sign.
__device__ __forceinline__ unsigned cvt8(const float* v, float scale) {
  unsigned w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], scale, 3);
  return w;
}

__device__ __forceinline__ unsigned sign_codes8(const float* v) {
  unsigned w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= ((__float_as_uint(v[i]) >> 31) << 3) << (4 * i);
  return w;
}

// Scale rules of the quantizer (the standard one and its variants; see include/fp4.h).
enum { kRuleStandard = 0, kRuleOcpFloor = 1, kRuleOas = 2, kRuleFit = 3 };

// E8M0 code of a group maximum `ab` (float bits, non-negative) under the standard rule:
// e = ceil(log2(alpha / 6)) clamped to [-127, 127], code e + 127.
__device__ __forceinline__ int mx_code_standard(unsigned ab) {
  const int code = (int)(ab >> 23) - 2 + ((ab & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  return code < 0 ? 0 : code;
}

template <int RULE>
__device__ __forceinline__ int mx_code(unsigned ab) {
  if constexpr (RULE == kRuleOcpFloor) {
    // e = floor(log2 alpha) - 2: the group maximum lands in [4, 8) and saturates above 6
    const int code = (int)(ab >> 23) - 2;
    return code < 0 ? 0 : code;
  } else if constexpr (RULE == kRuleOas) {
    // overflow-aware: when alpha / 2^e is in (3, 3.5] (mantissa in (0.5, 0.75] with the exponent
    // rounded up) use e - 1, so the maximum lands in (6, 7] and saturates to 6
    const int code = mx_code_standard(ab);
    const unsigned m = ab & 0x7FFFFFu;
    return (code > 0 && m > 0x400000u && m <= 0x600000u) ? code - 1 : code;
  } else {
    return mx_code_standard(ab);
  }
}

// 2^(code - 127) as a float32 (code 0 gives the subnormal 2^-127).
__device__ __forceinline__ float pow2_of_code(int code) {
  return code > 0 ? __uint_as_float((unsigned)code << 23) : __uint_as_float(0x00400000u);
}

// E2M1 values of eight codes in one dword (element 2j in the low nibble of byte j).
__device__ __forceinline__ void e2m1_values8(unsigned w, float* q) {
  const v2f f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const v2f f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const v2f f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const v2f f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  q[0] = f0[0]; q[1] = f0[1]; q[2] = f1[0]; q[3] = f1[1];
  q[4] = f2[0]; q[5] = f2[1]; q[6] = f3[0]; q[7] = f3[1];
}

// Squared error of n elements in float32, accumulated in element order: d = fl32(y - q * s),
// acc = fl32(acc + fl32(d * d)), with q * s exact (MX) or rounded once (NV).
template <int NE>
__device__ __forceinline__ float group_sse(const float* y, const unsigned* words, float s) {
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < NE / 8; ++w) {
    float q[8];
    e2m1_values8(words[w], q);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float d = y[8 * w + i] - q[i] * s;
      acc = acc + d * d;
    }
  }
  return acc;
}

// Rotate one 32-element chunk (v, float32, widened from bf16) by the Hadamard block B and
// quantize it to MXFP4 under the scale rule: returns the E8M0 code, writes the four code
// dwords. For B >= 64 the 2 / 4 chunks of a block must sit in adjacent lanes of one quad
// (lane & 1, lane & 2 give their position) and all of them must take part.
template <int B, int RULE>
__device__ __forceinline__ int mx_rotate_quantize_chunk(float v[32], v4u& out) {
  fwht<B>(v);
  const float c = __uint_as_float(hadamard_constant_bits(B));
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] *= c;
    amax = fmaxf(amax, fabsf(v[i]));
  }
  int code = mx_code<RULE>(__float_as_uint(amax));
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = cvt8(v + 8 * j, __uint_as_float((unsigned)code << 23));
  if constexpr (RULE == kRuleFit) {
    // data-free scale fitting: try the neighbouring exponents (smaller first), keep a strictly
    // smaller float32 squared error
    unsigned ow[4] = {out[0], out[1], out[2], out[3]};
    float best = group_sse<32>(v, ow, pow2_of_code(code));
    const int base = code;
#pragma unroll
    for (int step = -1; step <= 1; step += 2) {
      const int cand = base + step;
      if (cand < 0 || cand > 254) continue;
      unsigned o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = cvt8(v + 8 * j, __uint_as_float((unsigned)cand << 23));
      const float e = group_sse<32>(v, o, pow2_of_code(cand));
      if (e < best) {
        best = e;
        code = cand;
        out = v4u{o[0], o[1], o[2], o[3]};
      }
    }
  }
  return code;
}

}  // namespace fp4
