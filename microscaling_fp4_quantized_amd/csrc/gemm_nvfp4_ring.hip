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
// tensor scales multiply the result in the epilogue.
//
// Design for CDNA4:
//  * Codes and scales stay 4- and 8-bit in LDS. K advances 256 per stage; a 2-deep ring
//    (144 KB) is filled by LDS DMA (buffer_load_dwordx4 ... lds) as in the MXFP4 kernel:
//    16-byte chunks of a row XOR-swizzled by the row's low five bits so the 32 rows of a
//    fragment read hit distinct banks, the A rows of both stages before the B rows so every
//    fragment read is a per-lane offset plus an immediate, the 16 E4M3 bytes of each row and
//    stage in their own buffer, one barrier per stage, the DMA of stage s+1 issued in four
//    parts across the k-blocks of stage s.
//  * Each wave reads its fragments as 16 bytes (32 codes of one row) per lane and
//    dequantizes them in registers right before the MFMAs: one packed convert per code
//    byte (v_cvt_scalef32_pk_f16_fp4) and one packed multiply by the group scale d, itself
//    converted exactly from E4M3 to an fp16 pair by one v_cvt_scalef32_pk_f16_fp8 per two
//    groups (the lane's two scale bytes of two blocks are gathered into one dword per stage).
//  * K order within a 64-element block: lane half h holds elements 32h .. 32h + 31, and
//    MFMA k-step j takes elements 32h + 8j .. + 7 from lane half h, for both operands. Every
//    product still pairs x_k with w_k, and the block's sum is unchanged up to the order of
//    the float32 additions, which the MFMA does not fix in any case.
//  * 8 waves (2 x 4), 128 x 64 outputs per wave as 4 x 2 fragments of 32 x 32; W is the row
//    operand and X the column operand of every MFMA, so each lane ends with four consecutive
//    output features of one token, staged through LDS for whole-row 16-byte stores of Y.
//  * Workgroup i runs on XCD i % 8; each XCD takes a contiguous range of tiles, walked
//    M-fastest within groups of 8 tile rows. Two tile widths in one launch, as in the MXFP4
//    kernel: when 256x256 tiles would leave the last round part-filled, the columns after
//    whole rounds of them are covered by 256x192 tiles (4 x 2 waves of 64 x 96).
//  * Fewer than 256 rows of X (and N >= 1024): 64-column tiles, 128 x 64 up to 128 rows, 256 x 64
//    above (two 128 x 64 row tiles where the 256-row grid would fill at most half the CUs), so
//    that enough workgroups stream W; rows past M repeat row M-1.
// Requires K % 256 == 0 and K < 2^25 (32-bit buffer offsets); other shapes use the general kernel.
#include <atomic>
#include <type_traits>

#include "common.hpp"

namespace fp4 {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int BM = 256;                  // tile rows (both widths)
constexpr int WAVES = 8, NT = WAVES * 64;
constexpr int BKB = 128;                 // code bytes of a row per stage (256 elements)
constexpr int SCB = 16;                  // E4M3 bytes of a row per stage (16 groups of 16)
constexpr int KBLK = 4;                  // 64-element blocks per stage (one DMA part each)
constexpr int LDS_BYTES = 2 * (BM + 256) * (BKB + SCB);  // the wide tile's 2-deep ring: 144 KB

// One tile shape: BM_ rows, BN columns, WGM x WGN waves, an NS_-deep ring of stages (the DMA of
// stage s + NS - 1 is issued while stage s is multiplied).
template <int BN_, int WGM_, int WGN_, int BM_ = BM, int NS_ = 2>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, NS = NS_;
  static constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  static constexpr int STAGE = (BM + BN) * BKB;                   // codes of one stage
  static constexpr int SC = (BM + BN) * SCB;                      // scales of one stage
  static constexpr int A_WL = BM / 8 / WAVES, B_WL = BN / 8 / WAVES;  // 1 KB code wave-loads per wave
  static constexpr int SC_LOADS = (BM + BN) / 64;                 // 64-row scale wave-loads
  static constexpr int SC_WL = (SC_LOADS + WAVES - 1) / WAVES;
  static constexpr int EP = WN * 4 + 16;                          // epilogue row pitch (bytes)
  static_assert(WGM * WGN == WAVES, "wave layout");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "whole 32x32 fragments");
  static_assert(A_WL * 8 * WAVES == BM && B_WL * 8 * WAVES == BN, "row split");
  static_assert(SC_LOADS * 64 == BM + BN, "scale split");
  static_assert(NS >= 2 && NS * (STAGE + SC) <= LDS_BYTES, "ring fits");
  static_assert(NS == 2 || SC_WL == 1, "at most one scale wave-load per wave (the wait counts assume it)");
  static_assert(WAVES * 32 * EP <= LDS_BYTES, "epilogue staging fits");
};
using Wide = Tile<256, 2, 4>;
using Narrow = Tile<192, 4, 2>;
using Skinny = Tile<64, 8, 1>;  // 129-255 rows: 256 x 64 tiles, 8 waves of 32 x 64
using Skinny128 = Tile<64, 4, 2, 128>;  // 65-128 rows: 128 x 64 tiles, 8 waves of 32 x 32
template <class C>
constexpr int lds_need() {  // the ring and scale buffers, or the epilogue staging if larger
  return C::NS * (C::STAGE + C::SC) > WAVES * 32 * C::EP ? C::NS * (C::STAGE + C::SC) : WAVES * 32 * C::EP;
}
constexpr float kNvNarrowCost = 0.84f;  // measured time of a 256x192 tile over a 256x256 one

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// Barrier of the LDS ring: wait for this wave's LDS reads (lgkmcnt(0)) but not for its
// in-flight DMA loads, then synchronise the workgroup.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Raw buffer resource over [base, base + bytes): stride 0, last word 0x00020000 (32-bit data
// format in the gfx9-family descriptor layout, which untyped loads need). Offsets at or past
// `bytes` read as zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const uint8_t* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, (int)bytes, 0x00020000);
}

// 16-byte chunk q of row r sits at slot q ^ swz(r) of the row. swz depends only on r % 32, so
// every 32-row fragment reads at the same lane offsets; over any 16 consecutive rows it takes each
// value twice, once on even and once on odd rows, so a fragment read hits distinct banks.
__device__ __forceinline__ int swz(int r) { return (r ^ ((r >> 3) & 3)) & 7; }

// Two E4M3 scale bytes (word W of w) -> the exact fp16 pair (d0, d1): every E4M3FN value,
// subnormals included, is an fp16 number, and the gfx950 FP8 convert with a unit scale gives it.
template <bool W>
__device__ __forceinline__ h2 e4m3_pair(unsigned w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, W);
}

// Eight E2M1 codes (one dword, element 2q in the low nibble of byte q) -> eight exact fp16
// e2m1 * d: a packed convert per code byte, then a packed multiply by the group scale (the
// product has at most 6 significant bits and lies in [2^-10, 2688]).
__device__ __forceinline__ v8h dequant8(unsigned codes, h2 dd) {
  v4u o;
  o[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * dd);
  o[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * dd);
  o[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * dd);
  o[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * dd);
  return __builtin_bit_cast(v8h, o);
}

// One output tile [m0, m0 + C::BM) x [n0, n0 + C::BN) over all of K.
template <bool OUT_BF16, class C>
__device__ __forceinline__ void nv_tile(uint8_t* smem, const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ Xs,
                                        const float* __restrict__ x_ts, const uint8_t* __restrict__ Wq,
                                        const uint8_t* __restrict__ Ws, const float* __restrict__ w_ts,
                                        void* __restrict__ Yv, int M, int N, int K, int m0, int n0) {
  constexpr int BM = C::BM;
  constexpr int WGN = C::WGN, WM = C::WM, WN = C::WN, FM = C::FM, FN = C::FN;
  constexpr int STAGE = C::STAGE, SC = C::SC, A_WL = C::A_WL, B_WL = C::B_WL, SC_WL = C::SC_WL;
  constexpr int NS = C::NS, D = NS - 1;  // D: stages fetched ahead
  // LDS: the A rows of the NS stages, then their B rows, then the scale buffers, so that a
  // fragment read is a per-lane offset of the stage plus an immediate.
  constexpr int A_ST = BM * BKB, B_ST = C::BN * BKB, B_BASE = NS * A_ST;
  uint8_t* scl = smem + NS * STAGE;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;
  const int KB = K / 2, KS = K / 16;
  const int nst = K / 256;

  // DMA sources: 8 rows x 128 bytes per code wave-load, 64 rows x 16 bytes per scale wave-load;
  // rows past M / N repeat the last row. Buffer form: a wave-uniform resource at the tile's first
  // row of each operand and a 32-bit per-lane offset (below 256 * K / 2 < 2^32: K < 2^25).
  const int rows_a = min(M - m0, BM), rows_b = min(N - n0, C::BN);
  const __amdgpu_buffer_rsrc_t rsA = buffer_rsrc(Xq + (size_t)m0 * KB, (unsigned)rows_a * KB);
  const __amdgpu_buffer_rsrc_t rsB = buffer_rsrc(Wq + (size_t)n0 * KB, (unsigned)rows_b * KB);
  const __amdgpu_buffer_rsrc_t rsXs = buffer_rsrc(Xs + (size_t)m0 * KS, (unsigned)rows_a * KS);
  const __amdgpu_buffer_rsrc_t rsWs = buffer_rsrc(Ws + (size_t)n0 * KS, (unsigned)rows_b * KS);
  unsigned offA[A_WL], offB[B_WL], offS[SC_WL];
#pragma unroll
  for (int i = 0; i < A_WL; ++i) {
    const int r = (wave * A_WL + i) * 8 + (lane >> 3), q = lane & 7;
    offA[i] = (unsigned)min(r, rows_a - 1) * KB + ((q ^ swz(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < B_WL; ++i) {
    const int r = (wave * B_WL + i) * 8 + (lane >> 3), q = lane & 7;
    offB[i] = (unsigned)min(r, rows_b - 1) * KB + ((q ^ swz(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < SC_WL; ++i) {
    const int rb = min(wave * SC_WL + i, C::SC_LOADS - 1) * 64;  // wave-uniform; waves past the last load skip
    const int r = rb + lane;
    offS[i] = rb < BM ? (unsigned)min(r, rows_a - 1) * KS : (unsigned)min(r - BM, rows_b - 1) * KS;
  }

  // Part p (0..KBLK-1) of the DMA of stage s: code wave-load i goes with part i % KBLK, and the
  // stage's scales (16 bytes per row) with part 0.
  auto issue_part = [&](int s, int p) {
    if (p == 0) {
      uint8_t* dst = scl + ((unsigned)s % NS) * SC;
#pragma unroll
      for (int i = 0; i < SC_WL; ++i)
        if (wave * SC_WL + i < C::SC_LOADS)
          __builtin_amdgcn_raw_ptr_buffer_load_lds((wave * SC_WL + i) * 64 < BM ? rsXs : rsWs,
                                                   (lds_void*)(dst + (wave * SC_WL + i) * 1024), 16,
                                                   offS[i], (unsigned)s * SCB, 0, 0);
    }
    uint8_t* bufa = smem + ((unsigned)s % NS) * A_ST;
    uint8_t* bufb = smem + B_BASE + ((unsigned)s % NS) * B_ST;
#pragma unroll
    for (int i = 0; i < A_WL; ++i)
      if (i % KBLK == p)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_void*)(bufa + (wave * A_WL + i) * 1024), 16,
                                                 offA[i], (unsigned)s * BKB, 0, 0);
#pragma unroll
    for (int i = 0; i < B_WL; ++i)
      if (i % KBLK == p)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_void*)(bufb + (wave * B_WL + i) * 1024), 16,
                                                 offB[i], (unsigned)s * BKB, 0, 0);
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int fr = lane & 31, fh = lane >> 5;
  // per-lane offsets of the lane's row in stage 0 (A: row wm0 + fr, B: row wn0 + fr) and of its
  // chunk 2 kb + h of block kb; the stage adds A_ST / B_ST, fragment i / j an immediate i * 4 KB
  const int ra = (wm0 + fr) * BKB, rb = B_BASE + (wn0 + fr) * BKB;
  int cx[KBLK];
#pragma unroll
  for (int kb = 0; kb < KBLK; ++kb) cx[kb] = ((2 * kb + fh) ^ swz(fr)) << 4;
  const unsigned psel = fh ? 0x07060302u : 0x05040100u;  // bytes 2h, 2h + 1 of two dwords

  // Stage s: wait for its DMA (this wave's, then everyone's at the barrier), then multiply it
  // while the parts of stage s+D refill the buffers of stage s-1, which every wave has finished
  // reading once past the barrier. The last D stages are peeled off so that the loop body issues
  // its DMA unconditionally. At the top of a stage s with s + D < nst this wave may still have the
  // loads of stages s+1 .. s+D-1 in flight: A_WL + B_WL each, plus its scale load if it has one.
  constexpr int LW = A_WL + B_WL;
  const bool has_sc = wave < C::SC_LOADS;
  auto run_stage = [&](int s, auto with_dma) {
    if constexpr (!decltype(with_dma)::value || D == 1) wait_vmcnt<0>();
    else if (has_sc) wait_vmcnt<(D - 1) * (LW + 1)>();
    else wait_vmcnt<(D - 1) * LW>();
    ring_barrier();
    const int la = ra + ((unsigned)s % NS) * A_ST, lb = rb + ((unsigned)s % NS) * B_ST;
    const uint8_t* sbuf = scl + ((unsigned)s % NS) * SC;
    // the lane's scale bytes of the stage: of each block's four (one dword), the two of its lane
    // half, gathered as word kb % 2 of dword kb / 2
    unsigned sg_a[FM][2], sg_b[FN][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const v4u t = *reinterpret_cast<const v4u*>(sbuf + (wm0 + i * 32 + fr) * SCB);
      sg_a[i][0] = __builtin_amdgcn_perm(t[1], t[0], psel);
      sg_a[i][1] = __builtin_amdgcn_perm(t[3], t[2], psel);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const v4u t = *reinterpret_cast<const v4u*>(sbuf + (BM + wn0 + j * 32 + fr) * SCB);
      sg_b[j][0] = __builtin_amdgcn_perm(t[1], t[0], psel);
      sg_b[j][1] = __builtin_amdgcn_perm(t[3], t[2], psel);
    }
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb) {
      if constexpr (decltype(with_dma)::value) issue_part(s + D, kb);
      // 16-byte chunk 2 kb + h of the row: elements 32h .. 32h + 31 of block kb
      v4u ca[FM], cb[FN];
      const int oa = la + cx[kb], ob = lb + cx[kb];
#pragma unroll
      for (int i = 0; i < FM; ++i) ca[i] = *reinterpret_cast<const v4u*>(smem + oa + i * 32 * BKB);
#pragma unroll
      for (int j = 0; j < FN; ++j) cb[j] = *reinterpret_cast<const v4u*>(smem + ob + j * 32 * BKB);
      // group scales of the lane's two 16-element groups of block kb (groups 4 kb + 2h and + 1)
      h2 da[FM], db[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) da[i] = (kb & 1) ? e4m3_pair<true>(sg_a[i][kb / 2]) : e4m3_pair<false>(sg_a[i][kb / 2]);
#pragma unroll
      for (int j = 0; j < FN; ++j) db[j] = (kb & 1) ? e4m3_pair<true>(sg_b[j][kb / 2]) : e4m3_pair<false>(sg_b[j][kb / 2]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {  // k-step t: dword t of the chunk (elements 32h + 8t .. + 7)
        v8h a[FM], b[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          a[i] = dequant8(ca[i][t], t < 2 ? __builtin_shufflevector(da[i], da[i], 0, 0)
                                          : __builtin_shufflevector(da[i], da[i], 1, 1));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          b[j] = dequant8(cb[j][t], t < 2 ? __builtin_shufflevector(db[j], db[j], 0, 0)
                                          : __builtin_shufflevector(db[j], db[j], 1, 1));
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[j], a[i], acc[i][j], 0, 0, 0);  // D[n][m]
      }
    }
  };
  if constexpr (D == 1) {
#pragma unroll
    for (int p = 0; p < KBLK; ++p) issue_part(0, p);
    for (int s = 0; s + 1 < nst; ++s) run_stage(s, std::true_type{});
    run_stage(nst - 1, std::false_type{});
  } else {
    for (int t = 0; t < D && t < nst; ++t)
#pragma unroll
      for (int p = 0; p < KBLK; ++p) issue_part(t, p);
    int s = 0;
    for (; s + D < nst; ++s) run_stage(s, std::true_type{});
    for (; s < nst; ++s) run_stage(s, std::false_type{});
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

// One C::BM x 64 tile per workgroup, tile index b -> (tm, tn) M-fastest; for fewer than 256 rows of X.
template <bool OUT_BF16, class C>
__global__ __launch_bounds__(NT) void gemm_nvfp4_ring_skinny(const uint8_t* __restrict__ Xq,
                                                             const uint8_t* __restrict__ Xs,
                                                             const float* __restrict__ x_ts,
                                                             const uint8_t* __restrict__ Wq,
                                                             const uint8_t* __restrict__ Ws,
                                                             const float* __restrict__ w_ts, void* __restrict__ Yv,
                                                             int M, int N, int K, int tiles_m) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int b = blockIdx.x, tm = b % tiles_m, tn = b / tiles_m;
  nv_tile<OUT_BF16, C>(smem, Xq, Xs, x_ts, Wq, Ws, w_ts, Yv, M, N, K, tm * C::BM, tn * C::BN);
}

template <bool B>
std::atomic<int> g_skinny_attr[2][64];

template <bool B, class C>
hipError_t launch_skinny(const uint8_t* Xq, const uint8_t* Xs, const float* x_ts, const uint8_t* Wq, const uint8_t* Ws,
                         const float* w_ts, int M, int N, int K, void* Y, int dev, int slot, hipStream_t st) {
  auto sk = gemm_nvfp4_ring_skinny<B, C>;
  const bool cached = dev >= 0 && dev < 64;
  if (!cached || !g_skinny_attr<B>[slot][dev].load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute((const void*)sk, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    if (cached) g_skinny_attr<B>[slot][dev].store(1, std::memory_order_release);
  }
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
  hipLaunchKernelGGL(sk, dim3(tiles_m * tiles_n), dim3(NT), lds_need<C>(), st, Xq, Xs, x_ts, Wq, Ws, w_ts, Y, M, N, K,
                     tiles_m);
  return hipGetLastError();
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
  // Above 128 rows, two 128-row tiles per 64 columns where one 256-row tile per 64 columns would
  // fill at most half the CUs: at 129-255 rows and N = 4096 (K = 4096) 25 against 35 us, while at
  // N = 14336 the 256-row tiles win (36-38 against 44-50 us).
  if (M <= 128 || (M < BM && 2 * ((N + 63) / 64) <= cus))
    return launch_skinny<B, Skinny128>(Xq, Xs, x_ts, Wq, Ws, w_ts, M, N, K, Y, dev, 1, st);
  if (M < BM) return launch_skinny<B, Skinny>(Xq, Xs, x_ts, Wq, Ws, w_ts, M, N, K, Y, dev, 0, st);
  int tn1, tn2;
  fp4_plan_tile_columns(tiles_m, N, cus, kNvNarrowCost, tn1, tn2);
  hipLaunchKernelGGL(kern, dim3(tiles_m * (tn1 + tn2)), dim3(NT), LDS_BYTES, st, Xq, Xs, x_ts, Wq, Ws, w_ts, Y, M, N,
                     K, tiles_m, tn1, tn2);
  return hipGetLastError();
}

}  // namespace
}  // namespace fp4

bool fp4_gemm_nvfp4_ring_fits(int64_t M, int64_t N, int64_t K) {
  return K % 256 == 0 && K < ((int64_t)1 << 25) && ((M >= 256 && N >= 256) || (M > 64 && N >= 1024));
}

hipError_t fp4_launch_gemm_nvfp4_ring(const uint8_t* Xq, const uint8_t* Xs, const float* x_ts, const uint8_t* Wq,
                                      const uint8_t* Ws, const float* w_ts, int64_t M, int64_t N, int64_t K, void* Y,
                                      int out_bf16, hipStream_t st) {
  return out_bf16 ? fp4::launch<true>(Xq, Xs, x_ts, Wq, Ws, w_ts, (int)M, (int)N, (int)K, Y, st)
                  : fp4::launch<false>(Xq, Xs, x_ts, Wq, Ws, w_ts, (int)M, (int)N, (int)K, Y, st);
}
