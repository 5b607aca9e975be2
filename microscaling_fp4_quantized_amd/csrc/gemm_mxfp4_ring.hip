// Large-tile W4A4 MXFP4 GEMM for gfx950: Y = dq(Xq) dq(Wq)^T with 256-row workgroup tiles.
//
// "Bridging the Gap Between Promise and Performance for Microscaling FP4
// Quantization" (gist.science, German edition), Technische Zusammenfassung §2
// "GPU-Kernel-Unterstützung (QuTLASS)": the 4-bit matmul of the online path.
//
// Design for CDNA4 (measured on MI355X):
//  * v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands runs at twice the rate of the
//    16x16x128 form, so every product is a 32x32x64 scaled MFMA; lane l carries 32 K
//    elements (one MXFP4 group) of row l % 32 and that group's E8M0 byte.
//  * 8 waves (2 per SIMD). The 256x256 tile uses a 2 x 4 wave layout, 128 x 64 outputs per
//    wave (128 accumulators), so one wave's LDS reads overlap the other wave's MFMAs.
//  * K advances in stages of 256 elements (128 bytes per row). A 2-deep LDS ring (3-deep for the
//    one-row-tile grids below) is filled
//    with buffer_load_dwordx4 ... lds (LDS DMA, no register staging; the stage's offset in the
//    scalar offset field); 16-byte chunks of a row are XOR-swizzled by the row's low five bits
//    so the 32 rows of a fragment read hit distinct banks. The buffer form, not
//    global_load_lds: the compiler counts a pending FLAT-encoded DMA as a possible LDS access
//    and so waits for every LDS read (lgkmcnt(0)) before each MFMA group while one is in
//    flight; with the buffer form it waits only for the fragments the MFMAs use.
//  * LDS holds the A rows of the ring's stages, then the B rows, then the scales: every fragment
//    read is one of four per-lane offsets (per k-step) plus the stage's base and an immediate,
//    and the loop carries about a dozen VALU instructions per stage (which compete with the
//    MFMAs for issue cycles on gfx950).
//  * K order within a stage: k-step ks takes chunk ks of each row in lane half 0 and chunk
//    ks + 4 in lane half 1, for both operands, so every product still pairs x_k with w_k and
//    a lane half's four E8M0 bytes of the stage are one dword, read once per stage; op_sel = ks
//    picks the byte.
//  * The workgroup barrier of the ring waits for LDS reads only (each wave has already
//    waited for its own DMA of the stage), so in-flight prefetches are not drained.
//  * E8M0 scales are DMA'd 16 bytes per row (two stages) into their own double buffer.
//  * Output tiles go through LDS so Y is written as whole row segments.
//  * Tile order: workgroup i runs on XCD i % 8; each XCD takes a contiguous range of tiles,
//    walked M-fastest within groups of 8 tile rows, so tiles running together share
//    A and B slices in that XCD's L2.
//  * Two tile widths in one launch. When the 256x256 tiles would leave the last round of
//    workgroups part-filled, the columns left after whole rounds of 256-wide tiles are
//    covered by 256x192 tiles (4 x 2 waves of 64 x 96), each about 0.78 of a wide tile's
//    time, so the last round is full of cheaper tiles.
//  * Fewer than 256 rows of X (and N >= 1024; 33-64 rows from N >= 8192): 64-column tiles, 128 x 64
//    up to 128 rows, 256 x 64 above (two 128 x 64 row tiles where the 256-row grid would fill at
//    most half the CUs), so that enough workgroups stream W; rows past M repeat row M-1. A stage then holds few MFMAs per wave, so their ring is 3
//    deep: the DMA of stage s + 2 is issued while stage s is multiplied (from HBM at N = 14336,
//    K = 4096: 128 rows 13.8 against 17.4 us with 2 deep; 4 or 5 deep measured no faster).
// Requires K % 512 == 0 (whole scale groups) and K < 2^25 (32-bit buffer offsets); other
// shapes use the general kernel.
#include <atomic>
#include <type_traits>

#include "common.hpp"

namespace fp4 {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 256;                  // workgroup tile rows (both widths)
constexpr int WAVES = 8, NT = WAVES * 64;
constexpr int BKB = 128;                 // bytes of K per row per stage (256 elements)
constexpr int KSTEPS = 4;                // 32x32x64 steps per stage
constexpr int LDS_BYTES = 2 * (BM + 256) * BKB + 2 * (BM + 256) * 16;  // the wide tile's 2-deep ring: 144 KB

// One tile shape: BM_ rows, BN columns, WGM x WGN waves, an NS_-deep ring of stages. The DMA of
// stage s + NS - 1 is issued while stage s is multiplied; the scale bytes come 16 per row for a
// pair of stages, in SCP pair buffers (pair j + SCP is fetched with stage 2 j + 2 SCP, during
// stage 2 j + 2 SCP - NS + 1, which must come after every read of stage 2 j + 1).
template <int BN_, int WGM_, int WGN_, int BM_ = BM, int NS_ = 2>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, NS = NS_, SCP = NS_ / 2 + 1;
  static constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  static constexpr int STAGE = (BM + BN) * BKB;
  static constexpr int A_WL = BM / 8 / WAVES, B_WL = BN / 8 / WAVES;  // 1 KB DMA wave-loads per wave
  static constexpr int SC_BYTES = (BM + BN) * 16;                      // scales of 2 stages
  static constexpr int SC_LOADS = (BM + BN) / 64;                      // 64-row scale wave-loads
  static constexpr int SC_WL = (SC_LOADS + WAVES - 1) / WAVES;
  static constexpr int EP = WN * 4 + 16;                               // epilogue row pitch (bytes)
  static constexpr int RING = NS * STAGE + SCP * SC_BYTES;
  static_assert(WGM * WGN == WAVES, "wave layout");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "whole 32x32 fragments");
  static_assert(A_WL * 8 * WAVES == BM && B_WL * 8 * WAVES == BN, "row split");
  static_assert(SC_LOADS * 64 == BM + BN, "scale split");
  static_assert(NS >= 2 && 2 * SCP >= NS + 1, "scale pair buffers outlive their reads");
  static_assert(NS == 2 || SC_WL == 1, "at most one scale wave-load per wave (the wait counts assume it)");
  static_assert(RING <= LDS_BYTES, "ring fits");
  static_assert(WAVES * 32 * EP <= LDS_BYTES, "epilogue staging fits");
};
using Wide = Tile<256, 2, 4>;
using Narrow = Tile<192, 4, 2>;
// Below 256 rows a stage holds few MFMAs per wave, so a deeper ring keeps more stages in flight.
using Skinny = Tile<64, 8, 1, 256, 3>;     // 129-255 rows: 256 x 64 tiles, 8 waves of 32 x 64
using Skinny128 = Tile<64, 4, 2, 128, 3>;  // 33-128 rows: 128 x 64 tiles, 8 waves of 32 x 32
template <class C>
constexpr int lds_need() {  // the ring and scale buffers, or the epilogue staging if larger
  return C::RING > WAVES * 32 * C::EP ? C::RING : WAVES * 32 * C::EP;
}
constexpr float kNarrowCost = 0.78f;  // measured time of a 256x192 tile over a 256x256 one (MXFP4)

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

template <int SEL>
__device__ __forceinline__ v16f mfma32(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, SEL, sa, SEL, sb);
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

// One output tile [m0, m0 + 256) x [n0, n0 + C::BN) over all of K.
template <bool OUT_BF16, class C>
__device__ __forceinline__ void ring_tile(uint8_t* smem, const uint8_t* __restrict__ Xq,
                                          const uint8_t* __restrict__ Xs, const uint8_t* __restrict__ Wq,
                                          const uint8_t* __restrict__ Ws, void* __restrict__ Yv, int M, int N,
                                          int K, int m0, int n0) {
  constexpr int BM = C::BM;
  constexpr int WGN = C::WGN, WM = C::WM, WN = C::WN, FM = C::FM, FN = C::FN;
  constexpr int STAGE = C::STAGE, A_WL = C::A_WL, B_WL = C::B_WL, SC_BYTES = C::SC_BYTES, SC_WL = C::SC_WL;
  constexpr int NS = C::NS, SCP = C::SCP, D = NS - 1;  // D: stages fetched ahead
  // ring slot of stage s, and scale pair buffer of stage s
  auto slot = [](int s) { return NS == 2 ? (s & 1) : (int)((unsigned)s % NS); };
  auto pair = [](int s) { return SCP == 2 ? ((s >> 1) & 1) : (int)(((unsigned)s >> 1) % SCP); };
  // LDS: the A rows of the NS stages, then their B rows, then the scale buffers, so that a
  // fragment read is a per-lane offset of the stage plus an immediate.
  constexpr int A_ST = BM * BKB, B_ST = C::BN * BKB, B_BASE = NS * A_ST;
  uint8_t* scl = smem + NS * STAGE;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;
  const int KB = K / 2, KS = K / 32;
  const int nst = K / 256;  // even

  // DMA sources: 8 rows x 128 bytes per wave-load; rows past M / N repeat the last row. The
  // loads take the buffer form: a wave-uniform resource at the tile's first row of each operand
  // (its range the rows the tile may touch) and a 32-bit per-lane offset, which stays below
  // 256 * K / 2 < 2^32 since the kernel requires K < 2^25.
  const int rows_a = min(M - m0, BM), rows_b = min(N - n0, C::BN);
  const __amdgpu_buffer_rsrc_t rsA = buffer_rsrc(Xq + (size_t)m0 * KB, (unsigned)rows_a * KB);
  const __amdgpu_buffer_rsrc_t rsB = buffer_rsrc(Wq + (size_t)n0 * KB, (unsigned)rows_b * KB);
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
  // scale rows: loads below BM / 64 are X's rows, the rest W's (wave-uniform per load)
  const __amdgpu_buffer_rsrc_t rsXs = buffer_rsrc(Xs + (size_t)m0 * KS, (unsigned)rows_a * KS);
  const __amdgpu_buffer_rsrc_t rsWs = buffer_rsrc(Ws + (size_t)n0 * KS, (unsigned)rows_b * KS);
#pragma unroll
  for (int i = 0; i < SC_WL; ++i) {
    const int rb = min(wave * SC_WL + i, C::SC_LOADS - 1) * 64;  // wave-uniform; waves past the last load skip
    const int r = rb + lane;
    offS[i] = rb < BM ? (unsigned)min(r, rows_a - 1) * KS : (unsigned)min(r - BM, rows_b - 1) * KS;
  }

  // Part p (0..KSTEPS-1) of the DMA of stage s: its codes, wave-load i going with part
  // i % KSTEPS, and on part 0 of an even stage the scales of stages s, s+1 (16 bytes per row).
  // The parts are issued one per k-step of the stage before, so no wave stalls on a burst of
  // nine loads while it could be issuing MFMAs.
  auto issue_part = [&](int s, int p) {
    if (p == 0 && (s & 1) == 0) {
      uint8_t* dst = scl + pair(s) * SC_BYTES;
#pragma unroll
      for (int i = 0; i < SC_WL; ++i)
        if (wave * SC_WL + i < C::SC_LOADS)
          __builtin_amdgcn_raw_ptr_buffer_load_lds((wave * SC_WL + i) * 64 < BM ? rsXs : rsWs,
                                                   (lds_void*)(dst + (wave * SC_WL + i) * 1024), 16,
                                                   offS[i], (unsigned)(s >> 1) * 16, 0, 0);
    }
    uint8_t* bufa = smem + slot(s) * A_ST;
    uint8_t* bufb = smem + B_BASE + slot(s) * B_ST;
#pragma unroll
    for (int i = 0; i < A_WL; ++i)
      if (i % KSTEPS == p)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_void*)(bufa + (wave * A_WL + i) * 1024), 16,
                                                 offA[i], (unsigned)s * BKB, 0, 0);
#pragma unroll
    for (int i = 0; i < B_WL; ++i)
      if (i % KSTEPS == p)
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
  // chunk ks + 4 h; the stage adds A_ST / B_ST, fragment i / j an immediate i * 4 KB
  const int ra = (wm0 + fr) * BKB, rb = B_BASE + (wn0 + fr) * BKB;
  int cx[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) cx[ks] = ((ks + 4 * fh) ^ swz(fr)) << 4;

  // Stage s: wait for its DMA (this wave's, then everyone's at the barrier), then multiply it
  // while the parts of stage s+D refill the buffer of stage s-1, which every wave has finished
  // reading once past the barrier. The last D stages are peeled off so that the loop body issues
  // its DMA unconditionally (a per-k-step condition makes the compiler wait on the DMA before
  // every LDS read).
  // This wave's loads still allowed in flight at the top of a stage s with s + D < nst: those of
  // stages s+1 .. s+D-1, i.e. A_WL + B_WL each, plus the scale load on the even ones if the wave
  // issues one (of D-1 consecutive stages from s+1, D/2 are even if s+1 is, else (D-1)/2).
  auto wait_stage = [&](int s, auto with_dma) {
    constexpr int L = (D - 1) * (A_WL + B_WL);
    if constexpr (!decltype(with_dma)::value || D == 1) {
      wait_vmcnt<0>();
    } else {
      if (wave >= C::SC_LOADS) wait_vmcnt<L>();
      else if (s & 1) wait_vmcnt<L + D / 2>();
      else wait_vmcnt<L + (D - 1) / 2>();
    }
  };
  auto run_stage = [&](int s, auto with_dma) {
    wait_stage(s, with_dma);
    ring_barrier();
    const int sl = slot(s);
    const int la = ra + sl * A_ST, lb = rb + sl * B_ST;
    // the lane half's 4 scale bytes of the stage (pair buffer (s >> 1) % SCP, bytes 8 (s & 1) +
    // 4 h .. + 3 of the row's 16): byte ks goes with k-step ks
    unsigned sg_a[FM], sg_b[FN];
    {
      const uint8_t* sbuf = scl + pair(s) * SC_BYTES + 8 * (s & 1) + 4 * fh;
#pragma unroll
      for (int i = 0; i < FM; ++i) sg_a[i] = *reinterpret_cast<const unsigned*>(sbuf + (wm0 + i * 32 + fr) * 16);
#pragma unroll
      for (int j = 0; j < FN; ++j) sg_b[j] = *reinterpret_cast<const unsigned*>(sbuf + (BM + wn0 + j * 32 + fr) * 16);
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if constexpr (decltype(with_dma)::value) issue_part(s + D, ks);
      v4u a[FM], b[FN];
      const int oa = la + cx[ks], ob = lb + cx[ks];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = *reinterpret_cast<const v4u*>(smem + oa + i * 32 * BKB);
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = *reinterpret_cast<const v4u*>(smem + ob + j * 32 * BKB);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const v8i av = v8i{(int)a[i][0], (int)a[i][1], (int)a[i][2], (int)a[i][3], 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v8i bv = v8i{(int)b[j][0], (int)b[j][1], (int)b[j][2], (int)b[j][3], 0, 0, 0, 0};
          switch (ks) {  // byte ks of the lane half's scale dword
            case 0: acc[i][j] = mfma32<0>(av, bv, acc[i][j], (int)sg_a[i], (int)sg_b[j]); break;
            case 1: acc[i][j] = mfma32<1>(av, bv, acc[i][j], (int)sg_a[i], (int)sg_b[j]); break;
            case 2: acc[i][j] = mfma32<2>(av, bv, acc[i][j], (int)sg_a[i], (int)sg_b[j]); break;
            default: acc[i][j] = mfma32<3>(av, bv, acc[i][j], (int)sg_a[i], (int)sg_b[j]); break;
          }
        }
      }
    }
  };
  if constexpr (D == 1) {
#pragma unroll
    for (int p = 0; p < KSTEPS; ++p) issue_part(0, p);
    for (int s = 0; s + 1 < nst; ++s) run_stage(s, std::true_type{});
    run_stage(nst - 1, std::false_type{});
  } else {
    for (int t = 0; t < D && t < nst; ++t)
#pragma unroll
      for (int p = 0; p < KSTEPS; ++p) issue_part(t, p);
    int s = 0;
    for (; s + D < nst; ++s) run_stage(s, std::true_type{});
    for (; s < nst; ++s) run_stage(s, std::false_type{});
  }

  // Epilogue: each wave stages one 32 x WN slab at a time in its own LDS region, then writes
  // whole 16-byte pieces of its rows, 64 per wave instruction: 4 float32 values per piece, or
  // 8 bf16 values (read back as two 16-byte halves of float32, rounded to nearest even).
  constexpr int EP = C::EP;
  constexpr int VPP = OUT_BF16 ? 8 : 4;  // values per 16-byte piece of Y
  constexpr int CPR = WN / VPP;          // pieces per row
  __syncthreads();  // every wave is done with the ring
  float* ep = reinterpret_cast<float*>(smem + wave * 32 * EP);
  const bool vec = N % VPP == 0;  // every piece starts 16-byte aligned (Y itself is)
  const bool vec4 = N % 4 == 0;   // bf16: every piece starts 8-byte aligned
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = 8 * (v >> 2) + 4 * fh + (v & 3);  // 32x32 accumulator layout
        ep[rr * (EP / 4) + j * 32 + fr] = acc[i][j][v];
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's slab is in LDS (wave-private region)
#pragma unroll
    for (int k = 0; k < 32 * CPR / 64; ++k) {
      const int cix = k * 64 + lane;
      const int rr = cix / CPR, cc = cix % CPR;
      float val[VPP];
#pragma unroll
      for (int h = 0; h < VPP / 4; ++h) {
        const v4f t = *reinterpret_cast<const v4f*>(&ep[rr * (EP / 4) + cc * VPP + 4 * h]);
#pragma unroll
        for (int q = 0; q < 4; ++q) val[4 * h + q] = t[q];
      }
      const int row = m0 + wm0 + i * 32 + rr;
      const int col = n0 + wn0 + cc * VPP;
      if (row >= M) continue;
      if constexpr (OUT_BF16) {
        __bf16* dst = reinterpret_cast<__bf16*>(Yv) + (size_t)row * N + col;
        v4u pk;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          pk[q] = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)val[2 * q]) |
                  ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)val[2 * q + 1]) << 16);
        if (vec && col + VPP <= N) {
          __builtin_nontemporal_store(pk, reinterpret_cast<v4u*>(dst));
        } else if (vec4 && col + VPP <= N) {  // rows 8-byte aligned only: two 8-byte halves
          typedef unsigned v2u_ __attribute__((ext_vector_type(2)));
          __builtin_nontemporal_store(v2u_{pk[0], pk[1]}, reinterpret_cast<v2u_*>(dst));
          __builtin_nontemporal_store(v2u_{pk[2], pk[3]}, reinterpret_cast<v2u_*>(dst) + 1);
        } else {
          for (int q = 0; q < VPP; ++q)
            if (col + q < N) dst[q] = (__bf16)val[q];
        }
      } else {
        float* dst = reinterpret_cast<float*>(Yv) + (size_t)row * N + col;
        if (vec && col + VPP <= N) {
          __builtin_nontemporal_store(v4f{val[0], val[1], val[2], val[3]}, reinterpret_cast<v4f*>(dst));
        } else {
          for (int q = 0; q < VPP; ++q)
            if (col + q < N) dst[q] = val[q];
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
__global__ __launch_bounds__(NT) void gemm_mxfp4_ring(const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ Xs,
                                                      const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Ws,
                                                      void* __restrict__ Yv, int M, int N, int K, int tiles_m, int tn1,
                                                      int tn2) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int T1 = tiles_m * tn1, T2 = tiles_m * tn2;
  int b = blockIdx.x, tm, tn;
  if (b < T1) {
    const int L = (T1 % 8 == 0) ? (b & 7) * (T1 >> 3) + (b >> 3) : b;
    map_tile(L, tiles_m, tn1, tm, tn);
    ring_tile<OUT_BF16, Wide>(smem, Xq, Xs, Wq, Ws, Yv, M, N, K, tm * BM, tn * Wide::BN);
  } else {
    b -= T1;
    const int L = (T1 % 8 == 0 && T2 % 8 == 0) ? (b & 7) * (T2 >> 3) + (b >> 3) : b;
    map_tile(L, tiles_m, tn2, tm, tn);
    ring_tile<OUT_BF16, Narrow>(smem, Xq, Xs, Wq, Ws, Yv, M, N, K, tm * BM, tn1 * Wide::BN + tn * Narrow::BN);
  }
}

// One C::BM x 64 tile per workgroup, tile index b -> (tm, tn) M-fastest; for fewer than 256 rows of X.
template <bool OUT_BF16, class C>
__global__ __launch_bounds__(NT) void gemm_mxfp4_ring_skinny(const uint8_t* __restrict__ Xq,
                                                             const uint8_t* __restrict__ Xs,
                                                             const uint8_t* __restrict__ Wq,
                                                             const uint8_t* __restrict__ Ws, void* __restrict__ Yv,
                                                             int M, int N, int K, int tiles_m) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int b = blockIdx.x, tm = b % tiles_m, tn = b / tiles_m;
  ring_tile<OUT_BF16, C>(smem, Xq, Xs, Wq, Ws, Yv, M, N, K, tm * C::BM, tn * C::BN);
}

template <bool B>
std::atomic<int> g_skinny_attr[2][64];

template <bool B, class C>
hipError_t launch_skinny(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws, int M, int N,
                         int K, void* Y, int dev, int slot, hipStream_t st) {
  auto sk = gemm_mxfp4_ring_skinny<B, C>;
  const bool cached = dev >= 0 && dev < 64;
  if (!cached || !g_skinny_attr<B>[slot][dev].load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute((const void*)sk, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    if (cached) g_skinny_attr<B>[slot][dev].store(1, std::memory_order_release);
  }
  const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
  hipLaunchKernelGGL(sk, dim3(tiles_m * tiles_n), dim3(NT), lds_need<C>(), st, Xq, Xs, Wq, Ws, Y, M, N, K, tiles_m);
  return hipGetLastError();
}

// per kernel instantiation and device: the dynamic-LDS limit has been raised
template <bool B>
std::atomic<int> g_attr_done[64];
std::atomic<int> g_cus[64];  // compute units per device, 0 until queried

template <bool B>
hipError_t launch(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws, int M, int N, int K,
                  void* Y, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  auto kern = gemm_mxfp4_ring<B>;
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
  // Below 256 rows: one 128-row tile per 64 columns up to 128 rows. Above, one 256-row tile per 64
  // columns when that grid fills more than half the CUs, else two 128-row tiles per 64 columns
  // (78 KB of LDS each, so two share a CU): at 129-255 rows and N = 4096 (K = 4096, W from HBM)
  // 10.2-12.0 against 14.1-15.8 us, while at N = 14336 the 256-row tiles win (15.5-17.2 against
  // 18.7-23.9 us).
  if (M <= 128 || (M < BM && 2 * ((N + 63) / 64) <= cus))
    return launch_skinny<B, Skinny128>(Xq, Xs, Wq, Ws, M, N, K, Y, dev, 1, st);
  if (M < BM) return launch_skinny<B, Skinny>(Xq, Xs, Wq, Ws, M, N, K, Y, dev, 0, st);
  int tn1, tn2;
  fp4_plan_tile_columns(tiles_m, N, cus, kNarrowCost, tn1, tn2);
  hipLaunchKernelGGL(kern, dim3(tiles_m * (tn1 + tn2)), dim3(NT), LDS_BYTES, st, Xq, Xs, Wq, Ws, Y, M, N, K, tiles_m,
                     tn1, tn2);
  return hipGetLastError();
}

}  // namespace
}  // namespace fp4

// 33-64 rows take the 128-row tiles only on layers of at least this many columns: there the
// one-row-tile grid has 128+ workgroups and beats the weight-streaming decode kernel (N = 8192,
// 64 rows: 11.0 against 14.0 us; N = 14336: 11.7 against 16.2 us), while at N = 4096 its 64
// workgroups lose (10.2 against 7.0 us at 40 rows).
static constexpr int64_t kMidN = 8192;
bool fp4_gemm_mxfp4_ring_fits(int64_t M, int64_t N, int64_t K) {
  return K % 512 == 0 && K < ((int64_t)1 << 25) &&
         ((M >= 256 && N >= 256) || (M > 64 && N >= 1024) || (M > 32 && N >= kMidN));
}

hipError_t fp4_launch_gemm_mxfp4_ring(const uint8_t* Xq, const uint8_t* Xs, const uint8_t* Wq, const uint8_t* Ws,
                                      int64_t M, int64_t N, int64_t K, void* Y, int out_bf16, hipStream_t st) {
  return out_bf16 ? fp4::launch<true>(Xq, Xs, Wq, Ws, (int)M, (int)N, (int)K, Y, st)
                  : fp4::launch<false>(Xq, Xs, Wq, Ws, (int)M, (int)N, (int)K, Y, st);
}
