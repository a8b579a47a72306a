// bf16 GEMM main loop shared by the prefill-side kernels of the latent-cache library (gfx950).
//
// One workgroup computes a BM x BN tile of C[m][n] = sum_k A[m][k] B[n][k] (both operands stored with
// rows contiguous along k) with WGM x WGN waves, each wave a (BM/WGM) x (BN/WGN) block of
// 32 x 32 x 16 bf16 MFMAs accumulated in fp32.  Operand tiles of 32 k stream through an NSTG-stage LDS
// ring by direct-to-LDS DMA (NSTG - 1 stages in flight, one barrier per stage);
// 64-byte tile rows keep their 16-byte chunks XOR-swizzled by row so that the MFMA operand reads are
// bank-conflict free.  The caller supplies per-row source addresses (any row mapping: cache rows of
// several sequences, weight rows, clamped edges) and writes the epilogue from the accumulators.
#pragma once

#include "common.h"

namespace mla {

// 16 bytes per lane from a per-lane 64-bit global address into LDS at lds_addr + 16 * lane
// (global_load_lds_dwordx4 without a scalar base).  Completion is awaited with MLA_WAIT_VMCNT.
__device__ __forceinline__ void dma16_ptr(const void* p, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(p), "s"(lds_addr)
      : "memory");  // M0 is rewritten here; no other instruction in these kernels reads M0
}

template <int BM, int BN, int NSTG_ = 4, int WGM_ = 2, int WGN_ = 2>
struct GemmCfg {
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sides are multiples of 64");
  static_assert(NSTG_ == 3 || NSTG_ == 4, "three or four stages");
  static constexpr int BK = 32, NSTG = NSTG_, WGM = WGM_, WGN = WGN_, NW = WGM * WGN, THREADS = 64 * NW;
  static constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave blocks are multiples of 32");
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = NSTG * STAGE;
  // DMA instructions (16 rows of 64 bytes each) per stage.  When both operands split evenly over the
  // waves, wave w issues A_IPW instructions of A and B_IPW of B; otherwise the NQ instructions of the
  // stage tile [A; B] are dealt out round-robin (wave w takes q = w, w + NW, ...), so the first NQ % NW
  // waves issue one more than the others.
  static constexpr int NQ = (BM + BN) / 16;
  static constexpr bool EVEN = BM % (16 * NW) == 0 && BN % (16 * NW) == 0;
  static constexpr int A_IPW = BM / (16 * NW), B_IPW = BN / (16 * NW);
  static constexpr int IPW = (NQ + NW - 1) / NW;  // the most DMA instructions any wave issues per stage
};

// Byte offset of (row, 16-byte chunk) in a stage tile with 64-byte rows.
__device__ __forceinline__ int gemm_swz(int row, int chunk) { return row * 64 + 16 * (chunk ^ ((row >> 2) & 3)); }

// Accumulator element e of block (fm, fn) of wave (wm, wn) = (w / WGN, w % WGN) is
// C[wm*WM + 32 fm + 8(e/4) + 4(lane/32) + e%4][wn*WN + 32 fn + lane%32].  K must be a multiple of 32.
// Returns with the ring idle (no DMA in flight); the caller synchronises before reusing the LDS.
template <class C, class ARow, class BRow>
__device__ __forceinline__ void gemm_tile_cfg(char* lds, int K, ARow a_row, BRow b_row, f32x16 (&acc)[C::FM][C::FN]) {
  constexpr int BM = C::WM * C::WGM;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = w / C::WGN, wn = w % C::WGN;
  // this wave's DMA instructions: source row pointers (own 16-byte chunk) and LDS offsets in the stage
  const char* src[C::IPW];
  uint32_t dst[C::IPW];
  auto row_src = [&](int row) -> const char* {
    const char* p = row < BM ? (const char*)a_row(row) : (const char*)b_row(row - BM);
    return p + 16 * ((lane & 3) ^ ((row >> 2) & 3));
  };
#pragma unroll
  for (int i = 0; i < C::IPW; ++i) {
    int q;
    if constexpr (C::EVEN) {
      q = i < C::A_IPW ? w * C::A_IPW + i : BM / 16 + w * C::B_IPW + (i - C::A_IPW);
    } else {
      q = min(w + C::NW * i, C::NQ - 1);  // past the last instruction: never issued
    }
    src[i] = row_src(16 * q + (lane >> 2));
    dst[i] = q * 1024;
  }
  // instructions this wave issues per stage (wave-uniform)
  const int cnt = C::EVEN ? C::IPW : (w + C::NW * (C::IPW - 1) < C::NQ ? C::IPW : C::IPW - 1);
  const uint32_t lds0 = lds_addr_of(lds);
  auto issue = [&](int kt) {
    const uint32_t base = lds0 + (kt % C::NSTG) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::IPW; ++i)
      if (C::EVEN || i + 1 < C::IPW || cnt == C::IPW) dma16_ptr(src[i] + kt * 64, base + dst[i]);
  };
  const int KT = K / C::BK;
  // own part of stage s is complete once only the stages issued after it may be outstanding
  auto wait_n = [&](int later) {  // later in 0 .. NSTG - 2, wave-uniform
    if (C::EVEN || cnt == C::IPW) {
      if (C::NSTG > 3 && later >= 2) {
        MLA_WAIT_VMCNT(2 * C::IPW);
      } else if (later >= 1) {
        MLA_WAIT_VMCNT(C::IPW);
      } else {
        MLA_WAIT_VMCNT(0);
      }
    } else {
      if (C::NSTG > 3 && later >= 2) {
        MLA_WAIT_VMCNT(2 * (C::IPW - 1));
      } else if (later >= 1) {
        MLA_WAIT_VMCNT(C::IPW - 1);
      } else {
        MLA_WAIT_VMCNT(0);
      }
    }
  };
  auto wait_stage = [&](int s) { wait_n(min(KT - 1, s + C::NSTG - 2) - s); };
  // operands of one k-slice of 16 (ks = 0, 1) of stage s
  struct Frag {
    bf16x8 a[C::FM], b[C::FN];
  };
  auto load = [&](Frag& f, int s, int ks) {
    const char* sa = lds + (s % C::NSTG) * C::STAGE;
    const char* sb = sa + C::A_BYTES;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
      f.a[i] = *(const bf16x8*)(sa + gemm_swz(wm * C::WM + 32 * i + (lane & 31), 2 * ks + (lane >> 5)));
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      f.b[j] = *(const bf16x8*)(sb + gemm_swz(wn * C::WN + 32 * j + (lane & 31), 2 * ks + (lane >> 5)));
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma32(f.a[i], f.b[j], acc[i][j]);
  };
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};
  // Stage s is read after the barrier that follows every wave's wait for its part of s; that barrier
  // also ends all reads of stage s-1, whose slot then receives stage s + NSTG - 1.  The second slice
  // of a stage is loaded before the first slice's MFMAs, the next stage's first slice right after its
  // barrier, so LDS latency hides under MFMAs that are already issued.
#pragma unroll
  for (int s = 0; s < C::NSTG - 1; ++s)
    if (s < KT) issue(s);
  wait_stage(0);
  lds_barrier();
  if (C::NSTG - 1 < KT) issue(C::NSTG - 1);
  // (the last stage is peeled off: a branch around the barrier part would join the two paths before
  // mma(f1), and the compiler's wait for f1 there would then also wait for the next stage's reads)
  Frag f0, f1;
  load(f0, 0, 0);
  for (int kt = 0; kt + 1 < KT; ++kt) {
    load(f1, kt, 1);
    mma(f0);
    wait_stage(kt + 1);
    lds_barrier();
    if (kt + C::NSTG < KT) issue(kt + C::NSTG);
    load(f0, kt + 1, 0);
    mma(f1);
  }
  load(f1, KT - 1, 1);
  mma(f0);
  mma(f1);
}

template <int BM, int BN, int NSTG, class ARow, class BRow>
__device__ __forceinline__ void gemm_tile(char* lds, int K, ARow a_row, BRow b_row,
                                          f32x16 (&acc)[GemmCfg<BM, BN, NSTG>::FM][GemmCfg<BM, BN, NSTG>::FN]) {
  gemm_tile_cfg<GemmCfg<BM, BN, NSTG>>(lds, K, a_row, b_row, acc);
}

}  // namespace mla
