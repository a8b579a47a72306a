// bf16 GEMM main loop shared by the prefill-side kernels of the latent-cache library (gfx950).
//
// One workgroup computes a BM x BN tile of C[m][n] = sum_k A[m][k] B[n][k] (both operands stored with
// rows contiguous along k) with four waves in a 2 x 2 layout, each wave a (BM/2) x (BN/2) block of
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

template <int BM, int BN, int NSTG_ = 4>
struct GemmCfg {
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sides are multiples of 64");
  static_assert(NSTG_ == 3 || NSTG_ == 4, "three or four stages");
  static constexpr int BK = 32, NSTG = NSTG_;
  static constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = NSTG * STAGE;
  // DMA instructions (16 rows of 64 bytes each) per wave and stage
  static constexpr int A_IPW = BM / 64, B_IPW = BN / 64, IPW = A_IPW + B_IPW;
};

// Byte offset of (row, 16-byte chunk) in a stage tile with 64-byte rows.
__device__ __forceinline__ int gemm_swz(int row, int chunk) { return row * 64 + 16 * (chunk ^ ((row >> 2) & 3)); }

// Accumulator element e of block (fm, fn) of wave (wm, wn) is C[wm*WM + 32 fm + 8(e/4) + 4(lane/32) + e%4]
// [wn*WN + 32 fn + lane%32].  K must be a multiple of 32.  Returns with the ring idle (no DMA in flight);
// the caller synchronises before reusing the LDS.
template <int BM, int BN, int NSTG, class ARow, class BRow>
__device__ __forceinline__ void gemm_tile(char* lds, int K, ARow a_row, BRow b_row,
                                          f32x16 (&acc)[GemmCfg<BM, BN, NSTG>::FM][GemmCfg<BM, BN, NSTG>::FN]) {
  using C = GemmCfg<BM, BN, NSTG>;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = w >> 1, wn = w & 1;
  const char* asrc[C::A_IPW];
  const char* bsrc[C::B_IPW];
#pragma unroll
  for (int i = 0; i < C::A_IPW; ++i) {
    const int row = 16 * (w * C::A_IPW + i) + (lane >> 2);
    asrc[i] = (const char*)a_row(row) + 16 * ((lane & 3) ^ ((row >> 2) & 3));
  }
#pragma unroll
  for (int i = 0; i < C::B_IPW; ++i) {
    const int row = 16 * (w * C::B_IPW + i) + (lane >> 2);
    bsrc[i] = (const char*)b_row(row) + 16 * ((lane & 3) ^ ((row >> 2) & 3));
  }
  const uint32_t lds0 = lds_addr_of(lds);
  auto issue = [&](int kt) {
    const uint32_t base = lds0 + (kt % C::NSTG) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::A_IPW; ++i) dma16_ptr(asrc[i] + kt * 64, base + (w * C::A_IPW + i) * 1024);
#pragma unroll
    for (int i = 0; i < C::B_IPW; ++i) dma16_ptr(bsrc[i] + kt * 64, base + C::A_BYTES + (w * C::B_IPW + i) * 1024);
  };
  const int KT = K / C::BK;
  // own part of stage s is complete once only the stages issued after it may be outstanding
  auto wait_stage = [&](int s) {
    const int later = min(KT - 1, s + C::NSTG - 2) - s;
    if (C::NSTG > 3 && later >= 2) {
      MLA_WAIT_VMCNT(2 * C::IPW);
    } else if (later >= 1) {
      MLA_WAIT_VMCNT(C::IPW);
    } else {
      MLA_WAIT_VMCNT(0);
    }
  };
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

}  // namespace mla
