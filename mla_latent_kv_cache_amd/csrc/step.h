// Device pieces shared by the append kernels and the fused decode-step prologue (gfx950).
#pragma once

#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int SM_MAXM = 64;  // few-token appends: at most 64 tokens (two 32-row MFMA blocks)
constexpr int KS_MAX = 16;   // model-width slices of the split-K append

// Split-K append, phase 1, workgroup (bx: 32 output columns, by: one of KS slices of the model width):
// 4 waves split the slice, MFMA 32x32x16 over up to two 32-token blocks, and the workgroup's partial
// sums (fp32, [KS][M][N]) go to the workspace.  The reduction and epilogue run in append_reduce.
__device__ __forceinline__ void append_splitk_tile(const AppendArgs& a, int KS, int bx, int by) {
  __shared__ float red[4][SM_MAXM][32];
  const int K = a.s.d_model, D = a.s.d_kv, NR = a.s.n_rope_cols(), N = D + NR;
  const int M = a.batch * a.t_new, MB = (M + 31) / 32;
  const int n0 = bx * 32, ks = by;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int kslice = K / KS, kw = kslice / 4, k0 = ks * kslice + w * kw;
  const bf16* x = (const bf16*)a.x;
  const int gn = n0 + (lane & 31);
  const bf16* wrow = gn < D ? (const bf16*)a.w_dkv + (size_t)gn * K : (const bf16*)a.w_krope + (size_t)(gn - D) * K;
  const bool nok = gn < N;
  const bf16x8 zero8 = {};
  constexpr int SB = 8;  // K steps of 16 per lane issued together (kw <= 128)
  bf16x8 bv[SB], a0[SB], a1[SB];
#pragma unroll
  for (int u = 0; u < SB; ++u) {
    const int kk = k0 + 16 * u + 8 * (lane >> 5);
    const bool kin = 16 * u < kw;
    bv[u] = (nok && kin) ? *(const bf16x8*)(wrow + kk) : zero8;
    a0[u] = ((lane & 31) < M && kin) ? *(const bf16x8*)(x + (size_t)(lane & 31) * K + kk) : zero8;
    a1[u] = (MB > 1 && 32 + (lane & 31) < M && kin) ? *(const bf16x8*)(x + (size_t)(32 + (lane & 31)) * K + kk) : zero8;
  }
  f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int u = 0; u < SB; ++u) {
    acc[0] = mfma32(a0[u], bv[u], acc[0]);
    if (MB > 1) acc[1] = mfma32(a1[u], bv[u], acc[1]);
  }
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[w][mb * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)][lane & 31] = acc[mb][e];
  __syncthreads();
  float* part = (float*)a.ws + (size_t)ks * M * N;
  for (int idx = threadIdx.x; idx < M * 32; idx += blockDim.x) {
    const int m = idx >> 5, c = idx & 31;
    if (n0 + c < N) part[(size_t)m * N + n0 + c] = red[0][m][c] + red[1][m][c] + red[2][m][c] + red[3][m][c];
  }
}

}  // namespace mla
