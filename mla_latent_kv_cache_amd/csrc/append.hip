// Latent-cache append on gfx950: c_kv = x . W_dkv and the per-head retained RoPE keys.
//
// The down-projection of the MHA2MLA key-designs section (Paper-Notes ACL2025 page, 关键设计):
// each token's latent row c_kv = x . W_dkv is shared by all heads, and each head keeps the keys of
// its r retained RoPE subspaces [2p, 2p+1], rotated at the token's position (the RoPE part cannot
// be merged into the matrices, so it is cached separately).  Both projections run as ONE GEMM over
// the row-concatenation [W_dkv^T ; W_krope] (N = d_kv + n_h*2r outputs per token); the epilogue
// rotates adjacent output-column pairs and stores c_kv either in the cache dtype or as int4 codes.
#include <hip/hip_fp16.h>

#include "common.h"
#include "gemm.h"
#include "kernels.h"
#include "step.h"

namespace mla {

namespace {

// ------------------------------------------------------------------ generic path (any dtype / format)
// One workgroup per token: x row staged in LDS, one thread per output column, then the epilogue.
template <typename T>
__global__ __launch_bounds__(256) void append_generic(AppendArgs a) {
  extern __shared__ float sh[];
  const int d = a.s.d_model, D = a.s.d_kv, NR = a.s.n_rope_cols(), N = D + NR;
  float* xs = sh;
  float* outs = sh + d;
  const int m = blockIdx.x;
  const T* x = (const T*)a.x + (size_t)m * d;
  for (int k = threadIdx.x; k < d; k += blockDim.x) xs[k] = to_f32(x[k]);
  __syncthreads();
  for (int n = threadIdx.x; n < N; n += blockDim.x) {
    const T* w = n < D ? (const T*)a.w_dkv + (size_t)n * d : (const T*)a.w_krope + (size_t)(n - D) * d;
    float acc = 0.f;
    for (int k = 0; k < d; ++k) acc = fmaf(xs[k], to_f32(w[k]), acc);
    outs[n] = acc;
  }
  __syncthreads();
  int pos;
  const size_t row = (size_t)cache_row(a, m, &pos);
  if (a.s.fmt == 0) {
    T* ckv = (T*)a.ckv + row * D;
    for (int n = threadIdx.x; n < D; n += blockDim.x) ckv[n] = from_f32<T>(outs[n]);
  } else if (a.s.fmt >= 2) {
    for (int g = threadIdx.x; g < D / 32; g += blockDim.x) store_group_win2(a, m / a.t_new, pos, g, outs + 32 * g, 1);
  } else {
    uint8_t* codes = (uint8_t*)a.ckv + row * (D / 2);
    __half* scales = (__half*)a.ckv_scale + row * (D / 32);
    for (int g = threadIdx.x; g < D / 32; g += blockDim.x) {
      float am = 0.f;
      for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(outs[32 * g + i]));
      __half s = int4_scale(am);
      float sf = __half2float(s);
      for (int i = 0; i < 16; ++i) {
        int c0 = int4_code(outs[32 * g + 2 * i], sf), c1 = int4_code(outs[32 * g + 2 * i + 1], sf);
        codes[16 * g + i] = (uint8_t)((c0 & 15) | ((c1 & 15) << 4));
      }
      scales[g] = s;
    }
  }
  const int r = a.s.r_pairs, R2 = a.s.r2(), half = a.s.d_head / 2;
  T* kr = (T*)a.krope + row * NR;
  for (int q = threadIdx.x; q < a.s.rope_heads * r; q += blockDim.x) {  // h: RoPE key head
    int h = q / r, j = q - h * r;
    int p = load_pair(a.pair_idx, h * r + j, half);
    float c = a.rope_cos[(size_t)pos * half + p], s = a.rope_sin[(size_t)pos * half + p];
    float x0 = outs[D + h * R2 + 2 * j], x1 = outs[D + h * R2 + 2 * j + 1];
    kr[h * R2 + 2 * j] = from_f32<T>(x0 * c - x1 * s);
    kr[h * R2 + 2 * j + 1] = from_f32<T>(x0 * s + x1 * c);
  }
}

// ------------------------------------------------------------------ MFMA path (bf16)
// Workgroup tile 128 tokens x 128 output columns, K step 64, 4 waves of 64x64 (2x2 MFMA 32x32x16
// blocks), LDS double buffer with padded rows.  Workgroups are renumbered so that the
// column tiles of one token block run on the same XCD (its L2 then serves the shared x rows).
constexpr int TM = 128, TN = 128, TK = 64, PITCH = TK + 8;

__global__ __launch_bounds__(256, 2) void append_mfma_bf16(AppendArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sA[2][TM * PITCH];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][TN * PITCH];
  __shared__ int rows[TM], poss[TM];  // cache row and position of every token of the tile
  const int K = a.s.d_model, D = a.s.d_kv, NR = a.s.n_rope_cols(), N = D + NR;
  const int M = a.batch * a.t_new;
  const int n_tiles = (N + TN - 1) / TN;
  const int total = gridDim.x;
  int bid = blockIdx.x;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int m0 = (bid / n_tiles) * TM, n0 = (bid % n_tiles) * TN;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid < TM && m0 + tid < M) {
    int pos;
    rows[tid] = cache_row(a, m0 + tid, &pos);
    poss[tid] = pos;
  }  // read in the epilogue, after the main loop's barriers
  const int wm = wid >> 1, wn = wid & 1;
  const bf16* x = (const bf16*)a.x;
  const bf16* wd = (const bf16*)a.w_dkv;
  const bf16* wr = (const bf16*)a.w_krope;

  bf16x8 ra[4], rb[4];
  const bf16x8 zero8 = {};
  auto gload = [&](int kt) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      int c = it * 256 + tid, row = c >> 3, kc = (c & 7) * 8;
      int gm = m0 + row, gn = n0 + row;
      ra[it] = gm < M ? *(const bf16x8*)(x + (size_t)gm * K + kt * TK + kc) : zero8;
      const bf16* wrow = gn < D ? wd + (size_t)gn * K : wr + (size_t)(gn - D) * K;
      rb[it] = gn < N ? *(const bf16x8*)(wrow + kt * TK + kc) : zero8;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      int c = it * 256 + tid, row = c >> 3, kc = (c & 7) * 8;
      *(bf16x8*)&sA[buf][row * PITCH + kc] = ra[it];
      *(bf16x8*)&sB[buf][row * PITCH + kc] = rb[it];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int KT = K / TK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *(const bf16x8*)&sA[buf][(wm * 64 + i * 32 + (lane & 31)) * PITCH + ks * 16 + (lane >> 5) * 8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bv[j] = *(const bf16x8*)&sB[buf][(wn * 64 + j * 32 + (lane & 31)) * PITCH + ks * 16 + (lane >> 5) * 8];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(av[i], bv[j], acc[i][j]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const int r = a.s.r_pairs, R2 = a.s.r2(), half = a.s.d_head / 2;
  if (a.s.fmt >= 2 && n0 < D) {
    // windowed latent (2-bit or int4 codes): the tile's latent columns go to LDS (token rows 0-63 in sA, 64-127 in sB, which the
    // main loop no longer reads), then one thread per (token, group of 32 columns) codes or windows it
    constexpr int SP = TN + 1;
    float* stg0 = (float*)&sA[0][0];
    float* stg1 = (float*)&sB[0][0];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cl = wn * 64 + j * 32;
        if (n0 + cl >= D) continue;  // uniform across the wave
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int ml = wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          (ml < 64 ? stg0 : stg1)[(ml & 63) * SP + cl + (lane & 31)] = acc[i][j][e];
        }
      }
    __syncthreads();
    const int ng = min(TN, D - n0) / 32;
    for (int idx = threadIdx.x; idx < TM * ng; idx += blockDim.x) {
      const int ml = idx / ng, g = idx - ml * ng, m = m0 + ml;
      if (m >= M) continue;
      store_group_win2(a, m / a.t_new, poss[ml], n0 / 32 + g, (ml < 64 ? stg0 : stg1) + (ml & 63) * SP + 32 * g, 1);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c0 = n0 + wn * 64 + j * 32;
      const int n = c0 + (lane & 31);
      if (c0 >= N) continue;  // uniform across the wave
      if (c0 < D) {
        if (a.s.fmt == 0) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int ml = wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            if (m0 + ml < M) ((bf16*)a.ckv)[(size_t)rows[ml] * D + n] = (bf16)acc[i][j][e];
          }
        } else if (a.s.fmt >= 2) {
          // staged through LDS above
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float v = acc[i][j][e];
            float am = fabsf(v);
#pragma unroll
            for (int msk = 1; msk < 32; msk <<= 1) am = fmaxf(am, shfl_xor(am, msk));
            __half s = int4_scale(am);
            int code = int4_code(v, __half2float(s));
            int partner = __shfl_xor(code, 1, 64);
            const int ml = wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            if (m0 + ml < M) {
              const size_t row = (size_t)rows[ml];
              if ((lane & 1) == 0)
                ((uint8_t*)a.ckv)[row * (D / 2) + (n >> 1)] = (uint8_t)((code & 15) | ((partner & 15) << 4));
              if ((lane & 31) == 0) ((__half*)a.ckv_scale)[row * (D / 32) + (n >> 5)] = s;
            }
          }
        }
      } else {
        const int rel = n - D;
        const int h = rel / (R2 > 0 ? R2 : 1);
        const int jj = (rel - h * R2) >> 1, comp = rel & 1;
        const bool colok = rel < NR;
        const int p = load_pair(a.pair_idx, colok ? h * r + jj : 0, half);
        // the 16 rows' table entries in one round of loads (clamped in-bounds indices, no branch)
        float cst[16], snt[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int ml = wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          const size_t t = (size_t)(m0 + ml < M ? poss[ml] : 0) * half + p;
          cst[e] = a.rope_cos[t];
          snt[e] = a.rope_sin[t];
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float v = acc[i][j][e];
          float partner = shfl_xor(v, 1);
          const int ml = wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (m0 + ml < M && colok) {
            const size_t row = (size_t)rows[ml];
            const float cs = cst[e], sn = snt[e];
            float x0 = comp ? partner : v, x1 = comp ? v : partner;
            float o = comp ? (x0 * sn + x1 * cs) : (x0 * cs - x1 * sn);
            ((bf16*)a.krope)[row * NR + rel] = (bf16)o;
          }
        }
      }
    }
  }
}

// 256 x 192 tiles in eight waves of 64 x 96 (two per SIMD, so that one wave's MFMAs run while the other
// waits at the stage barrier or for its LDS operands): 133 us against 150 us with four waves of 128 x 96
// (one per SIMD) for the 16384 x 768 x 4096 down-projection of a 4 x 4096-token prompt (same-box A/B,
// identical cache rows).
using AppCfg8 = GemmCfg<256, 192, 4, 4, 2>;

// Epilogue of accumulator block (I, J): 32 output columns (one per lane, mod 32) x 32 tokens.
template <class C, int I, int J>
__device__ __forceinline__ void append_gemm_block(const AppendArgs& a, const f32x16& v, const int* rows,
                                                  const int* poss, int m0, int n0, int M) {
  const int D = a.s.d_kv, NR = a.s.n_rope_cols(), N = D + NR;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w / C::WGN, wn = w % C::WGN;
  const int c0 = n0 + wn * C::WN + J * 32;
  const int n = c0 + (lane & 31);
  if (c0 >= N) return;  // uniform across the wave
  const int r = a.s.r_pairs, R2 = a.s.r2(), half = a.s.d_head / 2;
  if (c0 < D) {
    if (a.s.fmt == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ml = wm * C::WM + I * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m0 + ml < M) ((bf16*)a.ckv)[(size_t)rows[ml] * D + n] = (bf16)v[e];
      }
    } else if (a.s.fmt >= 2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ml = wm * C::WM + I * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const bool ok = m0 + ml < M;
        store_lane_win2(a, ok, (m0 + ml) / a.t_new, ok ? poss[ml] : 0, n >> 5, v[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float am = fabsf(v[e]);
#pragma unroll
        for (int msk = 1; msk < 32; msk <<= 1) am = fmaxf(am, shfl_xor(am, msk));
        const __half s = int4_scale(am);
        const int code = int4_code(v[e], __half2float(s));
        const int partner = __shfl_xor(code, 1, 64);
        const int ml = wm * C::WM + I * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m0 + ml < M) {
          const size_t row = (size_t)rows[ml];
          if ((lane & 1) == 0)
            ((uint8_t*)a.ckv)[row * (D / 2) + (n >> 1)] = (uint8_t)((code & 15) | ((partner & 15) << 4));
          if ((lane & 31) == 0) ((__half*)a.ckv_scale)[row * (D / 32) + (n >> 5)] = s;
        }
      }
    }
  } else {
    const int rel = n - D;
    const int h = rel / (R2 > 0 ? R2 : 1);
    const int jj = (rel - h * R2) >> 1, comp = rel & 1;
    const bool colok = rel < NR;
    const int p = load_pair(a.pair_idx, colok ? h * r + jj : 0, half);
    // the 16 rows' table entries in one round of loads (clamped in-bounds indices, no branch: a load
    // under the store's condition would be waited for before the next one is issued)
    float cst[16], snt[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int ml = wm * C::WM + I * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      const size_t t = (size_t)(m0 + ml < M ? poss[ml] : 0) * half + p;
      cst[e] = a.rope_cos[t];
      snt[e] = a.rope_sin[t];
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float partner = shfl_xor(v[e], 1);
      const int ml = wm * C::WM + I * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (m0 + ml < M && colok) {
        const float cs = cst[e], sn = snt[e];
        const float x0 = comp ? partner : v[e], x1 = comp ? v[e] : partner;
        const float o = comp ? (x0 * sn + x1 * cs) : (x0 * cs - x1 * sn);
        ((bf16*)a.krope)[(size_t)rows[ml] * NR + rel] = (bf16)o;
      }
    }
  }
}
// All blocks, unrolled at compile time (the accumulators stay in registers).
template <class C, int I, int J>
__device__ __forceinline__ void append_gemm_blocks(const AppendArgs& a, f32x16 (&acc)[C::FM][C::FN],
                                                   const int* rows, const int* poss, int m0, int n0, int M) {
  append_gemm_block<C, I, J>(a, acc[I][J], rows, poss, m0, n0, M);
  if constexpr (J + 1 < C::FN) {
    append_gemm_blocks<C, I, J + 1>(a, acc, rows, poss, m0, n0, M);
  } else if constexpr (I + 1 < C::FM) {
    append_gemm_blocks<C, I + 1, 0>(a, acc, rows, poss, m0, n0, M);
  }
}

// ------------------------------------------------------------------ MFMA path for long prompts (bf16)
// Tiles of 256 tokens x 192 output columns through the shared GEMM main loop (gemm.h, four stages,
// one workgroup of eight waves per CU, a K loop over the whole model width); the tokens' cache rows and
// positions are resolved once per tile.  Same epilogue as the 128 x 128 path.
template <class C>
__global__ __launch_bounds__(C::THREADS, 1) void append_gemm_bf16(AppendArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];
  __shared__ int rows[256], poss[256];
  const int K = a.s.d_model, D = a.s.d_kv, NR = a.s.n_rope_cols(), N = D + NR;
  const int M = a.batch * a.t_new;
  const int n_tiles = (N + 191) / 192;
  const int total = gridDim.x;
  int bid = blockIdx.x;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int m0 = (bid / n_tiles) * 256, n0 = (bid % n_tiles) * 192;  // consecutive tiles share tokens
  const int tid = threadIdx.x;
  if (tid < 256 && m0 + tid < M) {
    int pos;
    rows[tid] = cache_row(a, m0 + tid, &pos);
    poss[tid] = pos;
  }
  __syncthreads();
  const bf16* x = (const bf16*)a.x;
  auto a_row = [&](int i) { return x + (size_t)min(m0 + i, M - 1) * K; };
  auto b_row = [&](int i) {
    const int n = min(n0 + i, N - 1);
    return n < D ? (const bf16*)a.w_dkv + (size_t)n * K : (const bf16*)a.w_krope + (size_t)(n - D) * K;
  };
  f32x16 acc[C::FM][C::FN];
  gemm_tile_cfg<C>(lds, K, a_row, b_row, acc);
  append_gemm_blocks<C, 0, 0>(a, acc, rows, poss, m0, n0, M);
}

// ------------------------------------------------------------------ MFMA path for few tokens (decode steps)
// M = batch * t_new <= 64 tokens: the GEMM is a weight read.  One workgroup per 32 output columns,
// 8 waves splitting the model width, MFMA 32x32x16 on up to two 32-token blocks, partial sums reduced
// in LDS, then the same epilogues as the large path (RoPE pairs, int4 groups of 32 columns).
constexpr int SM_WAVES = 8;

__global__ __launch_bounds__(512, 1) void append_small_bf16(AppendArgs a) {
  __shared__ float red[SM_WAVES][SM_MAXM][32];
  __shared__ float fin[SM_MAXM][33];
  __shared__ int rows[SM_MAXM], poss[SM_MAXM];
  const int K = a.s.d_model, D = a.s.d_kv, NR = a.s.n_rope_cols(), N = D + NR;
  const int M = a.batch * a.t_new;
  const int MB = (M + 31) / 32;
  const int n0 = blockIdx.x * 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int kw = K / SM_WAVES, k0 = w * kw;
  if (threadIdx.x < M) {  // cache row and position of every token, resolved once
    int pos;
    rows[threadIdx.x] = cache_row(a, threadIdx.x, &pos);
    poss[threadIdx.x] = pos;
  }
  const bf16* x = (const bf16*)a.x;
  const int gn = n0 + (lane & 31);
  const bf16* wrow = gn < D ? (const bf16*)a.w_dkv + (size_t)gn * K : (const bf16*)a.w_krope + (size_t)(gn - D) * K;
  const bool nok = gn < N;
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  const bf16x8 zero8 = {};
  // the wave's slice of the model width in batches of 8 K-steps (128 wide); every load of a batch is
  // issued before its MFMAs, and the next batch's loads before this batch's MFMAs
  constexpr int SB = 8;
  bf16x8 bv[2][SB], a0[2][SB];
  auto load_batch = [&](int st, int k) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int kk = k + 16 * u + 8 * (lane >> 5);
      const bool kin = k + 16 * u < k0 + kw;
      bv[st][u] = (nok && kin) ? *(const bf16x8*)(wrow + kk) : zero8;
      a0[st][u] = ((lane & 31) < M && kin) ? *(const bf16x8*)(x + (size_t)(lane & 31) * K + kk) : zero8;
    }
  };
  auto mma_batch = [&](int st, int k) {
#pragma unroll
    for (int u = 0; u < SB; ++u) acc[0] = mfma32(a0[st][u], bv[st][u], acc[0]);
    if (MB > 1) {  // second block of 32 tokens: its activations are read as they are used
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int kk = k + 16 * u + 8 * (lane >> 5);
        const int m1 = 32 + (lane & 31);
        bf16x8 a1 = (m1 < M && k + 16 * u < k0 + kw) ? *(const bf16x8*)(x + (size_t)m1 * K + kk) : zero8;
        acc[1] = mfma32(a1, bv[st][u], acc[1]);
      }
    }
  };
  load_batch(0, k0);
  for (int k = k0; k < k0 + kw; k += 2 * 16 * SB) {
    if (k + 16 * SB < k0 + kw) load_batch(1, k + 16 * SB);
    mma_batch(0, k);
    if (k + 16 * SB >= k0 + kw) break;
    if (k + 32 * SB < k0 + kw) load_batch(0, k + 32 * SB);
    mma_batch(1, k + 16 * SB);
  }
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[w][mb * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)][lane & 31] = acc[mb][e];
  __syncthreads();
  for (int idx = threadIdx.x; idx < MB * 32 * 32; idx += blockDim.x) {
    int m = idx >> 5, c = idx & 31;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < SM_WAVES; ++ww) v += red[ww][m][c];
    fin[m][c] = v;
  }
  __syncthreads();
  append_epilogue(a, &fin[0][0], 33, rows, poss, n0, M);
}

// ------------------------------------------------------------------ few tokens with a workspace
// Phase 1: workgroup (32 output columns, one of KS slices of the model width); 4 waves split the
// slice, MFMA 32x32x16 on up to two 32-token blocks, partial sums of the slice -> workspace (fp32,
// [KS][M][N]).  Phase 2: one workgroup of 1024 threads per 32 columns sums the KS partials (one
// output element per thread, all KS loads in one round) and runs the epilogue.

__global__ __launch_bounds__(256) void append_splitk_bf16(AppendArgs a, int KS) {
  __shared__ SplitKLds sm;
  append_splitk_tile(a, KS, blockIdx.x, blockIdx.y, sm);
}

__global__ __launch_bounds__(1024) void append_reduce(AppendArgs a, int KS) {
  __shared__ float fin[SM_MAXM][33];
  __shared__ int rows[SM_MAXM], poss[SM_MAXM];
  const int D = a.s.d_kv, N = D + a.s.n_rope_cols();
  const int M = a.batch * a.t_new;
  const int n0 = blockIdx.x * 32;
  if (threadIdx.x < M) {
    int pos;
    rows[threadIdx.x] = cache_row(a, threadIdx.x, &pos);
    poss[threadIdx.x] = pos;
  }
  const float* part = (const float*)a.ws;
  for (int idx = threadIdx.x; idx < M * 32; idx += blockDim.x) {
    const int m = idx >> 5, c = idx & 31;
    float v[KS_MAX];
#pragma unroll
    for (int ks = 0; ks < KS_MAX; ++ks) v[ks] = (ks < KS && n0 + c < N) ? part[((size_t)ks * M + m) * N + n0 + c] : 0.f;
    float sum = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS_MAX; ++ks) sum += v[ks];
    fin[m][c] = sum;
  }
  __syncthreads();
  append_epilogue(a, &fin[0][0], 33, rows, poss, n0, M);
}

// ------------------------------------------------------------------ standalone int4 quantiser
__global__ __launch_bounds__(256) void quantize_int4_kernel(const float* in, int64_t n_groups, uint8_t* codes,
                                                            uint16_t* scales) {
  int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_groups) return;
  const float* x = in + g * 32;
  float v[32];
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = x[i];
    am = fmaxf(am, fabsf(v[i]));
  }
  __half s = int4_scale(am);
  float sf = __half2float(s);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int c0 = int4_code(v[2 * i], sf), c1 = int4_code(v[2 * i + 1], sf);
    codes[g * 16 + i] = (uint8_t)((c0 & 15) | ((c1 & 15) << 4));
  }
  scales[g] = __half_as_ushort(s);
}

// ------------------------------------------------------------------ standalone 2-bit quantiser
__global__ __launch_bounds__(256) void quantize_int2_kernel(const float* in, int64_t n_groups, uint8_t* codes,
                                                            uint16_t* meta) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_groups) return;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = in[g * 32 + i];
  code_group2(v, codes + g * 8, (uint32_t*)meta + g);
}

}  // namespace

bool append_uses_mfma(const Shape& s) {
  return s.dtype == 1 && s.d_model % TK == 0 && s.d_kv % 32 == 0;
}

int append_ksplit(const Shape& s, int tokens) {
  if (!append_uses_mfma(s) || tokens > SM_MAXM || tokens <= 0) return 0;
  // as many model-width slices as possible (<= KS_MAX), each 4 waves x <= 8 K-steps of 16 (<= 512 wide)
  for (int ks = KS_MAX; ks >= 1; ks /= 2)
    if (s.d_model % (ks * 64) == 0 && s.d_model / ks <= 512) return ks;
  return 0;
}

size_t append_workspace_bytes(const Shape& s, int tokens) {
  const int ks = append_ksplit(s, tokens);
  return ks ? (size_t)ks * tokens * (s.d_kv + s.n_rope_cols()) * sizeof(float) : 0;
}


bool append_fits(const Shape& s) {
  return append_uses_mfma(s) || (size_t)(s.d_model + s.d_kv + s.n_rope_cols()) * sizeof(float) <= 65536;
}

hipError_t launch_append_reduce(const AppendArgs& a, int ks, hipStream_t st) {
  const int N = a.s.d_kv + a.s.n_rope_cols();
  hipLaunchKernelGGL(append_reduce, dim3((N + 31) / 32), dim3(1024), 0, st, a, ks);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  const int M = a.batch * a.t_new;
  const int N = a.s.d_kv + a.s.n_rope_cols();
  const int ks = a.ws ? append_ksplit(a.s, M) : 0;
  if (ks > 0) {
    hipLaunchKernelGGL(append_splitk_bf16, dim3((N + 31) / 32, ks), dim3(256), 0, st, a, ks);
    hipLaunchKernelGGL(append_reduce, dim3((N + 31) / 32), dim3(1024), 0, st, a, ks);
  } else if (append_uses_mfma(a.s) && M <= SM_MAXM && a.s.d_model % (SM_WAVES * 16) == 0) {
    hipLaunchKernelGGL(append_small_bf16, dim3((N + 31) / 32), dim3(SM_WAVES * 64), 0, st, a);
  } else if (append_uses_mfma(a.s) && a.s.d_model % 32 == 0 && ((M + 255) / 256) * ((N + 191) / 192) >= 192) {
    // long prompts: enough 256 x 192 tiles to fill most CUs
    const int grid = ((M + 255) / 256) * ((N + 191) / 192);
    hipLaunchKernelGGL(append_gemm_bf16<AppCfg8>, dim3(grid), dim3(AppCfg8::THREADS), 0, st, a);
  } else if (append_uses_mfma(a.s)) {
    int grid = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
    hipLaunchKernelGGL(append_mfma_bf16, dim3(grid), dim3(256), 0, st, a);
  } else {
    size_t shmem = (size_t)(a.s.d_model + N) * sizeof(float);
    if (a.s.dtype == 0)
      hipLaunchKernelGGL(append_generic<float>, dim3(M), dim3(256), shmem, st, a);
    else
      hipLaunchKernelGGL(append_generic<bf16>, dim3(M), dim3(256), shmem, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_int4(const float* in, int64_t n_groups, uint8_t* codes, uint16_t* scales, hipStream_t st) {
  int64_t blocks = (n_groups + 255) / 256;
  hipLaunchKernelGGL(quantize_int4_kernel, dim3((unsigned)blocks), dim3(256), 0, st, in, n_groups, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_int2(const float* in, int64_t n_groups, uint8_t* codes, uint16_t* meta, hipStream_t st) {
  const int64_t blocks = (n_groups + 255) / 256;
  hipLaunchKernelGGL(quantize_int2_kernel, dim3((unsigned)blocks), dim3(256), 0, st, in, n_groups, codes, meta);
  return hipGetLastError();
}

}  // namespace mla
