// Causal prefill over the latent cache on gfx950 (unabsorbed form).
//
// The MHA2MLA key-designs section (Paper-Notes ACL2025 page, 关键设计) recovers K_nope and V of head h
// from the latent: K_nope = c_kv . W_uk,h and V = c_kv . W_uv,h, with the retained RoPE keys cached
// separately.  For a whole prompt the minimum-work form rebuilds K and V once per token and runs plain
// causal attention with d_h = 128:
//   1. reconstruction GEMMs (MFMA):  K^[b,h,t, 0:dn] = c_kv[b,t] . W_uk,h        (dn = d_h - 2r)
//                                     V^T[b,h, :, t] = W_uv,h^T . c_kv[b,t]      (stored transposed)
//   2. causal flash attention (MFMA): head dims in the order [nope(h) | rope(h)], so the key row is
//      K^ followed by the cache's k_rope (already rotated) and the query row is q[nope(h)] followed by
//      the rotated retained pairs; q . k is unchanged by applying the same permutation to both.
#include <hip/hip_fp16.h>

#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

// ------------------------------------------------------------------ 1. reconstruction GEMM
// out = A . B^T over the latent width, tile 128 x 128, K step 64, 4 waves of 64 x 64.
//   MODE 0: A = latent rows of the cache (token m = (b, t)), B = W_uk rows (n = h*dn + i) -> K^
//   MODE 1: A = W_uv rows (m = h*d_h + e), B = latent rows (token n = (b, t))             -> V^T
constexpr int GT = 128, GK = 64, GP = GK + 8;

template <int MODE>
__global__ __launch_bounds__(256, 2) void rec_gemm(PrefillArgs a, int M, int N) {
  __shared__ __attribute__((aligned(16))) bf16 sA[2][GT * GP];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][GT * GP];
  const int K = a.s.d_kv, S = a.seq_len, dn = a.s.d_nope(), dh = a.s.d_head, NH = a.s.n_heads;
  const int n_tiles = (N + GT - 1) / GT;
  const int total = gridDim.x;
  int bid = blockIdx.x;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int m0 = (bid / n_tiles) * GT, n0 = (bid % n_tiles) * GT;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const bf16* ckv = (const bf16*)a.ckv;
  const bf16* wmat = MODE == 0 ? (const bf16*)a.w_uk : (const bf16*)a.w_uv;

  auto latent_row = [&](int tok) -> const bf16* {
    int b = tok / S, t = tok - b * S;
    return ckv + ((size_t)b * a.t_max + t) * K;
  };
  auto a_row = [&](int m) -> const bf16* { return MODE == 0 ? latent_row(m) : wmat + (size_t)m * K; };
  auto b_row = [&](int n) -> const bf16* { return MODE == 0 ? wmat + (size_t)n * K : latent_row(n); };

  bf16x8 ra[4], rb[4];
  const bf16x8 zero8 = {};
  auto gload = [&](int kt) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      int c = it * 256 + tid, row = c >> 3, kc = (c & 7) * 8;
      int gm = m0 + row, gn = n0 + row;
      ra[it] = gm < M ? *(const bf16x8*)(a_row(gm) + kt * GK + kc) : zero8;
      rb[it] = gn < N ? *(const bf16x8*)(b_row(gn) + kt * GK + kc) : zero8;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      int c = it * 256 + tid, row = c >> 3, kc = (c & 7) * 8;
      *(bf16x8*)&sA[buf][row * GP + kc] = ra[it];
      *(bf16x8*)&sB[buf][row * GP + kc] = rb[it];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int KT = K / GK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *(const bf16x8*)&sA[buf][(wm * 64 + i * 32 + (lane & 31)) * GP + ks * 16 + (lane >> 5) * 8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bv[j] = *(const bf16x8*)&sB[buf][(wn * 64 + j * 32 + (lane & 31)) * GP + ks * 16 + (lane >> 5) * 8];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(av[i], bv[j], acc[i][j]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }
  bf16* outk = (bf16*)(a.ws + a.plan.off_k);
  bf16* outv = (bf16*)(a.ws + a.plan.off_vt);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m >= M) continue;
        const bf16 v = (bf16)acc[i][j][e];
        if (MODE == 0) {
          int b = m / S, t = m - b * S, h = n / dn, ii = n - h * dn;
          outk[(((size_t)b * NH + h) * S + t) * dn + ii] = v;
        } else {
          int h = m / dh, e2 = m - h * dh, b = n / S, t = n - b * S;
          outv[(((size_t)b * NH + h) * dh + e2) * S + t] = v;
        }
      }
    }
}

// ------------------------------------------------------------------ 2. causal flash attention, d_h = 128
// Workgroup = (query tile of 128 rows, head, sequence); 4 waves of 32 query rows; key tiles of 64.
//   S^T[key][q] = K^[key] . Q^[q]      MFMA 32x32x16, A = key rows (LDS), B = query rows (registers):
//                                       lane l owns query l%32, so row max / sum stay in the lane
//                                       plus one cross-half shuffle
//   O^T[e][q]  += V^T[e][key] P[q][key] MFMA 32x32x16, A = V^T rows (LDS), B = P from the score
//                                       registers; within every 16 keys the V^T tile stores keys in
//                                       the order the score layout hands them out
// Query tiles are scheduled longest first (causal work grows with the tile index).
constexpr int FQ = 128, FKV = 64, KP = 128 + 8, VP = FKV + 8;

__global__ __launch_bounds__(256, 2) void prefill_attn(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 ks[2][FKV * KP];
  __shared__ __attribute__((aligned(16))) bf16 vs[2][128 * VP];
  __shared__ int nope_idx[128];
  __shared__ int pairs[64];
  const int S = a.seq_len, NH = a.s.n_heads, dn = a.s.d_nope(), r = a.s.r_pairs, R2 = a.s.r2(), half = 64;
  const int nqt = (S + FQ - 1) / FQ;
  const int qt = nqt - 1 - (int)blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int q0 = qt * FQ;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hb = lane >> 5, ql = lane & 31;
  const int myq = q0 + 32 * w + ql;

  if (tid == 0) {
    int n = 0;
    for (int j = 0; j < r; ++j) pairs[j] = load_pair(a.pair_idx, h * r + j, half);
    for (int i = 0; i < half; ++i) {
      bool kept = false;
      for (int j = 0; j < r; ++j) kept |= (pairs[j] == i);
      if (!kept) {
        nope_idx[n++] = 2 * i;
        nope_idx[n++] = 2 * i + 1;
      }
    }
  }
  // ---- stage the raw query rows of the tile in LDS (reusing the key buffers)
  bf16* qs = &ks[0][0];  // [128][128], 32 KB
  const bf16* qg = (const bf16*)a.q;
  for (int c = tid; c < FQ * 16; c += 256) {
    int row = c >> 4, ch = c & 15;
    int t = min(q0 + row, S - 1);
    *(uint4*)&qs[row * 128 + ch * 8] = *(const uint4*)(qg + (((size_t)b * S + t) * NH + h) * 128 + ch * 8);
  }
  __syncthreads();
  // ---- query operands: dims [nope(h) | rotated retained pairs], scaled by log2(e)/sqrt(d_h)
  const float scale = kLog2e / sqrtf(128.f);
  bf16x8 qv[8];
  {
    const bf16* qrow = qs + (32 * w + ql) * 128;
    const int pos = min(myq, S - 1);
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = 16 * s8 + 8 * hb + u;
        float v;
        if (e < dn) {
          v = (float)qrow[nope_idx[e]];
        } else {
          const int j = (e - dn) >> 1, c = (e - dn) & 1;
          const int p = pairs[j];
          const float x0 = (float)qrow[2 * p], x1 = (float)qrow[2 * p + 1];
          const float cs = a.rope_cos[(size_t)pos * half + p], sn = a.rope_sin[(size_t)pos * half + p];
          v = c ? (x0 * sn + x1 * cs) : (x0 * cs - x1 * sn);
        }
        qv[s8][u] = (bf16)(v * scale);
      }
    }
  }
  __syncthreads();

  const bf16* khat = (const bf16*)(a.ws + a.plan.off_k) + ((size_t)b * NH + h) * S * dn;
  const bf16* vt = (const bf16*)(a.ws + a.plan.off_vt) + ((size_t)b * NH + h) * 128 * S;
  const bf16* kr = (const bf16*)a.krope;
  const int nkc = dn / 8;  // 16-byte chunks of a key row that come from K^
  const int n_kv = min((S + FKV - 1) / FKV, (q0 + FQ - 1) / FKV + 1);

  u32x4 kreg[4], vreg[2][2];
  // every load of a thread reads the same 16-byte column chunk: from K^ (nope dims) or from k_rope
  const int kch = tid & 15;
  const bool from_rope = kch >= nkc;
  const bf16* kbase = from_rope ? kr + (size_t)h * R2 + (kch - nkc) * 8 : khat + kch * 8;
  const size_t krow_stride = from_rope ? (size_t)NH * R2 : (size_t)dn;
  const size_t kseq_off = from_rope ? (size_t)b * a.t_max * NH * R2 : 0;
  auto gload = [&](int kv0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      int t = min(kv0 + it * 16 + (tid >> 4), S - 1);
      kreg[it] = *(const u32x4*)(kbase + kseq_off + (size_t)t * krow_stride);
    }
    if (kv0 + FKV <= S) {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        int pidx = it * 256 + tid, row = pidx >> 2, g = pidx & 3;
        const bf16* src = vt + (size_t)row * S + kv0 + 16 * g;
        vreg[it][0] = *(const u32x4*)(src);
        vreg[it][1] = *(const u32x4*)(src + 8);
      }
    } else {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        int pidx = it * 256 + tid, row = pidx >> 2, g = pidx & 3;
        int k0 = kv0 + 16 * g;
        const bf16* src = vt + (size_t)row * S;
        bf16x8 lo, hi;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          lo[u] = k0 + u < S ? src[k0 + u] : (bf16)0.f;
          hi[u] = k0 + 8 + u < S ? src[k0 + 8 + u] : (bf16)0.f;
        }
        vreg[it][0] = __builtin_bit_cast(u32x4, lo);
        vreg[it][1] = __builtin_bit_cast(u32x4, hi);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      int c = it * 256 + tid, row = c >> 4, ch = c & 15;
      *(u32x4*)&ks[buf][row * KP + ch * 8] = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      int pidx = it * 256 + tid, row = pidx >> 2, g = pidx & 3;
      // keys 16g + {0..3, 8..11} first, then {4..7, 12..15}
      u32x4 x = vreg[it][0], y = vreg[it][1];
      *(u32x4*)&vs[buf][row * VP + 16 * g] = u32x4{x.x, x.y, y.x, y.y};
      *(u32x4*)&vs[buf][row * VP + 16 * g + 8] = u32x4{x.z, x.w, y.z, y.w};
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int wq_lo = q0 + 32 * w, wq_hi = wq_lo + 31;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int it = 0; it < n_kv; ++it) {
    const int buf = it & 1, kv0 = it * FKV;
    if (it + 1 < n_kv) gload(kv0 + FKV);
    if (kv0 <= wq_hi) {  // wave-uniform: some key of the tile is visible to some row of the wave
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          bf16x8 av = *(const bf16x8*)&ks[buf][(kb * 32 + ql) * KP + 16 * s8 + 8 * hb];
          sacc[kb] = mfma32(av, qv[s8], sacc[kb]);
        }
      }
      const bool need_mask = kv0 + FKV - 1 > wq_lo || kv0 + FKV > S;
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (need_mask) {
            int key = kv0 + kb * 32 + 8 * (e >> 2) + 4 * hb + (e & 3);
            if (key > myq || key >= S) sacc[kb][e] = -INFINITY;
          }
          mt = fmaxf(mt, sacc[kb][e]);
        }
      mt = fmaxf(mt, shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      const float alpha = exp2f(m_run - m_new);
      float rs = 0.f;
      bf16x8 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float p = exp2f(sacc[kb][e] - m_new);
          rs += p;
          pb[kb][e >> 3][e & 7] = (bf16)p;
        }
      rs += shfl_xor(rs, 32);
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        oacc[db] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            bf16x8 av = *(const bf16x8*)&vs[buf][(db * 32 + ql) * VP + kb * 32 + 16 * c + 8 * hb];
            oacc[db] = mfma32(av, pb[kb][c], oacc[db]);
          }
      }
    }
    if (it + 1 < n_kv) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store through LDS (rows of 128 output dims, 16-byte stores)
  const float inv = 1.f / l_run;
  bf16* os = &ks[0][0] + w * 32 * KP;  // [32][KP] per wave
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) os[ql * KP + db * 32 + 8 * (e >> 2) + 4 * hb + (e & 3)] = (bf16)(oacc[db][e] * inv);
  __builtin_amdgcn_wave_barrier();
  __syncthreads();
  bf16* og = (bf16*)a.out;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int c = i * 64 + lane, row = c >> 4, ch = c & 15;
    int t = q0 + 32 * w + row;
    if (t < S) *(uint4*)(og + (((size_t)b * S + t) * NH + h) * 128 + ch * 8) = *(const uint4*)&os[row * KP + ch * 8];
  }
}

}  // namespace

bool prefill_supported(const Shape& s) {
  return s.dtype == 1 && s.fmt == 0 && s.d_head == 128 && (s.r2() % 8) == 0 && s.d_kv % GK == 0;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

PrefillPlan plan_prefill(const Shape& s, int batch, int seq_len) {
  PrefillPlan p{};
  size_t off = 0;
  p.off_k = off;
  off = align256(off + (size_t)batch * s.n_heads * seq_len * s.d_nope() * 2);
  p.off_vt = off;
  off = align256(off + (size_t)batch * s.n_heads * s.d_head * seq_len * 2);
  p.off_q = off;
  p.total = off;
  return p;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  const int S = a.seq_len, B = a.batch, NH = a.s.n_heads;
  {
    const int M = B * S, N = NH * a.s.d_nope();
    if (N > 0) {
      int grid = ((M + GT - 1) / GT) * ((N + GT - 1) / GT);
      hipLaunchKernelGGL(rec_gemm<0>, dim3(grid), dim3(256), 0, st, a, M, N);
    }
  }
  {
    const int M = NH * a.s.d_head, N = B * S;
    int grid = ((M + GT - 1) / GT) * ((N + GT - 1) / GT);
    hipLaunchKernelGGL(rec_gemm<1>, dim3(grid), dim3(256), 0, st, a, M, N);
  }
  dim3 g((S + FQ - 1) / FQ, NH, B);
  hipLaunchKernelGGL(prefill_attn, g, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
