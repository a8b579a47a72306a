// Decode over the latent cache on gfx950 (absorbed form).
//
// Per the MHA2MLA key-designs section (Paper-Notes ACL2025 page, 关键设计): K_nope of head h is
// c_kv . W_uk,h and V is c_kv . W_uv,h, while the retained RoPE keys are cached separately.  So
//   score(h, n) = q_nope,h . (c_n W_uk,h) + q_rope,h . k_rope(n, h) = (W_uk,h q_nope,h) . c_n + ...
// and the head output is (sum_n p_n c_n) . W_uv,h.  Three launches:
//   1. qprep:   q~ = W_uk,h q_nope (latent query) and the rotated retained query pairs, both scaled by
//               log2(e)/sqrt(d_h) so the softmax runs on exp2;
//   2. attn:    split-K over each sequence's tokens; per 32-token tile the latent rows are staged in LDS
//               once and used by all heads for both products (scores and p . c); running max / sum per
//               head (online softmax); partial (m, l, o) per split in the workspace;
//   3. combine: merges the splits and applies W_uv,h.
#include <hip/hip_fp16.h>

#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int QB = 16;     // batch rows per qprep workgroup
constexpr int CB = 8;      // batch rows per combine workgroup
constexpr int MAX_DH = 256;

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int b) {
  int L = a.seq_lens[b];
  return L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
}

// ------------------------------------------------------------------ 1. query preparation
// Workgroup (head h, 64 latent columns, up to QB batch rows): the 4 waves split the NoPE dims, each
// lane owns one latent column, and the partial sums meet in LDS.  Workgroups with blockIdx.y == 0
// also rotate the retained query pairs.
template <typename T>
__global__ __launch_bounds__(256) void decode_qprep(DecodeArgs a) {
  const int h = blockIdx.x, k = blockIdx.y * 64 + (threadIdx.x & 63), b0 = blockIdx.z * QB;
  const int ty = threadIdx.x >> 6;
  const int D = a.s.d_kv, dh = a.s.d_head, r = a.s.r_pairs, dn = a.s.d_nope(), half = dh / 2, NH = a.s.n_heads;
  __shared__ int nope_idx[MAX_DH];
  __shared__ float qn[MAX_DH][QB];
  __shared__ float red[4][QB][64];
  if (threadIdx.x == 0) {
    int n = 0;
    for (int i = 0; i < half; ++i) {
      bool kept = false;
      for (int j = 0; j < r; ++j) kept |= (load_pair(a.pair_idx, h * r + j, half) == i);
      if (!kept) {
        nope_idx[n++] = 2 * i;
        nope_idx[n++] = 2 * i + 1;
      }
    }
  }
  __syncthreads();
  const T* q = (const T*)a.q;
  for (int idx = threadIdx.x; idx < QB * dn; idx += blockDim.x) {
    int bb = idx / dn, i = idx - bb * dn, b = b0 + bb;
    qn[i][bb] = b < a.batch ? to_f32(q[((size_t)b * NH + h) * dh + nope_idx[i]]) : 0.f;
  }
  __syncthreads();
  float acc[QB];
#pragma unroll
  for (int bb = 0; bb < QB; ++bb) acc[bb] = 0.f;
  const int per = (dn + 3) / 4, i0 = ty * per, i1 = min(dn, i0 + per);
  const T* wuk = (const T*)a.w_uk + (size_t)h * dn * D + k;
  if (k < D) {
    int i = i0;
    for (; i + 4 <= i1; i += 4) {
      float wv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) wv[u] = to_f32(wuk[(size_t)(i + u) * D]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int bb = 0; bb < QB; ++bb) acc[bb] = fmaf(wv[u], qn[i + u][bb], acc[bb]);
    }
    for (; i < i1; ++i) {
      float wv = to_f32(wuk[(size_t)i * D]);
#pragma unroll
      for (int bb = 0; bb < QB; ++bb) acc[bb] = fmaf(wv, qn[i][bb], acc[bb]);
    }
  }
#pragma unroll
  for (int bb = 0; bb < QB; ++bb) red[ty][bb][threadIdx.x & 63] = acc[bb];
  __syncthreads();
  const float scale = kLog2e / sqrtf((float)dh);
  T* qt = (T*)(a.ws + a.plan.off_qt);
  for (int idx = threadIdx.x; idx < QB * 64; idx += blockDim.x) {
    int bb = idx >> 6, kk = idx & 63, b = b0 + bb, kc = blockIdx.y * 64 + kk;
    if (b < a.batch && kc < D) {
      float v = red[0][bb][kk] + red[1][bb][kk] + red[2][bb][kk] + red[3][bb][kk];
      qt[((size_t)b * NH + h) * D + kc] = from_f32<T>(v * scale);
    }
  }
  if (blockIdx.y != 0) return;
  float* qr = (float*)(a.ws + a.plan.off_qr);
  for (int idx = threadIdx.x; idx < QB * r; idx += blockDim.x) {
    int bb = idx / r, j = idx - bb * r, b = b0 + bb;
    if (b >= a.batch) continue;
    int L = clamp_len(a, b);
    int pos = L > 0 ? L - 1 : 0;
    int p = load_pair(a.pair_idx, h * r + j, half);
    float x0 = to_f32(q[((size_t)b * NH + h) * dh + 2 * p]), x1 = to_f32(q[((size_t)b * NH + h) * dh + 2 * p + 1]);
    float c = a.rope_cos[(size_t)pos * half + p], s = a.rope_sin[(size_t)pos * half + p];
    qr[((size_t)b * NH + h) * 2 * r + 2 * j] = (x0 * c - x1 * s) * scale;
    qr[((size_t)b * NH + h) * 2 * r + 2 * j + 1] = (x0 * s + x1 * c) * scale;
  }
}

// ------------------------------------------------------------------ latent element access
template <typename T, int FMT>
__device__ __forceinline__ float latent(const DecodeArgs& a, size_t row, int k) {
  const int D = a.s.d_kv;
  if (FMT == 0) return to_f32(((const T*)a.ckv)[row * D + k]);
  uint32_t byte = ((const uint8_t*)a.ckv)[row * (D / 2) + (k >> 1)];
  float s = __half2float(((const __half*)a.ckv_scale)[row * (D / 32) + (k >> 5)]);
  return int4_dequant(nibble(byte, k & 1), s);
}

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

// ------------------------------------------------------------------ 2a. attention, generic VALU path
template <typename T, int FMT>
__global__ __launch_bounds__(256) void decode_attn_generic(DecodeArgs a) {
  const int split = blockIdx.x, b = blockIdx.y;
  const int D = a.s.d_kv, NH = a.s.n_heads, R2 = a.s.r2(), S = a.plan.n_splits;
  const int L = clamp_len(a, b);
  const int t0 = split * a.plan.chunk;
  const int n = min(t0 + a.plan.chunk, L) - t0;
  extern __shared__ float sh[];
  float* qs = sh;              // D
  float* qrs = qs + D;         // R2
  float* sc = qrs + R2 + 1;    // chunk
  __shared__ float red[8];
  float* ml = (float*)(a.ws + a.plan.off_ml) + ((size_t)b * S + split) * NH * 2;
  float* po = (float*)(a.ws + a.plan.off_o) + ((size_t)b * S + split) * NH * D;
  const T* qt = (const T*)(a.ws + a.plan.off_qt) + (size_t)b * NH * D;
  const float* qr = (const float*)(a.ws + a.plan.off_qr) + (size_t)b * NH * R2;
  const size_t row0 = (size_t)b * a.t_max + t0;
  for (int h = 0; h < NH; ++h) {
    if (n <= 0) {
      for (int k = threadIdx.x; k < D; k += blockDim.x) po[(size_t)h * D + k] = 0.f;
      if (threadIdx.x == 0) {
        ml[2 * h] = -INFINITY;
        ml[2 * h + 1] = 0.f;
      }
      continue;
    }
    for (int k = threadIdx.x; k < D; k += blockDim.x) qs[k] = to_f32(qt[(size_t)h * D + k]);
    for (int j = threadIdx.x; j < R2; j += blockDim.x) qrs[j] = qr[h * R2 + j];
    __syncthreads();
    float mloc = -INFINITY;
    for (int t = threadIdx.x; t < n; t += blockDim.x) {
      float s = 0.f;
      for (int k = 0; k < D; ++k) s = fmaf(qs[k], latent<T, FMT>(a, row0 + t, k), s);
      const T* kr = (const T*)a.krope + ((row0 + t) * NH + h) * R2;
      for (int j = 0; j < R2; ++j) s = fmaf(qrs[j], to_f32(kr[j]), s);
      sc[t] = s;
      mloc = fmaxf(mloc, s);
    }
    const float m = block_reduce(mloc, red, true);
    float lloc = 0.f;
    for (int t = threadIdx.x; t < n; t += blockDim.x) {
      float p = exp2f(sc[t] - m);
      sc[t] = p;
      lloc += p;
    }
    const float l = block_reduce(lloc, red, false);
    __syncthreads();
    for (int k = threadIdx.x; k < D; k += blockDim.x) {
      float o = 0.f;
      for (int t = 0; t < n; ++t) o = fmaf(sc[t], latent<T, FMT>(a, row0 + t, k), o);
      po[(size_t)h * D + k] = o;
    }
    if (threadIdx.x == 0) {
      ml[2 * h] = m;
      ml[2 * h + 1] = l;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ 2b. attention, MFMA path
// 32 heads, bf16.  Four waves split the latent width: wave w owns latent columns [w*DW, (w+1)*DW)
// for both products, so each wave stages only its own slice of every 32-token tile in LDS.
//   scores   S^T[n][h] = sum_k C[n][k] q~[h][k]      MFMA 32x32x16, A = C rows (ds_read_b128),
//                                                     B = q~ (registers); partial over the wave's
//                                                     columns, summed across waves through LDS
//   output   O^T[k][h] += sum_n C[n][k] P[h][n]      MFMA 32x32x16, A = C^T through the LDS
//                                                     transpose read, B = P straight from the
//                                                     score registers (same lane -> head mapping)
// Lane l owns head l%32 in both products, so the per-head max / sum / rescale stay in registers
// (one cross-half shuffle).  The next tile's rows and RoPE keys are prefetched into registers.  The
// dense 512-wide variant needs more than 256 registers per lane and runs at one wave per SIMD.
template <int DW, int R2, int FMT>
__global__ __launch_bounds__(256, (DW == 128 && FMT == 0) ? 1 : 2) void decode_attn_mfma(DecodeArgs a) {
  constexpr int CP = DW + 16;  // LDS row pitch in elements (conflict-free b128 and transpose reads)
  constexpr int NS = DW / 16;  // score k-steps per wave
  constexpr int NB = DW / 32;  // output blocks per wave
  constexpr int D = 4 * DW;
  __shared__ __attribute__((aligned(16))) bf16 cbuf[4][32 * CP];
  __shared__ f32x4 sbuf[2][4][4][64];

  const int split = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hb = lane >> 5, h = lane & 31;
  const int S = a.plan.n_splits;
  const int L = clamp_len(a, b);
  const int t0 = split * a.plan.chunk;
  const int t1 = min(t0 + a.plan.chunk, L);
  float* pml = (float*)(a.ws + a.plan.off_ml) + ((size_t)b * S + split) * 32 * 2;
  float* po = (float*)(a.ws + a.plan.off_o) + ((size_t)b * S + split) * 32 * D;

  if (t0 >= t1) {
    for (int idx = lane; idx < 32 * DW / 4; idx += 64) {
      int hh = idx / (DW / 4), c4 = idx - hh * (DW / 4);
      *(f32x4*)&po[(size_t)hh * D + w * DW + 4 * c4] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (w == 0 && lane < 32) {
      pml[2 * lane] = -INFINITY;
      pml[2 * lane + 1] = 0.f;
    }
    return;
  }

  // latent query operands (B of the score product) and the rotated query pairs
  const bf16* qt = (const bf16*)(a.ws + a.plan.off_qt) + ((size_t)b * 32 + h) * D + w * DW + 8 * hb;
  bf16x8 qv[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) qv[s] = *(const bf16x8*)(qt + 16 * s);
  float qr[R2];
  {
    const float* qrp = (const float*)(a.ws + a.plan.off_qr) + ((size_t)b * 32 + h) * R2;
#pragma unroll
    for (int c = 0; c < R2; ++c) qr[c] = qrp[c];
  }

  f32x16 oacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const size_t rowb = (size_t)b * a.t_max;
  const bf16* krb = (const bf16*)a.krope + rowb * 32 * R2;
  bf16* cw = cbuf[w];

  // ---- register prefetch of one tile: this wave's latent slice and its share of the RoPE keys
  constexpr int CPR = (FMT == 0) ? DW / 8 : DW / 32;  // 16-byte chunks per row
  constexpr int CCH = 32 * CPR / 64;                  // chunks per lane
  u32x4 creg[CCH];
  uint16_t sreg[CCH];
  typedef bf16 kv_t __attribute__((ext_vector_type(R2)));
  kv_t kreg[4];

  auto load_tile = [&](int tt) {
#pragma unroll
    for (int it = 0; it < CCH; ++it) {
      int c = it * 64 + lane, row = c / CPR, q = c - row * CPR;
      int tok = tt + row;
      if (tok < t1) {
        if (FMT == 0) {
          creg[it] = *(const u32x4*)((const bf16*)a.ckv + (rowb + tok) * D + w * DW + 8 * q);
        } else {
          creg[it] = *(const u32x4*)((const uint8_t*)a.ckv + (rowb + tok) * (D / 2) + (w * DW + 32 * q) / 2);
          sreg[it] = ((const uint16_t*)a.ckv_scale)[(rowb + tok) * (D / 32) + (w * DW) / 32 + q];
        }
      } else {
        creg[it] = u32x4{0u, 0u, 0u, 0u};
        sreg[it] = 0;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int tok = tt + 8 * w + 4 * hb + i;
      kreg[i] = tok < t1 ? *(const kv_t*)(krb + ((size_t)tok * 32 + h) * R2) : kv_t{};
    }
  };
  auto stage_tile = [&]() {
#pragma unroll
    for (int it = 0; it < CCH; ++it) {
      int c = it * 64 + lane, row = c / CPR, q = c - row * CPR;
      if (FMT == 0) {
        *(u32x4*)&cw[row * CP + 8 * q] = creg[it];
      } else {
        float s = __half2float(__ushort_as_half(sreg[it]));
        const uint32_t wd[4] = {creg[it].x, creg[it].y, creg[it].z, creg[it].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (bf16)int4_dequant(nibble(wd[u] >> (8 * (e >> 1)), e & 1), s);
          *(bf16x8*)&cw[row * CP + 32 * q + 8 * u] = v;
        }
      }
    }
  };

  load_tile(t0);
  int par = 0;
  for (int tt = t0; tt < t1; tt += 32, par ^= 1) {
    stage_tile();
    // RoPE term of rows 8w + 4hb + i (result elements 4w + i), taken before the registers refill
    float rt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < R2; ++c) acc = fmaf(qr[c], (float)kreg[i][c], acc);
      rt[i] = acc;
    }
    if (tt + 32 < t1) load_tile(tt + 32);
    __builtin_amdgcn_wave_barrier();

    // scores over this wave's latent columns
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8 av = *(const bf16x8*)&cw[(lane & 31) * CP + 16 * s + 8 * hb];
      sacc = mfma32(av, qv[s], sacc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (w == j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[4 * j + i] += rt[i];
      }
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4)
      sbuf[par][w][e4][lane] = f32x4{sacc[4 * e4], sacc[4 * e4 + 1], sacc[4 * e4 + 2], sacc[4 * e4 + 3]};
    __syncthreads();
    float sc[16];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      f32x4 v = sbuf[par][0][e4][lane];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) v += sbuf[par][ww][e4][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * e4 + i] = v[i];
    }
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      int n = 8 * (e >> 2) + 4 * hb + (e & 3);
      if (tt + n >= t1) sc[e] = -INFINITY;
      mt = fmaxf(mt, sc[e]);
    }
    mt = fmaxf(mt, shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    float p[16], rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = exp2f(sc[e] - m_new);
      rs += p[e];
    }
    rs += shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    bf16x8 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[c][e] = (bf16)p[8 * c + e];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      oacc[blk] *= alpha;
      const int col = blk * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row0 = 16 * c + 4 * hb + ((lane & 15) >> 2);
        bf16x4 x0 = lds_read_tr16(&cw[row0 * CP + col]);
        bf16x4 x1 = lds_read_tr16(&cw[(row0 + 8) * CP + col]);
        oacc[blk] = mfma32(cat(x0, x1), pb[c], oacc[blk]);
      }
    }
    asm volatile("" ::: "memory");
  }

#pragma unroll
  for (int blk = 0; blk < NB; ++blk)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      int k = w * DW + blk * 32 + 8 * e4 + 4 * hb;
      *(f32x4*)&po[(size_t)h * D + k] =
          f32x4{oacc[blk][4 * e4], oacc[blk][4 * e4 + 1], oacc[blk][4 * e4 + 2], oacc[blk][4 * e4 + 3]};
    }
  if (w == 0 && hb == 0) {
    pml[2 * h] = m_run;
    pml[2 * h + 1] = l_run;
  }
}

// ------------------------------------------------------------------ 3. combine + W_uv
// Workgroup (head h, CB batch rows).  Merge weights per (row, split) from the split maxima, the merged
// normalised latent output of every row in LDS, then out = o . W_uv,h^T with each thread pair sharing
// one output dim (16-byte weight loads, halves of the latent width, one shuffle).
template <typename T>
__global__ __launch_bounds__(256) void decode_combine(DecodeArgs a) {
  const int h = blockIdx.x, b0 = blockIdx.y * CB;
  const int D = a.s.d_kv, dh = a.s.d_head, NH = a.s.n_heads, S = a.plan.n_splits;
  extern __shared__ float sh[];
  float* ob = sh;                // [CB][D]
  float* wts = ob + CB * D;      // [CB][S]
  __shared__ float inv_den[CB];
  const float* ml = (const float*)(a.ws + a.plan.off_ml);
  const float* po = (const float*)(a.ws + a.plan.off_o);
  if (threadIdx.x < CB) {
    int bb = threadIdx.x, b = b0 + bb;
    float den = 0.f;
    if (b < a.batch) {
      float M = -INFINITY;
      for (int s = 0; s < S; ++s) M = fmaxf(M, ml[(((size_t)b * S + s) * NH + h) * 2]);
      for (int s = 0; s < S; ++s) {
        float ms = ml[(((size_t)b * S + s) * NH + h) * 2], ls = ml[(((size_t)b * S + s) * NH + h) * 2 + 1];
        float wv = (M == -INFINITY || ms == -INFINITY) ? 0.f : exp2f(ms - M);
        wts[bb * S + s] = wv;
        den += wv * ls;
      }
    } else {
      for (int s = 0; s < S; ++s) wts[bb * S + s] = 0.f;
    }
    inv_den[bb] = den > 0.f ? 1.f / den : 0.f;
  }
  __syncthreads();
  const size_t sstride = (size_t)NH * D;
  for (int idx = threadIdx.x; idx < CB * D; idx += blockDim.x) {
    int bb = idx / D, k = idx - bb * D, b = b0 + bb;
    float o = 0.f;
    if (b < a.batch) {
      const float* p = po + ((size_t)b * S * NH + h) * D + k;
      const float* wr = wts + bb * S;
      int s = 0;
      for (; s + 4 <= S; s += 4) {
        float v0 = p[(size_t)s * sstride], v1 = p[(size_t)(s + 1) * sstride];
        float v2 = p[(size_t)(s + 2) * sstride], v3 = p[(size_t)(s + 3) * sstride];
        o = fmaf(wr[s], v0, o);
        o = fmaf(wr[s + 1], v1, o);
        o = fmaf(wr[s + 2], v2, o);
        o = fmaf(wr[s + 3], v3, o);
      }
      for (; s < S; ++s) o = fmaf(wr[s], p[(size_t)s * sstride], o);
    }
    ob[idx] = o * inv_den[bb];
  }
  __syncthreads();
  const T* wuv = (const T*)a.w_uv + (size_t)h * dh * D;
  T* out = (T*)a.out;
  const int hk = D / 2;
  for (int e2 = threadIdx.x; e2 < 2 * dh; e2 += blockDim.x) {
    const int e = e2 >> 1, part = e2 & 1;
    const int k0 = part * hk, k1 = part ? D : hk;
    float acc[CB];
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) acc[bb] = 0.f;
    const T* wr = wuv + (size_t)e * D;
    int k = k0;
    if (sizeof(T) == 2 && (D % 16) == 0) {
      for (; k + 8 <= k1; k += 8) {
        bf16x8 wv = *(const bf16x8*)(wr + k);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          float wf = (float)wv[u];
#pragma unroll
          for (int bb = 0; bb < CB; ++bb) acc[bb] = fmaf(wf, ob[bb * D + k + u], acc[bb]);
        }
      }
    }
    for (; k < k1; ++k) {
      float wv = to_f32(wr[k]);
#pragma unroll
      for (int bb = 0; bb < CB; ++bb) acc[bb] = fmaf(wv, ob[bb * D + k], acc[bb]);
    }
#pragma unroll
    for (int bb = 0; bb < CB; ++bb) acc[bb] += __shfl_xor(acc[bb], 1, 64);
    if (part == 0) {
#pragma unroll
      for (int bb = 0; bb < CB; ++bb) {
        int b = b0 + bb;
        if (b < a.batch) out[((size_t)b * NH + h) * dh + e] = from_f32<T>(acc[bb]);
      }
    }
  }
}

template <typename T>
void launch_generic_attn(const DecodeArgs& a, hipStream_t st) {
  size_t shmem = (size_t)(a.s.d_kv + a.s.r2() + 1 + a.plan.chunk) * sizeof(float);
  dim3 grid(a.plan.n_splits, a.batch);
  if (a.s.fmt == 0)
    hipLaunchKernelGGL((decode_attn_generic<T, 0>), grid, dim3(256), shmem, st, a);
  else
    hipLaunchKernelGGL((decode_attn_generic<T, 1>), grid, dim3(256), shmem, st, a);
}

template <int DW, int R2>
void launch_mfma_attn(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.plan.n_splits, a.batch);
  if (a.s.fmt == 0)
    hipLaunchKernelGGL((decode_attn_mfma<DW, R2, 0>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_attn_mfma<DW, R2, 1>), grid, dim3(256), 0, st, a);
}

}  // namespace

bool decode_uses_mfma(const Shape& s) {
  return s.dtype == 1 && s.n_heads == 32 && (s.d_kv == 256 || s.d_kv == 512) && (s.r_pairs == 2 || s.r_pairs == 4);
}

bool decode_fits(const Shape& s, const DecodePlan& p) {
  const size_t lim = 65536;
  if ((size_t)(CB * s.d_kv + CB * p.n_splits) * sizeof(float) > lim) return false;
  if (!decode_uses_mfma(s) && (size_t)(s.d_kv + s.r2() + 1 + p.chunk) * sizeof(float) > lim) return false;
  return true;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

DecodePlan plan_decode(const Shape& s, int batch, int max_seq_len) {
  DecodePlan p{};
  const long long target_wg = 512;
  long long per = ((long long)max_seq_len * batch + target_wg - 1) / target_wg;
  int chunk = (int)(((per + 63) / 64) * 64);
  if (chunk < 64) chunk = 64;
  if (chunk > 2048) chunk = 2048;
  p.chunk = chunk;
  p.n_splits = max_seq_len > 0 ? (max_seq_len + chunk - 1) / chunk : 1;
  const size_t esz = s.dtype == 0 ? 4 : 2;
  size_t off = 0;
  p.off_qt = off;
  off = align256(off + (size_t)batch * s.n_heads * s.d_kv * esz);
  p.off_qr = off;
  off = align256(off + (size_t)batch * s.n_heads * (s.r2() > 0 ? s.r2() : 1) * 4);
  p.off_ml = off;
  off = align256(off + (size_t)batch * p.n_splits * s.n_heads * 2 * 4);
  p.off_o = off;
  off = align256(off + (size_t)batch * p.n_splits * s.n_heads * s.d_kv * 4);
  p.total = off;
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st, int phase_mask) {
  const int nh = a.s.n_heads;
  if (phase_mask & 1) {
    dim3 gq(nh, (a.s.d_kv + 63) / 64, (a.batch + QB - 1) / QB);
    if (a.s.dtype == 0)
      hipLaunchKernelGGL(decode_qprep<float>, gq, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(decode_qprep<bf16>, gq, dim3(256), 0, st, a);
  }
  if (phase_mask & 2) {
    if (decode_uses_mfma(a.s)) {
      if (a.s.d_kv == 512 && a.s.r_pairs == 4) launch_mfma_attn<128, 8>(a, st);
      else if (a.s.d_kv == 512 && a.s.r_pairs == 2) launch_mfma_attn<128, 4>(a, st);
      else if (a.s.d_kv == 256 && a.s.r_pairs == 4) launch_mfma_attn<64, 8>(a, st);
      else launch_mfma_attn<64, 4>(a, st);
    } else if (a.s.dtype == 0) {
      launch_generic_attn<float>(a, st);
    } else {
      launch_generic_attn<bf16>(a, st);
    }
  }
  if (phase_mask & 4) {
    size_t shc = (size_t)(CB * a.s.d_kv + CB * a.plan.n_splits) * sizeof(float);
    dim3 gc(nh, (a.batch + CB - 1) / CB);
    if (a.s.dtype == 0)
      hipLaunchKernelGGL(decode_combine<float>, gc, dim3(256), shc, st, a);
    else
      hipLaunchKernelGGL(decode_combine<bf16>, gc, dim3(256), shc, st, a);
  }
  return hipGetLastError();
}

}  // namespace mla
