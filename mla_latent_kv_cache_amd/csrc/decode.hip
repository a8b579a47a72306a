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

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int QB = 16;     // batch rows per qprep workgroup (QB * d_nope <= 4 * 512)
constexpr int MAX_DH = 256;

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int b) {
  int L = a.seq_lens[b];
  return L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
}

// ------------------------------------------------------------------ work split (see DecodePlan)
// Every function below is called by all 64 lanes of a wave and returns wave-uniform values.
__device__ __forceinline__ int wave_isum(int v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ int wave_iscan(int v) {  // inclusive prefix sum over lanes
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}
__device__ int work_chunk(const DecodeArgs& a) {
  int tot = 0;
  for (int i = threadIdx.x & 63; i < a.batch; i += 64) tot += clamp_len(a, i);
  tot = wave_isum(tot);
  const int per = (tot + a.plan.target - 1) / a.plan.target;
  const int chunk = ((per + 63) / 64) * 64;
  return __builtin_amdgcn_readfirstlane(chunk < 64 ? 64 : (chunk > a.plan.cmax ? a.plan.cmax : chunk));
}
struct WorkItem {
  int b, t0, t1;  // sequence and token range [t0, t1), non-empty when found
};
// Item `item` of the split; false when the batch has fewer items.
__device__ bool locate_item(const DecodeArgs& a, int item, WorkItem& wi) {
  const int chunk = work_chunk(a), lane = threadIdx.x & 63;
  int base = 0;
  for (int c0 = 0; c0 < a.batch; c0 += 64) {
    const int i = c0 + lane;
    const int L = i < a.batch ? clamp_len(a, i) : 0;
    const int cnt = (L + chunk - 1) / chunk;
    const int incl = wave_iscan(cnt);
    const int total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
    if (item < base + total) {
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(base + incl > item);
      const int ln = (int)__builtin_ctzll(hit);
      const int first = base + __shfl(incl - cnt, ln, 64);
      // the values are wave-uniform; readfirstlane lets the compiler keep them (and the addresses
      // derived from them) in scalar registers
      wi.b = __builtin_amdgcn_readfirstlane(c0 + ln);
      wi.t0 = __builtin_amdgcn_readfirstlane((item - first) * chunk);
      wi.t1 = __builtin_amdgcn_readfirstlane(min(wi.t0 + chunk, __shfl(L, ln, 64)));
      return true;
    }
    base += total;
  }
  return false;
}
// First item and item count of sequence b.
__device__ void sequence_items(const DecodeArgs& a, int b, int& first, int& count) {
  const int chunk = work_chunk(a), lane = threadIdx.x & 63;
  int before = 0;
  for (int i = lane; i < b; i += 64) before += (clamp_len(a, i) + chunk - 1) / chunk;
  first = __builtin_amdgcn_readfirstlane(wave_isum(before));
  count = (clamp_len(a, b) + chunk - 1) / chunk;
}

// ------------------------------------------------------------------ 1. query preparation
// Workgroup (head h, 64 latent columns, up to QB batch rows), 8 waves splitting the NoPE dims: every
// lane issues all of its W_uk loads at once, accumulates QB rows, and the partial sums meet in LDS.
// Workgroups with blockIdx.y == 0 also rotate the retained query pairs.
constexpr int QW = 8, QMAXI = 32;  // waves per workgroup, NoPE dims per wave (d_h - 2r <= 256)

template <typename T>
__global__ __launch_bounds__(512) void decode_qprep(DecodeArgs a) {
  const int h = blockIdx.x, kk = threadIdx.x & 63, k = blockIdx.y * 64 + kk, b0 = blockIdx.z * QB;
  const int ty = threadIdx.x >> 6;
  const int D = a.s.d_kv, dh = a.s.d_head, r = a.s.r_pairs, dn = a.s.d_nope(), half = dh / 2, NH = a.s.n_heads;
  __shared__ int nope_idx[MAX_DH];
  __shared__ int kept[MAX_DH / 2];
  __shared__ __attribute__((aligned(16))) float qn[MAX_DH][QB];
  __shared__ float red[QW][QB][64];
  // this thread's W_uk column over its share of the NoPE dims, loaded first (independent of the rest)
  const int per = (dn + QW - 1) / QW, i0 = ty * per, i1 = min(dn, i0 + per);
  const T* wuk = (const T*)a.w_uk + (size_t)h * dn * D + min(k, D - 1);
  float wv[QMAXI];
#pragma unroll
  for (int u = 0; u < QMAXI; ++u) {
    if (u < per) wv[u] = to_f32(wuk[(size_t)min(i0 + u, dn - 1) * D]);
  }
  build_nope_idx(a.pair_idx, h, r, half, kept, nope_idx);
  __syncthreads();
  const T* q = (const T*)a.q;
  {  // gather the NoPE query dims of the QB rows in one round (QB * d_nope <= 4 * blockDim)
    float g[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = threadIdx.x + u * blockDim.x, bb = idx / max(dn, 1), i = idx - bb * max(dn, 1), b = b0 + bb;
      g[u] = (idx < QB * dn && b < a.batch) ? to_f32(q[((size_t)b * NH + h) * dh + nope_idx[i]]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = threadIdx.x + u * blockDim.x, bb = idx / max(dn, 1), i = idx - bb * max(dn, 1);
      if (idx < QB * dn) qn[i][bb] = g[u];
    }
  }
  __syncthreads();
  float acc[QB];
#pragma unroll
  for (int bb = 0; bb < QB; ++bb) acc[bb] = 0.f;
#pragma unroll
  for (int u = 0; u < QMAXI; ++u) {
    if (i0 + u >= i1 || k >= D) break;
    const f32x4* qrow = (const f32x4*)qn[i0 + u];
#pragma unroll
    for (int b4 = 0; b4 < QB / 4; ++b4) {
      f32x4 qq = qrow[b4];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[4 * b4 + c] = fmaf(wv[u], qq[c], acc[4 * b4 + c]);
    }
  }
#pragma unroll
  for (int bb = 0; bb < QB; ++bb) red[ty][bb][kk] = acc[bb];
  __syncthreads();
  const float scale = kLog2e / sqrtf((float)dh);
  T* qt = (T*)(a.ws + a.plan.off_qt);
  for (int idx = threadIdx.x; idx < QB * 64; idx += blockDim.x) {
    int bb = idx >> 6, c = idx & 63, b = b0 + bb, kc = blockIdx.y * 64 + c;
    if (b < a.batch && kc < D) {
      float v = 0.f;
#pragma unroll
      for (int t = 0; t < QW; ++t) v += red[t][bb][c];
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

// 1b. query preparation on MFMA (bf16, d_h - 2r <= 128, latent width a multiple of 128).
// Workgroup (head h, 128 latent columns, 32 sequences); wave w owns 32 of the columns.
//   q~[b][k] = sum_i q_nope[b][i] W_uk,h[i][k]:  A = gathered NoPE query rows (LDS, rows b),
//   B = W_uk tile (LDS, rows i, k contiguous) through the transpose read; K = NoPE dims padded to 128.
__global__ __launch_bounds__(256) void decode_qprep_mfma(DecodeArgs a) {
  constexpr int WP = 128 + 8;  // LDS pitch of both tiles (elements)
  __shared__ __attribute__((aligned(16))) bf16 wt[128 * WP];
  __shared__ __attribute__((aligned(16))) bf16 qa[32 * WP];
  __shared__ int nope_idx[MAX_DH];
  __shared__ int kept[MAX_DH / 2];
  const int h = blockIdx.x, kb = blockIdx.y * 128, b0 = blockIdx.z * 32;
  const int D = a.s.d_kv, dh = a.s.d_head, r = a.s.r_pairs, dn = a.s.d_nope(), half = dh / 2, NH = a.s.n_heads;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hb = lane >> 5;
  // W_uk rows i < dn, columns kb .. kb+127: 16 chunks of 16 bytes per row, issued first
  const bf16* wuk = (const bf16*)a.w_uk + (size_t)h * dn * D + kb;
  u32x4 wreg[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = u * 256 + tid, row = c >> 4, ch = c & 15;
    wreg[u] = row < dn ? *(const u32x4*)(wuk + (size_t)row * D + ch * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  build_nope_idx(a.pair_idx, h, r, half, kept, nope_idx);
  __syncthreads();
  const bf16* q = (const bf16*)a.q;
  bf16 g[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {  // q_nope of 32 rows x 128 padded dims: 16 per thread
    const int c = u * 256 + tid, bb = c >> 7, i = c & 127, b = b0 + bb;
    g[u] = (i < dn && b < a.batch) ? q[((size_t)b * NH + h) * dh + nope_idx[i]] : (bf16)0.f;
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = u * 256 + tid, row = c >> 4, ch = c & 15;
    *(u32x4*)&wt[row * WP + ch * 8] = wreg[u];
  }
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int c = u * 256 + tid, bb = c >> 7, i = c & 127;
    qa[bb * WP + i] = g[u];
  }
  __syncthreads();
  f32x16 acc = f32x16{};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const bf16x8 av = *(const bf16x8*)&qa[(lane & 31) * WP + 16 * s + 8 * hb];
    const int col = 32 * w + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int row0 = 16 * s + 8 * hb + ((lane & 15) >> 2);
    const bf16x4 x0 = lds_read_tr16(&wt[row0 * WP + col]);
    const bf16x4 x1 = lds_read_tr16(&wt[(row0 + 4) * WP + col]);
    acc = mfma32(av, cat(x0, x1), acc);
  }
  const float scale = kLog2e / sqrtf((float)dh);
  bf16* qt = (bf16*)(a.ws + a.plan.off_qt);
  const int k = kb + 32 * w + (lane & 31);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int b = b0 + 8 * (e >> 2) + 4 * hb + (e & 3);
    if (b < a.batch) qt[((size_t)b * NH + h) * D + k] = (bf16)(acc[e] * scale);
  }
  if (blockIdx.y != 0) return;
  float* qr = (float*)(a.ws + a.plan.off_qr);
  for (int idx = tid; idx < 32 * r; idx += blockDim.x) {
    const int bb = idx / r, j = idx - bb * r, b = b0 + bb;
    if (b >= a.batch) continue;
    const int L = clamp_len(a, b);
    const int pos = L > 0 ? L - 1 : 0;
    const int p = load_pair(a.pair_idx, h * r + j, half);
    const float x0 = (float)q[((size_t)b * NH + h) * dh + 2 * p], x1 = (float)q[((size_t)b * NH + h) * dh + 2 * p + 1];
    const float c = a.rope_cos[(size_t)pos * half + p], sn = a.rope_sin[(size_t)pos * half + p];
    qr[((size_t)b * NH + h) * 2 * r + 2 * j] = (x0 * c - x1 * sn) * scale;
    qr[((size_t)b * NH + h) * 2 * r + 2 * j + 1] = (x0 * sn + x1 * c) * scale;
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
  WorkItem wi;
  if (!locate_item(a, blockIdx.x, wi)) return;
  const int b = wi.b, t0 = wi.t0, n = wi.t1 - wi.t0;
  const int D = a.s.d_kv, NH = a.s.n_heads, R2 = a.s.r2();
  extern __shared__ float sh[];
  float* qs = sh;              // D
  float* qrs = qs + D;         // R2
  float* sc = qrs + R2 + 1;    // chunk
  __shared__ float red[8];
  float* ml = (float*)(a.ws + a.plan.off_ml) + (size_t)blockIdx.x * NH * 2;
  float* po = (float*)(a.ws + a.plan.off_o) + (size_t)blockIdx.x * NH * D;
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

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hb = lane >> 5, h = lane & 31;
  WorkItem wi;
  if (!locate_item(a, blockIdx.x, wi)) return;
  const int b = wi.b, t0 = wi.t0, t1 = wi.t1;
  float* pml = (float*)(a.ws + a.plan.off_ml) + (size_t)blockIdx.x * 32 * 2;
  float* po = (float*)(a.ws + a.plan.off_o) + (size_t)blockIdx.x * 32 * D;

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

  // ---- register prefetch, two tiles deep: this wave's latent slice and its share of the RoPE keys
  constexpr int CPR = (FMT == 0) ? DW / 8 : DW / 32;  // 16-byte chunks per row
  constexpr int CCH = 32 * CPR / 64;                  // chunks per lane
  typedef bf16 kv_t __attribute__((ext_vector_type(R2)));
  u32x4 creg[2][CCH];
  uint16_t sreg[2][CCH];
  kv_t kreg[2][4];

  auto load_tile = [&](auto bsel, int tt) {
    constexpr int B = decltype(bsel)::value;
#pragma unroll
    for (int it = 0; it < CCH; ++it) {
      int c = it * 64 + lane, row = c / CPR, q = c - row * CPR;
      int tok = min(tt + row, t1 - 1);  // rows past the sequence repeat its last row (masked below)
      if (FMT == 0) {
        creg[B][it] = *(const u32x4*)((const bf16*)a.ckv + (rowb + tok) * D + w * DW + 8 * q);
      } else {
        creg[B][it] = *(const u32x4*)((const uint8_t*)a.ckv + (rowb + tok) * (D / 2) + (w * DW + 32 * q) / 2);
        sreg[B][it] = ((const uint16_t*)a.ckv_scale)[(rowb + tok) * (D / 32) + (w * DW) / 32 + q];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int tok = min(tt + 8 * w + 4 * hb + i, t1 - 1);
      kreg[B][i] = *(const kv_t*)(krb + ((size_t)tok * 32 + h) * R2);
    }
  };
  auto stage_tile = [&](auto bsel) {
    constexpr int B = decltype(bsel)::value;
#pragma unroll
    for (int it = 0; it < CCH; ++it) {
      int c = it * 64 + lane, row = c / CPR, q = c - row * CPR;
      if (FMT == 0) {
        *(u32x4*)&cw[row * CP + 8 * q] = creg[B][it];
      } else {
        float s = __half2float(__ushort_as_half(sreg[B][it]));
        const uint32_t wd[4] = {creg[B][it].x, creg[B][it].y, creg[B][it].z, creg[B][it].w};
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

  int par = 0;
  // one 32-token tile: stage registers -> LDS, refill them with the tile two ahead, then both products
  auto step = [&](auto bsel, int tt) {
    constexpr int B = decltype(bsel)::value;
    stage_tile(bsel);
    // RoPE term of rows 8w + 4hb + i (result elements 4w + i), taken before the registers refill
    float rt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < R2; ++c) acc = fmaf(qr[c], (float)kreg[B][i][c], acc);
      rt[i] = acc;
    }
    if (tt + 64 < t1) load_tile(bsel, tt + 64);
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
    par ^= 1;
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
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  load_tile(B0{}, t0);
  if (t0 + 32 < t1) load_tile(B1{}, t0 + 32);
  for (int tt = t0; tt < t1; tt += 64) {
    step(B0{}, tt);
    if (tt + 32 < t1) step(B1{}, tt + 32);
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

// ------------------------------------------------------------------ 2c. attention, dense MFMA path with LDS DMA
// Same math and lane mapping as 2b, but every tile reaches LDS through global_load_lds_dwordx4 (no
// staging registers): a ring of three tile slots (separate LDS arrays, so the compiler can tell the
// slot being read from the slots still being filled), two tiles in flight while the third is used,
// explicit vmcnt waits.  Each wave moves only what it reads: its latent column slice (rows XOR-swizzled
// in 16-byte chunks so that both the row reads and the transpose reads are bank-conflict free) and the
// RoPE keys of its 8 rows of the tile.  Rows past the sequence repeat its last row and are masked.
template <int DW>
__device__ __forceinline__ int swz(int row, int chunk) {
  if (DW == 128) return chunk ^ (((row & 7) << 1) | ((row >> 3) & 1));
  const int m = row >> 1;
  return chunk ^ (((m & 3) << 1) | ((m >> 2) & 1));
}
// byte offset of element (row, col) inside one wave's slice of a tile
template <int DW>
__device__ __forceinline__ int slice_off(int row, int col) {
  return row * (DW * 2) + 16 * swz<DW>(row, col >> 3) + (col & 7) * 2;
}


// NSLOT tile slots in the DMA ring (2: one tile in flight while one is used; 3: two in flight), NSB
// buffers for the cross-wave exchange of partial scores (2 saves one barrier per tile).
template <int DW, int R2, int NSLOT, int NSB>
__global__ __launch_bounds__(256, 1) void decode_attn_dma(DecodeArgs a) {
  constexpr int NS = DW / 16, NB = DW / 32, D = 4 * DW;
  constexpr int CSL = 32 * DW * 2;       // bytes of one wave's latent slice of a tile
  constexpr int KSL = 8 * 32 * R2 * 2;   // bytes of one wave's RoPE rows of a tile
  constexpr int NC = CSL / 1024, NK = KSL / 1024;
  constexpr int RB = DW * 2;             // bytes per slice row
  constexpr float kRescale = 8.f;        // log2 headroom before the running max must be raised
  __shared__ __attribute__((aligned(1024))) char cs0[4 * CSL], cs1[4 * CSL], cs2[NSLOT > 2 ? 4 * CSL : 16];
  __shared__ __attribute__((aligned(1024))) char ks0[4 * KSL], ks1[4 * KSL], ks2[NSLOT > 2 ? 4 * KSL : 16];
  __shared__ f32x4 sbuf[NSB][4][4][64];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hb = lane >> 5, h = lane & 31;
  WorkItem wi;
  if (!locate_item(a, blockIdx.x, wi)) return;
  const int b = wi.b, t0 = wi.t0, t1 = wi.t1;
  float* pml = (float*)(a.ws + a.plan.off_ml) + (size_t)blockIdx.x * 32 * 2;
  float* po = (float*)(a.ws + a.plan.off_o) + (size_t)blockIdx.x * 32 * D;

  // DMA addresses: a wave-uniform tile base (SGPRs) plus per-lane offsets that do not change per tile
  const size_t rowb = (size_t)b * a.t_max;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const char* cbase = (const char*)a.ckv + (rowb * D + wu * DW) * 2;
  const char* kseq = (const char*)a.krope + rowb * 32 * R2 * 2;  // this sequence's RoPE rows
  const char* kbase = kseq + 8 * wu * 32 * R2 * 2;                 // ... from the wave's first row
  uint32_t coff[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int off = 1024 * j + 16 * lane, row = off / RB;
    coff[j] = row * (D * 2) + 16 * swz<DW>(row, (off % RB) / 16);
  }
  const uint32_t c_lds[3] = {lds_addr_of(cs0) + wu * CSL, lds_addr_of(cs1) + wu * CSL, lds_addr_of(cs2) + wu * CSL};
  const uint32_t k_lds[3] = {lds_addr_of(ks0) + wu * KSL, lds_addr_of(ks1) + wu * KSL, lds_addr_of(ks2) + wu * KSL};
  auto issue_slot = [&](auto ssel, int tt) {
    constexpr int SL = decltype(ssel)::value;
    if (tt + 32 <= t1) {
      const char* cb = cbase + (size_t)tt * (D * 2);
#pragma unroll
      for (int j = 0; j < NC; ++j) dma16(cb, coff[j], c_lds[SL] + 1024 * j);
    } else {  // last, partial tile: rows past the sequence repeat its last row (masked later)
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int off = 1024 * j + 16 * lane, row = off / RB;
        const int tok = min(tt + row, t1 - 1);
        dma16(cbase, (uint32_t)(tok * (D * 2) + 16 * swz<DW>(row, (off % RB) / 16)), c_lds[SL] + 1024 * j);
      }
    }
    // the wave's RoPE rows 8w .. 8w+7 of the tile are one contiguous block
    if (tt + 8 * wu + 8 <= t1) {
      const char* kb = kbase + (size_t)tt * (32 * R2 * 2);
#pragma unroll
      for (int j = 0; j < NK; ++j) dma16(kb, (uint32_t)(1024 * j + 16 * lane), k_lds[SL] + 1024 * j);
    } else {
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const int off = 1024 * j + 16 * lane, tk = off / (64 * R2), within = off % (64 * R2);
        const int tok = min(tt + 8 * wu + tk, t1 - 1);  // absolute position, >= 0
        dma16(kseq, (uint32_t)(tok * (64 * R2) + within), k_lds[SL] + 1024 * j);
      }
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  issue_slot(S0{}, t0);
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
  // the query operands (and the first tile) must be complete before the loop: the compiler would
  // otherwise guard their first use inside the loop with a vmcnt(0) on every iteration
  MLA_WAIT_VMCNT(0);
  if (NSLOT > 2 && t0 + 32 < t1) issue_slot(S1{}, t0 + 32);

  f32x16 oacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) oacc[i] = f32x16{};
  // running max per head (log2 domain), raised lazily: p = exp2(s - m_run) may reach 2^kRescale
  float m_run = -INFINITY, l_run = 0.f;
  typedef bf16 kv_t __attribute__((ext_vector_type(R2)));
  int par = 0;

  auto step = [&](auto ssel, int tt) {
    constexpr int SL = decltype(ssel)::value;
    char* cs = SL == 0 ? cs0 : (SL == 1 ? cs1 : cs2);
    char* kss = SL == 0 ? ks0 : (SL == 1 ? ks1 : ks2);
    constexpr int NX = (SL + NSLOT - 1) % NSLOT;  // slot that receives the tile NSLOT-1 ahead
    const int ahead = tt + 32 * (NSLOT - 1);
    if (NSLOT > 2) {
      // this tile is complete once at most the next tile's loads (NC + NK) are outstanding
      if (tt + 32 < t1) {
        MLA_WAIT_VMCNT(NC + NK);
      } else {
        MLA_WAIT_VMCNT(0);
      }
    } else {
      MLA_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_wave_barrier();
    if (ahead < t1) issue_slot(std::integral_constant<int, NX>{}, ahead);

    const char* cw = cs + w * CSL;
    float rt[4];
    {
      const char* kw = kss + w * KSL;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kv_t kk = *(const kv_t*)(kw + ((4 * hb + i) * 32 + h) * R2 * 2);
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < R2; ++c) acc = fmaf(qr[c], (float)kk[c], acc);
        rt[i] = acc;
      }
    }
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8 av = *(const bf16x8*)(cw + slice_off<DW>(lane & 31, 16 * s + 8 * hb));
      sacc = mfma32(av, qv[s], sacc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (w == j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[4 * j + i] += rt[i];
      }
    if (NSB == 1) lds_barrier();  // every wave has read the previous tile's partial scores
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4)
      sbuf[NSB == 1 ? 0 : par][w][e4][lane] = f32x4{sacc[4 * e4], sacc[4 * e4 + 1], sacc[4 * e4 + 2], sacc[4 * e4 + 3]};
    lds_barrier();
    float sc[16];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int pb_ = NSB == 1 ? 0 : par;
      f32x4 v = sbuf[pb_][0][e4][lane];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) v += sbuf[pb_][ww][e4][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * e4 + i] = v[i];
    }
    par ^= 1;
    if (tt + 32 > t1) {  // last, partial tile: mask rows past the sequence
      asm volatile("" ::: "memory");  // keep this a branch (not if-converted into every tile)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (tt + 8 * (e >> 2) + 4 * hb + (e & 3) >= t1) sc[e] = -INFINITY;
    }
    float mt = sc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mt = fmaxf(mt, sc[e]);
    mt = fmaxf(mt, shfl_xor(mt, 32));
    // raise the running max only when this tile exceeds it by more than the headroom (rare after the
    // first tile); a raise rescales the latent accumulators of that head
    const bool raise = mt > m_run + kRescale;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      asm volatile("" ::: "memory");  // keep this a branch (not if-converted into every tile)
      const float m_new = raise ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) oacc[blk] *= alpha;
      m_run = m_new;
    }
    float p[16], rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = __builtin_amdgcn_exp2f(sc[e] - m_run);
      rs += p[e];
    }
    rs += shfl_xor(rs, 32);
    l_run += rs;
    bf16x8 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[c][e] = (bf16)p[8 * c + e];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int col = blk * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row0 = 16 * c + 4 * hb + ((lane & 15) >> 2);
        bf16x4 x0 = lds_read_tr16((const bf16*)(cw + slice_off<DW>(row0, col)));
        bf16x4 x1 = lds_read_tr16((const bf16*)(cw + slice_off<DW>(row0 + 8, col)));
        oacc[blk] = mfma32(cat(x0, x1), pb[c], oacc[blk]);
      }
    }
  };

  if (NSLOT > 2) {
    for (int tt = t0; tt < t1; tt += 96) {
      step(S0{}, tt);
      if (tt + 32 < t1) step(S1{}, tt + 32);
      if (tt + 64 < t1) step(S2{}, tt + 64);
    }
  } else {
    for (int tt = t0; tt < t1; tt += 64) {
      step(S0{}, tt);
      if (tt + 32 < t1) step(S1{}, tt + 32);
    }
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

// ------------------------------------------------------------------ 3. combine: merge, then W_uv
// 3a. merge: one wave per (sequence, head).  Weights exp2(m_s - M) from the split maxima, denominator
//     sum_s w_s l_s, normalised latent output o = sum_s w_s o_s / den into the workspace (fp32).  Each
//     lane owns KPL latent columns and keeps the loads of four splits in flight.
template <int KPL>
__global__ __launch_bounds__(256) void decode_merge(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int D = a.s.d_kv, NH = a.s.n_heads;
  if (pair >= a.batch * NH) return;
  const int b = pair / NH, h = pair - b * NH;
  int first, S;
  sequence_items(a, b, first, S);
  const float* ml = (const float*)(a.ws + a.plan.off_ml) + ((size_t)first * NH + h) * 2;
  const float* po = (const float*)(a.ws + a.plan.off_o) + ((size_t)first * NH + h) * D;
  // running merge over groups of 8 splits; each group's (m, l) and latent rows are loaded in one round
  float M = -INFINITY, den = 0.f, acc[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float ms[8], ls[8], v[8][KPL];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = s0 + u < S;
      ms[u] = ok ? ml[(size_t)(s0 + u) * NH * 2] : -INFINITY;
      ls[u] = ok ? ml[(size_t)(s0 + u) * NH * 2 + 1] : 0.f;
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const int k = lane + 64 * i;
        v[u][i] = (ok && k < D) ? po[(size_t)(s0 + u) * NH * D + k] : 0.f;
      }
    }
    float gm = M;
#pragma unroll
    for (int u = 0; u < 8; ++u) gm = fmaxf(gm, ms[u]);
    if (gm == -INFINITY) continue;  // nothing seen yet (empty splits only)
    const float c = exp2f(M - gm);  // rescale of what was merged so far (0 when M = -inf)
    den *= c;
#pragma unroll
    for (int i = 0; i < KPL; ++i) acc[i] *= c;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wv = ms[u] == -INFINITY ? 0.f : exp2f(ms[u] - gm);
      den = fmaf(wv, ls[u], den);
#pragma unroll
      for (int i = 0; i < KPL; ++i) acc[i] = fmaf(wv, v[u][i], acc[i]);
    }
    M = gm;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float* ob = (float*)(a.ws + a.plan.off_ob) + ((size_t)b * NH + h) * D;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int k = lane + 64 * i;
    if (k < D) ob[k] = acc[i] * inv;
  }
}

// 3b. out[b,h,:] = o[b,h,:] . W_uv,h^T.
//   bf16 path: MFMA.  Workgroup (head h, 32 output dims, 32 sequences), 4 waves splitting the latent
//   width.  Each merged fp32 row is split exactly into bf16 hi + lo parts (two MFMAs), so the product
//   keeps ~16 significant bits of o; W_uv rows are read once as 16-byte operand loads.
//   other shapes (fp32, latent widths not a multiple of 64): one thread per (row, output dim).
__global__ __launch_bounds__(256) void decode_project_mfma(DecodeArgs a) {
  __shared__ float red[4][32][33];
  const int h = blockIdx.x, e0 = blockIdx.y * 32, b0 = blockIdx.z * 32;
  const int D = a.s.d_kv, dh = a.s.d_head, NH = a.s.n_heads;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int kw = D / 4, k0 = w * kw;  // this wave's quarter of the latent width (multiple of 16)
  const float* ob = (const float*)(a.ws + a.plan.off_ob);
  const bf16* wuv = (const bf16*)a.w_uv + (size_t)h * dh * D;
  const int b = b0 + (lane & 31), e = e0 + (lane & 31);
  const bool bok = b < a.batch, eok = e < dh;
  const float* orow = ob + ((size_t)b * NH + h) * D;
  const bf16* wrow = wuv + (size_t)e * D;
  f32x16 acc = f32x16{};
  constexpr int MAXS = 8;  // K steps of 16 per batch of loads
  for (int kb = k0; kb < k0 + kw; kb += 16 * MAXS) {
    f32x4 o0[MAXS], o1[MAXS];
    bf16x8 wv[MAXS];
#pragma unroll
    for (int u = 0; u < MAXS; ++u) {
      const int k = kb + 16 * u + 8 * (lane >> 5);
      const bool kin = kb + 16 * u < k0 + kw;
      o0[u] = (bok && kin) ? *(const f32x4*)(orow + k) : f32x4{0.f, 0.f, 0.f, 0.f};
      o1[u] = (bok && kin) ? *(const f32x4*)(orow + k + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
      wv[u] = (eok && kin) ? *(const bf16x8*)(wrow + k) : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < MAXS; ++u) {
      bf16x8 hi, lo;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        hi[c] = (bf16)o0[u][c];
        lo[c] = (bf16)(o0[u][c] - (float)hi[c]);
        hi[4 + c] = (bf16)o1[u][c];
        lo[4 + c] = (bf16)(o1[u][c] - (float)hi[4 + c]);
      }
      acc = mfma32(hi, wv[u], acc);
      acc = mfma32(lo, wv[u], acc);
    }
  }
  // D[row = sequence][col = output dim]: lane holds col lane%32, rows 8(i/4) + 4(lane/32) + i%4
#pragma unroll
  for (int i = 0; i < 16; ++i) red[w][8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)][lane & 31] = acc[i];
  __syncthreads();
  bf16* out = (bf16*)a.out;
  for (int idx = threadIdx.x; idx < 32 * 32; idx += blockDim.x) {
    const int bb = idx >> 5, ee = idx & 31;
    const float v = red[0][bb][ee] + red[1][bb][ee] + red[2][bb][ee] + red[3][bb][ee];
    if (b0 + bb < a.batch && e0 + ee < dh) out[((size_t)(b0 + bb) * NH + h) * dh + e0 + ee] = (bf16)v;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void decode_project_vec(DecodeArgs a) {
  const int D = a.s.d_kv, dh = a.s.d_head, NH = a.s.n_heads;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.batch * NH * dh) return;
  const int e = idx % dh, bh = idx / dh, h = bh % NH;
  const float* o = (const float*)(a.ws + a.plan.off_ob) + (size_t)bh * D;
  const T* wr = (const T*)a.w_uv + ((size_t)h * dh + e) * D;
  float acc = 0.f;
  for (int k = 0; k < D; ++k) acc = fmaf(o[k], to_f32(wr[k]), acc);
  ((T*)a.out)[idx] = from_f32<T>(acc);
}

template <typename T>
void launch_generic_attn(const DecodeArgs& a, hipStream_t st) {
  size_t shmem = (size_t)(a.s.d_kv + a.s.r2() + 1 + a.plan.cmax) * sizeof(float);
  dim3 grid(a.plan.max_items);
  if (a.s.fmt == 0)
    hipLaunchKernelGGL((decode_attn_generic<T, 0>), grid, dim3(256), shmem, st, a);
  else
    hipLaunchKernelGGL((decode_attn_generic<T, 1>), grid, dim3(256), shmem, st, a);
}

template <int DW, int R2>
void launch_mfma_attn(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.plan.max_items);
  if (a.s.fmt == 0)
    hipLaunchKernelGGL((decode_attn_dma<DW, R2, (DW == 128 && R2 == 8) ? 3 : 3, (DW == 128 && R2 == 8) ? 1 : 2>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_attn_mfma<DW, R2, 1>), grid, dim3(256), 0, st, a);
}

}  // namespace

bool decode_uses_mfma(const Shape& s) {
  return s.dtype == 1 && s.n_heads == 32 && (s.d_kv == 256 || s.d_kv == 512) && (s.r_pairs == 2 || s.r_pairs == 4);
}

bool decode_fits(const Shape& s, const DecodePlan& p) {
  if (s.d_kv > 1024) return false;
  if (!decode_uses_mfma(s) && (size_t)(s.d_kv + s.r2() + 1 + p.cmax) * sizeof(float) > 65536) return false;
  return true;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

DecodePlan plan_decode(const Shape& s, int batch, int max_seq_len) {
  DecodePlan p{};
  // one workgroup per CU for the specialised dense kernels (their LDS ring fills a CU), two otherwise
  p.target = (decode_uses_mfma(s) && s.fmt == 0) ? 256 : 512;
  p.cmax = 2048;
  if (!decode_uses_mfma(s)) {  // the generic kernel keeps a chunk of scores in LDS
    const long long room = 65536 / 4 - (long long)s.d_kv - s.r2() - 1;
    const long long c = room > 0 ? (room / 64) * 64 : 64;
    if (c < p.cmax) p.cmax = (int)(c < 64 ? 64 : c);
  }
  // items = sum_b ceil(L_b / chunk) < sum_b L_b / chunk + batch; chunk >= sum / target unless clamped
  const long long B = batch, Lm = max_seq_len;
  long long by_min = B * ((Lm + 63) / 64);                          // chunk = 64
  long long by_max = (B * Lm + p.cmax - 1) / p.cmax;                // chunk = cmax
  long long bound = (by_max > p.target ? by_max : p.target) + B;
  long long items = by_min < bound ? by_min : bound;
  p.max_items = (int)(items < 1 ? 1 : items);
  const size_t esz = s.dtype == 0 ? 4 : 2;
  size_t off = 0;
  p.off_qt = off;
  off = align256(off + (size_t)batch * s.n_heads * s.d_kv * esz);
  p.off_qr = off;
  off = align256(off + (size_t)batch * s.n_heads * (s.r2() > 0 ? s.r2() : 1) * 4);
  p.off_ml = off;
  off = align256(off + (size_t)p.max_items * s.n_heads * 2 * 4);
  p.off_o = off;
  off = align256(off + (size_t)p.max_items * s.n_heads * s.d_kv * 4);
  p.off_ob = off;
  off = align256(off + (size_t)batch * s.n_heads * s.d_kv * 4);
  p.total = off;
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st, int phase_mask) {
  const int nh = a.s.n_heads;
  if (phase_mask & 1) {
    dim3 gq(nh, (a.s.d_kv + 63) / 64, (a.batch + QB - 1) / QB);
    if (a.s.dtype == 1 && a.s.d_nope() <= 128 && a.s.d_kv % 128 == 0)
      hipLaunchKernelGGL(decode_qprep_mfma, dim3(nh, a.s.d_kv / 128, (a.batch + 31) / 32), dim3(256), 0, st, a);
    else if (a.s.dtype == 0)
      hipLaunchKernelGGL(decode_qprep<float>, gq, dim3(64 * QW), 0, st, a);
    else
      hipLaunchKernelGGL(decode_qprep<bf16>, gq, dim3(64 * QW), 0, st, a);
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
    const int pairs = a.batch * nh, gm = (pairs + 3) / 4, kpl = (a.s.d_kv + 63) / 64;
    if (kpl <= 1) hipLaunchKernelGGL(decode_merge<1>, dim3(gm), dim3(256), 0, st, a);
    else if (kpl <= 2) hipLaunchKernelGGL(decode_merge<2>, dim3(gm), dim3(256), 0, st, a);
    else if (kpl <= 4) hipLaunchKernelGGL(decode_merge<4>, dim3(gm), dim3(256), 0, st, a);
    else if (kpl <= 8) hipLaunchKernelGGL(decode_merge<8>, dim3(gm), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(decode_merge<16>, dim3(gm), dim3(256), 0, st, a);
    const int n = a.batch * nh * a.s.d_head;
    if (a.s.dtype == 0) {
      hipLaunchKernelGGL(decode_project_vec<float>, dim3((n + 255) / 256), dim3(256), 0, st, a);
    } else if (a.s.d_kv % 64 == 0) {
      dim3 gp(nh, (a.s.d_head + 31) / 32, (a.batch + 31) / 32);
      hipLaunchKernelGGL(decode_project_mfma, gp, dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL(decode_project_vec<bf16>, dim3((n + 255) / 256), dim3(256), 0, st, a);
    }
  }
  return hipGetLastError();
}

}  // namespace mla
