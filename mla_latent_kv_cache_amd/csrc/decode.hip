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

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "step.h"

namespace mla {

namespace {

constexpr int QB = 16;     // batch rows per qprep workgroup (QB * d_nope <= 4 * 512)
constexpr int MLS = 4;     // floats per (work item, head) entry of the split statistics: m, l, A, unused
constexpr int MAX_DH = 256;

// Cache sequence read by query sequence b (several queries per cache sequence in multi-query decode).
__device__ __forceinline__ int cseq(const DecodeArgs& a, int b) { return a.qn > 1 ? b / a.qn : b; }
// Keys visible to query sequence b: its cache sequence's length (clamped to the host bound), less the
// newer queries of the same sequence.
__device__ __forceinline__ int clamp_len_of(const DecodeArgs& a, int b, int L) {  // L: seq_lens[cseq(b)]
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  if (a.qn > 1) {
    L -= a.qn - 1 - b % a.qn;
    L = L < 0 ? 0 : L;
  }
  return L;
}
__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int b) { return clamp_len_of(a, b, a.seq_lens[cseq(a, b)]); }
// Cache row of position pos of query sequence b (contiguous or through the page table).
__device__ __forceinline__ int seq_row(const DecodeArgs& a, int b, int pos) {
  return cache_row_of(a.pm, a.t_max, cseq(a, b), pos);
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
// Coded positions visible to query sequence b with L = clamp_len(b) visible keys.  With a window of bf16 rows
// (windowed formats, a.win > 0) the cache sequence's own last min(Lc, win) positions are ring rows, where Lc is
// its appended length (L plus the newer queries of the same sequence); the query sees [0, min(L, Lc - win)) as
// codes and the rest of its keys from the ring.  Without a window every key is coded.
__device__ __forceinline__ int coded_len(const DecodeArgs& a, int b, int L) {
  if (a.win <= 0 || L <= 0) return L;
  const int Lc = L + (a.qn > 1 ? a.qn - 1 - b % a.qn : 0);
  return min(L, Lc - min(Lc, a.win));
}
// Items of query sequence b (L visible keys): its coded positions are cut into chunks, and the last item also
// takes the window rows; a sequence with no coded rows has one item, its window.  WIN = false: a kernel of a
// format without a window (a.win is 0 there, so both forms count the same items; the constant one keeps the
// window arithmetic out of the kernels that never need it).
template <bool WIN = true>
__device__ __forceinline__ int item_count(const DecodeArgs& a, int b, int L, int chunk) {
  const int lq = WIN ? coded_len(a, b, L) : L, nq = (lq + chunk - 1) / chunk;
  return (nq == 0 && L > 0) ? 1 : nq;
}
// Lengths of sequences lane, lane + 64, ... : the first block's is returned in L0 (the callers reuse it,
// so that batches of up to 64 sequences read their lengths once), the chunk from their sum.
__device__ int work_chunk(const DecodeArgs& a, int& L0) {
  const int lane = threadIdx.x & 63;
  L0 = lane < a.batch ? clamp_len(a, lane) : 0;
  int tot = L0;
  for (int i = lane + 64; i < a.batch; i += 64) tot += clamp_len(a, i);
  tot = wave_isum(tot);
  const int per = (tot + a.plan.target - 1) / a.plan.target;
  const int chunk = ((per + 31) / 32) * 32;  // whole 32-row tiles (a 64-row minimum below)
  return __builtin_amdgcn_readfirstlane(chunk < 64 ? 64 : (chunk > a.plan.cmax ? a.plan.cmax : chunk));
}
__device__ int work_chunk(const DecodeArgs& a) {
  int L0;
  return work_chunk(a, L0);
}
struct WorkItem {
  int b, t0, t1;  // sequence and coded (or dense) token range [t0, t1)
  int w0, w1;     // window rows [w0, w1) of the sequence's last item (fmt 2), else empty
  int L;          // the sequence's (clamped) length
};
// Item `item` of the split; false when the batch has fewer items (WIN as for item_count).
template <bool WIN = true>
__device__ bool locate_item(const DecodeArgs& a, int item, WorkItem& wi) {
  int L0;
  const int chunk = work_chunk(a, L0), lane = threadIdx.x & 63;
  int base = 0;
  for (int c0 = 0; c0 < a.batch; c0 += 64) {
    const int i = c0 + lane;
    const int L = c0 == 0 ? L0 : (i < a.batch ? clamp_len(a, i) : 0);
    const int cnt = item_count<WIN>(a, i, L, chunk);
    const int incl = wave_iscan(cnt);
    const int total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
    if (item < base + total) {
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(base + incl > item);
      const int ln = (int)__builtin_ctzll(hit);
      const int first = base + __shfl(incl - cnt, ln, 64);
      const int Lb = __shfl(L, ln, 64), lq = WIN ? coded_len(a, c0 + ln, Lb) : Lb, nq = (lq + chunk - 1) / chunk;
      const int j = item - first;
      const bool last = j + 1 >= nq;
      // the values are wave-uniform; readfirstlane lets the compiler keep them (and the addresses
      // derived from them) in scalar registers
      wi.b = __builtin_amdgcn_readfirstlane(c0 + ln);
      wi.t0 = __builtin_amdgcn_readfirstlane(min(j * chunk, lq));
      wi.t1 = __builtin_amdgcn_readfirstlane(min(j * chunk + chunk, lq));
      wi.w0 = __builtin_amdgcn_readfirstlane(last ? lq : 0);
      wi.w1 = __builtin_amdgcn_readfirstlane(last ? Lb : 0);
      wi.L = __builtin_amdgcn_readfirstlane(Lb);
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
  for (int i = lane; i < b; i += 64) before += item_count(a, i, clamp_len(a, i), chunk);
  first = __builtin_amdgcn_readfirstlane(wave_isum(before));
  count = item_count(a, b, clamp_len(a, b), chunk);
}

// Rows of a fused split-K append (FuseArgs) at positions [t0, t1) of sequence b, written by the calling
// workgroup from the LDS scratch `lds`; true when there were any (the caller then waits for vmcnt 0
// before loading them).
__device__ __forceinline__ bool fused_rows(const FuseArgs& f, int b, int t0, int t1, float* lds) {
  if (f.ks == 0) return false;
  int sp = f.a.start_pos[b];
  sp = sp < 0 ? 0 : (sp > f.a.max_start ? f.a.max_start : sp);
  const int lo = max(t0, sp), hi = min(t1, sp + f.a.t_new);
  if (lo >= hi) return false;
  append_rows_fused(f.a, f.ks, b, sp, lo, hi, lds);
  return true;
}
// As fused_rows for the sequence's last item [t0, L), guessing that the new rows are the sequence's last
// t_new positions (a decode step's usual layout): the reduction's loads are issued together with the
// start position's instead of after it.  Returns 1 when the guess held (the rows are written), -1 when
// it does not apply or the start position differs (nothing written: the caller runs fused_rows).
// between() runs once the reduction's first loads are in flight (the caller issues its own loads there).
template <class Between>
__device__ __forceinline__ int fused_rows_last(const FuseArgs& f, int b, int t0, int L, float* lds, Between&& between) {
  const int g = L - f.a.t_new;
  if (f.ks == 0 || g < t0 || g < 0 || g > f.a.max_start) return -1;
  return append_rows_fused(f.a, f.ks, b, g, g, L, lds, true, between) ? 1 : -1;
}
// Extra workgroup max_items + b of a fused launch: the new rows of sequence b past its decode range.
__device__ __forceinline__ void fused_orphans(const DecodeArgs& a, const FuseArgs& f, float* lds) {
  const int b = blockIdx.x - a.plan.max_items;
  if (f.ks == 0 || b >= a.batch) return;
  fused_rows(f, b, clamp_len(a, b), 0x7fffffff, lds);
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
  build_nope_idx(a.pair_idx, a.s.rope_head(h), r, half, kept, nope_idx);
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
    int p = load_pair(a.pair_idx, a.s.rope_head(h) * r + j, half);
    float x0 = to_f32(q[((size_t)b * NH + h) * dh + 2 * p]), x1 = to_f32(q[((size_t)b * NH + h) * dh + 2 * p + 1]);
    float c = a.rope_cos[(size_t)pos * half + p], s = a.rope_sin[(size_t)pos * half + p];
    qr[((size_t)b * NH + h) * 2 * r + 2 * j] = (x0 * c - x1 * s) * scale;
    qr[((size_t)b * NH + h) * 2 * r + 2 * j + 1] = (x0 * s + x1 * c) * scale;
  }
}

// 1b. query preparation on MFMA (bf16, d_h <= 128 and a multiple of 8, latent width a multiple of 128,
// 16-byte aligned query rows).  Workgroup (head h, 128 latent columns, 32 sequences); wave w owns 32 of
// the columns.  q~[b][k] = sum_i q_nope[b][i] W_uk,h[i][k] runs over the head's own dims d (K = 128):
// A = the query rows as they are (LDS, rows b, zero past d_h), B = W_uk row i stored at LDS row
// nope_idx[i] (the i-th non-retained dim), every other row zero.  So nothing waits for the retained
// pairs before the query loads: the workgroup issues all of its global loads at its start.
constexpr int QP_WP = 128 + 8;  // LDS pitch of both q-prep tiles (elements)
struct QprepLds {
  __attribute__((aligned(16))) bf16 wt[128 * QP_WP];
  __attribute__((aligned(16))) bf16 qa[32 * QP_WP];
  int dest[128];  // LDS row of W_uk row i (rows i >= d_nope are zero)
};
__device__ __forceinline__ void qprep_mfma_tile(const DecodeArgs& a, int bx, int by, int bz, QprepLds& sm) {
  constexpr int WP = QP_WP;
  bf16* wt = sm.wt;
  bf16* qa = sm.qa;
  int* dest = sm.dest;
  const int h = bx, kb = by * 128, b0 = bz * 32;
  const int D = a.s.d_kv, dh = a.s.d_head, r = a.s.r_pairs, dn = a.s.d_nope(), half = dh / 2, NH = a.s.n_heads;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hb = lane >> 5;
  // global loads, in the order their values are needed: the retained pairs (wave 0), the rotation's
  // pairs and lengths (by == 0), the W_uk tile (rows i < d_nope, columns kb .. kb+127), the query rows.
  // Raw values first, clamped once every load is in flight (a use inside the loads' branches would wait
  // for each load in turn).
  const bool rot = by == 0 && tid < 32 * r;
  const int rbb = rot ? tid / r : 0, rj = rot ? tid - rbb * r : 0, rb = b0 + rbb;
  const bool rok = rot && rb < a.batch;
  int pk_raw = 0, rp_raw = 0, rL_raw = 0;
  const int g = a.s.rope_head(h);  // the head's row of the pair table
  if (tid < r) pk_raw = a.pair_idx[g * r + tid];
  if (rok) {
    rp_raw = a.pair_idx[g * r + rj];
    rL_raw = a.seq_lens[cseq(a, rb)];
  }
  // (the tile loads read a clamped in-bounds address and are zeroed afterwards: a load under a branch
  // would be waited for inside it)
  const bf16* q = (const bf16*)a.q;
  const bf16* wuk = dn > 0 ? (const bf16*)a.w_uk + (size_t)h * dn * D + kb : q;
  u32x4 wreg[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = u * 256 + tid, row = c >> 4, ch = c & 15;
    wreg[u] = *(const u32x4*)(dn > 0 ? wuk + (size_t)min(row, dn - 1) * D + ch * 8 : q);
  }
  u32x4 qreg[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {  // 32 rows x 16 chunks of 8 dims
    const int c = u * 256 + tid, bb = c >> 4, ch = c & 15, b = min(b0 + bb, a.batch - 1);
    qreg[u] = *(const u32x4*)(q + ((size_t)b * NH + h) * dh + 8 * min(ch, dh / 8 - 1));
  }
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (((u * 256 + tid) >> 4) >= dn) wreg[u] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = u * 256 + tid;
    if (8 * (c & 15) >= dh || b0 + (c >> 4) >= a.batch) qreg[u] = u32x4{0u, 0u, 0u, 0u};
  }
  const int pk = tid < r ? (pk_raw < 0 ? 0 : (pk_raw >= half ? half - 1 : pk_raw)) : -1;
  const int rp = rp_raw < 0 ? 0 : (rp_raw >= half ? half - 1 : rp_raw);
  const int rL = rok ? clamp_len_of(a, rb, rL_raw) : 0;
  if (w == 0) {
    // kept pairs as a 64-bit mask (lane j < r holds pair j), then lane l places dims 2l, 2l+1: the
    // non-retained pairs below d_h first, in ascending order, then the rest
    uint64_t km = 0;
    for (int j = 0; j < r; ++j) km |= 1ull << __builtin_amdgcn_readlane(pk, j);
    const bool nope = 2 * lane < dh && !((km >> lane) & 1ull);
    const uint64_t m = __builtin_amdgcn_ballot_w64(nope);
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const int pos = nope ? 2 * __builtin_popcountll(m & below)
                         : 2 * __builtin_popcountll(m) + 2 * __builtin_popcountll(~m & below);
    dest[pos] = 2 * lane;
    dest[pos + 1] = 2 * lane + 1;
  }
  // the rotation's RoPE factors (their addresses need the pair and the length)
  float rc = 0.f, rs = 0.f;
  if (rok) {
    const int pos = rL > 0 ? rL - 1 : 0;
    rc = a.rope_cos[(size_t)pos * half + rp];
    rs = a.rope_sin[(size_t)pos * half + rp];
  }
  lds_barrier();
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = u * 256 + tid, row = c >> 4, ch = c & 15;
    *(u32x4*)&wt[dest[row] * WP + ch * 8] = wreg[u];
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = u * 256 + tid, bb = c >> 4, ch = c & 15;
    *(u32x4*)&qa[bb * WP + ch * 8] = qreg[u];
  }
  lds_barrier();
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
  if (rok) {  // the retained pairs of the query, rotated to the sequence's last position
    float* qr = (float*)(a.ws + a.plan.off_qr);
    const float x0 = (float)qa[rbb * WP + 2 * rp], x1 = (float)qa[rbb * WP + 2 * rp + 1];
    qr[((size_t)rb * NH + h) * 2 * r + 2 * rj] = (x0 * rc - x1 * rs) * scale;
    qr[((size_t)rb * NH + h) * 2 * r + 2 * rj + 1] = (x0 * rs + x1 * rc) * scale;
  }
  if (by == 0) {  // more than 256 (sequence, pair) entries: the rest in turn
    float* qr = (float*)(a.ws + a.plan.off_qr);
    for (int idx = tid + 256; idx < 32 * r; idx += 256) {
      const int bb = idx / r, j = idx - bb * r, b = b0 + bb;
      if (b >= a.batch) continue;
      const int L = clamp_len(a, b), pos = L > 0 ? L - 1 : 0;
      const int p = load_pair(a.pair_idx, g * r + j, half);
      const float x0 = (float)qa[bb * WP + 2 * p], x1 = (float)qa[bb * WP + 2 * p + 1];
      const float c = a.rope_cos[(size_t)pos * half + p], sn = a.rope_sin[(size_t)pos * half + p];
      qr[((size_t)b * NH + h) * 2 * r + 2 * j] = (x0 * c - x1 * sn) * scale;
      qr[((size_t)b * NH + h) * 2 * r + 2 * j + 1] = (x0 * sn + x1 * c) * scale;
    }
  }
}

__global__ __launch_bounds__(256) void decode_qprep_mfma(DecodeArgs a) {
  __shared__ QprepLds sm;
  qprep_mfma_tile(a, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

// Decode-step prologue: the new tokens' split-K append (phase 1) and the query preparation depend on
// nothing of each other, so one launch runs both: workgroups [0, n_app) take append tiles, the rest
// query-preparation tiles.
__global__ __launch_bounds__(256) void decode_step_prologue(AppendArgs aa, int ks, DecodeArgs da) {
  const int nx = (aa.s.d_kv + aa.s.n_rope_cols() + 31) / 32, n_app = nx * ks;
  // one LDS block for either role (a workgroup runs one of them), so that more workgroups fit on a CU
  __shared__ union {
    SplitKLds app;
    QprepLds qp;
  } sm;
  const int bid = blockIdx.x;
  if (bid < n_app) {
    append_splitk_tile(aa, ks, bid % nx, bid / nx, sm.app);
  } else {
    const int j = bid - n_app, nh = da.s.n_heads, ny = da.s.d_kv / 128;
    qprep_mfma_tile(da, j % nh, (j / nh) % ny, j / (nh * ny), sm.qp);
  }
}

// ------------------------------------------------------------------ latent element access
// Element k of the latent of position pos of sequence b in the 2-bit format: a bf16 ring row inside the
// window, else fp32(z + code * s) of the coded row.
__device__ __forceinline__ float latent2(const DecodeArgs& a, int b, int pos, bool win, int k) {
  const int D = a.s.d_kv;
  if (win) return (float)((const bf16*)a.ckv_win)[((size_t)cseq(a, b) * a.win + pos % a.win) * D + k];
  const size_t row = (size_t)seq_row(a, b, pos);
  const uint32_t byte = ((const uint8_t*)a.ckv)[row * (D / 4) + (k >> 2)];
  const uint32_t m = ((const uint32_t*)a.ckv_scale)[row * (D / 32) + (k >> 5)];
  const float sc = __half2float(__ushort_as_half((unsigned short)(m & 0xFFFF)));
  const float z = __half2float(__ushort_as_half((unsigned short)(m >> 16)));
  return fmaf((float)((byte >> (2 * (k & 3))) & 3u), sc, z);
}

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
// One workgroup per work item, all heads in turn.  The item's rows (its coded or dense range, then for the
// 2-bit format the window of its sequence's last item) are taken in runs of at most plan.cmax rows, whose
// scores fit the LDS buffer; runs after the first merge into the head's running max / sum / output
// (a single run, the usual case, computes exactly the one-pass result).
template <typename T, int FMT>
__global__ __launch_bounds__(256) void decode_attn_generic(DecodeArgs a) {
  WorkItem wi;
  if (!locate_item(a, blockIdx.x, wi)) return;
  const int b = wi.b;
  const int D = a.s.d_kv, NH = a.s.n_heads, R2 = a.s.r2();
  constexpr int KPT = 4;  // latent columns per thread (d_kv <= 1024)
  extern __shared__ float sh[];
  float* qs = sh;              // D
  float* qrs = qs + D;         // R2
  float* sc = qrs + R2 + 1;    // cmax
  __shared__ float red[8];
  float* ml = (float*)(a.ws + a.plan.off_ml) + (size_t)blockIdx.x * NH * MLS;
  float* po = (float*)(a.ws + a.plan.off_o) + (size_t)blockIdx.x * NH * D;
  const T* qt = (const T*)(a.ws + a.plan.off_qt) + (size_t)b * NH * D;
  const float* qr = (const float*)(a.ws + a.plan.off_qr) + (size_t)b * NH * R2;
  // element k of the latent at position pos (from the window when `win`)
  auto lat = [&](int pos, bool win, int k) {
    if constexpr (FMT == 2) return latent2(a, b, pos, win, k);
    else if constexpr (FMT == 3)  // int4 codes with a window of bf16 rows
      return win ? (float)((const bf16*)a.ckv_win)[((size_t)cseq(a, b) * a.win + pos % a.win) * a.s.d_kv + k]
                 : latent<T, 1>(a, (size_t)seq_row(a, b, pos), k);
    else return latent<T, FMT>(a, (size_t)seq_row(a, b, pos), k);
  };
  for (int h = 0; h < NH; ++h) {
    for (int k = threadIdx.x; k < D; k += blockDim.x) qs[k] = to_f32(qt[(size_t)h * D + k]);
    for (int j = threadIdx.x; j < R2; j += blockDim.x) qrs[j] = qr[h * R2 + j];
    __syncthreads();
    float m_run = -INFINITY, l_run = 0.f, o[KPT] = {0.f, 0.f, 0.f, 0.f};
    for (int seg = 0; seg < 2; ++seg) {
      const int s0 = seg ? wi.w0 : wi.t0, s1 = seg ? wi.w1 : wi.t1;
      const bool win = seg == 1;
      for (int r0 = s0; r0 < s1; r0 += a.plan.cmax) {
        const int n = min(s1 - r0, a.plan.cmax);
        float mloc = -INFINITY;
        for (int t = threadIdx.x; t < n; t += blockDim.x) {
          float s = 0.f;
          for (int k = 0; k < D; ++k) s = fmaf(qs[k], lat(r0 + t, win, k), s);
          const T* kr = (const T*)a.krope + ((size_t)seq_row(a, b, r0 + t) * a.s.rope_heads + a.s.rope_head(h)) * R2;
          for (int j = 0; j < R2; ++j) s = fmaf(qrs[j], to_f32(kr[j]), s);
          sc[t] = s;
          mloc = fmaxf(mloc, s);
        }
        const float m_new = fmaxf(m_run, block_reduce(mloc, red, true));
        const float alpha = exp2f(m_run - m_new);  // 0 before the first run
        float lloc = 0.f;
        for (int t = threadIdx.x; t < n; t += blockDim.x) {
          const float p = exp2f(sc[t] - m_new);
          sc[t] = p;
          lloc += p;
        }
        l_run = l_run * alpha + block_reduce(lloc, red, false);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          const int k = threadIdx.x + i * blockDim.x;
          if (k >= D) continue;
          float acc = 0.f;
          for (int t = 0; t < n; ++t) acc = fmaf(sc[t], lat(r0 + t, win, k), acc);
          o[i] = o[i] * alpha + acc;
        }
        m_run = m_new;
        __syncthreads();  // sc is rewritten by the next run
      }
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int k = threadIdx.x + i * blockDim.x;
      if (k < D) po[(size_t)h * D + k] = o[i];
    }
    if (threadIdx.x == 0) {
      ml[MLS * h] = m_run;
      ml[MLS * h + 1] = l_run;
    }
    __syncthreads();
  }
}

// Partial result of one work item for the kernels whose four waves each hold DW latent columns of all
// 32 heads in the 32x32x16 MFMA accumulator layout (lane (h, hb): rows 8(e/4) + 4 hb + e%4 of each
// 32-column block).  fp32 format: O as is.  fp16 format: A = max |O| over the head's row (the four
// waves meet in `red`, LDS for 128 floats that no wave uses between the two barriers here) and O / A
// rounded to fp16, so the stored values lie in [-1, 1] whatever the latent magnitudes.  Split
// statistics: (m, l, A) per head.
template <int DW>
__device__ __forceinline__ void store_partial(const DecodeArgs& a, const f32x16 (&oacc)[DW / 32], float* red,
                                              char* stage, float m_run, float l_run, bool write_ml = true) {
  constexpr int NB = DW / 32, D = 4 * DW;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hb = lane >> 5, h = lane & 31;
  float* pml = (float*)(a.ws + a.plan.off_ml) + (size_t)blockIdx.x * 32 * MLS;
  float A = 1.f;
  if (a.plan.f16) {
    float am = 0.f;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(oacc[blk][e]));
    am = fmaxf(am, shfl_xor(am, 32));
    lds_barrier();
    if (hb == 0) red[w * 32 + h] = am;
    lds_barrier();
    A = fmaxf(fmaxf(red[h], red[32 + h]), fmaxf(red[64 + h], red[96 + h]));
    const float inv = A > 0.f ? 1.f / A : 0.f;
    _Float16* po = (_Float16*)(a.ws + a.plan.off_o) + (size_t)blockIdx.x * 32 * D;
    // through the wave's own staging area ([32 heads][DW] fp16, 16-byte chunks XOR-swizzled by row), so that
    // the rows leave as 16-byte stores, DW * 2 contiguous bytes per head, instead of 8-byte pieces 2 * D
    // bytes apart
    constexpr int CH = DW / 8;  // 16-byte chunks per row
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int kl = blk * 32 + 8 * e4 + 4 * hb;
        f16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (_Float16)(oacc[blk][4 * e4 + i] * inv);
        *(f16x4*)(stage + h * (DW * 2) + 16 * ((kl >> 3) ^ (h & (CH - 1))) + 2 * (kl & 7)) = v;
      }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 32 * CH / 64; ++i) {
      const int c = i * 64 + lane, row = c / CH, ch = c % CH;
      const u32x4 v = *(const u32x4*)(stage + row * (DW * 2) + 16 * (ch ^ (row & (CH - 1))));
      *(u32x4*)&po[(size_t)row * D + w * DW + 8 * ch] = v;
    }
  } else {
    float* po = (float*)(a.ws + a.plan.off_o) + (size_t)blockIdx.x * 32 * D;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int k = w * DW + blk * 32 + 8 * e4 + 4 * hb;
        *(f32x4*)&po[(size_t)h * D + k] =
            f32x4{oacc[blk][4 * e4], oacc[blk][4 * e4 + 1], oacc[blk][4 * e4 + 2], oacc[blk][4 * e4 + 3]};
      }
  }
  if (w == 0 && hb == 0) {
    if (write_ml) {
      pml[MLS * h] = m_run;
      pml[MLS * h + 1] = l_run;
    }
    pml[MLS * h + 2] = A;
  }
}

// ------------------------------------------------------------------ 2b. attention, MFMA path
// 32 heads, bf16.  Four waves split the latent width: wave w owns latent columns [w*DW, (w+1)*DW)
// for both products, so each wave stages only its own slice of every 32-token tile in LDS.
//   scores   S^T[n][h] = sum_k C[n][k] q~[h][k]      MFMA 32x32x16, A = C rows (ds_read_b128),
//                                                     B = q~ (registers); partial over the wave's
//                                                     columns, reduced per head through LDS: wave w
//                                                     sums heads 8w .. 8w+7 (4 scores per lane), adds
//                                                     their RoPE terms and owns their softmax
//   output   O^T[k][h] += sum_n C[n][k] P[h][n]      MFMA 32x32x16, A = C^T through the LDS
//                                                     transpose read, B = the owners' bf16 P from LDS
// Lane l owns head l%32 of the output accumulators; a raise of a head's running max reaches every wave
// as a rescale factor with a flag.  The next tile's rows and the RoPE keys of the lane's own head and
// tokens are prefetched into registers.  The dense 512-wide variant needs more than 256 registers per
// lane and runs at one wave per SIMD.
template <int DW, int R2, int FMT, bool PG>
__global__ __launch_bounds__(256, (DW == 128 && FMT == 0) ? 1 : 2) void decode_attn_mfma(DecodeArgs a, FuseArgs f) {
  constexpr int CP = DW + 16;  // LDS row pitch in elements (conflict-free b128 and transpose reads)
  constexpr int NS = DW / 16;  // score k-steps per wave
  constexpr int NB = DW / 32;  // output blocks per wave
  constexpr int D = 4 * DW;
  __shared__ __attribute__((aligned(16))) bf16 cbuf[4][32 * CP];
  __shared__ f32x4 sbuf[4][4][64];  // partial scores of every wave (then the end-of-item reduction)
  // per tile, from the owner of each head: bf16 probabilities [head][40] (the K order of the PV product),
  // and after a raise the per-head rescale factors with a flag per owner wave
  __shared__ __attribute__((aligned(16))) bf16 pbuf[32 * 40];
  __shared__ float abuf[32];
  __shared__ int fbuf[4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hb = lane >> 5, h = lane & 31;
  // the code layout (0 dense, 1 int4, 2 2-bit) and whether the format keeps a window of bf16 rows (fmt 2: 2-bit
  // codes, fmt 3: int4 codes)
  constexpr int CODEC = FMT == 3 ? 1 : FMT;
  constexpr bool HAS_WIN = FMT >= 2;
  static_assert(sizeof(cbuf) >= fuse_scratch_bytes(D, 32 * R2), "fused append scratch");
  if (blockIdx.x >= a.plan.max_items) {
    fused_orphans(a, f, (float*)cbuf);
    return;
  }
  WorkItem wi;
  if (!locate_item<HAS_WIN>(a, blockIdx.x, wi)) return;
  const int b = wi.b;
  // the tile loop runs over [wi.t0, wi.t1) and then (windowed formats) over the window [wi.w0, wi.w1), whose rows
  // come from the ring (the WIN instances of load_tile / step); t1 is the end of the current run
  int t1 = wi.t1;
  if (fused_rows(f, b, wi.t0, wi.t1, (float*)cbuf)) MLA_WAIT_VMCNT(0);

  // latent query operands (B of the score product) and the rotated query pairs
  const bf16* qt = (const bf16*)(a.ws + a.plan.off_qt) + ((size_t)b * 32 + h) * D + w * DW + 8 * hb;
  bf16x8 qv[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) qv[s] = *(const bf16x8*)(qt + 16 * s);
  // partial scores are reduced per head: this lane sums head xh = 8w + lane%8 at tokens xt0 .. xt0+3 of
  // each tile (source lane xsrc, entry xe4 of every wave's partial tile), adds their RoPE terms and runs
  // their softmax; its probabilities go to row xh of pbuf at kq .. kq+3
  const int xe4 = (lane >> 3) & 3, xhb = lane >> 5, xh = 8 * w + (lane & 7);
  const int xsrc = 32 * xhb + xh, xt0 = 8 * xe4 + 4 * xhb;
  const int kq = 16 * (xe4 >> 1) + 8 * xhb + 4 * (xe4 & 1);
  float qr[R2];
  {
    const float* qrp = (const float*)(a.ws + a.plan.off_qr) + ((size_t)b * 32 + xh) * R2;
#pragma unroll
    for (int c = 0; c < R2; ++c) qr[c] = qrp[c];
  }

  f32x16 oacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // a tile's 32 rows are consecutive cache rows (a page holds a multiple of 64 positions and tiles start
  // at multiples of 32 from the item's start), so a paged cache (PG) needs one row lookup per tile
  const size_t rowb = (size_t)cseq(a, b) * a.t_max;
  const bf16* krb = (const bf16*)a.krope;
  bf16* cw = cbuf[w];
  // RoPE key rows: NRH key heads of R2 dims (NRH = 32, or fewer when query heads share keys)
  const int NRH = a.s.rope_heads, KRW = NRH * R2;

  // ---- register prefetch, two tiles deep: this wave's latent slice and its share of the RoPE keys (loads
  // with the non-temporal hint: each cache row is read once per query)
  // 16-byte chunks per row of the wave's slice: 8 bf16, 32 int4 or 64 2-bit latents each
  constexpr int CPR = (CODEC == 0) ? DW / 8 : (CODEC == 1 ? DW / 32 : DW / 64);
  constexpr int CCH = 32 * CPR / 64;                  // chunks per lane
  typedef bf16 kv_t __attribute__((ext_vector_type(R2)));
  // per chunk: one fp16 scale (int4) or two (s, z) pairs of fp16 (2-bit: two groups of 32)
  using meta_t = std::conditional_t<CODEC == 2, uint2, uint16_t>;
  u32x4 creg[2][CCH];
  meta_t sreg[2][CCH];
  kv_t kreg[2][4];

  // full tiles: a wave-uniform tile base plus per-lane offsets that do not change per tile
  constexpr int RBY = CODEC == 0 ? D * 2 : (CODEC == 1 ? D / 2 : D / 4);  // latent bytes per cache row
  constexpr int MBY = CODEC == 2 ? 4 : 2;                                  // metadata bytes per group
  uint32_t coff[CCH], soff[CCH];
#pragma unroll
  for (int it = 0; it < CCH; ++it) {
    const int c = it * 64 + lane, row = c / CPR, q = c - row * CPR;
    coff[it] = row * RBY + (CODEC == 0 ? 2 * (w * DW + 8 * q) : (CODEC == 1 ? (w * DW + 32 * q) / 2 : (w * DW + 64 * q) / 4));
    soff[it] = MBY * (row * (D / 32) + (w * DW) / 32 + (CODEC == 2 ? 2 * q : q));
  }
  const uint32_t koff = ((xt0 * NRH + a.s.rope_head(xh)) * R2) * 2;  // RoPE keys of the lane's 4 tokens, head xh
  // window items (2-bit format) stage their bf16 rows straight from the ring in stage_window and
  // prefetch only the RoPE keys here
  auto load_tile = [&](auto bsel, auto winsel, int tt) {
    constexpr int B = decltype(bsel)::value;
    constexpr bool WIN = decltype(winsel)::value;
    // window tiles of a paged cache: the window starts at L - window, so a tile of its rows may cross a page
    // boundary; each lane looks up the rows of its 4 tokens (only their RoPE keys are loaded for a window
    // tile, the latents come from the ring).  (Gated first on the kernel's own constants, so that formats
    // without a window do not see this code at all.)
    if constexpr (PG && HAS_WIN) {
      if constexpr (WIN) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = min(tt + xt0 + i, t1 - 1);
          kreg[B][i] = __builtin_nontemporal_load(
              (const kv_t*)(krb + ((size_t)seq_row(a, b, tok) * NRH + a.s.rope_head(xh)) * R2));
        }
        return;
      }
    }
    // row0: the tile's first row (paged) or the sequence's (contiguous); tb: the tile's offset from it
    const size_t row0 = PG ? (size_t)__builtin_amdgcn_readfirstlane(seq_row(a, b, tt)) : rowb;
    const int tb = PG ? 0 : tt;
    if (tt + 32 <= t1) {
      const char* cb = (const char*)a.ckv + (row0 + tb) * RBY;
      const char* sb = (const char*)a.ckv_scale + (row0 + tb) * (D / 32) * MBY;
      const char* kb = (const char*)(krb + row0 * KRW) + (size_t)tb * KRW * 2 + koff;
      if constexpr (!WIN) {
#pragma unroll
        for (int it = 0; it < CCH; ++it) {
          creg[B][it] = __builtin_nontemporal_load((const u32x4*)(cb + coff[it]));
          if constexpr (CODEC != 0) sreg[B][it] = *(const meta_t*)(sb + soff[it]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) kreg[B][i] = __builtin_nontemporal_load((const kv_t*)(kb + i * KRW * 2));
      return;
    }
    if constexpr (!WIN) {
#pragma unroll
      for (int it = 0; it < CCH; ++it) {
        const int row = (it * 64 + lane) / CPR;
        const int tok = min(tt + row, t1 - 1);  // rows past the sequence repeat its last row (masked below)
        const char* cb = (const char*)a.ckv + (row0 + tok - tt + tb) * RBY;
        const char* sb = (const char*)a.ckv_scale + (row0 + tok - tt + tb) * (D / 32) * MBY;
        creg[B][it] = __builtin_nontemporal_load((const u32x4*)(cb + coff[it] - row * RBY));
        if constexpr (CODEC != 0) sreg[B][it] = *(const meta_t*)(sb + soff[it] - MBY * row * (D / 32));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int tok = min(tt + xt0 + i, t1 - 1);
      kreg[B][i] = __builtin_nontemporal_load((const kv_t*)(krb + row0 * KRW + ((size_t)(tok - tt + tb) * NRH + a.s.rope_head(xh)) * R2));
    }
  };
  auto stage_tile = [&](auto bsel) {
    constexpr int B = decltype(bsel)::value;
#pragma unroll
    for (int it = 0; it < CCH; ++it) {
      int c = it * 64 + lane, row = c / CPR, q = c - row * CPR;
      if constexpr (CODEC == 0) {
        *(u32x4*)&cw[row * CP + 8 * q] = creg[B][it];
      } else if constexpr (CODEC == 2) {
        const uint32_t wd[4] = {creg[B][it].x, creg[B][it].y, creg[B][it].z, creg[B][it].w};
        const uint32_t mg[2] = {sreg[B][it].x, sreg[B][it].y};
#pragma unroll
        for (int u = 0; u < 4; ++u) {  // word u: latents 16u .. 16u+15 of the chunk, group u / 2
          const float sc = __half2float(__ushort_as_half((unsigned short)(mg[u >> 1] & 0xFFFF)));
          const float z = __half2float(__ushort_as_half((unsigned short)(mg[u >> 1] >> 16)));
#pragma unroll
          for (int hlf = 0; hlf < 2; ++hlf) {
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              // the 2-bit code as an fp32 bit pattern 2^23 + code, minus 2^23: the code exactly
              const float code = __uint_as_float(((wd[u] >> (2 * (8 * hlf + e))) & 3u) | 0x4B000000u) - 8388608.0f;
              v[e] = (bf16)fmaf(code, sc, z);
            }
            *(bf16x8*)&cw[row * CP + 64 * q + 16 * u + 8 * hlf] = v;
          }
        }
      } else {
        float s = __half2float(__ushort_as_half(sreg[B][it]));
        const uint32_t wd[4] = {creg[B][it].x, creg[B][it].y, creg[B][it].z, creg[B][it].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            // nibble e of the word as a signed 4-bit code (sign-extending bit-field extract), converted
            // exactly, then times the scale as int4_dequant
            const float code = (float)(((int)(wd[u] << (28 - 4 * e))) >> 28);
            v[e] = (bf16)(code * s);
          }
          *(bf16x8*)&cw[row * CP + 32 * q + 8 * u] = v;
        }
      }
    }
  };

  // a tile of window rows: this wave's slice of rows tt .. tt+31 from the ring, global -> LDS
  // (in two halves of four 16-byte chunks per lane, to stay within the registers the prefetch leaves)
  auto stage_window = [&](int tt) {
    constexpr int WCPR = DW / 8, WCH = 32 * WCPR / 64, HALF = WCH / 2;  // chunks per row slice, per lane
    const bf16* ring = (const bf16*)a.ckv_win + (size_t)cseq(a, b) * a.win * D + w * DW;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      u32x4 tmp[HALF];
#pragma unroll
      for (int it = 0; it < HALF; ++it) {
        const int c = (hf * HALF + it) * 64 + lane, row = c / WCPR, q = c - row * WCPR;
        const int tok = min(tt + row, t1 - 1);  // rows past the range repeat its last row (masked below)
        tmp[it] = *(const u32x4*)(ring + (size_t)(tok % a.win) * D + 8 * q);
      }
#pragma unroll
      for (int it = 0; it < HALF; ++it) {
        const int c = (hf * HALF + it) * 64 + lane, row = c / WCPR, q = c - row * WCPR;
        *(u32x4*)&cw[row * CP + 8 * q] = tmp[it];
      }
    }
  };

  // one 32-token tile: stage registers -> LDS, refill them with the tile two ahead, then both products
  auto step = [&](auto bsel, auto winsel, int tt) {
    constexpr int B = decltype(bsel)::value;
    if constexpr (decltype(winsel)::value) stage_window(tt);
    else stage_tile(bsel);
    // RoPE terms of the lane's 4 tokens of head xh, taken before the registers refill
    float rt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < R2; ++c) acc = fmaf(qr[c], (float)kreg[B][i][c], acc);
      rt[i] = acc;
    }
    if (tt + 64 < t1) load_tile(bsel, winsel, tt + 64);
    __builtin_amdgcn_wave_barrier();

    // partial scores over this wave's latent columns, reduced per head through LDS
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8 av = *(const bf16x8*)&cw[(lane & 31) * CP + 16 * s + 8 * hb];
      sacc = mfma32(av, qv[s], sacc);
    }
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4)
      sbuf[w][e4][lane] = f32x4{sacc[4 * e4], sacc[4 * e4 + 1], sacc[4 * e4 + 2], sacc[4 * e4 + 3]};
    __syncthreads();
    f32x4 v = sbuf[0][xe4][xsrc];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) v += sbuf[ww][xe4][xsrc];
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = v[i] + rt[i];
    if (tt + 32 > t1) {  // last, partial tile: mask rows past the sequence
      asm volatile("" ::: "memory");  // keep this a branch (not if-converted into every tile)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tt + xt0 + i >= t1) sc[i] = -INFINITY;
    }
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = fmaxf(mt, shfl_xor(mt, 8));
    mt = fmaxf(mt, shfl_xor(mt, 16));
    mt = fmaxf(mt, shfl_xor(mt, 32));
    // the running max is raised only when a tile exceeds it by more than 2^8 (rare after the first
    // tile); a raise rescales the latent accumulators of that head (in every wave, through abuf)
    const bool raise = mt > m_run + 8.f;
    const bool any = __builtin_amdgcn_ballot_w64(raise) != 0;
    if (any) {
      asm volatile("" ::: "memory");  // keep this a branch (not if-converted into every tile)
      const float m_new = raise ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      if (lane < 8) abuf[xh] = alpha;
    }
    if (lane == 0) fbuf[w] = any ? 1 : 0;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m_run);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);  // per lane; the 8 lanes of a head are summed at the end
    bf16x4 pw;
#pragma unroll
    for (int i = 0; i < 4; ++i) pw[i] = (bf16)p[i];
    *(bf16x4*)&pbuf[xh * 40 + kq] = pw;
    __syncthreads();
    const int fl = fbuf[h >> 3];
    if (__builtin_amdgcn_ballot_w64(fl != 0)) {  // a raise in this tile: rescale those heads
      asm volatile("" ::: "memory");
      const float al = fl ? abuf[h] : 1.f;
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) oacc[blk] *= al;
    }
    bf16x8 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) pb[c] = *(const bf16x8*)&pbuf[h * 40 + 16 * c + 8 * hb];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
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
  auto run = [&](auto winsel, int ra, int rb) {
    t1 = rb;
    load_tile(B0{}, winsel, ra);
    if (ra + 32 < rb) load_tile(B1{}, winsel, ra + 32);
    for (int tt = ra; tt < rb; tt += 64) {
      step(B0{}, winsel, tt);
      if (tt + 32 < rb) step(B1{}, winsel, tt + 32);
    }
  };
  if (wi.t0 < wi.t1) run(std::false_type{}, wi.t0, wi.t1);
  if constexpr (HAS_WIN) {
    if (wi.w0 < wi.w1) run(std::true_type{}, wi.w0, wi.w1);
  }

  // row sums were kept per lane: sum the 8 lanes of each head, then its owner writes m and l
  l_run += shfl_xor(l_run, 8);
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  store_partial<DW>(a, oacc, (float*)sbuf, (char*)cbuf[w], m_run, l_run, false);  // cbuf[w]: this wave's own
  if (lane < 8) {
    float* pml = (float*)(a.ws + a.plan.off_ml) + (size_t)blockIdx.x * 32 * MLS;
    pml[MLS * xh] = m_run;
    pml[MLS * xh + 1] = l_run;
  }
}

// ------------------------------------------------------------------ 2c. attention, dense MFMA path with LDS DMA
// Same math as 2b, but every tile reaches LDS through global_load_lds_dwordx4 (no staging registers): a
// ring of three tile slots (separate LDS arrays, so the compiler can tell the slot being read from the
// slots still being filled), two tiles in flight while the third is used, explicit vmcnt waits.  Each
// wave moves its latent column slice, which only it reads (rows XOR-swizzled in 16-byte chunks so that
// both the row reads and the transpose reads are bank-conflict free), and the RoPE keys of rows
// 8w .. 8w+7 of the tile, which every wave reads after the tile's first barrier.  Rows past the sequence
// repeat its last row and are masked.
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


// Byte L of wave w's block inside a RoPE tile slot of the DMA kernel: the keys of heads 8w .. 8w+7, i.e.
// 32 pieces of 16*R2 bytes, one per token row of 64*R2 bytes.
template <int R2>
__device__ __forceinline__ char* own_at(char* kss, int w, int L) {
  return kss + (L / (16 * R2)) * (64 * R2) + w * (16 * R2) + L % (16 * R2);
}

// NSLOT tile slots in the DMA ring (2: one tile in flight while one is used; 3: two in flight).
// Partial scores are reduced per head: wave w sums, over the four column slices, the scores of heads
// 8w .. 8w+7 only (4 per lane), adds their RoPE terms and owns their softmax (running max, lazy raise,
// exp, row sum).  It hands the other waves bf16 probabilities (and, after a raise, the per-head rescale
// factors) through the part of the RoPE slot that only it reads, its own heads' keys, once it has read
// them; the next RoPE load into that slot therefore waits for the following tile's first barrier.  Per
// lane and tile: 4 partial-score reads, 4 exponentials, two probability reads, two barriers.
// CR (compact RoPE rows): the cache holds 8 RoPE key heads per row, query heads 4g .. 4g+3 sharing key
// head g (a layer converted from a grouped-query source); each wave loads its 8 rows of them (1 KB) into
// the end of its part of the RoPE slot and spreads them to the per-head layout before the tile's first
// barrier, so that everything after reads the per-head layout as usual.
template <int DW, int R2, int NSLOT, bool PG, bool CR = false>
__global__ __launch_bounds__(256, 1) void decode_attn_dma(DecodeArgs a, FuseArgs f) {
  static_assert(!CR || R2 == 8, "compact RoPE rows hold 8 key heads of 8 dims");
  constexpr int NS = DW / 16, NB = DW / 32, D = 4 * DW;
  constexpr int CSL = 32 * DW * 2;       // bytes of one wave's latent slice of a tile
  constexpr int KSL = 8 * 32 * R2 * 2;   // bytes of one wave's RoPE rows of a tile (per-head layout)
  constexpr int RRB = (CR ? 8 : 32) * R2 * 2;  // RoPE bytes per cache row
  constexpr int KDST = CR ? KSL - 1024 : 0;    // where a wave's RoPE rows land in its part of the slot
  constexpr int NC = CSL / 1024, NK = 8 * RRB / 1024;
  constexpr int RB = DW * 2;             // bytes per slice row
  constexpr float kRescale = 8.f;        // log2 headroom before the running max must be raised
  __shared__ __attribute__((aligned(1024))) char cs0[4 * CSL], cs1[4 * CSL], cs2[NSLOT > 2 ? 4 * CSL : 16];
  __shared__ __attribute__((aligned(1024))) char ks0[4 * KSL], ks1[4 * KSL], ks2[NSLOT > 2 ? 4 * KSL : 16];
  __shared__ f32x4 sbuf[4][4][64];  // partial scores of every wave, then the end-of-item reduction

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hb = lane >> 5, h = lane & 31;
  // a fused append's rows are formed in slot 2 (its first DMA is issued after the wait before the loop)
  constexpr bool CAN_FUSE = NSLOT > 2 && 4 * CSL >= fuse_scratch_bytes(D, 32 * R2);
  if (blockIdx.x >= a.plan.max_items) {
    if constexpr (CAN_FUSE) fused_orphans(a, f, (float*)cs2);
    return;
  }
  WorkItem wi;
  if (!locate_item<false>(a, blockIdx.x, wi)) return;
  const int b = wi.b, t0 = wi.t0, t1 = wi.t1;

  // DMA addresses: a wave-uniform tile base (SGPRs) plus per-lane offsets that do not change per tile
  // a tile's 32 rows are consecutive cache rows (pages hold multiples of 64 positions, tiles start at
  // multiples of 32 from the item's start): a paged cache (PG) needs one row lookup per tile, then
  // per-lane offsets from it
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const size_t rowb = (size_t)cseq(a, b) * a.t_max;
  // contiguous cache: the sequence's bases, a tile at a fixed offset from them
  const char* cbase = (const char*)a.ckv + (rowb * D + wu * DW) * 2;
  const char* kseq = (const char*)a.krope + rowb * RRB;
  const char* kbase = kseq + 8 * wu * RRB;
  uint32_t coff[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int off = 1024 * j + 16 * lane, row = off / RB;
    coff[j] = row * (D * 2) + 16 * swz<DW>(row, (off % RB) / 16);
  }
  // paged cache: lane i holds the pool page of the item's i-th page (an item of at most 2048 rows spans
  // at most 33 pages of 64 or more rows), read once here instead of once per tile
  int pid = 0, pg0 = 0;
  if constexpr (PG) {
    pg0 = t0 / a.pm.page;
    if ((pg0 + lane) * a.pm.page < t1 && pg0 + lane < a.pm.pps) {
      const int pg = a.pm.bt[(size_t)cseq(a, b) * a.pm.pps + pg0 + lane];
      pid = pg < 0 ? 0 : (pg >= a.pm.n_pages ? a.pm.n_pages - 1 : pg);
    }
  }
  const uint32_t c_lds[3] = {lds_addr_of(cs0) + wu * CSL, lds_addr_of(cs1) + wu * CSL, lds_addr_of(cs2) + wu * CSL};
  const uint32_t k_lds[3] = {lds_addr_of(ks0) + wu * KSL, lds_addr_of(ks1) + wu * KSL, lds_addr_of(ks2) + wu * KSL};
  auto issue_slot = [&](auto ssel, int tt, auto parts) {
    constexpr int SL = decltype(ssel)::value;
    constexpr int PARTS = decltype(parts)::value;  // 1: latent rows, 2: RoPE rows, 3: both
    // bases: the tile's rows (paged) or the sequence's rows (contiguous); tb = the tile's first position
    // relative to the base
    const char *cb0, *kt;
    int tb;
    if constexpr (PG) {
      const int pi = __builtin_amdgcn_readfirstlane(tt / a.pm.page - pg0);
      const size_t prow = (size_t)__builtin_amdgcn_readlane(pid, pi) * a.pm.page + tt % a.pm.page;
      cb0 = (const char*)a.ckv + (prow * D + wu * DW) * 2;
      kt = (const char*)a.krope + prow * RRB;
      tb = 0;
    } else {
      cb0 = cbase;
      kt = kseq;
      tb = tt;
    }
    if (!(PARTS & 1)) {
    } else if (tt + 32 <= t1) {
      const char* cb = cb0 + (size_t)tb * (D * 2);
#pragma unroll
      for (int j = 0; j < NC; ++j) dma16_nt(cb, coff[j], c_lds[SL] + 1024 * j);
    } else {  // last, partial tile: rows past the sequence repeat its last row (masked later)
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int off = 1024 * j + 16 * lane, row = off / RB;
        const int tok = min(tt + row, t1 - 1) - tt + tb;
        dma16_nt(cb0, (uint32_t)(tok * (D * 2) + 16 * swz<DW>(row, (off % RB) / 16)), c_lds[SL] + 1024 * j);
      }
    }
    // the wave's RoPE rows 8w .. 8w+7 of the tile are one contiguous block
    if (!(PARTS & 2)) {
    } else if (tt + 8 * wu + 8 <= t1) {
      const char* kb = (PG ? kt + 8 * wu * RRB : kbase) + (size_t)tb * RRB;
#pragma unroll
      for (int j = 0; j < NK; ++j) dma16_nt(kb, (uint32_t)(1024 * j + 16 * lane), k_lds[SL] + KDST + 1024 * j);
    } else {
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const int off = 1024 * j + 16 * lane, tk = off / RRB, within = off % RRB;
        const int tok = min(tt + 8 * wu + tk, t1 - 1) - tt + tb;  // row relative to the base, >= 0
        dma16_nt(kt, (uint32_t)(tok * RRB + within), k_lds[SL] + KDST + 1024 * j);
      }
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using PC = std::integral_constant<int, 1>;
  using PK = std::integral_constant<int, 2>;
  using PB = std::integral_constant<int, 3>;
  // the first tile and the query operands; issued before the item's new rows (if any) are known, so
  // that no workgroup waits for that look-up before its stream starts (a tile that holds a new row is
  // loaded again once the row is formed, below)
  const bf16* qt = (const bf16*)(a.ws + a.plan.off_qt) + ((size_t)b * 32 + h) * D + w * DW + 8 * hb;
  bf16x8 qv[NS];
  // this lane reduces head xh = 8w + lane%8 at tokens xt0 .. xt0+3 of each tile (from the partial
  // scores of source lane xsrc, entry xe4) and writes their probabilities at byte xpo of the wave's
  // probability block (the K order of the PV product, see pb below)
  const int xg = lane >> 3, xe4 = xg & 3, xhb = xg >> 2, xh = 8 * w + (lane & 7);
  const int xsrc = 32 * xhb + xh, xt0 = 8 * xe4 + 4 * xhb;
  const int xpo = ((2 * (xe4 >> 1) + xhb) * 8 + (lane & 7)) * 16 + 8 * (xe4 & 1);
  float qr[R2];
  const float* qrp = (const float*)(a.ws + a.plan.off_qr) + ((size_t)b * 32 + xh) * R2;
  bool started = false;
  auto start_loads = [&]() {
    if (started) return;
    started = true;
    issue_slot(S0{}, t0, PB{});
#pragma unroll
    for (int s = 0; s < NS; ++s) qv[s] = *(const bf16x8*)(qt + 16 * s);
#pragma unroll
    for (int c = 0; c < R2; ++c) qr[c] = qrp[c];
  };
  // new rows of a fused append in this item: reduced while the first tile and the query operands load,
  // and waited for with them below; when one lies in the first tile, that tile is loaded again after the
  // rows are written.  The sequence's last item first assumes a decode step's layout (the new rows are
  // the sequence's last t_new positions): its reduction's loads go out first, with the start position's,
  // and the item's own loads follow while they are in flight.
  int sp = -1;
  if constexpr (CAN_FUSE) {
    if (f.ks > 0 && t1 == wi.L && fused_rows_last(f, b, t0, wi.L, (float*)cs2, start_loads) > 0) sp = wi.L - f.a.t_new;
  }
  start_loads();
  if constexpr (CAN_FUSE) {
    if (f.ks > 0) {
      if (sp < 0 && fused_rows(f, b, t0, t1, (float*)cs2)) {
        sp = f.a.start_pos[b];  // the value fused_rows used (a cached re-read)
        sp = sp < 0 ? 0 : (sp > f.a.max_start ? f.a.max_start : sp);
      }
      if (sp >= 0 && sp < t0 + 32) {  // a new row in the first tile (only rows in [t0, t1) are written)
        MLA_WAIT_VMCNT(0);  // the rows are written and the first load has landed
        issue_slot(S0{}, t0, PB{});
      }
    }
  }
  // the query operands (and the first tile) must be complete before the loop: the compiler would
  // otherwise guard their first use inside the loop with a vmcnt(0) on every iteration
  MLA_WAIT_VMCNT(0);
  if (NSLOT > 2 && t0 + 32 < t1) issue_slot(S1{}, t0 + 32, PB{});

  f32x16 oacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) oacc[i] = f32x16{};
  // running max per head (log2 domain), raised lazily: p = exp2(s - m_run) may reach 2^kRescale
  float m_run = -INFINITY, l_run = 0.f;
  typedef bf16 kv_t __attribute__((ext_vector_type(R2)));

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
    if constexpr (CR) {
      // lane l holds key head l % 8 of row l / 8 (16 bytes); it writes them for query heads 4g .. 4g+3
      char* kr = kss + wu * KSL;
      const bf16x8 kv8 = *(const bf16x8*)(kr + KDST + 16 * lane);
      const int row = lane >> 3, g = lane & 7;
#pragma unroll
      for (int i = 0; i < 4; ++i) *(bf16x8*)(kr + row * (32 * R2 * 2) + (4 * g + i) * (R2 * 2)) = kv8;
    }
    __builtin_amdgcn_wave_barrier();
    if (ahead < t1) issue_slot(std::integral_constant<int, NX>{}, ahead, PC{});

    const char* cw = cs + w * CSL;
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8 av = *(const bf16x8*)(cw + slice_off<DW>(lane & 31, 16 * s + 8 * hb));
      sacc = mfma32(av, qv[s], sacc);
    }
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4)
      sbuf[w][e4][lane] = f32x4{sacc[4 * e4], sacc[4 * e4 + 1], sacc[4 * e4 + 2], sacc[4 * e4 + 3]};
    lds_barrier();  // partial scores and every wave's RoPE rows of this tile are in LDS
    // the RoPE slot of the previous tile is free now: every wave has read its probabilities
    if (ahead < t1) issue_slot(std::integral_constant<int, NX>{}, ahead, PK{});
    f32x4 v = sbuf[0][xe4][xsrc];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) v += sbuf[ww][xe4][xsrc];
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kv_t kk = *(const kv_t*)(kss + ((xt0 + i) * 32 + xh) * R2 * 2);
      float acc = v[i];
#pragma unroll
      for (int c = 0; c < R2; ++c) acc = fmaf(qr[c], (float)kk[c], acc);
      sc[i] = acc;
    }
    if (tt + 32 > t1) {  // last, partial tile: mask rows past the sequence
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tt + xt0 + i >= t1) sc[i] = -INFINITY;
    }
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = fmaxf(mt, shfl_xor(mt, 8));
    mt = fmaxf(mt, shfl_xor(mt, 16));
    mt = fmaxf(mt, shfl_xor(mt, 32));
    const bool raise = mt > m_run + kRescale;
    const bool any = __builtin_amdgcn_ballot_w64(raise) != 0;
    if (any) {
      asm volatile("" ::: "memory");
      const float m_new = raise ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      if (lane < 8) *(float*)own_at<R2>(kss, w, 512 + 4 * lane) = alpha;
    }
    if (lane == 0) *(int*)own_at<R2>(kss, w, 544) = any ? 1 : 0;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m_run);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    bf16x4 pv;
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = (bf16)p[i];
    *(bf16x4*)own_at<R2>(kss, w, xpo) = pv;
    lds_barrier();  // probabilities of every head
    const int fl = *(const int*)own_at<R2>(kss, h >> 3, 544);
    if (__builtin_amdgcn_ballot_w64(fl != 0)) {  // a raise in this tile: rescale those heads
      asm volatile("" ::: "memory");
      const float al = fl ? *(const float*)own_at<R2>(kss, h >> 3, 512 + 4 * (h & 7)) : 1.f;
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) oacc[blk] *= al;
    }
    bf16x8 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) pb[c] = *(const bf16x8*)own_at<R2>(kss, h >> 3, ((2 * c + hb) * 8 + (h & 7)) * 16);
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

  // row sums were kept per lane: sum the 8 lanes of each head, then its owner writes m and l
  l_run += shfl_xor(l_run, 8);
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  // (the wave's latent slice of slot 0 is its own and free: its last DMA has landed, its last PV is done)
  store_partial<DW>(a, oacc, (float*)sbuf, cs0 + wu * CSL, m_run, l_run, false);
  if (lane < 8) {
    float* pml = (float*)(a.ws + a.plan.off_ml) + (size_t)blockIdx.x * 32 * MLS;
    pml[MLS * xh] = m_run;
    pml[MLS * xh + 1] = l_run;
  }
}

// ------------------------------------------------------------------ 2d. attention, one tile stream per wave
// For shapes whose 16-token tiles are small (latent width 256 in bf16, int4 latents): the workgroup takes
// a work item and each wave a quarter of it in whole tiles, streamed through the wave's own LDS ring by
// direct-to-LDS DMA with no barrier.  Scores and the softmax are computed once per tile (no exchange
// between waves); the four waves merge (m, l, O) through LDS at the end, so the workspace holds one
// partial result per work item as for the other kernels.
//   scores  S[t][h] = C[t] . q~[h]: MFMA 16x16x32, A = latent rows (int4: dequantised in registers with
//           the (token, group) scale), B = q~ in registers, two blocks of 16 heads.  Lane chunk c of a
//           32-wide k-step covers latent columns [c D/4, (c+1) D/4), so its operands are contiguous.
//   PV      O^T[k][h] += C^T[k][t] P[t][h]: MFMA 32x32x16 over the tile's 16 tokens, A = transposed
//           latent reads (bf16: 16-bit transpose read; int4: 4-bit transpose read giving two column
//           blocks at once, codes scaled per token), B = P from a per-wave LDS scratch (P^T rows).
// Latent rows keep their 16-byte chunks XOR-swizzled by token so that both operand reads avoid bank
// conflicts.  Softmax uses a per-head reference set from the first tile's maximum; it is only raised
// when a head's tile sum leaves [0, 2^64] (scores 64 log2-units above it), which restarts the wave's
// range instead of rescaling O (the accumulators fill half the register file).
template <int D, int R2, int FMT, int NSLOT>
struct WaveTile {
  static constexpr int TT = 16;
  static constexpr int RB = FMT == 0 ? D * 2 : D / 2;      // latent bytes per token
  static constexpr int LB = TT * RB;
  static constexpr int SRB = FMT == 1 ? (D / 32) * 2 : 0;  // scale bytes per token
  static constexpr int SB = TT * SRB;
  static constexpr int KRB = 32 * R2 * 2;                  // RoPE key bytes per token
  static constexpr int KB = TT * KRB;
  static constexpr int SLOT = LB + SB + KB;
  static constexpr int PS = 32 * TT * 2;                   // P^T scratch [32 heads][16 tokens] bf16
  static constexpr int ST = FMT == 1 ? (D / 32) * TT * 2 : 0;  // scales transposed [group][token]
  static constexpr int WAVE_BYTES = NSLOT * SLOT + PS + ST;
  static constexpr int LDS_BYTES = 4 * WAVE_BYTES;
  static constexpr int NL = LB / 1024, NK = KB / 1024, NSC = SB / 256;  // DMA instructions per tile
  static constexpr int IPT = NL + NK + NSC;
  static constexpr int NSK = D / 32;  // score k-steps (lane chunks of D/4 columns, 8 per k-step)
  static constexpr int NB = D / 32;   // 32-column output blocks
  static constexpr int SWM = (RB / 16 < 16 ? RB / 16 : 16) - 1;
  static_assert(LB % 1024 == 0 && KB % 1024 == 0 && SB % 256 == 0, "DMA granularity");
  static_assert(LDS_BYTES <= 160 * 1024 && 4 * WAVE_BYTES >= 65536 + 2048, "LDS");  // merge: 2 KB + 64 KB
  static_assert(NSLOT == 2 || NSLOT == 3, "ring depth");
};

// Score operand from eight int4 codes in fp16, in the element order (n0, n4, n1, n5, n2, n6, n3, n7):
// each 16-bit half is built as fp16(1024 + (n ^ 8)) from the bits, 1032 subtracted exactly, then scaled
// (one rounding, 11-bit mantissa) with packed fp16 arithmetic.
__device__ __forceinline__ f16x8 dequant8h(uint32_t wd, uint32_t s2) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const uint32_t u = wd ^ 0x88888888u;
  const f16x2 off = {(_Float16)1032.f, (_Float16)1032.f}, sc = __builtin_bit_cast(f16x2, s2);
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 v = (__builtin_bit_cast(f16x2, ((u >> (4 * i)) & 0x000F000Fu) | 0x64006400u) - off) * sc;
    r[2 * i] = v[0];
    r[2 * i + 1] = v[1];
  }
  return r;
}
// Eight signed nibbles of `wd` (low first), element i times s[i], as bf16 (PV operand).
__device__ __forceinline__ bf16x8 dequant8v(uint32_t wd, const float* s) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)((float)(((int)(wd << (28 - 4 * i))) >> 28) * s[i]);
  return r;
}

template <int D, int R2, int FMT, int NSLOT, bool PG>
__global__ __launch_bounds__(256, 1) void decode_attn_wave(DecodeArgs a, FuseArgs f) {
  using W = WaveTile<D, R2, FMT, NSLOT>;
  constexpr int TT = W::TT, SWM = W::SWM;
  constexpr float kSumLimit = 18446744073709551616.f;  // 2^64
  __shared__ __attribute__((aligned(1024))) char lds[W::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  static_assert(W::LDS_BYTES >= fuse_scratch_bytes(D, 32 * R2), "fused append scratch");
  if (blockIdx.x >= a.plan.max_items) {
    fused_orphans(a, f, (float*)lds);
    return;
  }
  WorkItem wi;
  if (!locate_item<false>(a, blockIdx.x, wi)) return;
  const int b = wi.b;
  if (fused_rows(f, b, wi.t0, wi.t1, (float*)lds)) MLA_WAIT_VMCNT(0);
  // the wave's quarter of the item, in whole tiles
  const int ntile = (wi.t1 - wi.t0 + TT - 1) / TT, per = (ntile + 3) / 4;
  const int u0 = wi.t0 + TT * min(ntile, w * per);
  const int u1 = min(wi.t1, wi.t0 + TT * min(ntile, (w + 1) * per));
  const int nt = u1 > u0 ? (u1 - u0 + TT - 1) / TT : 0;

  char* mine = lds + w * W::WAVE_BYTES;
  char* pscr = mine + NSLOT * W::SLOT;  // P^T [32 heads][16 tokens]
  char* stp = pscr + W::PS;             // scales [group][16 tokens] (int4)
  const uint32_t mine_lds = lds_addr_of(mine);
  // a tile's TT rows are consecutive cache rows (pages hold multiples of 64 positions; tiles start at
  // multiples of TT from the item's start): a paged cache (PG) needs one row lookup per tile
  const size_t rowb = (size_t)cseq(a, b) * a.t_max;
  // tile j of the wave -> slot j % NSLOT; rows past the wave's range repeat its last row (masked later)
  auto issue = [&](int j) {
    // per-lane offsets are recomputed at every call (an opaque copy of the lane id keeps the compiler
    // from hoisting ~NL + NSC + NK of them into registers for the whole loop)
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int tt = u0 + TT * j;
    const uint32_t base = mine_lds + (j % NSLOT) * W::SLOT;
    const int last = u1 - 1;
    size_t prow;
    if constexpr (PG) prow = (size_t)__builtin_amdgcn_readfirstlane(seq_row(a, b, tt));
    else prow = rowb + tt;
    const char* lat = (const char*)a.ckv + prow * W::RB;
    const char* scl = FMT == 1 ? (const char*)a.ckv_scale + prow * W::SRB : (const char*)a.ckv;
    const char* kro = (const char*)a.krope + prow * W::KRB;
#pragma unroll
    for (int i = 0; i < W::NL; ++i) {
      const int off = 1024 * i + 16 * lane, row = off / W::RB, pos = (off % W::RB) / 16;
      const int tok = min(tt + row, last);
      dma16_nt(lat, (uint32_t)((tok - tt) * W::RB + 16 * (pos ^ (row & SWM))), base + 1024 * i);
    }
#pragma unroll
    for (int i = 0; i < W::NSC; ++i) {
      constexpr int SRB1 = W::SRB > 0 ? W::SRB : 1;  // (no scale rows for bf16 latents: NSC == 0)
      const int off = 256 * i + 4 * lane, row = off / SRB1, within = off % SRB1;
      const int tok = min(tt + row, last);
      dma4(scl, (uint32_t)((tok - tt) * W::SRB + within), base + W::LB + 256 * i);
    }
#pragma unroll
    for (int i = 0; i < W::NK; ++i) {
      const int off = 1024 * i + 16 * lane, row = off / W::KRB, within = off % W::KRB;
      const int tok = min(tt + row, last);
      dma16_nt(kro, (uint32_t)((tok - tt) * W::KRB + within), base + W::LB + W::SB + 1024 * i);
    }
  };
  constexpr int PF = NSLOT - 1;  // tiles in flight ahead of the one being computed

  // q~ operands (B of the score MFMA): head 16 hb2 + lane%16, columns c D/4 + 8 s .. +7 (c = lane/16);
  // int4 latents use fp16 operands with the columns in the dequantiser's order (0,4,1,5,2,6,3,7).
  // And the rotated query pairs of the lane's two heads.
  const int hl = lane & 15, c4 = lane >> 4;
  const bf16* qt = (const bf16*)(a.ws + a.plan.off_qt) + (size_t)b * 32 * D;
  bf16x8 qv[2][FMT == 0 ? W::NSK : 1];
  f16x8 qh[2][FMT == 1 ? W::NSK : 1];
#pragma unroll
  for (int hb2 = 0; hb2 < 2; ++hb2)
#pragma unroll
    for (int s = 0; s < W::NSK; ++s) {
      const bf16x8 v = *(const bf16x8*)(qt + (size_t)(16 * hb2 + hl) * D + c4 * (D / 4) + 8 * s);
      if (FMT == 0) {
        qv[hb2][FMT == 0 ? s : 0] = v;
      } else {
        constexpr int PERM[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
        for (int i = 0; i < 8; ++i) qh[hb2][FMT == 1 ? s : 0][i] = (_Float16)(float)v[PERM[i]];
      }
    }
  float qr[2][R2];
  {
    const float* qrp = (const float*)(a.ws + a.plan.off_qr) + (size_t)b * 32 * R2;
#pragma unroll
    for (int hb2 = 0; hb2 < 2; ++hb2)
#pragma unroll
      for (int c = 0; c < R2; ++c) qr[hb2][c] = qrp[(16 * hb2 + hl) * R2 + c];
  }
  MLA_WAIT_VMCNT(0);  // query operands complete before the loop
  asm volatile("" ::: "memory");

  f32x16 oacc[W::NB];
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  typedef bf16 kv_t __attribute__((ext_vector_type(R2)));

  bool restart;
  do {  // runs again only after a restart (see below)
  restart = false;
#pragma unroll
  for (int j = 0; j < PF; ++j)
    if (j < nt) issue(j);
#pragma unroll
  for (int g = 0; g < W::NB; ++g) oacc[g] = f32x16{};
  l_run[0] = l_run[1] = 0.f;
  bool any_pv = false;  // some tile has been added to O since the last (re)start
  for (int j = 0; j < nt; ++j) {
    // own DMA of tile j complete once only the later issued tiles may be outstanding
    if (NSLOT == 3 && j + 1 < nt) {
      MLA_WAIT_VMCNT(W::IPT);
    } else {
      MLA_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // the previous tile's LDS reads are done: its slot is free
    asm volatile("" ::: "memory");
    if (j + PF < nt) issue(j + PF);
    const char* lt = mine + (j % NSLOT) * W::SLOT;
    const char* sct = lt + W::LB;
    const char* kt = lt + W::LB + W::SB;
    const int tt = u0 + TT * j;
    const int st = lane & 15;  // this lane's token row for the score operand

    // ---- scores
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if (FMT == 0) {
#pragma unroll
      for (int s = 0; s < W::NSK; ++s) {
        const int chunk = c4 * (D / 32) + s;
        const bf16x8 av = *(const bf16x8*)(lt + st * W::RB + 16 * (chunk ^ (st & SWM)));
        sacc[0] = mfma16(av, qv[0][FMT == 0 ? s : 0], sacc[0]);
        sacc[1] = mfma16(av, qv[1][FMT == 0 ? s : 0], sacc[1]);
      }
    } else {
      constexpr int GPC = D / 128;  // 32-column groups per lane chunk (16-byte code chunks)
      uint32_t sc2[GPC];            // the token's scale of each group, in both fp16 halves
#pragma unroll
      for (int q4 = 0; q4 < GPC; ++q4) {
        const uint32_t hs = *(const unsigned short*)(sct + st * W::SRB + 2 * (c4 * GPC + q4));
        sc2[q4] = hs | (hs << 16);
      }
#pragma unroll
      for (int q4 = 0; q4 < GPC; ++q4) {
        const int chunk = c4 * GPC + q4;
        const u32x4 cw = *(const u32x4*)(lt + st * W::RB + 16 * (chunk ^ (st & SWM)));
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const f16x8 av = dequant8h(cw[s2], sc2[q4]);
          sacc[0] = mfma16h(av, qh[0][FMT == 1 ? 4 * q4 + s2 : 0], sacc[0]);
          sacc[1] = mfma16h(av, qh[1][FMT == 1 ? 4 * q4 + s2 : 0], sacc[1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // this tile's scales, transposed to [group][token] for the PV operand
      constexpr int GPL = (D / 32) / 4;  // groups per lane (64 lanes = 16 tokens x 4)
#pragma unroll
      for (int u = 0; u < GPL; ++u) {
        const int t = lane >> 2, g = GPL * (lane & 3) + u;
        *(__half*)(stp + (g * TT + t) * 2) = *(const __half*)(sct + t * W::SRB + 2 * g);
      }
    }
    // RoPE term of the lane's 2 x 4 (token, head) pairs: tokens 4 c4 + e, heads hl + 16 hb2
#pragma unroll
    for (int hb2 = 0; hb2 < 2; ++hb2)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const kv_t kk = *(const kv_t*)(kt + (4 * c4 + e) * W::KRB + (16 * hb2 + hl) * R2 * 2);
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < R2; ++c) acc = fmaf(qr[hb2][c], (float)kk[c], acc);
        sacc[hb2][e] += acc;
      }
    if (tt + TT > u1) {  // last, partial tile: mask rows past the range
      asm volatile("" ::: "memory");
#pragma unroll
      for (int hb2 = 0; hb2 < 2; ++hb2)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (tt + 4 * c4 + e >= u1) sacc[hb2][e] = -INFINITY;
    }

    // ---- softmax with a lazily raised reference (per head: lanes hl, hl+16, hl+32, hl+48 share it)
    float p[2][4], rs[2];
#pragma unroll
    for (int hb2 = 0; hb2 < 2; ++hb2) {
      rs[hb2] = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[hb2][e] = __builtin_amdgcn_exp2f(sacc[hb2][e] - m_run[hb2]);
        rs[hb2] += p[hb2][e];
      }
      rs[hb2] += shfl_xor(rs[hb2], 16);
      rs[hb2] += shfl_xor(rs[hb2], 32);
    }
    const bool raise0 = !(rs[0] <= kSumLimit), raise1 = !(rs[1] <= kSumLimit);
    if (__builtin_amdgcn_ballot_w64(raise0 || raise1)) {
      asm volatile("" ::: "memory");  // keep this a branch (first tile; later only for extreme inputs)
#pragma unroll
      for (int hb2 = 0; hb2 < 2; ++hb2) {
        float mt = fmaxf(fmaxf(sacc[hb2][0], sacc[hb2][1]), fmaxf(sacc[hb2][2], sacc[hb2][3]));
        mt = fmaxf(mt, shfl_xor(mt, 16));
        mt = fmaxf(mt, shfl_xor(mt, 32));
        if (hb2 == 0 ? raise0 : raise1) m_run[hb2] = fmaxf(m_run[hb2], mt);
      }
      if (any_pv) {
        // a head's scores outgrew its reference by ~2^64 after tiles were accumulated: start the
        // wave's range again with the raised references (O and l restart from zero; the loop only
        // comes back here after a further jump of that size, so restarts are bounded)
        MLA_WAIT_VMCNT(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
        restart = true;
        break;
      }
#pragma unroll
      for (int hb2 = 0; hb2 < 2; ++hb2) {
        rs[hb2] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[hb2][e] = __builtin_amdgcn_exp2f(sacc[hb2][e] - m_run[hb2]);
          rs[hb2] += p[hb2][e];
        }
        rs[hb2] += shfl_xor(rs[hb2], 16);
        rs[hb2] += shfl_xor(rs[hb2], 32);
      }
    }
    l_run[0] += rs[0];
    l_run[1] += rs[1];
    // P^T[head][token] in bf16: the lane's 4 tokens of each of its two heads
#pragma unroll
    for (int hb2 = 0; hb2 < 2; ++hb2) {
      bf16x4 pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[e] = (bf16)p[hb2][e];
      *(bf16x4*)(pscr + ((16 * hb2 + hl) * TT + 4 * c4) * 2) = pv;
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");

    // ---- PV: B = P^T[head l%32][tokens 8 hb .. +7]
    const int hb = lane >> 5, grp = lane >> 4, jl = lane & 15;
    const bf16x8 pbv = *(const bf16x8*)(pscr + ((lane & 31) * TT + 8 * hb) * 2);
    if (FMT == 0) {
#pragma unroll
      for (int g = 0; g < W::NB; ++g) {
        const int c0 = 32 * g + 16 * (grp & 1);
        const int col = c0 + 4 * (jl & 3);
        const int r0 = 8 * hb + (jl >> 2), r1 = r0 + 4;
        const bf16x4 x0 = lds_read_tr16((const bf16*)(lt + r0 * W::RB + 16 * ((col >> 3) ^ (r0 & SWM)) + 2 * (col & 7)));
        const bf16x4 x1 = lds_read_tr16((const bf16*)(lt + r1 * W::RB + 16 * ((col >> 3) ^ (r1 & SWM)) + 2 * (col & 7)));
        oacc[g] = mfma32(cat(x0, x1), pbv, oacc[g]);
      }
    } else {
      __builtin_amdgcn_wave_barrier();  // the transposed scales were written by other lanes
      asm volatile("" ::: "memory");
#pragma unroll
      for (int g = 0; g < W::NB; g += 2) {
        // addressing lane jl: token 8 hb + (jl & 7), block g + (jl >> 3), 16 columns from 16 (grp & 1)
        const int r = 8 * hb + (jl & 7), gg = g + (jl >> 3);
        typedef int v2i __attribute__((ext_vector_type(2)));
        const v2i t4 = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(lt + r * W::RB + 16 * (gg ^ (r & SWM)) + 8 * (grp & 1)));
        float s0[8], s1[8];
        {
          typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
          const f16x8 f0 = *(const f16x8*)(stp + (g * TT + 8 * hb) * 2);
          const f16x8 f1 = *(const f16x8*)(stp + ((g + 1) * TT + 8 * hb) * 2);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            s0[q] = (float)f0[q];
            s1[q] = (float)f1[q];
          }
        }
        oacc[g] = mfma32(dequant8v((uint32_t)t4.x, s0), pbv, oacc[g]);
        oacc[g + 1] = mfma32(dequant8v((uint32_t)t4.y, s1), pbv, oacc[g + 1]);
        __builtin_amdgcn_sched_barrier(0);  // bound the live operands (the accumulators fill half the file)
      }
    }
    any_pv = true;
  }
  } while (restart);

  // ---- merge the four waves: weights exp2(m_w - M) per head, then O summed over waves in LDS
  __syncthreads();  // every wave is done with its ring (its last wait drained its DMA)
  float* mm = (float*)lds;  // [4][32] references, then [4][32] weights
  float* ll = mm + 128;     // [4][32]
  float* wt = mm + 256;     // [4][32]
  if (lane < 16) {
    mm[w * 32 + lane] = m_run[0];
    mm[w * 32 + 16 + lane] = m_run[1];
    ll[w * 32 + lane] = l_run[0];
    ll[w * 32 + 16 + lane] = l_run[1];
  }
  __syncthreads();
  float* pml = (float*)(a.ws + a.plan.off_ml) + (size_t)blockIdx.x * 32 * MLS;
  if (w == 0 && lane < 32) {
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, mm[ww * 32 + lane]);
    float L = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = mm[ww * 32 + lane];
      const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      wt[ww * 32 + lane] = f;
      L = fmaf(f, ll[ww * 32 + lane], L);
    }
    pml[MLS * lane] = M;
    pml[MLS * lane + 1] = L;
  }
  __syncthreads();
  // O in rounds of 128 columns: every wave stores its raw accumulators (straight from the accumulation
  // registers), then wave w forms columns [32 w, 32 w + 32) as the weighted sum over the four waves
  // [4 waves][32 heads][128 columns], rows padded to OBP floats: the 32 heads a store instruction writes
  // then fall on different banks (a 128-float pitch put them all on the same ones)
  constexpr int OBP = 132;
  static_assert(2048 + 4 * 32 * OBP * 4 <= W::LDS_BYTES, "merge buffer");
  float* ob = (float*)(lds + 2048);
  const int h = lane & 31, hb = lane >> 5;
  // lane's heads: 8 it + lane / 8 (it = 0..3), 4 columns 32 w + 4 (lane % 8) of every 128-column round
  f32x4 vr[D / 128][4];
#pragma unroll
  for (int r = 0; r < D / 128; ++r) {
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x16& o = oacc[4 * r + gg];
        const int col = 32 * gg + 8 * e4 + 4 * hb;
        *(f32x4*)&ob[(w * 32 + h) * OBP + col] = f32x4{o[4 * e4], o[4 * e4 + 1], o[4 * e4 + 2], o[4 * e4 + 3]};
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int hh = 8 * it + (lane >> 3), col = 32 * w + 4 * (lane & 7);
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) v += wt[ww * 32 + hh] * *(const f32x4*)&ob[(ww * 32 + hh) * OBP + col];
      vr[r][it] = v;
    }
    __syncthreads();
  }
  const int col = 32 * w + 4 * (lane & 7);
  if (a.plan.f16) {  // A = max |O| per head: 4 columns x 8 lanes x rounds in a wave, then the 4 waves
    float* red = ob;  // [4 waves][32 heads]
    float am[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < D / 128; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) m = fmaxf(m, fabsf(vr[r][it][c]));
      m = fmaxf(m, shfl_xor(m, 1));
      m = fmaxf(m, shfl_xor(m, 2));
      am[it] = fmaxf(m, shfl_xor(m, 4));
      if ((lane & 7) == 0) red[w * 32 + 8 * it + (lane >> 3)] = am[it];
    }
    __syncthreads();
    _Float16* po = (_Float16*)(a.ws + a.plan.off_o) + (size_t)blockIdx.x * 32 * D;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int hh = 8 * it + (lane >> 3);
      const float A = fmaxf(fmaxf(red[hh], red[32 + hh]), fmaxf(red[64 + hh], red[96 + hh]));
      const float inv = A > 0.f ? 1.f / A : 0.f;
#pragma unroll
      for (int r = 0; r < D / 128; ++r) {
        f16x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (_Float16)(vr[r][it][c] * inv);
        *(f16x4*)&po[(size_t)hh * D + 128 * r + col] = v;
      }
      if (w == 0 && (lane & 7) == 0) pml[MLS * hh + 2] = A;
    }
  } else {
    float* po = (float*)(a.ws + a.plan.off_o) + (size_t)blockIdx.x * 32 * D;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int hh = 8 * it + (lane >> 3);
#pragma unroll
      for (int r = 0; r < D / 128; ++r) *(f32x4*)&po[(size_t)hh * D + 128 * r + col] = vr[r][it];
      if (w == 0 && (lane & 7) == 0) pml[MLS * hh + 2] = 1.f;
    }
  }
}

// Grid of the specialised attention kernels: the work items, plus one workgroup per sequence for the
// rows of a fused append that lie past its decode range.
inline dim3 attn_grid(const DecodeArgs& a, const FuseArgs& f) { return dim3(a.plan.max_items + (f.ks ? a.batch : 0)); }

template <int D, int R2, int FMT, int NSLOT>
void launch_wave_attn(const DecodeArgs& a, const FuseArgs& f, hipStream_t st) {
  if (a.pm.bt)
    hipLaunchKernelGGL((decode_attn_wave<D, R2, FMT, NSLOT, true>), attn_grid(a, f), dim3(256), 0, st, a, f);
  else
    hipLaunchKernelGGL((decode_attn_wave<D, R2, FMT, NSLOT, false>), attn_grid(a, f), dim3(256), 0, st, a, f);
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
  const float* ml = (const float*)(a.ws + a.plan.off_ml) + ((size_t)first * NH + h) * MLS;
  const float* po = (const float*)(a.ws + a.plan.off_o) + ((size_t)first * NH + h) * D;
  // running merge over groups of 8 splits; each group's (m, l) and latent rows are loaded in one round
  float M = -INFINITY, den = 0.f, acc[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float ms[8], ls[8], v[8][KPL];
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // unconditional loads (see merge_splits), masked slots re-read the last
      const int su = min(s0 + u, S - 1);
      ms[u] = s0 + u < S ? ml[(size_t)su * NH * MLS] : -INFINITY;
      ls[u] = ml[(size_t)su * NH * MLS + 1];
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const int k = lane + 64 * i;
        v[u][i] = k < D ? po[(size_t)su * NH * D + k] : 0.f;
      }
    }
    float gm = M;
#pragma unroll
    for (int u = 0; u < 8; ++u) gm = fmaxf(gm, ms[u]);
    // no branch here (the group's loads would be sunk past it): with nothing seen yet (gm = -inf) the
    // reference 0 gives every weight and the rescale exp2(-inf) = 0, leaving den and acc at zero
    const float ref = gm == -INFINITY ? 0.f : gm;
    const float c = exp2f(M - ref);  // rescale of what was merged so far (0 when M = -inf)
    den *= c;
#pragma unroll
    for (int i = 0; i < KPL; ++i) acc[i] *= c;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wv = exp2f(ms[u] - ref);  // 0 for an empty or masked split (ms = -inf)
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

// o = hi + lo, hi = bf16(o), lo = bf16(o - hi): KPL consecutive values to two LDS rows
template <int KPL>
__device__ __forceinline__ void write_hilo(bf16* hi, bf16* lo, const float (&v)[KPL]) {
  constexpr int NE = KPL < 8 ? KPL : 8;
  typedef __bf16 vec_t __attribute__((ext_vector_type(NE)));
#pragma unroll
  for (int c = 0; c < KPL / NE; ++c) {
    vec_t hv, lv;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      hv[e] = (bf16)v[NE * c + e];
      lv[e] = (bf16)(v[NE * c + e] - (float)hv[e]);
    }
    *(vec_t*)(hi + NE * c) = hv;
    *(vec_t*)(lo + NE * c) = lv;
  }
}

// 3c. merge and W_uv in one launch (bf16, latent width 256 or 512, head dim a multiple of 16).
//   Workgroup (head h, up to 16 consecutive sequences).  Each wave first issues the W_uv,h loads of its
//   blocks of 16 output dims (they do not depend on the merge), then merges: waves are spread over the
//   sequences (1, 2 or 4 waves per sequence, the waves of one sequence taking every wps-th group of 8
//   splits), each lane owning KPL = d_kv / 64 consecutive latent columns; waves sharing a sequence meet
//   in LDS.  The normalised row is split exactly into bf16 hi + lo parts (o = hi + lo up to the rounding
//   of lo) kept in LDS.  Projection: MFMA 16x16x32 with A = rows of W_uv,h (16 output dims) and B = the
//   sequences' hi and lo rows (16 columns, unused ones ignored).
constexpr int CB_MAXS = 16;  // sequences per combine workgroup (MFMA columns)
constexpr int CB_NW = 8;     // waves per combine workgroup

// Merge of the split partials (stats m, l, A and the row O/A) of one (sequence, head): groups g0,
// g0 + gstep, ... of G splits, the loads of a group all issued before any is used.  Returns the running
// max M, the denominator and the unnormalised row.
template <int KPL, bool F16>
__device__ __forceinline__ void merge_splits(const DecodeArgs& a, int first, int g0, int gstep, int S, int h,
                                             float& M, float& den, float (&acc)[KPL]) {
  constexpr int D = 64 * KPL, G = F16 ? 8 : 4;  // splits per group (loads in flight: 32 registers)
  const int NH = a.s.n_heads, lane = threadIdx.x & 63;
  typedef _Float16 hv_t __attribute__((ext_vector_type(KPL)));
  typedef float fv_t __attribute__((ext_vector_type(KPL)));
  typedef typename std::conditional<F16, hv_t, fv_t>::type pv_t;
  const float* ml = (const float*)(a.ws + a.plan.off_ml) + ((size_t)first * NH + h) * MLS;
  const size_t row0 = ((size_t)first * NH + h) * D + KPL * lane;
  M = -INFINITY;
  den = 0.f;
#pragma unroll
  for (int i = 0; i < KPL; ++i) acc[i] = 0.f;
  for (int s0 = G * g0; s0 < S; s0 += G * gstep) {
    float ms[G], ls[G], as[G];
    pv_t v[G];
    // every load of the group is issued unconditionally, so that they are all in flight together: a slot
    // past the sequence's last split re-reads that split and is masked out through its maximum below
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int su = min(s0 + u, S - 1);
      const float* e = ml + (size_t)su * NH * MLS;
      ms[u] = e[0];
      ls[u] = e[1];
      as[u] = F16 ? e[2] : 1.f;
      const size_t at = row0 + (size_t)su * NH * D;
      v[u] = *(const pv_t*)((const typename std::conditional<F16, _Float16, float>::type*)(a.ws + a.plan.off_o) + at);
    }
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (s0 + u >= S) ms[u] = -INFINITY;
    float gm = M;
#pragma unroll
    for (int u = 0; u < G; ++u) gm = fmaxf(gm, ms[u]);
    // no branch here (the group's loads would be sunk past it): with nothing seen yet (gm = -inf) the
    // reference 0 gives every weight and the rescale exp2(-inf) = 0, leaving den and acc at zero
    const float ref = gm == -INFINITY ? 0.f : gm;
    const float c = exp2f(M - ref);  // rescale of what was merged so far (0 when M = -inf)
    den *= c;
#pragma unroll
    for (int i = 0; i < KPL; ++i) acc[i] *= c;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const float wv = exp2f(ms[u] - ref);  // 0 for an empty or masked split (ms = -inf)
      den = fmaf(wv, ls[u], den);
      const float wa = wv * as[u];
#pragma unroll
      for (int i = 0; i < KPL; ++i) acc[i] = fmaf(wa, (float)v[u][i], acc[i]);
    }
    M = gm;
  }
}

// One workgroup of CB_NW waves per (head, part of the head's output dims, block of up to CB_MAXS
// sequences).  Waves share the sequences (CB_NW / nseq waves per sequence, each merging every wps-th
// group of splits, the groups' states combined through LDS), then project the block's merged rows with
// W_uv on MFMA: wave w computes 16 output dims of the workgroup's part (and more if the part is wider
// than 16 CB_NW) for all sequences of the block at once.  Splitting the output dims over gridDim.y
// workgroups repeats the merge but divides the W_uv rows each workgroup reads (the larger cost).
template <int KPL>
__global__ __launch_bounds__(64 * CB_NW) void decode_combine(DecodeArgs a, int sb) {
  constexpr int D = 64 * KPL, PITCH = D + 8;  // LDS row pitch in bf16 (16-byte shift per row)
  constexpr int NKS = D / 32;                  // k-steps per output block
  __shared__ __attribute__((aligned(16))) bf16 ohi[CB_MAXS][PITCH], olo[CB_MAXS][PITCH];
  __shared__ float st_m[CB_NW], st_d[CB_NW];
  __shared__ __attribute__((aligned(16))) float st_acc[CB_NW][64 * KPL];
  const int h = blockIdx.x, b0 = blockIdx.z * sb;
  const int NH = a.s.n_heads, dh = a.s.d_head, nblk = dh / 16 / gridDim.y, eb0 = blockIdx.y * nblk;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nseq = min(sb, a.batch - b0);
  const bf16* wuv = (const bf16*)a.w_uv + (size_t)h * dh * D;
  const int col = lane & 15, kq = 8 * (lane >> 4);
  bf16x8 wv[NKS];  // W_uv rows of output block w, loaded together with the wave's first merge loads
  auto load_wuv = [&]() {
    if (w < nblk) {
      const bf16* wrow = wuv + (size_t)(16 * (eb0 + w) + col) * D + kq;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) wv[ks] = *(const bf16x8*)(wrow + 32 * ks);
    }
  };

  // waves per sequence: a power of two, CB_NW / wps sequences in flight
  int wps = 1;
  while (wps < CB_NW && nseq * wps * 2 <= CB_NW) wps *= 2;
  int L0;  // length of sequence `lane` (one read serves the chunk, the item offsets and the counts)
  const int chunk = work_chunk(a, L0);
  const int cnt0 = item_count(a, lane, L0, chunk);
  bool loaded = false;
  for (int j = w / wps; j < nseq; j += CB_NW / wps) {
    const int b = b0 + j, q = w % wps;
    int before = lane < b ? cnt0 : 0;
    for (int i = lane + 64; i < b; i += 64) before += item_count(a, i, clamp_len(a, i), chunk);
    const int first = __builtin_amdgcn_readfirstlane(wave_isum(before));
    const int S = b < 64 ? __builtin_amdgcn_readfirstlane(__shfl(cnt0, b, 64)) : item_count(a, b, clamp_len(a, b), chunk);
    float M, den, acc[KPL];
    if (!loaded) {  // after the sequence lengths: waiting for them does not wait for these
      load_wuv();
      loaded = true;
    }
    if (a.plan.f16)
      merge_splits<KPL, true>(a, first, q, wps, S, h, M, den, acc);
    else
      merge_splits<KPL, false>(a, first, q, wps, S, h, M, den, acc);
    if (wps > 1) {  // partial state of this wave's split groups to LDS (one sequence per wave group)
      if (lane == 0) {
        st_m[w] = M;
        st_d[w] = den;
      }
#pragma unroll
      for (int i = 0; i < KPL / 4; ++i)
        *(f32x4*)&st_acc[w][KPL * lane + 4 * i] = f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
      continue;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int i = 0; i < KPL; ++i) acc[i] *= inv;
    write_hilo<KPL>(&ohi[j][KPL * lane], &olo[j][KPL * lane], acc);
  }
  if (!loaded) load_wuv();
  if (wps > 1) {
    __syncthreads();
    const int w0 = w;  // first wave of each group combines its group's states
    if (w0 % wps == 0 && w0 / wps < nseq) {
      float Mt = -INFINITY;
      for (int u = 0; u < wps; ++u) Mt = fmaxf(Mt, st_m[w0 + u]);
      float den = 0.f, acc[KPL];
#pragma unroll
      for (int i = 0; i < KPL; ++i) acc[i] = 0.f;
      for (int u = 0; u < wps; ++u) {
        const float c = st_m[w0 + u] == -INFINITY ? 0.f : exp2f(st_m[w0 + u] - Mt);
        den = fmaf(c, st_d[w0 + u], den);
#pragma unroll
        for (int i = 0; i < KPL; ++i) acc[i] = fmaf(c, st_acc[w0 + u][KPL * lane + i], acc[i]);
      }
      const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
      for (int i = 0; i < KPL; ++i) acc[i] *= inv;
      const int j = w0 / wps;
      write_hilo<KPL>(&ohi[j][KPL * lane], &olo[j][KPL * lane], acc);
    }
  }
  __syncthreads();

  auto project = [&](int eb, const bf16x8(&wk)[NKS]) {
    f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      r = mfma16(wk[ks], *(const bf16x8*)&ohi[col][32 * ks + kq], r);
      r = mfma16(wk[ks], *(const bf16x8*)&olo[col][32 * ks + kq], r);
    }
    // D[row = output dim 16 eb + 4 (lane / 16) + i][col = sequence b0 + lane % 16]
    if (col < nseq) {
      bf16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (bf16)r[i];
      *(bf16x4*)((bf16*)a.out + ((size_t)(b0 + col) * NH + h) * dh + 16 * eb + 4 * (lane >> 4)) = o;
    }
  };
  if (w < nblk) project(eb0 + w, wv);
  for (int eb = eb0 + w + CB_NW; eb < eb0 + nblk; eb += CB_NW) {  // parts wider than 16 * CB_NW
    const bf16* wrow = wuv + (size_t)(16 * eb + col) * D + kq;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) wv[ks] = *(const bf16x8*)(wrow + 32 * ks);
    project(eb, wv);
  }
}

template <typename T>
void launch_generic_attn(const DecodeArgs& a, hipStream_t st) {
  size_t shmem = (size_t)(a.s.d_kv + a.s.r2() + 1 + a.plan.cmax) * sizeof(float);
  dim3 grid(a.plan.max_items);
  if (a.s.fmt == 0)
    hipLaunchKernelGGL((decode_attn_generic<T, 0>), grid, dim3(256), shmem, st, a);
  else if (a.s.fmt == 1)
    hipLaunchKernelGGL((decode_attn_generic<T, 1>), grid, dim3(256), shmem, st, a);
  else if (a.s.fmt == 2)
    hipLaunchKernelGGL((decode_attn_generic<T, 2>), grid, dim3(256), shmem, st, a);
  else
    hipLaunchKernelGGL((decode_attn_generic<T, 3>), grid, dim3(256), shmem, st, a);
}

template <int DW, int R2>
void launch_mfma_attn(const DecodeArgs& a, const FuseArgs& f, hipStream_t st) {
  if (a.s.fmt == 0 && a.s.compact_rope()) {
    if constexpr (R2 == 8) {  // 8 key heads (decode_uses_mfma admits no other compact shape here)
      if (a.pm.bt)
        hipLaunchKernelGGL((decode_attn_dma<DW, R2, 3, true, true>), attn_grid(a, f), dim3(256), 0, st, a, f);
      else
        hipLaunchKernelGGL((decode_attn_dma<DW, R2, 3, false, true>), attn_grid(a, f), dim3(256), 0, st, a, f);
    }
  } else if (a.s.fmt == 0)
    if (a.pm.bt)
      hipLaunchKernelGGL((decode_attn_dma<DW, R2, 3, true>), attn_grid(a, f), dim3(256), 0, st, a, f);
    else
      hipLaunchKernelGGL((decode_attn_dma<DW, R2, 3, false>), attn_grid(a, f), dim3(256), 0, st, a, f);
  else if (a.s.fmt == 1)
    if (a.pm.bt)
      hipLaunchKernelGGL((decode_attn_mfma<DW, R2, 1, true>), attn_grid(a, f), dim3(256), 0, st, a, f);
    else
      hipLaunchKernelGGL((decode_attn_mfma<DW, R2, 1, false>), attn_grid(a, f), dim3(256), 0, st, a, f);
  else if (a.s.fmt == 2)
    if (a.pm.bt)
      hipLaunchKernelGGL((decode_attn_mfma<DW, R2, 2, true>), attn_grid(a, f), dim3(256), 0, st, a, f);
    else
      hipLaunchKernelGGL((decode_attn_mfma<DW, R2, 2, false>), attn_grid(a, f), dim3(256), 0, st, a, f);
  else if (a.pm.bt)
    hipLaunchKernelGGL((decode_attn_mfma<DW, R2, 3, true>), attn_grid(a, f), dim3(256), 0, st, a, f);
  else
    hipLaunchKernelGGL((decode_attn_mfma<DW, R2, 3, false>), attn_grid(a, f), dim3(256), 0, st, a, f);
}

}  // namespace

// Latent width 256 (bf16 or int4).  At width 512 the register-staged kernel is as fast for int4 (its
// dequantisation runs on two workgroups per CU) and the DMA ring kernel faster for bf16.
bool decode_uses_wave(const Shape& s) {
  return s.dtype == 1 && s.fmt <= 1 && s.n_heads == 32 && (s.r_pairs == 2 || s.r_pairs == 4) && s.d_kv == 256 &&
         !s.compact_rope();
}

// Specialised attention kernels that run the second phase of a split-K append (see FuseArgs).
static bool attn_takes_append(const Shape& s) {
  return s.fmt <= 1 && (decode_uses_wave(s) || (decode_uses_mfma(s) && (s.fmt == 1 || s.d_kv == 512)));
}

// (at latent width 256 the dense and int4 formats take the per-wave kernel; the 2-bit format runs the
// register-staged kernel at width 512 only)
// Shared RoPE keys: the int4 / 2-bit kernel indexes them per key head (any divisor of the heads); the
// dense DMA kernel has a compact instance for 8 key heads of 4 pairs.
bool decode_uses_mfma(const Shape& s) {
  return s.dtype == 1 && s.n_heads == 32 && (s.d_kv == 512 || (s.d_kv == 256 && s.fmt <= 1)) &&
         (s.r_pairs == 2 || s.r_pairs == 4) &&
         (!s.compact_rope() || (s.d_kv == 512 && (s.fmt != 0 || (s.rope_heads == 8 && s.r_pairs == 4))));
}

bool decode_uses_combine(const Shape& s) {
  return s.dtype == 1 && (s.d_kv == 256 || s.d_kv == 512) && s.d_head % 16 == 0 && s.d_head <= 512;
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
  p.target = (decode_uses_wave(s) || (decode_uses_mfma(s) && s.fmt == 0)) ? 256 : 512;
  p.cmax = 2048;
  p.f16 = decode_uses_combine(s) && (decode_uses_mfma(s) || decode_uses_wave(s)) ? 1 : 0;
  if (!decode_uses_mfma(s)) {  // the generic kernel keeps a chunk of scores in LDS
    const long long room = 65536 / 4 - (long long)s.d_kv - s.r2() - 1;
    const long long c = room > 0 ? (room / 64) * 64 : 64;
    if (c < p.cmax) p.cmax = (int)(c < 64 ? 64 : c);
  }
  // items = sum_b ceil(L_b / chunk) < sum_b L_b / chunk + batch; chunk >= sum / target unless clamped
  // (with a window, fmt 2, a sequence has at most that many: only its coded rows are cut)
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
  off = align256(off + (size_t)p.max_items * s.n_heads * MLS * 4);
  p.off_o = off;
  off = align256(off + (size_t)p.max_items * s.n_heads * s.d_kv * 4);
  p.off_ob = off;
  off = align256(off + (size_t)batch * s.n_heads * s.d_kv * 4);
  p.total = off;
  return p;
}

// Shape and alignment conditions of the MFMA query preparation (the fused step's prologue runs it).
static bool qprep_uses_mfma(const DecodeArgs& a) {
  return a.s.dtype == 1 && a.s.d_head <= 128 && a.s.d_head % 8 == 0 && a.s.d_kv % 128 == 0 &&
         ((uintptr_t)a.q & 15) == 0;
}

bool decode_step_fusable(const AppendArgs& aa, const DecodeArgs& da) {
  const int M = aa.batch * aa.t_new;
  return aa.ws != nullptr && append_ksplit(aa.s, M) > 0 && qprep_uses_mfma(da);
}

hipError_t launch_decode_step(const AppendArgs& aa, const DecodeArgs& da, hipStream_t st, int phase_mask) {
  const int M = aa.batch * aa.t_new;
  const int ks = append_ksplit(aa.s, M);
  const int nx = (aa.s.d_kv + aa.s.n_rope_cols() + 31) / 32;
  const int n_qp = da.s.n_heads * (da.s.d_kv / 128) * ((da.batch + 31) / 32);
  if (phase_mask & 1) hipLaunchKernelGGL(decode_step_prologue, dim3(nx * ks + n_qp), dim3(256), 0, st, aa, ks, da);
  // the split-K reduction runs inside the attention launch when its kernel takes it
  if (aa.t_new <= FUSE_MAXR && attn_takes_append(da.s) && !aa.pm.bt) {
    FuseArgs f{aa, ks};
    return launch_decode(da, st, phase_mask & 6, &f);
  }
  if (phase_mask & 2) {
    hipError_t e = launch_append_reduce(aa, ks, st);
    if (e != hipSuccess) return e;
  }
  return launch_decode(da, st, phase_mask & 6);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st, int phase_mask, const FuseArgs* fuse) {
  FuseArgs nf{};
  nf.ks = 0;
  const FuseArgs& f = fuse ? *fuse : nf;
  const int nh = a.s.n_heads;
  if (phase_mask & 1) {
    dim3 gq(nh, (a.s.d_kv + 63) / 64, (a.batch + QB - 1) / QB);
    if (qprep_uses_mfma(a))
      hipLaunchKernelGGL(decode_qprep_mfma, dim3(nh, a.s.d_kv / 128, (a.batch + 31) / 32), dim3(256), 0, st, a);
    else if (a.s.dtype == 0)
      hipLaunchKernelGGL(decode_qprep<float>, gq, dim3(64 * QW), 0, st, a);
    else
      hipLaunchKernelGGL(decode_qprep<bf16>, gq, dim3(64 * QW), 0, st, a);
  }
  if (phase_mask & 2) {
    if (decode_uses_wave(a.s)) {
      const int r = a.s.r_pairs;
      if (a.s.fmt == 1 && r == 4) launch_wave_attn<256, 8, 1, 3>(a, f, st);
      else if (a.s.fmt == 1) launch_wave_attn<256, 4, 1, 3>(a, f, st);
      else if (r == 4) launch_wave_attn<256, 8, 0, 2>(a, f, st);
      else launch_wave_attn<256, 4, 0, 3>(a, f, st);
    } else if (decode_uses_mfma(a.s)) {
      // latent width 512 (width 256 takes the per-wave kernel above)
      if (a.s.r_pairs == 4) launch_mfma_attn<128, 8>(a, f, st);
      else launch_mfma_attn<128, 4>(a, f, st);
    } else if (a.s.dtype == 0) {
      launch_generic_attn<float>(a, st);
    } else {
      launch_generic_attn<bf16>(a, st);
    }
  }
  if ((phase_mask & 4) && decode_uses_combine(a.s)) {
    // output dims in two parts when a head's W_uv rows exceed 64 KB and split into whole 16-wide blocks
    // (the rows each workgroup pulls through its CU bound the launch); sequences per workgroup: about one
    // workgroup per CU, at most 16 (the MFMA width)
    const bool wide = (size_t)a.s.d_head * a.s.d_kv * 2 > 65536;
    const int parts = wide && (a.s.d_head / 16) % 2 == 0 ? 2 : 1;
    const int sb = std::max(1, std::min(CB_MAXS, a.batch * nh * parts / 256));
    dim3 g(nh, parts, (a.batch + sb - 1) / sb);
    if (a.s.d_kv == 512)
      hipLaunchKernelGGL(decode_combine<8>, g, dim3(64 * CB_NW), 0, st, a, sb);
    else
      hipLaunchKernelGGL(decode_combine<4>, g, dim3(64 * CB_NW), 0, st, a, sb);
  } else if (phase_mask & 4) {
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
