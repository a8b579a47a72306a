// Device pieces shared by the append kernels and the fused decode step (gfx950).
#pragma once

#include <hip/hip_fp16.h>

#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int SM_MAXM = 64;  // few-token appends: at most 64 tokens (two 32-row MFMA blocks)
constexpr int KS_MAX = 16;   // model-width slices of the split-K append

// Cache row (contiguous or through the page table) and position of token m of an append (t_new
// consecutive tokens per sequence).
__device__ __forceinline__ int cache_row(const AppendArgs& a, int m, int* pos_out) {
  int b = m / a.t_new;
  int i = m - b * a.t_new;
  int sp = a.start_pos[b];
  sp = sp < 0 ? 0 : (sp > a.max_start ? a.max_start : sp);
  int pos = sp + i;
  *pos_out = pos;
  return cache_row_of(a.pm, a.t_max, b, pos);
}

// Output elements of the append epilogue, one function per kind so that every path that writes cache
// rows from fp32 projections runs the same arithmetic.
// Latent column n of a dense cache row.
__device__ __forceinline__ void store_latent(const AppendArgs& a, size_t row, int n, float v) {
  ((bf16*)a.ckv)[row * a.s.d_kv + n] = (bf16)v;
}
// int4 group g of a cache row from its 32 projected values v(c) = vals[c * stride].
__device__ __forceinline__ void store_group(const AppendArgs& a, size_t row, int g, const float* vals, int stride) {
  const int D = a.s.d_kv;
  float am = 0.f;
  for (int c = 0; c < 32; ++c) am = fmaxf(am, fabsf(vals[c * stride]));
  __half s = int4_scale(am);
  float sf = __half2float(s);
  uint8_t* codes = (uint8_t*)a.ckv + row * (D / 2) + 16 * g;
  for (int i = 0; i < 16; ++i) {
    int c0 = int4_code(vals[2 * i * stride], sf), c1 = int4_code(vals[(2 * i + 1) * stride], sf);
    codes[i] = (uint8_t)((c0 & 15) | ((c1 & 15) << 4));
  }
  ((__half*)a.ckv_scale)[row * (D / 32) + g] = s;
}
// ---- latents with a window of recent bf16 rows (fmt 2: 2-bit codes, fmt 3: int4 codes)
// Group of 32 latent values of one token (already rounded to bf16): z = fp16(min), s = fp16(max(max - z,
// 0) / 3), both saturating at the largest finite fp16; code = clamp(rint((x - z) / s), 0, 3) with an fp32
// subtraction and an IEEE fp32 division (s == 0: code 0).  Row `row` of the code store holds 8 bytes per
// group (element 4i + j at bits 2j of byte i) and one (s, z) pair of fp16 per group.
__device__ __forceinline__ __half sat_half(float v) {
  __half h = __float2half_rn(v);
  if (__hisinf(h)) h = __ushort_as_half((unsigned short)(v > 0.f ? 0x7BFF : 0xFBFF));
  return h;
}
__device__ __forceinline__ int int2_code(float x, float z, float s) {
  if (s == 0.f) return 0;
  const float q = rintf(__fdiv_rn(x - z, s));
  return (int)fminf(fmaxf(q, 0.f), 3.f);
}
__device__ __forceinline__ void code_group2(const float* v, uint8_t* codes, uint32_t* meta) {
  float lo = v[0], hi = v[0];
  for (int c = 1; c < 32; ++c) {
    lo = fminf(lo, v[c]);
    hi = fmaxf(hi, v[c]);
  }
  const __half zh = sat_half(lo);
  const float z = __half2float(zh);
  const __half sh = sat_half(__fdiv_rn(fmaxf(hi - z, 0.f), 3.0f));
  const float sc = __half2float(sh);
  for (int i = 0; i < 8; ++i) {
    int byte = 0;
    for (int j = 0; j < 4; ++j) byte |= int2_code(v[4 * i + j], z, sc) << (2 * j);
    codes[i] = (uint8_t)byte;
  }
  *meta = (uint32_t)__half_as_ushort(sh) | ((uint32_t)__half_as_ushort(zh) << 16);
}
__device__ __forceinline__ void store_group2(const AppendArgs& a, size_t row, int g, const float* v) {
  const int D = a.s.d_kv;
  code_group2(v, (uint8_t*)a.ckv + row * (D / 4) + 8 * g, (uint32_t*)a.ckv_scale + row * (D / 32) + g);
}
// A row group leaving (or never entering) the window of a windowed format, from its bf16 values v[0..31]:
// the 2-bit codec (fmt 2) or the int4 codec (fmt 3).
__device__ __forceinline__ void store_group_coded(const AppendArgs& a, size_t row, int g, const float* v) {
  if (a.s.fmt == 3)
    store_group(a, row, g, v, 1);
  else
    store_group2(a, row, g, v);
}
// Position that ring slot `slot` holds before an append that starts at position sp: the one in
// [sp - W, sp) congruent to slot modulo W (negative: the slot has not been used yet).
__device__ __forceinline__ int ring_occupant(int sp, int W, int slot) {
  const int base = sp - W;
  return base + (((slot - base) % W) + W) % W;
}
__device__ __forceinline__ int clamped_start(const AppendArgs& a, int b) {
  const int sp = a.start_pos[b];
  return sp < 0 ? 0 : (sp > a.max_start ? a.max_start : sp);
}
// Latent group g of the new token at position pos of sequence b, fp32 projections v(c) = vals[c * stride].
// The append ends at end = start + t_new.  A token at pos < end - W is coded at once; any other goes to
// ring slot pos % W, whose previous occupant (a position that leaves the window now) is coded first.
// Each (token, group) is handled by exactly one caller, and only it reads or writes that ring slot's
// group, so the read-before-write order needs no synchronisation.
__device__ __forceinline__ void store_group_win2(const AppendArgs& a, int b, int pos, int g, const float* vals,
                                                 int stride) {
  const int D = a.s.d_kv, W = a.win;
  const int sp = clamped_start(a, b);
  float v[32];
  for (int c = 0; c < 32; ++c) v[c] = (float)(bf16)vals[c * stride];
  if (pos < sp + a.t_new - W) {
    store_group_coded(a, (size_t)cache_row_of(a.pm, a.t_max, b, pos), g, v);
    return;
  }
  const int slot = pos % W;
  bf16* ring = (bf16*)a.ckv_win + ((size_t)b * W + slot) * D + 32 * g;
  const int p_old = ring_occupant(sp, W, slot);
  if (p_old >= 0) {
    float o[32];
    for (int c = 0; c < 32; ++c) o[c] = (float)ring[c];
    store_group_coded(a, (size_t)cache_row_of(a.pm, a.t_max, b, p_old), g, o);
  }
  for (int c = 0; c < 32; ++c) ring[c] = (bf16)v[c];
}
// The same for accumulator layouts in which the 32 lanes of each half-wave hold the 32 columns of one
// group of one token (column = lane % 32); `ok` is false for lanes past the last token.  Called by all 64
// lanes (the group reductions and the code packing are shuffles within each half).
__device__ __forceinline__ void store_lane_win2(const AppendArgs& a, bool ok, int b, int pos, int g, float val) {
  const int c = threadIdx.x & 31, D = a.s.d_kv, W = a.win;
  const float vb = (float)(bf16)val;
  bool direct = false, evict = false;
  int p_old = 0;
  float x = vb;
  bf16* ring = nullptr;
  if (ok) {
    const int sp = clamped_start(a, b);
    direct = pos < sp + a.t_new - W;
    if (!direct) {
      const int slot = pos % W;
      ring = (bf16*)a.ckv_win + ((size_t)b * W + slot) * D + 32 * g;
      p_old = ring_occupant(sp, W, slot);
      evict = p_old >= 0;
      if (evict) x = (float)ring[c];
    }
  }
  if (a.s.fmt == 3) {  // int4 codes of the bf16 values: group absmax, scale, nibbles packed by lane pairs
    float am = fabsf(x);
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) am = fmaxf(am, shfl_xor(am, m));
    const __half s4 = int4_scale(am);
    const int code = int4_code(x, __half2float(s4));
    const int partner = __shfl_xor(code, 1, 64);
    if (direct || evict) {
      const size_t row = (size_t)cache_row_of(a.pm, a.t_max, b, direct ? pos : p_old);
      if ((c & 1) == 0) ((uint8_t*)a.ckv)[row * (D / 2) + 16 * g + (c >> 1)] = (uint8_t)((code & 15) | ((partner & 15) << 4));
      if (c == 0) ((__half*)a.ckv_scale)[row * (D / 32) + g] = s4;
    }
    if (ok && !direct) ring[c] = (bf16)vb;
    return;
  }
  float lo = x, hi = x;
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) {
    lo = fminf(lo, shfl_xor(lo, m));
    hi = fmaxf(hi, shfl_xor(hi, m));
  }
  const __half zh = sat_half(lo);
  const float z = __half2float(zh);
  const __half sh = sat_half(__fdiv_rn(fmaxf(hi - z, 0.f), 3.0f));
  const float sc = __half2float(sh);
  const int code = int2_code(x, z, sc);
  const int c1 = __shfl_xor(code, 1, 64), c2 = __shfl_xor(code, 2, 64), c3 = __shfl_xor(code, 3, 64);
  if (direct || evict) {
    const size_t row = (size_t)cache_row_of(a.pm, a.t_max, b, direct ? pos : p_old);
    if ((c & 3) == 0)
      ((uint8_t*)a.ckv)[row * (D / 4) + 8 * g + (c >> 2)] = (uint8_t)(code | (c1 << 2) | (c2 << 4) | (c3 << 6));
    if (c == 0)
      ((uint32_t*)a.ckv_scale)[row * (D / 32) + g] =
          (uint32_t)__half_as_ushort(sh) | ((uint32_t)__half_as_ushort(zh) << 16);
  }
  if (ok && !direct) ring[c] = (bf16)vb;
}

// Retained RoPE pair at offset rel (even) of a row's RoPE block: rotate (x0, x1) at position pos.
__device__ __forceinline__ void store_rope_pair(const AppendArgs& a, size_t row, int pos, int rel, float x0, float x1) {
  const int r = a.s.r_pairs, R2 = a.s.r2(), NR = a.s.n_rope_cols(), half = a.s.d_head / 2;
  int h = rel / R2, jj = (rel - h * R2) >> 1;
  int p = load_pair(a.pair_idx, h * r + jj, half);
  float cs = a.rope_cos[(size_t)pos * half + p], sn = a.rope_sin[(size_t)pos * half + p];
  ((bf16*)a.krope)[row * NR + rel] = (bf16)(x0 * cs - x1 * sn);
  ((bf16*)a.krope)[row * NR + rel + 1] = (bf16)(x0 * sn + x1 * cs);
}

// Epilogue of the few-token paths for output columns n0 .. n0 + 31 (one int4 group or 16 RoPE pairs):
// element (m, c) of fin[m * ld + c] is column n0 + c of token m (fp32); rows[m] / poss[m] are the
// token's cache row and position.
__device__ __forceinline__ void append_epilogue(const AppendArgs& a, const float* fin, int ld, const int* rows,
                                                const int* poss, int n0, int M) {
  const int D = a.s.d_kv, NR = a.s.n_rope_cols();
  if (n0 < D) {
    if (a.s.fmt == 0) {
      for (int idx = threadIdx.x; idx < M * 32; idx += blockDim.x) {
        int m = idx >> 5, c = idx & 31;
        store_latent(a, (size_t)rows[m], n0 + c, fin[m * ld + c]);
      }
    } else if (a.s.fmt == 1) {
      for (int m = threadIdx.x; m < M; m += blockDim.x) store_group(a, (size_t)rows[m], n0 / 32, fin + m * ld, 1);
    } else {
      for (int m = threadIdx.x; m < M; m += blockDim.x) store_group_win2(a, m / a.t_new, poss[m], n0 / 32, fin + m * ld, 1);
    }
  } else {
    for (int idx = threadIdx.x; idx < M * 16; idx += blockDim.x) {
      int m = idx >> 4, cp = 2 * (idx & 15);
      int rel = n0 + cp - D;
      if (rel >= NR) continue;
      store_rope_pair(a, (size_t)rows[m], poss[m], rel, fin[m * ld + cp], fin[m * ld + cp + 1]);
    }
  }
}

// Split-K append, phase 2 for the tokens of sequence b at cache positions [p_lo, p_hi) (at most
// FUSE_MAXR, all of them new tokens of this append; sp = the sequence's clamped start position): each
// output column's KS partial sums are added in the order append_reduce uses, then the epilogue writes the
// cache rows, all columns at once.  Dense and int4 latents in contiguous caches only: the 2-bit format's
// append and a paged cache's are never fused into the attention launch (which keeps the page lookup out
// of the attention kernels).  The rows' RoPE tables (every pair of the rows' positions, when d_head <=
// 2 FUSE_HALF_MAX and there are at most 4 rows) and this thread's pair indices are loaded together with
// the partial sums, so that the whole reduction waits for one round of loads.  With `verify`, sp is a
// guess: the start position is loaded with the rest and, when its clamped value differs, the function
// returns false before writing anything.  `lds` holds fuse_scratch_bytes(D, NR) bytes.  Called by every
// thread of the workgroup.  The stores are not waited for: the caller waits for vmcnt 0 before any load
// that reads the rows.
constexpr int FUSE_MAXR = 8;
// Threads of the attention workgroups that run the reduction (a constant: blockDim is read from memory).
constexpr int FUSE_NT = 256;
constexpr int FUSE_HALF_MAX = 64;  // RoPE pairs per head whose tables are staged (d_head <= 128)
constexpr int fuse_scratch_bytes(int D, int NR) {
  return FUSE_MAXR * (D + NR + 4) * 4 + 2 * FUSE_MAXR * 4 + 2 * FUSE_MAXR * FUSE_HALF_MAX * 4;
}
struct NoLoads {
  __device__ void operator()() const {}
};
template <class Between = NoLoads>
__device__ __forceinline__ bool append_rows_fused(const AppendArgs& a, int KS, int b, int sp, int p_lo, int p_hi,
                                                  float* lds, bool verify = false, Between&& between = Between{}) {
  const int D = a.s.d_kv, NR = a.s.n_rope_cols(), N = D + NR, M = a.batch * a.t_new, ld = N + 4;
  const int R = p_hi - p_lo, half = a.s.d_head / 2, r = a.s.r_pairs, R2 = a.s.r2();
  int* rows = (int*)(lds + FUSE_MAXR * ld);
  int* poss = rows + FUSE_MAXR;
  float* cst = (float*)(poss + FUSE_MAXR);  // [R][half] cos, then [R][half] sin of the rows' positions
  float* sst = cst + FUSE_MAXR * FUSE_HALF_MAX;
  const int m0 = b * a.t_new + (p_lo - sp);
  const int sp_src = verify ? a.start_pos[b] : sp;  // issued with the loads below
  if ((int)threadIdx.x < R) {
    rows[threadIdx.x] = b * a.t_max + p_lo + threadIdx.x;
    poss[threadIdx.x] = p_lo + threadIdx.x;
  }
  // Every load below reads an in-bounds address whether or not its value is used, and no load sits
  // under a branch or next to a use of its value (either would make the compiler wait for it before the
  // next load goes out); the partial sums go out first, then the pair indices of the RoPE pairs this
  // thread writes and the rows' cos / sin entries (up to 4 rows: more take the per-pair loads below),
  // then the caller's own loads (between()).  Without RoPE columns (no pair table or RoPE tables to
  // read) those side loads read the first word of the partial sums instead.
  constexpr int RPT = 2;  // RoPE pairs per thread: 4 rows x 128 pairs over 256 threads
  constexpr int CPT = 1;  // table entries per thread: 4 rows x FUSE_HALF_MAX over 256 threads
  const bool staged = NR > 0 && half <= FUSE_HALF_MAX && R * (NR / 2) <= RPT * FUSE_NT &&
                      R * half <= CPT * FUSE_NT;
  const float* part = (const float*)a.ws;
  int praw[RPT];
  float cv[CPT], sv[CPT];
  auto side_loads = [&]() {
    const int32_t* pi_src = NR > 0 ? a.pair_idx : (const int32_t*)part;
    const float* cos_src = NR > 0 ? a.rope_cos : part;
    const float* sin_src = NR > 0 ? a.rope_sin : part;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int idx = threadIdx.x + i * FUSE_NT;
      const int rel = NR > 0 ? 2 * (idx % (NR / 2)) : 0, hh = NR > 0 ? rel / R2 : 0, jj = (rel - hh * R2) >> 1;
      praw[i] = pi_src[hh * r + jj];
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = min((int)threadIdx.x + i * FUSE_NT, R * half - 1), m = idx / half;
      const size_t at = NR > 0 ? (size_t)(p_lo + m) * half + (idx - m * half) : 0;
      cv[i] = cos_src[at];
      sv[i] = sin_src[at];
    }
  };
  // partial sums: rounds of 4 FUSE_NT columns, 16 bytes per thread and slice when rows hold whole 16-byte
  // chunks
  if (N % 4 == 0) {
    const size_t slice = (size_t)M * N / 4;  // one model-width slice of partial sums, in float4
    auto round = [&](int base, bool first) {
      const int f0 = base + 4 * (int)threadIdx.x, m = f0 / N, n = f0 - m * N;
      const bool ok = f0 < R * N;
      const f32x4* src = (const f32x4*)(part + (size_t)(m0 + (ok ? m : 0)) * N + (ok ? n : 0));
      f32x4 v[KS_MAX];
#pragma unroll
      for (int ks = 0; ks < KS_MAX; ++ks) v[ks] = src[min(ks, KS - 1) * slice];  // slices past KS unused
      if (first) {
        side_loads();
        between();
      }
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS_MAX; ++ks)
        if (ks < KS) sum += v[ks];
      if (ok) *(f32x4*)&lds[m * ld + n] = sum;
    };
    // the first round outside any loop: a loop around the caller's loads, whose values it does not use,
    // makes the compiler wait for every earlier load before entering it
    round(0, true);
    if (R * N > 4 * FUSE_NT)
      for (int base = 4 * FUSE_NT; base < R * N; base += 4 * FUSE_NT) round(base, false);
  } else {
    side_loads();
    between();
    for (int base = 0; base < R * N; base += 4 * FUSE_NT) {
      float v[4][KS_MAX];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int idx = base + it * FUSE_NT + threadIdx.x;
        const int m = idx / N, n = idx - m * N;
#pragma unroll
        for (int ks = 0; ks < KS_MAX; ++ks)
          v[it][ks] = (ks < KS && idx < R * N) ? part[((size_t)ks * M + m0 + m) * N + n] : 0.f;
      }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int idx = base + it * FUSE_NT + threadIdx.x;
        float sum = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS_MAX; ++ks) sum += v[it][ks];
        if (idx < R * N) lds[(idx / N) * ld + idx % N] = sum;
      }
    }
  }
  int pidx[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) pidx[i] = staged ? (praw[i] < 0 ? 0 : (praw[i] >= half ? half - 1 : praw[i])) : 0;
  if (staged) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = threadIdx.x + i * FUSE_NT;
      if (idx < R * half) {
        cst[idx] = cv[i];
        sst[idx] = sv[i];
      }
    }
  }
  lds_barrier();
  if (verify) {
    const int spc = sp_src < 0 ? 0 : (sp_src > a.max_start ? a.max_start : sp_src);
    if (spc != sp) return false;  // the same value in every thread: nothing was written to memory
  }
  if (a.s.fmt == 0) {
    for (int idx = threadIdx.x; idx < R * D; idx += FUSE_NT) {
      const int m = idx / D, n = idx - m * D;
      store_latent(a, (size_t)rows[m], n, lds[m * ld + n]);
    }
  } else {
    for (int idx = threadIdx.x; idx < R * (D / 32); idx += FUSE_NT) {
      const int m = idx / (D / 32), g = idx - m * (D / 32);
      store_group(a, (size_t)rows[m], g, lds + m * ld + 32 * g, 1);
    }
  }
  if (staged) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int idx = threadIdx.x + i * FUSE_NT;
      if (idx < R * (NR / 2)) {
        const int m = idx / (NR / 2), rel = 2 * (idx - m * (NR / 2));
        const float x0 = lds[m * ld + D + rel], x1 = lds[m * ld + D + rel + 1];
        const float cs = cst[m * half + pidx[i]], sn = sst[m * half + pidx[i]];
        bf16* kr = (bf16*)a.krope + (size_t)rows[m] * NR + rel;
        kr[0] = (bf16)(x0 * cs - x1 * sn);
        kr[1] = (bf16)(x0 * sn + x1 * cs);
      }
    }
  } else {
    for (int idx = threadIdx.x; idx < R * (NR / 2); idx += FUSE_NT) {
      const int m = idx / (NR / 2), rel = 2 * (idx - m * (NR / 2));
      store_rope_pair(a, (size_t)rows[m], poss[m], rel, lds[m * ld + D + rel], lds[m * ld + D + rel + 1]);
    }
  }
  lds_barrier();  // the scratch may be reused
  return true;
}

// Split-K append, phase 1, workgroup (bx: 32 output columns, by: one of KS slices of the model width):
// 4 waves split the slice, MFMA 32x32x16 over up to two 32-token blocks, and the workgroup's partial
// sums (fp32, [KS][M][N]) go to the workspace.  The reduction and epilogue run in append_reduce.
// LDS of one split-K append tile (the caller provides it, so that a launch that also runs other tiles can
// overlay their LDS).
struct SplitKLds {
  float red[4][SM_MAXM][32];
};
__device__ __forceinline__ void append_splitk_tile(const AppendArgs& a, int KS, int bx, int by, SplitKLds& sm) {
  auto& red = sm.red;
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
  for (int idx = threadIdx.x; idx < M * 32; idx += 256) {  // 256 threads (4 waves) per workgroup
    const int m = idx >> 5, c = idx & 31;
    if (n0 + c < N) part[(size_t)m * N + n0 + c] = red[0][m][c] + red[1][m][c] + red[2][m][c] + red[3][m][c];
  }
}

}  // namespace mla
