// Causal prefill over the latent cache on gfx950 (unabsorbed form).
//
// The MHA2MLA key-designs section (Paper-Notes ACL2025 page, 关键设计) recovers K_nope and V of head h
// from the latent: K_nope = c_kv . W_uk,h and V = c_kv . W_uv,h, with the retained RoPE keys cached
// separately.  For a whole prompt the minimum-work form rebuilds K and V once per token and runs plain
// causal attention with d_h = 128:
//   1. reconstruction GEMMs (MFMA): K[b,h,t,:] = NoPE dims from c_kv[b,t] . W_uk,h and the retained
//      dims copied from the cache's rotated k_rope, in the original head-dim order;
//      V^T[b,h,:,t] = W_uv,h^T . c_kv[b,t] (stored transposed, keys permuted within groups of 16)
//   2. causal flash attention (MFMA) over those rows with the query's retained pairs rotated.
#include <hip/hip_fp16.h>

#include "common.h"
#include "gemm.h"
#include "kernels.h"

namespace mla {

namespace {

// ------------------------------------------------------------------ 1. reconstruction GEMMs
// Through the shared GEMM main loop (gemm.h), K = d_kv, three stages (72 KB of LDS, two workgroups per
// CU so that one's epilogue overlaps the other's main loop).  The tile is staged in LDS in the output
// layout and written as whole 16-byte row chunks.
//   keys:   tile = 256 tokens x one head.  A = latent rows of the cache (token m = (b, t)), B = W_uk,h
//           rows: column e < d_nope is the GEMM result for NoPE dim nope_idx[e]; the remaining dims
//           come from the cache's rotated RoPE keys (pair j -> dims 2p_j, 2p_j + 1).  Written to
//           K[b, h, t, 0:128] in the ORIGINAL head-dim order, so queries need no permutation.
//   values: tile = one head's 128 dims x 256 tokens.  A = W_uv,h rows, B = latent rows (token n = (b, t),
//           t < s_pad; columns t >= S are written as zeros) -> V^T[b, h, e, pos(t)], keys permuted
//           within every 16 by pos() below.
using RecK = GemmCfg<256, 128, 3>;
using RecV = GemmCfg<128, 256, 3>;

// Position of key t in a V^T row: within each group of 16 keys the second and third runs of 4 swap
// places, which is the order in which the score MFMA's result registers hand out the keys (see the
// attention kernel), so P feeds the PV MFMA without any data movement.
__device__ __forceinline__ int vt_pos(int t) {
  const int k = t & 15;
  return (t & ~15) | (((k >> 2) & 1) << 3) | ((k >> 3) << 2) | (k & 3);
}

// Byte offset of element `col` of row `row` in a staging tile with `pitch`-byte rows, 16-byte chunks
// XOR-swizzled by the low row bits (rows 4 apart land in different banks).
__device__ __forceinline__ int stage_off(int row, int col, int pitch) {
  return row * pitch + 16 * ((col >> 3) ^ (row & 7)) + 2 * (col & 7);
}

// Hardware dispatch places workgroup k on XCD k % 8; logical tile t runs on XCD t / (total / 8), so
// consecutive logical tiles (which share an operand tile) share an L2.
__device__ __forceinline__ int xcd_tile(int bid, int total) {
  return (total & 7) == 0 ? (bid & 7) * (total >> 3) + (bid >> 3) : bid;
}

// (head, token tile) of reconstruction workgroup k.  When the head count is a multiple of 8, XCD x (which
// hardware dispatch gives workgroups k = x mod 8) takes heads x, x + 8, ... of every token tile, token tile
// by token tile: its heads' weight rows (n_h / 8 x 128 KB) stay in its L2 for the whole launch, and each
// latent tile is read once per XCD by the n_h / 8 workgroups that run it at the same time.  (With every head
// on every XCD, the 4 MB of all heads' weights did not fit beside the latent tiles in one L2 and were
// fetched again for every token tile.)
__device__ __forceinline__ void rec_tile(int bid, int total, int NH, int& hh, int& tile) {
  if ((NH & 7) == 0 && (total & 7) == 0) {
    const int x = bid & 7, j = bid >> 3, hpx = NH >> 3;
    tile = j / hpx;
    hh = x + 8 * (j - tile * hpx);
  } else {
    const int t = xcd_tile(bid, total);
    hh = t % NH;
    tile = t / NH;
  }
}

// Latent rows 0 .. S-1 of every sequence of a quantised cache, dequantised as the decode kernels do (int4:
// fp32(code) * fp32(scale); 2-bit: fp32(z + code * s) in one rounding; for the windowed formats the last
// `win` positions from the bf16 ring, slot t % win) and rounded to bf16 into the workspace [batch, S, d_kv]: the latent operand of the
// reconstruction GEMMs.  One lane per 8 latent values (16 output bytes).
__global__ __launch_bounds__(256) void prefill_stage_latent(PrefillArgs a) {
  const int D = a.s.d_kv, S = a.seq_len, per_row = D / 8;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)a.batch * S * per_row) return;
  const int c8 = (int)(idx % per_row);
  const size_t bt = idx / per_row;
  const int b = (int)(bt / S), t = (int)(bt - (size_t)b * S);
  bf16x8 v;
  if (a.s.fmt >= 2 && t >= S - min(S, a.win)) {
    v = *(const bf16x8*)((const bf16*)a.ckv_win + ((size_t)b * a.win + t % a.win) * D + 8 * c8);
  } else {
    const size_t row = (size_t)cache_row_of(a.pm, a.t_max, b, t);
    const _Float16* meta = (const _Float16*)a.ckv_scale;
    if (a.s.fmt == 1 || a.s.fmt == 3) {
      const uint32_t w = *(const uint32_t*)((const uint8_t*)a.ckv + row * (D / 2) + 4 * c8);
      const float sc = (float)meta[row * (D / 32) + c8 / 4];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (bf16)((float)((int)(w << (28 - 4 * i)) >> 28) * sc);
    } else {
      const uint32_t w = *(const uint16_t*)((const uint8_t*)a.ckv + row * (D / 4) + 2 * c8);
      const size_t g = (row * (D / 32) + c8 / 4) * 2;
      const float sc = (float)meta[g], z = (float)meta[g + 1];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (bf16)__builtin_fmaf((float)((w >> (2 * i)) & 3u), sc, z);
    }
  }
  *(bf16x8*)((bf16*)(a.ws + a.plan.off_lat) + ((size_t)b * S + t) * D + 8 * c8) = v;
}

__global__ __launch_bounds__(RecK::THREADS, 2) void rec_k_gemm(PrefillArgs a, int M) {
  __shared__ __attribute__((aligned(1024))) char lds[RecK::LDS_BYTES];
  __shared__ int dim_of[128];
  __shared__ int kept[64];
  __shared__ int crow[256], orow[256];  // cache row and output row of every token of the tile (-1: none)
  __shared__ int lrow[256];             // latent row of every token (the cache row, or the staged copy's)
  const int K = a.s.d_kv, S = a.seq_len, SP = a.plan.s_pad, dn = a.s.d_nope(), NH = a.s.n_heads;
  const int r = a.s.r_pairs, R2 = a.s.r2();
  int hh, tile;
  rec_tile(blockIdx.x, gridDim.x, NH, hh, tile);
  const int m0 = tile * 256;
  const int tid = threadIdx.x;
  if (tid < 128) dim_of[tid] = 0;  // duplicate pairs leave entries unset: keep them in range
  if (tid < 256) {
    const int m = m0 + tid;
    const int b = m / S, t = m - b * S;
    crow[tid] = m < M ? cache_row_of(a.pm, a.t_max, b, t) : -1;
    orow[tid] = m < M ? (b * NH + hh) * SP + t : -1;
    lrow[tid] = m < M ? (a.lat_staged ? m : crow[tid]) : -1;  // staged rows: [b * S + t]
  }
  const int gh = a.s.rope_head(hh), NRH = a.s.rope_heads;  // the head's RoPE key head
  __syncthreads();
  // the head's retained pairs (for the head-dim table) are loaded now and used after the GEMM: their round
  // trip runs under its first stages instead of before them (a __syncthreads would wait for them)
  const int kp = tid < r ? load_pair(a.pair_idx, gh * r + tid, 64) : 0;
  const int rp = tid < R2 ? load_pair(a.pair_idx, gh * r + (tid >> 1), 64) : 0;
  const bf16* ckv = (const bf16*)(a.lat_staged ? (const void*)(a.ws + a.plan.off_lat) : a.ckv);
  const int last = lrow[min(M - 1 - m0, 255)];
  auto a_row = [&](int i) {
    const int c = lrow[i];
    return ckv + (size_t)(c >= 0 ? c : last) * K;
  };
  auto b_row = [&](int i) -> const bf16* {  // rows past d_nope load valid rows (their results are unused)
    if (dn == 0) return ckv;
    return (const bf16*)a.w_uk + ((size_t)hh * dn + min(i, dn - 1)) * K;
  };
  // retained dims of the keys: the cache's rotated k_rope of (token, head).  Up to 16 of them per row: each
  // thread owns one row and loads them (4 bytes each) before the GEMM; they are written after it.
  const bf16* kr = (const bf16*)a.krope;
  uint32_t kv[8];
  const int kc = tid < 256 ? crow[tid] : -1;
  {
    const uint32_t* src = (const uint32_t*)(kr + ((size_t)(kc >= 0 ? kc : 0) * NRH + gh) * R2);
#pragma unroll
    for (int q = 0; q < 8; ++q) kv[q] = (kc >= 0 && R2 <= 16 && 2 * q < R2) ? src[q] : 0u;
  }
  f32x16 acc[RecK::FM][RecK::FN];
  gemm_tile_cfg<RecK>(lds, K, a_row, b_row, acc);
  __syncthreads();  // the ring is idle; its LDS becomes the staging tile [256 tokens][128 dims]
  // the head-dim table (ascending non-retained dims, then the retained pairs' dims), from the loads above
  for (int i = tid; i < 64; i += RecK::THREADS) kept[i] = 0;
  __syncthreads();
  if (tid < r) kept[kp] = 1;
  __syncthreads();
  if (tid < 64) {
    const int l = tid;
    const bool k0 = kept[l] != 0;
    const uint64_t m0 = __builtin_amdgcn_ballot_w64(k0);
    const uint64_t below = l ? (~0ull >> (64 - l)) : 0ull;
    if (!k0) {
      const int pos = l - __builtin_popcountll(m0 & below);
      dim_of[2 * pos] = 2 * l;
      dim_of[2 * pos + 1] = 2 * l + 1;
    }
  }
  if (tid < R2) dim_of[dn + tid] = 2 * rp + (tid & 1);
  __syncthreads();

  const int lane = tid & 63, w = tid >> 6, wm = w / RecK::WGN, wn = w % RecK::WGN;
#pragma unroll
  for (int j = 0; j < RecK::FN; ++j) {
    const int col = wn * RecK::WN + 32 * j + (lane & 31);
    if (col < dn) {
      const int d = dim_of[col];
#pragma unroll
      for (int i = 0; i < RecK::FM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = wm * RecK::WM + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          *(bf16*)(lds + stage_off(row, d, 256)) = (bf16)acc[i][j][e];
        }
    }
  }
  // retained dims from the registers loaded before the GEMM; more than 16 take a slower loop
  if (R2 <= 16 && tid < 256) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (2 * q < R2) *(uint32_t*)(lds + stage_off(tid, dim_of[dn + 2 * q], 256)) = kv[q];
  } else if (R2 > 16) {
    for (int idx = tid; idx < 256 * R2; idx += RecK::THREADS) {
      const int row = idx / R2, q = idx - row * R2, c = crow[row];
      const bf16 v = c >= 0 ? kr[((size_t)c * NRH + gh) * R2 + q] : (bf16)0.f;
      *(bf16*)(lds + stage_off(row, dim_of[dn + q], 256)) = v;
    }
  }
  __syncthreads();
  bf16* outk = (bf16*)(a.ws + a.plan.off_k);
  constexpr int KROWS = RecK::THREADS / 16;  // rows stored per round
#pragma unroll 4
  for (int it = 0; it < 256 / KROWS; ++it) {
    const int row = it * KROWS + (tid >> 4), ch = tid & 15, o = orow[row];
    if (o >= 0) *(u32x4*)(outk + (size_t)o * 128 + ch * 8) = *(const u32x4*)(lds + row * 256 + 16 * (ch ^ (row & 7)));
  }
}

__global__ __launch_bounds__(RecV::THREADS, 2) void rec_vt_gemm(PrefillArgs a, int N) {
  __shared__ __attribute__((aligned(1024))) char lds[RecV::LDS_BYTES];
  __shared__ int crow[256];  // cache row of every token column of the tile (clamped to valid rows)
  __shared__ size_t orow[32];  // output offset of every 8-position chunk (-1: none)
  const int K = a.s.d_kv, S = a.seq_len, SP = a.plan.s_pad, NH = a.s.n_heads;
  int hh, tile;
  rec_tile(blockIdx.x, gridDim.x, NH, hh, tile);
  const int n0 = tile * 256;
  const int tid = threadIdx.x;
  if (tid < 256) {
    const int n = min(n0 + tid, N - 1), b = n / SP, t = n - b * SP;
    crow[tid] = a.lat_staged ? b * S + min(t, S - 1) : cache_row_of(a.pm, a.t_max, b, min(t, S - 1));
    if (tid < 32) {
      const int nc = n0 + 8 * tid, bc = nc / SP, tc = nc - bc * SP;
      orow[tid] = nc < N ? ((size_t)(bc * NH + hh) * 128) * SP + tc : ~(size_t)0;
    }
  }
  __syncthreads();
  const bf16* ckv = (const bf16*)(a.lat_staged ? (const void*)(a.ws + a.plan.off_lat) : a.ckv);
  auto a_row = [&](int i) { return (const bf16*)a.w_uv + ((size_t)hh * 128 + i) * K; };
  auto b_row = [&](int i) { return ckv + (size_t)crow[i] * K; };
  f32x16 acc[RecV::FM][RecV::FN];
  gemm_tile_cfg<RecV>(lds, K, a_row, b_row, acc);
  __syncthreads();  // staging tile [128 dims][256 positions]

  const int lane = tid & 63, w = tid >> 6, wm = w / RecV::WGN, wn = w % RecV::WGN;
#pragma unroll
  for (int j = 0; j < RecV::FN; ++j) {
    const int col = wn * RecV::WN + 32 * j + (lane & 31), n = n0 + col, t = n % SP;
    const bool live = n < N && t < S;
    const int p = vt_pos(col);
#pragma unroll
    for (int i = 0; i < RecV::FM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * RecV::WM + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        *(bf16*)(lds + stage_off(row, p, 512)) = live ? (bf16)acc[i][j][e] : (bf16)0.f;
      }
  }
  __syncthreads();
  bf16* outv = (bf16*)(a.ws + a.plan.off_vt);
  constexpr int VROWS = RecV::THREADS / 32;  // rows stored per round
#pragma unroll 4
  for (int it = 0; it < 128 / VROWS; ++it) {
    const int row = it * VROWS + (tid >> 5), ch = tid & 31;
    const size_t o = orow[ch];  // eight positions never straddle two sequences (s_pad is a multiple of 64)
    if (o != ~(size_t)0) *(u32x4*)(outv + o + (size_t)row * SP) = *(const u32x4*)(lds + row * 512 + 16 * (ch ^ (row & 7)));
  }
}

// ------------------------------------------------------------------ 2. causal flash attention, d_h = 128
// Workgroup = (256 query rows, head, sequence), 8 waves of 32 rows, two per SIMD running half a tile
// apart so that one wave's softmax overlaps the other's MFMAs.  Key tiles of 64 stream through a 4-slot
// LDS ring by direct-to-LDS DMA (two tiles in flight), one workgroup barrier per tile:
//   S^T[key][q] = K[key] . Q[q]       MFMA 32x32x16, A = key rows from LDS, B = query rows in registers;
//                                      lane l owns query l%32, so row max / sum need one cross-half shuffle
//   O^T[e][q]  += V^T[e][key] P[q][key] MFMA 32x32x16, A = V^T rows from LDS, B = P straight from the
//                                      score registers (V^T keys are stored in the matching order)
// K rows (256 B) are stored with their 16-byte chunks XOR-swizzled by row, V^T rows (128 B) by row/2, so
// both operand reads are bank-conflict free.  Softmax uses a lazily raised reference instead of the
// running max: the tile's maximum is computed (and O rescaled) only when a row sum leaves [0, 2^16].  All query tiles of one (sequence, head) run
// on one XCD, longest first, so their shared K / V^T reads hit that XCD's L2.
constexpr int FQ = 256, FKV = 64, FNS = 4;
constexpr int KT_BYTES = FKV * 256, VT_BYTES = 128 * FKV * 2, SLOT = KT_BYTES + VT_BYTES;

// Schedule of a block of 16 operand reads from LDS and the 16 MFMAs that use them: ten reads ahead,
// then one MFMA per read, so that the matrix core does not wait for LDS latency between MFMAs (four
// waves of a CU read LDS at once; ten ahead measured ~5% faster than six).
__device__ __forceinline__ void lds_ahead_16() {
  __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);  // MFMA
}

// One query tile of one (sequence, head) pair, all 8 waves of the workgroup.
__device__ __forceinline__ void attend_query_tile(const PrefillArgs& a, char* ring, int pair, int qt) {
  const int S = a.seq_len, SP = a.plan.s_pad, NH = a.s.n_heads, r = a.s.r_pairs;
  const int b = pair / NH, h = pair - b * NH;
  const int q0 = qt * FQ;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hb = lane >> 5, ql = lane & 31;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int myq = q0 + 32 * w + ql;
  const int n_kv = min(SP / FKV, (min(q0 + FQ, S) - 1) / FKV + 1);

  // ---- DMA: wave w fills K rows 8w..8w+7 (two 1 KB instructions) and V^T rows 16w..16w+15 (two)
  const char* kg = (const char*)(a.ws + a.plan.off_k) + (size_t)pair * SP * 256;
  const char* vg = (const char*)(a.ws + a.plan.off_vt) + (size_t)pair * 128 * SP * 2;
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int krow = 8 * wu + 4 * i + (lane >> 4), kpos = lane & 15;
    koff[i] = krow * 256 + 16 * (kpos ^ (krow & 15));
    const int vrow = 16 * wu + 8 * i + (lane >> 3), vpos = lane & 7;
    voff[i] = vrow * SP * 2 + 16 * (vpos ^ ((vrow >> 1) & 7));
  }
  // the first eight retained pairs of the head, read before anything else is in flight
  constexpr int RP = 8;
  int pp[RP];
#pragma unroll
  for (int j = 0; j < RP; ++j)
    if (j < r) pp[j] = load_pair(a.pair_idx, a.s.rope_head(h) * r + j, 64);
  MLA_WAIT_VMCNT(0);
  const uint32_t ring_lds = lds_addr_of(ring);
  auto issue = [&](int kt) {
    const int slot = kt % FNS;
    const uint32_t kl = ring_lds + slot * SLOT + wu * 2048, vl = ring_lds + slot * SLOT + KT_BYTES + wu * 2048;
    const char* kb = kg + (size_t)kt * FKV * 256;
    const char* vb = vg + (size_t)kt * FKV * 2;
    dma16(kb, koff[0], kl);
    dma16(kb, koff[1], kl + 1024);
    dma16(vb, voff[0], vl);
    dma16(vb, voff[1], vl + 1024);
  };
  issue(0);
  if (n_kv > 1) issue(1);

  // ---- query operand: Q[row][16s + 8hb .. +7] in the original dim order, retained pairs rotated at the
  // row's position, scaled by log2(e)/sqrt(d_h)
  const int pos = min(myq, S - 1);
  const bf16* qrow = (const bf16*)a.q + (((size_t)b * S + pos) * NH + h) * 128 + 8 * hb;
  bf16x8 qv[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qv[s] = *(const bf16x8*)(qrow + 16 * s);
  // rotation factors of the first eight retained pairs, loaded in the same round as the query rows
  float pc[RP], ps[RP];
#pragma unroll
  for (int j = 0; j < RP; ++j)
    if (j < r) {
      pc[j] = a.rope_cos[(size_t)pos * 64 + pp[j]];
      ps[j] = a.rope_sin[(size_t)pos * 64 + pp[j]];
    }
  MLA_WAIT_VMCNT(0);  // query rows (and tiles 0, 1) complete before the loop
  {
    float x[8][8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int u = 0; u < 8; ++u) x[s][u] = (float)qv[s][u];
    // pair p = dims 2p, 2p+1 sits in k-step p/8, half-wave (p/4)%2, elements 2(p%4), 2(p%4)+1
    auto rotate = [&](int p, float cs, float sn) {
      if (hb != ((p >> 2) & 1)) return;
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int u2 = 0; u2 < 4; ++u2)
          if ((p >> 3) == s && (p & 3) == u2) {
            const float x0 = x[s][2 * u2], x1 = x[s][2 * u2 + 1];
            x[s][2 * u2] = x0 * cs - x1 * sn;
            x[s][2 * u2 + 1] = x0 * sn + x1 * cs;
          }
    };
#pragma unroll
    for (int j = 0; j < RP; ++j)
      if (j < r) rotate(pp[j], pc[j], ps[j]);
    for (int j = RP; j < r; ++j) {
      const int p = load_pair(a.pair_idx, a.s.rope_head(h) * r + j, 64);
      rotate(p, a.rope_cos[(size_t)pos * 64 + p], a.rope_sin[(size_t)pos * 64 + p]);
    }
    const float scale = kLog2e / sqrtf(128.f);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int u = 0; u < 8; ++u) qv[s][u] = (bf16)(x[s][u] * scale);
  }

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int wq_lo = q0 + 32 * wu, wq_hi = wq_lo + 31;  // wave-uniform (scalar) bounds
  constexpr float kSumLimit = 65536.f;
  f32x16 sacc[2];
  bf16x8 pb[2][2];

  // M phase of tile kt: O += P(kt-1) V(kt-1) (when tile kt-1 was visible), then S = K(kt) Q (when visible)
  auto phase_m = [&](int kt) {
    if (kt > 0 && (kt - 1) * FKV <= wq_hi) {
      const char* vs = ring + ((kt - 1) % FNS) * SLOT + KT_BYTES;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int row = db * 32 + ql;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const bf16x8 av = *(const bf16x8*)(vs + row * 128 + 16 * ((4 * kb + 2 * c + hb) ^ ((row >> 1) & 7)));
            oacc[db] = mfma32(av, pb[kb][c], oacc[db]);
          }
      }
      lds_ahead_16();
    }
    // keep the two products apart: hoisting the score operands above the PV product would raise the
    // register pressure past two waves per SIMD
    __builtin_amdgcn_sched_barrier(0);
    if (kt < n_kv && kt * FKV <= wq_hi) {
      const char* ks = ring + (kt % FNS) * SLOT;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        const int row = kb * 32 + ql;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          const bf16x8 av = *(const bf16x8*)(ks + row * 256 + 16 * ((2 * s8 + hb) ^ (row & 15)));
          sacc[kb] = mfma32(av, qv[s8], sacc[kb]);
        }
      }
      lds_ahead_16();
    }
  };
  // V phase of tile kt: mask, online softmax (lazy rescale), P(kt) in bf16 for the next M phase
  auto phase_v = [&](int kt) {
    if (kt < 0 || kt * FKV > wq_hi) return;
    const int kv0 = kt * FKV;
    if (kv0 + FKV - 1 > wq_lo || kv0 + FKV > S) {
      asm volatile("" ::: "memory");  // keep this a branch (only diagonal / last tiles pay for it)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kv0 + kb * 32 + 8 * (e >> 2) + 4 * hb + (e & 3);
          if (key > myq || key >= S) sacc[kb][e] = -INFINITY;
        }
    }
    // p = exp2(s - m_run) with the running reference m_run; the exact tile maximum is only needed when
    // a row's sum leaves [0, 2^16] (its largest term grew past 2^16, or m_run is still -inf on the
    // first tile, which gives inf / NaN): then m_run is raised to the maximum seen, O and l are
    // rescaled and the tile is recomputed.  The reference cancels in O / l either way.
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(sacc[kb][e] - m_run);
        rs += p;
        pb[kb][e >> 3][e & 7] = (bf16)p;
      }
    rs += shfl_xor(rs, 32);
    const bool raise = !(rs <= kSumLimit);
    if (__builtin_amdgcn_ballot_w64(raise)) {
      asm volatile("" ::: "memory");  // keep this a branch (rare after the first tile)
      float mt = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[kb][e]);
      mt = fmaxf(mt, shfl_xor(mt, 32));
      const float m_new = raise ? fmaxf(m_run, mt) : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      m_run = m_new;
      rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(sacc[kb][e] - m_run);
          rs += p;
          pb[kb][e >> 3][e & 7] = (bf16)p;
        }
      rs += shfl_xor(rs, 32);
    }
    l_run += rs;
  };

  // The two waves sharing a SIMD (w and w + 4) run half a tile apart: waves 0-3 pass the barrier of
  // tile kt before M(kt), waves 4-7 after M(kt-1), so that waves 4-7 run V(kt-1) while waves 0-3 run
  // M(kt) and M(kt) while waves 0-3 run V(kt).  Every wave meets the same n_kv + 1 barriers.  A slot is
  // refilled two tiles later, after barrier kt; the last reads of tile kt-2 (PV in M(kt-1)) precede that
  // barrier in both groups, so four slots suffice.
  const bool lagging = wu >= 4;
  auto sync_tile = [&](int kt) {
    // the own part of tile kt is complete once only tile kt+1's 4 loads may be outstanding
    if (kt + 1 < n_kv) {
      MLA_WAIT_VMCNT(4);
    } else {
      MLA_WAIT_VMCNT(0);
    }
    lds_barrier();
    if (kt + 2 < n_kv) issue(kt + 2);
  };
  if (lagging) sync_tile(0);
  for (int kt = 0; kt < n_kv; ++kt) {
    if (!lagging) sync_tile(kt);
    phase_m(kt);
    if (lagging) sync_tile(kt + 1);
    phase_v(kt);
  }
  if (!lagging) sync_tile(n_kv);
  phase_m(n_kv);  // PV of the last tile

  // ---- normalise and store through LDS (rows of 128 output dims, 16-byte stores)
  __syncthreads();  // all waves are done with the ring (no DMA is outstanding after the last tile)
  const float inv = 1.f / l_run;
  constexpr int OP = 136;  // row pitch in elements
  bf16* os = (bf16*)ring + w * 32 * OP;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (bf16)(oacc[db][4 * e4 + i] * inv);
      *(bf16x4*)&os[ql * OP + db * 32 + 8 * e4 + 4 * hb] = v;
    }
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  bf16* og = (bf16*)a.out;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = i * 64 + lane, row = c >> 4, ch = c & 15;
    const int t = q0 + 32 * w + row;
    if (t < S) *(u32x4*)(og + (((size_t)b * S + t) * NH + h) * 128 + ch * 8) = *(const u32x4*)&os[row * OP + ch * 8];
  }
}

// Workgroup i of a (sequence, head) pair takes query tiles nqt-1-i and i, so every workgroup carries
// the same causal work (nqt + 1 units of 256 x 256); a middle tile of an odd count runs alone.
// Hardware dispatch places workgroup k on XCD k % 8: all workgroups of a pair share one XCD (and its
// L2) when the pair count is a multiple of 8.
__global__ __launch_bounds__(512, 1) void prefill_attn(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char ring[FNS * SLOT];
  const int nqt = (a.seq_len + FQ - 1) / FQ, npw = (nqt + 1) / 2, pairs = a.batch * a.s.n_heads;
  const int k = blockIdx.x;
  int pair, i;
  if ((pairs & 7) == 0) {
    const int j = k >> 3;
    pair = (k & 7) + 8 * (j / npw);
    i = j % npw;
  } else {
    pair = k / npw;
    i = k % npw;
  }
  attend_query_tile(a, ring, pair, nqt - 1 - i);
  if (nqt - 1 - i != i) {
    __syncthreads();  // the ring and the output staging area are reused
    attend_query_tile(a, ring, pair, i);
  }
}

}  // namespace

bool prefill_supported(const Shape& s) {
  return s.dtype == 1 && s.fmt >= 0 && s.fmt <= 3 && s.d_head == 128 && s.d_kv % 64 == 0;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

PrefillPlan plan_prefill(const Shape& s, int batch, int seq_len) {
  PrefillPlan p{};
  p.s_pad = ((seq_len + FKV - 1) / FKV) * FKV;
  size_t off = 0;
  p.off_k = off;
  off = align256(off + (size_t)batch * s.n_heads * p.s_pad * 128 * 2);
  p.off_vt = off;
  off = align256(off + (size_t)batch * s.n_heads * 128 * p.s_pad * 2);
  p.off_lat = off;
  if (s.fmt != 0) off = align256(off + (size_t)batch * seq_len * s.d_kv * 2);
  p.total = off;
  return p;
}

hipError_t launch_prefill(const PrefillArgs& a0, hipStream_t st) {
  PrefillArgs a = a0;
  const int S = a.seq_len, B = a.batch, NH = a.s.n_heads, SP = a.plan.s_pad;
  if (a.s.fmt != 0) {  // quantised latent: dequantised copy first
    const size_t lanes = (size_t)B * S * (a.s.d_kv / 8);
    hipLaunchKernelGGL(prefill_stage_latent, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, st, a);
    a.lat_staged = 1;
  }
  hipLaunchKernelGGL(rec_k_gemm, dim3(((B * S + 255) / 256) * NH), dim3(RecK::THREADS), 0, st, a, B * S);
  hipLaunchKernelGGL(rec_vt_gemm, dim3(NH * ((B * SP + 255) / 256)), dim3(RecV::THREADS), 0, st, a, B * SP);
  const int nqt = (S + FQ - 1) / FQ;
  hipLaunchKernelGGL(prefill_attn, dim3(B * NH * ((nqt + 1) / 2)), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
