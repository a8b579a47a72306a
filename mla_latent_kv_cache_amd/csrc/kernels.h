// Internal launch interface between the C-ABI layer (api.cpp) and the gfx950 kernels.
// Everything here is validated by the caller; launchers only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

struct Shape {
  int d_model, n_heads, d_head, r_pairs, d_kv;
  int dtype;  // 0 f32, 1 bf16
  int fmt;    // 0 dense, 1 int4 g32, 2 int2 g32 with a bf16 window of recent rows, 3 int4 g32 with that window
  int rope_heads;  // RoPE key heads (n_heads, or a divisor: consecutive query heads share one)
  __host__ __device__ int r2() const { return 2 * r_pairs; }
  __host__ __device__ int d_nope() const { return d_head - 2 * r_pairs; }
  __host__ __device__ int n_rope_cols() const { return rope_heads * 2 * r_pairs; }
  // RoPE key head (row of the pair table and of W_krope, slot of a cache row's keys) of query head h
  __host__ __device__ int rope_head(int h) const { return h / (n_heads / rope_heads); }
  __host__ __device__ bool compact_rope() const { return rope_heads != n_heads; }
};

// Where the rows of a cache sequence live: contiguous (b * t_max + pos) when bt is null, else through a
// page table [sequences, pps] of page ids (clamped to [0, n_pages)) over a pool of `page`-row pages.
struct PageMap {
  const int32_t* bt;
  int page, pps, n_pages;
};
__device__ __forceinline__ int cache_row_of(const PageMap& pm, int t_max, int cb, int pos) {
  if (!pm.bt) return cb * t_max + pos;
  int pg = pm.bt[(size_t)cb * pm.pps + pos / pm.page];
  pg = pg < 0 ? 0 : (pg >= pm.n_pages ? pm.n_pages - 1 : pg);
  return pg * pm.page + pos % pm.page;
}

struct AppendArgs {
  Shape s;
  const void *x, *w_dkv, *w_krope;
  const int32_t* pair_idx;
  const float *rope_cos, *rope_sin;
  const int32_t* start_pos;
  int batch, t_new, max_start, t_max;
  void *ckv, *ckv_scale, *krope;
  char* ws = nullptr;  // optional workspace (few-token appends split the model width over workgroups)
  void* ckv_win = nullptr;  // fmt 2: ring of the last `win` rows per sequence [batch, win, d_kv] bf16
  int win = 0;
  PageMap pm{};
};

// Few-token append with a workspace: number of model-width slices and the workspace it needs
// (0 when the shape does not use the split path).
int append_ksplit(const Shape& s, int tokens);
size_t append_workspace_bytes(const Shape& s, int tokens);

// Decode work split.  The kernels read the batch's lengths L_b on the device and cut its tokens into
// work items of `chunk` tokens: chunk = clamp(round_up(ceil(sum_b L_b / target), 32), 64, cmax), and
// sequence b owns ceil(L_b / chunk) consecutive items (in batch order).  With a window of bf16 rows
// (fmt 2) only the coded positions [0, L_b - W_b), W_b = min(L_b, win), are cut, and the sequence's last
// item also reads the window [L_b - W_b, L_b) (one item when there are no coded positions).  Ragged batches therefore
// spread over about `target` workgroups like uniform ones.  max_items bounds the item count for any
// lengths within max_seq_len; the per-item partial results are laid out by item.
struct DecodePlan {
  int target;     // desired number of work items
  int cmax;       // largest chunk (multiple of 64)
  int max_items;  // grid size of the attention launch, >= 1
  int f16;        // partial latent rows stored as fp16 O / A with A = max |O| of the row (else fp32 O)
  size_t off_qt, off_qr, off_ml, off_o, off_ob, total;
};
DecodePlan plan_decode(const Shape& s, int batch, int max_seq_len);

struct DecodeArgs {
  Shape s;
  const void *q, *w_uk, *w_uv;
  const int32_t* pair_idx;
  const float *rope_cos, *rope_sin;
  const void *ckv, *ckv_scale, *krope;
  int batch, t_max, max_seq_len;
  const int32_t* seq_lens;
  void* out;
  char* ws;
  DecodePlan plan;
  const void* ckv_win = nullptr;  // fmt 2: ring of the last `win` rows per sequence [batch, win, d_kv] bf16
  int win = 0;
  PageMap pm{};
  // queries per cache sequence: `batch` counts queries, query v reads cache sequence v / qn with
  // length seq_lens[v / qn] - (qn - 1 - v % qn) (multi-query decode; 1 otherwise)
  int qn = 1;
};

// Prefill workspace: K [b, h, s_pad, 128] and V^T [b, h, 128, s_pad] bf16, s_pad = seq_len rounded up
// to the 64-key tile; for a quantised latent (fmt 1, 2) also the dequantised latent rows [b, seq_len, d_kv]
// bf16 that the reconstruction reads.
struct PrefillPlan {
  int s_pad;
  size_t off_k, off_vt, off_lat, total;
};
PrefillPlan plan_prefill(const Shape& s, int batch, int seq_len);

struct PrefillArgs {
  Shape s;
  const void *q, *w_uk, *w_uv;
  const int32_t* pair_idx;
  const float *rope_cos, *rope_sin;
  const void *ckv, *krope;
  int batch, t_max, seq_len;
  void* out;
  char* ws;
  PrefillPlan plan;
  PageMap pm{};
  const void* ckv_scale = nullptr;  // fmt 1: fp16 scales; fmt 2: fp16 (s, z) pairs
  const void* ckv_win = nullptr;    // fmt 2: ring of the last `win` rows per sequence [batch, win, d_kv] bf16
  int win = 0;
  int lat_staged = 0;  // set by the launcher: latent rows come from the workspace's dequantised copy
};

hipError_t launch_append(const AppendArgs& a, hipStream_t st);  // uses a.ws when set and useful
// phase_mask bit 0: q-prep, bit 1: attention, bit 2: combine
// Split-K append whose second phase runs inside the decode attention launch (ks == 0: none): the
// workgroup whose token range holds a new token writes its cache row first; rows outside every range
// go to `batch` extra workgroups.
struct FuseArgs {
  AppendArgs a;
  int ks;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st, int phase_mask = 7, const FuseArgs* fuse = nullptr);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);
// Decode step: split-K append of the new tokens (aa.ws = its partial sums) and decode (da), with the
// append's first phase and the query preparation in one launch.  Requires decode_step_fusable().
// phase_mask bit 0: that first launch; bit 1: the attention (with the append's reduction inside it, or
// before it); bit 2: the combine.
hipError_t launch_append_reduce(const AppendArgs& a, int ks, hipStream_t st);
bool decode_step_fusable(const AppendArgs& aa, const DecodeArgs& da);
hipError_t launch_decode_step(const AppendArgs& aa, const DecodeArgs& da, hipStream_t st, int phase_mask = 7);
hipError_t launch_quantize_int4(const float* in, int64_t n_groups, uint8_t* codes, uint16_t* scales, hipStream_t st);
hipError_t launch_quantize_int2(const float* in, int64_t n_groups, uint8_t* codes, uint16_t* meta, hipStream_t st);

// Shape predicates for the specialised paths (host side, used for dispatch and tests).
bool append_uses_mfma(const Shape& s);
bool decode_uses_mfma(const Shape& s);
bool decode_uses_wave(const Shape& s);  // per-wave tile streams (int4 latents, latent width 256)
bool decode_uses_combine(const Shape& s);  // merge and W_uv projection in one launch
bool prefill_supported(const Shape& s);
// Dynamic LDS of the generic kernels fits the 64 KiB a launch may request.
bool append_fits(const Shape& s);
bool decode_fits(const Shape& s, const DecodePlan& p);

}  // namespace mla
