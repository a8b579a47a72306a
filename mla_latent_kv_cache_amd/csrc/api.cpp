// C ABI of the latent-cache library: host-side argument checks, workspace sizing and dispatch.
// Every check runs before anything is enqueued, so a rejected call has no side effects.
#include "../../include/mla.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "kernels.h"

using mla::Shape;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Formats whose last `window` rows per sequence are bf16 rows in a ring.
bool windowed(const mla_config* c) {
  return c->cache_fmt == MLA_CACHE_INT2_G32_WIN || c->cache_fmt == MLA_CACHE_INT4_G32_WIN;
}

// Shape-only checks shared by every entry point.
int check_config(const mla_config* c) {
  if (!c) return MLA_ERR_INVALID_ARG;
  if (c->d_model <= 0 || c->n_heads <= 0 || c->d_head <= 0 || c->d_kv <= 0) return MLA_ERR_INVALID_ARG;
  if (c->d_head % 2 != 0 || c->r_pairs < 0 || 2 * c->r_pairs > c->d_head) return MLA_ERR_INVALID_ARG;
  if (c->dtype != MLA_F32 && c->dtype != MLA_BF16) return MLA_ERR_INVALID_ARG;
  if (c->cache_fmt != MLA_CACHE_DENSE && c->cache_fmt != MLA_CACHE_INT4_G32 && c->cache_fmt != MLA_CACHE_INT2_G32_WIN &&
      c->cache_fmt != MLA_CACHE_INT4_G32_WIN)
    return MLA_ERR_INVALID_ARG;
  if (c->rope_heads < 0 || (c->rope_heads > 0 && c->n_heads % c->rope_heads != 0)) return MLA_ERR_INVALID_ARG;
  if (c->d_head > 256) return MLA_ERR_UNSUPPORTED;
  if (c->cache_fmt != MLA_CACHE_DENSE && (c->dtype != MLA_BF16 || c->d_kv % 32 != 0)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

Shape shape_of(const mla_config* c) {
  return Shape{c->d_model, c->n_heads, c->d_head, c->r_pairs, c->d_kv, c->dtype, c->cache_fmt,
               c->rope_heads > 0 ? c->rope_heads : c->n_heads};
}

// A pointer that must be present (non-null, 16-byte aligned) when `needed`.
int check_ptr(const void* p, bool needed) {
  if (!needed) return MLA_OK;
  if (!p) return MLA_ERR_INVALID_ARG;
  return aligned16(p) ? MLA_OK : MLA_ERR_ALIGNMENT;
}

#define MLA_TRY(expr)          \
  do {                         \
    int rc_ = (expr);          \
    if (rc_ != MLA_OK) return rc_; \
  } while (0)

int check_weights(const mla_config* c, const mla_weights* w, bool need_dkv, bool need_up) {
  if (!w) return MLA_ERR_INVALID_ARG;
  const bool has_rope = c->r_pairs > 0;
  const bool has_nope = c->d_head - 2 * c->r_pairs > 0;
  MLA_TRY(check_ptr(w->w_dkv, need_dkv));
  MLA_TRY(check_ptr(w->w_krope, need_dkv && has_rope));
  MLA_TRY(check_ptr(w->w_uk, need_up && has_nope));
  MLA_TRY(check_ptr(w->w_uv, need_up));
  MLA_TRY(check_ptr(w->pair_idx, has_rope));
  MLA_TRY(check_ptr(w->rope_cos, has_rope));
  MLA_TRY(check_ptr(w->rope_sin, has_rope));
  if (has_rope && w->rope_len <= 0) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

int check_cache(const mla_config* c, const mla_cache* k) {
  if (!k) return MLA_ERR_INVALID_ARG;
  if (k->batch < 0 || k->t_max <= 0) return MLA_ERR_INVALID_ARG;
  MLA_TRY(check_ptr(k->ckv, true));
  MLA_TRY(check_ptr(k->krope, c->r_pairs > 0));
  MLA_TRY(check_ptr(k->ckv_scale, c->cache_fmt != MLA_CACHE_DENSE));
  if (windowed(c)) {
    if (k->window < 0) return MLA_ERR_INVALID_ARG;
    MLA_TRY(check_ptr(k->ckv_window, k->window > 0));
  }
  if (k->block_table) {
    if (((uintptr_t)k->block_table & 3u) != 0) return MLA_ERR_ALIGNMENT;
    if (k->page_size <= 0 || k->page_size % 64 != 0 || k->pages_per_seq <= 0 || k->n_pages <= 0)
      return MLA_ERR_INVALID_ARG;
    if ((long long)k->pages_per_seq * k->page_size != k->t_max) return MLA_ERR_INVALID_ARG;
    if ((long long)k->n_pages * k->page_size > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  } else if ((long long)k->batch * k->t_max > 0x7fffffffLL) {
    return MLA_ERR_UNSUPPORTED;  // cache rows are indexed with 32-bit integers
  }
  return MLA_OK;
}

// Positions [0, limit) must fit in the cache and, when RoPE is used, in the RoPE tables.
int check_positions(const mla_config* c, const mla_weights* w, const mla_cache* k, long long limit) {
  if (limit > k->t_max) return MLA_ERR_CAPACITY;
  if (c->r_pairs > 0 && limit > w->rope_len) return MLA_ERR_CAPACITY;
  return MLA_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// The page table of a paged cache (nothing for a contiguous one).
template <typename Args>
void set_pages(Args& a, const mla_cache* k) {
  if (!k->block_table) return;
  a.pm = mla::PageMap{k->block_table, k->page_size, k->pages_per_seq, k->n_pages};
}
// The bf16 ring of the 2-bit format (nothing for the other formats), and the page table.
template <typename Args>
void set_window(Args& a, const mla_config* c, const mla_cache* k) {
  set_pages(a, k);
  if (!windowed(c)) return;
  a.ckv_win = k->ckv_window;
  a.win = k->window;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_CAPACITY: return "positions exceed cache or RoPE table capacity";
    case MLA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

static int append_impl(const mla_config* cfg, const mla_weights* w, mla_cache* cache, const void* x,
                       const int32_t* start_pos, int32_t t_new, int32_t max_start_pos, void* workspace,
                       size_t ws_bytes, bool use_ws, hipStream_t stream) {
  MLA_TRY(check_config(cfg));
  MLA_TRY(check_weights(cfg, w, true, false));
  MLA_TRY(check_cache(cfg, cache));
  if (t_new < 0 || max_start_pos < 0) return MLA_ERR_INVALID_ARG;
  if (t_new == 0 || cache->batch == 0) return MLA_OK;
  MLA_TRY(check_ptr(x, true));
  MLA_TRY(check_ptr(start_pos, true));
  MLA_TRY(check_positions(cfg, w, cache, (long long)max_start_pos + t_new));
  if ((long long)cache->batch * t_new > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  const Shape s = shape_of(cfg);
  if (!mla::append_fits(s)) return MLA_ERR_UNSUPPORTED;
  char* ws = nullptr;
  if (use_ws) {
    const size_t need = mla::append_workspace_bytes(s, cache->batch * t_new);
    if (need > 0) {
      if (!workspace || ws_bytes < need) return MLA_ERR_WORKSPACE;
      if (!aligned16(workspace)) return MLA_ERR_ALIGNMENT;
      ws = (char*)workspace;
    }
  }
  mla::AppendArgs a{s, x, w->w_dkv, w->w_krope, w->pair_idx, w->rope_cos, w->rope_sin,
                    start_pos, cache->batch, t_new, max_start_pos, cache->t_max,
                    cache->ckv, cache->ckv_scale, cache->krope, ws};
  set_window(a, cfg, cache);
  return from_hip(mla::launch_append(a, stream));
}

int mla_cache_append(const mla_config* cfg, const mla_weights* w, mla_cache* cache, const void* x,
                     const int32_t* start_pos, int32_t t_new, int32_t max_start_pos, hipStream_t stream) {
  return append_impl(cfg, w, cache, x, start_pos, t_new, max_start_pos, nullptr, 0, false, stream);
}

size_t mla_cache_append_workspace_bytes(const mla_config* cfg, int32_t batch, int32_t t_new) {
  if (check_config(cfg) != MLA_OK || batch < 0 || t_new < 0) return 0;
  return mla::append_workspace_bytes(shape_of(cfg), batch * t_new);
}

int mla_cache_append_ws(const mla_config* cfg, const mla_weights* w, mla_cache* cache, const void* x,
                        const int32_t* start_pos, int32_t t_new, int32_t max_start_pos, void* workspace,
                        size_t ws_bytes, hipStream_t stream) {
  return append_impl(cfg, w, cache, x, start_pos, t_new, max_start_pos, workspace, ws_bytes, true, stream);
}

size_t mla_decode_workspace_bytes(const mla_config* cfg, int32_t batch, int32_t max_seq_len) {
  if (check_config(cfg) != MLA_OK || batch < 0 || max_seq_len < 0) return 0;
  return mla::plan_decode(shape_of(cfg), batch, max_seq_len).total;
}

static int decode_impl(int phase_mask, const mla_config* cfg, const mla_weights* w, const mla_cache* cache,
                       const void* q, const int32_t* seq_lens, int32_t max_seq_len, void* out, void* workspace,
                       size_t ws_bytes, hipStream_t stream, int q_len = 1) {
  MLA_TRY(check_config(cfg));
  MLA_TRY(check_weights(cfg, w, false, true));
  MLA_TRY(check_cache(cfg, cache));
  if (max_seq_len < 0 || q_len < 1) return MLA_ERR_INVALID_ARG;
  if (cache->batch == 0) return MLA_OK;
  MLA_TRY(check_ptr(q, true));
  MLA_TRY(check_ptr(seq_lens, true));
  MLA_TRY(check_ptr(out, true));
  MLA_TRY(check_positions(cfg, w, cache, max_seq_len));
  // the kernels count the batch's queries and tokens in 32-bit integers
  const long long nq = (long long)cache->batch * q_len;
  if (nq * (max_seq_len > 0 ? max_seq_len : 1) >= (1LL << 31)) return MLA_ERR_UNSUPPORTED;
  const Shape s = shape_of(cfg);
  const mla::DecodePlan plan = mla::plan_decode(s, (int)nq, max_seq_len);
  if (!mla::decode_fits(s, plan)) return MLA_ERR_UNSUPPORTED;
  // the specialised kernel addresses one sequence's cache rows with 32-bit byte offsets
  if (mla::decode_uses_mfma(s) && (size_t)cache->t_max * s.d_kv * 2 >= ((size_t)1 << 31)) return MLA_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < plan.total) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGNMENT;
  mla::DecodeArgs a{s, q, w->w_uk, w->w_uv, w->pair_idx, w->rope_cos, w->rope_sin,
                    cache->ckv, cache->ckv_scale, cache->krope, (int)nq, cache->t_max, max_seq_len,
                    seq_lens, out, (char*)workspace, plan};
  set_window(a, cfg, cache);
  a.qn = q_len;
  return from_hip(mla::launch_decode(a, stream, phase_mask));
}

int mla_decode(const mla_config* cfg, const mla_weights* w, const mla_cache* cache, const void* q,
               const int32_t* seq_lens, int32_t max_seq_len, void* out, void* workspace, size_t ws_bytes,
               hipStream_t stream) {
  return decode_impl(7, cfg, w, cache, q, seq_lens, max_seq_len, out, workspace, ws_bytes, stream);
}

size_t mla_decode_multi_workspace_bytes(const mla_config* cfg, int32_t batch, int32_t q_len, int32_t max_seq_len) {
  if (check_config(cfg) != MLA_OK || batch < 0 || q_len < 1 || max_seq_len < 0) return 0;
  if ((long long)batch * q_len > 0x7fffffffLL) return 0;
  return mla::plan_decode(shape_of(cfg), batch * q_len, max_seq_len).total;
}

int mla_decode_multi(const mla_config* cfg, const mla_weights* w, const mla_cache* cache, const void* q, int32_t q_len,
                     const int32_t* seq_lens, int32_t max_seq_len, void* out, void* workspace, size_t ws_bytes,
                     hipStream_t stream) {
  return decode_impl(7, cfg, w, cache, q, seq_lens, max_seq_len, out, workspace, ws_bytes, stream, q_len);
}

int mla_decode_phase(int phase, const mla_config* cfg, const mla_weights* w, const mla_cache* cache,
                     const void* q, const int32_t* seq_lens, int32_t max_seq_len, void* out, void* workspace,
                     size_t ws_bytes, hipStream_t stream) {
  if (phase < 1 || phase > 3) return MLA_ERR_INVALID_ARG;
  return decode_impl(1 << (phase - 1), cfg, w, cache, q, seq_lens, max_seq_len, out, workspace, ws_bytes, stream);
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t mla_decode_step_workspace_bytes(const mla_config* cfg, int32_t batch, int32_t t_new, int32_t max_seq_len) {
  if (check_config(cfg) != MLA_OK || batch < 0 || t_new < 0 || max_seq_len < 0) return 0;
  const Shape s = shape_of(cfg);
  return align256(mla::append_workspace_bytes(s, batch * t_new)) + mla::plan_decode(s, batch, max_seq_len).total;
}

static int decode_step_impl(const mla_config* cfg, const mla_weights* w, mla_cache* cache, const void* x,
                            const int32_t* start_pos, int32_t t_new, int32_t max_start_pos, const void* q,
                            const int32_t* seq_lens, int32_t max_seq_len, void* out, void* workspace,
                            size_t ws_bytes, hipStream_t stream, bool static_ws, int phase_mask = 7);

int mla_decode_step(const mla_config* cfg, const mla_weights* w, mla_cache* cache, const void* x,
                    const int32_t* start_pos, int32_t t_new, int32_t max_start_pos, const void* q,
                    const int32_t* seq_lens, int32_t max_seq_len, void* out, void* workspace, size_t ws_bytes,
                    hipStream_t stream) {
  return decode_step_impl(cfg, w, cache, x, start_pos, t_new, max_start_pos, q, seq_lens, max_seq_len, out, workspace,
                          ws_bytes, stream, false);
}

int mla_decode_step_phase(int phase, const mla_config* cfg, const mla_weights* w, mla_cache* cache, const void* x,
                          const int32_t* start_pos, int32_t t_new, int32_t max_start_pos, const void* q,
                          const int32_t* seq_lens, int32_t max_seq_len, void* out, void* workspace, size_t ws_bytes,
                          hipStream_t stream) {
  if (phase < 1 || phase > 3) return MLA_ERR_INVALID_ARG;
  return decode_step_impl(cfg, w, cache, x, start_pos, t_new, max_start_pos, q, seq_lens, max_seq_len, out, workspace,
                          ws_bytes, stream, false, 1 << (phase - 1));
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free decode step
// The workspace of mla_decode_step_static lives in this file-scope device array: each GPU the library runs on
// holds one copy until the process ends.  Host code never uses the array's name as an address (on the host it
// names a stand-in, not device memory): its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[MLA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's scratch array (nullptr with MLA_ERR_HIP if it cannot be found).
int current_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return MLA_ERR_HIP;
  *ptr = g_scratch_ptr[dev];
  return MLA_OK;
}
}  // namespace

extern "C" {

int mla_decode_step_static(const mla_config* cfg, const mla_weights* w, mla_cache* cache, const void* x,
                           const int32_t* start_pos, int32_t t_new, int32_t max_start_pos, const void* q,
                           const int32_t* seq_lens, int32_t max_seq_len, void* out, hipStream_t stream) {
  // the size check first, so that an oversized request is rejected before the device is touched
  if (check_config(cfg) == MLA_OK && cache && cache->batch >= 0 && t_new >= 0 && max_seq_len >= 0 &&
      mla_decode_step_workspace_bytes(cfg, cache->batch, t_new, max_seq_len) > (size_t)MLA_STATIC_SCRATCH_BYTES)
    return MLA_ERR_WORKSPACE;
  return decode_step_impl(cfg, w, cache, x, start_pos, t_new, max_start_pos, q, seq_lens, max_seq_len, out, nullptr,
                          MLA_STATIC_SCRATCH_BYTES, stream, true);
}

}  // extern "C"

static int decode_step_impl(const mla_config* cfg, const mla_weights* w, mla_cache* cache, const void* x,
                            const int32_t* start_pos, int32_t t_new, int32_t max_start_pos, const void* q,
                            const int32_t* seq_lens, int32_t max_seq_len, void* out, void* workspace,
                            size_t ws_bytes, hipStream_t stream, bool static_ws, int phase_mask) {
  // validation of both halves, as the separate calls do it
  MLA_TRY(check_config(cfg));
  MLA_TRY(check_weights(cfg, w, true, true));
  MLA_TRY(check_cache(cfg, cache));
  if (t_new < 0 || max_start_pos < 0 || max_seq_len < 0) return MLA_ERR_INVALID_ARG;
  if (cache->batch == 0) return MLA_OK;
  const Shape s = shape_of(cfg);
  if (t_new > 0) {
    MLA_TRY(check_ptr(x, true));
    MLA_TRY(check_ptr(start_pos, true));
    MLA_TRY(check_positions(cfg, w, cache, (long long)max_start_pos + t_new));
    if ((long long)cache->batch * t_new > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
    if (!mla::append_fits(s)) return MLA_ERR_UNSUPPORTED;
  }
  MLA_TRY(check_ptr(q, true));
  MLA_TRY(check_ptr(seq_lens, true));
  MLA_TRY(check_ptr(out, true));
  MLA_TRY(check_positions(cfg, w, cache, max_seq_len));
  if ((long long)cache->batch * max_seq_len >= (1LL << 31)) return MLA_ERR_UNSUPPORTED;
  const mla::DecodePlan plan = mla::plan_decode(s, cache->batch, max_seq_len);
  if (!mla::decode_fits(s, plan)) return MLA_ERR_UNSUPPORTED;
  if (mla::decode_uses_mfma(s) && (size_t)cache->t_max * s.d_kv * 2 >= ((size_t)1 << 31)) return MLA_ERR_UNSUPPORTED;
  const size_t app_bytes = align256(mla::append_workspace_bytes(s, cache->batch * t_new));
  if (ws_bytes < app_bytes + plan.total) return MLA_ERR_WORKSPACE;
  if (static_ws) MLA_TRY(current_scratch(&workspace));  // the last step before enqueueing: a lookup, no allocation
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGNMENT;
  char* wsa = (char*)workspace;
  char* wsd = wsa + app_bytes;
  mla::AppendArgs aa{s, x, w->w_dkv, w->w_krope, w->pair_idx, w->rope_cos, w->rope_sin,
                     start_pos, cache->batch, t_new, max_start_pos, cache->t_max,
                     cache->ckv, cache->ckv_scale, cache->krope, app_bytes > 0 ? wsa : nullptr};
  mla::DecodeArgs da{s, q, w->w_uk, w->w_uv, w->pair_idx, w->rope_cos, w->rope_sin,
                     cache->ckv, cache->ckv_scale, cache->krope, cache->batch, cache->t_max, max_seq_len,
                     seq_lens, out, wsd, plan};
  set_window(aa, cfg, cache);
  set_window(da, cfg, cache);
  if (t_new > 0 && mla::decode_step_fusable(aa, da))
    return from_hip(mla::launch_decode_step(aa, da, stream, phase_mask));
  if (t_new > 0 && (phase_mask & 1)) MLA_TRY(from_hip(mla::launch_append(aa, stream)));
  return from_hip(mla::launch_decode(da, stream, phase_mask));
}

extern "C" {

size_t mla_prefill_workspace_bytes(const mla_config* cfg, int32_t batch, int32_t seq_len) {
  if (check_config(cfg) != MLA_OK || batch < 0 || seq_len < 0) return 0;
  return mla::plan_prefill(shape_of(cfg), batch, seq_len).total;
}

int mla_prefill(const mla_config* cfg, const mla_weights* w, const mla_cache* cache, const void* q,
                int32_t seq_len, void* out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  MLA_TRY(check_config(cfg));
  MLA_TRY(check_weights(cfg, w, false, true));
  MLA_TRY(check_cache(cfg, cache));
  if (seq_len < 0) return MLA_ERR_INVALID_ARG;
  const Shape s = shape_of(cfg);
  if (!mla::prefill_supported(s)) return MLA_ERR_UNSUPPORTED;
  if (seq_len == 0 || cache->batch == 0) return MLA_OK;
  MLA_TRY(check_ptr(q, true));
  MLA_TRY(check_ptr(out, true));
  MLA_TRY(check_positions(cfg, w, cache, seq_len));
  const mla::PrefillPlan plan = mla::plan_prefill(s, cache->batch, seq_len);
  if (!workspace || ws_bytes < plan.total) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_ALIGNMENT;
  mla::PrefillArgs a{s, q, w->w_uk, w->w_uv, w->pair_idx, w->rope_cos, w->rope_sin, cache->ckv, cache->krope,
                     cache->batch, cache->t_max, seq_len, out, (char*)workspace, plan};
  set_window(a, cfg, cache);
  a.ckv_scale = cache->ckv_scale;
  return from_hip(mla::launch_prefill(a, stream));
}

int mla_rope_tables(int32_t rope_len, int32_t d_head, double theta, float* cos_out, float* sin_out) {
  if (rope_len < 0 || d_head <= 0 || d_head % 2 != 0 || !(theta > 0.0) || !std::isfinite(theta))
    return MLA_ERR_INVALID_ARG;
  if (rope_len == 0) return MLA_OK;
  if (!cos_out || !sin_out) return MLA_ERR_INVALID_ARG;
  const int half = d_head / 2;
  for (int p = 0; p < half; ++p) {
    // subspace p turns at theta^(-2p/d_head) per position; angles and their cosines in fp64
    const double freq = std::pow(theta, -2.0 * p / d_head);
    for (int32_t t = 0; t < rope_len; ++t) {
      const double ang = (double)t * freq;
      cos_out[(size_t)t * half + p] = (float)std::cos(ang);
      sin_out[(size_t)t * half + p] = (float)std::sin(ang);
    }
  }
  return MLA_OK;
}

int mla_quantize_int4(const float* in, int64_t n_groups, uint8_t* codes, uint16_t* scales, hipStream_t stream) {
  if (n_groups < 0) return MLA_ERR_INVALID_ARG;
  if (n_groups == 0) return MLA_OK;
  if (!in || !codes || !scales) return MLA_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(codes) || !aligned16(scales)) return MLA_ERR_ALIGNMENT;
  if (n_groups > ((int64_t)1 << 36)) return MLA_ERR_UNSUPPORTED;
  return from_hip(mla::launch_quantize_int4(in, n_groups, codes, scales, stream));
}

int mla_quantize_int2(const float* in, int64_t n_groups, uint8_t* codes, uint16_t* meta, hipStream_t stream) {
  if (n_groups < 0) return MLA_ERR_INVALID_ARG;
  if (n_groups == 0) return MLA_OK;
  if (!in || !codes || !meta) return MLA_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(codes) || !aligned16(meta)) return MLA_ERR_ALIGNMENT;
  if (n_groups > ((int64_t)1 << 36)) return MLA_ERR_UNSUPPORTED;
  return from_hip(mla::launch_quantize_int2(in, n_groups, codes, meta, stream));
}

}  // extern "C"
