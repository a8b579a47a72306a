/*
 * mla.h -- C ABI of the MHA2MLA latent-cache attention library (gfx950 / MI355X).
 *
 * The method (Paper-Notes ACL2025 page "MHA2MLA: Towards Economical Inference by Enabling
 * DeepSeek's Multi-Head Latent Attention in Any Transformer-based LLMs", section 关键设计,
 * "key designs"): an MHA layer is converted so that its KV cache holds, per token,
 *   - the latent c_kv = x . W_dkv (d_kv values shared by all heads; W_dkv = U_trunc of the
 *     joint SVD of [W_k,nope ; W_v]), and
 *   - per head, the keys of the r RoPE subspaces [2p, 2p+1] that head keeps (chosen offline by
 *     the 2-norm contribution score), already rotated at the token's position.
 * K_nope and V of head h are recovered from c_kv through that head's up-projections W_uk,h and
 * W_uv,h (the split of Sigma V^T); the RoPE part is computed separately because it cannot be
 * merged into the matrices.  The optional 4-bit and 2-bit latents follow the page's remark that
 * the latent composes with 4-bit or 2-bit KV-cache quantisation; the 2-bit one keeps the most recent
 * tokens unquantised, as the README page's quantised-cache evaluation does (residual length 128).
 *
 * Conventions for every entry point
 *   - All pointers to tensors are DEVICE pointers to caller-owned memory unless marked [host].
 *     The library never allocates, frees or synchronises device memory; scratch space comes from
 *     the caller's workspace, sized by the matching *_workspace_bytes call (mla_decode_step_static
 *     alone uses a static buffer the library holds per GPU instead, see there).
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream).  The calls keep no
 *     mutable global state (apart from that static buffer) and may be made from several host
 *     threads; calls that share output buffers or a workspace must be ordered by the caller (same
 *     stream or events).
 *   - Return value: MLA_OK (0) or a negative mla_status.  Every argument check runs on the host
 *     before anything is enqueued, so a call that returns an error has written nothing.
 *     MLA_ERR_HIP reports a failed launch (hipGetLastError after enqueueing); work enqueued
 *     before the failing launch may have run.
 *   - Dense row-major layouts; all tensor pointers must be 16-byte aligned (MLA_ERR_ALIGNMENT).
 *   - Weights use the [out_features, in_features] layout (each output's weights contiguous).
 *   - dtype MLA_F32: activations, weights, cache and outputs are fp32.  MLA_BF16: bf16 storage
 *     with fp32 accumulation and fp32 softmax.  RoPE tables are always fp32.
 *   - Device-resident per-sequence integers (start_pos, seq_lens) are trusted to lie within the
 *     host-side bound passed next to them; the kernels clamp to that bound, so a larger device
 *     value cannot make them access memory outside the buffers described here.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, inconsistent shape            */
  MLA_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype/format/shape combination)     */
  MLA_ERR_ALIGNMENT = -3,   /* a tensor pointer is not 16-byte aligned                        */
  MLA_ERR_WORKSPACE = -4,   /* workspace null or smaller than *_workspace_bytes               */
  MLA_ERR_CAPACITY = -5,    /* positions would exceed the cache's t_max or the RoPE table     */
  MLA_ERR_HIP = -6          /* a kernel launch failed                                          */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

typedef enum {
  MLA_CACHE_DENSE = 0,       /* c_kv stored in the config dtype                                */
  MLA_CACHE_INT4_G32 = 1,    /* c_kv as int4 codes, groups of 32 latent dims, fp16 absmax scale;
                                k_rope stays in the config dtype (BF16 only)                    */
  MLA_CACHE_INT2_G32_WIN = 2,/* c_kv of the last `window` positions of each sequence as bf16 rows
                                in a ring, older positions as affine 2-bit codes (groups of 32
                                latent dims, fp16 scale and offset); k_rope bf16 (BF16 only)    */
  MLA_CACHE_INT4_G32_WIN = 3 /* the same window of bf16 rows, older positions as the INT4_G32 codes
                                of their bf16 values (BF16 only)                                */
} mla_cache_fmt;

/* Layer shape.  d_head even; 0 <= r_pairs <= d_head/2; d_kv >= 1 (multiple of 32 for the quantised
 * formats). */
typedef struct {
  int32_t d_model;   /* model width d                                            */
  int32_t n_heads;   /* attention heads n_h                                      */
  int32_t d_head;    /* head dim d_h                                             */
  int32_t r_pairs;   /* RoPE subspaces kept per head, r (2r key dims per head)   */
  int32_t d_kv;      /* latent width (rank of the joint SVD), shared by all heads */
  int32_t dtype;     /* mla_dtype                                                 */
  int32_t cache_fmt; /* mla_cache_fmt                                             */
  int32_t rope_heads;/* RoPE key heads n_rh: 0 (= n_heads, keys per query head) or a divisor of
                        n_heads; query head h then uses RoPE key head h / (n_heads / n_rh), the
                        layout of a layer converted from a grouped-query source (one key head per
                        KV head, shared by its query heads; Paper-Notes page, 关键发现: GQA models
                        migrate as MHA ones do).  Else MLA_ERR_INVALID_ARG                     */
} mla_config;

/* Converted weights (read-only, device).  n_rh = rope_heads (n_h when 0), g(h) = h / (n_h / n_rh) the
 * RoPE key head of query head h.  nope(h) = the d_h - 2r dims of head h whose subspace is not kept,
 * ascending; rope(h) = dims 2p, 2p+1 for p = pair_idx[g(h)][j], j = 0..r-1.                      */
typedef struct {
  const void *w_dkv;        /* [d_kv, d_model]           W_dkv^T (down-projection, U_trunc)      */
  const void *w_krope;      /* [n_rh*2r, d_model]        rows (g, j, c) = column 2p+c of key head g
                                                          of W_k, p = pair_idx[g][j]               */
  const void *w_uk;         /* [n_h, d_h-2r, d_kv]       W_uk,h^T: row i rebuilds K dim nope(h)[i] */
  const void *w_uv;         /* [n_h, d_h, d_kv]          W_uv,h^T: row e rebuilds V dim e          */
  const int32_t *pair_idx;  /* [n_rh, r] int32, ascending per key head, each in [0, d_h/2)      */
  const float *rope_cos;    /* [rope_len, d_h/2] fp32: cos(pos * theta^(-2p/d_h))               */
  const float *rope_sin;    /* [rope_len, d_h/2] fp32: sin(...)                                 */
  int32_t rope_len;         /* rows of the RoPE tables (positions 0..rope_len-1)                */
} mla_weights;

/* Latent cache for `batch` sequences of up to t_max tokens each.
 *   DENSE:    ckv   [batch, t_max, d_kv]      config dtype
 *   INT4_G32: ckv   [batch, t_max, d_kv/2]    uint8, byte i = (code[2i] & 15) | (code[2i+1] & 15) << 4,
 *                                             codes two's-complement in [-7, 7]
 *             ckv_scale [batch, t_max, d_kv/32] fp16 (ignored / may be NULL for DENSE)
 *   INT2_G32_WIN:
 *             ckv   [batch, t_max, d_kv/4]    uint8, byte i = code[4i] | code[4i+1] << 2 | code[4i+2] << 4
 *                                             | code[4i+3] << 6, codes in [0, 3]; row pos holds position
 *                                             pos once it has left the window
 *             ckv_scale [batch, t_max, d_kv/32, 2] fp16 (s, z) per group; value = fp32(z + code * s)
 *             ckv_window [batch, window, d_kv] bf16 ring: slot pos % window holds position pos while
 *                                             pos >= L - window (L = the sequence's length)
 *             window >= 0 (0: every row is codes); ckv_window may be NULL when window == 0
 *   INT4_G32_WIN: ckv and ckv_scale as INT4_G32 (row pos holds position pos once it has left the window),
 *             ckv_window and window as INT2_G32_WIN
 *   all:      krope [batch, t_max, n_rh, 2r]  config dtype, pair (j, c) of key head g at index g*2r + 2j + c
 * ckv_window and window are read for the windowed formats (INT2_G32_WIN, INT4_G32_WIN) only.
 *
 * Paged caches (block_table != NULL; every format): ckv, ckv_scale and krope hold a pool of
 * n_pages pages of page_size rows each (the row layouts above, n_pages * page_size rows in place of
 * batch * t_max), and position pos of sequence b is pool row
 *     block_table[b * pages_per_seq + pos / page_size] * page_size + pos % page_size.
 * page_size is a multiple of 64; t_max must equal pages_per_seq * page_size; n_pages * page_size <= 2^31 - 1.
 * block_table [batch, pages_per_seq] int32 (device, 4-byte aligned); entries are clamped to
 * [0, n_pages), so a bad entry cannot make a kernel leave the pool.  Sequences may share pages (the
 * multi-query decode below reads one sequence's pages from several queries).  The windowed formats page
 * their codes, scales and RoPE keys; their ring ckv_window stays [batch, window, d_kv], one per sequence. */
typedef struct {
  void *ckv;
  void *ckv_scale;
  void *krope;
  int32_t batch;
  int32_t t_max;
  void *ckv_window;
  int32_t window;
  const int32_t *block_table; /* NULL: sequence b's position pos is row b * t_max + pos              */
  int32_t page_size;
  int32_t pages_per_seq;
  int32_t n_pages;
} mla_cache;

/* ---------------------------------------------------------------- append
 * Writes t_new tokens per sequence into the cache (down-projection and partial RoPE; the
 * key-designs section's latent c_kv = x . W_dkv and the per-head retained RoPE keys).
 *   x          [cache->batch, t_new, d_model] activations (config dtype)
 *   start_pos  [cache->batch] int32 (device): token i of sequence b goes to position start_pos[b]+i
 *   max_start_pos  host bound on start_pos[]: requires max_start_pos + t_new <= t_max and
 *                  <= rope_len (else MLA_ERR_CAPACITY)
 * Per token:  c_kv = x . W_dkv (fp32 accumulate, then rounded to the dtype, or quantised:
 *             s = fp16(absmax/7), code = clamp(rint(c/s), -7, 7), IEEE fp32 divisions);
 *             k_rope[h, j] = rotate((x . W_krope)[h, j, 0:2], pos * theta^(-2p/d_h)).
 * Windowed formats: each append must extend its sequences (start_pos[b] = the current length, all earlier
 *             positions written by earlier appends).  A row c_kv is rounded to bf16; rows that end up
 *             among the last `window` positions go to the ring, every other row (a new one, or one
 *             pushed out of the ring) is quantised from its bf16 value per group of 32 -- INT2_G32_WIN:
 *             z = fp16(min), s = fp16(max(max - z, 0) / 3), code = clamp(rint((c - z) / s), 0, 3)
 *             (fp32 arithmetic, IEEE division; s == 0 gives codes 0; infinite fp16 values saturate);
 *             INT4_G32_WIN: the int4 codec above on the bf16 values.
 * t_new == 0 or batch == 0 is a no-op returning MLA_OK.                                        */
int mla_cache_append(const mla_config *cfg, const mla_weights *w, mla_cache *cache, const void *x,
                     const int32_t *start_pos, int32_t t_new, int32_t max_start_pos, hipStream_t stream);

/* The same append with a caller workspace.  For a few tokens (batch * t_new <= 64, the decode-step
 * case) the down-projection is then split over the model width across many workgroups, with partial
 * sums in the workspace and a second launch that reduces them and stores the rows; otherwise the call
 * behaves like mla_cache_append and ignores the workspace.
 * Workspace: mla_cache_append_workspace_bytes(cfg, batch, t_new) bytes (0: none needed, may be NULL).  */
size_t mla_cache_append_workspace_bytes(const mla_config *cfg, int32_t batch, int32_t t_new);
int mla_cache_append_ws(const mla_config *cfg, const mla_weights *w, mla_cache *cache, const void *x,
                        const int32_t *start_pos, int32_t t_new, int32_t max_start_pos, void *workspace,
                        size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- decode
 * One query token per sequence attends to its cached tokens (the absorbed form of the
 * key-designs section: W_uk,h folded into the query, W_uv,h applied after the weighted latent sum).
 *   q          [batch, n_h, d_h] raw query (x . W_q, before RoPE, original head-dim order)
 *   seq_lens   [batch] int32 (device): L_b cached tokens, the query sits at position L_b - 1
 *              (append it first); L_b == 0 gives a zero output row.  Windowed formats: L_b must be the
 *              sequence's appended length (the ring holds its last `window` positions)
 *   max_seq_len  host bound on seq_lens[], 0 <= max_seq_len <= t_max and <= rope_len
 *   out        [batch, n_h, d_h] per-head attention outputs (before the output projection)
 * Scores are (q_hat . k_hat) / sqrt(d_h) with softmax over positions 0..L_b-1.
 * Workspace: mla_decode_workspace_bytes(cfg, batch, max_seq_len) bytes.                        */
size_t mla_decode_workspace_bytes(const mla_config *cfg, int32_t batch, int32_t max_seq_len);
int mla_decode(const mla_config *cfg, const mla_weights *w, const mla_cache *cache, const void *q,
               const int32_t *seq_lens, int32_t max_seq_len, void *out, void *workspace, size_t ws_bytes,
               hipStream_t stream);

/* The three launches of mla_decode one at a time, for callers that interleave other work between
 * them or time them separately.  Same arguments as mla_decode; the phases share the workspace and
 * must run in order 1, 2, 3 on the same stream:
 *   phase 1  latent query q~ = W_uk,h q_nope and the rotated retained query pairs
 *   phase 2  split-K attention over the cache (partial max / sum / latent output per split)
 *   phase 3  merge of the splits and the W_uv,h up-projection into `out`
 * phase outside 1..3 returns MLA_ERR_INVALID_ARG.                                               */
int mla_decode_phase(int phase, const mla_config *cfg, const mla_weights *w, const mla_cache *cache,
                     const void *q, const int32_t *seq_lens, int32_t max_seq_len, void *out, void *workspace,
                     size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- decode step
 * One serving step: mla_cache_append_ws of the new tokens (t_new per sequence) followed by
 * mla_decode over the updated cache, in one call.  The append's first phase and the decode's query
 * preparation do not depend on each other and share one launch; results are identical to the two
 * calls.  Arguments as for those calls; seq_lens[b] must count the appended tokens (normally
 * start_pos[b] + t_new) and max_seq_len bound them.
 * Workspace: mla_decode_step_workspace_bytes(cfg, batch, t_new, max_seq_len) bytes, 16-byte aligned
 * (the append's partial sums followed by the decode workspace).                                 */
size_t mla_decode_step_workspace_bytes(const mla_config *cfg, int32_t batch, int32_t t_new, int32_t max_seq_len);
int mla_decode_step(const mla_config *cfg, const mla_weights *w, mla_cache *cache, const void *x,
                    const int32_t *start_pos, int32_t t_new, int32_t max_start_pos, const void *q,
                    const int32_t *seq_lens, int32_t max_seq_len, void *out, void *workspace, size_t ws_bytes,
                    hipStream_t stream);

/* The three phases of mla_decode_step one at a time (for callers that time them or interleave other work):
 *   phase 1  the append's first launch (split-K partial sums of the new rows, or the whole append when the
 *            step does not split it) and the query preparation
 *   phase 2  the attention (the append's reduction runs inside this launch when the step fuses it)
 *   phase 3  the merge of the splits and the W_uv,h up-projection into `out`
 * Same arguments as mla_decode_step; phases run in order 1, 2, 3 on the same stream and workspace; running
 * 1, 2, 3 once gives the results of mla_decode_step.  phase outside 1..3 returns MLA_ERR_INVALID_ARG.  */
int mla_decode_step_phase(int phase, const mla_config *cfg, const mla_weights *w, mla_cache *cache, const void *x,
                          const int32_t *start_pos, int32_t t_new, int32_t max_start_pos, const void *q,
                          const int32_t *seq_lens, int32_t max_seq_len, void *out, void *workspace, size_t ws_bytes,
                          hipStream_t stream);

/* ---------------------------------------------------------------- allocation-free decode step
 * For callers that cannot allocate device memory (code under HIP graph capture, serving loops or harnesses that
 * forbid allocation): mla_decode_step with no workspace argument.  The workspace comes from a static device
 * buffer of MLA_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on until the process ends (the
 * buffer of the current device, hipGetDevice; the stream and every pointer must belong to that device).  The
 * call allocates and frees nothing; its first call on a device looks the buffer's address up once.
 * Every call on one GPU shares that buffer: calls that overlap on one GPU (other streams, other host threads)
 * race and must be ordered by the caller.  Nothing in the buffer needs clearing between calls: every byte a
 * call reads is written earlier in the same call.
 * Returns MLA_ERR_WORKSPACE when mla_decode_step_workspace_bytes(cfg, batch, t_new, max_seq_len) exceeds
 * MLA_STATIC_SCRATCH_BYTES (for example a Llama-2-7B-shaped layer at 64 sequences x 8192 positions needs
 * 45.3 MiB), before touching the device; every other argument and error as for mla_decode_step.      */
#define MLA_STATIC_SCRATCH_BYTES (64u << 20)
int mla_decode_step_static(const mla_config *cfg, const mla_weights *w, mla_cache *cache, const void *x,
                           const int32_t *start_pos, int32_t t_new, int32_t max_start_pos, const void *q,
                           const int32_t *seq_lens, int32_t max_seq_len, void *out, hipStream_t stream);

/* ---------------------------------------------------------------- multi-query decode
 * q_len query tokens per sequence at once (e.g. tokens proposed for speculative decoding), each attending
 * causally: with L_b cached tokens (the q_len new ones appended first), query i sits at position
 * L_b - q_len + i and attends to positions 0 .. L_b - q_len + i; a query at a negative position gives a
 * zero output row.  Same computation per query as mla_decode (q_len == 1 is mla_decode).
 *   q    [batch, q_len, n_h, d_h] raw queries;   out [batch, q_len, n_h, d_h]
 * Every cache format, contiguous or paged.  Windowed formats: seq_lens are the appended lengths, so the ring
 * holds positions L_b - window .. L_b - 1 of every query's cache sequence; a query sees the coded rows before
 * that range and the ring rows up to its own position.
 * Workspace: mla_decode_multi_workspace_bytes(cfg, batch, q_len, max_seq_len) bytes.               */
size_t mla_decode_multi_workspace_bytes(const mla_config *cfg, int32_t batch, int32_t q_len, int32_t max_seq_len);
int mla_decode_multi(const mla_config *cfg, const mla_weights *w, const mla_cache *cache, const void *q, int32_t q_len,
                     const int32_t *seq_lens, int32_t max_seq_len, void *out, void *workspace, size_t ws_bytes,
                     hipStream_t stream);

/* ---------------------------------------------------------------- prefill
 * Causal attention of seq_len query tokens per sequence, at positions 0..seq_len-1, over the
 * cache rows 0..seq_len-1 (append them first).  Unabsorbed form of the key-designs section: K_nope and
 * V of every head are recovered from the latent (c_kv . W_uk,h and c_kv . W_uv,h) and the retained RoPE
 * keys, which cannot be merged into the matrices, are read from the cache; for a whole prompt this
 * rebuilds each token's keys and values once instead of folding W_uk,h into every query.
 *   q    [batch, seq_len, n_h, d_h] raw queries;   out [batch, seq_len, n_h, d_h]
 * BF16 layers with d_head 128 and d_kv a multiple of 64 (MLA_ERR_UNSUPPORTED otherwise), any cache format:
 * a quantised latent (INT4_G32, INT2_G32_WIN, INT4_G32_WIN; contiguous or paged) is first dequantised into the workspace
 * exactly as decode reads it (int4: code * scale; 2-bit: z + code * s, the window's rows from the ring; then
 * rounded to bf16).  Windowed formats: every sequence's appended length must be seq_len (the ring then holds
 * positions seq_len - window .. seq_len - 1).
 * Workspace: mla_prefill_workspace_bytes(cfg, batch, seq_len) bytes.                           */
size_t mla_prefill_workspace_bytes(const mla_config *cfg, int32_t batch, int32_t seq_len);
int mla_prefill(const mla_config *cfg, const mla_weights *w, const mla_cache *cache, const void *q,
                int32_t seq_len, void *out, void *workspace, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- RoPE tables
 * The rotation tables of the partial RoPE (key-designs section: each retained 2-D subspace [2p, 2p+1] of a
 * head turns with its own frequency, theta^(-2p/d_head) per position): for positions t in [0, rope_len)
 * and subspaces p in [0, d_head/2), cos_out[t][p] = cos(t * theta^(-2p/d_head)) and sin_out likewise,
 * computed in fp64 on the host and rounded to fp32 -- the rope_cos / rope_sin of mla_weights.
 *   cos_out, sin_out  [host] caller-owned [rope_len, d_head/2] fp32 buffers (may be NULL when rope_len == 0)
 * Returns MLA_ERR_INVALID_ARG for rope_len < 0, an odd or non-positive d_head, theta not finite and > 0,
 * or a NULL buffer.  Synchronous host code; touches no device.                                      */
int mla_rope_tables(int32_t rope_len, int32_t d_head, double theta, float *cos_out, float *sin_out);

/* ---------------------------------------------------------------- int4 codec
 * The latent quantiser of the INT4_G32 cache on its own, for bit-exact checks of the codes (the key-designs
 * section's remark that the latent composes with 4-bit KV-cache quantisation; the group-32 absmax format
 * with fp16 scales is this library's, the pages fix none).
 *   in [n_groups*32] fp32 -> codes [n_groups*16] uint8 (packed as above), scales [n_groups] fp16 bits. */
int mla_quantize_int4(const float *in, int64_t n_groups, uint8_t *codes, uint16_t *scales, hipStream_t stream);

/* ---------------------------------------------------------------- 2-bit codec
 * The latent quantiser of the INT2_G32_WIN cache on its own (values already on the bf16 grid in the
 * cache; any fp32 values here), for bit-exact checks of the codes (the key-designs section's remark that the
 * latent composes with 2-bit KV-cache quantisation; the affine group-32 format with fp16 scale and offset is
 * this library's, the pages fix none).
 *   in [n_groups*32] fp32 -> codes [n_groups*8] uint8 (packed as above), meta [n_groups*2] fp16 bits
 *   (s, z per group).                                                                           */
int mla_quantize_int2(const float *in, int64_t n_groups, uint8_t *codes, uint16_t *meta, hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char *mla_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H_ */
