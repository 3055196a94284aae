/*
 * liblbca: learned block-compressed attention on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Device pointers are HIP device
 * memory owned by the caller; the library allocates nothing, keeps no state
 * between calls (except the static scratch array of
 * lbca_attend_decode_noalloc, part of the loaded code object), never frees a
 * caller buffer, and only enqueues work on the stream the caller passes (a
 * hipStream_t, 0 = the null stream).  Every call is asynchronous with respect
 * to the host unless stated otherwise.
 *
 * Errors: every entry point returns an int status.  Argument validation runs on
 * the host BEFORE any device work is enqueued; an argument error returns
 * LBCA_ERR_INVALID_ARG / LBCA_ERR_UNSUPPORTED / LBCA_ERR_WORKSPACE and leaves
 * every output untouched.  LBCA_ERR_HIP means a HIP launch reported an error
 * (outputs unspecified).  Nothing aborts or throws across the ABI.  Values the
 * host cannot see (positions held in device memory) are checked by the
 * kernels: a sequence whose position does not fit the buffers it was given
 * gets NaN outputs instead of out-of-bounds accesses.
 *
 * Layout conventions: a tensor has the shape given, its last (feature)
 * dimension contiguous, and its element type given by a dtype field
 * (LBCA_F32 = IEEE float32, LBCA_BF16 = bfloat16 bit patterns).  Every
 * tensor with a feature dimension (queries, keys, values, logits, outputs
 * and their gradients) also takes an lbca_strides field (named after it
 * with an _st suffix): int64 element strides of its other dimensions, so a
 * slice of a longer cache, a head-interleaved [batch, rows, heads, dim]
 * buffer seen as [batch, heads, rows, dim], or the query part of a fused
 * projection output is passed in place.  A zeroed lbca_strides means dense
 * row-major.  Per-head or per-sequence scalars (lse, sink, head_w),
 * positions, index lists and the pooling biases are dense.  Device pointers
 * to bf16/f32 data must be 16-byte aligned.  Positions are 0-based token
 * indices (int64).
 *
 * Method (pages cited by title and section):
 *  - "mSeek: learned KV-cache compression in a 3B model" (mSeek), section
 *    "How LBCA works": each completed block of m old tokens is replaced by one
 *    learned entry (per-channel softmax of content logits over the block,
 *    weighted sum of its keys and values); a query attends over every visible
 *    summary plus the exact raw local window; incomplete blocks stay raw.
 *  - "HCA: Heavily Compressed Attention (toy implementation)" (HCA), section
 *    "What is implemented": single-series pooling with a learnable positional
 *    bias; dense attention over all causally visible compressed entries plus a
 *    sliding-window branch; shared-KV MQA; RMSNorm; partial RoPE; sink.
 *  - "CSA: Compressed Sparse Attention (toy implementation)" (CSA), section
 *    "What is implemented": dual overlapped pooling; lightning indexer with
 *    ReLU scores and learned head weights; top-k over causally visible entries;
 *    shared-KV MQA core attention with the same treatment and a -t rotation
 *    of the rotated output dims.
 */
#ifndef LBCA_H
#define LBCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LBCA_ABI_VERSION 2

#if defined(__GNUC__)
#define LBCA_API __attribute__((visibility("default")))
#else
#define LBCA_API
#endif

/* status codes */
#define LBCA_OK 0
#define LBCA_ERR_INVALID_ARG (-1)  /* null required pointer, bad size, shape mismatch */
#define LBCA_ERR_UNSUPPORTED (-2)  /* valid but not implemented (dtype, dim, flag mix) */
#define LBCA_ERR_WORKSPACE (-3)    /* workspace missing or too small */
#define LBCA_ERR_HIP (-4)          /* a HIP runtime call failed */
#define LBCA_ERR_TOO_LARGE (-5)    /* beyond the static scratch of lbca_attend_decode_noalloc */

/* element types */
#define LBCA_F32 0
#define LBCA_BF16 1

/* visibility rules */
#define LBCA_EXCLUSIVE 0 /* mSeek LBCA: a block is pooled once complete AND wholly
                            older than the W-token window; raw span = first
                            unpooled token .. t (W .. W+m-1 tokens). */
#define LBCA_OVERLAP 1   /* HCA/CSA: every complete block is visible; the raw
                            window is the last W tokens [max(0,t-W+1), t]. */

/* Element strides of one tensor argument: s[i] is the distance, in
 * elements, between neighbours along dimension i, outermost first, for every
 * dimension but the last (which is contiguous); a tensor of rank r uses
 * s[0 .. r-2] and the rest are ignored.  All zero: dense row-major for the
 * documented shape.  Rules (INVALID_ARG otherwise): strides >= 0; each
 * stride times the element size a multiple of 16 bytes (rows stay aligned for
 * 16-byte loads); an output's elements must not overlap one another (for the
 * dimensions of extent > 1, sorted by stride, each stride covers the extent
 * of everything inside it).  Every stride but the outermost must be below 2^31
 * elements, dense defaults included (UNSUPPORTED otherwise), and the calls
 * that address cache rows with 32-bit offsets state their own bound on a
 * slice's span. */
typedef struct lbca_strides {
  int64_t s[3];
} lbca_strides;

LBCA_API int lbca_abi_version(void);

/* Static, never-NULL description of a status code. */
LBCA_API const char* lbca_status_string(int status);

/*
 * Host-only visibility rule for a query at position t (mSeek "How LBCA works",
 * steps 4-5; HCA/CSA "What is implemented").  Writes the number of visible
 * pooled entries (entries 0 .. n_pooled-1) and the first raw position; the raw
 * span is [raw_begin, t].
 *   EXCLUSIVE: n_pooled = floor(max(0, t+1-W) / m), raw_begin = n_pooled*m
 *   OVERLAP:   n_pooled = floor((t+1) / m),         raw_begin = max(0, t-W+1)
 * Errors: INVALID_ARG if t < 0, m < 1, W < 1, bad mode or a NULL output.
 * The kernels apply the same rule on the device.
 */
LBCA_API int lbca_visible_range(int64_t t, int64_t m, int64_t W, int32_t mode,
                       int64_t* n_pooled, int64_t* raw_begin);

/* ------------------------------------------------------------------------ */
/* Block pooling (mSeek "How LBCA works" steps 2-3; HCA "What is implemented"
 * item 1; CSA "What is implemented" item 1).
 *
 * Single-series mode (xb == NULL): entry j pools tokens [j*m, (j+1)*m):
 *   w[s,c]   = softmax over s in block j of (z[s,c] + bias[h, s-j*m, c])
 *   out_x[j,c] = sum_s w[s,c] * x[s,c];  out_v[j,c] = sum_s w[s,c] * v[s,c]
 * With v == NULL only out_x is written (HCA shared K=V series).
 * Dual mode (xb != NULL, CSA): entry i takes ONE softmax per channel over the
 * logits z[s]+bias[s-i*m] of block i and zb[s]+bias_b[s-(i-1)*m] of block i-1
 * (block i alone for i = 0), and sums the matching rows of x and xb.
 *
 * Optional entry treatment (shared series only, v == NULL): with
 * rmsnorm_eps >= 0 each pooled row is RMS-normalised (unit weight); with
 * rope_dims > 0 its last rope_dims dims are then rotated at the entry's block
 * start position j*m (rotate-half pairs (k, k+r/2), angle pos*base^(-2k/r),
 * angles reduced in double precision).  This is the per-entry part of the
 * HCA/CSA core-attention treatment, applied once when the entry is written;
 * lbca_attend_decode reads stored entries as-is.
 *
 *   x, v, z, xb, zb   [batch, heads, tokens, dim]; row r holds position pos_base+r
 *   bias, bias_b      [heads, block, dim] float32
 *   out_x, out_v      [batch, heads, entries, dim]; entry j is row j
 *   blocks [block_begin, block_end) are pooled; every other out row is left as is.
 * Dtypes: x/v/xb/out in x_dtype, z/zb in z_dtype (each F32 or BF16); math in fp32.
 * Constraints: dim a power of two in [8, 512]; rope_dims % 16 == 0, <= dim.
 * Errors: INVALID_ARG if a token row needed is outside [0, tokens) or
 * block_end > entries; UNSUPPORTED for treatment with v != NULL.
 */
typedef struct lbca_pool_args {
  const void* x;
  const void* v;
  const void* z;
  const float* bias;
  const void* xb;
  const void* zb;
  const float* bias_b;
  void* out_x;
  void* out_v;
  int64_t batch, heads, tokens, dim, block, entries;
  int64_t block_begin, block_end;
  int64_t pos_base;
  int32_t x_dtype, z_dtype;
  float rmsnorm_eps; /* < 0: off */
  int32_t rope_dims; /* 0: off */
  float rope_base;
  lbca_strides x_st, v_st, z_st, xb_st, zb_st, out_x_st, out_v_st;
} lbca_pool_args;

LBCA_API int lbca_pool_blocks(const lbca_pool_args* a, void* stream);

/* ------------------------------------------------------------------------ */
/* Gradients of single-series pooling (mSeek "How LBCA works" steps 2-3: with
 * a = z + bias[h, s - j*m] and w = softmax over block j's tokens per channel,
 * out_x[j] = sum w x, out_v[j] = sum w v).  For upstream gradients grad_x[j]
 * (and grad_v[j]) of the pooled rows of blocks [block_begin, block_end):
 *   dx[s] = w[s] * grad_x[j]          dv[s] = w[s] * grad_v[j]
 *   dz[s] = w[s] * (grad_x[j] * (x[s] - out_x[j]) + grad_v[j] * (v[s] - out_v[j]))
 *   dbias[h, i] = sum over sequences b and blocks j of dz[b, h, j*m + i]
 * with the entries recomputed in fp32.  Token rows of those blocks are
 * written in dx, dv, dz; every other row is left as is.  dbias is overwritten
 * (zeros for an empty range).  Results are bitwise reproducible.
 * Treatment (shared series only; HCA/CSA "What is implemented"): with
 * rmsnorm_eps >= 0 and/or rope_dims > 0 the stored entries were
 * rope(rmsnorm(out_x[j])) at position j*m (as lbca_pool_blocks writes them)
 * and grad_x is the gradient of those; it is taken back through the rotation
 * and the RMSNorm before the formulas above.
 * Dual mode (xb != NULL, CSA "What is implemented" item 1): entry j's softmax
 * also covers block j-1 of the b-series (xb, zb, bias_b); its rows get dxb,
 * dzb and its bias offsets dbias_b by the same formulas (entry 0 has no
 * b-part); b-series rows of blocks [max(block_begin,1)-1, block_end-1) are
 * written.
 *
 *   x, v, z            [batch, heads, tokens, dim]; row r holds position pos_base+r
 *   bias               [heads, block, dim] float32
 *   grad_x, grad_v     [batch, heads, entries, dim]   (x_dtype)
 *   dx, dv / dz        [batch, heads, tokens, dim]    (x_dtype / z_dtype)
 *   dbias              [heads, block, dim] float32
 *   xb, zb, dxb, dzb   [batch, heads, tokens, dim]; bias_b, dbias_b [heads, block, dim]
 * v, grad_v and dv are all NULL without values; xb, zb, bias_b, dxb, dzb,
 * dbias_b all NULL outside dual mode.  Treatment and dual mode need a shared
 * series (no values).
 * Constraints: dim a power of two in [8, 512], block * dim <= 8192 (dual:
 * 2 * block * dim <= 8192), heads <= 65535.  Workspace (lbca_pool_blocks_backward_workspace bytes,
 * 16-byte aligned, caller-owned, no initialisation needed): the bias-gradient
 * partials.  Errors as lbca_pool_blocks, plus WORKSPACE.
 */
typedef struct lbca_pool_grad_args {
  const void* x;
  const void* v;
  const void* z;
  const float* bias;
  const void* grad_x;
  const void* grad_v;
  void* dx;
  void* dv;
  void* dz;
  float* dbias;
  int64_t batch, heads, tokens, dim, block, entries;
  int64_t block_begin, block_end;
  int64_t pos_base;
  int32_t x_dtype, z_dtype;
  float rmsnorm_eps; /* treatment of the stored entries: < 0 off */
  int32_t rope_dims; /* 0: off */
  float rope_base;
  const void* xb;    /* dual mode: the b-series, its bias and outputs */
  const void* zb;
  const float* bias_b;
  void* dxb;
  void* dzb;
  float* dbias_b;
  lbca_strides x_st, v_st, z_st, grad_x_st, grad_v_st, dx_st, dv_st, dz_st, xb_st, zb_st, dxb_st, dzb_st;
} lbca_pool_grad_args;

LBCA_API int lbca_pool_blocks_backward_workspace(const lbca_pool_grad_args* a, size_t* bytes);
LBCA_API int lbca_pool_blocks_backward(const lbca_pool_grad_args* a, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ------------------------------------------------------------------------ */
/* Decode-time cache step (mSeek "How LBCA works" steps 1-3: the newest token
 * joins the raw cache; a block that is complete and, under the EXCLUSIVE rule,
 * wholly older than the window is pooled into one entry; HCA "What is
 * implemented" item 1 for the OVERLAP rule, where every complete block is an
 * entry).
 *
 * Raw cache: a mirrored ring of `ring` slots.  Position s is stored in rows
 * (s mod ring) and (s mod ring) + ring of the raw buffers, so every run of at
 * most `ring` consecutive positions is one contiguous range of rows.  For
 * sequence b whose new token sits at t = pos[b] (positions before t appended
 * by earlier calls, in order) one call:
 *   1. writes x_new[b], v_new[b], z_new[b] to both rows of position t;
 *   2. pools block j into entry row j when it becomes visible at t:
 *      EXCLUSIVE: t+1-W > 0 and (t+1-W) % m == 0, j = (t+1-W)/m - 1;
 *      OVERLAP:   (t+1) % m == 0,                 j = (t+1)/m - 1;
 *      exactly as lbca_pool_blocks (bias, treatment), reading the block's
 *      tokens from the ring; skipped when j >= entries;
 *   3. writes raw_pos_base[b] = rb - (rb mod ring), rb = raw_begin(t), so that
 *      lbca_attend_decode with raw rows = 2 * ring and this raw_pos_base reads
 *      the raw span of t from the ring.
 * Dual mode (xb_new != NULL, CSA "What is implemented" item 1): the b-series
 * token (xb_new, zb_new) goes to its own ring (raw_xb, raw_zb) and entry j
 * pools block j of the a-series with block j-1 of the b-series under one
 * softmax per channel (bias_b for the b part), as lbca_pool_blocks in dual mode.
 * The ring must hold every token a step reads: ring >= W + m (EXCLUSIVE: the
 * oldest token of the due block is t+1-W-m) or ring >= max(W, m) (OVERLAP),
 * and in dual mode, which also reads block j-1, ring >= W + 2 m (EXCLUSIVE) or
 * ring >= max(W, 2 m) (OVERLAP).  Sequences with t < 0 are skipped.
 *
 *   x_new, v_new   [batch, heads, dim]          x_dtype
 *   z_new          [batch, heads, dim]          z_dtype
 *   raw_x, raw_v   [batch, heads, 2*ring, dim]  x_dtype
 *   raw_z          [batch, heads, 2*ring, dim]  z_dtype
 *   bias           [heads, block, dim] float32
 *   out_x, out_v   [batch, heads, entries, dim] x_dtype
 *   pos            [batch] int64 (device);  raw_pos_base [batch] int64 (device, written)
 *   xb_new, zb_new, raw_xb, raw_zb, bias_b: the b-series, as x_new, z_new,
 *   raw_x, raw_z, bias (all NULL outside dual mode)
 * v_new, raw_v and out_v are all NULL for a shared series (x is key and value).
 * Treatment flags as lbca_pool_blocks (shared series only; dual mode has no values).
 * Constraints: dim a power of two in [8, 512].
 * Errors: INVALID_ARG for a NULL required pointer, a ring below the bound,
 * bad sizes or mode; UNSUPPORTED for treatment with v.
 */
typedef struct lbca_cache_args {
  const void* x_new;
  const void* v_new;
  const void* z_new;
  void* raw_x;
  void* raw_v;
  void* raw_z;
  const float* bias;
  void* out_x;
  void* out_v;
  const int64_t* pos;
  int64_t* raw_pos_base;
  int64_t batch, heads, dim, block, window, ring, entries;
  int32_t mode, x_dtype, z_dtype;
  float rmsnorm_eps; /* < 0: off */
  int32_t rope_dims; /* 0: off */
  float rope_base;
  const void* xb_new; /* dual mode: the b-series */
  const void* zb_new;
  void* raw_xb;
  void* raw_zb;
  const float* bias_b;
  lbca_strides x_new_st, v_new_st, z_new_st, raw_x_st, raw_v_st, raw_z_st, out_x_st, out_v_st;
  lbca_strides xb_new_st, zb_new_st, raw_xb_st, raw_zb_st;
} lbca_cache_args;

LBCA_API int lbca_cache_append(const lbca_cache_args* a, void* stream);

/* ------------------------------------------------------------------------ */
/* One decode step of an LBCA layer in one launch (mSeek "How LBCA works"
 * steps 1-4 and "Repository layout", generation through the LBCA cache):
 * the cache step and the attention of lbca_cache_append + lbca_attend_decode,
 * fused, for the EXCLUSIVE rule with separate K and V series.  For sequence b
 * at t = pos[b] (positions before t appended by earlier calls, in order):
 *   1. k_new[b], v_new[b], z_new[b] go to both ring rows of position t, as
 *      lbca_cache_append;
 *   2. when t completes a block ((t+1) % block == 0) it is pooled into entry
 *      j = (t+1)/block - 1 (skipped when j >= entries), bitwise as
 *      lbca_pool_blocks.  Unlike lbca_cache_append, which pools a block on
 *      the step that makes it visible, this pools it on its last token: under
 *      EXCLUSIVE a block is visible only once it is wholly older than the
 *      window, so no query of the same step reads it, and the one launch
 *      needs no ordering between its cache and attention work.  A caller that
 *      starts decoding after a prefill has pooled every block completed by
 *      then (not only the visible ones);
 *   3. raw_pos_base[b] is written as lbca_cache_append writes it;
 *   4. out[b], lse[b] are lbca_attend_decode's for q[b] at t over the pooled
 *      entries and the ring (raw rows 2 * ring), the row at t being k_new[b]
 *      and v_new[b] themselves.
 *
 *   q                [batch, q_heads, dim]          dtype
 *   k_new, v_new     [batch, kv_heads, dim]         dtype
 *   z_new            [batch, kv_heads, dim]         z_dtype (pooling logits)
 *   raw_k, raw_v     [batch, kv_heads, 2*ring, dim] dtype
 *   raw_z            [batch, kv_heads, 2*ring, dim] z_dtype
 *   bias             [kv_heads, block, dim] float32
 *   pooled_k/v       [batch, kv_heads, entries, dim] dtype
 *   pos              [batch] int64 (device);  raw_pos_base [batch] int64 (device, written)
 *   sink             [q_heads] float32 or NULL
 *   out              [batch, q_heads, dim] float32;  lse [batch, q_heads] float32 or NULL
 * Supported: dtype BF16 with dim 64 or 128, z_dtype F32 or BF16, ring >=
 * window + block, and the constraints of lbca_attend_decode and
 * lbca_cache_append.  One launch when the decode rows are not split across
 * workgroups (lbca_decode_step_workspace reports 0), else a second (merge).
 * Workspace as lbca_attend_decode (the same split partials).
 */
typedef struct lbca_step_args {
  const void* q;
  const void* k_new;
  const void* v_new;
  const void* z_new;
  void* raw_k;
  void* raw_v;
  void* raw_z;
  const float* bias;
  void* pooled_k;
  void* pooled_v;
  const int64_t* pos;
  int64_t* raw_pos_base;
  const float* sink;
  float* out;
  float* lse;
  int64_t batch, q_heads, kv_heads, dim, block, window, ring, entries;
  int32_t dtype, z_dtype;
  float scale;
  lbca_strides q_st, k_new_st, v_new_st, z_new_st, raw_k_st, raw_v_st, raw_z_st, pooled_k_st, pooled_v_st,
      out_st;
} lbca_step_args;

LBCA_API int lbca_decode_step_workspace(const lbca_step_args* a, size_t* bytes);
LBCA_API int lbca_decode_step(const lbca_step_args* a, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Decode attention: one query per sequence (mSeek "How LBCA works" step 4;
 * HCA "What is implemented" item 2; CSA "What is implemented" item 3).
 *
 * For query head h (KV head h / G, G = q_heads / kv_heads) of sequence b at
 * position t = pos[b], the visible rows are the pooled entries j < n_pooled(t)
 * (or, with sel_idx, the listed entries that are visible; -1 and invisible
 * ids are skipped) followed by the raw span [raw_begin(t), t], read from the
 * raw buffer row (position - raw_pos_base[b]).  One softmax over
 *   logit = scale * q . k_row
 * for all of them, plus exp(sink[h]) in the denominator when sink != NULL.
 *   out[b,h,:] = sum softmax * v_row;  lse[b,h] = log(sum exp(logit) [+ exp(sink)])
 * Shared series (pooled_v == raw_v == NULL): the row is both key and value.
 * Treatment (shared series only): rmsnorm_eps >= 0 normalises q and every RAW
 * row; rope_dims > 0 rotates q at t and every raw row at its position, and
 * rotates the output's last rope_dims dims by -t.  Pooled entries are used as
 * stored (write them with the same treatment through lbca_pool_blocks).
 *
 *   q            [batch, q_heads, dim]               dtype
 *   pooled_k/v   [batch, kv_heads, entries, dim]     dtype
 *   raw_k/v      [batch, kv_heads, raw_rows, dim]    dtype
 *   pos          [batch] int64 (device)
 *   raw_pos_base [batch] int64 (device) or NULL = 0
 *   sel_idx      [batch, k_sel] int32 (device) or NULL
 *   sink         [q_heads] float32 (device) or NULL
 *   out          [batch, q_heads, dim] float32;  lse [batch, q_heads] float32 or NULL
 * Supported: dtype BF16 with dim in {64,128,256,512}, G <= 64, rope_dims in
 * {0, 64, 128}, pooled and raw slices of one (sequence, KV head) below 2 GiB
 * (entries * dim and raw_rows * dim < 2^30), k_sel <= 32768, batch <= 65535
 * (MFMA path); dtype F32 with dim % 64 == 0, dim <= 512 and no treatment.
 * A sequence whose visible rows do not fit (n_pooled > entries, raw span
 * outside the raw buffer, t < 0) gets NaN in out and lse.
 * Workspace: lbca_attend_decode_workspace reports the bytes (0 when the rows
 * of a sequence are not split across workgroups; otherwise the split
 * partials).  Pass at least that many bytes of device memory, 16-byte
 * aligned; contents on entry do not matter.  Calls sharing one workspace must
 * not overlap.
 */
typedef struct lbca_decode_args {
  const void* q;
  const void* pooled_k;
  const void* pooled_v;
  const void* raw_k;
  const void* raw_v;
  const int64_t* pos;
  const int64_t* raw_pos_base;
  const int32_t* sel_idx;
  const float* sink;
  float* out;
  float* lse;
  int64_t batch, q_heads, kv_heads, dim, entries, raw_rows, k_sel;
  int64_t block, window;
  int32_t mode, dtype;
  float scale;
  float rmsnorm_eps; /* < 0: off */
  int32_t rope_dims; /* 0: off */
  float rope_base;
  lbca_strides q_st, pooled_k_st, pooled_v_st, raw_k_st, raw_v_st, out_st;
} lbca_decode_args;

LBCA_API int lbca_attend_decode_workspace(const lbca_decode_args* a, size_t* bytes);
LBCA_API int lbca_attend_decode(const lbca_decode_args* a, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Decode attention that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, validation, kernels and results as
 * lbca_attend_decode; the split partials go to a static scratch array that the
 * library holds in every GPU's memory until the process ends instead of a
 * caller workspace.  The scratch is at most LBCA_NOALLOC_SCRATCH_BYTES; a call
 * whose lbca_attend_decode_workspace size exceeds it returns
 * LBCA_ERR_TOO_LARGE before any device work.  The stream must belong to the
 * calling thread's current device.  Every call on one GPU shares that GPU's
 * scratch: calls that overlap on one GPU (other streams, other threads) race.
 * The scratch needs no initialisation (the kernels overwrite every partial
 * they read).  No hipMalloc, hipFree or allocating library call is made; the
 * first call on a device looks the scratch address up once.
 */
#define LBCA_NOALLOC_SCRATCH_BYTES (16u << 20)
LBCA_API int lbca_attend_decode_noalloc(const lbca_decode_args* a, void* stream);

/* ------------------------------------------------------------------------ */
/* Prefill attention over a chunk of q_len consecutive queries (mSeek "How LBCA
 * works" steps 4-5 and its chunked bounded-memory path): query i of the chunk
 * sits at position t = q_pos0 + i and sees exactly what lbca_attend_decode
 * would show it at t (per-query visibility), so chunked prefill equals
 * one-shot prefill.  A chunked caller pools the blocks the chunk's last query
 * may see before calling this.
 *
 *   q            [batch, q_len, q_heads, dim]            dtype
 *   pooled_k/v   [batch, kv_heads, entries, dim]         dtype (v NULL: shared)
 *   raw_k/v      [batch, kv_heads, raw_rows, dim]        row r = position raw_pos_base + r
 *   sink         [q_heads] float32 or NULL
 *   out          [batch, q_len, q_heads, dim]            out_dtype (F32 or BF16)
 *   lse          [batch, q_len, q_heads] float32 or NULL
 * Supported: BF16 with dim in {64,128}, scale > 0, positions and
 * q_len * (q_heads / kv_heads) below 2^31 (MFMA path); F32 with dim % 64 == 0,
 * dim <= 512.  Errors: INVALID_ARG if some query's pooled entries exceed
 * `entries` or its raw span leaves the raw buffer (checked on the host).
 */
typedef struct lbca_prefill_args {
  const void* q;
  const void* pooled_k;
  const void* pooled_v;
  const void* raw_k;
  const void* raw_v;
  const float* sink;
  void* out;
  float* lse;
  int64_t batch, q_len, q_heads, kv_heads, dim, entries, raw_rows;
  int64_t q_pos0, raw_pos_base, block, window;
  int32_t mode, dtype, out_dtype;
  float scale;
  lbca_strides q_st, pooled_k_st, pooled_v_st, raw_k_st, raw_v_st, out_st;
} lbca_prefill_args;

LBCA_API int lbca_attend_prefill(const lbca_prefill_args* a, void* stream);

/* ------------------------------------------------------------------------ */
/* Gradients of lbca_attend_prefill.  The forward is mSeek "How LBCA works"
 * steps 4-5; the layer is trained end to end (mSeek "Experiment at a glance"),
 * which needs these.  For each query row with forward output O and
 * log-sum-exp lse (sink included), over the rows it sees (same visibility as
 * the forward): P = exp(scale q.k - lse), D = dO . O, dS = P (dO . v - D), and
 *   grad_q = scale sum_k dS k,  grad_k += scale dS q,  grad_v += P dO,
 *   grad_sink[h] += -sum_rows exp(sink[h] - lse) D.
 *
 *   q, grad_out      [batch, q_len, q_heads, dim]          dtype
 *   pooled_k/v       [batch, kv_heads, entries, dim]       dtype
 *   raw_k/v          [batch, kv_heads, raw_rows, dim]      row r = position raw_pos_base + r
 *                    (v NULL: one series is both K and V; its gradient, the
 *                    sum of both roles, goes to grad_pooled_k / grad_raw_k and
 *                    grad_pooled_v / grad_raw_v must be NULL)
 *   out              [batch, q_len, q_heads, dim]          out_dtype (F32 or BF16): the forward's output
 *   lse              [batch, q_len, q_heads] float32       the forward's lse
 *   sink             [q_heads] float32 or NULL             the forward's sink
 *   grad_q           [batch, q_len, q_heads, dim] float32  overwritten
 *   grad_pooled_k/v  [batch, kv_heads, entries, dim] float32
 *   grad_raw_k/v     [batch, kv_heads, raw_rows, dim] float32
 *   grad_sink        [q_heads] float32 or NULL (needs sink)
 * accumulate = 0: the key, value and sink gradients are overwritten (rows that
 * no query of the call sees get 0); 1: added to them, so a chunked backward
 * calls this once per chunk of queries.
 * Supported: dtype BF16, dim 64 or 128, scale > 0, batch * q_len * q_heads
 * and raw_pos_base + raw_rows + block + window below 2^31,
 * batch * kv_heads <= 65535.  The visibility
 * checks of lbca_attend_prefill apply (INVALID_ARG).
 * Workspace (lbca_attend_prefill_backward_workspace; 16-byte aligned,
 * contents on entry do not matter, calls sharing one must not overlap): D per
 * query row (4 * batch * q_len * q_heads bytes, rounded up to 256), then one
 * fp32 partial gradient per pooled entry, K and V (K only when shared), and
 * run of 512 query positions: 4 * batch * kv_heads * T * S * 128 * nser * dim
 * bytes with T = ceil(n / 128) for the n entries the last query sees, S =
 * ceil((q_pos0 + q_len - max(f, q_pos0)) / 512), f = block + window - 1
 * (EXCLUSIVE) or block - 1 (OVERLAP) the first position that sees entry 0,
 * nser = 2 (1 shared).  grad_q and grad_sink are summed with floating-point
 * atomics, so their last bits can differ from run to run.
 */
typedef struct lbca_prefill_grad_args {
  const void* q;
  const void* pooled_k;
  const void* pooled_v;
  const void* raw_k;
  const void* raw_v;
  const float* sink;
  const void* out;
  const float* lse;
  const void* grad_out;
  float* grad_q;
  float* grad_pooled_k;
  float* grad_pooled_v;
  float* grad_raw_k;
  float* grad_raw_v;
  float* grad_sink;
  int64_t batch, q_len, q_heads, kv_heads, dim, entries, raw_rows;
  int64_t q_pos0, raw_pos_base, block, window;
  int32_t mode, dtype, out_dtype, accumulate;
  float scale;
  lbca_strides q_st, pooled_k_st, pooled_v_st, raw_k_st, raw_v_st, out_st, grad_out_st;
  lbca_strides grad_q_st, grad_pooled_k_st, grad_pooled_v_st, grad_raw_k_st, grad_raw_v_st;
} lbca_prefill_grad_args;

LBCA_API int lbca_attend_prefill_backward_workspace(const lbca_prefill_grad_args* a, size_t* bytes);
LBCA_API int lbca_attend_prefill_backward(const lbca_prefill_grad_args* a, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* CSA lightning indexer + top-k (CSA "What is implemented" item 2).
 * For sequence b at position t = pos[b], the visible compressed keys are
 * j < n_vis = min(floor((t+1)/block), entries) (OVERLAP rule).  Score
 *   I_j = sum_h head_w[b,h] * relu(q_idx[b,h,:] . keys[b,j,:])   (fp32)
 * and select the k largest; ties go to the lower index; if n_vis < k all
 * visible ids are selected and the rest of the row is -1.  out_idx holds the
 * chosen ids in ascending order; out_score (optional) their scores (NaN where
 * padded).  -0.0 and +0.0 compare equal; scores must not be NaN.
 *
 *   q_idx [batch, heads, dim] dtype;  head_w [batch, heads] float32
 *   keys  [batch, entries, dim] dtype;  pos [batch] int64 (device)
 *   out_idx [batch, k] int32;  out_score [batch, k] float32 or NULL
 * Supported: dtype BF16; dim in {32, 64, 128}; heads <= 16;
 * 1 <= k <= 2048; entries <= 65536.  Workspace (csa_index_topk_workspace,
 * 16-byte aligned, caller-owned, contents need no initialisation): the fp32
 * scores, batch x entries rounded up to 4; plus, when the selection runs in
 * two stages (entries span P = ceil(entries / 4096) >= 3 slices of 4096,
 * 4 k <= 4096 and P k <= 16384), batch x (P k rounded up to 4) candidate
 * (key, id) pairs of 8 bytes.
 * Sequences with t < 0 get an all -1 row.
 */
typedef struct csa_index_args {
  const void* q_idx;
  const float* head_w;
  const void* keys;
  const int64_t* pos;
  int32_t* out_idx;
  float* out_score;
  int64_t batch, heads, dim, entries, k, block;
  int32_t dtype;
  lbca_strides q_idx_st, keys_st;
} csa_index_args;

LBCA_API int csa_index_topk_workspace(const csa_index_args* a, size_t* bytes);
LBCA_API int csa_index_topk(const csa_index_args* a, void* workspace, size_t workspace_bytes,
                   void* stream);

/* ------------------------------------------------------------------------ */
/* CSA sparse prefill of a chunk of q_len consecutive queries (CSA "What is
 * implemented", second and third items, applied to every query of a chunk).
 * Query i of sequence b sits at t = q_pos0 + i.  It scores the indexer keys
 * visible at t (OVERLAP rule, j < floor((t+1)/block)), keeps its own top-k
 * exactly as csa_index_topk would, and attends to those entries plus its raw
 * window [max(0, t-window+1), t] under one softmax, exactly as
 * lbca_attend_decode with sel_idx would at t (MQA: one shared K = V series;
 * RMSNorm / partial RoPE of q and the raw rows, the output's last rope_dims
 * turned back by -t; entries are used as stored, already treated).
 *
 *   q_idx    [batch, q_len, idx_heads, idx_dim] dtype;  head_w [batch, q_len, idx_heads] float32
 *   idx_keys [batch, entries, idx_dim] dtype
 *   q        [batch, q_len, q_heads, dim] dtype
 *   entries  [batch, entries, dim] dtype  (pooled, treated)
 *   raw      [batch, raw_rows, dim] dtype  row r = position raw_pos_base + r (host scalar)
 *   sink     [q_heads] float32 or NULL
 *   out      [batch, q_len, q_heads, dim] float32;  lse [batch, q_len, q_heads] float32 or NULL
 *   out_idx  [batch, q_len, k] int32 or NULL: each query's selection (ascending, -1 padded)
 * Supported: dtype BF16; idx_dim in {32, 64, 128}, idx_heads <= 16,
 * 1 <= k <= 2048, entries <= 65536; dim 512 with q_heads a multiple of 32 up
 * to 64; batch * q_len <= 65535; entries * dim and raw_rows * dim < 2^30.
 * Errors: INVALID_ARG if the last query's visible entries exceed `entries`
 * or some query's raw window leaves the raw buffer (checked on the host).
 * Workspace (csa_sparse_prefill_workspace; 16-byte aligned, caller-owned,
 * contents on entry do not matter): per-query positions and selections, the
 * fp32 scores (batch * q_len rows of entries), and split partials when a
 * query's rows are split.  Calls sharing one workspace must not overlap.
 */
typedef struct csa_prefill_args {
  const void* q_idx;
  const float* head_w;
  const void* idx_keys;
  const void* q;
  const void* entries;
  const void* raw;
  const float* sink;
  float* out;
  float* lse;
  int32_t* out_idx;
  int64_t batch, q_len, idx_heads, idx_dim, q_heads, dim, n_entries, raw_rows, k;
  int64_t q_pos0, raw_pos_base, block, window;
  int32_t dtype;
  float scale;
  float rmsnorm_eps; /* < 0: off */
  int32_t rope_dims; /* 0: off */
  float rope_base;
  lbca_strides q_idx_st, idx_keys_st, q_st, entries_st, raw_st, out_st;
} csa_prefill_args;

LBCA_API int csa_sparse_prefill_workspace(const csa_prefill_args* a, size_t* bytes);
LBCA_API int csa_sparse_prefill(const csa_prefill_args* a, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ------------------------------------------------------------------------ */
/* Grouped projection GEMM: the projections around the path (CSA "What is
 * implemented" items 2 and 3: low-rank indexer queries and the grouped output
 * projection; HCA "What is implemented": the grouped output projection).
 *   C[g][i][j] = sum_l A[g][i][l] * W[g][j][l]     (fp32 accumulation)
 * for g < groups, i < m, j < n, l < k.  Weights are stored [out, in]:
 *   A  at a + g * a_group_stride + i * lda + l     a_dtype (F32 rounded to bf16, or BF16)
 *   W  at w + g * w_group_stride + j * ldw + l     BF16
 *   C  at c + g * c_group_stride + i * ldc + j     c_dtype (F32 or BF16), overwritten
 * (strides in elements).  Low-rank indexer queries: groups = 1, A = the query
 * latents [tokens, d_c], W = [heads * d_I, d_c], C = [tokens, heads * d_I].
 * Grouped output projection, stage 1: groups = g, A = the attention output
 * [tokens, H * c] with a_group_stride (H/g) * c and lda = H * c, W = [g, d_g,
 * (H/g) * c], C = [tokens, g * d_g] with c_group_stride d_g; stage 2: groups =
 * 1, A = that C, W = [d_model, g * d_g].
 * Constraints: k a multiple of 8; lda, ldw >= k and multiples of 8; ldc >= n;
 * A and W group strides multiples of 8; every 128-row band of A
 * or W below 2 GiB; groups and ceil(m / 128) at most 65535.  C must not
 * overlap A or W.  Errors: INVALID_ARG for NULL or misaligned pointers and bad
 * sizes, UNSUPPORTED for dtypes, k or strides outside the constraints.
 */
typedef struct lbca_gemm_args {
  const void* a;
  const void* w;
  void* c;
  int64_t groups, m, n, k;
  int64_t lda, ldw, ldc;
  int64_t a_group_stride, w_group_stride, c_group_stride;
  int32_t a_dtype, c_dtype;
} lbca_gemm_args;

LBCA_API int lbca_grouped_gemm(const lbca_gemm_args* a, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LBCA_H */
