// C-ABI entry points of liblbca: host-side validation, then one launcher call.
// Validation never touches the GPU, so every argument error is reported
// (and testable) on a machine without one.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "lbca_internal.h"

namespace {

bool is_dtype(int32_t d) { return d == LBCA_F32 || d == LBCA_BF16; }
bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
constexpr int64_t kMaxElems = int64_t(1) << 46;  // guards products against overflow

bool sane_product(std::initializer_list<int64_t> dims) {
  int64_t p = 1;
  for (int64_t d : dims) {
    if (d < 0) return false;
    if (d == 0) return true;
    if (p > kMaxElems / d) return false;
    p *= d;
  }
  return true;
}

int check_treatment(float eps, int32_t rope_dims, float rope_base, int64_t dim) {
  if (isnan(eps) || isinf(eps)) return LBCA_ERR_INVALID_ARG;
  if (rope_dims < 0 || rope_dims > dim) return LBCA_ERR_INVALID_ARG;
  if (rope_dims > 0 && (rope_dims % 16 != 0)) return LBCA_ERR_UNSUPPORTED;
  if (rope_dims > 0 && !(rope_base > 1.0f && isfinite(rope_base))) return LBCA_ERR_INVALID_ARG;
  return LBCA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LBCA_OK : LBCA_ERR_HIP; }

}  // namespace

extern "C" {

int lbca_abi_version(void) { return LBCA_ABI_VERSION; }

const char* lbca_status_string(int status) {
  switch (status) {
    case LBCA_OK: return "ok";
    case LBCA_ERR_INVALID_ARG: return "invalid argument";
    case LBCA_ERR_UNSUPPORTED: return "unsupported dtype, dimension or flag combination";
    case LBCA_ERR_WORKSPACE: return "workspace missing or too small";
    case LBCA_ERR_HIP: return "HIP runtime error";
    case LBCA_ERR_TOO_LARGE: return "sizes need more than the static scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

int lbca_visible_range(int64_t t, int64_t m, int64_t W, int32_t mode, int64_t* n_pooled,
                       int64_t* raw_begin) {
  if (!n_pooled || !raw_begin || t < 0 || m < 1 || W < 1) return LBCA_ERR_INVALID_ARG;
  if (mode == LBCA_EXCLUSIVE) {
    const int64_t x = t + 1 - W;
    *n_pooled = x > 0 ? x / m : 0;
    *raw_begin = *n_pooled * m;
  } else if (mode == LBCA_OVERLAP) {
    *n_pooled = (t + 1) / m;
    *raw_begin = t - W + 1 > 0 ? t - W + 1 : 0;
  } else {
    return LBCA_ERR_INVALID_ARG;
  }
  return LBCA_OK;
}

// ---------------------------------------------------------------------------
int lbca_pool_blocks(const lbca_pool_args* a, void* stream) {
  if (!a || !a->x || !a->z || !a->bias || !a->out_x) return LBCA_ERR_INVALID_ARG;
  if ((a->v == nullptr) != (a->out_v == nullptr)) return LBCA_ERR_INVALID_ARG;
  const bool dual = a->xb != nullptr || a->zb != nullptr || a->bias_b != nullptr;
  if (dual && !(a->xb && a->zb && a->bias_b)) return LBCA_ERR_INVALID_ARG;
  if (dual && a->v) return LBCA_ERR_UNSUPPORTED;
  if (!is_dtype(a->x_dtype) || !is_dtype(a->z_dtype)) return LBCA_ERR_INVALID_ARG;
  if (a->batch < 0 || a->heads < 1 || a->tokens < 0 || a->block < 1 || a->entries < 0)
    return LBCA_ERR_INVALID_ARG;
  if (!pow2(a->dim) || a->dim < 8) return a->dim > 0 ? LBCA_ERR_UNSUPPORTED : LBCA_ERR_INVALID_ARG;
  if (a->dim > 512) return LBCA_ERR_UNSUPPORTED;
  if (a->block_begin < 0 || a->block_end < a->block_begin || a->block_end > a->entries)
    return LBCA_ERR_INVALID_ARG;
  if (!sane_product({a->batch, a->heads, a->tokens, a->dim}) ||
      !sane_product({a->batch, a->heads, a->entries, a->dim}) ||
      !sane_product({a->heads, a->block, a->dim}) || a->block_end > kMaxElems / a->block)
    return LBCA_ERR_INVALID_ARG;
  const bool treat = a->rmsnorm_eps >= 0.f || a->rope_dims != 0;
  int st = check_treatment(a->rmsnorm_eps, a->rope_dims, a->rope_base, a->dim);
  if (st != LBCA_OK) return st;
  if (treat && a->v) return LBCA_ERR_UNSUPPORTED;
  if (!aligned16(a->x) || !aligned16(a->v) || !aligned16(a->z) || !aligned16(a->bias) ||
      !aligned16(a->xb) || !aligned16(a->zb) || !aligned16(a->bias_b) || !aligned16(a->out_x) ||
      !aligned16(a->out_v))
    return LBCA_ERR_INVALID_ARG;
  if (a->block_end > a->block_begin) {
    const int64_t first_block = (dual && a->block_begin > 0) ? a->block_begin - 1 : a->block_begin;
    const int64_t lo = first_block * a->block - a->pos_base;
    const int64_t hi = a->block_end * a->block - a->pos_base;
    if (lo < 0 || hi > a->tokens) return LBCA_ERR_INVALID_ARG;
  }
  if (a->batch == 0 || a->block_end == a->block_begin) return LBCA_OK;
  return hip_status(lbca::launch_pool(*a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
static int validate_pool_grad(const lbca_pool_grad_args* a) {
  if (!a || !a->x || !a->z || !a->bias || !a->grad_x || !a->dx || !a->dz || !a->dbias)
    return LBCA_ERR_INVALID_ARG;
  const bool has_v = a->v != nullptr;
  if ((a->grad_v != nullptr) != has_v || (a->dv != nullptr) != has_v) return LBCA_ERR_INVALID_ARG;
  const bool dual = a->xb || a->zb || a->bias_b || a->dxb || a->dzb || a->dbias_b;
  if (dual && !(a->xb && a->zb && a->bias_b && a->dxb && a->dzb && a->dbias_b)) return LBCA_ERR_INVALID_ARG;
  if (!is_dtype(a->x_dtype) || !is_dtype(a->z_dtype)) return LBCA_ERR_INVALID_ARG;
  if (a->batch < 0 || a->heads < 1 || a->tokens < 0 || a->block < 1 || a->entries < 0)
    return LBCA_ERR_INVALID_ARG;
  if (!pow2(a->dim) || a->dim < 8) return a->dim > 0 ? LBCA_ERR_UNSUPPORTED : LBCA_ERR_INVALID_ARG;
  if (a->dim > 512) return LBCA_ERR_UNSUPPORTED;
  if (a->block_begin < 0 || a->block_end < a->block_begin || a->block_end > a->entries)
    return LBCA_ERR_INVALID_ARG;
  if (!sane_product({a->batch, a->heads, a->tokens, a->dim}) ||
      !sane_product({a->batch, a->heads, a->entries, a->dim}) ||
      !sane_product({a->heads, a->block, a->dim}) || a->block_end > kMaxElems / a->block)
    return LBCA_ERR_INVALID_ARG;
  const bool treat = a->rmsnorm_eps >= 0.f || a->rope_dims != 0;
  const int st = check_treatment(a->rmsnorm_eps, a->rope_dims, a->rope_base, a->dim);
  if (st != LBCA_OK) return st;
  if ((treat || dual) && has_v) return LBCA_ERR_UNSUPPORTED;
  if ((dual ? 2 : 1) * a->block * a->dim > 8192 || a->heads > 65535) return LBCA_ERR_UNSUPPORTED;  // 4 tokens per lane
  if (!aligned16(a->x) || !aligned16(a->v) || !aligned16(a->z) || !aligned16(a->bias) ||
      !aligned16(a->grad_x) || !aligned16(a->grad_v) || !aligned16(a->dx) || !aligned16(a->dv) ||
      !aligned16(a->dz) || !aligned16(a->dbias) || !aligned16(a->xb) || !aligned16(a->zb) ||
      !aligned16(a->bias_b) || !aligned16(a->dxb) || !aligned16(a->dzb) || !aligned16(a->dbias_b))
    return LBCA_ERR_INVALID_ARG;
  if (a->block_end > a->block_begin) {
    const int64_t first_block = (dual && a->block_begin > 0) ? a->block_begin - 1 : a->block_begin;
    const int64_t lo = first_block * a->block - a->pos_base;
    const int64_t hi = a->block_end * a->block - a->pos_base;
    if (lo < 0 || hi > a->tokens) return LBCA_ERR_INVALID_ARG;
  }
  return LBCA_OK;
}

int lbca_pool_blocks_backward_workspace(const lbca_pool_grad_args* a, size_t* bytes) {
  if (!bytes) return LBCA_ERR_INVALID_ARG;
  const int st = validate_pool_grad(a);
  if (st != LBCA_OK) return st;
  *bytes = lbca::pool_grad_workspace_bytes(*a);
  return LBCA_OK;
}

int lbca_pool_blocks_backward(const lbca_pool_grad_args* a, void* workspace, size_t workspace_bytes,
                              void* stream) {
  const int st = validate_pool_grad(a);
  if (st != LBCA_OK) return st;
  const size_t need = lbca::pool_grad_workspace_bytes(*a);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return LBCA_ERR_WORKSPACE;
  return hip_status(lbca::launch_pool_grad(*a, workspace, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
static int validate_cache(const lbca_cache_args* a) {
  if (!a || !a->x_new || !a->z_new || !a->raw_x || !a->raw_z || !a->bias || !a->out_x || !a->pos ||
      !a->raw_pos_base)
    return LBCA_ERR_INVALID_ARG;
  const bool has_v = a->v_new != nullptr;
  if ((a->raw_v != nullptr) != has_v || (a->out_v != nullptr) != has_v) return LBCA_ERR_INVALID_ARG;
  const bool dual = a->xb_new || a->zb_new || a->raw_xb || a->raw_zb || a->bias_b;
  if (dual && !(a->xb_new && a->zb_new && a->raw_xb && a->raw_zb && a->bias_b)) return LBCA_ERR_INVALID_ARG;
  if (dual && has_v) return LBCA_ERR_UNSUPPORTED;
  if (!is_dtype(a->x_dtype) || !is_dtype(a->z_dtype)) return LBCA_ERR_INVALID_ARG;
  if (a->mode != LBCA_EXCLUSIVE && a->mode != LBCA_OVERLAP) return LBCA_ERR_INVALID_ARG;
  if (a->batch < 0 || a->heads < 1 || a->block < 1 || a->window < 1 || a->entries < 0 || a->ring < 1)
    return LBCA_ERR_INVALID_ARG;
  if (!pow2(a->dim) || a->dim < 8) return a->dim > 0 ? LBCA_ERR_UNSUPPORTED : LBCA_ERR_INVALID_ARG;
  if (a->dim > 512) return LBCA_ERR_UNSUPPORTED;
  // every token a step reads must still be in the ring
  const int64_t need = a->mode == LBCA_EXCLUSIVE ? a->window + a->block
                                                  : (a->window > a->block ? a->window : a->block);
  if (a->window > kMaxElems || a->block > kMaxElems || a->ring < need) return LBCA_ERR_INVALID_ARG;
  if (dual && a->ring < (a->mode == LBCA_EXCLUSIVE ? a->window + 2 * a->block : 2 * a->block))
    return LBCA_ERR_INVALID_ARG;  // block j-1 of the b-series is read too
  if (a->batch > INT32_MAX / a->heads) return LBCA_ERR_UNSUPPORTED;  // one workgroup per (sequence, head)
  if (!sane_product({a->batch, a->heads, 2 * a->ring, a->dim}) ||
      !sane_product({a->batch, a->heads, a->entries, a->dim}) || !sane_product({a->heads, a->block, a->dim}))
    return LBCA_ERR_INVALID_ARG;
  const bool treat = a->rmsnorm_eps >= 0.f || a->rope_dims != 0;
  int st = check_treatment(a->rmsnorm_eps, a->rope_dims, a->rope_base, a->dim);
  if (st != LBCA_OK) return st;
  if (treat && has_v) return LBCA_ERR_UNSUPPORTED;
  if (!aligned16(a->x_new) || !aligned16(a->v_new) || !aligned16(a->z_new) || !aligned16(a->raw_x) ||
      !aligned16(a->raw_v) || !aligned16(a->raw_z) || !aligned16(a->bias) || !aligned16(a->out_x) ||
      !aligned16(a->out_v) || !aligned16(a->xb_new) || !aligned16(a->zb_new) || !aligned16(a->raw_xb) ||
      !aligned16(a->raw_zb) || !aligned16(a->bias_b))
    return LBCA_ERR_INVALID_ARG;
  return LBCA_OK;
}

int lbca_cache_append(const lbca_cache_args* a, void* stream) {
  const int st = validate_cache(a);
  if (st != LBCA_OK) return st;
  if (a->batch == 0) return LBCA_OK;
  return hip_status(lbca::launch_cache_append(*a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
static int validate_decode(const lbca_decode_args* a) {
  if (!a || !a->q || !a->pooled_k || !a->raw_k || !a->pos || !a->out) return LBCA_ERR_INVALID_ARG;
  if ((a->pooled_v == nullptr) != (a->raw_v == nullptr)) return LBCA_ERR_INVALID_ARG;
  if (!is_dtype(a->dtype)) return LBCA_ERR_INVALID_ARG;
  if (a->batch < 0 || a->q_heads < 1 || a->kv_heads < 1 || a->q_heads % a->kv_heads != 0)
    return LBCA_ERR_INVALID_ARG;
  if (a->dim < 1 || a->entries < 0 || a->raw_rows < 1 || a->block < 1 || a->window < 1)
    return LBCA_ERR_INVALID_ARG;
  if (a->mode != LBCA_EXCLUSIVE && a->mode != LBCA_OVERLAP) return LBCA_ERR_INVALID_ARG;
  if (a->sel_idx && a->k_sel < 1) return LBCA_ERR_INVALID_ARG;
  if (!isfinite(a->scale)) return LBCA_ERR_INVALID_ARG;
  if (!sane_product({a->batch, a->kv_heads, a->entries, a->dim}) ||
      !sane_product({a->batch, a->kv_heads, a->raw_rows, a->dim}) ||
      !sane_product({a->batch, a->q_heads, a->dim}) || !sane_product({a->batch, a->k_sel}))
    return LBCA_ERR_INVALID_ARG;
  const bool treat = a->rmsnorm_eps >= 0.f || a->rope_dims != 0;
  int st = check_treatment(a->rmsnorm_eps, a->rope_dims, a->rope_base, a->dim);
  if (st != LBCA_OK) return st;
  if (treat && a->pooled_v) return LBCA_ERR_UNSUPPORTED;
  const int64_t G = a->q_heads / a->kv_heads;
  if (a->dtype == LBCA_BF16) {
    if (!(a->dim == 64 || a->dim == 128 || a->dim == 256 || a->dim == 512)) return LBCA_ERR_UNSUPPORTED;
    if (G > 64) return LBCA_ERR_UNSUPPORTED;
    if (!(a->rope_dims == 0 || a->rope_dims == 64 || a->rope_dims == 128)) return LBCA_ERR_UNSUPPORTED;
    // rows are addressed by 32-bit byte offsets within one (sequence, KV head)
    // slice; the merge grid's y/x carry batch and (KV head, head group)
    if (a->entries * a->dim * 2 >= (int64_t(1) << 31) || a->raw_rows * a->dim * 2 >= (int64_t(1) << 31) ||
        a->k_sel > 32768 || a->batch > 65535 || a->kv_heads * ((G + 15) / 16) > 65535)
      return LBCA_ERR_UNSUPPORTED;
  } else {
    if (a->dim % 64 != 0 || a->dim > 512) return LBCA_ERR_UNSUPPORTED;
    if (treat) return LBCA_ERR_UNSUPPORTED;
  }
  if (!aligned16(a->q) || !aligned16(a->pooled_k) || !aligned16(a->pooled_v) ||
      !aligned16(a->raw_k) || !aligned16(a->raw_v) || !aligned16(a->out))
    return LBCA_ERR_INVALID_ARG;
  // the selected ids of one workgroup's row range are staged in LDS; the
  // planner reports sizes that no split count (at most 64) can cover
  if (lbca::plan_decode(*a).unsupported) return LBCA_ERR_UNSUPPORTED;
  return LBCA_OK;
}

int lbca_attend_decode_workspace(const lbca_decode_args* a, size_t* bytes) {
  if (!bytes) return LBCA_ERR_INVALID_ARG;
  int st = validate_decode(a);
  if (st != LBCA_OK) return st;
  *bytes = lbca::plan_decode(*a).ws_bytes;
  return LBCA_OK;
}

int lbca_attend_decode(const lbca_decode_args* a, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int st = validate_decode(a);
  if (st != LBCA_OK) return st;
  const lbca::DecodePlan plan = lbca::plan_decode(*a);
  if (plan.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.ws_bytes || !aligned16(workspace)))
    return LBCA_ERR_WORKSPACE;
  if (a->batch == 0) return LBCA_OK;
  return hip_status(lbca::launch_decode(*a, plan, workspace, static_cast<hipStream_t>(stream)));
}

int lbca_attend_decode_noalloc(const lbca_decode_args* a, void* stream) {
  int st = validate_decode(a);
  if (st != LBCA_OK) return st;
  const lbca::DecodePlan plan = lbca::plan_decode(*a);
  if (plan.ws_bytes > LBCA_NOALLOC_SCRATCH_BYTES) return LBCA_ERR_TOO_LARGE;
  if (a->batch == 0) return LBCA_OK;
  void* ws = nullptr;
  if (plan.ws_bytes > 0 && lbca::static_scratch(&ws) != hipSuccess) return LBCA_ERR_HIP;
  return hip_status(lbca::launch_decode(*a, plan, ws, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// lbca_decode_step: the decode and cache-step arguments it stands for
static void step_parts(const lbca_step_args* a, lbca_decode_args* d, lbca_cache_args* c) {
  *d = lbca_decode_args{};
  d->q = a->q; d->pooled_k = a->pooled_k; d->pooled_v = a->pooled_v;
  d->raw_k = a->raw_k; d->raw_v = a->raw_v; d->pos = a->pos; d->raw_pos_base = a->raw_pos_base;
  d->sel_idx = nullptr; d->sink = a->sink; d->out = a->out; d->lse = a->lse;
  d->batch = a->batch; d->q_heads = a->q_heads; d->kv_heads = a->kv_heads; d->dim = a->dim;
  d->entries = a->entries; d->raw_rows = 2 * a->ring; d->k_sel = 0;
  d->block = a->block; d->window = a->window; d->mode = LBCA_EXCLUSIVE; d->dtype = a->dtype;
  d->scale = a->scale; d->rmsnorm_eps = -1.f; d->rope_dims = 0; d->rope_base = 0.f;
  *c = lbca_cache_args{};
  c->x_new = a->k_new; c->v_new = a->v_new; c->z_new = a->z_new;
  c->raw_x = a->raw_k; c->raw_v = a->raw_v; c->raw_z = a->raw_z; c->bias = a->bias;
  c->out_x = a->pooled_k; c->out_v = a->pooled_v; c->pos = a->pos; c->raw_pos_base = a->raw_pos_base;
  c->batch = a->batch; c->heads = a->kv_heads; c->dim = a->dim; c->block = a->block; c->window = a->window;
  c->ring = a->ring; c->entries = a->entries; c->mode = LBCA_EXCLUSIVE; c->x_dtype = a->dtype;
  c->z_dtype = a->z_dtype; c->rmsnorm_eps = -1.f; c->rope_dims = 0; c->rope_base = 0.f;
}

static int validate_step(const lbca_step_args* a, lbca_decode_args* d, lbca_cache_args* c) {
  if (!a || !a->k_new || !a->v_new || !a->pooled_v || !a->raw_v || !a->raw_pos_base) return LBCA_ERR_INVALID_ARG;
  if (a->ring < 1 || a->ring > kMaxElems) return LBCA_ERR_INVALID_ARG;
  step_parts(a, d, c);
  int st = validate_decode(d);
  if (st != LBCA_OK) return st;
  st = validate_cache(c);
  if (st != LBCA_OK) return st;
  if (a->dtype != LBCA_BF16 || !(a->dim == 64 || a->dim == 128)) return LBCA_ERR_UNSUPPORTED;
  return LBCA_OK;
}

int lbca_decode_step_workspace(const lbca_step_args* a, size_t* bytes) {
  if (!bytes) return LBCA_ERR_INVALID_ARG;
  lbca_decode_args d;
  lbca_cache_args c;
  const int st = validate_step(a, &d, &c);
  if (st != LBCA_OK) return st;
  *bytes = lbca::plan_decode(d).ws_bytes;
  return LBCA_OK;
}

int lbca_decode_step(const lbca_step_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  lbca_decode_args d;
  lbca_cache_args c;
  const int st = validate_step(a, &d, &c);
  if (st != LBCA_OK) return st;
  const lbca::DecodePlan plan = lbca::plan_decode(d);
  if (plan.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.ws_bytes || !aligned16(workspace)))
    return LBCA_ERR_WORKSPACE;
  if (a->batch == 0) return LBCA_OK;
  return hip_status(lbca::launch_decode_step(d, c, plan, workspace, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
int lbca_attend_prefill(const lbca_prefill_args* a, void* stream) {
  if (!a || !a->q || !a->pooled_k || !a->raw_k || !a->out) return LBCA_ERR_INVALID_ARG;
  if ((a->pooled_v == nullptr) != (a->raw_v == nullptr)) return LBCA_ERR_INVALID_ARG;
  if (!is_dtype(a->dtype) || !is_dtype(a->out_dtype)) return LBCA_ERR_INVALID_ARG;
  if (a->batch < 0 || a->q_len < 0 || a->q_heads < 1 || a->kv_heads < 1 ||
      a->q_heads % a->kv_heads != 0)
    return LBCA_ERR_INVALID_ARG;
  if (a->dim < 1 || a->entries < 0 || a->raw_rows < 1 || a->block < 1 || a->window < 1 ||
      a->q_pos0 < 0)
    return LBCA_ERR_INVALID_ARG;
  if (a->mode != LBCA_EXCLUSIVE && a->mode != LBCA_OVERLAP) return LBCA_ERR_INVALID_ARG;
  if (!isfinite(a->scale)) return LBCA_ERR_INVALID_ARG;
  if (!sane_product({a->batch, a->q_len, a->q_heads, a->dim}) ||
      !sane_product({a->batch, a->kv_heads, a->entries, a->dim}) ||
      !sane_product({a->batch, a->kv_heads, a->raw_rows, a->dim}) || a->q_pos0 > kMaxElems)
    return LBCA_ERR_INVALID_ARG;
  if (a->dtype == LBCA_BF16) {
    if (!(a->dim == 64 || a->dim == 128)) return LBCA_ERR_UNSUPPORTED;
    // positive scale (folded into the exponent after the row max); 32-bit rows and positions
    if (!(a->scale > 0.f) || a->q_len * (a->q_heads / a->kv_heads) >= (int64_t(1) << 31) ||
        a->q_pos0 + a->q_len >= (int64_t(1) << 31) || a->batch * a->kv_heads >= (int64_t(1) << 31))
      return LBCA_ERR_UNSUPPORTED;
  } else {
    if (a->dim % 64 != 0 || a->dim > 512) return LBCA_ERR_UNSUPPORTED;
  }
  if (!aligned16(a->q) || !aligned16(a->pooled_k) || !aligned16(a->pooled_v) ||
      !aligned16(a->raw_k) || !aligned16(a->raw_v) || !aligned16(a->out))
    return LBCA_ERR_INVALID_ARG;
  if (a->q_len > 0) {
    // n_pooled(t) and raw_begin(t) never decrease with t: the extreme queries bound all.
    int64_t np_last, rb_first, np0, rb_last;
    lbca_visible_range(a->q_pos0 + a->q_len - 1, a->block, a->window, a->mode, &np_last, &rb_last);
    lbca_visible_range(a->q_pos0, a->block, a->window, a->mode, &np0, &rb_first);
    if (np_last > a->entries) return LBCA_ERR_INVALID_ARG;
    if (rb_first - a->raw_pos_base < 0) return LBCA_ERR_INVALID_ARG;
    if (a->q_pos0 + a->q_len - 1 - a->raw_pos_base >= a->raw_rows) return LBCA_ERR_INVALID_ARG;
  }
  if (a->batch == 0 || a->q_len == 0) return LBCA_OK;
  return hip_status(lbca::launch_prefill(*a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
static int validate_prefill_grad(const lbca_prefill_grad_args* a) {
  if (!a || !a->q || !a->pooled_k || !a->raw_k || !a->out || !a->lse || !a->grad_out || !a->grad_q ||
      !a->grad_pooled_k || !a->grad_raw_k)
    return LBCA_ERR_INVALID_ARG;
  const bool shared = a->pooled_v == nullptr;
  if ((a->raw_v == nullptr) != shared || (a->grad_pooled_v == nullptr) != shared ||
      (a->grad_raw_v == nullptr) != shared)
    return LBCA_ERR_INVALID_ARG;
  if (a->grad_sink && !a->sink) return LBCA_ERR_INVALID_ARG;
  if (!is_dtype(a->dtype) || !is_dtype(a->out_dtype)) return LBCA_ERR_INVALID_ARG;
  if (a->accumulate != 0 && a->accumulate != 1) return LBCA_ERR_INVALID_ARG;
  if (a->batch < 0 || a->q_len < 0 || a->q_heads < 1 || a->kv_heads < 1 || a->q_heads % a->kv_heads != 0)
    return LBCA_ERR_INVALID_ARG;
  if (a->dim < 1 || a->entries < 0 || a->raw_rows < 1 || a->block < 1 || a->window < 1 || a->q_pos0 < 0 ||
      a->raw_pos_base < 0)
    return LBCA_ERR_INVALID_ARG;
  if (a->mode != LBCA_EXCLUSIVE && a->mode != LBCA_OVERLAP) return LBCA_ERR_INVALID_ARG;
  if (!isfinite(a->scale)) return LBCA_ERR_INVALID_ARG;
  if (!sane_product({a->batch, a->q_len, a->q_heads, a->dim}) ||
      !sane_product({a->batch, a->kv_heads, a->entries, a->dim}) ||
      !sane_product({a->batch, a->kv_heads, a->raw_rows, a->dim}) || a->q_pos0 > kMaxElems ||
      a->raw_pos_base > kMaxElems)
    return LBCA_ERR_INVALID_ARG;
  if (a->dtype != LBCA_BF16 || !(a->dim == 64 || a->dim == 128) || !(a->scale > 0.f)) return LBCA_ERR_UNSUPPORTED;
  const int64_t lim = int64_t(1) << 31;
  if (a->batch * a->q_len * a->q_heads >= lim || a->q_pos0 + a->q_len >= lim ||
      a->raw_pos_base + a->raw_rows + a->block + a->window >= lim || a->batch * a->kv_heads > 65535)
    return LBCA_ERR_UNSUPPORTED;
  if (!aligned16(a->q) || !aligned16(a->pooled_k) || !aligned16(a->pooled_v) || !aligned16(a->raw_k) ||
      !aligned16(a->raw_v) || !aligned16(a->out) || !aligned16(a->grad_out) || !aligned16(a->grad_q) ||
      !aligned16(a->grad_pooled_k) || !aligned16(a->grad_pooled_v) || !aligned16(a->grad_raw_k) ||
      !aligned16(a->grad_raw_v))
    return LBCA_ERR_INVALID_ARG;
  if (a->q_len > 0) {
    int64_t np_last, rb_first, np0, rb_last;
    lbca_visible_range(a->q_pos0 + a->q_len - 1, a->block, a->window, a->mode, &np_last, &rb_last);
    lbca_visible_range(a->q_pos0, a->block, a->window, a->mode, &np0, &rb_first);
    if (np_last > a->entries) return LBCA_ERR_INVALID_ARG;
    if (rb_first - a->raw_pos_base < 0) return LBCA_ERR_INVALID_ARG;
    if (a->q_pos0 + a->q_len - 1 - a->raw_pos_base >= a->raw_rows) return LBCA_ERR_INVALID_ARG;
  }
  return LBCA_OK;
}

int lbca_attend_prefill_backward_workspace(const lbca_prefill_grad_args* a, size_t* bytes) {
  if (!bytes) return LBCA_ERR_INVALID_ARG;
  const int st = validate_prefill_grad(a);
  if (st != LBCA_OK) return st;
  *bytes = lbca::prefill_grad_workspace_bytes(*a);
  return LBCA_OK;
}

int lbca_attend_prefill_backward(const lbca_prefill_grad_args* a, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  const int st = validate_prefill_grad(a);
  if (st != LBCA_OK) return st;
  const size_t need = lbca::prefill_grad_workspace_bytes(*a);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return LBCA_ERR_WORKSPACE;
  // q_len == 0 without accumulate still zeroes the key, value and sink gradients
  if (a->batch == 0 || (a->q_len == 0 && a->accumulate)) return LBCA_OK;
  return hip_status(lbca::launch_prefill_grad(*a, workspace, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
static int validate_index(const csa_index_args* a) {
  if (!a || !a->q_idx || !a->head_w || !a->keys || !a->pos || !a->out_idx) return LBCA_ERR_INVALID_ARG;
  if (!is_dtype(a->dtype)) return LBCA_ERR_INVALID_ARG;
  if (a->dtype != LBCA_BF16) return LBCA_ERR_UNSUPPORTED;
  if (a->batch < 0 || a->heads < 1 || a->entries < 0 || a->block < 1 || a->k < 1)
    return LBCA_ERR_INVALID_ARG;
  if (!(a->dim == 32 || a->dim == 64 || a->dim == 128)) return a->dim > 0 ? LBCA_ERR_UNSUPPORTED : LBCA_ERR_INVALID_ARG;
  if (a->heads > 16 || a->k > 2048 || a->entries > 65536) return LBCA_ERR_UNSUPPORTED;
  if (!sane_product({a->batch, a->entries, a->dim})) return LBCA_ERR_INVALID_ARG;
  if (!aligned16(a->q_idx) || !aligned16(a->keys) || !aligned16(a->head_w) ||
      !aligned16(a->out_idx) || !aligned16(a->out_score))
    return LBCA_ERR_INVALID_ARG;
  return LBCA_OK;
}

int csa_index_topk_workspace(const csa_index_args* a, size_t* bytes) {
  if (!bytes) return LBCA_ERR_INVALID_ARG;
  int st = validate_index(a);
  if (st != LBCA_OK) return st;
  *bytes = lbca::index_workspace_bytes(*a);
  return LBCA_OK;
}

// ---------------------------------------------------------------------------
namespace {

int validate_csa_prefill(const csa_prefill_args* a) {
  if (!a || !a->q_idx || !a->head_w || !a->idx_keys || !a->q || !a->entries || !a->raw || !a->out)
    return LBCA_ERR_INVALID_ARG;
  if (!is_dtype(a->dtype)) return LBCA_ERR_INVALID_ARG;
  if (a->dtype != LBCA_BF16) return LBCA_ERR_UNSUPPORTED;
  if (a->batch < 0 || a->q_len < 0 || a->idx_heads < 1 || a->idx_dim < 1 || a->q_heads < 1 || a->dim < 1 ||
      a->n_entries < 0 || a->raw_rows < 1 || a->k < 1 || a->q_pos0 < 0 || a->block < 1 || a->window < 1)
    return LBCA_ERR_INVALID_ARG;
  if (!isfinite(a->scale)) return LBCA_ERR_INVALID_ARG;
  if (!sane_product({a->batch, a->q_len, a->q_heads, a->dim}) ||
      !sane_product({a->batch, a->q_len, a->idx_heads, a->idx_dim}) ||
      !sane_product({a->batch, a->n_entries, a->dim}) || !sane_product({a->batch, a->raw_rows, a->dim}) ||
      !sane_product({a->batch, a->q_len, a->n_entries}) || !sane_product({a->batch, a->q_len, a->k}) ||
      a->q_pos0 > kMaxElems || a->raw_pos_base < -kMaxElems || a->raw_pos_base > kMaxElems)
    return LBCA_ERR_INVALID_ARG;
  const int st = check_treatment(a->rmsnorm_eps, a->rope_dims, a->rope_base, a->dim);
  if (st != LBCA_OK) return st;
  if (!(a->idx_dim == 32 || a->idx_dim == 64 || a->idx_dim == 128) || a->idx_heads > 16 || a->k > 2048 ||
      a->n_entries > 65536)
    return LBCA_ERR_UNSUPPORTED;
  if (a->dim != 512 || a->q_heads % 32 != 0 || a->q_heads > 64 || a->batch * a->q_len > 65535 ||
      a->n_entries * a->dim >= (int64_t(1) << 30) || a->raw_rows * a->dim >= (int64_t(1) << 30))
    return LBCA_ERR_UNSUPPORTED;
  if (!aligned16(a->q_idx) || !aligned16(a->head_w) || !aligned16(a->idx_keys) || !aligned16(a->q) ||
      !aligned16(a->entries) || !aligned16(a->raw) || !aligned16(a->out) || !aligned16(a->out_idx))
    return LBCA_ERR_INVALID_ARG;
  if (a->q_len > 0) {
    const int64_t t_last = a->q_pos0 + a->q_len - 1;
    if ((t_last + 1) / a->block > a->n_entries) return LBCA_ERR_INVALID_ARG;
    const int64_t lo = a->q_pos0 - a->window + 1 > 0 ? a->q_pos0 - a->window + 1 : 0;
    if (lo < a->raw_pos_base || t_last - a->raw_pos_base >= a->raw_rows) return LBCA_ERR_INVALID_ARG;
  }
  return LBCA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The two calls a chunk runs (selection over rows = batch * q_len queries, then
// the selected-entry attention over the same rows) and their workspace layout:
// positions, raw bases, selections, index workspace, decode workspace.
struct CsaPrefillPlan {
  csa_index_args ia;
  lbca_decode_args da;
  lbca::DecodePlan dp;
  size_t off_rpb, off_idx, off_index, off_decode, total;
};

CsaPrefillPlan plan_csa_prefill(const csa_prefill_args* a) {
  CsaPrefillPlan pl{};
  const int64_t rows = a->batch * a->q_len;
  pl.ia.q_idx = a->q_idx; pl.ia.head_w = a->head_w; pl.ia.keys = a->idx_keys;
  pl.ia.out_idx = a->out_idx; pl.ia.out_score = nullptr;
  pl.ia.batch = rows; pl.ia.heads = a->idx_heads; pl.ia.dim = a->idx_dim; pl.ia.entries = a->n_entries;
  pl.ia.k = a->k; pl.ia.block = a->block; pl.ia.dtype = a->dtype;
  pl.da.q = a->q; pl.da.pooled_k = a->entries; pl.da.raw_k = a->raw; pl.da.sink = a->sink;
  pl.da.out = a->out; pl.da.lse = a->lse;
  pl.da.batch = rows; pl.da.q_heads = a->q_heads; pl.da.kv_heads = 1; pl.da.dim = a->dim;
  pl.da.entries = a->n_entries; pl.da.raw_rows = a->raw_rows; pl.da.k_sel = a->k;
  pl.da.block = a->block; pl.da.window = a->window; pl.da.mode = LBCA_OVERLAP; pl.da.dtype = a->dtype;
  pl.da.scale = a->scale; pl.da.rmsnorm_eps = a->rmsnorm_eps; pl.da.rope_dims = a->rope_dims;
  pl.da.rope_base = a->rope_base;
  pl.da.sel_idx = reinterpret_cast<const int32_t*>(1);  // planned as a selection; set at launch
  if (rows > 0) pl.dp = lbca::plan_decode(pl.da);  // (its split sizing divides by the rows)
  const size_t r = (size_t)rows;
  pl.off_rpb = align256(r * sizeof(int64_t));
  pl.off_idx = pl.off_rpb + align256(r * sizeof(int64_t));
  pl.off_index = pl.off_idx + (a->out_idx ? 0 : align256(r * (size_t)a->k * sizeof(int32_t)));
  pl.off_decode = pl.off_index + align256(lbca::index_workspace_bytes(pl.ia));
  pl.total = pl.off_decode + pl.dp.ws_bytes;
  return pl;
}

}  // namespace

int csa_sparse_prefill_workspace(const csa_prefill_args* a, size_t* bytes) {
  if (!bytes) return LBCA_ERR_INVALID_ARG;
  const int st = validate_csa_prefill(a);
  if (st != LBCA_OK) return st;
  const CsaPrefillPlan pl = plan_csa_prefill(a);
  if (pl.dp.unsupported) return LBCA_ERR_UNSUPPORTED;  // selected ids beyond what the splits can stage
  *bytes = pl.total;
  return LBCA_OK;
}

int csa_sparse_prefill(const csa_prefill_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = validate_csa_prefill(a);
  if (st != LBCA_OK) return st;
  CsaPrefillPlan pl = plan_csa_prefill(a);
  if (pl.dp.unsupported) return LBCA_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < pl.total || !aligned16(workspace)) return LBCA_ERR_WORKSPACE;
  if (a->batch * a->q_len == 0) return LBCA_OK;
  char* ws = static_cast<char*>(workspace);
  int64_t* pos = reinterpret_cast<int64_t*>(ws);
  int64_t* rpb = reinterpret_cast<int64_t*>(ws + pl.off_rpb);
  int32_t* idx = a->out_idx ? a->out_idx : reinterpret_cast<int32_t*>(ws + pl.off_idx);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  pl.ia.pos = pos;
  pl.ia.out_idx = idx;
  hipError_t e = lbca::launch_index_topk_chunk(pl.ia, a->q_len, a->q_pos0, a->raw_pos_base, pos, rpb,
                                               ws + pl.off_index, s);
  if (e != hipSuccess) return LBCA_ERR_HIP;
  pl.da.pos = pos;
  pl.da.raw_pos_base = rpb;
  pl.da.sel_idx = idx;
  return hip_status(lbca::launch_decode(pl.da, pl.dp, ws + pl.off_decode, s, (int)a->q_len));
}

int lbca_grouped_gemm(const lbca_gemm_args* a, void* stream) {
  if (!a || !a->a || !a->w || !a->c) return LBCA_ERR_INVALID_ARG;
  if (!is_dtype(a->a_dtype) || !is_dtype(a->c_dtype)) return LBCA_ERR_INVALID_ARG;
  if (a->groups < 0 || a->m < 0 || a->n < 0 || a->k < 1) return LBCA_ERR_INVALID_ARG;
  if (a->lda < a->k || a->ldw < a->k || a->ldc < a->n || a->a_group_stride < 0 || a->w_group_stride < 0 ||
      a->c_group_stride < 0)
    return LBCA_ERR_INVALID_ARG;
  if (!aligned16(a->a) || !aligned16(a->w) || !aligned16(a->c)) return LBCA_ERR_INVALID_ARG;
  if (!sane_product({a->groups, a->m, a->lda}) || !sane_product({a->groups, a->n, a->ldw}) ||
      !sane_product({a->groups, a->m, a->ldc}) || a->a_group_stride > kMaxElems || a->w_group_stride > kMaxElems ||
      a->c_group_stride > kMaxElems)
    return LBCA_ERR_INVALID_ARG;
  if (a->k % 8 || a->lda % 8 || a->ldw % 8 || a->a_group_stride % 8 || a->w_group_stride % 8)
    return LBCA_ERR_UNSUPPORTED;
  const int64_t ka = a->a_dtype == LBCA_F32 ? 4 : 2;
  // 128-row bands are addressed with 32-bit byte offsets; the grid's y and z
  // carry row tiles and groups
  if ((127 * a->lda + a->k) * ka >= (int64_t(1) << 31) || (127 * a->ldw + a->k) * 2 >= (int64_t(1) << 31) ||
      a->groups > 65535 || (a->m + 127) / 128 > 65535 || (a->n + 127) / 128 > INT32_MAX)
    return LBCA_ERR_UNSUPPORTED;
  if (a->groups == 0 || a->m == 0 || a->n == 0) return LBCA_OK;
  return hip_status(lbca::launch_gemm(*a, static_cast<hipStream_t>(stream)));
}

int csa_index_topk(const csa_index_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate_index(a);
  if (st != LBCA_OK) return st;
  const size_t need = lbca::index_workspace_bytes(*a);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return LBCA_ERR_WORKSPACE;
  if (a->batch == 0) return LBCA_OK;
  return hip_status(lbca::launch_index_topk(*a, workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
