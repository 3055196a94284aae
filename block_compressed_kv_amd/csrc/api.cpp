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

int64_t esize(int32_t dtype) { return dtype == LBCA_F32 ? 4 : 2; }

// One tensor argument's strides: with all used strides zero, fills in the
// dense row-major ones for outer extents ext (outermost first) and feature dim
// d; then checks the rules of lbca_strides (non-negative, rows 16-byte
// aligned, every element within kMaxElems of the base and, for an output, no
// two elements at one address).  An absent tensor (ptr NULL) is not checked.
int fix_strides(lbca_strides& st, const void* ptr, std::initializer_list<int64_t> ext, int64_t d, int32_t dtype,
                bool output) {
  const int n = (int)ext.size();
  const int64_t* e = ext.begin();
  bool zero = true;
  for (int i = 0; i < n; ++i) zero = zero && st.s[i] == 0;
  if (zero) {
    int64_t s = d;
    for (int i = n - 1; i >= 0; --i) {
      st.s[i] = s;
      if (e[i] > 1) s = s <= kMaxElems / e[i] ? s * e[i] : kMaxElems + 1;
    }
  }
  for (int i = n; i < 3; ++i) st.s[i] = 0;
  if (!ptr) return LBCA_OK;
  for (int i = 1; i < n; ++i)
    if (st.s[i] >= (int64_t(1) << 31)) return LBCA_ERR_UNSUPPORTED;  // the kernels hold inner strides in 32 bits
  bool empty = d == 0;
  for (int i = 0; i < n; ++i) {
    if (st.s[i] < 0 || st.s[i] > kMaxElems || (st.s[i] * esize(dtype)) % 16 != 0) return LBCA_ERR_INVALID_ARG;
    empty = empty || e[i] == 0;
  }
  if (empty) return LBCA_OK;
  int64_t far = d;  // one past the furthest element
  for (int i = 0; i < n; ++i) {
    if (e[i] > 1 && st.s[i] > (kMaxElems - far) / (e[i] - 1)) return LBCA_ERR_INVALID_ARG;
    far += (e[i] - 1) * st.s[i];
  }
  if (output) {  // dimensions of extent > 1 in stride order, each past everything inside it
    int idx[3], k = 0;
    for (int i = 0; i < n; ++i)
      if (e[i] > 1) idx[k++] = i;
    for (int i = 1; i < k; ++i)
      for (int j = i; j > 0 && st.s[idx[j]] < st.s[idx[j - 1]]; --j) {
        const int t = idx[j];
        idx[j] = idx[j - 1];
        idx[j - 1] = t;
      }
    int64_t cover = d;
    for (int j = 0; j < k; ++j) {
      if (st.s[idx[j]] < cover) return LBCA_ERR_INVALID_ARG;
      cover += (e[idx[j]] - 1) * st.s[idx[j]];
    }
  }
  return LBCA_OK;
}

// Elements spanned by `rows` rows of row stride sr (one sequence and head's slice).
int64_t slice_span(int64_t rows, int64_t sr, int64_t d) { return rows > 0 ? (rows - 1) * sr + d : 0; }

#define LBCA_TRY(x)                 \
  do {                              \
    const int st_ = (x);            \
    if (st_ != LBCA_OK) return st_; \
  } while (0)

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
static int strides_pool(lbca_pool_args* a) {
  const int64_t B = a->batch, H = a->heads, T = a->tokens, N = a->entries, d = a->dim;
  LBCA_TRY(fix_strides(a->x_st, a->x, {B, H, T}, d, a->x_dtype, false));
  LBCA_TRY(fix_strides(a->v_st, a->v, {B, H, T}, d, a->x_dtype, false));
  LBCA_TRY(fix_strides(a->z_st, a->z, {B, H, T}, d, a->z_dtype, false));
  LBCA_TRY(fix_strides(a->xb_st, a->xb, {B, H, T}, d, a->x_dtype, false));
  LBCA_TRY(fix_strides(a->zb_st, a->zb, {B, H, T}, d, a->z_dtype, false));
  LBCA_TRY(fix_strides(a->out_x_st, a->out_x, {B, H, N}, d, a->x_dtype, true));
  LBCA_TRY(fix_strides(a->out_v_st, a->out_v, {B, H, N}, d, a->x_dtype, true));
  return LBCA_OK;
}

int lbca_pool_blocks(const lbca_pool_args* ap, void* stream) {
  if (!ap) return LBCA_ERR_INVALID_ARG;
  lbca_pool_args args = *ap;
  lbca_pool_args* a = &args;
  if (!a->x || !a->z || !a->bias || !a->out_x) return LBCA_ERR_INVALID_ARG;
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
  LBCA_TRY(strides_pool(a));
  if (a->batch == 0 || a->block_end == a->block_begin) return LBCA_OK;
  return hip_status(lbca::launch_pool(*a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
static int strides_pool_grad(lbca_pool_grad_args* a) {
  const int64_t B = a->batch, H = a->heads, T = a->tokens, N = a->entries, d = a->dim;
  const int32_t xt = a->x_dtype, zt = a->z_dtype;
  LBCA_TRY(fix_strides(a->x_st, a->x, {B, H, T}, d, xt, false));
  LBCA_TRY(fix_strides(a->v_st, a->v, {B, H, T}, d, xt, false));
  LBCA_TRY(fix_strides(a->z_st, a->z, {B, H, T}, d, zt, false));
  LBCA_TRY(fix_strides(a->xb_st, a->xb, {B, H, T}, d, xt, false));
  LBCA_TRY(fix_strides(a->zb_st, a->zb, {B, H, T}, d, zt, false));
  LBCA_TRY(fix_strides(a->grad_x_st, a->grad_x, {B, H, N}, d, xt, false));
  LBCA_TRY(fix_strides(a->grad_v_st, a->grad_v, {B, H, N}, d, xt, false));
  LBCA_TRY(fix_strides(a->dx_st, a->dx, {B, H, T}, d, xt, true));
  LBCA_TRY(fix_strides(a->dv_st, a->dv, {B, H, T}, d, xt, true));
  LBCA_TRY(fix_strides(a->dz_st, a->dz, {B, H, T}, d, zt, true));
  LBCA_TRY(fix_strides(a->dxb_st, a->dxb, {B, H, T}, d, xt, true));
  LBCA_TRY(fix_strides(a->dzb_st, a->dzb, {B, H, T}, d, zt, true));
  return LBCA_OK;
}

static int validate_pool_grad(lbca_pool_grad_args* a) {
  if (!a->x || !a->z || !a->bias || !a->grad_x || !a->dx || !a->dz || !a->dbias)
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
  return strides_pool_grad(a);
}

int lbca_pool_blocks_backward_workspace(const lbca_pool_grad_args* ap, size_t* bytes) {
  if (!bytes || !ap) return LBCA_ERR_INVALID_ARG;
  lbca_pool_grad_args args = *ap;
  lbca_pool_grad_args* a = &args;
  const int st = validate_pool_grad(a);
  if (st != LBCA_OK) return st;
  *bytes = lbca::pool_grad_workspace_bytes(*a);
  return LBCA_OK;
}

int lbca_pool_blocks_backward(const lbca_pool_grad_args* ap, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!ap) return LBCA_ERR_INVALID_ARG;
  lbca_pool_grad_args args = *ap;
  lbca_pool_grad_args* a = &args;
  const int st = validate_pool_grad(a);
  if (st != LBCA_OK) return st;
  const size_t need = lbca::pool_grad_workspace_bytes(*a);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return LBCA_ERR_WORKSPACE;
  return hip_status(lbca::launch_pool_grad(*a, workspace, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
static int strides_cache(lbca_cache_args* a) {
  const int64_t B = a->batch, H = a->heads, R = 2 * a->ring, N = a->entries, d = a->dim;
  const int32_t xt = a->x_dtype, zt = a->z_dtype;
  LBCA_TRY(fix_strides(a->x_new_st, a->x_new, {B, H}, d, xt, false));
  LBCA_TRY(fix_strides(a->v_new_st, a->v_new, {B, H}, d, xt, false));
  LBCA_TRY(fix_strides(a->z_new_st, a->z_new, {B, H}, d, zt, false));
  LBCA_TRY(fix_strides(a->xb_new_st, a->xb_new, {B, H}, d, xt, false));
  LBCA_TRY(fix_strides(a->zb_new_st, a->zb_new, {B, H}, d, zt, false));
  LBCA_TRY(fix_strides(a->raw_x_st, a->raw_x, {B, H, R}, d, xt, true));
  LBCA_TRY(fix_strides(a->raw_v_st, a->raw_v, {B, H, R}, d, xt, true));
  LBCA_TRY(fix_strides(a->raw_z_st, a->raw_z, {B, H, R}, d, zt, true));
  LBCA_TRY(fix_strides(a->raw_xb_st, a->raw_xb, {B, H, R}, d, xt, true));
  LBCA_TRY(fix_strides(a->raw_zb_st, a->raw_zb, {B, H, R}, d, zt, true));
  LBCA_TRY(fix_strides(a->out_x_st, a->out_x, {B, H, N}, d, xt, true));
  LBCA_TRY(fix_strides(a->out_v_st, a->out_v, {B, H, N}, d, xt, true));
  return LBCA_OK;
}

static int validate_cache(lbca_cache_args* a) {
  if (!a->x_new || !a->z_new || !a->raw_x || !a->raw_z || !a->bias || !a->out_x || !a->pos ||
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
  return strides_cache(a);
}

int lbca_cache_append(const lbca_cache_args* ap, void* stream) {
  if (!ap) return LBCA_ERR_INVALID_ARG;
  lbca_cache_args args = *ap;
  lbca_cache_args* a = &args;
  const int st = validate_cache(a);
  if (st != LBCA_OK) return st;
  if (a->batch == 0) return LBCA_OK;
  return hip_status(lbca::launch_cache_append(*a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
static int strides_decode(lbca_decode_args* a) {
  const int64_t B = a->batch, Hq = a->q_heads, Hk = a->kv_heads, d = a->dim;
  const int32_t dt = a->dtype;
  LBCA_TRY(fix_strides(a->q_st, a->q, {B, Hq}, d, dt, false));
  LBCA_TRY(fix_strides(a->pooled_k_st, a->pooled_k, {B, Hk, a->entries}, d, dt, false));
  LBCA_TRY(fix_strides(a->pooled_v_st, a->pooled_v, {B, Hk, a->entries}, d, dt, false));
  LBCA_TRY(fix_strides(a->raw_k_st, a->raw_k, {B, Hk, a->raw_rows}, d, dt, false));
  LBCA_TRY(fix_strides(a->raw_v_st, a->raw_v, {B, Hk, a->raw_rows}, d, dt, false));
  LBCA_TRY(fix_strides(a->out_st, a->out, {B, Hq}, d, LBCA_F32, true));
  if (dt == LBCA_BF16) {
    // rows are addressed by 32-bit byte offsets within one (sequence, KV head) slice
    const int64_t lim = int64_t(1) << 30;
    if (slice_span(a->entries, a->pooled_k_st.s[2], d) >= lim ||
        slice_span(a->entries, a->pooled_v_st.s[2], d) >= lim ||
        slice_span(a->raw_rows, a->raw_k_st.s[2], d) >= lim || slice_span(a->raw_rows, a->raw_v_st.s[2], d) >= lim)
      return LBCA_ERR_UNSUPPORTED;
  }
  return LBCA_OK;
}

static int validate_decode(lbca_decode_args* a) {
  if (!a->q || !a->pooled_k || !a->raw_k || !a->pos || !a->out) return LBCA_ERR_INVALID_ARG;
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
    if (a->k_sel > 32768 || a->batch > 65535 || a->kv_heads * ((G + 15) / 16) > 65535)
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
  return strides_decode(a);
}

int lbca_attend_decode_workspace(const lbca_decode_args* ap, size_t* bytes) {
  if (!bytes || !ap) return LBCA_ERR_INVALID_ARG;
  lbca_decode_args args = *ap;
  lbca_decode_args* a = &args;
  int st = validate_decode(a);
  if (st != LBCA_OK) return st;
  *bytes = lbca::plan_decode(*a).ws_bytes;
  return LBCA_OK;
}

int lbca_attend_decode(const lbca_decode_args* ap, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!ap) return LBCA_ERR_INVALID_ARG;
  lbca_decode_args args = *ap;
  lbca_decode_args* a = &args;
  int st = validate_decode(a);
  if (st != LBCA_OK) return st;
  const lbca::DecodePlan plan = lbca::plan_decode(*a);
  if (plan.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.ws_bytes || !aligned16(workspace)))
    return LBCA_ERR_WORKSPACE;
  if (a->batch == 0) return LBCA_OK;
  return hip_status(lbca::launch_decode(*a, plan, workspace, static_cast<hipStream_t>(stream)));
}

int lbca_attend_decode_noalloc(const lbca_decode_args* ap, void* stream) {
  if (!ap) return LBCA_ERR_INVALID_ARG;
  lbca_decode_args args = *ap;
  lbca_decode_args* a = &args;
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
  d->q_st = a->q_st; d->pooled_k_st = a->pooled_k_st; d->pooled_v_st = a->pooled_v_st;
  d->raw_k_st = a->raw_k_st; d->raw_v_st = a->raw_v_st; d->out_st = a->out_st;
  *c = lbca_cache_args{};
  c->x_new = a->k_new; c->v_new = a->v_new; c->z_new = a->z_new;
  c->raw_x = a->raw_k; c->raw_v = a->raw_v; c->raw_z = a->raw_z; c->bias = a->bias;
  c->out_x = a->pooled_k; c->out_v = a->pooled_v; c->pos = a->pos; c->raw_pos_base = a->raw_pos_base;
  c->batch = a->batch; c->heads = a->kv_heads; c->dim = a->dim; c->block = a->block; c->window = a->window;
  c->ring = a->ring; c->entries = a->entries; c->mode = LBCA_EXCLUSIVE; c->x_dtype = a->dtype;
  c->z_dtype = a->z_dtype; c->rmsnorm_eps = -1.f; c->rope_dims = 0; c->rope_base = 0.f;
  c->x_new_st = a->k_new_st; c->v_new_st = a->v_new_st; c->z_new_st = a->z_new_st;
  c->raw_x_st = a->raw_k_st; c->raw_v_st = a->raw_v_st; c->raw_z_st = a->raw_z_st;
  c->out_x_st = a->pooled_k_st; c->out_v_st = a->pooled_v_st;
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
static int strides_prefill(lbca_prefill_args* a) {
  const int64_t B = a->batch, Tq = a->q_len, Hq = a->q_heads, Hk = a->kv_heads, d = a->dim;
  const int32_t dt = a->dtype;
  LBCA_TRY(fix_strides(a->q_st, a->q, {B, Tq, Hq}, d, dt, false));
  LBCA_TRY(fix_strides(a->pooled_k_st, a->pooled_k, {B, Hk, a->entries}, d, dt, false));
  LBCA_TRY(fix_strides(a->pooled_v_st, a->pooled_v, {B, Hk, a->entries}, d, dt, false));
  LBCA_TRY(fix_strides(a->raw_k_st, a->raw_k, {B, Hk, a->raw_rows}, d, dt, false));
  LBCA_TRY(fix_strides(a->raw_v_st, a->raw_v, {B, Hk, a->raw_rows}, d, dt, false));
  LBCA_TRY(fix_strides(a->out_st, a->out, {B, Tq, Hq}, d, a->out_dtype, true));
  if (dt == LBCA_BF16) {
    // cache rows are read through buffer resources with 31-bit byte offsets
    auto big = [&](int64_t rows, const lbca_strides& st) {
      return rows * (st.s[2] > d ? st.s[2] : d) * 2 >= (int64_t(1) << 31);
    };
    if (big(a->entries, a->pooled_k_st) || big(a->entries, a->pooled_v_st) || big(a->raw_rows, a->raw_k_st) ||
        big(a->raw_rows, a->raw_v_st))
      return LBCA_ERR_UNSUPPORTED;
  }
  return LBCA_OK;
}

int lbca_attend_prefill(const lbca_prefill_args* ap, void* stream) {
  if (!ap) return LBCA_ERR_INVALID_ARG;
  lbca_prefill_args args = *ap;
  lbca_prefill_args* a = &args;
  if (!a->q || !a->pooled_k || !a->raw_k || !a->out) return LBCA_ERR_INVALID_ARG;
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
  LBCA_TRY(strides_prefill(a));
  if (a->batch == 0 || a->q_len == 0) return LBCA_OK;
  return hip_status(lbca::launch_prefill(*a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
static int strides_prefill_grad(lbca_prefill_grad_args* a) {
  const int64_t B = a->batch, Tq = a->q_len, Hq = a->q_heads, Hk = a->kv_heads, d = a->dim;
  const int64_t N = a->entries, R = a->raw_rows;
  const int32_t dt = a->dtype, f = LBCA_F32;
  LBCA_TRY(fix_strides(a->q_st, a->q, {B, Tq, Hq}, d, dt, false));
  LBCA_TRY(fix_strides(a->grad_out_st, a->grad_out, {B, Tq, Hq}, d, dt, false));
  LBCA_TRY(fix_strides(a->out_st, a->out, {B, Tq, Hq}, d, a->out_dtype, false));
  LBCA_TRY(fix_strides(a->pooled_k_st, a->pooled_k, {B, Hk, N}, d, dt, false));
  LBCA_TRY(fix_strides(a->pooled_v_st, a->pooled_v, {B, Hk, N}, d, dt, false));
  LBCA_TRY(fix_strides(a->raw_k_st, a->raw_k, {B, Hk, R}, d, dt, false));
  LBCA_TRY(fix_strides(a->raw_v_st, a->raw_v, {B, Hk, R}, d, dt, false));
  LBCA_TRY(fix_strides(a->grad_q_st, a->grad_q, {B, Tq, Hq}, d, f, true));
  LBCA_TRY(fix_strides(a->grad_pooled_k_st, a->grad_pooled_k, {B, Hk, N}, d, f, true));
  LBCA_TRY(fix_strides(a->grad_pooled_v_st, a->grad_pooled_v, {B, Hk, N}, d, f, true));
  LBCA_TRY(fix_strides(a->grad_raw_k_st, a->grad_raw_k, {B, Hk, R}, d, f, true));
  LBCA_TRY(fix_strides(a->grad_raw_v_st, a->grad_raw_v, {B, Hk, R}, d, f, true));
  return LBCA_OK;
}

static int validate_prefill_grad(lbca_prefill_grad_args* a) {
  if (!a->q || !a->pooled_k || !a->raw_k || !a->out || !a->lse || !a->grad_out || !a->grad_q ||
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
  return strides_prefill_grad(a);
}

int lbca_attend_prefill_backward_workspace(const lbca_prefill_grad_args* ap, size_t* bytes) {
  if (!bytes || !ap) return LBCA_ERR_INVALID_ARG;
  lbca_prefill_grad_args args = *ap;
  lbca_prefill_grad_args* a = &args;
  const int st = validate_prefill_grad(a);
  if (st != LBCA_OK) return st;
  *bytes = lbca::prefill_grad_workspace_bytes(*a);
  return LBCA_OK;
}

int lbca_attend_prefill_backward(const lbca_prefill_grad_args* ap, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!ap) return LBCA_ERR_INVALID_ARG;
  lbca_prefill_grad_args args = *ap;
  lbca_prefill_grad_args* a = &args;
  const int st = validate_prefill_grad(a);
  if (st != LBCA_OK) return st;
  const size_t need = lbca::prefill_grad_workspace_bytes(*a);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return LBCA_ERR_WORKSPACE;
  // q_len == 0 without accumulate still zeroes the key, value and sink gradients
  if (a->batch == 0 || (a->q_len == 0 && a->accumulate)) return LBCA_OK;
  return hip_status(lbca::launch_prefill_grad(*a, workspace, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
static int validate_index(csa_index_args* a) {
  if (!a->q_idx || !a->head_w || !a->keys || !a->pos || !a->out_idx) return LBCA_ERR_INVALID_ARG;
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
  LBCA_TRY(fix_strides(a->q_idx_st, a->q_idx, {a->batch, a->heads}, a->dim, a->dtype, false));
  LBCA_TRY(fix_strides(a->keys_st, a->keys, {a->batch, a->entries}, a->dim, a->dtype, false));
  return LBCA_OK;
}

int csa_index_topk_workspace(const csa_index_args* ap, size_t* bytes) {
  if (!bytes || !ap) return LBCA_ERR_INVALID_ARG;
  csa_index_args args = *ap;
  csa_index_args* a = &args;
  int st = validate_index(a);
  if (st != LBCA_OK) return st;
  *bytes = lbca::index_workspace_bytes(*a);
  return LBCA_OK;
}

// ---------------------------------------------------------------------------
namespace {

int validate_csa_prefill(csa_prefill_args* a) {
  if (!a->q_idx || !a->head_w || !a->idx_keys || !a->q || !a->entries || !a->raw || !a->out)
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
  if (a->dim != 512 || a->q_heads % 32 != 0 || a->q_heads > 64 || a->batch * a->q_len > 65535)
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
  const int64_t B = a->batch, Tq = a->q_len, N = a->n_entries;
  LBCA_TRY(fix_strides(a->q_idx_st, a->q_idx, {B, Tq, a->idx_heads}, a->idx_dim, a->dtype, false));
  LBCA_TRY(fix_strides(a->idx_keys_st, a->idx_keys, {B, N}, a->idx_dim, a->dtype, false));
  LBCA_TRY(fix_strides(a->q_st, a->q, {B, Tq, a->q_heads}, a->dim, a->dtype, false));
  LBCA_TRY(fix_strides(a->entries_st, a->entries, {B, N}, a->dim, a->dtype, false));
  LBCA_TRY(fix_strides(a->raw_st, a->raw, {B, a->raw_rows}, a->dim, a->dtype, false));
  LBCA_TRY(fix_strides(a->out_st, a->out, {B, Tq, a->q_heads}, a->dim, LBCA_F32, true));
  // rows are addressed by 32-bit byte offsets within one sequence's cache
  const int64_t lim = int64_t(1) << 30;
  if (slice_span(N, a->entries_st.s[1], a->dim) >= lim || slice_span(a->raw_rows, a->raw_st.s[1], a->dim) >= lim)
    return LBCA_ERR_UNSUPPORTED;
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
  // a query chunk's rows: [sequence, query, head] strides (launch_index_topk_chunk)
  pl.ia.q_idx_st = a->q_idx_st;
  pl.ia.keys_st = a->idx_keys_st;
  pl.da.q = a->q; pl.da.pooled_k = a->entries; pl.da.raw_k = a->raw; pl.da.sink = a->sink;
  pl.da.out = a->out; pl.da.lse = a->lse;
  pl.da.batch = rows; pl.da.q_heads = a->q_heads; pl.da.kv_heads = 1; pl.da.dim = a->dim;
  pl.da.entries = a->n_entries; pl.da.raw_rows = a->raw_rows; pl.da.k_sel = a->k;
  pl.da.block = a->block; pl.da.window = a->window; pl.da.mode = LBCA_OVERLAP; pl.da.dtype = a->dtype;
  pl.da.scale = a->scale; pl.da.rmsnorm_eps = a->rmsnorm_eps; pl.da.rope_dims = a->rope_dims;
  pl.da.rope_base = a->rope_base;
  // rows of a query chunk: q and out as [sequence, query, head]; the caches as
  // one KV head per sequence
  pl.da.q_st = a->q_st;
  pl.da.out_st = a->out_st;
  pl.da.pooled_k_st = lbca_strides{{a->entries_st.s[0], 0, a->entries_st.s[1]}};
  pl.da.raw_k_st = lbca_strides{{a->raw_st.s[0], 0, a->raw_st.s[1]}};
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

int csa_sparse_prefill_workspace(const csa_prefill_args* ap, size_t* bytes) {
  if (!bytes || !ap) return LBCA_ERR_INVALID_ARG;
  csa_prefill_args args = *ap;
  csa_prefill_args* a = &args;
  const int st = validate_csa_prefill(a);
  if (st != LBCA_OK) return st;
  const CsaPrefillPlan pl = plan_csa_prefill(a);
  if (pl.dp.unsupported) return LBCA_ERR_UNSUPPORTED;  // selected ids beyond what the splits can stage
  *bytes = pl.total;
  return LBCA_OK;
}

int csa_sparse_prefill(const csa_prefill_args* ap, void* workspace, size_t workspace_bytes, void* stream) {
  if (!ap) return LBCA_ERR_INVALID_ARG;
  csa_prefill_args args = *ap;
  csa_prefill_args* a = &args;
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

int csa_index_topk(const csa_index_args* ap, void* workspace, size_t workspace_bytes, void* stream) {
  if (!ap) return LBCA_ERR_INVALID_ARG;
  csa_index_args args = *ap;
  csa_index_args* a = &args;
  int st = validate_index(a);
  if (st != LBCA_OK) return st;
  const size_t need = lbca::index_workspace_bytes(*a);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return LBCA_ERR_WORKSPACE;
  if (a->batch == 0) return LBCA_OK;
  return hip_status(lbca::launch_index_topk(*a, workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
