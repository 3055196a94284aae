// Decode-time cache step: append each sequence's newest token to a mirrored
// raw ring and pool the block that becomes visible at that token.
//
// Method: "mSeek: learned KV-cache compression in a 3B model", section "How LBCA
// works" (steps 1-3: new tokens join the raw cache; a block that is complete
// and has left the W-token window becomes one pooled entry); "HCA: Heavily
// Compressed Attention (toy implementation)", "What is implemented" (every
// complete block is an entry, with RMSNorm and partial RoPE at its start).
//
// Design: one 256-thread workgroup per (sequence, head) row.  The first L =
// dim/8 lanes copy the new token's key, value and logit rows (16-byte
// vectors) into both rows of its ring slot.  On the step that makes a block
// visible, the whole workgroup pools it: its m tokens sit in m consecutive
// ring rows (the mirror keeps any run of at most `ring` positions
// contiguous), the 256 / L lane groups take token phases, and the phases are
// merged and the entry finished exactly as in the pooling kernels (shared
// code), so an entry written here is bitwise the one lbca_pool_blocks writes.
// Under the OVERLAP rule the due block ends with the new token, which the
// workgroup's barrier after the copy makes visible to every lane.  In dual
// (CSA) mode a second ring holds the b-series and the entry's softmax also
// folds block j-1 of it ("CSA: Compressed Sparse Attention (toy
// implementation)", "What is implemented", dual overlapped pooling).
#include "cache_common.h"

namespace lbca {

template <typename TX, typename TZ, bool HAS_V, bool TREAT, bool DUAL, bool DN>
__global__ __launch_bounds__(256) void cache_append_kernel(CacheParams p) {
  __shared__ float part[32][256];  // cross-wave phase merge
  // every argument field in one batch of scalar loads (otherwise they come in
  // dependent rounds, one per basic block)
  asm volatile("" ::"s"(p.x_new), "s"(p.v_new), "s"(p.z_new), "s"(p.raw_x), "s"(p.raw_v), "s"(p.raw_z), "s"(p.xb_new),
               "s"(p.zb_new), "s"(p.raw_xb), "s"(p.raw_zb),
               "s"(p.pos), "s"(p.raw_pos_base), "s"(p.heads), "s"(p.dim), "s"(p.m), "s"(p.W), "s"(p.ring),
               "s"(p.entries), "s"(p.mode), "s"(p.lanes_per_row), "s"(p.log2_lanes));
  // row = sequence * heads + head (the host keeps it below 2^31)
  cache_row<TX, TZ, HAS_V, TREAT, DUAL, false, true, true, DN>(p, blockIdx.x, part, true);
}

template <typename TX, typename TZ, bool DN>
static hipError_t launch_cache_d(const CacheParams& p, bool has_v, bool treat, bool dual, dim3 grid, hipStream_t s) {
  if (has_v) cache_append_kernel<TX, TZ, true, false, false, DN><<<grid, 256, 0, s>>>(p);
  else if (dual && treat) cache_append_kernel<TX, TZ, false, true, true, DN><<<grid, 256, 0, s>>>(p);
  else if (dual) cache_append_kernel<TX, TZ, false, false, true, DN><<<grid, 256, 0, s>>>(p);
  else if (treat) cache_append_kernel<TX, TZ, false, true, false, DN><<<grid, 256, 0, s>>>(p);
  else cache_append_kernel<TX, TZ, false, false, false, DN><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

template <typename TX, typename TZ>
static hipError_t launch_cache_typed(const CacheParams& p, bool has_v, bool treat, bool dual, dim3 grid, bool dn,
                                     hipStream_t s) {
  return dn ? launch_cache_d<TX, TZ, true>(p, has_v, treat, dual, grid, s)
            : launch_cache_d<TX, TZ, false>(p, has_v, treat, dual, grid, s);
}

hipError_t launch_cache_append(const lbca_cache_args& a, hipStream_t stream) {
  CacheParams p;
  p.x_new = a.x_new; p.v_new = a.v_new; p.z_new = a.z_new;
  p.raw_x = a.raw_x; p.raw_v = a.raw_v; p.raw_z = a.raw_z;
  p.bias = a.bias; p.out_x = a.out_x; p.out_v = a.out_v;
  p.pos = a.pos; p.raw_pos_base = a.raw_pos_base;
  p.xb_new = a.xb_new; p.zb_new = a.zb_new; p.raw_xb = a.raw_xb; p.raw_zb = a.raw_zb; p.bias_b = a.bias_b;
  p.heads = a.heads; p.dim = a.dim; p.m = a.block; p.W = a.window; p.ring = a.ring; p.entries = a.entries;
  p.mode = a.mode;
  p.lanes_per_row = (int)(a.dim / 8);
  p.log2_lanes = __builtin_ctz((unsigned)p.lanes_per_row);
  p.eps = a.rmsnorm_eps;
  p.rope_dims = a.rope_dims;
  p.log2_base = a.rope_dims > 0 ? log2((double)a.rope_base) : 0.0;
  set_cache_strides(p, a);
  const dim3 grid((unsigned)(a.batch * a.heads));
  const bool has_v = a.v_new != nullptr;
  const bool treat = a.rmsnorm_eps >= 0.f || a.rope_dims > 0;
  const bool dual = a.xb_new != nullptr;
  const int64_t B = a.batch, H = a.heads, R = 2 * a.ring, N = a.entries, d = a.dim;
  const bool dn =
      dense_strides(a.x_new, a.x_new_st, {B, H}, d) && dense_strides(a.v_new, a.v_new_st, {B, H}, d) &&
      dense_strides(a.z_new, a.z_new_st, {B, H}, d) && dense_strides(a.xb_new, a.xb_new_st, {B, H}, d) &&
      dense_strides(a.zb_new, a.zb_new_st, {B, H}, d) && dense_strides(a.raw_x, a.raw_x_st, {B, H, R}, d) &&
      dense_strides(a.raw_v, a.raw_v_st, {B, H, R}, d) && dense_strides(a.raw_z, a.raw_z_st, {B, H, R}, d) &&
      dense_strides(a.raw_xb, a.raw_xb_st, {B, H, R}, d) && dense_strides(a.raw_zb, a.raw_zb_st, {B, H, R}, d) &&
      dense_strides(a.out_x, a.out_x_st, {B, H, N}, d) && dense_strides(a.out_v, a.out_v_st, {B, H, N}, d);
  if (a.x_dtype == LBCA_BF16) {
    if (a.z_dtype == LBCA_BF16) return launch_cache_typed<bf16_t, bf16_t>(p, has_v, treat, dual, grid, dn, stream);
    return launch_cache_typed<bf16_t, float>(p, has_v, treat, dual, grid, dn, stream);
  }
  if (a.z_dtype == LBCA_BF16) return launch_cache_typed<float, bf16_t>(p, has_v, treat, dual, grid, dn, stream);
  return launch_cache_typed<float, float>(p, has_v, treat, dual, grid, dn, stream);
}

}  // namespace lbca
