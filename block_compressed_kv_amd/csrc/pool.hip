// Block pooling kernels (single series, shared series, dual overlapped series).
//
// Method: "mSeek: learned KV-cache compression in a 3B model", section "How LBCA
// works" (steps 2-3); "HCA: Heavily Compressed Attention (toy implementation)",
// "What is implemented" (single-series pooling with a learnable positional
// bias); "CSA: Compressed Sparse Attention (toy implementation)", "What is
// implemented" (dual overlapped pooling, one joint softmax per channel).
//
// Design: pooling reads every token-channel once (8 B/element for bf16 K+V
// with fp32 logits) and writes 1/m of that, so it is HBM-bound.  A group of
// L = dim/8 lanes covers one token row; each lane owns 8 consecutive channels,
// so every load is a 16-byte vector and a group's loads cover whole 128-byte
// lines.  The softmax over the block is an online softmax in registers,
// advanced four tokens at a time (one rescale exp per four data exps).
// An output row may be split over P token phases (groups that take tokens
// phase, phase+P, ...): with many rows (pooling a whole history) P = 1 and
// every group streams its own block; with few rows (the single block that
// falls out of the window at a decode step) P grows so that every lane has
// one short burst of loads in flight, and the P partial states are merged in
// a fixed tree order, by lane exchanges inside a wave and through LDS across
// waves (a sequential merge by one group costs more than the loads).  The
// optional HCA/CSA entry treatment (RMSNorm, partial
// RoPE at the block start) runs on the finished fp32 row before the single
// rounding to the storage type.
#include "lbca_internal.h"
#include "pool_common.h"

#ifndef LBCA_POOL_MAX_PHASES
#define LBCA_POOL_MAX_PHASES 64  // upper bound on token phases per output row
#endif

namespace lbca {

struct PoolParams {
  const void* x;
  const void* v;
  const void* z;
  const float* bias;
  const void* xb;
  const void* zb;
  const float* bias_b;
  void* out_x;
  void* out_v;
  Str x_st, v_st, z_st, xb_st, zb_st, ox_st, ov_st;  // {sequence, head, row}
  int64_t heads, tokens, dim, m, entries, block_begin, n_blocks, pos_base, total_rows;
  int lanes_per_row;  // L = dim / 8, a power of two <= 64
  int log2_lanes;
  int log2_phases;    // P = token phases per output row
  float eps;          // < 0: no RMSNorm
  int rope_dims;      // 0: no RoPE
  double log2_base;
};

// The strides of a pooling pass: the arguments', or, when every tensor of the
// call is dense (DN), the row-major ones worked out from the sizes.
struct PoolStr {
  Str x, v, z, xb, zb, ox, ov;
};
template <bool DN>
__device__ __forceinline__ PoolStr pool_strides(const PoolParams& p) {
  if constexpr (DN) {
    const Str tok{p.heads * p.tokens * p.dim, p.tokens * p.dim, p.dim};
    const Str ent{p.heads * p.entries * p.dim, p.entries * p.dim, p.dim};
    return PoolStr{tok, tok, tok, tok, tok, ent, ent};
  } else {
    return PoolStr{p.x_st, p.v_st, p.z_st, p.xb_st, p.zb_st, p.ox_st, p.ov_st};
  }
}

template <typename TX, typename TZ, bool DUAL, bool HAS_V, bool TREAT, bool DN>
__global__ __launch_bounds__(256) void pool_kernel(PoolParams p) {
  const PoolStr S = pool_strides<DN>(p);
  __shared__ float part[32][256];  // [state value][thread], used when P > 1
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int L = p.lanes_per_row;
  const int li = lane & (L - 1);                 // lane inside the group
  const int gb = tid >> p.log2_lanes;            // group inside the workgroup
  const int P = 1 << p.log2_phases;
  const int phase = gb & (P - 1);
  const int groups = 256 >> p.log2_lanes;
  const int64_t rows_per_wg = groups >> p.log2_phases;
  const int64_t row = (int64_t)blockIdx.x * rows_per_wg + (gb >> p.log2_phases);
  const bool active = row < p.total_rows;
  const int64_t rr = active ? row : 0;

  const int64_t j = p.block_begin + rr % p.n_blocks;  // entry index
  const int64_t bh = rr / p.n_blocks;                // sequence * heads + head
  const int64_t h = bh % p.heads, b = bh / p.heads;
  const int64_t dim = p.dim;
  const int64_t c0 = (int64_t)li * 8;
  auto at = [&](Str st, int64_t r) { return b * st.s0 + h * st.s1 + r * st.s2 + c0; };
  const float* bias_h = p.bias + h * p.m * dim + c0;

  PoolAcc<TX, TZ, HAS_V> acc;
  acc.init();
  if (active) {
    const int64_t r0 = j * p.m - p.pos_base;  // token row of the entry's own block
    acc.run(static_cast<const TX*>(p.x) + at(S.x, r0), HAS_V ? static_cast<const TX*>(p.v) + at(S.v, r0) : nullptr,
            static_cast<const TZ*>(p.z) + at(S.z, r0), bias_h, phase, P, p.m, dim, RowPitch{S.x.s2, S.v.s2, S.z.s2});
    if (DUAL && j > 0) {
      const int64_t rb = r0 - p.m;  // preceding block, b-series
      acc.run(static_cast<const TX*>(p.xb) + at(S.xb, rb), nullptr, static_cast<const TZ*>(p.zb) + at(S.zb, rb),
              p.bias_b + h * p.m * dim + c0, phase, P, p.m, dim, RowPitch{S.xb.s2, 0, S.zb.s2});
    }
  }

  finish_entry<TX, TZ, HAS_V, TREAT>(acc, part, L, P, phase, active, dim, c0, j * p.m,
                                     EntryTreat{p.eps, p.rope_dims, p.log2_base},
                                     static_cast<TX*>(p.out_x) + at(S.ox, j),
                                     HAS_V ? static_cast<TX*>(p.out_v) + at(S.ov, j) : nullptr);
}

template <typename TX, typename TZ, bool DN>
static hipError_t launch_typed_d(const PoolParams& p, bool dual, bool has_v, bool treat, dim3 grid, hipStream_t s) {
  if (dual) {
    if (treat) pool_kernel<TX, TZ, true, false, true, DN><<<grid, 256, 0, s>>>(p);
    else pool_kernel<TX, TZ, true, false, false, DN><<<grid, 256, 0, s>>>(p);
  } else if (has_v) {
    pool_kernel<TX, TZ, false, true, false, DN><<<grid, 256, 0, s>>>(p);
  } else {
    if (treat) pool_kernel<TX, TZ, false, false, true, DN><<<grid, 256, 0, s>>>(p);
    else pool_kernel<TX, TZ, false, false, false, DN><<<grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

template <typename TX, typename TZ>
static hipError_t launch_typed(const PoolParams& p, bool dual, bool has_v, bool treat, dim3 grid, bool dn,
                               hipStream_t s) {
  return dn ? launch_typed_d<TX, TZ, true>(p, dual, has_v, treat, grid, s)
            : launch_typed_d<TX, TZ, false>(p, dual, has_v, treat, grid, s);
}

hipError_t launch_pool(const lbca_pool_args& a, hipStream_t stream) {
  PoolParams p;
  p.x = a.x; p.v = a.v; p.z = a.z; p.bias = a.bias;
  p.xb = a.xb; p.zb = a.zb; p.bias_b = a.bias_b;
  p.out_x = a.out_x; p.out_v = a.out_v;
  p.x_st = a.x_st; p.v_st = a.v_st; p.z_st = a.z_st; p.xb_st = a.xb_st; p.zb_st = a.zb_st;
  p.ox_st = a.out_x_st; p.ov_st = a.out_v_st;
  p.heads = a.heads; p.tokens = a.tokens; p.dim = a.dim; p.m = a.block; p.entries = a.entries;
  p.block_begin = a.block_begin; p.n_blocks = a.block_end - a.block_begin;
  p.pos_base = a.pos_base;
  p.total_rows = a.batch * a.heads * p.n_blocks;
  p.lanes_per_row = (int)(a.dim / 8);
  p.log2_lanes = __builtin_ctz((unsigned)p.lanes_per_row);
  p.eps = a.rmsnorm_eps;
  p.rope_dims = a.rope_dims;
  p.log2_base = a.rope_dims > 0 ? log2((double)a.rope_base) : 0.0;
  if (p.total_rows == 0) return hipSuccess;
  // token phases: grow P (<= groups per workgroup, <= m) until ~8K groups are busy
  const int groups = 256 / p.lanes_per_row;
  int lp = 0;
  while ((1 << (lp + 1)) <= groups && (1 << (lp + 1)) <= a.block && (1 << (lp + 1)) <= LBCA_POOL_MAX_PHASES &&
         p.total_rows * (int64_t(1) << lp) < 8192)
    ++lp;
  p.log2_phases = lp;
  const int64_t rows_per_wg = groups >> lp;
  dim3 grid((unsigned)((p.total_rows + rows_per_wg - 1) / rows_per_wg));
  const bool dual = a.xb != nullptr, has_v = a.v != nullptr;
  const bool treat = a.rmsnorm_eps >= 0.f || a.rope_dims > 0;
  const int64_t B = a.batch, H = a.heads, T = a.tokens, N = a.entries, d = a.dim;
  const bool dn = dense_strides(a.x, a.x_st, {B, H, T}, d) && dense_strides(a.v, a.v_st, {B, H, T}, d) &&
                  dense_strides(a.z, a.z_st, {B, H, T}, d) && dense_strides(a.xb, a.xb_st, {B, H, T}, d) &&
                  dense_strides(a.zb, a.zb_st, {B, H, T}, d) && dense_strides(a.out_x, a.out_x_st, {B, H, N}, d) &&
                  dense_strides(a.out_v, a.out_v_st, {B, H, N}, d);
  if (a.x_dtype == LBCA_BF16) {
    if (a.z_dtype == LBCA_BF16) return launch_typed<bf16_t, bf16_t>(p, dual, has_v, treat, grid, dn, stream);
    return launch_typed<bf16_t, float>(p, dual, has_v, treat, grid, dn, stream);
  }
  if (a.z_dtype == LBCA_BF16) return launch_typed<float, bf16_t>(p, dual, has_v, treat, grid, dn, stream);
  return launch_typed<float, float>(p, dual, has_v, treat, grid, dn, stream);
}

}  // namespace lbca
