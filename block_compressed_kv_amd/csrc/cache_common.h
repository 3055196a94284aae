// The decode-time cache step of one (sequence, head) row, shared by
// lbca_cache_append and the fused lbca_decode_step.
//
// Method: "mSeek: learned KV-cache compression in a 3B model", section "How LBCA
// works" (steps 1-3: new tokens join the raw cache; a block that is complete
// and has left the W-token window becomes one pooled entry); "HCA: Heavily
// Compressed Attention (toy implementation)", "What is implemented" (every
// complete block is an entry, with RMSNorm and partial RoPE at its start).
#pragma once
#include "lbca_internal.h"
#include "pool_common.h"

namespace lbca {

struct CacheParams {
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
  const void* xb_new;  // dual (CSA) mode: the b-series
  const void* zb_new;
  void* raw_xb;
  void* raw_zb;
  const float* bias_b;
  int64_t heads, dim, m, W, ring, entries;
  int mode;
  int lanes_per_row;  // L = dim / 8
  int log2_lanes;
  float eps;
  int rope_dims;
  double log2_base;
};

// 16-byte vector i of row r (8 elements are one vector in bf16, two in fp32).
template <typename T>
__device__ __forceinline__ uint4 ld16(const T* r, int i) { return reinterpret_cast<const uint4*>(r)[i]; }
template <typename T>
__device__ __forceinline__ void st16(T* r, int i, uint4 v) { reinterpret_cast<uint4*>(r)[i] = v; }

// The cache step of one (sequence, head) row, run by the first 256 threads of
// the workgroup (member); wider workgroups' other threads pass member = false
// and only take part in the barriers.  AT_COMPLETION pools a block on the step
// of its last token (lbca_decode_step) instead of the step that makes it
// visible (lbca_cache_append).  COPY: the token append and the raw base (no
// barrier: the first L threads' work); POOL: the due block (every thread of the
// workgroup calls it when it pools, for the barriers).
template <typename TX, typename TZ, bool HAS_V, bool TREAT, bool DUAL, bool AT_COMPLETION, bool COPY = true,
          bool POOL = true>
__device__ __forceinline__ void cache_row(const CacheParams& p, unsigned row, float (*part)[256], bool member) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int L = p.lanes_per_row;
  const int li = lane & (L - 1);
  const int phase = tid >> p.log2_lanes;  // every lane group is a token phase of this row
  const int P = 256 >> p.log2_lanes;
  const unsigned b = row / (unsigned)p.heads, h = row % (unsigned)p.heads;
  const int64_t dim = p.dim, ring = p.ring;
  const int64_t c0 = (int64_t)li * 8;
  // the new token's rows first: their addresses do not depend on the position
  constexpr bool X2 = sizeof(TX) == 4, Z2 = sizeof(TZ) == 4;  // two vectors per 8 fp32 elements
  const int64_t src = (int64_t)row * dim + c0;
  const TX* xs = static_cast<const TX*>(p.x_new) + src;
  const TX* vs = static_cast<const TX*>(p.v_new) + src;
  const TZ* zs = static_cast<const TZ*>(p.z_new) + src;
  const TX* xbs = static_cast<const TX*>(p.xb_new) + src;
  const TZ* zbs = static_cast<const TZ*>(p.zb_new) + src;
  uint4 x0 = {}, x1 = {}, v0 = {}, v1 = {}, z0 = {}, z1 = {}, xb0 = {}, xb1 = {}, zb0 = {}, zb1 = {};
  if (COPY && member && phase == 0) {
    x0 = ld16(xs, 0);
    if constexpr (X2) x1 = ld16(xs, 1);
    if constexpr (HAS_V) {
      v0 = ld16(vs, 0);
      if constexpr (X2) v1 = ld16(vs, 1);
    }
    z0 = ld16(zs, 0);
    if constexpr (Z2) z1 = ld16(zs, 1);
    if constexpr (DUAL) {
      xb0 = ld16(xbs, 0);
      if constexpr (X2) xb1 = ld16(xbs, 1);
      zb0 = ld16(zbs, 0);
      if constexpr (Z2) zb1 = ld16(zbs, 1);
    }
  }
  const int64_t t = p.pos[b];
  if (t < 0) return;
  const int64_t series = (int64_t)row * 2 * ring * dim + c0;  // ring rows of this (sequence, head)

  // 1. the new token into both rows of its slot
  const int64_t slot = t % ring;
  if (COPY && member && phase == 0) {
    const int64_t d0 = series + slot * dim, d1 = d0 + ring * dim;
    TX* rx = static_cast<TX*>(p.raw_x);
    TZ* rz = static_cast<TZ*>(p.raw_z);
    st16(rx + d0, 0, x0);
    st16(rx + d1, 0, x0);
    if constexpr (X2) {
      st16(rx + d0, 1, x1);
      st16(rx + d1, 1, x1);
    }
    if constexpr (HAS_V) {
      TX* rv = static_cast<TX*>(p.raw_v);
      st16(rv + d0, 0, v0);
      st16(rv + d1, 0, v0);
      if constexpr (X2) {
        st16(rv + d0, 1, v1);
        st16(rv + d1, 1, v1);
      }
    }
    st16(rz + d0, 0, z0);
    st16(rz + d1, 0, z0);
    if constexpr (Z2) {
      st16(rz + d0, 1, z1);
      st16(rz + d1, 1, z1);
    }
    if constexpr (DUAL) {
      TX* rxb = static_cast<TX*>(p.raw_xb);
      TZ* rzb = static_cast<TZ*>(p.raw_zb);
      st16(rxb + d0, 0, xb0);
      st16(rxb + d1, 0, xb0);
      st16(rzb + d0, 0, zb0);
      st16(rzb + d1, 0, zb0);
      if constexpr (X2) {
        st16(rxb + d0, 1, xb1);
        st16(rxb + d1, 1, xb1);
      }
      if constexpr (Z2) {
        st16(rzb + d0, 1, zb1);
        st16(rzb + d1, 1, zb1);
      }
    }
  }
  // 2. the raw base that maps t's raw span onto ring rows
  int64_t n_pooled, raw_begin;
  visible_range(t, p.m, p.W, p.mode, &n_pooled, &raw_begin);
  if (COPY && h == 0 && tid == 0) p.raw_pos_base[b] = raw_begin - raw_begin % ring;
  if constexpr (!POOL) return;
  // 3. the block that becomes visible at t (or, AT_COMPLETION, whose last token is t), if any
  const int64_t x = (p.mode == LBCA_EXCLUSIVE && !AT_COMPLETION) ? t + 1 - p.W : t + 1;
  if (x <= 0 || x % p.m != 0) return;
  const int64_t j = x / p.m - 1;
  if (j >= p.entries) return;
  __syncthreads();  // the copied token (the last one of an OVERLAP or just-completed block) is visible to every lane
  const int64_t r0 = (j * p.m) % ring;  // first ring row of the block
  PoolAcc<TX, TZ, HAS_V> acc;
  acc.init();
  if (member)
    acc.run(static_cast<const TX*>(p.raw_x) + series + r0 * dim,
            HAS_V ? static_cast<const TX*>(p.raw_v) + series + r0 * dim : nullptr,
            static_cast<const TZ*>(p.raw_z) + series + r0 * dim, p.bias + h * p.m * dim + c0, phase, P, p.m, dim);
  if (member && DUAL && j > 0) {  // block j-1 of the b-series, under the same softmax
    const int64_t rb0 = ((j - 1) * p.m) % ring;
    acc.run(static_cast<const TX*>(p.raw_xb) + series + rb0 * dim, nullptr,
            static_cast<const TZ*>(p.raw_zb) + series + rb0 * dim, p.bias_b + h * p.m * dim + c0, phase, P, p.m, dim);
  }
  const int64_t o = ((int64_t)row * p.entries + j) * dim + c0;
  finish_entry<TX, TZ, HAS_V, TREAT>(acc, part, L, P, phase, true, dim, c0, j * p.m,
                                     EntryTreat{p.eps, p.rope_dims, p.log2_base}, static_cast<TX*>(p.out_x) + o,
                                     HAS_V ? static_cast<TX*>(p.out_v) + o : nullptr, member);
}


}  // namespace lbca
