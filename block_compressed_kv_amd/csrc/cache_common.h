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
  // element strides: token inputs {sequence, head}; rings and pooled outputs
  // {sequence, head, row}
  Str xn, vn, zn, xbn, zbn, rx, rv, rz, rxb, rzb, ox, ov;
};

// The strides of a cache step: the arguments', or, when every tensor of the
// call is dense (DN), the row-major ones worked out from the sizes.
struct CacheStr {
  Str xn, vn, zn, xbn, zbn, rx, rv, rz, rxb, rzb, ox, ov;
};
template <bool DN>
__device__ __forceinline__ CacheStr cache_strides(const CacheParams& p) {
  if constexpr (DN) {
    const Str tok{p.heads * p.dim, p.dim, 0};
    const Str ring{p.heads * 2 * p.ring * p.dim, 2 * p.ring * p.dim, p.dim};
    const Str ent{p.heads * p.entries * p.dim, p.entries * p.dim, p.dim};
    return CacheStr{tok, tok, tok, tok, tok, ring, ring, ring, ring, ring, ent, ent};
  } else {
    return CacheStr{p.xn, p.vn, p.zn, p.xbn, p.zbn, p.rx, p.rv, p.rz, p.rxb, p.rzb, p.ox, p.ov};
  }
}

inline void set_cache_strides(CacheParams& c, const lbca_cache_args& a) {
  c.xn = a.x_new_st; c.vn = a.v_new_st; c.zn = a.z_new_st; c.xbn = a.xb_new_st; c.zbn = a.zb_new_st;
  c.rx = a.raw_x_st; c.rv = a.raw_v_st; c.rz = a.raw_z_st; c.rxb = a.raw_xb_st; c.rzb = a.raw_zb_st;
  c.ox = a.out_x_st; c.ov = a.out_v_st;
}

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
          bool POOL = true, bool DN = false>
__device__ __forceinline__ void cache_row(const CacheParams& p, unsigned row, float (*part)[256], bool member) {
  const CacheStr S = cache_strides<DN>(p);
  const int tid = threadIdx.x, lane = tid & 63;
  const int L = p.lanes_per_row;
  const int li = lane & (L - 1);
  const int phase = tid >> p.log2_lanes;  // every lane group is a token phase of this row
  const int P = 256 >> p.log2_lanes;
  const unsigned b = row / (unsigned)p.heads, h = row % (unsigned)p.heads;
  const int64_t dim = p.dim, ring = p.ring;
  const int64_t c0 = (int64_t)li * 8;
  auto tok = [&](Str st) { return (int64_t)b * st.s0 + (int64_t)h * st.s1 + c0; };
  auto at = [&](Str st, int64_t r) { return tok(st) + r * st.s2; };
  // the new token's rows first: their addresses do not depend on the position
  constexpr bool X2 = sizeof(TX) == 4, Z2 = sizeof(TZ) == 4;  // two vectors per 8 fp32 elements
  const TX* xs = static_cast<const TX*>(p.x_new) + tok(S.xn);
  const TX* vs = static_cast<const TX*>(p.v_new) + tok(S.vn);
  const TZ* zs = static_cast<const TZ*>(p.z_new) + tok(S.zn);
  const TX* xbs = static_cast<const TX*>(p.xb_new) + tok(S.xbn);
  const TZ* zbs = static_cast<const TZ*>(p.zb_new) + tok(S.zbn);
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

  // 1. the new token into both rows of its slot
  const int64_t slot = t % ring;
  if (COPY && member && phase == 0) {
    // both ring rows of the slot in one series: its first 16-byte vectors, then (X2/Z2) the second
    auto put = [&](auto* base, Str st, uint4 a0, uint4 a1, bool two) {
      auto* r0 = base + at(st, slot);
      auto* r1 = r0 + ring * st.s2;
      st16(r0, 0, a0);
      st16(r1, 0, a0);
      if (two) {
        st16(r0, 1, a1);
        st16(r1, 1, a1);
      }
    };
    put(static_cast<TX*>(p.raw_x), S.rx, x0, x1, X2);
    if constexpr (HAS_V) put(static_cast<TX*>(p.raw_v), S.rv, v0, v1, X2);
    put(static_cast<TZ*>(p.raw_z), S.rz, z0, z1, Z2);
    if constexpr (DUAL) {
      put(static_cast<TX*>(p.raw_xb), S.rxb, xb0, xb1, X2);
      put(static_cast<TZ*>(p.raw_zb), S.rzb, zb0, zb1, Z2);
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
    acc.run(static_cast<const TX*>(p.raw_x) + at(S.rx, r0),
            HAS_V ? static_cast<const TX*>(p.raw_v) + at(S.rv, r0) : nullptr,
            static_cast<const TZ*>(p.raw_z) + at(S.rz, r0), p.bias + h * p.m * dim + c0, phase, P, p.m, dim,
            RowPitch{S.rx.s2, S.rv.s2, S.rz.s2});
  if (member && DUAL && j > 0) {  // block j-1 of the b-series, under the same softmax
    const int64_t rb0 = ((j - 1) * p.m) % ring;
    acc.run(static_cast<const TX*>(p.raw_xb) + at(S.rxb, rb0), nullptr,
            static_cast<const TZ*>(p.raw_zb) + at(S.rzb, rb0), p.bias_b + h * p.m * dim + c0, phase, P, p.m, dim,
            RowPitch{S.rxb.s2, 0, S.rzb.s2});
  }
  finish_entry<TX, TZ, HAS_V, TREAT>(acc, part, L, P, phase, true, dim, c0, j * p.m,
                                     EntryTreat{p.eps, p.rope_dims, p.log2_base},
                                     static_cast<TX*>(p.out_x) + at(S.ox, j),
                                     HAS_V ? static_cast<TX*>(p.out_v) + at(S.ov, j) : nullptr, member);
}


}  // namespace lbca
