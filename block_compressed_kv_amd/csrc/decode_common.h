// Decode parameters and per-sequence visibility shared by the decode kernels.
#pragma once
#include "device_util.h"
#include "lbca_internal.h"

namespace lbca {

struct DecodeParams {
  const bf16_t* q;
  const bf16_t* pk;
  const bf16_t* pv;
  const bf16_t* rk;
  const bf16_t* rv;
  const int64_t* pos;
  const int64_t* rpb;
  const int32_t* sel;
  const float* sink;
  float* out;
  float* lse;
  float* ws_ml;    // [units * splits][16][2]
  float* ws_acc;   // [units * splits][16][D] unnormalised fp32 partials (decode_kernel)
  bf16_t* ws_o;    // [units * splits][16][D] normalised bf16 partials (wide path)
  int64_t hq, hkv, G, entries, raw_rows, k_sel, m, W;
  int mode, splits, head_groups;
  int units;       // batch * kv_heads * head_groups
  int wide_twins;  // wide path: workgroups per (sequence, KV head, split), one per head-block set
  float scale_log2;
  float eps;
  int rope_dims;
  double log2_base;
  int qrows;  // > 1: consecutive rows b share cache sequence b / qrows (a query chunk)
  // fused cache step (lbca_decode_step): the new token's K and V rows
  // [batch, kv_heads, dim], read in place of the raw row at the position; the
  // raw base is worked out from the position and the ring size
  const bf16_t* tk;
  const bf16_t* tv;
  int64_t ring;  // > 0 only in the fused step
  // element strides.  q_st, o_st: {sequence, query of a chunk, head} (query
  // row b is query b % qrows of sequence b / qrows); pk/pv/rk/rv:
  // {sequence, KV head, row}; tk, tv: {sequence, KV head}
  Str q_st, o_st, pk_st, pv_st, rk_st, rv_st, tk_st, tv_st;
};

// Element offset of head h of query row b in q (q_st) or out (o_st).
__device__ __forceinline__ int64_t qrow_off(Str st, int qrows, int64_t b, int64_t h) {
  if (qrows > 1) return (b / qrows) * st.s0 + (b % qrows) * st.s1 + h * st.s2;
  return b * st.s0 + h * st.s2;
}

// Puts the argument fields a decode prologue needs into registers before its
// first branch.  Left to itself the compiler loads kernel arguments one basic
// block at a time, and at kernel start each of those dependent rounds is a
// full memory round trip before the first row load can be issued; an empty
// asm that takes every field as an input makes them one batch.
__device__ __forceinline__ void preload_params(const DecodeParams& p) {
  asm volatile("" ::"s"(p.q), "s"(p.pk), "s"(p.pv), "s"(p.rk), "s"(p.rv), "s"(p.pos), "s"(p.rpb), "s"(p.sel),
               "s"(p.hq), "s"(p.hkv), "s"(p.G), "s"(p.entries), "s"(p.raw_rows), "s"(p.k_sel), "s"(p.m), "s"(p.W),
               "s"(p.mode), "s"(p.splits), "s"(p.head_groups), "s"(p.units), "s"(p.wide_twins));
}
// The strides that place the query and the cache slices (strided calls).
__device__ __forceinline__ void preload_strides(const DecodeParams& p) {
  asm volatile("" ::"s"(p.q_st.s0), "s"(p.q_st.s1), "s"(p.q_st.s2), "s"(p.pk_st.s0), "s"(p.pk_st.s1),
               "s"(p.pk_st.s2), "s"(p.pv_st.s0), "s"(p.pv_st.s1), "s"(p.pv_st.s2), "s"(p.rk_st.s0),
               "s"(p.rk_st.s1), "s"(p.rk_st.s2), "s"(p.rv_st.s0), "s"(p.rv_st.s1), "s"(p.rv_st.s2));
}

// The strides a decode workgroup places its rows with: the arguments', or,
// when every tensor of the call is dense (DN), the row-major ones worked out
// from the sizes, which leaves the stride arguments unread.
struct DecStr {
  Str q, o, pk, pv, rk, rv, tk, tv;
};
// (qrows: the query rows per cache sequence, 1 outside a query chunk)
template <bool DN, int D>
__device__ __forceinline__ DecStr dec_strides(const DecodeParams& p, int qrows) {
  if constexpr (DN) {
    const Str qs{(int64_t)qrows * p.hq * D, p.hq * D, D};
    const Str ps{p.hkv * p.entries * D, p.entries * D, D};
    const Str rs{p.hkv * p.raw_rows * D, p.raw_rows * D, D};
    const Str ts{p.hkv * D, D, 0};
    return DecStr{qs, qs, ps, ps, rs, rs, ts, ts};
  } else {
    return DecStr{p.q_st, p.o_st, p.pk_st, p.pv_st, p.rk_st, p.rv_st, p.tk_st, p.tv_st};
  }
}

// A uniform value (a position, a raw base) requested before the row loads
// and used after them.  A plain load of it is taken as uniform and moved to
// scalar registers right after issue, which waits for it at once; a load
// through the scalar cache queues behind the row traffic and arrives late.
// Here the load goes out first as a vector load whose address the compiler
// takes as per-lane (an opaque zero), so nothing waits for it until
// uniform_value(), placed after the row loads, reads lane 0 (vector loads
// return in order, so that wait covers this load only).
struct EarlyI64 {
  int64_t v;
};
__device__ __forceinline__ EarlyI64 load_early(const int64_t* ptr) {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return EarlyI64{ptr[z]};
}
__device__ __forceinline__ int64_t uniform_value(EarlyI64 e) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)e.v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)e.v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// a % b for a >= 0, b > 0, in 32-bit arithmetic when both fit (the 64-bit
// remainder is a long instruction sequence).
__device__ __forceinline__ int64_t mod_nonneg(int64_t a, int64_t b) {
  if (((uint64_t)a | (uint64_t)b) < (uint64_t(1) << 32)) return (int64_t)((uint32_t)a % (uint32_t)b);
  return a % b;
}

struct SeqView {
  int64_t t, raw_begin, raw_row0;
  int n_pooled, n_sel, n_raw;
  bool ok;
};

// t: the sequence's position, base: position of raw row 0.
__device__ __forceinline__ SeqView seq_view(const DecodeParams& p, int64_t b, int64_t t, int64_t base) {
  SeqView v;
  v.t = t;
  int64_t np = 0, rb = 0;
  bool ok = v.t >= 0;
  if (ok) visible_range(v.t, p.m, p.W, p.mode, &np, &rb);
  ok = ok && np <= p.entries && rb - base >= 0 && v.t - base < p.raw_rows;
  v.ok = ok;
  v.n_pooled = (int)np;
  v.n_sel = ok ? (int)(p.sel ? p.k_sel : np) : 0;
  v.n_raw = ok ? (int)(v.t - rb + 1) : 0;
  v.raw_begin = rb;
  v.raw_row0 = rb - base;
  return v;
}
__device__ __forceinline__ SeqView seq_view(const DecodeParams& p, int64_t b) {
  const int64_t t = p.pos[b];
  int64_t base = p.rpb ? p.rpb[b] : 0;
  if (p.ring > 0 && t >= 0) {  // fused cache step: the base it writes for t
    int64_t np, rb;
    visible_range(t, p.m, p.W, p.mode, &np, &rb);
    base = rb - mod_nonneg(rb, p.ring);
  }
  return seq_view(p, b, t, base);
}

// Wide-row MQA decode (512 dims, shared series, query heads in blocks of 32
// per KV head): launched by launch_decode when the plan selects it.
// dn: every tensor of the call dense (instances that work the strides out from the sizes).
hipError_t launch_decode_wide(const DecodeParams& p, int rope_dims, bool treat, int head_blocks, bool dn,
                              hipStream_t stream);
// norm: the partials are the wide path's normalised bf16 outputs (ws_o).
void launch_decode_merge(const DecodeParams& p, int64_t batch, int64_t dim, bool norm, hipStream_t stream);

}  // namespace lbca
