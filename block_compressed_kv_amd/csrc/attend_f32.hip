// fp32 attention rows (decode and prefill) on the vector ALUs.
//
// Method: "mSeek: learned KV-cache compression in a 3B model", "How LBCA works"
// (steps 4-5): a query at t attends, under one softmax, over the visible pooled
// entries and the raw span; with an optional sink logit in the denominator
// ("HCA"/"CSA" toy-implementation pages, "What is implemented").
//
// One wave per (sequence, query, head).  Lanes score 64 visible rows at a time
// (each lane one row, q broadcast from LDS), a wave-wide online softmax keeps
// the running max and sum, then every probability is broadcast to accumulate
// the value rows, each lane owning dim/64 output dims.  fp32 throughout: this
// is the exact-arithmetic path for fp32 caches.
#include "device_util.h"
#include "lbca_internal.h"

namespace lbca {

struct RowsParams {
  const float* q;
  const float* pk;
  const float* pv;
  const float* rk;
  const float* rv;
  const int64_t* pos;      // device positions (decode) or null
  int64_t q_pos0;          // first query position (prefill)
  const int64_t* rpb_dev;  // device raw_pos_base (decode) or null
  int64_t rpb_host;
  const int32_t* sel;
  const float* sink;
  void* out;
  int out_bf16;
  float* lse;
  int64_t q_len, hq, hkv, G, entries, raw_rows, k_sel, m, W;
  int mode;
  float scale;
  // element strides: q and out {sequence, query, head}; caches {sequence, KV head, row}
  Str q_st, o_st, pk_st, pv_st, rk_st, rv_st;
};

template <int D>
__global__ __launch_bounds__(64) void rows_f32_kernel(RowsParams p) {
  constexpr int DPL = D / 64;
  __shared__ float qs[D];
  const int lane = threadIdx.x;
  const int64_t id = blockIdx.x;  // ((b * q_len + i) * hq + h)
  const int64_t h = id % p.hq;
  const int64_t bi = id / p.hq;
  const int64_t i = bi % p.q_len;
  const int64_t b = bi / p.q_len;
  const int64_t kvh = h / p.G;
  const int64_t t = p.pos ? p.pos[b] : p.q_pos0 + i;
  const int64_t base = p.rpb_dev ? p.rpb_dev[b] : p.rpb_host;
  int64_t np = 0, rb = 0;
  bool ok = t >= 0;
  if (ok) visible_range(t, p.m, p.W, p.mode, &np, &rb);
  ok = ok && np <= p.entries && rb - base >= 0 && t - base < p.raw_rows;
  float o[DPL];
  const int64_t orow = b * p.o_st.s0 + i * p.o_st.s1 + h * p.o_st.s2 + lane * DPL;
  if (!ok) {
    for (int c = 0; c < DPL; ++c) o[c] = __builtin_nanf("");
  } else {
    const float* qrow = p.q + b * p.q_st.s0 + i * p.q_st.s1 + h * p.q_st.s2;
    for (int d = lane; d < D; d += 64) qs[d] = qrow[d];
    __syncthreads();
    const int64_t n_sel = p.sel ? p.k_sel : np;
    const int64_t n_raw = t - rb + 1;
    const int64_t n_tot = n_sel + n_raw;
    const float* kpool = p.pk + b * p.pk_st.s0 + kvh * p.pk_st.s1;
    const float* kraw = p.rk + b * p.rk_st.s0 + kvh * p.rk_st.s1 + (rb - base) * p.rk_st.s2;
    const float* vpool = p.pv ? p.pv + b * p.pv_st.s0 + kvh * p.pv_st.s1 : kpool;
    const float* vraw = p.rv ? p.rv + b * p.rv_st.s0 + kvh * p.rv_st.s1 + (rb - base) * p.rv_st.s2 : kraw;
    const int64_t vps = p.pv ? p.pv_st.s2 : p.pk_st.s2, vrs = p.rv ? p.rv_st.s2 : p.rk_st.s2;
    float m_run = kNegInf, l_run = 0.f;
    for (int c = 0; c < DPL; ++c) o[c] = 0.f;
    for (int64_t g0 = 0; g0 < n_tot; g0 += 64) {
      // each lane scores one row
      const int64_t v = g0 + lane;
      bool rok = v < n_tot;
      const float* krow = nullptr;
      if (rok) {
        if (v < n_sel) {
          const int64_t e = p.sel ? (int64_t)p.sel[b * p.k_sel + v] : v;
          rok = e >= 0 && e < np;
          krow = kpool + e * p.pk_st.s2;
        } else {
          krow = kraw + (v - n_sel) * p.rk_st.s2;
        }
      }
      float s = kNegInf;
      if (rok) {
        float dot = 0.f;
        for (int d = 0; d < D; d += 4) {
          const float4 k4 = *reinterpret_cast<const float4*>(krow + d);
          dot = fmaf(qs[d], k4.x, dot);
          dot = fmaf(qs[d + 1], k4.y, dot);
          dot = fmaf(qs[d + 2], k4.z, dot);
          dot = fmaf(qs[d + 3], k4.w, dot);
        }
        s = dot * p.scale;
      }
      const float gmax = group_max<64>(s);
      const float nm = fmaxf(m_run, gmax);
      const float mu = nm == kNegInf ? 0.f : nm;
      const float corr = expf(m_run - mu);
      const float pr = expf(s - mu);
      l_run = l_run * corr + group_sum<64>(pr);
      for (int c = 0; c < DPL; ++c) o[c] *= corr;
      m_run = nm;
      const int cnt = (int)(n_tot - g0 < 64 ? n_tot - g0 : 64);
      for (int r = 0; r < cnt; ++r) {
        const float pw = __shfl(pr, r, 64);
        if (pw == 0.f) continue;  // masked row (uniform across the wave)
        const int64_t vv = g0 + r;
        const float* vrow;
        if (vv < n_sel) {
          const int64_t e = p.sel ? (int64_t)p.sel[b * p.k_sel + vv] : vv;
          vrow = vpool + e * vps;
        } else {
          vrow = vraw + (vv - n_sel) * vrs;
        }
        for (int c = 0; c < DPL; ++c) o[c] = fmaf(pw, vrow[lane * DPL + c], o[c]);
      }
    }
    float den = l_run;
    if (p.sink) den += expf(p.sink[h] - m_run);
    const float inv = 1.f / den;
    for (int c = 0; c < DPL; ++c) o[c] *= inv;
    if (lane == 0 && p.lse) p.lse[id] = m_run + logf(den);
  }
  if (!ok && lane == 0 && p.lse) p.lse[id] = __builtin_nanf("");
  if (p.out_bf16) {
    bf16_t* out = static_cast<bf16_t*>(p.out) + orow;
    for (int c = 0; c < DPL; ++c) out[c].bits = (uint16_t)(pack_bf16x2(o[c], 0.f) & 0xffff);
  } else {
    float* out = static_cast<float*>(p.out) + orow;
    for (int c = 0; c < DPL; ++c) out[c] = o[c];
  }
}

hipError_t launch_rows_f32(const RowsParams& rp, int64_t dim, int64_t batch, hipStream_t s) {
  const dim3 grid((unsigned)(batch * rp.q_len * rp.hq));
  switch (dim) {
    case 64: rows_f32_kernel<64><<<grid, 64, 0, s>>>(rp); break;
    case 128: rows_f32_kernel<128><<<grid, 64, 0, s>>>(rp); break;
    case 192: rows_f32_kernel<192><<<grid, 64, 0, s>>>(rp); break;
    case 256: rows_f32_kernel<256><<<grid, 64, 0, s>>>(rp); break;
    case 320: rows_f32_kernel<320><<<grid, 64, 0, s>>>(rp); break;
    case 384: rows_f32_kernel<384><<<grid, 64, 0, s>>>(rp); break;
    case 448: rows_f32_kernel<448><<<grid, 64, 0, s>>>(rp); break;
    case 512: rows_f32_kernel<512><<<grid, 64, 0, s>>>(rp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const lbca_prefill_args& a, hipStream_t stream) {
  RowsParams rp{};
  rp.q = static_cast<const float*>(a.q);
  rp.pk = static_cast<const float*>(a.pooled_k);
  rp.pv = static_cast<const float*>(a.pooled_v);
  rp.rk = static_cast<const float*>(a.raw_k);
  rp.rv = static_cast<const float*>(a.raw_v);
  rp.pos = nullptr;
  rp.q_pos0 = a.q_pos0;
  rp.rpb_dev = nullptr;
  rp.rpb_host = a.raw_pos_base;
  rp.sel = nullptr;
  rp.sink = a.sink;
  rp.out = a.out;
  rp.out_bf16 = a.out_dtype == LBCA_BF16;
  rp.lse = a.lse;
  rp.q_len = a.q_len;
  rp.hq = a.q_heads; rp.hkv = a.kv_heads; rp.G = a.q_heads / a.kv_heads;
  rp.entries = a.entries; rp.raw_rows = a.raw_rows; rp.k_sel = 0;
  rp.m = a.block; rp.W = a.window; rp.mode = a.mode; rp.scale = a.scale;
  rp.q_st = a.q_st; rp.o_st = a.out_st;
  rp.pk_st = a.pooled_k_st; rp.pv_st = a.pooled_v_st; rp.rk_st = a.raw_k_st; rp.rv_st = a.raw_v_st;
  return launch_rows_f32(rp, a.dim, a.batch, stream);
}

hipError_t launch_decode_f32(const lbca_decode_args& a, hipStream_t stream) {
  RowsParams rp{};
  rp.q = static_cast<const float*>(a.q);
  rp.pk = static_cast<const float*>(a.pooled_k);
  rp.pv = static_cast<const float*>(a.pooled_v);
  rp.rk = static_cast<const float*>(a.raw_k);
  rp.rv = static_cast<const float*>(a.raw_v);
  rp.pos = a.pos;
  rp.q_pos0 = 0;
  rp.rpb_dev = a.raw_pos_base;
  rp.rpb_host = 0;
  rp.sel = a.sel_idx;
  rp.sink = a.sink;
  rp.out = a.out;
  rp.out_bf16 = 0;
  rp.lse = a.lse;
  rp.q_len = 1;
  rp.hq = a.q_heads; rp.hkv = a.kv_heads; rp.G = a.q_heads / a.kv_heads;
  rp.entries = a.entries; rp.raw_rows = a.raw_rows; rp.k_sel = a.sel_idx ? a.k_sel : 0;
  rp.m = a.block; rp.W = a.window; rp.mode = a.mode; rp.scale = a.scale;
  // q and out [batch, heads, dim] as {sequence, query (one), head}
  rp.q_st = lbca_strides{{a.q_st.s[0], 0, a.q_st.s[1]}};
  rp.o_st = lbca_strides{{a.out_st.s[0], 0, a.out_st.s[1]}};
  rp.pk_st = a.pooled_k_st; rp.pv_st = a.pooled_v_st; rp.rk_st = a.raw_k_st; rp.rv_st = a.raw_v_st;
  return launch_rows_f32(rp, a.dim, a.batch, stream);
}

}  // namespace lbca
