// Decode attention over pooled entries plus the raw window (split-K flash-decode).
//
// Method: "mSeek: learned KV-cache compression in a 3B model", "How LBCA works"
// (step 4: attend over every completed summary plus the exact local window);
// "HCA: Heavily Compressed Attention (toy implementation)" and "CSA: Compressed
// Sparse Attention (toy implementation)", "What is implemented" (shared-KV MQA,
// RMSNorm on queries and entries, partial RoPE with the -t output rotation,
// attention sink, selected entries plus the sliding window).
//
// bf16 path (MFMA).  One wave per workgroup.  A wave owns 16 query heads of one
// KV head (GQA groups are padded to 16; MQA with 64 heads uses 4 head groups)
// and a contiguous range of R-row tiles of the visible-row list (pooled or
// selected entries, then the raw span).  Scores are computed transposed,
// S^T[row, head] = K[row, :] . Q[head, :], with v_mfma_f32_16x16x32_bf16 whose
// A operand is read straight from global memory in row-major K layout, so
// every lane holds all scores of one head and the softmax max/sum need only
// two cross-lane steps.  P^T is already the B-operand layout of
// v_mfma_f32_16x16x16_bf16 for O^T = V^T P^T; V rows go through LDS so the
// A operand (8 rows of one dim per lane) can be gathered.  Each wave writes an
// unnormalised partial (acc, running max, running sum); a merge kernel combines
// the splits in a fixed order (bitwise reproducible), adds the sink and
// applies the -t rotation.
//
// fp32 path (VALU).  One wave per (query, head): lanes score 64 rows at a time,
// then broadcast each probability to accumulate V.  Used for fp32 decode and
// fp32 prefill.
#include "device_util.h"
#include "lbca_internal.h"

namespace lbca {

typedef short s16x4 __attribute__((ext_vector_type(4)));

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
  float* ws_acc;  // [wg][16][D]
  float* ws_ml;   // [wg][16][2]
  int64_t hq, hkv, G, entries, raw_rows, k_sel, m, W;
  int mode, splits, head_groups, dim;
  float scale_log2;
  float eps;
  int rope_dims;
  double log2_base;
};

struct SeqView {
  int64_t t, n_pooled, n_sel, n_raw, raw_begin, raw_row0;
  bool ok;
};

__device__ __forceinline__ SeqView seq_view(const DecodeParams& p, int64_t b) {
  SeqView v;
  v.t = p.pos[b];
  const int64_t base = p.rpb ? p.rpb[b] : 0;
  int64_t np = 0, rb = 0;
  bool ok = v.t >= 0;
  if (ok) visible_range(v.t, p.m, p.W, p.mode, &np, &rb);
  ok = ok && np <= p.entries && rb - base >= 0 && v.t - base < p.raw_rows;
  v.ok = ok;
  v.n_pooled = np;
  v.n_sel = ok ? (p.sel ? p.k_sel : np) : 0;
  v.n_raw = ok ? v.t - rb + 1 : 0;
  v.raw_begin = rb;
  v.raw_row0 = rb - base;
  return v;
}

__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  f[0] = lo_bf16(u.x); f[1] = hi_bf16(u.x); f[2] = lo_bf16(u.y); f[3] = hi_bf16(u.y);
  f[4] = lo_bf16(u.z); f[5] = hi_bf16(u.z); f[6] = lo_bf16(u.w); f[7] = hi_bf16(u.w);
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 u;
  u.x = pack_bf16x2(f[0], f[1]); u.y = pack_bf16x2(f[2], f[3]);
  u.z = pack_bf16x2(f[4], f[5]); u.w = pack_bf16x2(f[6], f[7]);
  return u;
}

// HCA/CSA treatment of one row held in MFMA operand layout: lane (., kq) holds
// dims 32*s + 8*kq + i of the row (s < D/32, i < 8); the 4 lanes of a row are
// lane, lane^16, lane^32, lane^48.  RMSNorm over all D dims, then RoPE on the
// last RD dims (rotate-half pairs (k, k+RD/2) sit in the same lane, RD/64 steps
// apart).  Every lane of the wave must call this (it shuffles).
template <int D, int RD>
__device__ __forceinline__ void treat_row(uint4 (&r)[D / 32], double pos, bool ok, float eps,
                                          double log2_base) {
  constexpr int KS = D / 32;
  const int kq = (threadIdx.x & 63) >> 4;
  if (eps >= 0.f) {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float f[8];
      unpack8(r[s], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = ok ? 1.f / sqrtf(ss / (float)D + eps) : 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float f[8];
      unpack8(r[s], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] *= inv;
      r[s] = pack8(f);
    }
  }
  if (RD > 0) {
    constexpr int SH = RD / 64;       // steps between pair partners
    constexpr int S0 = KS - 2 * SH;   // first rotated step
#pragma unroll
    for (int s = S0; s < S0 + SH; ++s) {
      float a[8], b[8];
      unpack8(r[s], a);
      unpack8(r[s + SH], b);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = 32 * (s - S0) + 8 * kq + i;
        float c, sn;
        rope_cos_sin(pos, k, RD, log2_base, &c, &sn);
        const float x1 = a[i], x2 = b[i];
        a[i] = x1 * c - x2 * sn;
        b[i] = x2 * c + x1 * sn;
      }
      r[s] = pack8(a);
      r[s + SH] = pack8(b);
    }
  }
}

template <int D, int R, bool SHARED, int RD, bool TREAT>
__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeParams p) {
  constexpr int KS = D / 32, NH = R / 16, DT = D / 16, PITCH = D + 8;
  __shared__ __attribute__((aligned(16))) bf16_t vtile[R * PITCH];

  const int lane = threadIdx.x, n = lane & 15, kq = lane >> 4;
  int64_t id = blockIdx.x;
  const int split = (int)(id % p.splits);
  id /= p.splits;
  const int hg = (int)(id % p.head_groups);
  id /= p.head_groups;
  const int64_t kvh = id % p.hkv;
  const int64_t b = id / p.hkv;
  const SeqView sv = seq_view(p, b);

  const int64_t tiles_p = (sv.n_sel + R - 1) / R;
  const int64_t tiles_total = tiles_p + (sv.n_raw + R - 1) / R;
  const int64_t per = (tiles_total + p.splits - 1) / p.splits;
  const int64_t t0 = split * per;
  const int64_t t1 = t0 + per < tiles_total ? t0 + per : tiles_total;

  // queries of this head group as B operands (zero for padded heads)
  const int64_t slot = (int64_t)hg * 16 + n;
  const bool head_ok = slot < p.G;
  const bf16_t* qrow = p.q + ((b * p.hkv + kvh) * p.G + slot) * D + 8 * kq;
  uint4 qr[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qr[s] = head_ok ? *reinterpret_cast<const uint4*>(qrow + 32 * s) : make_uint4(0, 0, 0, 0);
  if (TREAT) treat_row<D, RD>(qr, (double)sv.t, head_ok, p.eps, p.log2_base);

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t kv_pool = (b * p.hkv + kvh) * p.entries;
  const int64_t kv_raw = (b * p.hkv + kvh) * p.raw_rows + sv.raw_row0;

  for (int64_t tile = t0; tile < t1; ++tile) {
    const bool is_raw = tile >= tiles_p;
    const int64_t v0 = is_raw ? (tile - tiles_p) * R : tile * R;
    const int64_t count = is_raw ? sv.n_raw : sv.n_sel;
    uint4 kr[NH][KS];
    uint4 vr[SHARED ? 1 : NH][SHARED ? 1 : KS];
    unsigned valid[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int64_t v = v0 + 16 * h + n;
      bool ok = v < count;
      int64_t row = 0;
      if (is_raw) {
        row = kv_raw + v;
      } else {
        int64_t e = v;
        if (p.sel) e = ok ? (int64_t)p.sel[b * p.k_sel + v] : -1;
        ok = ok && e >= 0 && e < sv.n_pooled;
        row = kv_pool + e;
      }
      const bf16_t* kp = (is_raw ? p.rk : p.pk) + row * D + 8 * kq;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kr[h][s] = ok ? *reinterpret_cast<const uint4*>(kp + 32 * s) : make_uint4(0, 0, 0, 0);
      if (!SHARED) {
        const bf16_t* vp = (is_raw ? p.rv : p.pv) + row * D + 8 * kq;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          vr[h][s] = ok ? *reinterpret_cast<const uint4*>(vp + 32 * s) : make_uint4(0, 0, 0, 0);
      }
      if (TREAT && is_raw) treat_row<D, RD>(kr[h], (double)(sv.raw_begin + v), ok, p.eps, p.log2_base);
      valid[h] = (unsigned)(__ballot(ok) & 0xffffull);
    }
    // value rows to LDS (row-major) for the transposed A-operand gather
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        *reinterpret_cast<uint4*>(&vtile[(16 * h + n) * PITCH + 32 * s + 8 * kq]) =
            SHARED ? kr[h][s] : vr[h][s];

    // S^T = K Q^T (16 rows x 16 heads per half)
    float sc[NH][4];
    float tmax = kNegInf;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[h][s]),
                                                     __builtin_bit_cast(bf16x8, qr[s]), c, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool vok = (valid[h] >> (4 * kq + j)) & 1u;
        sc[h][j] = vok ? c[j] * p.scale_log2 : kNegInf;
        tmax = fmaxf(tmax, sc[h][j]);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float nm = fmaxf(m_run, tmax);
    const float mu = nm == kNegInf ? 0.f : nm;
    const float corr = exp2f(m_run - mu);
    float psum = 0.f;
    s16x4 pop[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float pj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pj[j] = exp2f(sc[h][j] - mu);
        psum += pj[j];
      }
      const uint32_t w0 = pack_bf16x2(pj[0], pj[1]), w1 = pack_bf16x2(pj[2], pj[3]);
      pop[h] = s16x4{(short)(w0 & 0xffff), (short)(w0 >> 16), (short)(w1 & 0xffff), (short)(w1 >> 16)};
    }
    l_run = fmaf(l_run, corr, psum);
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] *= corr;
    m_run = nm;
    __syncthreads();
    // O^T += V^T P^T
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const bf16_t* vb = &vtile[(16 * h + 4 * kq) * PITCH + n];
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        s16x4 a;
        a[0] = (short)vb[16 * t].bits;
        a[1] = (short)vb[PITCH + 16 * t].bits;
        a[2] = (short)vb[2 * PITCH + 16 * t].bits;
        a[3] = (short)vb[3 * PITCH + 16 * t].bits;
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pop[h], acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  if (head_ok) {
    const int64_t wg = blockIdx.x;
    float* dst = p.ws_acc + (wg * 16 + n) * D + 4 * kq;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      *reinterpret_cast<float4*>(dst + 16 * t) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    if (kq == 0) {
      p.ws_ml[(wg * 16 + n) * 2] = m_run;
      p.ws_ml[(wg * 16 + n) * 2 + 1] = l_run;
    }
  }
}

// Combine the splits of one (sequence, query head): fixed order, then sink,
// normalisation, LSE and the -t rotation of the last rope_dims dims.
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeParams p) {
  __shared__ float orow[512];
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / p.hq, h = bh % p.hq;
  const int64_t kvh = h / p.G, g = h % p.G;
  const int64_t hg = g / 16, n = g % 16;
  const int D = p.dim;
  const SeqView sv = seq_view(p, b);
  float* out = p.out + bh * D;
  if (!sv.ok) {
    for (int d = threadIdx.x; d < D; d += blockDim.x) out[d] = __builtin_nanf("");
    if (threadIdx.x == 0 && p.lse) p.lse[bh] = __builtin_nanf("");
    return;
  }
  const int64_t wg0 = ((b * p.hkv + kvh) * p.head_groups + hg) * p.splits;
  float M = kNegInf;
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.ws_ml[((wg0 + s) * 16 + n) * 2]);
  float L = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    const float* ml = p.ws_ml + ((wg0 + s) * 16 + n) * 2;
    L += ml[1] * exp2f(ml[0] - M);
  }
  if (p.sink) L += exp2f(p.sink[h] * kLog2e - M);
  const float invL = 1.f / L;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float o = 0.f;
    for (int s = 0; s < p.splits; ++s) {
      const float w = exp2f(p.ws_ml[((wg0 + s) * 16 + n) * 2] - M);
      o = fmaf(p.ws_acc[((wg0 + s) * 16 + n) * D + d], w, o);
    }
    orow[d] = o * invL;
  }
  __syncthreads();
  const int r = p.rope_dims, half = r / 2;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float o = orow[d];
    if (r > 0 && d >= D - r) {
      const bool lo = d < D - half;
      const int k = lo ? d - (D - r) : d - (D - half);
      float c, sn;
      rope_cos_sin(-(double)sv.t, k, r, p.log2_base, &c, &sn);
      const float other = lo ? orow[d + half] : orow[d - half];
      o = lo ? o * c - other * sn : o * c + other * sn;
    }
    out[d] = o;
  }
  if (threadIdx.x == 0 && p.lse) p.lse[bh] = (M + log2f(L)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------------------
// fp32 path: one wave per (sequence, query, head); decode and prefill.
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
  const int64_t orow = id * D + lane * DPL;
  if (!ok) {
    for (int c = 0; c < DPL; ++c) o[c] = __builtin_nanf("");
  } else {
    const float* qrow = p.q + id * D;
    for (int d = lane; d < D; d += 64) qs[d] = qrow[d];
    __syncthreads();
    const int64_t n_sel = p.sel ? p.k_sel : np;
    const int64_t n_raw = t - rb + 1;
    const int64_t n_tot = n_sel + n_raw;
    const int64_t kv_pool = (b * p.hkv + kvh) * p.entries;
    const int64_t kv_raw = (b * p.hkv + kvh) * p.raw_rows + (rb - base);
    const float* vpool = p.pv ? p.pv : p.pk;
    const float* vraw = p.rv ? p.rv : p.rk;
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
          krow = p.pk + (kv_pool + e) * D;
        } else {
          krow = p.rk + (kv_raw + (v - n_sel)) * D;
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
          vrow = vpool + (kv_pool + e) * D;
        } else {
          vrow = vraw + (kv_raw + (vv - n_sel)) * D;
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
  return launch_rows_f32(rp, a.dim, a.batch, stream);
}

// ---------------------------------------------------------------------------
static int rows_per_tile(int64_t dim) { return dim >= 512 ? 16 : 32; }

DecodePlan plan_decode(const lbca_decode_args& a) {
  DecodePlan pl{};
  if (a.dtype != LBCA_BF16) {
    pl.tile_rows = 64;
    pl.head_groups = 1;
    pl.splits = 1;
    pl.ws_bytes = 0;
    return pl;
  }
  const int64_t G = a.q_heads / a.kv_heads;
  pl.tile_rows = rows_per_tile(a.dim);
  pl.head_groups = (int)((G + 15) / 16);
  // Upper bound of visible rows from the buffer capacities.
  const int64_t sel_max = a.sel_idx ? a.k_sel : a.entries;
  const int64_t raw_span = a.mode == LBCA_EXCLUSIVE ? a.window + a.block - 1 : a.window;
  const int64_t raw_max = raw_span < a.raw_rows ? raw_span : a.raw_rows;
  const int64_t tiles = (sel_max + pl.tile_rows - 1) / pl.tile_rows + (raw_max + pl.tile_rows - 1) / pl.tile_rows;
  // Aim for ~4 waves per CU over 256 CUs, never more splits than tiles.
  const int64_t units = a.batch * a.kv_heads * pl.head_groups;
  int64_t splits = units > 0 ? (1024 + units - 1) / units : 1;
  if (splits > tiles) splits = tiles;
  if (splits < 1) splits = 1;
  pl.splits = (int)splits;
  const size_t wgs = (size_t)(units > 0 ? units : 1) * (size_t)splits;
  pl.ws_bytes = wgs * 16 * (size_t)a.dim * sizeof(float) + wgs * 16 * 2 * sizeof(float);
  return pl;
}

template <int D, int R>
static hipError_t launch_partial_d(const DecodeParams& p, bool shared, int rd, bool treat, dim3 g,
                                   hipStream_t s) {
  if (!treat) {
    if (shared) decode_partial_kernel<D, R, true, 0, false><<<g, 64, 0, s>>>(p);
    else decode_partial_kernel<D, R, false, 0, false><<<g, 64, 0, s>>>(p);
    return hipGetLastError();
  }
  if (!shared) return hipErrorInvalidValue;
  switch (rd) {
    case 0: decode_partial_kernel<D, R, true, 0, true><<<g, 64, 0, s>>>(p); break;
    case 64:
      if (D < 64) return hipErrorInvalidValue;
      decode_partial_kernel<D, R, true, (D >= 64 ? 64 : 0), true><<<g, 64, 0, s>>>(p);
      break;
    case 128:
      if (D < 128) return hipErrorInvalidValue;
      decode_partial_kernel<D, R, true, (D >= 128 ? 128 : 0), true><<<g, 64, 0, s>>>(p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const lbca_decode_args& a, const DecodePlan& plan, void* ws,
                         hipStream_t stream) {
  const int64_t G = a.q_heads / a.kv_heads;
  if (a.dtype != LBCA_BF16) {
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
    rp.hq = a.q_heads; rp.hkv = a.kv_heads; rp.G = G;
    rp.entries = a.entries; rp.raw_rows = a.raw_rows; rp.k_sel = a.sel_idx ? a.k_sel : 0;
    rp.m = a.block; rp.W = a.window; rp.mode = a.mode; rp.scale = a.scale;
    return launch_rows_f32(rp, a.dim, a.batch, stream);
  }
  DecodeParams p{};
  p.q = static_cast<const bf16_t*>(a.q);
  p.pk = static_cast<const bf16_t*>(a.pooled_k);
  p.pv = static_cast<const bf16_t*>(a.pooled_v);
  p.rk = static_cast<const bf16_t*>(a.raw_k);
  p.rv = static_cast<const bf16_t*>(a.raw_v);
  p.pos = a.pos; p.rpb = a.raw_pos_base; p.sel = a.sel_idx; p.sink = a.sink;
  p.out = a.out; p.lse = a.lse;
  const size_t wgs = (size_t)a.batch * a.kv_heads * plan.head_groups * plan.splits;
  p.ws_acc = static_cast<float*>(ws);
  p.ws_ml = static_cast<float*>(ws) + wgs * 16 * a.dim;
  p.hq = a.q_heads; p.hkv = a.kv_heads; p.G = G;
  p.entries = a.entries; p.raw_rows = a.raw_rows; p.k_sel = a.sel_idx ? a.k_sel : 0;
  p.m = a.block; p.W = a.window; p.mode = a.mode;
  p.splits = plan.splits; p.head_groups = plan.head_groups; p.dim = (int)a.dim;
  p.scale_log2 = a.scale * kLog2e;
  p.eps = a.rmsnorm_eps;
  p.rope_dims = a.rope_dims;
  p.log2_base = a.rope_dims > 0 ? log2((double)a.rope_base) : 0.0;
  const bool shared = a.pooled_v == nullptr;
  const bool treat = a.rmsnorm_eps >= 0.f || a.rope_dims > 0;
  const dim3 g((unsigned)wgs);
  hipError_t e;
  switch (a.dim) {
    case 64: e = launch_partial_d<64, 32>(p, shared, a.rope_dims, treat, g, stream); break;
    case 128: e = launch_partial_d<128, 32>(p, shared, a.rope_dims, treat, g, stream); break;
    case 256: e = launch_partial_d<256, 32>(p, shared, a.rope_dims, treat, g, stream); break;
    case 512: e = launch_partial_d<512, 16>(p, shared, a.rope_dims, treat, g, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  decode_merge_kernel<<<dim3((unsigned)(a.batch * a.q_heads)), 128, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace lbca
