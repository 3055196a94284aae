// Decode attention over pooled entries plus the raw window (split-K flash-decode).
//
// Method: "mSeek: learned KV-cache compression in a 3B model", "How LBCA works"
// (step 4: attend over every completed summary plus the exact local window);
// "HCA: Heavily Compressed Attention (toy implementation)" and "CSA: Compressed
// Sparse Attention (toy implementation)", "What is implemented" (shared-KV MQA,
// RMSNorm on queries and entries, partial RoPE with the -t output rotation,
// attention sink, selected entries plus the sliding window).
//
// Work unit = (sequence, KV head, group of 16 query heads).  GQA groups are
// padded to 16 heads; MQA with 64 heads is 4 units per KV head, whose
// workgroups read the same rows (L2 hits after the first).
//
// A workgroup (NW waves) owns a contiguous range of the unit's visible-row
// list (pooled or selected entries, then the raw span) cut into R-row tiles;
// wave w takes tiles w, w+NW, ... and, where registers allow, keeps the next
// tile's global loads in flight (two tile buffers used in turn) while it
// computes the current one.  Scores are computed transposed,
// S^T[row, head] = K[row, :] . Q[head, :], with v_mfma_f32_16x16x32_bf16 whose
// A operand is loaded straight from global memory in row-major K layout: every
// lane holds scores of one head, and the softmax max/sum need one 16-lane and
// one 32-lane swap.  P^T is already the B operand of v_mfma_f32_16x16x16_bf16
// for O^T = V^T P^T; V rows are staged row-major in a per-wave LDS tile and
// each A operand is one transposing LDS read (ds_read_b64_tr_b16).
//
// Small decodes are bound by each wave's instruction chain, not by bytes, so
// the per-tile path is kept short: raw v_exp_f32, lane swaps instead of LDS
// permutes, the accumulator rescale skipped when no running max moved, 32-bit
// index arithmetic, and a single-barrier merge of the waves.  With one split
// the workgroup finishes its heads (sink, normalisation, -t rotation, LSE);
// with several, each workgroup writes an unnormalised partial (acc, max, sum)
// and decode_merge_kernel combines them in a fixed order (bitwise
// reproducible).  No device-scope fence is used anywhere: on this multi-XCD
// part a device-scope release/acquire writes back and invalidates the XCD's L2.
#include "device_util.h"
#include "lbca_internal.h"

#ifndef LBCA_DECODE_TARGET_WAVES
#define LBCA_DECODE_TARGET_WAVES 1024  // waves a decode launch aims for (256 CUs x 4 SIMDs)
#endif

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
  float* ws_acc;   // [units * splits][16][D]
  int64_t hq, hkv, G, entries, raw_rows, k_sel, m, W;
  int mode, splits, head_groups;
  float scale_log2;
  float eps;
  int rope_dims;
  double log2_base;
};

struct SeqView {
  int64_t t, raw_begin, raw_row0;
  int n_pooled, n_sel, n_raw;
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
  v.n_pooled = (int)np;
  v.n_sel = ok ? (int)(p.sel ? p.k_sel : np) : 0;
  v.n_raw = ok ? (int)(v.t - rb + 1) : 0;
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

// A wave reads back LDS its own lanes wrote: order the accesses at wave scope.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// HCA/CSA treatment of one row held in MFMA operand layout: lane (., kq) holds
// dims 32*s + 8*kq + i of the row (s < D/32, i < 8); the 4 lanes of a row are
// lane, lane^16, lane^32, lane^48.  RMSNorm over all D dims, then RoPE on the
// last RD dims (rotate-half pairs (k, k+RD/2) sit in the same lane, RD/64 steps
// apart).  Every lane of the wave must call this (it uses lane swaps).
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
    ss = xor16_sum(ss);
    ss = xor32_sum(ss);
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
  if constexpr (RD > 0) {
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

template <int D, int R, bool SHARED>
struct Tile {
  uint4 k[R / 16][D / 32];
  uint4 v[SHARED ? 1 : R / 16][SHARED ? 1 : D / 32];
  unsigned valid[R / 16];
};

// Issue the global loads of one tile (rows beyond the list or unusable
// selected ids are zero and marked invalid).
template <int D, int R, bool SHARED>
__device__ __forceinline__ void load_tile(Tile<D, R, SHARED>& T, const DecodeParams& p,
                                          const SeqView& sv, int64_t b, int64_t kv_pool,
                                          int64_t kv_raw, int tiles_p, int tile, int n, int kq) {
  constexpr int KS = D / 32, NH = R / 16;
  const bool is_raw = tile >= tiles_p;
  const int v0 = is_raw ? (tile - tiles_p) * R : tile * R;
  const int count = is_raw ? sv.n_raw : sv.n_sel;
  // base addresses selected as integers (a pointer select from the argument
  // block otherwise becomes a private-memory lookup)
  const uintptr_t kbase = is_raw ? reinterpret_cast<uintptr_t>(p.rk) : reinterpret_cast<uintptr_t>(p.pk);
  const uintptr_t vbase = is_raw ? reinterpret_cast<uintptr_t>(p.rv) : reinterpret_cast<uintptr_t>(p.pv);
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int v = v0 + 16 * h + n;
    bool ok = v < count;
    int64_t row;
    if (is_raw) {
      row = kv_raw + v;
    } else {
      int64_t e = v;
      if (p.sel) e = ok ? (int64_t)p.sel[b * p.k_sel + v] : -1;
      ok = ok && e >= 0 && e < sv.n_pooled;
      row = kv_pool + e;
    }
    const bf16_t* kp = reinterpret_cast<const bf16_t*>(kbase) + row * D + 8 * kq;
    if (ok) {
#pragma unroll
      for (int s = 0; s < KS; ++s) T.k[h][s] = *reinterpret_cast<const uint4*>(kp + 32 * s);
      if constexpr (!SHARED) {
        const bf16_t* vp = reinterpret_cast<const bf16_t*>(vbase) + row * D + 8 * kq;
#pragma unroll
        for (int s = 0; s < KS; ++s) T.v[h][s] = *reinterpret_cast<const uint4*>(vp + 32 * s);
      }
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        T.k[h][s] = make_uint4(0, 0, 0, 0);
        if constexpr (!SHARED) T.v[h][s] = make_uint4(0, 0, 0, 0);
      }
    }
    T.valid[h] = (unsigned)(__ballot(ok) & 0xffffull);
  }
}

template <int D, int R, int NW, bool SHARED, int RD, bool TREAT>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeParams p) {
  constexpr int KS = D / 32, NH = R / 16, DT = D / 16, PITCH = D + 16;
  constexpr int STAGE = R * PITCH;                   // bf16 elements of one wave's value stage
  constexpr bool PREFETCH = D <= 128;                // second tile buffer fits in registers
  constexpr bool PAR_MERGE = NW * 16 * D * 4 <= NW * STAGE * 2;
  static_assert(NW * STAGE * 2 >= 16 * D * 4, "merge buffer must fit in the stages");
  __shared__ __attribute__((aligned(16))) bf16_t lds[NW * STAGE];
  __shared__ float s_ml[NW][16][2];
  __shared__ float s_w[NW][16];
  __shared__ float s_M[16], s_L[16], s_inv[16], s_lse[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kq = lane >> 4;
  const int split = blockIdx.x;
  const int hg = (int)(blockIdx.y % (unsigned)p.head_groups);
  const int64_t kvh = blockIdx.y / (unsigned)p.head_groups;
  const int64_t b = blockIdx.z;
  const int64_t unit = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int slot0 = hg * 16;
  const int nvalid = (int)(p.G - slot0 < 16 ? p.G - slot0 : 16);
  const int64_t head0 = kvh * p.G + slot0;  // first query head of the unit
  const bool head_ok = n < nvalid;

  // queries of this head group as B operands (zero for padded heads); their
  // addresses do not depend on the position, so they load alongside it
  uint4 qr[KS];
  {
    const bf16_t* qrow = p.q + (b * p.hq + head0 + n) * D + 8 * kq;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qr[s] = head_ok ? *reinterpret_cast<const uint4*>(qrow + 32 * s) : make_uint4(0, 0, 0, 0);
  }
  const SeqView sv = seq_view(p, b);
  if (!sv.ok) {  // rows do not fit the buffers: NaN, written once per unit
    if (split == 0) {
      for (int i = tid; i < nvalid * D; i += blockDim.x)
        p.out[(b * p.hq + head0 + i / D) * D + i % D] = __builtin_nanf("");
      if (p.lse && tid < nvalid) p.lse[b * p.hq + head0 + tid] = __builtin_nanf("");
    }
    return;
  }
  if constexpr (TREAT) treat_row<D, RD>(qr, (double)sv.t, head_ok, p.eps, p.log2_base);

  const int tiles_p = (sv.n_sel + R - 1) / R;
  const int tiles_total = tiles_p + (sv.n_raw + R - 1) / R;
  const int per = (tiles_total + p.splits - 1) / p.splits;
  const int t0 = split * per;
  const int t1 = t0 + per < tiles_total ? t0 + per : tiles_total;
  const int64_t kv_pool = (b * p.hkv + kvh) * p.entries;
  const int64_t kv_raw = (b * p.hkv + kvh) * p.raw_rows + sv.raw_row0;

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16_t* vt = lds + wave * STAGE;
  // transposing-read base of this lane: row 4*kq + n/4, column 4*(n%4)
  const bf16_t* trb = vt + (4 * kq + (n >> 2)) * PITCH + 4 * (n & 3);

  auto process = [&](Tile<D, R, SHARED>& T, int tile) {
    if constexpr (TREAT) {
      if (tile >= tiles_p) {
        const int v0 = (tile - tiles_p) * R;
#pragma unroll
        for (int h = 0; h < NH; ++h)
          treat_row<D, RD>(T.k[h], (double)(sv.raw_begin + v0 + 16 * h + n), (T.valid[h] >> n) & 1u,
                           p.eps, p.log2_base);
      }
    }
    // value rows to this wave's LDS stage (row-major)
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        *reinterpret_cast<uint4*>(&vt[(16 * h + n) * PITCH + 32 * s + 8 * kq]) =
            SHARED ? T.k[h][s] : T.v[h][s];
    // S^T = K Q^T, 16 rows x 16 heads per half
    float sc[NH][4];
    float tmax = kNegInf;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, T.k[h][s]),
                                                     __builtin_bit_cast(bf16x8, qr[s]), c, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool vok = (T.valid[h] >> (4 * kq + j)) & 1u;
        sc[h][j] = vok ? c[j] * p.scale_log2 : kNegInf;
        tmax = fmaxf(tmax, sc[h][j]);
      }
    }
    tmax = xor16_max(tmax);
    tmax = xor32_max(tmax);
    const float nm = fmaxf(m_run, tmax);
    const float mu = nm == kNegInf ? 0.f : nm;
    const float corr = fast_exp2(m_run - mu);
    float psum = 0.f;
    s16x4 pop[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float pj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pj[j] = fast_exp2(sc[h][j] - mu);
        psum += pj[j];
      }
      const uint32_t w0 = pack_bf16x2(pj[0], pj[1]), w1 = pack_bf16x2(pj[2], pj[3]);
      pop[h] = s16x4{(short)(w0 & 0xffff), (short)(w0 >> 16), (short)(w1 & 0xffff), (short)(w1 >> 16)};
    }
    l_run = fmaf(l_run, corr, psum);
    if (__ballot(corr != 1.f)) {  // some head's running max moved
#pragma unroll
      for (int t = 0; t < DT; ++t) acc[t] *= corr;
    }
    m_run = nm;
    wave_lds_sync();
    // O^T += V^T P^T.  With two 16-row halves the k=32 MFMA takes this lane's 8
    // probabilities (rows 4kq+j of both halves) as its B operand and two
    // transposing reads (the same rows of one dim) as its A operand.
    if constexpr (NH == 2) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(
          (uint16_t)pop[0][0] | ((uint32_t)(uint16_t)pop[0][1] << 16),
          (uint16_t)pop[0][2] | ((uint32_t)(uint16_t)pop[0][3] << 16),
          (uint16_t)pop[1][0] | ((uint32_t)(uint16_t)pop[1][1] << 16),
          (uint16_t)pop[1][2] | ((uint32_t)(uint16_t)pop[1][3] << 16)));
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const s16x4 a0 = lds_read_tr16(trb + 16 * t), a1 = lds_read_tr16(trb + 16 * PITCH + 16 * t);
        const bf16x8 a = __builtin_bit_cast(bf16x8, s16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[t], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int t = 0; t < DT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_read_tr16(trb + 16 * h * PITCH + 16 * t),
                                                              pop[h], acc[t], 0, 0, 0);
    }
  };

  int tile = t0 + wave;
  if constexpr (PREFETCH) {
    if (tile < t1) {
      Tile<D, R, SHARED> ta, tb;
      load_tile<D, R, SHARED>(ta, p, sv, b, kv_pool, kv_raw, tiles_p, tile, n, kq);
      while (true) {  // two buffers used in turn: no register copies between tiles
        int nt = tile + NW;
        if (nt < t1) load_tile<D, R, SHARED>(tb, p, sv, b, kv_pool, kv_raw, tiles_p, nt, n, kq);
        process(ta, tile);
        if (nt >= t1) break;
        tile = nt;
        nt = tile + NW;
        if (nt < t1) load_tile<D, R, SHARED>(ta, p, sv, b, kv_pool, kv_raw, tiles_p, nt, n, kq);
        process(tb, tile);
        if (nt >= t1) break;
        tile = nt;
      }
    }
  } else {
    Tile<D, R, SHARED> tt;
    for (; tile < t1; tile += NW) {
      load_tile<D, R, SHARED>(tt, p, sv, b, kv_pool, kv_raw, tiles_p, tile, n, kq);
      process(tt, tile);
    }
  }
  l_run = xor16_sum(l_run);
  l_run = xor32_sum(l_run);

  // ---- merge the NW waves (fixed order) ----
  if (kq == 0) {
    s_ml[wave][n][0] = m_run;
    s_ml[wave][n][1] = l_run;
  }
  __syncthreads();  // every wave is done with its stage: the LDS is free
  if (tid < 16) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_ml[w][tid][0]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sw = s_ml[w][tid][0] == kNegInf ? 0.f : fast_exp2(s_ml[w][tid][0] - M);
      s_w[w][tid] = sw;
      L = fmaf(s_ml[w][tid][1], sw, L);
    }
    s_M[tid] = M;
    s_L[tid] = L;
  }
  __syncthreads();
  float* buf = reinterpret_cast<float*>(lds);
  if constexpr (PAR_MERGE) {  // every wave writes its scaled acc to its own slice
    if (head_ok) {
      const float sw = s_w[wave][n];
      float* dst = buf + (wave * 16 + n) * D + 4 * kq;
#pragma unroll
      for (int t = 0; t < DT; ++t)
        *reinterpret_cast<float4*>(dst + 16 * t) =
            make_float4(acc[t][0] * sw, acc[t][1] * sw, acc[t][2] * sw, acc[t][3] * sw);
    }
    __syncthreads();
  } else {  // accumulate into one buffer, wave after wave
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (wave == w && head_ok) {
        const float sw = s_w[w][n];
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          float4* dst = reinterpret_cast<float4*>(&buf[n * D + 16 * t + 4 * kq]);
          float4 v = make_float4(acc[t][0] * sw, acc[t][1] * sw, acc[t][2] * sw, acc[t][3] * sw);
          if (w > 0) {
            const float4 o = *dst;
            v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
          }
          *dst = v;
        }
      }
      __syncthreads();
    }
  }
  auto merged = [&](int sl, int d) {  // combined unnormalised acc of slot sl, dim d
    if constexpr (PAR_MERGE) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) o += buf[(w * 16 + sl) * D + d];
      return o;
    } else {
      return buf[sl * D + d];
    }
  };

  constexpr int r = RD, half = RD / 2;
  if (p.splits == 1) {
    if (tid < nvalid) {
      float L = s_L[tid];
      const float M = s_M[tid];
      if (p.sink) L += exp2f(p.sink[head0 + tid] * kLog2e - M);
      s_inv[tid] = 1.f / L;
      s_lse[tid] = (M + log2f(L)) * 0.69314718055994531f;
    }
    __syncthreads();
    const int items = nvalid * (D - half);  // plain dims, then rotate-half pairs
    for (int i = tid; i < items; i += blockDim.x) {
      const int sl = i / (D - half), d = i % (D - half);
      float* o = p.out + (b * p.hq + head0 + sl) * D;
      const float inv = s_inv[sl];
      if (d < D - r) {
        o[d] = merged(sl, d) * inv;
      } else if constexpr (RD > 0) {
        const int k = d - (D - r);
        const float x1 = merged(sl, d) * inv, x2 = merged(sl, d + half) * inv;
        float c, sn;
        rope_cos_sin(-(double)sv.t, k, r, p.log2_base, &c, &sn);
        o[d] = x1 * c - x2 * sn;
        o[d + half] = x2 * c + x1 * sn;
      }
    }
    if (p.lse && tid < nvalid) p.lse[b * p.hq + head0 + tid] = s_lse[tid];
    return;
  }
  // ---- split partial to the workspace; decode_merge_kernel combines the splits ----
  const int64_t part = unit * p.splits + split;
  for (int i = tid; i < nvalid * D; i += blockDim.x)
    p.ws_acc[(part * 16) * D + i] = merged(i / D, i % D);
  if (tid < nvalid) {
    p.ws_ml[(part * 16 + tid) * 2] = s_M[tid];
    p.ws_ml[(part * 16 + tid) * 2 + 1] = s_L[tid];
  }
}

// Combine the splits of one unit (16 query-head slots): every split's partial
// is loaded at once (no dependent chain), weights exp2(m_s - M) in a fixed
// order, then sink, normalisation, LSE and the -t rotation.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p, int D) {
  __shared__ float s_m[64][16], s_l[64][16];
  __shared__ float s_w[64][16];
  __shared__ float s_inv[16], s_lse[16];
  const int tid = threadIdx.x;
  const int64_t unit = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int hg = (int)(blockIdx.x % (unsigned)p.head_groups);
  const int64_t kvh = blockIdx.x / (unsigned)p.head_groups;
  const int64_t b = blockIdx.y;
  const int slot0 = hg * 16;
  const int nvalid = (int)(p.G - slot0 < 16 ? p.G - slot0 : 16);
  const int64_t head0 = kvh * p.G + slot0;
  const SeqView sv = seq_view(p, b);
  if (!sv.ok) return;  // the decode kernel already wrote NaN for this unit
  const int S = p.splits;
  const int64_t part0 = unit * S;
  for (int i = tid; i < S * 16; i += blockDim.x) {
    const int s = i >> 4, slot = i & 15;
    if (slot < nvalid) {
      s_m[s][slot] = p.ws_ml[((part0 + s) * 16 + slot) * 2];
      s_l[s][slot] = p.ws_ml[((part0 + s) * 16 + slot) * 2 + 1];
    }
  }
  __syncthreads();
  if (tid < nvalid) {
    float M = kNegInf;
    for (int s = 0; s < S; ++s) M = fmaxf(M, s_m[s][tid]);
    float L = 0.f;
    for (int s = 0; s < S; ++s) {
      const float sw = s_m[s][tid] == kNegInf ? 0.f : exp2f(s_m[s][tid] - M);
      s_w[s][tid] = sw;
      L = fmaf(s_l[s][tid], sw, L);
    }
    if (p.sink) L += exp2f(p.sink[head0 + tid] * kLog2e - M);
    s_inv[tid] = 1.f / L;
    s_lse[tid] = (M + log2f(L)) * 0.69314718055994531f;
  }
  __syncthreads();
  const float* pa = p.ws_acc + part0 * 16 * D;
  auto combined = [&](int sl, int d) {
    float o = 0.f;
#pragma unroll 8
    for (int s = 0; s < S; ++s) o = fmaf(pa[(s * 16 + sl) * D + d], s_w[s][sl], o);
    return o * s_inv[sl];
  };
  const int r = p.rope_dims, half = r >> 1;
  const int items = nvalid * (D - half);
  for (int i = tid; i < items; i += blockDim.x) {
    const int sl = i / (D - half), d = i % (D - half);
    float* o = p.out + (b * p.hq + head0 + sl) * D;
    if (d < D - r) {
      o[d] = combined(sl, d);
    } else {
      const int k = d - (D - r);
      const float x1 = combined(sl, d), x2 = combined(sl, d + half);
      float c, sn;
      rope_cos_sin(-(double)sv.t, k, r, p.log2_base, &c, &sn);
      o[d] = x1 * c - x2 * sn;
      o[d + half] = x2 * c + x1 * sn;
    }
  }
  if (p.lse && tid < nvalid) p.lse[b * p.hq + head0 + tid] = s_lse[tid];
}

// ---------------------------------------------------------------------------
static int rows_per_tile(int64_t dim) { return dim >= 512 ? 16 : 32; }
static int waves_per_wg(int64_t dim) { return dim <= 128 ? 8 : 4; }

DecodePlan plan_decode(const lbca_decode_args& a) {
  DecodePlan pl{};
  if (a.dtype != LBCA_BF16) return pl;  // fp32 path needs no workspace
  const int64_t G = a.q_heads / a.kv_heads;
  pl.tile_rows = rows_per_tile(a.dim);
  pl.head_groups = (int)((G + 15) / 16);
  const int nw = waves_per_wg(a.dim);
  // upper bound of the visible-row list from the buffer capacities
  const int64_t sel_max = a.sel_idx ? a.k_sel : a.entries;
  const int64_t raw_span = a.mode == LBCA_EXCLUSIVE ? a.window + a.block - 1 : a.window;
  const int64_t raw_max = raw_span < a.raw_rows ? raw_span : a.raw_rows;
  const int64_t rows = sel_max + raw_max;
  const int64_t tiles = (sel_max + pl.tile_rows - 1) / pl.tile_rows + (raw_max + pl.tile_rows - 1) / pl.tile_rows;
  const int64_t units = a.batch * a.kv_heads * pl.head_groups;
  // waves per unit: enough for ~LBCA_DECODE_TARGET_WAVES in total, never more
  // than there are tiles; split partials (16 heads x dim fp32 per workgroup, for
  // every head group of a KV head) kept under a quarter of the K/V bytes.
  int64_t wpu = units > 0 ? (LBCA_DECODE_TARGET_WAVES + units - 1) / units : 1;
  if (wpu > tiles) wpu = tiles;
  int64_t s = (wpu + nw - 1) / nw;
  const int64_t kv_bytes = rows * a.dim * 2 * (a.pooled_v ? 2 : 1);
  const int64_t part_bytes = (int64_t)pl.head_groups * 16 * (a.dim + 2) * 4;
  const int64_t by_traffic = kv_bytes / (4 * part_bytes) > 0 ? kv_bytes / (4 * part_bytes) : 1;
  if (s > by_traffic) s = by_traffic;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  pl.splits = (int)s;
  if (s == 1) return pl;
  const size_t u = (size_t)units;
  pl.ws_bytes = u * s * 16 * 2 * sizeof(float) + u * s * 16 * (size_t)a.dim * sizeof(float);
  return pl;
}

template <int D, int R, int NW>
static hipError_t launch_d(const DecodeParams& p, bool shared, int rd, bool treat, dim3 g,
                           hipStream_t s) {
  const dim3 blk(NW * 64);
  if (!treat) {
    if (shared) decode_kernel<D, R, NW, true, 0, false><<<g, blk, 0, s>>>(p);
    else decode_kernel<D, R, NW, false, 0, false><<<g, blk, 0, s>>>(p);
    return hipGetLastError();
  }
  if (!shared) return hipErrorInvalidValue;
  switch (rd) {
    case 0: decode_kernel<D, R, NW, true, 0, true><<<g, blk, 0, s>>>(p); break;
    case 64:
      if constexpr (D >= 64) decode_kernel<D, R, NW, true, 64, true><<<g, blk, 0, s>>>(p);
      break;
    case 128:
      if constexpr (D >= 128) decode_kernel<D, R, NW, true, 128, true><<<g, blk, 0, s>>>(p);
      else return hipErrorInvalidValue;
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const lbca_decode_args& a, const DecodePlan& plan, void* ws,
                         hipStream_t stream) {
  if (a.dtype != LBCA_BF16) return launch_decode_f32(a, stream);
  const int64_t G = a.q_heads / a.kv_heads;
  DecodeParams p{};
  p.q = static_cast<const bf16_t*>(a.q);
  p.pk = static_cast<const bf16_t*>(a.pooled_k);
  p.pv = static_cast<const bf16_t*>(a.pooled_v);
  p.rk = static_cast<const bf16_t*>(a.raw_k);
  p.rv = static_cast<const bf16_t*>(a.raw_v);
  p.pos = a.pos; p.rpb = a.raw_pos_base; p.sel = a.sel_idx; p.sink = a.sink;
  p.out = a.out; p.lse = a.lse;
  const size_t units = (size_t)a.batch * a.kv_heads * plan.head_groups;
  if (plan.splits > 1) {
    p.ws_ml = static_cast<float*>(ws);
    p.ws_acc = p.ws_ml + units * plan.splits * 16 * 2;
  }
  p.hq = a.q_heads; p.hkv = a.kv_heads; p.G = G;
  p.entries = a.entries; p.raw_rows = a.raw_rows; p.k_sel = a.sel_idx ? a.k_sel : 0;
  p.m = a.block; p.W = a.window; p.mode = a.mode;
  p.splits = plan.splits; p.head_groups = plan.head_groups;
  p.scale_log2 = a.scale * kLog2e;
  p.eps = a.rmsnorm_eps;
  p.rope_dims = a.rope_dims;
  p.log2_base = a.rope_dims > 0 ? log2((double)a.rope_base) : 0.0;
  const bool shared = a.pooled_v == nullptr;
  const bool treat = a.rmsnorm_eps >= 0.f || a.rope_dims > 0;
  const dim3 g((unsigned)plan.splits, (unsigned)(a.kv_heads * plan.head_groups), (unsigned)a.batch);
  hipError_t e;
  switch (a.dim) {
    case 64: e = launch_d<64, 32, 8>(p, shared, a.rope_dims, treat, g, stream); break;
    case 128: e = launch_d<128, 32, 8>(p, shared, a.rope_dims, treat, g, stream); break;
    case 256: e = launch_d<256, 32, 4>(p, shared, a.rope_dims, treat, g, stream); break;
    case 512: e = launch_d<512, 16, 4>(p, shared, a.rope_dims, treat, g, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || plan.splits == 1) return e;
  decode_merge_kernel<<<dim3((unsigned)(a.kv_heads * plan.head_groups), (unsigned)a.batch), 256, 0,
                        stream>>>(p, (int)a.dim);
  return hipGetLastError();
}

}  // namespace lbca
