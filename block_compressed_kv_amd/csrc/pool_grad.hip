// Gradients of single-series block pooling (key, value, logit and bias rows).
//
// Method: "mSeek: learned KV-cache compression in a 3B model", section "How LBCA
// works" (steps 2-3: per channel, w = softmax over the block's tokens of
// z + bias, entry = sum w x).  The chain rule through that definition gives,
// for token s of block j with upstream gradient rows g (key) and gv (value):
//   dx[s] = w[s] g,   dv[s] = w[s] gv,
//   dz[s] = w[s] (g (x[s] - entry_x) + gv (v[s] - entry_v)),
//   dbias[h, s - j m] = dz[s] summed over sequences and blocks.
//
// Design: one 256-thread workgroup per (head, chunk of consecutive blocks of
// that head's (sequence, block) list), so every block of a workgroup shares
// the bias rows, staged once in LDS.  L = dim/8 lanes cover a token row (8
// channels per lane, 16-byte vectors); the 256/L lane groups take token
// phases, at most four tokens per lane, held in registers as loaded, and the
// next block's rows are requested while the current one is worked.  Per block
// each lane's online-softmax state (channel max, weight sum, weighted key and
// value sums) is merged over the phases in a fixed order (lane exchanges
// inside a wave, the four waves' states through LDS), so the entry is
// recomputed in fp32 (not read back rounded), and each lane writes its
// tokens' gradients and adds their logit gradients to its bias partial.  Workgroup partials of the bias gradient go
// to the workspace; a second kernel sums them per (head, offset, channel) in
// chunk order, so every output is bitwise reproducible.  HBM-bound: per token
// channel it reads x, v, z and writes dx, dv, dz once.
#include "lbca_internal.h"
#include "device_util.h"

namespace lbca {

struct PoolGradParams {
  const void* x;
  const void* v;
  const void* z;
  const float* bias;
  const void* gx;
  const void* gv;
  void* dx;
  void* dv;
  void* dz;
  float* dbias;
  const void* xb;  // dual (CSA) mode: the b-series and its outputs
  const void* zb;
  const float* bias_b;
  void* dxb;
  void* dzb;
  float* dbias_b;
  float* part;  // [heads][chunks][M2][dim] bias-gradient partials (M2 = m, or 2m in dual mode)
  float eps;    // treatment of the entry (shared series): < 0 no RMSNorm
  int rope_dims;
  double log2_base;
  int64_t batch, heads, tokens, dim, m, entries, block_begin, n_blocks, pos_base;
  int chunks, per_chunk;  // workgroups per head, blocks per workgroup
  int log2_lanes;
  // element strides {sequence, head, row}: token rows and their gradients, entry gradients
  Str x_st, v_st, z_st, xb_st, zb_st, dx_st, dv_st, dz_st, dxb_st, dzb_st, gx_st, gv_st;
};

constexpr int kGradNT = 256;  // threads per workgroup (4 waves)
constexpr int kGradNW = kGradNT / 64;
constexpr int kGradTPL = 4;    // tokens per lane at most: m * dim <= kGradNT * 8 * kGradTPL = 8192

// Raw rows of one block for this lane: up to kGradTPL tokens of 8 channels,
// kept packed as loaded (16-byte vectors) so that the next block's loads can
// be in flight while the current block is worked.
template <typename TX, typename TZ, bool HAS_V>
struct BlockRows {
  static constexpr int NX = (int)(sizeof(TX) * 8 / 16), NZ = (int)(sizeof(TZ) * 8 / 16);
  uint4 x[kGradTPL][NX], v[kGradTPL][HAS_V ? NX : 1], z[kGradTPL][NZ];
  // token slot k's rows at xp[k], vp[k], zp[k]
  __device__ __forceinline__ void load(const TX* const* xp, const TX* const* vp, const TZ* const* zp,
                                       const bool* present) {
#pragma unroll
    for (int k = 0; k < kGradTPL; ++k) {
      if (!present[k]) continue;
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        x[k][i] = reinterpret_cast<const uint4*>(xp[k])[i];
        if constexpr (HAS_V) v[k][i] = reinterpret_cast<const uint4*>(vp[k])[i];
      }
#pragma unroll
      for (int i = 0; i < NZ; ++i) z[k][i] = reinterpret_cast<const uint4*>(zp[k])[i];
    }
  }
};

template <typename T, int N>
__device__ __forceinline__ void unpack_row(const uint4 (&u)[N], float* f) {
  if constexpr (sizeof(T) == 2) {
    f[0] = lo_bf16(u[0].x); f[1] = hi_bf16(u[0].x); f[2] = lo_bf16(u[0].y); f[3] = hi_bf16(u[0].y);
    f[4] = lo_bf16(u[0].z); f[5] = hi_bf16(u[0].z); f[6] = lo_bf16(u[0].w); f[7] = hi_bf16(u[0].w);
  } else {
    f[0] = __uint_as_float(u[0].x); f[1] = __uint_as_float(u[0].y);
    f[2] = __uint_as_float(u[0].z); f[3] = __uint_as_float(u[0].w);
    f[4] = __uint_as_float(u[1].x); f[5] = __uint_as_float(u[1].y);
    f[6] = __uint_as_float(u[1].z); f[7] = __uint_as_float(u[1].w);
  }
}

// Per channel online-softmax state of a set of tokens: max mx, sum l of
// 2^(a - mx), and the 2^(a - mx)-weighted sums of keys and values.
struct GradState {
  float mx[8], l[8], sx[8], sv[8];
};

// Combines `lo` (the lower phases) and `hi` into `lo` (two empty states stay empty).
__device__ __forceinline__ void combine_state(GradState& lo, const GradState& hi) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float nm = fmaxf(lo.mx[c], hi.mx[c]);
    const bool none = nm == kNegInf;
    const float a = none ? 0.f : fast_exp2(lo.mx[c] - nm), b = none ? 0.f : fast_exp2(hi.mx[c] - nm);
    lo.l[c] = lo.l[c] * a + hi.l[c] * b;
    lo.sx[c] = lo.sx[c] * a + hi.sx[c] * b;
    lo.sv[c] = lo.sv[c] * a + hi.sv[c] * b;
    lo.mx[c] = nm;
  }
}

// Merges the states of every phase of the block into every lane, in a fixed
// order: lane exchanges inside a wave (lanes lane ^ L, ^2L, ..), then the
// waves' states through LDS, read and combined in wave order by every lane
// (a workgroup of eight waves, two tokens per lane, measured slower: 4.0
// against 3.0 ms for a 32K history at batch 16).
// Called by every thread of the workgroup.
__device__ __forceinline__ void merge_phases(GradState& st, float (*red)[64][32], int L, int li) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = L; off < 64; off <<= 1) {
    GradState lo, hi;
    if (off == 16 || off == 32) {
      // a swap of a register with itself: lower row's (half's) value first on both lanes
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float* src[4] = {&st.mx[c], &st.l[c], &st.sx[c], &st.sv[c]};
        float* dl[4] = {&lo.mx[c], &lo.l[c], &lo.sx[c], &lo.sv[c]};
        float* dh[4] = {&hi.mx[c], &hi.l[c], &hi.sx[c], &hi.sv[c]};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t u = __float_as_uint(*src[q]);
          const auto r = off == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                                   : __builtin_amdgcn_permlane32_swap(u, u, false, false);
          *dl[q] = __uint_as_float(r[0]);
          *dh[q] = __uint_as_float(r[1]);
        }
      }
    } else {
      const bool lower = (lane & off) == 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float om = __shfl_xor(st.mx[c], off, 64), ol = __shfl_xor(st.l[c], off, 64);
        const float ox = __shfl_xor(st.sx[c], off, 64), ov = __shfl_xor(st.sv[c], off, 64);
        lo.mx[c] = lower ? st.mx[c] : om; hi.mx[c] = lower ? om : st.mx[c];
        lo.l[c] = lower ? st.l[c] : ol;   hi.l[c] = lower ? ol : st.l[c];
        lo.sx[c] = lower ? st.sx[c] : ox; hi.sx[c] = lower ? ox : st.sx[c];
        lo.sv[c] = lower ? st.sv[c] : ov; hi.sv[c] = lower ? ov : st.sv[c];
      }
    }
    combine_state(lo, hi);
    st = lo;
  }
  if (lane < L) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      red[wave][li][c] = st.mx[c];
      red[wave][li][8 + c] = st.l[c];
      red[wave][li][16 + c] = st.sx[c];
      red[wave][li][24 + c] = st.sv[c];
    }
  }
  __syncthreads();
  GradState acc;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    acc.mx[c] = red[0][li][c];
    acc.l[c] = red[0][li][8 + c];
    acc.sx[c] = red[0][li][16 + c];
    acc.sv[c] = red[0][li][24 + c];
  }
#pragma unroll
  for (int w = 1; w < kGradNW; ++w) {
    GradState t;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      t.mx[c] = red[w][li][c];
      t.l[c] = red[w][li][8 + c];
      t.sx[c] = red[w][li][16 + c];
      t.sv[c] = red[w][li][24 + c];
    }
    combine_state(acc, t);
  }
  __syncthreads();  // `red` free for the next block
  st = acc;
}

// The gradient of the treated entry y = rope(rmsnorm(e)) with respect to e,
// for this lane's channels c0.. of a row held by the L lanes of a group
// (every group holds the same row): the rotation back by the entry's angle
// (partner dims k + r/2 sit r/16 lanes away; freq[k]: turns per position of
// pair k, an LDS table), then the RMSNorm gradient
// (g - u mean(g u)) / r with row sums over the group.  Every lane calls it.
__device__ __forceinline__ void treat_grad(float (&g)[8], const float (&e)[8], int L, int64_t c0, int64_t dim,
                                           double block_pos, float eps, int rope_dims, const double* freq) {
  const int lane = threadIdx.x & 63;
  if (rope_dims > 0) {
    const int r = rope_dims, half = r >> 1;
    const int64_t first = dim - r;
    const bool lo_half = c0 >= first && c0 < first + half;
    const bool hi_half = c0 >= first + half;
    const int src = lo_half ? lane + (half >> 3) : (hi_half ? lane - (half >> 3) : lane);
    float prt[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) prt[c] = __shfl(g[c], src, 64);
    if (lo_half || hi_half) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int k = (int)(c0 + c - first) - (hi_half ? half : 0);
        float cs, sn;
        rope_cos_sin_turns(block_pos * freq[k], &cs, &sn);
        g[c] = lo_half ? g[c] * cs + prt[c] * sn : g[c] * cs - prt[c] * sn;
      }
    }
  }
  if (eps >= 0.f) {
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) ss = fmaf(e[c], e[c], ss);
    for (int o = L >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float inv_r = 1.f / sqrtf(ss / (float)dim + eps);
    float gu = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) gu = fmaf(g[c], e[c] * inv_r, gu);
    for (int o = L >> 1; o > 0; o >>= 1) gu += __shfl_xor(gu, o, 64);
    const float mean_gu = gu / (float)dim;
#pragma unroll
    for (int c = 0; c < 8; ++c) g[c] = (g[c] - e[c] * inv_r * mean_gu) * inv_r;
  }
}

template <typename TX, typename TZ, bool HAS_V, bool TREAT, bool DUAL>
__global__ __launch_bounds__(kGradNT) void pool_grad_kernel(PoolGradParams p) {
  __shared__ float red[kGradNW][64][32];
  __shared__ __attribute__((aligned(16))) float s_bias[8192];  // bias rows of the token set, M2 * dim <= 8192
  __shared__ double s_freq[TREAT ? 256 : 1];                     // RoPE turns per position, pair k
  const int tid = threadIdx.x, lane = tid & 63;
  const int L = 1 << p.log2_lanes;
  const int li = lane & (L - 1);
  const int phase = tid >> p.log2_lanes;
  const int P = kGradNT >> p.log2_lanes;
  const int h = (int)blockIdx.y, chunk = (int)blockIdx.x;
  const int64_t dim = p.dim, m = p.m;
  const int64_t M2 = DUAL ? 2 * m : m;  // tokens of an entry's softmax: block j (and block j-1 of the b-series)
  const int64_t c0 = (int64_t)li * 8;
  const int64_t list_n = p.batch * p.n_blocks;  // (sequence, block) pairs of this head
  const int64_t k0 = (int64_t)chunk * p.per_chunk;
  const int64_t k1 = k0 + p.per_chunk < list_n ? k0 + p.per_chunk : list_n;

  // this lane's token slots: offset u = phase + P k of the token set, present when < M2;
  // slots u >= m (dual mode) are block j-1 of the b-series
  bool has[kGradTPL], is_b[kGradTPL];
  int64_t uoff[kGradTPL];  // row offset from the entry's own block start
#pragma unroll
  for (int k = 0; k < kGradTPL; ++k) {
    const int64_t u = phase + (int64_t)P * k;
    has[k] = u < M2;
    is_b[k] = DUAL && u >= m;
    uoff[k] = is_b[k] ? u - 2 * m : u;
  }
  // element offset of this lane's channels of token row r of sequence b
  auto at = [&](Str st, int64_t b, int64_t r) __attribute__((always_inline)) {
    return b * st.s0 + (int64_t)h * st.s1 + r * st.s2 + c0;
  };
  // (sequence, entry) of list item kk and the token rows of this lane's slots
  auto block_of = [&](int64_t kk, int64_t& b, int64_t& j, int64_t (&row)[kGradTPL], bool (&present)[kGradTPL]) {
    b = kk / p.n_blocks;
    j = p.block_begin + kk % p.n_blocks;
#pragma unroll
    for (int k = 0; k < kGradTPL; ++k) {
      row[k] = j * m - p.pos_base + uoff[k];
      present[k] = has[k] && !(is_b[k] && j == 0);  // entry 0 has no b-part
    }
  };
  auto load_rows = [&](BlockRows<TX, TZ, HAS_V>& br, int64_t b, const int64_t (&row)[kGradTPL],
                       const bool (&present)[kGradTPL]) __attribute__((always_inline)) {
    const TX* xp[kGradTPL];
    const TX* vp[kGradTPL];
    const TZ* zp[kGradTPL];
#pragma unroll
    for (int k = 0; k < kGradTPL; ++k) {
      xp[k] = is_b[k] ? static_cast<const TX*>(p.xb) + at(p.xb_st, b, row[k])
                      : static_cast<const TX*>(p.x) + at(p.x_st, b, row[k]);
      vp[k] = HAS_V ? static_cast<const TX*>(p.v) + at(p.v_st, b, row[k]) : nullptr;
      zp[k] = is_b[k] ? static_cast<const TZ*>(p.zb) + at(p.zb_st, b, row[k])
                      : static_cast<const TZ*>(p.z) + at(p.z_st, b, row[k]);
    }
    br.load(xp, vp, zp, present);
  };
  BlockRows<TX, TZ, HAS_V> cur;
  {
    int64_t b, j, row[kGradTPL];
    bool present[kGradTPL];
    block_of(k0, b, j, row, present);
    load_rows(cur, b, row, present);
  }
  if constexpr (TREAT) {
    if (tid < p.rope_dims / 2) s_freq[tid] = rope_turns_per_pos(tid, p.rope_dims, p.log2_base);
  }
  for (int64_t e = tid * 4; e < m * dim; e += kGradNT * 4) {
    *reinterpret_cast<float4*>(&s_bias[e]) = *reinterpret_cast<const float4*>(p.bias + h * m * dim + e);
    if constexpr (DUAL)
      *reinterpret_cast<float4*>(&s_bias[m * dim + e]) = *reinterpret_cast<const float4*>(p.bias_b + h * m * dim + e);
  }
  __syncthreads();

  float db[kGradTPL][8];
#pragma unroll
  for (int k = 0; k < kGradTPL; ++k)
#pragma unroll
    for (int c = 0; c < 8; ++c) db[k][c] = 0.f;

  for (int64_t kk = k0; kk < k1; ++kk) {
    int64_t b, j, row[kGradTPL];
    bool present[kGradTPL];
    block_of(kk, b, j, row, present);
    float g[8], gvv[8];
    load8(static_cast<const TX*>(p.gx) + at(p.gx_st, b, j), g);
    if constexpr (HAS_V) load8(static_cast<const TX*>(p.gv) + at(p.gv_st, b, j), gvv);
    // logits (log2 units) of this lane's tokens, then the next block's rows go out
    float a[kGradTPL][8];
#pragma unroll
    for (int k = 0; k < kGradTPL; ++k) {
      if (!present[k]) continue;
      float zz[8];
      unpack_row<TZ>(cur.z[k], zz);
      const float* br = &s_bias[(phase + P * k) * dim + c0];
#pragma unroll
      for (int c = 0; c < 8; ++c) a[k][c] = (zz[c] + br[c]) * kLog2e;
    }
    BlockRows<TX, TZ, HAS_V> nxt;
    if (kk + 1 < k1) {
      int64_t bn, jn, rown[kGradTPL];
      bool presn[kGradTPL];
      block_of(kk + 1, bn, jn, rown, presn);
      load_rows(nxt, bn, rown, presn);
    }
    // this lane's state, then the block's
    GradState st;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float mx = kNegInf;
#pragma unroll
      for (int k = 0; k < kGradTPL; ++k)
        if (present[k]) mx = fmaxf(mx, a[k][c]);
      st.mx[c] = mx;
      st.l[c] = st.sx[c] = st.sv[c] = 0.f;
    }
    // a[k][c] becomes the token's weight relative to this lane's maximum
#pragma unroll
    for (int k = 0; k < kGradTPL; ++k) {
      if (!present[k]) continue;
      float xs[8], vs[8];
      unpack_row<TX>(cur.x[k], xs);
      if constexpr (HAS_V) unpack_row<TX>(cur.v[k], vs);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        a[k][c] = fast_exp2(a[k][c] - st.mx[c]);
        st.l[c] += a[k][c];
        st.sx[c] = fmaf(a[k][c], xs[c], st.sx[c]);
        if constexpr (HAS_V) st.sv[c] = fmaf(a[k][c], vs[c], st.sv[c]);
      }
    }
    float lmx[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) lmx[c] = st.mx[c];
    merge_phases(st, red, L, li);
    // the block's entry, and the factor that turns a lane weight into the softmax weight
    float scale[8], ex[8], ev[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float inv = 1.f / st.l[c];
      ex[c] = st.sx[c] * inv;
      ev[c] = st.sv[c] * inv;
      scale[c] = lmx[c] == kNegInf ? 0.f : fast_exp2(lmx[c] - st.mx[c]) * inv;
    }
    // the upstream gradient of a treated entry, taken back to the pooled row
    if constexpr (TREAT) treat_grad(g, ex, L, c0, dim, (double)(j * m), p.eps, p.rope_dims, s_freq);
    // gradients of this lane's tokens
#pragma unroll
    for (int k = 0; k < kGradTPL; ++k) {
      if (!present[k]) continue;
      float xs[8], vs[8];
      unpack_row<TX>(cur.x[k], xs);
      if constexpr (HAS_V) unpack_row<TX>(cur.v[k], vs);
      float ox[8], ov[8], oz[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float w = a[k][c] * scale[c];
        ox[c] = w * g[c];
        float da = g[c] * (xs[c] - ex[c]);
        if constexpr (HAS_V) {
          ov[c] = w * gvv[c];
          da = fmaf(gvv[c], vs[c] - ev[c], da);
        }
        oz[c] = w * da;
        db[k][c] += oz[c];
      }
      store8(is_b[k] ? static_cast<TX*>(p.dxb) + at(p.dxb_st, b, row[k]) : static_cast<TX*>(p.dx) + at(p.dx_st, b, row[k]),
             ox);
      if constexpr (HAS_V) store8(static_cast<TX*>(p.dv) + at(p.dv_st, b, row[k]), ov);
      store8(is_b[k] ? static_cast<TZ*>(p.dzb) + at(p.dzb_st, b, row[k]) : static_cast<TZ*>(p.dz) + at(p.dz_st, b, row[k]),
             oz);
    }
    cur = nxt;
  }
  // this workgroup's bias-gradient partial (rows u of the token set)
  float* part = p.part + (((int64_t)h * p.chunks + chunk) * M2) * dim + c0;
#pragma unroll
  for (int k = 0; k < kGradTPL; ++k)
    if (has[k]) store8(part + (phase + (int64_t)P * k) * dim, db[k]);
}

// dbias[h, i, c] (and, in dual mode, dbias_b[h, i, c] from rows m + i) = sum
// over chunks (in order) of the partials.
__global__ __launch_bounds__(256) void pool_grad_bias_kernel(PoolGradParams p, int dual) {
  const int64_t M2 = dual ? 2 * p.m : p.m;
  const int64_t n = p.heads * M2 * p.dim;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const int64_t md = M2 * p.dim;
  const int64_t h = e / md, r = e % md;
  const float* src = p.part + h * p.chunks * md + r;
  float s = 0.f;
  for (int c = 0; c < p.chunks; ++c) s += src[(int64_t)c * md];
  const int64_t u = r / p.dim, ch = r % p.dim;
  if (u < p.m) p.dbias[(h * p.m + u) * p.dim + ch] = s;
  else p.dbias_b[(h * p.m + u - p.m) * p.dim + ch] = s;
}

// Workgroups per head: about 1024 in all, each over consecutive blocks.
static void grad_plan(const lbca_pool_grad_args& a, int* chunks, int* per_chunk) {
  const int64_t list_n = a.batch * (a.block_end - a.block_begin);
  int64_t per = (list_n * a.heads + 1023) / 1024;
  if (per < 1) per = 1;
  const int64_t ch = list_n > 0 ? (list_n + per - 1) / per : 0;
  *chunks = (int)ch;
  *per_chunk = (int)per;
}

size_t pool_grad_workspace_bytes(const lbca_pool_grad_args& a) {
  int chunks, per;
  grad_plan(a, &chunks, &per);
  const int64_t m2 = a.xb ? 2 * a.block : a.block;
  return (size_t)a.heads * (size_t)chunks * (size_t)(m2 * a.dim) * sizeof(float);
}

template <typename TX, typename TZ>
static void launch_grad_typed(const PoolGradParams& p, bool has_v, bool treat, bool dual, dim3 grid, hipStream_t s) {
  if (has_v) pool_grad_kernel<TX, TZ, true, false, false><<<grid, kGradNT, 0, s>>>(p);
  else if (dual && treat) pool_grad_kernel<TX, TZ, false, true, true><<<grid, kGradNT, 0, s>>>(p);
  else if (dual) pool_grad_kernel<TX, TZ, false, false, true><<<grid, kGradNT, 0, s>>>(p);
  else if (treat) pool_grad_kernel<TX, TZ, false, true, false><<<grid, kGradNT, 0, s>>>(p);
  else pool_grad_kernel<TX, TZ, false, false, false><<<grid, kGradNT, 0, s>>>(p);
}

hipError_t launch_pool_grad(const lbca_pool_grad_args& a, void* ws, hipStream_t stream) {
  PoolGradParams p;
  p.x = a.x; p.v = a.v; p.z = a.z; p.bias = a.bias; p.gx = a.grad_x; p.gv = a.grad_v;
  p.dx = a.dx; p.dv = a.dv; p.dz = a.dz; p.dbias = a.dbias; p.part = static_cast<float*>(ws);
  p.xb = a.xb; p.zb = a.zb; p.bias_b = a.bias_b; p.dxb = a.dxb; p.dzb = a.dzb; p.dbias_b = a.dbias_b;
  p.eps = a.rmsnorm_eps; p.rope_dims = a.rope_dims;
  p.log2_base = a.rope_dims > 0 ? log2((double)a.rope_base) : 0.0;
  p.batch = a.batch; p.heads = a.heads; p.tokens = a.tokens; p.dim = a.dim; p.m = a.block;
  p.entries = a.entries; p.block_begin = a.block_begin; p.n_blocks = a.block_end - a.block_begin;
  p.pos_base = a.pos_base;
  p.x_st = a.x_st; p.v_st = a.v_st; p.z_st = a.z_st; p.xb_st = a.xb_st; p.zb_st = a.zb_st;
  p.dx_st = a.dx_st; p.dv_st = a.dv_st; p.dz_st = a.dz_st; p.dxb_st = a.dxb_st; p.dzb_st = a.dzb_st;
  p.gx_st = a.grad_x_st; p.gv_st = a.grad_v_st;
  grad_plan(a, &p.chunks, &p.per_chunk);
  p.log2_lanes = __builtin_ctz((unsigned)(a.dim / 8));
  const bool dual = a.xb != nullptr;
  const bool treat = a.rmsnorm_eps >= 0.f || a.rope_dims > 0;
  if (p.chunks > 0) {
    const dim3 grid((unsigned)p.chunks, (unsigned)a.heads);
    const bool has_v = a.v != nullptr;
    if (a.x_dtype == LBCA_BF16) {
      if (a.z_dtype == LBCA_BF16) launch_grad_typed<bf16_t, bf16_t>(p, has_v, treat, dual, grid, stream);
      else launch_grad_typed<bf16_t, float>(p, has_v, treat, dual, grid, stream);
    } else {
      if (a.z_dtype == LBCA_BF16) launch_grad_typed<float, bf16_t>(p, has_v, treat, dual, grid, stream);
      else launch_grad_typed<float, float>(p, has_v, treat, dual, grid, stream);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n = a.heads * (dual ? 2 : 1) * a.block * a.dim;
  pool_grad_bias_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(p, dual ? 1 : 0);
  return hipGetLastError();
}

}  // namespace lbca
