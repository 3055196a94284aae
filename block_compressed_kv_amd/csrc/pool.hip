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
#include "device_util.h"
#include "lbca_internal.h"

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
  int64_t heads, tokens, dim, m, entries, block_begin, n_blocks, pos_base, total_rows;
  int lanes_per_row;  // L = dim / 8, a power of two <= 64
  int log2_lanes;
  int log2_phases;    // P = token phases per output row
  float eps;          // < 0: no RMSNorm
  int rope_dims;      // 0: no RoPE
  double log2_base;
};

template <typename TX, typename TZ, bool HAS_V>
struct PoolAcc {
  float mx[8], l[8], ax[8], av[8];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int c = 0; c < 8; ++c) { mx[c] = kNegInf; l[c] = 0.f; ax[c] = 0.f; av[c] = 0.f; }
  }

  // Fold NT tokens, `stride` rows apart, into the state (bias rows stride apart too).
  template <int NT>
  __device__ __forceinline__ void fold(const TX* xs, const TX* vs, const TZ* zs, const float* bs,
                                       int64_t stride) {
    float a[NT][8];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      float zz[8], bb[8];
      load8(zs + i * stride, zz);
      load8(bs + i * stride, bb);
#pragma unroll
      for (int c = 0; c < 8; ++c) a[i][c] = (zz[c] + bb[c]) * kLog2e;
    }
    float xv[NT][8], vv[NT][8];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      load8(xs + i * stride, xv[i]);
      if constexpr (HAS_V) load8(vs + i * stride, vv[i]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float g = a[0][c];
#pragma unroll
      for (int i = 1; i < NT; ++i) g = fmaxf(g, a[i][c]);
      const float nm = fmaxf(mx[c], g);
      const float corr = exp2f(mx[c] - nm);
      float sl = 0.f, sx = 0.f, sv = 0.f;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const float p = exp2f(a[i][c] - nm);
        sl += p;
        sx = fmaf(p, xv[i][c], sx);
        if constexpr (HAS_V) sv = fmaf(p, vv[i][c], sv);
      }
      l[c] = fmaf(l[c], corr, sl);
      ax[c] = fmaf(ax[c], corr, sx);
      if constexpr (HAS_V) av[c] = fmaf(av[c], corr, sv);
      mx[c] = nm;
    }
  }

  // Fold tokens first, first+P, ... (< count) of a block whose token 0 is at
  // xs/vs/zs (row pitch dim) and whose bias row 0 is at bs.
  __device__ __forceinline__ void run(const TX* xs, const TX* vs, const TZ* zs, const float* bs,
                                      int64_t first, int64_t P, int64_t count, int64_t dim) {
    const int64_t stride = P * dim;
    int64_t i = first;
    for (; i + 3 * P < count; i += 4 * P)
      fold<4>(xs + i * dim, HAS_V ? vs + i * dim : nullptr, zs + i * dim, bs + i * dim, stride);
    for (; i < count; i += P)
      fold<1>(xs + i * dim, HAS_V ? vs + i * dim : nullptr, zs + i * dim, bs + i * dim, stride);
  }

  // Combine channel c of two partial states, lower token phase first
  // (branch-free; two empty states stay empty).
  __device__ __forceinline__ void combine1(int c, float lmx, float ll, float lax, float lav,
                                           float hmx, float hl, float hax, float hav) {
    const float nm = fmaxf(lmx, hmx);
    const bool none = nm == kNegInf;
    const float a = none ? 0.f : exp2f(lmx - nm), b = none ? 0.f : exp2f(hmx - nm);
    l[c] = ll * a + hl * b;
    ax[c] = lax * a + hax * b;
    av[c] = HAS_V ? lav * a + hav * b : 0.f;
    mx[c] = nm;
  }

  // Merge with the state of lane (lane ^ OFF), OFF = 16 or 32, through the
  // gfx950 lane swaps (VALU, no LDS round trip).  A swap of a register with
  // itself leaves the same two values in the same two result slots on both
  // lanes of a pair (the lower row's or half's value in the first, the other
  // in the second), so both lanes combine the same states in the same order.
  template <int OFF>
  __device__ __forceinline__ void merge_swap() {
    typedef float f2 __attribute__((ext_vector_type(2)));
    auto sw = [](float x) -> f2 {
      const uint32_t u = __float_as_uint(x);
      if constexpr (OFF == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return f2{__uint_as_float(r[0]), __uint_as_float(r[1])};
      } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return f2{__uint_as_float(r[0]), __uint_as_float(r[1])};
      }
    };
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const f2 m2 = sw(mx[c]), l2 = sw(l[c]), x2 = sw(ax[c]);
      const f2 v2 = HAS_V ? sw(av[c]) : f2{0.f, 0.f};
      combine1(c, m2[0], l2[0], x2[0], v2[0], m2[1], l2[1], x2[1], v2[1]);
    }
  }

  // Merge with the state of lane (lane ^ off); `lower`: this lane holds the
  // lower phase.  Both lanes of a pair evaluate the same expression.
  __device__ __forceinline__ void merge_xor(int off, bool lower) {
    if (off == 16) return merge_swap<16>();
    if (off == 32) return merge_swap<32>();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float omx = __shfl_xor(mx[c], off, 64), ol = __shfl_xor(l[c], off, 64);
      const float oax = __shfl_xor(ax[c], off, 64);
      const float oav = HAS_V ? __shfl_xor(av[c], off, 64) : 0.f;
      combine1(c, lower ? mx[c] : omx, lower ? l[c] : ol, lower ? ax[c] : oax, lower ? av[c] : oav,
               lower ? omx : mx[c], lower ? ol : l[c], lower ? oax : ax[c], lower ? oav : av[c]);
    }
  }
};

template <typename TX, typename TZ, bool DUAL, bool HAS_V, bool TREAT>
__global__ __launch_bounds__(256) void pool_kernel(PoolParams p) {
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
  const int64_t h = bh % p.heads;
  const int64_t dim = p.dim;
  const int64_t c0 = (int64_t)li * 8;
  const int64_t series = bh * p.tokens * dim + c0;
  const float* bias_h = p.bias + h * p.m * dim + c0;

  PoolAcc<TX, TZ, HAS_V> acc;
  acc.init();
  if (active) {
    const int64_t r0 = j * p.m - p.pos_base;  // token row of the entry's own block
    acc.run(static_cast<const TX*>(p.x) + series + r0 * dim,
            HAS_V ? static_cast<const TX*>(p.v) + series + r0 * dim : nullptr,
            static_cast<const TZ*>(p.z) + series + r0 * dim, bias_h, phase, P, p.m, dim);
    if (DUAL && j > 0) {
      const int64_t rb = r0 - p.m;  // preceding block, b-series
      acc.run(static_cast<const TX*>(p.xb) + series + rb * dim, nullptr,
              static_cast<const TZ*>(p.zb) + series + rb * dim, p.bias_b + h * p.m * dim + c0,
              phase, P, p.m, dim);
    }
  }

  // Merge the P phases of a row in a fixed order: inside a wave by lane
  // exchanges (phases of a row sit in consecutive groups), then across the
  // row's waves through LDS, read by the row's first wave.
  if (P > 1) {
    const int span = L * P;  // lanes of one row
    for (int off = L; off < 64 && off < span; off <<= 1) acc.merge_xor(off, (lane & off) == 0);
    if (span > 64) {
      const int wave = tid >> 6, waves_per_row = span >> 6;
      if (lane < L) {  // the wave's lowest phase group holds its merge
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          part[c][tid] = acc.mx[c];
          part[8 + c][tid] = acc.l[c];
          part[16 + c][tid] = acc.ax[c];
          part[24 + c][tid] = acc.av[c];
        }
      }
      __syncthreads();
      if ((wave & (waves_per_row - 1)) == 0) {
        for (int w = 1; w < waves_per_row; ++w) {
          const int src = tid + 64 * w;
#pragma unroll
          for (int c = 0; c < 8; ++c)
            acc.combine1(c, acc.mx[c], acc.l[c], acc.ax[c], acc.av[c], part[c][src], part[8 + c][src],
                         part[16 + c][src], part[24 + c][src]);
        }
      }
    }
  }

  float ox[8], ov[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float inv = active ? 1.f / acc.l[c] : 0.f;
    ox[c] = acc.ax[c] * inv;
    ov[c] = acc.av[c] * inv;
  }

  if constexpr (TREAT) {
    if (p.eps >= 0.f) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss = fmaf(ox[c], ox[c], ss);
      for (int o = L >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
      const float inv = 1.f / sqrtf(ss / (float)dim + p.eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) ox[c] *= inv;
    }
    if (p.rope_dims > 0) {
      const int r = p.rope_dims, half = r >> 1;
      const int64_t first = dim - r;
      const bool lo_half = c0 >= first && c0 < first + half;
      const bool hi_half = c0 >= first + half;
      const int src = lo_half ? lane + (half >> 3) : (hi_half ? lane - (half >> 3) : lane);
      float prt[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) prt[c] = __shfl(ox[c], src, 64);
      if (lo_half || hi_half) {
        const double pos = (double)(j * p.m);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int k = (int)(c0 + c - first) - (hi_half ? half : 0);
          float cs, sn;
          rope_cos_sin(pos, k, r, p.log2_base, &cs, &sn);
          ox[c] = lo_half ? ox[c] * cs - prt[c] * sn : ox[c] * cs + prt[c] * sn;
        }
      }
    }
  }

  if (active && phase == 0) {
    const int64_t o = (bh * p.entries + j) * dim + c0;
    store8(static_cast<TX*>(p.out_x) + o, ox);
    if constexpr (HAS_V) store8(static_cast<TX*>(p.out_v) + o, ov);
  }
}

template <typename TX, typename TZ>
static hipError_t launch_typed(const PoolParams& p, bool dual, bool has_v, bool treat, dim3 grid,
                               hipStream_t s) {
  if (dual) {
    if (treat) pool_kernel<TX, TZ, true, false, true><<<grid, 256, 0, s>>>(p);
    else pool_kernel<TX, TZ, true, false, false><<<grid, 256, 0, s>>>(p);
  } else if (has_v) {
    pool_kernel<TX, TZ, false, true, false><<<grid, 256, 0, s>>>(p);
  } else {
    if (treat) pool_kernel<TX, TZ, false, false, true><<<grid, 256, 0, s>>>(p);
    else pool_kernel<TX, TZ, false, false, false><<<grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_pool(const lbca_pool_args& a, hipStream_t stream) {
  PoolParams p;
  p.x = a.x; p.v = a.v; p.z = a.z; p.bias = a.bias;
  p.xb = a.xb; p.zb = a.zb; p.bias_b = a.bias_b;
  p.out_x = a.out_x; p.out_v = a.out_v;
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
  if (a.x_dtype == LBCA_BF16) {
    if (a.z_dtype == LBCA_BF16) return launch_typed<bf16_t, bf16_t>(p, dual, has_v, treat, grid, stream);
    return launch_typed<bf16_t, float>(p, dual, has_v, treat, grid, stream);
  }
  if (a.z_dtype == LBCA_BF16) return launch_typed<float, bf16_t>(p, dual, has_v, treat, grid, stream);
  return launch_typed<float, float>(p, dual, has_v, treat, grid, stream);
}

}  // namespace lbca
