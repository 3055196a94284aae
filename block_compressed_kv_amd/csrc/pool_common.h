// Per-channel online softmax of block pooling and the finishing of a pooled
// row (phase merge, normalisation, optional HCA/CSA treatment, store), shared
// by the pooling kernels and the decode-time cache step.
//
// Method: "mSeek: learned KV-cache compression in a 3B model", section "How LBCA
// works" (steps 2-3: per-channel softmax of content logits plus a positional
// bias over the block, weighted sums of its keys and values); "HCA: Heavily
// Compressed Attention (toy implementation)", "What is implemented" (RMSNorm
// and partial RoPE of the entry at its block start).
#pragma once
#include "device_util.h"

namespace lbca {

// Row strides (elements) of the token series a pooling pass reads.
struct RowPitch {
  int64_t x, v, z;
};

template <typename TX, typename TZ, bool HAS_V>
struct PoolAcc {
  float mx[8], l[8], ax[8], av[8];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int c = 0; c < 8; ++c) { mx[c] = kNegInf; l[c] = 0.f; ax[c] = 0.f; av[c] = 0.f; }
  }

  // Fold NT tokens into the state: token i at xs + i * st.x, vs + i * st.v,
  // zs + i * st.z, its bias row at bs + i * sb.
  template <int NT>
  __device__ __forceinline__ void fold(const TX* xs, const TX* vs, const TZ* zs, const float* bs,
                                       const RowPitch& st, int64_t sb) {
    float a[NT][8];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      float zz[8], bb[8];
      load8(zs + i * st.z, zz);
      load8(bs + i * sb, bb);
#pragma unroll
      for (int c = 0; c < 8; ++c) a[i][c] = (zz[c] + bb[c]) * kLog2e;
    }
    float xv[NT][8], vv[NT][8];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      load8(xs + i * st.x, xv[i]);
      if constexpr (HAS_V) load8(vs + i * st.v, vv[i]);
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
  // xs/vs/zs (row strides rp) and whose bias row 0 is at bs (row pitch dim).
  __device__ __forceinline__ void run(const TX* xs, const TX* vs, const TZ* zs, const float* bs,
                                      int64_t first, int64_t P, int64_t count, int64_t dim, const RowPitch& rp) {
    const RowPitch st{P * rp.x, P * rp.v, P * rp.z};
    const int64_t sb = P * dim;
    int64_t i = first;
    for (; i + 3 * P < count; i += 4 * P)
      fold<4>(xs + i * rp.x, HAS_V ? vs + i * rp.v : nullptr, zs + i * rp.z, bs + i * dim, st, sb);
    for (; i < count; i += P)
      fold<1>(xs + i * rp.x, HAS_V ? vs + i * rp.v : nullptr, zs + i * rp.z, bs + i * dim, st, sb);
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

// Entry treatment of a finished pooled row (RMSNorm with unit weight when
// eps >= 0, then RoPE of the last rope_dims dims at the block start).
struct EntryTreat {
  float eps;
  int rope_dims;
  double log2_base;
};

// Finishes one pooled row whose P token phases sit in P consecutive groups of
// L lanes (this lane: channels c0 .. c0+7 of phase `phase`): merges the phases
// in a fixed order (inside a wave by lane exchanges, across the row's waves
// through `part`, read by the row's first wave), normalises, applies the
// treatment and stores channels c0.. of the entry (phase-0 lanes of active
// rows).  Every thread of the workgroup calls it (lane exchanges, barrier);
// in a workgroup wider than the pooling threads (the first 256), the others
// pass member = false and only take part in the barrier.
template <typename TX, typename TZ, bool HAS_V, bool TREAT>
__device__ __forceinline__ void finish_entry(PoolAcc<TX, TZ, HAS_V>& acc, float (*part)[256], int L, int P,
                                             int phase, bool active, int64_t dim, int64_t c0, int64_t block_pos,
                                             const EntryTreat& tr, TX* out_x, TX* out_v, bool member = true) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (P > 1) {
    const int span = L * P;  // lanes of one row
    for (int off = L; off < 64 && off < span; off <<= 1) acc.merge_xor(off, (lane & off) == 0);
    if (span > 64) {
      const int wave = tid >> 6, waves_per_row = span >> 6;
      if (member && lane < L) {  // the wave's lowest phase group holds its merge
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          part[c][tid] = acc.mx[c];
          part[8 + c][tid] = acc.l[c];
          part[16 + c][tid] = acc.ax[c];
          part[24 + c][tid] = acc.av[c];
        }
      }
      __syncthreads();
      if (member && (wave & (waves_per_row - 1)) == 0) {
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
    if (tr.eps >= 0.f) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss = fmaf(ox[c], ox[c], ss);
      for (int o = L >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
      const float inv = 1.f / sqrtf(ss / (float)dim + tr.eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) ox[c] *= inv;
    }
    if (tr.rope_dims > 0) {
      const int r = tr.rope_dims, half = r >> 1;
      const int64_t first = dim - r;
      const bool lo_half = c0 >= first && c0 < first + half;
      const bool hi_half = c0 >= first + half;
      const int src = lo_half ? lane + (half >> 3) : (hi_half ? lane - (half >> 3) : lane);
      float prt[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) prt[c] = __shfl(ox[c], src, 64);
      if (lo_half || hi_half) {
        const double pos = (double)block_pos;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int k = (int)(c0 + c - first) - (hi_half ? half : 0);
          float cs, sn;
          rope_cos_sin(pos, k, r, tr.log2_base, &cs, &sn);
          ox[c] = lo_half ? ox[c] * cs - prt[c] * sn : ox[c] * cs + prt[c] * sn;
        }
      }
    }
  }

  if (member && active && phase == 0) {
    store8(out_x, ox);
    if constexpr (HAS_V) store8(out_v, ov);
  }
}

}  // namespace lbca
