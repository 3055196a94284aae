// Prefill attention for a chunk of consecutive queries, each with its own
// visibility (pooled entries j < n_pooled(t) plus the raw span [raw_begin(t), t]).
//
// Method: "mSeek: learned KV-cache compression in a 3B model", "How LBCA works"
// (steps 4-5, and the chunked bounded-memory path that must agree with the
// clear reference): a query sees every completed summary older than its
// window plus its exact raw window, never a summary holding a later token.
//
// bf16 path (MFMA).  A workgroup of 4 waves owns one (sequence, KV head) and
// 128 consecutive rows of the flattened (position, query head in the GQA group)
// space; each wave holds 32 of those rows (two 16-row groups) as B operands.
// The workgroup walks the union of its rows' visible rows in 32-row tiles:
// first the pooled prefix [0, n_pooled(last position)), then the raw band
// [raw_begin(first position), last position].  K and V tiles are staged in LDS
// (double buffered, the next tile's global loads in flight during the current
// tile's MFMAs, one barrier per tile).  Scores are computed transposed,
// S^T = K Q^T (v_mfma_f32_16x16x32_bf16), so each lane owns one query row's
// scores and the row max/sum need two cross-lane steps; O^T = V^T P^T uses
// v_mfma_f32_16x16x16_bf16 with P^T straight from the score registers.  A
// per-element mask applies each row's own visibility inside every tile.
#include "device_util.h"
#include "lbca_internal.h"

namespace lbca {

typedef short s16x4p __attribute__((ext_vector_type(4)));

struct PrefillParams {
  const bf16_t* q;
  const bf16_t* pk;
  const bf16_t* pv;
  const bf16_t* rk;
  const bf16_t* rv;
  const float* sink;
  void* out;
  float* lse;
  int64_t q_len, hq, hkv, G, entries, raw_rows, q_pos0, raw_pos_base, m, W;
  int mode, out_bf16, row_blocks;
  float scale_log2;
};

template <int D, bool SHARED>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
  constexpr int KS = D / 32, DT = D / 16, KT = 32, PITCH = D + 8;
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int LOADS = (KT * CH) / 256;      // chunks per thread per tile
  static_assert(LOADS >= 1 && (KT * CH) % 256 == 0, "tile must split evenly");
  __shared__ __attribute__((aligned(16))) bf16_t ks[2][KT * PITCH];
  __shared__ __attribute__((aligned(16))) bf16_t vs[SHARED ? 1 : 2][SHARED ? 16 : KT * PITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kq = lane >> 4;
  const int64_t bid = blockIdx.x;
  const int64_t rblk = bid % p.row_blocks;
  const int64_t bh = bid / p.row_blocks;
  const int64_t kvh = bh % p.hkv, b = bh / p.hkv;
  const int64_t rows_total = p.q_len * p.G;
  const int64_t row0 = rblk * 128;
  const int64_t row_last = (row0 + 127 < rows_total ? row0 + 127 : rows_total - 1);
  const int64_t p_first = p.q_pos0 + row0 / p.G;
  const int64_t p_last = p.q_pos0 + row_last / p.G;

  // my two 16-row query groups
  uint4 qr[2][KS];
  int64_t my_np[2], my_rb[2], my_pos[2], my_out[2];
  bool my_ok[2];
#pragma unroll
  for (int gq = 0; gq < 2; ++gq) {
    const int64_t r = row0 + wave * 32 + gq * 16 + n;
    const bool ok = r < rows_total;
    const int64_t rr = ok ? r : rows_total - 1;
    const int64_t pl = rr / p.G, g = rr % p.G;
    const int64_t t = p.q_pos0 + pl;
    visible_range(t, p.m, p.W, p.mode, &my_np[gq], &my_rb[gq]);
    my_pos[gq] = t;
    my_ok[gq] = ok;
    my_out[gq] = ((b * p.q_len + pl) * p.hq + kvh * p.G + g) * D;
    const bf16_t* qrow = p.q + my_out[gq] + 8 * kq;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qr[gq][s] = ok ? *reinterpret_cast<const uint4*>(qrow + 32 * s) : make_uint4(0, 0, 0, 0);
  }

  int64_t NP, RB, dummy;
  visible_range(p_last, p.m, p.W, p.mode, &NP, &dummy);
  visible_range(p_first, p.m, p.W, p.mode, &dummy, &RB);
  const int64_t T1 = (NP + KT - 1) / KT;
  const int64_t T2 = (p_last - RB + 1 + KT - 1) / KT;
  const int64_t T = T1 + T2;
  const int64_t kv_pool = (b * p.hkv + kvh) * p.entries;
  const int64_t kv_raw = (b * p.hkv + kvh) * p.raw_rows - p.raw_pos_base;

  uint4 kreg[LOADS], vreg[SHARED ? 1 : LOADS];
  auto load_tile = [&](int64_t tile) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i;
      const int r = c / CH, col = c % CH;
      int64_t row;
      bool ok;
      const bf16_t *kb, *vb;
      if (tile < T1) {
        const int64_t j = tile * KT + r;
        ok = j < NP;
        row = kv_pool + j;
        kb = p.pk;
        vb = p.pv;
      } else {
        const int64_t s = RB + (tile - T1) * KT + r;
        ok = s <= p_last;
        row = kv_raw + s;
        kb = p.rk;
        vb = p.rv;
      }
      kreg[i] = ok ? *reinterpret_cast<const uint4*>(kb + row * D + col * 8) : make_uint4(0, 0, 0, 0);
      if (!SHARED)
        vreg[i] = ok ? *reinterpret_cast<const uint4*>(vb + row * D + col * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = tid + 256 * i;
      const int r = c / CH, col = c % CH;
      *reinterpret_cast<uint4*>(&ks[buf][r * PITCH + col * 8]) = kreg[i];
      if (!SHARED) *reinterpret_cast<uint4*>(&vs[buf][r * PITCH + col * 8]) = vreg[i];
    }
  };

  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.f, 0.f};
  f32x4 acc[2][DT];
#pragma unroll
  for (int gq = 0; gq < 2; ++gq)
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[gq][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (T > 0) load_tile(0);
  for (int64_t tile = 0; tile < T; ++tile) {
    const int buf = (int)(tile & 1);
    store_tile(buf);
    __syncthreads();
    if (tile + 1 < T) load_tile(tile + 1);
    const bf16_t* kt = ks[buf];
    const bf16_t* vt = SHARED ? ks[buf] : vs[buf];
    const bool pooled = tile < T1;
    const int64_t base = pooled ? tile * KT : RB + (tile - T1) * KT;

    float sc[2][2][4];  // [group][half][j]
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      uint4 kop[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kop[s] = *reinterpret_cast<const uint4*>(&kt[(16 * hh + n) * PITCH + 32 * s + 8 * kq]);
#pragma unroll
      for (int gq = 0; gq < 2; ++gq) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[s]),
                                                       __builtin_bit_cast(bf16x8, qr[gq][s]), c, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t x = base + 16 * hh + 4 * kq + j;  // entry id or position
          const bool vis = pooled ? (x < my_np[gq]) : (x >= my_rb[gq] && x <= my_pos[gq]);
          sc[gq][hh][j] = vis ? c[j] * p.scale_log2 : kNegInf;
        }
      }
    }
    s16x4p pop[2][2];
#pragma unroll
    for (int gq = 0; gq < 2; ++gq) {
      float tmax = kNegInf;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int j = 0; j < 4; ++j) tmax = fmaxf(tmax, sc[gq][hh][j]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float nm = fmaxf(m_run[gq], tmax);
      const float mu = nm == kNegInf ? 0.f : nm;
      const float corr = exp2f(m_run[gq] - mu);
      float psum = 0.f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float pj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pj[j] = exp2f(sc[gq][hh][j] - mu);
          psum += pj[j];
        }
        const uint32_t w0 = pack_bf16x2(pj[0], pj[1]), w1 = pack_bf16x2(pj[2], pj[3]);
        pop[gq][hh] = s16x4p{(short)(w0 & 0xffff), (short)(w0 >> 16), (short)(w1 & 0xffff), (short)(w1 >> 16)};
      }
      l_run[gq] = fmaf(l_run[gq], corr, psum);
      m_run[gq] = nm;
#pragma unroll
      for (int t = 0; t < DT; ++t) acc[gq][t] *= corr;
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bf16_t* vb = &vt[(16 * hh + 4 * kq) * PITCH + n];
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        s16x4p a;
        a[0] = (short)vb[16 * t].bits;
        a[1] = (short)vb[PITCH + 16 * t].bits;
        a[2] = (short)vb[2 * PITCH + 16 * t].bits;
        a[3] = (short)vb[3 * PITCH + 16 * t].bits;
#pragma unroll
        for (int gq = 0; gq < 2; ++gq)
          acc[gq][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pop[gq][hh], acc[gq][t], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int gq = 0; gq < 2; ++gq) {
    float l = l_run[gq];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (!my_ok[gq]) continue;
    const int64_t h = (my_out[gq] / D) % p.hq;
    if (p.sink) l += exp2f(p.sink[h] * kLog2e - m_run[gq]);
    const float inv = 1.f / l;
    if (p.out_bf16) {
      bf16_t* o = static_cast<bf16_t*>(p.out) + my_out[gq] + 4 * kq;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        uint2 w;
        w.x = pack_bf16x2(acc[gq][t][0] * inv, acc[gq][t][1] * inv);
        w.y = pack_bf16x2(acc[gq][t][2] * inv, acc[gq][t][3] * inv);
        *reinterpret_cast<uint2*>(o + 16 * t) = w;
      }
    } else {
      float* o = static_cast<float*>(p.out) + my_out[gq] + 4 * kq;
#pragma unroll
      for (int t = 0; t < DT; ++t)
        *reinterpret_cast<float4*>(o + 16 * t) =
            make_float4(acc[gq][t][0] * inv, acc[gq][t][1] * inv, acc[gq][t][2] * inv, acc[gq][t][3] * inv);
    }
    if (p.lse && kq == 0) p.lse[my_out[gq] / D] = (m_run[gq] + log2f(l)) * 0.69314718055994531f;
  }
}

hipError_t launch_prefill(const lbca_prefill_args& a, hipStream_t stream) {
  if (a.dtype != LBCA_BF16) return launch_prefill_f32(a, stream);
  PrefillParams p{};
  p.q = static_cast<const bf16_t*>(a.q);
  p.pk = static_cast<const bf16_t*>(a.pooled_k);
  p.pv = static_cast<const bf16_t*>(a.pooled_v);
  p.rk = static_cast<const bf16_t*>(a.raw_k);
  p.rv = static_cast<const bf16_t*>(a.raw_v);
  p.sink = a.sink;
  p.out = a.out;
  p.lse = a.lse;
  p.q_len = a.q_len; p.hq = a.q_heads; p.hkv = a.kv_heads; p.G = a.q_heads / a.kv_heads;
  p.entries = a.entries; p.raw_rows = a.raw_rows; p.q_pos0 = a.q_pos0; p.raw_pos_base = a.raw_pos_base;
  p.m = a.block; p.W = a.window; p.mode = a.mode;
  p.out_bf16 = a.out_dtype == LBCA_BF16;
  p.scale_log2 = a.scale * kLog2e;
  p.row_blocks = (int)((a.q_len * p.G + 127) / 128);
  const dim3 grid((unsigned)(a.batch * a.kv_heads * p.row_blocks));
  const bool shared = a.pooled_v == nullptr;
  switch (a.dim) {
    case 64:
      if (shared) prefill_kernel<64, true><<<grid, 256, 0, stream>>>(p);
      else prefill_kernel<64, false><<<grid, 256, 0, stream>>>(p);
      break;
    case 128:
      if (shared) prefill_kernel<128, true><<<grid, 256, 0, stream>>>(p);
      else prefill_kernel<128, false><<<grid, 256, 0, stream>>>(p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lbca
