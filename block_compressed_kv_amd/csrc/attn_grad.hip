// Gradients of prefill attention over pooled entries plus the raw window.
//
// Method: "mSeek: learned KV-cache compression in a 3B model", "How LBCA
// works" steps 4-5 (the forward: one softmax per query over the pooled
// entries j < n_pooled(t) and the raw span [raw_begin(t), t]) and "Experiment
// at a glance" (the layer is trained end to end, so its gradients are needed).
// With P = exp(scale * q.k - lse) (lse from the forward, sink included),
// D = dO . O per query row, dP = dO . v and dS = P (dP - D):
//   dV_j = sum_rows P dO,  dK_j = scale sum_rows dS q,  dQ = scale sum_j dS k_j,
//   dsink_h = -sum_rows exp(sink_h - lse) D.
//
// Work split (bf16, dims 64 and 128).  A workgroup of 4 waves owns 128
// consecutive keys of one series (pooled entries, or raw positions) of one
// (sequence, KV head); wave w owns keys 32w..32w+31 and keeps their K and V
// rows in registers as MFMA operands, with dK and dV accumulating in
// registers.  It walks the query rows that can see its keys (the flattened
// (position, GQA head) rows of that KV head: every row from the first that
// sees its first key for pooled entries, split across workgroups in runs of
// 1024 rows; the window band for raw positions) in tiles of 32 rows staged
// through LDS (next tile prefetched into registers while the current one
// computes).  Per tile and wave, on v_mfma_f32_32x32x16_bf16:
//   S = Q K^T and dP = dO V^T       (rows x the wave's keys, contraction dims)
//   dV^T += dO^T P, dK^T += Q^T dS  (contraction over the 32 rows; P and dS
//                                    feed straight from the accumulator layout,
//                                    dO^T and Q^T come from transposing LDS reads)
//   dQ  = dS K                      (dS goes through LDS transposed; each wave
//                                    covers 32 dims, then adds its partial to
//                                    the fp32 dQ with atomics)
// Pooled-entry gradients are added with atomics (several query runs touch one
// entry); raw-position gradients have one owner and are stored.
#include "device_util.h"
#include "lbca_internal.h"

namespace lbca {

namespace {

constexpr int GK = 128;      // keys per workgroup
constexpr int GQ = 32;       // query rows per tile
constexpr int QSPLIT = 1024; // query rows per workgroup on the pooled series

struct GradParams {
  const bf16_t* q;
  const bf16_t* dout;
  const float* lse;
  const float* dvec;
  const bf16_t* pk;
  const bf16_t* pv;
  const bf16_t* rk;
  const bf16_t* rv;
  float* dq;
  float* dpk;
  float* dpv;
  float* drk;
  float* drv;
  int64_t q_len, hq, hkv, G, entries, raw_rows, q_pos0, raw_pos_base, m, W;
  int mode, accumulate, shared;
  int n_pool, pool_tiles, pool_splits, raw_tiles;
  float scale, scale_log2;
};

// Position of 16-byte chunk c of row r in an LDS tile of 32 query rows: 8
// consecutive rows read at one chunk, and 4 consecutive rows read at 4 aligned
// chunks (two transposing 16-lane groups), land in distinct banks.
template <int D>
__device__ __forceinline__ int qswz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

// 8 bf16 of one column from two transposing LDS reads (rows r..r+3 at a, then
// rows at b), as one MFMA operand
__device__ __forceinline__ bf16x8 tr_pair(const bf16_t* a, const bf16_t* b) {
  const s16x4 lo = lds_read_tr16(a), hi = lds_read_tr16(b);
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 pack8(const float* f) {
  const uint4 u = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                             pack_bf16x2(f[6], f[7]));
  return __builtin_bit_cast(bf16x8, u);
}

template <int D>
__global__ __launch_bounds__(256, 1) void attn_grad_kernel(GradParams p) {
  constexpr int DS = D / 16;                  // 16-dim slices of the S / dP contraction
  constexpr int DB = D / 32;                  // 32-dim blocks of dV^T / dK^T
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int NCH = GQ * CH / 256;          // chunks per thread per tile and tensor
  static_assert(NCH == 1 || NCH == 2, "staging holds one or two chunks per tensor");
  constexpr int KSL = D == 128 ? 8 : 4;       // 16-key slices of the wave's dQ contraction
  __shared__ __attribute__((aligned(16))) bf16_t sq[2][GQ * D];
  __shared__ __attribute__((aligned(16))) bf16_t sdo[2][GQ * D];
  __shared__ __attribute__((aligned(16))) bf16_t sdst[GK * GQ];  // dS^T: row = key, 32 query columns
  __shared__ __attribute__((aligned(16))) float s_l2[2][GQ];
  __shared__ __attribute__((aligned(16))) float s_dv[2][GQ];
  __shared__ __attribute__((aligned(16))) int s_a[2][GQ];       // pooled: n_pooled(t); raw: raw_begin(t)
  __shared__ __attribute__((aligned(16))) int s_b[2][GQ];       // raw: t
  __shared__ __attribute__((aligned(16))) int s_row[2][GQ];     // flat query-row index, -1 if not this tile's

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5, j16 = lane & 15, g4 = lane >> 4;
  const int bh = blockIdx.y;
  const int b = bh / (int)p.hkv, kvh = bh % (int)p.hkv;
  const int G = (int)p.G;
  const int rows_total = (int)p.q_len * G;
  const int wi = blockIdx.x;
  const bool pooled = wi < p.pool_tiles * p.pool_splits;

  int k0, nkeys, row_begin, row_end;
  if (pooled) {
    const int tile = wi / p.pool_splits, split = wi % p.pool_splits;
    k0 = tile * GK;
    nkeys = min(GK, p.n_pool - k0);
    // first position whose pooled prefix includes entry k0
    const int64_t t_first = p.mode == LBCA_EXCLUSIVE ? (int64_t)(k0 + 1) * p.m + p.W - 1 : (int64_t)(k0 + 1) * p.m - 1;
    const int64_t i_first = t_first - p.q_pos0 > 0 ? t_first - p.q_pos0 : 0;
    row_begin = (int)(i_first * G) + split * QSPLIT;
    row_end = min(row_begin + QSPLIT, rows_total);
    if (row_begin >= rows_total) return;  // nothing in this run: the entries' gradients were set beforehand
  } else {
    k0 = (wi - p.pool_tiles * p.pool_splits) * GK;
    nkeys = (int)min((int64_t)GK, p.raw_rows - k0);
    // queries t seeing some position in [p0, p1]: t >= p0 and raw_begin(t) <= p1
    const int64_t p0 = p.raw_pos_base + k0, p1 = p0 + nkeys - 1;
    const int64_t t_last = p.mode == LBCA_EXCLUSIVE ? (p1 / p.m + 1) * p.m + p.W - 2 : p1 + p.W - 1;
    const int64_t lo = p0 > p.q_pos0 ? p0 : p.q_pos0;
    const int64_t hi = t_last < p.q_pos0 + p.q_len - 1 ? t_last : p.q_pos0 + p.q_len - 1;
    row_begin = (int)((lo - p.q_pos0) * G);
    row_end = hi >= lo ? (int)((hi - p.q_pos0 + 1) * G) : row_begin;
  }

  const int64_t key_base = pooled ? (int64_t)bh * p.entries + k0 : (int64_t)bh * p.raw_rows + k0;
  const bf16_t* kser = pooled ? p.pk : p.rk;
  const bf16_t* vser = pooled ? (p.shared ? p.pk : p.pv) : (p.shared ? p.rk : p.rv);

  // this wave's K and V rows as B operands (N = key, K = dims 16 s + 8 h ..)
  const int key_rel = 32 * wave + n;
  const bool key_ok = key_rel < nkeys;
  uint4 kb[DS], vb[DS];
  {
    const bf16_t* kr = kser + (key_base + (key_ok ? key_rel : 0)) * D + 8 * h;
    const bf16_t* vr = vser + (key_base + (key_ok ? key_rel : 0)) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      kb[s] = key_ok ? *reinterpret_cast<const uint4*>(kr + 16 * s) : make_uint4(0, 0, 0, 0);
      vb[s] = key_ok ? *reinterpret_cast<const uint4*>(vr + 16 * s) : make_uint4(0, 0, 0, 0);
    }
  }
  // K as the B operand of dQ (N = dim, K = keys): this wave's 32 dims over its
  // key range (all 128 keys at 128 dims; at 64 dims the waves split dims x key halves)
  const int dq_db = D == 128 ? wave : (wave & 1);
  const int dq_kb = D == 128 ? 0 : 64 * (wave >> 1);
  bf16x8 kt[KSL];
#pragma unroll
  for (int s = 0; s < KSL; ++s) {
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kk = dq_kb + 16 * s + 8 * h + j;
      e[j] = kk < nkeys ? reinterpret_cast<const uint16_t*>(kser)[(key_base + kk) * D + 32 * dq_db + n] : (uint16_t)0;
    }
    const uint4 u = make_uint4(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                               e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16));
    kt[s] = __builtin_bit_cast(bf16x8, u);
  }

  f32x16 dva[DB], dka[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dva[i] = dka[i] = f32x16{};

  // staging of one query tile (held in named registers: NCH chunks of Q and of
  // dO per thread, plus one row's bookkeeping for threads 0..31)
  uint4 stq0 = make_uint4(0, 0, 0, 0), stq1 = stq0, sto0 = stq0, sto1 = stq0;
  float st_l2 = 0.f, st_dv = 0.f;
  int st_a = 0, st_b = 0, st_row = -1;
  auto fetch = [&](int rt) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = tid + 256 * c, row = idx / CH, ch = idx % CH;
      const int gr = rt + row;
      uint4 vq = make_uint4(0, 0, 0, 0), vo = vq;
      if (gr < row_end) {
        const int i = gr / G, hg = gr - i * G;
        const int64_t off = (((int64_t)b * p.q_len + i) * p.hq + (int64_t)kvh * G + hg) * D + 8 * ch;
        vq = *reinterpret_cast<const uint4*>(p.q + off);
        vo = *reinterpret_cast<const uint4*>(p.dout + off);
      }
      if (c == 0) { stq0 = vq; sto0 = vo; }
      else { stq1 = vq; sto1 = vo; }
    }
    if (tid < GQ) {
      const int gr = rt + tid;
      if (gr < row_end) {
        const int i = gr / G, hg = gr - i * G;
        const int64_t rid = ((int64_t)b * p.q_len + i) * p.hq + (int64_t)kvh * G + hg;
        st_row = (int)rid;
        st_l2 = p.lse[rid] * kLog2e;
        st_dv = p.dvec[rid];
        int64_t np, rb;
        visible_range(p.q_pos0 + i, p.m, p.W, p.mode, &np, &rb);
        st_a = pooled ? (int)np : (int)rb;
        st_b = (int)(p.q_pos0 + i);
      } else {
        st_row = -1;
        st_l2 = __builtin_inff();
        st_dv = 0.f;
        st_a = pooled ? 0 : 0x7fffffff;
        st_b = -1;
      }
    }
  };
  auto stash = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = tid + 256 * c, row = idx / CH, ch = idx % CH;
      const int pos = row * D + 8 * (ch ^ qswz<D>(row));
      *reinterpret_cast<uint4*>(&sq[buf][pos]) = c == 0 ? stq0 : stq1;
      *reinterpret_cast<uint4*>(&sdo[buf][pos]) = c == 0 ? sto0 : sto1;
    }
    if (tid < GQ) {
      s_l2[buf][tid] = st_l2;
      s_dv[buf][tid] = st_dv;
      s_a[buf][tid] = st_a;
      s_b[buf][tid] = st_b;
      s_row[buf][tid] = st_row;
    }
  };

  // this lane's key as a pooled entry id or a raw position
  const int my_key = pooled ? k0 + key_rel : (int)(p.raw_pos_base + k0 + key_rel);

  if (row_begin < row_end) {
    fetch(row_begin);
    stash(0);
  }
  __syncthreads();
  int buf = 0;
  for (int rt = row_begin; rt < row_end; rt += GQ) {
    const bool more = rt + GQ < row_end;
    if (more) fetch(rt + GQ);
    const bf16_t* tq = sq[buf];
    const bf16_t* tdo = sdo[buf];

    // S = Q K^T, dP = dO V^T: lane (key n, h) gets rows 8 (e / 4) + 4 h + e % 4
    f32x16 sacc = {}, dpacc = {};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const int pos = n * D + 8 * ((2 * s + h) ^ qswz<D>(n));
      const bf16x8 aq = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&tq[pos]));
      const bf16x8 ao = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&tdo[pos]));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, __builtin_bit_cast(bf16x8, kb[s]), sacc, 0, 0, 0);
      dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, __builtin_bit_cast(bf16x8, vb[s]), dpacc, 0, 0, 0);
    }

    // probabilities and scaled dS, masked by each row's visibility
    float pe[16], dse[16];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r0 = 8 * qq + 4 * h;
      const float4 l2 = *reinterpret_cast<const float4*>(&s_l2[buf][r0]);
      const float4 dv = *reinterpret_cast<const float4*>(&s_dv[buf][r0]);
      const int4 va = *reinterpret_cast<const int4*>(&s_a[buf][r0]);
      const int4 vbv = *reinterpret_cast<const int4*>(&s_b[buf][r0]);
      const float l2a[4] = {l2.x, l2.y, l2.z, l2.w}, dva4[4] = {dv.x, dv.y, dv.z, dv.w};
      const int aa[4] = {va.x, va.y, va.z, va.w}, bb[4] = {vbv.x, vbv.y, vbv.z, vbv.w};
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int e = 4 * qq + rr;
        const bool vis = key_ok && (pooled ? my_key < aa[rr] : (aa[rr] <= my_key && my_key <= bb[rr]));
        const float pr = vis ? fast_exp2(sacc[e] * p.scale_log2 - l2a[rr]) : 0.f;
        pe[e] = pr;
        dse[e] = pr * (dpacc[e] - dva4[rr]) * p.scale;
      }
    }
    const bf16x8 pb0 = pack8(pe), pb1 = pack8(pe + 8);
    const bf16x8 db0 = pack8(dse), db1 = pack8(dse + 8);

    // dS^T into LDS: row key_rel, query columns 8 qq + 4 h .. +3
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const uint2 w2 = make_uint2(pack_bf16x2(dse[4 * qq], dse[4 * qq + 1]), pack_bf16x2(dse[4 * qq + 2], dse[4 * qq + 3]));
      *reinterpret_cast<uint2*>(&sdst[key_rel * GQ + 8 * (qq ^ ((key_rel >> 2) & 3)) + 4 * h]) = w2;
    }

    // dV^T += dO^T P, dK^T += Q^T dS over the tile's rows: k slice ks holds
    // rows 16 ks + 4 h .. +3 and 16 ks + 8 + 4 h .. +3 (the accumulator order)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ra = 16 * ks + 4 * (g4 >> 1) + (j16 >> 2), rb2 = ra + 8;
#pragma unroll
      for (int dbk = 0; dbk < DB; ++dbk) {
        const int c = 4 * dbk + 2 * (g4 & 1) + ((j16 & 3) >> 1);
        const int pa = ra * D + 8 * (c ^ qswz<D>(ra)) + 4 * (j16 & 1);
        const int pbb = rb2 * D + 8 * (c ^ qswz<D>(rb2)) + 4 * (j16 & 1);
        const bf16x8 aot = tr_pair(&tdo[pa], &tdo[pbb]);
        const bf16x8 aqt = tr_pair(&tq[pa], &tq[pbb]);
        dva[dbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aot, ks ? pb1 : pb0, dva[dbk], 0, 0, 0);
        dka[dbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aqt, ks ? db1 : db0, dka[dbk], 0, 0, 0);
      }
    }
    __syncthreads();

    // dQ (rows x this wave's 32 dims) = dS K over the wave's key range
    f32x16 dqa = {};
#pragma unroll
    for (int s = 0; s < KSL; ++s) {
      const int ka = dq_kb + 16 * s + 8 * (g4 >> 1) + (j16 >> 2), kb2 = ka + 4;
      const int c = 2 * (g4 & 1) + ((j16 & 3) >> 1);
      const bf16x8 ad = tr_pair(&sdst[ka * GQ + 8 * (c ^ ((ka >> 2) & 3)) + 4 * (j16 & 1)],
                                &sdst[kb2 * GQ + 8 * (c ^ ((kb2 >> 2) & 3)) + 4 * (j16 & 1)]);
      dqa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, kt[s], dqa, 0, 0, 0);
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int4 rid = *reinterpret_cast<const int4*>(&s_row[buf][8 * qq + 4 * h]);
      const int ra[4] = {rid.x, rid.y, rid.z, rid.w};
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (ra[rr] >= 0) unsafeAtomicAdd(p.dq + (int64_t)ra[rr] * D + 32 * dq_db + n, dqa[4 * qq + rr]);
    }

    if (more) stash(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // dK, dV of this wave's keys: lane (key n, h) holds dims 32 db + 8 qq + 4 h .. +3
  if (!key_ok) return;
  const int64_t krow = (key_base + key_rel) * D;
  float* gk = pooled ? p.dpk : p.drk;
  float* gv = pooled ? p.dpv : p.drv;
#pragma unroll
  for (int dbk = 0; dbk < DB; ++dbk)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int d = 32 * dbk + 8 * qq + 4 * h;
      float kv[4], vv[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        vv[rr] = dva[dbk][4 * qq + rr];
        kv[rr] = dka[dbk][4 * qq + rr] + (p.shared ? vv[rr] : 0.f);
      }
      if (pooled) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          unsafeAtomicAdd(gk + krow + d + rr, kv[rr]);
          if (!p.shared) unsafeAtomicAdd(gv + krow + d + rr, vv[rr]);
        }
      } else {
        float4* pk4 = reinterpret_cast<float4*>(gk + krow + d);
        float4 k4 = make_float4(kv[0], kv[1], kv[2], kv[3]);
        if (p.accumulate) {
          const float4 o = *pk4;
          k4.x += o.x; k4.y += o.y; k4.z += o.z; k4.w += o.w;
        }
        *pk4 = k4;
        if (!p.shared) {
          float4* pv4 = reinterpret_cast<float4*>(gv + krow + d);
          float4 v4 = make_float4(vv[0], vv[1], vv[2], vv[3]);
          if (p.accumulate) {
            const float4 o = *pv4;
            v4.x += o.x; v4.y += o.y; v4.z += o.z; v4.w += o.w;
          }
          *pv4 = v4;
        }
      }
    }
}

// D = dO . O per query row, dq set to zero, and the sink gradient.  Grid:
// (runs of 64 flattened (sequence, position) rows, query heads); threads of
// one row hold 8 dims each.
struct PrepParams {
  const bf16_t* dout;
  const void* out;
  const float* lse;
  const float* sink;
  float* dvec;
  float* dq;
  float* dsink;
  int64_t rows;  // batch * q_len
  int64_t hq, dim;
  int out_f32;
};

__global__ __launch_bounds__(256) void attn_grad_prep_kernel(PrepParams p) {
  __shared__ float red[4];
  const int tpr = (int)p.dim / 8;           // threads per row: 8 or 16
  const int rpp = 256 / tpr;                // rows per pass
  const int tid = threadIdx.x, sub = tid % tpr, rloc = tid / tpr;
  const int hh = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  float sink_acc = 0.f;
  const float sk = p.sink ? p.sink[hh] : 0.f;
  for (int r = rloc; r < 64; r += rpp) {
    const int64_t row = r0 + r;
    if (row >= p.rows) break;
    const int64_t rid = row * p.hq + hh;
    const int64_t off = rid * p.dim + 8 * sub;
    float go[8], o[8];
    load8(p.dout + off, go);
    if (p.out_f32) load8(static_cast<const float*>(p.out) + off, o);
    else load8(static_cast<const bf16_t*>(p.out) + off, o);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(go[i], o[i], acc);
    for (int w = tpr / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w);
    const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    store8(p.dq + off, z);
    if (sub == 0) {
      p.dvec[rid] = acc;
      if (p.sink) sink_acc -= __expf(sk - p.lse[rid]) * acc;
    }
  }
  if (!p.dsink) return;
  for (int w = 32; w >= 1; w >>= 1) sink_acc += __shfl_xor(sink_acc, w);
  if ((tid & 63) == 0) red[tid >> 6] = sink_acc;
  __syncthreads();
  if (tid == 0) unsafeAtomicAdd(p.dsink + hh, red[0] + red[1] + red[2] + red[3]);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = 0.f;
}

hipError_t zero_f32(float* x, int64_t n, hipStream_t stream) {
  if (!x || n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  fill_zero_kernel<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, stream>>>(x, n);
  return hipGetLastError();
}

}  // namespace

size_t prefill_grad_workspace_bytes(const lbca_prefill_grad_args& a) {
  return (size_t)((a.batch * a.q_len * a.q_heads * 4 + 15) / 16 * 16);
}

hipError_t launch_prefill_grad(const lbca_prefill_grad_args& a, void* workspace, hipStream_t stream) {
  const bool shared = a.pooled_v == nullptr;
  const int64_t G = a.q_heads / a.kv_heads;
  float* dvec = static_cast<float*>(workspace);
  hipError_t e;
  if (!a.accumulate) {
    const int64_t pooled_elems = a.batch * a.kv_heads * a.entries * a.dim;
    if ((e = zero_f32(a.grad_pooled_k, pooled_elems, stream)) != hipSuccess) return e;
    if (!shared && (e = zero_f32(a.grad_pooled_v, pooled_elems, stream)) != hipSuccess) return e;
    if ((e = zero_f32(a.grad_sink, a.q_heads, stream)) != hipSuccess) return e;
    if (a.q_len == 0) {  // no queries: every raw row's gradient is zero too
      const int64_t raw_elems = a.batch * a.kv_heads * a.raw_rows * a.dim;
      if ((e = zero_f32(a.grad_raw_k, raw_elems, stream)) != hipSuccess) return e;
      if (!shared && (e = zero_f32(a.grad_raw_v, raw_elems, stream)) != hipSuccess) return e;
    }
  }
  if (a.q_len == 0) return hipSuccess;
  PrepParams pp{};
  pp.dout = static_cast<const bf16_t*>(a.grad_out);
  pp.out = a.out;
  pp.lse = a.lse;
  pp.sink = a.grad_sink ? a.sink : nullptr;
  pp.dvec = dvec;
  pp.dq = a.grad_q;
  pp.dsink = a.grad_sink;
  pp.rows = a.batch * a.q_len;
  pp.hq = a.q_heads;
  pp.dim = a.dim;
  pp.out_f32 = a.out_dtype == LBCA_F32;
  attn_grad_prep_kernel<<<dim3((unsigned)((pp.rows + 63) / 64), (unsigned)a.q_heads), 256, 0, stream>>>(pp);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  GradParams p{};
  p.q = static_cast<const bf16_t*>(a.q);
  p.dout = static_cast<const bf16_t*>(a.grad_out);
  p.lse = a.lse;
  p.dvec = dvec;
  p.pk = static_cast<const bf16_t*>(a.pooled_k);
  p.pv = static_cast<const bf16_t*>(a.pooled_v);
  p.rk = static_cast<const bf16_t*>(a.raw_k);
  p.rv = static_cast<const bf16_t*>(a.raw_v);
  p.dq = a.grad_q;
  p.dpk = a.grad_pooled_k;
  p.dpv = a.grad_pooled_v;
  p.drk = a.grad_raw_k;
  p.drv = a.grad_raw_v;
  p.q_len = a.q_len; p.hq = a.q_heads; p.hkv = a.kv_heads; p.G = G;
  p.entries = a.entries; p.raw_rows = a.raw_rows; p.q_pos0 = a.q_pos0; p.raw_pos_base = a.raw_pos_base;
  p.m = a.block; p.W = a.window;
  p.mode = a.mode;
  p.accumulate = a.accumulate;
  p.shared = shared;
  int64_t np_last, rb_last;
  lbca_visible_range(a.q_pos0 + a.q_len - 1, a.block, a.window, a.mode, &np_last, &rb_last);
  p.n_pool = (int)np_last;
  p.pool_tiles = (int)((np_last + GK - 1) / GK);
  if (p.pool_tiles > 0) {
    const int64_t t_first = a.mode == LBCA_EXCLUSIVE ? a.block + a.window - 1 : a.block - 1;
    const int64_t i_first = t_first - a.q_pos0 > 0 ? t_first - a.q_pos0 : 0;
    const int64_t rows = (a.q_len - i_first) * G;
    p.pool_splits = (int)((rows + QSPLIT - 1) / QSPLIT);
  }
  p.raw_tiles = (int)((a.raw_rows + GK - 1) / GK);
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  const dim3 grid((unsigned)(p.pool_tiles * p.pool_splits + p.raw_tiles), (unsigned)(a.batch * a.kv_heads));
  if (a.dim == 128) attn_grad_kernel<128><<<grid, 256, 0, stream>>>(p);
  else attn_grad_kernel<64><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace lbca
