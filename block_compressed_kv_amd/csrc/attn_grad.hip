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
// registers.  Each lane works out once which query positions see its key (an
// interval: from the first position whose pooled prefix holds the entry on,
// or the positions whose window holds the raw position), so a score's mask is
// two integer compares.  The workgroup walks the positions that can see any of
// its keys (for pooled entries split across workgroups in runs of 512
// positions) in tiles of 32 positions of one query head, the heads of the GQA
// group innermost, staged through LDS with the next tile prefetched into
// registers.  Per tile and wave, on v_mfma_f32_32x32x16_bf16:
//   S = Q K^T and dP = dO V^T       (positions x the wave's keys, over dims)
//   dV^T += dO^T P, dK^T += Q^T dS  (over the 32 positions; P and dS feed
//                                    straight from the accumulator layout, dO^T
//                                    and Q^T come from transposing LDS reads)
//   dQ  = dS K                      (dS goes through LDS transposed; each wave
//                                    covers 32 dims, then adds its partial to
//                                    the fp32 dQ with atomics)
// Raw-position gradients have one owner and are stored; a pooled entry's
// gradient is the sum over the runs that touch it, so each run stores its
// partial in the workspace and a reduction kernel adds them up (many runs
// adding into the same entries with atomics at the same time serialise).
#include "device_util.h"
#include "lbca_internal.h"

namespace lbca {

namespace {

constexpr int GK = 128;      // keys per workgroup
constexpr int GQ = 32;       // query positions per tile
constexpr int PSPLIT = 512;  // query positions per workgroup on the pooled series

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
  float* part;  // pooled-entry partials: [batch * kv_heads][pool tile][split][128 keys][K, V][dim]
  float* drk;
  float* drv;
  int64_t entries, raw_rows;
  int q_len, hq, hkv, G, q_pos0, raw_pos_base, m, W;
  int mode, accumulate, shared;
  int n_pool, pool_tiles, pool_splits, raw_tiles;
  float scale, scale_log2;
};

// Element strides of the gradient kernel's tensors: q, dout, dq {sequence,
// query, head}; K, V and the raw gradients {sequence, KV head, row}.  A kernel
// argument of its own: held in GradParams they made the register allocation
// of the 128-dim kernel spill.
struct GradStrides {
  Str q, dout, dq, pk, pv, rk, rv, drk, drv;
};

// Position of 16-byte chunk c of row r in an LDS tile of 32 query rows: 8
// consecutive rows read at one chunk, and 4 consecutive rows read at 4 aligned
// chunks (two transposing 16-lane groups), land in distinct banks.
template <int D>
__device__ __forceinline__ int qswz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1);
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

// DN: every tensor of the call dense; the kernel then works its offsets out
// from the sizes and leaves the strides unread.
template <int D, bool DN>
__global__ __launch_bounds__(512, 1) void attn_grad_kernel(GradParams p, GradStrides ST) {
  constexpr int DS = D / 16;                  // 16-dim slices of the S / dP contraction
  constexpr int DB = D / 32;                  // 32-dim blocks of dV^T / dK^T
  constexpr int DBH = DB / 2;                 // blocks of one wave's half of the dims
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int KSL = D == 128 ? 8 : 4;       // 16-key slices of a wave's dQ contraction
  constexpr int TCH = GQ * CH;                // chunks of one tile of one tensor
  static_assert(2 * TCH == 512 || TCH == 512, "staging: one chunk per thread and tensor, or one in all");
  __shared__ __attribute__((aligned(16))) bf16_t sk[GK * D];     // the workgroup's K rows
  __shared__ __attribute__((aligned(16))) bf16_t sv[GK * D];     // and V rows
  __shared__ __attribute__((aligned(16))) bf16_t sq[2][GQ * D];
  __shared__ __attribute__((aligned(16))) bf16_t sdo[2][GQ * D];
  __shared__ __attribute__((aligned(16))) bf16_t sdst[GK * GQ];  // dS^T: row = key, 32 query columns
  __shared__ __attribute__((aligned(16))) float s_l2[2][GQ];
  __shared__ __attribute__((aligned(16))) float s_dv[2][GQ];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 3, dh = wave >> 2;  // this wave's 32 keys and half of the dims
  const int n = lane & 31, h = lane >> 5, j16 = lane & 15, g4 = lane >> 4;
  const int bh = blockIdx.y;
  const int b = bh / p.hkv, kvh = bh % p.hkv;
  const int G = p.G;
  const int q_end = p.q_pos0 + p.q_len;  // one past the last query position
  const int wi = blockIdx.x;
  const bool pooled = wi < p.pool_tiles * p.pool_splits;

  // keys [k0, k0 + nkeys) of one series; query positions [t_begin, t_end)
  int k0, nkeys, t_begin, t_end;
  if (pooled) {
    const int tile = wi / p.pool_splits, split = wi % p.pool_splits;
    k0 = tile * GK;
    nkeys = min(GK, p.n_pool - k0);
    // first position whose pooled prefix includes entry k0
    const int t_first = p.mode == LBCA_EXCLUSIVE ? (k0 + 1) * p.m + p.W - 1 : (k0 + 1) * p.m - 1;
    t_begin = max(t_first, p.q_pos0) + split * PSPLIT;
    t_end = min(t_begin + PSPLIT, q_end);
    if (t_begin >= q_end) return;  // nothing in this run: the entries' gradients were set beforehand
  } else {
    k0 = (wi - p.pool_tiles * p.pool_splits) * GK;
    nkeys = (int)min((int64_t)GK, p.raw_rows - k0);
    // queries seeing some position in [p0, p1]: t >= p0 and raw_begin(t) <= p1
    const int p0 = p.raw_pos_base + k0, p1 = p0 + nkeys - 1;
    const int t_last = p.mode == LBCA_EXCLUSIVE ? (p1 / p.m + 1) * p.m + p.W - 2 : p1 + p.W - 1;
    t_begin = max(p0, p.q_pos0);
    t_end = max(t_begin, min(t_last + 1, q_end));
  }

  // first K and V rows of the workgroup and their row strides (a shared series
  // reads values with the key strides; strides as values: a select between
  // argument fields by reference would become a private-memory lookup)
  const bf16_t* kser = pooled ? p.pk : p.rk;
  const bf16_t* vser = pooled ? (p.shared ? p.pk : p.pv) : (p.shared ? p.rk : p.rv);
  int64_t ksr = D, vsr = D;
  if constexpr (DN) {
    const int64_t key_base = pooled ? (int64_t)bh * p.entries + k0 : (int64_t)bh * p.raw_rows + k0;
    kser += key_base * D;
    vser += key_base * D;
  } else {
    const int64_t ks0 = pooled ? ST.pk.s0 : ST.rk.s0, ks1 = pooled ? ST.pk.s1 : ST.rk.s1;
    const int64_t vs0 = p.shared ? ks0 : pooled ? ST.pv.s0 : ST.rv.s0;
    const int64_t vs1 = p.shared ? ks1 : pooled ? ST.pv.s1 : ST.rv.s1;
    ksr = pooled ? ST.pk.s2 : ST.rk.s2;
    vsr = p.shared ? ksr : pooled ? ST.pv.s2 : ST.rv.s2;
    kser += b * ks0 + kvh * ks1 + k0 * ksr;
    vser += b * vs0 + kvh * vs1 + k0 * vsr;
  }

  // the workgroup's K and V rows into LDS (rows past the series read as
  // zeros), chunk c of row r at position c ^ qswz(r)
  for (int idx = tid; idx < GK * CH; idx += 512) {
    const int r = idx / CH, c = idx % CH;
    const bool ok = r < nkeys;
    const uint4 vk = ok ? *reinterpret_cast<const uint4*>(kser + r * ksr + 8 * c) : make_uint4(0, 0, 0, 0);
    const uint4 vv = ok ? *reinterpret_cast<const uint4*>(vser + r * vsr + 8 * c) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&sk[r * D + 8 * (c ^ qswz<D>(r))]) = vk;
    *reinterpret_cast<uint4*>(&sv[r * D + 8 * (c ^ qswz<D>(r))]) = vv;
  }
  const int key_rel = 32 * kw + n;
  const bool key_ok = key_rel < nkeys;
  // the query positions that see this lane's key: [vis_lo, vis_hi]
  int vis_lo, vis_hi;
  if (!key_ok) {
    vis_lo = 0x7fffffff;
    vis_hi = -1;
  } else if (pooled) {
    const int j = k0 + key_rel;
    vis_lo = p.mode == LBCA_EXCLUSIVE ? (j + 1) * p.m + p.W - 1 : (j + 1) * p.m - 1;
    vis_hi = 0x7fffffff;
  } else {
    const int pos = p.raw_pos_base + k0 + key_rel;
    vis_lo = pos;
    vis_hi = p.mode == LBCA_EXCLUSIVE ? (pos / p.m + 1) * p.m + p.W - 2 : pos + p.W - 1;
  }
  // dQ is the first half's job: wave kw covers 32 dims (all 128 keys at 128
  // dims; at 64 dims the four waves split dims x key halves)
  const bool do_dq = dh == 0;
  const int dq_db = D == 128 ? kw : (kw & 1);
  const int dq_kb = D == 128 ? 0 : 64 * (kw >> 1);

  f32x16 dva[DBH], dka[DBH];
#pragma unroll
  for (int i = 0; i < DBH; ++i) dva[i] = dka[i] = f32x16{};

  // tiles: 32 positions (from t_begin) x each query head of the group, heads inner
  const int n_tiles = ((t_end - t_begin + GQ - 1) / GQ) * G;
  const int qh0 = kvh * G;

  // staging of one tile: one 16-byte chunk of Q and of dO per thread at 128
  // dims (Q by threads 0..255 and dO by 256..511 at 64 dims); threads 0..31
  // also one row's lse and D
  constexpr bool BOTH = TCH == 512;
  const int st_idx = BOTH ? tid : (tid & (TCH - 1));
  const int st_row = st_idx / CH, st_ch = st_idx % CH;
  const int st_pos = st_row * D + 8 * (st_ch ^ qswz<D>(st_row));
  uint4 stq, sto;
  float st_l2, st_dv;
  auto fetch = [&](int it) __attribute__((always_inline)) {
    const int tp = t_begin + GQ * (it / G), hq = qh0 + it % G;
    const int t = min(tp + st_row, t_end - 1);  // rows past the run repeat its last row (masked)
    const int64_t i = t - p.q_pos0;
    if constexpr (DN) {  // one row offset serves q and dout
      const int64_t off = (((int64_t)b * p.q_len + i) * p.hq + hq) * D + 8 * st_ch;
      if (BOTH || tid < TCH) stq = *reinterpret_cast<const uint4*>(p.q + off);
      if (BOTH || tid >= TCH) sto = *reinterpret_cast<const uint4*>(p.dout + off);
    } else {
      if (BOTH || tid < TCH)
        stq = *reinterpret_cast<const uint4*>(p.q + (int64_t)b * ST.q.s0 + i * ST.q.s1 + (int64_t)hq * ST.q.s2 +
                                              8 * st_ch);
      if (BOTH || tid >= TCH)
        sto = *reinterpret_cast<const uint4*>(p.dout + (int64_t)b * ST.dout.s0 + i * ST.dout.s1 +
                                              (int64_t)hq * ST.dout.s2 + 8 * st_ch);
    }
    const int tr = min(tp + (tid & 31), t_end - 1);
    const int64_t rid = ((int64_t)b * p.q_len + (tr - p.q_pos0)) * p.hq + hq;
    if (tid < GQ) {
      st_l2 = p.lse[rid];
      st_dv = p.dvec[rid];
    }
  };
  auto stash = [&](int it, int buf) __attribute__((always_inline)) {
    if (BOTH || tid < TCH) *reinterpret_cast<uint4*>(&sq[buf][st_pos]) = stq;
    if (BOTH || tid >= TCH) *reinterpret_cast<uint4*>(&sdo[buf][st_pos]) = sto;
    if (tid < GQ) {
      const int tp = t_begin + GQ * (it / G);
      const bool ok = tp + tid < t_end;
      s_l2[buf][tid] = ok ? st_l2 * kLog2e : __builtin_inff();
      s_dv[buf][tid] = ok ? st_dv : 0.f;
    }
  };

  if (n_tiles > 0) {
    fetch(0);
    stash(0, 0);
  }
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < n_tiles;
    if (more) fetch(it + 1);
    const bf16_t* tq = sq[buf];
    const bf16_t* tdo = sdo[buf];
    const int tp = t_begin + GQ * (it / G), hq = qh0 + it % G;

    // S = Q K^T, dP = dO V^T: lane (key n, h) gets rows 8 (e / 4) + 4 h + e % 4
    f32x16 sacc = {}, dpacc = {};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const int pos = n * D + 8 * ((2 * s + h) ^ qswz<D>(n));
      const bf16x8 aq = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&tq[pos]));
      const bf16x8 ao = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&tdo[pos]));
      const int kpos = key_rel * D + 8 * ((2 * s + h) ^ qswz<D>(key_rel));
      const bf16x8 bk = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sk[kpos]));
      const bf16x8 bv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&sv[kpos]));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bk, sacc, 0, 0, 0);
      dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, bv, dpacc, 0, 0, 0);
    }

    // probabilities and scaled dS; row r sees this lane's key iff its position is
    // in [vis_lo, vis_hi] (rows past the run have lse +inf, so P = 0)
    // (computed in place: sacc becomes P, dpacc becomes dS)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r0 = 8 * qq + 4 * h;
      const float4 l2 = *reinterpret_cast<const float4*>(&s_l2[buf][r0]);
      const float4 dv = *reinterpret_cast<const float4*>(&s_dv[buf][r0]);
      const float l2a[4] = {l2.x, l2.y, l2.z, l2.w}, dva4[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int e = 4 * qq + rr, t = tp + r0 + rr;
        const bool vis = t >= vis_lo && t <= vis_hi;
        const float x = vis ? sacc[e] * p.scale_log2 - l2a[rr] : kNegInf;
        const float pr = fast_exp2(x);
        sacc[e] = pr;
        dpacc[e] = pr * (dpacc[e] - dva4[rr]) * p.scale;
      }
    }
    uint32_t pw[8], dw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pw[i] = pack_bf16x2(sacc[2 * i], sacc[2 * i + 1]);
      dw[i] = pack_bf16x2(dpacc[2 * i], dpacc[2 * i + 1]);
    }
    const bf16x8 pb0 = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    const bf16x8 pb1 = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
    const bf16x8 db0 = __builtin_bit_cast(bf16x8, make_uint4(dw[0], dw[1], dw[2], dw[3]));
    const bf16x8 db1 = __builtin_bit_cast(bf16x8, make_uint4(dw[4], dw[5], dw[6], dw[7]));

    // dS^T into LDS (one wave of each pair): row key_rel, query columns 8 qq + 4 h .. +3
    if (do_dq) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        *reinterpret_cast<uint2*>(&sdst[key_rel * GQ + 8 * (qq ^ ((key_rel >> 2) & 3)) + 4 * h]) =
            make_uint2(dw[2 * qq], dw[2 * qq + 1]);
    }

    // dV^T += dO^T P, dK^T += Q^T dS over the tile's rows, on this wave's half
    // of the dims: k slice ks holds rows 16 ks + 4 h .. +3 and 16 ks + 8 + 4 h
    // .. +3 (the accumulator order)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ra = 16 * ks + 4 * (g4 >> 1) + (j16 >> 2), rb2 = ra + 8;
#pragma unroll
      for (int i = 0; i < DBH; ++i) {
        const int c = 4 * (DBH * dh + i) + 2 * (g4 & 1) + ((j16 & 3) >> 1);
        const int pa = ra * D + 8 * (c ^ qswz<D>(ra)) + 4 * (j16 & 1);
        const int pbb = rb2 * D + 8 * (c ^ qswz<D>(rb2)) + 4 * (j16 & 1);
        const bf16x8 aot = tr_pair(&tdo[pa], &tdo[pbb]);
        const bf16x8 aqt = tr_pair(&tq[pa], &tq[pbb]);
        dva[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aot, ks ? pb1 : pb0, dva[i], 0, 0, 0);
        dka[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aqt, ks ? db1 : db0, dka[i], 0, 0, 0);
      }
    }
    __syncthreads();
    // The next tile into the other buffer (free since the last barrier) before
    // this tile's dQ atomics: the store waits for the tile's loads, and
    // vector-memory operations complete in order, so placed after the atomics
    // it would wait for them too.
    if (more) stash(it + 1, buf ^ 1);

    // dQ (rows x this wave's 32 dims) = dS K over its key range; K^T from LDS
    if (do_dq) {
      f32x16 dqa = {};
#pragma unroll
      for (int s = 0; s < KSL; ++s) {
        const int ka = dq_kb + 16 * s + 8 * (g4 >> 1) + (j16 >> 2), kb2 = ka + 4;
        const int c = 2 * (g4 & 1) + ((j16 & 3) >> 1);
        const bf16x8 ad = tr_pair(&sdst[ka * GQ + 8 * (c ^ ((ka >> 2) & 3)) + 4 * (j16 & 1)],
                                  &sdst[kb2 * GQ + 8 * (c ^ ((kb2 >> 2) & 3)) + 4 * (j16 & 1)]);
        const int ck = 4 * dq_db + 2 * (g4 & 1) + ((j16 & 3) >> 1);
        const bf16x8 bk = tr_pair(&sk[ka * D + 8 * (ck ^ qswz<D>(ka)) + 4 * (j16 & 1)],
                                  &sk[kb2 * D + 8 * (ck ^ qswz<D>(kb2)) + 4 * (j16 & 1)]);
        dqa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, bk, dqa, 0, 0, 0);
      }
      float* dqrow = DN ? p.dq + (((int64_t)b * p.q_len + (tp - p.q_pos0)) * p.hq + hq) * D + 32 * dq_db + n
                        : p.dq + (int64_t)b * ST.dq.s0 + (int64_t)(tp - p.q_pos0) * ST.dq.s1 +
                              (int64_t)hq * ST.dq.s2 + 32 * dq_db + n;
      const int64_t rstride = DN ? (int64_t)p.hq * D : (int64_t)ST.dq.s1;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 8 * (e >> 2) + 4 * h + (e & 3);
        if (tp + r < t_end) unsafeAtomicAdd(dqrow + r * rstride, dqa[e]);
      }
    }
    __syncthreads();
  }

  // dK, dV of this wave's keys and dims: lane (key n, h) holds dims
  // 32 (DBH dh + i) + 8 qq + 4 h .. +3
  if (!key_ok) return;
  const int64_t krel = k0 + key_rel;
  const int64_t krow = DN ? ((int64_t)bh * p.raw_rows + krel) * D : 0;  // dense: one offset for K and V
  float* const gk_row = DN ? p.drk + krow : p.drk + (int64_t)b * ST.drk.s0 + (int64_t)kvh * ST.drk.s1 + krel * ST.drk.s2;
  float* const gv_row = p.shared ? nullptr
                        : DN     ? p.drv + krow
                                 : p.drv + (int64_t)b * ST.drv.s0 + (int64_t)kvh * ST.drv.s1 + krel * ST.drv.s2;
  // a run's partial: row (bh, tile, split, key) of K then (separate series) V
  const int nser = p.shared ? 1 : 2;
  const int64_t prow = pooled ? ((((int64_t)bh * p.pool_tiles + wi / p.pool_splits) * p.pool_splits + wi % p.pool_splits) *
                                     GK + key_rel) * nser * D
                              : 0;
#pragma unroll
  for (int i = 0; i < DBH; ++i)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int d = 32 * (DBH * dh + i) + 8 * qq + 4 * h;
      float kv[4], vv[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        vv[rr] = dva[i][4 * qq + rr];
        kv[rr] = dka[i][4 * qq + rr] + (p.shared ? vv[rr] : 0.f);
      }
      if (pooled) {
        *reinterpret_cast<float4*>(p.part + prow + d) = make_float4(kv[0], kv[1], kv[2], kv[3]);
        if (!p.shared) *reinterpret_cast<float4*>(p.part + prow + D + d) = make_float4(vv[0], vv[1], vv[2], vv[3]);
      } else {
        float4* pk4 = reinterpret_cast<float4*>(gk_row + d);
        float4 k4 = make_float4(kv[0], kv[1], kv[2], kv[3]);
        if (p.accumulate) {
          const float4 o = *pk4;
          k4.x += o.x; k4.y += o.y; k4.z += o.z; k4.w += o.w;
        }
        *pk4 = k4;
        if (!p.shared) {
          float4* pv4 = reinterpret_cast<float4*>(gv_row + d);
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
  int64_t hq, dim, q_len;
  int out_f32;
  Str do_st, o_st, dq_st;  // {sequence, query, head}
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
    const int64_t sb = row / p.q_len, si = row % p.q_len;
    auto at = [&](Str st) { return sb * st.s0 + si * st.s1 + (int64_t)hh * st.s2 + 8 * sub; };
    float go[8], o[8];
    load8(p.dout + at(p.do_st), go);
    if (p.out_f32) load8(static_cast<const float*>(p.out) + at(p.o_st), o);
    else load8(static_cast<const bf16_t*>(p.out) + at(p.o_st), o);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(go[i], o[i], acc);
    for (int w = tpr / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w);
    const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    store8(p.dq + at(p.dq_st), z);
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

// Pooled-entry gradients: the sum of the partials of the runs that touched the
// entry's 128-key tile (entries no query sees get 0), stored or added.  One
// thread per 4 dims of one entry.
struct ReduceParams {
  const float* part;
  float* gk;
  float* gv;
  int64_t entries;
  int64_t total;  // batch * kv_heads * entries * dim / 4
  int dim, n_pool, pool_tiles, pool_splits, shared, accumulate;
  int q_pos0, q_end, block, window, mode, hkv;
  Str gk_st, gv_st;  // {sequence, KV head, entry}
};

__global__ __launch_bounds__(256) void attn_grad_reduce_kernel(ReduceParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.total) return;
  const int q4 = p.dim / 4;
  const int d = (int)(i % q4) * 4;
  const int64_t row = i / q4;  // (bh, entry)
  const int j = (int)(row % p.entries);
  const int64_t bh = row / p.entries;
  float4 k4 = make_float4(0.f, 0.f, 0.f, 0.f), v4 = k4;
  if (j < p.n_pool) {
    const int tile = j / GK, k0 = tile * GK;
    const int t_first = p.mode == LBCA_EXCLUSIVE ? (k0 + 1) * p.block + p.window - 1 : (k0 + 1) * p.block - 1;
    const int start = t_first > p.q_pos0 ? t_first : p.q_pos0;
    const int runs = (p.q_end - start + PSPLIT - 1) / PSPLIT;
    const int nser = p.shared ? 1 : 2;
    const float* src = p.part + (((bh * p.pool_tiles + tile) * p.pool_splits) * GK + (j - k0)) * nser * p.dim + d;
    const int64_t step = (int64_t)GK * nser * p.dim;
    for (int r = 0; r < runs; ++r) {
      const float4 a = *reinterpret_cast<const float4*>(src + r * step);
      k4.x += a.x; k4.y += a.y; k4.z += a.z; k4.w += a.w;
      if (!p.shared) {
        const float4 c = *reinterpret_cast<const float4*>(src + r * step + p.dim);
        v4.x += c.x; v4.y += c.y; v4.z += c.z; v4.w += c.w;
      }
    }
  }
  const int64_t b = bh / p.hkv, kvh = bh % p.hkv;
  float4* gk4 = reinterpret_cast<float4*>(p.gk + b * p.gk_st.s0 + kvh * p.gk_st.s1 + (int64_t)j * p.gk_st.s2 + d);
  if (p.accumulate) {
    const float4 o = *gk4;
    k4.x += o.x; k4.y += o.y; k4.z += o.z; k4.w += o.w;
  }
  *gk4 = k4;
  if (!p.shared) {
    float4* gv4 = reinterpret_cast<float4*>(p.gv + b * p.gv_st.s0 + kvh * p.gv_st.s1 + (int64_t)j * p.gv_st.s2 + d);
    if (p.accumulate) {
      const float4 o = *gv4;
      v4.x += o.x; v4.y += o.y; v4.z += o.z; v4.w += o.w;
    }
    *gv4 = v4;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = 0.f;
}

// Zeroes rows [n0][n1][n2] of dim floats at element strides st.
__global__ __launch_bounds__(256) void zero_rows_kernel(float* x, Str st, int64_t n1, int64_t n2, int64_t rows,
                                                        int dim) {
  const int per = dim / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows * per; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / per, c = (i % per) * 4;
    const int64_t r2 = r % n2, r1 = (r / n2) % n1, r0 = r / (n1 * n2);
    *reinterpret_cast<float4*>(x + r0 * st.s0 + r1 * st.s1 + r2 * st.s2 + c) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

hipError_t zero_rows(float* x, const lbca_strides& st, int64_t n0, int64_t n1, int64_t n2, int64_t dim,
                     hipStream_t stream) {
  const int64_t rows = n0 * n1 * n2;
  if (!x || rows <= 0) return hipSuccess;
  const int64_t blocks = (rows * (dim / 4) + 255) / 256;
  zero_rows_kernel<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, stream>>>(x, st, n1, n2, rows, (int)dim);
  return hipGetLastError();
}

hipError_t zero_f32(float* x, int64_t n, hipStream_t stream) {
  if (!x || n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  fill_zero_kernel<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, stream>>>(x, n);
  return hipGetLastError();
}

// pooled-entry tiles of 128 keys, and query runs of 512 positions the first
// tile's entries are seen by (every later tile is seen by no more)
struct GradPlan {
  int n_pool = 0, pool_tiles = 0, pool_splits = 0;
  size_t dvec_bytes = 0, part_bytes = 0;
};

GradPlan grad_plan(const lbca_prefill_grad_args& a) {
  GradPlan g;
  g.dvec_bytes = (size_t)((a.batch * a.q_len * a.q_heads * 4 + 255) / 256 * 256);
  if (a.q_len == 0) return g;
  int64_t np_last, rb_last;
  lbca_visible_range(a.q_pos0 + a.q_len - 1, a.block, a.window, a.mode, &np_last, &rb_last);
  g.n_pool = (int)np_last;
  g.pool_tiles = (int)((np_last + GK - 1) / GK);
  if (g.pool_tiles > 0) {
    const int64_t t_first = a.mode == LBCA_EXCLUSIVE ? a.block + a.window - 1 : a.block - 1;
    const int64_t t0 = t_first > a.q_pos0 ? t_first : a.q_pos0;
    g.pool_splits = (int)((a.q_pos0 + a.q_len - t0 + PSPLIT - 1) / PSPLIT);
  }
  const int nser = a.pooled_v == nullptr ? 1 : 2;
  g.part_bytes = (size_t)(a.batch * a.kv_heads) * g.pool_tiles * g.pool_splits * GK * nser * a.dim * 4;
  return g;
}

}  // namespace

size_t prefill_grad_workspace_bytes(const lbca_prefill_grad_args& a) {
  const GradPlan g = grad_plan(a);
  return g.dvec_bytes + g.part_bytes;
}

hipError_t launch_prefill_grad(const lbca_prefill_grad_args& a, void* workspace, hipStream_t stream) {
  const bool shared = a.pooled_v == nullptr;
  const int64_t G = a.q_heads / a.kv_heads;
  const GradPlan g = grad_plan(a);
  float* dvec = static_cast<float*>(workspace);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + g.dvec_bytes);
  hipError_t e;
  if (!a.accumulate) {
    if ((e = zero_f32(a.grad_sink, a.q_heads, stream)) != hipSuccess) return e;
    if (a.q_len == 0) {  // no queries: every key and value gradient is zero
      const int64_t B = a.batch, H = a.kv_heads, N = a.entries, R = a.raw_rows, d = a.dim;
      if ((e = zero_rows(a.grad_pooled_k, a.grad_pooled_k_st, B, H, N, d, stream)) != hipSuccess) return e;
      if (!shared && (e = zero_rows(a.grad_pooled_v, a.grad_pooled_v_st, B, H, N, d, stream)) != hipSuccess)
        return e;
      if ((e = zero_rows(a.grad_raw_k, a.grad_raw_k_st, B, H, R, d, stream)) != hipSuccess) return e;
      if (!shared && (e = zero_rows(a.grad_raw_v, a.grad_raw_v_st, B, H, R, d, stream)) != hipSuccess) return e;
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
  pp.q_len = a.q_len;
  pp.do_st = a.grad_out_st; pp.o_st = a.out_st; pp.dq_st = a.grad_q_st;
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
  p.part = part;
  p.drk = a.grad_raw_k;
  p.drv = a.grad_raw_v;
  p.entries = a.entries;
  p.raw_rows = a.raw_rows;
  p.q_len = (int)a.q_len; p.hq = (int)a.q_heads; p.hkv = (int)a.kv_heads; p.G = (int)G;
  p.q_pos0 = (int)a.q_pos0; p.raw_pos_base = (int)a.raw_pos_base;
  p.m = (int)a.block; p.W = (int)a.window;
  p.mode = a.mode;
  p.accumulate = a.accumulate;
  p.shared = shared;
  p.n_pool = g.n_pool;
  p.pool_tiles = g.pool_tiles;
  p.pool_splits = g.pool_splits;
  p.raw_tiles = (int)((a.raw_rows + GK - 1) / GK);
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  GradStrides gs;
  gs.q = a.q_st; gs.dout = a.grad_out_st; gs.dq = a.grad_q_st;
  gs.pk = a.pooled_k_st; gs.pv = a.pooled_v_st; gs.rk = a.raw_k_st; gs.rv = a.raw_v_st;
  gs.drk = a.grad_raw_k_st; gs.drv = a.grad_raw_v_st;
  const dim3 grid((unsigned)(p.pool_tiles * p.pool_splits + p.raw_tiles), (unsigned)(a.batch * a.kv_heads));
  const int64_t B = a.batch, Tq = a.q_len, Hq = a.q_heads, Hk = a.kv_heads, d = a.dim;
  const bool dn = dense_strides(a.q, a.q_st, {B, Tq, Hq}, d) && dense_strides(a.grad_out, a.grad_out_st, {B, Tq, Hq}, d) &&
                  dense_strides(a.grad_q, a.grad_q_st, {B, Tq, Hq}, d) &&
                  dense_strides(a.pooled_k, a.pooled_k_st, {B, Hk, a.entries}, d) &&
                  dense_strides(a.pooled_v, a.pooled_v_st, {B, Hk, a.entries}, d) &&
                  dense_strides(a.raw_k, a.raw_k_st, {B, Hk, a.raw_rows}, d) &&
                  dense_strides(a.raw_v, a.raw_v_st, {B, Hk, a.raw_rows}, d) &&
                  dense_strides(a.grad_raw_k, a.grad_raw_k_st, {B, Hk, a.raw_rows}, d) &&
                  dense_strides(a.grad_raw_v, a.grad_raw_v_st, {B, Hk, a.raw_rows}, d);
  if (a.dim == 128) dn ? attn_grad_kernel<128, true><<<grid, 512, 0, stream>>>(p, gs)
                       : attn_grad_kernel<128, false><<<grid, 512, 0, stream>>>(p, gs);
  else dn ? attn_grad_kernel<64, true><<<grid, 512, 0, stream>>>(p, gs)
          : attn_grad_kernel<64, false><<<grid, 512, 0, stream>>>(p, gs);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  ReduceParams rp{};
  rp.part = part;
  rp.gk = a.grad_pooled_k;
  rp.gv = a.grad_pooled_v;
  rp.entries = a.entries;
  rp.total = a.batch * a.kv_heads * a.entries * a.dim / 4;
  rp.dim = (int)a.dim;
  rp.n_pool = g.n_pool;
  rp.pool_tiles = g.pool_tiles;
  rp.pool_splits = g.pool_splits;
  rp.shared = shared;
  rp.accumulate = a.accumulate;
  rp.q_pos0 = (int)a.q_pos0;
  rp.q_end = (int)(a.q_pos0 + a.q_len);
  rp.block = (int)a.block;
  rp.window = (int)a.window;
  rp.mode = a.mode;
  rp.hkv = (int)a.kv_heads;
  rp.gk_st = a.grad_pooled_k_st; rp.gv_st = a.grad_pooled_v_st;
  if (rp.total > 0)
    attn_grad_reduce_kernel<<<(unsigned)((rp.total + 255) / 256), 256, 0, stream>>>(rp);
  return hipGetLastError();
}

}  // namespace lbca
