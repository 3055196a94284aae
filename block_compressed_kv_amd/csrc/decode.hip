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
// wave w takes tiles w, w+NW, ... and keeps up to three tiles' global loads
// in flight (register buffers refilled as soon as they are consumed); with one
// split the first pooled tiles are requested before the position is read.
// Scores are computed transposed,
// S^T[row, head] = K[row, :] . Q[head, :], with v_mfma_f32_16x16x32_bf16 whose
// A operand is loaded straight from global memory in row-major K layout: every
// lane holds scores of one head, and the softmax max/sum need one 16-lane and
// one 32-lane swap.  P^T is already the B operand of the MFMA for
// O^T = V^T P^T; V rows are staged row-major in a per-wave LDS tile and each
// A operand is gathered with transposing LDS reads (ds_read_b64_tr_b16).
//
// When there are too few units to occupy every CU, DS "twin" workgroups share
// a unit: each computes the full Q.K scores (identical softmax state, so no
// merge is needed) but only 1/DS of the output dims, loading all K rows and
// only its slice of V.  Twins get linear workgroup ids 8 apart, which the
// dispatcher places on the same XCD, so the second read of K hits its L2.
//
// Small decodes are bound by each wave's instruction chain and by memory
// latency rather than by bytes, so the per-tile path is kept short: raw
// v_exp_f32, lane swaps instead of LDS permutes, the accumulator rescale
// skipped when no running max moved, 32-bit index arithmetic, and a
// single-barrier merge of the waves.  With one split the workgroup finishes
// its heads (sink, normalisation, -t rotation, LSE); with several, each
// workgroup writes an unnormalised partial (acc, max, sum) and
// decode_merge_kernel combines them in a fixed order (bitwise reproducible).
// No device-scope fence is used anywhere: on this multi-XCD part a
// device-scope release/acquire writes back and invalidates the XCD's L2.
#include <mutex>
#include <type_traits>

#include "cache_common.h"
#include "decode_common.h"

#ifndef LBCA_DECODE_TILES_PER_WAVE
#define LBCA_DECODE_TILES_PER_WAVE 4  // tiles per wave above which a unit's rows are split
#endif

namespace lbca {

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
// apart).  freq[k] = turns per position of pair k (an LDS table, so the
// double-precision frequencies are not held in registers through the tile
// loop).  Every lane of the wave must call this (it uses lane swaps).
template <int D, int RD>
__device__ __forceinline__ void treat_row(uint4 (&r)[D / 32], double pos, bool ok, float eps,
                                          const double* freq) {
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
        rope_cos_sin_turns(pos * freq[k], &c, &sn);
        const float x1 = a[i], x2 = b[i];
        a[i] = x1 * c - x2 * sn;
        b[i] = x2 * c + x1 * sn;
      }
      r[s] = pack8(a);
      r[s + SH] = pack8(b);
    }
  }
}

// One R-row tile in registers: all D dims of K (MFMA A operands) and this
// workgroup's slice of V (DV dims) when V is a separate series.
template <int D, int R, int DS, bool SHARED>
struct Tile {
  uint4 k[R / 16][D / 32];
  uint4 v[SHARED ? 1 : R / 16][SHARED ? 1 : D / 32 / DS];
  unsigned valid[R / 16];
};

// Byte addresses of one (sequence, KV head) slice: the pooled and raw rows of
// K and V (V aliases K for a shared series), and a stand-in row that rows
// outside the list read instead (this head group's first query row: always
// valid memory and already in cache, so such loads cost no HBM traffic).
struct Slices {
  uintptr_t pk, pv, rk, rv, dummy;
  uintptr_t tk, tv;  // fused cache step: the new token's rows
  uint32_t pks, pvs, rks, rvs;  // row strides in bytes
};

// Selected ids of one workgroup's range are staged in LDS (a global load of
// an id right before the rows it names would make every wait on it a wait
// for all older loads of the wave).
constexpr int kSelLds = 1024;

template <int D, int R, int DS, bool SHARED>
__device__ __forceinline__ void clear_valid(Tile<D, R, DS, SHARED>& T) {
#pragma unroll
  for (int h = 0; h < R / 16; ++h) T.valid[h] = 0;
}

// Issue the loads of one tile of the visible-row list.  Tile ids: [0, tiles_p)
// pooled or selected rows, [tiles_p, pad_p) empty, [pad_p, ...) raw rows.  A
// tile that is not live (outside this workgroup's range) has no rows.  Rows
// not in the list read the stand-in row and get a clear valid bit (their
// scores are masked and their values zeroed when staged): the loads of a tile
// carry no branch, since a load that may be skipped makes the compiler wait
// for every older load before the next use of any.  Tiles past the range are
// not loaded at all: each load instruction costs address-unit time even when
// its data is cached, and a wave cannot end before its loads return.
// ids: the selected ids of list positions r0, r0+1, ... (LDS).
template <int D, int R, int DS, bool SHARED, bool FUSED = false>
__device__ __forceinline__ void load_tile(Tile<D, R, DS, SHARED>& T, const int* ids, int r0,
                                          bool sel, const Slices& sl, const SeqView& sv,
                                          int tiles_p, int pad_p, int tile, bool live, int n,
                                          int kq, int dv0) {
  constexpr int KS = D / 32, NH = R / 16, KV = KS / DS;
  const bool is_raw = tile >= pad_p;
  const bool empty = !is_raw && tile >= tiles_p;
  const int v0 = is_raw ? (tile - pad_p) * R : tile * R;
  const int count = (!live || empty) ? 0 : is_raw ? sv.n_raw : sv.n_sel;
  const uintptr_t kb = is_raw ? sl.rk : sl.pk;  // wave-uniform selects
  const uintptr_t vb = is_raw ? sl.rv : sl.pv;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int v = v0 + 16 * h + n;
    bool ok = v < count;
    int row;
    if (is_raw) {
      row = (int)sv.raw_row0 + v;
    } else {
      row = v;
      if (sel) row = ids[ok ? min(v - r0, kSelLds - 1) : 0];
      ok = ok && row >= 0 && row < sv.n_pooled;
    }
    const uint64_t off = (uint64_t)(uint32_t)row * (is_raw ? sl.rks : sl.pks) + 16u * kq;
    // fused cache step: the raw row at the position is the new token's input row
    const bool tok = FUSED && is_raw && v == sv.n_raw - 1;
    const uintptr_t kp = ok ? (tok ? sl.tk + 16u * kq : kb + off) : sl.dummy + 16u * kq;
#pragma unroll
    for (int s = 0; s < KS; ++s) T.k[h][s] = ldg16(kp + 64u * s);
    if constexpr (!SHARED) {
      const uint64_t offv = (uint64_t)(uint32_t)row * (is_raw ? sl.rvs : sl.pvs) + 16u * kq;
      const uintptr_t vp = (ok ? (tok ? sl.tv + 16u * kq : vb + offv) : sl.dummy + 16u * kq) + 2u * dv0;
#pragma unroll
      for (int s = 0; s < KV; ++s) T.v[h][s] = ldg16(vp + 64u * s);
    }
    T.valid[h] = (unsigned)(__ballot(ok) & 0xffffull);
  }
}

// One decode workgroup's work (workgroup id bid).  FUSED (lbca_decode_step):
// the raw row at the position is read from the new token's input and the raw
// base follows from the position; the workgroup that owns split 0 of a
// (sequence, KV head) also appends the token to the ring (cp): its rows are
// requested first and stored once the position is known; when the token
// completes a block it returns that cache row (else -1), so the caller pools
// the block after the decode.
template <int D, int R, int NW, int DS, bool SHARED, int RD, bool TREAT, bool SPEC, bool FUSED, bool DN,
          typename TZ = float>
__device__ __forceinline__ int decode_body(const DecodeParams& p, unsigned bid, const CacheParams* cp = nullptr) {
  constexpr int KS = D / 32, NH = R / 16;
  constexpr int DV = D / DS;                         // output dims of this workgroup
  constexpr int KV = DV / 32, DT = DV / 16, PITCH = DV + 16;
  constexpr int STAGE = R * PITCH;                   // bf16 elements of one wave's value stage
  constexpr bool PAR_MERGE = NW * 16 * DV * 4 <= NW * STAGE * 2;
  static_assert(NW * STAGE * 2 >= 16 * DV * 4, "merge buffer must fit in the stages");
  static_assert(RD <= DV, "rotated dims must lie in one dim slice");
  __shared__ __attribute__((aligned(16))) bf16_t lds[NW * STAGE];
  __shared__ float s_ml[NW][16][2];
  __shared__ float s_w[NW][16];
  __shared__ float s_M[16], s_L[16], s_inv[16], s_lse[16];
  __shared__ float s_sink[16];  // sink logits of the head slots (the one-barrier merge)
  __shared__ double s_freq[RD > 0 ? RD / 2 : 1];  // RoPE turns per position, pair k
  __shared__ int s_ids[SPEC ? 1 : kSelLds];        // selected ids of this workgroup's range

  preload_params(p);
  if constexpr (!DN) preload_strides(p);
  const DecStr ST = dec_strides<DN, D>(p, 1);  // one query row per sequence here
  if constexpr (FUSED)  // the cache-step fields too, in the same batch of scalar loads
    asm volatile("" ::"s"(cp->x_new), "s"(cp->v_new), "s"(cp->z_new), "s"(cp->raw_x), "s"(cp->raw_v),
                 "s"(cp->raw_z), "s"(cp->raw_pos_base), "s"(cp->ring), "s"(p.ring));
  CacheStr CS{};  // the cache step's strides (fused step; dense: from the decode's sizes)
  if constexpr (FUSED) {
    if constexpr (DN) {
      const Str tok{p.hkv * D, D, 0}, ring{p.hkv * p.raw_rows * D, p.raw_rows * D, D};
      CS.xn = CS.vn = CS.zn = tok;
      CS.rx = CS.rv = CS.rz = ring;
    } else {
      CS = cache_strides<false>(*cp);
    }
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile choices stay scalar
  const int n = lane & 15, kq = lane >> 4;
  // linear id -> (unit, split, dim slice); twins of a unit sit 8 ids apart (same XCD)
  unsigned u = bid, dh = 0;
  if constexpr (DS > 1) {
    const unsigned rest = bid >> 3;
    dh = rest % DS;
    u = (rest / DS) * 8 + (bid & 7);
  }
  if (u >= (unsigned)p.units * (unsigned)p.splits) return -1;  // padding of the XCD mapping
  const int split = (int)(u % (unsigned)p.splits);
  const unsigned unit = u / (unsigned)p.splits;
  const unsigned uy = (unsigned)(p.hkv * p.head_groups);
  const int64_t b = unit / uy;
  const unsigned y = unit % uy;
  const int hg = (int)(y % (unsigned)p.head_groups);
  const int64_t kvh = y / (unsigned)p.head_groups;
  const int dv0 = (int)dh * DV;                      // first output dim of this workgroup
  const int slot0 = hg * 16;
  const int nvalid = (int)(p.G - slot0 < 16 ? p.G - slot0 : 16);
  const int64_t head0 = kvh * p.G + slot0;  // first query head of the unit
  const bool head_ok = n < nvalid;
  const int own_row = (FUSED && split == 0 && dh == 0 && hg == 0) ? (int)(b * p.hkv + kvh) : -1;
  // fused step: the owner's first dim/8 lanes request the new token's rows
  // before anything else, so the wait for them is covered by the wait for the
  // position (vector loads return in order)
  uint4 tok_k = {}, tok_v = {}, tok_z0 = {}, tok_z1 = {};
  const bool tok_lane = FUSED && own_row >= 0 && tid < D / 8;
  if constexpr (FUSED) {
    if (tok_lane) {
      tok_k = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(cp->x_new) + b * CS.xn.s0 +
                                              kvh * CS.xn.s1 + 8 * tid);
      tok_v = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(cp->v_new) + b * CS.vn.s0 +
                                              kvh * CS.vn.s1 + 8 * tid);
      const TZ* zs = static_cast<const TZ*>(cp->z_new) + b * CS.zn.s0 + kvh * CS.zn.s1 + 8 * tid;
      tok_z0 = reinterpret_cast<const uint4*>(zs)[0];
      if constexpr (sizeof(TZ) == 4) tok_z1 = reinterpret_cast<const uint4*>(zs)[1];
    }
  }

  // the position first: it is waited for after the first rows are requested
  const EarlyI64 e_pos = load_early(p.pos + b);
  const EarlyI64 e_base = load_early(p.rpb ? p.rpb + b : p.pos + b);
  // queries of this head group as B operands; their addresses do not depend
  // on the position, so they load alongside it.  Padded head slots load head
  // 0's row: a lane's scores, softmax state and output column belong to its
  // own head, and padded heads are never written.  (Loads without a branch
  // keep the count of loads after the position exact for the wait on it.)
  uint4 qr[KS];
  {
    const bf16_t* qrow = p.q + (DN ? (b * p.hq + head0 + (head_ok ? n : 0)) * D
                                   : b * ST.q.s0 + (head0 + (head_ok ? n : 0)) * ST.q.s2) + 8 * kq;
#pragma unroll
    for (int s = 0; s < KS; ++s) qr[s] = *reinterpret_cast<const uint4*>(qrow + 32 * s);
  }
  // Addresses of this (sequence, KV head) slice (none depends on the position).
  Slices sl;
  {
    if constexpr (DN) {  // dense: one slice offset per series (pooled, raw)
      const uint64_t sp = (uint64_t)((b * p.hkv + kvh) * p.entries) * (D * 2);
      const uint64_t sr = (uint64_t)((b * p.hkv + kvh) * p.raw_rows) * (D * 2);
      sl.pk = reinterpret_cast<uintptr_t>(p.pk) + sp;
      sl.rk = reinterpret_cast<uintptr_t>(p.rk) + sr;
      sl.pv = SHARED ? sl.pk : reinterpret_cast<uintptr_t>(p.pv) + sp;
      sl.rv = SHARED ? sl.rk : reinterpret_cast<uintptr_t>(p.rv) + sr;
    } else {
      sl.pk = reinterpret_cast<uintptr_t>(p.pk + b * ST.pk.s0 + kvh * ST.pk.s1);
      sl.rk = reinterpret_cast<uintptr_t>(p.rk + b * ST.rk.s0 + kvh * ST.rk.s1);
      sl.pv = SHARED ? sl.pk : reinterpret_cast<uintptr_t>(p.pv + b * ST.pv.s0 + kvh * ST.pv.s1);
      sl.rv = SHARED ? sl.rk : reinterpret_cast<uintptr_t>(p.rv + b * ST.rv.s0 + kvh * ST.rv.s1);
    }
    sl.pks = 2u * (uint32_t)ST.pk.s2;
    sl.rks = 2u * (uint32_t)ST.rk.s2;
    sl.pvs = SHARED ? sl.pks : 2u * (uint32_t)ST.pv.s2;
    sl.rvs = SHARED ? sl.rks : 2u * (uint32_t)ST.rv.s2;
    sl.dummy = reinterpret_cast<uintptr_t>(p.q + (DN ? (b * p.hq + head0) * D : b * ST.q.s0 + head0 * ST.q.s2));
    if constexpr (FUSED) {
      sl.tk = reinterpret_cast<uintptr_t>(p.tk + b * ST.tk.s0 + kvh * ST.tk.s1);
      sl.tv = reinterpret_cast<uintptr_t>(p.tv + b * ST.tv.s0 + kvh * ST.tv.s1);
    } else {
      sl.tk = sl.tv = 0;
    }
  }
  // Each wave keeps TMAX tiles in flight.  SPEC instances (one split, no
  // selection, launched as such by the host) request their first TMAX tiles,
  // the pooled tiles w, w+NW, ..., now, before the position arrives
  // (visibility is applied once the position is known), and move the raw
  // tiles past slot TMAX*NW of the list.
  constexpr int TMAX = D <= 64 ? 4 : D <= 128 ? (DS > 1 ? 3 : 2) : 1;
  static_assert(!SPEC || D <= 128, "early tiles of wide rows would spill");
  Tile<D, R, DS, SHARED> T[TMAX];
  constexpr bool spec = SPEC;
  if constexpr (SPEC) {
#pragma unroll
    for (int i = 0; i < TMAX; ++i) {
      // no buffer rows left (the first tile is always requested, reading the
      // stand-in row past the buffer, so every path has the same loads)
      if (i > 0 && (wave + i * NW) * R >= p.entries) break;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int e = (wave + i * NW) * R + 16 * h + n;
        const uint64_t off = (uint64_t)e * sl.pks + 16u * kq;
        const bool in = e < p.entries;  // rows past the buffer read the stand-in row
        const uintptr_t kp = in ? sl.pk + off : sl.dummy + 16u * kq;
#pragma unroll
        for (int s = 0; s < KS; ++s) T[i].k[h][s] = ldg16(kp + 64u * s);
        if constexpr (!SHARED) {
          const uint64_t offv = (uint64_t)e * sl.pvs + 16u * kq;
          const uintptr_t vp = (in ? sl.pv + offv : sl.dummy + 16u * kq) + 2u * dv0;
#pragma unroll
          for (int s = 0; s < KV; ++s) T[i].v[h][s] = ldg16(vp + 64u * s);
        }
      }
    }
  }
  int64_t base = 0;
  if constexpr (FUSED) {  // the raw base the cache step writes for this position
    const int64_t t = uniform_value(e_pos);
    int64_t np = 0, rb = 0;
    if (t >= 0) visible_range(t, p.m, p.W, p.mode, &np, &rb);
    base = rb - mod_nonneg(rb, p.ring);
    (void)e_base;
  } else {
    base = p.rpb ? uniform_value(e_base) : 0;
  }
  const SeqView sv = seq_view(p, b, uniform_value(e_pos), base);
  // fused step: the cache row is handed back only when the token completes a
  // block that fits the pooled buffer (the caller then pools it), so the other
  // steps end without the cache step reading the position again
  int pool_row = -1;
  if constexpr (FUSED) {
    const int64_t x = sv.t + 1;
    if (own_row >= 0 && sv.t >= 0 && x % cp->m == 0 && x / cp->m - 1 < cp->entries) pool_row = own_row;
  }
  // Fused step: the token into both ring rows of its slot, and the raw base
  // (lbca_cache_append's rule), once the position is known.  (Stored after
  // the decode work instead, the stores lengthen the owner workgroups' tails:
  // 14.6 against 14.3 us per layer-step.)
  {
    if constexpr (FUSED) {
    if (tok_lane && sv.t >= 0) {
      const int64_t ring = cp->ring, slot = mod_nonneg(sv.t, ring);
      bf16_t* rk = static_cast<bf16_t*>(cp->raw_x) + b * CS.rx.s0 + kvh * CS.rx.s1 + slot * CS.rx.s2 + 8 * tid;
      bf16_t* rv = static_cast<bf16_t*>(cp->raw_v) + b * CS.rv.s0 + kvh * CS.rv.s1 + slot * CS.rv.s2 + 8 * tid;
      TZ* rz = static_cast<TZ*>(cp->raw_z) + b * CS.rz.s0 + kvh * CS.rz.s1 + slot * CS.rz.s2 + 8 * tid;
      const int64_t d0 = 0, d1 = ring * CS.rx.s2, v1 = ring * CS.rv.s2, z1 = ring * CS.rz.s2;
      *reinterpret_cast<uint4*>(rk + d0) = tok_k;
      *reinterpret_cast<uint4*>(rk + d1) = tok_k;
      *reinterpret_cast<uint4*>(rv + d0) = tok_v;
      *reinterpret_cast<uint4*>(rv + v1) = tok_v;
      reinterpret_cast<uint4*>(rz + d0)[0] = tok_z0;
      reinterpret_cast<uint4*>(rz + z1)[0] = tok_z0;
      if constexpr (sizeof(TZ) == 4) {
        reinterpret_cast<uint4*>(rz + d0)[1] = tok_z1;
        reinterpret_cast<uint4*>(rz + z1)[1] = tok_z1;
      }
      if (kvh == 0 && tid == 0) cp->raw_pos_base[b] = base;
    }
    }
  }
  if (!sv.ok) {  // rows do not fit the buffers: NaN, written once per unit and slice
    if (split == 0) {
      for (int i = tid; i < nvalid * DV; i += blockDim.x)
        p.out[b * ST.o.s0 + (head0 + i / DV) * ST.o.s2 + dv0 + i % DV] = __builtin_nanf("");
      if (p.lse && dh == 0 && tid < nvalid) p.lse[b * p.hq + head0 + tid] = __builtin_nanf("");
    }
    return pool_row;
  }
  if constexpr (TREAT) {
    if constexpr (RD > 0) {
      if (tid < RD / 2) s_freq[tid] = rope_turns_per_pos(tid, RD, p.log2_base);
      __syncthreads();
    }
    treat_row<D, RD>(qr, (double)sv.t, head_ok, p.eps, s_freq);
  }

  const int tiles_p = (sv.n_sel + R - 1) / R;
  const int pad_p = spec && tiles_p < TMAX * NW ? TMAX * NW : tiles_p;  // first raw tile
  const int tiles_total = pad_p + (sv.n_raw + R - 1) / R;
  const int per = (tiles_total + p.splits - 1) / p.splits;
  const int t0 = split * per;
  const int t1 = t0 + per < tiles_total ? t0 + per : tiles_total;

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16_t* vt = lds + wave * STAGE;
  // transposing-read base of this lane: row 4*kq + n/4, column 4*(n%4)
  const bf16_t* trb = vt + (4 * kq + (n >> 2)) * PITCH + 4 * (n & 3);

  auto process = [&](Tile<D, R, DS, SHARED>& T, int tile) {
    if constexpr (TREAT) {
      if (tile >= pad_p) {
        const int v0 = (tile - pad_p) * R;
#pragma unroll
        for (int h = 0; h < NH; ++h)
          treat_row<D, RD>(T.k[h], (double)(sv.raw_begin + v0 + 16 * h + n), (T.valid[h] >> n) & 1u,
                           p.eps, s_freq);
      }
    }
    // this workgroup's slice of the value rows to the wave's LDS stage (row-major)
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int s = 0; s < KV; ++s) {
        uint4 val;
        if constexpr (SHARED) {  // shared series: V is the (treated) K row, slice dh
          // bitwise select: a conditional pick between array elements would be
          // turned into a dynamically indexed (private memory) array
          val = T.k[h][s];
#pragma unroll
          for (int q = 1; q < DS; ++q) {
            const uint32_t mk = (int)dh == q ? 0xffffffffu : 0u;
            const uint4 w = T.k[h][q * KV + s];
            val = make_uint4((val.x & ~mk) | (w.x & mk), (val.y & ~mk) | (w.y & mk),
                             (val.z & ~mk) | (w.z & mk), (val.w & ~mk) | (w.w & mk));
          }
        } else {
          val = T.v[h][s];
        }
        if (!((T.valid[h] >> n) & 1u)) val = make_uint4(0, 0, 0, 0);  // rows past the list may hold anything
        *reinterpret_cast<uint4*>(&vt[(16 * h + n) * PITCH + 32 * s + 8 * kq]) = val;
      }
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
    uint32_t pw[NH][2];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float pj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pj[j] = fast_exp2(sc[h][j] - mu);
        psum += pj[j];
      }
      pw[h][0] = pack_bf16x2(pj[0], pj[1]);
      pw[h][1] = pack_bf16x2(pj[2], pj[3]);
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
      const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pw[0][0], pw[0][1], pw[1][0], pw[1][1]));
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const s16x4 a0 = lds_read_tr16(trb + 16 * t), a1 = lds_read_tr16(trb + 16 * PITCH + 16 * t);
        const bf16x8 a = __builtin_bit_cast(bf16x8, s16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[t], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const s16x4 pb = __builtin_bit_cast(s16x4, make_uint2(pw[h][0], pw[h][1]));
#pragma unroll
        for (int t = 0; t < DT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_read_tr16(trb + 16 * h * PITCH + 16 * t),
                                                              pb, acc[t], 0, 0, 0);
      }
    }
  };

  // Tile loop: buffer i is computed, then refilled with the tile TMAX*NW
  // further on, so up to TMAX tiles' loads overlap the computation; selected
  // ids are fetched one refill ahead.  Tiles without a visible row (empty
  // padding, past the range) are not computed.
  // selected ids of this range to LDS (the host sizes ranges to fit)
  const bool sel = !SPEC && p.sel != nullptr;  // SPEC instances are launched without a selection
  const int r0 = t0 * R;
  if (sel) {
    int nr = (t1 < tiles_p ? t1 : tiles_p) * R;
    nr = (nr < sv.n_sel ? nr : sv.n_sel) - r0;
    nr = nr < kSelLds ? nr : kSelLds;
    const int32_t* src = p.sel + b * p.k_sel + r0;
    for (int i = tid; i < nr; i += NW * 64) s_ids[i] = src[i];
    __syncthreads();
  }
  if constexpr (TMAX == 1) {
    // wide rows: one buffer, loaded then computed (a refill issued during the
    // computation would need a second buffer and spill)
#pragma unroll 1
    for (int ti = t0 + wave; ti < t1; ti += NW) {
      load_tile<D, R, DS, SHARED, FUSED>(T[0], s_ids, r0, sel, sl, sv, tiles_p, pad_p, ti, true, n, kq, dv0);
      unsigned any = 0;
#pragma unroll
      for (int h = 0; h < NH; ++h) any |= T[0].valid[h];
      if (any) process(T[0], ti);
    }
  } else {
    const int step = TMAX * NW;
    if constexpr (SPEC) {  // first tiles already requested: set their valid bits
#pragma unroll
      for (int i = 0; i < TMAX; ++i)
#pragma unroll
        for (int h = 0; h < NH; ++h)
          T[i].valid[h] = (unsigned)(__ballot((wave + i * NW) * R + 16 * h + n < sv.n_sel) & 0xffffull);
    } else {
#pragma unroll
      for (int i = 0; i < TMAX; ++i) {
        const int ti = t0 + wave + i * NW;
        if (ti < t1) load_tile<D, R, DS, SHARED, FUSED>(T[i], s_ids, r0, sel, sl, sv, tiles_p, pad_p, ti, true, n, kq, dv0);
        else clear_valid(T[i]);
      }
    }
#pragma unroll 1
    for (int g0 = t0 + wave; g0 < t1; g0 += step) {
#pragma unroll
      for (int i = 0; i < TMAX; ++i) {
        const int ti = g0 + i * NW;
        unsigned any = 0;
#pragma unroll
        for (int h = 0; h < NH; ++h) any |= T[i].valid[h];
        if (any) process(T[i], ti);
        const int nt = ti + step;
        if (nt < t1) load_tile<D, R, DS, SHARED, FUSED>(T[i], s_ids, r0, sel, sl, sv, tiles_p, pad_p, nt, true, n, kq, dv0);
        else clear_valid(T[i]);
      }
    }
  }
  l_run = xor16_sum(l_run);
  l_run = xor32_sum(l_run);

  // ---- merge the NW waves (fixed order) ----
  float* buf = reinterpret_cast<float*>(lds);
  if constexpr (PAR_MERGE) {
    // the sink logits of the head slots (requested now: the loads overlap the
    // barrier's wait)
    const float sink_r = p.sink && wave == 0 && kq == 0 ? p.sink[head0 + (head_ok ? n : 0)] : 0.f;
    // Every wave leaves its (max, sum) and its unscaled acc in its own stage
    // (a wave's LDS operations complete in order, so its last reads of the
    // stage are done), one barrier publishes them, and each output thread
    // forms the wave weights of its slot itself.
    if (kq == 0) {
      s_ml[wave][n][0] = m_run;
      s_ml[wave][n][1] = l_run;
      if (wave == 0) s_sink[n] = sink_r;
    }
    if (head_ok) {
      float* dst = reinterpret_cast<float*>(vt) + n * DV + 4 * kq;
#pragma unroll
      for (int t = 0; t < DT; ++t)
        *reinterpret_cast<float4*>(dst + 16 * t) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    }
    __syncthreads();
    // weights exp2(m_w - M) of the waves for slot sl, M and L = sum_w l_w sw_w
    auto weights = [&](int sl, float (&sw)[NW], float& M, float& L) __attribute__((always_inline)) {
      M = kNegInf;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, s_ml[w][sl][0]);
      L = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        sw[w] = s_ml[w][sl][0] == kNegInf ? 0.f : fast_exp2(s_ml[w][sl][0] - M);
        L = fmaf(s_ml[w][sl][1], sw[w], L);
      }
    };
    auto merged = [&](int sl, int dl, const float (&sw)[NW]) __attribute__((always_inline)) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) o = fmaf(buf[w * (STAGE / 2) + sl * DV + dl], sw[w], o);
      return o;
    };
    if (p.splits == 1) {
      constexpr int r = RD, half = RD / 2;
      const bool rot = RD > 0 && (int)dh == DS - 1;
      const int per_slot = rot ? DV - half : DV;
      const int items = nvalid * per_slot;
      for (int i = tid; i < items; i += blockDim.x) {
        const int sl = i / per_slot, dl = i % per_slot;
        float sw[NW], M, L;
        weights(sl, sw, M, L);
        if (p.sink) L += exp2f(s_sink[sl] * kLog2e - M);
        const float inv = 1.f / L;
        const int d = dv0 + dl;
        float* o = p.out + b * ST.o.s0 + (head0 + sl) * ST.o.s2;
        if (!rot || d < D - r) {
          o[d] = merged(sl, dl, sw) * inv;
        } else if constexpr (RD > 0) {
          const int k = d - (D - r);
          const float x1 = merged(sl, dl, sw) * inv, x2 = merged(sl, dl + half, sw) * inv;
          float c, sn;
          rope_cos_sin_turns(-(double)sv.t * s_freq[k], &c, &sn);
          o[d] = x1 * c - x2 * sn;
          o[d + half] = x2 * c + x1 * sn;
        }
      }
      if (p.lse && dh == 0 && tid < nvalid) {
        float sw[NW], M, L;
        weights(tid, sw, M, L);
        if (p.sink) L += exp2f(s_sink[tid] * kLog2e - M);
        p.lse[b * p.hq + head0 + tid] = (M + log2f(L)) * 0.69314718055994531f;
      }
      return pool_row;
    }
    // split partial to the workspace; decode_merge_kernel combines the splits
    const int64_t part = (int64_t)unit * p.splits + split;
    for (int i = tid; i < nvalid * DV; i += blockDim.x) {
      float sw[NW], M, L;
      weights(i / DV, sw, M, L);
      p.ws_acc[(part * 16 + i / DV) * D + dv0 + i % DV] = merged(i / DV, i % DV, sw);
    }
    if (dh == 0 && tid < nvalid) {
      float sw[NW], M, L;
      weights(tid, sw, M, L);
      p.ws_ml[(part * 16 + tid) * 2] = M;
      p.ws_ml[(part * 16 + tid) * 2 + 1] = L;
    }
    return pool_row;
  } else {
    // the waves' acc summed into one buffer, wave after wave (the stages are
    // too small for a slice per wave)
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
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (wave == w && head_ok) {
        const float sw = s_w[w][n];
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          float4* dst = reinterpret_cast<float4*>(&buf[n * DV + 16 * t + 4 * kq]);
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
    if (p.splits == 1) {
      if (tid < nvalid) {
        float L = s_L[tid];
        const float M = s_M[tid];
        if (p.sink) L += exp2f(p.sink[head0 + tid] * kLog2e - M);
        s_inv[tid] = 1.f / L;
        s_lse[tid] = (M + log2f(L)) * 0.69314718055994531f;
      }
      __syncthreads();
      constexpr int r = RD, half = RD / 2;
      const bool rot = RD > 0 && (int)dh == DS - 1;
      const int per_slot = rot ? DV - half : DV;
      const int items = nvalid * per_slot;
      for (int i = tid; i < items; i += blockDim.x) {
        const int sl = i / per_slot, dl = i % per_slot;
        const int d = dv0 + dl;
        float* o = p.out + b * ST.o.s0 + (head0 + sl) * ST.o.s2;
        const float inv = s_inv[sl];
        if (!rot || d < D - r) {
          o[d] = buf[sl * DV + dl] * inv;
        } else if constexpr (RD > 0) {
          const int k = d - (D - r);
          const float x1 = buf[sl * DV + dl] * inv, x2 = buf[sl * DV + dl + half] * inv;
          float c, sn;
          rope_cos_sin_turns(-(double)sv.t * s_freq[k], &c, &sn);
          o[d] = x1 * c - x2 * sn;
          o[d + half] = x2 * c + x1 * sn;
        }
      }
      if (p.lse && dh == 0 && tid < nvalid) p.lse[b * p.hq + head0 + tid] = s_lse[tid];
      return pool_row;
    }
    const int64_t part = (int64_t)unit * p.splits + split;
    for (int i = tid; i < nvalid * DV; i += blockDim.x)
      p.ws_acc[(part * 16 + i / DV) * D + dv0 + i % DV] = buf[(i / DV) * DV + i % DV];
    if (dh == 0 && tid < nvalid) {
      p.ws_ml[(part * 16 + tid) * 2] = s_M[tid];
      p.ws_ml[(part * 16 + tid) * 2 + 1] = s_L[tid];
    }
  }
  return pool_row;
}

// Combine the splits of one unit (16 query-head slots) over one chunk of CK
// output dims (blockIdx.z): weights exp2(m_s - M), sink, normalisation, LSE
// and the -t rotation.  CK is the rotated width when dims rotate (the last
// chunk is then exactly the rotated dims).  1024 threads: thread (sg, slot, u),
// u < CK/4, sums the float4 at dims c0 + 4u over splits s = sg, sg + NG, ...
// (NG = 256 / CK split groups; all loads independent); the groups are added
// in LDS in a fixed order, and thread (slot, u < CK/8) finishes the pair of
// float4s at c0 + 4u and c0 + 4u + CK/2 (a rotate-half pair in the last chunk).
// NORM: each split's partial is its own normalised output in bf16 (the wide
// path), weighted by exp2(m_s - M) * l_s instead of exp2(m_s - M).
constexpr int kMergeGroups = 4;  // for 64-dim chunks
template <int D, int R, int NW, int DS, bool SHARED, int RD, bool TREAT, bool SPEC, bool DN = true>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeParams p) {
  decode_body<D, R, NW, DS, SHARED, RD, TREAT, SPEC, false, DN>(p, blockIdx.x);
}

// Fused decode step (lbca_decode_step, EXCLUSIVE rule, K and V series): the
// decode launch of decode_kernel, each workgroup reading its position's raw
// row from the new token's input.  The workgroup that owns split 0 of a
// (sequence, KV head) also runs that row's cache step: the token append, and,
// on the step whose token completes a block, the pooling of that block after
// its decode work, with its first 256
// threads (bitwise as lbca_pool_blocks).  No query of the step reads what the
// cache step writes: the row at the position comes from the input, and under
// EXCLUSIVE a block is visible only once it is wholly older than the window.
// (Separate cache workgroups would be given the decode's registers and could
// not share a CU with a decode workgroup.)
struct StepParams {
  DecodeParams d;
  CacheParams c;
};

template <int D, int R, int NW, int DS, bool SPEC, typename TZ, bool DN>
__global__ __launch_bounds__(NW * 64) void decode_step_kernel(StepParams sp) {
  static_assert(NW * 64 >= 256, "the cache step needs 256 threads");
  __shared__ float part[32][256];  // the cache step's cross-wave phase merge
  const int row = decode_body<D, R, NW, DS, false, 0, false, SPEC, true, DN, TZ>(sp.d, blockIdx.x, &sp.c);
  if (row >= 0)
    cache_row<bf16_t, TZ, true, false, false, true, false, true, DN>(sp.c, row, part, threadIdx.x < 256);
}

template <bool NORM>
__global__ __launch_bounds__(1024) void decode_merge_kernel(DecodeParams p, int D, int CK) {
  __shared__ float s_w[64][16];                 // split weights
  __shared__ float s_red[16][16], s_red2[16][16];  // per-wave max and sum of each slot
  __shared__ float s_inv[16], s_lse[16];
  __shared__ float4 s_part[kMergeGroups][16][32];  // [group][slot][float4 of the chunk], CK <= 128
  using PT = typename std::conditional<NORM, uint2, float4>::type;  // one partial's 4 dims
  constexpr int kPre = 8;  // partials per thread requested before the weights are known
  const int tid = threadIdx.x;
  const int64_t unit = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int hg = (int)(blockIdx.x % (unsigned)p.head_groups);
  const int64_t kvh = blockIdx.x / (unsigned)p.head_groups;
  const int64_t b = blockIdx.y;
  const int slot0 = hg * 16;
  const int nvalid = (int)(p.G - slot0 < 16 ? p.G - slot0 : 16);
  const int64_t head0 = kvh * p.G + slot0;
  const int S = p.splits;
  const int64_t part0 = unit * S;
  const int nf = CK / 4;   // float4s per slot in the chunk
  const int NG = 256 / CK;  // split groups
  const int c0 = (int)blockIdx.z * CK;
  const int u0 = tid % nf, sl0 = (tid / nf) % 16, sg = tid / (nf * 16);
  const bool mine = sg < NG && sl0 < nvalid;
  const int64_t off = (part0 * 16 + sl0) * D + c0 + 4 * u0;
  const PT* pa = reinterpret_cast<const PT*>(NORM ? static_cast<const void*>(p.ws_o + off)
                                                  : static_cast<const void*>(p.ws_acc + off));
  const int64_t pstride = (int64_t)16 * D / 4;  // one split on, in units of PT
  // this thread's first partials (splits sg, sg + NG, ...) go out with the maxima
  PT pre[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i)
    if (mine && sg + i * NG < S) pre[i] = pa[(int64_t)(sg + i * NG) * pstride];
  // Split weights, one thread per (split s = tid / 16, slot tid % 16) (S <= 64):
  // the slot's max and sum over splits go over the four splits of a wave by
  // lane exchanges, then over the waves through LDS, both in a fixed order.
  const int ws = tid >> 4, wsl = tid & 15, wave = tid >> 6;
  const int nwv = (S + 3) >> 2;  // waves holding splits
  float2 ml = make_float2(kNegInf, 0.f);
  if (ws < S) ml = *reinterpret_cast<const float2*>(&p.ws_ml[(part0 * 16 + tid) * 2]);
  const SeqView sv = seq_view(p, b);
  if (!sv.ok) return;  // the decode kernel already wrote NaN for this unit
  float M = fmaxf(ml.x, __shfl_xor(ml.x, 16, 64));
  M = fmaxf(M, __shfl_xor(M, 32, 64));
  if (wave < nwv && (tid & 63) < 16) s_red[wave][wsl] = M;
  __syncthreads();
  M = s_red[0][wsl];
#pragma unroll
  for (int w = 1; w < 16; ++w)
    if (w < nwv) M = fmaxf(M, s_red[w][wsl]);
  const float sw = ml.x == kNegInf ? 0.f : exp2f(ml.x - M);
  if (ws < S) s_w[ws][wsl] = NORM ? sw * ml.y : sw;
  float L = ml.y * sw;
  L += __shfl_xor(L, 16, 64);
  L += __shfl_xor(L, 32, 64);
  if (wave < nwv && (tid & 63) < 16) s_red2[wave][wsl] = L;
  __syncthreads();
  if (tid < nvalid) {
    L = s_red2[0][tid];
    for (int w = 1; w < nwv; ++w) L += s_red2[w][tid];
    if (p.sink) L += exp2f(p.sink[head0 + tid] * kLog2e - M);
    s_inv[tid] = 1.f / L;
    s_lse[tid] = (M + log2f(L)) * 0.69314718055994531f;
  }
  __syncthreads();
  if (mine) {
    auto add = [&](float4& x, const PT& a, float w) {
      if constexpr (NORM) {
        x.x = fmaf(lo_bf16(a.x), w, x.x); x.y = fmaf(hi_bf16(a.x), w, x.y);
        x.z = fmaf(lo_bf16(a.y), w, x.z); x.w = fmaf(hi_bf16(a.y), w, x.w);
      } else {
        x.x = fmaf(a.x, w, x.x); x.y = fmaf(a.y, w, x.y); x.z = fmaf(a.z, w, x.z); x.w = fmaf(a.w, w, x.w);
      }
    };
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kPre; ++i)
      if (sg + i * NG < S) add(x, pre[i], s_w[sg + i * NG][sl0]);
    for (int s = sg + kPre * NG; s < S; s += NG) add(x, pa[(int64_t)s * pstride], s_w[s][sl0]);
    s_part[sg][sl0][u0] = x;
  }
  __syncthreads();
  const int sl = tid / (nf / 2), u = tid % (nf / 2);
  if (sl < nvalid) {
    const float inv = s_inv[sl];
    float o1[4], o2[4];
    {
      float4 x = s_part[0][sl][u], y = s_part[0][sl][u + nf / 2];
      for (int g = 1; g < NG; ++g) {
        const float4 a = s_part[g][sl][u], c = s_part[g][sl][u + nf / 2];
        x.x += a.x; x.y += a.y; x.z += a.z; x.w += a.w;
        y.x += c.x; y.y += c.y; y.z += c.z; y.w += c.w;
      }
      o1[0] = x.x * inv; o1[1] = x.y * inv; o1[2] = x.z * inv; o1[3] = x.w * inv;
      o2[0] = y.x * inv; o2[1] = y.y * inv; o2[2] = y.z * inv; o2[3] = y.w * inv;
    }
    const int d1 = c0 + 4 * u, d2 = d1 + CK / 2;
    const int r = p.rope_dims;
    if (r > 0 && c0 == D - r) {  // rotate-half pairs (d1 + e, d2 + e) by -t
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float cs, sn;
        rope_cos_sin(-(double)sv.t, d1 + e - c0, r, p.log2_base, &cs, &sn);
        const float x1 = o1[e], x2 = o2[e];
        o1[e] = x1 * cs - x2 * sn;
        o2[e] = x2 * cs + x1 * sn;
      }
    }
    float* o = p.out + qrow_off(p.o_st, p.qrows, b, head0 + sl);
    *reinterpret_cast<float4*>(o + d1) = make_float4(o1[0], o1[1], o1[2], o1[3]);
    *reinterpret_cast<float4*>(o + d2) = make_float4(o2[0], o2[1], o2[2], o2[3]);
  }
  if (p.lse && blockIdx.z == 0 && tid < nvalid) p.lse[b * p.hq + head0 + tid] = s_lse[tid];
}

void launch_decode_merge(const DecodeParams& p, int64_t batch, int64_t dim, bool norm, hipStream_t stream) {
  // chunks of the rotated width when dims rotate, else of min(dim, 64)
  const int ck = p.rope_dims > 0 ? p.rope_dims : (dim < 64 ? (int)dim : 64);
  const dim3 grid((unsigned)(p.hkv * p.head_groups), (unsigned)batch, (unsigned)(dim / ck));
  if (norm) decode_merge_kernel<true><<<grid, 1024, 0, stream>>>(p, (int)dim, ck);
  else decode_merge_kernel<false><<<grid, 1024, 0, stream>>>(p, (int)dim, ck);
}

// ---------------------------------------------------------------------------
static int rows_per_tile(int64_t dim) { return dim >= 512 ? 16 : 32; }
static int waves_per_wg(int64_t dim) { return dim <= 128 ? 8 : 4; }

// Wide-row MQA path (512 dims, shared series, query heads in 32-head blocks):
// workgroups per (sequence, KV head) along the row list.  Enough splits to
// give about LBCA_WIDE_TARGET_WGS row ranges (one CU streams only about
// 40 GB/s), but at least LBCA_WIDE_MIN_TILES 32-row tiles per range (a
// split's bf16 partial, 32 KB per head block, stays at most the rows it
// reads; with few rows, as in a CSA step over its selection, one tile per
// range measured 16.9 against 18.8 us for two), and enough that each range's
// selected ids fit the LDS stage.  With 64 query
// heads each range is worked by two 4-wave "twin" workgroups, one per 32-head
// block (LBCA_WIDE_TWINS), rather than one 8-wave workgroup for both.
#ifndef LBCA_WIDE_TWINS
#define LBCA_WIDE_TWINS 1
#endif
#ifndef LBCA_WIDE_TARGET_WGS
#define LBCA_WIDE_TARGET_WGS 128
#endif
#ifndef LBCA_WIDE_MIN_TILES
#define LBCA_WIDE_MIN_TILES 1
#endif
constexpr int kWideSelLds = 1024;  // matches the wide kernel's id stage

constexpr int64_t kWideOneGroupRows = 512;

static DecodePlan plan_decode_wide(const lbca_decode_args& a, int64_t G) {
  DecodePlan pl{};
  pl.tile_rows = 32;
  pl.head_groups = (int)(G / 16);
  pl.dim_splits = 1;
  pl.wide_blocks = (int)(G / 32);
  const int64_t sel_max = a.sel_idx ? a.k_sel : a.entries;
  const int64_t raw_span = a.mode == LBCA_EXCLUSIVE ? a.window + a.block - 1 : a.window;
  const int64_t raw_max = raw_span < a.raw_rows ? raw_span : a.raw_rows;
  const int64_t tiles = (sel_max + 31) / 32 + (raw_max + 31) / 32;
  pl.wide_twins = 1;
  // one 4-wave workgroup per 32-head block, unless there are so many rows (a
  // query chunk) that one 8-wave workgroup per row already fills the chip and
  // gathers the row's entries once for both blocks
  if (LBCA_WIDE_TWINS && pl.wide_blocks == 2 && a.batch * a.kv_heads < kWideOneGroupRows) {
    pl.wide_twins = 2;
    pl.wide_blocks = 1;
  }
  const int64_t per_split = a.batch * a.kv_heads;  // (sequence, KV head) ranges per split
  int64_t s = (LBCA_WIDE_TARGET_WGS + per_split - 1) / per_split;
  const int64_t by_rows = (tiles + LBCA_WIDE_MIN_TILES - 1) / LBCA_WIDE_MIN_TILES;
  if (s > by_rows) s = by_rows;
  if (s > 64) s = 64;  // the merge combines at most 64 splits
  if (a.sel_idx) {
    // every range's selected ids must fit the LDS stage; with more ids than
    // 64 ranges can stage there is no valid plan (unsupported)
    const int64_t need = (tiles + kWideSelLds / 32 - 1) / (kWideSelLds / 32);
    if (need > 64) {
      pl.unsupported = 1;
      return pl;
    }
    if (s < need) s = need;
  }
  if (s < 1) s = 1;
  // ranges hold ceil(tiles / s) tiles each; drop the splits that would get none
  // (260 tiles over 32 splits leave three empty), so no workgroup writes an
  // empty partial and the merge reads fewer.  The range size is unchanged, so
  // the selected ids per range still fit.  With treated rows and more than
  // one tile per range (no selection) a raw tile counts twice (it is
  // normalised and rotated in LDS first), and the ranges split that cost;
  // decode_wide_kernel applies the same rule (wide_ranges).
  const int64_t per = (tiles + s - 1) / s;
  const bool treat = a.rmsnorm_eps >= 0.f || a.rope_dims > 0;
  if (treat && !a.sel_idx && per >= 2) {
    const int64_t tiles_r = (raw_max + 31) / 32;
    const int64_t cost = tiles + tiles_r, pc = (cost + s - 1) / s;
    s = (cost + pc - 1) / pc;
  } else if (per > 0) {
    s = (tiles + per - 1) / per;
  }
  pl.splits = (int)s;
  if (s == 1) return pl;
  const size_t u = (size_t)(a.batch * a.kv_heads * pl.head_groups);
  pl.ws_bytes = u * s * 16 * 2 * sizeof(float) + u * s * 16 * (size_t)a.dim * sizeof(bf16_t);
  return pl;
}

DecodePlan plan_decode(const lbca_decode_args& a) {
  DecodePlan pl{};
  if (a.dtype != LBCA_BF16) return pl;  // fp32 path needs no workspace
  const int64_t G = a.q_heads / a.kv_heads;
  if (a.dim == 512 && a.pooled_v == nullptr && G % 32 == 0) return plan_decode_wide(a, G);
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
  // Splits: only when a unit's tiles would give its waves more than
  // LBCA_DECODE_TILES_PER_WAVE each (one workgroup per unit keeps every tile's
  // loads in flight at once and needs no merge launch, which costs more than
  // the few extra tiles per wave); split partials (16 heads x dim fp32 per
  // workgroup, for every head group of a KV head) kept under a quarter of the
  // K/V bytes.
  int64_t s = (tiles + nw * LBCA_DECODE_TILES_PER_WAVE - 1) / (nw * LBCA_DECODE_TILES_PER_WAVE);
  const int64_t kv_bytes = rows * a.dim * 2 * (a.pooled_v ? 2 : 1);
  const int64_t part_bytes = (int64_t)pl.head_groups * 16 * (a.dim + 2) * 4;
  const int64_t by_traffic = kv_bytes / (4 * part_bytes) > 0 ? kv_bytes / (4 * part_bytes) : 1;
  if (s > by_traffic) s = by_traffic;
  if (s > 64) s = 64;  // the merge combines at most 64 splits
  if (s < 1) s = 1;
  // a workgroup's range of selected ids must fit its LDS stage; with more ids
  // than 64 ranges can stage there is no valid plan (unsupported)
  if (a.sel_idx) {
    const int64_t tiles_per_ids = kSelLds / pl.tile_rows;
    const int64_t need = (tiles + tiles_per_ids - 1) / tiles_per_ids;
    if (need > 64) {
      pl.unsupported = 1;
      return pl;
    }
    if (s < need) s = need;
  }
  pl.splits = (int)s;
  // dim-split twins when the workgroups would not cover the 256 CUs, and
  // always for 512 dims (a full-width accumulator does not fit beside a tile)
  pl.dim_splits = ((a.dim == 512 || (a.dim >= 128 && units * s < 256)) && a.rope_dims <= a.dim / 2) ? 2 : 1;
  if (s == 1) return pl;
  const size_t u = (size_t)units;
  pl.ws_bytes = u * s * 16 * 2 * sizeof(float) + u * s * 16 * (size_t)a.dim * sizeof(float);
  return pl;
}

// DN: every tensor of the call dense (instances that work the strides out
// from the sizes).  Strided calls run the same instance family, so their
// results equal the dense ones bit for bit.
template <int D, int R, int NW, int DS, bool DN>
static hipError_t launch_dd(const DecodeParams& p, bool shared, int rd, bool treat, dim3 g, hipStream_t s) {
  const dim3 blk(NW * 64);
  if (!treat) {
    if constexpr (D <= 128) {  // early-request instances for one split without selection
      if (p.splits == 1 && p.sel == nullptr) {
        if (shared) decode_kernel<D, R, NW, DS, true, 0, false, true, DN><<<g, blk, 0, s>>>(p);
        else decode_kernel<D, R, NW, DS, false, 0, false, true, DN><<<g, blk, 0, s>>>(p);
        return hipGetLastError();
      }
    }
    if (shared) decode_kernel<D, R, NW, DS, true, 0, false, false, DN><<<g, blk, 0, s>>>(p);
    else decode_kernel<D, R, NW, DS, false, 0, false, false, DN><<<g, blk, 0, s>>>(p);
    return hipGetLastError();
  }
  if (!shared) return hipErrorInvalidValue;
  switch (rd) {
    case 0: decode_kernel<D, R, NW, DS, true, 0, true, false, DN><<<g, blk, 0, s>>>(p); break;
    case 64:
      if constexpr (D / DS >= 64) decode_kernel<D, R, NW, DS, true, 64, true, false, DN><<<g, blk, 0, s>>>(p);
      else return hipErrorInvalidValue;
      break;
    case 128:
      if constexpr (D / DS >= 128) decode_kernel<D, R, NW, DS, true, 128, true, false, DN><<<g, blk, 0, s>>>(p);
      else return hipErrorInvalidValue;
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int R, int NW, int DS>
static hipError_t launch_d(const DecodeParams& p, bool shared, int rd, bool treat, dim3 g, bool dn,
                           hipStream_t s) {
  return dn ? launch_dd<D, R, NW, DS, true>(p, shared, rd, treat, g, s)
            : launch_dd<D, R, NW, DS, false>(p, shared, rd, treat, g, s);
}

// Whether every tensor of a decode call has dense row-major strides.
static bool decode_dense(const lbca_decode_args& a, int qrows) {
  const int64_t B = a.batch / qrows, Hk = a.kv_heads, d = a.dim;
  auto q_like = [&](const void* ptr, const lbca_strides& st) {
    return qrows > 1 ? dense_strides(ptr, st, {B, (int64_t)qrows, a.q_heads}, d)
                     : dense_strides(ptr, st, {a.batch, a.q_heads}, d);
  };
  return q_like(a.q, a.q_st) && q_like(a.out, a.out_st) &&
         dense_strides(a.pooled_k, a.pooled_k_st, {B, Hk, a.entries}, d) &&
         dense_strides(a.pooled_v, a.pooled_v_st, {B, Hk, a.entries}, d) &&
         dense_strides(a.raw_k, a.raw_k_st, {B, Hk, a.raw_rows}, d) &&
         dense_strides(a.raw_v, a.raw_v_st, {B, Hk, a.raw_rows}, d);
}

// Query and output strides as {sequence, query, head}: a decode call's q and
// out are [batch, heads, dim]; a query chunk's (qrows > 1) [batch, qrows,
// heads, dim].  A shared series reads its values with the key strides.
static void set_strides(DecodeParams& p, const lbca_decode_args& a, int qrows) {
  auto qform = [&](const lbca_strides& s) {
    return qrows > 1 ? s : lbca_strides{{s.s[0], 0, s.s[1]}};
  };
  p.q_st = qform(a.q_st);
  p.o_st = qform(a.out_st);
  p.pk_st = a.pooled_k_st;
  p.rk_st = a.raw_k_st;
  p.pv_st = a.pooled_v ? a.pooled_v_st : a.pooled_k_st;
  p.rv_st = a.raw_v ? a.raw_v_st : a.raw_k_st;
}

hipError_t launch_decode(const lbca_decode_args& a, const DecodePlan& plan, void* ws,
                         hipStream_t stream, int qrows) {
  if (a.dtype != LBCA_BF16) return launch_decode_f32(a, stream);
  const int64_t G = a.q_heads / a.kv_heads;
  DecodeParams p{};
  p.qrows = qrows;
  if (qrows > 1 && plan.wide_blocks == 0) return hipErrorInvalidValue;  // shared cache rows: wide path only
  p.q = static_cast<const bf16_t*>(a.q);
  p.pk = static_cast<const bf16_t*>(a.pooled_k);
  p.pv = static_cast<const bf16_t*>(a.pooled_v);
  p.rk = static_cast<const bf16_t*>(a.raw_k);
  p.rv = static_cast<const bf16_t*>(a.raw_v);
  p.pos = a.pos; p.rpb = a.raw_pos_base; p.sel = a.sel_idx; p.sink = a.sink;
  p.out = a.out; p.lse = a.lse;
  set_strides(p, a, qrows);
  const bool dn = decode_dense(a, qrows);
  const size_t units = (size_t)a.batch * a.kv_heads * plan.head_groups;
  if (plan.splits > 1) {
    p.ws_ml = static_cast<float*>(ws);
    p.ws_acc = p.ws_ml + units * plan.splits * 16 * 2;
    p.ws_o = reinterpret_cast<bf16_t*>(p.ws_acc);
  }
  p.wide_twins = plan.wide_twins;
  p.hq = a.q_heads; p.hkv = a.kv_heads; p.G = G;
  p.entries = a.entries; p.raw_rows = a.raw_rows; p.k_sel = a.sel_idx ? a.k_sel : 0;
  p.m = a.block; p.W = a.window; p.mode = a.mode;
  p.splits = plan.splits; p.head_groups = plan.head_groups;
  p.units = (int)units;
  p.scale_log2 = a.scale * kLog2e;
  p.eps = a.rmsnorm_eps;
  p.rope_dims = a.rope_dims;
  p.log2_base = a.rope_dims > 0 ? log2((double)a.rope_base) : 0.0;
  const bool shared = a.pooled_v == nullptr;
  const bool treat = a.rmsnorm_eps >= 0.f || a.rope_dims > 0;
  if (plan.wide_blocks > 0) {
    hipError_t e = launch_decode_wide(p, a.rope_dims, treat, plan.wide_blocks, dn, stream);
    if (e != hipSuccess || plan.splits == 1) return e;
    launch_decode_merge(p, a.batch, a.dim, true, stream);
    return hipGetLastError();
  }
  const size_t pairs = units * plan.splits;  // (unit, split) pairs
  const int ds = plan.dim_splits;
  const dim3 g((unsigned)(ds == 1 ? pairs : (pairs + 7) / 8 * 8 * ds));
  hipError_t e;
  switch (a.dim * 4 + ds) {
    case 64 * 4 + 1: e = launch_d<64, 32, 8, 1>(p, shared, a.rope_dims, treat, g, dn, stream); break;
    case 128 * 4 + 1: e = launch_d<128, 32, 8, 1>(p, shared, a.rope_dims, treat, g, dn, stream); break;
    case 128 * 4 + 2: e = launch_d<128, 32, 8, 2>(p, shared, a.rope_dims, treat, g, dn, stream); break;
    case 256 * 4 + 1: e = launch_d<256, 32, 4, 1>(p, shared, a.rope_dims, treat, g, dn, stream); break;
    case 256 * 4 + 2: e = launch_d<256, 32, 4, 2>(p, shared, a.rope_dims, treat, g, dn, stream); break;
    case 512 * 4 + 2: e = launch_d<512, 16, 4, 2>(p, shared, a.rope_dims, treat, g, dn, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || plan.splits == 1) return e;
  launch_decode_merge(p, a.batch, a.dim, false, stream);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused decode step: the decode launch of launch_decode with the cache rows'
// workgroups appended (plus the merge when the rows are split).
// dn: every tensor of the call dense (instances that work the strides out from the sizes).
template <int D, int DS, typename TZ>
static void launch_step_d(const StepParams& sp, bool spec, bool dn, unsigned grid, hipStream_t s) {
  if (dn) {
    if (spec) decode_step_kernel<D, 32, 8, DS, true, TZ, true><<<grid, 512, 0, s>>>(sp);
    else decode_step_kernel<D, 32, 8, DS, false, TZ, true><<<grid, 512, 0, s>>>(sp);
  } else {
    if (spec) decode_step_kernel<D, 32, 8, DS, true, TZ, false><<<grid, 512, 0, s>>>(sp);
    else decode_step_kernel<D, 32, 8, DS, false, TZ, false><<<grid, 512, 0, s>>>(sp);
  }
}

hipError_t launch_decode_step(const lbca_decode_args& da, const lbca_cache_args& ca, const DecodePlan& plan,
                              void* ws, hipStream_t stream) {
  StepParams sp{};
  DecodeParams& p = sp.d;
  p.qrows = 1;
  p.q = static_cast<const bf16_t*>(da.q);
  p.pk = static_cast<const bf16_t*>(da.pooled_k);
  p.pv = static_cast<const bf16_t*>(da.pooled_v);
  p.rk = static_cast<const bf16_t*>(da.raw_k);
  p.rv = static_cast<const bf16_t*>(da.raw_v);
  p.pos = da.pos; p.rpb = nullptr; p.sel = nullptr; p.sink = da.sink;
  p.out = da.out; p.lse = da.lse;
  set_strides(p, da, 1);
  p.tk = static_cast<const bf16_t*>(ca.x_new);
  p.tv = static_cast<const bf16_t*>(ca.v_new);
  p.tk_st = ca.x_new_st;
  p.tv_st = ca.v_new_st;
  p.ring = ca.ring;
  const size_t units = (size_t)da.batch * da.kv_heads * plan.head_groups;
  if (plan.splits > 1) {
    p.ws_ml = static_cast<float*>(ws);
    p.ws_acc = p.ws_ml + units * plan.splits * 16 * 2;
  }
  p.hq = da.q_heads; p.hkv = da.kv_heads; p.G = da.q_heads / da.kv_heads;
  p.entries = da.entries; p.raw_rows = da.raw_rows; p.k_sel = 0;
  p.m = da.block; p.W = da.window; p.mode = da.mode;
  p.splits = plan.splits; p.head_groups = plan.head_groups;
  p.units = (int)units;
  p.scale_log2 = da.scale * kLog2e;
  p.eps = -1.f;
  CacheParams& c = sp.c;
  c.x_new = ca.x_new; c.v_new = ca.v_new; c.z_new = ca.z_new;
  c.raw_x = ca.raw_x; c.raw_v = ca.raw_v; c.raw_z = ca.raw_z;
  c.bias = ca.bias; c.out_x = ca.out_x; c.out_v = ca.out_v;
  c.pos = ca.pos; c.raw_pos_base = ca.raw_pos_base;
  c.heads = ca.heads; c.dim = ca.dim; c.m = ca.block; c.W = ca.window; c.ring = ca.ring; c.entries = ca.entries;
  c.mode = ca.mode;
  c.lanes_per_row = (int)(ca.dim / 8);
  c.log2_lanes = __builtin_ctz((unsigned)c.lanes_per_row);
  c.eps = -1.f;
  set_cache_strides(c, ca);
  const size_t pairs = units * plan.splits;
  const int ds = plan.dim_splits;
  const unsigned grid = (unsigned)(ds == 1 ? pairs : (pairs + 7) / 8 * 8 * ds);
  const bool spec = plan.splits == 1;
  const bool zf = ca.z_dtype == LBCA_F32;
  const int64_t B = ca.batch, H = ca.heads, R = 2 * ca.ring, d = ca.dim;
  const bool dn = decode_dense(da, 1) && dense_strides(ca.x_new, ca.x_new_st, {B, H}, d) &&
                  dense_strides(ca.v_new, ca.v_new_st, {B, H}, d) && dense_strides(ca.z_new, ca.z_new_st, {B, H}, d) &&
                  dense_strides(ca.raw_z, ca.raw_z_st, {B, H, R}, d);
  switch (da.dim * 4 + ds) {
    case 64 * 4 + 1:
      zf ? launch_step_d<64, 1, float>(sp, spec, dn, grid, stream)
         : launch_step_d<64, 1, bf16_t>(sp, spec, dn, grid, stream);
      break;
    case 128 * 4 + 1:
      zf ? launch_step_d<128, 1, float>(sp, spec, dn, grid, stream)
         : launch_step_d<128, 1, bf16_t>(sp, spec, dn, grid, stream);
      break;
    case 128 * 4 + 2:
      zf ? launch_step_d<128, 2, float>(sp, spec, dn, grid, stream)
         : launch_step_d<128, 2, bf16_t>(sp, spec, dn, grid, stream);
      break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  launch_decode_merge(p, da.batch, da.dim, false, stream);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Static scratch of lbca_attend_decode_noalloc: the split partials of the
// decode kernels live in this file-scope device array instead of a caller
// workspace.  Each GPU holds its own copy at its own address; host code must
// use the address hipGetSymbolAddress reports for the current device (the
// array's name is only a host-side stand-in), looked up once per device.
static __device__ __align__(256) unsigned char scratch[LBCA_NOALLOC_SCRATCH_BYTES];

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

}  // namespace lbca
