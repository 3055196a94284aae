// Prefill attention for a chunk of consecutive queries, each with its own
// visibility (pooled entries j < n_pooled(t) plus the raw span [raw_begin(t), t]).
//
// Method: "mSeek: learned KV-cache compression in a 3B model", "How LBCA works"
// (steps 4-5, and the chunked bounded-memory path that must agree with the
// clear reference): a query sees every completed summary older than its
// window plus its exact raw window, never a summary holding a later token.
//
// bf16 path (MFMA, a dense contraction).  At 128 dims prefill128_kernel
// (below, on 32x32x16 MFMAs) runs; prefill_kernel, described here, serves 64
// dims.  A workgroup of 8 waves (two per
// SIMD, so one wave's softmax arithmetic runs beside the other's MFMAs) owns
// one (sequence, KV head) and 256 consecutive rows of the flattened (position,
// query head in the GQA group) space; each wave holds 32 of those rows (two
// 16-row groups) as B operands.  The workgroup walks the union of its rows'
// visible rows in tiles of 32 rows at 128 dims (64 at 64 dims): the pooled
// prefix [0, n_pooled(last position)), then the raw band [raw_begin(first
// position), last position].  K and V tiles go straight from global memory to
// LDS (global_load_lds_dwordx4, no staging registers) in a chunk-swizzled
// layout, so the 16-byte K reads and the transposing V reads of a 16-lane
// group hit distinct banks; four buffers keep two tiles' loads in flight, one
// barrier per tile.  The loop is software-pipelined: a tile's softmax runs
// while the next tile's Q.K MFMAs execute.  Scores are computed
// transposed, S^T = K Q^T with v_mfma_f32_16x16x32_bf16, so each lane owns one
// query row's scores and the row max/sum need a 16- and a 32-lane swap; P^T
// is then directly the B operand of O^T = V^T P^T (k = 32 keys: two 16-key
// blocks), whose A operand comes from two transposing LDS reads
// (ds_read_b64_tr_b16).  Tiles visible to every row skip the per-element mask;
// a row's reference max moves only when a score exceeds it by 2^8, so the
// accumulator rescale runs on few tiles.
#include <type_traits>

#include "device_util.h"
#include "lbca_internal.h"

namespace lbca {

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
  // element strides: q and out {sequence, query, head}; caches {sequence, KV head, row}
  Str q_st, o_st, pk_st, pv_st, rk_st, rv_st;
};

// Element offset of (sequence b, query t, head h) in q (q_st) or out (o_st).
__device__ __forceinline__ int64_t qoff(Str st, int64_t b, int64_t t, int64_t h) {
  return b * st.s0 + t * st.s1 + h * st.s2;
}

// The strides a prefill workgroup uses: the arguments', or, when every tensor
// of the call is dense (DN), the row-major ones worked out from the sizes.
struct PreStr {
  Str q, o, pk, pv, rk, rv;
};
template <bool DN, int D>
__device__ __forceinline__ PreStr pre_strides(const PrefillParams& p) {
  if constexpr (DN) {
    const Str qs{p.q_len * p.hq * D, p.hq * D, D};
    const Str ps{p.hkv * p.entries * D, p.entries * D, D};
    const Str rs{p.hkv * p.raw_rows * D, p.raw_rows * D, D};
    return PreStr{qs, qs, ps, ps, rs, rs};
  } else {
    return PreStr{p.q_st, p.o_st, p.pk_st, p.pv_st, p.rk_st, p.rv_st};
  }
}

// Chunk swizzle of an LDS tile row (16-byte chunks).  A 16-byte read serves
// 16 lanes per pass over the 64 banks, so at 128 dims (a row spans all 64
// banks) 16 consecutive rows read at one chunk index, and 4 consecutive rows
// read at 4 aligned chunks (the transposing V reads), must land on 16 distinct
// chunk positions.  Unchanged when the row moves by 16.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (2 * (r >> 1)) & 7;
}

// Wait until at most N vector-memory operations of this wave are in flight
// (other counters untouched).
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// All transposing V reads of one tile (16 ds_read_b64_tr_b16) in one block
// that also waits for them.  Written as one asm block because the compiler
// cannot tell which LDS buffer the intrinsic form reads and would wait for
// every tile load still in flight; the block's outputs are early-clobber and
// all used, and it ends with the wait for its own reads.  Slot o = (c*DT+t)*2+h
// holds rows 32c + 16h + 4kq.. of column 16t + n (c: 32-key chunk, h: half).
template <int D>
__device__ __forceinline__ void read_v_tiles(s16x4 (&r)[16], const bf16_t* vt, int n, int kq, int swz_tr) {
  constexpr int DT = D / 16;
  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) bf16_t*)(vt);
  uint32_t ad[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
    ad[t] = base + 2u * (uint32_t)((4 * kq + (n >> 2)) * D + 4 * (n & 1) + 8 * ((2 * t + ((n & 3) >> 1)) ^ swz_tr));
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n"
        "ds_read_b64_tr_b16 %1, %16 offset:4096\n"
        "ds_read_b64_tr_b16 %2, %17\n"
        "ds_read_b64_tr_b16 %3, %17 offset:4096\n"
        "ds_read_b64_tr_b16 %4, %18\n"
        "ds_read_b64_tr_b16 %5, %18 offset:4096\n"
        "ds_read_b64_tr_b16 %6, %19\n"
        "ds_read_b64_tr_b16 %7, %19 offset:4096\n"
        "ds_read_b64_tr_b16 %8, %20\n"
        "ds_read_b64_tr_b16 %9, %20 offset:4096\n"
        "ds_read_b64_tr_b16 %10, %21\n"
        "ds_read_b64_tr_b16 %11, %21 offset:4096\n"
        "ds_read_b64_tr_b16 %12, %22\n"
        "ds_read_b64_tr_b16 %13, %22 offset:4096\n"
        "ds_read_b64_tr_b16 %14, %23\n"
        "ds_read_b64_tr_b16 %15, %23 offset:4096\n"
        "s_waitcnt lgkmcnt(0)\n"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]),
          "=&v"(r[14]), "=&v"(r[15])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
        : "memory");
  } else {
    static_assert(D == 64, "transposing V reads are laid out for 64 or 128 dims");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n"
        "ds_read_b64_tr_b16 %1, %16 offset:2048\n"
        "ds_read_b64_tr_b16 %2, %17\n"
        "ds_read_b64_tr_b16 %3, %17 offset:2048\n"
        "ds_read_b64_tr_b16 %4, %18\n"
        "ds_read_b64_tr_b16 %5, %18 offset:2048\n"
        "ds_read_b64_tr_b16 %6, %19\n"
        "ds_read_b64_tr_b16 %7, %19 offset:2048\n"
        "ds_read_b64_tr_b16 %8, %16 offset:4096\n"
        "ds_read_b64_tr_b16 %9, %16 offset:6144\n"
        "ds_read_b64_tr_b16 %10, %17 offset:4096\n"
        "ds_read_b64_tr_b16 %11, %17 offset:6144\n"
        "ds_read_b64_tr_b16 %12, %18 offset:4096\n"
        "ds_read_b64_tr_b16 %13, %18 offset:6144\n"
        "ds_read_b64_tr_b16 %14, %19 offset:4096\n"
        "ds_read_b64_tr_b16 %15, %19 offset:6144\n"
        "s_waitcnt lgkmcnt(0)\n"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]),
          "=&v"(r[14]), "=&v"(r[15])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
  }
}

// Workgroup shape at 128 dims: waves and 16-row query groups per wave
#ifndef LBCA_PREFILL_WAVES
#define LBCA_PREFILL_WAVES 8
#endif
#ifndef LBCA_PREFILL_QG
#define LBCA_PREFILL_QG 2
#endif
// VALU instructions the scheduler places after each Q.K MFMA of the next tile
// (0: the compiler's own order)
#ifndef LBCA_PREFILL_SCHED
#define LBCA_PREFILL_SCHED 0
#endif
// 1: the 128-dim path runs prefill_kernel instead of prefill128_kernel
#ifndef LBCA_PREFILL_V1
#define LBCA_PREFILL_V1 0
#endif

template <int D, bool SHARED, int NWV, int QG, bool DN>
__global__ __launch_bounds__(NWV * 64, 1) void prefill_kernel(PrefillParams p) {
  constexpr int NT = NWV * 64;
  constexpr int KT = D <= 64 ? 64 : 32;  // keys per tile (registers bound it at 128 dims)
  constexpr int KB = KT / 16;            // 16-key blocks per tile
  constexpr int KS = D / 32;             // 32-wide head-dim chunks (Q.K contraction)
  constexpr int DT = D / 16;             // 16-wide output dim blocks
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int CALLS = KT * CH / NT;    // LDS loads per thread per tile and series
  constexpr int ROWS = NWV * QG * 16;    // query rows per workgroup
  constexpr int LPT = CALLS * (SHARED ? 1 : 2);  // vector-memory ops per wave per tile
  static_assert(KT * CH % NT == 0, "every thread loads whole chunks");
  // four tile buffers, each its own array so the compiler can tell a read of
  // one from the loads into another
  constexpr int VSZ = SHARED ? 8 : KT * D;
  __shared__ __attribute__((aligned(16))) bf16_t ks0[KT * D], ks1[KT * D], ks2[KT * D], ks3[KT * D];
  __shared__ __attribute__((aligned(16))) bf16_t vs0[VSZ], vs1[VSZ], vs2[VSZ], vs3[VSZ];
  auto kbuf = [&](auto c) __attribute__((always_inline)) -> bf16_t* {
    if constexpr (decltype(c)::value == 0) return ks0;
    else if constexpr (decltype(c)::value == 1) return ks1;
    else if constexpr (decltype(c)::value == 2) return ks2;
    else return ks3;
  };
  auto vbuf = [&](auto c) __attribute__((always_inline)) -> bf16_t* {
    if constexpr (SHARED) return kbuf(c);
    else if constexpr (decltype(c)::value == 0) return vs0;
    else if constexpr (decltype(c)::value == 1) return vs1;
    else if constexpr (decltype(c)::value == 2) return vs2;
    else return vs3;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (LDS load bases)
  const int n = lane & 15, kq = lane >> 4;
  const int swz_n = swz<D>(n), swz_tr = swz<D>(4 * kq + (n >> 2));  // (invariant under +16 rows)
  const int bid = blockIdx.x;
  const int rblk = bid % p.row_blocks;
  const int bh = bid / p.row_blocks;
  const int kvh = bh % (int)p.hkv, b = bh / (int)p.hkv;
  const int G = (int)p.G;
  const int rows_total = (int)p.q_len * G;
  const int row0 = rblk * ROWS;
  const int row_last = row0 + ROWS - 1 < rows_total ? row0 + ROWS - 1 : rows_total - 1;
  const int q0 = (int)p.q_pos0;
  const int p_first = q0 + row0 / G, p_last = q0 + row_last / G;
  const PreStr ST = pre_strides<DN, D>(p);

  // this wave's 16-row query groups: B operands and per-row visibility
  uint4 qr[QG][KS];
  int my_np[QG], my_rb[QG], my_pos[QG];
  int my_rr[QG];  // flat row (position in the chunk * G + head in the group)
  bool my_ok[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const int r = row0 + wave * (QG * 16) + g * 16 + n;
    const bool ok = r < rows_total;
    const int rr = ok ? r : rows_total - 1;
    const int pl = rr / G, hg = rr - pl * G;
    int64_t np, rb;
    visible_range(q0 + pl, p.m, p.W, p.mode, &np, &rb);
    my_np[g] = (int)np;
    my_rb[g] = (int)rb;
    my_pos[g] = q0 + pl;
    my_ok[g] = ok;
    my_rr[g] = rr;
    const bf16_t* qrow = p.q + qoff(ST.q, b, pl, (int64_t)kvh * G + hg) + 8 * kq;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qr[g][s] = ok ? *reinterpret_cast<const uint4*>(qrow + 32 * s) : make_uint4(0, 0, 0, 0);
  }

  int64_t t64a, t64b;
  visible_range(p_last, p.m, p.W, p.mode, &t64a, &t64b);
  const int NP = (int)t64a, RBmax = (int)t64b;
  visible_range(p_first, p.m, p.W, p.mode, &t64a, &t64b);
  const int NPmin = (int)t64a, RB = (int)t64b;
  const int T1 = (NP + KT - 1) / KT;
  const int T = T1 + (p_last - RB + 1 + KT - 1) / KT;
  // slice bases as integers (a pointer select from the argument block would
  // become a private-memory lookup)
  // row strides in bytes; a shared series reads values with the key strides
  const uint32_t pks = 2u * (uint32_t)ST.pk.s2, rks = 2u * (uint32_t)ST.rk.s2;
  const uint32_t pvs = SHARED ? pks : 2u * (uint32_t)ST.pv.s2, rvs = SHARED ? rks : 2u * (uint32_t)ST.rv.s2;
  const int64_t b64 = b, kvh64 = kvh;
  const uintptr_t pk_base = reinterpret_cast<uintptr_t>(p.pk + b64 * ST.pk.s0 + kvh64 * ST.pk.s1);
  const uintptr_t pv_base =
      SHARED ? pk_base : reinterpret_cast<uintptr_t>(p.pv + b64 * ST.pv.s0 + kvh64 * ST.pv.s1);
  // raw bases at position 0 (row -raw_pos_base)
  const uintptr_t rk_base = reinterpret_cast<uintptr_t>(p.rk + b64 * ST.rk.s0 + kvh64 * ST.rk.s1) -
                            (uintptr_t)(p.raw_pos_base * rks);
  const uintptr_t rv_base =
      SHARED ? rk_base
             : reinterpret_cast<uintptr_t>(p.rv + b64 * ST.rv.s0 + kvh64 * ST.rv.s1) -
                   (uintptr_t)(p.raw_pos_base * rvs);

  // LDS layout: row r of a tile holds its 16-byte chunks in swizzled order,
  // chunk c at position c ^ swz(r), so that the 16-byte K reads of 8 rows and
  // the transposing V reads of 4 rows land on distinct banks without padding.
  // Tile loads go straight to LDS (global_load_lds_dwordx4: lane i of a wave
  // writes 16 bytes at the wave's LDS base + 16 i), so each lane loads the
  // global chunk that belongs at its slot.  Rows past the list re-read its
  // last row (finite data; their scores are masked, so their weights are 0).
  auto load_tile = [&](int tile, auto bufc) __attribute__((always_inline)) {
    const bool pooled = tile < T1;
    const int x0 = pooled ? tile * KT : RB + (tile - T1) * KT;
    const int lim = pooled ? NP : p_last + 1;
    const uintptr_t kb = pooled ? pk_base : rk_base, vb = pooled ? pv_base : rv_base;
    const uint32_t ks = pooled ? pks : rks, vs = pooled ? pvs : rvs;
#pragma unroll
    for (int i = 0; i < CALLS; ++i) {
      const int slot = i * NT + tid;
      const int r = slot / CH, pos = slot % CH;
      const int x = x0 + r < lim ? x0 + r : lim - 1;
      const uint32_t col = 16u * (pos ^ swz<D>(r));
      const int dst = (i * NT + wave * 64) * 8;  // bf16 elements, wave-uniform
      __builtin_amdgcn_global_load_lds(reinterpret_cast<gbl_void*>(kb + (uint64_t)(uint32_t)x * ks + col),
                                       (lds_void*)(kbuf(bufc) + dst), 16, 0, 0);
      if constexpr (!SHARED)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<gbl_void*>(vb + (uint64_t)(uint32_t)x * vs + col),
                                         (lds_void*)(vbuf(bufc) + dst), 16, 0, 0);
    }
  };

  float m_run[QG], l_run[QG];
  f32x4 acc[QG][DT];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    m_run[g] = kNegInf;
    l_run[g] = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // S^T = K Q^T: 16 keys x 16 rows per MFMA; each K operand feeds QG MFMAs
  auto qk = [&](const bf16_t* kt, f32x4 (&sc)[KB][QG]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      uint4 ka[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        ka[s] = *reinterpret_cast<const uint4*>(&kt[(16 * kb + n) * D + 8 * ((4 * s + kq) ^ swz_n)]);
#pragma unroll
      for (int g = 0; g < QG; ++g) sc[kb][g] = f32x4{0.f, 0.f, 0.f, 0.f};
      // the QG accumulation chains interleaved: consecutive MFMAs are independent
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int g = 0; g < QG; ++g)
          sc[kb][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[s]),
                                                               __builtin_bit_cast(bf16x8, qr[g][s]), sc[kb][g], 0, 0, 0);
    }
  };

  // Softmax of one tile in two parts.  Part A (branches): the mask where some
  // row does not see the whole tile, the tile max and the lazy rescale.  Part
  // B (branch-free): exponentials, row sums and the bf16 pack of P^T, issued
  // in the same block as the next tile's Q.K MFMAs so the two interleave.
  auto softmax_a = [&](int tile, f32x4 (&sc)[KB][QG], float (&mu)[QG]) __attribute__((always_inline)) {
    const bool pooled = tile < T1;
    const int x0 = pooled ? tile * KT : RB + (tile - T1) * KT;
    const bool full = pooled ? (tile + 1) * KT <= NPmin : (x0 >= RBmax && x0 + KT - 1 <= p_first);
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      if (!full) {  // one uniform branch around the whole mask
        // visible x: [lo, hi] (pooled: [0, n_pooled - 1]; raw: [raw_begin, t])
        const int lo = pooled ? 0 : my_rb[g], hi = pooled ? my_np[g] - 1 : my_pos[g];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int x = x0 + 16 * kb + 4 * kq + j;
            sc[kb][g][j] = (x >= lo && x <= hi) ? sc[kb][g][j] : kNegInf;
          }
      }
      // Running max with lazy rescaling: the reference max of a row moves only
      // when a score exceeds it by more than 2^8 (any reference gives the same
      // softmax; weights stay below 2^8, far from fp32 or bf16 overflow), so
      // the fp32 accumulators are rescaled on few tiles.  The scale is folded
      // into the exponent: p = 2^(s * scale*log2(e) - m).
      float tmax = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) tmax = fmaxf(tmax, sc[kb][g][j]);
      tmax = xor16_max(tmax);
      tmax = xor32_max(tmax) * p.scale_log2;
      if (__ballot(tmax > m_run[g] + 8.f)) {
        const float nm = fmaxf(m_run[g], tmax);
        const float corr = nm == kNegInf ? 1.f : fast_exp2(m_run[g] - nm);
        l_run[g] *= corr;
#pragma unroll
        for (int t = 0; t < DT; ++t) acc[g][t] *= corr;
        m_run[g] = nm;
      }
      mu[g] = m_run[g] == kNegInf ? 0.f : m_run[g];
    }
  };
  auto softmax_b = [&](f32x4 (&sc)[KB][QG], const float (&mu)[QG], uint4 (&pb)[KB / 2][QG])
                       __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      float psum = 0.f;
      uint32_t w[KB][2];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float pj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pj[j] = fast_exp2(fmaf(sc[kb][g][j], p.scale_log2, -mu[g]));
          psum += pj[j];
        }
        w[kb][0] = pack_bf16x2(pj[0], pj[1]);
        w[kb][1] = pack_bf16x2(pj[2], pj[3]);
      }
#pragma unroll
      for (int c = 0; c < KB / 2; ++c) pb[c][g] = make_uint4(w[2 * c][0], w[2 * c][1], w[2 * c + 1][0], w[2 * c + 1][1]);
      l_run[g] += psum;
    }
  };
  // O^T += V^T P^T: k = 32 keys (two 16-key blocks); A from two transposing reads,
  // lane (n, kq) at row 4kq + n/4 (+16 per key block), column 16t + 4(n%4)
  auto pv = [&](const uint4 (&pb)[KB / 2][QG], const bf16_t* vt) __attribute__((always_inline)) {
    s16x4 va[16];
    read_v_tiles<D>(va, vt, n, kq, swz_tr);
#pragma unroll
    for (int c = 0; c < KB / 2; ++c)
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const s16x4 a0 = va[(c * DT + t) * 2], a1 = va[(c * DT + t) * 2 + 1];
        const bf16x8 a = __builtin_bit_cast(bf16x8, s16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
#pragma unroll
        for (int g = 0; g < QG; ++g)
          acc[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, pb[c][g]), acc[g][t], 0, 0, 0);
      }
  };

  // Tile loop, software-pipelined and unrolled by the four buffers: step
  // `tile` waits for tile+1's loads (tile+2's may stay in flight), then a
  // barrier (every wave's part has landed; the buffer of tile-1 is free),
  // requests tile+3 into that buffer, runs part A of tile's softmax, issues
  // tile+1's Q.K MFMAs interleaved with part B, then tile's P.V MFMAs.
  f32x4 s_a[KB][QG], s_b[KB][QG];  // scores of the current and the next tile, roles alternating
  auto step = [&](int tile, auto bufc, f32x4 (&s_cur)[KB][QG], f32x4 (&s_next)[KB][QG]) __attribute__((always_inline)) {
    constexpr int B = decltype(bufc)::value;
    if (tile + 1 < T) {
      if (tile + 2 < T) vmcnt_wait<LPT>();
      else vmcnt_wait<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (tile + 3 < T) load_tile(tile + 3, std::integral_constant<int, (B + 3) % 4>{});
    float mu[QG];
    softmax_a(tile, s_cur, mu);
    uint4 pb[KB / 2][QG];
    if (tile + 1 < T) {
      qk(kbuf(std::integral_constant<int, (B + 1) % 4>{}), s_next);
      softmax_b(s_cur, mu, pb);
#if LBCA_PREFILL_SCHED
      // per 16-key block of the next tile: its K reads, then each MFMA beside
      // a share of the exponentials
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
#pragma unroll
        for (int i = 0; i < KS * QG; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, LBCA_PREFILL_SCHED, 0);
        }
      }
#endif
    } else {
      softmax_b(s_cur, mu, pb);
    }
    pv(pb, vbuf(bufc));
  };
  if (0 < T) load_tile(0, std::integral_constant<int, 0>{});
  if (1 < T) load_tile(1, std::integral_constant<int, 1>{});
  if (2 < T) load_tile(2, std::integral_constant<int, 2>{});
  if (T > 2) vmcnt_wait<2 * LPT>();
  else if (T > 1) vmcnt_wait<LPT>();
  else vmcnt_wait<0>();
  __builtin_amdgcn_s_barrier();
  if (T > 0) qk(kbuf(std::integral_constant<int, 0>{}), s_a);
  for (int tile = 0; tile < T; tile += 4) {
    step(tile, std::integral_constant<int, 0>{}, s_a, s_b);
    if (tile + 1 >= T) break;
    step(tile + 1, std::integral_constant<int, 1>{}, s_b, s_a);
    if (tile + 2 >= T) break;
    step(tile + 2, std::integral_constant<int, 2>{}, s_a, s_b);
    if (tile + 3 >= T) break;
    step(tile + 3, std::integral_constant<int, 3>{}, s_b, s_a);
  }

#pragma unroll
  for (int g = 0; g < QG; ++g) {
    float l = xor16_sum(l_run[g]);
    l = xor32_sum(l);
    if (!my_ok[g]) continue;
    const int pl = my_rr[g] / G;
    const int64_t h = (int64_t)kvh * G + (my_rr[g] - pl * G);
    const int64_t ooff = qoff(ST.o, b, pl, h);
    if (p.sink) l += fast_exp2(p.sink[h] * kLog2e - m_run[g]);
    const float inv = 1.f / l;
    if (p.out_bf16) {
      bf16_t* o = static_cast<bf16_t*>(p.out) + ooff + 4 * kq;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        uint2 w;
        w.x = pack_bf16x2(acc[g][t][0] * inv, acc[g][t][1] * inv);
        w.y = pack_bf16x2(acc[g][t][2] * inv, acc[g][t][3] * inv);
        *reinterpret_cast<uint2*>(o + 16 * t) = w;
      }
    } else {
      float* o = static_cast<float*>(p.out) + ooff + 4 * kq;
#pragma unroll
      for (int t = 0; t < DT; ++t)
        *reinterpret_cast<float4*>(o + 16 * t) =
            make_float4(acc[g][t][0] * inv, acc[g][t][1] * inv, acc[g][t][2] * inv, acc[g][t][3] * inv);
    }
    if (p.lse && kq == 0) p.lse[((int64_t)b * p.q_len + pl) * p.hq + h] = (m_run[g] + log2f(l)) * 0.69314718055994531f;
  }
}

// Raw buffer resource over [base, base + bytes) (bytes below 2^31) and a
// 16-byte load from it at vector offset + scalar offset; offsets at or past
// the limit read zeros without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(uintptr_t base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ldb16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0));
}

// ---------------------------------------------------------------------------
// 128-dim prefill on 32x32 MFMA tiles with a register-staged, four-buffer tile
// pipeline.
//
// Same work split as prefill_kernel (8 waves, 256 rows of the flattened
// (position, GQA head) space per workgroup, 32-key tiles, a per-query visible
// span), but each wave holds its 32 query rows as one 32-column block and uses
// v_mfma_f32_32x32x16_bf16, which moves twice the flops per cycle of the
// 16x16x32 form on this part:
//   S^T (32 keys x 32 rows) = K (32 x 16 dims) Q^T, eight MFMAs per tile; lane
//   (n, h) then holds 16 scores of query row n: keys 8j + 4h + r (j, r < 4), so
//   a row's max and sum need one 32-lane swap;
//   O^T (4 x 32 dims x 32 rows) += V^T P^T, two MFMAs of 16 keys per 32-dim
//   block: P^T is the score layout itself (key k-slot order 4h..4h+3,
//   8+4h..8+4h+3, then +16), V^T comes from transposing LDS reads in the same
//   key order.
// The loop: tile u goes global -> registers at step u-4 and registers -> LDS
// buffer u % 4 at step u-2 (plain stores, so the compiler counts every LDS
// operation; one barrier per step makes a tile visible).  Step t issues the
// reads of V(t) and K(t+1), then the exponentials of tile t beside the Q.K
// MFMAs of tile t+1, then P.V of tile t and the mask and max of tile t+1; the
// (rare) accumulator rescale closes the step.
template <bool SHARED, bool DN>
__global__ __launch_bounds__(512, 1) void prefill128_kernel(PrefillParams p) {
  constexpr int D = 128, NWV = 8, NT = 512, KT = 32, DC = D / 16, DB = D / 32, CH = 16;
  constexpr int ROWS = NWV * 32;  // 256
  constexpr int TILE = KT * D;    // bf16 elements of one K (or V) tile
  static_assert(KT * CH == NT, "one 16-byte chunk per thread per tile and series");
  __shared__ __attribute__((aligned(16))) bf16_t lds[4 * (SHARED ? 1 : 2) * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int bid = blockIdx.x;
  const int rblk = bid % p.row_blocks;
  const int bh = bid / p.row_blocks;
  const int kvh = bh % (int)p.hkv, b = bh / (int)p.hkv;
  const int G = (int)p.G;
  const int rows_total = (int)p.q_len * G;
  const int row0 = rblk * ROWS;
  const int row_last = row0 + ROWS - 1 < rows_total ? row0 + ROWS - 1 : rows_total - 1;
  const int q0 = (int)p.q_pos0;
  const int p_first = q0 + row0 / G, p_last = q0 + row_last / G;
  const PreStr ST = pre_strides<DN, D>(p);

  // this lane's query row (B operand: dims 16c + 8h .. +8) and its visibility
  uint4 qr[DC];
  int my_np, my_rb, my_pos;
  int my_rr;  // flat row (position in the chunk * G + head in the group)
  bool my_ok;
  {
    const int r = row0 + wave * 32 + n;
    my_ok = r < rows_total;
    const int rr = my_ok ? r : rows_total - 1;
    const int pl = rr / G, hg = rr - pl * G;
    int64_t np, rb;
    visible_range(q0 + pl, p.m, p.W, p.mode, &np, &rb);
    my_np = (int)np;
    my_rb = (int)rb;
    my_pos = q0 + pl;
    my_rr = rr;
    const bf16_t* qrow = p.q + qoff(ST.q, b, pl, (int64_t)kvh * G + hg) + 8 * h;
#pragma unroll
    for (int c = 0; c < DC; ++c)
      qr[c] = my_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * c) : make_uint4(0, 0, 0, 0);
  }

  int64_t t64a, t64b;
  visible_range(p_last, p.m, p.W, p.mode, &t64a, &t64b);
  const int NP = (int)t64a, RBmax = (int)t64b;
  visible_range(p_first, p.m, p.W, p.mode, &t64a, &t64b);
  const int NPmin = (int)t64a, RB = (int)t64b;
  const int T1 = (NP + KT - 1) / KT;
  const int T = T1 + (p_last - RB + 1 + KT - 1) / KT;
  // row strides in bytes; a shared series reads values with the key strides
  const uint32_t pks = 2u * (uint32_t)ST.pk.s2, rks = 2u * (uint32_t)ST.rk.s2;
  const uint32_t pvs = SHARED ? pks : 2u * (uint32_t)ST.pv.s2, rvs = SHARED ? rks : 2u * (uint32_t)ST.rv.s2;
  const int64_t b64 = b, kvh64 = kvh;
  const uintptr_t pk_base = reinterpret_cast<uintptr_t>(p.pk + b64 * ST.pk.s0 + kvh64 * ST.pk.s1);
  const uintptr_t pv_base =
      SHARED ? pk_base : reinterpret_cast<uintptr_t>(p.pv + b64 * ST.pv.s0 + kvh64 * ST.pv.s1);
  // raw bases at position 0 (row -raw_pos_base)
  const uintptr_t rk_base = reinterpret_cast<uintptr_t>(p.rk + b64 * ST.rk.s0 + kvh64 * ST.rk.s1) -
                            (uintptr_t)(p.raw_pos_base * rks);
  const uintptr_t rv_base =
      SHARED ? rk_base
             : reinterpret_cast<uintptr_t>(p.rv + b64 * ST.rv.s0 + kvh64 * ST.rv.s1) -
                   (uintptr_t)(p.raw_pos_base * rvs);

  // LDS tile layout: row r holds its 16-byte chunks in swizzled order, chunk
  // x at position x ^ swz(r); this thread's chunk of every tile is LDS slot
  // 8 * tid = (row tid / 16, position tid % 16), global chunk position ^ swz.
  const int st_r = tid / CH, st_c = tid % CH;
  const uint32_t st_goff = 16u * (uint32_t)(st_c ^ swz<D>(st_r));
  // tile u lives in buffer u % 4 (compile-time below, so buffer bases fold into
  // the LDS instructions' offsets)
  auto kbuf = [&](auto c) -> bf16_t* { return lds + decltype(c)::value * (SHARED ? 1 : 2) * TILE; };
  auto vbuf = [&](auto c) -> bf16_t* { return SHARED ? kbuf(c) : kbuf(c) + TILE; };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // two tiles' chunks in flight between global memory and LDS: tile u goes to
  // staging slot u % 2 at step u - 4 and into LDS at step u - 2
  uint4 stg_k[2], stg_v[2];
  // (captures by value: a select between references to the bases would become
  // a private-memory table lookup)
  // Tile rows come through buffer resources (scalar base and byte limit) with
  // a wave-uniform tile offset and this thread's fixed vector offset: no
  // vector address register that later instructions could overwrite while a
  // load is in flight (which would make the compiler wait for it), and rows
  // past the span's end (the last tile's tail) read as zeros without touching
  // memory.  Each span's limit is its last visible row.
  const int64_t raw_n = (int64_t)p_last + 1 - p.raw_pos_base;  // raw rows up to the last position
  const uintptr_t rk_slice = rk_base + (uintptr_t)(p.raw_pos_base * rks);
  const uintptr_t rv_slice = rv_base + (uintptr_t)(p.raw_pos_base * rvs);
  const int64_t pk_lim = (int64_t)NP * pks, pv_lim = (int64_t)NP * pvs, rk_lim = raw_n * rks, rv_lim = raw_n * rvs;
  const __amdgpu_buffer_rsrc_t rs_pk = make_rsrc(pk_base, pk_lim);
  const __amdgpu_buffer_rsrc_t rs_pv = make_rsrc(pv_base, pv_lim);
  const __amdgpu_buffer_rsrc_t rs_rk = make_rsrc(rk_slice, rk_lim);
  const __amdgpu_buffer_rsrc_t rs_rv = make_rsrc(rv_slice, rv_lim);
  const uint32_t st_voff = (uint32_t)(st_r * D * 2) + st_goff;  // (dense rows)
  auto fetch = [=, &stg_k, &stg_v](int u, auto slot) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    (void)stg_v;
    const bool pooled = u < T1;
    const int r0 = pooled ? u * KT : RB - (int)p.raw_pos_base + (u - T1) * KT;  // first row of the tile
    if constexpr (DN) {
      const int soff = r0 * (D * 2);
      stg_k[SL] = ldb16(pooled ? rs_pk : rs_rk, st_voff, soff);
      if constexpr (!SHARED) stg_v[SL] = ldb16(pooled ? rs_pv : rs_rv, st_voff, soff);
    } else {
      // strided rows: the descriptor is built per tile from a selected base and
      // limit (a select between two descriptors goes through private memory)
      const uint32_t ks = pooled ? pks : rks;
      stg_k[SL] = ldb16(make_rsrc(pooled ? pk_base : rk_slice, pooled ? pk_lim : rk_lim),
                        (uint32_t)st_r * ks + st_goff, (int)(r0 * ks));
      if constexpr (!SHARED) {
        const uint32_t vs = pooled ? pvs : rvs;
        stg_v[SL] = ldb16(make_rsrc(pooled ? pv_base : rv_slice, pooled ? pv_lim : rv_lim),
                          (uint32_t)st_r * vs + st_goff, (int)(r0 * vs));
      }
    }
  };
  auto stash = [&](auto c, auto slot) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    *reinterpret_cast<uint4*>(kbuf(c) + 8 * tid) = stg_k[SL];
    if constexpr (!SHARED) *reinterpret_cast<uint4*>(vbuf(c) + 8 * tid) = stg_v[SL];
  };

  float m_run = kNegInf, mu = 0.f, l_run = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  auto is_full = [&](int u) -> bool {
    const bool pooled = u < T1;
    const int x0 = pooled ? u * KT : RB + (u - T1) * KT;
    return pooled ? (u + 1) * KT <= NPmin : (x0 >= RBmax && x0 + KT - 1 <= p_first);
  };
  // K A operands of dim chunks [c0, c0 + 4): lane (key n, h), dims 16c + 8h .. +8
  auto read_k = [&](auto c, int c0, uint4 (&ka)[4]) __attribute__((always_inline)) {
    const bf16_t* kt = kbuf(c) + n * D;
    const int sw = swz<D>(n);
#pragma unroll
    for (int i = 0; i < 4; ++i) ka[i] = *reinterpret_cast<const uint4*>(kt + 8 * ((2 * (c0 + i) + h) ^ sw));
  };
  // V^T A operands: lane (dim 16 (q % 2) + i, h = q / 2) of 16-lane group q, for
  // 32-dim block db and key half kh: keys 16kh + 4h.. and 16kh + 8 + 4h.., two
  // transposing reads (lane j of the group points at row base + j / 4,
  // dims 4 (j % 4) ..+4 of its 16-dim half)
  const int vq = lane >> 4, vj = lane & 15;
  const int v_row = 4 * (vq >> 1) + (vj >> 2), v_col = 16 * (vq & 1) + 4 * (vj & 3);
  auto read_v = [&](auto c, s16x4 (&va)[DB][2][2]) __attribute__((always_inline)) {
    const bf16_t* vt = vbuf(c);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 16 * kh + 8 * u + v_row;
          const int col = 32 * db + v_col;
          const bf16_t* a = vt + r * D + 8 * ((col >> 3) ^ swz<D>(r)) + (col & 7);
          va[db][kh][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a));
        }
  };
  auto qk = [&](const uint4 (&ka)[4], int c0, f32x16& sc) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[i]),
                                                   __builtin_bit_cast(bf16x8, qr[c0 + i]), sc, 0, 0, 0);
  };
  // mask (tiles some row does not fully see) and this lane's max of the tile in
  // scaled log2 units (the row max over the row's two lanes is taken only when
  // some lane's max passes the reference)
  auto mask_max = [&](int u, bool full, f32x16& sc) __attribute__((always_inline)) -> float {
    if (!full) {
      const bool pooled = u < T1;
      const int x0 = pooled ? u * KT : RB + (u - T1) * KT;
      const int lo = pooled ? 0 : my_rb, hi = pooled ? my_np - 1 : my_pos;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int x = x0 + 8 * (e >> 2) + 4 * h + (e & 3);
        sc[e] = (x >= lo && x <= hi) ? sc[e] : kNegInf;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc[e]);
    return mx * p.scale_log2;
  };
  // lazy reference max: moves only when a score passes it by 2^8; the
  // accumulators (which hold every tile before this one) are rescaled then
  auto rescale = [&](float tmax) __attribute__((always_inline)) {
    if (__ballot(tmax > m_run + 8.f)) {
      const float nm = fmaxf(m_run, xor32_max(tmax));  // the row's max over its two lanes
      const float corr = nm == kNegInf ? 1.f : fast_exp2(m_run - nm);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= corr;
      m_run = nm;
    }
    mu = m_run == kNegInf ? 0.f : m_run;
  };
  // P^T B operands (16 keys each): the score layout itself, rounded to bf16
  auto exps = [&](const f32x16& sc, uint4 (&pb)[2]) __attribute__((always_inline)) {
    float pj[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) pj[e] = fast_exp2(fmaf(sc[e], p.scale_log2, -mu));
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ps += pj[e];
    l_run += ps;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
      pb[kh] = make_uint4(pack_bf16x2(pj[8 * kh + 0], pj[8 * kh + 1]), pack_bf16x2(pj[8 * kh + 2], pj[8 * kh + 3]),
                          pack_bf16x2(pj[8 * kh + 4], pj[8 * kh + 5]), pack_bf16x2(pj[8 * kh + 6], pj[8 * kh + 7]));
  };
  auto pv = [&](const s16x4 (&va)[DB][2][2], const uint4 (&pb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4 a0 = va[db][kh][0], a1 = va[db][kh][1];
        const bf16x8 a = __builtin_bit_cast(bf16x8, s16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pb[kh]), acc[db], 0, 0, 0);
      }
  };

  // prologue: tiles 0 and 1 into LDS, tiles 2 and 3 in flight; scores of tile 0
  f32x16 s_a = f32x16{}, s_b = f32x16{};
  if (T > 0) {
    fetch(0, I0{});
    stash(I0{}, I0{});
    if (T > 1) {
      fetch(1, I1{});
      stash(I1{}, I1{});
    }
    if (T > 2) fetch(2, I0{});
    if (T > 3) fetch(3, I1{});
    __syncthreads();
#pragma unroll
    for (int c0 = 0; c0 < DC; c0 += 4) {
      uint4 ka[4];
      read_k(I0{}, c0, ka);
      qk(ka, c0, s_a);
    }
    rescale(mask_max(0, is_full(0), s_a));
  }
  // step t (tile t in buffer C): S(t) in s_cur (masked, mu set for it); S(t+1) into s_next
  auto step = [&](int t, auto c, f32x16& s_cur, f32x16& s_next) __attribute__((always_inline)) {
    constexpr int C = decltype(c)::value;
    using CN = std::integral_constant<int, (C + 1) % 4>;
    using CS = std::integral_constant<int, (C + 2) % 4>;
    using SL = std::integral_constant<int, C % 2>;  // staging slot of tiles t+2 and t+4
    __syncthreads();  // tile t+1 (stored last step) visible; tile t-2's buffer free
    if (t + 2 < T) {
      stash(CS{}, SL{});  // waits for its rows (fetched two steps ago)
      if (t + 4 < T) fetch(t + 4, SL{});
    }
    uint4 ka0[4], ka1[4];
    read_k(CN{}, 0, ka0);
    read_k(CN{}, 4, ka1);
    uint4 pb[2];
    exps(s_cur, pb);  // the exponentials of tile t beside the Q.K MFMAs of tile t+1
    s_next = f32x16{};
    qk(ka0, 0, s_next);
    qk(ka1, 4, s_next);
    s16x4 va[DB][2][2];
    read_v(c, va);
    pv(va, pb);       // P.V of tile t, then the mask and max of tile t+1
    rescale(mask_max(t + 1, is_full(t + 1), s_next));
  };
  for (int t = 0;; t += 4) {  // every tile but the last: one step per buffer
    if (t + 1 >= T) break;
    step(t, I0{}, s_a, s_b);
    if (t + 2 >= T) break;
    step(t + 1, I1{}, s_b, s_a);
    if (t + 3 >= T) break;
    step(t + 2, I2{}, s_a, s_b);
    if (t + 4 >= T) break;
    step(t + 3, I3{}, s_b, s_a);
  }
  if (T > 0) {  // the last tile: scores in s_a (even) or s_b (odd), buffer (T-1) % 4
    const int tl = T - 1;
    if (tl & 1) s_a = s_b;
    __syncthreads();
    uint4 pb[2];
    exps(s_a, pb);
    s16x4 va[DB][2][2];
    const bf16_t* vt = lds + (tl & 3) * (SHARED ? 1 : 2) * TILE + (SHARED ? 0 : TILE);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 16 * kh + 8 * u + v_row;
          const int col = 32 * db + v_col;
          const bf16_t* a = vt + r * D + 8 * ((col >> 3) ^ swz<D>(r)) + (col & 7);
          va[db][kh][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a));
        }
    pv(va, pb);
  }

  // finish: the row's sum over its two lanes, sink, normalisation, LSE; lane
  // (n, h) writes dims 32 db + 8 j + 4 h .. +4 of its row
  float l = xor32_sum(l_run);
  if (!my_ok) return;
  const int pl = my_rr / G;
  const int64_t head = (int64_t)kvh * G + (my_rr - pl * G);
  const int64_t ooff = qoff(ST.o, b, pl, head);
  if (p.sink) l += fast_exp2(p.sink[head] * kLog2e - m_run);
  const float inv = 1.f / l;
  if (p.out_bf16) {
    bf16_t* o = static_cast<bf16_t*>(p.out) + ooff + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint2 w;
        w.x = pack_bf16x2(acc[db][4 * j + 0] * inv, acc[db][4 * j + 1] * inv);
        w.y = pack_bf16x2(acc[db][4 * j + 2] * inv, acc[db][4 * j + 3] * inv);
        *reinterpret_cast<uint2*>(o + 32 * db + 8 * j) = w;
      }
  } else {
    float* o = static_cast<float*>(p.out) + ooff + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(o + 32 * db + 8 * j) =
            make_float4(acc[db][4 * j + 0] * inv, acc[db][4 * j + 1] * inv, acc[db][4 * j + 2] * inv,
                        acc[db][4 * j + 3] * inv);
  }
  if (p.lse && h == 0) p.lse[((int64_t)b * p.q_len + pl) * p.hq + head] = (m_run + log2f(l)) * 0.69314718055994531f;
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
  p.q_st = a.q_st; p.o_st = a.out_st;
  p.pk_st = a.pooled_k_st; p.pv_st = a.pooled_v_st; p.rk_st = a.raw_k_st; p.rv_st = a.raw_v_st;
  const bool shared = a.pooled_v == nullptr;
  const int64_t B = a.batch, Hk = a.kv_heads, d = a.dim;
  const bool dn = dense_strides(a.q, a.q_st, {B, a.q_len, a.q_heads}, d) &&
                  dense_strides(a.out, a.out_st, {B, a.q_len, a.q_heads}, d) &&
                  dense_strides(a.pooled_k, a.pooled_k_st, {B, Hk, a.entries}, d) &&
                  dense_strides(a.pooled_v, a.pooled_v_st, {B, Hk, a.entries}, d) &&
                  dense_strides(a.raw_k, a.raw_k_st, {B, Hk, a.raw_rows}, d) &&
                  dense_strides(a.raw_v, a.raw_v_st, {B, Hk, a.raw_rows}, d);
  auto go = [&](auto kern, int waves, int rows) {
    p.row_blocks = (int)((a.q_len * p.G + rows - 1) / rows);
    const dim3 grid((unsigned)(a.batch * a.kv_heads * p.row_blocks));
    kern<<<grid, waves * 64, 0, stream>>>(p);
  };
  switch (a.dim) {
    case 64:
      if (shared) dn ? go(prefill_kernel<64, true, 8, 2, true>, 8, 256) : go(prefill_kernel<64, true, 8, 2, false>, 8, 256);
      else dn ? go(prefill_kernel<64, false, 8, 2, true>, 8, 256) : go(prefill_kernel<64, false, 8, 2, false>, 8, 256);
      break;
    case 128:
#if LBCA_PREFILL_V1
      {
        constexpr int W128 = LBCA_PREFILL_WAVES, Q128 = LBCA_PREFILL_QG;
        if (shared) go(prefill_kernel<128, true, W128, Q128, false>, W128, W128 * Q128 * 16);
        else go(prefill_kernel<128, false, W128, Q128, false>, W128, W128 * Q128 * 16);
      }
#else
      if (shared) dn ? go(prefill128_kernel<true, true>, 8, 256) : go(prefill128_kernel<true, false>, 8, 256);
      else dn ? go(prefill128_kernel<false, true>, 8, 256) : go(prefill128_kernel<false, false>, 8, 256);
#endif
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lbca
