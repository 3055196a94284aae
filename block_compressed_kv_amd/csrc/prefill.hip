// Prefill attention for a chunk of consecutive queries, each with its own
// visibility (pooled entries j < n_pooled(t) plus the raw span [raw_begin(t), t]).
//
// Method: "mSeek: learned KV-cache compression in a 3B model", "How LBCA works"
// (steps 4-5, and the chunked bounded-memory path that must agree with the
// clear reference): a query sees every completed summary older than its
// window plus its exact raw window, never a summary holding a later token.
//
// bf16 path (MFMA, a dense contraction).  A workgroup of 8 waves (two per
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
};

// Chunk swizzle of an LDS tile row (16-byte chunks): 8 consecutive rows read at
// one chunk index, or 4 consecutive rows read at two adjacent chunks, hit
// distinct banks.  Unchanged when the row moves by 16.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return (2 * r) & 15;
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

template <int D, bool SHARED, int NWV, int QG>
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

  // this wave's 16-row query groups: B operands and per-row visibility
  uint4 qr[QG][KS];
  int my_np[QG], my_rb[QG], my_pos[QG];
  int64_t my_out[QG];
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
    my_out[g] = (((int64_t)b * p.q_len + pl) * p.hq + (int64_t)kvh * G + hg) * D;
    const bf16_t* qrow = p.q + my_out[g] + 8 * kq;
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
  const uintptr_t pk_base = reinterpret_cast<uintptr_t>(p.pk) + ((int64_t)bh * p.entries) * (D * 2);
  const uintptr_t pv_base = reinterpret_cast<uintptr_t>(SHARED ? p.pk : p.pv) + ((int64_t)bh * p.entries) * (D * 2);
  const uintptr_t rk_base = reinterpret_cast<uintptr_t>(p.rk) + ((int64_t)bh * p.raw_rows - p.raw_pos_base) * (D * 2);
  const uintptr_t rv_base = reinterpret_cast<uintptr_t>(SHARED ? p.rk : p.rv) + ((int64_t)bh * p.raw_rows - p.raw_pos_base) * (D * 2);

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
#pragma unroll
    for (int i = 0; i < CALLS; ++i) {
      const int slot = i * NT + tid;
      const int r = slot / CH, pos = slot % CH;
      const int x = x0 + r < lim ? x0 + r : lim - 1;
      const uint64_t off = (uint64_t)(int64_t)x * (D * 2) + 16u * (pos ^ swz<D>(r));
      const int dst = (i * NT + wave * 64) * 8;  // bf16 elements, wave-uniform
      __builtin_amdgcn_global_load_lds(reinterpret_cast<gbl_void*>(kb + off), (lds_void*)(kbuf(bufc) + dst), 16, 0, 0);
      if constexpr (!SHARED)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<gbl_void*>(vb + off), (lds_void*)(vbuf(bufc) + dst), 16, 0, 0);
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
    const int64_t h = (my_out[g] / D) % p.hq;
    if (p.sink) l += fast_exp2(p.sink[h] * kLog2e - m_run[g]);
    const float inv = 1.f / l;
    if (p.out_bf16) {
      bf16_t* o = static_cast<bf16_t*>(p.out) + my_out[g] + 4 * kq;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        uint2 w;
        w.x = pack_bf16x2(acc[g][t][0] * inv, acc[g][t][1] * inv);
        w.y = pack_bf16x2(acc[g][t][2] * inv, acc[g][t][3] * inv);
        *reinterpret_cast<uint2*>(o + 16 * t) = w;
      }
    } else {
      float* o = static_cast<float*>(p.out) + my_out[g] + 4 * kq;
#pragma unroll
      for (int t = 0; t < DT; ++t)
        *reinterpret_cast<float4*>(o + 16 * t) =
            make_float4(acc[g][t][0] * inv, acc[g][t][1] * inv, acc[g][t][2] * inv, acc[g][t][3] * inv);
    }
    if (p.lse && kq == 0) p.lse[my_out[g] / D] = (m_run[g] + log2f(l)) * 0.69314718055994531f;
  }
}

// ---------------------------------------------------------------------------
// 128-dim prefill with a register-staged, four-buffer tile pipeline.
//
// Same work split, operand layouts and softmax as prefill_kernel (8 waves, 256
// rows of the flattened (position, GQA head) space per workgroup, 32-key tiles,
// S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16), but the loop is
// arranged so that every phase pairs matrix work with independent vector work
// and the LDS reads of a phase are issued one phase ahead:
//   tile u: global rows -> registers at step u-4, registers -> LDS buffer
//   u % 4 at step u-2 (one barrier per step makes it visible);
//   step t: the reads of V(t) and K(t+1) go out first, then
//     block A: exponentials of tile t beside the Q.K MFMAs of tile t+1,
//     block B: the P.V MFMAs of tile t beside the mask and max of tile t+1,
//   and the (rare) accumulator rescale for tile t+1 closes the step.
// Plain LDS stores and the transposing-read builtin let the compiler count
// LDS operations exactly (no LDS DMA whose waits it cannot place).
template <bool SHARED>
__global__ __launch_bounds__(512, 1) void prefill128_kernel(PrefillParams p) {
  constexpr int D = 128, NWV = 8, NT = 512, QG = 2, KT = 32, KB = 2, KS = 4, DT = 8, CH = 16;
  constexpr int ROWS = NWV * QG * 16;  // 256
  constexpr int TILE = KT * D;         // bf16 elements of one K (or V) tile
  static_assert(KT * CH == NT, "one 16-byte chunk per thread per tile and series");
  __shared__ __attribute__((aligned(16))) bf16_t lds[4 * (SHARED ? 1 : 2) * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, kq = lane >> 4;
  const int swz_n = swz<D>(n), swz_tr = swz<D>(4 * kq + (n >> 2));
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

  uint4 qr[QG][KS];
  int my_np[QG], my_rb[QG], my_pos[QG];
  int64_t my_out[QG];
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
    my_out[g] = (((int64_t)b * p.q_len + pl) * p.hq + (int64_t)kvh * G + hg) * D;
    const bf16_t* qrow = p.q + my_out[g] + 8 * kq;
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
  const uintptr_t pk_base = reinterpret_cast<uintptr_t>(p.pk) + ((int64_t)bh * p.entries) * (D * 2);
  const uintptr_t pv_base = reinterpret_cast<uintptr_t>(SHARED ? p.pk : p.pv) + ((int64_t)bh * p.entries) * (D * 2);
  const uintptr_t rk_base = reinterpret_cast<uintptr_t>(p.rk) + ((int64_t)bh * p.raw_rows - p.raw_pos_base) * (D * 2);
  const uintptr_t rv_base = reinterpret_cast<uintptr_t>(SHARED ? p.rk : p.rv) + ((int64_t)bh * p.raw_rows - p.raw_pos_base) * (D * 2);

  // this thread's chunk of every tile: LDS slot (r, c) = element 8 * tid holds
  // global chunk c ^ swz(r) of tile row r (the swizzled layout of prefill_kernel)
  const int st_r = tid / CH, st_c = tid % CH;
  const uint32_t st_goff = 16u * (uint32_t)(st_c ^ swz<D>(st_r));
  // tile u lives in buffer u % 4 (compile-time below, so buffer bases fold into
  // the LDS instructions' offsets)
  auto kbuf = [&](auto c) -> bf16_t* { return lds + decltype(c)::value * (SHARED ? 1 : 2) * TILE; };
  auto vbuf = [&](auto c) -> bf16_t* { return SHARED ? kbuf(c) : kbuf(c) + TILE; };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // two tiles' chunks in flight between global memory and LDS: tile u goes to
  // staging slot u % 2 at step u - 4 and into LDS at step u - 2
  uint4 stg_k[2], stg_v[2];
  // (captures by value: a select between references to the bases would become
  // a private-memory table lookup)
  auto fetch = [=, &stg_k, &stg_v](int u, auto slot) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    (void)stg_v;
    const bool pooled = u < T1;
    const int x0 = pooled ? u * KT : RB + (u - T1) * KT;
    const int lim = pooled ? NP : p_last + 1;
    const int x = x0 + st_r < lim ? x0 + st_r : lim - 1;  // rows past the list re-read its last row
    const uint64_t off = (uint64_t)(int64_t)x * (D * 2) + st_goff;
    const uintptr_t kb = pooled ? pk_base : rk_base, vb = pooled ? pv_base : rv_base;
    // global (not flat) loads: a flat load also counts against the LDS counter,
    // so every wait for an LDS read would wait for these rows too
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
    stg_k[SL] = __builtin_bit_cast(uint4, *reinterpret_cast<g_u32x4*>(kb + off));
    if constexpr (!SHARED) stg_v[SL] = __builtin_bit_cast(uint4, *reinterpret_cast<g_u32x4*>(vb + off));
  };
  auto stash = [&](auto c, auto slot) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    *reinterpret_cast<uint4*>(kbuf(c) + 8 * tid) = stg_k[SL];
    if constexpr (!SHARED) *reinterpret_cast<uint4*>(vbuf(c) + 8 * tid) = stg_v[SL];
  };

  // row sums come from the MFMA: an all-ones A operand against P^T gives every
  // lane its row's sum of the bf16 weights (the same weights P.V uses)
  float m_run[QG], mu[QG];
  f32x4 acc[QG][DT], lsum[QG];
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    m_run[g] = kNegInf;
    mu[g] = 0.f;
    lsum[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto is_full = [&](int u) -> bool {
    const bool pooled = u < T1;
    const int x0 = pooled ? u * KT : RB + (u - T1) * KT;
    return pooled ? (u + 1) * KT <= NPmin : (x0 >= RBmax && x0 + KT - 1 <= p_first);
  };
  auto read_k = [&](auto c, int kb, uint4 (&ka)[KS]) __attribute__((always_inline)) {
    const bf16_t* kt = kbuf(c);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      ka[s] = *reinterpret_cast<const uint4*>(&kt[(16 * kb + n) * D + 8 * ((4 * s + kq) ^ swz_n)]);
  };
  // V^T operand: lane (n, kq) at row 4kq + n/4 (+16 for the second key block),
  // column 16t + 4(n%4) (+ 8 ^ swizzle), two transposing reads per 16-dim block
  auto read_v = [&](auto c, s16x4 (&va)[2 * DT]) __attribute__((always_inline)) {
    const bf16_t* vt = vbuf(c);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const bf16_t* a = vt + (4 * kq + (n >> 2)) * D + 4 * (n & 1) + 8 * ((2 * t + ((n & 3) >> 1)) ^ swz_tr);
      va[2 * t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a));
      va[2 * t + 1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a + 16 * D));
    }
  };
  // S^T of one 16-key block: 16 keys x 16 rows per MFMA, each K operand feeding QG MFMAs
  auto qk = [&](const uint4 (&ka)[KS], f32x4 (&sc)[QG]) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < QG; ++g) sc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int g = 0; g < QG; ++g)
        sc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[s]),
                                                        __builtin_bit_cast(bf16x8, qr[g][s]), sc[g], 0, 0, 0);
  };
  // mask (tiles some row does not fully see) and this lane's max of the tile in
  // scaled log2 units (the row max over the row's four lanes is taken only when
  // some lane's max passes the reference)
  auto mask_max = [&](int u, bool full, f32x4 (&sc)[KB][QG], float (&tmax)[QG]) __attribute__((always_inline)) {
    const bool pooled = u < T1;
    const int x0 = pooled ? u * KT : RB + (u - T1) * KT;
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      if (!full) {
        const int lo = pooled ? 0 : my_rb[g], hi = pooled ? my_np[g] - 1 : my_pos[g];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int x = x0 + 16 * kb + 4 * kq + j;
            sc[kb][g][j] = (x >= lo && x <= hi) ? sc[kb][g][j] : kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sc[kb][g][j]);
      tmax[g] = mx * p.scale_log2;
    }
  };
  // lazy reference max: moves only when a score passes it by 2^8; the
  // accumulators (which hold every tile before this one) are rescaled then
  auto rescale = [&](const float (&tmax)[QG]) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      if (__ballot(tmax[g] > m_run[g] + 8.f)) {
        const float nm = fmaxf(m_run[g], xor32_max(xor16_max(tmax[g])));  // the row's max
        const float corr = nm == kNegInf ? 1.f : fast_exp2(m_run[g] - nm);
        lsum[g] *= corr;
#pragma unroll
        for (int t = 0; t < DT; ++t) acc[g][t] *= corr;
        m_run[g] = nm;
      }
      mu[g] = m_run[g] == kNegInf ? 0.f : m_run[g];
    }
  };
  auto exps = [&](const f32x4 (&sc)[KB][QG], uint4 (&pb)[QG]) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      uint32_t w[KB][2];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float pj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) pj[j] = fast_exp2(fmaf(sc[kb][g][j], p.scale_log2, -mu[g]));
        w[kb][0] = pack_bf16x2(pj[0], pj[1]);
        w[kb][1] = pack_bf16x2(pj[2], pj[3]);
      }
      pb[g] = make_uint4(w[0][0], w[0][1], w[1][0], w[1][1]);
    }
  };
  auto pv = [&](const s16x4 (&va)[2 * DT], const uint4 (&pb)[QG]) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < QG; ++g) lsum[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8, pb[g]), lsum[g], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const s16x4 a0 = va[2 * t], a1 = va[2 * t + 1];
      const bf16x8 a = __builtin_bit_cast(bf16x8, s16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
#pragma unroll
      for (int g = 0; g < QG; ++g)
        acc[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, pb[g]), acc[g][t], 0, 0, 0);
    }
  };

  // prologue: tiles 0 and 1 into LDS, tile 2 in flight; scores of tile 0
  f32x4 s_a[KB][QG], s_b[KB][QG];
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
    for (int kb = 0; kb < KB; ++kb) {
      uint4 ka[KS];
      read_k(I0{}, kb, ka);
      qk(ka, s_a[kb]);
    }
    float tm[QG];
    mask_max(0, is_full(0), s_a, tm);
    rescale(tm);
  }
  // step t (buffer of tile t: C): S(t) in s_cur (masked, mu set for it); S(t+1) into s_next
  auto step = [&](int t, auto c, f32x4 (&s_cur)[KB][QG], f32x4 (&s_next)[KB][QG]) __attribute__((always_inline)) {
    constexpr int C = decltype(c)::value;
    using CN = std::integral_constant<int, (C + 1) % 4>;
    using CS = std::integral_constant<int, (C + 2) % 4>;
    using SL = std::integral_constant<int, C % 2>;  // staging slot of tiles t+2 and t+4
    __syncthreads();  // tile t+1 (stored last step) visible; tile t-2's buffer free
    if (t + 2 < T) {
      stash(CS{}, SL{});  // waits for its rows (fetched two steps ago)
      if (t + 4 < T) fetch(t + 4, SL{});
    }
    uint4 ka0[KS], ka1[KS];
    read_k(CN{}, 0, ka0);
    read_k(CN{}, 1, ka1);
    uint4 pb[QG];
    // block A: exponentials of tile t beside the Q.K MFMAs of tile t+1
    exps(s_cur, pb);
    qk(ka0, s_next[0]);
    qk(ka1, s_next[1]);
    s16x4 va[2 * DT];
    read_v(c, va);
    // block B: P.V MFMAs of tile t, then the mask and max of tile t+1
    pv(va, pb);
    float tm[QG];
    mask_max(t + 1, is_full(t + 1), s_next, tm);
    rescale(tm);
  };
  using I3 = std::integral_constant<int, 3>;
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
    if (tl & 1) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int g = 0; g < QG; ++g) s_a[kb][g] = s_b[kb][g];
    }
    __syncthreads();
    uint4 pb[QG];
    exps(s_a, pb);
    s16x4 va[2 * DT];
    const bf16_t* vt = lds + (tl & 3) * (SHARED ? 1 : 2) * TILE + (SHARED ? 0 : TILE);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const bf16_t* a = vt + (4 * kq + (n >> 2)) * D + 4 * (n & 1) + 8 * ((2 * t + ((n & 3) >> 1)) ^ swz_tr);
      va[2 * t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a));
      va[2 * t + 1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a + 16 * D));
    }
    pv(va, pb);
  }
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    float l = lsum[g][0];
    if (!my_ok[g]) continue;
    const int64_t h = (my_out[g] / D) % p.hq;
    if (p.sink) l += fast_exp2(p.sink[h] * kLog2e - m_run[g]);
    const float inv = 1.f / l;
    if (p.out_bf16) {
      bf16_t* o = static_cast<bf16_t*>(p.out) + my_out[g] + 4 * kq;
#pragma unroll
      for (int tt = 0; tt < DT; ++tt) {
        uint2 w;
        w.x = pack_bf16x2(acc[g][tt][0] * inv, acc[g][tt][1] * inv);
        w.y = pack_bf16x2(acc[g][tt][2] * inv, acc[g][tt][3] * inv);
        *reinterpret_cast<uint2*>(o + 16 * tt) = w;
      }
    } else {
      float* o = static_cast<float*>(p.out) + my_out[g] + 4 * kq;
#pragma unroll
      for (int tt = 0; tt < DT; ++tt)
        *reinterpret_cast<float4*>(o + 16 * tt) =
            make_float4(acc[g][tt][0] * inv, acc[g][tt][1] * inv, acc[g][tt][2] * inv, acc[g][tt][3] * inv);
    }
    if (p.lse && kq == 0) p.lse[my_out[g] / D] = (m_run[g] + log2f(l)) * 0.69314718055994531f;
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
  const bool shared = a.pooled_v == nullptr;
  auto go = [&](auto kern, int waves, int rows) {
    p.row_blocks = (int)((a.q_len * p.G + rows - 1) / rows);
    const dim3 grid((unsigned)(a.batch * a.kv_heads * p.row_blocks));
    kern<<<grid, waves * 64, 0, stream>>>(p);
  };
  switch (a.dim) {
    case 64:
      if (shared) go(prefill_kernel<64, true, 8, 2>, 8, 256);
      else go(prefill_kernel<64, false, 8, 2>, 8, 256);
      break;
    case 128:
#if LBCA_PREFILL_V1
      {
        constexpr int W128 = LBCA_PREFILL_WAVES, Q128 = LBCA_PREFILL_QG;
        if (shared) go(prefill_kernel<128, true, W128, Q128>, W128, W128 * Q128 * 16);
        else go(prefill_kernel<128, false, W128, Q128>, W128, W128 * Q128 * 16);
      }
#else
      if (shared) go(prefill128_kernel<true>, 8, 256);
      else go(prefill128_kernel<false>, 8, 256);
#endif
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lbca
