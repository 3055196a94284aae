// Decode attention for wide shared-series rows: 512-dim entries read as both
// key and value by blocks of 32 query heads (HCA and CSA core attention).
//
// Method: "HCA: Heavily Compressed Attention (toy implementation)" and "CSA:
// Compressed Sparse Attention (toy implementation)", "What is implemented":
// multi-query attention in which every query head reads the same compressed
// entry as key and value, RMSNorm on queries and entries, RoPE on the last
// dims (entries at their block start, raw tokens at their position, queries at
// t, the output rotated back by -t), an attention sink in the denominator, and
// for CSA only the selected entries plus the sliding window.
//
// Work split: a range is (sequence, KV head, split), a contiguous run of
// 32-row tiles of the visible-row list (pooled or selected entries, then the
// raw span).  One workgroup works a range for HB 32-head blocks; with 64
// query heads the host either launches one 8-wave workgroup (HB = 2) or two
// 4-wave "twin" workgroups (HB = 1, one per head block) whose linear ids are
// 8 apart, so both land on the same XCD and the second read of a tile is an
// L2 hit.  A CU streams at most about 40 GB/s, so the host picks enough splits
// to spread the rows over most CUs, few enough that the split partials stay
// small.
//
// 4 x HB waves: wave (hb, q) owns head block hb and the 128-dim quarter q of
// the rows and of the output.  Tiles go straight from global memory to LDS
// (global_load_lds_dwordx4, four rows per instruction, 16-byte chunks
// swizzled per row so that both read patterns below are free of bank
// conflicts); the waves of a quarter copy its rows between them, a ring of
// three tiles keeps two tiles' copies in flight, and one barrier per tile
// publishes a landed tile (and frees the oldest slot for the next copy).
// Scores are computed transposed with v_mfma_f32_32x32x16_bf16, S^T[row,
// head] = K Q^T, each wave over its quarter of the dims; the four partials of
// a head block are summed through LDS in a fixed order, so its waves hold the
// same scores and softmax state.  In the 32x32 accumulator layout lane (n, g)
// holds head n and rows 8j + 4g + i, which is exactly the B operand P^T of
// O^T = V^T P^T for k = 16 rows when the rows of a 16-row block are taken in
// the order {4g..4g+3, 8+4g..8+4g+3}; the A operand V^T comes from two
// transposing LDS reads (ds_read_b64_tr_b16) in that same row order.
// Raw-window rows are normalised and rotated in LDS when they land (row sums
// of squares summed over the quarters); the queries are normalised and
// rotated in registers.  Reads of copied tiles are asm blocks that wait for
// themselves: the compiler cannot tell which ring slot a plain read touches
// and would wait for every copy in flight.
//
// The running max moves lazily (only when a score exceeds it by 2^8); with
// one split the workgroup finishes the heads (sink, normalisation, LSE, -t
// rotation), otherwise it writes its own normalised output in bf16 plus its
// (max, sum) in fp32 for decode_merge_kernel, in the 16-head-unit layout of
// the other decode path (half the bytes of an fp32 partial).
// No device-scope fence is used.
#include <type_traits>

#include "decode_common.h"

namespace lbca {

constexpr int kWideSel = 1024;  // selected ids staged per workgroup range

namespace {

constexpr int WD = 512;            // row dims
constexpr int WTR = 32;            // rows per tile
constexpr int WQ = 128;            // dims per wave
constexpr int WKST = WQ / 16;      // 16-dim k-steps of one wave's score MFMAs
constexpr int WDB = WQ / 32;       // 32-dim output blocks of one wave
constexpr int WQB = WTR * WQ * 2;  // bytes of one wave's quarter tile
constexpr int WSLOTS = 3;          // ring depth (tiles)

// 16-byte chunk swizzle of tile row r (16 chunks per quarter row; the LDS
// serves 16 chunks per cycle): 16 consecutive rows read at one chunk, and 4
// rows (from a multiple of 4) read at 4 chunks of an aligned group, fall on 16
// distinct bank groups.  Rows 16 apart share the swizzle.
__device__ __forceinline__ int wswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Workgroup barrier for LDS traffic between waves: this wave's LDS accesses
// complete, then s_barrier; the asm's memory clobber keeps the compiler from
// moving memory accesses across it.  Global-to-LDS copies still in flight are
// not waited for (a release fence would wait for them, since they write LDS);
// each wave waits for its own copies with vm_wait before reading them.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n s_barrier" ::: "memory");
}

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  // vmcnt is split over bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// The 8 score A operands of one quarter tile (row n, chunk (2ks + g) ^ swz(n)):
// one per-lane address per k-step.
__device__ __forceinline__ void wide_k_reads(uint4 (&r)[WKST], const uint32_t (&a)[WKST]) {
  asm volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %9\n"
      "ds_read_b128 %2, %10\n"
      "ds_read_b128 %3, %11\n"
      "ds_read_b128 %4, %12\n"
      "ds_read_b128 %5, %13\n"
      "ds_read_b128 %6, %14\n"
      "ds_read_b128 %7, %15\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// The P^T B operands of this lane for both 16-row blocks: the 8-byte words of
// the waves that finished rows j = 0..3 (512 bytes apart), pr[j]; and the A
// operands of O^T += V^T P^T for both 16-row blocks of a quarter tile
// and the wave's 4 output blocks: lane (i, mq, g) reads rows 16kb + 4g + i/4
// and 16kb + 8 + 4g + i/4 at dims 32*db + 16*mq + 4*(i%4); the transposing
// reads give lane (m, g) dims 32*db + m of rows {4g.., 8+4g..} of block kb.
// a[2*db + h]: address of (row r1 + 8h, block db) in block 0; block 1 is
// 4096 bytes on (same swizzle).  r[kb][2*db + h].  All reads in one block
// with one wait.
__device__ __forceinline__ void wide_ptr_reads(uint2 (&pr)[4], uint32_t pa, s16x4 (&r)[2][8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64 %0, %20\n"
      "ds_read_b64 %1, %20 offset:512\n"
      "ds_read_b64 %2, %20 offset:1024\n"
      "ds_read_b64 %3, %20 offset:1536\n"
      "ds_read_b64_tr_b16 %4, %21\n"
      "ds_read_b64_tr_b16 %5, %22\n"
      "ds_read_b64_tr_b16 %6, %23\n"
      "ds_read_b64_tr_b16 %7, %24\n"
      "ds_read_b64_tr_b16 %8, %25\n"
      "ds_read_b64_tr_b16 %9, %26\n"
      "ds_read_b64_tr_b16 %10, %27\n"
      "ds_read_b64_tr_b16 %11, %28\n"
      "ds_read_b64_tr_b16 %12, %21 offset:4096\n"
      "ds_read_b64_tr_b16 %13, %22 offset:4096\n"
      "ds_read_b64_tr_b16 %14, %23 offset:4096\n"
      "ds_read_b64_tr_b16 %15, %24 offset:4096\n"
      "ds_read_b64_tr_b16 %16, %25 offset:4096\n"
      "ds_read_b64_tr_b16 %17, %26 offset:4096\n"
      "ds_read_b64_tr_b16 %18, %27 offset:4096\n"
      "ds_read_b64_tr_b16 %19, %28 offset:4096\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(pr[0]), "=&v"(pr[1]), "=&v"(pr[2]), "=&v"(pr[3]),
        "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[0][2]), "=&v"(r[0][3]), "=&v"(r[0][4]), "=&v"(r[0][5]),
        "=&v"(r[0][6]), "=&v"(r[0][7]), "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[1][2]), "=&v"(r[1][3]),
        "=&v"(r[1][4]), "=&v"(r[1][5]), "=&v"(r[1][6]), "=&v"(r[1][7])
      : "v"(pa), "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// This lane's float4 j of the head block's four partials (4 KB apart): the
// rows 8j + 4g + i this wave finishes.
__device__ __forceinline__ void wide_x4_reads(float4 (&r)[4], uint32_t a) {
  asm volatile(
      "ds_read_b128 %0, %4\n"
      "ds_read_b128 %1, %4 offset:4096\n"
      "ds_read_b128 %2, %4 offset:8192\n"
      "ds_read_b128 %3, %4 offset:12288\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a)
      : "memory");
}

__device__ __forceinline__ void unpack8w(const uint4& u, float* f) {
  f[0] = lo_bf16(u.x); f[1] = hi_bf16(u.x); f[2] = lo_bf16(u.y); f[3] = hi_bf16(u.y);
  f[4] = lo_bf16(u.z); f[5] = hi_bf16(u.z); f[6] = lo_bf16(u.w); f[7] = hi_bf16(u.w);
}
__device__ __forceinline__ uint4 pack8w(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

}  // namespace

template <int HB, int RD, bool TREAT, bool SEL, bool DN>
__global__ __launch_bounds__(256 * HB) void decode_wide_kernel(DecodeParams p) {
  static_assert(HB == 1 || HB == 2, "one or two 32-head blocks");
  static_assert(RD == 0 || RD == 64 || RD == 128, "rotated dims");
  constexpr int NI = 8 / HB;  // copy instructions per wave per tile (four rows each)
  __shared__ __attribute__((aligned(16))) uint8_t ring[WSLOTS * 4 * WQB];  // [slot][quarter] 32 rows
  __shared__ __attribute__((aligned(16))) float xs[HB][4][16 * 64];      // partial scores per wave
  __shared__ float ts[4][WTR];                                           // raw rows: partial sums of squares
  __shared__ float tq[HB][4][32];                                        // queries: partial sums of squares
  __shared__ float s_mx[HB][4][32];                                      // row-slice maxima / sums per head
  __shared__ __attribute__((aligned(16))) uint2 s_p[HB][4][64];          // P (bf16) of rows 8j.. per lane
  __shared__ int s_ids[SEL ? kWideSel : 1];
  __shared__ double s_freq[RD > 0 ? RD / 2 : 1];

  preload_params(p);
  if constexpr (!DN) preload_strides(p);
  const DecStr ST = dec_strides<DN, WD>(p, p.qrows);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = wave & 3, hb = wave >> 2;  // dim quarter, head block
  const int n = lane & 31, g = lane >> 5;

  const int S = p.splits;
  // linear id -> (range, twin); twins of a range sit 8 ids apart (same XCD)
  unsigned u = blockIdx.x, tw = 0;
  if (p.wide_twins > 1) {
    const unsigned rest = blockIdx.x >> 3;
    tw = rest & 1u;
    u = (rest >> 1) * 8 + (blockIdx.x & 7);
  }
  if (u >= (unsigned)(p.units / p.head_groups) * (unsigned)S) return;  // padding of the XCD mapping
  const int split = (int)(u % (unsigned)S);
  const unsigned bk = u / (unsigned)S;
  const int64_t kvh = bk % (unsigned)p.hkv;
  const int64_t b = bk / (unsigned)p.hkv;
  const int hbg = (int)tw * HB + hb;            // head block of this wave within the KV head
  const int64_t head0 = kvh * p.G + 32 * hbg;  // first query head of this wave's block

  const EarlyI64 e_pos = load_early(p.pos + b);  // requested first, used after the first copies
  const EarlyI64 e_base = load_early(p.rpb ? p.rpb + b : p.pos + b);
  // query B operands (head n, dims 128q + 16ks + 8g ..); their addresses do
  // not depend on the position, so they load while it is on its way.  With a
  // selection they are requested before the tile range is worked out, else
  // after it (each order measured the faster for its path, by 0.1-0.4 us).
  uint4 qb[WKST];
  if constexpr (SEL) {
    const bf16_t* qrow = p.q + qrow_off(ST.q, p.qrows, b, head0 + n) + WQ * q + 8 * g;
#pragma unroll
    for (int ks = 0; ks < WKST; ++ks) qb[ks] = *reinterpret_cast<const uint4*>(qrow + 16 * ks);
  }
  // Tile range of this split from the buffer capacities (no position needed,
  // so the first copies go out before it arrives): list positions [0, cap_sel)
  // of pooled or selected entries, then [0, cap_raw) of the raw span.  Rows
  // outside the runtime list are masked.
  const int cap_sel = (int)(p.sel ? p.k_sel : p.entries);
  const int64_t raw_span = p.mode == 0 ? p.W + p.m - 1 : p.W;
  const int cap_raw = (int)(raw_span < p.raw_rows ? raw_span : p.raw_rows);
  const int tiles_p = (cap_sel + WTR - 1) / WTR;
  const int tiles_r = (cap_raw + WTR - 1) / WTR;
  const int tiles = tiles_p + tiles_r;
  int t0, t1;
  if (TREAT && !SEL && S < tiles) {
    // ranges split a cost in which a raw tile (treated in LDS) counts twice;
    // a range takes the tiles whose cost ends inside it
    const int cost = tiles + tiles_r, pc = (cost + S - 1) / S;
    const int c0 = split * pc < cost ? split * pc : cost, c1 = c0 + pc < cost ? c0 + pc : cost;
    t0 = c0 <= tiles_p ? c0 : tiles_p + (c0 - tiles_p) / 2;
    t1 = c1 <= tiles_p ? c1 : tiles_p + (c1 - tiles_p) / 2;
  } else {
    const int per = (tiles + S - 1) / S;
    t0 = split * per < tiles ? split * per : tiles;
    t1 = t0 + per < tiles ? t0 + per : tiles;
  }
  const int r0 = t0 * WTR;  // first list position of the range

  if constexpr (!SEL) {
    const bf16_t* qrow = p.q + qrow_off(ST.q, p.qrows, b, head0 + n) + WQ * q + 8 * g;
#pragma unroll
    for (int ks = 0; ks < WKST; ++ks) qb[ks] = *reinterpret_cast<const uint4*>(qrow + 16 * ks);
  }
  // Selected ids of this range (the host sizes ranges to fit), after the
  // queries: storing an id to the LDS waits for its load and so for the
  // queries too (loads complete in order), but the queries then stream while
  // the ids are on their way (requested first, they measured 17.1 against
  // 16.9 us per CSA call).
  if constexpr (SEL) {
    int nr = (t1 < tiles_p ? t1 : tiles_p) * WTR;
    nr = (nr < cap_sel ? nr : cap_sel) - r0;
    nr = nr < kWideSel ? nr : kWideSel;
    const int32_t* src = p.sel + b * p.k_sel + r0;
    for (int i = tid; i < nr; i += 256 * HB) s_ids[i] = src[i];
    lds_barrier();
  }
  SeqView sv;  // filled once the position arrives (after the first copies)

  // ---- tile copies: the waves of quarter q copy its 32 rows between them ----
  const int64_t cb = p.qrows > 1 ? (int64_t)((unsigned)b / (unsigned)p.qrows) : b;  // cache sequence
  const uintptr_t pk_slice = reinterpret_cast<uintptr_t>(p.pk + cb * ST.pk.s0 + kvh * ST.pk.s1);
  const uintptr_t rk_slice = reinterpret_cast<uintptr_t>(p.rk + cb * ST.rk.s0 + kvh * ST.rk.s1);
  const uint32_t pks = 2u * (uint32_t)ST.pk.s2, rks = 2u * (uint32_t)ST.rk.s2;  // row strides, bytes
  const uintptr_t dummy = reinterpret_cast<uintptr_t>(p.q + qrow_off(ST.q, p.qrows, b, kvh * p.G));  // 1 KB, cached
  const int rq = lane >> 4, c_lane = lane & 15;  // row within 4 and LDS chunk this lane writes
  // Row v of the tile's part of the list -> (valid, buffer row).
  auto locate = [&](bool raw, int v, int64_t& row) __attribute__((always_inline)) -> bool {
    if (raw) {
      row = sv.raw_row0 + v;
      return v < sv.n_raw;
    }
    bool ok = v < sv.n_sel;
    int id = v;
    if constexpr (SEL) {
      const int li = v - r0;
      id = s_ids[ok ? (li < kWideSel ? li : kWideSel - 1) : 0];
      ok = ok && id >= 0 && id < sv.n_pooled;
    }
    row = id;
    return ok;
  };
  // Whether every row of the tile is in the list and its rows are consecutive.
  auto tile_full = [&](bool raw, int v0) __attribute__((always_inline)) {
    return raw ? v0 + WTR <= sv.n_raw : (!SEL && v0 + WTR <= sv.n_sel);
  };
  // byte offset of this lane's copy j (row 4(hb*NI + j) + rq) within its row,
  // plus (dense rows) the row's offset within a run of rows
  uint32_t lane_off[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int r = 4 * (hb * NI + j) + rq;
    lane_off[j] = (DN ? (uint32_t)(r * WD * 2) : 0u) + (uint32_t)(WQ * 2 * q) + 16u * (uint32_t)(c_lane ^ wswz(r));
  }
  // a run's row offset of copy j for row stride rs (strided rows)
  auto run_off = [&](int j, uint32_t rs) __attribute__((always_inline)) -> uint64_t {
    return DN ? 0 : (uint64_t)(uint32_t)(4 * (hb * NI + j) + rq) * rs;
  };
  // Issues this wave's NI copies of `tile` into ring slot `slot`.
  auto issue = [&](int tile, int slot) __attribute__((always_inline)) {
    const bool raw = tile >= tiles_p;
    const int v0 = raw ? (tile - tiles_p) * WTR : tile * WTR;
    const uintptr_t sb = raw ? rk_slice : pk_slice;
    const uint32_t rs = raw ? rks : pks;
    uint8_t* dst0 = ring + slot * (4 * WQB) + q * WQB + hb * NI * 1024;
    if (tile_full(raw, v0)) {  // consecutive rows, all in the list
      const uintptr_t base = sb + (uint64_t)(raw ? sv.raw_row0 + v0 : (int64_t)v0) * rs;
#pragma unroll
      for (int j = 0; j < NI; ++j)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<gbl_void*>(base + run_off(j, rs) + lane_off[j]),
                                         (lds_void*)(dst0 + j * 1024), 16, 0, 0);
      return;
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = 4 * (hb * NI + j) + rq;
      int64_t row;
      const bool ok = locate(raw, v0 + r, row);
      const uint32_t coff = (uint32_t)(WQ * 2 * q) + 16u * (uint32_t)(c_lane ^ wswz(r));
      const uintptr_t ga = (ok ? sb + (uint64_t)row * rs : dummy) + coff;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<gbl_void*>(ga), (lds_void*)(dst0 + j * 1024), 16, 0, 0);
    }
  };
  // Copies of a pooled or selected tile before the position is known: rows
  // within the buffer capacities (the list bounds are applied by the mask).
  auto issue_early = [&](int tile, int slot) __attribute__((always_inline)) {
    const int v0 = tile * WTR;
    uint8_t* dst0 = ring + slot * (4 * WQB) + q * WQB + hb * NI * 1024;
    if (!SEL && v0 + WTR <= cap_sel) {
      const uintptr_t base = pk_slice + (uint64_t)v0 * pks;
#pragma unroll
      for (int j = 0; j < NI; ++j)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<gbl_void*>(base + run_off(j, pks) + lane_off[j]),
                                         (lds_void*)(dst0 + j * 1024), 16, 0, 0);
      return;
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = 4 * (hb * NI + j) + rq;
      const int v = v0 + r;
      bool ok = v < cap_sel;
      int id = v;
      if constexpr (SEL) {
        const int li = v - r0;
        id = s_ids[ok ? (li < kWideSel ? li : kWideSel - 1) : 0];
        ok = ok && id >= 0 && id < p.entries;
      }
      const uint32_t coff = (uint32_t)(WQ * 2 * q) + 16u * (uint32_t)(c_lane ^ wswz(r));
      const uintptr_t ga = (ok ? pk_slice + (uint64_t)id * pks : dummy) + coff;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<gbl_void*>(ga), (lds_void*)(dst0 + j * 1024), 16, 0, 0);
    }
  };
  // the first two tiles: pooled ones now, raw ones once the position is known
  // (raw tiles come last, so the copies stay in tile order)
  if (t0 < t1 && t0 < tiles_p) issue_early(t0, 0);
  if (t0 + 1 < t1 && t0 + 1 < tiles_p) issue_early(t0 + 1, 1);
  if constexpr (RD > 0) {  // RoPE turns per position (published by the barrier below)
    if (tid < RD / 2) s_freq[tid] = rope_turns_per_pos(tid, RD, p.log2_base);
  }
  sv = seq_view(p, b, uniform_value(e_pos), p.rpb ? uniform_value(e_base) : 0);
  if (!sv.ok) {  // rows do not fit the buffers: NaN, written once
    vm_wait<0>();
    if (split == 0) {
      const int64_t h0 = kvh * p.G + 32 * HB * (int)tw;
      for (int i = tid; i < 32 * HB * WD; i += 256 * HB)
        p.out[qrow_off(ST.o, p.qrows, b, h0 + i / WD) + i % WD] = __builtin_nanf("");
      if (p.lse && tid < 32 * HB) p.lse[b * p.hq + h0 + tid] = __builtin_nanf("");
    }
    return;
  }
  if (t0 < t1 && t0 >= tiles_p) issue(t0, 0);
  if (t0 + 1 < t1 && t0 + 1 >= tiles_p) issue(t0 + 1, 1);

  // ---- query treatment in registers: RMSNorm over all 512 dims, RoPE on the last RD ----
  if constexpr (RD > 0) lds_barrier();  // s_freq
  if constexpr (TREAT) {
    float inv = 1.f;
    if (p.eps >= 0.f) {
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < WKST; ++ks) {
        float f[8];
        unpack8w(qb[ks], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
      }
      ss = xor32_sum(ss);
      if (g == 0) tq[hb][q][n] = ss;
      lds_barrier();
      inv = 1.f / sqrtf((((tq[hb][0][n] + tq[hb][1][n]) + tq[hb][2][n]) + tq[hb][3][n]) / (float)WD + p.eps);
    }
    constexpr int K0 = (WQ - RD) / 16, SHK = RD / 32;  // first rotated k-step; partner k-steps on
#pragma unroll
    for (int ks = 0; ks < WKST; ++ks) {
      const bool rot = RD > 0 && q == 3 && ks >= K0;
      if (rot && ks >= K0 + SHK) continue;  // written with its partner
      float f[8];
      unpack8w(qb[ks], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= inv;
      if (rot) {
        float h[8];
        unpack8w(qb[ks + SHK], h);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          h[e] *= inv;
          const int k = 16 * (ks - K0) + 8 * g + e;
          float cs, sn;
          rope_cos_sin_turns((double)sv.t * s_freq[k], &cs, &sn);
          const float x1 = f[e], x2 = h[e];
          f[e] = x1 * cs - x2 * sn;
          h[e] = x2 * cs + x1 * sn;
        }
        qb[ks + SHK] = pack8w(h);
      }
      qb[ks] = pack8w(f);
    }
  }

  // per-lane LDS byte offsets within a quarter tile.  Score A operands: row n,
  // chunk (2ks + g) ^ swz(n).
  uint32_t koff[WKST];
#pragma unroll
  for (int ks = 0; ks < WKST; ++ks) koff[ks] = (uint32_t)(n * WQ * 2 + 16 * ((2 * ks + g) ^ wswz(n)));
  // Transposing reads of rows r1 = 4g + i/4 and r1 + 8, chunk 4db + 2mq + (i%4)/2
  // (swizzled), 8-byte half i%2.
  uint32_t toff[8];
  {
    const int i = lane & 15, mq = (lane >> 4) & 1;
    const int r1 = 4 * g + (i >> 2), cl = 2 * mq + ((i & 3) >> 1);
#pragma unroll
    for (int db = 0; db < WDB; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = r1 + 8 * h;
        toff[2 * db + h] = (uint32_t)(r * WQ * 2 + 16 * ((4 * db + cl) ^ wswz(r)) + 8 * (i & 1));
      }
  }
  const uint32_t ring_a = (uint32_t)(uintptr_t)(lds_u8*)(ring) + (uint32_t)(q * WQB);
  // this wave finishes rows 8q + 4g + i of its head block: its float4 of each partial
  const uint32_t xs_a = (uint32_t)(uintptr_t)(lds_u8*)(reinterpret_cast<uint8_t*>(&xs[hb][0][0])) + 16u * (q * 64 + lane);
  const uint32_t p_a = (uint32_t)(uintptr_t)(lds_u8*)(reinterpret_cast<uint8_t*>(&s_p[hb][0][0])) + 8u * lane;

  float m_run = kNegInf, l_run = 0.f;  // running max (this head block) and row-slice sum
  float m_oth = kNegInf;                // running max of the other head block (for the decision)
  f32x16 acc[WDB];
#pragma unroll
  for (int db = 0; db < WDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;

  // Software-pipelined tile loop.  Step `tile` reads from LDS and issues the
  // score MFMAs of tile + 1, then the P.V MFMAs of tile, and writes tile + 1's
  // partial scores; while the P.V MFMAs run: barrier A (the partials are
  // visible, and every wave is past its reads of tile's ring slot, which then
  // receives the copy of tile + 3), the softmax of tile + 1 (the four partials
  // of its rows summed in a fixed order, P against the running max, P and the
  // row-slice maxima to LDS), the wait for this wave's copies of tile + 2,
  // barrier C (P visible, tile + 2 landed) and the rescale decision.  When a
  // head's tile max exceeds its running max by more than 2^8 (the first tile,
  // and rarely after), every wave rescales, recomputes P and adds a barrier.
  // One buffer each for the partial scores, P and the maxima suffices: every
  // write of them follows a barrier that follows every wave's last read of the
  // previous contents.
  if (t0 < t1) {
    if (t0 + 1 < t1) vm_wait<NI>();
    else vm_wait<0>();
  }
  lds_barrier();  // the first tile landed

  // Raw rows of `tile` (ring slot sl): RMSNorm over all 512 dims, RoPE on the
  // last RD, in LDS, by head block 0's waves.  Every wave calls it (barriers).
  auto treat_raw = [&](int tile, int sl) __attribute__((always_inline)) {
    if constexpr (TREAT) {
      if (tile >= tiles_p) {
        // lane (n, g): row n, chunks c = g, g+2, ..., g+14 of quarter q (a
        // rotate-half partner chunk is RD/16 chunks on: same parity, same lane)
        uint8_t* rowp = ring + sl * (4 * WQB) + q * WQB + n * (WQ * 2);
        if (hb == 0 && p.eps >= 0.f) {
          float ss = 0.f;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            float f[8];
            unpack8w(*reinterpret_cast<const uint4*>(rowp + 16 * ((2 * u + g) ^ wswz(n))), f);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
          }
          ss = xor32_sum(ss);
          if (g == 0) ts[q][n] = ss;
        }
        lds_barrier();
        if (hb == 0) {
          float inv = 1.f;
          if (p.eps >= 0.f) inv = 1.f / sqrtf((((ts[0][n] + ts[1][n]) + ts[2][n]) + ts[3][n]) / (float)WD + p.eps);
          const double pos = (double)(sv.raw_begin + (tile - tiles_p) * WTR + n);
          constexpr int RC0 = (WQ - RD) / 8;  // first rotated chunk of the last quarter
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int c = 2 * u + g;
            const bool rot = RD > 0 && q == 3 && c >= RC0;
            const bool rot_lo = rot && c < RC0 + RD / 16;
            if (rot && !rot_lo) continue;  // written with its partner
            uint8_t* ap = rowp + 16 * (c ^ wswz(n));
            float f[8];
            unpack8w(*reinterpret_cast<const uint4*>(ap), f);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] *= inv;
            if (rot_lo) {
              uint8_t* bp = rowp + 16 * ((c + RD / 16) ^ wswz(n));
              float h[8];
              unpack8w(*reinterpret_cast<const uint4*>(bp), h);
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                h[e] *= inv;
                const int k = 8 * (c - RC0) + e;
                float cs, sn;
                rope_cos_sin_turns(pos * s_freq[k], &cs, &sn);
                const float x1 = f[e], x2 = h[e];
                f[e] = x1 * cs - x2 * sn;
                h[e] = x2 * cs + x1 * sn;
              }
              *reinterpret_cast<uint4*>(bp) = pack8w(h);
            }
            *reinterpret_cast<uint4*>(ap) = pack8w(f);
          }
        }
        lds_barrier();  // treated rows visible to every wave
      }
    }
  };
  // Score MFMAs of the quarter tile at LDS address sa, two independent chains.
  auto qk_issue = [&](uint32_t sa, f32x16& c0, f32x16& c1) __attribute__((always_inline)) {
    uint4 ka[WKST];
    uint32_t kad[WKST];
#pragma unroll
    for (int ks = 0; ks < WKST; ++ks) kad[ks] = sa + koff[ks];
    wide_k_reads(ka, kad);
#pragma unroll
    for (int e = 0; e < 16; ++e) c0[e] = c1[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < WKST; ks += 2) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[ks]),
                                                   __builtin_bit_cast(bf16x8, qb[ks]), c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[ks + 1]),
                                                   __builtin_bit_cast(bf16x8, qb[ks + 1]), c1, 0, 0, 0);
    }
  };
  // O^T += V^T P^T for the quarter tile at sa, two 16-row blocks: P^T of block
  // kb is this lane's P of rows j = 2kb, 2kb + 1 (from the waves that finished them).
  auto pv = [&](uint32_t sa) __attribute__((always_inline)) {
    uint2 pr[4];
    s16x4 va[2][8];
    uint32_t ta[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) ta[k] = sa + toff[k];
    wide_ptr_reads(pr, p_a, va, ta);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pr[2 * kb].x, pr[2 * kb].y, pr[2 * kb + 1].x, pr[2 * kb + 1].y));
#pragma unroll
      for (int db = 0; db < WDB; ++db) {
        const s16x4 a0 = va[kb][2 * db], a1 = va[kb][2 * db + 1];
        const bf16x8 a = __builtin_bit_cast(bf16x8, s16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[db], 0, 0, 0);
      }
    }
  };
  auto write_xs = [&](const f32x16& c0, const f32x16& c1) __attribute__((always_inline)) {
    float* xw = xs[hb][q];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(&xw[(j * 64 + lane) * 4]) =
          make_float4(c0[4 * j] + c1[4 * j], c0[4 * j + 1] + c1[4 * j + 1], c0[4 * j + 2] + c1[4 * j + 2],
                      c0[4 * j + 3] + c1[4 * j + 3]);
  };
  // Rows 8q + 4g + i (i < 4) of `tile`: the four partials summed in a fixed
  // order, masked, scaled into the exponent's units; P against the running
  // max to LDS, and this wave's row-slice max for the decision.
  auto softmax = [&](int tile, float (&s4)[4], float (&pj)[4]) __attribute__((always_inline)) {
    const bool raw = tile >= tiles_p;
    const int v0 = raw ? (tile - tiles_p) * WTR : tile * WTR;
    uint32_t mk = 0xffffffffu;  // valid rows of the tile (lane n: row n)
    if (!tile_full(raw, v0)) {
      int64_t row;
      const bool ok = locate(raw, v0 + n, row);
      mk = (uint32_t)(__ballot(ok) & 0xffffffffull);
    }
    {
      float4 xr[4];
      wide_x4_reads(xr, xs_a);
      float4 t = xr[0];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        t.x += xr[w].x; t.y += xr[w].y; t.z += xr[w].z; t.w += xr[w].w;
      }
      s4[0] = t.x * p.scale_log2; s4[1] = t.y * p.scale_log2;
      s4[2] = t.z * p.scale_log2; s4[3] = t.w * p.scale_log2;
    }
    if (mk != 0xffffffffu) {  // a tile with rows outside the list
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (!((mk >> (8 * q + 4 * g + e)) & 1u)) s4[e] = kNegInf;
    }
    const float mu = m_run == kNegInf ? 0.f : m_run;
#pragma unroll
    for (int e = 0; e < 4; ++e) pj[e] = fast_exp2(s4[e] - mu);
    s_p[hb][q][lane] = make_uint2(pack_bf16x2(pj[0], pj[1]), pack_bf16x2(pj[2], pj[3]));
    const float lm = xor32_max(fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3])));
    if (g == 0) s_mx[hb][q][n] = lm;
  };
  // After barrier C: the tile max of head n in both head blocks (every wave
  // tracks both running maxima, so the decision is the same in all waves).
  auto decide = [&](const float (&s4)[4], float (&pj)[4]) __attribute__((always_inline)) {
    const float tm = fmaxf(fmaxf(s_mx[hb][0][n], s_mx[hb][1][n]), fmaxf(s_mx[hb][2][n], s_mx[hb][3][n]));
    float tm_o = kNegInf;
    if constexpr (HB > 1)
      tm_o = fmaxf(fmaxf(s_mx[hb ^ 1][0][n], s_mx[hb ^ 1][1][n]), fmaxf(s_mx[hb ^ 1][2][n], s_mx[hb ^ 1][3][n]));
    if (__ballot(tm > m_run + 8.f || tm_o > m_oth + 8.f)) {  // rescale to the tile max, recompute P
      const float nm = fmaxf(m_run, tm);
      const float corr = nm == kNegInf ? 1.f : fast_exp2(m_run - nm);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < WDB; ++db) acc[db] *= corr;
      m_run = nm;
      m_oth = fmaxf(m_oth, tm_o);
      const float mu = m_run == kNegInf ? 0.f : m_run;
#pragma unroll
      for (int e = 0; e < 4; ++e) pj[e] = fast_exp2(s4[e] - mu);
      s_p[hb][q][lane] = make_uint2(pack_bf16x2(pj[0], pj[1]), pack_bf16x2(pj[2], pj[3]));
      lds_barrier();  // nobody has read the first P yet
    }
    l_run += (pj[0] + pj[1]) + (pj[2] + pj[3]);
  };

  const auto slot_addr = [&](int sl) { return ring_a + (uint32_t)(sl * 4 * WQB); };  // this wave's quarter
  float s4[4], pj[4];
  if (t0 < t1) {  // prologue: scores and P of the first tile
    treat_raw(t0, 0);
    f32x16 c0, c1;
    qk_issue(slot_addr(0), c0, c1);
    write_xs(c0, c1);
    lds_barrier();  // A
    if (t0 + 2 < t1) issue(t0 + 2, 2);
    softmax(t0, s4, pj);
    if (t0 + 1 < t1) {  // this wave's copies of t0 + 1 landed
      if (t0 + 2 < t1) vm_wait<NI>();
      else vm_wait<0>();
    }
    lds_barrier();  // C
    decide(s4, pj);
  }
  int slot = 0;  // ring slot of `tile`
#pragma unroll 1
  for (int tile = t0; tile < t1; ++tile) {
    const int nslot = slot == WSLOTS - 1 ? 0 : slot + 1;
    const bool more = tile + 1 < t1;
    f32x16 c0, c1;
    if (more) {
      treat_raw(tile + 1, nslot);
      qk_issue(slot_addr(nslot), c0, c1);
    }
    pv(slot_addr(slot));
    if (more) {
      write_xs(c0, c1);
      lds_barrier();  // A
      if (tile + 3 < t1) issue(tile + 3, slot);
      softmax(tile + 1, s4, pj);
      if (tile + 2 < t1) {  // this wave's copies of tile + 2 landed
        if (tile + 3 < t1) vm_wait<NI>();
        else vm_wait<0>();
      }
      lds_barrier();  // C
      decide(s4, pj);
    }
    slot = nslot;
  }
  const float M = m_run;
  float L;
  {  // the row sums of the four slices (same scale in every wave), fixed order
    const float lw = xor32_sum(l_run);
    lds_barrier();  // every wave is past its last read of s_mx
    if (g == 0) s_mx[hb][q][n] = lw;
    lds_barrier();
    L = ((s_mx[hb][0][n] + s_mx[hb][1][n]) + s_mx[hb][2][n]) + s_mx[hb][3][n];
  }

  const int64_t head = head0 + n;
  if (S == 1) {
    if (p.sink) L += exp2f(p.sink[head] * kLog2e - M);
    const float inv = 1.f / L;
#pragma unroll
    for (int db = 0; db < WDB; ++db) acc[db] *= inv;
    if constexpr (RD > 0) {
      if (q == 3) {  // -t rotation of the last RD dims: blocks db and db + RD/64
        constexpr int B0 = WDB - RD / 32, SH = RD / 64;
#pragma unroll
        for (int db = B0; db < B0 + SH; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int k = 32 * (db - B0) + 8 * (e >> 2) + 4 * g + (e & 3);
            float cs, sn;
            rope_cos_sin_turns(-(double)sv.t * s_freq[k], &cs, &sn);
            const float x1 = acc[db][e], x2 = acc[db + SH][e];
            acc[db][e] = x1 * cs - x2 * sn;
            acc[db + SH][e] = x2 * cs + x1 * sn;
          }
      }
    }
    float* o = p.out + qrow_off(ST.o, p.qrows, b, head) + WQ * q + 4 * g;
#pragma unroll
    for (int db = 0; db < WDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(o + 32 * db + 8 * j) =
            make_float4(acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2], acc[db][4 * j + 3]);
    if (p.lse && q == 0 && g == 0) p.lse[b * p.hq + head] = (M + log2f(L)) * 0.69314718055994531f;
    return;
  }
  // split partial in the 16-head-unit layout: unit (b, kvh, 16-head group), part = unit * S + split;
  // this split's own normalised output in bf16 (zero where no row of the range is visible)
  const int64_t unit = (b * p.hkv + kvh) * p.head_groups + 2 * hbg + (n >> 4);
  const int64_t part = unit * S + split;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  bf16_t* o = p.ws_o + (part * 16 + (n & 15)) * WD + WQ * q + 4 * g;
#pragma unroll
  for (int db = 0; db < WDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint2*>(o + 32 * db + 8 * j) =
          make_uint2(pack_bf16x2(acc[db][4 * j] * inv, acc[db][4 * j + 1] * inv),
                     pack_bf16x2(acc[db][4 * j + 2] * inv, acc[db][4 * j + 3] * inv));
  if (q == 0 && g == 0) {
    p.ws_ml[(part * 16 + (n & 15)) * 2] = M;
    p.ws_ml[(part * 16 + (n & 15)) * 2 + 1] = L;
  }
}

hipError_t launch_decode_wide(const DecodeParams& p, int rope_dims, bool treat, int head_blocks, bool dn,
                              hipStream_t stream) {
  const unsigned pairs = (unsigned)(p.units / p.head_groups) * (unsigned)p.splits;  // (sequence, KV head, split)
  const dim3 grid(p.wide_twins > 1 ? (pairs + 7) / 8 * 8 * (unsigned)p.wide_twins : pairs);
  const bool sel = p.sel != nullptr;
  auto go = [&](auto kern, int hb) {
    kern<<<grid, 256 * hb, 0, stream>>>(p);
    return hipGetLastError();
  };
  auto pick = [&](auto hbc, auto dnc) -> hipError_t {
    constexpr int HB = decltype(hbc)::value;
    constexpr bool DN = decltype(dnc)::value;
    if (!treat)
      return sel ? go(decode_wide_kernel<HB, 0, false, true, DN>, HB) : go(decode_wide_kernel<HB, 0, false, false, DN>, HB);
    switch (rope_dims) {
      case 0:
        return sel ? go(decode_wide_kernel<HB, 0, true, true, DN>, HB) : go(decode_wide_kernel<HB, 0, true, false, DN>, HB);
      case 64:
        return sel ? go(decode_wide_kernel<HB, 64, true, true, DN>, HB) : go(decode_wide_kernel<HB, 64, true, false, DN>, HB);
      case 128:
        return sel ? go(decode_wide_kernel<HB, 128, true, true, DN>, HB)
                   : go(decode_wide_kernel<HB, 128, true, false, DN>, HB);
      default: return hipErrorInvalidValue;
    }
  };
  using T = std::true_type;
  using F = std::false_type;
  if (head_blocks == 2) return dn ? pick(std::integral_constant<int, 2>{}, T{}) : pick(std::integral_constant<int, 2>{}, F{});
  if (head_blocks == 1) return dn ? pick(std::integral_constant<int, 1>{}, T{}) : pick(std::integral_constant<int, 1>{}, F{});
  return hipErrorInvalidValue;
}

}  // namespace lbca
