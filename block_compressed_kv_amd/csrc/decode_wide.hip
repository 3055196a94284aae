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
// Work split: a workgroup owns (sequence, KV head, split), a contiguous range
// of 32-row tiles of the visible-row list (pooled or selected entries, then
// the raw span), for all query heads of the KV head (one or two blocks of 32):
// each tile crosses from memory to a CU once.  A CU streams at most about
// 40 GB/s, so the host picks enough splits to spread the rows over most CUs,
// few enough that the split partials stay small.
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
// rotation), otherwise it writes its unnormalised partial for
// decode_merge_kernel in the 16-head-unit layout of the other decode path.
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

// 16-byte chunk swizzle of tile row r (16 chunks per quarter row): 8
// consecutive rows at one chunk, and 4 rows (from a multiple of 4) at two
// adjacent chunks (even first), fall on distinct bank groups.  Rows 16 apart
// differ by 4.
__device__ __forceinline__ int wswz(int r) { return (2 * r + (r >> 2)) & 7; }

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

// The 8 score A operands of one quarter tile (row n, chunk (2ks + g) ^ swz(n)
// = 8*(ks/4) + ((2*(ks%4) + g) ^ swz(n))): four per-lane addresses, the
// k-steps 4..7 128 bytes further.
__device__ __forceinline__ void wide_k_reads(uint4 (&r)[WKST], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %9\n"
      "ds_read_b128 %2, %10\n"
      "ds_read_b128 %3, %11\n"
      "ds_read_b128 %4, %8 offset:128\n"
      "ds_read_b128 %5, %9 offset:128\n"
      "ds_read_b128 %6, %10 offset:128\n"
      "ds_read_b128 %7, %11 offset:128\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

// The A operands of O^T += V^T P^T for one 16-row block of a quarter tile and
// the wave's 4 output blocks: lane (i, mq, g) reads rows rb + 4g + i/4 and
// rb + 8 + 4g + i/4 at dims 32*db + 16*mq + 4*(i%4); the transposing reads
// give lane (m, g) dims 32*db + m of rows {rb+4g.., rb+8+4g..}.  The swizzled
// chunk of block db is 8*(db/2) + (chunk of db%2), so four per-lane addresses
// (two rows x db parity) and an immediate offset cover the 8 reads.
// a: (row 1, even db), (row 1, odd db), (row 2, even db), (row 2, odd db).
__device__ __forceinline__ void wide_tr_reads(s16x4 (&r)[8], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n"
      "ds_read_b64_tr_b16 %1, %10\n"
      "ds_read_b64_tr_b16 %2, %9\n"
      "ds_read_b64_tr_b16 %3, %11\n"
      "ds_read_b64_tr_b16 %4, %8 offset:128\n"
      "ds_read_b64_tr_b16 %5, %10 offset:128\n"
      "ds_read_b64_tr_b16 %6, %9 offset:128\n"
      "ds_read_b64_tr_b16 %7, %11 offset:128\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

// Two 16-byte rows of every wave's partial scores (float4 j0 and j0+1 of
// this lane; the waves' partials are 4 KB apart).  An asm block like the tile
// reads: a plain read would make the compiler wait for the copies in flight.
__device__ __forceinline__ void wide_x_reads(float4 (&r)[8], uint32_t a) {
  asm volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %8 offset:4096\n"
      "ds_read_b128 %2, %8 offset:8192\n"
      "ds_read_b128 %3, %8 offset:12288\n"
      "ds_read_b128 %4, %8 offset:1024\n"
      "ds_read_b128 %5, %8 offset:5120\n"
      "ds_read_b128 %6, %8 offset:9216\n"
      "ds_read_b128 %7, %8 offset:13312\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7])
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

template <int HB, int RD, bool TREAT, bool SEL>
__global__ __launch_bounds__(256 * HB) void decode_wide_kernel(DecodeParams p) {
  static_assert(HB == 1 || HB == 2, "one or two 32-head blocks");
  static_assert(RD == 0 || RD == 64 || RD == 128, "rotated dims");
  constexpr int NI = 8 / HB;  // copy instructions per wave per tile (four rows each)
  __shared__ __attribute__((aligned(16))) uint8_t ring[WSLOTS * 4 * WQB];  // [slot][quarter] 32 rows
  __shared__ __attribute__((aligned(16))) float xs[HB][4][16 * 64];      // partial scores per wave
  __shared__ float ts[4][WTR];                                           // raw rows: partial sums of squares
  __shared__ float tq[HB][4][32];                                        // queries: partial sums of squares
  __shared__ int s_ids[SEL ? kWideSel : 1];
  __shared__ double s_freq[RD > 0 ? RD / 2 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = wave & 3, hb = wave >> 2;  // dim quarter, head block
  const int n = lane & 31, g = lane >> 5;

  const int S = p.splits;
  const int split = (int)(blockIdx.x % (unsigned)S);
  const unsigned bk = blockIdx.x / (unsigned)S;
  const int64_t kvh = bk % (unsigned)p.hkv;
  const int64_t b = bk / (unsigned)p.hkv;
  const int64_t head0 = kvh * p.G + 32 * hb;  // first query head of this wave's block

  // query B operands (head n, dims 128q + 16ks + 8g ..); their addresses do
  // not depend on the position, so they load alongside it
  uint4 qb[WKST];
  {
    const bf16_t* qrow = p.q + (b * p.hq + head0 + n) * WD + WQ * q + 8 * g;
#pragma unroll
    for (int ks = 0; ks < WKST; ++ks) qb[ks] = *reinterpret_cast<const uint4*>(qrow + 16 * ks);
  }
  const SeqView sv = seq_view(p, b);
  if (!sv.ok) {  // rows do not fit the buffers: NaN, written once
    if (split == 0) {
      const int64_t h0 = kvh * p.G;
      for (int i = tid; i < 32 * HB * WD; i += 256 * HB) p.out[(b * p.hq + h0) * WD + i] = __builtin_nanf("");
      if (p.lse && tid < 32 * HB) p.lse[b * p.hq + h0 + tid] = __builtin_nanf("");
    }
    return;
  }

  const int tiles_p = (sv.n_sel + WTR - 1) / WTR;
  const int tiles = tiles_p + (sv.n_raw + WTR - 1) / WTR;
  const int per = (tiles + S - 1) / S;
  const int t0 = split * per < tiles ? split * per : tiles;
  const int t1 = t0 + per < tiles ? t0 + per : tiles;
  const int r0 = t0 * WTR;  // first list position of the range

  if constexpr (SEL) {  // selected ids of this range (the host sizes ranges to fit)
    int nr = (t1 < tiles_p ? t1 : tiles_p) * WTR;
    nr = (nr < sv.n_sel ? nr : sv.n_sel) - r0;
    nr = nr < kWideSel ? nr : kWideSel;
    const int32_t* src = p.sel + b * p.k_sel + r0;
    for (int i = tid; i < nr; i += 256 * HB) s_ids[i] = src[i];
  }
  if constexpr (RD > 0) {
    if (tid < RD / 2) s_freq[tid] = rope_turns_per_pos(tid, RD, p.log2_base);
  }
  if constexpr (SEL || RD > 0) lds_barrier();

  // ---- tile copies: the waves of quarter q copy its 32 rows between them ----
  const uintptr_t pk_slice = reinterpret_cast<uintptr_t>(p.pk) + (uint64_t)((b * p.hkv + kvh) * p.entries) * (WD * 2);
  const uintptr_t rk_slice = reinterpret_cast<uintptr_t>(p.rk) + (uint64_t)((b * p.hkv + kvh) * p.raw_rows) * (WD * 2);
  const uintptr_t dummy = reinterpret_cast<uintptr_t>(p.q + (b * p.hq + kvh * p.G) * WD);  // 1 KB, cached
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
  // Issues this wave's NI copies of `tile` into ring slot `slot`.
  auto issue = [&](int tile, int slot) __attribute__((always_inline)) {
    const bool raw = tile >= tiles_p;
    const int v0 = raw ? (tile - tiles_p) * WTR : tile * WTR;
    const uintptr_t sb = raw ? rk_slice : pk_slice;
    uint8_t* dst0 = ring + slot * (4 * WQB) + q * WQB + hb * NI * 1024;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = 4 * (hb * NI + j) + rq;
      int64_t row;
      const bool ok = locate(raw, v0 + r, row);
      const uint32_t coff = (uint32_t)(WQ * 2 * q) + 16u * (uint32_t)(c_lane ^ wswz(r));
      const uintptr_t ga = (ok ? sb + (uint64_t)row * (WD * 2) : dummy) + coff;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<gbl_void*>(ga), (lds_void*)(dst0 + j * 1024), 16, 0, 0);
    }
  };
  if (t0 < t1) issue(t0, 0);
  if (t0 + 1 < t1) issue(t0 + 1, 1);

  // ---- query treatment in registers: RMSNorm over all 512 dims, RoPE on the last RD ----
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
  // chunk 8*(ks/4) + ((2*(ks%4) + g) ^ swz(n)).
  uint32_t koff[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) koff[k] = (uint32_t)(n * WQ * 2 + 16 * ((2 * k + g) ^ wswz(n)));
  // Transposing reads of rows r1 = 4g + i/4 and r1 + 8 (block 0); block 1 is
  // 16 rows on, whose swizzle differs by 4, i.e. the db parities swap.
  uint32_t toff[4];
  {
    const int i = lane & 15, mq = (lane >> 4) & 1;
    const int r1 = 4 * g + (i >> 2), cl = 2 * mq + ((i & 3) >> 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = r1 + 8 * (k >> 1), par = k & 1;
      toff[k] = (uint32_t)(r * WQ * 2 + 16 * ((4 * par + cl) ^ wswz(r)) + 8 * (i & 1));
    }
  }
  const uint32_t ring_a = (uint32_t)(uintptr_t)(lds_u8*)(ring) + (uint32_t)(q * WQB);
  const uint32_t xs_a = (uint32_t)(uintptr_t)(lds_u8*)(reinterpret_cast<uint8_t*>(&xs[hb][0][0])) + 16u * lane;

  float m_run = kNegInf, l_run = 0.f;
  f32x16 acc[WDB];
#pragma unroll
  for (int db = 0; db < WDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;

  int slot = 0;
#pragma unroll 1
  for (int tile = t0; tile < t1; ++tile) {
    // this wave's copies of the tile landed (the next tile's may stay in flight) ...
    if (tile + 1 < t1) vm_wait<NI>();
    else vm_wait<0>();
    // ... and every wave's: the tile is complete, the previous tile's slot and
    // the partial-score buffers are free
    lds_barrier();
    if (tile + 2 < t1) issue(tile + 2, slot == 0 ? 2 : slot - 1);
    const uint32_t sa = ring_a + (uint32_t)(slot * 4 * WQB);  // this wave's quarter tile (LDS address)
    const bool raw = tile >= tiles_p;
    const int v0 = raw ? (tile - tiles_p) * WTR : tile * WTR;
    if constexpr (TREAT) {
      if (raw) {  // raw rows: RMSNorm over all 512 dims, RoPE on the last RD (head block 0's waves)
        // lane (n, g): row n, chunks c = g, g+2, ..., g+14 of quarter q (a
        // rotate-half partner chunk is RD/16 chunks on: same parity, same lane)
        uint8_t* rowp = ring + slot * (4 * WQB) + q * WQB + n * (WQ * 2);
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
          const double pos = (double)(sv.raw_begin + v0 + n);
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
    // valid rows of the tile (lane n: row n)
    uint32_t mk;
    {
      int64_t row;
      const bool ok = locate(raw, v0 + n, row);
      mk = (uint32_t)(__ballot(ok) & 0xffffffffull);
    }
    // partial scores over this wave's dims: S^T[row, head], rows 8j + 4g + i
    f32x16 sc;
    {
      uint4 ka[WKST];
      const uint32_t kad[4] = {sa + koff[0], sa + koff[1], sa + koff[2], sa + koff[3]};
      wide_k_reads(ka, kad);
      f32x16 s2;
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = s2[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < WKST; ks += 2) {  // two independent chains
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[ks]),
                                                     __builtin_bit_cast(bf16x8, qb[ks]), sc, 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[ks + 1]),
                                                     __builtin_bit_cast(bf16x8, qb[ks + 1]), s2, 0, 0, 0);
      }
      sc += s2;
    }
    float* xw = xs[hb][q];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(&xw[(j * 64 + lane) * 4]) =
          make_float4(sc[4 * j], sc[4 * j + 1], sc[4 * j + 2], sc[4 * j + 3]);
    lds_barrier();
    // full scores: the head block's four partials in a fixed order (identical in its waves)
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
      float4 xr[8];  // [j - 2jh][quarter]
      wide_x_reads(xr, xs_a + 2048u * jh);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        float4 t = xr[4 * jj];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const float4 o = xr[4 * jj + w];
          t.x += o.x; t.y += o.y; t.z += o.z; t.w += o.w;
        }
        const int j = 2 * jh + jj;
        sc[4 * j] = t.x; sc[4 * j + 1] = t.y; sc[4 * j + 2] = t.z; sc[4 * j + 3] = t.w;
      }
    }
    // mask, scale into the exponent's units, running max (moves lazily)
    float tmax = kNegInf;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 8 * j + 4 * g + e;
        const float v = ((mk >> row) & 1u) ? sc[4 * j + e] * p.scale_log2 : kNegInf;
        sc[4 * j + e] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = xor32_max(tmax);
    if (__ballot(tmax > m_run + 8.f)) {
      const float nm = fmaxf(m_run, tmax);
      const float corr = nm == kNegInf ? 1.f : fast_exp2(m_run - nm);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < WDB; ++db) acc[db] *= corr;
      m_run = nm;
    }
    const float mu = m_run == kNegInf ? 0.f : m_run;
    float psum = 0.f;
    uint32_t pw[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float pj[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pj[e] = fast_exp2(sc[4 * j + e] - mu);
        psum += pj[e];
      }
      pw[2 * j] = pack_bf16x2(pj[0], pj[1]);
      pw[2 * j + 1] = pack_bf16x2(pj[2], pj[3]);
    }
    l_run += psum;
    // O^T += V^T P^T, two 16-row blocks: P^T of block kb is this lane's rows of j = 2kb, 2kb+1
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s16x4 va[8];
      const uint32_t o = sa + 4096u * kb;
      const uint32_t ta[4] = {o + toff[kb], o + toff[1 - kb], o + toff[2 + kb], o + toff[3 - kb]};
      wide_tr_reads(va, ta);
      const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pw[4 * kb], pw[4 * kb + 1], pw[4 * kb + 2], pw[4 * kb + 3]));
#pragma unroll
      for (int db = 0; db < WDB; ++db) {
        const s16x4 a0 = va[2 * db], a1 = va[2 * db + 1];
        const bf16x8 a = __builtin_bit_cast(bf16x8, s16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[db], 0, 0, 0);
      }
    }
    slot = slot == WSLOTS - 1 ? 0 : slot + 1;
  }
  const float M = m_run;
  float L = xor32_sum(l_run);

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
    float* o = p.out + (b * p.hq + head) * WD + WQ * q + 4 * g;
#pragma unroll
    for (int db = 0; db < WDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(o + 32 * db + 8 * j) =
            make_float4(acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2], acc[db][4 * j + 3]);
    if (p.lse && q == 0 && g == 0) p.lse[b * p.hq + head] = (M + log2f(L)) * 0.69314718055994531f;
    return;
  }
  // split partial in the 16-head-unit layout: unit (b, kvh, 16-head group), part = unit * S + split
  const int64_t unit = (b * p.hkv + kvh) * p.head_groups + 2 * hb + (n >> 4);
  const int64_t part = unit * S + split;
  float* o = p.ws_acc + (part * 16 + (n & 15)) * WD + WQ * q + 4 * g;
#pragma unroll
  for (int db = 0; db < WDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(o + 32 * db + 8 * j) =
          make_float4(acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2], acc[db][4 * j + 3]);
  if (q == 0 && g == 0) {
    p.ws_ml[(part * 16 + (n & 15)) * 2] = M;
    p.ws_ml[(part * 16 + (n & 15)) * 2 + 1] = L;
  }
}

hipError_t launch_decode_wide(const DecodeParams& p, int rope_dims, bool treat, int head_blocks,
                              hipStream_t stream) {
  const unsigned seqs = (unsigned)(p.units / (2 * head_blocks));  // sequences x KV heads
  const dim3 grid(seqs * (unsigned)p.splits);
  const bool sel = p.sel != nullptr;
  auto go = [&](auto kern, int hb) {
    kern<<<grid, 256 * hb, 0, stream>>>(p);
    return hipGetLastError();
  };
  auto pick = [&](auto hbc) -> hipError_t {
    constexpr int HB = decltype(hbc)::value;
    if (!treat) return sel ? go(decode_wide_kernel<HB, 0, false, true>, HB) : go(decode_wide_kernel<HB, 0, false, false>, HB);
    switch (rope_dims) {
      case 0: return sel ? go(decode_wide_kernel<HB, 0, true, true>, HB) : go(decode_wide_kernel<HB, 0, true, false>, HB);
      case 64: return sel ? go(decode_wide_kernel<HB, 64, true, true>, HB) : go(decode_wide_kernel<HB, 64, true, false>, HB);
      case 128: return sel ? go(decode_wide_kernel<HB, 128, true, true>, HB) : go(decode_wide_kernel<HB, 128, true, false>, HB);
      default: return hipErrorInvalidValue;
    }
  };
  if (head_blocks == 2) return pick(std::integral_constant<int, 2>{});
  if (head_blocks == 1) return pick(std::integral_constant<int, 1>{});
  return hipErrorInvalidValue;
}

}  // namespace lbca
