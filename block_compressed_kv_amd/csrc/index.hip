// CSA lightning indexer scores and top-k selection.
//
// Method: "CSA: Compressed Sparse Attention (toy implementation)", "What is
// implemented" (second item): per-head ReLU relevance of the indexer queries
// against the compressed indexer keys, mixed by learned head weights, then a
// top-k restricted to causally visible entries.
//
// Scoring is HBM-bound (a 64-dim bf16 key is read once and meets every indexer
// head): one wave scores 64 keys with v_mfma_f32_16x16x32_bf16, A = key rows
// read straight from global memory, B = the indexer queries (heads padded to
// 16); each lane then holds one head's dot products for 4 keys, applies
// w_h * relu(.) and a 16-lane reduction sums the heads.  Scores go to the
// workspace in fp32.
//
// Selection is exact and deterministic: an MSB-first radix select over the
// order-preserving 32-bit image of the fp32 scores (held in registers) finds
// the k-th largest key, then block-wide scans in index order take every
// larger score and the lowest-index ties, writing the chosen ids in ascending
// order.
#include "device_util.h"
#include "lbca_internal.h"

namespace lbca {

struct IndexParams {
  const bf16_t* q;
  const float* w;
  const bf16_t* keys;
  const int64_t* pos;
  int32_t* out_idx;
  float* out_score;
  float* scores;  // [B][stride]
  uint32_t* cand_key;  // two-stage selection: [B][slices * k] order keys of the slices' top-k
  int32_t* cand_id;    // [B][slices * k] their entry ids (-1: padding)
  int64_t heads, entries, k, m, stride;  // stride: entries rounded up to 4 (16-byte rows)
  int slices;                            // two-stage selection: slices of kSliceLen entries
  int64_t cstride;                       // candidates per sequence, rounded up to 4
  int64_t qrows;                         // chunk scoring: query rows per key sequence
  // element strides: queries {sequence, query of a chunk, head}, keys {sequence, entry}
  Str q_st, k_st;
};

__device__ __forceinline__ int64_t n_visible(const IndexParams& p, int64_t b) {
  const int64_t t = p.pos[b];
  if (t < 0) return 0;
  const int64_t n = (t + 1) / p.m;
  return n < p.entries ? n : p.entries;
}

// Sum over each 16-lane row with DPP moves; the total lands in lane 15 of the row.
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xF, 0xF, true));
  return x;
}

// One wave scores 64 keys.  Every load is issued up front and carries no
// branch (keys past the visible ones read the last visible key; padded heads
// read head 0's query and have weight 0), so the loads overlap and each wait
// covers only what it needs.
template <int DI>
__global__ __launch_bounds__(256) void index_score_kernel(IndexParams p) {
  constexpr int KS = DI / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kq = lane >> 4;
  const int64_t b = blockIdx.y;
  const int64_t nv = n_visible(p, b);
  const int64_t key0 = ((int64_t)blockIdx.x * 4 + wave) * 64;
  if (key0 >= nv) return;  // whole wave beyond the visible keys
  const bool head_ok = n < p.heads;
  const bf16_t* qrow = p.q + b * p.q_st.s0 + (head_ok ? n : 0) * p.q_st.s2 + 8 * kq;
  uint4 qr[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qr[s] = *reinterpret_cast<const uint4*>(qrow + 32 * s);
  const float wv = p.w[b * p.heads + (head_ok ? n : 0)];
  uint4 kv[4][KS];
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    int64_t key = key0 + 16 * hh + n;
    key = key < nv ? key : nv - 1;
    const bf16_t* krow = p.keys + b * p.k_st.s0 + key * p.k_st.s1 + 8 * kq;
#pragma unroll
    for (int s = 0; s < KS; ++s) kv[hh][s] = *reinterpret_cast<const uint4*>(krow + 32 * s);
  }
  const float wh = head_ok ? wv : 0.f;
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv[hh][s]),
                                                   __builtin_bit_cast(bf16x8, qr[s]), c, 0, 0, 0);
    // lane (n, kq) holds head n's dot products with keys kbase .. kbase + 3
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = row16_sum(wh * fmaxf(c[j], 0.f));
    const int64_t kbase = key0 + 16 * hh + 4 * kq;
    if (n == 15) {
      float* dst = p.scores + b * p.stride + kbase;
      if (kbase + 3 < nv) {
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (kbase + j < nv) dst[j] = v[j];
      }
    }
  }
}

// Sum over aligned groups of HP lanes (8 or 16) inside each 16-lane row; every
// lane of a group gets the total (quad swaps, then the half-row and row mirrors).
template <int HP>
__device__ __forceinline__ float lane_group_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  if constexpr (HP == 16)
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

#ifndef LBCA_CHUNK_Q
#define LBCA_CHUNK_Q 64
#endif
constexpr int kChunkQ = LBCA_CHUNK_Q;  // queries per workgroup of the chunk scorer

// Chunk scoring: one wave holds 64 keys in registers and runs every query of
// its workgroup's group of kChunkQ over them; the MFMA's 16 B columns carry QP
// queries' heads at once (HP = 16 / QP head slots each, padded heads weigh 0),
// so a key tile read once serves the whole query group.  The next query's
// rows are requested before the current one is scored.
template <int DI, int QP>
__global__ __launch_bounds__(256) void index_score_chunk_kernel(IndexParams p) {
  constexpr int KS = DI / 32, HP = 16 / QP;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kq = lane >> 4;
  const int qo = n / HP, hd = n % HP;
  const int64_t seq = blockIdx.z;
  const int64_t q0 = (int64_t)blockIdx.y * kChunkQ;
  const int64_t qn = p.qrows - q0 < kChunkQ ? p.qrows - q0 : kChunkQ;
  const int64_t r0 = seq * p.qrows + q0;
  const int64_t nv_last = n_visible(p, r0 + qn - 1);  // positions grow along the chunk
  const int64_t key0 = ((int64_t)blockIdx.x * 4 + wave) * 64;
  if (key0 >= nv_last) return;  // no query of the group sees these keys
  uint4 kv[4][KS];
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    int64_t key = key0 + 16 * hh + n;
    key = key < nv_last ? key : nv_last - 1;
    const bf16_t* krow = p.keys + seq * p.k_st.s0 + key * p.k_st.s1 + 8 * kq;
#pragma unroll
    for (int s = 0; s < KS; ++s) kv[hh][s] = *reinterpret_cast<const uint4*>(krow + 32 * s);
  }
  const bool head_ok = hd < p.heads;
  const int hsafe = head_ok ? hd : 0;
  // query slot i + qo of the group: its row (clamped into the group), rows and weight
  auto row_of = [&](int64_t i) { return r0 + (i + qo < qn ? i + qo : i); };
  // query row r (query r - seq * qrows of the sequence), this lane's head
  const bf16_t* qseq = p.q + seq * p.q_st.s0 + hsafe * p.q_st.s2 + 8 * kq;
  auto qrow_of = [&](int64_t rr) { return qseq + (rr - seq * p.qrows) * p.q_st.s1; };
  uint4 qr[KS];
  int64_t r = row_of(0);
#pragma unroll
  for (int s = 0; s < KS; ++s) qr[s] = *reinterpret_cast<const uint4*>(qrow_of(r) + 32 * s);
  float wv = p.w[r * p.heads + hsafe];
  int64_t tpos = p.pos[r];
  for (int64_t i = 0; i < qn; i += QP) {
    // request the next slot's rows first
    const int64_t rn = row_of(i + QP < qn ? i + QP : i);
    uint4 qn_r[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qn_r[s] = *reinterpret_cast<const uint4*>(qrow_of(rn) + 32 * s);
    const float wn = p.w[rn * p.heads + hsafe];
    const int64_t tn = p.pos[rn];
    const bool q_ok = i + qo < qn;
    const float wh = head_ok && q_ok ? wv : 0.f;
    int64_t nv = tpos < 0 ? 0 : (tpos + 1) / p.m;
    nv = nv < p.entries ? nv : p.entries;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv[hh][s]),
                                                     __builtin_bit_cast(bf16x8, qr[s]), c, 0, 0, 0);
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = lane_group_sum<HP>(wh * fmaxf(c[j], 0.f));
      const int64_t kbase = key0 + 16 * hh + 4 * kq;
      if (hd == 0 && q_ok) {
        float* dst = p.scores + r * p.stride + kbase;
        if (kbase + 3 < nv) {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (kbase + j < nv) dst[j] = v[j];
        }
      }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) qr[s] = qn_r[s];
    r = rn;
    wv = wn;
    tpos = tn;
  }
}

__global__ void fill_rows_kernel(int64_t* pos, int64_t* rpb, int64_t rows, int64_t q_len, int64_t q_pos0,
                                 int64_t raw_pos_base) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  pos[r] = q_pos0 + r % q_len;
  rpb[r] = raw_pos_base;
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS round trips):
// shifts by 1, 2, 4, 8 within each 16-lane row, then lane 15 of a row added
// to the next row, then lane 31 added to the upper half.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Over the wave's lanes in order, with values v (>= 0) and a running count
// `before` ahead of lane 0: the first lane where before + (inclusive sum)
// reaches `target`; *base gets before + the sum of the lanes ahead of it.
__device__ __forceinline__ int wave_crossing(int v, int target, int before, int* base) {
  const int x = wave_incl_scan(v);
  const uint64_t hit = __ballot(before + x >= target);
  const int L = hit ? (int)__builtin_ctzll(hit) : 63;
  *base = before + __builtin_amdgcn_readlane(x - v, L);
  return L;
}

// Key back to the score it was made from (order_key is a bijection on floats
// other than -0).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Entries per slice of the two-stage selection (1024 threads x 4 keys).
constexpr int kSliceLen = 4096;

// MODE 0: one workgroup per sequence over all its visible scores.
// MODE 1 (first stage of two): workgroup (slice, sequence) over the visible
// scores of entries [slice * kSliceLen, +kSliceLen); it writes the slice's
// top-k as (order key, entry id) candidates in index order, padded with
// (0, -1) when the slice has at most k visible entries.  The top-k of the
// whole sequence is among the slices' top-k (each of its members is in the
// top-k of its own slice under the same order and tie rule).
// MODE 2 (second stage): one workgroup per sequence over the slices *
// k candidates; candidate order is index order, so the same tie rule (lower
// index first) is the lower candidate position, and padding (key 0, below
// every finite score's key) is never chosen.
// Every thread keeps KPT scores (as order-preserving
// 32-bit keys) of entries r * 1024 + tid in registers.  The k-th largest key is
// found by a radix select over 12 + 10 + 10 bits: each pass counts the keys
// that still match the digits chosen so far into an LDS histogram, and a scan
// from the top bin finds the bin holding the k-th largest.  The first pass is
// workgroup-wide; the keys of its chosen bin are then compacted, and wave 0
// alone runs the other two passes over that list (no workgroup barriers).
// The selection then takes every key above it and the lowest-index keys equal
// to it: each element's output slot is the number of selected elements before
// it in index order, from per-(round, wave) counts scanned across the block.
template <int KPT, int MODE>
__global__ __launch_bounds__(1024) void topk_kernel(IndexParams p) {
  static_assert(MODE != 1 || KPT * 1024 == kSliceLen, "a first-stage workgroup holds one slice");
  // LDS: the scores when more than 8 per thread are staged there (copied
  // straight from global memory), then the histograms (4 interleaved copies
  // per bin in the workgroup-wide passes, so lanes of one wave that hit the
  // same bin mostly hit different words)
  constexpr int STAGE = KPT <= 32 ? KPT * 1024 : 0;
  constexpr int LDS_WORDS = STAGE > 4096 * 5 ? STAGE : 4096 * 5;  // histogram + candidate list
  __shared__ __attribute__((aligned(16))) int lds_words[LDS_WORDS];
  int* hist = lds_words;
  __shared__ int s_gt[KPT * 16], s_eq[KPT * 16];
  __shared__ int s_part[1024];
  __shared__ int s_nc;
  __shared__ int s_pick[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = MODE == 1 ? blockIdx.y : blockIdx.x;
  const int nvis = (int)n_visible(p, b);
  const int K = (int)p.k;
  const int base = MODE == 1 ? (int)blockIdx.x * kSliceLen : 0;  // entry id of item 0
  // items of this workgroup: visible scores (MODE 0), the slice's visible
  // scores (MODE 1), or every candidate slot (MODE 2)
  const int nv = MODE == 0 ? nvis
               : MODE == 1 ? (nvis - base < 0 ? 0 : (nvis - base < kSliceLen ? nvis - base : kSliceLen))
                           : p.slices * K;
  const float* sc = p.scores + b * p.stride + base;
  const uint32_t* ck = p.cand_key + b * p.cstride;
  const int32_t* cid = p.cand_id + b * p.cstride;
  int32_t* oi = p.out_idx + b * K;
  float* os = p.out_score ? p.out_score + b * K : nullptr;
  const int64_t wofs = b * p.cstride + (int64_t)(MODE == 1 ? (int)blockIdx.x : 0) * K;  // MODE 1 output
  uint32_t* wk = p.cand_key + wofs;
  int32_t* wi = p.cand_id + wofs;

  if constexpr (MODE == 2) {
    // real candidates: min(k, visible entries of the slice) at the head of each slice's block
    int n_real = 0;
    for (int q = 0; q < p.slices; ++q) {
      const int c = nvis - q * kSliceLen;
      n_real += c <= 0 ? 0 : (c < K ? c : K);
    }
    if (n_real <= K) {  // all of them, in order, then padding
      for (int i = tid; i < K; i += blockDim.x) {
        int q = 0, at = i, id = -1;
        uint32_t key = 0;
        for (; q < p.slices; ++q) {
          const int c0 = nvis - q * kSliceLen, c = c0 <= 0 ? 0 : (c0 < K ? c0 : K);
          if (at < c) {
            id = cid[q * K + at];
            key = ck[q * K + at];
            break;
          }
          at -= c;
        }
        oi[i] = id;
        if (os) os[i] = id >= 0 ? key_score(key) : __builtin_nanf("");
      }
      return;
    }
  } else if (nv <= K) {
    for (int i = tid; i < K; i += blockDim.x) {
      const bool in = i < nv;
      if constexpr (MODE == 0) {
        oi[i] = in ? (int32_t)i : -1;
        if (os) os[i] = in ? sc[i] : __builtin_nanf("");
      } else {
        wk[i] = in ? order_key(sc[i]) : 0u;
        wi[i] = in ? (int32_t)(base + i) : -1;
      }
    }
    return;
  }

  uint32_t key[KPT];
  int32_t cidr[MODE == 2 ? KPT : 1];  // second stage: the candidates' entry ids, requested with their keys
  // Up to 8 keys per thread go straight to registers while the first pass's
  // histogram is cleared; more are staged through the LDS in 16-byte copies.
  constexpr bool DIRECT = KPT <= 8;
  if constexpr (DIRECT) {
    uint32_t rk[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int i = r * 1024 + tid;
      const int j = i < nv ? i : 0;  // a clamped index: every thread issues every load
      rk[r] = MODE == 2 ? ck[j] : __float_as_uint(sc[j]);
      if constexpr (MODE == 2) cidr[r] = cid[j];
    }
    for (int i = tid; i < 4096; i += 1024) *reinterpret_cast<int4*>(&hist[4 * i]) = make_int4(0, 0, 0, 0);
    if (tid == 0) s_nc = 0;
#pragma unroll
    for (int r = 0; r < KPT; ++r)
      key[r] = r * 1024 + tid < nv ? (MODE == 2 ? rk[r] : order_key(__uint_as_float(rk[r]))) : 0u;
    __syncthreads();  // histogram cleared
  } else if constexpr (STAGE > 0) {
    // 16-byte copies of the visible scores to LDS (lane i of a wave writes
    // bytes 16 i of the wave's 1 KB), the last nv % 4 scores one by one
    // (MODE 2: the candidates' keys, 4 bytes each as well)
    const int nc = nv >> 2;
    uint32_t* stage = reinterpret_cast<uint32_t*>(lds_words);
    const uint32_t* src = MODE == 2 ? ck : reinterpret_cast<const uint32_t*>(sc);
    for (int c0 = wave * 64; c0 < nc; c0 += 1024) {
      if (c0 + lane < nc)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<gbl_void*>(reinterpret_cast<uintptr_t>(src + 4 * (c0 + lane))),
                                         (lds_void*)(stage + 4 * c0), 16, 0, 0);
    }
    if (tid < nv - 4 * nc) stage[4 * nc + tid] = src[4 * nc + tid];
    if constexpr (MODE == 2) {
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const int i = r * 1024 + tid;
        cidr[r] = cid[i < nv ? i : 0];
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies landed
    __syncthreads();
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int i = r * 1024 + tid;
      key[r] = i < nv ? (MODE == 2 ? stage[i] : order_key(__uint_as_float(stage[i]))) : 0u;
    }
    __syncthreads();  // the LDS becomes the histogram
  } else {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int i = r * 1024 + tid;
      key[r] = i < nv ? (MODE == 2 ? ck[i] : order_key(sc[i])) : 0u;
      if constexpr (MODE == 2) cidr[r] = cid[i < nv ? i : 0];
    }
  }

  uint32_t prefix = 0, pmask = 0;
  int remaining = K;
  // candidate list (keys of the chosen first-pass bin) in the LDS past the histogram
  constexpr int kCandMax = (LDS_WORDS - 4 * 4096) > 4096 ? 4096 : (LDS_WORDS - 4 * 4096);
  uint32_t* cand = reinterpret_cast<uint32_t*>(lds_words + 4 * 4096);
  int n_cand = -1;
  auto count = [&](int bin) {
    const int4 h = *reinterpret_cast<const int4*>(&hist[4 * bin]);
    return h.x + h.y + h.z + h.w;
  };
  // One block-wide radix pass over the keys still matching the digits chosen
  // so far (from the compacted list when there is one).
  auto block_pass = [&](int pass) __attribute__((always_inline)) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
    const int nb = pass == 0 ? 4096 : 1024;
    if (!(DIRECT && pass == 0)) {  // (the direct load cleared the first histogram)
      for (int i = tid; i < nb; i += 1024) *reinterpret_cast<int4*>(&hist[4 * i]) = make_int4(0, 0, 0, 0);
      __syncthreads();
    }
    // Keys past the visible entries are 0 and every visible key is at least
    // 2^23 (order image of a finite float), so they fall in bin 0 of the first
    // pass (never the chosen one) and never match a later prefix.
    if (pass > 0 && n_cand >= 0) {
      for (int c = tid; c < n_cand; c += 1024) {
        const uint32_t k = cand[c];
        if ((k & pmask) == prefix) atomicAdd(&hist[4 * ((k >> shift) & (uint32_t)(nb - 1)) + (lane & 3)], 1);
      }
    } else {
#pragma unroll
      for (int r = 0; r < KPT; ++r)
        if ((key[r] & pmask) == prefix)
          atomicAdd(&hist[4 * ((key[r] >> shift) & (uint32_t)(nb - 1)) + (lane & 3)], 1);
    }
    __syncthreads();
    // find the bin holding the remaining-th largest key: thread t sums bins
    // nb-1-t*per .. nb-(t+1)*per (per = nb/1024) into s_part[t]; then one wave
    // narrows it down: 16 threads per lane, then the thread, then its bins
    const int per = nb / 1024;
    {
      int local = 0;
      for (int j = 0; j < per; ++j) local += count(nb - 1 - tid * per - j);
      s_part[tid] = local;
    }
    __syncthreads();
    if (wave == 0) {
      int l16 = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) l16 += s_part[16 * lane + j];
      int bs;
      const int L = wave_crossing(l16, remaining, 0, &bs);  // lane holding the crossing
      const int tv = lane < 16 ? s_part[16 * L + lane] : 0;
      const int J = wave_crossing(tv, remaining, bs, &bs);
      const int t = 16 * L + J;
      const int bv = lane < per ? count(nb - 1 - t * per - lane) : 0;
      const int jb = wave_crossing(bv, remaining, bs, &bs);
      if (lane == 0) {
        s_pick[0] = nb - 1 - t * per - jb;
        s_pick[1] = remaining - bs;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_pick[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    remaining = s_pick[1];
  };

  block_pass(0);
  {  // compact the chosen bin's keys (if they fit) for the later passes
    const int nbin = count(s_pick[0]);
    __syncthreads();  // every wave has read the count; the list may overwrite LDS past the histogram
    if (nbin <= kCandMax) {
      if constexpr (!DIRECT) {
        if (tid == 0) s_nc = 0;
        __syncthreads();
      }
      // one LDS atomic per wave: lane offsets from a scan of per-thread counts
      int mine = 0;
#pragma unroll
      for (int r = 0; r < KPT; ++r) mine += (key[r] & pmask) == prefix;
      const int incl = wave_incl_scan(mine);
      int wb = 0;
      if (lane == 63) wb = atomicAdd(&s_nc, incl);
      int at = __builtin_amdgcn_readlane(wb, 63) + incl - mine;
#pragma unroll
      for (int r = 0; r < KPT; ++r)
        if ((key[r] & pmask) == prefix) cand[at++] = key[r];
      __syncthreads();
      n_cand = s_nc;
    }
  }
  if (n_cand >= 0) {
    // The two 10-bit passes over the compacted list in wave 0 alone (no
    // workgroup barriers): a private 1024-bin histogram, lane L counting the
    // descending bins 1023 - 16 L .. 1008 - 16 L.  A wave's LDS operations
    // complete in order, so each clear, count and read sees the one before.
    if (wave == 0) {
#pragma unroll
      for (int pass = 1; pass < 3; ++pass) {
        const int shift = pass == 1 ? 10 : 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<int4*>(&hist[16 * lane + 4 * j]) = make_int4(0, 0, 0, 0);
        for (int c = lane; c < n_cand; c += 64) {
          const uint32_t k = cand[c];
          if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 1023u], 1);
        }
        const int blk = 63 - lane;  // storage block of this lane's descending bins
        int sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int4 h = *reinterpret_cast<const int4*>(&hist[16 * blk + 4 * j]);
          sum += (h.x + h.y) + (h.z + h.w);
        }
        int bs;
        const int L = wave_crossing(sum, remaining, 0, &bs);
        const int bv = lane < 16 ? hist[16 * (63 - L) + 15 - lane] : 0;
        const int J = wave_crossing(bv, remaining, bs, &bs);
        prefix |= (uint32_t)(16 * (63 - L) + 15 - J) << shift;
        pmask |= 1023u << shift;
        remaining -= bs;
      }
      if (lane == 0) {
        s_pick[0] = (int)prefix;
        s_pick[1] = remaining;
      }
    }
    __syncthreads();
    prefix = (uint32_t)s_pick[0];
    remaining = s_pick[1];
  } else {
    block_pass(1);
    block_pass(2);
  }
  const uint32_t thr = prefix;       // key of the k-th largest score
  const int need_eq = remaining;     // keys equal to it to take, lowest index first

  // counts above / equal to the threshold per (round, wave), then one wave
  // turns them into exclusive prefixes in index order (round-major)
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const bool in = r * 1024 + tid < nv;
    const uint64_t gm = __ballot(in && key[r] > thr), em = __ballot(in && key[r] == thr);
    if (lane == 0) {
      s_gt[r * 16 + wave] = __popcll(gm);
      s_eq[r * 16 + wave] = __popcll(em);
    }
  }
  __syncthreads();
  if (wave == 0) {
    constexpr int PER = KPT * 16 / 64;  // entries per lane
    int lg = 0, lq = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      lg += s_gt[lane * PER + j];
      lq += s_eq[lane * PER + j];
    }
    const int xg = wave_incl_scan(lg), xq = wave_incl_scan(lq);
    int cg = xg - lg, cq = xq - lq;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int g = s_gt[lane * PER + j], q = s_eq[lane * PER + j];
      s_gt[lane * PER + j] = cg;
      s_eq[lane * PER + j] = cq;
      cg += g;
      cq += q;
    }
  }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const int i = r * 1024 + tid;
    const bool in = i < nv;
    const bool gt = in && key[r] > thr, eq = in && key[r] == thr;
    const uint64_t gm = __ballot(gt), em = __ballot(eq);
    const int gb = s_gt[r * 16 + wave] + __popcll(gm & below);
    const int eb = s_eq[r * 16 + wave] + __popcll(em & below);
    int slot = -1;
    if (gt) slot = gb + (eb < need_eq ? eb : need_eq);
    else if (eq && eb < need_eq) slot = gb + eb;
    if (slot >= 0) {
      if constexpr (MODE == 0) {
        oi[slot] = (int32_t)i;
        if (os) os[slot] = sc[i];
      } else if constexpr (MODE == 1) {
        wk[slot] = key[r];
        wi[slot] = (int32_t)(base + i);
      } else {
        oi[slot] = cidr[r];
        if (os) os[slot] = key_score(key[r]);
      }
    }
  }
}

// Two-stage selection when the entries span at least 3 slices and each slice
// keeps at most a quarter of its entries; the second stage holds every
// candidate in registers (at most 16 per thread).
static int select_slices(const csa_index_args& a) {
  const int64_t P = (a.entries + kSliceLen - 1) / kSliceLen;
  if (P < 3 || a.k * 4 > kSliceLen || P * a.k > 16 * 1024) return 0;
  return (int)P;
}

size_t index_workspace_bytes(const csa_index_args& a) {
  size_t bytes = (size_t)a.batch * (size_t)((a.entries + 3) & ~int64_t(3)) * sizeof(float);
  const int P = select_slices(a);
  if (P > 0) bytes += (size_t)a.batch * (size_t)((P * a.k + 3) & ~int64_t(3)) * (sizeof(uint32_t) + sizeof(int32_t));
  return bytes;
}

static hipError_t launch_topk(const IndexParams& p, const csa_index_args& a, hipStream_t stream);

static IndexParams index_params(const csa_index_args& a, void* ws) {
  IndexParams p{};
  p.q = static_cast<const bf16_t*>(a.q_idx);
  p.w = a.head_w;
  p.keys = static_cast<const bf16_t*>(a.keys);
  p.pos = a.pos;
  p.out_idx = a.out_idx;
  p.out_score = a.out_score;
  p.scores = static_cast<float*>(ws);
  p.heads = a.heads; p.entries = a.entries; p.k = a.k; p.m = a.block;
  p.stride = (a.entries + 3) & ~int64_t(3);
  p.slices = select_slices(a);
  if (p.slices > 0) {
    p.cstride = (p.slices * a.k + 3) & ~int64_t(3);
    p.cand_key = reinterpret_cast<uint32_t*>(p.scores + a.batch * p.stride);
    p.cand_id = reinterpret_cast<int32_t*>(p.cand_key + a.batch * p.cstride);
  }
  p.qrows = 1;
  p.q_st = lbca_strides{{a.q_idx_st.s[0], 0, a.q_idx_st.s[1]}};  // [batch, heads, dim]
  p.k_st = a.keys_st;
  return p;
}

hipError_t launch_index_topk(const csa_index_args& a, void* ws, hipStream_t stream) {
  const IndexParams p = index_params(a, ws);
  if (a.entries > 0) {
    const dim3 grid((unsigned)((a.entries + 255) / 256), (unsigned)a.batch);
    switch (a.dim) {
      case 32: index_score_kernel<32><<<grid, 256, 0, stream>>>(p); break;
      case 64: index_score_kernel<64><<<grid, 256, 0, stream>>>(p); break;
      case 128: index_score_kernel<128><<<grid, 256, 0, stream>>>(p); break;
      default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_topk(p, a, stream);
}

hipError_t launch_index_topk_chunk(const csa_index_args& a, int64_t q_len, int64_t q_pos0, int64_t raw_pos_base,
                                   int64_t* pos_ws, int64_t* rpb_ws, void* ws, hipStream_t stream) {
  fill_rows_kernel<<<(unsigned)((a.batch + 255) / 256), 256, 0, stream>>>(pos_ws, rpb_ws, a.batch, q_len, q_pos0,
                                                                          raw_pos_base);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  IndexParams p = index_params(a, ws);
  p.pos = pos_ws;
  p.qrows = q_len;
  p.q_st = a.q_idx_st;  // a query chunk's rows: {sequence, query, head}
  if (a.entries > 0) {
    const dim3 grid((unsigned)((a.entries + 255) / 256), (unsigned)((q_len + kChunkQ - 1) / kChunkQ),
                    (unsigned)(a.batch / q_len));
    const bool two = a.heads <= 8;
    switch (a.dim * 2 + (two ? 1 : 0)) {
      case 32 * 2 + 1: index_score_chunk_kernel<32, 2><<<grid, 256, 0, stream>>>(p); break;
      case 32 * 2: index_score_chunk_kernel<32, 1><<<grid, 256, 0, stream>>>(p); break;
      case 64 * 2 + 1: index_score_chunk_kernel<64, 2><<<grid, 256, 0, stream>>>(p); break;
      case 64 * 2: index_score_chunk_kernel<64, 1><<<grid, 256, 0, stream>>>(p); break;
      case 128 * 2 + 1: index_score_chunk_kernel<128, 2><<<grid, 256, 0, stream>>>(p); break;
      case 128 * 2: index_score_chunk_kernel<128, 1><<<grid, 256, 0, stream>>>(p); break;
      default: return hipErrorInvalidValue;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_topk(p, a, stream);
}

// From this many rows on, one selection workgroup per row already fills the
// chip, and the slice stage would only add a pass over the candidates.
constexpr int64_t kOneStageRows = 256;

static hipError_t launch_topk(const IndexParams& p, const csa_index_args& a, hipStream_t stream) {
  const dim3 g((unsigned)a.batch);
  if (p.slices > 0 && a.batch < kOneStageRows) {
    topk_kernel<4, 1><<<dim3((unsigned)p.slices, (unsigned)a.batch), 1024, 0, stream>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nc = p.slices * a.k;
    if (nc <= 4096) topk_kernel<4, 2><<<g, 1024, 0, stream>>>(p);
    else if (nc <= 8192) topk_kernel<8, 2><<<g, 1024, 0, stream>>>(p);
    else topk_kernel<16, 2><<<g, 1024, 0, stream>>>(p);
    return hipGetLastError();
  }
  if (a.entries <= 4096) topk_kernel<4, 0><<<g, 1024, 0, stream>>>(p);
  else if (a.entries <= 16384) topk_kernel<16, 0><<<g, 1024, 0, stream>>>(p);
  else if (a.entries <= 32768) topk_kernel<32, 0><<<g, 1024, 0, stream>>>(p);
  else topk_kernel<64, 0><<<g, 1024, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace lbca
