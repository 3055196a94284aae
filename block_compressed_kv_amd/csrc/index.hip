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
  float* scores;  // [B][entries]
  int64_t heads, entries, k, m;
};

__device__ __forceinline__ int64_t n_visible(const IndexParams& p, int64_t b) {
  const int64_t t = p.pos[b];
  if (t < 0) return 0;
  const int64_t n = (t + 1) / p.m;
  return n < p.entries ? n : p.entries;
}

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
  const bf16_t* qrow = p.q + (b * p.heads + n) * DI + 8 * kq;
  uint4 qr[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qr[s] = head_ok ? *reinterpret_cast<const uint4*>(qrow + 32 * s) : make_uint4(0, 0, 0, 0);
  const float wh = head_ok ? p.w[b * p.heads + n] : 0.f;
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    const int64_t key = key0 + 16 * hh + n;
    const bool ok = key < nv;
    const bf16_t* krow = p.keys + (b * p.entries + key) * DI + 8 * kq;
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 kv = ok ? *reinterpret_cast<const uint4*>(krow + 32 * s) : make_uint4(0, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv),
                                                   __builtin_bit_cast(bf16x8, qr[s]), c, 0, 0, 0);
    }
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = wh * fmaxf(c[j], 0.f);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += __shfl_xor(v[j], o, 64);
    const int64_t kbase = key0 + 16 * hh + 4 * kq;  // keys of lane (., kq): kbase .. kbase+3
    if (n == 0) {
      float* dst = p.scores + b * p.entries + kbase;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (kbase + j < nv) dst[j] = v[j];
    }
  }
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one value per thread over a 1024-thread block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_sums, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_sums[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int s = lane < 16 ? wave_sums[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    if (lane < 16) wave_sums[16 + lane] = s;  // inclusive prefix of wave totals
  }
  __syncthreads();
  const int before = wave > 0 ? wave_sums[16 + wave - 1] : 0;
  if (total) *total = wave_sums[16 + 15];
  const int r = before + x - v;
  __syncthreads();
  return r;
}

// One workgroup per sequence; every thread keeps KPT scores (as order-preserving
// 32-bit keys) of entries r * 1024 + tid in registers.  The k-th largest key is
// found by a radix select over 12 + 10 + 10 bits: each pass counts the keys
// that still match the digits chosen so far into an LDS histogram, and a
// block-wide scan from the top bin finds the bin holding the k-th largest.
// The selection then takes every key above it and the lowest-index keys equal
// to it: each element's output slot is the number of selected elements before
// it in index order, from per-(round, wave) counts scanned across the block.
template <int KPT>
__global__ __launch_bounds__(1024) void topk_kernel(IndexParams p) {
  __shared__ int hist[4096];
  __shared__ int scan_buf[32];
  __shared__ int s_gt[KPT * 16], s_eq[KPT * 16];
  __shared__ int s_pick[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = blockIdx.x;
  const int nv = (int)n_visible(p, b);
  const int K = (int)p.k;
  const float* sc = p.scores + b * p.entries;
  int32_t* oi = p.out_idx + b * K;
  float* os = p.out_score ? p.out_score + b * K : nullptr;

  if (nv <= K) {
    for (int i = tid; i < K; i += blockDim.x) {
      const bool in = i < nv;
      oi[i] = in ? (int32_t)i : -1;
      if (os) os[i] = in ? sc[i] : __builtin_nanf("");
    }
    return;
  }

  uint32_t key[KPT];
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const int i = r * 1024 + tid;
    key[r] = i < nv ? order_key(sc[i]) : 0u;
  }

  uint32_t prefix = 0, pmask = 0;
  int remaining = K;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
    const int nb = pass == 0 ? 4096 : 1024;
    for (int i = tid; i < nb; i += 1024) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const bool in = r * 1024 + tid < nv && (key[r] & pmask) == prefix;
      if (in) atomicAdd(&hist[(key[r] >> shift) & (uint32_t)(nb - 1)], 1);
    }
    __syncthreads();
    // bins from the top: thread t holds bins nb-1-t*per .. nb-per-t*per
    const int per = nb / 1024;
    int local = 0;
    for (int j = 0; j < per; ++j) local += hist[nb - 1 - tid * per - j];
    const int above = block_exclusive_scan(local, scan_buf, nullptr);
    if (above < remaining && remaining <= above + local) {
      int c = above;
      for (int j = 0; j < per; ++j) {
        const int bin = nb - 1 - tid * per - j;
        const int h = hist[bin];
        if (c + h >= remaining) {
          s_pick[0] = bin;
          s_pick[1] = remaining - c;
          break;
        }
        c += h;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_pick[0] << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    remaining = s_pick[1];
    __syncthreads();
  }
  const uint32_t thr = prefix;       // key of the k-th largest score
  const int need_eq = remaining;     // keys equal to it to take, lowest index first

  // counts above / equal to the threshold per (round, wave), scanned in index order
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
  for (int e0 = 0; e0 < KPT * 16; e0 += 1024) {  // entries in index order (round-major)
    const int e = e0 + tid;
    const bool ok = e < KPT * 16;
    int gt_tot, eq_tot;
    const int g = ok ? s_gt[e] : 0, q = ok ? s_eq[e] : 0;
    const int gp = block_exclusive_scan(g, scan_buf, &gt_tot);
    const int qp = block_exclusive_scan(q, scan_buf, &eq_tot);
    if (ok) {
      s_gt[e] = gp + (e0 > 0 ? hist[0] : 0);
      s_eq[e] = qp + (e0 > 0 ? hist[1] : 0);
    }
    __syncthreads();
    if (tid == 0) {  // running totals for the next 1024 entries
      hist[0] = (e0 > 0 ? hist[0] : 0) + gt_tot;
      hist[1] = (e0 > 0 ? hist[1] : 0) + eq_tot;
    }
    __syncthreads();
  }
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
      oi[slot] = (int32_t)i;
      if (os) os[slot] = sc[i];
    }
  }
}

size_t index_workspace_bytes(const csa_index_args& a) {
  return (size_t)a.batch * (size_t)a.entries * sizeof(float);
}

hipError_t launch_index_topk(const csa_index_args& a, void* ws, hipStream_t stream) {
  IndexParams p{};
  p.q = static_cast<const bf16_t*>(a.q_idx);
  p.w = a.head_w;
  p.keys = static_cast<const bf16_t*>(a.keys);
  p.pos = a.pos;
  p.out_idx = a.out_idx;
  p.out_score = a.out_score;
  p.scores = static_cast<float*>(ws);
  p.heads = a.heads; p.entries = a.entries; p.k = a.k; p.m = a.block;
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
  const dim3 g((unsigned)a.batch);
  if (a.entries <= 4096) topk_kernel<4><<<g, 1024, 0, stream>>>(p);
  else if (a.entries <= 16384) topk_kernel<16><<<g, 1024, 0, stream>>>(p);
  else if (a.entries <= 32768) topk_kernel<32><<<g, 1024, 0, stream>>>(p);
  else topk_kernel<64><<<g, 1024, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace lbca
