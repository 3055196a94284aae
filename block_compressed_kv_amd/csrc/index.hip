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
// order-preserving 32-bit image of the fp32 scores finds the k-th largest key,
// then a block-wide scan in index order takes every larger score and the
// lowest-index ties, writing the chosen ids in ascending order.
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

__global__ __launch_bounds__(1024) void topk_kernel(IndexParams p) {
  __shared__ int hist[256];
  __shared__ int scan_buf[32];
  __shared__ uint32_t s_prefix, s_remaining;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t nv = n_visible(p, b);
  const int64_t K = p.k;
  const float* sc = p.scores + b * p.entries;
  int32_t* oi = p.out_idx + b * K;
  float* os = p.out_score ? p.out_score + b * K : nullptr;

  if (nv <= K) {
    for (int64_t i = tid; i < K; i += blockDim.x) {
      const bool in = i < nv;
      oi[i] = in ? (int32_t)i : -1;
      if (os) os[i] = in ? sc[i] : __builtin_nanf("");
    }
    return;
  }

  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int64_t i = tid; i < nv; i += blockDim.x) {
      const uint32_t key = order_key(sc[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t above = 0;
      int d = 255;
      for (; d > 0; --d) {
        const uint32_t h = (uint32_t)hist[d];
        if (above + h >= remaining) break;
        above += h;
      }
      s_prefix = prefix | ((uint32_t)d << shift);
      s_remaining = remaining - above;
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    mask |= 0xffu << shift;
    __syncthreads();
  }
  const uint32_t thr = prefix;        // key of the k-th largest score
  const int need_eq = (int)remaining; // ties at thr to take, lowest index first

  const int64_t chunk = (nv + blockDim.x - 1) / blockDim.x;
  const int64_t c0 = tid * chunk;
  const int64_t c1 = c0 + chunk < nv ? c0 + chunk : nv;
  int n_gt = 0, n_eq = 0;
  for (int64_t i = c0; i < c1; ++i) {
    const uint32_t key = order_key(sc[i]);
    n_gt += key > thr;
    n_eq += key == thr;
  }
  const int eq_off = block_exclusive_scan(n_eq, scan_buf, nullptr);
  int take_eq = need_eq - eq_off;
  take_eq = take_eq < 0 ? 0 : (take_eq > n_eq ? n_eq : take_eq);
  int out = block_exclusive_scan(n_gt + take_eq, scan_buf, nullptr);
  int eq_seen = 0;
  for (int64_t i = c0; i < c1; ++i) {
    const float f = sc[i];
    const uint32_t key = order_key(f);
    bool pick = key > thr;
    if (key == thr) {
      pick = eq_seen < take_eq;
      ++eq_seen;
    }
    if (pick) {
      oi[out] = (int32_t)i;
      if (os) os[out] = f;
      ++out;
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
  topk_kernel<<<dim3((unsigned)a.batch), 1024, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace lbca
