// Grouped projection GEMM for the projections around the attention path.
//
// Method: "CSA: Compressed Sparse Attention (toy implementation)", "What is
// implemented": low-rank indexer queries (the query latent times one matrix
// that makes every indexer head's query) and the grouped output projection
// (consecutive query heads in g groups, each group's concatenated outputs
// times its own matrix, then the concatenated group results times the output
// matrix); "HCA: Heavily Compressed Attention (toy implementation)", "What is
// implemented": the same grouped output projection.  Each is one or two calls
// of
//   C[g][i][j] = sum_l A[g][i][l] * W[g][j][l]      (fp32 accumulation)
// with weights stored [out_features, in_features] (both operands contiguous
// along the contraction).
//
// A workgroup of 4 waves owns a 128 x 128 tile of C; wave (wm, wn) owns a
// 64 x 64 quarter as 2 x 2 blocks of v_mfma_f32_32x32x16_bf16 (the faster of
// the bf16 MFMA forms on this part).  K advances in 64-wide steps: the next
// step's A and W rows are loaded into registers (buffer resources: rows past M
// or N read zeros; an fp32 A is rounded to bf16 on the way) while the current
// step's are multiplied from LDS, then stored into the other LDS buffer; one
// barrier per step.  LDS rows hold their 16-byte chunks in swizzled order so
// that each MFMA operand read (one chunk of 32 consecutive rows, 16 lanes per
// pass) hits distinct banks.  Two workgroups fit on a CU (64 KB of LDS each).
#include <type_traits>
#include "device_util.h"
#include "lbca_internal.h"

namespace lbca {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;

struct GemmParams {
  const void* a;
  const bf16_t* w;
  void* c;
  int64_t m, n, k, lda, ldw, ldc, a_gs, w_gs, c_gs;
  int a_f32, c_f32;
  int c_vec;  // C rows and groups start on 16-byte (fp32) / 8-byte (bf16) boundaries
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ldb(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0));
}
// position of chunk x of LDS row r: a 128-byte row spans half the banks, so
// rows of one parity share a bank half; a 16-byte read serves 16 lanes per
// pass, 16 consecutive rows, so the xor spreads the 8 rows of each parity over
// all 8 chunk slots
__device__ __forceinline__ int gswz(int r, int x) { return x ^ ((r >> 1) & 7); }

template <bool AF32, bool CF32>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t sa[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sw[2][BN * BK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int n32 = lane & 31, h = lane >> 5;
  const int g = blockIdx.z;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int ka = p.a_f32 ? 4 : 2;  // bytes per A element

  // this group's A rows [m0, m0 + BM) and W rows [n0, n0 + BN) as buffer
  // resources limited to the last valid row
  const char* abase = static_cast<const char*>(p.a) + (g * p.a_gs + m0 * p.lda) * ka;
  const char* wbase = reinterpret_cast<const char*>(p.w + g * p.w_gs + n0 * p.ldw);
  const int64_t arows = p.m - m0 < BM ? p.m - m0 : BM, wrows = p.n - n0 < BN ? p.n - n0 : BN;
  const __amdgpu_buffer_rsrc_t ra = rsrc(abase, ((arows - 1) * p.lda + p.k) * ka);
  const __amdgpu_buffer_rsrc_t rw = rsrc(wbase, ((wrows - 1) * p.ldw + p.k) * 2);

  // staging: each thread moves 4 A chunks and 4 W chunks (8 bf16 each) per step;
  // chunk s of this thread: tile row (tid / 8) + 32 s, chunk tid % 8
  const int st_x = tid & 7, st_r = tid >> 3;
  // bf16 A: the chunks are stored to the LDS as loaded; a chunk past K is
  // zeroed in a branch that only the tail step takes.
  uint4 stg_a[4], stg_w[4];
  auto fetch16 = [&](int64_t k0) __attribute__((always_inline)) {
    const bool tail = k0 + BK > p.k;
    const bool live = !tail || k0 + 8 * st_x < p.k;  // K is a multiple of 8
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = st_r + 32 * s;
      stg_a[s] = ldb(ra, (uint32_t)(((int64_t)r * p.lda + k0 + 8 * st_x) * 2), 0);
      stg_w[s] = ldb(rw, (uint32_t)(((int64_t)r * p.ldw + k0 + 8 * st_x) * 2), 0);
      if (!live) {
        stg_a[s] = make_uint4(0, 0, 0, 0);
        stg_w[s] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto stash16 = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = st_r + 32 * s;
      *reinterpret_cast<uint4*>(&sa[buf][r * BK + 8 * gswz(r, st_x)]) = stg_a[s];
      *reinterpret_cast<uint4*>(&sw[buf][r * BK + 8 * gswz(r, st_x)]) = stg_w[s];
    }
  };
  // fp32 A: the loaded words are kept until the stash, which rounds them to
  // bf16 and, on the one step that runs past K (a uniform branch), zeroes the
  // chunks beyond K, so every load of the next step stays in flight while this
  // step's MFMAs run (rounding right after the load would wait for it there).
  uint4 f32_lo[4], f32_hi[4], f32_w[4];
  bool f32_tail = false;
  uint32_t f32_keep = ~0u;  // all ones, or zero for a chunk past K
  auto fetch32 = [&](int64_t k0) __attribute__((always_inline)) {
    f32_tail = k0 + BK > p.k;
    f32_keep = k0 + 8 * st_x < p.k ? ~0u : 0u;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = st_r + 32 * s;
      const uint32_t off = (uint32_t)(((int64_t)r * p.lda + k0 + 8 * st_x) * 4);
      f32_lo[s] = ldb(ra, off, 0);
      f32_hi[s] = ldb(ra, off + 16, 0);
      f32_w[s] = ldb(rw, (uint32_t)(((int64_t)r * p.ldw + k0 + 8 * st_x) * 2), 0);
    }
  };
  auto stash32_as = [&](int buf, uint32_t m, auto masked) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = st_r + 32 * s;
      const uint4 lo = f32_lo[s], hi = f32_hi[s];
      uint4 a = make_uint4(pack_bf16x2(__uint_as_float(lo.x), __uint_as_float(lo.y)),
                           pack_bf16x2(__uint_as_float(lo.z), __uint_as_float(lo.w)),
                           pack_bf16x2(__uint_as_float(hi.x), __uint_as_float(hi.y)),
                           pack_bf16x2(__uint_as_float(hi.z), __uint_as_float(hi.w)));
      uint4 w = f32_w[s];
      if constexpr (decltype(masked)::value) {
        a = make_uint4(a.x & m, a.y & m, a.z & m, a.w & m);
        w = make_uint4(w.x & m, w.y & m, w.z & m, w.w & m);
      }
      *reinterpret_cast<uint4*>(&sa[buf][r * BK + 8 * gswz(r, st_x)]) = a;
      *reinterpret_cast<uint4*>(&sw[buf][r * BK + 8 * gswz(r, st_x)]) = w;
    }
  };
  auto fetch = [&](int64_t k0) __attribute__((always_inline)) {
    if constexpr (AF32)
      fetch32(k0);
    else
      fetch16(k0);
  };
  auto stash = [&](int buf) __attribute__((always_inline)) {
    if constexpr (AF32) {
      if (f32_tail)
        stash32_as(buf, f32_keep, std::true_type{});
      else
        stash32_as(buf, ~0u, std::false_type{});
    } else {
      stash16(buf);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // one 64-wide step from LDS buffer buf: for each 16-wide k slice kk, the A
  // operand of block row i is (row 64 wm + 32 i + n32, k 16 kk + 8 h ..), the W
  // operand of block column j is (row 64 wn + 32 j + n32, same k)
  auto mma = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      uint4 fa[2], fw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra_ = 64 * wm + 32 * i + n32, rw_ = 64 * wn + 32 * i + n32;
        fa[i] = *reinterpret_cast<const uint4*>(&sa[buf][ra_ * BK + 8 * gswz(ra_, 2 * kk + h)]);
        fw[i] = *reinterpret_cast<const uint4*>(&sw[buf][rw_ * BK + 8 * gswz(rw_, 2 * kk + h)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fw[j]),
                                                              __builtin_bit_cast(bf16x8, fa[i]), acc[i][j], 0, 0, 0);
    }
  };

  const int64_t steps = (p.k + BK - 1) / BK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int64_t s = 0; s < steps; ++s) {
    const int buf = (int)(s & 1);
    if (s + 1 < steps) fetch((s + 1) * BK);
    mma(buf);
    if (s + 1 < steps) stash(buf ^ 1);
    __syncthreads();
  }

  // acc[i][j] is C^T of the 32 x 32 block (MFMA A = W rows, B = A rows): lane
  // (n32, h) holds C row 64 wm + 32 i + n32, columns 64 wn + 32 j + 8 q + 4 h + r
  // for element 4 q + r
  const int64_t row = m0 + 64 * wm + n32;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t r = row + 32 * i;
    if (r >= p.m) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n0 + 64 * wn + 32 * j + 8 * q + 4 * h;
        const int64_t o = g * p.c_gs + r * p.ldc + col;
        const f32x16& v = acc[i][j];
        if (p.c_vec && col + 3 < p.n) {
          if constexpr (CF32) {
            *reinterpret_cast<float4*>(static_cast<float*>(p.c) + o) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
          } else {
            uint2 w2;
            w2.x = pack_bf16x2(v[4 * q], v[4 * q + 1]);
            w2.y = pack_bf16x2(v[4 * q + 2], v[4 * q + 3]);
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(p.c) + o) = w2;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (col + e >= p.n) break;
            if constexpr (CF32) static_cast<float*>(p.c)[o + e] = v[4 * q + e];
            else {
              const uint32_t w1 = pack_bf16x2(v[4 * q + e], 0.f);
              static_cast<uint16_t*>(p.c)[o + e] = (uint16_t)(w1 & 0xffffu);
            }
          }
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm(const lbca_gemm_args& a, hipStream_t stream) {
  GemmParams p{};
  p.a = a.a;
  p.w = static_cast<const bf16_t*>(a.w);
  p.c = a.c;
  p.m = a.m; p.n = a.n; p.k = a.k;
  p.lda = a.lda; p.ldw = a.ldw; p.ldc = a.ldc;
  p.a_gs = a.a_group_stride; p.w_gs = a.w_group_stride; p.c_gs = a.c_group_stride;
  p.a_f32 = a.a_dtype == LBCA_F32;
  p.c_f32 = a.c_dtype == LBCA_F32;
  p.c_vec = a.ldc % 4 == 0 && a.c_group_stride % 4 == 0;
  const dim3 grid((unsigned)((a.n + BN - 1) / BN), (unsigned)((a.m + BM - 1) / BM), (unsigned)a.groups);
  if (p.a_f32) {
    if (p.c_f32) gemm_kernel<true, true><<<grid, 256, 0, stream>>>(p);
    else gemm_kernel<true, false><<<grid, 256, 0, stream>>>(p);
  } else {
    if (p.c_f32) gemm_kernel<false, true><<<grid, 256, 0, stream>>>(p);
    else gemm_kernel<false, false><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace lbca
