// Probes of this part's measured ceilings, reported beside the kernels'
// roofline fractions: a streaming HBM read, a streaming copy (read and
// write), LDS read bandwidth, a bf16 MFMA loop and an empty kernel (the
// launch floor).  Built into libceilings.so, a library of its own
// that only the benchmark loads; nothing here is part of the attention path.
//
// Each entry point checks its sizes and returns a hipError_t value (0 = success).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Grid-stride read of n16 16-byte vectors, eight loads in flight per thread;
// each thread writes the xor of what it read (so no load can be dropped).
__global__ __launch_bounds__(256) void read_kernel(const u32x4_t* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Grid-stride copy of n16 16-byte vectors, eight loads in flight per thread
// before their stores.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                   int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) __builtin_nontemporal_store(v[j], dst + i + j * stride);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// LDS read bandwidth: 256 threads fill 64 KB of LDS from src, then each
// thread reads 16 bytes per step at a lane-contiguous address (the 64 lanes of
// a wave cover 1 KB, free of bank conflicts), eight reads in flight, for
// `iters` steps; every thread writes the xor of what it read.
__global__ __launch_bounds__(256) void lds_kernel(const u32x4_t* __restrict__ src, uint32_t* __restrict__ out,
                                                  int iters) {
  __shared__ u32x4_t buf[4096];  // 64 KB
  for (int i = threadIdx.x; i < 4096; i += 256) buf[i] = src[i];
  __syncthreads();
  uint32_t acc = 0;
  int idx = threadIdx.x;
  for (int it = 0; it < iters; ++it) {
    u32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = buf[(idx + j * 512) & 4095];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    idx = (idx + 256 + (int)(acc & 1u) * 64) & 4095;  // the next addresses depend on the data read
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Four independent chains of v_mfma_f32_32x32x16_bf16 per wave (32768 flops
// each); every thread writes one sum of its accumulators.
__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ out, int iters) {
  const float s = 1e-3f * (float)(threadIdx.x & 63);
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(s + 0.25f * e);
    b[e] = (__bf16)(0.5f - s);
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = c0[0] + c1[5] + c2[10] + c3[15];
}

// Eight independent chains of v_mfma_f32_16x16x32_bf16 per wave (16384 flops
// each), the instruction the attention kernels use.
__global__ __launch_bounds__(256) void mfma16_kernel(float* __restrict__ out, int iters) {
  const float s = 1e-3f * (float)(threadIdx.x & 63);
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(s + 0.25f * e);
    b[e] = (__bf16)(0.5f - s);
  }
  f32x4_t c[8] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) r += c[k][k & 3];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from src with `grid` workgroups of 256
// threads; out holds grid * 256 uint32.
__attribute__((visibility("default"))) int ceil_read(const void* src, size_t bytes, void* out, int grid,
                                                     void* stream) {
  if (!src || !out || grid < 1 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  read_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4_t*>(src),
                                                                  (int64_t)(bytes / 16),
                                                                  static_cast<uint32_t*>(out));
  return (int)hipGetLastError();
}

// Copies `bytes` (a multiple of 16) from src to dst with `grid` workgroups of 256 threads.
__attribute__((visibility("default"))) int ceil_copy(const void* src, void* dst, size_t bytes, int grid,
                                                     void* stream) {
  if (!src || !dst || grid < 1 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  copy_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4_t*>(src),
                                                                  static_cast<u32x4_t*>(dst), (int64_t)(bytes / 16));
  return (int)hipGetLastError();
}

// grid workgroups of 256 threads, each thread 8 * iters LDS reads of 16 bytes
// after copying 64 KB of src (at least 64 KB) into LDS; out holds grid * 256 uint32.
__attribute__((visibility("default"))) int ceil_lds(const void* src, void* out, int grid, int iters, void* stream) {
  if (!src || !out || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
  lds_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4_t*>(src),
                                                                 static_cast<uint32_t*>(out), iters);
  return (int)hipGetLastError();
}

// grid workgroups of 4 waves, each wave 4 * iters MFMAs of 32768 flops; out
// holds grid * 256 floats.
__attribute__((visibility("default"))) int ceil_mfma(void* out, int grid, int iters, void* stream) {
  if (!out || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
  mfma_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<float*>(out), iters);
  return (int)hipGetLastError();
}

// grid workgroups of 4 waves, each wave 8 * iters MFMAs of 16384 flops; out
// holds grid * 256 floats.
__attribute__((visibility("default"))) int ceil_mfma16(void* out, int grid, int iters, void* stream) {
  if (!out || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
  mfma16_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<float*>(out), iters);
  return (int)hipGetLastError();
}

__attribute__((visibility("default"))) int ceil_empty(void* stream) {
  empty_kernel<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>();
  return (int)hipGetLastError();
}

}  // extern "C"
