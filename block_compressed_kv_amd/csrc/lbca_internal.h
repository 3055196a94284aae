// Internal launcher declarations of liblbca (host side).
#pragma once
#include <hip/hip_runtime.h>

#include <initializer_list>

#include "lbca.h"

namespace lbca {

// Element strides of one tensor argument as the kernels hold them,
// outermost dimension first: the outermost (sequence) stride in 64 bits, the
// other two in 32 (the entry points reject inner strides of 2^31 elements or
// more), which keeps the kernels' scalar registers free.
struct Str {
  int64_t s0;
  int32_t s1, s2;
  Str() = default;
  Str(const lbca_strides& a) : s0(a.s[0]), s1((int32_t)a.s[1]), s2((int32_t)a.s[2]) {}
  __host__ __device__ constexpr Str(int64_t a, int64_t b, int64_t c) : s0(a), s1((int32_t)b), s2((int32_t)c) {}
};

// Whether the strides of a tensor with outer extents ext (outermost first) and
// feature dim d are the dense row-major ones (dimensions of extent 1 aside,
// whose strides are never used).  An absent tensor counts as dense.
inline bool dense_strides(const void* ptr, const lbca_strides& st, std::initializer_list<int64_t> ext, int64_t d) {
  if (!ptr) return true;
  const int n = (int)ext.size();
  const int64_t* e = ext.begin();
  int64_t s = d;
  for (int i = n - 1; i >= 0; --i) {
    if (e[i] > 1 && st.s[i] != s) return false;
    s *= e[i] > 0 ? e[i] : 1;
  }
  return true;
}

// Host validation has already run when these are called; they only pick the
// kernel instance and launch it on `stream`.
hipError_t launch_pool(const lbca_pool_args& a, hipStream_t stream);
hipError_t launch_cache_append(const lbca_cache_args& a, hipStream_t stream);
size_t pool_grad_workspace_bytes(const lbca_pool_grad_args& a);
hipError_t launch_pool_grad(const lbca_pool_grad_args& a, void* ws, hipStream_t stream);

struct DecodePlan {
  int tile_rows;     // rows per wave tile
  int head_groups;   // ceil(G / 16): 16-head groups per KV head (MFMA path)
  int splits;        // workgroups along the row list of one (sequence, KV head, head group)
  int dim_splits;    // twin workgroups per (unit, split), each owning 1/dim_splits of the dims
  int wide_blocks;   // > 0: wide-row MQA kernel with this many 32-head blocks per workgroup
  int wide_twins;    // wide-row workgroups per (sequence, KV head, split)
  size_t ws_bytes;   // split partials (acc, max, sum); 0 with one split
  int unsupported;   // 1: no launch shape covers these sizes (too many selected ids)
};
DecodePlan plan_decode(const lbca_decode_args& a);
// qrows > 1 (wide-row path only): rows b of the call are queries of a chunk,
// and consecutive groups of qrows rows read cache sequence b / qrows
hipError_t launch_decode(const lbca_decode_args& a, const DecodePlan& plan, void* ws,
                         hipStream_t stream, int qrows = 1);

// Address of the calling thread's current device's copy of the static decode
// scratch (LBCA_NOALLOC_SCRATCH_BYTES), looked up once per device.
hipError_t static_scratch(void** ptr);
hipError_t launch_decode_step(const lbca_decode_args& da, const lbca_cache_args& ca, const DecodePlan& plan,
                              void* ws, hipStream_t stream);

hipError_t launch_prefill(const lbca_prefill_args& a, hipStream_t stream);
hipError_t launch_prefill_f32(const lbca_prefill_args& a, hipStream_t stream);
size_t prefill_grad_workspace_bytes(const lbca_prefill_grad_args& a);
hipError_t launch_prefill_grad(const lbca_prefill_grad_args& a, void* workspace, hipStream_t stream);
hipError_t launch_decode_f32(const lbca_decode_args& a, hipStream_t stream);

hipError_t launch_gemm(const lbca_gemm_args& a, hipStream_t stream);

size_t index_workspace_bytes(const csa_index_args& a);
hipError_t launch_index_topk(const csa_index_args& a, void* ws, hipStream_t stream);
// Query chunk: a.batch = sequences * q_len rows (q_idx [rows, heads, dim],
// head_w [rows, heads], out_idx [rows, k]); keys [sequences, entries, dim];
// row r sits at q_pos0 + r % q_len.  Writes the rows' positions to pos_ws and
// raw_pos_base to rpb_ws (rows int64 each), then scores and selects.
hipError_t launch_index_topk_chunk(const csa_index_args& a, int64_t q_len, int64_t q_pos0, int64_t raw_pos_base,
                                   int64_t* pos_ws, int64_t* rpb_ws, void* ws, hipStream_t stream);

}  // namespace lbca
