// Internal launcher declarations of liblbca (host side).
#pragma once
#include <hip/hip_runtime.h>

#include "lbca.h"

namespace lbca {

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
