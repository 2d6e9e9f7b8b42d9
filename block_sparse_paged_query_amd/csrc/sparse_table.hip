// Page-16 sparse block table and prefill token positions.
//
// [SPA] vllm.models.minimax_m3.amd.ops.sparse_pa:
//   _write_sparse_block_table_row_from_values (the per-row compaction),
//   minimax_m3_build_sparse_block_table_decode / _prefill (one row per query
//   token, decode rows right-aligned, prefill rows by request id and position).
// [NV4] vllm.models.minimax_m3.amd.sparse_attention_nvfp4,
//   MiniMaxM3SparseRocmNvfp4MetadataBuilder.build (per-token request id and
//   absolute position of prefill tokens).
//
// One wave per query row; the row's slot list is compacted into LDS with a
// ballot per 64 ids, then the row is written as 16-byte stores of 4 page ids.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

__global__ __launch_bounds__(256) void sparse_table_kernel(const TableArgs a) {
  __shared__ int lists[4][kMaxTopK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= a.total_q) return;  // whole wave leaves; no workgroup barrier below
  int req, abs_pos;
  if (a.query_req_id != nullptr) {
    req = a.query_req_id[row];
    abs_pos = a.query_abs_pos[row];
    if (req < 0 || req >= a.num_reqs) {
      req = 0;
      abs_pos = -1;
    }
  } else {
    decode_row_position(a.seq_lens, a.dql, row, &req, &abs_pos);
  }
  const RowSlots rs = compact_row(a.topk + (int64_t)row * a.topk_stride, a.topk_k,
                                  a.block_table + (int64_t)req * a.bt_stride, a.bt_cols, abs_pos, lists[wave]);
  // lanes read entries other lanes wrote: LDS requests of one wave complete in order
  __builtin_amdgcn_wave_barrier();
  int32_t* dst = a.sparse_bt + (int64_t)row * a.sbt_stride;
  const int width = a.topk_k * kPagesPerBlock;
  const bool vec_ok = (a.sbt_stride % 4) == 0 && ((uintptr_t)a.sparse_bt % 16) == 0;
  if (vec_ok) {
    // lane writes 4 consecutive entries: half a slot
    for (int e = lane * 4; e < width; e += 256) {
      const int slot = e >> 3, j = e & 7;
      int4 v;
      if (slot < rs.n_slots) {
        const int base = lists[wave][slot] * a.block_page_stride + j;
        v = make_int4(base, base + 1, base + 2, base + 3);
      } else {
        v = make_int4(0, 0, 0, 0);
      }
      *reinterpret_cast<int4*>(dst + e) = v;
    }
  } else {
    for (int e = lane; e < width; e += 64) {
      const int slot = e >> 3;
      dst[e] = slot < rs.n_slots ? lists[wave][slot] * a.block_page_stride + (e & 7) : 0;
    }
  }
  if (lane == 0) a.sparse_ctx[row] = rs.ctx;
}

hipError_t launch_sparse_table(const TableArgs& a, hipStream_t stream) {
  const int blocks = (a.total_q + 3) / 4;
  log_launch("sparse_table_kernel: %d rows, top-k %d, %d workgroups of 4 waves", a.total_q, a.topk_k, blocks);
  hipLaunchKernelGGL(sparse_table_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void query_positions_kernel(const int32_t* __restrict__ cu,
                                                              const int32_t* __restrict__ context_lens, int num_reqs,
                                                              int total_q, int32_t* req_id, int32_t* abs_pos) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= total_q) return;
  if (t >= cu[num_reqs] || t < cu[0]) {
    req_id[t] = 0;
    abs_pos[t] = -1;
    return;
  }
  int lo = 0, hi = num_reqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  req_id[t] = lo;
  abs_pos[t] = context_lens[lo] + (t - cu[lo]);
}

hipError_t launch_query_positions(const int32_t* cu, const int32_t* context_lens, int num_reqs, int total_q,
                                  int32_t* req_id, int32_t* abs_pos, hipStream_t stream) {
  log_launch("query_positions_kernel: %d rows, %d requests", total_q, num_reqs);
  hipLaunchKernelGGL(query_positions_kernel, dim3((total_q + 255) / 256), dim3(256), 0, stream, cu, context_lens,
                     num_reqs, total_q, req_id, abs_pos);
  return hipGetLastError();
}

}  // namespace msa
