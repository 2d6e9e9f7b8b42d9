// Internal launch interfaces between the C ABI (msa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// Launch log: while the environment variable MSA_LOG is set to a value other
// than "0" (read at each launch), every kernel launch writes one line to
// stderr with the kernel and its launch shape.
void log_launch(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

// Arguments of the attends (decode rows, prefill query tiles).
struct AttendArgs {
  const void* q;
  void* out;
  const int32_t* topk;
  int64_t topk_stride;
  int32_t topk_k;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t bt_cols;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_q;
  int32_t dql;
  int32_t num_reqs;
  // Cache geometry, in units of sub_stride bytes (one 16-token page of one
  // layer).  Token t (0..15) of the j-th 16-token page (j < 8) of sparse
  // block `phys`, kv head h, starts at
  //   k_base + (phys * blk_units + j) * sub_stride + h * head_stride + t * row_stride
  // (NVFP4: the K slot of head h, token rows inside the slot as the format
  // gives them); V at the same offsets from v_base, which has the V page
  // offset, the V slot or the in-row offset of V folded in.  A block's
  // pages are inside the cache when phys * blk_units + v_unit_offset + 7 <
  // num_units.
  const uint8_t* k_base;
  const uint8_t* v_base;
  int32_t blk_units;
  int32_t head_stride;
  int64_t sub_stride;
  int32_t row_stride;
  int64_t num_units;
  int32_t v_unit_offset;
  const float* k_scale;
  const float* v_scale;
  float softmax_scale;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t head_dim;
  int32_t nsplit;
  int32_t total_rows;
  float* ws_o;    // [rows][Hq][nsplit][D]
  float* ws_ml;   // [rows][Hq][nsplit][2]
  int32_t num_cus;   // compute units of the device (launch shaping)
  // Prefill at 4-8 query heads per kv head: device workspace of perm_cap x
  // 32 bytes for the row order of each query tile (QT bytes a tile), or NULL
  // to keep the natural order.
  int8_t* row_perm;
  int32_t perm_cap;
};

hipError_t launch_attend_decode(const AttendArgs& a, int fmt, int rows, hipStream_t stream);

// Matrix-core prefill over query tiles: bf16, fp8 or NVFP4 pages; head_dim
// 128 (or 64 for bf16 and fp8); 1 to 16 query heads per kv head (every shape
// the C ABI accepts).
hipError_t launch_prefill_blocks(const AttendArgs& a, int fmt, hipStream_t stream);

struct TableArgs {
  const int32_t* topk;
  int64_t topk_stride;
  int32_t topk_k;
  int32_t total_q;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t bt_cols;
  int32_t num_reqs;
  const int32_t* seq_lens;
  int32_t dql;
  const int32_t* query_req_id;
  const int32_t* query_abs_pos;
  int32_t block_page_stride;
  int32_t* sparse_bt;
  int64_t sbt_stride;
  int32_t* sparse_ctx;
};

hipError_t launch_sparse_table(const TableArgs& a, hipStream_t stream);

hipError_t launch_query_positions(const int32_t* cu, const int32_t* context_lens, int num_reqs, int total_q,
                                  int32_t* req_id, int32_t* abs_pos, hipStream_t stream);

hipError_t launch_index_insert(const void* k, int64_t ks0, int64_t ks1, int n, int d, int esize, void* cache,
                               int64_t cs0, int64_t cs1, int num_blocks, int block_size, const int64_t* slots,
                               int64_t slot_stride, hipStream_t stream);

// Test hook: each row's K / V in sparse-table order through the decode
// attend's gather (launch_gather_dequant_decode) or the prefill attend's
// staged copy (launch_gather_dequant_prefill); head_dim 128, or 64 for bf16
// and fp8 pages.
hipError_t launch_gather_dequant_decode(const AttendArgs& a, int fmt, const int32_t* sbt, int64_t sbt_stride,
                                        const int32_t* sctx, int bps, int rows, int width_tokens, float* k_out,
                                        float* v_out, hipStream_t stream);
hipError_t launch_gather_dequant_prefill(const AttendArgs& a, int fmt, const int32_t* sbt, int64_t sbt_stride,
                                         const int32_t* sctx, int bps, int rows, int width_tokens, float* k_out,
                                         float* v_out, hipStream_t stream);

}  // namespace msa
