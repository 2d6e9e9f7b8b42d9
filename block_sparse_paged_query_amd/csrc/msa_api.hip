// C ABI of libmsa: argument validation (before any HIP call), workspace and
// split selection, and launches on the caller's stream.  Declarations and the
// contract of every entry point are in include/msa.h.
#include <stdio.h>
#include <stdarg.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/msa.h"
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

void log_launch(const char* fmt, ...) {
  const char* v = getenv("MSA_LOG");
  if (v == nullptr || v[0] == 0 || strcmp(v, "0") == 0) return;
  char line[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof(line), fmt, ap);
  va_end(ap);
  fprintf(stderr, "[msa] %s\n", line);
}

}  // namespace msa

namespace {

thread_local char g_last_error[512] = "";

msa_status_t fail(msa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

msa_status_t ok() {
  g_last_error[0] = 0;
  return MSA_OK;
}

msa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MSA_CHECK(cond, st, ...) \
  do {                           \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

int fmt_of(int32_t kv_dtype) {
  switch (kv_dtype) {
    case MSA_BF16: return msa::kFmtBf16;
    case MSA_FP8_E4M3FN: return msa::kFmtFp8;
    case MSA_NVFP4: return msa::kFmtNvfp4;
    default: return -1;
  }
}

// Layout-dependent checks of a cache descriptor (the attends and the hook).
msa_status_t check_kv_geometry(const msa_kv_cache_t* kv) {
  const int esz = kv->kv_dtype == MSA_BF16 ? 2 : 1;
  int64_t page_min = 0;
  if (kv->kv_layout == MSA_KV_PAGE16) {
    MSA_CHECK(kv->block_page_stride == 8 || kv->block_page_stride == 16, MSA_ERR_INVALID_ARGUMENT,
              "block_page_stride %d: 8 (separate K/V planes) or 16 (both sides in a block)", kv->block_page_stride);
    page_min = kv->kv_dtype == MSA_NVFP4 ? (int64_t)2 * kv->num_kv_heads * 9 * kv->head_dim
                                         : (int64_t)kv->num_kv_heads * 16 * kv->head_dim * esz;
  } else if (kv->kv_layout == MSA_KV_ROWS128) {
    MSA_CHECK(kv->kv_dtype != MSA_NVFP4, MSA_ERR_UNSUPPORTED, "K|V-interleaved 128-token pages hold bf16 or fp8");
    MSA_CHECK(kv->block_page_stride == 8, MSA_ERR_INVALID_ARGUMENT,
              "block_page_stride %d: 128-token pages need 8 (one page per block)", kv->block_page_stride);
    MSA_CHECK(kv->v_pages == nullptr ||
                  kv->v_pages == static_cast<const uint8_t*>(kv->k_pages) + (int64_t)kv->head_dim * esz,
              MSA_ERR_INVALID_ARGUMENT, "v_pages must be NULL or k_pages + head_dim elements");
    page_min = (int64_t)kv->num_kv_heads * msa::kBlockTokens * 2 * kv->head_dim * esz;
    const int64_t sub = (int64_t)msa::kPageTokens * 2 * kv->head_dim * esz;
    MSA_CHECK(kv->page_stride_bytes % sub == 0, MSA_ERR_INVALID_ARGUMENT,
              "page stride %lld bytes: 128-token pages need a multiple of 16 rows (%lld bytes)",
              (long long)kv->page_stride_bytes, (long long)sub);
    MSA_CHECK(kv->page_stride_bytes / sub <= INT32_MAX, MSA_ERR_INVALID_ARGUMENT, "page stride %lld bytes too large",
              (long long)kv->page_stride_bytes);
    MSA_CHECK(kv->page_stride_bytes <= 0 || kv->num_pages <= INT64_MAX / (kv->page_stride_bytes / sub),
              MSA_ERR_INVALID_ARGUMENT, "num_pages %lld out of range", (long long)kv->num_pages);
  } else {
    return fail(MSA_ERR_INVALID_ARGUMENT, "kv_layout %d: 0 (16-token pages) or 1 (K|V-interleaved 128-token pages)",
                kv->kv_layout);
  }
  MSA_CHECK(kv->num_pages >= 0 && kv->num_pages <= (INT64_MAX >> 4), MSA_ERR_INVALID_ARGUMENT,
            "num_pages %lld out of range", (long long)kv->num_pages);
  MSA_CHECK(kv->page_stride_bytes >= page_min && kv->page_stride_bytes % 16 == 0, MSA_ERR_INVALID_ARGUMENT,
            "page stride %lld bytes: need a multiple of 16 and >= %lld", (long long)kv->page_stride_bytes,
            (long long)page_min);
  return MSA_OK;
}

// The kernels' view of a checked descriptor: base pointers and strides such
// that token t of the j-th 16-token page of block b, kv head h, starts at
// base + (b * blk_units + j) * sub + h * head + t * row; the buffer holds
// num_units units of sub bytes, V pages v_unit_offset units after K's.
struct KvGeometry {
  const uint8_t* k_base;
  const uint8_t* v_base;
  int32_t blk_units, head;
  int64_t sub;
  int32_t row;
  int64_t num_units;
  int32_t v_unit_offset;
};

KvGeometry kv_geometry(const msa_kv_cache_t* kv) {
  KvGeometry g;
  const int esz = kv->kv_dtype == MSA_BF16 ? 2 : 1;
  const uint8_t* k = static_cast<const uint8_t*>(kv->k_pages);
  const int64_t ps = kv->page_stride_bytes;
  if (kv->kv_layout == MSA_KV_ROWS128) {
    const int32_t row = 2 * kv->head_dim * esz;
    g.k_base = k;
    g.v_base = k ? k + (int64_t)kv->head_dim * esz : nullptr;
    g.sub = (int64_t)msa::kPageTokens * row;
    g.blk_units = (int32_t)(ps / g.sub);
    g.head = msa::kBlockTokens * row;
    g.row = row;
    g.num_units = kv->num_pages * g.blk_units;
    g.v_unit_offset = 0;
  } else if (kv->kv_dtype == MSA_NVFP4) {
    g.k_base = k;
    g.v_base = k ? k + 9 * kv->head_dim : nullptr;
    g.sub = ps;
    g.blk_units = kv->block_page_stride;
    g.head = 2 * 9 * kv->head_dim;
    g.row = 0;
    g.num_units = kv->num_pages;
    g.v_unit_offset = 0;
  } else {
    const int32_t row = kv->head_dim * esz;
    g.v_unit_offset = kv->block_page_stride - msa::kPagesPerBlock;
    g.k_base = k;
    g.v_base = kv->v_pages ? static_cast<const uint8_t*>(kv->v_pages) + g.v_unit_offset * ps : nullptr;
    g.sub = ps;
    g.blk_units = kv->block_page_stride;
    g.head = msa::kPageTokens * row;
    g.row = row;
    g.num_units = kv->num_pages;
  }
  return g;
}

// Validation shared by the attends.
msa_status_t check_attend(const void* q, int32_t q_dtype, int32_t rows, int32_t num_q_heads, const msa_kv_cache_t* kv,
                          const int32_t* topk, int64_t topk_row_stride, int32_t topk_k, const int32_t* block_table,
                          int64_t bt_row_stride, int32_t bt_cols, const void* out, float softmax_scale) {
  MSA_CHECK(kv != nullptr, MSA_ERR_INVALID_ARGUMENT, "kv cache descriptor is NULL");
  MSA_CHECK(rows >= 0, MSA_ERR_INVALID_ARGUMENT, "row count %d is negative", rows);
  MSA_CHECK(q_dtype == MSA_BF16, MSA_ERR_UNSUPPORTED, "q dtype %d: only bf16 queries are served", q_dtype);
  MSA_CHECK(fmt_of(kv->kv_dtype) >= 0, MSA_ERR_UNSUPPORTED, "kv dtype %d: bf16, fp8 e4m3fn or nvfp4 pages only",
            kv->kv_dtype);
  MSA_CHECK(kv->head_dim == 64 || kv->head_dim == 128, MSA_ERR_UNSUPPORTED, "head_dim %d: 64 or 128 only",
            kv->head_dim);
  MSA_CHECK(kv->kv_dtype != MSA_NVFP4 || kv->head_dim == 128, MSA_ERR_UNSUPPORTED,
            "nvfp4 pages need head_dim 128 (got %d)", kv->head_dim);
  MSA_CHECK(kv->num_kv_heads >= 1, MSA_ERR_INVALID_ARGUMENT, "num_kv_heads %d < 1", kv->num_kv_heads);
  MSA_CHECK(num_q_heads >= 1 && num_q_heads % kv->num_kv_heads == 0, MSA_ERR_INVALID_ARGUMENT,
            "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads, kv->num_kv_heads);
  MSA_CHECK(num_q_heads / kv->num_kv_heads <= 16, MSA_ERR_UNSUPPORTED,
            "%d query heads per kv head: at most 16 are served", num_q_heads / kv->num_kv_heads);
  {
    const msa_status_t st = check_kv_geometry(kv);
    if (st != MSA_OK) return st;
  }
  MSA_CHECK(topk_k >= 1 && topk_k <= msa::kMaxTopK, MSA_ERR_UNSUPPORTED, "topk_k %d: 1..%d", topk_k, msa::kMaxTopK);
  MSA_CHECK(topk_row_stride >= topk_k, MSA_ERR_INVALID_ARGUMENT, "topk row stride %lld < topk_k %d",
            (long long)topk_row_stride, topk_k);
  MSA_CHECK(bt_cols >= 0 && bt_row_stride >= bt_cols, MSA_ERR_INVALID_ARGUMENT,
            "block_table: %d columns, row stride %lld", bt_cols, (long long)bt_row_stride);
  MSA_CHECK(softmax_scale == softmax_scale, MSA_ERR_INVALID_ARGUMENT, "softmax_scale is NaN");
  if (rows > 0) {
    MSA_CHECK(q && out && topk && block_table && kv->k_pages, MSA_ERR_INVALID_ARGUMENT,
              "q, out, topk, block_table and k_pages must be non-NULL");
    const bool v_plane = kv->kv_dtype != MSA_NVFP4 && kv->kv_layout == MSA_KV_PAGE16;
    MSA_CHECK(!v_plane || kv->v_pages, MSA_ERR_INVALID_ARGUMENT, "v_pages is NULL");
    MSA_CHECK(((uintptr_t)q % 16) == 0 && ((uintptr_t)out % 16) == 0 && ((uintptr_t)kv->k_pages % 16) == 0 &&
                  (!v_plane || ((uintptr_t)kv->v_pages % 16) == 0),
              MSA_ERR_INVALID_ARGUMENT, "q, out and page buffers must be 16-byte aligned");
  }
  return MSA_OK;
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

msa::AttendArgs attend_args(const void* q, int32_t num_q_heads, const msa_kv_cache_t* kv, const int32_t* topk,
                            int64_t topk_row_stride, int32_t topk_k, const int32_t* block_table, int64_t bt_row_stride,
                            int32_t bt_cols, float softmax_scale, void* out) {
  msa::AttendArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.out = out;
  a.topk = topk;
  a.topk_stride = topk_row_stride;
  a.topk_k = topk_k;
  a.block_table = block_table;
  a.bt_stride = bt_row_stride;
  a.bt_cols = bt_cols;
  const KvGeometry g = kv_geometry(kv);
  a.k_base = g.k_base;
  a.v_base = g.v_base;
  a.blk_units = g.blk_units;
  a.sub_stride = g.sub;
  a.head_stride = g.head;
  a.row_stride = g.row;
  a.num_units = g.num_units;
  a.v_unit_offset = g.v_unit_offset;
  a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale;
  a.softmax_scale = softmax_scale;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = kv->num_kv_heads;
  a.group = num_q_heads / kv->num_kv_heads;
  a.head_dim = kv->head_dim;
  a.nsplit = 1;
  a.num_cus = device_cus();
  return a;
}

size_t split_bytes(int64_t rows, int32_t num_q_heads, int32_t head_dim, int32_t nsplit) {
  return (size_t)(rows * num_q_heads * nsplit) * (size_t)(head_dim + 2) * sizeof(float) + 256;
}


// Splits per (row, kv head): enough workgroups for two per compute unit, each
// split keeping at least one 128-token block per wave.
int choose_splits(int64_t rows, int32_t num_kv_heads, int32_t topk_k, int cus) {
  const int64_t units = rows * num_kv_heads;
  if (units <= 0) return 1;
  int64_t ns = (2 * (int64_t)cus + units - 1) / units;
  const int64_t max_ns = topk_k > 1 ? topk_k : 1;   // 4 chunks per block, 4 waves per split
  if (ns > max_ns) ns = max_ns;
  if (ns > 64) ns = 64;
  return ns < 1 ? 1 : (int)ns;
}

}  // namespace

extern "C" {

MSA_API const char* msa_last_error(void) { return g_last_error; }

MSA_API msa_status_t msa_build_sparse_block_table(const int32_t* topk, int64_t topk_row_stride, int32_t topk_k,
                                                  int32_t total_q, const int32_t* block_table, int64_t bt_row_stride,
                                                  int32_t bt_cols, int32_t num_reqs, const int32_t* seq_lens,
                                                  int32_t decode_query_len, const int32_t* query_req_id,
                                                  const int32_t* query_abs_pos, int32_t block_page_stride,
                                                  int32_t* sparse_bt, int64_t sbt_row_stride, int32_t* sparse_ctx,
                                                  hipStream_t stream) {
  MSA_CHECK(total_q >= 0 && num_reqs >= 0, MSA_ERR_INVALID_ARGUMENT, "negative total_q %d or num_reqs %d", total_q,
            num_reqs);
  MSA_CHECK(topk_k >= 1 && topk_k <= msa::kMaxTopK, MSA_ERR_UNSUPPORTED, "topk_k %d: 1..%d", topk_k, msa::kMaxTopK);
  MSA_CHECK(topk_row_stride >= topk_k, MSA_ERR_INVALID_ARGUMENT, "topk row stride %lld < topk_k %d",
            (long long)topk_row_stride, topk_k);
  MSA_CHECK(bt_cols >= 0 && bt_row_stride >= bt_cols, MSA_ERR_INVALID_ARGUMENT,
            "block_table: %d columns, row stride %lld", bt_cols, (long long)bt_row_stride);
  MSA_CHECK(block_page_stride >= 1, MSA_ERR_INVALID_ARGUMENT, "block_page_stride %d < 1", block_page_stride);
  MSA_CHECK(sbt_row_stride >= (int64_t)topk_k * msa::kPagesPerBlock, MSA_ERR_INVALID_ARGUMENT,
            "sparse_bt row stride %lld < 8 * topk_k", (long long)sbt_row_stride);
  MSA_CHECK((query_req_id == nullptr) == (query_abs_pos == nullptr), MSA_ERR_INVALID_ARGUMENT,
            "prefill mode needs both query_req_id and query_abs_pos");
  if (query_req_id == nullptr) {
    MSA_CHECK(decode_query_len >= 1, MSA_ERR_INVALID_ARGUMENT, "decode_query_len %d < 1", decode_query_len);
    MSA_CHECK((int64_t)total_q == (int64_t)num_reqs * decode_query_len, MSA_ERR_INVALID_ARGUMENT,
              "decode mode: %d top-k rows for %d requests of %d tokens each", total_q, num_reqs,
              decode_query_len);
  }
  if (total_q == 0) return ok();
  MSA_CHECK(topk && sparse_bt && sparse_ctx && (block_table || bt_cols == 0), MSA_ERR_INVALID_ARGUMENT,
            "topk, block_table, sparse_bt and sparse_ctx must be non-NULL");
  MSA_CHECK(query_req_id != nullptr || seq_lens != nullptr, MSA_ERR_INVALID_ARGUMENT, "decode mode needs seq_lens");
  MSA_CHECK(num_reqs >= 1, MSA_ERR_INVALID_ARGUMENT, "rows without requests");
  msa::TableArgs a;
  a.topk = topk;
  a.topk_stride = topk_row_stride;
  a.topk_k = topk_k;
  a.total_q = total_q;
  a.block_table = block_table;
  a.bt_stride = bt_row_stride;
  a.bt_cols = bt_cols;
  a.num_reqs = num_reqs;
  a.seq_lens = seq_lens;
  a.dql = decode_query_len;
  a.query_req_id = query_req_id;
  a.query_abs_pos = query_abs_pos;
  a.block_page_stride = block_page_stride;
  a.sparse_bt = sparse_bt;
  a.sbt_stride = sbt_row_stride;
  a.sparse_ctx = sparse_ctx;
  return hip_status(msa::launch_sparse_table(a, stream), "sparse table launch");
}

MSA_API msa_status_t msa_query_token_positions(const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                               int32_t num_reqs, int32_t total_q, int32_t* query_req_id,
                                               int32_t* query_abs_pos, hipStream_t stream) {
  MSA_CHECK(num_reqs >= 0 && total_q >= 0, MSA_ERR_INVALID_ARGUMENT, "negative num_reqs %d or total_q %d", num_reqs,
            total_q);
  if (total_q == 0) return ok();
  MSA_CHECK(cu_seqlens_q && query_req_id && query_abs_pos && (context_lens || num_reqs == 0),
            MSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  return hip_status(msa::launch_query_positions(cu_seqlens_q, context_lens, num_reqs, total_q, query_req_id,
                                                query_abs_pos, stream),
                    "query positions launch");
}

MSA_API size_t msa_decode_workspace_size(int32_t total_q, int32_t num_q_heads, int32_t head_dim, int32_t topk_k) {
  if (total_q <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  const int max_ns = topk_k > 64 ? 64 : (topk_k < 1 ? 1 : topk_k);
  return split_bytes(total_q, num_q_heads, head_dim, max_ns);
}

// Decode: validate every host-visible argument, then (if `launch`) enqueue.
static msa_status_t decode_impl(bool launch, const void* q, int32_t q_dtype, int32_t num_reqs,
                                int32_t decode_query_len, int32_t num_q_heads, const msa_kv_cache_t* kv,
                                const int32_t* topk, int64_t topk_row_stride, int32_t topk_k,
                                const int32_t* block_table, int64_t bt_row_stride, int32_t bt_cols,
                                const int32_t* seq_lens, float softmax_scale, void* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  MSA_CHECK(num_reqs >= 0 && decode_query_len >= 1, MSA_ERR_INVALID_ARGUMENT, "num_reqs %d, decode_query_len %d",
            num_reqs, decode_query_len);
  const int64_t rows64 = (int64_t)num_reqs * decode_query_len;
  MSA_CHECK(rows64 <= (1 << 24), MSA_ERR_UNSUPPORTED, "%lld decode rows: at most 2^24", (long long)rows64);
  const int32_t rows = (int32_t)rows64;
  msa_status_t st = check_attend(q, q_dtype, rows, num_q_heads, kv, topk, topk_row_stride, topk_k, block_table,
                                 bt_row_stride, bt_cols, out, softmax_scale);
  if (st != MSA_OK) return st;
  if (rows == 0) return ok();
  MSA_CHECK(seq_lens != nullptr, MSA_ERR_INVALID_ARGUMENT, "seq_lens is NULL");
  if (!launch) return ok();
  msa::AttendArgs a = attend_args(q, num_q_heads, kv, topk, topk_row_stride, topk_k, block_table, bt_row_stride,
                                  bt_cols, softmax_scale, out);
  a.seq_lens = seq_lens;
  a.dql = decode_query_len;
  a.num_reqs = num_reqs;
  a.total_rows = rows;
  int ns = choose_splits(rows, kv->num_kv_heads, topk_k, device_cus());
  while (ns > 1 && (workspace == nullptr || split_bytes(rows, num_q_heads, kv->head_dim, ns) > workspace_bytes)) --ns;
  a.nsplit = ns;
  if (ns > 1) {
    const uintptr_t base = ((uintptr_t)workspace + 255) & ~(uintptr_t)255;
    a.ws_o = reinterpret_cast<float*>(base);
    a.ws_ml = a.ws_o + (size_t)rows * num_q_heads * ns * kv->head_dim;
  }
  return hip_status(msa::launch_attend_decode(a, fmt_of(kv->kv_dtype), rows, stream),
                    "decode launch");
}

MSA_API msa_status_t msa_sparse_decode(const void* q, int32_t q_dtype, int32_t num_reqs, int32_t decode_query_len,
                                       int32_t num_q_heads, const msa_kv_cache_t* kv, const int32_t* topk,
                                       int64_t topk_row_stride, int32_t topk_k, const int32_t* block_table,
                                       int64_t bt_row_stride, int32_t bt_cols, const int32_t* seq_lens,
                                       float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  return decode_impl(true, q, q_dtype, num_reqs, decode_query_len, num_q_heads, kv, topk, topk_row_stride, topk_k,
                     block_table, bt_row_stride, bt_cols, seq_lens, softmax_scale, out, workspace, workspace_bytes,
                     stream);
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace: the split-K partials go to a fixed
// device array instead.  With at least 512 (row, kv head) units the decode
// runs one split and needs no scratch; below that it takes
// ns = ceil(512 / units) splits (units * ns < 1024), and the partials of a
// row head are (D + 2) fp32 per split, so a group of <= 16 query heads at
// D <= 128 needs at most 1023 * 16 * 130 * 4 B + 256 B of alignment slack:
// the array below is never too small for the split count the decode picks.
// ---------------------------------------------------------------------------
constexpr size_t kDecodeScratchBytes = size_t(9) << 20;
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The array's device address on the current device (host code must use this,
// never the array's name, which is a host-side stand-in).
msa_status_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MSA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MSA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}
}  // namespace

MSA_API size_t msa_decode_noalloc_scratch_bytes(void) { return kDecodeScratchBytes; }

MSA_API msa_status_t msa_sparse_decode_noalloc(const void* q, int32_t q_dtype, int32_t num_reqs,
                                               int32_t decode_query_len, int32_t num_q_heads,
                                               const msa_kv_cache_t* kv, const int32_t* topk,
                                               int64_t topk_row_stride, int32_t topk_k, const int32_t* block_table,
                                               int64_t bt_row_stride, int32_t bt_cols, const int32_t* seq_lens,
                                               float softmax_scale, void* out, hipStream_t stream) {
  msa_status_t st = decode_impl(false, q, q_dtype, num_reqs, decode_query_len, num_q_heads, kv, topk,
                                topk_row_stride, topk_k, block_table, bt_row_stride, bt_cols, seq_lens,
                                softmax_scale, out, nullptr, 0, stream);
  if (st != MSA_OK) return st;
  const int64_t rows = (int64_t)num_reqs * decode_query_len;
  if (rows == 0) return ok();
  const int ns = choose_splits(rows, kv->num_kv_heads, topk_k, device_cus());
  const size_t need = ns > 1 ? split_bytes(rows, num_q_heads, kv->head_dim, ns) : 0;
  MSA_CHECK(need <= kDecodeScratchBytes, MSA_ERR_WORKSPACE_TOO_SMALL,
            "decode of %lld rows x %d heads in %d splits needs %zu bytes of scratch; the library holds %zu "
            "(use msa_sparse_decode with a workspace)",
            (long long)rows, num_q_heads, ns, need, kDecodeScratchBytes);
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != MSA_OK) return st;
  return decode_impl(true, q, q_dtype, num_reqs, decode_query_len, num_q_heads, kv, topk, topk_row_stride, topk_k,
                     block_table, bt_row_stride, bt_cols, seq_lens, softmax_scale, out, ws, kDecodeScratchBytes,
                     stream);
}

// A query tile's row order takes a byte per row of the tile (QT = 32, 48 or
// 64 rows at 8-6, 5 and 4 query heads per kv head).  A request of n rows has
// ceil(n / QT) tiles, so at QT = 32 total_q rows in any number of requests
// have at most total_q + ceil(total_q / 32) tiles; the larger tiles fit this
// size unless most requests hold a single row (the tiles past it keep their
// natural order).
MSA_API size_t msa_prefill_workspace_size(int32_t total_q, int32_t num_q_heads, int32_t head_dim, int32_t topk_k) {
  (void)num_q_heads;
  (void)head_dim;
  (void)topk_k;
  if (total_q <= 0) return 0;
  return 32 * ((size_t)total_q + ((size_t)total_q + 31) / 32);
}

// Prefill: validate every host-visible argument, then (if `launch`) enqueue.
static msa_status_t prefill_impl(bool launch, const void* q, int32_t q_dtype, int32_t total_q, int32_t num_q_heads,
                                 const msa_kv_cache_t* kv, const int32_t* topk, int64_t topk_row_stride,
                                 int32_t topk_k, const int32_t* block_table, int64_t bt_row_stride, int32_t bt_cols,
                                 int32_t num_reqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                 float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  MSA_CHECK(total_q >= 0 && num_reqs >= 0, MSA_ERR_INVALID_ARGUMENT, "negative total_q %d or num_reqs %d", total_q,
            num_reqs);
  MSA_CHECK(total_q <= (1 << 24), MSA_ERR_UNSUPPORTED, "%d prefill rows: at most 2^24", total_q);
  msa_status_t st = check_attend(q, q_dtype, total_q, num_q_heads, kv, topk, topk_row_stride, topk_k, block_table,
                                 bt_row_stride, bt_cols, out, softmax_scale);
  if (st != MSA_OK) return st;
  if (total_q == 0) return ok();
  MSA_CHECK(num_reqs >= 1 && cu_seqlens_q && seq_lens, MSA_ERR_INVALID_ARGUMENT,
            "prefill needs num_reqs >= 1, cu_seqlens_q and seq_lens");
  if (!launch) return ok();
  msa::AttendArgs a = attend_args(q, num_q_heads, kv, topk, topk_row_stride, topk_k, block_table, bt_row_stride,
                                  bt_cols, softmax_scale, out);
  a.seq_lens = seq_lens;
  a.cu_seqlens_q = cu_seqlens_q;
  a.num_reqs = num_reqs;
  a.dql = 1;
  a.total_rows = total_q;
  if (workspace != nullptr && workspace_bytes >= 32) {
    a.row_perm = static_cast<int8_t*>(workspace);
    a.perm_cap = (int32_t)std::min<size_t>(workspace_bytes / 32, (size_t)INT32_MAX);
  }
  return hip_status(msa::launch_prefill_blocks(a, fmt_of(kv->kv_dtype), stream), "prefill launch");
}

MSA_API msa_status_t msa_sparse_prefill(const void* q, int32_t q_dtype, int32_t total_q, int32_t num_q_heads,
                                        const msa_kv_cache_t* kv, const int32_t* topk, int64_t topk_row_stride,
                                        int32_t topk_k, const int32_t* block_table, int64_t bt_row_stride,
                                        int32_t bt_cols, int32_t num_reqs, const int32_t* cu_seqlens_q,
                                        const int32_t* seq_lens, float softmax_scale, void* out, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  return prefill_impl(true, q, q_dtype, total_q, num_q_heads, kv, topk, topk_row_stride, topk_k, block_table,
                      bt_row_stride, bt_cols, num_reqs, cu_seqlens_q, seq_lens, softmax_scale, out, workspace,
                      workspace_bytes, stream);
}

MSA_API msa_status_t msa_sparse_attention(
    const void* q, int32_t q_dtype, int32_t num_tokens, int32_t num_q_heads, const msa_kv_cache_t* kv,
    const int32_t* topk, int64_t topk_row_stride, int32_t topk_k, int32_t num_decode_tokens,
    int32_t decode_query_len, const int32_t* decode_block_table, int64_t decode_bt_row_stride,
    int32_t decode_bt_cols, const int32_t* decode_seq_lens, int32_t num_prefill_reqs,
    const int32_t* prefill_block_table, int64_t prefill_bt_row_stride, int32_t prefill_bt_cols,
    const int32_t* prefill_cu_seqlens_q, const int32_t* prefill_seq_lens, float softmax_scale, void* out,
    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  MSA_CHECK(kv != nullptr, MSA_ERR_INVALID_ARGUMENT, "kv cache descriptor is NULL");
  MSA_CHECK(num_tokens >= 0 && num_decode_tokens >= 0 && num_decode_tokens <= num_tokens, MSA_ERR_INVALID_ARGUMENT,
            "num_decode_tokens %d of num_tokens %d", num_decode_tokens, num_tokens);
  MSA_CHECK(decode_query_len >= 1 && num_decode_tokens % decode_query_len == 0, MSA_ERR_INVALID_ARGUMENT,
            "num_decode_tokens %d is not a multiple of decode_query_len %d", num_decode_tokens, decode_query_len);
  MSA_CHECK(num_q_heads >= 1 && kv->head_dim >= 1, MSA_ERR_INVALID_ARGUMENT, "num_q_heads %d, head_dim %d",
            num_q_heads, kv->head_dim);
  const int32_t nd = num_decode_tokens, np = num_tokens - num_decode_tokens;
  const int64_t row_bytes = (int64_t)num_q_heads * kv->head_dim * 2;   // bf16 q / out rows
  const uint8_t* qp = q ? static_cast<const uint8_t*>(q) + (int64_t)nd * row_bytes : nullptr;
  uint8_t* op = out ? static_cast<uint8_t*>(out) + (int64_t)nd * row_bytes : nullptr;
  const int32_t* tp = topk ? topk + (int64_t)nd * topk_row_stride : nullptr;
  // validate both parts before enqueuing either
  msa_status_t st = decode_impl(false, q, q_dtype, nd / decode_query_len, decode_query_len, num_q_heads, kv, topk,
                                topk_row_stride, topk_k, decode_block_table, decode_bt_row_stride, decode_bt_cols,
                                decode_seq_lens, softmax_scale, out, workspace, workspace_bytes, stream);
  if (st != MSA_OK) return st;
  st = prefill_impl(false, qp, q_dtype, np, num_q_heads, kv, tp, topk_row_stride, topk_k, prefill_block_table,
                    prefill_bt_row_stride, prefill_bt_cols, num_prefill_reqs, prefill_cu_seqlens_q, prefill_seq_lens,
                    softmax_scale, op, nullptr, 0, stream);
  if (st != MSA_OK) return st;
  st = decode_impl(true, q, q_dtype, nd / decode_query_len, decode_query_len, num_q_heads, kv, topk, topk_row_stride,
                   topk_k, decode_block_table, decode_bt_row_stride, decode_bt_cols, decode_seq_lens, softmax_scale,
                   out, workspace, workspace_bytes, stream);
  if (st != MSA_OK) return st;
  // (stream order: the decode's split-K merge has read its partials before
  // the prefill reuses the workspace)
  return prefill_impl(true, qp, q_dtype, np, num_q_heads, kv, tp, topk_row_stride, topk_k, prefill_block_table,
                      prefill_bt_row_stride, prefill_bt_cols, num_prefill_reqs, prefill_cu_seqlens_q,
                      prefill_seq_lens, softmax_scale, op, workspace, workspace_bytes, stream);
}

MSA_API msa_status_t msa_insert_index_cache(const void* index_k, int64_t k_stride0, int64_t k_stride1, int32_t n,
                                            int32_t d, int32_t dtype, void* index_cache, int64_t c_stride0,
                                            int64_t c_stride1, int64_t c_stride2, int32_t num_blocks,
                                            int32_t cache_block_size, const int64_t* slot_mapping,
                                            int64_t slot_stride, hipStream_t stream) {
  MSA_CHECK(n >= 0 && d >= 0 && num_blocks >= 0 && cache_block_size >= 0, MSA_ERR_INVALID_ARGUMENT,
            "negative size (n %d, d %d, blocks %d, block size %d)", n, d, num_blocks, cache_block_size);
  if (n == 0 || d == 0 || num_blocks == 0 || cache_block_size == 0) return ok();
  MSA_CHECK(c_stride2 == 1, MSA_ERR_INVALID_ARGUMENT, "index cache: element stride %lld along the key dimension, 1 needed", (long long)c_stride2);
  int esize = 0;
  switch (dtype) {
    case MSA_BF16:
    case MSA_FP16: esize = 2; break;
    case MSA_FP32: esize = 4; break;
    case MSA_FP8_E4M3FN: esize = 1; break;
    default: return fail(MSA_ERR_UNSUPPORTED, "index key dtype %d: bf16, fp16, fp32 or fp8 only", dtype);
  }
  MSA_CHECK(index_k && index_cache && slot_mapping, MSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  return hip_status(msa::launch_index_insert(index_k, k_stride0, k_stride1, n, d, esize, index_cache, c_stride0,
                                             c_stride1, num_blocks, cache_block_size, slot_mapping, slot_stride,
                                             stream),
                    "index cache launch");
}

MSA_API msa_status_t msa_debug_gather_dequant(const msa_kv_cache_t* kv, const int32_t* sparse_bt,
                                              int64_t sbt_row_stride, const int32_t* sparse_ctx, int32_t total_q,
                                              int32_t sbt_width, int32_t path, float* k_out, float* v_out,
                                              hipStream_t stream) {
  MSA_CHECK(kv != nullptr && total_q >= 0, MSA_ERR_INVALID_ARGUMENT, "NULL kv or negative total_q");
  MSA_CHECK(fmt_of(kv->kv_dtype) >= 0, MSA_ERR_UNSUPPORTED, "kv dtype %d: bf16, fp8 e4m3fn or nvfp4 pages only",
            kv->kv_dtype);
  MSA_CHECK(kv->num_kv_heads >= 1, MSA_ERR_INVALID_ARGUMENT, "num_kv_heads %d < 1", kv->num_kv_heads);
  MSA_CHECK(path == 0 || path == 1, MSA_ERR_INVALID_ARGUMENT, "path %d: 0 (decode gather) or 1 (prefill staging)",
            path);
  MSA_CHECK(kv->head_dim == 128 || (kv->head_dim == 64 && kv->kv_dtype != MSA_NVFP4), MSA_ERR_UNSUPPORTED,
            "head_dim %d: 128, or 64 for bf16 / fp8 pages", kv->head_dim);
  {
    const msa_status_t st = check_kv_geometry(kv);
    if (st != MSA_OK) return st;
  }
  MSA_CHECK(sbt_width >= msa::kPagesPerBlock && sbt_width % msa::kPagesPerBlock == 0 &&
                sbt_width <= msa::kPagesPerBlock * msa::kMaxTopK,
            MSA_ERR_INVALID_ARGUMENT, "sbt_width %d: a multiple of 8 in 8..%d", sbt_width,
            msa::kPagesPerBlock * msa::kMaxTopK);
  MSA_CHECK(sbt_row_stride >= sbt_width, MSA_ERR_INVALID_ARGUMENT, "sparse_bt row stride %lld < sbt_width %d",
            (long long)sbt_row_stride, sbt_width);
  if (total_q == 0) return ok();
  const bool v_plane = kv->kv_dtype != MSA_NVFP4 && kv->kv_layout == MSA_KV_PAGE16;
  MSA_CHECK(sparse_bt && sparse_ctx && k_out && v_out && kv->k_pages && (!v_plane || kv->v_pages),
            MSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  msa::AttendArgs a;
  memset(&a, 0, sizeof(a));
  const KvGeometry g = kv_geometry(kv);
  a.k_base = g.k_base;
  a.v_base = g.v_base;
  a.blk_units = g.blk_units;
  a.sub_stride = g.sub;
  a.head_stride = g.head;
  a.row_stride = g.row;
  a.num_units = g.num_units;
  a.v_unit_offset = g.v_unit_offset;
  a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale;
  a.num_kv_heads = kv->num_kv_heads;
  a.head_dim = kv->head_dim;
  const int width_tokens = sbt_width * msa::kPageTokens;
  const int fmt = fmt_of(kv->kv_dtype);
  const hipError_t e = path == 0
      ? msa::launch_gather_dequant_decode(a, fmt, sparse_bt, sbt_row_stride, sparse_ctx, kv->block_page_stride,
                                          total_q, width_tokens, k_out, v_out, stream)
      : msa::launch_gather_dequant_prefill(a, fmt, sparse_bt, sbt_row_stride, sparse_ctx, kv->block_page_stride,
                                           total_q, width_tokens, k_out, v_out, stream);
  return hip_status(e, "gather dequant hook launch");
}

}  // extern "C"
