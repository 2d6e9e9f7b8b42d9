// Device helpers shared by the libmsa kernels (gfx950 / CDNA4, wave64).
//
// Page titles cited:
//   [FI]  vllm.models.minimax_m3.nvidia.sparse_attention_flashinfer
//   [NV4] vllm.models.minimax_m3.amd.sparse_attention_nvfp4
//   [SPA] vllm.models.minimax_m3.amd.ops.sparse_pa
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// GCC-style vectors: the matrix-core and conversion builtins are declared on them.
typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
typedef _Float16 f16x8 __attribute__((__vector_size__(16)));
typedef _Float16 f16x2 __attribute__((__vector_size__(4)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x2 __attribute__((__vector_size__(8)));

constexpr int kBlockTokens = 128;   // a sparse block ([SPA]: SPARSE_BLOCK_SIZE)
constexpr int kPageTokens = 16;     // page-16 numbering ([SPA] rebase_block_table_to_page16)
constexpr int kPagesPerBlock = 8;   // 128 / 16
constexpr int kMaxTopK = 1024;      // longest top-k row the attends stage in LDS

enum KvFormat : int { kFmtBf16 = 0, kFmtFp8 = 1, kFmtNvfp4 = 2 };

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Matrix cores: D = A * B + C on a 16x16 tile with a 32-deep reduction.
// Lane l = 16 * g + r holds A[r][8g .. 8g+7], B[8g .. 8g+7][r] and returns
// C[4g .. 4g+3][r] (layout checked on the device against a host product).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Exact conversions.  The scaled-convert instructions apply only the exponent
// of their scale operand, so they are always called with 1.0 here; E4M3 block
// scales are applied with a separate (exact) fp16 multiply.
// ---------------------------------------------------------------------------
// Two E4M3FN codes (bytes 0,1 or 2,3 of w) -> two bf16, exact.
template <bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  bf16x2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi);
  return __builtin_bit_cast(uint32_t, v);
}
// Two E4M3FN codes -> two fp16, exact (E4M3FN is a subset of fp16).
template <bool kHi>
__device__ __forceinline__ f16x2 fp8x2_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHi);
}
// Byte kByte of w (two e2m1 codes, low nibble first) -> two fp16, exact.
template <int kByte>
__device__ __forceinline__ f16x2 fp4x2_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, kByte);
}

__device__ __forceinline__ uint32_t f16x2_bits(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ f16x2 bits_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

// bf16 -> fp16 pair (exact for |x| in the fp16 normal range).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  return f16x2_bits(v);
}

// Two floats -> packed bf16 / fp16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 v = {(_Float16)a, (_Float16)b};
  return f16x2_bits(v);
}

// Halves of two packed pairs: (a.lo, b.lo) or (a.hi, b.hi).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Word 3 of a raw buffer descriptor (unit stride, no swizzle, 32-bit data
// format): a load at or past num_records bytes returns 0 and touches no memory.
constexpr int kRawBufferWord3 = 0x00020000;

// A byte pointer into LDS (direct-to-LDS copies take one).
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// ---------------------------------------------------------------------------
// NVFP4 slot byte order, head_dim 128 ([NV4] customize_spec leaves the bytes
// inside a page to the kernels).  A slot holds 16 tokens: 1024 code bytes
// (two e2m1 codes per byte, the low nibble the even element), then 128
// E4M3FN scale bytes (one per 16 elements).
//   K slot, token-major: code byte c of token t at t * 64 + c, scale u at
//     1024 + t * 8 + u.
//   V slot, tokens in groups of 4: the 4-byte unit w (elements 8w .. 8w+7) of
//     token t at ((t / 4 * 16 + w) * 4 + t % 4) * 4, scale u at
//     1024 + (t / 4 * 8 + u) * 4 + t % 4 -- a decode lane reads its 8 elements
//     of 4 tokens (16 bytes) and their 4 scales (4 bytes) in one load each.
// ---------------------------------------------------------------------------
constexpr int kNvfp4SlotBytes = 9 * 128;
constexpr int kNvfp4ScaleBase = 1024;
__device__ __forceinline__ int nvfp4_code_byte(bool v_slot, int t, int c) {
  return v_slot ? ((t / 4 * 16 + c / 4) * 4 + t % 4) * 4 + c % 4 : t * 64 + c;
}
__device__ __forceinline__ int nvfp4_scale_byte(bool v_slot, int t, int u) {
  return kNvfp4ScaleBase + (v_slot ? (t / 4 * 8 + u) * 4 + t % 4 : t * 8 + u);
}

// ---------------------------------------------------------------------------
// Row compaction ([SPA] _write_sparse_block_table_row_from_values).
//
// Run by all 64 lanes of one wave.  Keeps the ids 0 <= id <= own block
// (id < bt_cols) of a top-k row; writes the physical block ids of the kept
// earlier ("full") blocks, in row order, to list[0 ..), then the own
// ("tail") block; returns the slot count and the attended context length.
// Stable order comes from a ballot plus a masked bit count per 64 ids.
// ---------------------------------------------------------------------------
struct RowSlots {
  int n_slots;
  int ctx;
};

__device__ __forceinline__ RowSlots compact_row(const int32_t* __restrict__ topk_row, int k,
                                                const int32_t* __restrict__ bt_row, int bt_cols,
                                                int abs_pos, int* list) {
  const int lane = threadIdx.x & 63;
  const int causal_len = abs_pos + 1 > 0 ? abs_pos + 1 : 0;
  const int self_blk = abs_pos >= 0 ? abs_pos / kBlockTokens : -1;
  int n_full = 0;
  bool has_tail = false;
  int tail_phys = 0;
  if (causal_len > 0) {
    for (int base = 0; base < k; base += 64) {
      const int t = base + lane;
      const int blk = t < k ? topk_row[t] : -1;
      const bool valid = blk >= 0 && blk <= self_blk && blk < bt_cols;
      const bool is_full = valid && blk < self_blk;
      const bool is_tail = valid && blk == self_blk;
      const int phys = valid ? bt_row[blk] : 0;
      const uint64_t fm = __ballot(is_full);
      const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(fm >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)fm, 0u));
      if (is_full) list[n_full + rank] = phys;
      n_full += __popcll(fm);
      const uint64_t tm = __ballot(is_tail);
      if (tm != 0) {
        has_tail = true;
        tail_phys = __shfl(phys, __ffsll((unsigned long long)tm) - 1);
      }
    }
  }
  if (has_tail && lane == 0) list[n_full] = tail_phys;
  RowSlots out;
  out.n_slots = n_full + (has_tail ? 1 : 0);
  out.ctx = has_tail ? n_full * kBlockTokens + (causal_len - self_blk * kBlockTokens)
                     : min(out.n_slots * kBlockTokens, causal_len);
  return out;
}

// Row position in decode: row i of request i / dql sits at
// seq_lens[r] - dql + i % dql ([FI] forward: right-aligned decode tokens).
__device__ __forceinline__ void decode_row_position(const int32_t* __restrict__ seq_lens, int dql, int row,
                                                    int* req, int* abs_pos) {
  const int r = row / dql;
  *req = r;
  *abs_pos = seq_lens[r] - dql + (row - r * dql);
}

}  // namespace msa
