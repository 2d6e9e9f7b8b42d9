// Test hook: dequantize the K and V of given (page, token) pairs with the
// exact conversions the attends use, then apply the per-tensor scale in fp32.
//
// [FI] vllm.models.minimax_m3.nvidia.sparse_attention_flashinfer,
//   MiniMaxM3SparseFlashInferImpl.forward: fp8 view of the cache, per-tensor
//   k / v scales.
// [NV4] vllm.models.minimax_m3.amd.sparse_attention_nvfp4, customize_spec:
//   NVFP4 slots (packed e2m1 data plus block scales), two per kv head.
//
// One thread per (token, kv head, pair of elements).
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

// `src`: bf16 / fp8 the token's row, NVFP4 the page's slot of the head.
__device__ __forceinline__ void dequant_pair(int fmt, const uint8_t* src, bool v_side, int slot, int e,
                                             float* x0, float* x1) {
  if (fmt == kFmtBf16) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(src + e * 2);
    *x0 = __uint_as_float(w << 16);
    *x1 = __uint_as_float(w & 0xffff0000u);
  } else if (fmt == kFmtFp8) {
    const uint32_t w = *reinterpret_cast<const uint16_t*>(src + e);
    const uint32_t b = fp8x2_to_bf16x2<false>(w);
    *x0 = __uint_as_float(b << 16);
    *x1 = __uint_as_float(b & 0xffff0000u);
  } else {
    // head_dim 128: codes, then scales
    const uint32_t code = src[nvfp4_code_byte(v_side, slot, e / 2)];
    const uint32_t sb = src[nvfp4_scale_byte(v_side, slot, e / 16)];
    const f16x2 sc = fp8x2_to_f16x2<false>(sb);
    const f16x2 s = {sc[0], sc[0]};
    const f16x2 v = fp4x2_to_f16x2<0>(code) * s;
    *x0 = (float)v[0];
    *x1 = (float)v[1];
  }
}

__global__ __launch_bounds__(256) void debug_dequant_kernel(const DequantArgs a) {
  const int D = a.head_dim, H = a.num_kv_heads;
  const int64_t total = (int64_t)a.n * H * (D / 2);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int e = (int)(idx % (D / 2)) * 2;
  const int h = (int)((idx / (D / 2)) % H);
  const int i = (int)(idx / ((int64_t)(D / 2) * H));
  const int64_t page = a.pages[i];
  const int slot = a.slots[i] & 15;
  const float ks = a.k_scale ? *a.k_scale : 1.f, vs = a.v_scale ? *a.v_scale : 1.f;
  float* ko = a.k_out + ((int64_t)i * H + h) * D + e;
  float* vo = a.v_out + ((int64_t)i * H + h) * D + e;
  // page-16 id -> unit of the cache (the V page offset is in v_base)
  const int64_t unit = page / a.block_page_stride * a.blk_units + page % a.block_page_stride;
  if (page < 0 || unit >= a.num_units || unit + a.v_unit_offset >= a.num_units) {
    ko[0] = ko[1] = vo[0] = vo[1] = __builtin_nanf("");
    return;
  }
  const int64_t off = unit * a.sub_stride + (int64_t)h * a.head_stride +
                      (a.fmt == kFmtNvfp4 ? 0 : (int64_t)slot * a.row_stride);
  float x0, x1;
  dequant_pair(a.fmt, a.k_base + off, false, slot, e, &x0, &x1);
  ko[0] = x0 * ks;
  ko[1] = x1 * ks;
  dequant_pair(a.fmt, a.v_base + off, true, slot, e, &x0, &x1);
  vo[0] = x0 * vs;
  vo[1] = x1 * vs;
}

hipError_t launch_debug_dequant(const DequantArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.n * a.num_kv_heads * (a.head_dim / 2);
  hipLaunchKernelGGL(debug_dequant_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace msa
