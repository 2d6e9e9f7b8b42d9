// Index-key side cache insert.
//
// [SPA] vllm.models.minimax_m3.amd.ops.sparse_pa, minimax_m3_insert_index_cache:
// keys [N, D] are scattered into a key-only cache [B, T, D], one int64 slot
// per key.  Slot s addresses block s / T, position s % T; negative slots
// (padding) and slots past the cache are skipped.  One thread per element.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

template <typename T>
__global__ __launch_bounds__(256) void index_insert_kernel(const T* __restrict__ k, int64_t ks0, int64_t ks1, int n,
                                                           int d, T* __restrict__ cache, int64_t cs0, int64_t cs1,
                                                           int64_t capacity, int block_size,
                                                           const int64_t* __restrict__ slots, int64_t slot_stride) {
  const int64_t total = (int64_t)n * d;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t i = idx / d, e = idx - i * d;
    const int64_t s = slots[i * slot_stride];
    if (s < 0 || s >= capacity) continue;
    cache[(s / block_size) * cs0 + (s % block_size) * cs1 + e] = k[i * ks0 + e * ks1];
  }
}

hipError_t launch_index_insert(const void* k, int64_t ks0, int64_t ks1, int n, int d, int esize, void* cache,
                               int64_t cs0, int64_t cs1, int num_blocks, int block_size, const int64_t* slots,
                               int64_t slot_stride, hipStream_t stream) {
  const int64_t total = (int64_t)n * d;
  const int64_t cap = (int64_t)num_blocks * block_size;
  int64_t blocks64 = (total + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 > 65536 ? 65536 : blocks64);
  log_launch("index_insert_kernel: %d keys of %d x %d bytes, %u workgroups", n, d, esize, blocks);
  switch (esize) {
    case 1:
      hipLaunchKernelGGL(index_insert_kernel<uint8_t>, dim3(blocks), dim3(256), 0, stream, (const uint8_t*)k, ks0,
                         ks1, n, d, (uint8_t*)cache, cs0, cs1, cap, block_size, slots, slot_stride);
      break;
    case 2:
      hipLaunchKernelGGL(index_insert_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream, (const uint16_t*)k, ks0,
                         ks1, n, d, (uint16_t*)cache, cs0, cs1, cap, block_size, slots, slot_stride);
      break;
    default:
      hipLaunchKernelGGL(index_insert_kernel<uint32_t>, dim3(blocks), dim3(256), 0, stream, (const uint32_t*)k, ks0,
                         ks1, n, d, (uint32_t*)cache, cs0, cs1, cap, block_size, slots, slot_stride);
      break;
  }
  return hipGetLastError();
}

}  // namespace msa
