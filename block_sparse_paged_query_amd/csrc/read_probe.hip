// Measurement hook: a plain HBM read of 4096-byte chunks in a given order,
// with the 16-byte non-temporal loads the decode's page reads use.  Each
// thread folds what it read into one word, so nothing is skipped.  Its rate
// is what this GPU's memory delivers to a kernel that only reads, the context
// for the attends' gathered-KV rates.
//
// One workgroup of 256 threads reads one chunk per step (16 bytes a thread);
// kReadProbeBlocks workgroups stride over the chunk list.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

extern const int kReadProbeBlocks = 4096;   // workgroups (out: kReadProbeBlocks * 256 words)

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ buf, const uint32_t* order,
                                                         uint32_t n_chunks, uint32_t* out) {
  uint32_t acc = 0;
  for (uint32_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const uint32_t id = order ? order[c] : c;
    if (id >= n_chunks) continue;   // a bad order entry reads nothing
    const u32x4 v = __builtin_nontemporal_load(buf + (size_t)id * 256 + threadIdx.x);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_read_probe(const void* buf, const uint32_t* order, uint32_t n_chunks, uint32_t* out,
                             hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kReadProbeBlocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), order, n_chunks, out);
  return hipGetLastError();
}

}  // namespace msa
