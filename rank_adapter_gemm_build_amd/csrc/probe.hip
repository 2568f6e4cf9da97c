// Bandwidth probe (diagnostics): what this GPU's HBM delivers to a plain streaming
// kernel, as the ceiling to set the LoRA kernels' traffic against.  The LoRA steps
// are read-dominated (weights and activations read once, the output rows read and
// written once), so the probe offers two forms: a pure read of `read_bytes`, and a
// read of `read_bytes` with one byte written for every `ratio` bytes read.
//
// Every lane moves 16 bytes per access.  The read form gives each workgroup one
// contiguous stretch of the buffer, read 16 accesses deep per lane (consecutive lanes
// on consecutive 16-byte chunks), and folds what it reads into one word per thread
// (written once at the end, so the loads cannot be dropped): measured on MI355X this
// reads at about 6.1-6.2 TB/s, against 5.2-5.6 TB/s for a grid-stride loop over the
// whole buffer.
#include <hip/hip_runtime.h>

#include "device_util.h"

namespace rax {

constexpr int kProbeUnroll = 16;
constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = min((size_t)blockIdx.x * per, n16), b1 = min(b0 + per, n16);
  uint32_t acc = 0;
  size_t i = b0 + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < b1; i += kProbeUnroll * kProbeThreads) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[i + u * kProbeThreads];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < b1; i += kProbeThreads) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// ratio 16-byte chunks read for each chunk written: out[j] = xor of in[j * ratio + q]
// over q (consecutive lanes read consecutive chunks of each of the ratio strides)
__global__ __launch_bounds__(256) void probe_read_write_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                               size_t n_out, int ratio) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t j = (size_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_out; j += stride) {
    uint4 a = make_uint4(0, 0, 0, 0);
    for (int q = 0; q < ratio; ++q) {
      const uint4 v = src[(size_t)q * n_out + j];
      a.x ^= v.x; a.y ^= v.y; a.z ^= v.z; a.w ^= v.w;
    }
    dst[j] = a;
  }
}

int probe_grid(size_t work) {
  const size_t want = (work + 255) / 256;
  return (int)std::min<size_t>(std::max<size_t>(want, 1), 256 * 16);   // 16 workgroups per CU at most
}

hipError_t launch_bandwidth_probe(const void* src, size_t read_bytes, void* dst, size_t dst_bytes, int ratio,
                                  hipStream_t stream) {
  if (!src || !dst || read_bytes < 16 || (reinterpret_cast<uintptr_t>(src) & 15) ||
      (reinterpret_cast<uintptr_t>(dst) & 15))
    return hipErrorInvalidValue;
  const size_t n16 = read_bytes / 16;
  if (ratio <= 0) {
    // four workgroups per CU, each with a contiguous stretch (at least one full pass)
    const int grid = (int)std::max<size_t>(1, std::min<size_t>(1024, n16 / (kProbeUnroll * kProbeThreads)));
    if ((size_t)grid * 256 * sizeof(uint32_t) > dst_bytes) return hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, static_cast<const uint4*>(src), n16,
                       static_cast<uint32_t*>(dst));
  } else {
    const size_t n_out = n16 / (size_t)ratio;
    if (n_out == 0 || n_out * 16 > dst_bytes) return hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_read_write_kernel, dim3(probe_grid(n_out)), dim3(256), 0, stream,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n_out, ratio);
  }
  return hipGetLastError();
}

}  // namespace rax
