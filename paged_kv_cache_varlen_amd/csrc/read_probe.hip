// Streaming-read ceiling of the device: the rate at which plain waves can
// pull a large buffer from HBM with 16-byte non-temporal loads (the same
// kind of load the decode path uses for K/V).  A measurement aid for the
// roofline figures, not part of the attention path; built as its own
// library (libpa_probe.so) so that libpa.so exports only the documented ABI.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Grid-stride over n16 16-byte words, U loads in flight per thread; the XOR
// of everything read is stored only if it is all ones, which keeps the loads
// without writing anything in practice.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p,
                                                          size_t n16, u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= v[k];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  if ((acc.x & acc.y & acc.z & acc.w) == 0xFFFFFFFFu) sink[0] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) of device memory at buf once, with
// `blocks` workgroups of 256 threads, on `stream` (hipStream_t; NULL = the
// null stream).  sink: 16 bytes of device memory the kernel may write.
// Returns 0, or a hipError_t value.
extern "C" int pa_probe_stream_read(const void* buf, size_t bytes, void* sink,
                                    int blocks, void* stream) {
  if (buf == nullptr || sink == nullptr || blocks < 1 || (bytes & 15) != 0 ||
      ((uintptr_t)buf & 15) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel<8>, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16,
                     static_cast<u32x4*>(sink));
  return (int)hipGetLastError();
}
