// Whole-block operations on the pool: the block copy of copy-on-write, and
// the expansion of block tables of larger blocks into 16-token block ids.
#include "pa_device.h"

namespace pa {

namespace {

constexpr int kCopyThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per (pair, pool) and slice of the block: 16-byte loads and
// stores, consecutive across the workgroup, non-temporal (a copied block is
// not read again by this launch; measured 4.95 -> 5.23 TB/s of reads plus
// writes for 4096 pairs of 32 KiB blocks).  A pair naming a block outside
// the pool (or the same block twice) is skipped.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    int64_t block_bytes, int64_t num_blocks, const int64_t* __restrict__ mapping,
    int64_t num_pairs) {
  const int64_t pair = blockIdx.x >> 1;
  if (pair >= num_pairs) return;
  const int64_t src = mapping[2 * pair], dst = mapping[2 * pair + 1];
  if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks || src == dst) return;
  uint8_t* pool = (blockIdx.x & 1) ? v_cache : k_cache;
  const u32x4* s = reinterpret_cast<const u32x4*>(pool + src * block_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(pool + dst * block_bytes);
  const int64_t n16 = block_bytes / 16;
  for (int64_t i = (int64_t)blockIdx.y * kCopyThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.y * kCopyThreads)
    __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

// out[b][j] = in[b][j / R] * R + j % R for the R = block_size / 16 sub-blocks
// of each block; negative (unused) entries stay -1.
__global__ __launch_bounds__(256) void expand_tables_kernel(
    const int32_t* __restrict__ in, int32_t in_stride, int32_t num_seqs, int R,
    int32_t* __restrict__ out) {
  const int64_t out_stride = (int64_t)in_stride * R;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)num_seqs * out_stride) return;
  const int64_t b = i / out_stride, j = i - b * out_stride;
  const int32_t id = in[b * in_stride + j / R];
  const int64_t e = (int64_t)id * R + j % R;
  out[i] = (id < 0 || e > INT32_MAX) ? -1 : (int32_t)e;
}

}  // namespace

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, int64_t block_bytes,
                              int64_t num_blocks, const int64_t* mapping,
                              int64_t num_pairs, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t n16 = block_bytes / 16;
  int64_t slices = (n16 + kCopyThreads - 1) / kCopyThreads;
  if (slices > 64) slices = 64;
  const dim3 grid((unsigned)(2 * num_pairs), (unsigned)slices);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, stream,
                     static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                     block_bytes, num_blocks, mapping, num_pairs);
  return hipGetLastError();
}

hipError_t launch_expand_tables(const int32_t* in, int32_t in_stride,
                                int32_t num_seqs, int R, int32_t* out,
                                hipStream_t stream) {
  const int64_t n = (int64_t)num_seqs * in_stride * R;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(expand_tables_kernel, dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, stream, in, in_stride, num_seqs, R, out);
  return hipGetLastError();
}

}  // namespace pa
