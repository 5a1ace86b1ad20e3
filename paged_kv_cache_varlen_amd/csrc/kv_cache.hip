// KV scatter into the block pool, and the logical gather back out of it.
// The tile layouts and the scatter's per-thread bodies are in kv_scatter.h.
#include "kv_scatter.h"

namespace pa {

namespace {

// One thread per (quad of new tokens, kv head, 8-dim chunk); pools of
// BS-token blocks.
template <int D, int BS>
__global__ __launch_bounds__(256) void write_kv_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int64_t k_stride, int64_t v_stride, const int64_t* __restrict__ slots,
    int64_t num_tokens, int Hkv, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, int64_t num_slots) {
  write_kv_thread<D, BS>((int64_t)blockIdx.x * blockDim.x + threadIdx.x, k, v, k_stride,
                         v_stride, slots, num_tokens, Hkv, k_cache, v_cache, num_slots);
}

// One thread per (quad of new tokens, kv head, 16-byte unit of each pool).
template <int D>
__global__ __launch_bounds__(256) void write_kv8_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int64_t k_stride, int64_t v_stride, const int64_t* __restrict__ slots,
    int64_t num_tokens, int Hkv, float k_scale, float v_scale,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    int64_t num_slots) {
  write_kv8_thread<D>((int64_t)blockIdx.x * blockDim.x + threadIdx.x, k, v, k_stride,
                      v_stride, slots, num_tokens, Hkv, k_scale, v_scale, k_cache,
                      v_cache, num_slots);
}

// One thread per (dense row, kv head, 8-dim chunk); pools of BS-token
// blocks.
template <int D, int BS>
__global__ __launch_bounds__(256) void gather_kv_kernel(
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    int64_t num_blocks, const int32_t* __restrict__ bt, int32_t bt_stride,
    const int32_t* __restrict__ seq_lens, const int64_t* __restrict__ kv_start,
    int32_t num_seqs, int64_t total_rows, int Hkv, uint16_t* __restrict__ k_out,
    uint16_t* __restrict__ v_out) {
  constexpr int kChunks = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = (int64_t)Hkv * kChunks;
  if (gid >= total_rows * per_row) return;
  const int64_t row = gid / per_row;
  const int rem = (int)(gid - row * per_row);
  const int g = rem / kChunks;
  const int c = rem - g * kChunks;
  // request owning this row: last b with kv_start[b] <= row
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (kv_start[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int64_t j = row - kv_start[b];
  if (j < 0 || j >= seq_lens[b] || j / BS >= bt_stride) return;
  int64_t blk = bt[(int64_t)b * bt_stride + j / BS];
  if (blk < 0 || blk >= num_blocks) return;
  const int t = (int)(j % BS);
  const int64_t tile = (blk * Hkv + g) * (int64_t)(BS * D);
  const int64_t dst = (row * Hkv + g) * D + c * 8;
  *reinterpret_cast<uint4*>(k_out + dst) =
      *reinterpret_cast<const uint4*>(k_cache + tile + ((int64_t)c * BS + t) * 8);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int d = c * 8 + jj;
    w[jj >> 1] |= (uint32_t)v_cache[tile + v_offset<D, BS>(t, d)] << ((jj & 1) * 16);
  }
  *reinterpret_cast<uint4*>(v_out + dst) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Workgroup size of a scatter launch: a small scatter (a decode step's) is
// limited by its scattered V stores per CU, so it is spread over up to 1024
// one-wave workgroups; larger ones use 256 threads.
unsigned scatter_block(int64_t threads) { return threads <= 64 * 1024 ? 64u : 256u; }

}  // namespace

hipError_t launch_write_kv(const uint16_t* k, const uint16_t* v,
                           int64_t k_stride, int64_t v_stride,
                           const int64_t* slot_mapping, int64_t num_tokens,
                           int num_kv_heads, int head_dim, uint16_t* k_cache,
                           uint16_t* v_cache, int64_t num_blocks,
                           hipStream_t stream, int block_size) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t threads = ((num_tokens + 3) / 4) * num_kv_heads * (head_dim / 8);
  const dim3 block(scatter_block(threads));
  const dim3 grid((unsigned)((threads + block.x - 1) / block.x));
  const int64_t num_slots = num_blocks * block_size;
  void (*fn)(const uint16_t*, const uint16_t*, int64_t, int64_t, const int64_t*, int64_t,
             int, uint16_t*, uint16_t*, int64_t);
  if (block_size == 8)
    fn = head_dim == 128 ? write_kv_kernel<128, 8> : write_kv_kernel<64, 8>;
  else
    fn = head_dim == 128 ? write_kv_kernel<128, kBlock> : write_kv_kernel<64, kBlock>;
  hipLaunchKernelGGL(fn, grid, block, 0, stream, k, v, k_stride, v_stride, slot_mapping,
                     num_tokens, num_kv_heads, k_cache, v_cache, num_slots);
  return hipGetLastError();
}

hipError_t launch_write_kv8(const uint16_t* k, const uint16_t* v,
                            int64_t k_stride, int64_t v_stride,
                            const int64_t* slot_mapping, int64_t num_tokens,
                            int num_kv_heads, int head_dim, float k_scale,
                            float v_scale, uint8_t* k_cache, uint8_t* v_cache,
                            int64_t num_blocks, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t threads = ((num_tokens + 3) / 4) * num_kv_heads * (head_dim / 4);
  const dim3 block(scatter_block(threads));
  const dim3 grid((unsigned)((threads + block.x - 1) / block.x));
  const int64_t num_slots = num_blocks * kBlock;
  if (head_dim == 128) {
    hipLaunchKernelGGL(write_kv8_kernel<128>, grid, block, 0, stream, k, v, k_stride,
                       v_stride, slot_mapping, num_tokens, num_kv_heads, k_scale,
                       v_scale, k_cache, v_cache, num_slots);
  } else {
    hipLaunchKernelGGL(write_kv8_kernel<64>, grid, block, 0, stream, k, v, k_stride,
                       v_stride, slot_mapping, num_tokens, num_kv_heads, k_scale,
                       v_scale, k_cache, v_cache, num_slots);
  }
  return hipGetLastError();
}

hipError_t launch_gather_kv(const uint16_t* k_cache, const uint16_t* v_cache,
                            int64_t num_blocks, const int32_t* block_tables,
                            int32_t bt_stride, const int32_t* seq_lens,
                            const int64_t* kv_start, int32_t num_seqs,
                            int64_t total_rows, int num_kv_heads, int head_dim,
                            uint16_t* k_out, uint16_t* v_out,
                            hipStream_t stream, int block_size) {
  if (total_rows == 0 || num_seqs == 0) return hipSuccess;
  const int64_t threads = total_rows * num_kv_heads * (head_dim / 8);
  const dim3 block(256);
  const dim3 grid((unsigned)((threads + 255) / 256));
  void (*fn)(const uint16_t*, const uint16_t*, int64_t, const int32_t*, int32_t,
             const int32_t*, const int64_t*, int32_t, int64_t, int, uint16_t*, uint16_t*);
  if (block_size == 8)
    fn = head_dim == 128 ? gather_kv_kernel<128, 8> : gather_kv_kernel<64, 8>;
  else
    fn = head_dim == 128 ? gather_kv_kernel<128, kBlock> : gather_kv_kernel<64, kBlock>;
  hipLaunchKernelGGL(fn, grid, block, 0, stream, k_cache, v_cache, num_blocks,
                     block_tables, bt_stride, seq_lens, kv_start, num_seqs, total_rows,
                     num_kv_heads, k_out, v_out);
  return hipGetLastError();
}

}  // namespace pa
