// Multi-head latent attention (MLA) over a paged latent cache: one 576-dim
// vector per token (512 latent + 64 rotary dims) shared by every query head,
// in blocks of 64 tokens; decode attends MQA-style on the latent.
//
// Cache layout: block n holds 64 * 576 bf16; token t, dim d of the block is
// element (((t / 16) * 18 + d / 32) * 16 + t % 16) * 32 + d % 32, so one
// 16-token x 32-dim piece is 1 KiB contiguous: a wave loads the score operand
// of 16 keys for one 32-dim k step with one 16-byte load per lane.
//
// Decode (mla_decode_kernel): one workgroup of four waves per (query token,
// key split, group of 16 query heads).  For each 16 keys, wave w loads the
// 32-dim chunks it owns (latent chunks 4w .. 4w+3, and one rotary chunk for
// w < 2), computes its share of S^T = K Q^T against the 16 heads, and adds
// the other waves' shares through LDS; all run the same online softmax, and
// wave w accumulates output dims 128w .. 128w+127.  The PV product needs each lane to
// hold 4 consecutive keys of one dim, while the cache rows hold consecutive
// dims of one key: an MFMA against a 0/1 selection matrix moves a 16-key x
// 16-dim piece of the key operand into that form (exact: every product is
// x * 1 or x * 0 and the sums have one nonzero term), so the latent is stored
// and read once.
#include "mfma_util.h"
#include "pa_device.h"

namespace pa {

namespace {


constexpr int kKc = kMlaDim / 32;      // 18 score k steps
constexpr int kLatC = kMlaLatent / 32;  // 16 latent chunks of 32 dims
constexpr int kMlaWaves = 4;
constexpr int kMlaThreads = 64 * kMlaWaves;
constexpr int kOwn = kLatC / kMlaWaves;  // latent chunks per wave
constexpr int kMlaStages = 4;            // 16-key tiles in flight + 1


// Workgroup barrier after this wave's LDS writes have completed.  Unlike
// __syncthreads() (a release/acquire fence, which also waits for every global
// load in flight) it leaves the tile prefetches in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Request of query token t: the last b with qsl[b] <= t (qsl non-decreasing,
// qsl[0] = 0).  The wave's 64 lanes test 64 evenly spaced candidates per
// round (one load each, in parallel): one round up to 64 requests, two up to
// 4096.
__device__ __forceinline__ int request_of(const int32_t* qsl, int num_seqs, int t) {
  const int lane = threadIdx.x & 63;
  int lo = 0, n = num_seqs;  // answer in [lo, lo + n)
  while (n > 1) {
    const int stride = (n + 63) / 64;
    const int bi = lo + lane * stride;
    const bool le = lane * stride < n && qsl[bi] <= t;
    const uint64_t m = __builtin_amdgcn_ballot_w64(le);
    const int k = m ? 63 - __builtin_clzll(m) : 0;
    lo += k * stride;
    n = min(stride, n - k * stride);
  }
  return lo;
}

// Keys token t sees (0 when its request's metadata is out of bounds).
__device__ __forceinline__ int visible_keys(const MlaParams& P, int t, int* b_out) {
  const int b = request_of(P.qsl, P.num_seqs, t);
  const int q0 = P.qsl[b], q1 = P.qsl[b + 1], L = P.seq_lens[b];
  *b_out = b;
  if (q0 < 0 || t < q0 || t >= q1 || q1 - q0 > L || L > P.max_seq_len ||
      (L + kMlaBlock - 1) / kMlaBlock > P.bt_stride)
    return 0;
  return L - (q1 - t) + 1;  // query t - q0 sits at L - Q + (t - q0)
}

__global__ __launch_bounds__(256) void mla_write_kv_kernel(
    const uint16_t* __restrict__ kv, int64_t stride, const int64_t* __restrict__ slots,
    int64_t num_tokens, uint16_t* __restrict__ cache, int64_t num_blocks) {
  // thread: (token, 8-dim piece); 72 pieces per token
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= num_tokens * (kMlaDim / 8)) return;
  const int64_t tok = i / (kMlaDim / 8);
  const int d = (int)(i - tok * (kMlaDim / 8)) * 8;
  const int64_t s = slots[tok];
  if (s < 0 || s >= num_blocks * kMlaBlock) return;
  const int64_t n = s / kMlaBlock;
  const int t = (int)(s - n * kMlaBlock);
  const int64_t off = n * (int64_t)kMlaBlock * kMlaDim +
                      (((t >> 4) * kKc + (d >> 5)) * 16 + (t & 15)) * 32 + (d & 31);
  *reinterpret_cast<uint4*>(cache + off) =
      *reinterpret_cast<const uint4*>(kv + tok * stride + d);
}

__global__ __launch_bounds__(kMlaThreads, 2) void mla_decode_kernel(MlaParams P) {
  // partial scores of the waves, two tiles deep
  __shared__ f32x4 sx[2][kMlaWaves][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  // Workgroup -> (unit u = (token, split), head group): workgroups are
  // dealt to the 8 XCDs round-robin, so the head groups of one unit get
  // indices with the same residue mod 8 (one XCD, one L2) and follow each
  // other there.
  const int nhg = P.Hq / 16;
  const int rest = blockIdx.x >> 3;
  const int hg = rest % nhg;
  const int u = (rest / nhg) * 8 + (blockIdx.x & 7);
  if (u >= P.num_q_tokens * P.max_splits) return;
  const int s = u % P.max_splits;
  const int t = u / P.max_splits;
  int b;
  const int nvis = visible_keys(P, t, &b);
  const int nsplit = (nvis + P.split - 1) / P.split;
  if (s >= nsplit) return;
  const int k0 = s * P.split, k1 = min(nvis, k0 + P.split);

  // Wave w owns latent chunks kOwn * w .. kOwn * w + kOwn - 1 (its output
  // dims) and, for w < 2, rotary chunk 16 + w: its share of the 18 score k
  // steps.  Its query operands: lane (r, g) of chunk c holds dims
  // 32c + 8g .. +7 of head r.
  const bool rot = w < kMlaDim / 32 - kLatC;
  auto chunk = [&](int i) { return i < kOwn ? kOwn * w + i : kLatC + w; };
  const uint16_t* qp = P.q + ((int64_t)t * P.Hq + hg * 16 + r) * kMlaDim + 8 * g;
  bf16x8 qop[kOwn + 1];
#pragma unroll
  for (int i = 0; i < kOwn + 1; ++i)
    if (i < kOwn || rot) qop[i] = *reinterpret_cast<const bf16x8*>(qp + 32 * chunk(i));
  // 0/1 selection operands: E_j[k][n] = 1 where k = 16j + n (lane (r, g)
  // holds rows 8g .. 8g+7 of column r)
  bf16x8 sel[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) sel[j][i] = (__bf16)((8 * g + i == 16 * j + r) ? 1.0f : 0.0f);

  // block ids of the split (at most 64), one per lane
  const int jb0 = k0 / kMlaBlock;
  const int nblk = (k1 + kMlaBlock - 1) / kMlaBlock - jb0;
  int idv = 0;
  if (lane < nblk) idv = P.bt[(int64_t)b * P.bt_stride + jb0 + lane];
  idv = idv < 0 ? 0 : (idv >= P.num_blocks ? (int)(P.num_blocks - 1) : idv);

  f32x4 acc[2 * kOwn];  // this wave's latent chunks x 2 dim tiles of 16
#pragma unroll
  for (int k = 0; k < 2 * kOwn; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lsum = 0.0f;
  const float c2 = P.scale_log2;

  const int ntiles = (k1 - k0 + 15) / 16;  // 16-key tiles of the split
  typedef bf16x8 Tile[kOwn + 1];
  auto load_tile = [&](Tile& kop, int tile) {
    const int key = k0 + 16 * tile;
    const int id = __builtin_amdgcn_readlane(idv, (key / kMlaBlock) - jb0);
    // the piece of (16-key tile, chunk) is [16 tokens][32 dims]: lane (r, g)
    // reads token r, dims 8g .. 8g+7
    const uint16_t* base = P.cache + (int64_t)id * kMlaBlock * kMlaDim +
                           ((key % kMlaBlock) >> 4) * kKc * 512 + r * 32 + g * 8;
    // one head group: every tile is read once (non-temporal); several: the
    // other groups' workgroups on this XCD read it again from L2
#pragma unroll
    for (int i = 0; i < kOwn + 1; ++i)
      if (i < kOwn || rot) {
        const bf16x8* src = reinterpret_cast<const bf16x8*>(base + chunk(i) * 512);
        kop[i] = nhg == 1 ? __builtin_nontemporal_load(src) : *src;
      }
  };
  auto compute = [&](const Tile& kop, int tile) {
    const int key0 = k0 + 16 * tile;
    // this wave's share of the scores; every wave then adds the shares of
    // all waves in the same order, so all hold the same sums
    f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kOwn; ++i) part = mfma32(kop[i], qop[i], part);
    if (rot) part = mfma32(kop[kOwn], qop[kOwn], part);
    sx[tile & 1][w][lane] = part;
    lds_barrier();
    f32x4 sc = sx[tile & 1][0][lane];
#pragma unroll
    for (int v = 1; v < kMlaWaves; ++v) sc += sx[tile & 1][v][lane];
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (key0 + 4 * g + i < k1) ? sc[i] : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = column_max(mx);
    const float mnew = fmaxf(mrun, mx * c2);
    const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(mrun - muse);
    mrun = mnew;
    bf16x4 p;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c2, -muse));
      psum += (float)p[i];
    }
    lsum = lsum * alpha + psum;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int k = 0; k < 2 * kOwn; ++k) acc[k] *= alpha;
    }
    // keys past the split end may be unwritten slots: their V rows are zeroed
    // (a 0 weight must not meet a NaN)
#pragma unroll
    for (int cc = 0; cc < kOwn; ++cc) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f32x4 tv = mfma32(kop[cc], sel[j], f32x4{0.f, 0.f, 0.f, 0.f});
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = (key0 + 4 * g + i < k1) ? (__bf16)tv[i] : (__bf16)0.0f;
        acc[2 * cc + j] = mfma16(v, p, acc[2 * cc + j]);
      }
    }
  };
  // Ring of kMlaStages tiles: the loads of tile i + kMlaStages - 1 are issued
  // before tile i is computed (prefetches past the end repeat the last tile);
  // every wave runs the same steps (one barrier each).
  Tile ring[kMlaStages];
#pragma unroll
  for (int k = 0; k < kMlaStages - 1; ++k) load_tile(ring[k], min(k, ntiles - 1));
  for (int i = 0; i < ntiles; i += kMlaStages) {
#pragma unroll
    for (int k = 0; k < kMlaStages; ++k) {
      load_tile(ring[(k + kMlaStages - 1) % kMlaStages],
                min(i + k + kMlaStages - 1, ntiles - 1));
      if (i + k < ntiles) compute(ring[k], i + k);
    }
  }

  float l = lsum;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const int h = hg * 16 + r;
  const int dim0 = 32 * kOwn * w + 4 * g;
  if (nsplit == 1) {
    const float inv = 1.0f / l;
    uint16_t* op = P.out + ((int64_t)t * P.Hq + h) * kMlaLatent + dim0;
#pragma unroll
    for (int k = 0; k < 2 * kOwn; ++k) {
      bf16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc[k][i] * inv);
      *reinterpret_cast<bf16x4*>(op + 16 * k) = o;
    }
    return;
  }
  const int64_t row = ((int64_t)t * P.Hq + h) * P.max_splits + s;
  float* ap = P.part_acc + row * kMlaLatent + dim0;
#pragma unroll
  for (int k = 0; k < 2 * kOwn; ++k) *reinterpret_cast<f32x4*>(ap + 16 * k) = acc[k];
  if (w == 0 && g == 0) P.part_ml[row] = make_float2(mrun, l);
}

// One wave per (query token, head) whose keys were split: online log-sum-exp
// over its splits in order; lane i holds dims 8i .. 8i+7.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaParams P) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row0 >= (int64_t)P.num_q_tokens * P.Hq) return;
  const int t = (int)(row0 / P.Hq);
  int b;
  const int nvis = visible_keys(P, t, &b);
  const int nsplit = (nvis + P.split - 1) / P.split;
  if (nsplit < 2 || nsplit > P.max_splits) return;
  float M = -INFINITY, den = 0.0f;
  f32x4 n0 = {0.f, 0.f, 0.f, 0.f}, n1 = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const int64_t row = row0 * P.max_splits + s;
    const float2 ml = P.part_ml[row];
    const f32x4* ap = reinterpret_cast<const f32x4*>(P.part_acc + row * kMlaLatent + 8 * lane);
    const f32x4 a0 = ap[0], a1 = ap[1];
    const float mn = fmaxf(M, ml.x);
    const float mu = (mn == -INFINITY) ? 0.0f : mn;
    const float c_old = __builtin_amdgcn_exp2f(M - mu);
    const float c_new = __builtin_amdgcn_exp2f(ml.x - mu);
    den = den * c_old + ml.y * c_new;
    n0 = n0 * c_old + a0 * c_new;
    n1 = n1 * c_old + a1 * c_new;
    M = mn;
  }
  const float inv = 1.0f / den;
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i] = (__bf16)(n0[i] * inv);
    o[i + 4] = (__bf16)(n1[i] * inv);
  }
  *reinterpret_cast<bf16x8*>(P.out + row0 * kMlaLatent + 8 * lane) = o;
}

}  // namespace

hipError_t launch_mla_write_kv(const uint16_t* kv, int64_t stride, const int64_t* slots,
                               int64_t num_tokens, uint16_t* cache, int64_t num_blocks,
                               hipStream_t stream) {
  const int64_t n = num_tokens * (kMlaDim / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_write_kv_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     stream, kv, stride, slots, num_tokens, cache, num_blocks);
  return hipGetLastError();
}

hipError_t launch_mla_decode(const MlaParams& P, hipStream_t stream) {
  if (P.num_q_tokens == 0 || P.num_seqs == 0) return hipSuccess;
  const int64_t units = (int64_t)P.num_q_tokens * P.max_splits;
  const int64_t wgs = (units + 7) / 8 * 8 * (P.Hq / 16);
  hipLaunchKernelGGL(mla_decode_kernel, dim3((unsigned)wgs), dim3(kMlaThreads), 0,
                     stream, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P.max_splits < 2) return e;
  const int64_t rows = (int64_t)P.num_q_tokens * P.Hq;
  hipLaunchKernelGGL(mla_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     stream, P);
  return hipGetLastError();
}

}  // namespace pa
