// KV scatter into the block pool ("reshape and cache"): the layouts of the
// pool tiles and the per-thread bodies of the scatter, shared by the scatter
// kernels and by the fused scatter + work-plan kernel.
//
// Every new token of the flattened batch is written to the physical slot
// slot_mapping[i] = block_id * 16 + offset ("vLLM v1 Deep Dive", Aside "KV
// cache and prefix caching"; "vLLM: An Exhaustive Technical Study" section
// 2.1, "Reaching the kernel").  One body for prefill chunks and decodes
// alike: the slot is all it needs.
//
// Pool tile layout (block n, kv head g) of a pool of BS-token blocks (BS = 16,
// or 8), BS*D bf16, H = D/2:
//   K(t, d) at ((d/8)*BS + t)*8 + d%8       -> 16 bytes per (t, 8-dim chunk)
//   V(t, d) at ((((d%H)/16*2 + d/H)*(BS/4) + t/4)*16 + d%16)*4 + t%4
//                                           -> 8 bytes per (4 tokens, dim)
// The attention kernel reads each tile with fully contiguous wave loads
// (16 bytes per lane for K, 8 for V) that land directly in MFMA operand
// order; a 16-key MFMA tile of a pool of 8-token blocks is two such tiles.
#pragma once

#include "pa_device.h"

namespace pa {

namespace {

// Offset of V(t, d) inside a tile of BS token slots.
template <int D, int BS = kBlock>
__device__ __forceinline__ int v_offset(int t, int d) {
  constexpr int H = D / 2;
  return ((((d % H) / 16 * 2 + d / H) * (BS / 4) + (t >> 2)) * 16 + d % 16) * 4 + (t & 3);
}

// Scatter thread gid (0 <= gid < ceil(T/4) * Hkv * D/8; larger gids do
// nothing), one per (quad of consecutive new tokens, kv head, 8-dim chunk): a
// 16-byte K copy per token; for V, when the quad's slots are the four slots
// 4m .. 4m+3 of one block (a prefill chunk's tokens), one 8-byte run per dim
// (the layout keeps 4 consecutive tokens of a dim together), otherwise
// 2-byte stores per token.  Copies are integer moves: exact bits.  Slots
// outside [0, num_slots) are skipped.  BS: tokens per block of the pool
// (slot s is offset s % BS of block s / BS).
template <int D, int BS = kBlock>
__device__ __forceinline__ void write_kv_thread(
    int64_t gid,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int64_t k_stride, int64_t v_stride, const int64_t* __restrict__ slots,
    int64_t num_tokens, int Hkv, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, int64_t num_slots) {
  constexpr int kChunks = D / 8;
  const int64_t per_quad = (int64_t)Hkv * kChunks;
  const int64_t nquads = (num_tokens + 3) >> 2;
  if (gid >= nquads * per_quad) return;
  const int64_t quad = gid / per_quad;
  const int rem = (int)(gid - quad * per_quad);
  const int g = rem / kChunks;
  const int c = rem - g * kChunks;
  const int64_t tok0 = quad * 4;
  const int ntok = (int)min((int64_t)4, num_tokens - tok0);

  int64_t s[4];
  uint4 vv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = -1;
    if (i < ntok) {
      s[i] = slots[tok0 + i];
      vv[i] = *reinterpret_cast<const uint4*>(v + (tok0 + i) * v_stride + g * D + c * 8);
      const uint4 kv = *reinterpret_cast<const uint4*>(k + (tok0 + i) * k_stride + g * D + c * 8);
      if (s[i] >= 0 && s[i] < num_slots) {
        const int64_t tile = ((s[i] / BS) * Hkv + g) * (int64_t)(BS * D);
        *reinterpret_cast<uint4*>(k_cache + tile + ((int64_t)c * BS + (s[i] % BS)) * 8) = kv;
      }
    }
  }
  const bool run = ntok == 4 && s[0] >= 0 && s[3] < num_slots && (s[0] & 3) == 0 &&
                   s[1] == s[0] + 1 && s[2] == s[0] + 2 && s[3] == s[0] + 3;
  if (run) {
    const int64_t tile = ((s[0] / BS) * Hkv + g) * (int64_t)(BS * D);
    const int t0 = (int)(s[0] % BS);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = c * 8 + j;
      uint32_t lo = 0, hi = 0;  // tokens 0,1 and 2,3 of the run at dim d
      const int sh = (j & 1) * 16;
      const uint32_t w0 = (&vv[0].x)[j >> 1] >> sh, w1 = (&vv[1].x)[j >> 1] >> sh;
      const uint32_t w2 = (&vv[2].x)[j >> 1] >> sh, w3 = (&vv[3].x)[j >> 1] >> sh;
      lo = (w0 & 0xffffu) | (w1 << 16);
      hi = (w2 & 0xffffu) | (w3 << 16);
      *reinterpret_cast<uint2*>(v_cache + tile + v_offset<D, BS>(t0, d)) = make_uint2(lo, hi);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i >= ntok || s[i] < 0 || s[i] >= num_slots) continue;
    const int64_t tile = ((s[i] / BS) * Hkv + g) * (int64_t)(BS * D);
    const int t = (int)(s[i] % BS);
    const uint32_t w[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = c * 8 + j;
      v_cache[tile + v_offset<D, BS>(t, d)] = (uint16_t)(w[j >> 1] >> ((j & 1) * 16));
    }
  }
}

// ---- 8-bit pools ------------------------------------------------------------
//
// E4M3 codes (OCP: bias 7, 3 mantissa bits, no infinities, largest finite
// 448), one fp32 scale per pool; the code of x is that of fp32(x) / scale,
// rounded to nearest (ties to even), saturated at +-448, NaN -> 0x7f.
// Tile (block n, kv head g) of 16*D bytes, H = D/2:
//   K(t, d), d = 32c + 8q + j, c = 2p + h:   ((p*4 + q)*16 + t)*16 + h*8 + j
//   V(t, d), d = dh*H + 16c + r, c = 2p + cc: ((p*4 + t/4)*16 + r)*16
//                                             + (2cc + dh)*4 + t%4
// so that every lane of an attention wave reads 16 contiguous bytes that
// hold two K operands (chunks 2p and 2p+1) or four 4-key V operands.

template <int D>
__device__ __forceinline__ int k8_offset(int t, int d) {
  const int c = d >> 5, q = (d >> 3) & 3, j = d & 7;
  return (((c >> 1) * 4 + q) * 16 + t) * 16 + (c & 1) * 8 + j;
}
template <int D>
__device__ __forceinline__ int v8_offset(int t, int d) {
  constexpr int H = D / 2;
  const int dh = d / H, c = (d % H) >> 4, r = d & 15;
  return (((c >> 1) * 4 + (t >> 2)) * 16 + r) * 16 + ((c & 1) * 2 + dh) * 4 + (t & 3);
}

// fp32(bf16 bits) / scale, the value whose code is stored.
__device__ __forceinline__ float scaled(uint32_t bits16, float scale) {
  return __uint_as_float(bits16 << 16) / scale;
}

// Codes of two values in the low 16 bits (a in byte 0, b in byte 1):
// saturate, convert with the hardware's round-to-nearest-even, and put the
// NaN code where the input was NaN.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  const bool na = a != a, nb = b != b;
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
  if (na) w = (w & 0xff00u) | 0x7fu;
  if (nb) w = (w & 0x00ffu) | 0x7f00u;
  return w;
}

// 8-bit scatter thread gid (0 <= gid < ceil(T/4) * Hkv * D/4; larger gids
// do nothing), one per (quad of consecutive new tokens, kv head, 16-byte
// unit u of the D/4 units a quad fills in each pool).  K: unit u belongs to token
// u / (D/16) of the quad (its own slot); V: unit u = (p, r) holds the quad's
// 4 tokens for 4 dims, one 16-byte store when the quad fills slots
// 4m .. 4m+3 of one block, single-byte stores per token otherwise.  Slots
// outside [0, num_slots) are skipped.
template <int D>
__device__ __forceinline__ void write_kv8_thread(
    int64_t gid,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int64_t k_stride, int64_t v_stride, const int64_t* __restrict__ slots,
    int64_t num_tokens, int Hkv, float k_scale, float v_scale,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    int64_t num_slots) {
  constexpr int kUnits = D / 4;       // 16-byte units per quad and pool
  constexpr int kKUnits = D / 16;     // K units per token
  constexpr int H = D / 2;
  const int64_t per_quad = (int64_t)Hkv * kUnits;
  const int64_t nquads = (num_tokens + 3) >> 2;
  if (gid >= nquads * per_quad) return;
  const int64_t quad = gid / per_quad;
  const int rem = (int)(gid - quad * per_quad);
  const int g = rem / kUnits;
  const int u = rem - g * kUnits;
  const int64_t tok0 = quad * 4;
  const int ntok = (int)min((int64_t)4, num_tokens - tok0);

  int64_t s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = i < ntok ? slots[tok0 + i] : -1;

  // K unit: token i, chunks c = 2p, 2p + 1, dims 8q .. 8q+7 of each
  {
    const int i = u / kKUnits, uk = u - i * kKUnits;
    const int p = uk >> 2, q = uk & 3;
    if (i < ntok && s[i] >= 0 && s[i] < num_slots) {
      const uint16_t* row = k + (tok0 + i) * k_stride + g * D;
      const uint4 a = *reinterpret_cast<const uint4*>(row + 64 * p + 8 * q);
      const uint4 b = *reinterpret_cast<const uint4*>(row + 64 * p + 32 + 8 * q);
      const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t* w = h ? wb : wa;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint32_t lo = e4m3_pair(scaled(w[2 * m] & 0xffffu, k_scale),
                                        scaled(w[2 * m] >> 16, k_scale));
          const uint32_t hi = e4m3_pair(scaled(w[2 * m + 1] & 0xffffu, k_scale),
                                        scaled(w[2 * m + 1] >> 16, k_scale));
          o[2 * h + m] = lo | (hi << 16);
        }
      }
      const int64_t tile = ((s[i] >> 4) * Hkv + g) * (int64_t)(kBlock * D);
      *reinterpret_cast<uint4*>(k_cache + tile + k8_offset<D>((int)(s[i] & 15), 64 * p + 8 * q)) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  // V unit (p, r): dims 16(2p + cc) + r + dh * H for (cc, dh) in byte-group
  // order (0,0), (0,1), (1,0), (1,1)
  {
    const int p = u >> 4, r = u & 15;
    int dims[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) dims[e] = 16 * (2 * p + (e >> 1)) + r + (e & 1) * H;
    uint32_t code[4][4];  // [token][dim group]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        uint32_t w = 0;
        if (i < ntok) {
          const uint16_t* row = v + (tok0 + i) * v_stride + g * D;
          w = e4m3_pair(scaled(row[dims[e]], v_scale), scaled(row[dims[e + 1]], v_scale));
        }
        code[i][e] = w & 0xffu;
        code[i][e + 1] = (w >> 8) & 0xffu;
      }
    }
    const bool run = ntok == 4 && s[0] >= 0 && s[3] < num_slots && (s[0] & 3) == 0 &&
                     s[1] == s[0] + 1 && s[2] == s[0] + 2 && s[3] == s[0] + 3;
    if (run) {
      const int64_t tile = ((s[0] >> 4) * Hkv + g) * (int64_t)(kBlock * D);
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = code[0][e] | (code[1][e] << 8) | (code[2][e] << 16) | (code[3][e] << 24);
      *reinterpret_cast<uint4*>(v_cache + tile + v8_offset<D>((int)(s[0] & 15), dims[0])) =
          make_uint4(o[0], o[1], o[2], o[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= ntok || s[i] < 0 || s[i] >= num_slots) continue;
        const int64_t tile = ((s[i] >> 4) * Hkv + g) * (int64_t)(kBlock * D);
        const int t = (int)(s[i] & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v_cache[tile + v8_offset<D>(t, dims[e])] = (uint8_t)code[i][e];
      }
    }
  }
}

}  // namespace

}  // namespace pa
