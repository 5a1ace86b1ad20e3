/*
 * CPU reference ("oracle") for the paged KV-cache varlen attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke entry point and the CPU
 * baseline leg of the benchmark do.  It shares no source, header or helper
 * with the HIP path.
 *
 * Plain, slow, obviously correct: loops in the order the definitions state
 * them, floating point in fp64.  bf16 inputs are widened exactly (the 16 bits
 * become the top half of an IEEE binary32, which converts exactly to binary64).
 *
 * Sources (the pages whose definitions these functions write out):
 *  - "vLLM v1 Deep Dive", Part 3 Runtime, Aside "KV cache and prefix caching"
 *    (supercharleszhu.github.io): a forward writes each new token's K/V into
 *    the physical slot block_id*block_size + offset given by slot_mapping, and
 *    reads K/V back per request through its block_table; a prefill query
 *    attends causally over cached prefix + new tokens, a decode query over all
 *    of its blocks, one launch for the whole batch.
 *  - Same page, "Step 4c - Mixed batches": query_start_loc is the prefix sum
 *    of per-request scheduled token counts.
 *  - "vLLM: An Exhaustive Technical Study for Kernel Engineers" (anthony-chaudhary.github.io) section 2.1
 *    "PagedAttention & the block manager" (block table maps logical block
 *    index to physical block id; write slot = block number * block_size +
 *    offset) and section 2.4 "Attention kernels & backends" (query heads that
 *    share one KV head are processed together).
 *
 * Readings taken where the pages are silent (each listed in the design notes):
 *  - attention is softmax(scale * q.k^T) v, the scale a caller argument;
 *  - seq_lens counts cached + new tokens, and the new tokens are the last
 *    Q_b positions, so query i of a Q_b-token chunk sits at p = L_b - Q_b + i
 *    and sees keys 0..p (bottom-right causal alignment);
 *  - query head h reads KV head floor(h / (Hq/Hkv));
 *  - slot_mapping entries < 0 are skipped;
 *  - the pool layout is the one documented with the C ABI (see k_index and
 *    v_index below: 16-token blocks, per (block, kv head) one K tile and one
 *    V tile of 16*D bf16 each, permuted inside the tile).
 */
#include <math.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "oracle.h"

/* ---- bf16 <-> fp64 (exact widening) ---------------------------------- */

static double bf16_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ---- pool layout (as documented with the C ABI) ----------------------- */

/* Element offset of K (block n, kv head g, token slot t, dim d).
 * Tile (n, g) starts at (n*Hkv + g) * bs * D; inside it K is stored as
 * D/8 chunks of [bs tokens][8 dims]. */
static size_t k_index(int64_t n, int64_t g, int64_t t, int64_t d, int64_t Hkv,
                      int64_t bs, int64_t D) {
  size_t tile = (size_t)((n * Hkv + g) * bs * D);
  size_t chunk = (size_t)(d / 8);
  return tile + (chunk * (size_t)bs + (size_t)t) * 8 + (size_t)(d % 8);
}

/* Element offset of V (block n, kv head g, token slot t, dim d).
 * Inside a tile, with H = D/2, d = dh*H + 16*c + r (dh < 2, r < 16) and
 * t = 4*tg + tl: order is [c][dh][tg][r][tl], i.e. 4 consecutive tokens of
 * one dim are contiguous and 64 such runs form a 512-byte region per
 * (c, dh). */
static size_t v_index(int64_t n, int64_t g, int64_t t, int64_t d, int64_t Hkv,
                      int64_t bs, int64_t D) {
  size_t tile = (size_t)((n * Hkv + g) * bs * D);
  int64_t H = D / 2;
  int64_t dh = d / H, c = (d % H) / 16, r = d % 16;
  int64_t tg = t / 4, tl = t % 4;
  return tile + (size_t)((((c * 2 + dh) * (bs / 4) + tg) * 16 + r) * 4 + tl);
}

/* ---- 8-bit KV cache: E4M3 codes and their tile layout ------------------- */

/* The pages name fp8 (E4M3) KV-cache quantisation with one fp32 scale per
 * tensor ("Quantization & compute kernels", the KV-cache quantisation axis,
 * in "vLLM: An Exhaustive Technical Study for Kernel Engineers").  The code
 * is OCP E4M3 ("E4M3FN"): sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; no infinities; S.1111.111 is NaN; normal values (1 + m/8) * 2^(e-7)
 * for e = 1..15 (largest finite 1.75 * 2^8 = 448); subnormals (m/8) * 2^-6. */
double oracle_e4m3_decode(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Encode one fp32 value: NaN -> 0x7f; magnitudes at or above 448 (and
 * infinities) saturate to 448; everything else rounds to the nearest code,
 * ties to the even mantissa.  Exact arithmetic in fp64 (the value is an
 * fp32, so a / 2^k and its rounding are exact). */
uint8_t oracle_e4m3_encode(float v) {
  if (isnan(v)) return 0x7f;
  uint8_t s = signbit(v) ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (a >= 448.0) return s | 0x7e;
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: multiples of 2^-9; 8 * 2^-9 is the smallest normal */
    double m = rint(a / ldexp(1.0, -9)); /* round to nearest, ties to even */
    return s | (uint8_t)m;               /* m == 8 is code 0x08 = 2^-6 */
  }
  int k;
  frexp(a, &k); /* a = f * 2^k, f in [0.5, 1) */
  int e = k - 1; /* a in [2^e, 2^(e+1)) */
  double m = rint((a / ldexp(1.0, e) - 1.0) * 8.0);
  if (m == 8.0) {
    m = 0.0;
    e += 1;
  }
  /* a < 448 keeps e + 7 <= 15 and excludes the NaN code */
  return s | (uint8_t)(((e + 7) << 3) | (int)m);
}

/* Byte offset of K (block n, kv head g, slot t, dim d) in an 8-bit pool.
 * Tile (n, g) starts at (n*Hkv + g) * bs * D.  With d = 32c + 8q + j
 * (q < 4, j < 8) and c = 2p + h: 16-byte units [p][q][t], each holding the
 * 8 dims of chunk c = 2p and then the 8 dims of chunk 2p + 1. */
static size_t k8_index(int64_t n, int64_t g, int64_t t, int64_t d, int64_t Hkv,
                       int64_t bs, int64_t D) {
  size_t tile = (size_t)((n * Hkv + g) * bs * D);
  int64_t c = d / 32, q = (d % 32) / 8, j = d % 8;
  int64_t p = c / 2, h = c % 2;
  return tile + (size_t)(((p * 4 + q) * bs + t) * 16 + h * 8 + j);
}

/* Byte offset of V (block n, kv head g, slot t, dim d) in an 8-bit pool.
 * With H = D/2, d = dh*H + 16c + r (dh < 2, r < 16), c = 2p + cc and
 * t = 4*tg + tl: 16-byte units [p][tg][r], each holding 4-token runs for
 * (cc, dh) = (0,0), (0,1), (1,0), (1,1). */
static size_t v8_index(int64_t n, int64_t g, int64_t t, int64_t d, int64_t Hkv,
                       int64_t bs, int64_t D) {
  size_t tile = (size_t)((n * Hkv + g) * bs * D);
  int64_t H = D / 2;
  int64_t dh = d / H, c = (d % H) / 16, r = d % 16;
  int64_t p = c / 2, cc = c % 2;
  int64_t tg = t / 4, tl = t % 4;
  return tile +
         (size_t)(((p * (bs / 4) + tg) * 16 + r) * 16 + (cc * 2 + dh) * 4 + tl);
}

size_t oracle_k8_index(int64_t n, int64_t g, int64_t t, int64_t d, int64_t Hkv,
                       int64_t bs, int64_t D) {
  return k8_index(n, g, t, d, Hkv, bs, D);
}

size_t oracle_v8_index(int64_t n, int64_t g, int64_t t, int64_t d, int64_t Hkv,
                       int64_t bs, int64_t D) {
  return v8_index(n, g, t, d, Hkv, bs, D);
}

size_t oracle_k_index(int64_t n, int64_t g, int64_t t, int64_t d, int64_t Hkv,
                      int64_t bs, int64_t D) {
  return k_index(n, g, t, d, Hkv, bs, D);
}

size_t oracle_v_index(int64_t n, int64_t g, int64_t t, int64_t d, int64_t Hkv,
                      int64_t bs, int64_t D) {
  return v_index(n, g, t, d, Hkv, bs, D);
}

/* ---- KV scatter (reshape-and-cache) ---------------------------------- */

/* For each new token t with slot s = slot_mapping[t] >= 0: block s / bs,
 * offset s % bs; copy the bits of k[t][g][d], v[t][g][d] there.  Every other
 * pool element is left as it was. */
void oracle_write_kv(uint16_t *k_cache, uint16_t *v_cache, const uint16_t *k,
                     const uint16_t *v, const int64_t *slot_mapping,
                     int64_t num_tokens, int64_t Hkv, int64_t bs, int64_t D) {
  /* kv heads write disjoint tiles, so they run in parallel; within a head the
   * tokens are applied in order (a repeated slot keeps the last token). */
#pragma omp parallel for schedule(static)
  for (int64_t g = 0; g < Hkv; ++g) {
    for (int64_t t = 0; t < num_tokens; ++t) {
      int64_t s = slot_mapping[t];
      if (s < 0) continue;
      int64_t n = s / bs, off = s % bs;
      for (int64_t d = 0; d < D; ++d) {
        size_t src = (size_t)((t * Hkv + g) * D + d);
        k_cache[k_index(n, g, off, d, Hkv, bs, D)] = k[src];
        v_cache[v_index(n, g, off, d, Hkv, bs, D)] = v[src];
      }
    }
  }
}

/* 8-bit scatter: the same slots as oracle_write_kv; each element x (bf16,
 * widened exactly to fp32) is stored as the E4M3 code of the fp32 quotient
 * x / scale (IEEE division, round to nearest). */
void oracle_write_kv_fp8(uint8_t *k_cache, uint8_t *v_cache, const uint16_t *k,
                         const uint16_t *v, const int64_t *slot_mapping,
                         int64_t num_tokens, int64_t Hkv, int64_t bs, int64_t D,
                         float k_scale, float v_scale) {
  /* kv heads in parallel, tokens in order within a head (as above) */
#pragma omp parallel for schedule(static)
  for (int64_t g = 0; g < Hkv; ++g) {
    for (int64_t t = 0; t < num_tokens; ++t) {
      int64_t s = slot_mapping[t];
      if (s < 0) continue;
      int64_t n = s / bs, off = s % bs;
      for (int64_t d = 0; d < D; ++d) {
        size_t src = (size_t)((t * Hkv + g) * D + d);
        float kx = (float)bf16_to_double(k[src]);
        float vx = (float)bf16_to_double(v[src]);
        float kq = kx / k_scale;
        float vq = vx / v_scale;
        k_cache[k8_index(n, g, off, d, Hkv, bs, D)] = oracle_e4m3_encode(kq);
        v_cache[v8_index(n, g, off, d, Hkv, bs, D)] = oracle_e4m3_encode(vq);
      }
    }
  }
}

/* ---- logical gather through the block tables -------------------------- */

/* Dense [sum L_b][Hkv][D]: row (start_b + j) holds logical token j of
 * sequence b, read from block block_tables[b][j / bs] at offset j % bs. */
void oracle_gather_kv(const uint16_t *k_cache, const uint16_t *v_cache,
                      const int32_t *block_tables, int64_t bt_stride,
                      const int32_t *seq_lens, int64_t num_seqs, int64_t Hkv,
                      int64_t bs, int64_t D, uint16_t *k_out, uint16_t *v_out) {
  int64_t row = 0;
  for (int64_t b = 0; b < num_seqs; ++b) {
    for (int64_t j = 0; j < seq_lens[b]; ++j, ++row) {
      int64_t n = block_tables[b * bt_stride + j / bs];
      for (int64_t g = 0; g < Hkv; ++g) {
        for (int64_t d = 0; d < D; ++d) {
          size_t dst = (size_t)((row * Hkv + g) * D + d);
          k_out[dst] = k_cache[k_index(n, g, j % bs, d, Hkv, bs, D)];
          v_out[dst] = v_cache[v_index(n, g, j % bs, d, Hkv, bs, D)];
        }
      }
    }
  }
}

/* ---- copy-on-write and larger blocks ------------------------------------ */

/* Copy-on-write ("vLLM: An Exhaustive Technical Study", section 2.1: a block
 * held by several requests is duplicated when one of them writes into it).
 * For each pair (src, dst) = (mapping[2i], mapping[2i+1]), in order, every
 * byte of block src is copied to block dst in both pools (a block is
 * block_bytes bytes: all kv heads, K or V).  Pairs naming a block outside
 * [0, num_blocks), or the same block twice, are skipped. */
void oracle_copy_blocks(uint8_t *k_cache, uint8_t *v_cache, int64_t block_bytes,
                        int64_t num_blocks, const int64_t *mapping,
                        int64_t num_pairs) {
  for (int64_t i = 0; i < num_pairs; ++i) {
    int64_t src = mapping[2 * i], dst = mapping[2 * i + 1];
    if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks || src == dst)
      continue;
    for (int64_t b = 0; b < block_bytes; ++b) {
      k_cache[dst * block_bytes + b] = k_cache[src * block_bytes + b];
      v_cache[dst * block_bytes + b] = v_cache[src * block_bytes + b];
    }
  }
}

/* Tables of bs-token blocks (bs = R * 16) in 16-token block ids.  With
 * block size bs, token t of a request is written to slot
 * table[t / bs] * bs + t % bs (same section); read as a pool of 16-token
 * blocks, that slot lies in 16-token block slot / 16.  So 16-token block j of
 * the request (tokens 16j .. 16j+15) is out[j] = slot(16j) / 16.  Entries
 * < 0 stay -1. */
void oracle_expand_block_tables(const int32_t *in, int64_t num_seqs,
                                int64_t in_stride, int64_t bs, int32_t *out) {
  int64_t R = bs / 16, out_stride = in_stride * R;
  for (int64_t b = 0; b < num_seqs; ++b) {
    for (int64_t j = 0; j < out_stride; ++j) {
      int64_t t = 16 * j;
      int64_t n = in[b * in_stride + t / bs];
      out[b * out_stride + j] = n < 0 ? -1 : (int32_t)((n * bs + t % bs) / 16);
    }
  }
}

/* ---- MLA latent cache ----------------------------------------------------- */

/* Multi-head latent attention ("vLLM: An Exhaustive Technical Study",
 * section 2.4, the MLA paragraph): one latent vector per token, shared by all
 * query heads, of MLA_DL = 512 latent + 64 rotary dims, in blocks of 64
 * tokens; decode attends MQA-style on the latent.  Reading: a query head's
 * score of token j is scale * (its 576-dim query . token j's 576-dim cached
 * vector), and its output is the softmax-weighted sum of the first
 * MLA_DV = 512 (latent) dims of those vectors.
 *
 * Cache layout (the library's choice, documented with the C ABI): block n
 * holds 64 * 576 bf16; token t, dim d of the block sits at
 * (((t / 16) * 18 + d / 32) * 16 + t % 16) * 32 + d % 32. */
#define MLA_BS 64
#define MLA_DL 576
#define MLA_DV 512

static size_t mla_index(int64_t n, int64_t t, int64_t d) {
  return (size_t)(n * MLA_BS * MLA_DL +
                  (((t / 16) * (MLA_DL / 32) + d / 32) * 16 + t % 16) * 32 + d % 32);
}

size_t oracle_mla_index(int64_t n, int64_t t, int64_t d) { return mla_index(n, t, d); }

/* For each token i with slot s = slot_mapping[i] >= 0: block s / 64, offset
 * s % 64; copy the bits of kv[i][0..575] there. */
void oracle_mla_write_kv(uint16_t *cache, const uint16_t *kv,
                         const int64_t *slot_mapping, int64_t num_tokens) {
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t s = slot_mapping[i];
    if (s < 0) continue;
    for (int64_t d = 0; d < MLA_DL; ++d)
      cache[mla_index(s / MLA_BS, s % MLA_BS, d)] = kv[i * MLA_DL + d];
  }
}

/* out[t][h][e] (fp64) for every query token t of every request b: query i of
 * the request's Q = qsl[b+1] - qsl[b] tokens sits at p = L - Q + i and sees
 * tokens 0..p; token j's vector is read from block block_tables[b][j / 64],
 * offset j % 64. */
void oracle_mla_decode(const uint16_t *q, const uint16_t *cache,
                       const int32_t *block_tables, int64_t bt_stride,
                       const int32_t *seq_lens, const int32_t *query_start_loc,
                       int64_t num_seqs, int64_t Hq, float scale, double *out,
                       int nthreads) {
  const double sigma = (double)scale;
  for (int64_t b = 0; b < num_seqs; ++b) {
    int64_t q0 = query_start_loc[b], Q = query_start_loc[b + 1] - q0;
    int64_t L = seq_lens[b];
    int64_t rows = Q * Hq;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic)
    for (int64_t r = 0; r < rows; ++r) {
      int64_t i = r / Hq, h = r % Hq, t = q0 + i, p = L - Q + i;
      double *s = (double *)malloc(sizeof(double) * (size_t)(p + 1));
      double m = -INFINITY;
      for (int64_t j = 0; j <= p; ++j) {
        int64_t n = block_tables[b * bt_stride + j / MLA_BS];
        double acc = 0.0;
        for (int64_t d = 0; d < MLA_DL; ++d)
          acc += bf16_to_double(q[(t * Hq + h) * MLA_DL + d]) *
                 bf16_to_double(cache[mla_index(n, j % MLA_BS, d)]);
        s[j] = sigma * acc;
        if (s[j] > m) m = s[j];
      }
      double den = 0.0;
      for (int64_t j = 0; j <= p; ++j) {
        s[j] = exp(s[j] - m);
        den += s[j];
      }
      for (int64_t e = 0; e < MLA_DV; ++e) {
        double num = 0.0;
        for (int64_t j = 0; j <= p; ++j) {
          int64_t n = block_tables[b * bt_stride + j / MLA_BS];
          num += s[j] * bf16_to_double(cache[mla_index(n, j % MLA_BS, e)]);
        }
        out[(t * Hq + h) * MLA_DV + e] = num / den;
      }
      free(s);
    }
  }
}

/* ---- attention ---------------------------------------------------------- */

/* Softmax-weighted sum over keys 0..p of one (query row, head), given the
 * scores s[0..p] already computed; v_at(j, d) supplies V.  Shared by the paged
 * and the dense form: the two differ only in how K and V are addressed. */
typedef double (*v_fetch_fn)(const void *ctx, int64_t j, int64_t d);

static void softmax_weighted_sum(const double *s, int64_t p, v_fetch_fn v_at,
                                 const void *ctx, int64_t D, double *out) {
  double m = s[0];
  for (int64_t j = 1; j <= p; ++j)
    if (s[j] > m) m = s[j];
  double denom = 0.0;
  for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
  for (int64_t j = 0; j <= p; ++j) {
    double w = exp(s[j] - m);
    denom += w;
    for (int64_t d = 0; d < D; ++d) out[d] += w * v_at(ctx, j, d);
  }
  for (int64_t d = 0; d < D; ++d) out[d] /= denom;
}

/* The pools one attention reads: bf16 (k_cache, v_cache) or 8-bit codes
 * (k8, v8) whose values are decode(code) * scale, in fp64. */
typedef struct {
  const uint16_t *k_cache, *v_cache;
  const uint8_t *k8, *v8;
  double k_scale, v_scale;
  const int32_t *bt_row;
  int64_t g, Hkv, bs, D;
} paged_ctx;

static double paged_k(const paged_ctx *c, int64_t j, int64_t d) {
  int64_t n = c->bt_row[j / c->bs];
  if (c->k8)
    return oracle_e4m3_decode(
               c->k8[k8_index(n, c->g, j % c->bs, d, c->Hkv, c->bs, c->D)]) *
           c->k_scale;
  return bf16_to_double(
      c->k_cache[k_index(n, c->g, j % c->bs, d, c->Hkv, c->bs, c->D)]);
}

static double paged_v(const void *ctx, int64_t j, int64_t d) {
  const paged_ctx *c = (const paged_ctx *)ctx;
  int64_t n = c->bt_row[j / c->bs];
  if (c->v8)
    return oracle_e4m3_decode(
               c->v8[v8_index(n, c->g, j % c->bs, d, c->Hkv, c->bs, c->D)]) *
           c->v_scale;
  return bf16_to_double(
      c->v_cache[v_index(n, c->g, j % c->bs, d, c->Hkv, c->bs, c->D)]);
}

/* One output row: query token t (global index) of sequence b, query head h;
 * pools and layout from *pools (its bt_row and g are set here). */
static void paged_row(const uint16_t *q, const paged_ctx *pools,
                      const int32_t *block_tables, int64_t bt_stride,
                      const int32_t *seq_lens, const int32_t *query_start_loc,
                      int64_t b, int64_t t, int64_t h, int64_t Hq, double sigma,
                      double *scores, double *out) {
  int64_t L = seq_lens[b];
  int64_t Q = query_start_loc[b + 1] - query_start_loc[b];
  int64_t i = t - query_start_loc[b];
  int64_t p = L - Q + i; /* position of this query; it sees keys 0..p */
  int64_t D = pools->D;
  paged_ctx c = *pools;
  c.bt_row = block_tables + b * bt_stride;
  c.g = h / (Hq / pools->Hkv);
  const uint16_t *qrow = q + (size_t)((t * Hq + h) * D);
  for (int64_t j = 0; j <= p; ++j) {
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d)
      dot += bf16_to_double(qrow[d]) * paged_k(&c, j, d);
    scores[j] = sigma * dot;
  }
  softmax_weighted_sum(scores, p, paged_v, &c, D, out);
}

/* Sequence that owns global query token t (query_start_loc is
 * non-decreasing). */
static int64_t seq_of_token(const int32_t *query_start_loc, int64_t num_seqs,
                            int64_t t) {
  for (int64_t b = 0; b < num_seqs; ++b)
    if (t < query_start_loc[b + 1]) return b;
  return -1;
}

/* Rows rows[2r] = query token t, rows[2r+1] = query head h (all rows when
 * rows is NULL: r = t * Hq + h); out[r][d]. */
static void attend_impl(const uint16_t *q, const paged_ctx *pools,
                        const int32_t *block_tables, int64_t bt_stride,
                        const int32_t *seq_lens, const int32_t *query_start_loc,
                        int64_t num_seqs, int64_t Hq, float scale,
                        int64_t max_seq_len, const int64_t *rows,
                        int64_t num_rows, double *scratch, double *out,
                        int nthreads) {
  double sigma = (double)scale;
  int64_t D = pools->D;
  (void)nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t r = 0; r < num_rows; ++r) {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    int64_t t = rows ? rows[2 * r] : r / Hq;
    int64_t h = rows ? rows[2 * r + 1] : r % Hq;
    int64_t b = seq_of_token(query_start_loc, num_seqs, t);
    paged_row(q, pools, block_tables, bt_stride, seq_lens, query_start_loc, b,
              t, h, Hq, sigma, scratch + (size_t)tid * (size_t)max_seq_len,
              out + (size_t)(r * D));
  }
}

/* out[t][h][d] (fp64) for every query token of every sequence. */
void oracle_attend(const uint16_t *q, const uint16_t *k_cache,
                   const uint16_t *v_cache, const int32_t *block_tables,
                   int64_t bt_stride, const int32_t *seq_lens,
                   const int32_t *query_start_loc, int64_t num_seqs,
                   int64_t Hq, int64_t Hkv, int64_t bs, int64_t D, float scale,
                   int64_t max_seq_len, double *scratch, double *out,
                   int nthreads) {
  paged_ctx pools = {k_cache, v_cache, NULL, NULL, 1.0, 1.0, NULL, 0, Hkv, bs, D};
  attend_impl(q, &pools, block_tables, bt_stride, seq_lens, query_start_loc,
              num_seqs, Hq, scale, max_seq_len, NULL,
              query_start_loc[num_seqs] * Hq, scratch, out, nthreads);
}

/* Selected rows only: rows[2r] = query token t, rows[2r+1] = query head h;
 * out_rows[r][d]. */
void oracle_attend_rows(const uint16_t *q, const uint16_t *k_cache,
                        const uint16_t *v_cache, const int32_t *block_tables,
                        int64_t bt_stride, const int32_t *seq_lens,
                        const int32_t *query_start_loc, int64_t num_seqs,
                        int64_t Hq, int64_t Hkv, int64_t bs, int64_t D,
                        float scale, int64_t max_seq_len, const int64_t *rows,
                        int64_t num_rows, double *scratch, double *out_rows,
                        int nthreads) {
  paged_ctx pools = {k_cache, v_cache, NULL, NULL, 1.0, 1.0, NULL, 0, Hkv, bs, D};
  attend_impl(q, &pools, block_tables, bt_stride, seq_lens, query_start_loc,
              num_seqs, Hq, scale, max_seq_len, rows, num_rows, scratch,
              out_rows, nthreads);
}

/* The same attention over 8-bit pools: K and V values are
 * decode(code) * k_scale and decode(code) * v_scale. */
void oracle_attend_fp8(const uint16_t *q, const uint8_t *k8, const uint8_t *v8,
                       float k_scale, float v_scale,
                       const int32_t *block_tables, int64_t bt_stride,
                       const int32_t *seq_lens, const int32_t *query_start_loc,
                       int64_t num_seqs, int64_t Hq, int64_t Hkv, int64_t bs,
                       int64_t D, float scale, int64_t max_seq_len,
                       const int64_t *rows, int64_t num_rows, double *scratch,
                       double *out, int nthreads) {
  paged_ctx pools = {NULL, NULL, k8, v8, (double)k_scale, (double)v_scale,
                     NULL, 0, Hkv, bs, D};
  if (!rows) num_rows = query_start_loc[num_seqs] * Hq;
  attend_impl(q, &pools, block_tables, bt_stride, seq_lens, query_start_loc,
              num_seqs, Hq, scale, max_seq_len, rows, num_rows, scratch, out,
              nthreads);
}

/* Dense form: K/V of sequence b are rows kv_start_b .. kv_start_b + L_b - 1
 * of contiguous [sum L][Hkv][D] arrays (kv_start = prefix sum of seq_lens).
 * No block tables; same scores and softmax. */
typedef struct {
  const uint16_t *v_dense;
  int64_t row0, g, Hkv, D;
} dense_ctx;

static double dense_v(const void *ctx, int64_t j, int64_t d) {
  const dense_ctx *c = (const dense_ctx *)ctx;
  return bf16_to_double(c->v_dense[(size_t)(((c->row0 + j) * c->Hkv + c->g) *
                                                c->D + d)]);
}

void oracle_attend_dense(const uint16_t *q, const uint16_t *k_dense,
                         const uint16_t *v_dense, const int32_t *seq_lens,
                         const int32_t *query_start_loc, int64_t num_seqs,
                         int64_t Hq, int64_t Hkv, int64_t D, float scale,
                         int64_t max_seq_len, double *scratch, double *out) {
  double sigma = (double)scale;
  int64_t row0 = 0;
  for (int64_t b = 0; b < num_seqs; ++b) {
    int64_t L = seq_lens[b];
    int64_t Q = query_start_loc[b + 1] - query_start_loc[b];
    for (int64_t i = 0; i < Q; ++i) {
      int64_t t = query_start_loc[b] + i;
      int64_t p = L - Q + i;
      for (int64_t h = 0; h < Hq; ++h) {
        int64_t g = h / (Hq / Hkv);
        const uint16_t *qrow = q + (size_t)((t * Hq + h) * D);
        for (int64_t j = 0; j <= p; ++j) {
          double dot = 0.0;
          for (int64_t d = 0; d < D; ++d)
            dot += bf16_to_double(qrow[d]) *
                   bf16_to_double(
                       k_dense[(size_t)(((row0 + j) * Hkv + g) * D + d)]);
          scratch[j] = sigma * dot;
        }
        dense_ctx c = {v_dense, row0, g, Hkv, D};
        softmax_weighted_sum(scratch, p, dense_v, &c, D,
                             out + (size_t)((t * Hq + h) * D));
      }
    }
    row0 += L;
  }
  (void)max_seq_len;
}

int oracle_abi_version(void) { return 1; }
