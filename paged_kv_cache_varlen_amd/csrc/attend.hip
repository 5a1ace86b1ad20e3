// Paged varlen causal attention over a mixed batch (chunked-prefill chunks and
// decodes in one launch), gfx950.
//
// What is computed ("Inside vLLM", Part 3, Step 4c and the Aside "KV cache and
// prefix caching"; "vLLM internals study" sections 2.1 and 2.4): for every
// query token of request b (its Q_b new tokens are the last Q_b of its L_b
// tokens, rows query_start_loc[b]..) and every query head h,
//     out = softmax_j(scale * q.K_j) V_j  over keys j = 0 .. p,  p = L_b - Q_b + i,
// K_j/V_j read from block block_tables[b][j/16], slot j%16, of the kv head
// h / G shared by the G query heads of its group.
//
// Structure (three kernels on one stream, no host synchronisation):
//   plan    one workgroup turns seq_lens / query_start_loc into a work list of
//           (request, query tile, logical key range) items, prefill items
//           first, and zeroes the work-queue head;
//   attend  persistent waves pull (item, kv head) units from the queue.  One
//           wave owns one unit: the query tile's columns (token x head of the
//           group) are MFMA columns, 16 keys (one block) are MFMA rows, so
//           every K/V tile is read once for all G heads.  Scores S^T = K Q^T
//           and the PV product O^T = V^T P^T run on v_mfma_f32_16x16x32_bf16;
//           the online softmax (running max / sum per column) is fp32 with
//           wavefront shuffles.  Items whose key range is the whole causal
//           range write bf16 out directly, split items write fp32 partials;
//   merge   log-sum-exp combination of the split partials in split order.
//
// Reduction order depends only on (Q_b, L_b) and logical key positions, so
// results are bitwise independent of physical block ids, of shared blocks and
// of the rest of the batch.
#include "pa_device.h"

namespace pa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

struct AttendParams {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  int64_t num_blocks;
  const int32_t* bt;
  int32_t bt_stride;
  const int32_t* seq_lens;
  const int32_t* qsl;
  int32_t num_seqs;
  int32_t num_q_tokens;
  int32_t Hq;
  int32_t Hkv;
  int32_t G;
  int32_t max_query_len;
  int32_t max_seq_len;
  float scale_log2;  // scale * log2(e): scores live in the exp2 domain
  uint16_t* out;
  PlanHeader* hdr;
  WorkItem* items;
  TokenSplit* token_split;
  float2* part_ml;
  float* part_acc;
  int64_t max_items;
  int64_t max_partials;
};

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

constexpr int kPlanThreads = 1024;

struct SeqCounts {
  int kind;      // -1: nothing to do
  int ntiles;
  int tq;        // tokens per tile
  int splitlen;  // logical tokens per split (0: unsplit)
  int items;
  int partials;
};

__device__ SeqCounts seq_counts(const AttendParams& P, int b) {
  SeqCounts c{-1, 0, 0, 0, 0, 0};
  const int q0 = P.qsl[b], q1 = P.qsl[b + 1];
  const int Q = q1 - q0, L = P.seq_lens[b];
  const bool ok = q0 >= 0 && Q >= 0 && q1 <= P.num_q_tokens && Q <= L &&
                  L <= P.max_seq_len && Q <= P.max_query_len &&
                  ((L + kBlock - 1) / kBlock) <= P.bt_stride;
  if (!ok) {
    atomicOr(&P.hdr->error, 2u);
    return c;
  }
  if (Q == 0) return c;
  const int tq_d = decode_tile_tokens(P.G);
  if (Q <= tq_d) {
    c.kind = kKindDecode;
    c.ntiles = 1;
    c.tq = Q;
    c.splitlen = kSplitDecode;
    const int ns = (L + kSplitDecode - 1) / kSplitDecode;
    c.items = ns;
    c.partials = ns > 1 ? Q * ns : 0;
    return c;
  }
  c.kind = kKindPrefill;
  c.tq = prefill_tile_tokens(P.G);
  c.ntiles = (Q + c.tq - 1) / c.tq;
  c.splitlen = (c.ntiles * P.Hkv < kPrefillUnsplitUnits) ? kSplitPrefill : 0;
  for (int t = 0; t < c.ntiles; ++t) {
    const int ntok = min(c.tq, Q - t * c.tq);
    const int pmax1 = L - Q + t * c.tq + ntok;
    const int ns = c.splitlen ? (pmax1 + c.splitlen - 1) / c.splitlen : 1;
    c.items += ns;
    c.partials += ns > 1 ? ntok * ns : 0;
  }
  return c;
}

// Exclusive scan over the workgroup; *total receives the sum.
__device__ int block_scan(int x, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int kWaves = kPlanThreads / 64;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) lds[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const int v = lane < kWaves ? lds[lane] : 0;
    int vi = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(vi, off);
      if (lane >= off) vi += y;
    }
    if (lane < kWaves) lds[lane] = vi - v;
    if (lane == kWaves - 1) lds[kWaves] = vi;
  }
  __syncthreads();
  const int res = incl - x + lds[wid];
  *total = lds[kWaves];
  __syncthreads();
  return res;
}

__device__ void emit_seq(const AttendParams& P, int b, const SeqCounts& c,
                         int ibase, int pbase) {
  const int q0 = P.qsl[b];
  const int Q = P.qsl[b + 1] - q0, L = P.seq_lens[b];
  if (c.kind == kKindDecode) {
    const int ns = c.items;
    const int pb = ns > 1 ? pbase : -1;
    for (int s = 0; s < ns; ++s) {
      WorkItem it;
      it.seq = b;
      it.tok0 = q0;
      it.ntok = Q;
      it.kind = kKindDecode;
      it.kv0 = s * kSplitDecode;
      it.kv1 = min(L, (s + 1) * kSplitDecode);
      it.split = s;
      it.pbase = pb;
      P.items[ibase + s] = it;
    }
    for (int k = 0; k < Q; ++k)
      P.token_split[q0 + k] = TokenSplit{pb < 0 ? -1 : pb + k * ns, ns};
    return;
  }
  // prefill: longest tiles (latest tokens) first
  int icur = ibase, pcur = pbase;
  for (int t = c.ntiles - 1; t >= 0; --t) {
    const int ntok = min(c.tq, Q - t * c.tq);
    const int pmax1 = L - Q + t * c.tq + ntok;
    const int ns = c.splitlen ? (pmax1 + c.splitlen - 1) / c.splitlen : 1;
    const int span = c.splitlen ? c.splitlen : pmax1;
    const int pb = ns > 1 ? pcur : -1;
    if (ns > 1) pcur += ntok * ns;
    for (int s = 0; s < ns; ++s) {
      WorkItem it;
      it.seq = b;
      it.tok0 = q0 + t * c.tq;
      it.ntok = ntok;
      it.kind = kKindPrefill;
      it.kv0 = s * span;
      it.kv1 = min(pmax1, (s + 1) * span);
      it.split = s;
      it.pbase = pb;
      P.items[icur++] = it;
    }
    for (int k = 0; k < ntok; ++k)
      P.token_split[q0 + t * c.tq + k] =
          TokenSplit{pb < 0 ? -1 : pb + k * ns, ns};
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(AttendParams P) {
  __shared__ int lds[kPlanThreads / 64 + 1];
  const int tid = threadIdx.x;
  if (tid == 0) {
    P.hdr->work_counter = 0;
    P.hdr->error = 0;
  }
  // Tokens of skipped requests keep this record: the merge leaves them alone.
  for (int t = tid; t < P.num_q_tokens; t += kPlanThreads)
    P.token_split[t] = TokenSplit{-1, 1};
  __syncthreads();
  // sweep 1: total prefill items, so that decode items go after them
  int pre_total = 0, all_items = 0, all_partials = 0;
  for (int base = 0; base < P.num_seqs; base += kPlanThreads) {
    const int b = base + tid;
    SeqCounts c{-1, 0, 0, 0, 0, 0};
    if (b < P.num_seqs) c = seq_counts(P, b);
    int t0, t1, t2;
    block_scan(c.kind == kKindPrefill ? c.items : 0, lds, &t0);
    block_scan(c.items, lds, &t1);
    block_scan(c.partials, lds, &t2);
    pre_total += t0;
    all_items += t1;
    all_partials += t2;
  }
  const bool fits = all_items <= P.max_items && all_partials <= P.max_partials;
  // sweep 2: write
  int pre_carry = 0, dec_carry = 0, part_carry = 0;
  for (int base = 0; base < P.num_seqs; base += kPlanThreads) {
    const int b = base + tid;
    SeqCounts c{-1, 0, 0, 0, 0, 0};
    if (b < P.num_seqs) c = seq_counts(P, b);
    int tp, td, tpart;
    const int ep = block_scan(c.kind == kKindPrefill ? c.items : 0, lds, &tp);
    const int ed = block_scan(c.kind == kKindDecode ? c.items : 0, lds, &td);
    const int epart = block_scan(c.partials, lds, &tpart);
    if (fits && c.kind >= 0) {
      const int ibase = c.kind == kKindPrefill ? pre_carry + ep
                                               : pre_total + dec_carry + ed;
      emit_seq(P, b, c, ibase, part_carry + epart);
    }
    pre_carry += tp;
    dec_carry += td;
    part_carry += tpart;
  }
  if (tid == 0) {
    P.hdr->num_items = fits ? (uint32_t)all_items : 0u;
    P.hdr->num_work = fits ? (uint32_t)all_items * (uint32_t)P.Hkv : 0u;
    if (!fits) P.hdr->error |= 1u;
  }
}

// ---------------------------------------------------------------------------
// attend
// ---------------------------------------------------------------------------

__device__ __forceinline__ bf16x8 load16(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D>
struct KVPair {
  bf16x8 k[2][D / 32];  // block a, block b: K rows in MFMA operand order
  bf16x8 v[2][D / 32];  // V^T rows: lanes' 4 keys at dims d and d + D/2
};

// One (item, kv head) unit on one wave.  CT = MFMA column tiles of 16;
// PIPE = 2 keeps the next block pair's loads in flight while the current pair
// is computed, PIPE = 1 loads and computes one pair at a time.
template <int D, int CT, int PIPE>
__device__ __forceinline__ void run_item(const AttendParams& P,
                                         const WorkItem& it, int kvh,
                                         int lane) {
  constexpr int KC = D / 32;  // 32-dim chunks = MFMA k-steps for QK^T
  constexpr int NT = D / 16;  // 16-dim output tiles for PV
  const int r = lane & 15, g = lane >> 4;
  const int b = it.seq;
  const int L = P.seq_lens[b];
  const int q0 = P.qsl[b];
  const int Q = P.qsl[b + 1] - q0;
  const int G = P.G;
  const int posbase = L - Q + (it.tok0 - q0);  // position of tile token 0
  const int ncols = it.ntok * G;

  // Q^T operand: column = (token, head-in-group); lane holds 8 dims.
  bf16x8 qop[CT][KC];
  int cpos[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = ct * 16 + r;
    const int tk = col / G;
    const int hh = col - tk * G;
    const bool valid = col < ncols;
    cpos[ct] = valid ? posbase + tk : -1;
    if (valid) {
      const uint16_t* qp =
          P.q + ((int64_t)(it.tok0 + tk) * P.Hq + kvh * G + hh) * D + 8 * g;
#pragma unroll
      for (int c = 0; c < KC; ++c) qop[ct][c] = load16(qp + 32 * c);
    } else {
#pragma unroll
      for (int c = 0; c < KC; ++c) qop[ct][c] = zero8();
    }
  }

  f32x4 acc[CT][NT];
  float mrun[CT], lsum[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    mrun[ct] = -INFINITY;
    lsum[ct] = 0.0f;
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[ct][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int jb0 = it.kv0 >> 4;
  const int jb1 = (it.kv1 + kBlock - 1) >> 4;
  const int nblk = jb1 - jb0;
  const int npairs = (nblk + 1) >> 1;
  const int32_t* btrow = P.bt + (int64_t)b * P.bt_stride;
  const int64_t tile_elems = (int64_t)kBlock * D;
  const int64_t maxblk = P.num_blocks - 1;

  // Physical block ids of 64 consecutive logical blocks, one per lane.
  int idv = 0;
  int chunk = -1;
  auto ensure_ids = [&](int rel) {
    const int want = rel >> 6;
    if (want != chunk) {
      chunk = want;
      const int j = jb0 + (want << 6) + lane;
      int id = j < jb1 ? btrow[j] : 0;
      id = id < 0 ? 0 : (id > maxblk ? (int)maxblk : id);
      idv = id;
    }
  };

  auto issue = [&](KVPair<D>& buf, int pr) {
    const int rel = 2 * pr;
    ensure_ids(rel);
    const int ia = __builtin_amdgcn_readlane(idv, rel & 63);
    const bool has_b = rel + 1 < nblk;
    const int ib = __builtin_amdgcn_readlane(idv, (rel + 1) & 63);
    const uint16_t* ka = P.k_cache + ((int64_t)ia * P.Hkv + kvh) * tile_elems;
    const uint16_t* va = P.v_cache + ((int64_t)ia * P.Hkv + kvh) * tile_elems;
#pragma unroll
    for (int c = 0; c < KC; ++c) buf.k[0][c] = load16(ka + c * 512 + lane * 8);
#pragma unroll
    for (int c = 0; c < KC; ++c)
      buf.v[0][c] = load16(va + c * 512 + (4 * r + g) * 8);
    if (has_b) {
      const uint16_t* kb = P.k_cache + ((int64_t)ib * P.Hkv + kvh) * tile_elems;
      const uint16_t* vb = P.v_cache + ((int64_t)ib * P.Hkv + kvh) * tile_elems;
#pragma unroll
      for (int c = 0; c < KC; ++c) buf.k[1][c] = load16(kb + c * 512 + lane * 8);
#pragma unroll
      for (int c = 0; c < KC; ++c)
        buf.v[1][c] = load16(vb + c * 512 + (4 * r + g) * 8);
    } else {
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        buf.k[1][c] = zero8();
        buf.v[1][c] = zero8();
      }
    }
  };

  auto compute = [&](KVPair<D>& buf, int pr) {
    const int kp0 = (jb0 + 2 * pr) * kBlock;  // logical position of key 0 of block a
    // keys at or past kv1 may be unwritten pool slots: zero their V so that
    // 0-weight x NaN cannot reach the accumulator.
    if (kp0 + 2 * kBlock > it.kv1) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool dead = kp0 + 16 * x + 4 * g + i >= it.kv1;
#pragma unroll
          for (int c = 0; c < KC; ++c) {
            if (dead) {
              buf.v[x][c][i] = (__bf16)0.0f;
              buf.v[x][c][i + 4] = (__bf16)0.0f;
            }
          }
        }
      }
    }
    const bool need_mask = kp0 + 2 * kBlock - 1 > posbase;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) sa = mfma(buf.k[0][c], qop[ct][c], sa);
#pragma unroll
      for (int c = 0; c < KC; ++c) sb = mfma(buf.k[1][c], qop[ct][c], sb);
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = sa[i] * P.scale_log2;
        x[i + 4] = sb[i] * P.scale_log2;
      }
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ka = kp0 + 4 * g + i;
          if (ka > cpos[ct]) x[i] = -INFINITY;
          if (ka + kBlock > cpos[ct]) x[i + 4] = -INFINITY;
        }
      }
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun[ct], mx);
      const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(mrun[ct] - muse);
      mrun[ct] = mnew;
      bf16x8 pop;
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const __bf16 pb = (__bf16)__builtin_amdgcn_exp2f(x[i] - muse);
        pop[i] = pb;
        psum += (float)pb;
      }
      lsum[ct] = lsum[ct] * alpha + psum;
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[ct][n] *= alpha;
#pragma unroll
      for (int n = 0; n < KC; ++n) {
        const bf16x8 vlo = __builtin_shufflevector(buf.v[0][n], buf.v[1][n], 0,
                                                   1, 2, 3, 8, 9, 10, 11);
        acc[ct][n] = mfma(vlo, pop, acc[ct][n]);
      }
#pragma unroll
      for (int n = 0; n < KC; ++n) {
        const bf16x8 vhi = __builtin_shufflevector(buf.v[0][n], buf.v[1][n], 4,
                                                   5, 6, 7, 12, 13, 14, 15);
        acc[ct][n + KC] = mfma(vhi, pop, acc[ct][n + KC]);
      }
    }
  };

  if (PIPE == 2) {
    if (npairs > 0) {
      KVPair<D> b0, b1;
      issue(b0, 0);
      for (int pr = 0; pr < npairs; pr += 2) {
        if (pr + 1 < npairs) issue(b1, pr + 1);
        compute(b0, pr);
        if (pr + 1 >= npairs) break;
        if (pr + 2 < npairs) issue(b0, pr + 2);
        compute(b1, pr + 1);
      }
    }
  } else {
    for (int pr = 0; pr < npairs; ++pr) {
      KVPair<D> b0;
      issue(b0, pr);
      compute(b0, pr);
    }
  }

  // epilogue
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    float l = lsum[ct];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int col = ct * 16 + r;
    if (col >= ncols) continue;
    const int tk = col / G;
    const int hh = col - tk * G;
    const int64_t t = it.tok0 + tk;
    const int h = kvh * G + hh;
    if (it.pbase < 0) {
      const float inv = 1.0f / l;
      uint16_t* op = P.out + (t * P.Hq + h) * D + 4 * g;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        bf16x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc[ct][n][i] * inv);
        *reinterpret_cast<bf16x4*>(op + 16 * n) = o;
      }
    } else {
      const int ns = P.token_split[t].nsplit;
      const int64_t slot = (int64_t)it.pbase + (int64_t)tk * ns + it.split;
      float* ap = P.part_acc + (slot * P.Hq + h) * D + 4 * g;
#pragma unroll
      for (int n = 0; n < NT; ++n)
        *reinterpret_cast<f32x4*>(ap + 16 * n) = acc[ct][n];
      if (g == 0) P.part_ml[slot * P.Hq + h] = make_float2(mrun[ct], l);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kAttendThreads)
__attribute__((amdgpu_waves_per_eu(kAttendWavesPerSimd, 8)))
void attend_kernel(AttendParams P) {
  const int lane = threadIdx.x & 63;
  const uint32_t num_work = P.hdr->num_work;
  const uint32_t Hkv = (uint32_t)P.Hkv;
  while (true) {
    uint32_t w = 0;
    if (lane == 0) w = atomicAdd(&P.hdr->work_counter, 1u);
    w = __shfl(w, 0);
    w = __builtin_amdgcn_readfirstlane(w);
    if (w >= num_work) break;
    const WorkItem it = P.items[w / Hkv];
    const int kvh = (int)(w % Hkv);
    if (it.kind == kKindPrefill)
      run_item<D, kPrefillColTiles, 1>(P, it, kvh, lane);
    else
      run_item<D, kDecodeColTiles, 2>(P, it, kvh, lane);
  }
}

// ---------------------------------------------------------------------------
// merge
// ---------------------------------------------------------------------------

// One wave per (token, head); lanes cover head_dim.
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(AttendParams P) {
  constexpr int PER = D / 64;
  const int64_t th = blockIdx.x;
  const int64_t t = th / P.Hq;
  const int h = (int)(th - t * P.Hq);
  const TokenSplit ts = P.token_split[t];
  if (ts.nsplit <= 1 || ts.pbase < 0) return;
  const int lane = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < ts.nsplit; ++s)
    M = fmaxf(M, P.part_ml[((int64_t)ts.pbase + s) * P.Hq + h].x);
  float den = 0.0f;
  float num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.0f;
  for (int s = 0; s < ts.nsplit; ++s) {
    const int64_t slot = (int64_t)ts.pbase + s;
    const float2 ml = P.part_ml[slot * P.Hq + h];
    const float w = __builtin_amdgcn_exp2f(ml.x - M);
    den += w * ml.y;
    const float* ap = P.part_acc + (slot * P.Hq + h) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] += w * ap[lane * PER + e];
  }
  const float inv = 1.0f / den;
  uint16_t* op = P.out + (t * P.Hq + h) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const __bf16 o = (__bf16)(num[e] * inv);
    op[lane * PER + e] = *reinterpret_cast<const uint16_t*>(&o);
  }
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, hipStream_t stream) {
  if (a.num_q_tokens == 0 || a.num_seqs == 0) return hipSuccess;
  AttendParams P;
  P.q = a.q;
  P.k_cache = a.k_cache;
  P.v_cache = a.v_cache;
  P.num_blocks = a.num_blocks;
  P.bt = a.block_tables;
  P.bt_stride = a.bt_stride;
  P.seq_lens = a.seq_lens;
  P.qsl = a.qsl;
  P.num_seqs = a.num_seqs;
  P.num_q_tokens = (int32_t)a.num_q_tokens;
  P.Hq = a.num_q_heads;
  P.Hkv = a.num_kv_heads;
  P.G = a.num_q_heads / a.num_kv_heads;
  P.max_query_len = a.max_query_len;
  P.max_seq_len = a.max_seq_len;
  P.scale_log2 = a.scale * kLog2e;
  P.out = a.out;
  char* ws = static_cast<char*>(a.workspace);
  P.hdr = reinterpret_cast<PlanHeader*>(ws);
  P.items = reinterpret_cast<WorkItem*>(ws + a.ws.items);
  P.token_split = reinterpret_cast<TokenSplit*>(ws + a.ws.token_split);
  P.part_ml = reinterpret_cast<float2*>(ws + a.ws.part_ml);
  P.part_acc = reinterpret_cast<float*>(ws + a.ws.part_acc);
  P.max_items = a.ws.max_items;
  P.max_partials = a.ws.max_partials;

  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // Persistent grid: enough waves to fill every CU at the kernel's
  // occupancy, never more than the work-unit bound.
  const int64_t max_work = a.ws.max_items * a.num_kv_heads;
  int64_t waves = (int64_t)a.num_cus * 4 * kAttendWavesPerSimd;
  if (waves > max_work) waves = max_work;
  const int64_t wgs = (waves + (kAttendThreads / 64) - 1) / (kAttendThreads / 64);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(attend_kernel<128>, dim3((unsigned)wgs),
                       dim3(kAttendThreads), 0, stream, P);
  else
    hipLaunchKernelGGL(attend_kernel<64>, dim3((unsigned)wgs),
                       dim3(kAttendThreads), 0, stream, P);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int64_t rows = a.num_q_tokens * a.num_q_heads;
  if (a.head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)rows), dim3(64), 0,
                       stream, P);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)rows), dim3(64), 0,
                       stream, P);
  return hipGetLastError();
}

}  // namespace pa
