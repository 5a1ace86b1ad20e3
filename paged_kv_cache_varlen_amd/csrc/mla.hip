// Multi-head latent attention (MLA) over a paged latent cache: one 576-dim
// vector per token (512 latent + 64 rotary dims) shared by every query head,
// in blocks of 64 tokens; decode attends MQA-style on the latent.
//
// Cache layout: block n holds 64 * 576 bf16; token t, dim d of the block is
// element (((t / 16) * 18 + d / 32) * 16 + t % 16) * 32 + d % 32.  A 16-token
// sub-tile is 18 KiB of [32-dim chunk][16 tokens][32 dims] (one KiB piece per
// chunk), so tokens 32s .. 32s+31 of a block (s = 0, 1) are 36 KiB contiguous.
//
// Decode (mla_decode_kernel).  The work is a stream of items: the requests
// in order, each group of G consecutive query tokens of a request in order
// (G = 1, or 128 / Hq for batches of multi-token requests with 16, 32 or 64
// heads), a few head items for the group's query stages, then the keys its
// last token sees in stages of SK (16 for up to 32 heads with G = 1, else
// 32).  The stream is cut into contiguous ranges of R = ceil(items /
// gridDim.x) items, one per workgroup, so every workgroup reads about the
// same latent bytes whatever the mix of lengths; a group whose keys are cut
// between workgroups leaves one partial result per workgroup, folded by
// mla_merge_kernel.
//
// A workgroup has one wave per 16 (token, head) rows of a group (for 16 and
// 32 heads with G = 1, one wave per (16 heads, quarter / half of the 512
// output dims)).  Its stages pass
// through a ring of four LDS buffers (18 KiB for SK = 16, two workgroups per
// CU; 36 KiB for SK = 32), filled three stages ahead by global-to-LDS loads
// that the waves share; each wave then reads the stage from LDS for
//  - the scores S^T = K Q^T (MFMA 16x16x32, keys x heads): the key operand
//    is one 16-byte LDS read per lane per 32-dim chunk and 16 keys, the
//    query operand stays in registers;
//  - the weighted sum O^T += V^T P^T (MFMA 16x16x32 over 32 keys, 16x16x16
//    over 16): the V^T operand
//    (four consecutive keys of one dim per lane, where the cache holds
//    consecutive dims of one key) comes from the LDS transpose read
//    ds_read_b64_tr_b16, so the latent is fetched from HBM once and needs
//    no transposed copy.
// Each 1 KiB piece of a stage lands in LDS XOR-swizzled: the 16-byte granule
// of (token k, 8-dim group g) sits at granule g * 16 + (k ^ (12 * (g & 1)))
// of its piece, which keeps both LDS read patterns free of bank conflicts.
#include "mfma_util.h"
#include "mla_device.h"

namespace pa {
namespace {

constexpr int kKc = kMlaDim / 32;              // 18 chunks of 32 dims
constexpr int kSubBytes = 16 * kMlaDim * 2;    // 18 KiB: 16 tokens
constexpr int kRing = 4;                       // LDS stage buffers
// A stage of SK keys (16 or 32): SK / 16 sub-tiles of 18 KiB, kPieces
// one-KiB loads, 64 / SK stages per block; a range's stage table holds
// kTable entries.
template <int SK>
struct Geo {
  static constexpr int kSubs = SK / 16;
  static constexpr int kStageBytes = kSubs * kSubBytes;
  static constexpr int kPieces = kStageBytes / 1024;
  static constexpr int kPerBlock = kMlaBlock / SK;
  static constexpr int kTable = mla_table_entries(SK);
};
constexpr int64_t kBlockElems = (int64_t)kMlaBlock * kMlaDim;
// A new maximum is taken only when a score exceeds the one in use by more
// than this (log2 units): the exponentials stay <= 2^8, and the rescale of
// the accumulators is skipped for most stages.
constexpr float kSlack = 8.0f;

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt not waited), as an immediate the
// compiler's own wait insertion sees.
constexpr int kWaitLgkm0 = 0xC07F;

// Scalar-memory load of a wave-uniform address (tracked by lgkmcnt, not by
// the vector-memory counter that orders the stage ring).
template <class T>
__device__ __forceinline__ T sload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// A request's metadata is in bounds: its tokens inside [0, T), Q <= L,
// L <= max_seq_len and its blocks inside its block-table row.
__device__ __forceinline__ bool req_ok(const MlaParams& P, int q0, int q1, int L) {
  return q0 >= 0 && q1 >= q0 && q1 <= P.num_q_tokens && q1 - q0 <= L &&
         L <= P.max_seq_len && (L + kMlaBlock - 1) / kMlaBlock <= P.bt_stride;
}

// Key stages of the first k groups of G query tokens of a request, all full
// groups, whose k'-th group's last token sees a + k' G keys: the sum of
// ceil((a + k' G) / SK).  With SK = m G that is floor((c + k') / m),
// c = floor((a + SK - 1) / G), whose partial sums have a closed form.
template <int SK>
__device__ __forceinline__ int64_t group_prefix(int64_t k, int64_t a, int G) {
  const int64_t m = SK / G, c = (a + SK - 1) / G;
  auto tri = [m](int64_t n) {  // sum_{x < n} floor(x / m)
    const int64_t q = n / m, r = n % m;
    return m * q * (q - 1) / 2 + q * r;
  };
  return tri(c + k) - tri(c);
}

// Stream items of a request of Q query tokens and L keys in groups of G:
// per group, qw head items, then the stages of the keys its last token sees
// (query i of the Q sees L - Q + 1 + i keys; a last partial group's last
// token sees L).
template <int SK>
__device__ __forceinline__ int64_t items_of(int Q, int L, int G, int qw) {
  if (Q <= 0) return 0;
  const int ng = (Q + G - 1) / G;
  return (int64_t)ng * qw + group_prefix<SK>(ng - 1, L - Q + G, G) + (L + SK - 1) / SK;
}

// Stream items of request b (vector loads, one request per lane; 0 past the
// end or out of bounds).
template <int SK>
__device__ __forceinline__ int64_t req_items(const MlaParams& P, int b, int qw, int G) {
  if (b >= P.num_seqs) return 0;
  const int q0 = P.qsl[b], q1 = P.qsl[b + 1], L = P.seq_lens[b];
  if (!req_ok(P, q0, q1, L)) return 0;
  return items_of<SK>(q1 - q0, L, G, qw);
}

__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Range of workgroup b of a grid of g: with g = 8 q + r, the workgroups
// b = x (mod 8) (those of XCD x) take ranges x q + min(x, r) + b / 8 onward,
// a bijection of [0, g).
__device__ __forceinline__ int xcd_range(int b, int g) {
  const int x = b & 7, q = g >> 3, r = g & 7;
  return x * q + min(x, r) + (b >> 3);
}

// Inclusive prefix sum over the wave's 64 lanes.
__device__ __forceinline__ int64_t wave_scan(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  return v;
}

// Position in the stream: request b (metadata q0, Q, L), its group i of
// ntok query tokens (tokens q0 + G i ..), stage j of the group's nst stages
// (those of the nvis keys its last token sees).  Every field is
// wave-uniform.
struct Cursor {
  int b, q0, Q, L;
  int i, j, nst, ntok, nvis;
};

template <int SK>
__device__ __forceinline__ void cursor_group(Cursor& c, int G) {
  c.ntok = min(G, c.Q - c.i * G);
  c.nvis = c.L - c.Q + c.i * G + c.ntok;
  c.nst = (c.nvis + SK - 1) / SK;
}

// Metadata of the requests b0 .. b0 + 63, one per lane (loaded once), and
// scalar loads past them.
struct ReqWindow {
  int b0, q0, q1, L;
  __device__ __forceinline__ void get(const MlaParams& P, int b, int& rq0, int& rq1,
                                      int& rL) const {
    if (b - b0 < 64) {
      rq0 = __builtin_amdgcn_readlane(q0, b - b0);
      rq1 = __builtin_amdgcn_readlane(q1, b - b0);
      rL = __builtin_amdgcn_readlane(L, b - b0);
    } else {
      rq0 = sload(P.qsl + b);
      rq1 = sload(P.qsl + b + 1);
      rL = sload(P.seq_lens + b);
    }
  }
};

// Next stage; past a request's last token the next request with tokens whose
// metadata is in bounds.  Called only while stages remain, which the
// stream's total guarantees; past num_seqs it stops on a dummy position,
// never used.
template <int SK>
__device__ __forceinline__ void cursor_next(Cursor& c, const MlaParams& P,
                                            const ReqWindow& win, int G) {
  if (++c.j < c.nst) return;
  c.j = 0;
  if (++c.i >= (c.Q + G - 1) / G) {
    c.i = 0;
    for (;;) {
      if (++c.b >= P.num_seqs) {
        c.b = P.num_seqs - 1;
        c.q0 = 0;
        c.Q = 1;
        c.L = 1;
        break;
      }
      int q0, q1, L;
      win.get(P, c.b, q0, q1, L);
      if (q1 > q0 && req_ok(P, q0, q1, L)) {
        c.q0 = q0;
        c.Q = q1 - q0;
        c.L = L;
        break;
      }
    }
  }
  cursor_group<SK>(c, G);
}

// Global-to-LDS copy of one KiB: lane i reads 16 bytes at gaddr + voff and
// writes them to LDS at laddr + 16 i (non-temporal: streamed once).  Inline
// assembly, so that the compiler's wait insertion does not track it (it
// would wait for every such load before any LDS read); the ring waits for
// them itself.  M0 holds the LDS address; five wait states after writing it
// and the SGPR address pair cover the hazards; M0 is restored.
__device__ __forceinline__ void dma_kib(uint64_t gaddr, uint32_t voff, uint32_t laddr) {
  // (the addresses are wave-uniform; readfirstlane makes that visible, so
  // that they sit in SGPRs.  It returns an int: each half goes through a
  // uint32_t, or the low half would be sign-extended into the high one.)
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)gaddr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(gaddr >> 32));
  gaddr = ((uint64_t)hi << 32) | lo;
  laddr = __builtin_amdgcn_readfirstlane(laddr);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 4\n\t"
      "global_load_lds_dwordx4 %1, %2 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(gaddr), "s"(laddr)
      : "memory");
}

// Entries of a range's stage table: a key stage is block id * 4 + which SK
// keys of the block (bit 31 clear); a query stage is kQStage | t0 << 6 |
// (ntok - 1) << 3 | k: (token, head) rows SK k .. SK k + SK - 1 of the group
// of ntok tokens from token t0 (its rows t0 Hq .. are consecutive in q;
// SK * 1152 bytes, fewer for the last), which precede the group's key
// stages.
constexpr uint32_t kQStage = 0x80000000u;

// This wave's share of a stage's loads: nl of its `pieces` one-KiB pieces,
// p0 .. p0 + nl - 1 modulo pieces (past the end they repeat pieces another
// wave also loads: the same bytes to the same place), so every wave issues
// exactly nl loads per stage, key stage or query stage.
template <int SK>
__device__ __forceinline__ void dma_stage(const MlaParams& P, uint32_t e, uint32_t lstage,
                                          uint32_t voff, int p0, int nl) {
  uint64_t g;
  int pieces;
  uint32_t vo;
  if (e & kQStage) {
    const int64_t t = (e & ~kQStage) >> 6;
    const int ntok = (int)((e >> 3) & 7) + 1;
    const int k = e & 7;
    g = (uint64_t)(uintptr_t)(P.q + (t * P.Hq + SK * k) * kMlaDim);
    pieces = min(SK, ntok * P.Hq - SK * k) * (kMlaDim * 2) / 1024;
    vo = (uint32_t)(16 * (threadIdx.x & 63));
  } else {
    g = (uint64_t)(uintptr_t)(P.cache + (int64_t)(e >> 2) * kBlockElems) +
        (uint64_t)(e & 3) * Geo<SK>::kStageBytes;
    pieces = Geo<SK>::kPieces;
    vo = voff;
  }
  for (int x = 0; x < nl; ++x) {
    int p = p0 + x;
    while (p >= pieces) p -= pieces;
    dma_kib(g + (uint64_t)p * 1024, vo, lstage + (uint32_t)p * 1024);
  }
}

// Wait until this wave has at most 2 nl (+ extra) ring loads in flight -- the
// two stages issued after the one about to be read, plus the result stores
// of a piece finished in the last three stages, which count too -- then meet
// the other waves: after the barrier every wave's share of the stage is in
// LDS, and every wave has finished reading the buffer that is refilled next.
// (The counter retires in order, so the wait covers the stage as long as
// the allowance is no more than the operations issued after it: `extra` is
// at most the stores a piece issues, and none where the wave stored none.
// No LDS read is outstanding here: each was consumed before.)
#define MLA_WAIT(N) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory")
template <int EXTRA>
__device__ __forceinline__ void ring_wait(int nl, bool tail, bool stores) {
  static_assert(24 + EXTRA <= 63, "vmcnt immediate");
  if (tail) {
    MLA_WAIT(0);
    return;
  }
  switch (nl + (stores ? 100 : 0)) {
    case 5: MLA_WAIT(10); break;
    case 6: MLA_WAIT(12); break;
    case 8: MLA_WAIT(16); break;
    case 9: MLA_WAIT(18); break;
    case 12: MLA_WAIT(24); break;
    case 105: MLA_WAIT(10 + EXTRA); break;
    case 106: MLA_WAIT(12 + EXTRA); break;
    case 108: MLA_WAIT(16 + EXTRA); break;
    case 109: MLA_WAIT(18 + EXTRA); break;
    case 112: MLA_WAIT(24 + EXTRA); break;
    default: MLA_WAIT(0); break;
  }
}
#undef MLA_WAIT

__device__ __forceinline__ s16x4 lds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
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

// DQ waves per 16 heads (4, 2 or 1), each with 512 / DQ output dims; stages
// of SK keys (16: 80 KiB of LDS, two workgroups per compute unit; 32: 160
// KiB, one).  GRP: groups of P.G query tokens (one wave per 16 of the
// group's (token, head) rows); otherwise one token per group.
template <int DQ, int SK, bool GRP>
__global__ __launch_bounds__(DQ == 1 ? 512 : 256, SK == 16 ? 2 : 1) void mla_decode_kernel(
    MlaParams P) {
  static_assert(!GRP || DQ == 1, "groups of tokens: one wave per 16 rows");
  constexpr int kTiles = kMlaLatent / 16 / DQ;  // 16-dim output tiles per wave
  constexpr int kSubs = Geo<SK>::kSubs;
  constexpr int kStageBytes = Geo<SK>::kStageBytes;
  constexpr int kPieces = Geo<SK>::kPieces;
  constexpr int kPerBlock = Geo<SK>::kPerBlock;
  constexpr int kTable = Geo<SK>::kTable;
  // LDS reads are issued at most this many chunks / tiles ahead of their
  // MFMAs: all of them would not fit in the registers beside the
  // accumulators (128 of them with one wave per 16 heads)
  constexpr int kScoreGroup = DQ == 1 ? 3 : 6;
  constexpr int kPvGroup = DQ == 1 ? 4 : 8;
  // With DQ waves per 16 heads, wave dq computes the scores over chunks
  // [c0, c1) only (4 or 5 of 18 for DQ = 4, 9 for DQ = 2) and the partial
  // sums are added through LDS in a fixed order, so all DQ waves hold the
  // same scores without each reading the whole key tile.
  constexpr int kMaxC = (kKc + DQ - 1) / DQ;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing * kStageBytes];
  // the range's stage table (query and key stages in stream order; its
  // last two slots hold the entry count and the key-stage count)
  __shared__ uint32_t stab[kTable];
  // partial scores of the waves (DQ > 1: 4 waves): [wave][sub-tile][lane]
  __shared__ f32x4 xsc[DQ > 1 ? 4 : 1][kSubs][64];
  // two workgroups per compute unit with 16-key stages: at most 80 KiB each
  static_assert(sizeof(ring) + sizeof(stab) + sizeof(xsc) <= (SK == 16 ? 81920u : 163840u),
                "LDS of the decode workgroup");

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int hg = w / DQ, dq = w % DQ;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = kKc * dq / DQ, nc = kKc * (dq + 1) / DQ - c0;  // this wave's score chunks

  // ---- records of tokens that no in-bounds request holds ----------------
  // (tokens t = w, w + grid, ..; every other token's record is written by
  // the workgroup holding its first stage, so each launch writes every
  // record once)
  if (P.seg && w == nw - 1) {
    for (int64_t t = blockIdx.x; t < P.num_q_tokens; t += gridDim.x) {
      const int b = request_of(P.qsl, P.num_seqs, (int)t);
      const int q0 = P.qsl[b], q1 = P.qsl[b + 1], L = P.seq_lens[b];
      if (!(req_ok(P, q0, q1, L) && t >= q0 && t < q1) && lane == 0) P.seg[t] = make_int2(0, 0);
    }
  }

  // ---- this workgroup's range [I0, I1) of the item stream ---------------
  // The stream: per group of G query tokens of a request, qw head items (the
  // cost of its query stages and of switching groups, in key-stage times),
  // then the key stages of its last token.  Each lane totals a contiguous
  // run of C requests; a scan over the lanes gives the stream length M and
  // the run holding item I0, whose requests a second scan walks.  (Every
  // wave computes the same.)
  const int G = GRP ? P.G : 1;
  const int qs = (G * P.Hq + SK - 1) / SK;  // query stages of a full group
  const int qw = mla_token_items(G * P.Hq, SK);
  const int C = (P.num_seqs + 63) / 64;
  int64_t tot = 0;
  int wq0 = 0, wq1 = 0, wL = 0;  // C == 1: lane b's request metadata, kept
  if (C == 1) {
    if (lane < P.num_seqs) {
      wq0 = P.qsl[lane];
      wq1 = P.qsl[lane + 1];
      wL = P.seq_lens[lane];
      if (req_ok(P, wq0, wq1, wL)) tot = items_of<SK>(wq1 - wq0, wL, G, qw);
    }
  } else {
#pragma unroll 4
    for (int k = 0; k < C; ++k) tot += req_items<SK>(P, lane * C + k, qw, G);
  }
  const int64_t incl = wave_scan(tot);
  const int64_t M = readlane64(incl, 63);
  const int64_t R = (M + gridDim.x - 1) / gridDim.x;
  // range rg of workgroup blockIdx.x: workgroups go to the 8 XCDs in turn,
  // and consecutive ranges (the pieces of one group, which read the same
  // query) are given to workgroups of one XCD, so that they share its L2
  const int rg = xcd_range(blockIdx.x, gridDim.x);
  const int64_t I0 = min((int64_t)rg * R, M);
  const int64_t I1 = min(I0 + R, M);
  if (I0 >= I1 || I1 - I0 > kTable - 2 - qs) return;
  const int lam = __builtin_ctzll(__builtin_amdgcn_ballot_w64(incl > I0));
  int64_t carry = readlane64(incl - tot, lam);
  int b0 = C == 1 ? lam : -1;
  int64_t s0 = I0 - carry;
  for (int k0 = 0; C > 1 && k0 < C; k0 += 64) {
    const int64_t it = k0 + lane < C ? req_items<SK>(P, lam * C + k0 + lane, qw, G) : 0;
    const int64_t inc = wave_scan(it) + carry;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(inc > I0);
    if (hit) {
      const int x = __builtin_ctzll(hit);
      b0 = lam * C + k0 + x;
      s0 = I0 - (readlane64(inc, x) - readlane64(it, x));
      break;
    }
    carry = readlane64(inc, 63);
  }
  b0 = __builtin_amdgcn_readfirstlane(b0);
  if (b0 < 0) return;

  ReqWindow win;
  if (C == 1) {  // every request is in the scan's registers
    win.b0 = 0;
    win.q0 = wq0;
    win.q1 = wq1;
    win.L = wL;
  } else {
    win.b0 = b0;
    const int b = b0 + lane;
    const bool in = b < P.num_seqs;
    win.q0 = in ? P.qsl[b] : 0;
    win.q1 = in ? P.qsl[b + 1] : 0;
    win.L = in ? P.seq_lens[b] : 0;
  }
  Cursor cur;
  cur.b = b0;
  int64_t kpos;  // stream index of the current group's first key stage
  {
    int q0, q1, L;
    win.get(P, b0, q0, q1, L);
    cur.q0 = q0;
    cur.Q = q1 - q0;
    cur.L = L;
    // group: the last i whose items start at or before s0 (group i starts
    // at i qw + the key stages of the groups before it, all full)
    const int64_t a = cur.L - cur.Q + G;
    int lo = 0, hi = (cur.Q + G - 1) / G - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)(mid + 1) * qw + group_prefix<SK>(mid + 1, a, G) > s0)
        hi = mid;
      else
        lo = mid + 1;
    }
    cur.i = lo;
    const int off = (int)(s0 - ((int64_t)lo * qw + group_prefix<SK>(lo, a, G)));
    // a range starting among the head items starts the group at stage 0
    cur.j = off < qw ? 0 : off - qw;
    kpos = I0 - off + qw;
    cursor_group<SK>(cur, G);
  }

  // ---- lane constants of the LDS layout ---------------------------------
  // key operand: lane (r, g) reads token r, dims 8g .. 8g+7 of a chunk
  const int offK = (g * 16 + (r ^ (12 * (g & 1)))) * 16;
  // V^T operand: the transpose read gives lane (g, r) element e from the
  // 8 bytes lane 16g + 4e + r / 4 points at, element r % 4; lane
  // 16g + 4e + q therefore points at token 4g + e, dims 4q .. 4q+3 of the
  // 16-dim tile, and lane (r, g) receives tokens 4g .. 4g+3 of dim r.
  const int vq = lane & 3, ve = (lane >> 2) & 3, vh = vq >> 1;
  const int offV = (vh * 16 + ((4 * g + ve) ^ (12 * vh))) * 16 + 8 * (vq & 1) +
                   512 * (dq * kTiles);
  // ring loads: lane i fetches granule (token (i % 16) ^ (12 (g & 1)), g) of
  // a key piece (bytes 16 i .. of a query piece)
  const uint32_t voff = (uint32_t)(((r ^ (12 * (g & 1))) * 64) + g * 16);
  const int nl = (kPieces + nw - 1) / nw;
  const int p0 = w * nl;
  const uint32_t lring =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)ring;

  // ---- the first group's query stages: issued before the table is built -
  // and its first key stage (block id read directly; the table's entry is
  // the same), by waves 1 .. nw - 1 only, nle pieces each: wave 0 builds the
  // table, and its block-id loads would otherwise wait for these loads (the
  // vector memory counter retires in order).  The ring waits still hold: a
  // wave that loads nle >= nl pieces of these stages waits for no fewer
  // loads than it needs, and wave 0 has none of them in flight.
  // (query stages of a group, and the table entry of its k-th)
  auto group_qs = [&](const Cursor& c) { return (c.ntok * P.Hq + SK - 1) / SK; };
  auto qentry = [&](const Cursor& c, int k) {
    return kQStage | ((uint32_t)(c.q0 + c.i * G) << 6) | ((uint32_t)(c.ntok - 1) << 3) |
           (uint32_t)k;
  };
  const int qs0 = group_qs(cur);
  const int pre = min(qs0, kRing - 1);
  const int pre2 = qs0 < kRing - 1 ? qs0 + 1 : pre;
  const int nle = nw > 1 ? (kPieces + nw - 2) / (nw - 1) : nl;
  const int p0e = nw > 1 ? (w - 1) * nle : 0;
  auto issue_first = [&]() {
    for (int k = 0; k < pre; ++k)
      dma_stage<SK>(P, qentry(cur, k), lring + k * kStageBytes, voff, p0e, nle);
    if (pre2 > pre) {
      int id = sload(P.bt + (int64_t)cur.b * P.bt_stride + cur.j / kPerBlock);
      id = id < 0 ? 0 : (id >= P.num_blocks ? (int)(P.num_blocks - 1) : id);
      dma_stage<SK>(P, ((uint32_t)id << 2) | (uint32_t)(cur.j % kPerBlock),
                    lring + qs0 * kStageBytes, voff, p0e, nle);
    }
  };
  if (w != 0 || nw == 1) issue_first();

  // ---- the range's stage table (wave 0; one gather) -----------------------
  // Group by group, for each group with key stages in the range: its query
  // stages, then (request - b0) << 14 | stage of each of those key stages;
  // then each lane turns its key entries into block ids with one
  // block-table load each.  At most R + qs entries (a group's query stages
  // are entries of the range only where its head items are, but the
  // first's).
  constexpr int kCap = kTable - 2;  // entries; then the two counts
  if (w == 0) {
    Cursor f = cur;
    int64_t fpos = kpos;
    int x = 0, nk = 0;
    for (;;) {
      const int64_t ka = max(I0, fpos), kb = min(I1, fpos + f.nst);
      if (kb > ka) {
        const int cnt = (int)(kb - ka), j0 = (int)(ka - fpos), qsf = group_qs(f);
        if (x + qsf + cnt > kCap) {
          x = -1;  // cannot happen with the launch's grid: it bounds R
          break;
        }
        if (lane < qsf) stab[x + lane] = qentry(f, lane);
        x += qsf;
        for (int y = lane; y < cnt; y += 64)
          stab[x + y] = ((uint32_t)(f.b - b0) << 14) | (uint32_t)(j0 + y);
        x += cnt;
        nk += cnt;
      }
      // the next group's key stages start past its head items
      fpos += f.nst + qw;
      if (fpos >= I1) break;
      f.j = f.nst - 1;
      cursor_next<SK>(f, P, win, G);
    }
#pragma unroll 4
    for (int y = lane; y < x; y += 64) {
      const uint32_t v = stab[y];
      if (v & kQStage) continue;
      const int b = b0 + (int)(v >> 14), j = (int)(v & 16383);
      int id = P.bt[(int64_t)b * P.bt_stride + j / kPerBlock];
      id = id < 0 ? 0 : (id >= P.num_blocks ? (int)(P.num_blocks - 1) : id);
      stab[y] = ((uint32_t)id << 2) | (uint32_t)(j % kPerBlock);
    }
    if (lane == 0) {
      stab[kCap] = (uint32_t)x;
      stab[kCap + 1] = (uint32_t)nk;
    }
  }
  // (an LDS-only barrier: __syncthreads() would also wait for the ring
  // loads just issued)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const int n = (int)__builtin_amdgcn_readfirstlane(stab[kCap]);
  const int nreal = (int)__builtin_amdgcn_readfirstlane(stab[kCap + 1]);  // key stages of the range
  if (n <= 0 || nreal <= 0) {  // (no LDS write of the ring may outlive the workgroup)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }

  // ---- rest of the prologue: entries pre2 .. kRing - 2 --------------------
  for (int k = pre2; k < kRing - 1 && k < n; ++k)
    dma_stage<SK>(P, __builtin_amdgcn_readfirstlane(stab[k]), lring + k * kStageBytes, voff, p0,
              nl);

  int stored = 0;         // ring waits left that allow for result stores
  int done = 0;           // key stages computed
  bool first_tok = true;  // the piece is of the range's first group
  const float c2 = P.scale_log2;
  int it = 0;             // table entry
  // Before entry `it` is read: wait for it (and meet the other waves), then
  // refill the buffer every wave has finished with.
  auto ring_step = [&]() {
    ring_wait<kTiles>(nl, it + kRing - 2 >= n, stored > 0);
    if (stored > 0) --stored;
    if (it + kRing - 1 < n)
      dma_stage<SK>(P, __builtin_amdgcn_readfirstlane(stab[it + kRing - 1]),
                lring + (uint32_t)((it + kRing - 1) % kRing) * kStageBytes, voff, p0, nl);
  };

  // The wave's 16 (token, head) rows of a group: rows 16 hg .. 16 hg + 15,
  // token tw of the group, heads 16 hg - tw Hq .. (one token's heads: Hq is
  // a multiple of 16).
  const int vrow = 16 * hg;
  const int tw = vrow / P.Hq;
  // One group's piece of the range per pass: its query stages, then its key
  // stages.  (The query operand lives within a pass.)  A wave whose token is
  // past a short group's last takes part in the waits and barriers only.
  while (done < nreal) {
    const bool active = !GRP || tw < cur.ntok;
    bf16x8 qop[kMaxC];  // lane (r, g): row vrow + r, dims 32 (c0 + i) + 8g .. +7
    const int qsg = group_qs(cur);
    for (int k = 0; k < qsg; ++k, ++it) {
      ring_step();
      if (active && k == vrow / SK) {
        // lane (r, g): row vrow + r (row vrow % SK + r of the stage), dims
        // 8g .. of each chunk
        const uint8_t* st = ring + (it % kRing) * kStageBytes +
                            (vrow % SK + r) * (kMlaDim * 2) + g * 16 + c0 * 64;
#pragma unroll
        for (int i = 0; i < kMaxC; ++i)
          if (i < nc) qop[i] = *reinterpret_cast<const bf16x8*>(st + i * 64);
        // the copies land before the buffer can be refilled
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      }
    }
    const int cnt = min(cur.nst - cur.j, nreal - done);
    f32x4 acc[kTiles];
#pragma unroll
    for (int k = 0; k < kTiles; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lsum = 0.0f;
    // keys the wave's token sees
    const int nvis = cur.L - cur.Q + 1 + cur.i * G + tw;
    for (int ks = 0; ks < cnt; ++ks, ++it) {
      ring_step();
      const int j = cur.j + ks;  // stage of the group
      const uint8_t* st = ring + (it % kRing) * kStageBytes;
      __bf16 pw[4 * kSubs];
      if (active) {
        // scores of the stage's 16-key sub-tiles
        f32x4 sc[kSubs];
#pragma unroll
        for (int u = 0; u < kSubs; ++u) sc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kMaxC; ++i) {
          if (i < nc) {
            const uint8_t* kp = st + (c0 + i) * 1024 + offK;
#pragma unroll
            for (int u = 0; u < kSubs; ++u)
              sc[u] = mfma32(*reinterpret_cast<const bf16x8*>(kp + u * kSubBytes), qop[i], sc[u]);
          }
          if (i % kScoreGroup == kScoreGroup - 1) __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (DQ > 1) {
          // add the head group's partial sums in wave order (the same sums in
          // every wave); the writes land before the barrier, and every wave
          // has read them before the next stage's barrier
#pragma unroll
          for (int u = 0; u < kSubs; ++u) xsc[w][u][lane] = sc[u];
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          const int w0 = hg * DQ;  // the head group's first wave
#pragma unroll
          for (int u = 0; u < kSubs; ++u) {
            sc[u] = xsc[w0][u][lane];
#pragma unroll
            for (int v = 1; v < DQ; ++v) sc[u] += xsc[w0 + v][u][lane];
          }
        }
        // online softmax over the stage's keys (lane (r, g): keys 4g .. 4g+3
        // of each sub-tile, row r); keys the token does not see get -inf (in a
        // group, an earlier token may see none of a stage: its weights are 0
        // while its maximum is still -inf)
        const int key0 = SK * j + 4 * g;
        float y[4 * kSubs];
#pragma unroll
        for (int u = 0; u < kSubs; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            y[4 * u + e] = key0 + 16 * u + e < nvis ? sc[u][e] * c2 : -INFINITY;
        float mx = y[0];
#pragma unroll
        for (int e = 1; e < 4 * kSubs; ++e) mx = fmaxf(mx, y[e]);
        mx = column_max(mx);
        if (__builtin_amdgcn_ballot_w64(mx > mrun + kSlack) != 0) {
          const float mnew = fmaxf(mrun, mx);
          const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);  // 0 on the first stage
#pragma unroll
          for (int k = 0; k < kTiles; ++k) acc[k] *= alpha;
          lsum *= alpha;
          mrun = mnew;
        }
        const float mref = mrun == -INFINITY ? 0.0f : mrun;
        float ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 4 * kSubs; ++e) {
          pw[e] = (__bf16)__builtin_amdgcn_exp2f(y[e] - mref);
          ps += (float)pw[e];
        }
        lsum += ps;
      }
      // weighted sum; in a stage the group's last token does not see to its
      // end, the V rows of the keys past what it sees (possibly unwritten
      // slots: a 0 weight must not meet a NaN) are first zeroed in LDS (the
      // other tokens' masked keys are written slots).  Every wave writes the
      // same zeros, and its own reads follow its own writes (LDS operations of
      // a wave complete in order), so no barrier is needed.
      if (SK * j + SK > cur.nvis) {
        const int kv = cur.nvis - SK * j;  // keys of the stage it sees
        uint8_t* sw = ring + (it % kRing) * kStageBytes;
        for (int q = lane; q < kSubs * (kMlaLatent / 32) * 64; q += 64) {
          const int u = q >> 10, c = (q >> 6) & 15, pos = q & 63;
          const int key = 16 * u + ((pos & 15) ^ (12 * ((pos >> 4) & 1)));
          if (key >= kv)
            *reinterpret_cast<u32x4*>(sw + u * kSubBytes + c * 1024 + pos * 16) =
                u32x4{0u, 0u, 0u, 0u};
        }
      }
      // (operands assembled by whole-vector casts and shuffles: assembled
      // element by element, the transpose reads' results were compiled to
      // copies of their first dwords)
      if (!active) continue;
      if constexpr (SK == 32) {
        bf16x8 pp;
#pragma unroll
        for (int e = 0; e < 8; ++e) pp[e] = pw[e];
#pragma unroll
        for (int mt = 0; mt < kTiles; ++mt) {
          const bf16x8 a = __builtin_shufflevector(
              __builtin_bit_cast(bf16x4, lds_read_tr(st + 512 * mt + offV)),
              __builtin_bit_cast(bf16x4, lds_read_tr(st + kSubBytes + 512 * mt + offV)), 0, 1,
              2, 3, 4, 5, 6, 7);
          acc[mt] = mfma32(a, pp, acc[mt]);
          if (mt % kPvGroup == kPvGroup - 1) __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        bf16x4 pp;
#pragma unroll
        for (int e = 0; e < 4; ++e) pp[e] = pw[e];
#pragma unroll
        for (int mt = 0; mt < kTiles; ++mt) {
          const bf16x4 a = __builtin_bit_cast(bf16x4, lds_read_tr(st + 512 * mt + offV));
          acc[mt] = mfma16(a, pp, acc[mt]);
          if (mt % kPvGroup == kPvGroup - 1) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // the group's piece is done: the wave's rows of the output, or of its
    // partial (a token that saw no key of the piece: weight 0, output 0)
    const bool whole = cur.j == 0 && cur.j + cnt == cur.nst;
    float l = lsum;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const int t = cur.q0 + cur.i * G + tw;
    const int h = vrow - tw * P.Hq + r;
    const int dim0 = dq * kTiles * 16 + 4 * g;
    if (!active) {
    } else if (whole) {
      uint16_t* op = P.out + ((int64_t)t * P.Hq + h) * kMlaLatent + dim0;
#pragma unroll
      for (int k = 0; k < kTiles; ++k) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[k][e] * inv);
        *reinterpret_cast<bf16x4*>(op + 16 * k) = o;
      }
    } else {
      // slot 2 rg: the range's first group; 2 rg + 1: its last (only these
      // two can be cut), G Hq rows each.  The piece's normalised output in
      // bf16, its (max, sum) in fp32.
      const int64_t row = (2 * (int64_t)rg + (first_tok ? 0 : 1)) * (G * P.Hq) + vrow + r;
      uint16_t* ap = P.part_out + row * kMlaLatent + dim0;
#pragma unroll
      for (int k = 0; k < kTiles; ++k) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[k][e] * inv);
        *reinterpret_cast<bf16x4*>(ap + 16 * k) = o;
      }
      if (dq == 0 && g == 0) P.part_ml[row] = make_float2(mrun, l);
    }
    // the workgroup holding the group's first key stage records, for each of
    // its tokens, which workgroups hold its pieces (this one, then whole
    // ranges, the last one (R items each) holding the group's last key
    // stage) and the token's place in the group; the first wave of each
    // token writes it
    if (cur.j == 0 && active && vrow % P.Hq == 0 && dq == 0 && lane == 0 && P.seg) {
      const int64_t last = kpos + cur.nst - 1;
      const int pieces = (int)(last / R - rg + 1);
      P.seg[t] = make_int2(rg, ((2 * pieces + (first_tok ? 0 : 1)) << 3) | tw);
    }
    // (the ring waits allow for result stores only where there are some)
    stored = active ? kRing - 1 : 0;
    first_tok = false;
    done += cnt;
    if (done < nreal) {
      kpos += cur.nst + qw;
      cur.j = cur.nst - 1;
      cursor_next<SK>(cur, P, win, G);
    }
  }
}

// One wave per (query token, head) whose keys were cut between workgroups:
// log-sum-exp over the pieces.  The lanes read the pieces' (max, sum) in
// parallel (64 pieces per round) along with the outputs of the first eight
// pieces, then every lane adds its 8 dims of each piece's output, weighted;
// lane i holds dims 8i .. 8i+7.  The decode
// writes every token's record in every launch ((0, 0) for tokens of
// out-of-bounds requests), so no stale record is read.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaParams P) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row0 >= (int64_t)P.num_q_tokens * P.Hq) return;
  const int t = (int)(row0 / P.Hq), h = (int)(row0 % P.Hq);
  // pieces of the token's group: the first in slot 2 w0 + flag (flag: the
  // group was not the first of w0's range), the others in slots 2 (w0 + s)
  // (their ranges begin inside the group); the token's rows are those of its
  // place tw in the group
  const int2 sg = P.seg[t];
  const int pieces = sg.y >> 4, flag = (sg.y >> 3) & 1, tw = sg.y & 7;
  if (pieces < 2 || sg.x < 0 || sg.x > P.grid - pieces || tw >= P.G) return;
  auto row_of = [&](int s) -> int64_t {
    const int64_t slot = s == 0 ? 2 * (int64_t)sg.x + flag : 2 * ((int64_t)sg.x + s);
    return slot * (P.G * P.Hq) + tw * P.Hq + h;
  };
  // out = sum_i w_i o_i / sum_i w_i, w_i = l_i 2^(m_i - M): o_i a piece's
  // normalised output (bf16), (m_i, l_i) its running max and sum
  float M = -INFINITY, den = 0.0f;
  float n[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // pieces whose outputs are loaded with the (max, sum) round (a token of
  // a few requests typically has 4 to 10)
  constexpr int kAhead = 8;
  for (int s0 = 0; s0 < pieces; s0 += 64) {
    const int cnt = min(64, pieces - s0);
    float2 ml = make_float2(-INFINITY, 0.0f);
    if (lane < cnt) ml = P.part_ml[row_of(s0 + lane)];
    // the first pieces' outputs do not depend on the (max, sum) values:
    // their loads go out in the same round
    bf16x8 oa[kAhead];
#pragma unroll
    for (int k = 0; k < kAhead; ++k)
      if (k < cnt)
        oa[k] = *reinterpret_cast<const bf16x8*>(P.part_out + row_of(s0 + k) * kMlaLatent +
                                                 8 * lane);
    float mx = ml.x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
    const float mn = fmaxf(M, mx);  // finite: the group's first piece saw a key of every token
    const float c_old = __builtin_amdgcn_exp2f(M - mn);
    const float wgt = lane < cnt ? ml.y * __builtin_amdgcn_exp2f(ml.x - mn) : 0.0f;
    float dl = wgt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) dl += __shfl_xor(dl, d);
    den = den * c_old + dl;
#pragma unroll
    for (int e = 0; e < 8; ++e) n[e] *= c_old;
#pragma unroll
    for (int k = 0; k < kAhead; ++k) {
      if (k < cnt) {
        const float wk = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wgt), k));
#pragma unroll
        for (int e = 0; e < 8; ++e) n[e] += wk * (float)oa[k][e];
      }
    }
    for (int k = kAhead; k < cnt; ++k) {
      const float wk = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wgt), k));
      const bf16x8 ok = *reinterpret_cast<const bf16x8*>(P.part_out + row_of(s0 + k) * kMlaLatent +
                                                         8 * lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) n[e] += wk * (float)ok[e];
    }
    M = mn;
  }
  const float inv = 1.0f / den;
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (__bf16)(n[e] * inv);
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
  const int hgs = P.Hq / 16;  // 1 .. 8
  const int dq = hgs == 1 ? 4 : (hgs == 2 ? 2 : 1);
  const dim3 block(64 * hgs * dq), grid((unsigned)P.grid);
  static_assert(mla_stage_keys(16) == 16 && mla_stage_keys(32) == 16 &&
                    mla_stage_keys(48) == 32,
                "the instances below follow the stage size the layout assumes");
  if (P.G > 1)  // groups of 128 / Hq tokens: 8 waves of 16 (token, head) rows
    hipLaunchKernelGGL((mla_decode_kernel<1, 32, true>), grid, dim3(512), 0, stream, P);
  else if (dq == 4)
    hipLaunchKernelGGL((mla_decode_kernel<4, 16, false>), grid, block, 0, stream, P);
  else if (dq == 2)
    hipLaunchKernelGGL((mla_decode_kernel<2, 16, false>), grid, block, 0, stream, P);
  else
    hipLaunchKernelGGL((mla_decode_kernel<1, 32, false>), grid, block, 0, stream, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P.grid < 2) return e;
  const int64_t rows = (int64_t)P.num_q_tokens * P.Hq;
  hipLaunchKernelGGL(mla_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     stream, P);
  return hipGetLastError();
}

}  // namespace pa
