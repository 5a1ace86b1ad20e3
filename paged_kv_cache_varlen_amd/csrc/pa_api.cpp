// C ABI of libpa.so: argument checks, workspace sizing and launches.  The
// operations and their sources are documented in include/pa.h.
#include "pa.h"

#include <cfloat>

#include <hip/hip_runtime_api.h>

#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "pa_device.h"
#include "mla_device.h"

namespace {

thread_local std::string g_last_error;

pa_status fail(pa_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

pa_status ok() {
  g_last_error.clear();
  return PA_OK;
}

pa_status hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Compute-unit count per device, read once.
int num_cus_of_current_device(hipError_t* err) {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    *err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (*err != hipSuccess) return 0;
    cache[dev] = n > 0 ? n : 1;
  }
  return cache[dev];
}

bool supported_head_dim(int32_t d) { return d == 64 || d == 128; }

pa_status check_heads(int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim) {
  if (num_q_heads <= 0 || num_kv_heads <= 0)
    return fail(PA_ERR_SHAPE, "num_q_heads and num_kv_heads must be > 0");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "num_q_heads must be a multiple of num_kv_heads");
  if (num_q_heads / num_kv_heads > pa::kMaxGroup)
    return fail(PA_ERR_UNSUPPORTED,
                "more than 16 query heads per kv head is not supported");
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer";
    case PA_ERR_SHAPE: return "invalid shape";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_METADATA: return "invalid metadata";
    case PA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// Checks shared by the scatter entry points (the 8-bit scales are checked by
// the caller, first).
pa_status check_scatter(const char* name, const void* k, const void* v,
                        int64_t k_token_stride, int64_t v_token_stride,
                        const int64_t* slot_mapping, int64_t num_tokens,
                        int32_t num_kv_heads, int32_t head_dim, const void* k_cache,
                        const void* v_cache, int64_t num_blocks) {
  if (num_tokens < 0 || num_blocks < 0)
    return fail(PA_ERR_SHAPE, "num_tokens and num_blocks must be >= 0");
  if (num_kv_heads <= 0) return fail(PA_ERR_SHAPE, "num_kv_heads must be > 0");
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (k_token_stride < row || v_token_stride < row)
    return fail(PA_ERR_SHAPE, "token strides must be >= num_kv_heads*head_dim");
  if ((k_token_stride % 8) || (v_token_stride % 8))
    return fail(PA_ERR_SHAPE, "token strides must be multiples of 8 elements");
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(PA_ERR_NULL, std::string(name) + ": NULL pointer");
  if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15)
    return fail(PA_ERR_SHAPE, "k, v and the pools must be 16-byte aligned");
  return PA_OK;
}

// The 8-bit variants: the pools' scales are checked before anything else.
pa_status check_fp8(float k_scale, float v_scale) {
  if (!(k_scale > 0.0f && k_scale <= FLT_MAX) || !(v_scale > 0.0f && v_scale <= FLT_MAX))
    return fail(PA_ERR_SHAPE, "8-bit pools: scales must be finite and > 0");
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_write_kv(const void* k, const void* v, int64_t k_token_stride,
                      int64_t v_token_stride, const int64_t* slot_mapping,
                      int64_t num_tokens, int32_t num_kv_heads,
                      int32_t head_dim, void* k_cache, void* v_cache,
                      int64_t num_blocks, void* stream) {
  pa_status s = check_scatter("pa_write_kv", k, v, k_token_stride, v_token_stride,
                              slot_mapping, num_tokens, num_kv_heads, head_dim, k_cache,
                              v_cache, num_blocks);
  if (s != PA_OK || num_tokens == 0) return s == PA_OK ? ok() : s;
  hipError_t e = pa::launch_write_kv(
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      k_token_stride, v_token_stride, slot_mapping, num_tokens, num_kv_heads,
      head_dim, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
      num_blocks, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_write_kv launch");
  return ok();
}

pa_status pa_write_kv_fp8(const void* k, const void* v, int64_t k_token_stride,
                          int64_t v_token_stride, const int64_t* slot_mapping,
                          int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, float k_scale, float v_scale,
                          void* k_cache, void* v_cache, int64_t num_blocks,
                          void* stream) {
  pa_status s = check_fp8(k_scale, v_scale);
  if (s != PA_OK) return s;
  s = check_scatter("pa_write_kv_fp8", k, v, k_token_stride, v_token_stride,
                    slot_mapping, num_tokens, num_kv_heads, head_dim, k_cache, v_cache,
                    num_blocks);
  if (s != PA_OK || num_tokens == 0) return s == PA_OK ? ok() : s;
  hipError_t e = pa::launch_write_kv8(
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      k_token_stride, v_token_stride, slot_mapping, num_tokens, num_kv_heads,
      head_dim, k_scale, v_scale, static_cast<uint8_t*>(k_cache),
      static_cast<uint8_t*>(v_cache), num_blocks, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_write_kv_fp8 launch");
  return ok();
}

size_t pa_attend_workspace_size(int32_t num_seqs, int64_t num_q_tokens,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_query_len,
                                int32_t max_seq_len) {
  if (num_seqs < 0 || num_q_tokens < 0 || max_query_len < 0 || max_seq_len < 0)
    return 0;
  if (check_heads(num_q_heads, num_kv_heads, head_dim) != PA_OK) return 0;
  return pa::workspace_layout(num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                              head_dim, max_query_len, max_seq_len)
      .total;
}

size_t pa_attend_cascade_workspace_size(int32_t num_seqs, int64_t num_q_tokens,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_query_len,
                                        int32_t max_seq_len) {
  if (num_seqs < 0 || num_q_tokens < 0 || max_query_len < 0 || max_seq_len < 0)
    return 0;
  if (check_heads(num_q_heads, num_kv_heads, head_dim) != PA_OK) return 0;
  return pa::workspace_layout(num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                              head_dim, max_query_len, max_seq_len)
      .cascade_total;
}

}  // extern "C"

namespace {

// Checks shared by the attention entry points; fills `a`.  With
// need_tensors = false (planning only) q, the pools and out may be NULL.
pa_status prepare_attend(const void* q, const void* k_cache,
                         const void* v_cache, int64_t num_blocks,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, const int32_t* query_start_loc,
                         int32_t num_seqs, int64_t num_q_tokens,
                         int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t max_query_len,
                         int32_t max_seq_len, float scale, void* out,
                         void* workspace, size_t workspace_bytes,
                         bool need_tensors, pa::AttendArgs* a, bool* empty,
                         int32_t prefix_len = -1) {
  *empty = false;
  if (num_seqs < 0 || num_q_tokens < 0 || num_blocks < 0 ||
      max_blocks_per_seq < 0 || max_query_len < 0 || max_seq_len < 0)
    return fail(PA_ERR_SHAPE, "pa_attend: negative size");
  if (num_q_tokens > INT32_MAX / 2)
    return fail(PA_ERR_SHAPE, "pa_attend: num_q_tokens too large");
  pa_status s = check_heads(num_q_heads, num_kv_heads, head_dim);
  if (s != PA_OK) return s;
  if (num_q_tokens == 0 || num_seqs == 0) {
    *empty = true;
    return PA_OK;
  }
  if (!block_tables || !seq_lens || !query_start_loc)
    return fail(PA_ERR_NULL, "pa_attend: NULL metadata pointer");
  if (need_tensors && (!q || !k_cache || !v_cache || !out))
    return fail(PA_ERR_NULL, "pa_attend: NULL pointer");
  if (max_blocks_per_seq == 0 || (need_tensors && num_blocks == 0))
    return fail(PA_ERR_SHAPE, "pa_attend: empty pool or block table");
  if (num_blocks > (int64_t)(UINT32_MAX / (uint32_t)num_kv_heads))
    return fail(PA_ERR_SHAPE, "pa_attend: num_blocks * num_kv_heads must fit in 32 bits");
  if (need_tensors && !(scale > 0.0f && scale <= FLT_MAX))
    return fail(PA_ERR_SHAPE, "pa_attend: scale must be finite and > 0");
  if (need_tensors &&
      (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) & 15))
    return fail(PA_ERR_SHAPE, "q, out and the pools must be 16-byte aligned");
  pa::WorkspaceLayout ws =
      pa::workspace_layout(num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                           head_dim, max_query_len, max_seq_len);
  // shared-prefix calls (prefix_len >= 0): the workspace also holds the
  // prefix section; the plan shares the largest multiple of 32 keys not above
  // common_prefix_len (every key range then covers whole pairs of blocks)
  const bool cascade = prefix_len >= 0;
  if (cascade && prefix_len > max_seq_len)
    return fail(PA_ERR_SHAPE, "common_prefix_len must be in [0, max_seq_len]");
  const size_t need = cascade ? ws.cascade_total : ws.total;
  if (!workspace || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE,
                std::string(cascade ? "shared-prefix attention" : "pa_attend") +
                    ": workspace needs " + std::to_string(need) + " bytes, got " +
                    std::to_string(workspace_bytes));
  if ((uintptr_t)workspace & 255)
    return fail(PA_ERR_WORKSPACE, "pa_attend: workspace must be 256-byte aligned");
  hipError_t e = hipSuccess;
  const int cus = num_cus_of_current_device(&e);
  if (e != hipSuccess) return hip_fail(e, "pa_attend device query");
  a->q = static_cast<const uint16_t*>(q);
  a->k_cache = static_cast<const uint16_t*>(k_cache);
  a->v_cache = static_cast<const uint16_t*>(v_cache);
  a->num_blocks = num_blocks;
  a->block_tables = block_tables;
  a->bt_stride = max_blocks_per_seq;
  a->seq_lens = seq_lens;
  a->qsl = query_start_loc;
  a->num_seqs = num_seqs;
  a->num_q_tokens = num_q_tokens;
  a->num_q_heads = num_q_heads;
  a->num_kv_heads = num_kv_heads;
  a->head_dim = head_dim;
  a->max_query_len = max_query_len;
  a->max_seq_len = max_seq_len;
  a->scale = scale;
  a->out = static_cast<uint16_t*>(out);
  a->workspace = workspace;
  a->ws = ws;
  a->num_cus = cus;
  a->cascade = cascade;
  a->prefix_len = cascade ? (prefix_len & ~31) : 0;
  a->kv8 = false;
  a->k_scale = 1.0f;
  a->v_scale = 1.0f;
  return PA_OK;
}

void set_fp8(float k_scale, float v_scale, pa::AttendArgs* a) {
  a->kv8 = true;
  a->k_scale = k_scale;
  a->v_scale = v_scale;
}

}  // namespace

extern "C" {

pa_status pa_attend_plan(const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, const int32_t* query_start_loc,
                         int32_t num_seqs, int64_t num_q_tokens,
                         int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t max_query_len,
                         int32_t max_seq_len, void* workspace,
                         size_t workspace_bytes, void* stream) {
  pa::AttendArgs a;
  bool empty;
  pa_status s = prepare_attend(nullptr, nullptr, nullptr, 0, block_tables,
                               max_blocks_per_seq, seq_lens, query_start_loc,
                               num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                               head_dim, max_query_len, max_seq_len, 0.0f,
                               nullptr, workspace, workspace_bytes, false, &a,
                               &empty);
  if (s != PA_OK) return s;
  if (empty) return ok();
  hipError_t e = pa::launch_plan(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_attend_plan launch");
  return ok();
}

pa_status pa_attend_plan_fp8(const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* seq_lens, const int32_t* query_start_loc,
                             int32_t num_seqs, int64_t num_q_tokens,
                             int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t max_query_len,
                             int32_t max_seq_len, void* workspace,
                             size_t workspace_bytes, void* stream) {
  pa::AttendArgs a;
  bool empty;
  pa_status s = prepare_attend(nullptr, nullptr, nullptr, 0, block_tables,
                               max_blocks_per_seq, seq_lens, query_start_loc,
                               num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                               head_dim, max_query_len, max_seq_len, 0.0f,
                               nullptr, workspace, workspace_bytes, false, &a,
                               &empty);
  if (s != PA_OK) return s;
  if (empty) return ok();
  a.kv8 = true;  // the plan's key ranges only; no scales are involved
  hipError_t e = pa::launch_plan(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_attend_plan_fp8 launch");
  return ok();
}

pa_status pa_attend_planned(const void* q, const void* k_cache,
                            const void* v_cache, int64_t num_blocks,
                            const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            const int32_t* query_start_loc, int32_t num_seqs,
                            int64_t num_q_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_query_len, int32_t max_seq_len,
                            float scale, void* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  pa::AttendArgs a;
  bool empty;
  pa_status s = prepare_attend(q, k_cache, v_cache, num_blocks, block_tables,
                               max_blocks_per_seq, seq_lens, query_start_loc,
                               num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                               head_dim, max_query_len, max_seq_len, scale, out,
                               workspace, workspace_bytes, true, &a, &empty);
  if (s != PA_OK) return s;
  if (empty) return ok();
  hipError_t e = pa::launch_planned(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_attend_planned launch");
  return ok();
}

pa_status pa_attend_merge(int32_t num_seqs, int64_t num_q_tokens,
                          int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t max_query_len,
                          int32_t max_seq_len, void* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  pa::AttendArgs a;
  bool empty;
  // metadata pointers are not read by the merge: pass placeholders through
  // the shared checks
  static const int32_t kNone[2] = {0, 0};
  pa_status s = prepare_attend(nullptr, nullptr, nullptr, 0, kNone, 1, kNone,
                               kNone, num_seqs, num_q_tokens, num_q_heads,
                               num_kv_heads, head_dim, max_query_len,
                               max_seq_len, 0.0f, out, workspace,
                               workspace_bytes, false, &a, &empty);
  if (s != PA_OK) return s;
  if (empty) return ok();
  if (!out) return fail(PA_ERR_NULL, "pa_attend_merge: NULL out");
  if ((uintptr_t)out & 15) return fail(PA_ERR_SHAPE, "out must be 16-byte aligned");
  hipError_t e = pa::launch_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_attend_merge launch");
  return ok();
}

pa_status pa_attend(const void* q, const void* k_cache, const void* v_cache,
                    int64_t num_blocks, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* seq_lens,
                    const int32_t* query_start_loc, int32_t num_seqs,
                    int64_t num_q_tokens, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim,
                    int32_t max_query_len, int32_t max_seq_len, float scale,
                    void* out, void* workspace, size_t workspace_bytes,
                    void* stream) {
  pa::AttendArgs a;
  bool empty;
  pa_status s = prepare_attend(q, k_cache, v_cache, num_blocks, block_tables,
                               max_blocks_per_seq, seq_lens, query_start_loc,
                               num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                               head_dim, max_query_len, max_seq_len, scale, out,
                               workspace, workspace_bytes, true, &a, &empty);
  if (s != PA_OK) return s;
  if (empty) return ok();
  hipError_t e = pa::launch_plan(a, static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = pa::launch_planned(a, static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = pa::launch_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_attend launch");
  return ok();
}

static_assert(PA_NOALLOC_SCRATCH_BYTES == pa::kStaticScratchBytes,
              "pa.h states the static scratch size");

pa_status pa_attend_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            int64_t num_blocks, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            const int32_t* query_start_loc, int32_t num_seqs,
                            int64_t num_q_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_query_len, int32_t max_seq_len, float scale,
                            void* out, void* stream) {
  // sizes first: a batch whose workspace exceeds the static scratch is
  // rejected before any device call (invalid sizes fall through to the
  // checks of prepare_attend, which report them)
  const size_t need = pa_attend_workspace_size(num_seqs, num_q_tokens, num_q_heads,
                                               num_kv_heads, head_dim, max_query_len,
                                               max_seq_len);
  if (need > pa::kStaticScratchBytes)
    return fail(PA_ERR_WORKSPACE,
                "pa_attend_noalloc: these sizes need " + std::to_string(need) +
                    " bytes of workspace; the static scratch holds " +
                    std::to_string(pa::kStaticScratchBytes) +
                    " (call pa_attend with a workspace instead)");
  // every argument check of pa_attend, against a workspace of the scratch's
  // size; the scratch's device address is bound once they have passed (the
  // placeholder is never dereferenced)
  pa::AttendArgs a;
  bool empty;
  void* const placeholder = reinterpret_cast<void*>(uintptr_t(256));
  pa_status s = prepare_attend(q, k_cache, v_cache, num_blocks, block_tables,
                               max_blocks_per_seq, seq_lens, query_start_loc,
                               num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                               head_dim, max_query_len, max_seq_len, scale, out,
                               placeholder, pa::kStaticScratchBytes, true, &a, &empty);
  if (s != PA_OK) return s;
  if (empty) return ok();
  void* ws = nullptr;
  hipError_t e = pa::scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e, "pa_attend_noalloc scratch lookup");
  a.workspace = ws;
  e = pa::launch_plan(a, static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = pa::launch_planned(a, static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = pa::launch_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_attend_noalloc launch");
  return ok();
}

pa_status pa_attend_planned_fp8(const void* q, const void* k_cache,
                                const void* v_cache, int64_t num_blocks,
                                const int32_t* block_tables,
                                int32_t max_blocks_per_seq,
                                const int32_t* seq_lens,
                                const int32_t* query_start_loc, int32_t num_seqs,
                                int64_t num_q_tokens, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_query_len, int32_t max_seq_len,
                                float scale, float k_scale, float v_scale,
                                void* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (check_fp8(k_scale, v_scale) != PA_OK) return PA_ERR_SHAPE;
  pa::AttendArgs a;
  bool empty;
  pa_status s = prepare_attend(q, k_cache, v_cache, num_blocks, block_tables,
                               max_blocks_per_seq, seq_lens, query_start_loc,
                               num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                               head_dim, max_query_len, max_seq_len, scale, out,
                               workspace, workspace_bytes, true, &a, &empty);
  if (s != PA_OK) return s;
  if (empty) return ok();
  set_fp8(k_scale, v_scale, &a);
  hipError_t e = pa::launch_planned(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_attend_planned_fp8 launch");
  return ok();
}

pa_status pa_attend_fp8(const void* q, const void* k_cache, const void* v_cache,
                        int64_t num_blocks, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* seq_lens,
                        const int32_t* query_start_loc, int32_t num_seqs,
                        int64_t num_q_tokens, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim,
                        int32_t max_query_len, int32_t max_seq_len, float scale,
                        float k_scale, float v_scale, void* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (check_fp8(k_scale, v_scale) != PA_OK) return PA_ERR_SHAPE;
  pa::AttendArgs a;
  bool empty;
  pa_status s = prepare_attend(q, k_cache, v_cache, num_blocks, block_tables,
                               max_blocks_per_seq, seq_lens, query_start_loc,
                               num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                               head_dim, max_query_len, max_seq_len, scale, out,
                               workspace, workspace_bytes, true, &a, &empty);
  if (s != PA_OK) return s;
  if (empty) return ok();
  set_fp8(k_scale, v_scale, &a);
  hipError_t e = pa::launch_plan(a, static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = pa::launch_planned(a, static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = pa::launch_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_attend_fp8 launch");
  return ok();
}

// ---- shared-prefix (cascade) attention --------------------------------------

pa_status pa_attend_plan_cascade(const int32_t* block_tables,
                                 int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens,
                                 const int32_t* query_start_loc, int32_t num_seqs,
                                 int64_t num_q_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_query_len, int32_t max_seq_len,
                                 int32_t common_prefix_len, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  pa::AttendArgs a;
  bool empty;
  pa_status s = prepare_attend(nullptr, nullptr, nullptr, 0, block_tables,
                               max_blocks_per_seq, seq_lens, query_start_loc,
                               num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                               head_dim, max_query_len, max_seq_len, 0.0f,
                               nullptr, workspace, workspace_bytes, false, &a,
                               &empty, common_prefix_len < 0 ? INT32_MAX : common_prefix_len);
  if (s != PA_OK) return s;
  if (empty) return ok();
  hipError_t e = pa::launch_plan(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_attend_plan_cascade launch");
  return ok();
}

// ---- scatter + plan in one launch -------------------------------------------

namespace {

pa_status write_plan_call(const char* name, bool kv8, const void* k, const void* v,
                          int64_t k_token_stride, int64_t v_token_stride,
                          const int64_t* slot_mapping, int64_t num_new_tokens,
                          float k_scale, float v_scale, void* k_cache, void* v_cache,
                          int64_t num_blocks, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* seq_lens,
                          const int32_t* query_start_loc, int32_t num_seqs,
                          int64_t num_q_tokens, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                          int32_t max_seq_len, int32_t common_prefix_len,
                          void* workspace, size_t workspace_bytes, void* stream) {
  pa_status s = kv8 ? check_fp8(k_scale, v_scale) : PA_OK;
  if (s != PA_OK) return s;
  s = check_scatter(name, k, v, k_token_stride, v_token_stride, slot_mapping,
                    num_new_tokens, num_kv_heads, head_dim, k_cache, v_cache, num_blocks);
  if (s != PA_OK) return s;
  pa::AttendArgs a;
  bool empty;
  s = prepare_attend(nullptr, nullptr, nullptr, num_blocks, block_tables,
                     max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                     num_q_tokens, num_q_heads, num_kv_heads, head_dim, max_query_len,
                     max_seq_len, 0.0f, nullptr, workspace, workspace_bytes, false, &a,
                     &empty, common_prefix_len < 0 ? -1 : common_prefix_len);
  if (s != PA_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (empty) {
    // nothing to plan: the scatter alone
    if (num_new_tokens == 0) return ok();
    e = kv8 ? pa::launch_write_kv8(static_cast<const uint16_t*>(k),
                                   static_cast<const uint16_t*>(v), k_token_stride,
                                   v_token_stride, slot_mapping, num_new_tokens,
                                   num_kv_heads, head_dim, k_scale, v_scale,
                                   static_cast<uint8_t*>(k_cache),
                                   static_cast<uint8_t*>(v_cache), num_blocks, st)
            : pa::launch_write_kv(static_cast<const uint16_t*>(k),
                                  static_cast<const uint16_t*>(v), k_token_stride,
                                  v_token_stride, slot_mapping, num_new_tokens,
                                  num_kv_heads, head_dim, static_cast<uint16_t*>(k_cache),
                                  static_cast<uint16_t*>(v_cache), num_blocks, st);
  } else {
    a.kv8 = kv8;
    pa::ScatterArgs sc;
    sc.k = static_cast<const uint16_t*>(k);
    sc.v = static_cast<const uint16_t*>(v);
    sc.k_stride = k_token_stride;
    sc.v_stride = v_token_stride;
    sc.slots = slot_mapping;
    sc.num_tokens = num_new_tokens;
    sc.Hkv = num_kv_heads;
    sc.k_scale = k_scale;
    sc.v_scale = v_scale;
    sc.k_cache = k_cache;
    sc.v_cache = v_cache;
    sc.num_slots = num_blocks * pa::kBlock;
    sc.per_block = 0;  // chosen by the launcher
    e = pa::launch_write_plan(a, sc, st);
  }
  if (e != hipSuccess) return hip_fail(e, (std::string(name) + " launch").c_str());
  return ok();
}

}  // namespace

pa_status pa_write_kv_plan(const void* k, const void* v, int64_t k_token_stride,
                           int64_t v_token_stride, const int64_t* slot_mapping,
                           int64_t num_new_tokens, void* k_cache, void* v_cache,
                           int64_t num_blocks, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                           const int32_t* query_start_loc, int32_t num_seqs,
                           int64_t num_q_tokens, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim,
                           int32_t max_query_len, int32_t max_seq_len,
                           int32_t common_prefix_len, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return write_plan_call("pa_write_kv_plan", false, k, v, k_token_stride, v_token_stride,
                         slot_mapping, num_new_tokens, 1.0f, 1.0f, k_cache, v_cache,
                         num_blocks, block_tables, max_blocks_per_seq, seq_lens,
                         query_start_loc, num_seqs, num_q_tokens, num_q_heads,
                         num_kv_heads, head_dim, max_query_len, max_seq_len,
                         common_prefix_len, workspace, workspace_bytes, stream);
}

pa_status pa_write_kv_plan_fp8(const void* k, const void* v, int64_t k_token_stride,
                               int64_t v_token_stride, const int64_t* slot_mapping,
                               int64_t num_new_tokens, float k_scale, float v_scale,
                               void* k_cache, void* v_cache, int64_t num_blocks,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, const int32_t* query_start_loc,
                               int32_t num_seqs, int64_t num_q_tokens,
                               int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_query_len,
                               int32_t max_seq_len, int32_t common_prefix_len,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return write_plan_call("pa_write_kv_plan_fp8", true, k, v, k_token_stride,
                         v_token_stride, slot_mapping, num_new_tokens, k_scale, v_scale,
                         k_cache, v_cache, num_blocks, block_tables, max_blocks_per_seq,
                         seq_lens, query_start_loc, num_seqs, num_q_tokens, num_q_heads,
                         num_kv_heads, head_dim, max_query_len, max_seq_len,
                         common_prefix_len, workspace, workspace_bytes, stream);
}

namespace {

// Attention (and optionally plan and merge) over a shared-prefix workspace.
pa_status cascade_call(const void* q, const void* k_cache, const void* v_cache,
                       int64_t num_blocks, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                       const int32_t* query_start_loc, int32_t num_seqs,
                       int64_t num_q_tokens, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_query_len, int32_t max_seq_len,
                       int32_t common_prefix_len, float scale, bool kv8,
                       float k_scale, float v_scale, void* out, void* workspace,
                       size_t workspace_bytes, void* stream, bool plan_and_merge,
                       const char* what) {
  if (kv8 && check_fp8(k_scale, v_scale) != PA_OK) return PA_ERR_SHAPE;
  pa::AttendArgs a;
  bool empty;
  pa_status s = prepare_attend(q, k_cache, v_cache, num_blocks, block_tables,
                               max_blocks_per_seq, seq_lens, query_start_loc,
                               num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                               head_dim, max_query_len, max_seq_len, scale, out,
                               workspace, workspace_bytes, true, &a, &empty,
                               common_prefix_len < 0 ? INT32_MAX : common_prefix_len);
  if (s != PA_OK) return s;
  if (empty) return ok();
  if (kv8) set_fp8(k_scale, v_scale, &a);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = plan_and_merge ? pa::launch_plan(a, st) : hipSuccess;
  if (e == hipSuccess) e = pa::launch_planned(a, st);
  if (e == hipSuccess && plan_and_merge) e = pa::launch_merge(a, st);
  if (e != hipSuccess) return hip_fail(e, what);
  return ok();
}

}  // namespace

pa_status pa_attend_planned_cascade(const void* q, const void* k_cache,
                                    const void* v_cache, int64_t num_blocks,
                                    const int32_t* block_tables,
                                    int32_t max_blocks_per_seq,
                                    const int32_t* seq_lens,
                                    const int32_t* query_start_loc,
                                    int32_t num_seqs, int64_t num_q_tokens,
                                    int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_query_len,
                                    int32_t max_seq_len, float scale, void* out,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return cascade_call(q, k_cache, v_cache, num_blocks, block_tables,
                      max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                      num_q_tokens, num_q_heads, num_kv_heads, head_dim,
                      max_query_len, max_seq_len, 0, scale, false, 1.0f, 1.0f,
                      out, workspace, workspace_bytes, stream, false,
                      "pa_attend_planned_cascade launch");
}

pa_status pa_attend_planned_cascade_fp8(
    const void* q, const void* k_cache, const void* v_cache, int64_t num_blocks,
    const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* seq_lens, const int32_t* query_start_loc, int32_t num_seqs,
    int64_t num_q_tokens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t max_query_len, int32_t max_seq_len, float scale,
    float k_scale, float v_scale, void* out, void* workspace,
    size_t workspace_bytes, void* stream) {
  return cascade_call(q, k_cache, v_cache, num_blocks, block_tables,
                      max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                      num_q_tokens, num_q_heads, num_kv_heads, head_dim,
                      max_query_len, max_seq_len, 0, scale, true, k_scale,
                      v_scale, out, workspace, workspace_bytes, stream, false,
                      "pa_attend_planned_cascade_fp8 launch");
}

pa_status pa_attend_merge_cascade(int32_t num_seqs, int64_t num_q_tokens,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_query_len,
                                  int32_t max_seq_len, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  pa::AttendArgs a;
  bool empty;
  static const int32_t kNone[2] = {0, 0};
  pa_status s = prepare_attend(nullptr, nullptr, nullptr, 0, kNone, 1, kNone,
                               kNone, num_seqs, num_q_tokens, num_q_heads,
                               num_kv_heads, head_dim, max_query_len,
                               max_seq_len, 0.0f, out, workspace,
                               workspace_bytes, false, &a, &empty, 0);
  if (s != PA_OK) return s;
  if (empty) return ok();
  if (!out) return fail(PA_ERR_NULL, "pa_attend_merge_cascade: NULL out");
  if ((uintptr_t)out & 15) return fail(PA_ERR_SHAPE, "out must be 16-byte aligned");
  hipError_t e = pa::launch_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_attend_merge_cascade launch");
  return ok();
}

pa_status pa_attend_cascade(const void* q, const void* k_cache,
                            const void* v_cache, int64_t num_blocks,
                            const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            const int32_t* query_start_loc, int32_t num_seqs,
                            int64_t num_q_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_query_len, int32_t max_seq_len,
                            int32_t common_prefix_len, float scale, void* out,
                            void* workspace, size_t workspace_bytes,
                            void* stream) {
  return cascade_call(q, k_cache, v_cache, num_blocks, block_tables,
                      max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                      num_q_tokens, num_q_heads, num_kv_heads, head_dim,
                      max_query_len, max_seq_len, common_prefix_len, scale, false,
                      1.0f, 1.0f, out, workspace, workspace_bytes, stream, true,
                      "pa_attend_cascade launch");
}

pa_status pa_attend_cascade_fp8(const void* q, const void* k_cache,
                                const void* v_cache, int64_t num_blocks,
                                const int32_t* block_tables,
                                int32_t max_blocks_per_seq,
                                const int32_t* seq_lens,
                                const int32_t* query_start_loc, int32_t num_seqs,
                                int64_t num_q_tokens, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_query_len, int32_t max_seq_len,
                                int32_t common_prefix_len, float scale,
                                float k_scale, float v_scale, void* out,
                                void* workspace, size_t workspace_bytes,
                                void* stream) {
  return cascade_call(q, k_cache, v_cache, num_blocks, block_tables,
                      max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                      num_q_tokens, num_q_heads, num_kv_heads, head_dim,
                      max_query_len, max_seq_len, common_prefix_len, scale, true,
                      k_scale, v_scale, out, workspace, workspace_bytes, stream,
                      true, "pa_attend_cascade_fp8 launch");
}

pa_status pa_validate_cascade_host(const int32_t* block_tables,
                                   int32_t max_blocks_per_seq,
                                   const int32_t* seq_lens,
                                   const int32_t* query_start_loc,
                                   int32_t num_seqs, int32_t common_prefix_len) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || common_prefix_len < 0)
    return fail(PA_ERR_SHAPE, "validate: negative size");
  if (num_seqs > 0 && (!block_tables || !seq_lens || !query_start_loc))
    return fail(PA_ERR_NULL, "validate: NULL pointer");
  const int64_t nshared = common_prefix_len / PA_BLOCK_SIZE;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const std::string at = " (request " + std::to_string(b) + ")";
    const int64_t Q = (int64_t)query_start_loc[b + 1] - query_start_loc[b];
    if ((int64_t)seq_lens[b] - Q < common_prefix_len)
      return fail(PA_ERR_METADATA, "a query lies inside the shared prefix" + at);
    if (nshared > max_blocks_per_seq)
      return fail(PA_ERR_METADATA, "block table row shorter than the shared prefix");
    for (int64_t j = 0; j < nshared; ++j)
      if (block_tables[(int64_t)b * max_blocks_per_seq + j] != block_tables[j])
        return fail(PA_ERR_METADATA, "shared prefix block differs from request 0's" + at);
  }
  return ok();
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, int64_t num_blocks,
                         int32_t num_kv_heads, int32_t head_dim, int32_t elem_bytes,
                         const int64_t* block_mapping, int64_t num_pairs,
                         void* stream) {
  if (num_blocks < 0 || num_pairs < 0)
    return fail(PA_ERR_SHAPE, "pa_copy_blocks: negative size");
  if (num_kv_heads <= 0) return fail(PA_ERR_SHAPE, "num_kv_heads must be > 0");
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (elem_bytes != 1 && elem_bytes != 2)
    return fail(PA_ERR_SHAPE, "elem_bytes must be 2 (bf16 pools) or 1 (8-bit pools)");
  if (num_pairs > (int64_t)1 << 30)
    return fail(PA_ERR_SHAPE, "pa_copy_blocks: too many pairs in one call");
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !block_mapping)
    return fail(PA_ERR_NULL, "pa_copy_blocks: NULL pointer");
  if (((uintptr_t)k_cache | (uintptr_t)v_cache) & 15)
    return fail(PA_ERR_SHAPE, "the pools must be 16-byte aligned");
  const int64_t block_bytes = (int64_t)num_kv_heads * PA_BLOCK_SIZE * head_dim * elem_bytes;
  hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, block_bytes, num_blocks,
                                        block_mapping, num_pairs,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_copy_blocks launch");
  return ok();
}

pa_status pa_expand_block_tables(const int32_t* block_tables, int32_t num_seqs,
                                 int32_t max_blocks_per_seq, int32_t block_size,
                                 int32_t* out, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 0)
    return fail(PA_ERR_SHAPE, "pa_expand_block_tables: negative size");
  if (block_size < PA_BLOCK_SIZE || block_size % PA_BLOCK_SIZE != 0 || block_size > (1 << 16))
    return fail(PA_ERR_UNSUPPORTED, "block_size must be a multiple of 16 (at most 65536)");
  const int R = block_size / PA_BLOCK_SIZE;
  if ((int64_t)max_blocks_per_seq * R > INT32_MAX)
    return fail(PA_ERR_SHAPE, "pa_expand_block_tables: expanded rows too long");
  if (num_seqs == 0 || max_blocks_per_seq == 0) return ok();
  if (!block_tables || !out) return fail(PA_ERR_NULL, "pa_expand_block_tables: NULL pointer");
  hipError_t e = pa::launch_expand_tables(block_tables, max_blocks_per_seq, num_seqs, R,
                                          out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_expand_block_tables launch");
  return ok();
}

// ---- multi-head latent attention ----------------------------------------

static_assert(pa::kMlaDim == PA_MLA_DIM && pa::kMlaLatent == PA_MLA_LATENT &&
                  pa::kMlaBlock == PA_MLA_BLOCK_SIZE,
              "MLA sizes of the header and the kernels agree");

size_t pa_mla_workspace_size(int64_t num_q_tokens, int32_t num_q_heads,
                             int32_t max_seq_len) {
  if (num_q_tokens < 0 || num_q_tokens >= pa::kMlaMaxTokens || num_q_heads <= 0 ||
      num_q_heads % 16 != 0 || max_seq_len < 0)
    return 0;
  return pa::mla_workspace_bytes(num_q_tokens, num_q_heads, max_seq_len);  // 0 past kMlaMaxGrid
}

pa_status pa_mla_write_kv(const void* kv, int64_t kv_token_stride,
                          const int64_t* slot_mapping, int64_t num_tokens, void* cache,
                          int64_t num_blocks, void* stream) {
  if (num_tokens < 0 || num_blocks < 0)
    return fail(PA_ERR_SHAPE, "pa_mla_write_kv: negative size");
  if (num_tokens == 0) return ok();
  if (!kv || !slot_mapping || !cache) return fail(PA_ERR_NULL, "pa_mla_write_kv: NULL pointer");
  if (kv_token_stride < PA_MLA_DIM || kv_token_stride % 8 != 0)
    return fail(PA_ERR_SHAPE, "kv_token_stride must be >= 576 and a multiple of 8");
  if (((uintptr_t)kv | (uintptr_t)cache) & 15)
    return fail(PA_ERR_SHAPE, "kv and the cache must be 16-byte aligned");
  hipError_t e = pa::launch_mla_write_kv(static_cast<const uint16_t*>(kv), kv_token_stride,
                                         slot_mapping, num_tokens,
                                         static_cast<uint16_t*>(cache), num_blocks,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_mla_write_kv launch");
  return ok();
}

pa_status pa_mla_decode(const void* q, const void* cache, int64_t num_blocks,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* seq_lens, const int32_t* query_start_loc,
                        int32_t num_seqs, int64_t num_q_tokens, int32_t num_q_heads,
                        int32_t max_seq_len, float scale, void* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || num_q_tokens < 0 || num_blocks < 0 || max_blocks_per_seq < 0 ||
      max_seq_len < 0)
    return fail(PA_ERR_SHAPE, "pa_mla_decode: negative size");
  if (num_q_heads <= 0 || num_q_heads % 16 != 0 || num_q_heads > 128)
    return fail(PA_ERR_UNSUPPORTED, "num_q_heads must be a multiple of 16, at most 128");
  if (num_q_tokens > INT32_MAX / 2)
    return fail(PA_ERR_SHAPE, "pa_mla_decode: num_q_tokens too large");
  if (max_seq_len > (1 << 18))
    return fail(PA_ERR_UNSUPPORTED, "pa_mla_decode: max_seq_len above 262144");
  if (num_seqs > pa::kMlaMaxSeqs)
    return fail(PA_ERR_UNSUPPORTED, "pa_mla_decode: num_seqs above 131072");
  if (num_q_tokens >= pa::kMlaMaxTokens)
    return fail(PA_ERR_UNSUPPORTED, "pa_mla_decode: num_q_tokens of 2^25 or more");
  if (num_blocks > pa::kMlaMaxBlocks)
    return fail(PA_ERR_UNSUPPORTED, "pa_mla_decode: num_blocks above 2^29");
  if (num_q_tokens == 0 || num_seqs == 0) return ok();
  if (!q || !cache || !block_tables || !seq_lens || !query_start_loc || !out)
    return fail(PA_ERR_NULL, "pa_mla_decode: NULL pointer");
  if (max_blocks_per_seq == 0 || num_blocks == 0 || max_seq_len == 0)
    return fail(PA_ERR_SHAPE, "pa_mla_decode: empty cache, block table or max_seq_len");
  if (!(scale > 0.0f && scale <= FLT_MAX))
    return fail(PA_ERR_SHAPE, "pa_mla_decode: scale must be finite and > 0");
  if (((uintptr_t)q | (uintptr_t)cache | (uintptr_t)out) & 15)
    return fail(PA_ERR_SHAPE, "q, out and the cache must be 16-byte aligned");
  const int group = pa::mla_group(num_q_heads, num_q_tokens, num_seqs);
  const pa::MlaLayout m = pa::mla_layout(num_q_tokens, num_q_heads, max_seq_len, group);
  if (m.grid <= 0)
    return fail(PA_ERR_UNSUPPORTED, "pa_mla_decode: more work than one launch takes");
  if (((int64_t)num_q_tokens * num_q_heads + 3) / 4 > INT32_MAX)
    return fail(PA_ERR_SHAPE, "pa_mla_decode: too many (token, head) rows");
  if (m.grid > 1) {
    if (!workspace || workspace_bytes < m.total)
      return fail(PA_ERR_WORKSPACE, "pa_mla_decode: workspace needs " +
                                        std::to_string(m.total) + " bytes, got " +
                                        std::to_string(workspace_bytes));
    if ((uintptr_t)workspace & 255)
      return fail(PA_ERR_WORKSPACE, "pa_mla_decode: workspace must be 256-byte aligned");
  }
  pa::MlaParams P;
  P.q = static_cast<const uint16_t*>(q);
  P.cache = static_cast<const uint16_t*>(cache);
  P.num_blocks = num_blocks;
  P.bt = block_tables;
  P.bt_stride = max_blocks_per_seq;
  P.seq_lens = seq_lens;
  P.qsl = query_start_loc;
  P.num_seqs = num_seqs;
  P.num_q_tokens = (int32_t)num_q_tokens;
  P.Hq = num_q_heads;
  P.max_seq_len = max_seq_len;
  P.grid = m.grid;
  P.G = group;
  P.scale_log2 = scale * 1.4426950408889634f;
  P.out = static_cast<uint16_t*>(out);
  char* ws = static_cast<char*>(workspace);
  P.seg = m.grid > 1 ? reinterpret_cast<int2*>(ws + m.seg) : nullptr;
  P.part_ml = m.grid > 1 ? reinterpret_cast<float2*>(ws + m.part_ml) : nullptr;
  P.part_out = m.grid > 1 ? reinterpret_cast<uint16_t*>(ws + m.part_out) : nullptr;
  hipError_t e = pa::launch_mla_decode(P, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_mla_decode launch");
  return ok();
}

pa_status pa_gather_kv(const void* k_cache, const void* v_cache,
                       int64_t num_blocks, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                       const int64_t* kv_start, int32_t num_seqs,
                       int64_t total_rows, int32_t num_kv_heads,
                       int32_t head_dim, void* k_out, void* v_out,
                       void* stream) {
  if (num_seqs < 0 || total_rows < 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return fail(PA_ERR_SHAPE, "pa_gather_kv: negative size");
  if (num_kv_heads <= 0) return fail(PA_ERR_SHAPE, "num_kv_heads must be > 0");
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (total_rows == 0 || num_seqs == 0) return ok();
  if (!k_cache || !v_cache || !block_tables || !seq_lens || !kv_start ||
      !k_out || !v_out)
    return fail(PA_ERR_NULL, "pa_gather_kv: NULL pointer");
  hipError_t e = pa::launch_gather_kv(
      static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
      num_blocks, block_tables, max_blocks_per_seq, seq_lens, kv_start, num_seqs,
      total_rows, num_kv_heads, head_dim, static_cast<uint16_t*>(k_out),
      static_cast<uint16_t*>(v_out), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_gather_kv launch");
  return ok();
}

pa_status pa_write_kv_bs(const void* k, const void* v, int64_t k_token_stride,
                         int64_t v_token_stride, const int64_t* slot_mapping,
                         int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                         void* k_cache, void* v_cache, int64_t num_blocks,
                         int32_t block_size, void* stream) {
  if (block_size != 8 && block_size != 16)
    return fail(PA_ERR_UNSUPPORTED,
                "pa_write_kv_bs: block_size must be 8 or 16 (larger blocks: 16-token "
                "pools, see pa_expand_block_tables)");
  pa_status s = check_scatter("pa_write_kv_bs", k, v, k_token_stride, v_token_stride,
                              slot_mapping, num_tokens, num_kv_heads, head_dim, k_cache,
                              v_cache, num_blocks);
  if (s != PA_OK || num_tokens == 0) return s == PA_OK ? ok() : s;
  hipError_t e = pa::launch_write_kv(
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), k_token_stride,
      v_token_stride, slot_mapping, num_tokens, num_kv_heads, head_dim,
      static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), num_blocks,
      static_cast<hipStream_t>(stream), block_size);
  if (e != hipSuccess) return hip_fail(e, "pa_write_kv_bs launch");
  return ok();
}

pa_status pa_attend_bs(const void* q, const void* k_cache, const void* v_cache,
                       int64_t num_blocks, int32_t block_size,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* seq_lens, const int32_t* query_start_loc,
                       int32_t num_seqs, int64_t num_q_tokens, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                       int32_t max_seq_len, float scale, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (block_size != 8 && block_size != 16)
    return fail(PA_ERR_UNSUPPORTED,
                "pa_attend_bs: block_size must be 8 or 16 (larger blocks: 16-token "
                "pools, see pa_expand_block_tables)");
  pa::AttendArgs a;
  bool empty;
  pa_status s = prepare_attend(q, k_cache, v_cache, num_blocks, block_tables,
                               max_blocks_per_seq, seq_lens, query_start_loc,
                               num_seqs, num_q_tokens, num_q_heads, num_kv_heads,
                               head_dim, max_query_len, max_seq_len, scale, out,
                               workspace, workspace_bytes, true, &a, &empty);
  if (s != PA_OK) return s;
  if (empty) return ok();
  a.block_size = block_size;
  hipError_t e = pa::launch_plan(a, static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = pa::launch_planned(a, static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = pa::launch_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pa_attend_bs launch");
  return ok();
}

pa_status pa_gather_kv_bs(const void* k_cache, const void* v_cache, int64_t num_blocks,
                          int32_t block_size, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* seq_lens,
                          const int64_t* kv_start, int32_t num_seqs, int64_t total_rows,
                          int32_t num_kv_heads, int32_t head_dim, void* k_out,
                          void* v_out, void* stream) {
  if (block_size != 8 && block_size != 16)
    return fail(PA_ERR_UNSUPPORTED, "pa_gather_kv_bs: block_size must be 8 or 16");
  if (num_seqs < 0 || total_rows < 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return fail(PA_ERR_SHAPE, "pa_gather_kv_bs: negative size");
  if (num_kv_heads <= 0) return fail(PA_ERR_SHAPE, "num_kv_heads must be > 0");
  if (!supported_head_dim(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (total_rows == 0 || num_seqs == 0) return ok();
  if (!k_cache || !v_cache || !block_tables || !seq_lens || !kv_start || !k_out || !v_out)
    return fail(PA_ERR_NULL, "pa_gather_kv_bs: NULL pointer");
  hipError_t e = pa::launch_gather_kv(
      static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
      num_blocks, block_tables, max_blocks_per_seq, seq_lens, kv_start, num_seqs,
      total_rows, num_kv_heads, head_dim, static_cast<uint16_t*>(k_out),
      static_cast<uint16_t*>(v_out), static_cast<hipStream_t>(stream), block_size);
  if (e != hipSuccess) return hip_fail(e, "pa_gather_kv_bs launch");
  return ok();
}

pa_status pa_validate_metadata_host(const int32_t* block_tables,
                                    int32_t max_blocks_per_seq,
                                    const int32_t* seq_lens,
                                    const int32_t* query_start_loc,
                                    int32_t num_seqs, int64_t num_q_tokens,
                                    int32_t max_query_len, int32_t max_seq_len,
                                    int64_t num_blocks,
                                    const int64_t* slot_mapping,
                                    int64_t num_slots) {
  if (num_seqs < 0 || num_q_tokens < 0 || max_blocks_per_seq < 0 || num_blocks < 0)
    return fail(PA_ERR_SHAPE, "validate: negative size");
  if (num_seqs > 0 && (!block_tables || !seq_lens || !query_start_loc))
    return fail(PA_ERR_NULL, "validate: NULL pointer");
  if (num_seqs > 0 && query_start_loc[0] != 0)
    return fail(PA_ERR_METADATA, "query_start_loc[0] != 0");
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t q0 = query_start_loc[b], q1 = query_start_loc[b + 1];
    const int64_t L = seq_lens[b];
    const std::string at = " (request " + std::to_string(b) + ")";
    if (q1 < q0) return fail(PA_ERR_METADATA, "query_start_loc decreases" + at);
    if (L < 0) return fail(PA_ERR_METADATA, "seq_len < 0" + at);
    if (q1 - q0 > L) return fail(PA_ERR_METADATA, "query length > seq_len" + at);
    if (L > max_seq_len) return fail(PA_ERR_METADATA, "seq_len > max_seq_len" + at);
    if (q1 - q0 > max_query_len)
      return fail(PA_ERR_METADATA, "query length > max_query_len" + at);
    const int64_t nb = (L + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE;
    if (nb > max_blocks_per_seq)
      return fail(PA_ERR_METADATA, "block table row too short" + at);
    for (int64_t j = 0; j < nb; ++j) {
      const int64_t id = block_tables[(int64_t)b * max_blocks_per_seq + j];
      if (id < 0 || id >= num_blocks)
        return fail(PA_ERR_METADATA, "block id out of range" + at);
    }
  }
  if (num_seqs > 0 && query_start_loc[num_seqs] != num_q_tokens)
    return fail(PA_ERR_METADATA, "query_start_loc[num_seqs] != num_q_tokens");
  if (slot_mapping && num_slots > 0) {
    std::unordered_set<int64_t> seen;
    seen.reserve((size_t)num_slots * 2);
    for (int64_t i = 0; i < num_slots; ++i) {
      const int64_t s = slot_mapping[i];
      if (s < 0) continue;
      if (s >= num_blocks * PA_BLOCK_SIZE)
        return fail(PA_ERR_METADATA, "slot out of range (token " + std::to_string(i) + ")");
      if (!seen.insert(s).second)
        return fail(PA_ERR_METADATA, "duplicate slot (token " + std::to_string(i) + ")");
    }
  }
  return ok();
}

pa_status pa_validate_metadata(const int32_t* block_tables,
                               int32_t max_blocks_per_seq,
                               const int32_t* seq_lens,
                               const int32_t* query_start_loc,
                               int32_t num_seqs, int64_t num_q_tokens,
                               int32_t max_query_len, int32_t max_seq_len,
                               int64_t num_blocks, const int64_t* slot_mapping,
                               int64_t num_slots) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || num_slots < 0)
    return fail(PA_ERR_SHAPE, "validate: negative size");
  if (num_seqs > 0 && (!block_tables || !seq_lens || !query_start_loc))
    return fail(PA_ERR_NULL, "validate: NULL pointer");
  std::vector<int32_t> bt((size_t)num_seqs * max_blocks_per_seq);
  std::vector<int32_t> sl(num_seqs), qsl(num_seqs + 1);
  std::vector<int64_t> sm(slot_mapping ? num_slots : 0);
  hipError_t e = hipSuccess;
  if (num_seqs > 0) {
    if (!bt.empty())
      e = hipMemcpy(bt.data(), block_tables, bt.size() * 4, hipMemcpyDeviceToHost);
    if (e == hipSuccess)
      e = hipMemcpy(sl.data(), seq_lens, sl.size() * 4, hipMemcpyDeviceToHost);
    if (e == hipSuccess)
      e = hipMemcpy(qsl.data(), query_start_loc, qsl.size() * 4, hipMemcpyDeviceToHost);
  }
  if (e == hipSuccess && !sm.empty())
    e = hipMemcpy(sm.data(), slot_mapping, sm.size() * 8, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "validate: copy to host");
  return pa_validate_metadata_host(bt.data(), max_blocks_per_seq, sl.data(),
                                   qsl.data(), num_seqs, num_q_tokens,
                                   max_query_len, max_seq_len, num_blocks,
                                   sm.empty() ? nullptr : sm.data(),
                                   (int64_t)sm.size());
}

}  // extern "C"
