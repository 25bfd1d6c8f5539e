// api.hip -- the extern "C" entry points of libpkv (declared in include/pkv.h).
// Host-side validation of scalar arguments, then kernel launches on the
// caller's stream.  Nothing here reads device memory or allocates.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "pkv_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A dispatch counts its work-items in 32 bits: at 256 per workgroup, at most
// 2^24 - 1 workgroups.
constexpr int64_t kMaxWorkgroups = (INT64_C(1) << 24) - 1;

// The checked build validates device data before launching (checks.hip); the
// regular build compiles the checks away without evaluating them.
#ifdef PKV_DEBUG_CHECKS
#define PKV_CHECK(call)                  \
  do {                                   \
    const pkv_status check_ = (call);    \
    if (check_ != PKV_OK) return check_; \
  } while (0)
#else
#define PKV_CHECK(call) \
  do {                  \
  } while (0)
#endif

pkv_status launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_DEVICE_DATA: return "device data breaks a precondition (checked build)";
    case PKV_ERR_SCRATCH_LIMIT:
      return "the call needs more scratch than the static buffer of "
             "pkv_paged_attention_varlen_noalloc holds (PKV_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int32_t pkv_debug_checks_enabled(void) {
#ifdef PKV_DEBUG_CHECKS
  return 1;
#else
  return 0;
#endif
}

uint32_t pkv_debug_check_flags(void) {
#ifdef PKV_DEBUG_CHECKS
  return pkv::last_check_flags();
#else
  return 0u;
#endif
}

}  // extern "C"

// Host checks of pkv_prepare_inputs' arguments.
static pkv_status prepare_args_status(const int32_t* num_scheduled_tokens,
                                      const int32_t* num_computed_tokens,
                                      const int32_t* block_table, int64_t bt_row_stride,
                                      int32_t num_reqs, int32_t num_tokens, int32_t qsl_len,
                                      int32_t block_size, int64_t num_blocks,
                                      const int32_t* req_indices, const int32_t* positions,
                                      const int64_t* slot_mapping,
                                      const int32_t* query_start_loc, const int32_t* seq_lens,
                                      const int32_t* logits_indices) {
  if (num_reqs < 0 || num_tokens < 0 || qsl_len < num_reqs + 1 || block_size < 1 ||
      num_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  if (!query_start_loc) return PKV_ERR_INVALID_ARG;
  if (num_reqs > 0 &&
      (!num_scheduled_tokens || !num_computed_tokens || !seq_lens || !logits_indices))
    return PKV_ERR_INVALID_ARG;
  if (num_tokens > 0 && (num_reqs == 0 || !block_table || bt_row_stride < 1 || !req_indices ||
                         !positions || !slot_mapping))
    return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

extern "C" {

pkv_status pkv_prepare_inputs(const int32_t* num_scheduled_tokens,
                              const int32_t* num_computed_tokens, const int32_t* block_table,
                              int64_t bt_row_stride, int32_t num_reqs, int32_t num_tokens,
                              int32_t qsl_len, int32_t block_size, int64_t num_blocks,
                              int32_t* req_indices, int32_t* positions, int64_t* slot_mapping,
                              int32_t* query_start_loc, int32_t* seq_lens,
                              int32_t* logits_indices, void* stream) {
  const pkv_status st = prepare_args_status(
      num_scheduled_tokens, num_computed_tokens, block_table, bt_row_stride, num_reqs,
      num_tokens, qsl_len, block_size, num_blocks, req_indices, positions, slot_mapping,
      query_start_loc, seq_lens, logits_indices);
  if (st != PKV_OK) return st;
  PKV_CHECK(pkv::check_prepare(num_scheduled_tokens, num_computed_tokens, block_table,
                               bt_row_stride, num_reqs, num_tokens, block_size, num_blocks,
                               static_cast<hipStream_t>(stream)));
  return launch_status(pkv::launch_prepare(
      num_scheduled_tokens, num_computed_tokens, block_table, bt_row_stride, num_reqs,
      num_tokens, qsl_len, block_size, num_blocks, req_indices, positions, slot_mapping,
      query_start_loc, seq_lens, logits_indices, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_prepare_input_ids(const int32_t* token_table, int64_t row_width,
                                 int32_t num_reqs, const int32_t* req_indices,
                                 const int32_t* positions, int32_t num_tokens,
                                 const int32_t* seq_lens, const int32_t* num_tokens_total,
                                 int64_t* token_indices, int32_t* input_ids,
                                 uint8_t* discard_request_mask, void* stream) {
  if (num_reqs < 0 || num_tokens < 0 || row_width < 1) return PKV_ERR_INVALID_ARG;
  if (num_tokens > 0 && (!token_table || !req_indices || !positions || !input_ids))
    return PKV_ERR_INVALID_ARG;
  if (num_reqs > 0 && (!seq_lens || !num_tokens_total || !discard_request_mask))
    return PKV_ERR_INVALID_ARG;
  PKV_CHECK(pkv::check_rows(req_indices, positions, num_tokens, num_reqs, row_width,
                            static_cast<hipStream_t>(stream)));
  return launch_status(pkv::launch_input_ids(
      token_table, row_width, num_reqs, req_indices, positions, num_tokens, seq_lens,
      num_tokens_total, token_indices, input_ids, discard_request_mask,
      static_cast<hipStream_t>(stream)));
}

pkv_status pkv_kv_cache_write(const void* key, const void* value, int64_t key_row_stride,
                              int64_t value_row_stride, void* key_cache, void* value_cache,
                              int64_t num_blocks, const int64_t* slot_mapping,
                              int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, pkv_dtype dtype, void* stream) {
  if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_INVALID_ARG;
  const int32_t esz = dtype == PKV_BF16 ? 2 : 4;
  if ((int64_t)head_dim * esz % 16 != 0 || head_dim > 256) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (key_row_stride < row || value_row_stride < row) return PKV_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache) ||
      key_row_stride * esz % 16 != 0 || value_row_stride * esz % 16 != 0)
    return PKV_ERR_INVALID_ARG;
  if (num_kv_heads > 65535) return PKV_ERR_UNSUPPORTED;
  PKV_CHECK(pkv::check_slots(slot_mapping, num_tokens, num_blocks * block_size, nullptr,
                             nullptr, static_cast<hipStream_t>(stream)));
  return launch_status(pkv::launch_kv_write(key, value, key_row_stride, value_row_stride,
                                            key_cache, value_cache, num_blocks, slot_mapping,
                                            num_tokens, num_kv_heads, head_dim, block_size, esz,
                                            static_cast<hipStream_t>(stream)));
}

pkv_status pkv_kv_cache_write_fp8(const void* key, const void* value, int64_t key_row_stride,
                                  int64_t value_row_stride, void* key_cache, void* value_cache,
                                  int64_t num_blocks, const int64_t* slot_mapping,
                                  int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, pkv_dtype dtype, const float* k_scale,
                                  const float* v_scale, void* stream) {
  if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_INVALID_ARG;
  if (block_size != pkv::kBlock || head_dim % 64 != 0 || head_dim > 256)
    return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  const int32_t esz = dtype == PKV_BF16 ? 2 : 4;
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping || !k_scale || !v_scale)
    return PKV_ERR_INVALID_ARG;
  if (key_row_stride < row || value_row_stride < row) return PKV_ERR_INVALID_ARG;
  if (!aligned16(key_cache) || !aligned16(value_cache) ||
      (reinterpret_cast<uintptr_t>(key) & (esz - 1)) != 0 ||
      (reinterpret_cast<uintptr_t>(value) & (esz - 1)) != 0 ||
      (reinterpret_cast<uintptr_t>(k_scale) & 3) != 0 ||
      (reinterpret_cast<uintptr_t>(v_scale) & 3) != 0)
    return PKV_ERR_INVALID_ARG;
  if (num_kv_heads > 65535) return PKV_ERR_UNSUPPORTED;
  PKV_CHECK(pkv::check_slots(slot_mapping, num_tokens, num_blocks * pkv::kBlock, k_scale,
                             v_scale, static_cast<hipStream_t>(stream)));
  return launch_status(pkv::launch_kv_write_fp8(key, value, key_row_stride, value_row_stride,
                                                key_cache, value_cache, num_blocks, slot_mapping,
                                                num_tokens, num_kv_heads, head_dim, esz, k_scale,
                                                v_scale, static_cast<hipStream_t>(stream)));
}

size_t pkv_paged_attention_workspace_bytes(int32_t num_reqs, int32_t num_tokens,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t max_query_len,
                                           int32_t max_seq_len, int32_t split_tokens,
                                           pkv_dtype dtype) {
  pkv::AttnPlan plan;
  if (!pkv::make_attn_plan(num_reqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                           max_query_len, max_seq_len, split_tokens, dtype, &plan))
    return 0;
  return plan.total_bytes;
}

pkv_status pkv_copy_blocks(void* key_cache, void* value_cache, int64_t num_blocks,
                           int64_t block_bytes, const int32_t* block_pairs, int32_t num_pairs,
                           void* stream) {
  if (num_blocks < 0 || block_bytes < 16 || num_pairs < 0) return PKV_ERR_INVALID_ARG;
  if (num_pairs > 0 && (!key_cache || !value_cache || !block_pairs)) return PKV_ERR_INVALID_ARG;
  if ((block_bytes & 15) != 0 || !aligned16(key_cache) || !aligned16(value_cache))
    return PKV_ERR_UNSUPPORTED;
  if (pkv::block_op_workgroups(block_bytes, num_pairs) > kMaxWorkgroups) return PKV_ERR_UNSUPPORTED;
  PKV_CHECK(pkv::check_block_list(block_pairs, num_pairs, true, num_blocks,
                                  static_cast<hipStream_t>(stream)));
  return launch_status(pkv::launch_copy_blocks(key_cache, value_cache, num_blocks, block_bytes,
                                               block_pairs, num_pairs,
                                               static_cast<hipStream_t>(stream)));
}

pkv_status pkv_zero_blocks(void* key_cache, void* value_cache, int64_t num_blocks,
                           int64_t block_bytes, const int32_t* block_ids, int32_t num_ids,
                           void* stream) {
  if (num_blocks < 0 || block_bytes < 16 || num_ids < 0) return PKV_ERR_INVALID_ARG;
  if (num_ids > 0 && (!key_cache || !value_cache || !block_ids)) return PKV_ERR_INVALID_ARG;
  if ((block_bytes & 15) != 0 || !aligned16(key_cache) || !aligned16(value_cache))
    return PKV_ERR_UNSUPPORTED;
  if (pkv::block_op_workgroups(block_bytes, num_ids) > kMaxWorkgroups) return PKV_ERR_UNSUPPORTED;
  PKV_CHECK(pkv::check_block_list(block_ids, num_ids, false, num_blocks,
                                  static_cast<hipStream_t>(stream)));
  return launch_status(pkv::launch_zero_blocks(key_cache, value_cache, num_blocks, block_bytes,
                                               block_ids, num_ids,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// What an attention call does: plan and run (pkv_paged_attention_varlen*),
// or one of the two (pkv_paged_attention_plan / pkv_paged_attention_run).
enum class AttnMode { kFused, kPlan, kRun };

// FNV-1a over the sizes a work list depends on.
static uint32_t plan_fingerprint(const pkv::AttnPlan& plan, int32_t num_reqs, int32_t num_tokens,
                                 int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim) {
  const int64_t v[] = {num_reqs,     num_tokens, max_query_len,      max_seq_len, num_q_heads,
                       num_kv_heads, head_dim,   plan.split_tokens, plan.max_splits};
  uint32_t h = 2166136261u;
  for (int64_t x : v)
    for (int k = 0; k < 8; ++k) h = (h ^ (uint32_t)((x >> (8 * k)) & 0xff)) * 16777619u;
  return h;
}

// Host checks of an attention call's sizes and its work-list plan (every
// attention entry point; `runs` for the calls that run the kernels).
static pkv_status attention_plan_for(bool runs, int32_t num_reqs, int32_t num_tokens,
                                     int32_t max_query_len, int32_t max_seq_len,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, float scale, pkv_dtype dtype,
                                     int32_t split_tokens, pkv::AttnPlan* plan) {
  if (num_reqs < 0 || num_tokens < 0 || max_query_len < 0 || max_seq_len < 0 ||
      num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 ||
      split_tokens < 0 || split_tokens % 32 != 0)
    return PKV_ERR_INVALID_ARG;
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_ERR_INVALID_ARG;
  if (runs && (!(scale > 0.f) || scale == HUGE_VALF)) return PKV_ERR_INVALID_ARG;  // and NaN
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (runs && block_size != pkv::kBlock) return PKV_ERR_UNSUPPORTED;
  const int32_t group = num_q_heads / num_kv_heads;
  if (dtype == PKV_BF16 && group > pkv::kPairsPerTile) return PKV_ERR_UNSUPPORTED;
  if (num_q_heads > 65535) return PKV_ERR_UNSUPPORTED;
  if (!pkv::make_attn_plan(num_reqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                           max_query_len, max_seq_len, split_tokens, dtype, plan))
    return PKV_ERR_INVALID_ARG;
  if (plan->grid > kMaxWorkgroups) return PKV_ERR_UNSUPPORTED;  // one workgroup per item + helpers
  return PKV_OK;
}

static bool workspace_fits(const pkv::AttnPlan& plan, const void* workspace,
                           size_t workspace_bytes) {
  return plan.total_bytes == 0 ||
         (workspace != nullptr && workspace_bytes >= plan.total_bytes &&
          (reinterpret_cast<uintptr_t>(workspace) & 255u) == 0);
}

static pkv_status attention_call(
    AttnMode mode, const void* q, int64_t q_row_stride, const void* key_cache,
    const void* value_cache, int64_t num_blocks, void* out, int64_t out_row_stride,
    const int32_t* query_start_loc, const int32_t* seq_lens, const int32_t* block_table,
    int64_t bt_row_stride, int32_t num_reqs, int32_t num_tokens, int32_t max_query_len,
    int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, float scale, pkv_dtype dtype, const float* k_scale,
    const float* v_scale, int32_t split_tokens, void* workspace, size_t workspace_bytes,
    void* stream) {
  const bool kv8 = k_scale != nullptr;
  const bool runs = mode != AttnMode::kPlan;
  pkv::AttnPlan plan;
  const pkv_status st =
      attention_plan_for(runs, num_reqs, num_tokens, max_query_len, max_seq_len, num_q_heads,
                         num_kv_heads, head_dim, block_size, scale, dtype, split_tokens, &plan);
  if (st != PKV_OK) return st;
  if (num_tokens == 0 || num_reqs == 0) return PKV_OK;
  if (!query_start_loc || !seq_lens) return PKV_ERR_INVALID_ARG;
  const int32_t esz = dtype == PKV_BF16 ? 2 : 4;
  if (runs) {
    if (!q || !key_cache || !value_cache || !out || !block_table) return PKV_ERR_INVALID_ARG;
    if (kv8 && (!v_scale || (reinterpret_cast<uintptr_t>(k_scale) & 3) != 0 ||
                (reinterpret_cast<uintptr_t>(v_scale) & 3) != 0))
      return PKV_ERR_INVALID_ARG;
    const int64_t row = (int64_t)num_q_heads * head_dim;
    if (q_row_stride < row || out_row_stride < row || bt_row_stride < 1 || num_blocks < 1)
      return PKV_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out) || !aligned16(key_cache) || !aligned16(value_cache) ||
        q_row_stride * esz % 16 != 0 || out_row_stride * esz % 16 != 0)
      return PKV_ERR_INVALID_ARG;
  }
  if (!workspace_fits(plan, workspace, workspace_bytes)) return PKV_ERR_WORKSPACE;

  pkv::AttnArgs a;
  a.q = q;
  a.q_stride = q_row_stride;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.num_blocks = num_blocks;
  a.out = out;
  a.out_stride = out_row_stride;
  a.qsl = query_start_loc;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.bt_stride = bt_row_stride;
  a.num_reqs = num_reqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.scale = scale;
  a.k_scale = kv8 ? k_scale : nullptr;
  a.v_scale = kv8 ? v_scale : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t fp = plan_fingerprint(plan, num_reqs, num_tokens, max_query_len, max_seq_len,
                                       num_q_heads, num_kv_heads, head_dim);
  // a run over a work list made earlier: a checked build compares its record
  const int32_t* planned =
      mode == AttnMode::kRun && plan.total_bytes > 0 ? static_cast<const int32_t*>(workspace)
                                                     : nullptr;
  (void)planned;  // read by the checked build only
  PKV_CHECK(pkv::check_attention(query_start_loc, seq_lens, runs ? block_table : nullptr,
                                 bt_row_stride, num_reqs, num_tokens, max_query_len, max_seq_len,
                                 num_blocks, a.k_scale, a.v_scale, planned, fp, s));
  if (dtype == PKV_BF16) {
    if (mode != AttnMode::kRun) {
      const hipError_t e = pkv::launch_attention_plan(a, plan, workspace, fp, s);
      if (e != hipSuccess) return launch_status(e);
    }
    if (!runs) return PKV_OK;
    return launch_status(pkv::launch_attention_run(a, plan, workspace, kv8, s));
  }
  if (!runs) return PKV_OK;  // the fp32 path has no work list
  return launch_status(pkv::launch_attention_f32(a, s));
}

extern "C" {

pkv_status pkv_paged_attention_varlen(
    const void* q, int64_t q_row_stride, const void* key_cache, const void* value_cache,
    int64_t num_blocks, void* out, int64_t out_row_stride, const int32_t* query_start_loc,
    const int32_t* seq_lens, const int32_t* block_table, int64_t bt_row_stride,
    int32_t num_reqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float scale, pkv_dtype dtype, int32_t split_tokens, void* workspace,
    size_t workspace_bytes, void* stream) {
  return attention_call(AttnMode::kFused, q, q_row_stride, key_cache, value_cache, num_blocks,
                        out, out_row_stride, query_start_loc, seq_lens, block_table,
                        bt_row_stride, num_reqs, num_tokens, max_query_len, max_seq_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, scale, dtype, nullptr,
                        nullptr, split_tokens, workspace, workspace_bytes, stream);
}

pkv_status pkv_paged_attention_varlen_fp8(
    const void* q, int64_t q_row_stride, const void* key_cache, const void* value_cache,
    int64_t num_blocks, void* out, int64_t out_row_stride, const int32_t* query_start_loc,
    const int32_t* seq_lens, const int32_t* block_table, int64_t bt_row_stride,
    int32_t num_reqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float scale, const float* k_scale, const float* v_scale, int32_t split_tokens,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_scale || !v_scale) return PKV_ERR_INVALID_ARG;
  return attention_call(AttnMode::kFused, q, q_row_stride, key_cache, value_cache, num_blocks,
                        out, out_row_stride, query_start_loc, seq_lens, block_table,
                        bt_row_stride, num_reqs, num_tokens, max_query_len, max_seq_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, scale, PKV_BF16,
                        k_scale, v_scale, split_tokens, workspace, workspace_bytes, stream);
}

pkv_status pkv_paged_attention_plan(const int32_t* query_start_loc, const int32_t* seq_lens,
                                    int32_t num_reqs, int32_t num_tokens, int32_t max_query_len,
                                    int32_t max_seq_len, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype,
                                    int32_t split_tokens, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return attention_call(AttnMode::kPlan, nullptr, 0, nullptr, nullptr, 0, nullptr, 0,
                        query_start_loc, seq_lens, nullptr, 0, num_reqs, num_tokens,
                        max_query_len, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                        pkv::kBlock, 1.f, dtype, nullptr, nullptr, split_tokens, workspace,
                        workspace_bytes, stream);
}

pkv_status pkv_prepare_inputs_and_plan(
    const int32_t* num_scheduled_tokens, const int32_t* num_computed_tokens,
    const int32_t* block_table, int64_t bt_row_stride, int32_t num_reqs, int32_t num_tokens,
    int32_t qsl_len, int32_t block_size, int64_t num_blocks, int32_t* req_indices,
    int32_t* positions, int64_t* slot_mapping, int32_t* query_start_loc, int32_t* seq_lens,
    int32_t* logits_indices, int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype, int32_t split_tokens,
    void* workspace, size_t workspace_bytes, void* stream) {
  pkv_status st = prepare_args_status(
      num_scheduled_tokens, num_computed_tokens, block_table, bt_row_stride, num_reqs,
      num_tokens, qsl_len, block_size, num_blocks, req_indices, positions, slot_mapping,
      query_start_loc, seq_lens, logits_indices);
  if (st != PKV_OK) return st;
  pkv::AttnPlan plan;
  st = attention_plan_for(false, num_reqs, num_tokens, max_query_len, max_seq_len, num_q_heads,
                          num_kv_heads, head_dim, pkv::kBlock, 1.f, dtype, split_tokens, &plan);
  if (st != PKV_OK) return st;
  // a work list exists for bf16 queries and a non-empty batch (as for
  // pkv_paged_attention_plan, which leaves the workspace alone otherwise)
  const bool listed = dtype == PKV_BF16 && num_tokens > 0 && num_reqs > 0;
  if (listed && !workspace_fits(plan, workspace, workspace_bytes)) return PKV_ERR_WORKSPACE;
#ifdef PKV_DEBUG_CHECKS
  // the checked build validates the prepare inputs, then the plan's inputs
  // on the device, so it runs the two calls one after the other
  st = pkv_prepare_inputs(num_scheduled_tokens, num_computed_tokens, block_table,
                          bt_row_stride, num_reqs, num_tokens, qsl_len, block_size, num_blocks,
                          req_indices, positions, slot_mapping, query_start_loc, seq_lens,
                          logits_indices, stream);
  if (st != PKV_OK || !listed) return st;
  return pkv_paged_attention_plan(query_start_loc, seq_lens, num_reqs, num_tokens,
                                  max_query_len, max_seq_len, num_q_heads, num_kv_heads,
                                  head_dim, dtype, split_tokens, workspace, workspace_bytes,
                                  stream);
#else
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!listed)
    return launch_status(pkv::launch_prepare(
        num_scheduled_tokens, num_computed_tokens, block_table, bt_row_stride, num_reqs,
        num_tokens, qsl_len, block_size, num_blocks, req_indices, positions, slot_mapping,
        query_start_loc, seq_lens, logits_indices, s));
  const pkv::PrepareArgs p = {num_scheduled_tokens, num_computed_tokens, block_table,
                              bt_row_stride,        num_reqs,            num_tokens,
                              qsl_len,              block_size,          num_blocks,
                              req_indices,          positions,           slot_mapping,
                              query_start_loc,      seq_lens,            logits_indices};
  const uint32_t fp = plan_fingerprint(plan, num_reqs, num_tokens, max_query_len, max_seq_len,
                                       num_q_heads, num_kv_heads, head_dim);
  return launch_status(pkv::launch_prepare_plan(p, plan, num_kv_heads, workspace, fp, s));
#endif
}

pkv_status pkv_paged_attention_run(
    const void* q, int64_t q_row_stride, const void* key_cache, const void* value_cache,
    int64_t num_blocks, void* out, int64_t out_row_stride, const int32_t* query_start_loc,
    const int32_t* seq_lens, const int32_t* block_table, int64_t bt_row_stride,
    int32_t num_reqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float scale, pkv_dtype dtype, const float* k_scale, const float* v_scale,
    int32_t split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if ((k_scale == nullptr) != (v_scale == nullptr)) return PKV_ERR_INVALID_ARG;
  if (k_scale != nullptr && dtype != PKV_BF16) return PKV_ERR_INVALID_ARG;
  return attention_call(AttnMode::kRun, q, q_row_stride, key_cache, value_cache, num_blocks,
                        out, out_row_stride, query_start_loc, seq_lens, block_table,
                        bt_row_stride, num_reqs, num_tokens, max_query_len, max_seq_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, scale, dtype, k_scale,
                        v_scale, split_tokens, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// pkv_paged_attention_varlen_noalloc: the workspace is a static device array
// ---------------------------------------------------------------------------

namespace {

// The attention workspace of the allocation-free entry point: one copy per
// device, held from module load until the process ends, shared by every call
// on that device.  In host code `scratch` names a host-side stand-in, not the
// device array: its device address comes from hipGetSymbolAddress.
__device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];  // per device, looked up once

// This device's address of `scratch` (the current device).  Concurrent first
// calls may each look it up; they store the same address.
pkv_status scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_LAUNCH;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PKV_ERR_LAUNCH;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *addr = p;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attention_varlen_noalloc(
    const void* q, int64_t q_row_stride, const void* key_cache, const void* value_cache,
    int64_t num_blocks, void* out, int64_t out_row_stride, const int32_t* query_start_loc,
    const int32_t* seq_lens, const int32_t* block_table, int64_t bt_row_stride,
    int32_t num_reqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float scale, pkv_dtype dtype, int32_t split_tokens, void* stream) {
  // the sizes first: a call the static array cannot hold is rejected before
  // anything touches the device
  const size_t need = pkv_paged_attention_workspace_bytes(
      num_reqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_query_len, max_seq_len,
      split_tokens, dtype);
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (need > 0 && num_tokens > 0 && num_reqs > 0) {
    const pkv_status st = scratch_address(&ws);
    if (st != PKV_OK) return st;
  }
  return attention_call(AttnMode::kFused, q, q_row_stride, key_cache, value_cache, num_blocks,
                        out, out_row_stride, query_start_loc, seq_lens, block_table,
                        bt_row_stride, num_reqs, num_tokens, max_query_len, max_seq_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, scale, dtype, nullptr,
                        nullptr, split_tokens, ws, ws ? (size_t)PKV_NOALLOC_SCRATCH_BYTES : 0,
                        stream);
}

}  // extern "C"
