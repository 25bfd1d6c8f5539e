// pkv_internal.h -- declarations shared by the libpkv HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// Attention path constants.
constexpr int kBlock = 16;          // tokens per KV block the attention kernels read
constexpr int kPairsPerTile = 16;   // MFMA N width: (query row, q head) pairs per tile
constexpr int kWaves = 4;           // waves per attention workgroup
constexpr int kPrefillTilesPerWave = 2;  // 16-pair tiles one wave owns in a prefill item
constexpr int kPrefillPairs = kWaves * kPrefillTilesPerWave * kPairsPerTile;  // 128
constexpr int kPlanReqs = 1024;      // threads of the plan kernel; requests it ranks at once
constexpr int kPlanMaxSplits = 2048; // partition counts the plan orders partition-major

// Host-side plan of one attention call (derived from host scalars only).
struct AttnPlan {
  int32_t group;          // q heads per kv head
  int32_t split_tokens;   // partition size of a decode context (multiple of 32)
  int32_t max_splits;     // partitions per decode context, upper bound
  int64_t max_items;      // upper bound on work items
  int64_t grid;           // workgroups of the main kernel: max_items + prompt helpers
  size_t items_offset;    // byte offsets inside the workspace
  size_t ml_offset;
  size_t o_offset;
  size_t total_bytes;
};

bool make_attn_plan(int32_t num_reqs, int32_t num_tokens, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                    int32_t max_seq_len, int32_t split_tokens, pkv_dtype dtype, AttnPlan* plan);

// One request's term of the batch checksum a work list records (summed mod
// 2^32 with qsl[0] * 374761393 over the requests).
__host__ __device__ inline uint32_t plan_batch_term(int32_t r, int32_t qsl_next, int32_t seq_len) {
  uint32_t t = (uint32_t)qsl_next * 2654435761u + (uint32_t)seq_len * 2246822519u +
               (uint32_t)r * 3266489917u;
  return t ^ (t >> 15);
}

// Device-data checks of the checked build (checks.hip; PKV_DEBUG_CHECKS).
uint32_t last_check_flags();
pkv_status check_prepare(const int32_t* nst, const int32_t* nct, const int32_t* block_table,
                         int64_t bt_stride, int32_t num_reqs, int32_t num_tokens,
                         int32_t block_size, int64_t num_blocks, hipStream_t stream);
pkv_status check_slots(const int64_t* slots, int32_t num_tokens, int64_t num_slots,
                       const float* k_scale, const float* v_scale, hipStream_t stream);
// block_table may be null (a plan call: nothing reads it).  With `plan`
// non-null (a run call), the work list's recorded fingerprint and batch
// checksum must match `fingerprint` and the batch.
pkv_status check_attention(const int32_t* qsl, const int32_t* seq_lens,
                           const int32_t* block_table, int64_t bt_stride, int32_t num_reqs,
                           int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
                           int64_t num_blocks, const float* k_scale, const float* v_scale,
                           const int32_t* plan, uint32_t fingerprint, hipStream_t stream);
pkv_status check_rows(const int32_t* req_indices, const int32_t* positions, int32_t num_tokens,
                      int32_t num_reqs, int64_t row_width, hipStream_t stream);
pkv_status check_block_list(const int32_t* ids, int32_t n, bool pairs, int64_t num_blocks,
                            hipStream_t stream);

hipError_t launch_prepare(const int32_t* nst, const int32_t* nct, const int32_t* block_table,
                          int64_t bt_stride, int32_t num_reqs, int32_t num_tokens,
                          int32_t qsl_len, int32_t block_size, int64_t num_blocks,
                          int32_t* req_indices, int32_t* positions, int64_t* slot_mapping,
                          int32_t* qsl, int32_t* seq_lens, int32_t* logits_indices,
                          hipStream_t stream);

// The arguments of pkv_prepare_inputs.
struct PrepareArgs {
  const int32_t* nst;
  const int32_t* nct;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t num_reqs;
  int32_t num_tokens;
  int32_t qsl_len;
  int32_t block_size;
  int64_t num_blocks;
  int32_t* req_indices;
  int32_t* positions;
  int64_t* slot_mapping;
  int32_t* qsl;
  int32_t* seq_lens;
  int32_t* logits_indices;
};

hipError_t launch_input_ids(const int32_t* token_table, int64_t row_width, int32_t num_reqs,
                            const int32_t* req_indices, const int32_t* positions,
                            int32_t num_tokens, const int32_t* seq_lens,
                            const int32_t* num_tokens_total, int64_t* token_indices,
                            int32_t* input_ids, uint8_t* discard, hipStream_t stream);

// Workgroups one copy / zero launch takes for `count` blocks (2 pools x chunks).
int64_t block_op_workgroups(int64_t block_bytes, int32_t count);

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, int64_t num_blocks,
                              int64_t block_bytes, const int32_t* pairs, int32_t num_pairs,
                              hipStream_t stream);

hipError_t launch_zero_blocks(void* key_cache, void* value_cache, int64_t num_blocks,
                              int64_t block_bytes, const int32_t* ids, int32_t num_ids,
                              hipStream_t stream);

hipError_t launch_kv_write(const void* key, const void* value, int64_t key_stride,
                           int64_t value_stride, void* key_cache, void* value_cache,
                           int64_t num_blocks, const int64_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t elem_bytes, hipStream_t stream);

hipError_t launch_kv_write_fp8(const void* key, const void* value, int64_t key_stride,
                               int64_t value_stride, void* key_cache, void* value_cache,
                               int64_t num_blocks, const int64_t* slot_mapping,
                               int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                               int32_t elem_bytes, const float* k_scale, const float* v_scale,
                               hipStream_t stream);

struct AttnArgs {
  const void* q;
  int64_t q_stride;
  const void* key_cache;
  const void* value_cache;
  int64_t num_blocks;
  void* out;
  int64_t out_stride;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t num_reqs;
  int32_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  float scale;
  const float* k_scale;  // FP8 pools: device scalars; null for 16-bit pools
  const float* v_scale;
};

// bf16 queries; kv8 selects FP8 E4M3 pools (a.k_scale / a.v_scale set).
// bf16 path: the work list (plan), then the main and reduce kernels over it
// (run); `fingerprint` identifies the sizes the list was made for.
hipError_t launch_attention_plan(const AttnArgs& a, const AttnPlan& plan, void* workspace,
                                 uint32_t fingerprint, hipStream_t stream);
hipError_t launch_attention_run(const AttnArgs& a, const AttnPlan& plan, void* workspace,
                                bool kv8, hipStream_t stream);
// prepare (p) and the bf16 work list (plan) of the same step in one launch;
// the list is read from the query_start_loc / seq_lens that p writes.
hipError_t launch_prepare_plan(const PrepareArgs& p, const AttnPlan& plan, int32_t num_kv_heads,
                               void* workspace, uint32_t fingerprint, hipStream_t stream);
hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t stream);

}  // namespace pkv
