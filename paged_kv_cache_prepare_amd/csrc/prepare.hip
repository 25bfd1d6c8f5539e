// prepare.hip -- flat-batch index tensors of one step, in one launch
// (prepare_rows.h: what is computed, and how the rows are shared out).
// Each 256-thread workgroup owns a range of 1024 flat rows; workgroup 0 also
// writes the per-request outputs.  Launch-latency bound.
#include "prepare_rows.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerGroup = 1024;

__global__ __launch_bounds__(kThreads) void prepare_kernel(
    const int32_t* __restrict__ nst, const int32_t* __restrict__ nct,
    const int32_t* __restrict__ block_table, int64_t bt_stride, int32_t num_reqs,
    int32_t num_tokens, int32_t qsl_len, int32_t block_size, int64_t num_blocks,
    int32_t* __restrict__ req_indices, int32_t* __restrict__ positions,
    int64_t* __restrict__ slot_mapping, int32_t* __restrict__ qsl,
    int32_t* __restrict__ seq_lens, int32_t* __restrict__ logits_indices) {
  const int64_t row_lo = (int64_t)blockIdx.x * kRowsPerGroup;
  const int64_t row_hi = min((int64_t)num_tokens, row_lo + kRowsPerGroup);
  prepare_rows<kThreads>(nst, nct, block_table, bt_stride, num_reqs, num_tokens, qsl_len,
                         block_size, num_blocks, req_indices, positions, slot_mapping, qsl,
                         seq_lens, logits_indices, row_lo, row_hi, blockIdx.x == 0);
}

}  // namespace

hipError_t launch_prepare(const int32_t* nst, const int32_t* nct, const int32_t* block_table,
                          int64_t bt_stride, int32_t num_reqs, int32_t num_tokens,
                          int32_t qsl_len, int32_t block_size, int64_t num_blocks,
                          int32_t* req_indices, int32_t* positions, int64_t* slot_mapping,
                          int32_t* qsl, int32_t* seq_lens, int32_t* logits_indices,
                          hipStream_t stream) {
  const int groups = max(1, (num_tokens + kRowsPerGroup - 1) / kRowsPerGroup);
  hipLaunchKernelGGL(prepare_kernel, dim3(groups), dim3(kThreads), 0, stream, nst, nct,
                     block_table, bt_stride, num_reqs, num_tokens, qsl_len, block_size,
                     num_blocks, req_indices, positions, slot_mapping, qsl, seq_lens,
                     logits_indices);
  return hipGetLastError();
}

}  // namespace pkv

// ---------------------------------------------------------------------------
// Input token ids and the discard mask.
//
// "Building the Batch" ("How they are computed") keeps every request's token
// list as one fixed-width row of a 2-D table, so the t-th new token of the
// request in row r sits at flat offset r * row_width + position; one gather
// then produces the step's input ids.  "vLLM's Model Runner -- the Persistent
// Batch, in Source" ("The batch contains rows that must not be sampled")
// marks a request whose sequence after this pass is still shorter than its
// known token count: its last row is sampled but the token is thrown away.
// One thread per flat row and per request; both read what prepare_kernel
// wrote, so this launch follows it on the same stream.
// ---------------------------------------------------------------------------
namespace pkv {
namespace {

__global__ __launch_bounds__(kThreads) void input_ids_kernel(
    const int32_t* __restrict__ token_table, int64_t row_width, int32_t num_reqs,
    const int32_t* __restrict__ req_indices, const int32_t* __restrict__ positions,
    int32_t num_tokens, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ num_tokens_total, int64_t* __restrict__ token_indices,
    int32_t* __restrict__ input_ids, uint8_t* __restrict__ discard) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < num_tokens) {
    const int32_t r = req_indices[i];
    const int32_t p = positions[i];
    int64_t k = -1;
    int32_t id = -1;
    if (r >= 0 && r < num_reqs && p >= 0 && p < row_width) {
      k = (int64_t)r * row_width + p;
      id = token_table[k];
    }
    if (token_indices != nullptr) token_indices[i] = k;
    input_ids[i] = id;
  }
  if (i < num_reqs) discard[i] = seq_lens[i] < num_tokens_total[i] ? 1 : 0;
}

}  // namespace

hipError_t launch_input_ids(const int32_t* token_table, int64_t row_width, int32_t num_reqs,
                            const int32_t* req_indices, const int32_t* positions,
                            int32_t num_tokens, const int32_t* seq_lens,
                            const int32_t* num_tokens_total, int64_t* token_indices,
                            int32_t* input_ids, uint8_t* discard, hipStream_t stream) {
  const int32_t n = max(num_tokens, num_reqs);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(input_ids_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, token_table, row_width, num_reqs, req_indices, positions,
                     num_tokens, seq_lens, num_tokens_total, token_indices, input_ids, discard);
  return hipGetLastError();
}

}  // namespace pkv
