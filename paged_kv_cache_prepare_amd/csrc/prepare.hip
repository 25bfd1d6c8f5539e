// prepare.hip -- flat-batch index tensors of one step, in one launch.
//
// Computes what "Building the Batch" ("How they are computed", "Reading and
// writing the KV cache") and "vLLM's Model Runner -- the Persistent Batch, in
// Source" ("The two things this method returns") build on the host with
// NumPy: request boundaries (query_start_loc), per-token request index and
// absolute position, the cache slot of every new token, and the per-request
// sequence length and last row.  Integer work only; launch-latency bound.
//
// Each workgroup owns a range of 1024 flat rows.  It walks the requests in
// chunks of 256, scanning num_scheduled_tokens in LDS to get each request's
// first row, and maps each of its rows to a request by binary search over
// the chunk's row starts.  Workgroup 0 also writes the per-request outputs
// and the padded tail of query_start_loc.  No cross-workgroup communication.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerGroup = 1024;

// Inclusive scan of one int per thread across a 256-thread workgroup.
// `wave_tot` is LDS scratch of 4 ints; returns the scan value and the total.
__device__ inline int block_scan_256(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int up = __shfl_up(v, off, 64);
    if (lane >= off) v += up;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  int before = 0;
  int sum = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int x = wave_tot[w];
    before += (w < wave) ? x : 0;
    sum += x;
  }
  *total = sum;
  return v + before;
}

__global__ __launch_bounds__(kThreads) void prepare_kernel(
    const int32_t* __restrict__ nst, const int32_t* __restrict__ nct,
    const int32_t* __restrict__ block_table, int64_t bt_stride, int32_t num_reqs,
    int32_t num_tokens, int32_t qsl_len, int32_t block_size, int64_t num_blocks,
    int32_t* __restrict__ req_indices, int32_t* __restrict__ positions,
    int64_t* __restrict__ slot_mapping, int32_t* __restrict__ qsl,
    int32_t* __restrict__ seq_lens, int32_t* __restrict__ logits_indices) {
  __shared__ int s_start[kThreads];
  __shared__ int s_nct[kThreads];
  __shared__ int s_wave[4];

  const int tid = threadIdx.x;
  const bool writer = blockIdx.x == 0;
  const int64_t row_lo = (int64_t)blockIdx.x * kRowsPerGroup;
  const int64_t row_hi = min((int64_t)num_tokens, row_lo + kRowsPerGroup);

  int carry = 0;  // rows owned by the requests before the current chunk
  for (int base = 0; base < num_reqs; base += kThreads) {
    if (!writer && carry >= row_hi) break;  // carry is uniform across the workgroup
    const int r = base + tid;
    const int n = r < num_reqs ? nst[r] : 0;
    const int c = r < num_reqs ? nct[r] : 0;
    int total;
    const int incl = block_scan_256(n, s_wave, &total);
    const int start = carry + incl - n;
    if (writer && r < num_reqs) {
      if (r == 0) qsl[0] = 0;
      qsl[r + 1] = carry + incl;
      seq_lens[r] = c + n;
      logits_indices[r] = carry + incl - 1;
    }
    s_start[tid] = start;
    s_nct[tid] = c;
    __syncthreads();

    const int in_chunk = min(kThreads, num_reqs - base);
    const int64_t lo = max(row_lo, (int64_t)carry);
    const int64_t hi = min(row_hi, (int64_t)carry + total);
    for (int64_t i = lo + tid; i < hi; i += kThreads) {
      // last request in the chunk whose first row is <= i; a request with no
      // rows shares its start with the next one, so it is never selected
      int a = 0, b = in_chunk - 1;
      while (a < b) {
        const int mid = (a + b + 1) >> 1;
        if (s_start[mid] <= i) a = mid; else b = mid - 1;
      }
      const int req = base + a;
      const int pos = s_nct[a] + (int)(i - s_start[a]);
      const int logical = pos / block_size;
      int64_t slot = -1;
      if (pos >= 0 && logical < bt_stride) {
        const int32_t phys = block_table[(int64_t)req * bt_stride + logical];
        if (phys >= 0 && phys < num_blocks)
          slot = (int64_t)phys * block_size + (pos - logical * block_size);
      }
      req_indices[i] = req;
      positions[i] = pos;
      slot_mapping[i] = slot;
    }
    carry += total;
    __syncthreads();  // s_start / s_wave are rewritten by the next chunk
  }

  // Rows past the device-side token total (host and device totals disagree).
  for (int64_t i = max(row_lo, (int64_t)carry) + tid; i < row_hi; i += kThreads) {
    req_indices[i] = -1;
    positions[i] = -1;
    slot_mapping[i] = -1;
  }
  if (writer) {
    if (num_reqs == 0 && tid == 0) qsl[0] = 0;
    for (int k = num_reqs + 1 + tid; k < qsl_len; k += kThreads) qsl[k] = carry;
  }
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
