// checks.hip -- device-data precondition checks of the checked build
// (libpkv_checked.so, compiled with PKV_DEBUG_CHECKS).
//
// The regular library documents its preconditions on device data and never
// reads that data on the host; its kernels stay inside their buffers when a
// precondition is broken, but the results are then unspecified.  The checked
// build runs one validation kernel per entry point first, on the same stream,
// waits for it, and returns PKV_ERR_DEVICE_DATA without launching the real
// kernels when any check fails.  The failed checks are ORed into a device
// word as PKV_CHECK_* bits (include/pkv.h).  Every check reads only inside
// the buffers the entry point describes.
#include <atomic>

#include "pkv_internal.h"

namespace pkv {
namespace {

__device__ uint32_t g_check_flags;

__device__ inline void flag(uint32_t bits) { atomicOr(&g_check_flags, bits); }

__global__ void check_reset_kernel() { g_check_flags = 0u; }

// Scheduler counts and the block-table entries prepare reads: the columns of
// every new token's position.
__global__ __launch_bounds__(1024) void check_prepare_kernel(
    const int32_t* nst, const int32_t* nct, const int32_t* block_table, int64_t bt_stride,
    int32_t num_reqs, int32_t num_tokens, int32_t block_size, int64_t num_blocks) {
  __shared__ unsigned long long total;
  if (threadIdx.x == 0) total = 0ull;
  __syncthreads();
  unsigned long long mine = 0ull;
  for (int r = threadIdx.x; r < num_reqs; r += blockDim.x) {
    const int n = nst[r], c = nct[r];
    if (n < 0 || c < 0) {
      flag(PKV_CHECK_COUNTS);
      continue;
    }
    mine += (unsigned long long)n;
    if (n == 0) continue;
    const int64_t first = c / block_size;
    const int64_t last = ((int64_t)c + n - 1) / block_size;
    for (int64_t j = first; j <= last; ++j) {
      if (j >= bt_stride) {
        flag(PKV_CHECK_BLOCK_ID);
        break;
      }
      const int32_t id = block_table[(int64_t)r * bt_stride + j];
      if (id < 0 || id >= num_blocks) flag(PKV_CHECK_BLOCK_ID);
    }
  }
  atomicAdd(&total, mine);
  __syncthreads();
  if (threadIdx.x == 0 && total != (unsigned long long)num_tokens) flag(PKV_CHECK_COUNTS);
}

// FP8 scales: finite and positive.
__device__ inline void check_scales(const float* k_scale, const float* v_scale) {
  const float ks = *k_scale, vs = *v_scale;
  if (!(ks > 0.f) || !(vs > 0.f) || isinf(ks) || isinf(vs)) flag(PKV_CHECK_SCALE);
}

// Slots in [-1, num_blocks * block_size), and no slot >= 0 twice (pairwise,
// for calls of at most kDupCheckRows rows); the FP8 scales when given.
__global__ __launch_bounds__(256) void check_slots_kernel(const int64_t* slots, int32_t num_tokens,
                                                          int64_t num_slots, bool dups,
                                                          const float* k_scale,
                                                          const float* v_scale) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0 && k_scale != nullptr) check_scales(k_scale, v_scale);
  if (i >= num_tokens) return;
  const int64_t s = slots[i];
  if (s < -1 || s >= num_slots) flag(PKV_CHECK_SLOT);
  if (!dups || s < 0) return;
  for (int64_t j = i + 1; j < num_tokens; ++j)
    if (slots[j] == s) {
      flag(PKV_CHECK_SLOT_DUP);
      return;
    }
}

// query_start_loc, the lengths, and every block-table entry a request's
// context reads (columns below ceil(seq_len / 16)).  One workgroup per request.
// A run call (plan != null) also compares the work list's recorded sizes and
// batch checksum with this call's (workgroup 0, serially).
__global__ __launch_bounds__(256) void check_attention_kernel(
    const int32_t* qsl, const int32_t* seq_lens, const int32_t* block_table, int64_t bt_stride,
    int32_t num_reqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
    int64_t num_blocks, const float* k_scale, const float* v_scale, const int32_t* plan,
    uint32_t fingerprint) {
  const int r = blockIdx.x;
  if (r == 0 && threadIdx.x == 0 && plan != nullptr) {
    uint32_t sum = (uint32_t)qsl[0] * 374761393u;
    for (int k = 0; k < num_reqs; ++k) sum += plan_batch_term(k, qsl[k + 1], seq_lens[k]);
    if ((uint32_t)plan[1] != fingerprint || (uint32_t)plan[2] != sum) flag(PKV_CHECK_PLAN);
  }
  const int q0 = qsl[r], q1 = qsl[r + 1];
  const int L = seq_lens[r];
  if (threadIdx.x == 0) {
    if (q0 < 0 || q1 < q0 || q1 > num_tokens) flag(PKV_CHECK_QSL);
    const int q_len = q1 - q0;
    if (L < 0 || (q_len > 0 && q_len > L) || L > max_seq_len || q_len > max_query_len)
      flag(PKV_CHECK_LENGTHS);
    if (r == 0 && k_scale != nullptr) check_scales(k_scale, v_scale);
  }
  if (q1 <= q0 || L <= 0 || block_table == nullptr) return;  // nothing to read
  const int64_t cols = ((int64_t)L + kBlock - 1) / kBlock;
  if (cols > bt_stride && threadIdx.x == 0) flag(PKV_CHECK_BLOCK_ID);
  const int64_t lim = cols < bt_stride ? cols : bt_stride;
  for (int64_t j = threadIdx.x; j < lim; j += blockDim.x) {
    const int32_t id = block_table[(int64_t)r * bt_stride + j];
    if (id < 0 || id >= num_blocks) flag(PKV_CHECK_BLOCK_ID);
  }
}

// Rows of the input-id gather: padding rows (-1, -1) or a request of the
// step and a position inside the token table.
__global__ __launch_bounds__(256) void check_rows_kernel(const int32_t* req_indices,
                                                         const int32_t* positions,
                                                         int32_t num_tokens, int32_t num_reqs,
                                                         int64_t row_width) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= num_tokens) return;
  const int32_t r = req_indices[i], p = positions[i];
  if (r == -1 && p == -1) return;
  if (r < 0 || r >= num_reqs || p < 0 || p >= row_width) flag(PKV_CHECK_ROW);
}

// Block ids of copy pairs (stride 2) or of a clear list (stride 1); for
// copies, destinations distinct and never a source (pairwise, at most
// kDupCheckRows pairs).
__global__ __launch_bounds__(256) void check_block_list_kernel(const int32_t* ids, int32_t n,
                                                               int32_t stride, int64_t num_blocks,
                                                               bool pairs_check) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  for (int c = 0; c < stride; ++c) {
    const int32_t id = ids[k * stride + c];
    if (id < 0 || id >= num_blocks) flag(PKV_CHECK_BLOCK_ID);
  }
  if (!pairs_check) return;
  const int32_t dst = ids[2 * k + 1];
  for (int64_t m = 0; m < n; ++m) {
    if ((m != k && ids[2 * m + 1] == dst) || ids[2 * m] == dst) {
      flag(PKV_CHECK_PAIRS);
      return;
    }
  }
}

constexpr int32_t kDupCheckRows = 1 << 16;

std::atomic<uint32_t> g_last_flags{0u};  // host copy of the last failure

// Reset the word, run `launch`, wait for the stream, report.
template <typename F>
pkv_status run_check(hipStream_t stream, F launch) {
  hipLaunchKernelGGL(check_reset_kernel, dim3(1), dim3(1), 0, stream);
  if (hipGetLastError() != hipSuccess) return PKV_ERR_LAUNCH;
  launch();
  if (hipGetLastError() != hipSuccess) return PKV_ERR_LAUNCH;
  uint32_t flags = 0u;
  if (hipMemcpyFromSymbolAsync(&flags, HIP_SYMBOL(g_check_flags), sizeof(flags), 0,
                               hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return PKV_ERR_LAUNCH;
  if (flags != 0u) {
    g_last_flags.store(flags, std::memory_order_relaxed);
    return PKV_ERR_DEVICE_DATA;
  }
  return PKV_OK;
}

unsigned grid_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

uint32_t last_check_flags() { return g_last_flags.load(std::memory_order_relaxed); }

pkv_status check_prepare(const int32_t* nst, const int32_t* nct, const int32_t* block_table,
                         int64_t bt_stride, int32_t num_reqs, int32_t num_tokens,
                         int32_t block_size, int64_t num_blocks, hipStream_t stream) {
  if (num_reqs == 0) return num_tokens == 0 ? PKV_OK : PKV_ERR_INVALID_ARG;
  return run_check(stream, [&] {
    hipLaunchKernelGGL(check_prepare_kernel, dim3(1), dim3(1024), 0, stream, nst, nct,
                       block_table, bt_stride, num_reqs, num_tokens, block_size, num_blocks);
  });
}

pkv_status check_slots(const int64_t* slots, int32_t num_tokens, int64_t num_slots,
                       const float* k_scale, const float* v_scale, hipStream_t stream) {
  if (num_tokens == 0) return PKV_OK;
  return run_check(stream, [&] {
    hipLaunchKernelGGL(check_slots_kernel, dim3(grid_for(num_tokens)), dim3(256), 0, stream,
                       slots, num_tokens, num_slots, num_tokens <= kDupCheckRows, k_scale,
                       v_scale);
  });
}

pkv_status check_attention(const int32_t* qsl, const int32_t* seq_lens,
                           const int32_t* block_table, int64_t bt_stride, int32_t num_reqs,
                           int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
                           int64_t num_blocks, const float* k_scale, const float* v_scale,
                           const int32_t* plan, uint32_t fingerprint, hipStream_t stream) {
  if (num_reqs == 0) return PKV_OK;
  return run_check(stream, [&] {
    hipLaunchKernelGGL(check_attention_kernel, dim3((unsigned)num_reqs), dim3(256), 0, stream,
                       qsl, seq_lens, block_table, bt_stride, num_reqs, num_tokens,
                       max_query_len, max_seq_len, num_blocks, k_scale, v_scale, plan,
                       fingerprint);
  });
}

pkv_status check_rows(const int32_t* req_indices, const int32_t* positions, int32_t num_tokens,
                      int32_t num_reqs, int64_t row_width, hipStream_t stream) {
  if (num_tokens == 0) return PKV_OK;
  return run_check(stream, [&] {
    hipLaunchKernelGGL(check_rows_kernel, dim3(grid_for(num_tokens)), dim3(256), 0, stream,
                       req_indices, positions, num_tokens, num_reqs, row_width);
  });
}

pkv_status check_block_list(const int32_t* ids, int32_t n, bool pairs, int64_t num_blocks,
                            hipStream_t stream) {
  if (n == 0) return PKV_OK;
  return run_check(stream, [&] {
    hipLaunchKernelGGL(check_block_list_kernel, dim3(grid_for(n)), dim3(256), 0, stream, ids, n,
                       pairs ? 2 : 1, num_blocks, pairs && n <= kDupCheckRows);
  });
}

}  // namespace pkv
