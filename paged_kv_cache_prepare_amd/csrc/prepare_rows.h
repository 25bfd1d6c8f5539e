// prepare_rows.h -- the index derivation of one step as a device function,
// shared by the prepare kernel and the fused prepare + plan kernel.
//
// Computes what "Building the Batch" ("How they are computed", "Reading and
// writing the KV cache") and "vLLM's Model Runner -- the Persistent Batch, in
// Source" ("The two things this method returns") build on the host with
// NumPy: request boundaries (query_start_loc), per-token request index and
// absolute position, the cache slot of every new token, and the per-request
// sequence length and last row.  Integer work only.
//
// A workgroup of T threads owns the flat rows [row_lo, row_hi).  It walks the
// requests in chunks of T, scanning num_scheduled_tokens in LDS to get each
// request's first row, and maps each of its rows to a request by binary search
// over the chunk's row starts.  The `writer` workgroup also writes the
// per-request outputs and the padded tail of query_start_loc (it walks every
// chunk, whatever its rows).  No cross-workgroup communication.
#pragma once

#include "pkv_internal.h"

namespace pkv {

// Inclusive scan of one int per thread across a T-thread workgroup (T a
// multiple of 64, at most 1024).  `wave_tot` is LDS scratch of T / 64 ints;
// returns the scan value and the total.  The caller synchronises before
// wave_tot is written again.
template <int T>
__device__ inline int prep_block_scan(int v, int* wave_tot, int* total) {
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
  for (int w = 0; w < T / 64; ++w) {
    const int x = wave_tot[w];
    before += (w < wave) ? x : 0;
    sum += x;
  }
  *total = sum;
  return v + before;
}

template <int T>
__device__ inline void prepare_rows(
    const int32_t* __restrict__ nst, const int32_t* __restrict__ nct,
    const int32_t* __restrict__ block_table, int64_t bt_stride, int32_t num_reqs,
    int32_t num_tokens, int32_t qsl_len, int32_t block_size, int64_t num_blocks,
    int32_t* __restrict__ req_indices, int32_t* __restrict__ positions,
    int64_t* __restrict__ slot_mapping, int32_t* __restrict__ qsl,
    int32_t* __restrict__ seq_lens, int32_t* __restrict__ logits_indices, int64_t row_lo,
    int64_t row_hi, bool writer) {
  __shared__ int s_start[T];
  __shared__ int s_nct[T];
  __shared__ int s_wave[T / 64];

  const int tid = threadIdx.x;
  int carry = 0;  // rows owned by the requests before the current chunk
  for (int base = 0; base < num_reqs; base += T) {
    if (!writer && carry >= row_hi) break;  // carry is uniform across the workgroup
    const int r = base + tid;
    const int n = r < num_reqs ? nst[r] : 0;
    const int c = r < num_reqs ? nct[r] : 0;
    int total;
    const int incl = prep_block_scan<T>(n, s_wave, &total);
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

    const int in_chunk = min(T, num_reqs - base);
    const int64_t lo = max(row_lo, (int64_t)carry);
    const int64_t hi = min(row_hi, (int64_t)carry + total);
    for (int64_t i = lo + tid; i < hi; i += T) {
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
  for (int64_t i = max(row_lo, (int64_t)carry) + tid; i < row_hi; i += T) {
    req_indices[i] = -1;
    positions[i] = -1;
    slot_mapping[i] = -1;
  }
  if (writer) {
    if (num_reqs == 0 && tid == 0) qsl[0] = 0;
    for (int k = num_reqs + 1 + tid; k < qsl_len; k += T) qsl[k] = carry;
  }
}

}  // namespace pkv
