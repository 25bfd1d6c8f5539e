// attention.hip -- paged, variable-length causal attention for gfx950.
//
// What is computed ("How vLLM Works Internally: A Deep Dive", "How the Kernel
// Works"): for every query row, look up its request's block table, fetch K
// from scattered physical blocks, score, softmax, and sum V with those
// weights.  A query at in-chunk offset t of a request with q_len new tokens
// and seq_len total tokens is at position seq_len - q_len + t and sees keys
// 0..that position.  Long decode contexts are split into partitions whose
// partial softmax results a second pass combines ("PagedAttention V2").
//
// bf16 path (three launches per call, all on the caller's stream):
//  1. plan:   one workgroup turns query_start_loc / seq_lens into a work list
//             in the workspace: prefill tiles first, then decode partitions,
//             longest contexts first.  Host code never reads device data, so
//             the list is built on the device.
//  2. main:   workgroups of 4 waves; prompt-chunk tiles and single-token
//             decodes of the same step run in this one launch (prefill
//             tiles on resident workgroups, one workgroup per decode item).
//             * decode item = (request, kv head, partition): the q heads of
//               the kv head (and, for short multi-token queries, their rows)
//               form the 16-wide N side of v_mfma_f32_16x16x32_bf16; the 4
//               waves split the partition's 32-token steps and merge their
//               (max, sum, acc) states through LDS at the end.
//             * prefill item = (request, kv head, 128 (row, head) pairs): each
//               wave owns 32 pairs (2 MFMA N tiles); the workgroup stages each
//               64-token K/V step in LDS once for all four waves.
//             Both walk the context two 16-token blocks at a time: K rows are
//             the MFMA A operand (16 tokens x 32 dims per load); S^T = K Q^T
//             lands with 4 tokens of one column per lane, which is exactly
//             the B-operand layout of P^T in O^T = V^T P^T, so the softmax
//             probabilities feed the second MFMA without leaving registers.
//             V runs are tiles of 16 dims x 4 tokens, so a lane's V^T
//             operand (4 tokens of one dim) is one contiguous 8-byte run.  Online softmax: running max by
//             two cross-lane shuffles, per-lane partial sums reduced once.
//  3. reduce: combines partition partials of split decode items.
// fp32 path: one wave per (row, q head), fp32 vector math, no partitions.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "pkv_internal.h"
#include "prepare_rows.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPrefillItemsWord = 4;  // workspace header word: prefill items at the list head
constexpr int kClaimWord = 32;        // workspace header words: prompt-tile tickets per XCD, finishers
constexpr int kXcds = 8;              // XCDs: workgroup b runs on XCD b % 8

// Compute units of the current device, cached per device id.  Concurrent
// first calls from several host threads may each query the device; they
// store the same value, and the atomics make that race benign.
int device_cu_count() {
  static std::atomic<int> cached[64];  // static storage: zero-initialised
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}
constexpr int kThreads = kWaves * 64;

__device__ inline bf16x8 ld_b128(const char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ inline f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline unsigned short bf16_bits(float x) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(x));
}

// Keep element k of a 4 x bf16 run iff bit k of `keep` is set.
__device__ inline u32x2 keep_bf16x4(u32x2 v, unsigned keep) {
  v.x &= ((keep & 1u) ? 0x0000FFFFu : 0u) | ((keep & 2u) ? 0xFFFF0000u : 0u);
  v.y &= ((keep & 4u) ? 0x0000FFFFu : 0u) | ((keep & 8u) ? 0xFFFF0000u : 0u);
  return v;
}

__device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Max / sum over the four lanes n, n + 16, n + 32, n + 48 that hold one MFMA
// column.  The row-swap permutes exchange 16-lane rows and 32-lane halves
// between two copies of x; combining both copies gives every lane the
// partner's value without an LDS round trip.  (The two results are copied
// to scalars before any bit cast: bit-casting a subscript of the builtin's
// result directly has been seen to read element 0 for both.)
__device__ inline void swap_rows16(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}

__device__ inline void swap_halves32(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}

__device__ inline float column_max(float x) {
  float a, b;
  swap_rows16(x, a, b);
  swap_halves32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}

__device__ inline float column_sum(float x) {
  float a, b;
  swap_rows16(x, a, b);
  swap_halves32(a + b, a, b);
  return a + b;
}

// The block table is read-only for the whole call.  Reading it through the
// constant address space lets wave-uniform lookups compile to scalar loads
// (counted by lgkmcnt), so they never wait behind in-flight K/V vector loads,
// also after a workgroup barrier.
typedef const __attribute__((address_space(4))) int32_t table_t;

__device__ inline table_t* table_row(const int32_t* block_table, int64_t row_stride, int r) {
  return (table_t*)(block_table + (int64_t)r * row_stride);
}

// Rows of request r, or 0 when its query_start_loc range leaves [0, num_tokens)
// (a broken precondition): such a request gets no work, so no kernel touches
// rows outside q / out.
__device__ inline int valid_q_len(const int32_t* qsl, int r, int num_tokens) {
  const int q0 = qsl[r], q1 = qsl[r + 1];
  return (q0 >= 0 && q1 <= num_tokens && q1 >= q0) ? q1 - q0 : 0;
}

// Partitions of one decode context; identical in plan, main and reduce.
__device__ inline int num_splits(int seq_len, int split_tokens, int max_splits) {
  return min(max_splits, max(1, ceil_div(max(seq_len, 1), split_tokens)));
}

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

__device__ inline int block_scan_1024(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int up = __shfl_up(v, off, 64);
    if (lane >= off) v += up;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int x = wave_tot[w];
    before += (w < wave) ? x : 0;
    sum += x;
  }
  __syncthreads();
  *total = sum;
  return v + before;
}

// First index in the non-decreasing s[0..n) whose value exceeds x (n if none).
__device__ inline int upper_bound_lds(const int* s, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s[mid] > x) hi = mid; else lo = mid + 1;
  }
  return lo;
}

struct PlanSmem {
  int wave[16];
  int len[kPlanReqs];    // seq_len by request (ordered path)
  int qlen[kPlanReqs];   // valid query rows by request (ordered path)
  int req[kPlanReqs];    // request at rank j (ordered path) / unused (chunked path)
  int incl[kPlanReqs];   // inclusive prefix of per-slot unit counts
  int aux[kPlanReqs];    // per-slot split count or tile count
  int dreq[kPlanReqs];   // decode requests by split count, largest first
  int dns[kPlanReqs];    // their split counts (non-increasing)
  int gt[kPlanMaxSplits + 1];  // decode requests with more than k splits
  int pk[kPlanMaxSplits + 1];  // decode units before split index k
};

// Work units of one request in a pass: prefill tiles (pass 0) or decode
// partitions (pass 1), from its valid query rows and seq_len.  *aux gets the
// tile count or the split count.
__device__ inline int plan_units_of(int q_len, int seq_len, int group, int split_tokens,
                                    int max_splits, int pass, int* aux) {
  const int pairs = q_len * group;
  int cnt = 0;
  if (pass == 0 && pairs > kPairsPerTile) cnt = ceil_div(pairs, kPrefillPairs);
  if (pass == 1 && pairs >= 1 && pairs <= kPairsPerTile)
    cnt = num_splits(seq_len, split_tokens, max_splits);
  *aux = cnt;
  return cnt;
}

__device__ inline int plan_units(const int32_t* qsl, const int32_t* seq_lens, int r,
                                 int num_tokens, int group, int split_tokens, int max_splits,
                                 int pass, int* aux) {
  const int pairs = valid_q_len(qsl, r, num_tokens) * group;
  int cnt = 0;
  if (pass == 0 && pairs > kPairsPerTile) cnt = ceil_div(pairs, kPrefillPairs);
  if (pass == 1 && pairs >= 1 && pairs <= kPairsPerTile)
    cnt = num_splits(seq_lens[r], split_tokens, max_splits);
  *aux = cnt;
  return cnt;
}

// The work list.  Item = (request, kv head, index, split count): index is the
// row tile of a prefill item (split count -1) or the partition of a decode
// item.  Items of one unit (a tile or a partition) are consecutive, one per kv
// head.  Prefill units come first, then decode units.
//
// Ordered path (num_reqs <= kPlanReqs and max_splits <= kPlanMaxSplits):
// requests are ranked by seq_len (to 1/1024 of the longest), longest first, so
// the longest work starts first and the tail of the launch holds the short
// items.  Prefill tiles of a
// request go latest rows first (they see the most keys).  Decode units go
// partition-major: partition 0 of every request, then partition 1, ...; the
// later partitions of a context are its shorter remainders, and requests that
// share prefix blocks read those blocks at about the same time.
// Chunked path (larger batches): request order, 1024 requests per scan.
// The list is built by one 1024-thread workgroup: the plan kernel, or
// workgroup 0 of the fused prepare + plan kernel once it has written
// query_start_loc and seq_lens.
__device__ __attribute__((always_inline)) inline void plan_body(
    const int32_t* qsl, const int32_t* seq_lens, int32_t num_reqs,
    int32_t num_tokens, int32_t num_kv_heads, int32_t group, int32_t split_tokens, int32_t max_splits,
    int64_t max_items, int4* __restrict__ items, int32_t* __restrict__ n_items,
    uint32_t fingerprint) {
  __shared__ PlanSmem sm;
  __shared__ uint32_t batch_sum;
  __shared__ int max_len;
  const int tid = threadIdx.x;
  const int H = num_kv_heads;
  int64_t carry = 0;  // units emitted so far; item index = unit * H + kv head
  int64_t pre_units = 0;  // prefill units (they head the list)
  // a checksum of the batch the list is made for (plan_batch_term), word 2
  if (tid == 0) {
    batch_sum = 0u;
    max_len = 0;
  }
  __syncthreads();
  const bool ordered = num_reqs <= kPlanReqs && max_splits <= kPlanMaxSplits;

  if (ordered) {
    // every per-request input is read once, up front, in one round trip
    const bool mine = tid < num_reqs;
    const int L = mine ? seq_lens[tid] : 0;
    const int QL = mine ? valid_q_len(qsl, tid, num_tokens) : 0;
    uint32_t part = (mine ? plan_batch_term(tid, qsl[tid + 1], L) : 0u) +
                    (tid == 0 ? (uint32_t)qsl[0] * 374761393u : 0u);
    int lmax = max(L, 0);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      part += __shfl_xor(part, off, 64);
      lmax = max(lmax, __shfl_xor(lmax, off, 64));
    }
    if ((tid & 63) == 0) {
      atomicAdd(&batch_sum, part);
      atomicMax(&max_len, lmax);
    }
    if (mine) {
      sm.len[tid] = L;
      sm.qlen[tid] = QL;
    }
    int* hist = sm.incl;   // requests per length bucket (the scans below reuse it)
    int* cursor = sm.aux;  // next free rank of each bucket
    hist[tid] = 0;
    __syncthreads();
    // Rank by seq_len, longest first, as a bucket sort over 1024 buckets of
    // the length range.  The order within a bucket follows the atomics and
    // may vary between calls: it only places prompt tiles, whose emission
    // below takes any order, and decode requests are sorted again by their
    // exact split count before pass 1 relies on an order.  No result depends
    // on the list's order (every item writes its own rows or partition).
    const int top = max(max_len, 1);
    const int bucket = mine ? (int)((int64_t)(top - min(max(L, 0), top)) * (kPlanReqs - 1) / top)
                            : 0;
    if (mine) atomicAdd(&hist[bucket], 1);
    __syncthreads();
    {
      const int h = hist[tid];
      int tot;
      const int incl = block_scan_1024(h, sm.wave, &tot);
      cursor[tid] = incl - h;
    }
    __syncthreads();
    if (mine) sm.req[atomicAdd(&cursor[bucket], 1)] = tid;
    __syncthreads();
    // pass 0: prefill tiles, in rank order
    {
      int tiles = 0;
      if (tid < num_reqs) {
        const int rq = sm.req[tid];
        plan_units_of(sm.qlen[rq], sm.len[rq], group, split_tokens, max_splits, 0, &tiles);
      }
      int total;
      const int incl = block_scan_1024(tiles, sm.wave, &total);
      sm.incl[tid] = incl;
      sm.aux[tid] = tiles;
      __syncthreads();
      const int n = (int)min((int64_t)total * H, max_items);
      for (int e = tid; e < n; e += kPlanReqs) {
        const int u = e / H, h = e - u * H;
        const int j = upper_bound_lds(sm.incl, num_reqs, u);
        const int k = u - (sm.incl[j] - sm.aux[j]);
        items[e] = make_int4(sm.req[j], h, sm.aux[j] - 1 - k, -1);
      }
      carry = total;
      pre_units = total;
    }
    // pass 1: decode partitions, partition-major.  The decode requests are
    // put in order of their split count, largest first, by a counting sort
    // over the counts 1..max_splits (equal counts keep no particular order).
    // Then the requests that have a partition k are exactly the first gt[k]
    // of them, gt[k] = #{decode requests with more than k splits}, and the
    // units of partition index k are pk[k] .. pk[k+1]-1 with pk the prefix
    // sum of gt.
    {
      int ns = 0, rq = -1;
      if (tid < num_reqs) {
        rq = sm.req[tid];
        plan_units_of(sm.qlen[rq], sm.len[rq], group, split_tokens, max_splits, 1, &ns);
      }
      for (int v = tid; v <= max_splits; v += kPlanReqs) sm.gt[v] = 0;
      __syncthreads();
      if (ns > 0) atomicAdd(&sm.gt[ns], 1);  // histogram of the split counts
      __syncthreads();
      // suffix sums of the histogram: slot i of the scan holds count
      // max_splits - i, two slots per thread (max_splits <= 2 * kPlanReqs)
      {
        const int i0 = 2 * tid, i1 = i0 + 1;
        const int h0 = i0 < max_splits ? sm.gt[max_splits - i0] : 0;
        const int h1 = i1 < max_splits ? sm.gt[max_splits - i1] : 0;
        int tot;
        const int excl = block_scan_1024(h0 + h1, sm.wave, &tot) - h0 - h1;
        __syncthreads();  // every histogram read is done
        if (i0 < max_splits) sm.gt[max_splits - i0] = excl;
        if (i1 < max_splits) sm.gt[max_splits - i1] = excl + h0;
        if (tid == 0) sm.gt[0] = tot;
      }
      __syncthreads();
      int pcarry;
      {
        const int k0 = 2 * tid, k1 = k0 + 1;
        const int g0 = k0 < max_splits ? sm.gt[k0] : 0;
        const int g1 = k1 < max_splits ? sm.gt[k1] : 0;
        const int excl = block_scan_1024(g0 + g1, sm.wave, &pcarry) - g0 - g1;
        if (k0 < max_splits) sm.pk[k0] = excl;
        if (k1 < max_splits) sm.pk[k1] = excl + g0;
        if (tid == 0) sm.pk[max_splits] = pcarry;
      }
      __syncthreads();  // every gt read is done before the cursors move
      // place: the requests with count v take ranks gt[v] .. gt[v-1]-1
      if (ns > 0) {
        const int pos = atomicAdd(&sm.gt[ns], 1);
        sm.dreq[pos] = rq;
        sm.dns[pos] = ns;
      }
      __syncthreads();
      const int base = (int)min(carry * H, max_items);
      const int n = (int)min((int64_t)pcarry * H, max_items - base);
      for (int e = tid; e < n; e += kPlanReqs) {
        const int idx = base + e;
        const int u = e / H, h = e - u * H;
        const int k = upper_bound_lds(sm.pk, max_splits + 1, u) - 1;
        const int j = u - sm.pk[k];
        items[idx] = make_int4(sm.dreq[j], h, k, sm.dns[j]);
      }
      carry += pcarry;
    }
  } else {
    {
      uint32_t part = tid == 0 ? (uint32_t)qsl[0] * 374761393u : 0u;
      for (int r = tid; r < num_reqs; r += kPlanReqs)
        part += plan_batch_term(r, qsl[r + 1], seq_lens[r]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
      if ((tid & 63) == 0) atomicAdd(&batch_sum, part);
    }
    for (int pass = 0; pass < 2; ++pass) {
      if (pass == 1) pre_units = carry;
      for (int rb = 0; rb < num_reqs; rb += kPlanReqs) {
        const int r = rb + tid;
        int cnt = 0, aux = 0;
        if (r < num_reqs)
          cnt = plan_units(qsl, seq_lens, r, num_tokens, group, split_tokens, max_splits, pass,
                           &aux);
        int total;
        const int incl = block_scan_1024(cnt, sm.wave, &total);
        sm.incl[tid] = incl;
        sm.aux[tid] = aux;
        __syncthreads();
        const int nslot = min(kPlanReqs, num_reqs - rb);
        const int64_t base = carry * H;
        const int64_t n = (int64_t)total * H;
        for (int64_t e = tid; e < n; e += kPlanReqs) {
          const int64_t idx = base + e;
          if (idx >= max_items) break;
          const int u = (int)(e / H), h = (int)(e - (int64_t)u * H);
          const int j = upper_bound_lds(sm.incl, nslot, u);
          const int k = u - (sm.incl[j] - sm.aux[j]);
          items[idx] = pass == 0 ? make_int4(rb + j, h, sm.aux[j] - 1 - k, -1)
                                 : make_int4(rb + j, h, k, sm.aux[j]);
        }
        carry += total;
        __syncthreads();  // incl / aux are rewritten by the next chunk
      }
    }
  }
  if (tid == 0) {
    const int64_t n = carry * H;
    *n_items = (int32_t)(n < max_items ? n : max_items);
    // the sizes and the batch the list was made for, so that a checked run
    // can tell
    n_items[1] = (int32_t)fingerprint;
    n_items[2] = (int32_t)batch_sum;
    const int64_t np = pre_units * H;
    n_items[kPrefillItemsWord] = (int32_t)(np < max_items ? np : max_items);
#pragma unroll
    for (int x = 0; x <= kXcds; ++x) n_items[kClaimWord + x] = 0;
  }
}

__global__ __launch_bounds__(kPlanReqs) void attn_plan_kernel(
    const int32_t* __restrict__ qsl, const int32_t* __restrict__ seq_lens, int32_t num_reqs,
    int32_t num_tokens, int32_t num_kv_heads, int32_t group, int32_t split_tokens, int32_t max_splits,
    int64_t max_items, int4* __restrict__ items, int32_t* __restrict__ n_items,
    uint32_t fingerprint) {
  plan_body(qsl, seq_lens, num_reqs, num_tokens, num_kv_heads, group, split_tokens, max_splits,
            max_items, items, n_items, fingerprint);
}

// The step's index tensors and its attention work list in one launch (the
// two are computed by the same step, and a launch boundary between them
// costs more than either): workgroup 0 writes the per-request outputs
// (query_start_loc, seq_lens, logits_indices, the padded tail), then builds
// the work list from them; workgroups 1, 2, ... map 1024 flat rows each.
// The per-request outputs are read back by the workgroup that wrote them,
// after a barrier.
__global__ __launch_bounds__(kPlanReqs) void prepare_plan_kernel(
    const int32_t* __restrict__ nst, const int32_t* __restrict__ nct,
    const int32_t* __restrict__ block_table, int64_t bt_stride, int32_t num_reqs,
    int32_t num_tokens, int32_t qsl_len, int32_t block_size, int64_t num_blocks,
    int32_t* __restrict__ req_indices, int32_t* __restrict__ positions,
    int64_t* __restrict__ slot_mapping, int32_t* qsl, int32_t* seq_lens,
    int32_t* __restrict__ logits_indices, int32_t num_kv_heads, int32_t group,
    int32_t split_tokens, int32_t max_splits, int64_t max_items, int4* __restrict__ items,
    int32_t* __restrict__ n_items, uint32_t fingerprint) {
  if (blockIdx.x == 0) {
    prepare_rows<kPlanReqs>(nst, nct, block_table, bt_stride, num_reqs, num_tokens, qsl_len,
                            block_size, num_blocks, req_indices, positions, slot_mapping, qsl,
                            seq_lens, logits_indices, 0, 0, true);
    __syncthreads();
    if (num_tokens > 0 && num_reqs > 0 && items != nullptr)
      plan_body(qsl, seq_lens, num_reqs, num_tokens, num_kv_heads, group, split_tokens,
                max_splits, max_items, items, n_items, fingerprint);
  } else {
    const int64_t row_lo = (int64_t)(blockIdx.x - 1) * kPlanReqs;
    prepare_rows<kPlanReqs>(nst, nct, block_table, bt_stride, num_reqs, num_tokens, qsl_len,
                            block_size, num_blocks, req_indices, positions, slot_mapping, qsl,
                            seq_lens, logits_indices, row_lo,
                            min((int64_t)num_tokens, row_lo + kPlanReqs), false);
  }
}

// ---------------------------------------------------------------------------
// main: shared step of the decode and prefill items
// ---------------------------------------------------------------------------

template <int D>
struct Geometry {
  static constexpr int KS = D / 32;                   // QK k-steps of 32 dims
  static constexpr int DT = D / 16;                   // PV output dim tiles
  static constexpr int64_t kHeadBytes = kBlock * D * 2;  // one (block, kv head) run
};

// Loads of one 32-token step: K rows of blocks j0 and j1 (A operand of S^T),
// and 4-token V^T runs of both blocks for every 16-dim tile.  A (block, kv
// head) V run is [dim / 16][token / 4][dim % 16][token % 4] x 2 bytes: tile dt
// is 512 contiguous bytes, and the 8 bytes of (dim 16 dt + n, tokens
// 4g..4g+3) sit at 512 dt + 128 g + 8 n.
template <int D>
struct StepLoads {
  bf16x8 k0[Geometry<D>::KS], k1[Geometry<D>::KS];
  u32x2 v0[Geometry<D>::DT], v1[Geometry<D>::DT];
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Buffer descriptor word 3 for raw 32-bit buffer accesses on CDNA.
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the decode K/V stream: non-temporal.  A decode item reads
// each context block once (shared prefix blocks are read by a few concurrent
// items at most), and the streaming policy sustains a markedly higher read
// rate on scattered 4 KB runs.  Prefill tiles keep the default policy: every
// tile of a prompt chunk re-reads the same blocks, which must stay cached.
// One exception: in a launch that also holds prompt tiles, a partition of a
// split context whose first block another request holds at the same position
// (a shared prefix) is read with the default policy.  Beside the prompt
// tiles' cached lines the streaming lines of a shared run are evicted before
// the slower sharers reach them; with the default policy they stay long
// enough to be read once from memory.  In a decode-only launch the sharers
// keep step and the streaming policy stays faster.
constexpr int kKvLoadPolicy = 2;
constexpr int kSharedKvLoadPolicy = 0;
constexpr int kPrefillLoadPolicy = 0;

// Descriptor of one (block, kv head) run of a pool.  Its record count bounds
// every access to that 16-token run in hardware; a masked block gets a count
// of 0, so its loads return zeros without touching memory.
template <int D>
__device__ inline rsrc_t run_rsrc(const char* run, bool valid) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(run), 0,
                                           valid ? (int)Geometry<D>::kHeadBytes : 0, kRsrcWord3);
}

struct StepRsrc {
  rsrc_t k0, k1, v0, v1;
  bool ok0, ok1;
};

template <int D, int POL>
__device__ inline void issue_step_loads(StepLoads<D>& ld, const StepRsrc& r, int k_lane,
                                        int v_lane) {
#pragma unroll
  for (int s = 0; s < Geometry<D>::KS; ++s) {
    ld.k0[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r.k0, k_lane + s * 1024, 0, POL));
    ld.k1[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r.k1, k_lane + s * 1024, 0, POL));
  }
#pragma unroll
  for (int dt = 0; dt < Geometry<D>::DT; ++dt) {
    ld.v0[dt] = __builtin_amdgcn_raw_buffer_load_b64(r.v0, v_lane + dt * (16 * kBlock * 2), 0, POL);
    ld.v1[dt] = __builtin_amdgcn_raw_buffer_load_b64(r.v1, v_lane + dt * (16 * kBlock * 2), 0, POL);
  }
}

// Online-softmax state of one 16-column tile held by a wave.
template <int D>
struct TileState {
  f32x4 o[Geometry<D>::DT];  // O^T: lane (n, g) holds dims 16*dt + 4*g + i of column n
  float m;                   // running max of raw scores (same in all lanes of a column)
  float l;                   // this lane's partial sum of exp weights
};

template <int D>
__device__ inline void tile_init(TileState<D>& st) {
#pragma unroll
  for (int dt = 0; dt < Geometry<D>::DT; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
}

// One 32-token step for one column tile: S^T = K Q^T, mask, online softmax,
// O^T += V^T P^T.  `kpos` is the position of element 0 of this lane's block-0
// run (block j0 start + 4 * g); element i of block 1 is at kpos + 16 + i.
template <int D, bool MASK>
__device__ inline void tile_step(TileState<D>& st, const bf16x8* qf, const StepLoads<D>& ld,
                                 const bf16x8* vf, int kpos, int p_col, bool ok0, bool ok1,
                                 float c2) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < Geometry<D>::KS; ++s) {
    s0 = mfma_bf16(ld.k0[s], qf[s], s0);
    s1 = mfma_bf16(ld.k1[s], qf[s], s1);
  }
  if (MASK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0[i] = (ok0 && kpos + i <= p_col) ? s0[i] : -INFINITY;
      s1[i] = (ok1 && kpos + 16 + i <= p_col) ? s1[i] : -INFINITY;
    }
  }
  float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                   fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
  mx = column_max(mx);
  const float m_new = fmaxf(st.m, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = fast_exp2((st.m - m_use) * c2);
  float p[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = fast_exp2((s0[i] - m_use) * c2);
    p[4 + i] = fast_exp2((s1[i] - m_use) * c2);
  }
  st.l = st.l * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
  st.m = m_new;
  bf16x8 pf;
#pragma unroll
  for (int i = 0; i < 8; ++i) pf[i] = static_cast<__bf16>(p[i]);
#pragma unroll
  for (int dt = 0; dt < Geometry<D>::DT; ++dt) {
    st.o[dt] *= alpha;
    st.o[dt] = mfma_bf16(vf[dt], pf, st.o[dt]);
  }
}

// V^T operand of one step: elements 0..3 = block j0 tokens 4g..4g+3, 4..7 =
// block j1 tokens 4g..4g+3.  Under MASK, tokens past the context or in an
// invalid block are zeroed (their probability is 0, but the pool may hold NaN
// there and 0 * NaN would poison the sum).
template <int D, bool MASK>
__device__ inline void build_v_operand(bf16x8* vf, const StepLoads<D>& ld, int kpos, int seq_len,
                                       bool ok0, bool ok1) {
  unsigned keep0 = 0xFu, keep1 = 0xFu;
  if (MASK) {
    keep0 = 0u;
    keep1 = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      keep0 |= (ok0 && kpos + i < seq_len) ? (1u << i) : 0u;
      keep1 |= (ok1 && kpos + 16 + i < seq_len) ? (1u << i) : 0u;
    }
  }
#pragma unroll
  for (int dt = 0; dt < Geometry<D>::DT; ++dt) {
    u32x2 a = ld.v0[dt], b = ld.v1[dt];
    if (MASK) {
      a = keep_bf16x4(a, keep0);
      b = keep_bf16x4(b, keep1);
    }
    vf[dt] = __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
  }
}

// Descriptors of the two blocks of one step (wave-uniform block ids).
template <int D>
__device__ inline StepRsrc make_step(const AttnArgs& a, int b0, int b1, const char* kbase,
                                     const char* vbase) {
  StepRsrc r;
  r.ok0 = b0 >= 0 && b0 < a.num_blocks;
  r.ok1 = b1 >= 0 && b1 < a.num_blocks;
  const int64_t stride = (int64_t)a.num_kv_heads * Geometry<D>::kHeadBytes;
  const int64_t o0 = (r.ok0 ? (int64_t)b0 : 0) * stride;
  const int64_t o1 = (r.ok1 ? (int64_t)b1 : 0) * stride;
  r.k0 = run_rsrc<D>(kbase + o0, r.ok0);
  r.k1 = run_rsrc<D>(kbase + o1, r.ok1);
  r.v0 = run_rsrc<D>(vbase + o0, r.ok0);
  r.v1 = run_rsrc<D>(vbase + o1, r.ok1);
  return r;
}

// Walks 32-token steps [s_begin, s_end) of one request for NT column tiles,
// software-pipelined: the loads of step s+1 are in flight while step s is
// computed, and the block ids of step s+2 are fetched with scalar loads (they
// are wave-uniform; scalar loads are counted apart from vector loads, so they
// never force the in-flight K/V loads to drain).  Steps whose keys all lie at
// or below p_unmasked (and whose blocks are valid) skip the causal / tail
// masking.
template <int D, int NT, int POL>
__device__ __attribute__((always_inline)) inline void walk_steps(
    TileState<D> (&st)[NT], const bf16x8 (&qf)[NT][Geometry<D>::KS], const int (&p_col)[NT],
    const AttnArgs& a, table_t* bt, int nblk, int s_begin, int s_end,
    int p_unmasked, int seq_len, const char* kbase, const char* vbase, float c2) {
  if (s_begin >= s_end) return;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  // K slab s of a run (1 KB): token n, dims 32s + 8g .. + 7 at 64 n + 16 g;
  // the 64 lanes of one load read the whole slab
  const int k_lane = 64 * n + 16 * g;
  const int v_lane = 128 * g + 8 * n;
  const int lim = min(nblk, (int)min<int64_t>(a.bt_stride, 0x7fffffff));
  const int last_col = (int)min<int64_t>(a.bt_stride, 0x7fffffff) - 1;

  // block ids of a step: always-valid addresses, validity applied after the load
  const int lim_walk = min(lim, 2 * s_end);  // blocks past the walk are never loaded
  auto ids_at = [&](int step) {
    const int j0 = 2 * step, j1 = j0 + 1;
    int b0 = bt[min(j0, last_col)];
    int b1 = bt[min(j1, last_col)];
    return int2{j0 < lim_walk ? b0 : -1, j1 < lim_walk ? b1 : -1};
  };
  auto compute = [&](const StepLoads<D>& ld, const StepRsrc& sb, int step) {
    const int kpos = step * 2 * kBlock + 4 * g;
    const bool mask = (step * 2 * kBlock + 2 * kBlock - 1 > p_unmasked) || !sb.ok0 || !sb.ok1;
    bf16x8 vf[Geometry<D>::DT];
    if (mask) {
      build_v_operand<D, true>(vf, ld, kpos, seq_len, sb.ok0, sb.ok1);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        tile_step<D, true>(st[nt], qf[nt], ld, vf, kpos, p_col[nt], sb.ok0, sb.ok1, c2);
    } else {
      build_v_operand<D, false>(vf, ld, kpos, seq_len, true, true);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        tile_step<D, false>(st[nt], qf[nt], ld, vf, kpos, p_col[nt], true, true, c2);
    }
  };

  StepLoads<D> A, B;
  int2 ids = ids_at(s_begin);
  StepRsrc sa = make_step<D>(a, ids.x, ids.y, kbase, vbase), sbk;
  issue_step_loads<D, POL>(A, sa, k_lane, v_lane);
  ids = ids_at(s_begin + 1);
  int step = s_begin;
  while (true) {
    // past the end the ids are -1: zero-count descriptors, no memory traffic
    sbk = make_step<D>(a, ids.x, ids.y, kbase, vbase);
    ids = ids_at(step + 2);
    issue_step_loads<D, POL>(B, sbk, k_lane, v_lane);
    compute(A, sa, step);
    if (++step >= s_end) break;
    sa = make_step<D>(a, ids.x, ids.y, kbase, vbase);
    ids = ids_at(step + 2);
    issue_step_loads<D, POL>(A, sa, k_lane, v_lane);
    compute(B, sbk, step);
    if (++step >= s_end) break;
  }
}

// ---------------------------------------------------------------------------
// FP8 E4M3 pools: the decode walk
// ---------------------------------------------------------------------------
//
// An FP8 run of one (block, kv head) is 16 * D bytes.  K runs are slabs of
// 64 dims, [dim / 64][token][dim % 64]; the 16-byte load of lane (n, g) in
// slab t is token n, dims 64t + 16g .. + 15 (one load instruction reads the
// whole 1 KB slab), and holds the A operands of QK k-steps 2t (its first 8
// bytes) and 2t + 1 (the last 8): the contraction over dims may run in any
// order as long as Q follows the same one.  V runs are laid out [dim / 64][token / 4][dim % 16][(dim / 16) % 4]
// [token % 4], so one 16-byte load of lane (n, g) holds tokens 4g..4g+3 of
// dims 64 dq + 16 dt + n for four 16-dim tiles dt: the V^T operand runs of
// four PV MFMAs.  Codes widen exactly to bf16; k_scale is folded into the
// softmax scale and v_scale into the output.

template <int D>
struct Geometry8 {
  static constexpr int kHeadBytes = kBlock * D;  // one (block, kv head) run
  static constexpr int KL = D / 64;               // 16-byte K loads per token row
  static constexpr int VL = D / 64;               // 16-byte V loads per lane and block
};

template <int D>
struct StepLoads8 {
  u32x4 k0[Geometry8<D>::KL], k1[Geometry8<D>::KL];
  u32x4 v0[Geometry8<D>::VL], v1[Geometry8<D>::VL];
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight E4M3 codes (bytes of a, then of b) as eight bf16 values (exact).
__device__ inline bf16x8 fp8x8_to_bf16(unsigned a, unsigned b) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a, 1.0f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a, 1.0f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.0f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int D>
__device__ inline rsrc_t run_rsrc8(const char* run, bool valid) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(run), 0,
                                           valid ? (int)Geometry8<D>::kHeadBytes : 0, kRsrcWord3);
}

template <int D>
__device__ inline StepRsrc make_step8(const AttnArgs& a, int b0, int b1, const char* kbase,
                                      const char* vbase) {
  StepRsrc r;
  r.ok0 = b0 >= 0 && b0 < a.num_blocks;
  r.ok1 = b1 >= 0 && b1 < a.num_blocks;
  const int64_t stride = (int64_t)a.num_kv_heads * Geometry8<D>::kHeadBytes;
  const int64_t o0 = (r.ok0 ? (int64_t)b0 : 0) * stride;
  const int64_t o1 = (r.ok1 ? (int64_t)b1 : 0) * stride;
  r.k0 = run_rsrc8<D>(kbase + o0, r.ok0);
  r.k1 = run_rsrc8<D>(kbase + o1, r.ok1);
  r.v0 = run_rsrc8<D>(vbase + o0, r.ok0);
  r.v1 = run_rsrc8<D>(vbase + o1, r.ok1);
  return r;
}

template <int D, int POL>
__device__ inline void issue_step_loads8(StepLoads8<D>& ld, const StepRsrc& r, int k_lane,
                                         int v_lane) {
#pragma unroll
  for (int t = 0; t < Geometry8<D>::KL; ++t) {
    ld.k0[t] = __builtin_amdgcn_raw_buffer_load_b128(r.k0, k_lane + 1024 * t, 0, POL);
    ld.k1[t] = __builtin_amdgcn_raw_buffer_load_b128(r.k1, k_lane + 1024 * t, 0, POL);
  }
#pragma unroll
  for (int q = 0; q < Geometry8<D>::VL; ++q) {
    ld.v0[q] = __builtin_amdgcn_raw_buffer_load_b128(r.v0, v_lane + 1024 * q, 0, POL);
    ld.v1[q] = __builtin_amdgcn_raw_buffer_load_b128(r.v1, v_lane + 1024 * q, 0, POL);
  }
}

// tile_step over FP8 loads: qf[s] must hold dims 64(s / 2) + 16g + 8(s % 2)
// .. + 7 of the lane's column.
template <int D, bool MASK>
__device__ inline void tile_step8(TileState<D>& st, const bf16x8* qf, const StepLoads8<D>& ld,
                                  int kpos, int p_col, bool ok0, bool ok1, int seq_len,
                                  float c2) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < Geometry8<D>::KL; ++t) {
    s0 = mfma_bf16(fp8x8_to_bf16(ld.k0[t].x, ld.k0[t].y), qf[2 * t], s0);
    s1 = mfma_bf16(fp8x8_to_bf16(ld.k1[t].x, ld.k1[t].y), qf[2 * t], s1);
    s0 = mfma_bf16(fp8x8_to_bf16(ld.k0[t].z, ld.k0[t].w), qf[2 * t + 1], s0);
    s1 = mfma_bf16(fp8x8_to_bf16(ld.k1[t].z, ld.k1[t].w), qf[2 * t + 1], s1);
  }
  unsigned keep0 = 0xFu, keep1 = 0xFu;
  if (MASK) {
    keep0 = 0u;
    keep1 = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0[i] = (ok0 && kpos + i <= p_col) ? s0[i] : -INFINITY;
      s1[i] = (ok1 && kpos + 16 + i <= p_col) ? s1[i] : -INFINITY;
      keep0 |= (ok0 && kpos + i < seq_len) ? (1u << i) : 0u;
      keep1 |= (ok1 && kpos + 16 + i < seq_len) ? (1u << i) : 0u;
    }
  }
  float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                   fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
  mx = column_max(mx);
  const float m_new = fmaxf(st.m, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = fast_exp2((st.m - m_use) * c2);
  float p[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = fast_exp2((s0[i] - m_use) * c2);
    p[4 + i] = fast_exp2((s1[i] - m_use) * c2);
  }
  st.l = st.l * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
  st.m = m_new;
  bf16x8 pf;
#pragma unroll
  for (int i = 0; i < 8; ++i) pf[i] = static_cast<__bf16>(p[i]);
#pragma unroll
  for (int q = 0; q < Geometry8<D>::VL; ++q) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u32x2 lo = __builtin_bit_cast(u32x2, fp8x8_to_bf16(ld.v0[q][w], 0u).lo);
      u32x2 hi = __builtin_bit_cast(u32x2, fp8x8_to_bf16(ld.v1[q][w], 0u).lo);
      if (MASK) {
        lo = keep_bf16x4(lo, keep0);
        hi = keep_bf16x4(hi, keep1);
      }
      const int dt = 4 * q + w;
      st.o[dt] *= alpha;
      st.o[dt] = mfma_bf16(__builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y}), pf,
                           st.o[dt]);
    }
  }
}

// walk_steps over FP8 pools (same pipeline: loads of step s+1 in flight while
// step s is computed).
template <int D, int POL>
__device__ __attribute__((always_inline)) inline void walk_steps8(
    TileState<D>& st, const bf16x8 (&qf)[Geometry<D>::KS], int p_col, const AttnArgs& a,
    table_t* bt, int nblk, int s_begin, int s_end, int p_unmasked, int seq_len,
    const char* kbase, const char* vbase, float c2) {
  if (s_begin >= s_end) return;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int k_lane = 64 * n + 16 * g;  // + 1024 t: token n, dims 64t + 16g .. + 15
  const int v_lane = (16 * g + n) * 16;
  const int lim = min(nblk, (int)min<int64_t>(a.bt_stride, 0x7fffffff));
  const int last_col = (int)min<int64_t>(a.bt_stride, 0x7fffffff) - 1;
  const int lim_walk = min(lim, 2 * s_end);
  auto ids_at = [&](int step) {
    const int j0 = 2 * step, j1 = j0 + 1;
    int b0 = bt[min(j0, last_col)];
    int b1 = bt[min(j1, last_col)];
    return int2{j0 < lim_walk ? b0 : -1, j1 < lim_walk ? b1 : -1};
  };
  auto compute = [&](const StepLoads8<D>& ld, const StepRsrc& sb, int step) {
    const int kpos = step * 2 * kBlock + 4 * g;
    const bool mask = (step * 2 * kBlock + 2 * kBlock - 1 > p_unmasked) || !sb.ok0 || !sb.ok1;
    if (mask)
      tile_step8<D, true>(st, qf, ld, kpos, p_col, sb.ok0, sb.ok1, seq_len, c2);
    else
      tile_step8<D, false>(st, qf, ld, kpos, p_col, true, true, seq_len, c2);
  };
  StepLoads8<D> A, B;
  int2 ids = ids_at(s_begin);
  StepRsrc sa = make_step8<D>(a, ids.x, ids.y, kbase, vbase), sbk;
  issue_step_loads8<D, POL>(A, sa, k_lane, v_lane);
  ids = ids_at(s_begin + 1);
  int step = s_begin;
  while (true) {
    sbk = make_step8<D>(a, ids.x, ids.y, kbase, vbase);
    ids = ids_at(step + 2);
    issue_step_loads8<D, POL>(B, sbk, k_lane, v_lane);
    compute(A, sa, step);
    if (++step >= s_end) break;
    sa = make_step8<D>(a, ids.x, ids.y, kbase, vbase);
    ids = ids_at(step + 2);
    issue_step_loads8<D, POL>(A, sa, k_lane, v_lane);
    compute(B, sbk, step);
    if (++step >= s_end) break;
  }
}

// ---------------------------------------------------------------------------
// decode item
// ---------------------------------------------------------------------------

template <int D>
struct DecodeSmem {
  float m[kWaves][kPairsPerTile];
  float l[kWaves][kPairsPerTile];
  float o[kWaves][kPairsPerTile][D + 4];
};

// KV8: the pools hold FP8 E4M3 codes; c2 already carries k_scale and vs is
// v_scale (1 for 16-bit pools).
template <int D, bool KV8>
__device__ void run_decode(const AttnArgs& a, int group, float c2, float vs, int r, int kvh,
                           int split, int nsplit, int max_splits, float* __restrict__ ml,
                           float* __restrict__ opart, DecodeSmem<D>& sm, bool with_prompts) {
  using Geo = Geometry<D>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n = lane & 15, g = lane >> 4;
  const int row0 = a.qsl[r];
  const int q_len = a.qsl[r + 1] - row0;
  const int L = a.seq_lens[r];
  const int pairs = q_len * group;

  // MFMA column n = (row t, head hh) pair n of this item
  const bool col_ok = n < pairs;
  const int t = col_ok ? n / group : 0;
  const int head = kvh * group + (col_ok ? n - t * group : 0);
  int p_col[1] = {col_ok ? L - q_len + t : -1};

  bf16x8 qf[1][Geo::KS];
  {
    const char* qrow = static_cast<const char*>(a.q) +
                       ((int64_t)(row0 + t) * a.q_stride + (int64_t)head * D) * 2;
#pragma unroll
    for (int s = 0; s < Geo::KS; ++s) {
      // the FP8 K loads pair k-steps 2t and 2t+1 over dims 64t + 16g .. + 15
      const int dim = KV8 ? 64 * (s >> 1) + 16 * g + 8 * (s & 1) : 32 * s + 8 * g;
      qf[0][s] = col_ok ? ld_b128(qrow + dim * 2)
                        : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  const int nblk = L > 0 ? ceil_div(L, kBlock) : 0;
  const int steps_all = ceil_div(nblk, 2);
  const int per_split = ceil_div(steps_all, nsplit);
  const int sp_begin = split * per_split;
  const int sp_end = min(steps_all, sp_begin + per_split);
  const int per_wave = ceil_div(max(0, sp_end - sp_begin), kWaves);
  const int w_begin = sp_begin + wave * per_wave;
  const int w_end = min(sp_end, w_begin + per_wave);

  table_t* bt = table_row(a.block_table, a.bt_stride, r);
  const int64_t run = KV8 ? Geometry8<D>::kHeadBytes : Geo::kHeadBytes;
  const char* kbase = static_cast<const char*>(a.key_cache) + kvh * run;
  const char* vbase = static_cast<const char*>(a.value_cache) + kvh * run;

  // A partition whose first block another request holds at the same position
  // (a shared prefix) is read with the default cache policy when prompt tiles
  // share the launch (kSharedKvLoadPolicy; 16-bit pools only: a second FP8
  // walk measured slower on every FP8 launch, shared or not).  Only split
  // contexts are checked: they exist when the batch has few (request, kv
  // head) items, so the check reads at most a few hundred table entries, once
  // per item.
  bool shared = false;
  if (!KV8 && with_prompts && nsplit > 1) {
    const int j0 = 2 * sp_begin;
    const int id0 = (j0 < nblk && j0 < a.bt_stride) ? bt[j0] : -1;
    bool hit = false;
    if (id0 >= 0 && id0 < a.num_blocks) {
      for (int rr = threadIdx.x; rr < a.num_reqs; rr += kThreads) {
        if (rr == r) continue;
        const int len = a.seq_lens[rr];
        if (len > 0 && j0 < ceil_div(len, kBlock) && a.block_table[(int64_t)rr * a.bt_stride + j0] == id0)
          hit = true;
      }
    }
    shared = __syncthreads_or(hit);
  }

  TileState<D> st[1];
  tile_init(st[0]);
  if (KV8) {
    walk_steps8<D, kKvLoadPolicy>(st[0], qf[0], p_col[0], a, bt, nblk, w_begin, w_end,
                                  L - q_len, L, kbase, vbase, c2);
  } else {
    if (shared)
      walk_steps<D, 1, kSharedKvLoadPolicy>(st, qf, p_col, a, bt, nblk, w_begin, w_end,
                                            L - q_len, L, kbase, vbase, c2);
    else
      walk_steps<D, 1, kKvLoadPolicy>(st, qf, p_col, a, bt, nblk, w_begin, w_end, L - q_len,
                                      L, kbase, vbase, c2);
  }

  // merge the four waves' states
  const float l_tot = column_sum(st[0].l);
  if (g == 0) {
    sm.m[wave][n] = st[0].m;
    sm.l[wave][n] = l_tot;
  }
#pragma unroll
  for (int dt = 0; dt < Geo::DT; ++dt)
    *reinterpret_cast<f32x4*>(&sm.o[wave][n][16 * dt + 4 * g]) = st[0].o[dt];
  __syncthreads();

  constexpr int kDimsPerThread = D / 16;  // 256 threads = 16 columns x 16 dim chunks
  const int cn = threadIdx.x >> 4;
  const int cd = (threadIdx.x & 15) * kDimsPerThread;
  if (cn < pairs) {
    float mw[kWaves];
    float mmax = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = sm.m[w][cn];
      mmax = fmaxf(mmax, mw[w]);
    }
    float lsum = 0.f;
    float acc[kDimsPerThread];
#pragma unroll
    for (int k = 0; k < kDimsPerThread; ++k) acc[k] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = (mw[w] == -INFINITY) ? 0.f : fast_exp2((mw[w] - mmax) * c2);
      lsum += f * sm.l[w][cn];
#pragma unroll
      for (int k = 0; k < kDimsPerThread; ++k) acc[k] += f * sm.o[w][cn][cd + k];
    }
#pragma unroll
    for (int k = 0; k < kDimsPerThread; ++k) acc[k] *= vs;
    const int tt = cn / group;
    const int hh = kvh * group + (cn - tt * group);
    if (nsplit == 1) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      unsigned short bits[kDimsPerThread];
#pragma unroll
      for (int k = 0; k < kDimsPerThread; ++k) bits[k] = bf16_bits(acc[k] * inv);
      char* dst = static_cast<char*>(a.out) +
                  ((int64_t)(row0 + tt) * a.out_stride + (int64_t)hh * D + cd) * 2;
      if (kDimsPerThread == 8) {
        u32x4 v;
        __builtin_memcpy(&v, bits, 16);
        *reinterpret_cast<u32x4*>(dst) = v;
      } else {
        u32x2 v;
        __builtin_memcpy(&v, bits, 8);
        *reinterpret_cast<u32x2*>(dst) = v;
      }
    } else {
      const int64_t idx =
          (((int64_t)r * a.num_kv_heads + kvh) * max_splits + split) * kPairsPerTile + cn;
      if ((threadIdx.x & 15) == 0) {
        ml[2 * idx] = mmax;
        ml[2 * idx + 1] = lsum;
      }
      float* dst = opart + idx * D + cd;
#pragma unroll
      for (int k = 0; k < kDimsPerThread; k += 4)
        *reinterpret_cast<f32x4*>(dst + k) = f32x4{acc[k], acc[k + 1], acc[k + 2], acc[k + 3]};
    }
  }
}

// ---------------------------------------------------------------------------
// prefill item: K/V staged in LDS, shared by the four waves
// ---------------------------------------------------------------------------
//
// One item = 128 (row, head) pairs of one request and kv head; wave w owns
// pairs [32w, 32w + 32) as two 16-column MFMA tiles.  The context is walked in
// 64-token steps (4 blocks).  Each step's K and V runs are fetched once per
// workgroup -- wave w fetches block w of the step through its buffer
// descriptors -- into registers while the previous step is computed, then
// written to the other half of a double-buffered LDS tile; one barrier per
// step.
//
// QK^T tile t of a step is block t (MFMA row m = token m of the block).  After
// S^T = K Q^T the lane group g of a column holds tokens 4g .. 4g+3 of blocks
// 2k and 2k+1, which is the P^T operand of PV k-step k; the V^T operand of a
// lane is the matching 4 + 4 tokens of one dim.
// LDS layouts are "operand-major": the 16 lanes of a lane group that read
// one MFMA operand fragment read one contiguous, aligned 256-byte run, which
// the gfx950 LDS serves without bank conflicts (spreading a 16-lane group
// over several rows costs extra cycles, measured with the LDS bank-conflict
// counter).  Every operand read is 16*lane or a lane base plus an immediate:
//  * K:   [block t][8-dim chunk c][16 tokens] x 16 bytes;
//  * V^T: per block, the pool's run as it is (tiles of 16 dims x 4 tokens);
//    a lane's operand (8 tokens of one dim) is two 8-byte reads 128 bytes
//    apart, and lane groups 2k, 2k+1 read 256 contiguous bytes each time.
// The staging loads pick, per lane, the global 16-byte chunk whose LDS slot
// makes each 16-lane write group fill one 256-byte segment as well.
// The softmax denominator is accumulated by one more MFMA per PV k-step, with
// an all-ones A operand: it sums exactly the bf16-rounded weights that the
// numerator uses.

constexpr int kPrefillStep = 64;  // tokens per prefill step (4 blocks)
constexpr float kLazyLog2 = 16.f;  // rescale when a column max grows by > 2^16

template <int D>
struct PrefillLayout {
  // One run per block of the step.  K runs are 64 bytes apart modulo 256 so
  // that the two blocks a K operand read touches fall in different banks.
  static constexpr int kRun = kBlock * D * 2 + 64;
  static constexpr int vRun = kBlock * D * 2;
  static constexpr int kBytes = 4 * kRun;  // one K buffer
  static constexpr int vBytes = 4 * vRun;  // one V buffer
  static constexpr int kOff0 = 0, kOff1 = kBytes;
  static constexpr int vOff0 = 2 * kBytes, vOff1 = 2 * kBytes + vBytes;
  static constexpr int total = 2 * kBytes + 2 * vBytes;
};

// FP8 pools: each wave copies its block's K and V runs into a double-buffered
// staging area and the MFMA operands are widened from there in registers.
// V runs are copied verbatim.  K runs are stored in 16-byte units swizzled
// within each 64-dim slab (token t's unit of dims 16 c .. + 15 at unit
// 4 t + (c + 2 ((t / 8) % 2)) % 4), 16 bytes apart from block to block, so
// that the 16 lanes of one operand read hit 16 different bank groups.
template <int D>
struct PrefillLayout8 {
  static constexpr int kRun = kBlock * D + 16;
  static constexpr int vRun = kBlock * D;
  static constexpr int kOff0 = 0, kOff1 = 4 * kRun;
  static constexpr int vOff0 = 8 * kRun, vOff1 = 8 * kRun + 4 * vRun;
  static constexpr int total = 8 * kRun + 8 * vRun;
};

template <int D>
struct PrefillSmem {
  char bytes[PrefillLayout<D>::total];
  alignas(4) unsigned char valid[2][4];  // per buffer: block b of the step is readable
};

// Zero element e of a (2 dims x 4 tokens) bf16 unit when first + e % 4 >= limit.
__device__ inline u32x4 keep_below4(u32x4 v, int first, int limit) {
  const unsigned lo = (first < limit) ? 0x0000FFFFu : 0u;
  const unsigned m0 = lo | ((first + 1 < limit) ? 0xFFFF0000u : 0u);
  const unsigned m1 = ((first + 2 < limit) ? 0x0000FFFFu : 0u) |
                      ((first + 3 < limit) ? 0xFFFF0000u : 0u);
  return u32x4{v.x & m0, v.y & m1, v.z & m0, v.w & m1};
}

template <typename T>
__device__ inline T lds_ld(const char* base, int off) {
  return *reinterpret_cast<const T*>(base + off);
}

// S^T = K Q^T for the two 16-row tiles t = 0, 1 of half h of a 64-key step
// (keys 32h..32h+31).  Rows are keys in a permuted order: row 4g + i of tile t
// is key 8g + 4t + i of the half, so the 4 + 4 weights a lane (n, g) ends up
// with are the 8 consecutive keys 8g..8g+7, all in block 2h + g / 2 -- one
// contiguous 16-byte run of each V dim, and of the P^T B operand.
template <int D, int NT>
// Q arrives pre-scaled by scale * log2(e) and each column's accumulator starts
// at -mref, so the result is already the log2 weight exponent of every key.
__device__ __attribute__((always_inline)) inline void prefill_qk_half(
    f32x4 (&s)[NT][2], const bf16x8 (&qf)[NT][Geometry<D>::KS], const char* kb, int h,
    const float (&mref)[NT]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    bf16x8 kf[Geometry<D>::KS];
#pragma unroll
    for (int k = 0; k < Geometry<D>::KS; ++k)
      kf[k] = lds_ld<bf16x8>(kb, 2 * h * PrefillLayout<D>::kRun + 64 * t + 1024 * k);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc = {-mref[nt], -mref[nt], -mref[nt], -mref[nt]};
#pragma unroll
      for (int k = 0; k < Geometry<D>::KS; ++k) acc = mfma_bf16(kf[k], qf[nt][k], acc);
      s[nt][t] = acc;
    }
  }
}

// Softmax weights of one half, P^T packed as the PV B operand: element j of
// lane (n, g) is key 8g + j of the half (tile 0 gives j < 4, tile 1 the rest).
// The scores are already log2 exponents relative to the column reference.
template <int NT>
__device__ __attribute__((always_inline)) inline void prefill_weights(bf16x8 (&p)[NT],
                                                                      const f32x4 (&s)[NT][2]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[nt][i] = static_cast<__bf16>(fast_exp2(s[nt][0][i]));
      p[nt][4 + i] = static_cast<__bf16>(fast_exp2(s[nt][1][i]));
    }
  }
}

// Mask, reference check and weights of one half.  Scores are held as
//   x = scale * log2(e) * (q . k) - mref,
// where mref is the column's reference max (log2 units).  The reference is
// refreshed only when some column's max grows by more than 2^kLazyLog2, i.e.
// some x exceeds kLazyLog2, or on the column's first key; then O and the
// denominator are rescaled.  Otherwise the stale reference is kept and the
// weights stay <= 2^kLazyLog2.  Numerator and denominator share the
// reference, so the result is unchanged.  Each lane compares its own max;
// the reference is column-uniform, so some lane of a column exceeds the bound
// exactly when the column max does, and only then are column maxima formed
// across lanes.  Weights are formed first and formed again in the rare refresh.
// Scores of keys a column must not see become -inf: keys past its query
// position, and every key of a block that holds no readable run.
template <int NT>
__device__ __attribute__((always_inline)) inline void prefill_mask_half(
    f32x4 (&s)[NT][2], unsigned valid, int step, int h, const int (&p_col)[NT]) {
  const int g = (threadIdx.x & 63) >> 4;
  const bool bok = (valid >> (2 * h + (g >> 1))) & 1u;
  asm volatile("");  // keep the masked path a branch of its own
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kpos = step * kPrefillStep + 32 * h + 8 * g + 4 * t + i;
        s[nt][t][i] = (bok && kpos <= p_col[nt]) ? s[nt][t][i] : -INFINITY;
      }
    }
}

// `later` holds scores of the step's other half formed with the same
// reference; a refresh shifts them too.
template <int D, int NT>
__device__ __attribute__((always_inline)) inline void prefill_softmax_half(
    bf16x8 (&p)[NT], f32x4 (&s)[NT][2], f32x4 (&later)[NT][2], f32x4 (&o)[NT][Geometry<D>::DT],
    f32x4 (&lacc)[NT], float (&mref)[NT], bool (&has_ref)[NT]) {
  float lmx[NT];
  bool need = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    lmx[nt] = fmaxf(fmaxf(fmaxf(s[nt][0][0], s[nt][0][1]), fmaxf(s[nt][0][2], s[nt][0][3])),
                    fmaxf(fmaxf(s[nt][1][0], s[nt][1][1]), fmaxf(s[nt][1][2], s[nt][1][3])));
    need = need | (!has_ref[nt] & (lmx[nt] != -INFINITY)) | (lmx[nt] > kLazyLog2);
  }
  prefill_weights<NT>(p, s);
  // Scheduling request for the block that ends here (the other half's QK or
  // PV MFMAs, this half's V operand reads and weights): two MFMAs, then
  // eight vector instructions, eight times, so the wave's own weights fill
  // the matrix unit's busy cycles.  Same-host A/B: prompt rows 1-2 % faster
  // (the 2048-token prompt 0.0904 -> 0.0887 ms, the 5000-token chunk 0.444
  // -> 0.441 ms), mixed steps and FP8 prompt rows unchanged; with one MFMA
  // per group the FP8 prompt rows were 2-3 % slower.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x402, 8, 0);  // VALU, transcendental included
  }
  if (__builtin_amdgcn_ballot_w64(need)) {  // wave-uniform, rare
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mx = column_max(lmx[nt]);
      const bool first = !has_ref[nt] && mx != -INFINITY;
      const bool grow = first || mx > kLazyLog2;
      // a column without a reference has only seen masked keys: O and its
      // denominator are still exactly 0
      const float shift = grow ? mx : 0.f;
      const float alpha = grow ? (has_ref[nt] ? fast_exp2(-mx) : 0.f) : 1.f;
      lacc[nt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < Geometry<D>::DT; ++dt) o[nt][dt] *= alpha;
      mref[nt] += shift;
      has_ref[nt] = has_ref[nt] || first;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s[nt][t] -= shift;
        later[nt][t] -= shift;
      }
    }
    prefill_weights<NT>(p, s);
  }
}

// V^T operands of half h, one per 16-dim tile.  They are read from LDS
// before the half's softmax, so their latency hides behind the exponentials.
template <int D>
__device__ __attribute__((always_inline)) inline void prefill_v_read(
    bf16x8 (&vf)[Geometry<D>::DT], const char* vb, int h) {
#pragma unroll
  for (int dt = 0; dt < Geometry<D>::DT; ++dt) {
    const u32x2 lo = lds_ld<u32x2>(vb, 2 * h * PrefillLayout<D>::vRun + dt * 512);
    const u32x2 hi = lds_ld<u32x2>(vb, 2 * h * PrefillLayout<D>::vRun + dt * 512 + 128);
    vf[dt] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
  }
}
// FP8 forms of the two operand reads.  K: lane (n, g) of tile t of half h
// reads token 8 ((n / 4) % 2) + 4t + n % 4 of block 2h + n / 8 (the row order
// of prefill_qk_half), dims 64 s + 16 g .. + 15 of each slab s: the A operands
// of k-steps 2s (first 8 codes) and 2s + 1 (Q is loaded in the same order).
// `kb` carries the lane's offset within a tile-0 read.
template <int D, int NT>
__device__ __attribute__((always_inline)) inline void prefill_qk_half8(
    f32x4 (&s)[NT][2], const bf16x8 (&qf)[NT][Geometry<D>::KS], const char* kb, int h,
    const float (&mref)[NT]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    bf16x8 kf[Geometry<D>::KS];
#pragma unroll
    for (int sl = 0; sl < D / 64; ++sl) {
      const u32x4 w = lds_ld<u32x4>(kb, 2 * h * PrefillLayout8<D>::kRun + 256 * t + 1024 * sl);
      kf[2 * sl] = fp8x8_to_bf16(w.x, w.y);
      kf[2 * sl + 1] = fp8x8_to_bf16(w.z, w.w);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc = {-mref[nt], -mref[nt], -mref[nt], -mref[nt]};
#pragma unroll
      for (int k = 0; k < Geometry<D>::KS; ++k) acc = mfma_bf16(kf[k], qf[nt][k], acc);
      s[nt][t] = acc;
    }
  }
}

// V: lane (n, g) reads, for each 64-dim group dq, the two 16-byte units of
// token groups 2 (g % 2) and 2 (g % 2) + 1 of block 2h + g / 2: word j of
// each holds 4 tokens of dim 64 dq + 16 j + n, so the pair is the V^T operand
// (keys 8 g .. + 7 of the half) of dim tile 4 dq + j.
template <int D>
__device__ __attribute__((always_inline)) inline void prefill_v_read8(
    bf16x8 (&vf)[Geometry<D>::DT], const char* vb, int h) {
#pragma unroll
  for (int dq = 0; dq < D / 64; ++dq) {
    const u32x4 lo = lds_ld<u32x4>(vb, 2 * h * PrefillLayout8<D>::vRun + 1024 * dq);
    const u32x4 hi = lds_ld<u32x4>(vb, 2 * h * PrefillLayout8<D>::vRun + 1024 * dq + 256);
#pragma unroll
    for (int j = 0; j < 4; ++j) vf[4 * dq + j] = fp8x8_to_bf16(lo[j], hi[j]);
  }
}

// O^T += V^T P^T over keys 32h..32h+31, and the denominators (an all-ones A
// operand sums exactly the bf16 weights the numerator uses).
template <int D, int NT>
__device__ __attribute__((always_inline)) inline void prefill_pv_half(
    f32x4 (&o)[NT][Geometry<D>::DT], f32x4 (&lacc)[NT], const bf16x8 (&p)[NT],
    const bf16x8 (&vf)[Geometry<D>::DT], bf16x8 ones) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) lacc[nt] = mfma_bf16(ones, p[nt], lacc[nt]);
#pragma unroll
  for (int dt = 0; dt < Geometry<D>::DT; ++dt) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[nt][dt] = mfma_bf16(vf[dt], p[nt], o[nt][dt]);
  }
}

// One 64-key step of a prefill tile from the staged K (kb) and V (vb) runs.
// `mask` (wave-uniform) is set on the diagonal steps and on steps with an
// unreadable block; only those pay for the per-key selects.
template <int D, int NT, bool KV8>
__device__ __attribute__((always_inline)) inline void prefill_step(
    f32x4 (&o)[NT][Geometry<D>::DT], f32x4 (&lacc)[NT], float (&mref)[NT], bool (&has_ref)[NT],
    const bf16x8 (&qf)[NT][Geometry<D>::KS], const char* kb, const char* vb, bool mask,
    unsigned valid, int step, const int (&p_col)[NT], bf16x8 ones) {
  f32x4 s0[NT][2], s1[NT][2];
  bf16x8 p0[NT], p1[NT];
  auto qk_half = [&](f32x4 (&sx)[NT][2], int h) {
    if constexpr (KV8)
      prefill_qk_half8<D, NT>(sx, qf, kb, h, mref);
    else
      prefill_qk_half<D, NT>(sx, qf, kb, h, mref);
  };
  auto v_read = [&](bf16x8 (&vx)[Geometry<D>::DT], int h) {
    if constexpr (KV8)
      prefill_v_read8<D>(vx, vb, h);
    else
      prefill_v_read<D>(vx, vb, h);
  };
  // The two MFMA-only stretches (QK of half 0, PV of half 1) run at raised
  // wave priority, so the SIMD's other wave gets the issue slots for its
  // vector work while this one keeps the matrix unit fed.
  __builtin_amdgcn_s_setprio(1);
  qk_half(s0, 0);
  __builtin_amdgcn_s_setprio(0);
  if (mask) prefill_mask_half<NT>(s0, valid, step, 0, p_col);
  qk_half(s1, 1);
  bf16x8 vf[Geometry<D>::DT];
  v_read(vf, 0);
  prefill_softmax_half<D, NT>(p0, s0, s1, o, lacc, mref, has_ref);
  if (mask) prefill_mask_half<NT>(s1, valid, step, 1, p_col);
  prefill_pv_half<D, NT>(o, lacc, p0, vf, ones);
  v_read(vf, 1);
  prefill_softmax_half<D, NT>(p1, s1, s0, o, lacc, mref, has_ref);
  __builtin_amdgcn_s_setprio(1);
  prefill_pv_half<D, NT>(o, lacc, p1, vf, ones);
  __builtin_amdgcn_s_setprio(0);
}

// KV8: the pools hold FP8 E4M3 codes (c2 already carries k_scale, vs is
// v_scale).  Each wave then copies its block's FP8 runs into the
// double-buffered FP8 staging area (PrefillLayout8) and every wave widens its
// operands from there in registers, with the same one barrier per step.
template <int D, bool KV8>
__device__ void run_prefill(const AttnArgs& a, int group, float c2, float vs, int r, int kvh,
                            int mtile, PrefillSmem<D>& sm) {
  using Geo = Geometry<D>;
  using Lay = PrefillLayout<D>;
  constexpr int NT = kPrefillTilesPerWave;
  constexpr int KQ = (int)(Geo::kHeadBytes / 1024);  // 16-byte loads per lane per run
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n = lane & 15, g = lane >> 4;
  const int row0 = a.qsl[r];
  const int q_len = a.qsl[r + 1] - row0;
  const int L = a.seq_lens[r];
  const int pairs = q_len * group;
  const int tile_base = mtile * kPrefillPairs;
  const int pbase = tile_base + wave * (NT * kPairsPerTile);
  const bool wave_has_rows = pbase < pairs;

  bf16x8 qf[NT][Geo::KS];
  int p_col[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int P = pbase + nt * kPairsPerTile + n;
    const bool ok = P < pairs;
    const int t = ok ? P / group : 0;
    const int head = kvh * group + (ok ? P - t * group : 0);
    p_col[nt] = ok ? L - q_len + t : -1;
    const char* qrow = static_cast<const char*>(a.q) +
                       ((int64_t)(row0 + t) * a.q_stride + (int64_t)head * D) * 2;
#pragma unroll
    for (int s = 0; s < Geo::KS; ++s) {
      // FP8 pools contract the dims of k-step s in the order of their K slabs
      const int dim = KV8 ? 64 * (s >> 1) + 16 * g + 8 * (s & 1) : 32 * s + 8 * g;
      bf16x8 v = ok ? ld_b128(qrow + dim * 2)
                    : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      // scores come out in log2 units: Q carries scale * log2(e), rounded
      // once to bf16 (2^-9 relative per element, well below the bf16
      // rounding of the weights)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = static_cast<__bf16>(static_cast<float>(v[e]) * c2);
      qf[nt][s] = v;
    }
  }
  // rows seen by this wave and by the whole workgroup
  const int t_lo = wave_has_rows ? pbase / group : 0;
  const int t_hi = wave_has_rows ? (min(pairs, pbase + NT * kPairsPerTile) - 1) / group : -1;
  const int p_lo = L - q_len + t_lo;
  const int p_hi = wave_has_rows ? L - q_len + t_hi : -1;
  const int wg_last = (min(pairs, tile_base + kPrefillPairs) - 1) / group;
  const int p_hi_wg = L - q_len + wg_last;
  const int nsteps = p_hi_wg >= 0 ? min(ceil_div(L, kPrefillStep), p_hi_wg / kPrefillStep + 1)
                                   : 0;

  table_t* bt = table_row(a.block_table, a.bt_stride, r);
  constexpr int64_t kRunBytes = KV8 ? Geometry8<D>::kHeadBytes : Geo::kHeadBytes;
  const char* kbase = static_cast<const char*>(a.key_cache) + kvh * kRunBytes;
  const char* vbase = static_cast<const char*>(a.value_cache) + kvh * kRunBytes;
  const int64_t blk_stride = (int64_t)a.num_kv_heads * kRunBytes;
  const int nblk = L > 0 ? ceil_div(L, kBlock) : 0;
  const int lim = min(nblk, (int)min<int64_t>(a.bt_stride, 0x7fffffff));
  const int last_col = (int)min<int64_t>(a.bt_stride, 0x7fffffff) - 1;

  // LDS layout of one buffer: a K area and a V area, each with one run per
  // block of the step (block b is the one wave b fetches), copied straight
  // from the pools by LDS-direct buffer loads (lane i of a load fills bytes
  // 16i..16i+15 of its 1 KB destination).
  //   K run: 1 KB per k-step s; lane (m = i & 15, gg = i >> 4) holds dims
  //          8(4s + gg)..+7 of token m, the MFMA A-operand order.
  //   V run: the pool run verbatim: 16-byte slot 32 dt + 8 u + p holds
  //          dims 16 dt + 2p and +1 of tokens 4u..4u+3.  A PV operand (8
  //          tokens of one dim) is two 8-byte reads of token groups 2c and
  //          2c+1, 128 bytes apart.
  // Source offsets of copy q: K token (lane & 15), dims 8(4q + (lane >> 4)),
  // which in the pool's 32-dim slabs is slab q at 64 (lane & 15) + 16 (lane
  // >> 4): each copy reads one whole 1 KB slab; V slot q * 64 + lane.  Both
  // are a lane base plus q times a constant.
  const int k_src = 64 * (lane & 15) + 16 * (lane >> 4);              // + 1024 q
  const int v_u = (lane >> 3) & 3;  // token group of this lane's V slots
  const int v_src = 16 * lane;      // + 1024 q
  typedef __attribute__((address_space(3))) void lds_void;
  // Issue this wave's copy of block `wave` of a step into LDS buffer `buf`.
  // Returns whether the block is readable (inside the context, id inside the
  // pool); a block that is not is not read at all.
  // FP8 copies of wave w's block: V verbatim; K slab c with lane i's unit from
  // token i / 4, dims 16 ((i % 4 - 2 ((i / 32) % 2)) % 4) .. + 15 (the swizzle
  // of PrefillLayout8).
  using L8 = PrefillLayout8<D>;
  static_assert(!KV8 || L8::total <= Lay::total, "FP8 staging must fit the 16-bit buffers");
  const int k8_src = 64 * (lane >> 2) + 16 * (((lane & 3) - 2 * ((lane >> 5) & 1)) & 3);
  auto fetch = [&](int step, int buf) {
    const int j = 4 * step + wave;
    const int id = bt[min(j, last_col)];
    const bool ok = j < lim && step < nsteps && id >= 0 && id < a.num_blocks;
    if (KV8) {
      if (ok) {
        const int64_t off = (int64_t)id * blk_stride;
        const rsrc_t rk8 = run_rsrc8<D>(kbase + off, true);
        const rsrc_t rv8 = run_rsrc8<D>(vbase + off, true);
        char* kdst = sm.bytes + (buf ? L8::kOff1 : L8::kOff0) + wave * L8::kRun;
        char* vdst = sm.bytes + (buf ? L8::vOff1 : L8::vOff0) + wave * L8::vRun;
#pragma unroll
        for (int c = 0; c < D / 64; ++c) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk8, (lds_void*)(kdst + c * 1024), 16,
                                                   k8_src + 1024 * c, 0, 0,
                                                   kPrefillLoadPolicy);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv8, (lds_void*)(vdst + c * 1024), 16,
                                                   16 * lane + 1024 * c, 0, 0,
                                                   kPrefillLoadPolicy);
        }
      }
      return ok;
    }
    if (ok) {
      const int64_t off = (int64_t)id * blk_stride;
      const rsrc_t rk_d = run_rsrc<D>(kbase + off, true);
      const rsrc_t rv_d = run_rsrc<D>(vbase + off, true);
      char* kdst = sm.bytes + (buf ? Lay::kOff1 : Lay::kOff0) + wave * Lay::kRun;
      char* vdst = sm.bytes + (buf ? Lay::vOff1 : Lay::vOff0) + wave * Lay::vRun;
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk_d, (lds_void*)(kdst + q * 1024), 16,
                                                 k_src + 1024 * q, 0, 0, kPrefillLoadPolicy);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv_d, (lds_void*)(vdst + q * 1024), 16,
                                                 v_src + 1024 * q, 0, 0, kPrefillLoadPolicy);
      }
    }
    return ok;
  };
  // After this wave's copies have landed: publish the block's validity (every
  // wave needs it for masking), zero the V run of a block that was not read,
  // and zero V tokens past the context in the last block (their weight is 0,
  // but the pool may hold NaN there and 0 * NaN would poison the sum).
  auto finish = [&](int step, int buf, bool ok) {
    if (KV8) {
      // FP8 V unit i holds tokens 4 (i / 16) .. + 3 (byte e of each word is
      // token 4 (i / 16) + e)
      char* vdst = sm.bytes + (buf ? L8::vOff1 : L8::vOff0) + wave * L8::vRun;
      if (lane == 0) sm.valid[buf][wave] = ok ? 1 : 0;
      const int tok0 = step * kPrefillStep + wave * kBlock + 4 * (lane >> 4);
      if (!ok || tok0 + 4 > L) {
        unsigned keep = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) keep |= (ok && tok0 + e < L) ? (0xFFu << (8 * e)) : 0u;
#pragma unroll
        for (int c = 0; c < D / 64; ++c) {
          u32x4* pv = reinterpret_cast<u32x4*>(vdst + c * 1024 + 16 * lane);
          const u32x4 v = ok ? *pv : u32x4{0u, 0u, 0u, 0u};
          *pv = u32x4{v.x & keep, v.y & keep, v.z & keep, v.w & keep};
        }
      }
      return;
    }
    char* vdst = sm.bytes + (buf ? Lay::vOff1 : Lay::vOff0) + wave * Lay::vRun;
    if (lane == 0) sm.valid[buf][wave] = ok ? 1 : 0;
    const int tok0 = step * kPrefillStep + wave * kBlock;  // first token of this block
    if (!ok) {
#pragma unroll
      for (int q = 0; q < KQ; ++q)
        *reinterpret_cast<u32x4*>(vdst + q * 1024 + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
    } else if (tok0 + kBlock > L) {
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
        u32x4* pv = reinterpret_cast<u32x4*>(vdst + q * 1024 + 16 * lane);
        *pv = keep_below4(*pv, tok0 + 4 * v_u, L);
      }
    }
  };
  // vmcnt(0): the LDS-direct copies are not tracked by the compiler's own
  // waits, so each wave waits for its copies before the workgroup barrier.
  auto wait_copies = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };
  // lane-constant LDS offsets of the MFMA operand reads
  // K operand row n of tile 0 is key 8(n / 4) + n % 4 of the half: block
  // n / 8 of the half, token 8((n / 4) % 2) + n % 4; lane (n, g) reads dims
  // 8(4k + g)..+7 of it.  V operand lane (n, g) reads dim 16 dt + n, keys
  // 8(g % 2)..+7 of block g / 2 of the half: token groups 2(g % 2) (at
  // 256 (g % 2) in each tile) and 2(g % 2) + 1 (128 bytes further).
  const int k_rd = (n >> 3) * Lay::kRun + (g * 16 + 8 * ((n >> 2) & 1) + (n & 3)) * 16;
  const int v_rd = (g >> 1) * Lay::vRun + (g & 1) * 256 + n * 8;
  // FP8: K operand unit of tile 0 (token tb = 8 ((n / 4) % 2) + n % 4 of
  // block n / 8, swizzled dims unit g), V units of token groups 2 (g % 2) and
  // 2 (g % 2) + 1 of block g / 2
  const int tb8 = 8 * ((n >> 2) & 1) + (n & 3);
  const int k8_rd = (n >> 3) * L8::kRun + 16 * (4 * tb8 + ((g + 2 * ((n >> 2) & 1)) & 3));
  const int v8_rd = (g >> 1) * L8::vRun + (g & 1) * 512 + 16 * n;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u,
                                                       0x3F803F80u});

  f32x4 o[NT][Geo::DT];  // O^T: lane (n, g) holds dims 16*dt + 4*g + i of column n
  f32x4 lacc[NT];        // softmax denominators (every row of a column holds the same sum)
  float mref[NT];        // reference max of the column in log2 units (0 until its first key)
  bool has_ref[NT];      // the column has seen a visible key
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int dt = 0; dt < Geo::DT; ++dt) o[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    lacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    mref[nt] = 0.f;
    has_ref[nt] = false;
  }

  {
    const bool ok0 = fetch(0, 0);
    wait_copies();
    finish(0, 0, ok0);
  }
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const bool ok_next = fetch(step + 1, buf ^ 1);
    if (step * kPrefillStep <= p_hi) {
      const char* kb = KV8 ? sm.bytes + (buf ? L8::kOff1 : L8::kOff0) + k8_rd
                           : sm.bytes + (buf ? Lay::kOff1 : Lay::kOff0) + k_rd;
      const char* vb = KV8 ? sm.bytes + (buf ? L8::vOff1 : L8::vOff0) + v8_rd
                           : sm.bytes + (buf ? Lay::vOff1 : Lay::vOff0) + v_rd;
      const unsigned vw = *reinterpret_cast<const unsigned*>(sm.valid[buf]);
      const unsigned valid = (vw & 1u) | ((vw >> 7) & 2u) | ((vw >> 14) & 4u) | ((vw >> 21) & 8u);
      const bool mask = (step * kPrefillStep + kPrefillStep - 1 > p_lo) || valid != 0xFu;
      // The step runs as two 32-key halves in a software pipeline: the QK
      // MFMAs of half 1 are issued next to the softmax of half 0, and the PV
      // MFMAs of half 0 next to the softmax of half 1, so each wave keeps its
      // matrix unit busy while its vector unit forms the weights.
      prefill_step<D, NT, KV8>(o, lacc, mref, has_ref, qf, kb, vb, mask, valid, step, p_col,
                               ones);
    }
    wait_copies();
    finish(step + 1, buf ^ 1, ok_next);
    __syncthreads();
  }

  if (!wave_has_rows) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float l_tot = lacc[nt][0];
    const int P = pbase + nt * kPairsPerTile + n;
    if (P < pairs) {
      const int t = P / group;
      const int head = kvh * group + (P - t * group);
      const float inv = l_tot > 0.f ? vs / l_tot : 0.f;
      char* dst = static_cast<char*>(a.out) +
                  ((int64_t)(row0 + t) * a.out_stride + (int64_t)head * D + 4 * g) * 2;
#pragma unroll
      for (int dt = 0; dt < Geo::DT; ++dt) {
        const f32x4 v = o[nt][dt];
        u16x4 b = {bf16_bits(v[0] * inv), bf16_bits(v[1] * inv), bf16_bits(v[2] * inv),
                   bf16_bits(v[3] * inv)};
        *reinterpret_cast<u16x4*>(dst + dt * 32) = b;
      }
    }
  }
}

template <int D>
union MainSmem {
  DecodeSmem<D> dec;
  PrefillSmem<D> pre;
};

// Two workgroups per CU (2 waves per SIMD, <= 256 registers per lane): one
// wave's softmax VALU work overlaps the other's MFMAs, and a decode item's
// start-up latency overlaps the other workgroup's loads.
//
// Prefill items (the head of the list) run on P resident workgroups; decode
// items are one workgroup each, dispatched after them, so the hardware
// dispatcher balances them.  A batch of prompt tiles only has P = min(prefill
// items, `slots`) (two per CU), each walking a fixed snake over the
// longest-first list.  A batch with decode items too has P = min(prefill
// items, `slots_mixed`) (one per CU), so each CU runs one MFMA-bound prompt
// tile beside HBM-bound decode items, and the prompt tiles are shared out
// dynamically: each resident workgroup takes its first item directly and
// claims the next ones in list order from a counter in the workspace header
// (one counter per XCD, over the items of that XCD's residue class), and
// `slots_mixed` helper workgroups placed after the decode items claim from
// the same counters once the dispatcher reaches them, i.e. as the decode
// items drain.  Without them the decode items finished 0.3 ms before the
// last prompt tiles on the 5000-token chunk + 200 decodes (FP8 pools), with
// one prompt workgroup per CU for that whole time.  The last claimant zeroes
// the counters for the next run over the same list.  (A whole-list
// claim form for prompt-only batches lost 3-16 %: 512 workgroups claiming at
// once serialise on one counter.)
template <int D, bool KV8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_main_kernel(
    AttnArgs a, int32_t group, float c2, const int4* __restrict__ items,
    const int32_t* __restrict__ n_items, int32_t max_splits, float* __restrict__ ml,
    float* __restrict__ opart, int32_t slots, int32_t slots_mixed, int32_t* __restrict__ claim) {
  __shared__ MainSmem<D> sm;
  __shared__ int next_idx[2];
  const int n = n_items[0];
  const int n_pre = n_items[kPrefillItemsWord];
  // FP8 pools: k_scale joins the softmax scale, v_scale the output
  const float c2k = KV8 ? c2 * *a.k_scale : c2;
  const float vs = KV8 ? *a.v_scale : 1.f;
  const bool mixed = n > n_pre && n_pre > 0;
  const int P = min(n_pre, mixed ? slots_mixed : slots);
  const int n_dec = n - n_pre;
  // helper workgroups after the decode items (as many as the grid holds)
  const int Hh = mixed ? max(0, min(slots_mixed, (int)gridDim.x - P - n_dec)) : 0;
  const int b = blockIdx.x;
  if (b < P || (mixed && b >= P + n_dec && b < P + n_dec + Hh)) {
    // Prompt-only launch: the first P workgroups stay resident and take
    // items b, 2P - 1 - b, 2P + b, ... (a snake over the longest-first list).
    // Launch with decode items: the P resident workgroups take item b, then
    // claim items in list order from a counter; the helper workgroups, which
    // the dispatcher starts once the decode items are all placed, claim too.
    // Claims stay on the workgroup's XCD: XCD x hands out the items past P
    // whose index is x mod 8 (for 8 kv heads, the tiles of one head), so a
    // head's K/V blocks keep being read through one L2.
    const int x = b % kXcds;
    const int first = P + (x - P % kXcds + kXcds) % kXcds;
    auto take = [&](int slot) {
      if (threadIdx.x == 0) next_idx[slot] = first + kXcds * atomicAdd(claim + x, 1);
      __syncthreads();
      return next_idx[slot];
    };
    int slot = 0;
    int idx = b < P ? b : take(slot);
    for (int k = 1; idx < n_pre; ++k) {
      const int4 it = items[idx];
      run_prefill<D, KV8>(a, group, c2k, vs, it.x, it.y, it.z, sm.pre);
      __syncthreads();
      slot ^= 1;
      idx = mixed ? take(slot) : k * P + ((k & 1) ? P - 1 - b : b);
    }
    // the last claimant leaves the counters zeroed for the next run
    if (mixed && threadIdx.x == 0 && atomicAdd(claim + kXcds, 1) == P + Hh - 1) {
#pragma unroll
      for (int y = 0; y <= kXcds; ++y) atomicExch(claim + y, 0);
    }
    return;
  }
  if (b >= P + n_dec) return;
  const int idx = n_pre + (b - P);
  if (idx >= n) return;
  const int4 it = items[idx];
  run_decode<D, KV8>(a, group, c2k, vs, it.x, it.y, it.z, it.w, max_splits, ml, opart, sm.dec,
                     n_pre > 0);
}

// ---------------------------------------------------------------------------
// reduce: combine the partitions of split decode items
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void attn_reduce_kernel(AttnArgs a, int32_t group, float c2,
                                                          int32_t split_tokens, int32_t max_splits,
                                                          const float* __restrict__ ml,
                                                          const float* __restrict__ opart) {
  const int r = blockIdx.x / a.num_kv_heads;
  const int kvh = blockIdx.x - r * a.num_kv_heads;
  const int row0 = a.qsl[r];
  const int q_len = valid_q_len(a.qsl, r, a.num_tokens);
  const int pairs = q_len * group;
  if (pairs < 1 || pairs > kPairsPerTile) return;
  const int nsplit = num_splits(a.seq_lens[r], split_tokens, max_splits);
  if (nsplit <= 1) return;
  if (a.k_scale != nullptr) c2 *= *a.k_scale;  // partial maxima are raw FP8 scores
  constexpr int kDimsPerThread = D / 16;
  const int cn = threadIdx.x >> 4;
  const int sl = threadIdx.x & 15;
  const int cd = sl * kDimsPerThread;
  if (cn >= pairs) return;  // the 16 lanes of a column leave together
  const int64_t base = (((int64_t)r * a.num_kv_heads + kvh) * max_splits) * kPairsPerTile + cn;
  // the largest partition maximum: the column's 16 lanes take every 16th
  // partition, then combine within their 16-lane segment
  float mmax = -INFINITY;
  for (int s = sl; s < nsplit; s += 16) mmax = fmaxf(mmax, ml[2 * (base + (int64_t)s * kPairsPerTile)]);
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, off, 16));
  // weighted sum over the partitions in ascending order; the loads of a
  // batch of partitions are all issued before any of them is used
  constexpr int kV = kDimsPerThread / 4;
  float lsum = 0.f;
  float acc[kDimsPerThread];
#pragma unroll
  for (int k = 0; k < kDimsPerThread; ++k) acc[k] = 0.f;
  auto batch = [&](int s0, auto u_count) {
    constexpr int U = decltype(u_count)::value;
    float2 mlv[U];
    f32x4 v[U][kV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t idx = base + (int64_t)min(s0 + u, nsplit - 1) * kPairsPerTile;
      mlv[u] = *reinterpret_cast<const float2*>(ml + 2 * idx);
#pragma unroll
      for (int k = 0; k < kV; ++k)
        v[u][k] = *reinterpret_cast<const f32x4*>(opart + idx * D + cd + 4 * k);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of its arithmetic
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = s0 + u < nsplit;  // a select, so the loads above stay hoisted
      const float ms = mlv[u].x;
      const float f = (ms == -INFINITY) ? 0.f : fast_exp2((ms - mmax) * c2);
      lsum = in ? lsum + f * mlv[u].y : lsum;
#pragma unroll
      for (int k = 0; k < kV; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[4 * k + i] = in ? acc[4 * k + i] + f * v[u][k][i] : acc[4 * k + i];
    }
  };
  int s0 = 0;
  for (; s0 + 8 <= nsplit; s0 += 8) batch(s0, std::integral_constant<int, 8>());
  for (; s0 < nsplit; s0 += 2) batch(s0, std::integral_constant<int, 2>());
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int tt = cn / group;
  const int hh = kvh * group + (cn - tt * group);
  unsigned short bits[kDimsPerThread];
#pragma unroll
  for (int k = 0; k < kDimsPerThread; ++k) bits[k] = bf16_bits(acc[k] * inv);
  char* dst = static_cast<char*>(a.out) +
              ((int64_t)(row0 + tt) * a.out_stride + (int64_t)hh * D + cd) * 2;
  if (kDimsPerThread == 8) {
    u32x4 v;
    __builtin_memcpy(&v, bits, 16);
    *reinterpret_cast<u32x4*>(dst) = v;
  } else {
    u32x2 v;
    __builtin_memcpy(&v, bits, 8);
    *reinterpret_cast<u32x2*>(dst) = v;
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one wave per (row, q head)
// ---------------------------------------------------------------------------

// Element of (dim, token) in a (block, kv head) K run: slabs of 32 dims,
// [dim / 32][token][dim % 32].
__device__ inline int k_slab_elem(int dim, int tok) {
  return ((dim >> 5) * kBlock + tok) * 32 + (dim & 31);
}

// Element of (dim, token) in a (block, kv head) V run: tiles of 16 dims x 4
// tokens, [dim / 16][token / 4][dim % 16][token % 4].
__device__ inline int v_tile_elem(int dim, int tok) {
  return ((dim >> 4) * (kBlock / 4) + (tok >> 2)) * 64 + (dim & 15) * 4 + (tok & 3);
}

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a, int32_t group) {
  constexpr int PER = D / 64;
  const int row = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int R = a.num_reqs;
  int lo = 0, hi = R - 1;  // last request whose first row is <= row
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.qsl[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int r = lo;
  const int row0 = a.qsl[r];
  const int q_len = a.qsl[r + 1] - row0;
  float* out = static_cast<float*>(a.out) + (int64_t)row * a.out_stride + (int64_t)h * D;
  if (row < row0 || row >= row0 + q_len) {  // inconsistent query_start_loc
#pragma unroll
    for (int k = 0; k < PER; ++k) out[lane + 64 * k] = 0.f;
    return;
  }
  const int L = a.seq_lens[r];
  const int p = L - q_len + (row - row0);
  const int kvh = h / group;
  const float* qrow = static_cast<const float*>(a.q) + (int64_t)row * a.q_stride + (int64_t)h * D;
  float qv[PER], o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    qv[k] = qrow[lane + 64 * k];
    o[k] = 0.f;
  }
  const float* kc = static_cast<const float*>(a.key_cache);
  const float* vc = static_cast<const float*>(a.value_cache);
  const int32_t* bt = a.block_table + (int64_t)r * a.bt_stride;
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j <= p; ++j) {
    const int lb = j / kBlock;
    if (lb >= a.bt_stride) break;
    const int32_t phys = bt[lb];
    if (phys < 0 || phys >= a.num_blocks) continue;
    const int off = j - lb * kBlock;
    const int64_t head_base = (int64_t)phys * a.num_kv_heads + kvh;
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k)
      dot += qv[k] * kc[head_base * D * kBlock + k_slab_elem(lane + 64 * k, off)];
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) dot += __shfl_xor(dot, sh, 64);
    const float s = dot * a.scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float pj = expf(s - m_new);
    l = l * alpha + pj;
#pragma unroll
    for (int k = 0; k < PER; ++k)
      o[k] = o[k] * alpha + pj * vc[head_base * D * kBlock + v_tile_elem(lane + 64 * k, off)];
    m = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) out[lane + 64 * k] = o[k] * inv;
}

// The work list: item count at workspace word 0, the plan fingerprint at
// word 1, the batch checksum at word 2, the prefill item count at word
// kPrefillItemsWord, items from plan.items_offset.
hipError_t launch_plan(const AttnArgs& a, const AttnPlan& plan, void* workspace,
                       uint32_t fingerprint, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(kPlanReqs), 0, stream, a.qsl, a.seq_lens,
                     a.num_reqs, a.num_tokens, a.num_kv_heads, plan.group, plan.split_tokens,
                     plan.max_splits, plan.max_items, reinterpret_cast<int4*>(ws + plan.items_offset),
                     reinterpret_cast<int32_t*>(ws), fingerprint);
  return hipGetLastError();
}

// prepare_plan_kernel: 1 + ceil(num_tokens / 1024) workgroups.  A plan
// without a work list (no tokens, no requests, or the fp32 path) leaves the
// workspace alone.
hipError_t launch_prepare_plan_k(const PrepareArgs& p, const AttnPlan& plan, int32_t num_kv_heads,
                                 void* workspace, uint32_t fingerprint, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  const bool listed = plan.max_items > 0 && p.num_tokens > 0 && p.num_reqs > 0 && ws != nullptr;
  const int groups = 1 + (p.num_tokens + kPlanReqs - 1) / kPlanReqs;
  hipLaunchKernelGGL(prepare_plan_kernel, dim3(groups), dim3(kPlanReqs), 0, stream, p.nst, p.nct,
                     p.block_table, p.bt_stride, p.num_reqs, p.num_tokens, p.qsl_len,
                     p.block_size, p.num_blocks, p.req_indices, p.positions, p.slot_mapping,
                     p.qsl, p.seq_lens, p.logits_indices, num_kv_heads, plan.group,
                     plan.split_tokens, plan.max_splits, plan.max_items,
                     listed ? reinterpret_cast<int4*>(ws + plan.items_offset) : nullptr,
                     listed ? reinterpret_cast<int32_t*>(ws) : nullptr, fingerprint);
  return hipGetLastError();
}

template <int D, bool KV8>
hipError_t launch_run_d(const AttnArgs& a, const AttnPlan& plan, void* workspace,
                        hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  int32_t* n_items = reinterpret_cast<int32_t*>(ws);
  int4* items = reinterpret_cast<int4*>(ws + plan.items_offset);
  float* ml = plan.max_splits > 1 ? reinterpret_cast<float*>(ws + plan.ml_offset) : nullptr;
  float* opart = plan.max_splits > 1 ? reinterpret_cast<float*>(ws + plan.o_offset) : nullptr;
  const float c2 = a.scale * kLog2e;
  hipError_t e = hipSuccess;
  if (plan.max_items > 0) {
    hipLaunchKernelGGL((attn_main_kernel<D, KV8>), dim3((unsigned)plan.grid),
                       dim3(kThreads), 0, stream, a, plan.group, c2, items, n_items,
                       plan.max_splits, ml, opart, 2 * device_cu_count(), device_cu_count(),
                       reinterpret_cast<int32_t*>(ws) + kClaimWord);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (plan.max_splits > 1) {
    hipLaunchKernelGGL(attn_reduce_kernel<D>, dim3(a.num_reqs * a.num_kv_heads), dim3(256), 0,
                       stream, a, plan.group, c2, plan.split_tokens, plan.max_splits, ml, opart);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

bool make_attn_plan(int32_t num_reqs, int32_t num_tokens, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                    int32_t max_seq_len, int32_t split_tokens, pkv_dtype dtype, AttnPlan* plan) {
  if (num_reqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || head_dim <= 0 || max_query_len < 0 ||
      max_seq_len < 0 || split_tokens < 0 || split_tokens % 32 != 0)
    return false;
  AttnPlan p = {};
  p.group = num_q_heads / num_kv_heads;
  if (dtype != PKV_BF16) {
    *plan = p;
    return true;
  }
  const int64_t pairs_per_req = (int64_t)num_reqs * num_kv_heads;
  int32_t st = split_tokens;
  if (st == 0) {
    // Partition long decode contexts only when the batch has fewer
    // (request, kv head) items than the chip has CUs, and then into about
    // one item per CU, each of at least 256 tokens: more, shorter items
    // measured slower (each pays its own set-up and merge, and a shared
    // prefix's partitions run less in step).  A batch of one request with
    // more query rows than one decode tile holds no decode item, so it gets
    // no partitions (and no reduce launch).
    const int64_t want = device_cu_count();
    const bool one_prompt = num_reqs == 1 && (int64_t)max_query_len * p.group > kPairsPerTile;
    if (pairs_per_req >= want || max_seq_len <= 256 || one_prompt) {
      st = ((std::max(max_seq_len, 1) + 31) / 32) * 32;
    } else {
      const int64_t per = ((int64_t)max_seq_len * pairs_per_req + want - 1) / want;
      st = (int32_t)std::max<int64_t>(256, ((per + 31) / 32) * 32);
    }
  }
  p.split_tokens = st;
  p.max_splits = std::max(1, (std::max(max_seq_len, 1) + st - 1) / st);
  const int64_t g = p.group;
  // A prefill request has q_len * G > 16, so at most T / (16 / G + 1) requests
  // are prefill requests; each adds at most one partial tile.
  const int64_t min_prefill_q = kPairsPerTile / g + 1;
  const int64_t prefill_reqs = std::min<int64_t>(num_reqs, num_tokens / min_prefill_q);
  const int64_t prefill_tiles =
      ((int64_t)num_tokens * g + kPrefillPairs - 1) / kPrefillPairs + prefill_reqs;
  p.max_items = (int64_t)num_kv_heads * ((int64_t)num_reqs * p.max_splits + prefill_tiles);
  if (num_tokens == 0) p.max_items = 0;
  // one workgroup per item, plus one helper per CU for the prompt tiles of a
  // batch that also holds decode items
  p.grid = p.max_items + (p.max_items > 0 && prefill_reqs > 0 ? device_cu_count() : 0);
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 256;  // header: item count
  p.items_offset = off;
  off = align(off + (size_t)p.max_items * sizeof(int4));
  if (p.max_splits > 1) {
    const size_t slots = (size_t)pairs_per_req * p.max_splits * kPairsPerTile;
    p.ml_offset = off;
    off = align(off + slots * 2 * sizeof(float));
    p.o_offset = off;
    off = align(off + slots * (size_t)head_dim * sizeof(float));
  }
  p.total_bytes = off;
  *plan = p;
  return true;
}

hipError_t launch_attention_plan(const AttnArgs& a, const AttnPlan& plan, void* workspace,
                                 uint32_t fingerprint, hipStream_t stream) {
  if (a.num_tokens == 0 || a.num_reqs == 0) return hipSuccess;
  return launch_plan(a, plan, workspace, fingerprint, stream);
}

hipError_t launch_prepare_plan(const PrepareArgs& p, const AttnPlan& plan, int32_t num_kv_heads,
                               void* workspace, uint32_t fingerprint, hipStream_t stream) {
  return launch_prepare_plan_k(p, plan, num_kv_heads, workspace, fingerprint, stream);
}

hipError_t launch_attention_run(const AttnArgs& a, const AttnPlan& plan, void* workspace,
                                bool kv8, hipStream_t stream) {
  if (a.num_tokens == 0 || a.num_reqs == 0) return hipSuccess;
  if (kv8) {
    if (a.head_dim == 128) return launch_run_d<128, true>(a, plan, workspace, stream);
    return launch_run_d<64, true>(a, plan, workspace, stream);
  }
  if (a.head_dim == 128) return launch_run_d<128, false>(a, plan, workspace, stream);
  return launch_run_d<64, false>(a, plan, workspace, stream);
}

hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0 || a.num_reqs == 0) return hipSuccess;
  const int group = a.num_q_heads / a.num_kv_heads;
  dim3 grid(a.num_tokens, a.num_q_heads);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, stream, a, group);
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, stream, a, group);
  return hipGetLastError();
}

}  // namespace pkv
