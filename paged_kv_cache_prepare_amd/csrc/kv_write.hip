// kv_write.hip -- scatter this step's K/V rows into the paged block pool.
//
// "Inside vLLM: Following One Request from the API to GPU Execution", Part 5:
// writes are token-granular -- token i's K and V rows go to cache slot
// slot_mapping[i] = block * block_size + offset.  HBM-bound copy; no math.
//
// One workgroup handles 16 consecutive tokens of one kv head.
//  * K pool rows [block][head][offset][:] are contiguous per token, so each
//    thread moves one 16-byte chunk (global load -> global store).
//  * V pool blocks are dim-major ([block][head][dim][offset]).  The 16 rows
//    are staged in LDS, then each thread writes one dimension for a run of
//    16 / element-size consecutive tokens: when those tokens occupy
//    consecutive offsets of one block (a prompt chunk) the run is a single
//    16-byte store and a whole block row is written by adjacent threads;
//    otherwise (scattered decode tokens) it falls back to element stores.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kTileTokens = 16;
constexpr int kMaxRowBytes = 1024;  // head_dim * element bytes

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int E>  // element bytes: 2 (bf16) or 4 (fp32)
__global__ __launch_bounds__(kThreads) void kv_write_kernel(
    const char* __restrict__ key, const char* __restrict__ value, int64_t key_stride,
    int64_t value_stride, char* __restrict__ key_cache, char* __restrict__ value_cache,
    int64_t num_blocks, const int64_t* __restrict__ slot_mapping, int32_t num_tokens,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
  using elem_t = typename std::conditional<E == 2, uint16_t, uint32_t>::type;
  constexpr int kVecElems = 16 / E;
  __shared__ u32x4 s_v[kTileTokens * kMaxRowBytes / 16];
  __shared__ int64_t s_slot[kTileTokens];

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTileTokens;
  const int h = blockIdx.y;
  const int chunks = head_dim * E / 16;  // 16-byte chunks per row
  const int64_t pool_slots = num_blocks * block_size;

  if (tid < kTileTokens) {
    int64_t s = -1;
    if (t0 + tid < num_tokens) {
      s = slot_mapping[t0 + tid];
      if (s >= pool_slots) s = -1;
    }
    s_slot[tid] = s < 0 ? -1 : s;
  }
  __syncthreads();

  for (int w = tid; w < kTileTokens * chunks; w += kThreads) {
    const int tk = w / chunks;
    const int c = w - tk * chunks;
    const int64_t s = s_slot[tk];
    u32x4 vv = {0u, 0u, 0u, 0u};
    if (s >= 0) {
      const int64_t row = t0 + tk;
      const u32x4 kv = *reinterpret_cast<const u32x4*>(
          key + (row * key_stride + (int64_t)h * head_dim) * E + c * 16);
      vv = *reinterpret_cast<const u32x4*>(
          value + (row * value_stride + (int64_t)h * head_dim) * E + c * 16);
      const int64_t blk = s / block_size;
      const int64_t off = s - blk * block_size;
      *reinterpret_cast<u32x4*>(
          key_cache + (((blk * num_kv_heads + h) * block_size + off) * head_dim) * E + c * 16) = kv;
    }
    s_v[tk * chunks + c] = vv;
  }
  __syncthreads();

  const elem_t* s_elems = reinterpret_cast<const elem_t*>(s_v);
  const int row_elems = head_dim;  // elements of one staged row
  constexpr int kGroups = kTileTokens / kVecElems;
  for (int w = tid; w < head_dim * kGroups; w += kThreads) {
    const int dim = w / kGroups;
    const int gi = w - dim * kGroups;
    const int tk0 = gi * kVecElems;
    const int64_t s0 = s_slot[tk0];
    bool run = s0 >= 0;
    elem_t vals[kVecElems];
#pragma unroll
    for (int j = 0; j < kVecElems; ++j) {
      vals[j] = s_elems[(tk0 + j) * row_elems + dim];
      run = run && s_slot[tk0 + j] == s0 + j;
    }
    if (run) {
      const int64_t blk = s0 / block_size;
      const int64_t off = s0 - blk * block_size;
      char* dst = value_cache + (((blk * num_kv_heads + h) * head_dim + dim) * block_size + off) * E;
      run = off + kVecElems <= block_size && (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
      if (run) {
        u32x4 packed;
        __builtin_memcpy(&packed, vals, 16);
        *reinterpret_cast<u32x4*>(dst) = packed;
      }
    }
    if (!run) {
#pragma unroll
      for (int j = 0; j < kVecElems; ++j) {
        const int64_t s = s_slot[tk0 + j];
        if (s < 0) continue;
        const int64_t blk = s / block_size;
        const int64_t off = s - blk * block_size;
        *reinterpret_cast<elem_t*>(
            value_cache + (((blk * num_kv_heads + h) * head_dim + dim) * block_size + off) * E) =
            vals[j];
      }
    }
  }
}

}  // namespace

hipError_t launch_kv_write(const void* key, const void* value, int64_t key_stride,
                           int64_t value_stride, void* key_cache, void* value_cache,
                           int64_t num_blocks, const int64_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t elem_bytes, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  dim3 grid((num_tokens + kTileTokens - 1) / kTileTokens, num_kv_heads);
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(kv_write_kernel<2>, grid, dim3(kThreads), 0, stream,
                       static_cast<const char*>(key), static_cast<const char*>(value),
                       key_stride, value_stride, static_cast<char*>(key_cache),
                       static_cast<char*>(value_cache), num_blocks, slot_mapping, num_tokens,
                       num_kv_heads, head_dim, block_size);
  } else {
    hipLaunchKernelGGL(kv_write_kernel<4>, grid, dim3(kThreads), 0, stream,
                       static_cast<const char*>(key), static_cast<const char*>(value),
                       key_stride, value_stride, static_cast<char*>(key_cache),
                       static_cast<char*>(value_cache), num_blocks, slot_mapping, num_tokens,
                       num_kv_heads, head_dim, block_size);
  }
  return hipGetLastError();
}

}  // namespace pkv
