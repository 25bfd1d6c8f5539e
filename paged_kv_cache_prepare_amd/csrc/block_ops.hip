// block_ops.hip -- whole-block copy and zeroing in both KV pools.
//
// Copy-on-write ("How vLLM Works Internally: A Deep Dive", "Copy-on-Write for
// Beam Search"): when a beam must write into a block it shares, the block is
// first duplicated into a freshly allocated one and the beam's table is
// pointed there.  Zeroing ("Inside vLLM: Following One Request from the API to
// GPU Execution", Part 2, new_block_ids_to_zero): freshly allocated blocks are
// cleared before the forward pass so that an earlier owner's bytes (NaNs
// included) cannot leak into attention.
//
// Every pool layout of this library stores one block as a single contiguous
// run of block_bytes bytes, so both operations are byte streams: HBM-bound,
// no arithmetic.  Work unit: one 16 KiB chunk of one pool of one listed
// block; 256 threads move it as four 16-byte vectors each, all loads issued
// before the first store.  Consecutive workgroups cover consecutive bytes of
// a block, K pool then V pool, so each wave's accesses are fully coalesced.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kVecs = 4;                                  // 16-byte vectors per thread
constexpr int64_t kChunkBytes = (int64_t)kThreads * kVecs * 16;

struct Unit {
  int64_t item;    // index into the pair / id list
  int pool;        // 0 = K pool, 1 = V pool
  int64_t offset;  // byte offset of the chunk inside the block
};

__device__ inline Unit unit_of(int64_t w, int64_t chunks) {
  Unit u;
  u.item = w / (2 * chunks);
  const int64_t rem = w - u.item * 2 * chunks;
  u.pool = rem >= chunks ? 1 : 0;
  u.offset = (rem - u.pool * chunks) * kChunkBytes;
  return u;
}

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache, int64_t num_blocks,
    int64_t block_bytes, int64_t chunks, const int32_t* __restrict__ pairs) {
  const Unit u = unit_of(blockIdx.x, chunks);
  const int64_t src = pairs[2 * u.item];
  const int64_t dst = pairs[2 * u.item + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint8_t* pool = u.pool ? value_cache : key_cache;
  const uint4* from = reinterpret_cast<const uint4*>(pool + src * block_bytes + u.offset);
  uint4* to = reinterpret_cast<uint4*>(pool + dst * block_bytes + u.offset);
  const int64_t nvec = min((int64_t)kThreads * kVecs, (block_bytes - u.offset) >> 4);
  uint4 v[kVecs];
#pragma unroll
  for (int j = 0; j < kVecs; ++j) {
    const int64_t e = (int64_t)j * kThreads + threadIdx.x;
    if (e < nvec) v[j] = from[e];
  }
#pragma unroll
  for (int j = 0; j < kVecs; ++j) {
    const int64_t e = (int64_t)j * kThreads + threadIdx.x;
    if (e < nvec) to[e] = v[j];
  }
}

__global__ __launch_bounds__(kThreads) void zero_blocks_kernel(
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache, int64_t num_blocks,
    int64_t block_bytes, int64_t chunks, const int32_t* __restrict__ ids) {
  const Unit u = unit_of(blockIdx.x, chunks);
  const int64_t b = ids[u.item];
  if (b < 0 || b >= num_blocks) return;
  uint8_t* pool = u.pool ? value_cache : key_cache;
  uint4* to = reinterpret_cast<uint4*>(pool + b * block_bytes + u.offset);
  const int64_t nvec = min((int64_t)kThreads * kVecs, (block_bytes - u.offset) >> 4);
#pragma unroll
  for (int j = 0; j < kVecs; ++j) {
    const int64_t e = (int64_t)j * kThreads + threadIdx.x;
    if (e < nvec) to[e] = make_uint4(0, 0, 0, 0);
  }
}

}  // namespace

int64_t block_op_workgroups(int64_t block_bytes, int32_t count) {
  return 2 * ((block_bytes + kChunkBytes - 1) / kChunkBytes) * (int64_t)count;
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, int64_t num_blocks,
                              int64_t block_bytes, const int32_t* pairs, int32_t num_pairs,
                              hipStream_t stream) {
  const int64_t groups = block_op_workgroups(block_bytes, num_pairs);
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)groups), dim3(kThreads), 0, stream,
                     static_cast<uint8_t*>(key_cache), static_cast<uint8_t*>(value_cache),
                     num_blocks, block_bytes, (block_bytes + kChunkBytes - 1) / kChunkBytes,
                     pairs);
  return hipGetLastError();
}

hipError_t launch_zero_blocks(void* key_cache, void* value_cache, int64_t num_blocks,
                              int64_t block_bytes, const int32_t* ids, int32_t num_ids,
                              hipStream_t stream) {
  const int64_t groups = block_op_workgroups(block_bytes, num_ids);
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_blocks_kernel, dim3((uint32_t)groups), dim3(kThreads), 0, stream,
                     static_cast<uint8_t*>(key_cache), static_cast<uint8_t*>(value_cache),
                     num_blocks, block_bytes, (block_bytes + kChunkBytes - 1) / kChunkBytes,
                     ids);
  return hipGetLastError();
}

}  // namespace pkv
