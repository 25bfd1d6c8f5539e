// kv_write.hip -- scatter this step's K/V rows into the paged block pool.
//
// "Inside vLLM: Following One Request from the API to GPU Execution", Part 5:
// writes are token-granular -- token i's K and V rows go to cache slot
// slot_mapping[i] = block * block_size + offset.  HBM-bound copy; no math.
//
// One workgroup handles 16 consecutive tokens of one kv head.
//  * K runs ([block][head] runs of head_dim x block_size) are slabs of 32
//    dims, [dim / 32][offset][dim % 32] (k_elem): each thread moves one
//    16-byte chunk of a token's row (global load -> global store), which
//    lands inside one slab row.
//  * V runs ([block][head] runs of head_dim x 16) are tiles of 16 dims x 4
//    offsets (v_elem), so that a decode token's row touches 8 cache lines
//    per head (head_dim 128) rather than 32: each partly written line costs
//    the next kernel HBM time when it is written back.  The 16 rows are
//    staged in LDS, then each thread writes one 16-byte unit (16 / (4 E)
//    dims x 4 offsets): one store when its 4 tokens fill aligned consecutive
//    offsets of one block (a prompt chunk), element stores otherwise.
//  * Pool stores are non-temporal: the rows are read back by the attention
//    call through its own loads, and streaming them out shortened the
//    following attention launch by 2-4 us on decode batches (measured).
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kTileTokens = 16;
constexpr int kMaxRowBytes = 1024;  // head_dim * element bytes

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Element of (dim, offset) inside one (block, head) K run of head_dim x
// block_size elements: slabs of KW dims ordered [dim / KW][offset][dim % KW],
// KW = 32 (KW = head_dim when 32 does not divide it).  One 32-dim slab of a
// 16-token block is what a wave-wide 16-byte load of the attention kernels
// reads at once.
__device__ inline int64_t k_elem(int dim, int off, int head_dim, int block_size) {
  const int kw = head_dim % 32 == 0 ? 32 : head_dim;
  return ((int64_t)(dim / kw) * block_size + off) * kw + dim % kw;
}

// Element of (dim, offset) inside one (block, head) V run of head_dim x
// block_size elements: tiles of DW dims x TG offsets ordered
// [dim / DW][offset / TG][dim % DW][offset % TG], DW = 16 and TG = 4 (DW =
// head_dim when 16 does not divide it, TG = block_size when 4 does not).  A
// decode token's row then lands in head_dim / 16 cache lines per head
// instead of one line per 4 dims.
__device__ inline int64_t v_elem(int dim, int off, int head_dim, int block_size) {
  const int dw = head_dim % 16 == 0 ? 16 : head_dim;
  const int tg = block_size % 4 == 0 ? 4 : block_size;
  return ((int64_t)(dim / dw) * (block_size / tg) + off / tg) * (dw * tg) + (dim % dw) * tg +
         off % tg;
}

template <int E>  // element bytes: 2 (bf16) or 4 (fp32)
__global__ __launch_bounds__(kThreads) void kv_write_kernel(
    const char* __restrict__ key, const char* __restrict__ value, int64_t key_stride,
    int64_t value_stride, char* __restrict__ key_cache, char* __restrict__ value_cache,
    int64_t num_blocks, const int64_t* __restrict__ slot_mapping, int32_t num_tokens,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
  using elem_t = typename std::conditional<E == 2, uint16_t, uint32_t>::type;
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
      const int off = (int)(s - blk * block_size);
      const int64_t run = (int64_t)head_dim * block_size;  // elements of one (block, head) run
      __builtin_nontemporal_store(kv, reinterpret_cast<u32x4*>(
          key_cache + ((blk * num_kv_heads + h) * run +
                       k_elem(c * (16 / E), off, head_dim, block_size)) * E));
    }
    s_v[tk * chunks + c] = vv;
  }
  __syncthreads();

  // V runs are tiles of 16 dims x 4 offsets (v_elem).  A 16-byte unit of a
  // tile is 16 / (4 E) dims x 4 offsets; it is one store when its 4 tokens
  // are this tile's consecutive slots starting at an offset divisible by 4
  // (a prompt chunk), element stores otherwise (scattered decode tokens).
  const elem_t* s_elems = reinterpret_cast<const elem_t*>(s_v);
  const int64_t run = (int64_t)head_dim * block_size;  // elements of one (block, head) run
  if (head_dim % 16 == 0 && block_size % 4 == 0) {
    constexpr int kDims = 4 / E;               // dims per 16-byte unit
    constexpr int kUnits = 16 / kDims;         // units per tile and token group
    const int units = (head_dim / 16) * 4 * kUnits;
    for (int w = tid; w < units; w += kThreads) {
      const int dim0 = (w / (4 * kUnits)) * 16 + (w % kUnits) * kDims;
      const int tk0 = 4 * ((w / kUnits) & 3);
      const int64_t s0 = s_slot[tk0];
      bool whole = s0 >= 0 && (s0 & 3) == 0;
      elem_t vals[4 * kDims];  // [dim][token]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        whole = whole && s_slot[tk0 + j] == s0 + j;
#pragma unroll
        for (int c = 0; c < kDims; ++c) vals[c * 4 + j] = s_elems[(tk0 + j) * head_dim + dim0 + c];
      }
      if (whole) {
        const int64_t blk = s0 / block_size;
        const int off = (int)(s0 - blk * block_size);
        u32x4 packed;
        __builtin_memcpy(&packed, vals, 16);
        __builtin_nontemporal_store(packed, reinterpret_cast<u32x4*>(
            value_cache + ((blk * num_kv_heads + h) * run + v_elem(dim0, off, head_dim, block_size)) * E));
        continue;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t s = s_slot[tk0 + j];
        if (s < 0) continue;
        const int64_t blk = s / block_size;
        const int off = (int)(s - blk * block_size);
        elem_t* dst = reinterpret_cast<elem_t*>(value_cache) + (blk * num_kv_heads + h) * run;
#pragma unroll
        for (int c = 0; c < kDims; ++c)
          __builtin_nontemporal_store(vals[c * 4 + j], &dst[v_elem(dim0 + c, off, head_dim, block_size)]);
      }
    }
  } else {  // untiled run ([dim][offset]): element stores
    for (int w = tid; w < kTileTokens * head_dim; w += kThreads) {
      const int tk = w / head_dim, dim = w - tk * head_dim;
      const int64_t s = s_slot[tk];
      if (s < 0) continue;
      const int64_t blk = s / block_size;
      const int off = (int)(s - blk * block_size);
      reinterpret_cast<elem_t*>(value_cache)[(blk * num_kv_heads + h) * run +
                                              v_elem(dim, off, head_dim, block_size)] =
          s_elems[tk * head_dim + dim];
    }
  }
}

// FP8 E4M3 cache ("How vLLM Works Internally: A Deep Dive", "FP8 KV Cache";
// the write call's kv_cache_dtype, k_scale and v_scale): each element is
// stored as the E4M3 code of value / scale (binary32 division, nearest with
// ties to even; finite magnitudes beyond 448 saturate).
//  * K pool: each (block, head) run of head_dim * 16 bytes is
//    [dim / 64][offset][dim % 64], one 16-byte store per 16 dims.
//  * V pool: each (block, head) run of head_dim * 16 bytes is
//    [dim / 64][offset / 4][dim % 16][(dim / 16) % 4][offset % 4]: 16
//    consecutive bytes are 4 tokens of 4 dims 16 apart, the unit the
//    attention kernels load.  The tile's codes are staged in LDS; a 16-byte
//    unit is stored whole when its 4 tokens are this tile's consecutive
//    slots of one block (a prompt chunk), byte by byte otherwise.
__device__ inline float fp8_prescale(float x, float scale) {
  const float q = x / scale;
  return (q != q) ? q : fminf(fmaxf(q, -448.f), 448.f);  // NaN stays NaN
}

// E4M3 codes of four values, element 0 in the low byte.
__device__ inline unsigned fp8x4(float a, float b, float c, float d) {
  unsigned w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int E>  // element bytes of key/value: 2 (bf16) or 4 (fp32)
__device__ inline float load_elem(const char* p) {
  if (E == 2) {
    const unsigned bits = (unsigned)*reinterpret_cast<const uint16_t*>(p) << 16;
    return __builtin_bit_cast(float, bits);
  }
  return *reinterpret_cast<const float*>(p);
}

constexpr int kMaxDim8 = 256;

template <int E>
__global__ __launch_bounds__(kThreads) void kv_write_fp8_kernel(
    const char* __restrict__ key, const char* __restrict__ value, int64_t key_stride,
    int64_t value_stride, uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    int64_t num_blocks, const int64_t* __restrict__ slot_mapping, int32_t num_tokens,
    int32_t num_kv_heads, int32_t head_dim, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale) {
  __shared__ uint8_t s_v[kTileTokens][kMaxDim8];
  __shared__ int64_t s_slot[kTileTokens];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTileTokens;
  const int h = blockIdx.y;
  const int64_t pool_slots = num_blocks * kTileTokens;
  const float ks = *k_scale, vs = *v_scale;
  const int64_t run = (int64_t)head_dim * kTileTokens;  // bytes of one (block, head) run

  if (tid < kTileTokens) {
    int64_t s = -1;
    if (t0 + tid < num_tokens) {
      s = slot_mapping[t0 + tid];
      if (s >= pool_slots) s = -1;
    }
    s_slot[tid] = s < 0 ? -1 : s;
  }
  __syncthreads();

  // K rows (and the V codes into LDS): one task = 16 dims of one token
  const int chunks = head_dim / 16;
  for (int w = tid; w < kTileTokens * chunks; w += kThreads) {
    const int tk = w / chunks;
    const int c = w - tk * chunks;
    const int64_t s = s_slot[tk];
    if (s < 0) continue;
    const int64_t row = t0 + tk;
    const char* kp = key + (row * key_stride + (int64_t)h * head_dim + 16 * c) * E;
    const char* vp = value + (row * value_stride + (int64_t)h * head_dim + 16 * c) * E;
    unsigned kw[4], vw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float k4[4], v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        k4[j] = fp8_prescale(load_elem<E>(kp + (4 * i + j) * E), ks);
        v4[j] = fp8_prescale(load_elem<E>(vp + (4 * i + j) * E), vs);
      }
      kw[i] = fp8x4(k4[0], k4[1], k4[2], k4[3]);
      vw[i] = fp8x4(v4[0], v4[1], v4[2], v4[3]);
    }
    const int64_t blk = s / kTileTokens;
    const int64_t off = s - blk * kTileTokens;
    __builtin_nontemporal_store(u32x4{kw[0], kw[1], kw[2], kw[3]},
                                reinterpret_cast<u32x4*>(key_cache + (blk * num_kv_heads + h) * run +
                                                         ((c >> 2) * kTileTokens + off) * 64 +
                                                         16 * (c & 3)));
    *reinterpret_cast<u32x4*>(&s_v[tk][16 * c]) = u32x4{vw[0], vw[1], vw[2], vw[3]};
  }
  __syncthreads();

  // V: one task = one 16-byte unit (4 tokens of the tile x 4 dims 16 apart)
  const int quads = head_dim / 64;
  for (int w = tid; w < 4 * quads * 16; w += kThreads) {
    const int n = w & 15;
    const int dq = (w >> 4) % quads;
    const int tg = w / (16 * quads);  // tokens 4tg..4tg+3 of the tile
    const int tk0 = 4 * tg;
    const int64_t s0 = s_slot[tk0];
    uint8_t b[16];  // b[4 dt + tt] = token tk0 + tt, dim 64 dq + 16 dt + n
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) b[4 * dt + tt] = s_v[tk0 + tt][64 * dq + 16 * dt + n];
    bool whole = s0 >= 0 && (s0 & 3) == 0;
#pragma unroll
    for (int tt = 1; tt < 4; ++tt) whole = whole && s_slot[tk0 + tt] == s0 + tt;
    if (whole) {
      const int64_t blk = s0 / kTileTokens;
      const int g = (int)(s0 - blk * kTileTokens) / 4;
      u32x4 v;
      __builtin_memcpy(&v, b, 16);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(value_cache + (blk * num_kv_heads + h) * run +
                                                              (((int64_t)dq * 4 + g) * 16 + n) * 16));
      continue;
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int64_t s = s_slot[tk0 + tt];
      if (s < 0) continue;
      const int64_t blk = s / kTileTokens;
      const int off = (int)(s - blk * kTileTokens);
      uint8_t* unit = value_cache + (blk * num_kv_heads + h) * run +
                      (((int64_t)dq * 4 + off / 4) * 16 + n) * 16 + off % 4;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) __builtin_nontemporal_store(b[4 * dt + tt], &unit[4 * dt]);
    }
  }
}

}  // namespace

hipError_t launch_kv_write_fp8(const void* key, const void* value, int64_t key_stride,
                               int64_t value_stride, void* key_cache, void* value_cache,
                               int64_t num_blocks, const int64_t* slot_mapping,
                               int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                               int32_t elem_bytes, const float* k_scale, const float* v_scale,
                               hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  dim3 grid((num_tokens + kTileTokens - 1) / kTileTokens, num_kv_heads);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(kv_write_fp8_kernel<2>, grid, dim3(kThreads), 0, stream,
                       static_cast<const char*>(key), static_cast<const char*>(value),
                       key_stride, value_stride, static_cast<uint8_t*>(key_cache),
                       static_cast<uint8_t*>(value_cache), num_blocks, slot_mapping, num_tokens,
                       num_kv_heads, head_dim, k_scale, v_scale);
  else
    hipLaunchKernelGGL(kv_write_fp8_kernel<4>, grid, dim3(kThreads), 0, stream,
                       static_cast<const char*>(key), static_cast<const char*>(value),
                       key_stride, value_stride, static_cast<uint8_t*>(key_cache),
                       static_cast<uint8_t*>(value_cache), num_blocks, slot_mapping, num_tokens,
                       num_kv_heads, head_dim, k_scale, v_scale);
  return hipGetLastError();
}

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
