// calib.hip -- measurement utilities of the benchmark (libpkv_calib.so): the
// shader clock seen by a spinning wave, and a plain read kernel over lists
// of 4 KB runs.  Not part of the paged KV-cache path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_calib.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int64_t kMaxTicks = 1000000000;  // 10 s of the 100 MHz counter
constexpr int kMaxRunKiB = 4;
constexpr int kInflightKiB = 32;  // bytes per wave in flight: 8 runs of 4 KiB, 16 of 2 KiB

// Exits once `ticks` ticks of the constant counter have passed; the counter
// only moves forward, so every wave reaches the end.
__global__ __launch_bounds__(64) void clock_kernel(uint64_t* out, uint64_t ticks) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0, c1 = c0;
  while (r1 - r0 < ticks) {
    __builtin_amdgcn_s_sleep(8);
    r1 = __builtin_amdgcn_s_memrealtime();
    c1 = __builtin_amdgcn_s_memtime();
  }
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

typedef const __attribute__((address_space(1))) u32x4 global_u32x4;

__device__ inline u32x4 nt_load(uint64_t addr) {
  return __builtin_nontemporal_load(reinterpret_cast<global_u32x4*>(addr));
}

// Wave w reads its runs kInflight at a time (32 KiB): all loads of a group
// are issued before any of them is used.  Lane l reads bytes 16 l + 1024 j
// of a run, j < KIB.
template <int KIB>
__global__ __launch_bounds__(256) void read_runs_kernel(const uint64_t* __restrict__ run_addr,
                                                        const int64_t* __restrict__ wave_begin,
                                                        int64_t num_waves, uint32_t* sink) {
  constexpr int kInflight = kInflightKiB / KIB;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= num_waves) return;
  const int lane = threadIdx.x & 63;
  const int64_t b = wave_begin[w], e = wave_begin[w + 1];
  uint32_t acc = 0u;
  for (int64_t r = b; r < e; r += kInflight) {
    u32x4 v[kInflight][KIB];
#pragma unroll
    for (int i = 0; i < kInflight; ++i) {
      // past the wave's list: read its last run again (same addresses, valid)
      const uint64_t run = run_addr[r + i < e ? r + i : e - 1];
#pragma unroll
      for (int j = 0; j < KIB; ++j) v[i][j] = nt_load(run + 16 * lane + 1024 * j);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the group is issued first
#pragma unroll
    for (int i = 0; i < kInflight; ++i)
#pragma unroll
      for (int j = 0; j < KIB; ++j)
        acc ^= (r + i < e) ? (v[i][j].x ^ v[i][j].y ^ v[i][j].z ^ v[i][j].w) : 0u;
  }
  sink[w * 64 + lane] = acc;
}

}  // namespace

extern "C" int pkv_calib_clock(uint64_t* out, int64_t ticks_100mhz, void* stream) {
  if (out == nullptr || ticks_100mhz < 1 || ticks_100mhz > kMaxTicks) return 1;
  hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), out,
                     (uint64_t)ticks_100mhz);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int pkv_calib_read_runs(const uint64_t* run_addr, const int64_t* wave_begin,
                                   int64_t num_waves, int32_t run_kib, uint32_t* sink,
                                   void* stream) {
  if (run_addr == nullptr || wave_begin == nullptr || sink == nullptr || num_waves < 1 ||
      num_waves > ((int64_t)1 << 31) * 4 - 4 || run_kib < 1 || run_kib > kMaxRunKiB ||
      run_kib == 3)
    return 1;
  const dim3 grid((unsigned)((num_waves + 3) / 4));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (run_kib == 4)
    hipLaunchKernelGGL(read_runs_kernel<4>, grid, dim3(256), 0, st, run_addr, wave_begin,
                       num_waves, sink);
  else if (run_kib == 2)
    hipLaunchKernelGGL(read_runs_kernel<2>, grid, dim3(256), 0, st, run_addr, wave_begin,
                       num_waves, sink);
  else if (run_kib == 1)
    hipLaunchKernelGGL(read_runs_kernel<1>, grid, dim3(256), 0, st, run_addr, wave_begin,
                       num_waves, sink);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
