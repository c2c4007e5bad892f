// Measurement probes for the decode benchmark (not part of the OScaR path):
//
//  * oscar_probe_stream -- the decode kernel's cache stream with the compute
//    taken out: the same grid (split, KV head, sequence), the same
//    workgroup size and LDS footprint (so one workgroup per compute unit),
//    two loader waves per workgroup copying the split's group blocks
//    (groups s, s + S, ...; 9472 bytes each) into an 8-stage LDS ring with
//    direct global -> LDS nontemporal loads, two groups in flight per
//    loader.  Its time per launch is what HBM gives this access pattern at
//    this size, launch costs included: the attainable bound of the decode
//    kernel.
//  * oscar_probe_clock -- one wave per compute unit reads the shader clock
//    counter and the constant-rate wall clock around a fixed loop; the ratio
//    of the two deltas is the shader clock the chip ran at.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/oscar_probe.h"

namespace {

constexpr int kBlockBytes = 9472;       // one group block of the packed cache
constexpr int kRing = 8;                // LDS stages
constexpr int kLoaders = 2;             // loader waves per workgroup
constexpr int kAhead = 2;               // groups in flight per loader
constexpr int kCopiesPerGroup = 10;     // 16-byte-per-lane copy instructions per group
constexpr int kThreads = 1024;          // 16 waves, as the decode kernel for 4 query heads per KV head
constexpr int kLdsBytes = 147780;       // the decode kernel's LDS footprint for 4 query heads per KV head
static_assert(kRing * kBlockBytes <= kLdsBytes, "ring fits");

struct ProbeSmem {
  uint8_t ring[kRing][kBlockBytes];
  uint8_t pad[kLdsBytes - kRing * kBlockBytes];   // keeps one workgroup per compute unit
};

__device__ __forceinline__ void copy16(const void* gptr, const uint8_t* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gptr), "s"(m0)
               : "memory");
}

// The copies of one group block into a stage: 9 contiguous kilobytes plus
// the last 256 bytes (16 lanes).
__device__ __forceinline__ void copy_group(uint8_t* stage, const uint8_t* blk, int lane) {
#pragma unroll
  for (int j = 0; j < 9; ++j) copy16(blk + 1024 * j + 16 * lane, stage + 1024 * j);
  if (lane < 16) copy16(blk + 9216 + 16 * lane, stage + 9216);
}

template <int N>
__device__ __forceinline__ void wait_groups(int rem) {
  if constexpr (N <= 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (rem >= N) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N * kCopiesPerGroup) : "memory");
    } else {
      wait_groups<N - 1>(rem);
    }
  }
}

__global__ __launch_bounds__(kThreads) void stream_probe_kernel(const uint8_t* __restrict__ blocks, int groups_cap,
                                                                 int num_kv_heads, uint32_t* __restrict__ sink) {
  __shared__ ProbeSmem sm;
  const int split = blockIdx.x;
  const int S = gridDim.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= kLoaders) return;
  const uint8_t* slice = blocks + (static_cast<size_t>(b) * num_kv_heads + h) * groups_cap * static_cast<size_t>(kBlockBytes);
  const int n_k = (groups_cap > split) ? (groups_cap - split + S - 1) / S : 0;
  const int n_mine = (n_k > wave) ? (n_k - wave + kLoaders - 1) / kLoaders : 0;
  int issued = 0;
  for (int j = 0; j < n_mine; ++j) {
    for (; issued < min(j + kAhead, n_mine); ++issued) {
      const int k = wave + issued * kLoaders;
      // stage k % kRing last held group k - kRing of this loader, whose
      // copies completed before group k - kRing + kAhead * kLoaders was issued
      copy_group(sm.ring[k % kRing], slice + static_cast<size_t>(split + k * S) * kBlockBytes, lane);
    }
    wait_groups<kAhead - 1>(issued - 1 - j);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // one word per loader wave, so that the copies have an observable effect
  if (lane == 0)
    sink[(static_cast<size_t>(b) * gridDim.y + h) * S * kLoaders + split * kLoaders + wave] =
        *reinterpret_cast<const uint32_t*>(sm.ring[wave]);
}

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* __restrict__ out, int iters) {
  const uint64_t c0 = clock64();
  const uint64_t r0 = wall_clock64();
  float x = static_cast<float>(threadIdx.x);
  for (int i = 0; i < iters; ++i) x = fmaf(x, 0.999999f, 1e-6f);
  const uint64_t c1 = clock64();
  const uint64_t r1 = wall_clock64();
  if (threadIdx.x == 0) {
    out[3 * blockIdx.x + 0] = c1 - c0;
    out[3 * blockIdx.x + 1] = r1 - r0;
    out[3 * blockIdx.x + 2] = (x == 12345.f) ? 1u : 0u;   // keeps the loop
  }
}

}  // namespace

extern "C" {

int32_t oscar_probe_stream(const uint8_t* blocks, int32_t batch, int32_t num_kv_heads, int32_t capacity,
                           int32_t splits, uint32_t* sink, void* stream) {
  if (!blocks || !sink || batch <= 0 || num_kv_heads <= 0 || capacity <= 0 || capacity % 128 != 0 || splits <= 0 ||
      batch > 65535 || num_kv_heads > 65535)
    return 1;
  if ((reinterpret_cast<uintptr_t>(blocks) & 15u) != 0) return 1;
  dim3 grid(splits, num_kv_heads, batch);
  hipLaunchKernelGGL(stream_probe_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), blocks,
                     capacity / 128, num_kv_heads, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int32_t oscar_probe_clock(uint64_t* out, int32_t num_blocks, int32_t iters, void* stream) {
  if (!out || num_blocks <= 0 || iters < 0) return 1;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(num_blocks), dim3(64), 0, static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int32_t oscar_probe_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

}  // extern "C"
