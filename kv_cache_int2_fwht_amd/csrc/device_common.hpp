// Device helpers shared by the OScaR kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

constexpr int kHeadDim = 128;
constexpr int kGroup = 128;
constexpr int kWave = 64;

// One 16-byte-per-lane global -> LDS load: lane l's 16 bytes at gptr land at
// LDS byte lds + 16 l (lanes switched off write nothing).  Issued as inline
// assembly; the issuing wave tracks completion with its own vector-memory
// counter waits.  The data is read once, so the loads carry the nontemporal
// hint (a streaming probe of the decode's cache reads runs at 6.1 TB/s with
// it against 5.5 TB/s without).
__device__ __forceinline__ void lds_load16(const void* gptr, const uint8_t* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gptr), "s"(m0)
               : "memory");
}

// ---------------------------------------------------------------------------
// Cross-lane moves (DPP).  Control words of the gfx9 DPP encoding.
// ---------------------------------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]: partner lane ^ 1
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]: partner lane ^ 2
constexpr int kDppRowRor4 = 0x124;  // rotate right by 4 within a 16-lane row
constexpr int kDppRowRor8 = 0x128;  // rotate right by 8 within a 16-lane row

// Index, in blocks of 9472 bytes, of the block of group g of KV head h of
// sequence b.  Contiguous cache: blocks [batch][heads][groups_cap].  Paged
// cache: page table[b * groups_cap + g] of a pool [pages][heads], the entry
// clamped to [0, num_pages) so that any entry stays inside the pool.  The
// callers pass uniform b, h and g, and the table is read-only for the whole
// launch, so the entry is read with a scalar load.
typedef __attribute__((address_space(4))) const int32_t* ConstI32Ptr;
__device__ __forceinline__ size_t group_block_index(const int32_t* table, int32_t num_pages, int groups_cap,
                                                    int num_kv_heads, int b, int h, int g) {
  if (table == nullptr) return (static_cast<size_t>(b) * num_kv_heads + h) * groups_cap + g;
  int page = ((ConstI32Ptr)(table))[static_cast<size_t>(b) * groups_cap + g];
  page = min(max(page, 0), num_pages - 1);
  return static_cast<size_t>(page) * num_kv_heads + h;
}

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, true));
}

template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double x) {
  const int64_t bits = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(bits & 0xffffffff), kCtrl, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(bits >> 32), kCtrl, 0xF, 0xF, true);
  return __longlong_as_double((static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo));
}

// Full-wave reductions through ds_swizzle-free shuffles (used outside hot loops).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// ---------------------------------------------------------------------------
// Number formats.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp16 bit pattern -> float (exact).
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  return static_cast<double>(f16_bits_to_f32(h));
}

// fp64 -> fp16 bits, round to nearest even, saturating at +-65504.  Rounds
// once from the double value (no intermediate float rounding), so the
// result is the fp16 value nearest to x.
__device__ __forceinline__ uint16_t f64_to_f16_bits_rne_sat(double x) {
  const uint16_t sign = (x < 0.0) ? 0x8000 : 0;
  double ax = fabs(x);
  if (!(ax <= 65504.0)) ax = 65504.0;  // saturate (NaN is not supported)
  if (ax < 0x1p-14) {
    // subnormal range: value = m * 2^-24 with m in [0, 1024]; m == 1024 is
    // the smallest normal, whose bit pattern is also 1024.
    const double m = rint(ax * 0x1p24);
    return sign | static_cast<uint16_t>(m);
  }
  int e = ilogb(ax);                       // 2^e <= ax < 2^(e+1), e in [-14, 15]
  double m = rint(ldexp(ax, 10 - e));      // in [1024, 2048]
  if (m >= 2048.0) { m = 1024.0; ++e; }
  if (e > 15) return sign | 0x7BFF;        // cannot happen after the clamp; kept for safety
  return sign | static_cast<uint16_t>(((e + 15) << 10) | (static_cast<int>(m) - 1024));
}

}  // namespace oscar
