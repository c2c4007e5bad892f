// OScaR quantizer kernel: Canalized Rotation + Omni-Token Scaling +
// per-channel INT2 for keys, per-token INT2 for values, 2-bit packing.
//
// Method: OScaR abstract (arXiv 2605.19660, fugumt.com record, "Abstract");
// ai-papers.net OScaR summary, section "OScaRの提案手法" and Fig. 4 (rotation
// first, then per-token L2 scaling).  The INT2 formula (asymmetric min/max,
// fp16 scale and zero-point, round half to even) and the packed layout are
// this library's readings of what the pages leave open.
//
// One workgroup (4 waves) quantizes one 128-token group of one (sequence,
// KV head).  Every quantity that decides an fp16 parameter or a code is
// computed in fp64: the Hadamard butterflies on bf16 inputs are then exact
// in practice, so the stored norms, scales, zero-points and codes are the
// ones an fp64 evaluation of the same formulas gives.  The memory reads are
// issued first, so that they overlap the transforms: the group's value rows
// straight into LDS (where they stay for both value passes), the key rows
// into registers.  The first key pass finds norms and per-channel ranges;
// after the block-wide reduction the second decides the codes, from the
// first pass's transformed keys kept in registers for half of each wave's
// tokens and from an identical transform repeated on the other half (read
// again from cache: keeping both halves would not fit the registers).  A
// code decision near a half-way point takes the correctly rounded division,
// on a branch of its own.
#include "device_common.hpp"
#include "internal.hpp"

namespace oscar {
namespace {

constexpr int kThreads = 256;
constexpr double kSqrt128 = 0x1.6a09e667f3bcdp+3;  // 8 * sqrt(2)

// The code of x for the levels (z, s): clamp(rne((x - z) / s), 0, 3), with
// the quotient taken as the product (x - z) * inv_s.  Within a hair of a
// half-way point that product can land on the other side of an exact tie
// than the correctly rounded quotient, so `near` reports a quotient within
// 1e-9 of one (|r - rne(r)| > 0.5 - 1e-9); code_exact decides those.
// inv_s == 0 encodes s == 0: r = 0, code 0, never near.
__device__ __forceinline__ uint32_t code_fast(double x, double z, double inv_s, bool& near) {
  const double r = (x - z) * inv_s;
  const double t = rint(r);
  near = fabs(r - t) > 0.5 - 1e-9;
  return static_cast<uint32_t>(fmin(fmax(t, 0.0), 3.0));
}
__device__ __forceinline__ uint32_t code_exact(double x, double z, double s) {
  return static_cast<uint32_t>(fmin(fmax(rint((x - z) / s), 0.0), 3.0));
}

// Minimum and maximum as the bare instructions.  fmin / fmax would first
// copy each operand the compiler cannot prove quiet (results of cross-lane
// moves, LDS loads and bit conversions) through a quieting max, one more
// instruction per operand.  The two agree on every input that is not a
// NaN; inputs holding NaN have no defined parameters either way.
__device__ __forceinline__ double min_q(double a, double b) {
  double r;
  asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ double max_q(double a, double b) {
  double r;
  asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float minf_q(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float maxf_q(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Keeps a rare branch a branch: without it the compiler computes the
// division of every code and selects, which costs more than the rest of the
// decision.
__device__ __forceinline__ void rare_path() { asm volatile("" ::: "memory"); }

// 32 channels 32L .. 32L+31 of one key row (bf16) -> the unnormalised
// Walsh-Hadamard transform Y = sqrt(128) H k in fp64 across the four lanes
// L = 0..3 of a quad: channel bits 0..4 in-lane, bits 5 and 6 across the
// quad (exact for bf16 inputs in practice).  key_row_load fetches the lane's
// 64 bytes of the row; key_fwht_raw transforms them.
__device__ __forceinline__ void key_row_load(const uint16_t* row, int L, uint4 (&raw)[4]) {
  const uint4* src = reinterpret_cast<const uint4*>(row + 32 * L);
#pragma unroll
  for (int q = 0; q < 4; ++q) raw[q] = src[q];
}
__device__ __forceinline__ void key_fwht_raw(const uint4 (&raw)[4], int L, bool rotate, double (&x)[32]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w = raw[q];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * q + 2 * e] = static_cast<double>(bf16lo_to_f32(ws[e]));
      x[8 * q + 2 * e + 1] = static_cast<double>(bf16hi_to_f32(ws[e]));
    }
  }
  if (!rotate) return;   // the rotation is switched off (ablation variants only)
#pragma unroll
  for (int bit = 1; bit < 32; bit <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & bit)) {
        const double p = x[i], r = x[i | bit];
        x[i] = p + r;
        x[i | bit] = p - r;
      }
    }
  }
  // across the quad: x + partner, or partner - x, as one fused multiply-add
  // with a factor of +-1 (the product is exact, so it rounds like the sum)
  const double s1 = (L & 1) ? -1.0 : 1.0;
  const double s2 = (L & 2) ? -1.0 : 1.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = fma(s1, x[i], dpp_f64<kDppQuadXor1>(x[i]));
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    x[i] = fma(s2, x[i], dpp_f64<kDppQuadXor2>(x[i]));
  }
}
__device__ __forceinline__ void key_fwht(const uint16_t* row, int L, bool rotate, double (&x)[32]) {
  uint4 raw[4];
  key_row_load(row, L, raw);
  key_fwht_raw(raw, L, rotate, x);
}

// Per-channel LDS arrays are read and written by the four lanes of a quad
// at channels 32 L + i (L = 0..3), 256 bytes apart: one bank.  One padding
// entry after every 32 channels puts the four lanes on four different banks.
constexpr int kChPadded = kHeadDim + kHeadDim / 32;
__device__ __forceinline__ int padc(int c) { return c + (c >> 5); }

struct QuantSmem {
  // The group's block is assembled here and written out at the end in whole
  // 16-byte pieces: its codes in `out_codes` (which reuses the key ranges'
  // space once the key parameters are known), its (s, z) pairs and norms in
  // `out_params`.
  union alignas(16) {
    struct {
      double red_min[16][kChPadded];   // per-channel min / max of the scaled keys, one row per (wave, 16-lane row)
      double red_max[16][kChPadded];
    } r;
    uint8_t out_codes[OSCAR_BLOCK_K_SZ];                        // key codes, then value codes
  } u;
  alignas(16) uint8_t out_params[OSCAR_BLOCK_BYTES - OSCAR_BLOCK_K_SZ];   // key (s, z), value (s, z), key norms
  double zs[kChPadded], ss[kChPadded], inv_s[kChPadded];   // key (z16, s16, 1 / s16) per channel (padc index)
  double inv_n[kGroup];                                  // 1 / (sqrt(128) n16) per token (0 if n16 = 0)
  double vz[kGroup], vs[kGroup], vinv[kGroup];           // value (z16, s16, 1 / s16) per token
  uint4 vrow[kGroup][kHeadDim / 8];                      // the group's values (bf16)
};

__global__ __launch_bounds__(kThreads, 2) void quantize_kv_kernel(QuantizeArgs a) {
  const int j = blockIdx.x;   // source group
  const int h = blockIdx.y;   // KV head
  const int b = blockIdx.z;   // sequence
  if (j >= a.num_groups[b]) return;
  const int groups_cap = a.capacity / kGroup;
  const int dst = a.dst_group_start[b] + j;
  if (dst < 0 || dst >= groups_cap) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const bool rotate = (a.flags & OSCAR_KEYS_UNROTATED) == 0;
  const bool scale = (a.flags & OSCAR_KEYS_UNSCALED) == 0;
  // this group's block (through the block table for a paged cache)
  uint8_t* const blk =
      a.blocks + group_block_index(a.block_table, a.num_pages, groups_cap, a.num_kv_heads, b, h, dst) * OSCAR_BLOCK_BYTES;
  const uint16_t* ksrc = a.k_src + b * a.sb + h * a.sh + static_cast<int64_t>(j) * kGroup * a.st;
  const uint16_t* vsrc = a.v_src + b * a.sb + h * a.sh + static_cast<int64_t>(j) * kGroup * a.st;

  __shared__ QuantSmem sm;

  // The memory reads first, so that they overlap the key transforms: the
  // wave's 32 value rows straight into LDS (4 rows per wave instruction),
  // then the key rows of both key passes into registers.
  {
    const uint16_t* vrows = vsrc + static_cast<int64_t>(wave * 32 + (lane >> 4)) * a.st + 8 * (lane & 15);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      lds_load16(vrows + static_cast<int64_t>(4 * i) * a.st, reinterpret_cast<const uint8_t*>(&sm.vrow[wave * 32 + 4 * i][0]));
  }

  // ---------------- keys, first pass: norms and per-channel ranges ----------------
  // Lane = (slot, L): 4 lanes per token, lane L holds channels 32L..32L+31.
  // A wave covers 16 tokens per pass, two passes: tokens wave*32 + pass*16 + slot.
  const int L = lane & 3;
  const int slot = lane >> 2;
  const int row = wave * 4 + (lane >> 4);
  uint4 kraw[2][4];
  key_row_load(ksrc + static_cast<int64_t>(wave * 32 + slot) * a.st, L, kraw[0]);
  key_row_load(ksrc + static_cast<int64_t>(wave * 32 + 16 + slot) * a.st, L, kraw[1]);
  // the first pass's transformed keys stay in registers until their codes
  // are decided after the block-wide reduction (the second pass's are
  // transformed again then: keeping both would not fit the registers)
  double xk[32];
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int t = wave * 32 + pass * 16 + slot;
    double x[32];
    uint4 raw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) raw[q] = pass ? kraw[1][q] : kraw[0][q];
    key_fwht_raw(raw, L, rotate, x);
    if (pass == 0) {
#pragma unroll
      for (int i = 0; i < 32; ++i) xk[i] = x[i];
    }
    // ||y||^2 = sum(Y^2) / 128 for the unnormalised transform Y = sqrt(128) y
    // (sum(k^2) when the rotation is off).
    double ssq = 0.0;
#pragma unroll
    for (int i = 0; i < 32; ++i) ssq = fma(x[i], x[i], ssq);
    ssq += dpp_f64<kDppQuadXor1>(ssq);   // a + b == b + a: all four lanes agree
    ssq += dpp_f64<kDppQuadXor2>(ssq);
    const double n = rotate ? sqrt(ssq * (1.0 / 128.0)) : sqrt(ssq);
    // without the scaling the stored norm is 1 and u = y
    const uint16_t n16_bits = scale ? f64_to_f16_bits_rne_sat(n) : uint16_t{0x3C00};
    const double n16 = f16_bits_to_f64(n16_bits);
    const double inv = (n16 > 0.0) ? 1.0 / (rotate ? n16 * kSqrt128 : n16) : 0.0;
    if (L == 0) {
      reinterpret_cast<uint16_t*>(sm.out_params + (OSCAR_BLOCK_K_NORM - OSCAR_BLOCK_K_SZ))[t] = n16_bits;
      sm.inv_n[t] = inv;
    }
    // per-channel min / max over the four token slots of each 16-lane row
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const double u = x[i] * inv;
      const double u4 = dpp_f64<kDppRowRor4>(u);
      double mn = min_q(u, u4);
      double mx = max_q(u, u4);
      mn = min_q(mn, dpp_f64<kDppRowRor8>(mn));
      mx = max_q(mx, dpp_f64<kDppRowRor8>(mx));
      if ((lane & 15) < 4) {
        if (pass == 0) {
          sm.u.r.red_min[row][padc(32 * L + i)] = mn;
          sm.u.r.red_max[row][padc(32 * L + i)] = mx;
        } else {   // the same lane wrote these entries in the first pass
          sm.u.r.red_min[row][padc(32 * L + i)] = min_q(sm.u.r.red_min[row][padc(32 * L + i)], mn);
          sm.u.r.red_max[row][padc(32 * L + i)] = max_q(sm.u.r.red_max[row][padc(32 * L + i)], mx);
        }
      }
    }
  }

  // ---------------- values, first pass: per-token ranges; rows kept in LDS ----------------
  // 16 lanes per token, 8 channels per lane, 4 tokens per wave pass.
  {
    const int cb = lane & 15;
    const int tslot = lane >> 4;
    // the copies of the wave's value rows (issued first) have landed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll 2
    for (int pass = 0; pass < 8; ++pass) {
      const int t = wave * 32 + pass * 4 + tslot;
      const uint4 w = sm.vrow[t][cb];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      float lo = bf16lo_to_f32(ws[0]), hi = lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f0 = bf16lo_to_f32(ws[e]), f1 = bf16hi_to_f32(ws[e]);
        lo = minf_q(lo, minf_q(f0, f1));
        hi = maxf_q(hi, maxf_q(f0, f1));
      }
      lo = minf_q(lo, dpp_f32<kDppQuadXor1>(lo));
      hi = maxf_q(hi, dpp_f32<kDppQuadXor1>(hi));
      lo = minf_q(lo, dpp_f32<kDppQuadXor2>(lo));
      hi = maxf_q(hi, dpp_f32<kDppQuadXor2>(hi));
      lo = minf_q(lo, dpp_f32<kDppRowRor4>(lo));
      hi = maxf_q(hi, dpp_f32<kDppRowRor4>(hi));
      lo = minf_q(lo, dpp_f32<kDppRowRor8>(lo));
      hi = maxf_q(hi, dpp_f32<kDppRowRor8>(hi));
      if (cb == 0) {   // the token's range, until its parameters are computed below
        sm.vz[t] = static_cast<double>(lo);
        sm.vs[t] = static_cast<double>(hi);
      }
    }
    // the parameters of the wave's 32 tokens, one per lane (computed once
    // per pass with 4 lanes active, the divisions and fp16 roundings cost
    // eight times as many instructions)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < 32) {
      const int t = wave * 32 + lane;
      const double lo = sm.vz[t], hi = sm.vs[t];
      const uint16_t s_bits = f64_to_f16_bits_rne_sat((hi - lo) / 3.0);
      const uint16_t z_bits = f64_to_f16_bits_rne_sat(lo);
      reinterpret_cast<uint32_t*>(sm.out_params + (OSCAR_BLOCK_V_SZ - OSCAR_BLOCK_K_SZ))[t] =
          static_cast<uint32_t>(s_bits) | (static_cast<uint32_t>(z_bits) << 16);
      const double s16 = f16_bits_to_f64(s_bits);
      sm.vz[t] = f16_bits_to_f64(z_bits);
      sm.vs[t] = s16;
      sm.vinv[t] = (s16 > 0.0) ? 1.0 / s16 : 0.0;
    }
  }
  __syncthreads();

  // ---------------- key parameters per channel ----------------
  if (tid < kHeadDim) {
    const int pt = padc(tid);
    double lo = sm.u.r.red_min[0][pt], hi = sm.u.r.red_max[0][pt];
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      lo = min_q(lo, sm.u.r.red_min[r][pt]);
      hi = max_q(hi, sm.u.r.red_max[r][pt]);
    }
    const uint16_t s_bits = f64_to_f16_bits_rne_sat((hi - lo) / 3.0);
    const uint16_t z_bits = f64_to_f16_bits_rne_sat(lo);
    reinterpret_cast<uint32_t*>(sm.out_params)[tid] =
        static_cast<uint32_t>(s_bits) | (static_cast<uint32_t>(z_bits) << 16);
    const double s16 = f16_bits_to_f64(s_bits);
    sm.zs[pt] = f16_bits_to_f64(z_bits);
    sm.ss[pt] = s16;
    sm.inv_s[pt] = (s16 > 0.0) ? 1.0 / s16 : 0.0;
  }

  __syncthreads();   // the key ranges are read: their space now takes the codes

  // ---------------- value codes: thread = (channel d, half of the group's tokens) ----------------
  {
    const int d = tid & (kHeadDim - 1);
    const int half = tid >> 7;
    const uint16_t* vr = reinterpret_cast<const uint16_t*>(&sm.vrow[0][0]);
    uint32_t words[4];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      uint32_t acc = 0, near_mask = 0;
#pragma unroll 4
      for (int e = 0; e < 16; ++e) {
        const int t = half * 64 + wd * 16 + e;
        const double v = static_cast<double>(bf16_to_f32(vr[t * kHeadDim + d]));
        bool near;
        acc |= code_fast(v, sm.vz[t], sm.vinv[t], near) << (2 * e);
        near_mask |= static_cast<uint32_t>(near) << e;
      }
      if (__any(near_mask != 0)) {
        rare_path();
        for (int e = 0; e < 16; ++e) {
          if ((near_mask >> e) & 1u) {
            const int t = half * 64 + wd * 16 + e;
            const double v = static_cast<double>(bf16_to_f32(vr[t * kHeadDim + d]));
            acc = (acc & ~(3u << (2 * e))) | (code_exact(v, sm.vz[t], sm.vs[t]) << (2 * e));
          }
        }
      }
      words[wd] = acc;
    }
    *reinterpret_cast<uint4*>(sm.u.out_codes + OSCAR_BLOCK_V_CODES + d * 32 + 16 * half) =
        make_uint4(words[0], words[1], words[2], words[3]);
  }
  __syncthreads();

  // ---------------- keys, second pass: codes (the second 16 tokens transformed again) ----------------
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int t = wave * 32 + pass * 16 + slot;
    double x[32];
    if (pass == 0) {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = xk[i];
    } else {
      key_fwht(ksrc + static_cast<int64_t>(t) * a.st, L, rotate, x);   // bit-identical to the first pass
    }
    const double inv = sm.inv_n[t];
    uint32_t w0 = 0, w1 = 0, near0 = 0, near1 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c0 = padc(32 * L + i), c1 = padc(32 * L + 16 + i);
      bool n0, n1;
      w0 |= code_fast(x[i] * inv, sm.zs[c0], sm.inv_s[c0], n0) << (2 * i);
      w1 |= code_fast(x[16 + i] * inv, sm.zs[c1], sm.inv_s[c1], n1) << (2 * i);
      near0 |= static_cast<uint32_t>(n0) << i;
      near1 |= static_cast<uint32_t>(n1) << i;
    }
    if (__any((near0 | near1) != 0)) {
      rare_path();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c0 = padc(32 * L + i), c1 = padc(32 * L + 16 + i);
        if ((near0 >> i) & 1u) w0 = (w0 & ~(3u << (2 * i))) | (code_exact(x[i] * inv, sm.zs[c0], sm.ss[c0]) << (2 * i));
        if ((near1 >> i) & 1u)
          w1 = (w1 & ~(3u << (2 * i))) | (code_exact(x[16 + i] * inv, sm.zs[c1], sm.ss[c1]) << (2 * i));
      }
    }
    *reinterpret_cast<uint2*>(sm.u.out_codes + OSCAR_BLOCK_K_CODES + t * 32 + 8 * L) = make_uint2(w0, w1);
  }
  __syncthreads();

  // ---------------- the block, written once with coalesced 16-byte stores ----------------
  static_assert(OSCAR_BLOCK_K_CODES == 0 && OSCAR_BLOCK_V_CODES + 4096 == OSCAR_BLOCK_K_SZ, "codes first");
  for (int i = tid; i < OSCAR_BLOCK_BYTES / 16; i += kThreads) {
    const uint4 w = (i < OSCAR_BLOCK_K_SZ / 16) ? reinterpret_cast<const uint4*>(sm.u.out_codes)[i]
                                                : reinterpret_cast<const uint4*>(sm.out_params)[i - OSCAR_BLOCK_K_SZ / 16];
    reinterpret_cast<uint4*>(blk)[i] = w;
  }
}

}  // namespace

hipError_t launch_quantize(const QuantizeArgs& a, int32_t batch, int32_t max_groups, hipStream_t s) {
  dim3 grid(max_groups, a.num_kv_heads, batch);
  hipLaunchKernelGGL(quantize_kv_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
