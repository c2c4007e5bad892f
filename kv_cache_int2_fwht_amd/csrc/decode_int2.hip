// Single-query GQA decode attention over the packed OScaR INT2 cache.
//
// What is computed (OScaR abstract, arXiv 2605.19660; ai-papers.net OScaR
// summary, sections "OScaRの提案手法" and "実験結果"): the query is rotated once
// by the same orthonormal Hadamard matrix as the keys; a quantized key token
// t of group g scores n16_t * sum_d Hq[d] * (s16_g[d] * c_td + z16_g[d]),
// evaluated as n16_t * (sum_d q'_d c_td + Z_g) with q' = Hq * s16_g and
// Z_g = Hq . z16_g formed once per group; values dequantize as
// vs16_t * c + vz16_t, so the weighted value sum is
// sum_t (p_t vs16_t) c_t + sum_t p_t vz16_t.  Tokens of the bf16 tail score
// q . k_t on their stored values.
//
// Both contractions over the codes run on the matrix cores as exact integer
// products (v_mfma_i32_16x16x64_i8): the 2-bit codes are spread to int8 with
// one mask per four codes (the code's bit position becomes a power-of-two
// weight 1, 4 or 16 that is divided out of the other operand), and the fp32
// operand (q' for the scores, p * vs for the values) is written as a 32-bit
// fixed-point integer with a per-group power-of-two scale and split into four
// signed base-256 digits, one matrix row per (head, digit).  The int32 results
// are recombined exactly and scaled back, so the only rounding is the 2^-26
// relative fixed-point step of q' and p * vs.
//
// Work split: grid (split, KV head, sequence); one 8-wave workgroup per
// compute unit; the waves claim the split's 128-token groups one at a time
// (prefetching the next group's bytes while computing the current one) and
// keep a base-2 online softmax each.  Lane
// roles inside a wave (lane = 16 * r + n, w = n >> 1, u = 2 (n & 1)):
//  * score / softmax lane (r, n): head r of the row block, the tokens
//    16w + 4b + u + c of the group (b = 0..3, c = 0..1; column n of tile
//    4c + b);
//  * q' lane (r, n): head r, the channels 16w + 4b + u + c;
//  * value lane (r, n): head r, channels 16j + n of channel tile j.
// With these sets, the four digits of the values a lane owns for one c land
// in four consecutive bytes of one MFMA operand row, so each lane stages
// its operand bytes with one 8-byte LDS write per digit row.
// The waves merge in LDS into one partial record per split; merge.hip
// combines the splits.
#include "decode_common.hpp"

namespace oscar {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// After the spread (spread_codes) the code at bit position 2r of its byte
// carries the weight 4^r (masks 0x03, 0x0C, 0x30, 0xC0); the other operand
// is multiplied by 64 / 4^r so that every code ends up with weight 64.
__device__ constexpr float kFac[4] = {64.f, 16.f, 4.f, 1.f};

// 16 packed codes (bits 2k..2k+1 = code k) -> 16 int8 lanes of an MFMA
// operand.  Byte b of output dword r holds code 4b + r times 4^r; the top
// field is flipped into int8 range, 64 * code - 128, and the -128 is
// cancelled by the accumulator's start value (field3_bias).
__device__ __forceinline__ v4i spread_codes(uint32_t x) {
  v4i o;
  o[0] = static_cast<int>(x & 0x03030303u);
  o[1] = static_cast<int>(x & 0x0C0C0C0Cu);
  o[2] = static_cast<int>(x & 0x30303030u);
  o[3] = static_cast<int>((x & 0xC0C0C0C0u) ^ 0x80808080u);
  return o;
}

// 128 * (sum of the A operand over the K positions that carry top-field
// codes), the start value that cancels the -128 offset of spread_codes in a
// two-step (K = 128) product with A halves a0, a1.
__device__ __forceinline__ v4i field3_bias(const v4i& a0, const v4i& a1) {
  const v4i b64 = {0, 0, 0, 0x40404040};   // 64 at the top-field positions
  v4i c = {0, 0, 0, 0};
  c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b64, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b64, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b64, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b64, c, 0, 0, 0);
  return c;
}

// Four signed base-256 digits of an integer v, |v| < 2^31 - 2^24, given as
// v_off = v + 0x808080: digit k is byte k of the result read as int8
// (balanced representation).
__device__ __forceinline__ uint32_t balanced_digits_off(int v_off) {
  return static_cast<uint32_t>(v_off) ^ 0x808080u;
}

// An integer within one unit of y (|y| < 2^30), plus 0x808080, for
// balanced_digits_off.  The offset and the rounding half are added in fp32
// and the sum is truncated: round half up wherever the sum is positive.
__device__ __forceinline__ int fixed_off(float y) { return static_cast<int>(y + 8421504.5f); }

// 2^x for x <= 0 with the hardware exponential: results below 2^-126 flush
// to zero (negligible weights in a softmax); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum over the 16 lanes of a DPP row of non-negative floats (compared as
// their bit patterns, which order them).
__device__ __forceinline__ float row_max16_nonneg(float x) {
  int v = __float_as_int(x);
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppQuadXor1, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppQuadXor2, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppRowRor4, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppRowRor8, 0xF, 0xF, true));
  return __int_as_float(v);
}

// Maximum over the 16 lanes of a DPP row of floats that are not NaN: each
// float is mapped to an int with the same order (negative values have their
// magnitude bits flipped), reduced, and mapped back (the map is its own
// inverse).
__device__ __forceinline__ int float_order_key(int bits) { return bits ^ ((bits >> 31) & 0x7FFFFFFF); }
__device__ __forceinline__ float row_max16_ordered(float x) {
  int v = float_order_key(__float_as_int(x));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppQuadXor1, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppQuadXor2, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppRowRor4, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppRowRor8, 0xF, 0xF, true));
  return __int_as_float(float_order_key(v));
}

// Recombine the four digit rows of one (head, column) of an MFMA result.
__device__ __forceinline__ float digits_value(const v4i& c) {
  const int hi = c[3] * 256 + c[2];
  const int lo = c[1] * 256 + c[0];
  return fmaf(static_cast<float>(hi), 65536.f, static_cast<float>(lo));
}

struct GroupBytes {
  uint2 kd[8];     // K codes of token tau(4c+b) (see lane roles), dwords 2g and 2g+1 of the row
  uint2 vd[8];     // V codes of channel 16j + n, dwords 2g and 2g+1 of the channel row
  uint32_t nrm[4];  // fp16 norms of tokens 16w + 4b + u + {0, 1}
  uint2 vsz[4];     // (vs | vz << 16) of tokens 16w + 4b + u + {0, 1}
  uint2 ksz[4];     // (s | z << 16) of channels 16w + 4b + u + {0, 1}
};

// Bytes of group g needed by the score phase: key codes, norms, key scales
// and zero-points, value scales and zero-points (used by the softmax).
__device__ __forceinline__ void load_score_side(GroupBytes& r, const DecodeInt2Args& a, size_t slice, int groups_cap,
                                                int g, int lane) {
  const int gl = lane >> 4;
  const int n = lane & 15;
  const int base = 16 * (n >> 1) + 2 * (n & 1);   // token / channel 16w + u
  const size_t row0 = slice * a.capacity + static_cast<size_t>(g) * kGroup;   // first token row
  const size_t grp = slice * groups_cap + g;
  const uint8_t* kc = a.k_codes + (row0 + base) * 32 + 8 * gl;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.kd[i] = *reinterpret_cast<const uint2*>(kc + (4 * (i & 3) + (i >> 2)) * 32);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    r.nrm[b] = *reinterpret_cast<const uint32_t*>(a.k_norm + row0 + base + 4 * b);
    r.vsz[b] = *reinterpret_cast<const uint2*>(a.v_sz + (row0 + base + 4 * b) * 2);
    r.ksz[b] = *reinterpret_cast<const uint2*>(a.k_sz + (grp * kHeadDim + base + 4 * b) * 2);
  }
}

// Bytes of group g needed by the value phase: the value codes.
__device__ __forceinline__ void load_value_side(GroupBytes& r, const DecodeInt2Args& a, size_t slice, int groups_cap,
                                                int g, int lane) {
  const int gl = lane >> 4;
  const int n = lane & 15;
  const size_t grp = slice * groups_cap + g;
  const uint8_t* vc = a.v_codes + (grp * kHeadDim + n) * 32 + 8 * gl;
#pragma unroll
  for (int j = 0; j < 8; ++j) r.vd[j] = *reinterpret_cast<const uint2*>(vc + j * 16 * 32);
}

__device__ __forceinline__ uint32_t pick(const uint2& v, int c) { return c ? v.y : v.x; }
__device__ __forceinline__ float f16_lo(uint32_t w) { return f16_bits_to_f32(static_cast<uint16_t>(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return f16_bits_to_f32(static_cast<uint16_t>(w >> 16)); }

// 4x4 byte transpose: y[k] byte b = x[b] byte k.
__device__ __forceinline__ void transpose4(const uint32_t (&x)[4], uint32_t (&y)[4]) {
  const uint32_t t01_lo = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);
  const uint32_t t01_hi = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);
  const uint32_t t23_lo = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
  const uint32_t t23_hi = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
  y[0] = __builtin_amdgcn_perm(t23_lo, t01_lo, 0x05040100u);
  y[1] = __builtin_amdgcn_perm(t23_lo, t01_lo, 0x07060302u);
  y[2] = __builtin_amdgcn_perm(t23_hi, t01_hi, 0x05040100u);
  y[3] = __builtin_amdgcn_perm(t23_hi, t01_hi, 0x07060302u);
}

// MFMA A operand staging: per (operand half or K step, lane group) a block of
// 16 rows x 16 bytes plus 16 bytes of padding, so that the 8-byte writes of
// a wave spread over all LDS banks.
constexpr int kOpRow = 16;
constexpr int kOpBlock = 16 * kOpRow + 16;

// Write the digit rows of the eight fixed-point values x[c][b] a lane owns
// (c = 0..1, b = 0..3) into operand block `blk` (a pointer to [2][4][kOpBlock]).
__device__ __forceinline__ void stage_digits(uint8_t* blk, const uint32_t (&x)[2][4], int gl, int n) {
  uint32_t y0[4], y1[4];
  transpose4(x[0], y0);
  transpose4(x[1], y1);
  const int w = n >> 1;
  uint8_t* dst = blk + ((w & 1) * 4 + (w >> 1)) * kOpBlock + 8 * (n & 1);
#pragma unroll
  for (int k = 0; k < 4; ++k) *reinterpret_cast<uint2*>(dst + (4 * gl + k) * kOpRow) = make_uint2(y0[k], y1[k]);
}

__device__ __forceinline__ v4i read_operand(const uint8_t* blk, int half, int gl, int n) {
  return *reinterpret_cast<const v4i*>(blk + (half * 4 + gl) * kOpBlock + n * kOpRow);
}

// Query set-up by one wave.  Lane l holds, for row block rb, the elements
// 8 (l % 16) .. 8 (l % 16) + 7 of head 4 rb + l / 16 (zero for heads >= G).
template <int G, int RB>
__device__ __forceinline__ void fetch_q_wave(const uint16_t* q, int lane, uint4 (&raw)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int head = 4 * rb + (lane >> 4);
    const uint4 v = reinterpret_cast<const uint4*>(q)[head < G ? 16 * head + (lane & 15) : 0];
    raw[rb] = (head < G) ? v : make_uint4(0u, 0u, 0u, 0u);
  }
}

// q_raw = q * scale and q_rot = (H q) * scale, H the orthonormal Sylvester
// Hadamard matrix of order 128 in natural order: butterflies (x, y) ->
// (x + y, x - y) over index pairs differing in one bit, the three low bits
// inside a lane, the four high bits across the 16 lanes of a row.
template <int RB>
__device__ __forceinline__ void rotate_q_wave(const uint4 (&raw)[RB], float scale, float (*q_raw)[kHeadDim],
                                              float (*q_rot)[kHeadDim], int lane) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = 4 * rb + (lane >> 4);
    const int d0 = 8 * (lane & 15);
    const uint32_t w[4] = {raw[rb].x, raw[rb].y, raw[rb].z, raw[rb].w};
    float x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16lo_to_f32(w[k]);
      x[2 * k + 1] = bf16hi_to_f32(w[k]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) q_raw[row][d0 + j] = x[j] * scale;
#pragma unroll
    for (int bit = 1; bit < 8; bit <<= 1)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (!(j & bit)) {
          const float a = x[j], b = x[j | bit];
          x[j] = a + b;
          x[j | bit] = a - b;
        }
#pragma unroll
    for (int lb = 1; lb < 16; lb <<= 1) {
      const bool upper = lane & lb;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float y = __shfl_xor(x[j], lb, kWave);
        x[j] = upper ? y - x[j] : x[j] + y;
      }
    }
    const float norm = scale * 0.088388347648318440550f;   // 1/sqrt(128)
#pragma unroll
    for (int j = 0; j < 8; ++j) q_rot[row][d0 + j] = x[j] * norm;
  }
}

template <int G>
struct Int2Cfg {
  static constexpr int kRB = (G + 3) / 4;  // 16-row blocks of (head, digit) rows
  static constexpr int kRows = kRB * 4;    // heads incl. zero padding
  // One workgroup per compute unit: 12 waves (3 per SIMD) while the kernel
  // fits in 168 VGPRs, 8 waves for 8 query heads per KV head.
  static constexpr int kWaves = (kRB == 1) ? 12 : 8;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kSlots = kWaves + 1;  // waves + the bf16-tail state
};

template <int G>
struct Int2Smem {
  float q_raw[Int2Cfg<G>::kRows][kHeadDim];   // q * sm_scale * log2(e)
  float q_rot[Int2Cfg<G>::kRows][kHeadDim];   // (H q) * sm_scale * log2(e)
  float tail_p[G][kGroup];                     // softmax weights of the bf16 tail tokens
  // per wave and row block: MFMA A operands staged as [half][lane group][row][16 bytes]
  uint8_t a_qk[Int2Cfg<G>::kWaves][Int2Cfg<G>::kRB][2 * 4 * kOpBlock];
  uint8_t a_pv[Int2Cfg<G>::kWaves][Int2Cfg<G>::kRB][2 * 4 * kOpBlock];
  MergeSmem<G, Int2Cfg<G>::kSlots> merge;
  int next_group;   // next group of this split not yet claimed by a wave
  int q_ready;      // set by wave 0 once q_raw, q_rot, next_group and the tail slot are written
};

// Running softmax state of one wave: per row block, m (uniform over the
// head's 16 lanes), per-lane partial l and sum p * vz, and acc for channels
// 16j + n.
template <int RB>
struct WaveRun {
  float m[RB], l[RB], z[RB], acc[RB][8];
};

// Score phase of one quantized 128-token group: scores on the matrix cores,
// online softmax update, p * vs staged as the value phase's A operand.
// Returns the softmax rescale factors in alpha and inv_p.
template <int G>
__device__ __forceinline__ void score_phase(const GroupBytes& cur, int t0, int t_end,
                                            const float (&qv)[Int2Cfg<G>::kRB][2][4], const float (&fac)[2],
                                            Int2Smem<G>& sm, WaveRun<Int2Cfg<G>::kRB>& st, int wave, int gl, int n,
                                            float (&alpha)[Int2Cfg<G>::kRB], float (&inv_p)[Int2Cfg<G>::kRB]) {
  constexpr int RB = Int2Cfg<G>::kRB;
  const int tok_base = t0 + 16 * (n >> 1) + 2 * (n & 1);
  // ---- q' = Hq * s16 as 4-digit fixed point (A operand), Z = Hq . z16 ----
  float Zg[RB], inv_q[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float qs[2][4];
    float zp = 0.f, amax = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint32_t w = pick(cur.ksz[b], c);
        qs[c][b] = fmaf(qv[rb][c][b], f16_lo(w), 0.f);   // one mixed-precision FMA
        zp = fmaf(qv[rb][c][b], f16_hi(w), zp);
        amax = fmaxf(amax, fabsf(qs[c][b]));
      }
    amax = row_max16_nonneg(amax);
    Zg[rb] = row_sum16(zp);
    int e;
    frexpf(amax, &e);                        // amax < 2^e
    const float sc = ldexpf(1.f, 24 - e);    // |q' * sc| < 2^24, |q' * sc * fac| < 2^30
    inv_q[rb] = ldexpf(1.f, e - 30);         // 1 / (sc * 64)
    uint32_t x[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < 4; ++b) x[c][b] = balanced_digits_off(fixed_off(qs[c][b] * (sc * fac[c])));
    stage_digits(sm.a_qk[wave][rb], x, gl, n);
  }
  wave_sync_lds();
  v4i aq[RB][2], bias[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    aq[rb][0] = read_operand(sm.a_qk[wave][rb], 0, gl, n);
    aq[rb][1] = read_operand(sm.a_qk[wave][rb], 1, gl, n);
    bias[rb] = field3_bias(aq[rb][0], aq[rb][1]);
  }

  // ---- scores: column n of tile i = 4c + b is token 16w + 4b + u + c ----
  float logit[RB][2][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = i >> 2, b = i & 3;
    const v4i b0 = spread_codes(cur.kd[i].x);
    const v4i b1 = spread_codes(cur.kd[i].y);
    const float n16 = c ? f16_hi(cur.nrm[b]) : f16_lo(cur.nrm[b]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[rb][0], b0, bias[rb], 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[rb][1], b1, acc, 0, 0, 0);
      logit[rb][c][b] = fmaf(fmaf(digits_value(acc), inv_q[rb], Zg[rb]), n16, 0.f);
    }
  }
  if (t0 + kGroup > t_end) {   // a group cut short by max_tokens: mask the tokens beyond it
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i >> 2, b = i & 3;
      const bool valid = tok_base + 4 * b + c < t_end;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) logit[rb][c][b] = valid ? logit[rb][c][b] : -INFINITY;
    }
  }

  // ---- online softmax (base 2) and p * vs as 4-digit fixed point ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float gm = logit[rb][0][0];
#pragma unroll
    for (int i = 1; i < 8; ++i) gm = fmaxf(gm, logit[rb][i >> 2][i & 3]);
    gm = row_max16_ordered(gm);
    const float m_new = (gm > st.m[rb]) ? gm : st.m[rb];   // finite: every group has a valid token
    alpha[rb] = fast_exp2(st.m[rb] - m_new);   // 0 while m was -inf
    st.m[rb] = m_new;
    float ls = 0.f, zs = 0.f, pmax = 0.f;
    float pv[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t w = pick(cur.vsz[b], c);
        const float p = fast_exp2(logit[rb][c][b] - m_new);
        ls += p;
        zs = fmaf(p, f16_hi(w), zs);
        pv[c][b] = fmaf(p, f16_lo(w), 0.f);
        pmax = fmaxf(pmax, pv[c][b]);
      }
    st.l[rb] = fmaf(st.l[rb], alpha[rb], ls);
    st.z[rb] = fmaf(st.z[rb], alpha[rb], zs);
    pmax = row_max16_nonneg(pmax);
    int e2;
    frexpf(pmax, &e2);                       // p * vs < 2^e2 for this head and group
    const float sc2 = ldexpf(1.f, 24 - e2);
    inv_p[rb] = ldexpf(1.f, e2 - 30);
    uint32_t x[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < 4; ++b) x[c][b] = balanced_digits_off(fixed_off(pv[c][b] * (sc2 * fac[c])));
    stage_digits(sm.a_pv[wave][rb], x, gl, n);
  }
}

// Value phase: weighted value codes on the matrix cores (channel tile j,
// column n = channel 16j + n), folded into the running accumulators.
template <int G>
__device__ __forceinline__ void value_phase(const GroupBytes& cur, Int2Smem<G>& sm, WaveRun<Int2Cfg<G>::kRB>& st,
                                            int wave, int gl, int n, const float (&alpha)[Int2Cfg<G>::kRB],
                                            const float (&inv_p)[Int2Cfg<G>::kRB]) {
  constexpr int RB = Int2Cfg<G>::kRB;
  wave_sync_lds();
  v4i ap[RB][2], bias[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    ap[rb][0] = read_operand(sm.a_pv[wave][rb], 0, gl, n);
    ap[rb][1] = read_operand(sm.a_pv[wave][rb], 1, gl, n);
    bias[rb] = field3_bias(ap[rb][0], ap[rb][1]);
  }

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const v4i b0 = spread_codes(cur.vd[j].x);
    const v4i b1 = spread_codes(cur.vd[j].y);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ap[rb][0], b0, bias[rb], 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ap[rb][1], b1, acc, 0, 0, 0);
      st.acc[rb][j] = fmaf(digits_value(acc), inv_p[rb], st.acc[rb][j] * alpha[rb]);
    }
  }
  // the next group rewrites a_qk / a_pv only after this wave has read them
  wave_sync_lds();
}

template <int G>
__global__ __launch_bounds__(Int2Cfg<G>::kThreads) void decode_int2_kernel(DecodeInt2Args a) {
  using C = Int2Cfg<G>;
  constexpr int RB = C::kRB;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int gl = lane >> 4;   // lane group: head of the row block / operand K slice
  const int n = lane & 15;

  __shared__ Int2Smem<G> sm;

  const int groups_cap = a.capacity / kGroup;
  int nq = a.n_quant[b];
  int nt = a.n_tail[b];
  nq = min(max(nq, 0) & ~(kGroup - 1), a.capacity);
  nt = min(max(nt, 0), kGroup - 1);
  if (a.k_tail == nullptr || a.v_tail == nullptr) nt = 0;
  const int total = min(nq + nt, a.max_tokens);
  // Split s owns the groups s, s + S, s + 2S, ... (S = number of splits):
  // at any moment the workgroups of a head read neighbouring groups, which
  // spreads the traffic over all memory channels.
  const int S = a.splits;
  const int n_groups = (total + kGroup - 1) / kGroup;
  const size_t slice = static_cast<size_t>(b) * a.num_kv_heads + h;
  const int qh0 = h * G;

  const int g_qend = min(n_groups, nq / kGroup);   // quantized groups end here; a tail group may follow
  int g = split + wave * S;
  // Wave 0 requests the query before any wave requests cache bytes (the
  // barrier orders the requests of the compute unit).  It then sets up the
  // query and the shared state and raises q_ready before requesting its own
  // first group, while the other waves request their first groups at once
  // and wait for q_ready only afterwards: no wave's start waits for another
  // wave's cache requests to be accepted.
  uint4 q_in[RB];
  if (wave == 0) fetch_q_wave<G, RB>(a.q + (static_cast<size_t>(b) * a.num_q_heads + qh0) * kHeadDim, lane, q_in);
  if (tid == 0) sm.q_ready = 0;
  __syncthreads();
  const int g_first = (g < g_qend) ? g : 0;
  GroupBytes cur;
  if (wave == 0) {
    rotate_q_wave<RB>(q_in, a.sm_scale * kLog2e, sm.q_raw, sm.q_rot, lane);
    clear_slot(sm.merge, C::kWaves);  // the tail slot stays empty unless a tail is seen
    if (lane == 0) sm.next_group = C::kWaves;   // next group index k (group split + k S)
    // every lane releases its own writes
    __hip_atomic_store(&sm.q_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  // The first group's loads are issued without a branch on the group (a wave
  // without a group reads group 0 of its slice, which always exists, and
  // ignores it), so that later waits count exactly the loads issued.
  load_score_side(cur, a, slice, groups_cap, g_first, lane);
  load_value_side(cur, a, slice, groups_cap, g_first, lane);
  while (__hip_atomic_load(&sm.q_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
    __builtin_amdgcn_s_sleep(1);

  // rotated query of this lane's head and channels 16w + 4b + u + c, per row block
  float qv[RB][2][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < 4; ++b) qv[rb][c][b] = sm.q_rot[rb * 4 + gl][16 * (n >> 1) + 4 * b + 2 * (n & 1) + c];
  // weight divisors of the bit pairs u + c this lane's values occupy
  const float fac[2] = {kFac[2 * (n & 1)], kFac[2 * (n & 1) + 1]};

  WaveRun<RB> st;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    st.m[rb] = -INFINITY;
    st.l[rb] = 0.f;
    st.z[rb] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[rb][j] = 0.f;
  }

  // Groups are handed out dynamically: each wave starts with the split's
  // group number `wave` and then claims the next unclaimed one,
  // so waves that get fewer issue slots simply process fewer groups.  One
  // register set per wave: the next group's score-side bytes are requested
  // as soon as the score phase has consumed the current ones, its value
  // codes as soon as the value phase has.
  while (g < g_qend) {
    float alpha[RB], inv_p[RB];
    score_phase<G>(cur, g * kGroup, total, qv, fac, sm, st, wave, gl, n, alpha, inv_p);
    int k_next = 0;
    if (lane == 0) k_next = atomicAdd(&sm.next_group, 1);
    const int g_next = split + __builtin_amdgcn_readfirstlane(k_next) * S;
    if (g_next < g_qend) load_score_side(cur, a, slice, groups_cap, g_next, lane);
    value_phase<G>(cur, sm, st, wave, gl, n, alpha, inv_p);
    if (g_next < g_qend) load_value_side(cur, a, slice, groups_cap, g_next, lane);
    g = g_next;
  }

  // ---- this wave's state -> merge slot ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = row_sum16(st.l[rb]);
    const float z_tot = row_sum16(st.z[rb]);
    const int hh = rb * 4 + gl;
    if (hh < G) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.merge.acc[wave][hh][16 * j + n] = st.acc[rb][j] + z_tot;
      if (n == 0) {
        sm.merge.m[wave][hh] = st.m[rb];
        sm.merge.l[wave][hh] = l_tot;
      }
    }
  }

  // ---- the bf16 tail (at most one partial group, after the quantized ones) ----
  const int g_tail = nq / kGroup;
  if (nt > 0 && g_tail < n_groups && g_tail % S == split && wave == (g_tail / S) % C::kWaves) {
    const int n_tok = min(nt, total - g_tail * kGroup);
    bf16_tokens_wave<G, C::kSlots>(a.k_tail + slice * kGroup * kHeadDim, a.v_tail + slice * kGroup * kHeadDim,
                                   n_tok, sm.q_raw, sm.tail_p, sm.merge, C::kWaves);
  }

  const size_t partial_base = (static_cast<size_t>(b) * a.num_q_heads + qh0) * a.splits;
  write_partial<G, C::kSlots>(sm.merge, a.partials, partial_base, split, a.splits);
}

template <int G>
hipError_t launch_g(const DecodeInt2Args& a, int32_t batch, hipStream_t s) {
  dim3 grid(a.splits, a.num_kv_heads, batch);
  hipLaunchKernelGGL(decode_int2_kernel<G>, grid, dim3(Int2Cfg<G>::kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_int2(const DecodeInt2Args& a, int32_t batch, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<1>(a, batch, s);
    case 2: return launch_g<2>(a, batch, s);
    case 4: return launch_g<4>(a, batch, s);
    case 8: return launch_g<8>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
