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
// Work split: grid (split, KV head, sequence); 4 waves per workgroup; each
// wave streams whole 128-token groups (prefetching the next group's bytes
// while computing the current one) with a base-2 online softmax.  Lane
// roles inside a wave (lane = 16 * r + n):
//  * score / softmax lane (r, n): head r of the row block, tokens 8n .. 8n+7
//    of the group (one per 16-token column tile i, token 8n + i);
//  * q' lane (r, n): head r, channels 8n .. 8n+7;
//  * value lane (r, n): head r, channels 16j + n of channel tile j.
// The waves merge in LDS into one partial record per split; merge.hip
// combines the splits.
#include "decode_common.hpp"

namespace oscar {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// 16 / (weight of a code at bit position 2r of its byte after the spread):
// r = 0 -> mask 0x03 (weight 1), r = 1 -> 0x0C (4), r = 2 -> 0x30 (16),
// r = 3 -> shifted down by 6 (weight 1).
__device__ constexpr float kInvWeight16[4] = {16.f, 4.f, 1.f, 16.f};

// 16 packed codes (bits 2k..2k+1 = code k) -> 16 int8 lanes of an MFMA
// operand.  Byte b of output dword r holds code 4b + r times its weight.
__device__ __forceinline__ v4i spread_codes(uint32_t x) {
  v4i o;
  o[0] = static_cast<int>(x & 0x03030303u);
  o[1] = static_cast<int>(x & 0x0C0C0C0Cu);
  o[2] = static_cast<int>(x & 0x30303030u);
  o[3] = static_cast<int>((x >> 6) & 0x03030303u);
  return o;
}

// Four signed base-256 digits of |v| < 2^31 - 2^24: digit k is byte k of the
// result read as int8 (balanced representation).
__device__ __forceinline__ uint32_t balanced_digits(int v) {
  return static_cast<uint32_t>(v + 0x808080) ^ 0x808080u;
}

// Recombine the four digit rows of one (head, column) of an MFMA result.
__device__ __forceinline__ float digits_value(const v4i& c) {
  const int hi = c[3] * 256 + c[2];
  const int lo = c[1] * 256 + c[0];
  return fmaf(static_cast<float>(hi), 65536.f, static_cast<float>(lo));
}

struct GroupBytes {
  uint2 kd[8];    // K codes of token 8n + i, dwords 2g and 2g+1 of the row (g = lane >> 4)
  uint2 vd[8];    // V codes of channel 16j + n, dwords 2g and 2g+1 of the channel row
  uint4 norm;     // fp16 norms of tokens 8n .. 8n+7
  uint4 vsz[2];   // (vs, vz) fp16 pairs of tokens 8n .. 8n+7
  uint4 ksz[2];   // (s, z) fp16 pairs of channels 8n .. 8n+7
};

__device__ __forceinline__ void load_group(GroupBytes& r, const DecodeInt2Args& a, size_t slice, int groups_cap,
                                           int g, int lane) {
  const int gl = lane >> 4;
  const int n = lane & 15;
  const size_t row0 = slice * a.capacity + static_cast<size_t>(g) * kGroup;   // first token row
  const size_t grp = slice * groups_cap + g;
  const uint8_t* kc = a.k_codes + (row0 + 8 * n) * 32 + 8 * gl;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.kd[i] = *reinterpret_cast<const uint2*>(kc + i * 32);
  const uint8_t* vc = a.v_codes + (grp * kHeadDim + n) * 32 + 8 * gl;
#pragma unroll
  for (int j = 0; j < 8; ++j) r.vd[j] = *reinterpret_cast<const uint2*>(vc + j * 16 * 32);
  r.norm = *reinterpret_cast<const uint4*>(a.k_norm + row0 + 8 * n);
  const uint4* vs = reinterpret_cast<const uint4*>(a.v_sz + (row0 + 8 * n) * 2);
  r.vsz[0] = vs[0];
  r.vsz[1] = vs[1];
  const uint4* ks = reinterpret_cast<const uint4*>(a.k_sz + (grp * kHeadDim + 8 * n) * 2);
  r.ksz[0] = ks[0];
  r.ksz[1] = ks[1];
}

__device__ __forceinline__ uint32_t word8(const uint4 (&w)[2], int j) {
  const uint4 x = w[j >> 2];
  switch (j & 3) {
    case 0: return x.x;
    case 1: return x.y;
    case 2: return x.z;
    default: return x.w;
  }
}
__device__ __forceinline__ uint32_t half8(const uint4& w, int i) {  // fp16 i of 8 packed in a uint4
  const uint32_t x = (i >> 1) == 0 ? w.x : (i >> 1) == 1 ? w.y : (i >> 1) == 2 ? w.z : w.w;
  return (i & 1) ? (x >> 16) : (x & 0xffffu);
}

template <int G>
struct Int2Cfg {
  static constexpr int kRB = (G + 3) / 4;  // 16-row blocks of (head, digit) rows
  static constexpr int kRows = kRB * 4;    // heads incl. zero padding
  static constexpr int kSlots = kDecodeWaves + 1;  // waves + the bf16-tail state
};

template <int G>
struct Int2Smem {
  float q_raw[Int2Cfg<G>::kRows][kHeadDim];   // q * sm_scale * log2(e)
  union {
    float q_rot[Int2Cfg<G>::kRows][kHeadDim];  // (H q) * sm_scale * log2(e); read once at the start
    float tail_p[G][kGroup];                    // softmax weights of the bf16 tail tokens
  } u;
  // per wave and row block: MFMA A operands staged as [half][lane group][row][16 bytes]
  uint8_t a_qk[kDecodeWaves][Int2Cfg<G>::kRB][2][4][16][16];
  uint8_t a_pv[kDecodeWaves][Int2Cfg<G>::kRB][2][4][16][16];
  MergeSmem<G, Int2Cfg<G>::kSlots> merge;
};

template <int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_int2_kernel(DecodeInt2Args a) {
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
  const int t_begin = split * a.tokens_per_split;
  const int t_end = min(t_begin + a.tokens_per_split, total);
  const size_t slice = static_cast<size_t>(b) * a.num_kv_heads + h;
  const int qh0 = h * G;

  if (wave == 0) clear_slot(sm.merge, kDecodeWaves);  // the tail slot stays empty unless a tail is seen
  load_and_rotate_q<G, C::kRows>(a.q + (static_cast<size_t>(b) * a.num_q_heads + qh0) * kHeadDim,
                                 a.sm_scale * kLog2e, sm.q_raw, sm.u.q_rot);

  // rotated query of this lane's head and channels 8n .. 8n+7, per row block
  float qv[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[rb][j] = sm.u.q_rot[rb * 4 + gl][8 * n + j];
  __syncthreads();  // q_rot shares storage with tail_p

  float m_run[RB], l_run[RB], z_run[RB], acc[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
    z_run[rb] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[rb][j] = 0.f;
  }

  const int g_begin = t_begin / kGroup;
  const int g_end = (t_end + kGroup - 1) / kGroup;
  const int g_qend = min(g_end, nq / kGroup);   // quantized groups end here; a tail group may follow
  int g = g_begin + wave;
  GroupBytes cur, nxt;
  if (g < g_qend) load_group(cur, a, slice, groups_cap, g, lane);
  for (; g < g_qend; g += kDecodeWaves) {
    const int g_next = g + kDecodeWaves;
    if (g_next < g_qend) load_group(nxt, a, slice, groups_cap, g_next, lane);
    const int t0 = g * kGroup;

    // ---- q' = Hq * s16 as 4-digit fixed point (A operand), Z = Hq . z16 ----
    float Zg[RB], inv_q[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float qs[8];
      float zp = 0.f, amax = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w = word8(cur.ksz, j);
        const float s = f16_bits_to_f32(static_cast<uint16_t>(w & 0xffffu));
        const float z = f16_bits_to_f32(static_cast<uint16_t>(w >> 16));
        qs[j] = qv[rb][j] * s;
        zp = fmaf(qv[rb][j], z, zp);
        amax = fmaxf(amax, fabsf(qs[j]));
      }
      amax = row_max16(amax);
      Zg[rb] = row_sum16(zp);
      int e;
      frexpf(amax, &e);                        // amax < 2^e
      const float sc = ldexpf(1.f, 26 - e);    // |q' * sc| < 2^26
      inv_q[rb] = ldexpf(1.f, e - 30);         // 1 / (sc * 16)
      uint8_t(*dst)[4][16][16] = sm.a_qk[wave][rb];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t dg = balanced_digits(static_cast<int>(qs[j] * (sc * kInvWeight16[j & 3])));
        // channel 8n + j sits in packed dword w = n >> 1 (operand half w & 1,
        // lane group w >> 1), byte 2 (n & 1) + (j >> 2), bit pair j & 3, i.e.
        // operand byte 4 (j & 3) + 2 (n & 1) + (j >> 2).
        const int half = (n >> 1) & 1, g4 = n >> 2, p = 4 * (j & 3) + 2 * (n & 1) + (j >> 2);
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[half][g4][4 * gl + k][p] = static_cast<uint8_t>(dg >> (8 * k));
      }
    }
    wave_sync_lds();
    v4i aq[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      aq[rb][0] = *reinterpret_cast<const v4i*>(sm.a_qk[wave][rb][0][gl][n]);
      aq[rb][1] = *reinterpret_cast<const v4i*>(sm.a_qk[wave][rb][1][gl][n]);
    }

    // ---- scores of tokens 8n + i (column n of tile i) ----
    float logit[RB][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const v4i b0 = spread_codes(cur.kd[i].x);
      const v4i b1 = spread_codes(cur.kd[i].y);
      const float n16 = f16_bits_to_f32(static_cast<uint16_t>(half8(cur.norm, i)));
      const bool valid = t0 + 8 * n + i < t_end;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        v4i c = {0, 0, 0, 0};
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[rb][0], b0, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[rb][1], b1, c, 0, 0, 0);
        logit[rb][i] = valid ? n16 * fmaf(digits_value(c), inv_q[rb], Zg[rb]) : -INFINITY;
      }
    }

    // ---- online softmax (base 2) and p * vs as 4-digit fixed point ----
    float vs[8], vz[8], vmax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = word8(cur.vsz, i);
      vs[i] = f16_bits_to_f32(static_cast<uint16_t>(w & 0xffffu));
      vz[i] = f16_bits_to_f32(static_cast<uint16_t>(w >> 16));
      vmax = fmaxf(vmax, vs[i]);
    }
    vmax = row_max16(vmax);
    int e2;
    frexpf(vmax, &e2);
    const float sc2 = ldexpf(1.f, 26 - e2);
    const float inv2 = ldexpf(1.f, e2 - 30);
    float alpha[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float gm = logit[rb][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) gm = fmaxf(gm, logit[rb][i]);
      gm = row_max16(gm);
      const float m_new = fmaxf(m_run[rb], gm);   // finite: every group has a valid token
      alpha[rb] = (m_run[rb] == -INFINITY) ? 0.f : exp2f(m_run[rb] - m_new);
      m_run[rb] = m_new;
      float ls = 0.f, zs = 0.f;
      uint8_t(*dst)[4][16][16] = sm.a_pv[wave][rb];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = exp2f(logit[rb][i] - m_new);
        ls += p;
        zs = fmaf(p, vz[i], zs);
        const uint32_t dg = balanced_digits(static_cast<int>(p * vs[i] * (sc2 * kInvWeight16[i & 3])));
        // token 8n + i sits in packed dword w = n >> 1 of its channel row
        // (K step w & 1, lane group w >> 1), byte 2 (n & 1) + (i >> 2), bit pair i & 3.
        const int ks = (n >> 1) & 1, g4 = n >> 2, p4 = 4 * (i & 3) + 2 * (n & 1) + (i >> 2);
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[ks][g4][4 * gl + k][p4] = static_cast<uint8_t>(dg >> (8 * k));
      }
      l_run[rb] = fmaf(l_run[rb], alpha[rb], ls);
      z_run[rb] = fmaf(z_run[rb], alpha[rb], zs);
    }
    wave_sync_lds();
    v4i ap[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      ap[rb][0] = *reinterpret_cast<const v4i*>(sm.a_pv[wave][rb][0][gl][n]);
      ap[rb][1] = *reinterpret_cast<const v4i*>(sm.a_pv[wave][rb][1][gl][n]);
    }

    // ---- weighted value codes: channel tile j, column n = channel 16j + n ----
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const v4i b0 = spread_codes(cur.vd[j].x);
      const v4i b1 = spread_codes(cur.vd[j].y);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        v4i c = {0, 0, 0, 0};
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(ap[rb][0], b0, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(ap[rb][1], b1, c, 0, 0, 0);
        acc[rb][j] = fmaf(digits_value(c), inv2, acc[rb][j] * alpha[rb]);
      }
    }
    if (g_next < g_qend) cur = nxt;
  }

  // ---- this wave's state -> merge slot ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = row_sum16(l_run[rb]);
    const float z_tot = row_sum16(z_run[rb]);
    const int hh = rb * 4 + gl;
    if (hh < G) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.merge.acc[wave][hh][16 * j + n] = acc[rb][j] + z_tot;
      if (n == 0) {
        sm.merge.m[wave][hh] = m_run[rb];
        sm.merge.l[wave][hh] = l_tot;
      }
    }
  }

  // ---- the bf16 tail (at most one partial group, after the quantized ones) ----
  const int g_tail = nq / kGroup;
  if (nt > 0 && g_tail >= g_begin && g_tail < g_end && wave == (g_tail - g_begin) % kDecodeWaves) {
    const int n_tok = min(nt, t_end - g_tail * kGroup);
    bf16_tokens_wave<G, C::kSlots>(a.k_tail + slice * kGroup * kHeadDim, a.v_tail + slice * kGroup * kHeadDim,
                                   n_tok, sm.q_raw, sm.u.tail_p, sm.merge, kDecodeWaves);
  }

  const size_t partial_base = (static_cast<size_t>(b) * a.num_q_heads + qh0) * a.splits;
  write_partial<G, C::kSlots>(sm.merge, a.partials, partial_base, split, a.splits);
}

template <int G>
hipError_t launch_g(const DecodeInt2Args& a, int32_t batch, hipStream_t s) {
  dim3 grid(a.splits, a.num_kv_heads, batch);
  hipLaunchKernelGGL(decode_int2_kernel<G>, grid, dim3(kDecodeThreads), 0, s, a);
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
