// Single-query GQA decode attention over the packed OScaR INT2 cache.
//
// What is computed (OScaR abstract, arXiv 2605.19660; ai-papers.net OScaR
// summary, sections "OScaRの提案手法" and "実験結果"): the query is rotated once
// by the same orthonormal Hadamard matrix as the keys; a quantized key token
// t of group g scores n16_t * sum_d Hq[d] * (s16_g[d] * c_td + z16_g[d]),
// which is evaluated as n16_t * (sum_d q'_d c_td + Z_g) with q' = Hq * s16_g
// and Z_g = Hq . z16_g formed once per group; tail tokens score q . k_t on
// their bf16 values.  Values dequantize as vs16_t * c + vz16_t, so the
// weighted sum is sum_t (p_t vs16_t) c_t + sum_t p_t vz16_t.
//
// Structure: grid (split, KV head, sequence), 4 waves per workgroup, each
// wave streams whole 128-token groups of the split with an online softmax
// (base 2); the waves merge in LDS and the last workgroup of each
// (sequence, KV head) merges the splits (decode_common.hpp).
//
// This version does the dot products on the VALU in fp32: lane = token for
// the scores, lane = channel pair for the value accumulation.
#include "decode_common.hpp"

namespace oscar {
namespace {

template <int G>
struct Int2Smem {
  float q_raw[G][kHeadDim];           // q * sm_scale * log2(e)
  float q_rot[G][kHeadDim];           // (H q) * sm_scale * log2(e)
  float qp[kDecodeWaves][G][kHeadDim];  // per wave: q' = q_rot * s16 of the current group
  float pv[kDecodeWaves][G][kGroup];    // per wave: p_t * vs16_t (or p_t for tail tokens)
  MergeSmem<G> merge;
};

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_int2_kernel(DecodeInt2Args a) {
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;

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
  load_and_rotate_q<G>(a.q + (static_cast<size_t>(b) * a.num_q_heads + qh0) * kHeadDim, a.sm_scale * kLog2e,
                       sm.q_raw, sm.q_rot);

  WaveState<G> st;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    st.m[hh] = -INFINITY;
    st.l[hh] = 0.f;
    st.acc[hh][0] = st.acc[hh][1] = 0.f;
  }

  const int g_begin = t_begin / kGroup;
  const int g_end = (t_end + kGroup - 1) / kGroup;  // t_end <= t_begin gives no groups
  for (int g = g_begin + wave; g < g_end; g += kDecodeWaves) {
    const int t0 = g * kGroup;
    const bool quant = t0 < nq;
    float logit[G][2];
    float vscale[2] = {1.f, 1.f};
    float vzero[2] = {0.f, 0.f};
    if (quant) {
      // --- fold the group's key scales into the query ---
      const uint2 sz = *reinterpret_cast<const uint2*>(a.k_sz + ((slice * groups_cap + g) * kHeadDim + 2 * lane) * 2);
      const float s0 = f16_bits_to_f32(sz.x & 0xffff), z0 = f16_bits_to_f32(sz.x >> 16);
      const float s1 = f16_bits_to_f32(sz.y & 0xffff), z1 = f16_bits_to_f32(sz.y >> 16);
      float Z[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float qa = sm.q_rot[hh][2 * lane], qb = sm.q_rot[hh][2 * lane + 1];
        sm.qp[wave][hh][2 * lane] = qa * s0;
        sm.qp[wave][hh][2 * lane + 1] = qb * s1;
        Z[hh] = wave_sum(qa * z0 + qb * z1);
      }
      wave_sync_lds();
      // --- scores: lane owns tokens t0 + lane and t0 + lane + 64 ---
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int t = t0 + lane + 64 * k;
        const size_t row = slice * a.capacity + t;
        const uint4* kr = reinterpret_cast<const uint4*>(a.k_codes + row * 32);
        const uint4 c0 = kr[0], c1 = kr[1];
        const uint32_t words[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float n16 = f16_bits_to_f32(a.k_norm[row]);
        const uint32_t vsz = reinterpret_cast<const uint32_t*>(a.v_sz)[row];
        vscale[k] = f16_bits_to_f32(vsz & 0xffff);
        vzero[k] = f16_bits_to_f32(vsz >> 16);
        float dot[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) dot[hh] = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float c = static_cast<float>((words[w] >> (2 * e)) & 3u);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) dot[hh] = fmaf(sm.qp[wave][hh][16 * w + e], c, dot[hh]);
          }
        }
        const bool valid = t < t_end && t >= t_begin;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) logit[hh][k] = valid ? n16 * (dot[hh] + Z[hh]) : -INFINITY;
      }
    } else {
      // --- bf16 tail tokens: exact q . k_t with the unrotated query ---
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int tt = lane + 64 * k;  // index inside the tail
        const int t = t0 + tt;
        const bool valid = tt < nt && t < t_end && t >= t_begin;
        float dot[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) dot[hh] = 0.f;
        if (valid) {
          const uint4* kr = reinterpret_cast<const uint4*>(a.k_tail + (slice * kGroup + tt) * kHeadDim);
#pragma unroll 4
          for (int c = 0; c < 16; ++c) {
            const uint4 w = kr[c];
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float k0 = bf16lo_to_f32(ws[e]), k1 = bf16hi_to_f32(ws[e]);
#pragma unroll
              for (int hh = 0; hh < G; ++hh) {
                dot[hh] = fmaf(sm.q_raw[hh][8 * c + 2 * e], k0, dot[hh]);
                dot[hh] = fmaf(sm.q_raw[hh][8 * c + 2 * e + 1], k1, dot[hh]);
              }
            }
          }
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) logit[hh][k] = valid ? dot[hh] : -INFINITY;
      }
    }
    // --- online softmax update (base 2) ---
    float alpha[G], zsum[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float gmax = wave_max(fmaxf(logit[hh][0], logit[hh][1]));
      const float m_new = fmaxf(st.m[hh], gmax);
      if (m_new == -INFINITY) {  // nothing valid yet (uniform across the wave)
        alpha[hh] = 1.f;
        zsum[hh] = 0.f;
        sm.pv[wave][hh][lane] = 0.f;
        sm.pv[wave][hh][lane + 64] = 0.f;
        continue;
      }
      alpha[hh] = (st.m[hh] == -INFINITY) ? 0.f : exp2f(st.m[hh] - m_new);
      const float p0 = exp2f(logit[hh][0] - m_new);  // -inf -> 0
      const float p1 = exp2f(logit[hh][1] - m_new);
      st.l[hh] = st.l[hh] * alpha[hh] + wave_sum(p0 + p1);
      st.m[hh] = m_new;
      zsum[hh] = wave_sum(p0 * vzero[0] + p1 * vzero[1]);
      sm.pv[wave][hh][lane] = p0 * vscale[0];
      sm.pv[wave][hh][lane + 64] = p1 * vscale[1];
    }
    wave_sync_lds();
    // --- value accumulation: lane owns channels 2*lane, 2*lane + 1 ---
    float add[G][2];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) add[hh][0] = add[hh][1] = 0.f;
    if (quant) {
      const uint8_t* vbase = a.v_codes + ((slice * groups_cap + g) * kHeadDim + 2 * lane) * 32;
      const uint4* r0 = reinterpret_cast<const uint4*>(vbase);
      const uint4* r1 = reinterpret_cast<const uint4*>(vbase + 32);
      const uint4 a0 = r0[0], a1 = r0[1], b0 = r1[0], b1 = r1[1];
      const uint32_t w0[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const uint32_t w1[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int w = 0; w < 8; ++w) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float c0 = static_cast<float>((w0[w] >> (2 * e)) & 3u);
          const float c1 = static_cast<float>((w1[w] >> (2 * e)) & 3u);
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            const float p = sm.pv[wave][hh][16 * w + e];
            add[hh][0] = fmaf(p, c0, add[hh][0]);
            add[hh][1] = fmaf(p, c1, add[hh][1]);
          }
        }
      }
    } else {
      const int n_valid = min(nt, kGroup);
      for (int tt = 0; tt < n_valid; ++tt) {
        const uint32_t vv = *reinterpret_cast<const uint32_t*>(a.v_tail + (slice * kGroup + tt) * kHeadDim + 2 * lane);
        const float v0 = bf16lo_to_f32(vv), v1 = bf16hi_to_f32(vv);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float p = sm.pv[wave][hh][tt];
          add[hh][0] = fmaf(p, v0, add[hh][0]);
          add[hh][1] = fmaf(p, v1, add[hh][1]);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      st.acc[hh][0] = st.acc[hh][0] * alpha[hh] + add[hh][0] + zsum[hh];
      st.acc[hh][1] = st.acc[hh][1] * alpha[hh] + add[hh][1] + zsum[hh];
    }
    wave_sync_lds();  // pv / qp are rewritten by the next group
  }

  const size_t partial_base = (static_cast<size_t>(b) * a.num_q_heads + qh0) * a.splits;
  finish_split<G>(st, sm.merge, a.partials, a.counters + slice,
                  a.out + (static_cast<size_t>(b) * a.num_q_heads + qh0) * kHeadDim, partial_base, split, a.splits);
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
