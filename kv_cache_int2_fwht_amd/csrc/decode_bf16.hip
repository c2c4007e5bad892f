// Split-K flash-decoding over unquantized bf16 keys and values: the
// reference decode step against which the INT2 path's speed-up is measured
// (the pages compare against BF16 FlashDecoding-v2: OScaR abstract, arXiv
// 2605.19660; ai-papers.net OScaR summary, section "実験結果").
//
// Same skeleton as the INT2 kernel: grid (split, KV head, sequence), 4 waves
// per workgroup, 128-token chunks per wave with a base-2 online softmax,
// in-LDS wave merge and a per-split partial record merged by merge.hip.
#include "decode_common.hpp"

namespace oscar {
namespace {

constexpr int kDecodeThreads = 512;   // 8 waves: one workgroup per compute unit
constexpr int kDecodeWaves = kDecodeThreads / kWave;

template <int G>
struct Bf16Smem {
  float q_raw[G][kHeadDim];
  float pv[kDecodeWaves][G][kGroup];
  MergeSmem<G, kDecodeWaves> merge;
};

// Per-wave state of G heads: m, l uniform across the wave; each lane owns
// channels 2*lane and 2*lane + 1 of acc.
template <int G>
struct WaveState {
  float m[G];
  float l[G];
  float acc[G][2];
};

template <int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_bf16_kernel(DecodeBf16Args a) {
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  __shared__ Bf16Smem<G> sm;

  const int len = min(max(a.seq_len[b], 0), min(a.capacity, a.max_tokens));
  // Split s owns the 128-token chunks s, s + S, s + 2S, ... (S = splits),
  // so the workgroups of a head read neighbouring chunks at any moment.
  const int S = a.splits;
  const int t_end = len;
  const size_t slice = static_cast<size_t>(b) * a.num_kv_heads + h;
  const int qh0 = h * G;
  load_and_rotate_q<G, G>(a.q + (static_cast<size_t>(b) * a.num_q_heads + qh0) * kHeadDim, a.sm_scale * kLog2e,
                          sm.q_raw, nullptr);

  WaveState<G> st;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    st.m[hh] = -INFINITY;
    st.l[hh] = 0.f;
    st.acc[hh][0] = st.acc[hh][1] = 0.f;
  }

  const int c_end = (len + kGroup - 1) / kGroup;
  for (int c = split + wave * S; c < c_end; c += kDecodeWaves * S) {
    const int t0 = c * kGroup;
    float logit[G][2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = t0 + lane + 64 * k;
      const bool valid = t < t_end;
      float dot[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) dot[hh] = 0.f;
      if (valid) {
        const uint4* kr = reinterpret_cast<const uint4*>(a.k + (slice * a.capacity + t) * kHeadDim);
#pragma unroll 4
        for (int ch = 0; ch < 16; ++ch) {
          const uint4 w = kr[ch];
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float k0 = bf16lo_to_f32(ws[e]), k1 = bf16hi_to_f32(ws[e]);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
              dot[hh] = fmaf(sm.q_raw[hh][8 * ch + 2 * e], k0, dot[hh]);
              dot[hh] = fmaf(sm.q_raw[hh][8 * ch + 2 * e + 1], k1, dot[hh]);
            }
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) logit[hh][k] = valid ? dot[hh] : -INFINITY;
    }
    float alpha[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float gmax = wave_max(fmaxf(logit[hh][0], logit[hh][1]));
      const float m_new = fmaxf(st.m[hh], gmax);
      if (m_new == -INFINITY) {
        alpha[hh] = 1.f;
        sm.pv[wave][hh][lane] = 0.f;
        sm.pv[wave][hh][lane + 64] = 0.f;
        continue;
      }
      alpha[hh] = (st.m[hh] == -INFINITY) ? 0.f : exp2f(st.m[hh] - m_new);
      const float p0 = exp2f(logit[hh][0] - m_new);
      const float p1 = exp2f(logit[hh][1] - m_new);
      st.l[hh] = st.l[hh] * alpha[hh] + wave_sum(p0 + p1);
      st.m[hh] = m_new;
      sm.pv[wave][hh][lane] = p0;
      sm.pv[wave][hh][lane + 64] = p1;
    }
    wave_sync_lds();
    float add[G][2];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) add[hh][0] = add[hh][1] = 0.f;
    const int n_valid = min(t_end - t0, kGroup);
    for (int tt = 0; tt < n_valid; ++tt) {
      const uint32_t vv = *reinterpret_cast<const uint32_t*>(a.v + (slice * a.capacity + t0 + tt) * kHeadDim + 2 * lane);
      const float v0 = bf16lo_to_f32(vv), v1 = bf16hi_to_f32(vv);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float p = sm.pv[wave][hh][tt];
        add[hh][0] = fmaf(p, v0, add[hh][0]);
        add[hh][1] = fmaf(p, v1, add[hh][1]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      st.acc[hh][0] = st.acc[hh][0] * alpha[hh] + add[hh][0];
      st.acc[hh][1] = st.acc[hh][1] * alpha[hh] + add[hh][1];
    }
    wave_sync_lds();
  }

#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    sm.merge.acc[wave][hh][2 * lane] = st.acc[hh][0];
    sm.merge.acc[wave][hh][2 * lane + 1] = st.acc[hh][1];
    if (lane == 0) {
      sm.merge.m[wave][hh] = st.m[hh];
      sm.merge.l[wave][hh] = st.l[hh];
    }
  }
  const size_t partial_base = (static_cast<size_t>(b) * a.num_q_heads + qh0) * a.splits;
  write_partial<G, kDecodeWaves>(sm.merge, a.partials, partial_base, split, a.splits);
}

template <int G>
hipError_t launch_g(const DecodeBf16Args& a, int32_t batch, hipStream_t s) {
  dim3 grid(a.splits, a.num_kv_heads, batch);
  hipLaunchKernelGGL(decode_bf16_kernel<G>, grid, dim3(kDecodeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeBf16Args& a, int32_t batch, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<1>(a, batch, s);
    case 2: return launch_g<2>(a, batch, s);
    case 4: return launch_g<4>(a, batch, s);
    case 8: return launch_g<8>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
