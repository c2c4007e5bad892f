// Split-K flash-decoding over unquantized bf16 keys and values: the
// reference decode step against which the INT2 path's speed-up is measured
// (the pages compare against BF16 FlashDecoding-v2: OScaR abstract, arXiv
// 2605.19660; ai-papers.net OScaR summary, section "実験結果").
//
// Grid (split, KV head, sequence), 8 waves per workgroup; each wave walks
// its 128-token chunks in steps of 32 tokens with a base-2 online softmax.
// Lane l = 16 tq + c owns channels 8c .. 8c+7 of the tokens 4s + tq of a
// step: key and value loads read whole rows (1 KB per wave instruction),
// the dot products are summed over the 16 lanes of a row with DPP, and the
// weighted values accumulate in registers (no LDS traffic per token).  The
// waves merge in LDS into a per-split partial record; merge.hip combines
// the splits.
#include "decode_common.hpp"

namespace oscar {
namespace {

constexpr int kDecodeThreads = 512;   // 8 waves: one workgroup per compute unit
constexpr int kDecodeWaves = kDecodeThreads / kWave;
constexpr int kSub = 32;              // tokens per wave step
constexpr int kSteps = kSub / 4;      // tokens per lane per step

template <int G>
struct Bf16Smem {
  float q_raw[G][kHeadDim];
  MergeSmem<G, kDecodeWaves> merge;
};

// Bytes of one 32-token step: lane l = 16 tq + c holds channels 8c .. 8c+7
// of tokens t0 + 4s + tq (s = 0..7), so every load instruction of the wave
// reads four whole 256-byte rows.
struct StepBytes {
  uint4 k[kSteps];
  uint4 v[kSteps];
};

__device__ __forceinline__ void unpack8(const uint4& w, float (&x)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16lo_to_f32(u[e]);
    x[2 * e + 1] = bf16hi_to_f32(u[e]);
  }
}

// Rows beyond the sequence are read as its last row (always in bounds) and
// masked out of the softmax.
__device__ __forceinline__ const uint4* row_ptr(const uint16_t* base, size_t slice_row0, int t, int last, int c) {
  return reinterpret_cast<const uint4*>(base + (slice_row0 + min(t, last)) * kHeadDim) + c;
}

// 16 bytes of K or V with the nontemporal hint (the cache is read once per
// step, as in the INT2 kernel's copies).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Maximum and sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float max_over_rows(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, kWave));
  return fmaxf(x, __shfl_xor(x, 32, kWave));
}
__device__ __forceinline__ float sum_over_rows(float x) {
  x += __shfl_xor(x, 16, kWave);
  return x + __shfl_xor(x, 32, kWave);
}

template <int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_bf16_kernel(DecodeBf16Args a) {
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int tq = lane >> 4;   // token within a group of four
  const int c = lane & 15;    // channels 8c .. 8c+7

  __shared__ Bf16Smem<G> sm;

  const int len = min(max(a.seq_len[b], 0), min(a.capacity, a.max_tokens));
  // Split s owns the 128-token chunks s, s + S, s + 2S, ... (S = splits),
  // so the workgroups of a head read neighbouring chunks at any moment.
  const int S = a.splits;
  const size_t slice = static_cast<size_t>(b) * a.num_kv_heads + h;
  const size_t row0 = slice * a.capacity;
  const int qh0 = h * G;
  const int last = max(len - 1, 0);
  load_and_rotate_q<G, G>(a.q + (static_cast<size_t>(b) * a.num_q_heads + qh0) * kHeadDim, a.sm_scale * kLog2e,
                          sm.q_raw, nullptr);
  float qreg[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int j = 0; j < 8; ++j) qreg[hh][j] = sm.q_raw[hh][8 * c + j];

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[hh][j] = 0.f;
  }

  // steps of 32 tokens: step i is tokens 32 (i % 4) of chunk split + (i / 4 * kWaves + wave) * S
  const int c_end = (len + kGroup - 1) / kGroup;
  auto step_t0 = [&](int i) { return (split + ((i >> 2) * kDecodeWaves + wave) * S) * kGroup + kSub * (i & 3); };
  auto has_step = [&](int i) { return split + ((i >> 2) * kDecodeWaves + wave) * S < c_end; };
  StepBytes cur;
  if (has_step(0)) {
    const int t0 = step_t0(0);
#pragma unroll
    for (int s2 = 0; s2 < kSteps; ++s2) {
      cur.k[s2] = load_stream(row_ptr(a.k, row0, t0 + 4 * s2 + tq, last, c));
      cur.v[s2] = load_stream(row_ptr(a.v, row0, t0 + 4 * s2 + tq, last, c));
    }
  }
  for (int i = 0; has_step(i); ++i) {
    const int t0 = step_t0(i);
    // ---- scores: per lane 8 channels, then the sum over the 16 lanes of a row ----
    float logit[G][kSteps];
#pragma unroll
    for (int s2 = 0; s2 < kSteps; ++s2) {
      float kx[8];
      unpack8(cur.k[s2], kx);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) d = fmaf(qreg[hh][j], kx[j], d);
        logit[hh][s2] = row_sum16(d);
      }
    }
    const bool more = has_step(i + 1);
    const int t1 = step_t0(i + 1);
    if (more) {
#pragma unroll
      for (int s2 = 0; s2 < kSteps; ++s2) cur.k[s2] = load_stream(row_ptr(a.k, row0, t1 + 4 * s2 + tq, last, c));
    }
    // ---- online softmax (base 2) over this step's tokens ----
    float p[G][kSteps];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float mx = -INFINITY;
#pragma unroll
      for (int s2 = 0; s2 < kSteps; ++s2) {
        if (t0 + 4 * s2 + tq >= len) logit[hh][s2] = -INFINITY;
        mx = fmaxf(mx, logit[hh][s2]);
      }
      mx = max_over_rows(mx);
      const float m_new = fmaxf(m[hh], mx);
      // every step holds a token of the sequence, so m_new is finite
      const float alpha = exp2f(m[hh] - m_new);
      m[hh] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < kSteps; ++s2) {
        p[hh][s2] = exp2f(logit[hh][s2] - m_new);
        ls += p[hh][s2];
      }
      l[hh] = fmaf(l[hh], alpha, ls);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[hh][j] *= alpha;
    }
    // ---- weighted values: this lane's tokens and channels ----
#pragma unroll
    for (int s2 = 0; s2 < kSteps; ++s2) {
      float vx[8];
      unpack8(cur.v[s2], vx);
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[hh][j] = fmaf(p[hh][s2], vx[j], acc[hh][j]);
    }
    if (more) {
#pragma unroll
      for (int s2 = 0; s2 < kSteps; ++s2) cur.v[s2] = load_stream(row_ptr(a.v, row0, t1 + 4 * s2 + tq, last, c));
    }
  }

  // ---- sums over the four token rows of the wave -> merge slot ----
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float lt = sum_over_rows(l[hh]);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[hh][j] = sum_over_rows(acc[hh][j]);
    if (tq == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.merge.acc[wave][hh][8 * c + j] = acc[hh][j];
      if (c == 0) {
        sm.merge.m[wave][hh] = m[hh];
        sm.merge.l[wave][hh] = lt;
      }
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
