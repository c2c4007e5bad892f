// Merge of the split-K partial softmax states into the attention output.
//
// Each decode workgroup leaves, per query head, a record (m, l, -, -,
// acc[128]) of its token range in base 2: m = max logit * log2(e),
// l = sum 2^(x - m), acc = sum 2^(x - m) * value.  Merging is the usual
// flash-decoding algebra: M = max m_s, w_s = 2^(m_s - M), out =
// sum_s w_s acc_s / sum_s w_s l_s, with out = 0 when every split is empty.
// The splits are combined in a fixed order, so the result is deterministic.
//
// One workgroup per (KV head, sequence), one wave per query head: lane s
// reads m_s and l_s of split s, every lane reads two channels of every
// split's acc, all loads are issued before any arithmetic waits on them.
#include "decode_common.hpp"

namespace oscar {
namespace {

constexpr int kChunk = 64;   // splits handled per pass (one per lane)

template <int G>
__global__ __launch_bounds__(kDecodeThreads) void merge_splits_kernel(const float* __restrict__ partials,
                                                                       float* __restrict__ out, int num_q_heads,
                                                                       int splits) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  for (int hh = wave; hh < G; hh += kDecodeWaves) {
    const int qh = h * G + hh;
    const float* base = partials + (static_cast<size_t>(b) * num_q_heads + qh) * splits * kPartialFloats;
    float M = -INFINITY;
    for (int c0 = 0; c0 < splits; c0 += kChunk) {
      const int s = c0 + lane;
      const float ms = (s < splits) ? base[static_cast<size_t>(s) * kPartialFloats] : -INFINITY;
      M = fmaxf(M, wave_max(ms));
    }
    float L = 0.f, a0 = 0.f, a1 = 0.f;
    if (M != -INFINITY) {
      for (int c0 = 0; c0 < splits; c0 += kChunk) {
        const int s = c0 + lane;
        float ms = -INFINITY, ls = 0.f;
        if (s < splits) {
          ms = base[static_cast<size_t>(s) * kPartialFloats];
          ls = base[static_cast<size_t>(s) * kPartialFloats + 1];
        }
        const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
        L += wave_sum(ls * w);
        const int cnt = min(kChunk, splits - c0);
        float2 v[kChunk];
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
          v[k] = (k < cnt) ? *reinterpret_cast<const float2*>(base + static_cast<size_t>(c0 + k) * kPartialFloats + 4 +
                                                              2 * lane)
                           : make_float2(0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
          const float wk = __shfl(w, k, kWave);
          a0 = fmaf(wk, v[k].x, a0);
          a1 = fmaf(wk, v[k].y, a1);
        }
      }
    }
    float2 r = (L > 0.f) ? make_float2(a0 / L, a1 / L) : make_float2(0.f, 0.f);
    *reinterpret_cast<float2*>(out + (static_cast<size_t>(b) * num_q_heads + qh) * kHeadDim + 2 * lane) = r;
  }
}

template <int G>
hipError_t launch_g(const float* partials, float* out, int batch, int num_kv_heads, int num_q_heads, int splits,
                    hipStream_t s) {
  hipLaunchKernelGGL(merge_splits_kernel<G>, dim3(num_kv_heads, batch), dim3(kDecodeThreads), 0, s, partials, out,
                     num_q_heads, splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const float* partials, float* out, int32_t batch, int32_t num_kv_heads, int32_t num_q_heads,
                        int32_t splits, hipStream_t s) {
  switch (num_q_heads / num_kv_heads) {
    case 1: return launch_g<1>(partials, out, batch, num_kv_heads, num_q_heads, splits, s);
    case 2: return launch_g<2>(partials, out, batch, num_kv_heads, num_q_heads, splits, s);
    case 4: return launch_g<4>(partials, out, batch, num_kv_heads, num_q_heads, splits, s);
    case 8: return launch_g<8>(partials, out, batch, num_kv_heads, num_q_heads, splits, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
