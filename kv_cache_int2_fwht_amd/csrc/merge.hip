// Merge of the split-K partial softmax states into the attention output.
//
// Each decode workgroup leaves, per query head, a record (m, l, -, -,
// acc[128]) of its token range in base 2: m = max logit * log2(e),
// l = sum 2^(x - m), acc = sum 2^(x - m) * value.  Merging is the usual
// flash-decoding algebra: M = max m_s, w_s = 2^(m_s - M), out =
// sum_s w_s acc_s / sum_s w_s l_s, with out = 0 when every split is empty.
// The splits are combined in a fixed order, so the result is deterministic.
//
// One workgroup per (query head, sequence), so that the partial records are
// read by many compute units at once.  Wave w merges the splits w, w + 4,
// ... (lane = two channels; the record's m and l are read by every lane
// from the same address), then wave 0 merges the four wave results.
#include "decode_common.hpp"

namespace oscar {
namespace {

constexpr int kMergeUnroll = 8;
constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / kWave;

__global__ __launch_bounds__(kMergeThreads) void merge_splits_kernel(const float* __restrict__ partials,
                                                                       float* __restrict__ out, int num_q_heads,
                                                                       int splits) {
  const int qh = blockIdx.x;
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  __shared__ float sm_m[kMergeWaves], sm_l[kMergeWaves];
  __shared__ float2 sm_acc[kMergeWaves][kWave];
  const float* base = partials + (static_cast<size_t>(b) * num_q_heads + qh) * splits * kPartialFloats;

  float M = -INFINITY, L = 0.f, a0 = 0.f, a1 = 0.f;
  for (int s0 = wave; s0 < splits; s0 += kMergeWaves * kMergeUnroll) {
    float2 ml[kMergeUnroll], v[kMergeUnroll];
#pragma unroll
    for (int k = 0; k < kMergeUnroll; ++k) {   // all loads of the batch first
      const int s = s0 + k * kMergeWaves;
      if (s < splits) {
        const float* rec = base + static_cast<size_t>(s) * kPartialFloats;
        ml[k] = *reinterpret_cast<const float2*>(rec);
        v[k] = *reinterpret_cast<const float2*>(rec + 4 + 2 * lane);
      } else {
        ml[k] = make_float2(-INFINITY, 0.f);
        v[k] = make_float2(0.f, 0.f);
      }
    }
    // the batch's maximum first, so that its weights are independent
    float Mb = ml[0].x;
#pragma unroll
    for (int k = 1; k < kMergeUnroll; ++k) Mb = fmaxf(Mb, ml[k].x);
    const float M_new = fmaxf(M, Mb);
    if (M_new == -INFINITY) continue;         // nothing seen yet (uniform over the wave)
    const float r = fast_exp2(M - M_new);     // 0 while M was -inf
    float Lb = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int k = 0; k < kMergeUnroll; ++k) {
      const float w = fast_exp2(ml[k].x - M_new);   // 0 for an empty split
      Lb = fmaf(ml[k].y, w, Lb);
      b0 = fmaf(v[k].x, w, b0);
      b1 = fmaf(v[k].y, w, b1);
    }
    L = fmaf(L, r, Lb);
    a0 = fmaf(a0, r, b0);
    a1 = fmaf(a1, r, b1);
    M = M_new;
  }
  if (lane == 0) {
    sm_m[wave] = M;
    sm_l[wave] = L;
  }
  sm_acc[wave][lane] = make_float2(a0, a1);
  __syncthreads();
  if (wave == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) Mt = fmaxf(Mt, sm_m[w]);
    float Lt = 0.f, r0 = 0.f, r1 = 0.f;
    if (Mt != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kMergeWaves; ++w) {
        const float f = fast_exp2(sm_m[w] - Mt);   // 0 for a wave that saw no split
        Lt = fmaf(sm_l[w], f, Lt);
        r0 = fmaf(sm_acc[w][lane].x, f, r0);
        r1 = fmaf(sm_acc[w][lane].y, f, r1);
      }
    }
    const float2 res = (Lt > 0.f) ? make_float2(r0 / Lt, r1 / Lt) : make_float2(0.f, 0.f);
    *reinterpret_cast<float2*>(out + (static_cast<size_t>(b) * num_q_heads + qh) * kHeadDim + 2 * lane) = res;
  }
}

}  // namespace

hipError_t launch_merge(const float* partials, float* out, int32_t batch, int32_t num_q_heads, int32_t splits,
                        hipStream_t s) {
  hipLaunchKernelGGL(merge_splits_kernel, dim3(num_q_heads, batch), dim3(kMergeThreads), 0, s, partials, out,
                     num_q_heads, splits);
  return hipGetLastError();
}

}  // namespace oscar
