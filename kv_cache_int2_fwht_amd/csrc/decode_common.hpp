// Split-K pieces shared by the INT2 and bf16 decode kernels: query rotation,
// the in-workgroup merge of per-wave softmax states, the partial record and
// the last-arriving-workgroup merge across splits.
//
// Softmax states are kept in base 2: logits are pre-multiplied by log2(e),
// m is the running maximum of those scaled logits, l = sum 2^(x - m), and
// acc[d] = sum 2^(x - m) * value[d].  Merging (m_i, l_i, acc_i) gives
// M = max m_i, L = sum l_i 2^(m_i - M), out = sum acc_i 2^(m_i - M) / L.
#pragma once

#include "device_common.hpp"
#include "internal.hpp"

namespace oscar {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = kDecodeThreads / kWave;
constexpr float kLog2e = 1.4426950408889634f;

// q [G][128] (bf16) -> dst_raw = q * scale, dst_rot = (H q) * scale with the
// orthonormal Sylvester Hadamard matrix (butterflies in LDS).  Block-wide.
template <int G>
__device__ void load_and_rotate_q(const uint16_t* q, float scale, float (*dst_raw)[kHeadDim],
                                  float (*dst_rot)[kHeadDim]) {
  const int tid = threadIdx.x;
  for (int i = tid; i < G * kHeadDim; i += kDecodeThreads) {
    const float v = bf16_to_f32(q[i]);
    dst_raw[i / kHeadDim][i % kHeadDim] = v * scale;
    dst_rot[i / kHeadDim][i % kHeadDim] = v;
  }
  __syncthreads();
  for (int bit = 1; bit < kHeadDim; bit <<= 1) {
    for (int i = tid; i < G * kHeadDim / 2; i += kDecodeThreads) {
      const int hh = i / (kHeadDim / 2);
      const int k = i % (kHeadDim / 2);
      // k enumerates the index pairs (lo, lo | bit) with lo's bit clear.
      const int lo = ((k & ~(bit - 1)) << 1) | (k & (bit - 1));
      const float x = dst_rot[hh][lo], y = dst_rot[hh][lo | bit];
      dst_rot[hh][lo] = x + y;
      dst_rot[hh][lo | bit] = x - y;
    }
    __syncthreads();
  }
  const float norm = scale * 0.088388347648318440550f;  // 1/sqrt(128)
  for (int i = tid; i < G * kHeadDim; i += kDecodeThreads) dst_rot[i / kHeadDim][i % kHeadDim] *= norm;
  __syncthreads();
}

// Per-wave state of G heads: m, l uniform across the wave; each lane owns
// channels 2*lane and 2*lane + 1 of acc.
template <int G>
struct WaveState {
  float m[G];
  float l[G];
  float acc[G][2];
};

template <int G>
struct MergeSmem {
  float m[kDecodeWaves][G];
  float l[kDecodeWaves][G];
  float acc[kDecodeWaves][G][kHeadDim];
  bool last;
};

// Merge the waves' states inside the workgroup, write this split's partial
// records, and let the last workgroup of the (sequence, KV head) merge every
// split into out.  Must be reached by all threads of the block.
template <int G>
__device__ void finish_split(const WaveState<G>& st, MergeSmem<G>& sm, float* partials, uint32_t* counter,
                             float* out_bh, size_t partial_base, int split, int splits) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      sm.m[wave][hh] = st.m[hh];
      sm.l[wave][hh] = st.l[hh];
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    sm.acc[wave][hh][2 * lane] = st.acc[hh][0];
    sm.acc[wave][hh][2 * lane + 1] = st.acc[hh][1];
  }
  __syncthreads();
  // partial record of head hh at partials[(partial_base + hh * splits + split) * 132]
  for (int i = tid; i < G * kHeadDim; i += kDecodeThreads) {
    const int hh = i / kHeadDim;
    const int d = i % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, sm.m[w][hh]);
    float Lsum = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float f = (sm.m[w][hh] == -INFINITY) ? 0.f : exp2f(sm.m[w][hh] - M);
      Lsum += sm.l[w][hh] * f;
      A += sm.acc[w][hh][d] * f;
    }
    float* rec = partials + (partial_base + static_cast<size_t>(hh) * splits + split) * kPartialFloats;
    rec[4 + d] = A;
    if (d == 0) {
      rec[0] = M;
      rec[1] = Lsum;
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(counter, 1u);
    sm.last = (prev == static_cast<uint32_t>(splits - 1));
  }
  __syncthreads();
  if (!sm.last) return;
  __threadfence();
  for (int i = tid; i < G * kHeadDim; i += kDecodeThreads) {
    const int hh = i / kHeadDim;
    const int d = i % kHeadDim;
    const float* base = partials + (partial_base + static_cast<size_t>(hh) * splits) * kPartialFloats;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, base[s * kPartialFloats]);
    float Lsum = 0.f, A = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < splits; ++s) {
        const float* rec = base + s * kPartialFloats;
        const float ms = rec[0];
        if (ms == -INFINITY) continue;
        const float f = exp2f(ms - M);
        Lsum += rec[1] * f;
        A += rec[4 + d] * f;
      }
    }
    out_bh[hh * kHeadDim + d] = (Lsum > 0.f) ? A / Lsum : 0.f;
  }
  if (tid == 0) atomicExch(counter, 0u);
}

}  // namespace oscar
