// Split-K pieces shared by the INT2 and bf16 decode kernels: query rotation,
// the in-workgroup merge of per-wave softmax states, the partial record and
// the per-split partial record (merged by merge.hip).
//
// Softmax states are kept in base 2: logits are pre-multiplied by log2(e),
// m is the running maximum of those scaled logits, l = sum 2^(x - m), and
// acc[d] = sum 2^(x - m) * value[d].  Merging (m_i, l_i, acc_i) gives
// M = max m_i, L = sum l_i 2^(m_i - M), out = sum acc_i 2^(m_i - M) / L.
#pragma once

#include "device_common.hpp"
#include "internal.hpp"

namespace oscar {

constexpr float kLog2e = 1.4426950408889634f;

// The query values a thread contributes to load_and_rotate_q: elements
// tid and tid + blockDim.x of q [G][128] (bf16), 0 beyond G rows.  Split
// from the rotation so that a kernel can issue these loads before other
// long-latency loads and wait for them alone.
template <int G, int kRows>
struct QueryRegs {
  float v[2];
};

template <int G, int kRows>
__device__ __forceinline__ QueryRegs<G, kRows> fetch_q(const uint16_t* q) {
  static_assert(kRows * kHeadDim <= 2 * 512, "two query elements per thread at >= 512 threads");
  QueryRegs<G, kRows> r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = threadIdx.x + k * blockDim.x;
    const float x = bf16_to_f32(q[i < G * kHeadDim ? i : 0]);   // unconditional load, no branch
    r.v[k] = (i < G * kHeadDim) ? x : 0.f;
  }
  return r;
}

// dst_raw = q * scale and, if dst_rot is given, dst_rot = (H q) * scale with
// the orthonormal Sylvester Hadamard matrix (butterflies in LDS).  Rows
// G .. kRows-1 of both are zero-filled.  Block-wide.
template <int G, int kRows>
__device__ void rotate_q(const QueryRegs<G, kRows>& r, float scale, float (*dst_raw)[kHeadDim],
                         float (*dst_rot)[kHeadDim]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + k * blockDim.x;
    if (i < kRows * kHeadDim) {
      dst_raw[i / kHeadDim][i % kHeadDim] = r.v[k] * scale;
      if (dst_rot) dst_rot[i / kHeadDim][i % kHeadDim] = r.v[k];
    }
  }
  __syncthreads();
  if (!dst_rot) return;
  for (int bit = 1; bit < kHeadDim; bit <<= 1) {
    for (int i = tid; i < G * kHeadDim / 2; i += blockDim.x) {
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
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) dst_rot[i / kHeadDim][i % kHeadDim] *= norm;
  __syncthreads();
}

// fetch_q followed by rotate_q.
template <int G, int kRows>
__device__ void load_and_rotate_q(const uint16_t* q, float scale, float (*dst_raw)[kHeadDim],
                                  float (*dst_rot)[kHeadDim]) {
  rotate_q<G, kRows>(fetch_q<G, kRows>(q), scale, dst_raw, dst_rot);
}

// Hardware 2^x (about 1 ulp; 2^-inf = 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Softmax states of G heads from kSlots producers (waves, plus extra slots
// such as a bf16-tail state) of one workgroup.  A producer that saw no
// token leaves m = -inf, l = 0, acc = 0.
template <int G, int kSlots>
struct MergeSmem {
  float m[kSlots][G];
  float l[kSlots][G];
  float acc[kSlots][G][kHeadDim];
};

template <int G, int kSlots>
__device__ void clear_slot(MergeSmem<G, kSlots>& sm, int slot) {
  // called by one wave
  const int lane = threadIdx.x & 63;
  for (int i = lane; i < G * kHeadDim; i += kWave) sm.acc[slot][i / kHeadDim][i % kHeadDim] = 0.f;
  if (lane < G) {
    sm.m[slot][lane] = -INFINITY;
    sm.l[slot][lane] = 0.f;
  }
}

// Merge the slots and write this split's partial records
// partials[(partial_base + hh * splits + split) * 132] = (m, l, -, -, acc[128]).
// Must be reached by all threads of the block after the slots are written
// (with a barrier first unless the caller has just passed one: kSync).
// The records of all splits are merged by merge_splits_kernel, launched
// after the decode kernel on the same stream.
template <int G, int kSlots, bool kSync = true>
__device__ void write_partial(MergeSmem<G, kSlots>& sm, float* partials, size_t partial_base, int split,
                              int splits) {
  const int tid = threadIdx.x;
  if (kSync) __syncthreads();
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) {
    const int hh = i / kHeadDim;
    const int d = i % kHeadDim;
    float m[kSlots];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSlots; ++w) {
      m[w] = sm.m[w][hh];
      M = fmaxf(M, m[w]);
    }
    float Lsum = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kSlots; ++w) {
        const float f = fast_exp2(m[w] - M);   // 0 for an empty slot (m = -inf)
        Lsum = fmaf(sm.l[w][hh], f, Lsum);
        A = fmaf(sm.acc[w][hh][d], f, A);
      }
    }
    float* rec = partials + (partial_base + static_cast<size_t>(hh) * splits + split) * kPartialFloats;
    rec[4 + d] = A;
    if (d == 0) {
      rec[0] = M;
      rec[1] = Lsum;
    }
  }
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Reductions over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every
// lane of the row receives the result.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f32<kDppRowRor4>(x));
  x = fmaxf(x, dpp_f32<kDppRowRor8>(x));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  x += dpp_f32<kDppRowRor4>(x);
  x += dpp_f32<kDppRowRor8>(x);
  return x;
}

// bf16 tokens (the not yet quantized tail) with plain VALU arithmetic: one
// wave scores up to 128 tokens with the unrotated query (lane = token) and
// accumulates their values (lane = channel pair), leaving a softmax state in
// `slot` of the merge buffer.  k, v: token-major bf16 rows of 128 channels.
template <int G, int kSlots>
__device__ void bf16_tokens_wave(const uint16_t* k, const uint16_t* v, int n_tok, const float (*q_raw)[kHeadDim],
                                 float (*pv)[kGroup], MergeSmem<G, kSlots>& sm, int slot) {
  const int lane = threadIdx.x & 63;
  float logit[G][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int tt = lane + 64 * kk;
    const bool valid = tt < n_tok;
    float dot[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) dot[hh] = 0.f;
    if (valid) {
      const uint4* kr = reinterpret_cast<const uint4*>(k + static_cast<size_t>(tt) * kHeadDim);
#pragma unroll 4
      for (int c = 0; c < 16; ++c) {
        const uint4 w = kr[c];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = bf16lo_to_f32(ws[e]), k1 = bf16hi_to_f32(ws[e]);
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            dot[hh] = fmaf(q_raw[hh][8 * c + 2 * e], k0, dot[hh]);
            dot[hh] = fmaf(q_raw[hh][8 * c + 2 * e + 1], k1, dot[hh]);
          }
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) logit[hh][kk] = valid ? dot[hh] : -INFINITY;
  }
  float mx[G], lsum[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    mx[hh] = wave_max(fmaxf(logit[hh][0], logit[hh][1]));
    const float p0 = (mx[hh] == -INFINITY) ? 0.f : exp2f(logit[hh][0] - mx[hh]);
    const float p1 = (mx[hh] == -INFINITY) ? 0.f : exp2f(logit[hh][1] - mx[hh]);
    lsum[hh] = wave_sum(p0 + p1);
    pv[hh][lane] = p0;
    pv[hh][lane + 64] = p1;
  }
  wave_sync_lds();
  float add[G][2];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) add[hh][0] = add[hh][1] = 0.f;
  for (int tt = 0; tt < n_tok; ++tt) {
    const uint32_t vv = *reinterpret_cast<const uint32_t*>(v + static_cast<size_t>(tt) * kHeadDim + 2 * lane);
    const float v0 = bf16lo_to_f32(vv), v1 = bf16hi_to_f32(vv);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float p = pv[hh][tt];
      add[hh][0] = fmaf(p, v0, add[hh][0]);
      add[hh][1] = fmaf(p, v1, add[hh][1]);
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    sm.acc[slot][hh][2 * lane] = add[hh][0];
    sm.acc[slot][hh][2 * lane + 1] = add[hh][1];
    if (lane == 0) {
      sm.m[slot][hh] = mx[hh];
      sm.l[slot][hh] = lsum[hh];
    }
  }
}

}  // namespace oscar
