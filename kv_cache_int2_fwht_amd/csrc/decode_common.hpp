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

// Wait until at most `rem` units of kPerUnit copies each of this wave are
// outstanding (rem <= N; the counter wait takes its count as an immediate).
template <int kPerUnit, int N>
__device__ __forceinline__ void wait_units_outstanding(int rem) {
  if constexpr (N <= 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (rem >= N) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N * kPerUnit) : "memory");
    } else {
      wait_units_outstanding<kPerUnit, N - 1>(rem);
    }
  }
}

// An LDS flag, read by lane 0 alone and broadcast to the wave (a read of
// one word by all 64 lanes occupies the LDS longer).
__device__ __forceinline__ int read_flag(const int* f, int lane) {
  int v = 0;
  if (lane == 0) v = __hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
  return __builtin_amdgcn_readfirstlane(v);
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

// Merge slots 0 .. kUse-1 and write this split's partial records
// partials[(partial_base + hh * splits + split) * 132] = (m, l, -, -, acc[128]).
// Slots from kUse on must be empty (leaving them out changes nothing: an
// empty slot has weight 0).  Must be reached by all threads of the block
// after the slots are written (with a barrier first unless the caller has
// just passed one: kSync).  The records of all splits are merged by
// merge_splits_kernel, launched after the decode kernel on the same stream.
template <int G, int kSlots, bool kSync = true, int kUse = kSlots>
__device__ void write_partial(MergeSmem<G, kSlots>& sm, float* partials, size_t partial_base, int split,
                              int splits) {
  const int tid = threadIdx.x;
  if (kSync) __syncthreads();
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) {
    const int hh = i / kHeadDim;
    const int d = i % kHeadDim;
    static_assert(kUse <= kSlots, "merging more slots than there are");
    float m[kUse];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kUse; ++w) {
      m[w] = sm.m[w][hh];
      M = fmaxf(M, m[w]);
    }
    float Lsum = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kUse; ++w) {
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

// bf16 tokens (the not yet quantized tail): one wave scores up to 64
// tokens on the matrix cores, exact bf16 x bf16 products of the query (not
// rotated, since the tail is stored as it is) and the keys accumulated in
// fp32, then accumulates the values with plain VALU arithmetic (lane =
// channel pair), leaving a softmax state in `slot` of the merge buffer.
// k, v: token-major bf16 rows of 128 channels; q: the G query rows (bf16);
// scale: sm_scale * log2(e).  Token `last` is read from the rows k_last /
// v_last instead when they are given (a token appended in the same launch).
// pv: LDS scratch of the weights, [64 tokens][G].
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kTailPart = 64;   // tokens per bf16_tokens_wave call

template <int G, int kSlots>
__device__ void bf16_tokens_wave(const uint16_t* k, const uint16_t* v, int n_tok, const uint16_t* q, float scale,
                                 float (*pv)[G], MergeSmem<G, kSlots>& sm, int slot,
                                 const uint16_t* k_last = nullptr, const uint16_t* v_last = nullptr, int last = -1) {
  static_assert(G <= 8, "query rows 0..G-1 of the 16-row operand, two row groups at most");
  constexpr int kTiles = kTailPart / 16;
  n_tok = min(n_tok, kTailPart);
  const int lane = threadIdx.x & 63;
  const int gl = lane >> 4;   // operand K slice / result row group (heads 4 gl .. 4 gl + 3)
  const int n = lane & 15;    // operand row (query head) / result column (token of the tile)
  // every load first: the query (A operand: head n, zero rows beyond G,
  // channels 32 ks + 8 gl .. +7), the key rows of the tiles (B operand) and
  // the value pairs of all tokens (lane = channel pair).  Tokens past n_tok
  // are masked (logit -inf, weight 0) but still read a row, which must hold
  // finite data (0 * NaN is NaN): row 0 of the part.  A token appended in
  // this launch (row `last`) is read from its source rows k_last / v_last,
  // since another wave may be storing it into the tail meanwhile; when that
  // is row 0, the part holds no other valid token and all of its rows read
  // the source rows (row stride 0).  One select per row keeps the address
  // arithmetic, and so the register count, of the plain tail.
  const bool own0 = k_last != nullptr && last == 0;
  const int stride = own0 ? 0 : kHeadDim;
  if (own0) {
    k = k_last;
    v = v_last;
  }
  uint4 qa[4], kb[kTiles][4];
  uint32_t vv[kTailPart];
  {
    const uint16_t* qrow = q + static_cast<size_t>(n < G ? n : 0) * kHeadDim + 8 * gl;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[ks] = *reinterpret_cast<const uint4*>(qrow + 32 * ks);
#pragma unroll
    for (int j = 0; j < kTiles; ++j) {
      const int tok = 16 * j + n;
      const uint16_t* krow = (k_last != nullptr && tok == last) ? k_last : k + (tok < n_tok ? tok : 0) * stride;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[j][ks] = *reinterpret_cast<const uint4*>(krow + 32 * ks + 8 * gl);
    }
#pragma unroll
    for (int e = 0; e < kTailPart; ++e) {
      const uint16_t* vrow = (v_last != nullptr && e == last) ? v_last : v + (e < n_tok ? e : 0) * stride;
      vv[e] = *reinterpret_cast<const uint32_t*>(vrow + 2 * lane);
    }
  }
  // scores: tile j = tokens 16 j .. 16 j + 15; lane holds rows 4 gl + r of column n
  float lg[kTiles][4];
#pragma unroll
  for (int j = 0; j < kTiles; ++j) {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, n < G ? qa[ks] : make_uint4(0, 0, 0, 0)),
                                                  __builtin_bit_cast(bf16x8_t, kb[j][ks]), c, 0, 0, 0);
    const bool valid = 16 * j + n < n_tok;
#pragma unroll
    for (int r = 0; r < 4; ++r) lg[j][r] = valid ? c[r] * scale : -INFINITY;
  }
  // softmax per head (max and sum over the tiles in-lane, then over the 16 lanes of the row)
  float mx[4], ls[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float m = lg[0][r];
#pragma unroll
    for (int j = 1; j < kTiles; ++j) m = fmaxf(m, lg[j][r]);
    mx[r] = row_max16(m);   // finite: token 0 of the part is always valid
    float l = 0.f;
#pragma unroll
    for (int j = 0; j < kTiles; ++j) {
      const float p = fast_exp2(lg[j][r] - mx[r]);   // 0 for masked tokens
      lg[j][r] = p;
      l += p;
    }
    ls[r] = row_sum16(l);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hh = 4 * gl + r;
    if (hh < G) {
#pragma unroll
      for (int j = 0; j < kTiles; ++j) pv[16 * j + n][hh] = lg[j][r];   // masked tokens get 0
    }
  }
  wave_sync_lds();
  // values
  float add[G][2];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) add[hh][0] = add[hh][1] = 0.f;
#pragma unroll
  for (int e = 0; e < kTailPart; ++e) {
    const float v0 = bf16lo_to_f32(vv[e]), v1 = bf16hi_to_f32(vv[e]);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float p = pv[e][hh];   // 0 past n_tok
      add[hh][0] = fmaf(p, v0, add[hh][0]);
      add[hh][1] = fmaf(p, v1, add[hh][1]);
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    sm.acc[slot][hh][2 * lane] = add[hh][0];
    sm.acc[slot][hh][2 * lane + 1] = add[hh][1];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hh = 4 * gl + r;
    if (hh < G && n == 0) {
      sm.m[slot][hh] = mx[r];
      sm.l[slot][hh] = ls[r];
    }
  }
}

}  // namespace oscar
