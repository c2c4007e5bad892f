// Split-K flash-decoding over unquantized bf16 keys and values: the
// reference decode step against which the INT2 path's speed-up is measured
// (the pages compare against BF16 FlashDecoding-v2: OScaR abstract, arXiv
// 2605.19660; ai-papers.net OScaR summary, section "実験結果").
//
// Grid (split, KV head, sequence), one workgroup per compute unit.  Split s
// owns the 128-token chunks s, s + S, ... of its (sequence, KV head), each
// cut into four 32-token pieces.  Two loader waves stream the pieces (keys
// then values, 16 KB) into an LDS ring with direct global -> LDS loads, two
// pieces in flight each; the compute waves take the pieces in a fixed order
// (so results repeat bit for bit) with a base-2 online softmax.  Scores are
// exact bf16 x bf16 products on the matrix cores (query rows x key rows,
// fp32 accumulation); the key rows sit in LDS with their 16-byte chunks
// permuted (chunk j of row t at j ^ (t mod 16)) so that the operand reads
// are free of bank conflicts.  The weighted values accumulate with VALU
// arithmetic: lane l = 16 tq + c owns channels 8c .. 8c+7 of the tokens
// 4s + tq of a piece (s = 0..7).  The compute waves merge in LDS into a
// per-split partial record; merge.hip combines the splits.
#include "decode_common.hpp"

namespace oscar {
namespace {

constexpr int kPieceTokens = 32;
constexpr int kPieceBytes = kPieceTokens * kHeadDim * 2 * 2;   // keys then values
constexpr int kCopiesPerPiece = kPieceBytes / 1024;            // 1 KB per copy instruction
constexpr int kSteps = kPieceTokens / 4;                       // tokens per lane per piece

template <int G>
struct Bf16Cfg {
  // 2 waves per SIMD: a compute wave holds the query, the accumulators and
  // one piece's keys or values (about 200 VGPRs for G = 4)
  static constexpr int kWaves = 8;
  static constexpr int kLoaders = 2;
  static constexpr int kCompute = kWaves - kLoaders;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kRing = (G <= 4) ? 8 : 6;   // pieces in LDS (a multiple of kLoaders)
  static constexpr int kAhead = 2;                 // pieces in flight per loader
  static_assert(kRing % kLoaders == 0 && kAhead * kLoaders <= kRing, "ring");
  static_assert(kAhead * kCopiesPerPiece <= 63, "vector-memory counter limit");
};

template <int G>
struct Bf16Smem {
  float q_raw[G][kHeadDim];
  uint8_t ring[Bf16Cfg<G>::kRing][kPieceBytes];
  MergeSmem<G, Bf16Cfg<G>::kCompute> merge;
  float pv[Bf16Cfg<G>::kCompute][kPieceTokens][G];   // a piece's softmax weights, per compute wave
  int filled[Bf16Cfg<G>::kRing];    // stage s holds piece k = s + kRing * (filled[s] - 1)
  int emptied[Bf16Cfg<G>::kRing];   // times stage s has been read
};

__device__ __forceinline__ void unpack8(const uint4& w, float (&x)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16lo_to_f32(u[e]);
    x[2 * e + 1] = bf16hi_to_f32(u[e]);
  }
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
__global__ __launch_bounds__(Bf16Cfg<G>::kThreads) void decode_bf16_kernel(DecodeBf16Args a) {
  using C = Bf16Cfg<G>;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int tq = lane >> 4;   // token within a group of four
  const int c = lane & 15;    // channels 8c .. 8c+7

  __shared__ Bf16Smem<G> sm;

  const int len = min(max(a.seq_len[b], 0), min(a.capacity, a.max_tokens));
  const int S = a.splits;
  const size_t slice = static_cast<size_t>(b) * a.num_kv_heads + h;
  const size_t row0 = slice * a.capacity;
  const int qh0 = h * G;
  const int last = max(len - 1, 0);
  // this split's pieces: piece k is tokens 32 (k % 4) of chunk split + (k / 4) S
  const int c_end = (len + kGroup - 1) / kGroup;
  const int n_chunks = (c_end > split) ? (c_end - split + S - 1) / S : 0;
  const int n_pieces = 4 * n_chunks;
  auto piece_t0 = [&](int k) { return (split + (k >> 2) * S) * kGroup + kPieceTokens * (k & 3); };

  if (tid < C::kRing) {
    sm.filled[tid] = 0;
    sm.emptied[tid] = 0;
  }
  load_and_rotate_q<G, G>(a.q + (static_cast<size_t>(b) * a.num_q_heads + qh0) * kHeadDim, a.sm_scale * kLog2e,
                          sm.q_raw, nullptr);   // ends with a barrier

  if (wave < C::kLoaders) {
    // ---- loaders: loader i copies the pieces i, i + kLoaders, ... with up
    // to kAhead of them in flight; piece k goes to stage k % kRing once its
    // previous occupant has been read.  Rows past the sequence are read as
    // its last row (always inside the buffer; the compute waves mask them).
    // A piece is published once the wave's in-order vector-memory counter
    // shows that only later pieces' copies are outstanding ----
    const int n_mine = (n_pieces > wave) ? (n_pieces - wave + C::kLoaders - 1) / C::kLoaders : 0;
    int issued = 0;
    for (int j = 0; j < n_mine; ++j) {
      for (; issued < min(j + C::kAhead, n_mine); ++issued) {
        const int k = wave + issued * C::kLoaders;
        const int s = k % C::kRing;
        while (read_flag(&sm.emptied[s], lane) < k / C::kRing) __builtin_amdgcn_s_sleep(1);
        const int t0 = piece_t0(k);
        uint8_t* stage = sm.ring[s];
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
          // lane l fills chunk l % 16 of piece row 4 i + l / 16, which holds
          // chunk (l % 16) ^ (row % 16) of the key row
          const int prow = 4 * i + (lane >> 4);
          const size_t row = row0 + min(t0 + prow, last);
          lds_load16(a.k + row * kHeadDim + 8 * ((lane & 15) ^ (prow & 15)), stage + 1024 * i);
        }
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
          const size_t row = row0 + min(t0 + 4 * i + (lane >> 4), last);
          lds_load16(a.v + row * kHeadDim + 8 * (lane & 15), stage + kPieceBytes / 2 + 1024 * i);
        }
      }
      // the counter wait is the release: the copies are in LDS before the
      // flag store issues
      wait_units_outstanding<kCopiesPerPiece, C::kAhead - 1>(issued - 1 - j);
      const int k = wave + j * C::kLoaders;
      if (lane == 0)
        __hip_atomic_store(&sm.filled[k % C::kRing], k / C::kRing + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    const int cw = wave - C::kLoaders;
    const int gl = lane >> 4;   // MFMA lane group: query rows 4 gl .. 4 gl + 3 / operand K slice
    const int n = lane & 15;    // MFMA row (query head) / column (token of the tile)
    const float scale = a.sm_scale * kLog2e;
    // A operand: query head n (zero rows from G on), channels 32 ks + 8 gl .. +7
    uint4 qa[4];
    {
      const uint16_t* qrow = a.q + ((static_cast<size_t>(b) * a.num_q_heads + qh0) + (n < G ? n : 0)) * kHeadDim + 8 * gl;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 v = *reinterpret_cast<const uint4*>(qrow + 32 * ks);
        qa[ks] = (n < G) ? v : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // running softmax state: m and l per head (wave-uniform), acc per lane
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      m[hh] = -INFINITY;
      l[hh] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[hh][j] = 0.f;
    }
    // piece k goes to SIMD k % 4 (a workgroup's wave w runs on SIMD w % 4),
    // whose compute waves take its pieces in turn: every SIMD gets a quarter
    // of the work, in a fixed assignment
    const int simd = wave % 4;
    const int first_i = (simd < C::kLoaders) ? 1 : 0;
    const int n_simd = (C::kWaves - 1 - simd) / 4 + 1 - first_i;
    float (*pv)[G] = sm.pv[cw];
    for (int k = simd + 4 * (wave / 4 - first_i); k < n_pieces; k += 4 * n_simd) {
      const int s = k % C::kRing;
      const int use = k / C::kRing;
      while (read_flag(&sm.filled[s], lane) <= use) __builtin_amdgcn_s_sleep(1);
      const uint8_t* stage = sm.ring[s];
      const int t0 = piece_t0(k);
      if (t0 >= len) {   // a piece past the end of the sequence (the rest of its last chunk): nothing to add
        if (lane == 0) __hip_atomic_store(&sm.emptied[s], use + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        continue;
      }
      // ---- scores on the matrix cores: tile j = tokens 16 j .. 16 j + 15;
      // lane holds rows 4 gl + r (heads) of column n ----
      float lg[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int prow = 16 * j + n;
        f32x4_t cacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const uint4 kb = *reinterpret_cast<const uint4*>(stage + 256 * prow + 16 * ((4 * ks + gl) ^ n));
          cacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[ks]),
                                                         __builtin_bit_cast(bf16x8_t, kb), cacc, 0, 0, 0);
        }
        const bool valid = t0 + prow < len;
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[j][r] = valid ? cacc[r] * scale : -INFINITY;
      }
      // the values of the piece, then the stage may be refilled
      uint4 vb[kSteps];
#pragma unroll
      for (int i = 0; i < kSteps; ++i)
        vb[i] = *reinterpret_cast<const uint4*>(stage + kPieceBytes / 2 + 1024 * i + 16 * lane);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (lane == 0) __hip_atomic_store(&sm.emptied[s], use + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      // ---- online softmax (base 2) per head: head 4 gl + r is row r of lane group gl ----
      float alpha[G];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mx = row_max16(fmaxf(lg[0][r], lg[1][r]));   // finite for the heads: a token is valid
        float mh[2], mn[2];
#pragma unroll
        for (int g2 = 0; g2 < (G + 3) / 4; ++g2) {
          const int hh = 4 * g2 + r;
          if (hh < G) {
            const float mxh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 16 * g2));
            mh[g2] = fmaxf(m[hh], mxh);
            alpha[hh] = fast_exp2(m[hh] - mh[g2]);   // 0 while m was -inf
            m[hh] = mh[g2];
          }
          mn[g2] = (hh < G) ? mh[g2] : 0.f;
        }
        const float m_row = ((G + 3) / 4 > 1 && gl == 1) ? mn[(G + 3) / 4 - 1] : mn[0];
        const float p0 = fast_exp2(lg[0][r] - m_row), p1 = fast_exp2(lg[1][r] - m_row);
        const float ps = row_sum16(p0 + p1);
#pragma unroll
        for (int g2 = 0; g2 < (G + 3) / 4; ++g2) {
          const int hh = 4 * g2 + r;
          if (hh < G) {
            l[hh] = fmaf(l[hh], alpha[hh],
                         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ps), 16 * g2)));
            if (gl == g2) {
              pv[n][hh] = p0;
              pv[16 + n][hh] = p1;
            }
          }
        }
      }
      wave_sync_lds();
      // ---- weighted values: this lane's tokens 4 i + tq and channels 8c .. 8c+7 ----
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[hh][j] *= alpha[hh];
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        float vx[8];
        unpack8(vb[i], vx);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float p = pv[4 * i + tq][hh];
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[hh][j] = fmaf(p, vx[j], acc[hh][j]);
        }
      }
      wave_sync_lds();   // pv is rewritten by the next piece only after these reads
    }
    // ---- sums over the four token rows of the wave -> merge slot ----
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[hh][j] = sum_over_rows(acc[hh][j]);
      if (tq == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.merge.acc[cw][hh][8 * c + j] = acc[hh][j];
        if (c == 0) {
          sm.merge.m[cw][hh] = m[hh];
          sm.merge.l[cw][hh] = l[hh];
        }
      }
    }
  }
  const size_t partial_base = (static_cast<size_t>(b) * a.num_q_heads + qh0) * a.splits;
  write_partial<G, C::kCompute>(sm.merge, a.partials, partial_base, split, a.splits);
}

template <int G>
hipError_t launch_g(const DecodeBf16Args& a, int32_t batch, hipStream_t s) {
  dim3 grid(a.splits, a.num_kv_heads, batch);
  hipLaunchKernelGGL(decode_bf16_kernel<G>, grid, dim3(Bf16Cfg<G>::kThreads), 0, s, a);
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
