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
// weight 1, 4 or 16, divided out of the other operand; the top field is
// stored as 64 - 64 c against a negated operand), and the fp32 operand (q'
// for the scores, p * vs for the values) is written as a 32-bit fixed-point
// integer with a per-group power-of-two scale and split into four signed
// base-256 digits, one matrix row per (head, digit).  The int32 results are
// recombined exactly and scaled back, so the only rounding is the
// fixed-point step of q' and p * vs (2^-24 of the group's largest value)
// and fp32 rounding.
//
// Work split: grid (split, KV head, sequence), about one workgroup per
// compute unit, all resident at once; split s owns the groups s, s + S, ...
// Inside a workgroup two loader waves stream the groups' blocks into an LDS
// ring with direct global -> LDS copies, and the compute waves take the
// groups in a fixed round-robin over the SIMDs, each keeping a base-2 online
// softmax (a fixed assignment keeps the summation order, so results repeat
// bit for bit).  Lane roles inside a compute wave (lane = 16 * r + n,
// w = n >> 1, u = 2 (n & 1)):
//  * score / softmax lane (r, n): head r of the row block, the tokens
//    16w + 4b + u + c of the group (b = 0..3, c = 0..1; column n of tile
//    4c + b);
//  * q' lane (r, n): head r, the channels 16w + 4b + u + c;
//  * value lane (r, n): head r, channels 16j + n of channel tile j.
// With these sets, the four digits of the values a lane owns for one c land
// in four consecutive bytes of one MFMA operand row, so each lane stages
// its operand bytes with one 8-byte LDS write per digit row.
// The compute waves' states (and the bf16 tail's) merge in LDS into one
// partial record per split; merge.hip combines the splits.
#include "decode_common.hpp"

namespace oscar {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// After the spread (spread_codes) the code at bit position 2r of its byte
// carries the weight 4^r (masks 0x03, 0x0C, 0x30); the other operand is
// multiplied by 64 / 4^r so that every code ends up with weight 64.  The top
// field is stored as 64 - 64 c (so that it fits int8) and its operand is
// negated: (-x) (64 - 64 c) = 64 x c - 64 x, the -64 x being cancelled by
// the accumulator's start value.
__device__ constexpr float kFac[4] = {64.f, 16.f, 4.f, -1.f};

// 16 packed codes (bits 2k..2k+1 = code k) -> 16 int8 lanes of an MFMA
// operand.  Byte b of output dword r holds code 4b + r times 4^r for r < 3;
// the top field holds 64 - 64 * code (one XOR turns 64 c into it), paired
// with a negated operand and the start value of field3_bias.
__device__ __forceinline__ v4i spread_codes(uint32_t x) {
  v4i o;
  o[0] = static_cast<int>(x & 0x03030303u);
  o[1] = static_cast<int>(x & 0x0C0C0C0Cu);
  o[2] = static_cast<int>(x & 0x30303030u);
  o[3] = static_cast<int>((x & 0xC0C0C0C0u) ^ 0x40404040u);
  return o;
}

// -64 * (sum of the A operand over the K positions that carry top-field
// codes): the start value of a two-step (K = 128) product with A halves a0,
// a1 that removes the constant 64 of the top field, leaving -64 c times the
// (negated) operand there.
__device__ __forceinline__ v4i field3_bias(const v4i& a0, const v4i& a1) {
  const v4i bm64 = {0, 0, 0, static_cast<int>(0xC0C0C0C0u)};   // -64 at the top-field positions
  v4i c = {0, 0, 0, 0};
  c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bm64, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bm64, c, 0, 0, 0);
  return c;
}

// Four signed base-256 digits of an integer v, |v| < 2^31 - 2^24, given as
// v_off = v + 0x808080: digit k is byte k of the result read as int8
// (balanced representation).
__device__ __forceinline__ uint32_t balanced_digits_off(int v_off) {
  return static_cast<uint32_t>(v_off) ^ 0x808080u;
}

// An integer within one unit of y (|y| < 2^30), plus 0x808080, for
// balanced_digits_off.  The offset and the rounding half are added in fp32
// and the sum is truncated: round half up wherever the sum is positive.
__device__ __forceinline__ int fixed_off(float y) { return static_cast<int>(y + 8421504.5f); }

// 2^x for x <= 0 with the hardware exponential: results below 2^-126 flush
// to zero (negligible weights in a softmax); 2^-inf = 0.
// Maximum over the 16 lanes of a DPP row of non-negative floats (compared as
// their bit patterns, which order them).
__device__ __forceinline__ float row_max16_nonneg(float x) {
  int v = __float_as_int(x);
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppQuadXor1, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppQuadXor2, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppRowRor4, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppRowRor8, 0xF, 0xF, true));
  return __int_as_float(v);
}

// Maximum over the 16 lanes of a DPP row of floats that are not NaN: each
// float is mapped to an int with the same order (negative values have their
// magnitude bits flipped), reduced, and mapped back (the map is its own
// inverse).
__device__ __forceinline__ int float_order_key(int bits) { return bits ^ ((bits >> 31) & 0x7FFFFFFF); }
__device__ __forceinline__ float row_max16_ordered(float x) {
  int v = float_order_key(__float_as_int(x));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppQuadXor1, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppQuadXor2, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppRowRor4, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppRowRor8, 0xF, 0xF, true));
  return __int_as_float(float_order_key(v));
}

// Recombine the four digit rows of one (head, column) of an MFMA result.
__device__ __forceinline__ float digits_value(const v4i& c) {
  const int hi = c[3] * 256 + c[2];
  const int lo = c[1] * 256 + c[0];
  return fmaf(static_cast<float>(hi), 65536.f, static_cast<float>(lo));
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
struct GroupBytes {
  u32x2 kd[8];      // K codes of token tau(4c+b) (see lane roles), dwords 2g and 2g+1 of the row
  u32x2 vd[8];      // V codes of channel 16j + n, dwords 2g and 2g+1 of the channel row
  uint32_t nrm[4];  // fp16 norms of tokens 16w + 4b + u + {0, 1}
  u32x2 vsz[4];     // (vs | vz << 16) of tokens 16w + 4b + u + {0, 1}
  u32x2 ksz[4];     // (s | z << 16) of channels 16w + 4b + u + {0, 1}
};

// A group's block in LDS, as a loader wave copies it with direct global ->
// LDS loads (16 bytes per lane per instruction, one contiguous kilobyte per
// wave instruction).  The copies permute the block's 16-byte pieces so that
// the compute waves' 8-byte operand reads are free of LDS bank conflicts
// (gfx950 serves 32 lanes of an 8-byte read per cycle from 64 four-byte
// banks, so each read instruction should cover 256 contiguous bytes per 32
// lanes):
//  * key codes: slot 16 (4 b + 2 c + hh) + n holds half hh (16 bytes) of the
//    row of token 16 (n >> 1) + 4 b + 2 (n & 1) + c, the token of column n of
//    score tile 4 c + b (see the lane roles above);
//  * value codes: slot 32 j + 16 hh + n holds half hh of the row of channel
//    16 j + n;
//  * key and value (s, z) pairs: 16-byte piece p (four channels or tokens) of
//    each 512-byte array at slot p ^ 2 ((p >> 4) & 1);
//  * norms: 16-byte piece p (eight tokens) at slot p ^ ((p >> 3) & 1) (a
//    4-byte read serves 32 lanes per cycle from 32 banks).
constexpr int kStageK = OSCAR_BLOCK_K_CODES;   // 4096 B: key code half rows
constexpr int kStageV = OSCAR_BLOCK_V_CODES;   // 4096 B: value code half rows
constexpr int kStageKsz = OSCAR_BLOCK_K_SZ;    // 512 B: (s, z) per channel
constexpr int kStageVsz = OSCAR_BLOCK_V_SZ;    // 512 B: (vs, vz) per token
constexpr int kStageNorm = OSCAR_BLOCK_K_NORM; // 256 B: fp16 norms
constexpr int kStageBytes = OSCAR_BLOCK_BYTES;
constexpr int kDmaPerGroup = 10;   // load instructions per group (the norms take one of them)
static_assert(kStageV == 4096 && kStageKsz == 8192 && kStageVsz == kStageKsz + 512 && kStageNorm == 9216 &&
                  kStageBytes == 9472,
              "the copy below assumes this block layout");

__device__ __forceinline__ int sz_piece_slot(int p) { return p ^ (((p >> 4) & 1) << 1); }   // an involution
__device__ __forceinline__ int norm_piece_slot(int p) { return p ^ ((p >> 3) & 1); }        // an involution

// Source byte offsets, inside a group block, of the 16 bytes a loader lane
// copies with each of the group's load instructions (fixed for the kernel).
struct LoaderLane {
  int k[4];   // key code slots 64 j + lane
  int v[4];   // value code slots 64 j + lane
  int sz;     // (s, z) slot lane of the 1 KB of pairs
  int nrm;    // norm slot lane (lanes 0..15)
};

__device__ __forceinline__ LoaderLane loader_lane(int lane) {
  LoaderLane o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sl = 64 * j + lane;
    const int cls = sl >> 4, n = sl & 15;
    const int b = cls >> 2, c = (cls >> 1) & 1, hh = cls & 1;
    o.k[j] = kStageK + 32 * (16 * (n >> 1) + 4 * b + 2 * (n & 1) + c) + 16 * hh;
    o.v[j] = kStageV + 32 * (16 * (sl >> 5) + n) + 16 * ((sl >> 4) & 1);
  }
  o.sz = kStageKsz + 512 * (lane >> 5) + 16 * sz_piece_slot(lane & 31);
  o.nrm = kStageNorm + 16 * norm_piece_slot(lane & 15);
  return o;
}

// The kDmaPerGroup loads that copy the group block at blk into a stage.
__device__ __forceinline__ void dma_group(uint8_t* stage, const uint8_t* blk, const LoaderLane& o, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) lds_load16(blk + o.k[j], stage + kStageK + 1024 * j);
#pragma unroll
  for (int j = 0; j < 4; ++j) lds_load16(blk + o.v[j], stage + kStageV + 1024 * j);
  lds_load16(blk + o.sz, stage + kStageKsz);
  if (lane < 16) lds_load16(blk + o.nrm, stage + kStageNorm);
}

// Byte offsets inside a stage of the operands a lane reads (see the lane
// roles above and the stage layout), fixed for the whole kernel, so that
// each read of a group is one of these plus an immediate.
struct StageLane {
  int k;      // key codes of tile 4 c + b: + 512 c + 1024 b
  int v;      // value codes of channel tile j: + 512 j
  int nrm[2]; // norms of tokens base + 4 b: nrm[b >> 1] + 8 (b & 1)
  int vsz[2]; // value (s, z) of tokens base + 4 b: vsz[b >> 1] + 16 b
  int ksz[2]; // key (s, z) of channels base + 4 b: ksz[b >> 1] + 16 b
};

__device__ __forceinline__ StageLane stage_lane(int lane) {
  const int gl = lane >> 4;
  const int n = lane & 15;
  const int w = n >> 1;
  StageLane o;
  const int half = 256 * (gl >> 1) + 16 * n + 8 * (gl & 1);
  o.k = kStageK + half;
  o.v = kStageV + half;
  // norms of tokens 16 w + 4 b + u (+1): piece 2 w + (b >> 1) at slot
  // (2 w + (b >> 1)) ^ s, s = w >> 2, at byte 8 (b & 1) + 2 u of the piece
  const int sn = w >> 2;
  o.nrm[0] = kStageNorm + 32 * w + 16 * sn + 4 * (n & 1);
  o.nrm[1] = kStageNorm + 32 * w + 16 * (1 - sn) + 4 * (n & 1);
  // (s, z) of channels / tokens 16 w + 4 b + u (+1): piece 4 w + b at slot
  // (4 w + b) ^ x, x = 2 (w >> 2): 4 w + b + x for b < 2, 4 w + b - x for b >= 2
  const int x = 2 * (w >> 2);
  const int pair = 64 * w + 8 * (n & 1);
  o.vsz[0] = kStageVsz + pair + 16 * x;
  o.vsz[1] = kStageVsz + pair - 16 * x;
  o.ksz[0] = kStageKsz + pair + 16 * x;
  o.ksz[1] = kStageKsz + pair - 16 * x;
  return o;
}

// Registers of the group being computed: 28 single LDS reads in one block,
// which waits for all of them at its end.  (Left to itself the compiler
// pairs reads 512 or 16 bytes apart into one paired instruction, which
// gfx950 serves with bank conflicts for these layouts; single reads of the
// layouts above have none.)
__device__ __forceinline__ void read_stage(GroupBytes& r, const uint8_t* stage, const StageLane& o) {
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(stage));
  const uint32_t ak = base + o.k, av = base + o.v;
  const uint32_t an0 = base + o.nrm[0], an1 = base + o.nrm[1];
  const uint32_t avs0 = base + o.vsz[0], avs1 = base + o.vsz[1];
  const uint32_t aks0 = base + o.ksz[0], aks1 = base + o.ksz[1];
  asm volatile(
      "ds_read_b64 %0, %28\n\t"
      "ds_read_b64 %1, %28 offset:1024\n\t"
      "ds_read_b64 %2, %28 offset:2048\n\t"
      "ds_read_b64 %3, %28 offset:3072\n\t"
      "ds_read_b64 %4, %28 offset:512\n\t"
      "ds_read_b64 %5, %28 offset:1536\n\t"
      "ds_read_b64 %6, %28 offset:2560\n\t"
      "ds_read_b64 %7, %28 offset:3584\n\t"
      "ds_read_b64 %8, %29\n\t"
      "ds_read_b64 %9, %29 offset:512\n\t"
      "ds_read_b64 %10, %29 offset:1024\n\t"
      "ds_read_b64 %11, %29 offset:1536\n\t"
      "ds_read_b64 %12, %29 offset:2048\n\t"
      "ds_read_b64 %13, %29 offset:2560\n\t"
      "ds_read_b64 %14, %29 offset:3072\n\t"
      "ds_read_b64 %15, %29 offset:3584\n\t"
      "ds_read_b32 %16, %30\n\t"
      "ds_read_b32 %17, %30 offset:8\n\t"
      "ds_read_b32 %18, %31\n\t"
      "ds_read_b32 %19, %31 offset:8\n\t"
      "ds_read_b64 %20, %32\n\t"
      "ds_read_b64 %21, %32 offset:16\n\t"
      "ds_read_b64 %22, %33 offset:32\n\t"
      "ds_read_b64 %23, %33 offset:48\n\t"
      "ds_read_b64 %24, %34\n\t"
      "ds_read_b64 %25, %34 offset:16\n\t"
      "ds_read_b64 %26, %35 offset:32\n\t"
      "ds_read_b64 %27, %35 offset:48\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.kd[0]), "=&v"(r.kd[1]), "=&v"(r.kd[2]), "=&v"(r.kd[3]), "=&v"(r.kd[4]), "=&v"(r.kd[5]),
        "=&v"(r.kd[6]), "=&v"(r.kd[7]), "=&v"(r.vd[0]), "=&v"(r.vd[1]), "=&v"(r.vd[2]), "=&v"(r.vd[3]),
        "=&v"(r.vd[4]), "=&v"(r.vd[5]), "=&v"(r.vd[6]), "=&v"(r.vd[7]), "=&v"(r.nrm[0]), "=&v"(r.nrm[1]),
        "=&v"(r.nrm[2]), "=&v"(r.nrm[3]), "=&v"(r.vsz[0]), "=&v"(r.vsz[1]), "=&v"(r.vsz[2]), "=&v"(r.vsz[3]),
        "=&v"(r.ksz[0]), "=&v"(r.ksz[1]), "=&v"(r.ksz[2]), "=&v"(r.ksz[3])
      : "v"(ak), "v"(av), "v"(an0), "v"(an1), "v"(avs0), "v"(avs1), "v"(aks0), "v"(aks1)
      : "memory");
}

__device__ __forceinline__ uint32_t pick(const u32x2& v, int c) { return c ? v.y : v.x; }
__device__ __forceinline__ float f16_lo(uint32_t w) { return f16_bits_to_f32(static_cast<uint16_t>(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return f16_bits_to_f32(static_cast<uint16_t>(w >> 16)); }

// 4x4 byte transpose: y[k] byte b = x[b] byte k.
__device__ __forceinline__ void transpose4(const uint32_t (&x)[4], uint32_t (&y)[4]) {
  const uint32_t t01_lo = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);
  const uint32_t t01_hi = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);
  const uint32_t t23_lo = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
  const uint32_t t23_hi = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
  y[0] = __builtin_amdgcn_perm(t23_lo, t01_lo, 0x05040100u);
  y[1] = __builtin_amdgcn_perm(t23_lo, t01_lo, 0x07060302u);
  y[2] = __builtin_amdgcn_perm(t23_hi, t01_hi, 0x05040100u);
  y[3] = __builtin_amdgcn_perm(t23_hi, t01_hi, 0x07060302u);
}

// MFMA A operand staging: per (operand half or K step, lane group) a block of
// 16 rows x 16 bytes plus 16 bytes of padding, so that the 8-byte writes of
// a wave spread over all LDS banks.
constexpr int kOpRow = 16;
constexpr int kOpBlock = 16 * kOpRow + 16;

// Write the digit rows of the eight fixed-point values x[c][b] a lane owns
// (c = 0..1, b = 0..3) into operand block `blk` (a pointer to [2][4][kOpBlock]).
__device__ __forceinline__ void stage_digits(uint8_t* blk, const uint32_t (&x)[2][4], int gl, int n) {
  uint32_t y0[4], y1[4];
  transpose4(x[0], y0);
  transpose4(x[1], y1);
  const int w = n >> 1;
  uint8_t* dst = blk + ((w & 1) * 4 + (w >> 1)) * kOpBlock + 8 * (n & 1);
#pragma unroll
  for (int k = 0; k < 4; ++k) *reinterpret_cast<uint2*>(dst + (4 * gl + k) * kOpRow) = make_uint2(y0[k], y1[k]);
}

__device__ __forceinline__ v4i read_operand(const uint8_t* blk, int half, int gl, int n) {
  return *reinterpret_cast<const v4i*>(blk + (half * 4 + gl) * kOpBlock + n * kOpRow);
}

// Query set-up by one wave.  Lane l holds, for row block rb, the elements
// 8 (l % 16) .. 8 (l % 16) + 7 of head 4 rb + l / 16 (zero for heads >= G).
template <int G, int RB>
__device__ __forceinline__ void fetch_q_wave(const uint16_t* q, int lane, uint4 (&raw)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int head = 4 * rb + (lane >> 4);
    const uint4 v = reinterpret_cast<const uint4*>(q)[head < G ? 16 * head + (lane & 15) : 0];
    raw[rb] = (head < G) ? v : make_uint4(0u, 0u, 0u, 0u);
  }
}

// q_raw = q * scale and q_rot = (H q) * scale, H the orthonormal Sylvester
// Hadamard matrix of order 128 in natural order: butterflies (x, y) ->
// (x + y, x - y) over index pairs differing in one bit, the three low bits
// inside a lane, the four high bits across the 16 lanes of a row.
template <int RB>
__device__ __forceinline__ void rotate_q_wave(const uint4 (&raw)[RB], float scale, float (*q_raw)[kHeadDim],
                                              float (*q_rot)[kHeadDim], int lane) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = 4 * rb + (lane >> 4);
    const int d0 = 8 * (lane & 15);
    const uint32_t w[4] = {raw[rb].x, raw[rb].y, raw[rb].z, raw[rb].w};
    float x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16lo_to_f32(w[k]);
      x[2 * k + 1] = bf16hi_to_f32(w[k]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) q_raw[row][d0 + j] = x[j] * scale;
#pragma unroll
    for (int bit = 1; bit < 8; bit <<= 1)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (!(j & bit)) {
          const float a = x[j], b = x[j | bit];
          x[j] = a + b;
          x[j | bit] = a - b;
        }
#pragma unroll
    for (int lb = 1; lb < 16; lb <<= 1) {
      const bool upper = lane & lb;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float y = __shfl_xor(x[j], lb, kWave);
        x[j] = upper ? y - x[j] : x[j] + y;
      }
    }
    const float norm = scale * 0.088388347648318440550f;   // 1/sqrt(128)
#pragma unroll
    for (int j = 0; j < 8; ++j) q_rot[row][d0 + j] = x[j] * norm;
  }
}

template <int G>
struct Int2Cfg {
  static constexpr int kRB = (G + 3) / 4;  // 16-row blocks of (head, digit) rows
  static constexpr int kRows = kRB * 4;    // heads incl. zero padding
  // One workgroup per compute unit: 16 waves (4 per SIMD) while the kernel
  // fits in 128 VGPRs, 8 waves for 8 query heads per KV head.  The first
  // kLoaders waves stream the cache into LDS; the others compute.  Every
  // SIMD spends about as long on its share of the groups as HBM takes to
  // deliver them, and with 4 waves instead of 3 it hides more of each
  // group's dependency stalls, so no backlog builds up on the two SIMDs
  // that also run the loaders.
  static constexpr int kWaves = (kRB == 1) ? 16 : 8;
  static constexpr int kLoaders = 2;
  static constexpr int kCompute = kWaves - kLoaders;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kSlots = kCompute + 2;  // one merge slot per compute wave + two for the bf16 tail
  static constexpr int kRing = 8;   // group stages in LDS (a multiple of kLoaders; 10 would not fit)
  static_assert(kWaves % 4 == 0 && kLoaders < 4, "compute waves on every SIMD");
  static constexpr int kAhead = 2;           // groups each loader has in flight (kAhead * kDmaPerGroup <= 63)
  static_assert(kRing % kLoaders == 0, "a stage is always refilled by the same loader");
  static_assert(kAhead * kDmaPerGroup <= 63, "vector-memory counter limit");
};

template <int G>
struct Int2Smem {
  float q_raw[Int2Cfg<G>::kRows][kHeadDim];   // q * sm_scale * log2(e)
  float q_rot[Int2Cfg<G>::kRows][kHeadDim];   // (H q) * sm_scale * log2(e)
  float tail_p[kGroup][G];                     // softmax weights of the bf16 tail tokens (two halves)
  // per compute wave and row block: an MFMA A operand staged as
  // [half][lane group][row][16 bytes] (the scores' q digits, then the
  // values' p digits)
  uint8_t a_op[Int2Cfg<G>::kCompute][Int2Cfg<G>::kRB][2 * 4 * kOpBlock];
  uint8_t ring[Int2Cfg<G>::kRing][kStageBytes];      // group stages
  // key (s, z) pairs of the split's last four groups, group k at [k % 4],
  // in the stage's piece order, fetched at the start by the waves that
  // compute them
  uint8_t last_ksz[4][512];
  MergeSmem<G, Int2Cfg<G>::kSlots> merge;              // final state of each compute wave, and of the bf16 tail
  int filled[Int2Cfg<G>::kRing];    // stage s holds group index k = s + kRing * (filled[s] - 1)
  int emptied[Int2Cfg<G>::kRing];   // times stage s has been read into registers
  int q_ready;                      // set by wave 0 once q_raw and q_rot are written
};

// Running softmax state of one wave: per row block, m (uniform over the
// head's 16 lanes), per-lane partial l and sum p * vz, and acc for channels
// 16j + n.
template <int RB>
struct WaveRun {
  float m[RB], l[RB], z[RB], acc[RB][8];
};

// The query side of a group's scores, which depends only on the group's key
// (s, z) pairs: the A operand q' = Hq * s16 as 4-digit fixed point (staged
// and read back), its top-field bias, Z = Hq . z16 and the scale back.
template <int RB>
struct QPrep {
  v4i aq[RB][2], bias[RB];
  float Zg[RB], inv_q[RB];
};

template <int G>
__device__ __forceinline__ void q_prep(const u32x2 (&ksz)[4], const float (&qv)[Int2Cfg<G>::kRB][2][4],
                                       const float (&fac)[2], Int2Smem<G>& sm, int wave, int gl, int n,
                                       QPrep<Int2Cfg<G>::kRB>& p) {
  constexpr int RB = Int2Cfg<G>::kRB;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float qs[2][4];
    float zp = 0.f, amax = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint32_t w = pick(ksz[b], c);
        qs[c][b] = fmaf(qv[rb][c][b], f16_lo(w), 0.f);   // one mixed-precision FMA
        zp = fmaf(qv[rb][c][b], f16_hi(w), zp);
        amax = fmaxf(amax, fabsf(qs[c][b]));
      }
    amax = row_max16_nonneg(amax);
    p.Zg[rb] = row_sum16(zp);
    int e;
    frexpf(amax, &e);                        // amax < 2^e
    const float sc = ldexpf(1.f, 24 - e);    // |q' * sc| < 2^24, |q' * sc * fac| < 2^30
    p.inv_q[rb] = ldexpf(1.f, e - 30);       // 1 / (sc * 64)
    uint32_t x[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < 4; ++b) x[c][b] = balanced_digits_off(fixed_off(qs[c][b] * (sc * fac[c])));
    stage_digits(sm.a_op[wave][rb], x, gl, n);
  }
  wave_sync_lds();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    p.aq[rb][0] = read_operand(sm.a_op[wave][rb], 0, gl, n);
    p.aq[rb][1] = read_operand(sm.a_op[wave][rb], 1, gl, n);
    p.bias[rb] = field3_bias(p.aq[rb][0], p.aq[rb][1]);
  }
}

// Score phase of one quantized 128-token group with its query side p:
// scores on the matrix cores, online softmax update, p * vs staged as the
// value phase's A operand.  Returns the softmax rescale factors in alpha
// and inv_p.
template <int G>
__device__ __forceinline__ void score_phase(const GroupBytes& cur, const QPrep<Int2Cfg<G>::kRB>& p, int t0, int t_end,
                                            Int2Smem<G>& sm, WaveRun<Int2Cfg<G>::kRB>& st, int wave, int gl, int n,
                                            const float (&fac)[2], float (&alpha)[Int2Cfg<G>::kRB],
                                            float (&inv_p)[Int2Cfg<G>::kRB]) {
  constexpr int RB = Int2Cfg<G>::kRB;
  const int tok_base = t0 + 16 * (n >> 1) + 2 * (n & 1);

  // ---- scores: column n of tile i = 4c + b is token 16w + 4b + u + c ----
  float logit[RB][2][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = i >> 2, b = i & 3;
    const v4i b0 = spread_codes(cur.kd[i].x);
    const v4i b1 = spread_codes(cur.kd[i].y);
    const float n16 = c ? f16_hi(cur.nrm[b]) : f16_lo(cur.nrm[b]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(p.aq[rb][0], b0, p.bias[rb], 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(p.aq[rb][1], b1, acc, 0, 0, 0);
      logit[rb][c][b] = fmaf(fmaf(digits_value(acc), p.inv_q[rb], p.Zg[rb]), n16, 0.f);
    }
  }
  if (t0 + kGroup > t_end) {   // a group cut short by max_tokens: mask the tokens beyond it
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i >> 2, b = i & 3;
      const bool valid = tok_base + 4 * b + c < t_end;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) logit[rb][c][b] = valid ? logit[rb][c][b] : -INFINITY;
    }
  }

  // ---- online softmax (base 2) and p * vs as 4-digit fixed point ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float gm = logit[rb][0][0];
#pragma unroll
    for (int i = 1; i < 8; ++i) gm = fmaxf(gm, logit[rb][i >> 2][i & 3]);
    gm = row_max16_ordered(gm);
    const float m_new = (gm > st.m[rb]) ? gm : st.m[rb];   // finite: every group has a valid token
    alpha[rb] = fast_exp2(st.m[rb] - m_new);   // 0 while m was -inf
    st.m[rb] = m_new;
    float ls = 0.f, zs = 0.f, pmax = 0.f;
    float pv[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t w = pick(cur.vsz[b], c);
        const float p = fast_exp2(logit[rb][c][b] - m_new);
        ls += p;
        zs = fmaf(p, f16_hi(w), zs);
        pv[c][b] = fmaf(p, f16_lo(w), 0.f);
        pmax = fmaxf(pmax, pv[c][b]);
      }
    st.l[rb] = fmaf(st.l[rb], alpha[rb], ls);
    st.z[rb] = fmaf(st.z[rb], alpha[rb], zs);
    pmax = row_max16_nonneg(pmax);
    int e2;
    frexpf(pmax, &e2);                       // p * vs < 2^e2 for this head and group
    const float sc2 = ldexpf(1.f, 24 - e2);
    inv_p[rb] = ldexpf(1.f, e2 - 30);
    uint32_t x[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < 4; ++b) x[c][b] = balanced_digits_off(fixed_off(pv[c][b] * (sc2 * fac[c])));
    stage_digits(sm.a_op[wave][rb], x, gl, n);
  }
}

// Value phase: weighted value codes on the matrix cores (channel tile j,
// column n = channel 16j + n), folded into the running accumulators.
template <int G>
__device__ __forceinline__ void value_phase(const GroupBytes& cur, Int2Smem<G>& sm, WaveRun<Int2Cfg<G>::kRB>& st,
                                            int wave, int gl, int n, const float (&alpha)[Int2Cfg<G>::kRB],
                                            const float (&inv_p)[Int2Cfg<G>::kRB]) {
  constexpr int RB = Int2Cfg<G>::kRB;
  wave_sync_lds();
  v4i ap[RB][2], bias[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    ap[rb][0] = read_operand(sm.a_op[wave][rb], 0, gl, n);
    ap[rb][1] = read_operand(sm.a_op[wave][rb], 1, gl, n);
    bias[rb] = field3_bias(ap[rb][0], ap[rb][1]);
  }

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const v4i b0 = spread_codes(cur.vd[j].x);
    const v4i b1 = spread_codes(cur.vd[j].y);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ap[rb][0], b0, bias[rb], 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ap[rb][1], b1, acc, 0, 0, 0);
      st.acc[rb][j] = fmaf(digits_value(acc), inv_p[rb], st.acc[rb][j] * alpha[rb]);
    }
  }
  // the next group rewrites a_op only after this wave has read it
  wave_sync_lds();
}

template <int G>
__global__ __launch_bounds__(Int2Cfg<G>::kThreads) void decode_int2_kernel(DecodeInt2Args a) {
  using C = Int2Cfg<G>;
  constexpr int RB = C::kRB;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: loop control in scalar registers
  const int lane = tid & 63;
  const int gl = lane >> 4;   // lane group: head of the row block / operand K slice
  const int n = lane & 15;

  __shared__ Int2Smem<G> sm;

  const int groups_cap = a.capacity / kGroup;
  // Split s owns the groups s, s + S, s + 2S, ... (S = number of splits):
  // at any moment the workgroups of a head read neighbouring groups, which
  // spreads the traffic over all memory channels.
  const int S = a.splits;
  const size_t slice = static_cast<size_t>(b) * a.num_kv_heads + h;
  const int qh0 = h * G;

  // Wave roles: waves 0 .. kLoaders-1 (started first) stream the cache,
  // the others (compute wave cw = wave - kLoaders) compute.
  const bool loader = wave < C::kLoaders;
  const int cw = wave - C::kLoaders;

  // Start-up.  Compute wave 0 requests the query; the loaders request their
  // first groups right after the barrier, before anything waits for the
  // sequence lengths: the first groups are chosen from the capacity alone
  // (always inside the buffer) and are simply not used if the sequence turns
  // out to be shorter.  (A wave issuing cache copies can stall on issue for
  // a while, so no wave issues them before the barrier.)
  uint4 q_in[RB];
  if (cw == 0) fetch_q_wave<G, RB>(a.q + (static_cast<size_t>(b) * a.num_q_heads + qh0) * kHeadDim, lane, q_in);
  if (tid < C::kRing) {
    sm.filled[tid] = 0;
    sm.emptied[tid] = 0;
  }
  if (tid == 0) sm.q_ready = 0;
  __syncthreads();

  // block of the split's k-th group (a table lookup for a paged cache)
  auto group_block = [&](int k) {
    return a.blocks + group_block_index(a.block_table, a.num_pages, groups_cap, a.num_kv_heads, b, h, split + k * S) *
                          static_cast<size_t>(kStageBytes);
  };
  int issued = 0;   // groups this loader has requested, in order (its j-th is k = wave + j kLoaders)
  if (loader) {
    const LoaderLane ll = loader_lane(lane);
    static_assert(C::kAhead * C::kLoaders <= C::kRing, "the first groups go to unused stages");
#pragma unroll
    for (int j = 0; j < C::kAhead; ++j) {
      const int k = wave + j * C::kLoaders;
      if (split + k * S >= groups_cap) break;
      dma_group(sm.ring[k % C::kRing], group_block(k), ll, lane);
      ++issued;
    }
  }

  // The lengths, read with scalar loads and waited for with the scalar
  // counter, so that the wait does not include the cache copies above.
  int nq, nt;
  asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(nq), "=&s"(nt)
               : "s"(a.n_quant + b), "s"(a.n_tail + b)
               : "memory");
  nq = min(max(nq, 0) & ~(kGroup - 1), a.capacity);
  nt = min(max(nt, 0), kGroup);
  if (a.k_tail == nullptr || a.v_tail == nullptr) nt = 0;
  const int total = min(nq + nt, a.max_tokens);
  const int n_groups = (total + kGroup - 1) / kGroup;
  const int g_qend = min(n_groups, nq / kGroup);   // quantized groups end here; a tail group may follow
  // this split's quantized groups: index k is group split + k S
  const int n_k = (g_qend > split) ? (g_qend - split + S - 1) / S : 0;

  WaveRun<RB> st;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    st.m[rb] = -INFINITY;
    st.l[rb] = 0.f;
    st.z[rb] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[rb][j] = 0.f;
  }

  if (loader) {
    // ---- loaders: stream the split's groups through the ring ----
    // Loader i copies the groups k = i, i + kLoaders, ... with up to kAhead
    // of them in flight; group k goes to stage k % kRing once its previous
    // occupant (k - kRing, the same loader's) has been read into registers.
    // A group is published once its copies have reached LDS, which the
    // wave's in-order vector-memory counter shows when only the loads of
    // later groups are outstanding.
    const int n_mine = (n_k > wave) ? (n_k - wave + C::kLoaders - 1) / C::kLoaders : 0;
    const LoaderLane ll = loader_lane(lane);
    // the block of the next group to request, looked up one request ahead
    // (a paged cache's table entry is then read long before it is needed)
    const uint8_t* next_blk = (issued < n_mine) ? group_block(wave + issued * C::kLoaders) : a.blocks;
    for (int j = 0; j < n_mine; ++j) {
      for (; issued < min(j + C::kAhead, n_mine); ++issued) {
        const int k = wave + issued * C::kLoaders;
        const int s = k % C::kRing;
        const int use = k / C::kRing;   // earlier occupants of the stage
        const uint8_t* blk = next_blk;
        if (issued + 1 < n_mine) next_blk = group_block(k + C::kLoaders);
        while (read_flag(&sm.emptied[s], lane) < use)
          __builtin_amdgcn_s_sleep(1);
        dma_group(sm.ring[s], blk, ll, lane);
      }
      // the counter wait is the release: the copies are in LDS before the
      // flag store issues (a release store would wait for every load)
      wait_units_outstanding<kDmaPerGroup, C::kAhead - 1>(issued - 1 - j);
      const int k = wave + j * C::kLoaders;
      // one lane stores the flag (a store of all 64 lanes to one word would
      // occupy the LDS for many cycles)
      if (lane == 0)
        __hip_atomic_store(&sm.filled[k % C::kRing], k / C::kRing + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // first groups requested for nothing included
  } else {
    if (wave >= C::kWaves - 2) {
      // ---- the bf16 tail (at most one group, after the quantized ones):
      // tokens 0..63 -> merge slot kCompute (last wave), 64..127 -> slot
      // kCompute + 1 (the wave before).  Done first, while the first groups
      // are still on their way, by the two compute waves with the fewest
      // groups ----
      const int half = C::kWaves - 1 - wave;   // 0: tokens 0..63, 1: tokens 64..127
      const int slot = C::kCompute + half;
      clear_slot(sm.merge, slot);              // stays empty unless tail tokens are seen
      const int g_tail = nq / kGroup;
      const bool owner = (g_tail % S == split);   // one workgroup per slice holds the tail
      const size_t tail_row0 = slice * kGroup * kHeadDim;
      const uint16_t* k_new = nullptr;
      const uint16_t* v_new = nullptr;
      if (a.k_new != nullptr && nt > 0 && owner) {
        // the token appended in this launch: stored at tail index nt - 1 (by
        // the first of the two waves), and attended from its source rows
        k_new = a.k_new + slice * kHeadDim;
        v_new = a.v_new + slice * kHeadDim;
        if (half == 0) {
          const size_t dst = tail_row0 + static_cast<size_t>(nt - 1) * kHeadDim + 2 * lane;
          *reinterpret_cast<uint32_t*>(a.k_tail + dst) = *reinterpret_cast<const uint32_t*>(k_new + 2 * lane);
          *reinterpret_cast<uint32_t*>(a.v_tail + dst) = *reinterpret_cast<const uint32_t*>(v_new + 2 * lane);
        }
      }
      const int t_begin = kTailPart * half;
      if (nt > 0 && g_tail < n_groups && owner) {
        const int n_tok = min(nt, total - g_tail * kGroup) - t_begin;   // this wave's tokens
        if (n_tok > 0) {
          const size_t row0 = tail_row0 + static_cast<size_t>(t_begin) * kHeadDim;
          bf16_tokens_wave<G, C::kSlots>(a.k_tail + row0, a.v_tail + row0, min(n_tok, kTailPart),
                                         a.q + (static_cast<size_t>(b) * a.num_q_heads + qh0) * kHeadDim,
                                         a.sm_scale * kLog2e, sm.tail_p + t_begin, sm.merge, slot, k_new, v_new,
                                         nt - 1 - t_begin);
        }
      }
    }
    if (cw == 0) {
      rotate_q_wave<RB>(q_in, a.sm_scale * kLog2e, sm.q_raw, sm.q_rot, lane);
      // every lane releases its own writes
      __hip_atomic_store(&sm.q_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    while (read_flag(&sm.q_ready, lane) == 0)
      __builtin_amdgcn_s_sleep(1);
    // query of this lane's head and channels 16w + 4b + u + c, per row block:
    // rotated like the keys (unrotated only for the ablation variant whose
    // keys were quantized unrotated)
    const float(*q_keys)[kHeadDim] = (a.flags & OSCAR_KEYS_UNROTATED) ? sm.q_raw : sm.q_rot;
    float qv[RB][2][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          qv[rb][c][b] = q_keys[rb * 4 + gl][16 * (n >> 1) + 4 * b + 2 * (n & 1) + c];
    // weight divisors of the bit pairs u + c this lane's values occupy
    const float fac[2] = {kFac[2 * (n & 1)], kFac[2 * (n & 1) + 1]};

    // ---- compute waves: group k goes to SIMD k % 4 (a workgroup's wave w
    // runs on SIMD w % 4), and the SIMD's compute waves take its groups in
    // turn, so that neighbouring groups, in particular the last ones to
    // arrive, are computed on different SIMDs.  The assignment is fixed,
    // which keeps the summation order, and so the result, the same from run
    // to run ----
    const int simd = wave % 4;
    const int first_i = (simd < C::kLoaders) ? 1 : 0;                  // SIMD's first compute wave: simd + 4 first_i
    const int n_simd = (C::kWaves - 1 - simd) / 4 + 1 - first_i;      // compute waves on this SIMD
    GroupBytes cur;
    const StageLane sl = stage_lane(lane);
    // This wave's last group, if it is one of the split's last four (those
    // land when the stream ends and bound the kernel's end): its key (s, z)
    // pairs are fetched now, straight into LDS, so that the query side of
    // its scores is ready before the group itself lands.
    const int k_first = simd + 4 * (wave / 4 - first_i);
    const int k_last = (k_first < n_k) ? k_first + (n_k - 1 - k_first) / (4 * n_simd) * (4 * n_simd) : -1;
    const bool late = k_last >= 0 && k_last + 4 >= n_k;
    if (late) {
      const uint8_t* src = group_block(k_last) + kStageKsz + 16 * sz_piece_slot(lane & 31);
      if (lane < 32) lds_load16(src, sm.last_ksz[k_last & 3]);
    }
    for (int k = k_first; k < n_k; k += 4 * n_simd) {
      const int s = k % C::kRing;
      const int use = k / C::kRing;
      QPrep<RB> qp;
      const bool prepped = late && k == k_last;
      if (prepped) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the fetch above
        const uint8_t* buf = sm.last_ksz[k_last & 3];
        u32x2 ksz[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) ksz[b] = *reinterpret_cast<const u32x2*>(buf + sl.ksz[b >> 1] - kStageKsz + 16 * b);
        q_prep<G>(ksz, qv, fac, sm, cw, gl, n, qp);
      }
      while (read_flag(&sm.filled[s], lane) <= use)
        __builtin_amdgcn_s_sleep(1);
      read_stage(cur, sm.ring[s], sl);
      // the stage may be refilled once every lane's reads have returned
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (lane == 0) __hip_atomic_store(&sm.emptied[s], use + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      // The last group of each SIMD (one of the split's last four) lands when
      // the stream ends and bounds the kernel's end, while the other waves
      // on its SIMD finish groups that landed earlier: it is issued first.
      if (k + 4 >= n_k) __builtin_amdgcn_s_setprio(2);
      const int g = split + k * S;
      if (!prepped) q_prep<G>(cur.ksz, qv, fac, sm, cw, gl, n, qp);
      float alpha[RB], inv_p[RB];
      score_phase<G>(cur, qp, g * kGroup, total, sm, st, cw, gl, n, fac, alpha, inv_p);
      value_phase<G>(cur, sm, st, cw, gl, n, alpha, inv_p);
    }
  }

  if (!loader) {
    // ---- this compute wave's state -> its merge slot ----
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float l_tot = row_sum16(st.l[rb]);
      const float z_tot = row_sum16(st.z[rb]);
      const int hh = rb * 4 + gl;
      if (hh < G) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.merge.acc[cw][hh][16 * j + n] = st.acc[rb][j] + z_tot;
        if (n == 0) {
          sm.merge.m[cw][hh] = st.m[rb];
          sm.merge.l[cw][hh] = l_tot;
        }
      }
    }
  }
  __syncthreads();

  const size_t partial_base = (static_cast<size_t>(b) * a.num_q_heads + qh0) * a.splits;
  // the two bf16-tail slots hold tokens only in the workgroup that owns the
  // tail group; elsewhere they are empty and left out of the merge
  const int g_tail = nq / kGroup;
  if (nt > 0 && g_tail < n_groups && g_tail % S == split)
    write_partial<G, C::kSlots, false>(sm.merge, a.partials, partial_base, split, a.splits);
  else
    write_partial<G, C::kSlots, false, C::kCompute>(sm.merge, a.partials, partial_base, split, a.splits);
}

template <int G>
hipError_t launch_g(const DecodeInt2Args& a, int32_t batch, hipStream_t s) {
  dim3 grid(a.splits, a.num_kv_heads, batch);
  hipLaunchKernelGGL(decode_int2_kernel<G>, grid, dim3(Int2Cfg<G>::kThreads), 0, s, a);
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
