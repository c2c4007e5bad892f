// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/oscar.h"

namespace oscar {

// Split-K plan of one decode call: the token range [0, max_tokens) of every
// (sequence, KV head) is cut into `splits` pieces of `tokens_per_split`
// tokens (a multiple of 128), one workgroup each.
struct SplitPlan {
  int32_t tokens_per_split;
  int32_t splits;
};

SplitPlan plan_int2(int32_t batch, int32_t num_kv_heads, int32_t max_tokens);
SplitPlan plan_bf16(int32_t batch, int32_t num_kv_heads, int32_t max_tokens);

// Partial softmax state record of one (query head, split): m, l, two pad
// words, acc[128]; 132 floats = 528 bytes (16-byte aligned).
constexpr int kPartialFloats = 132;

// Workspace layout: partials [batch][num_q_heads][splits][132] floats.
size_t partial_bytes(int32_t batch, int32_t num_q_heads, int32_t splits);

struct QuantizeArgs {
  uint8_t* blocks;
  const uint16_t* k_src;
  const uint16_t* v_src;
  int64_t sb, sh, st;
  const int32_t* dst_group_start;
  const int32_t* num_groups;
  const int32_t* block_table;   // paged cache: page of each (sequence, group); nullptr = contiguous
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t capacity;
  int32_t flags;   // OSCAR_KEYS_*
};

struct DecodeInt2Args {
  const uint8_t* blocks;
  const int32_t* block_table;   // paged cache: page of each (sequence, group); nullptr = contiguous
  int32_t num_pages;
  uint16_t* k_tail;        // written only when a token is appended (k_new given)
  uint16_t* v_tail;
  const uint16_t* k_new;   // token appended to the tail in this launch ([B][Hkv][128]), or null
  const uint16_t* v_new;
  const int32_t* n_quant;
  const int32_t* n_tail;
  const uint16_t* q;
  float* partials;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t capacity;
  int32_t max_tokens;
  int32_t tokens_per_split;
  int32_t splits;
  float sm_scale;
  int32_t flags;   // OSCAR_KEYS_*
};

struct DecodeBf16Args {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seq_len;
  const uint16_t* q;
  float* partials;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t capacity;
  int32_t max_tokens;
  int32_t tokens_per_split;
  int32_t splits;
  float sm_scale;
};

hipError_t launch_quantize(const QuantizeArgs& a, int32_t batch, int32_t max_groups, hipStream_t s);
hipError_t launch_decode_int2(const DecodeInt2Args& a, int32_t batch, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeBf16Args& a, int32_t batch, hipStream_t s);
hipError_t launch_merge(const float* partials, float* out, int32_t batch, int32_t num_q_heads, int32_t splits,
                        hipStream_t s);

}  // namespace oscar
