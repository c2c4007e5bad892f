/*
 * oscar.h -- C ABI of the OScaR INT2 KV-cache library for AMD Instinct MI355X
 * (gfx950).
 *
 * The library implements two things:
 *
 *  1. The OScaR key/value quantizer.  Each key is rotated by the orthonormal
 *     128-point Hadamard matrix ("Canalized Rotation"), divided by its own L2
 *     norm, which is kept in fp16 ("Omni-Token Scaling"), and quantized to
 *     INT2 per channel over groups of 128 tokens.  Values are quantized to
 *     INT2 per token.  Sources: OScaR abstract (arXiv 2605.19660, fugumt.com
 *     record, "Abstract"); ai-papers.net OScaR summary, section
 *     "OScaRの提案手法" and Fig. 4.
 *  2. Single-query grouped-query attention over the packed cache (one decode
 *     step), the operation whose speed-up over bf16 flash-decoding the pages
 *     report (ai-papers.net summary, section "実験結果"; abstract), plus a bf16
 *     flash-decoding kernel over unquantized keys/values that serves as the
 *     speed-up denominator.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All buffers are device memory owned by the caller; the library never
 *    allocates, frees or synchronizes.  Every compute call is asynchronous on
 *    the given stream (a hipStream_t passed as void*; NULL = default stream).
 *  - Host-side arguments are validated before anything is launched.  A
 *    failing call launches nothing, returns a non-zero oscar_status and
 *    records a message retrievable with oscar_last_error() on the same host
 *    thread.  Nothing throws across this boundary.
 *  - Values that live in device memory (lengths, group starts) are
 *    preconditions stated per call; kernels skip work that would fall
 *    outside the buffers described by oscar_kv_cache instead of faulting.
 *  - fp16 and bf16 numbers are passed as uint16_t bit patterns.
 *  - head_dim and the quantization group are both fixed at 128.
 *
 * Packed cache layout (the pages fix only "INT2"; the byte layout is this
 * library's):
 *  - 2-bit codes, four per byte, least significant bits first:
 *    byte = c0 | c1 << 2 | c2 << 4 | c3 << 6.
 *  - blocks : uint8 [batch][num_kv_heads][capacity/128][OSCAR_BLOCK_BYTES];
 *             one 9472-byte block per group of 128 tokens, which holds
 *             everything a decode step reads for that group, so that the
 *             step streams whole blocks:
 *      [OSCAR_BLOCK_K_CODES, +4096) key codes, [128 tokens][32 bytes]; byte
 *                               i of a token row holds channels 4i..4i+3 of
 *                               the rotated, scaled key;
 *      [OSCAR_BLOCK_V_CODES, +4096) value codes, [128 channels][32 bytes];
 *                               byte j of a channel row holds tokens
 *                               4j..4j+3 of the group;
 *      [OSCAR_BLOCK_K_SZ, +512)    fp16 [128 channels][2]: the group's key
 *                               (scale s, zero-point z) per channel;
 *      [OSCAR_BLOCK_V_SZ, +512)    fp16 [128 tokens][2]: each token's value
 *                               (s, z);
 *      [OSCAR_BLOCK_K_NORM, +256)  fp16 [128 tokens]: each key's L2 norm
 *                               (after the rotation, which keeps it).
 *  - k_tail, v_tail : bf16 [batch][num_kv_heads][128][128]; the tokens of
 *              the current, not yet complete group (at most 127 are read).
 *  Paged cache (block_table != NULL): the blocks live in a pool of pages,
 *  blocks : uint8 [num_pages][num_kv_heads][OSCAR_BLOCK_BYTES], one page per
 *  group of 128 tokens holding that group's block for every KV head; group g
 *  of sequence b is page block_table[b * (capacity/128) + g].  Pages may be
 *  assigned in any order; two groups written by the same call must not share
 *  a page.  The kernels clamp a table entry to [0, num_pages) before using
 *  it, so a stale entry reaches some page of the pool, never memory outside
 *  it.
 *  Dequantization: key (rotated domain) = n * (s * c + z) with the group's
 *  (s, z) for that channel; value = s * c + z with the token's (s, z).
 *  blocks must be 256-byte aligned (every block then is), the tails
 *  16-byte aligned.
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OSCAR_ABI_VERSION 3
#define OSCAR_HEAD_DIM 128
#define OSCAR_GROUP 128

/* One group's block in the packed cache (byte offsets, see the layout above). */
#define OSCAR_BLOCK_K_CODES 0
#define OSCAR_BLOCK_V_CODES 4096
#define OSCAR_BLOCK_K_SZ 8192
#define OSCAR_BLOCK_V_SZ 8704
#define OSCAR_BLOCK_K_NORM 9216
#define OSCAR_BLOCK_BYTES 9472

typedef enum oscar_status {
  OSCAR_OK = 0,
  OSCAR_EINVAL = 1,        /* null/misaligned pointer, negative or zero size, bad stride */
  OSCAR_EUNSUPPORTED = 2,  /* head_dim or group != 128, Hq not a multiple of Hkv, GQA ratio > 8 */
  OSCAR_EWORKSPACE = 3,    /* workspace smaller than oscar_decode_workspace_bytes() */
  OSCAR_EHIP = 4           /* no usable device, or the HIP launch failed */
} oscar_status;

/* Caller-owned packed cache (see the layout above). */
/* oscar_kv_cache.flags: key-quantizer variants for the Token Norm Imbalance
 * ablation (ai-papers.net OScaR summary, sections "TNIという根本課題の特定"
 * and "OScaRの提案手法").  0 is the method: keys rotated, then scaled. */
#define OSCAR_KEYS_UNROTATED 1   /* no Hadamard rotation: keys quantized as they are */
#define OSCAR_KEYS_UNSCALED 2    /* no per-token L2 scaling: the stored norm is 1 */

typedef struct oscar_kv_cache {
  int32_t batch;
  int32_t num_kv_heads;
  int32_t head_dim;        /* must be 128 */
  int32_t group;           /* must be 128 */
  int32_t capacity;        /* tokens per sequence; a positive multiple of 128 */
  int32_t flags;           /* OSCAR_KEYS_* bits; the quantizer and the decode of a cache must agree */
  uint8_t* blocks;          /* [batch][num_kv_heads][capacity/128][OSCAR_BLOCK_BYTES], or the page pool */
  uint16_t* k_tail;        /* read by the decode calls, written by oscar_decode_attn_append only; */
  uint16_t* v_tail;        /* may be NULL if no tail is ever used */
  /* Paged layout (a block table as in paged-attention serving): NULL for the
   * contiguous layout above; else device int32 [batch][capacity/128], the
   * page of each group (4-byte aligned), and blocks is the pool of
   * num_pages pages (see the layout above). */
  const int32_t* block_table;
  int32_t num_pages;       /* pages in the pool (> 0) when block_table is set; ignored otherwise */
  int32_t reserved;        /* must be 0 */
} oscar_kv_cache;

/* Version of this ABI (OSCAR_ABI_VERSION). */
int32_t oscar_abi_version(void);

/* Static text of a status code. */
const char* oscar_status_string(oscar_status status);

/* Message of the last failing call made on this host thread ("" if none). */
const char* oscar_last_error(void);

/*
 * oscar_quantize_kv -- prefill and group append.
 *
 * Quantizes whole 128-token groups of bf16 keys and values into the packed
 * cache (OScaR abstract; ai-papers.net summary, "OScaRの提案手法"): for keys,
 * Hadamard rotation, per-token L2 norm stored in fp16, division by that
 * stored norm, per-channel INT2 over the group; for values, per-token INT2.
 * INT2 is asymmetric: s = (max - min) / 3 and z = min, both stored in fp16
 * (round to nearest even, saturating at +-65504), code =
 * clamp(round_half_even((x - z) / s), 0, 3), code 0 where s == 0; a key
 * whose stored norm is 0 is scaled to 0.  The rotation, norm, scaling,
 * min/max and the division deciding each code are evaluated in fp64.
 *
 * k_src, v_src : bf16 sources; element (b, h, t, d) at
 *                src + b*src_stride_b + h*src_stride_h + t*src_stride_t + d
 *                (strides in elements, channels contiguous).  Source token
 *                t belongs to source group t / 128.
 * dst_group_start : device int32[batch]; source group j of sequence b is
 *                written to cache group dst_group_start[b] + j.
 * num_groups   : device int32[batch]; number of source groups of sequence b
 *                to quantize (0 allowed).  Groups whose destination falls
 *                outside [0, capacity/128) are skipped.
 * max_groups   : host upper bound of num_groups[] (sizes the grid); 0 is a
 *                no-op.
 * Group append: pass the tail buffer as source (strides 128*128*Hkv,
 * 128*128, 128), dst_group_start = n_quant / 128 and num_groups = 1 for the
 * sequences whose tail is full, 0 otherwise.
 */
oscar_status oscar_quantize_kv(const oscar_kv_cache* cache,
                               const uint16_t* k_src, const uint16_t* v_src,
                               int64_t src_stride_b, int64_t src_stride_h,
                               int64_t src_stride_t,
                               const int32_t* dst_group_start,
                               const int32_t* num_groups, int32_t max_groups,
                               void* stream);

/*
 * Bytes of workspace that oscar_decode_attn / oscar_decode_attn_bf16 need
 * for this shape: the split-K partial softmax states (m, l, acc[128]) of
 * every query head and split.  Returns 0 for invalid shapes.  The
 * workspace needs no initialisation.
 */
size_t oscar_decode_workspace_bytes(int32_t batch, int32_t num_kv_heads,
                                    int32_t num_q_heads, int32_t max_tokens);

/*
 * oscar_decode_attn -- one decode step over the packed INT2 cache: the step
 * whose speed the pages report against BF16 FlashDecoding-v2 (OScaR
 * abstract, fugumt.com record, "Abstract"; ai-papers.net OScaR summary,
 * section "実験結果"), with the keys as the summary's section "OScaRの提案手法"
 * stores them (rotated, then scaled per token), so the query is rotated the
 * same way.
 *
 * For every sequence b and query head j (KV head j / (num_q_heads /
 * num_kv_heads)): rotate q by the same Hadamard matrix, score each quantized
 * token as sm_scale * n * (Hq . (s * c + z)), score each tail token as
 * sm_scale * (q . k_tail), take the softmax over all n_quant[b] + n_tail[b]
 * tokens and write out = sum_t p_t * value_t (values dequantized as
 * s * c + z, tail values as stored).  The token range is split across
 * workgroups; a second kernel on the same stream merges their partial
 * softmax states in a fixed order, so results are deterministic.  An empty
 * sequence gives out = 0.
 *
 * n_quant      : device int32[batch]; quantized tokens, a multiple of 128,
 *                <= capacity (precondition).
 * n_tail       : device int32[batch]; tail tokens, 0..128 (precondition).
 * max_tokens   : host upper bound of n_quant[b] + n_tail[b]; sizes the grid
 *                and the workspace.  Tokens beyond it are not read.
 * q            : bf16 [batch][num_q_heads][128].
 * sm_scale     : logit scale (usually 1/sqrt(128)).
 * out          : fp32 [batch][num_q_heads][128].
 * ws, ws_bytes : workspace of at least oscar_decode_workspace_bytes(batch,
 *                num_kv_heads, num_q_heads, max_tokens) bytes.  Calls that
 *                share a workspace must not overlap (ordering them on one
 *                stream is enough).
 */
oscar_status oscar_decode_attn(const oscar_kv_cache* cache,
                               const int32_t* n_quant, const int32_t* n_tail,
                               int32_t max_tokens, const uint16_t* q,
                               int32_t num_q_heads, float sm_scale, float* out,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * oscar_decode_attn_append -- a decode step that first appends the step's
 * own key and value to the bf16 tail, in the same launch (the decode-time
 * append of the group-append workflow: the pages quantize a group once it
 * is complete, ai-papers.net OScaR summary, section "OScaRの提案手法").
 *
 * n_tail[b] counts the new token: it is stored at tail index n_tail[b] - 1
 * of every KV head of sequence b and attended together with the rest.
 * Preconditions: 1 <= n_tail[b] <= 128 and n_quant[b] + 128 <= capacity
 * (the tail's group lies inside the cache).  When n_tail[b] reaches 128 the
 * caller quantizes the tail (oscar_quantize_kv with k_tail / v_tail as the
 * source and destination group n_quant[b] / 128) before the next append,
 * and continues with n_quant[b] + 128 and n_tail[b] = 0.
 *
 * k_new, v_new : bf16 [batch][num_kv_heads][128], 16-byte aligned.
 * cache->k_tail and cache->v_tail must be given.  Other arguments and the
 * result as in oscar_decode_attn.
 */
oscar_status oscar_decode_attn_append(const oscar_kv_cache* cache,
                                      const int32_t* n_quant, const int32_t* n_tail,
                                      int32_t max_tokens, const uint16_t* q,
                                      const uint16_t* k_new, const uint16_t* v_new,
                                      int32_t num_q_heads, float sm_scale, float* out,
                                      void* ws, size_t ws_bytes, void* stream);

/*
 * The two halves of oscar_decode_attn, for callers that combine partial
 * softmax states themselves (for instance a sequence split across devices:
 * each device scores its own tokens, the records are gathered along the
 * split axis and merged once).
 *
 * oscar_decode_num_splits -- records per (sequence, query head) that
 * oscar_decode_attn_splits writes for this shape (0 for invalid shapes).
 *
 * oscar_decode_attn_splits -- the first kernel of oscar_decode_attn: same
 * arguments except out.  The record format is this library's (the pages
 * describe no kernel); the merge is the standard combination of partial
 * softmax states.  It writes, at the start of ws, the float records
 * [batch][num_q_heads][S][132] (S = oscar_decode_num_splits(batch,
 * num_kv_heads, max_tokens)); record (b, j, r) = (m, l, unused, unused,
 * acc[128]) over the tokens of split r of sequence b, in base 2:
 * m = max_t x_t with x_t = logit_t * log2(e) (-inf if the split saw no
 * token), l = sum_t 2^(x_t - m), acc[d] = sum_t 2^(x_t - m) * value_t[d]
 * (l = acc = 0 for an empty split).
 *
 * oscar_decode_merge -- out[b][j] = sum_r w_r acc_r / sum_r w_r l_r with
 * w_r = 2^(m_r - max_r m_r), over the num_splits records of (b, j) stored
 * as above at partials; records with m = -inf are skipped and out = 0 if
 * all are.  Records are combined in a fixed order (deterministic).
 * partials, out: device memory, 16-byte aligned; batch <= 65535.
 */
int32_t oscar_decode_num_splits(int32_t batch, int32_t num_kv_heads, int32_t max_tokens);

oscar_status oscar_decode_attn_splits(const oscar_kv_cache* cache,
                                      const int32_t* n_quant, const int32_t* n_tail,
                                      int32_t max_tokens, const uint16_t* q,
                                      int32_t num_q_heads, float sm_scale,
                                      void* ws, size_t ws_bytes, void* stream);

oscar_status oscar_decode_merge(const float* partials, int32_t batch,
                                int32_t num_q_heads, int32_t num_splits,
                                float* out, void* stream);

/*
 * oscar_decode_attn_noalloc -- oscar_decode_attn without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * The split records live in a device array inside the library,
 * OSCAR_NOALLOC_SCRATCH_BYTES large; every device the library runs on holds
 * its own copy until the process ends.  The call allocates nothing and frees
 * nothing.  Its first call on a device looks up that device's copy (the
 * device current on the calling thread is the one used).  Arguments and
 * result as in oscar_decode_attn.
 *
 * Limits: a shape whose records need more than OSCAR_NOALLOC_SCRATCH_BYTES
 * (oscar_decode_workspace_bytes() > OSCAR_NOALLOC_SCRATCH_BYTES) is refused
 * with OSCAR_EWORKSPACE before anything is launched.  Every call on a device
 * shares that device's array: calls that may overlap on one device (on
 * different streams, or from different threads without ordering) race and
 * give wrong results; calls ordered on one stream are safe.  Every call
 * writes all the records it reads, so nothing needs clearing between calls.
 */
#define OSCAR_NOALLOC_SCRATCH_BYTES (4 << 20)

oscar_status oscar_decode_attn_noalloc(const oscar_kv_cache* cache,
                                       const int32_t* n_quant, const int32_t* n_tail,
                                       int32_t max_tokens, const uint16_t* q,
                                       int32_t num_q_heads, float sm_scale, float* out,
                                       void* stream);

/*
 * oscar_decode_attn_bf16 -- the same decode step over unquantized bf16
 * keys and values: plain split-K flash-decoding, the counterpart of the
 * BF16 FlashDecoding-v2 baseline the pages compare against (ai-papers.net
 * OScaR summary, section "実験結果"; OScaR abstract).
 *
 * k, v    : bf16 [batch][num_kv_heads][capacity][128].
 * seq_len : device int32[batch]; tokens of sequence b, <= capacity
 *           (precondition).
 * Other arguments as in oscar_decode_attn.
 */
oscar_status oscar_decode_attn_bf16(const uint16_t* k, const uint16_t* v,
                                    int32_t batch, int32_t num_kv_heads,
                                    int32_t capacity, const int32_t* seq_len,
                                    int32_t max_tokens, const uint16_t* q,
                                    int32_t num_q_heads, float sm_scale,
                                    float* out, void* ws, size_t ws_bytes,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H */
