// Host side of the C ABI declared in include/oscar.h: argument validation,
// split planning, workspace layout, launches and error reporting.
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "internal.hpp"

namespace oscar {
namespace {

thread_local char g_last_error[512] = "";

oscar_status fail(oscar_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
oscar_status fail(oscar_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

oscar_status ok() {
  g_last_error[0] = '\0';
  return OSCAR_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int device_count() {
  static std::once_flag once;
  static int count = 0;
  std::call_once(once, [] {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess) n = 0;
    count = n;
  });
  return count;
}

oscar_status check_device(const char* fn) {
  if (device_count() <= 0) return fail(OSCAR_EHIP, "%s: no HIP device available", fn);
  return OSCAR_OK;
}

oscar_status launched(hipError_t e, const char* fn) {
  if (e != hipSuccess) return fail(OSCAR_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

// One workgroup per compute unit (256 on MI355X), all resident at once: as
// many splits per (sequence, KV head) as fit, so that no workgroup waits for
// another to finish.  A split covers whole 128-token groups.
#ifndef OSCAR_TARGET_BLOCKS
#define OSCAR_TARGET_BLOCKS 256
#endif
constexpr int64_t kTargetBlocks = OSCAR_TARGET_BLOCKS;

SplitPlan make_plan(int32_t batch, int32_t num_kv_heads, int32_t max_tokens) {
  const int64_t heads = static_cast<int64_t>(batch) * num_kv_heads;
  const int64_t T = max_tokens > 0 ? max_tokens : 0;
  const int64_t groups = (T + OSCAR_GROUP - 1) / OSCAR_GROUP;
  int64_t s = kTargetBlocks / (heads > 0 ? heads : 1);
  s = s < 1 ? 1 : s;
  s = (groups > 0 && s > groups) ? groups : s;
  const int64_t tps = ((groups + s - 1) / s) * OSCAR_GROUP;   // whole groups per split
  SplitPlan p;
  p.tokens_per_split = static_cast<int32_t>(tps > 0 ? tps : OSCAR_GROUP);
  p.splits = static_cast<int32_t>(T > 0 ? (T + p.tokens_per_split - 1) / p.tokens_per_split : 1);
  return p;
}

}  // namespace

SplitPlan plan_int2(int32_t batch, int32_t num_kv_heads, int32_t max_tokens) {
  // The INT2 kernel deals the groups out round-robin (split s takes groups
  // s, s + S, ...), so it uses every split that fits, up to one per group.
  SplitPlan p = make_plan(batch, num_kv_heads, max_tokens);
  const int64_t heads = static_cast<int64_t>(batch) * num_kv_heads;
  const int64_t groups = (static_cast<int64_t>(max_tokens > 0 ? max_tokens : 0) + OSCAR_GROUP - 1) / OSCAR_GROUP;
  int64_t s = kTargetBlocks / (heads > 0 ? heads : 1);
  s = s < 1 ? 1 : s;
  s = (groups > 0 && s > groups) ? groups : s;
  p.splits = static_cast<int32_t>(groups > 0 ? s : 1);
  return p;
}
SplitPlan plan_bf16(int32_t batch, int32_t num_kv_heads, int32_t max_tokens) {
  return make_plan(batch, num_kv_heads, max_tokens);
}

size_t partial_bytes(int32_t batch, int32_t num_q_heads, int32_t splits) {
  return static_cast<size_t>(batch) * num_q_heads * splits * kPartialFloats * sizeof(float);
}

namespace {

oscar_status check_heads(const char* fn, int32_t batch, int32_t num_kv_heads, int32_t num_q_heads) {
  if (batch <= 0 || num_kv_heads <= 0 || num_q_heads <= 0)
    return fail(OSCAR_EINVAL, "%s: batch, num_kv_heads and num_q_heads must be positive", fn);
  if (batch > 65535 || num_kv_heads > 65535)
    return fail(OSCAR_EINVAL, "%s: batch and num_kv_heads must be <= 65535", fn);
  if (num_q_heads % num_kv_heads != 0)
    return fail(OSCAR_EUNSUPPORTED, "%s: num_q_heads (%d) is not a multiple of num_kv_heads (%d)", fn,
                num_q_heads, num_kv_heads);
  const int g = num_q_heads / num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(OSCAR_EUNSUPPORTED, "%s: query heads per KV head must be 1, 2, 4 or 8 (got %d)", fn, g);
  return OSCAR_OK;
}

oscar_status check_cache(const char* fn, const oscar_kv_cache* c) {
  if (!c) return fail(OSCAR_EINVAL, "%s: cache descriptor is NULL", fn);
  if (c->head_dim != OSCAR_HEAD_DIM) return fail(OSCAR_EUNSUPPORTED, "%s: head_dim must be 128 (got %d)", fn, c->head_dim);
  if (c->group != OSCAR_GROUP) return fail(OSCAR_EUNSUPPORTED, "%s: group must be 128 (got %d)", fn, c->group);
  if (c->batch <= 0 || c->num_kv_heads <= 0) return fail(OSCAR_EINVAL, "%s: batch and num_kv_heads must be positive", fn);
  if (c->batch > 65535 || c->num_kv_heads > 65535) return fail(OSCAR_EINVAL, "%s: batch and num_kv_heads must be <= 65535", fn);
  if (c->capacity <= 0 || c->capacity % OSCAR_GROUP != 0)
    return fail(OSCAR_EINVAL, "%s: capacity must be a positive multiple of 128 (got %d)", fn, c->capacity);
  if ((c->flags & ~(OSCAR_KEYS_UNROTATED | OSCAR_KEYS_UNSCALED)) != 0)
    return fail(OSCAR_EINVAL, "%s: unknown bits in cache->flags (0x%x)", fn, static_cast<unsigned>(c->flags));
  if (!c->blocks) return fail(OSCAR_EINVAL, "%s: cache->blocks is NULL", fn);
  if ((reinterpret_cast<uintptr_t>(c->blocks) & 255u) != 0)
    return fail(OSCAR_EINVAL, "%s: cache->blocks is not 256-byte aligned", fn);
  if ((c->k_tail && !aligned16(c->k_tail)) || (c->v_tail && !aligned16(c->v_tail)))
    return fail(OSCAR_EINVAL, "%s: tail buffers must be 16-byte aligned", fn);
  if (c->reserved != 0) return fail(OSCAR_EINVAL, "%s: cache->reserved must be 0", fn);
  if (c->block_table) {
    if ((reinterpret_cast<uintptr_t>(c->block_table) & 3u) != 0)
      return fail(OSCAR_EINVAL, "%s: cache->block_table is not 4-byte aligned", fn);
    if (c->num_pages <= 0) return fail(OSCAR_EINVAL, "%s: a paged cache needs num_pages > 0 (got %d)", fn, c->num_pages);
  }
  return OSCAR_OK;
}

// Split records of oscar_decode_attn_noalloc: a file-scope device array, so
// that the call needs no workspace from the caller.  In host code the name
// `scratch` is only a stand-in for the symbol: host code uses the device
// address that hipGetSymbolAddress returns for the current device (each
// device holds its own copy of the array), never the name itself.
static __device__ __align__(256) uint8_t scratch[OSCAR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr with an error set if
// the lookup fails.
oscar_status scratch_on_current_device(const char* fn, void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(OSCAR_EHIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(OSCAR_EHIP, "%s: device %d beyond the %d supported", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(OSCAR_EHIP, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return OSCAR_OK;
}

}  // namespace
}  // namespace oscar

using namespace oscar;

extern "C" {

int32_t oscar_abi_version(void) { return OSCAR_ABI_VERSION; }

const char* oscar_status_string(oscar_status status) {
  switch (status) {
    case OSCAR_OK: return "ok";
    case OSCAR_EINVAL: return "invalid argument";
    case OSCAR_EUNSUPPORTED: return "unsupported shape";
    case OSCAR_EWORKSPACE: return "workspace too small";
    case OSCAR_EHIP: return "HIP error";
  }
  return "unknown status";
}

const char* oscar_last_error(void) { return g_last_error; }

oscar_status oscar_quantize_kv(const oscar_kv_cache* cache, const uint16_t* k_src, const uint16_t* v_src,
                               int64_t src_stride_b, int64_t src_stride_h, int64_t src_stride_t,
                               const int32_t* dst_group_start, const int32_t* num_groups, int32_t max_groups,
                               void* stream) {
  const char* fn = "oscar_quantize_kv";
  oscar_status st = check_cache(fn, cache);
  if (st != OSCAR_OK) return st;
  if (!k_src || !v_src || !dst_group_start || !num_groups)
    return fail(OSCAR_EINVAL, "%s: source or group arrays are NULL", fn);
  if (!aligned16(k_src) || !aligned16(v_src)) return fail(OSCAR_EINVAL, "%s: sources must be 16-byte aligned", fn);
  if (src_stride_b < 0 || src_stride_h < 0 || src_stride_t < OSCAR_HEAD_DIM)
    return fail(OSCAR_EINVAL, "%s: strides must be non-negative and the token stride >= 128", fn);
  if (src_stride_b % 8 || src_stride_h % 8 || src_stride_t % 8)
    return fail(OSCAR_EINVAL, "%s: strides must be multiples of 8 elements (16 bytes)", fn);
  if (max_groups < 0) return fail(OSCAR_EINVAL, "%s: max_groups must be >= 0", fn);
  if (max_groups > cache->capacity / OSCAR_GROUP)
    return fail(OSCAR_EINVAL, "%s: max_groups (%d) exceeds the cache's %d groups", fn, max_groups,
                cache->capacity / OSCAR_GROUP);
  if (max_groups == 0) return ok();
  if ((st = check_device(fn)) != OSCAR_OK) return st;
  QuantizeArgs a;
  a.blocks = cache->blocks;
  a.block_table = cache->block_table;
  a.num_pages = cache->block_table ? cache->num_pages : 0;
  a.k_src = k_src;
  a.v_src = v_src;
  a.sb = src_stride_b;
  a.sh = src_stride_h;
  a.st = src_stride_t;
  a.dst_group_start = dst_group_start;
  a.num_groups = num_groups;
  a.num_kv_heads = cache->num_kv_heads;
  a.capacity = cache->capacity;
  a.flags = cache->flags;
  return launched(launch_quantize(a, cache->batch, max_groups, static_cast<hipStream_t>(stream)), fn);
}

size_t oscar_decode_workspace_bytes(int32_t batch, int32_t num_kv_heads, int32_t num_q_heads, int32_t max_tokens) {
  if (batch <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 || max_tokens < 0) return 0;
  if (num_q_heads % num_kv_heads != 0) return 0;
  const SplitPlan pi = plan_int2(batch, num_kv_heads, max_tokens);
  const SplitPlan pb = plan_bf16(batch, num_kv_heads, max_tokens);
  const int32_t splits = pi.splits > pb.splits ? pi.splits : pb.splits;
  return partial_bytes(batch, num_q_heads, splits);
}

}  // extern "C"

namespace {

// Validation and launch of the INT2 decode kernel (the split records); out
// is checked only when the caller also merges.
oscar_status decode_int2_splits(const char* fn, const oscar_kv_cache* cache, const int32_t* n_quant,
                                const int32_t* n_tail, int32_t max_tokens, const uint16_t* q, int32_t num_q_heads,
                                float sm_scale, const uint16_t* k_new, const uint16_t* v_new, const float* out, bool with_out, void* ws, size_t ws_bytes,
                                hipStream_t s, int32_t* splits_out) {
  oscar_status st = check_cache(fn, cache);
  if (st != OSCAR_OK) return st;
  if ((st = check_heads(fn, cache->batch, cache->num_kv_heads, num_q_heads)) != OSCAR_OK) return st;
  if (!n_quant || !n_tail || !q || !ws || (with_out && !out)) return fail(OSCAR_EINVAL, "%s: NULL argument", fn);
  if (!aligned16(q) || !aligned16(ws) || (with_out && !aligned16(out)))
    return fail(OSCAR_EINVAL, "%s: q, out and ws must be 16-byte aligned", fn);
  if (max_tokens < 0) return fail(OSCAR_EINVAL, "%s: max_tokens must be >= 0", fn);
  if (max_tokens > cache->capacity + OSCAR_GROUP - 1)
    return fail(OSCAR_EINVAL, "%s: max_tokens (%d) exceeds capacity + 127", fn, max_tokens);
  const size_t need = oscar_decode_workspace_bytes(cache->batch, cache->num_kv_heads, num_q_heads, max_tokens);
  if (ws_bytes < need) return fail(OSCAR_EWORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, ws_bytes, need);
  if ((st = check_device(fn)) != OSCAR_OK) return st;
  const SplitPlan p = plan_int2(cache->batch, cache->num_kv_heads, max_tokens);
  DecodeInt2Args a;
  a.blocks = cache->blocks;
  a.block_table = cache->block_table;
  a.num_pages = cache->block_table ? cache->num_pages : 0;
  a.k_tail = cache->k_tail;
  a.v_tail = cache->v_tail;
  a.k_new = k_new;
  a.v_new = v_new;
  a.n_quant = n_quant;
  a.n_tail = n_tail;
  a.q = q;
  a.partials = static_cast<float*>(ws);
  a.num_kv_heads = cache->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.capacity = cache->capacity;
  a.flags = cache->flags;
  a.max_tokens = max_tokens;
  a.tokens_per_split = p.tokens_per_split;
  a.splits = p.splits;
  a.sm_scale = sm_scale;
  *splits_out = p.splits;
  return launched(launch_decode_int2(a, cache->batch, s), fn);
}

}  // namespace

extern "C" {

int32_t oscar_decode_num_splits(int32_t batch, int32_t num_kv_heads, int32_t max_tokens) {
  if (batch <= 0 || num_kv_heads <= 0 || max_tokens < 0) return 0;
  return plan_int2(batch, num_kv_heads, max_tokens).splits;
}

oscar_status oscar_decode_attn_splits(const oscar_kv_cache* cache, const int32_t* n_quant, const int32_t* n_tail,
                                      int32_t max_tokens, const uint16_t* q, int32_t num_q_heads, float sm_scale,
                                      void* ws, size_t ws_bytes, void* stream) {
  int32_t splits = 0;
  return decode_int2_splits("oscar_decode_attn_splits", cache, n_quant, n_tail, max_tokens, q, num_q_heads,
                            sm_scale, nullptr, nullptr, nullptr, false, ws, ws_bytes, static_cast<hipStream_t>(stream),
                            &splits);
}

oscar_status oscar_decode_merge(const float* partials, int32_t batch, int32_t num_q_heads, int32_t num_splits,
                                float* out, void* stream) {
  const char* fn = "oscar_decode_merge";
  if (!partials || !out) return fail(OSCAR_EINVAL, "%s: NULL argument", fn);
  if (!aligned16(partials) || !aligned16(out))
    return fail(OSCAR_EINVAL, "%s: partials and out must be 16-byte aligned", fn);
  if (batch <= 0 || batch > 65535 || num_q_heads <= 0 || num_splits <= 0)
    return fail(OSCAR_EINVAL, "%s: batch must be in [1, 65535], num_q_heads and num_splits positive", fn);
  oscar_status st = check_device(fn);
  if (st != OSCAR_OK) return st;
  return launched(launch_merge(partials, out, batch, num_q_heads, num_splits, static_cast<hipStream_t>(stream)),
                  fn);
}

oscar_status oscar_decode_attn(const oscar_kv_cache* cache, const int32_t* n_quant, const int32_t* n_tail,
                               int32_t max_tokens, const uint16_t* q, int32_t num_q_heads, float sm_scale,
                               float* out, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "oscar_decode_attn";
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t splits = 0;
  oscar_status st = decode_int2_splits(fn, cache, n_quant, n_tail, max_tokens, q, num_q_heads, sm_scale, nullptr,
                                       nullptr, out, true, ws, ws_bytes, s, &splits);
  if (st != OSCAR_OK) return st;
  return launched(launch_merge(static_cast<const float*>(ws), out, cache->batch, num_q_heads, splits, s), fn);
}

oscar_status oscar_decode_attn_append(const oscar_kv_cache* cache, const int32_t* n_quant, const int32_t* n_tail,
                                      int32_t max_tokens, const uint16_t* q, const uint16_t* k_new,
                                      const uint16_t* v_new, int32_t num_q_heads, float sm_scale, float* out,
                                      void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "oscar_decode_attn_append";
  if (!k_new || !v_new) return fail(OSCAR_EINVAL, "%s: NULL k_new or v_new", fn);
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(OSCAR_EINVAL, "%s: k_new and v_new must be 16-byte aligned", fn);
  if (cache && (!cache->k_tail || !cache->v_tail))
    return fail(OSCAR_EINVAL, "%s: the cache has no tail buffers to append to", fn);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t splits = 0;
  oscar_status st = decode_int2_splits(fn, cache, n_quant, n_tail, max_tokens, q, num_q_heads, sm_scale, k_new,
                                       v_new, out, true, ws, ws_bytes, s, &splits);
  if (st != OSCAR_OK) return st;
  return launched(launch_merge(static_cast<const float*>(ws), out, cache->batch, num_q_heads, splits, s), fn);
}

oscar_status oscar_decode_attn_noalloc(const oscar_kv_cache* cache, const int32_t* n_quant, const int32_t* n_tail,
                                       int32_t max_tokens, const uint16_t* q, int32_t num_q_heads, float sm_scale,
                                       float* out, void* stream) {
  const char* fn = "oscar_decode_attn_noalloc";
  // the size check comes first, so that a shape beyond the array is refused
  // before anything touches the device
  const size_t need = (cache != nullptr && num_q_heads > 0)
                          ? oscar_decode_workspace_bytes(cache->batch, cache->num_kv_heads, num_q_heads, max_tokens)
                          : 0;
  if (need > OSCAR_NOALLOC_SCRATCH_BYTES)
    return fail(OSCAR_EWORKSPACE, "%s: this shape needs %zu bytes of split records, more than the %d-byte scratch array",
                fn, need, OSCAR_NOALLOC_SCRATCH_BYTES);
  oscar_status st = check_cache(fn, cache);
  if (st != OSCAR_OK) return st;
  if ((st = check_heads(fn, cache->batch, cache->num_kv_heads, num_q_heads)) != OSCAR_OK) return st;
  if ((st = check_device(fn)) != OSCAR_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_on_current_device(fn, &ws)) != OSCAR_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t splits = 0;
  st = decode_int2_splits(fn, cache, n_quant, n_tail, max_tokens, q, num_q_heads, sm_scale, nullptr, nullptr, out,
                          true, ws, OSCAR_NOALLOC_SCRATCH_BYTES, s, &splits);
  if (st != OSCAR_OK) return st;
  return launched(launch_merge(static_cast<const float*>(ws), out, cache->batch, num_q_heads, splits, s), fn);
}

oscar_status oscar_decode_attn_bf16(const uint16_t* k, const uint16_t* v, int32_t batch, int32_t num_kv_heads,
                                    int32_t capacity, const int32_t* seq_len, int32_t max_tokens, const uint16_t* q,
                                    int32_t num_q_heads, float sm_scale, float* out, void* ws, size_t ws_bytes,
                                    void* stream) {
  const char* fn = "oscar_decode_attn_bf16";
  oscar_status st = check_heads(fn, batch, num_kv_heads, num_q_heads);
  if (st != OSCAR_OK) return st;
  if (!k || !v || !seq_len || !q || !out || !ws) return fail(OSCAR_EINVAL, "%s: NULL argument", fn);
  if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(out) || !aligned16(ws))
    return fail(OSCAR_EINVAL, "%s: k, v, q, out and ws must be 16-byte aligned", fn);
  if (capacity <= 0) return fail(OSCAR_EINVAL, "%s: capacity must be positive", fn);
  if (max_tokens < 0 || max_tokens > capacity)
    return fail(OSCAR_EINVAL, "%s: max_tokens must be in [0, capacity]", fn);
  const size_t need = oscar_decode_workspace_bytes(batch, num_kv_heads, num_q_heads, max_tokens);
  if (ws_bytes < need) return fail(OSCAR_EWORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, ws_bytes, need);
  if ((st = check_device(fn)) != OSCAR_OK) return st;
  const SplitPlan p = plan_bf16(batch, num_kv_heads, max_tokens);
  DecodeBf16Args a;
  a.k = k;
  a.v = v;
  a.seq_len = seq_len;
  a.q = q;
  a.partials = static_cast<float*>(ws);
  a.num_kv_heads = num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.capacity = capacity;
  a.max_tokens = max_tokens;
  a.tokens_per_split = p.tokens_per_split;
  a.splits = p.splits;
  a.sm_scale = sm_scale;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = launched(launch_decode_bf16(a, batch, s), fn)) != OSCAR_OK) return st;
  return launched(launch_merge(a.partials, out, batch, num_q_heads, p.splits, s), fn);
}

}  // extern "C"

