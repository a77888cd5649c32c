// Host side of the C ABI (include/pa.h): argument checks, split planning and
// kernel dispatch.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/pa.h"
#include "../../include/pa_probe.h"
#include "pa_launch.h"

namespace {

thread_local char g_last_error[512] = "";

pa_status fail(pa_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

pa_status ok() {
  g_last_error[0] = '\0';
  return PA_OK;
}

pa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes(int dt) {
  switch (dt) {
    case PA_DTYPE_F32: return 4;
    case PA_DTYPE_F16: return 2;
    case PA_DTYPE_BF16: return 2;
    case PA_DTYPE_FP8_E4M3: return 1;
    case PA_DTYPE_INT8: return 1;
    default: return 0;
  }
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape / type checks shared by decode and prefill.
pa_status check_attention_shape(int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                int max_blocks, pa_dtype q_dtype, pa_dtype cache_dtype,
                                pa_dtype v_cache_dtype) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "head counts and max_blocks_per_seq must be positive");
  if (num_q_heads % num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > 16)
    return fail(PA_ERR_UNSUPPORTED, "more than 16 query heads per KV head");
  if (num_kv_heads > 65535) return fail(PA_ERR_UNSUPPORTED, "too many KV heads");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d (supported: 8, 16, 32, 64)", block_size);
  if (elem_bytes(q_dtype) == 0 || elem_bytes(cache_dtype) == 0 || elem_bytes(v_cache_dtype) == 0)
    return fail(PA_ERR_INVALID_ARG, "unknown dtype code");
  const bool q16 = q_dtype == PA_DTYPE_BF16 || q_dtype == PA_DTYPE_F16;
  const bool same = q_dtype == cache_dtype && q_dtype != PA_DTYPE_FP8_E4M3 && q_dtype != PA_DTYPE_INT8;
  const bool fp8 = cache_dtype == PA_DTYPE_FP8_E4M3 && q16;
  const bool i8 = cache_dtype == PA_DTYPE_INT8 && q16;
  if (!same && !fp8 && !i8) return fail(PA_ERR_UNSUPPORTED, "unsupported (q, cache) dtype pair");
  // V: the K format, or (beside an fp8 K pool) the query type
  if (v_cache_dtype != cache_dtype && !(fp8 && v_cache_dtype == q_dtype))
    return fail(PA_ERR_UNSUPPORTED, "unsupported (K cache, V cache) dtype pair");
  return PA_OK;
}

struct Plan {
  int mode;
  int chunk;      // units of 32 tokens
  int max_parts;
  int max_len;
  size_t workspace;
};

constexpr int kUnit = 32;              // tokens per unit of decode work
constexpr int kMaxPlanSeqs = 8000;     // sequences whose plan fits in 64 KB of LDS

// Resolved partition request: > 0 fixed partitions of that many tokens,
// 0 balanced cut, -1 never split; any other value is invalid.
bool valid_request(int request, int block_size) {
  if (request == 0 || request == -1) return true;
  return request > 0 && request % kUnit == 0 && request % block_size == 0;
}

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

size_t workspace_for(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int max_parts) {
  const size_t rows = (size_t)num_seqs * num_q_heads * max_parts;
  return up256(rows * head_dim * sizeof(float)) + 2 * up256(rows * sizeof(float)) +
         up256((size_t)num_seqs * num_kv_heads * sizeof(int));
}

void fill_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int max_len,
               int request, Plan* plan) {
  const int umax = (max_len + kUnit - 1) / kUnit;
  plan->max_len = max_len;
  if (request == -1) {
    plan->mode = pa::kSplitNone;
    plan->chunk = umax > 0 ? umax : 1;
    plan->max_parts = 1;
    plan->workspace = 0;
    return;
  }
  if (request == 0) {
    // Balanced cut: ranges of at least max(2 units, a sixteenth of the
    // longest context), so a pair splits into at most 17 partials.
    plan->mode = pa::kSplitBalanced;
    plan->chunk = std::max(2, (umax + 15) / 16);
    plan->max_parts = (umax + plan->chunk - 1) / plan->chunk + 1;
  } else {
    plan->mode = pa::kSplitFixed;
    plan->chunk = request / kUnit;
    plan->max_parts = std::max(1, (umax + plan->chunk - 1) / plan->chunk);
  }
  plan->workspace = workspace_for(num_seqs, num_q_heads, num_kv_heads, head_dim, plan->max_parts);
}

pa_status plan_decode(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int max_blocks, int max_seq_len, int partition_size,
                      Plan* plan) {
  const long long cap = (long long)max_blocks * block_size;
  if (cap > (1 << 30)) return fail(PA_ERR_UNSUPPORTED, "block table too wide");
  if (max_seq_len < 0) return fail(PA_ERR_INVALID_ARG, "max_seq_len < 0");
  if (num_seqs > kMaxPlanSeqs)
    return fail(PA_ERR_UNSUPPORTED, "num_seqs %d > %d per call", num_seqs, kMaxPlanSeqs);
  if (!valid_request(partition_size, block_size))
    return fail(PA_ERR_INVALID_ARG,
                "partition_size %d: use 0, -1 or a positive multiple of 32 and of block_size",
                partition_size);
  const int max_len = (max_seq_len == 0 || max_seq_len > cap) ? (int)cap : max_seq_len;
  const long long units = (long long)num_seqs * ((max_len + kUnit - 1) / kUnit) * num_kv_heads;
  if (units > (1LL << 30))
    return fail(PA_ERR_UNSUPPORTED, "batch too large: %lld (sequence, KV head, 32-token) units",
                units);
  fill_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_len, partition_size, plan);
  return PA_OK;
}

// Workspace of pa_decode_noalloc, for callers that cannot allocate: a
// file-scope device array (each GPU the library runs on holds its own copy
// until the process ends).  In host code `scratch` names a host-side stand-in;
// kernels get the device address that hipGetSymbolAddress returns, looked up
// once per device on the first call made on it.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's copy of `scratch`.
pa_status scratch_address(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device ordinal %d >= %d", dev, kMaxDevices);
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] {
    slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
    if (slot.err == hipSuccess && slot.ptr == nullptr) slot.err = hipErrorInvalidSymbol;
  });
  if (slot.err != hipSuccess) return hip_status(slot.err, "hipGetSymbolAddress(scratch)");
  *out = slot.ptr;
  return PA_OK;
}

enum class Stage { kBoth, kAttention, kReduce };

// Checks a decode call and fills its kernel parameters; *work is false when
// there is nothing to enqueue (no sequences).
pa_status decode_setup(pa::DecodeParams* params, bool* work, void* out, const void* q,
                       const void* k_pool, const void* v_pool, const int32_t* block_tables,
                       const int32_t* seq_lens, float scale, int32_t block_size, int32_t num_seqs,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_blocks_per_seq, int32_t max_seq_len, pa_dtype q_dtype,
                       pa_dtype cache_dtype, pa_dtype v_cache_dtype, float k_scale, float v_scale,
                       int32_t partition_size, void* workspace, size_t workspace_bytes,
                       const float* k_scales, const float* v_scales, const void* new_k,
                       const void* new_v, int64_t new_k_stride, int64_t new_v_stride,
                       bool use_scratch) {
  *work = false;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs < 0");
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "num_seqs > 65535");
  pa_status st = check_attention_shape(num_q_heads, num_kv_heads, head_dim, block_size,
                                       max_blocks_per_seq, q_dtype, cache_dtype, v_cache_dtype);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_INVALID_ARG, "scale, k_scale and v_scale must be finite");
  const bool append = new_k != nullptr || new_v != nullptr;
  if (append) {
    if (!new_k || !new_v) return fail(PA_ERR_INVALID_ARG, "append needs both new_k and new_v");
    if (q_dtype != cache_dtype || v_cache_dtype != cache_dtype ||
        (q_dtype != PA_DTYPE_BF16 && q_dtype != PA_DTYPE_F16))
      return fail(PA_ERR_UNSUPPORTED, "append supports bf16/f16 queries with a cache of the same type");
    const int64_t dense = (int64_t)num_kv_heads * head_dim;
    if (new_k_stride == 0) new_k_stride = dense;
    if (new_v_stride == 0) new_v_stride = dense;
    if (new_k_stride < dense || new_v_stride < dense || (new_k_stride * 2) % 16 || (new_v_stride * 2) % 16)
      return fail(PA_ERR_INVALID_ARG, "new-token strides must be >= num_kv_heads * head_dim and keep rows 16-byte aligned");
    if (!aligned(new_k, 16) || !aligned(new_v, 16))
      return fail(PA_ERR_INVALID_ARG, "misaligned new-token pointer");
  }
  if (cache_dtype == PA_DTYPE_INT8) {
    if (!k_scales || !v_scales)
      return fail(PA_ERR_INVALID_ARG, "an int8 cache needs its per-block scales (pa_decode_int8)");
    if (!aligned(k_scales, 4) || !aligned(v_scales, 4))
      return fail(PA_ERR_INVALID_ARG, "misaligned per-block scales");
  }
  Plan plan;
  st = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                   max_seq_len, partition_size, &plan);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !seq_lens)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer (tensors need 16 bytes, int arrays 4)");
  if (use_scratch && plan.workspace > 0) {
    // the no-allocation entry: the library's own device array, never hipMalloc
    if (plan.workspace > kScratchBytes)
      return fail(PA_ERR_WORKSPACE,
                  "this call needs %zu bytes of split-KV workspace; the no-allocation entry holds "
                  "at most %zu (use pa_decode with a caller workspace)",
                  plan.workspace, kScratchBytes);
    st = scratch_address(&workspace);
    if (st != PA_OK) return st;
    workspace_bytes = kScratchBytes;
  }
  if (plan.workspace > 0) {
    if (!workspace || workspace_bytes < plan.workspace)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.workspace,
                  workspace_bytes);
    if (!aligned(workspace, 256)) return fail(PA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  }

  pa::DecodeParams& p = *params;
  p = pa::DecodeParams{};
  p.out = out;
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  if (plan.workspace > 0) {
    const size_t rows = (size_t)num_seqs * num_q_heads * plan.max_parts;
    char* ws = static_cast<char*>(workspace);
    const size_t o_bytes = up256(rows * head_dim * sizeof(float));
    const size_t ml_bytes = up256(rows * sizeof(float));
    p.part_o = reinterpret_cast<float*>(ws);
    p.part_m = reinterpret_cast<float*>(ws + o_bytes);
    p.part_l = reinterpret_cast<float*>(ws + o_bytes + ml_bytes);
    p.nparts = reinterpret_cast<int*>(ws + o_bytes + 2 * ml_bytes);
  }
  p.qk_scale_log2 = scale * k_scale * 1.4426950408889634f;
  p.v_scale = v_scale;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks = max_blocks_per_seq;
  p.max_len = plan.max_len;
  p.mode = plan.mode;
  p.chunk = plan.chunk;
  p.max_parts = plan.max_parts;
  p.q_dtype = q_dtype;
  p.cache_dtype = cache_dtype;
  p.v_cache_dtype = v_cache_dtype;
  p.k_scales = k_scales;
  p.v_scales = v_scales;
  p.new_k = append ? new_k : nullptr;
  p.new_v = append ? new_v : nullptr;
  p.new_k_stride = new_k_stride;
  p.new_v_stride = new_v_stride;
  *work = true;
  return PA_OK;
}

pa_status decode_impl(Stage stage, void* out, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                      float scale, int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                      int32_t max_seq_len, pa_dtype q_dtype, pa_dtype cache_dtype,
                      pa_dtype v_cache_dtype, float k_scale, float v_scale,
                      int32_t partition_size, void* workspace, size_t workspace_bytes,
                      void* stream, const float* k_scales = nullptr,
                      const float* v_scales = nullptr, const void* new_k = nullptr,
                      const void* new_v = nullptr, int64_t new_k_stride = 0,
                      int64_t new_v_stride = 0, bool use_scratch = false) {
  pa::DecodeParams p;
  bool work = false;
  const pa_status st = decode_setup(&p, &work, out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                                    block_size, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                    max_blocks_per_seq, max_seq_len, q_dtype, cache_dtype,
                                    v_cache_dtype, k_scale, v_scale, partition_size, workspace,
                                    workspace_bytes, k_scales, v_scales, new_k, new_v, new_k_stride,
                                    new_v_stride, use_scratch);
  if (st != PA_OK) return st;
  if (!work) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (stage != Stage::kReduce) {
    hipError_t e = pa::launch_decode_attention(p, s);
    if (e != hipSuccess) return hip_status(e, "decode attention launch");
  }
  if (stage != Stage::kAttention) {
    hipError_t e = pa::launch_decode_reduce(p, s);
    if (e != hipSuccess) return hip_status(e, "decode reduce launch");
  }
  return ok();
}

}  // namespace

namespace pa {
// Status with a message for pa_last_error(), for the other host-side files.
pa_status report(pa_status code, const char* message) {
  if (code == PA_OK) return ok();
  return fail(code, "%s", message);
}
}  // namespace pa

extern "C" {

static pa_status scatter_impl(const void* key, const void* value, void* k_pool, void* v_pool,
                              const int64_t* slot_mapping, int32_t num_tokens,
                              int64_t key_token_stride, int64_t value_token_stride,
                              int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, pa_dtype src_dtype, pa_dtype k_cache_dtype,
                              pa_dtype v_cache_dtype, float k_scale, float v_scale, void* stream,
                              const float* k_scales, const float* v_scales) {
  const pa_dtype cache_dtype = k_cache_dtype;
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0 || block_size <= 0)
    return fail(PA_ERR_INVALID_ARG, "negative size or non-positive heads/block_size");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d (supported: 8, 16, 32, 64)", block_size);
  const int seb = elem_bytes(src_dtype), ceb = elem_bytes(cache_dtype);
  if (seb == 0 || ceb == 0 || elem_bytes(v_cache_dtype) == 0)
    return fail(PA_ERR_INVALID_ARG, "unknown dtype code");
  if (src_dtype == PA_DTYPE_INT8) return fail(PA_ERR_UNSUPPORTED, "int8 is not a source type");
  const bool same = src_dtype == cache_dtype;
  const bool quant = cache_dtype == PA_DTYPE_FP8_E4M3 && src_dtype != PA_DTYPE_FP8_E4M3;
  const bool i8 = cache_dtype == PA_DTYPE_INT8 && src_dtype != PA_DTYPE_FP8_E4M3;
  if (!same && !quant && !i8) return fail(PA_ERR_UNSUPPORTED, "unsupported (src, cache) dtype pair");
  if (i8 && (!k_scales || !v_scales))
    return fail(PA_ERR_INVALID_ARG, "an int8 cache needs its per-block scales (pa_reshape_and_cache_int8)");
  if (i8 && (!aligned(k_scales, 4) || !aligned(v_scales, 4)))
    return fail(PA_ERR_INVALID_ARG, "misaligned per-block scales");
  // V: the K format, or (beside an fp8 K pool) the source type
  if (v_cache_dtype != cache_dtype && !(quant && v_cache_dtype == src_dtype))
    return fail(PA_ERR_UNSUPPORTED, "unsupported (K cache, V cache) dtype pair");
  if (quant && !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0 && v_scale > 0))
    return fail(PA_ERR_INVALID_ARG, "fp8 scales must be finite and positive");
  const int64_t dense = (int64_t)num_kv_heads * head_dim;
  if (key_token_stride == 0) key_token_stride = dense;
  if (value_token_stride == 0) value_token_stride = dense;
  if (key_token_stride < dense || value_token_stride < dense)
    return fail(PA_ERR_INVALID_ARG, "token stride smaller than num_kv_heads * head_dim");
  if ((key_token_stride * seb) % 16 || (value_token_stride * seb) % 16)
    return fail(PA_ERR_INVALID_ARG, "token strides must keep rows 16-byte aligned");
  if (num_tokens == 0) return ok();
  if (!key || !value || !k_pool || !v_pool || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer");
  pa::ScatterParams p{};
  p.key = key;
  p.value = value;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.slot_mapping = slot_mapping;
  p.key_stride = key_token_stride;
  p.value_stride = value_token_stride;
  p.num_tokens = num_tokens;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.src_dtype = src_dtype;
  p.cache_dtype = cache_dtype;
  p.v_cache_dtype = v_cache_dtype;
  p.src_elem_bytes = seb;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.k_scales = k_scales;
  p.v_scales = v_scales;
  return hip_status(pa::launch_scatter(p, static_cast<hipStream_t>(stream)), "scatter launch");
}

pa_status pa_reshape_and_cache_kv(const void* key, const void* value, void* k_pool, void* v_pool,
                                  const int64_t* slot_mapping, int32_t num_tokens,
                                  int64_t key_token_stride, int64_t value_token_stride,
                                  int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, pa_dtype src_dtype, pa_dtype k_cache_dtype,
                                  pa_dtype v_cache_dtype, float k_scale, float v_scale, void* stream) {
  return scatter_impl(key, value, k_pool, v_pool, slot_mapping, num_tokens, key_token_stride,
                      value_token_stride, num_blocks, num_kv_heads, head_dim, block_size, src_dtype,
                      k_cache_dtype, v_cache_dtype, k_scale, v_scale, stream, nullptr, nullptr);
}

pa_status pa_reshape_and_cache_int8(const void* key, const void* value, void* k_pool, void* v_pool,
                                    const float* k_scales, const float* v_scales,
                                    const int64_t* slot_mapping, int32_t num_tokens,
                                    int64_t key_token_stride, int64_t value_token_stride,
                                    int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, pa_dtype src_dtype, void* stream) {
  return scatter_impl(key, value, k_pool, v_pool, slot_mapping, num_tokens, key_token_stride,
                      value_token_stride, num_blocks, num_kv_heads, head_dim, block_size, src_dtype,
                      PA_DTYPE_INT8, PA_DTYPE_INT8, 1.0f, 1.0f, stream, k_scales, v_scales);
}

pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_pool, void* v_pool,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int64_t key_token_stride, int64_t value_token_stride,
                               int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, pa_dtype src_dtype, pa_dtype cache_dtype,
                               float k_scale, float v_scale, void* stream) {
  return pa_reshape_and_cache_kv(key, value, k_pool, v_pool, slot_mapping, num_tokens,
                                 key_token_stride, value_token_stride, num_blocks, num_kv_heads,
                                 head_dim, block_size, src_dtype, cache_dtype, cache_dtype, k_scale,
                                 v_scale, stream);
}

pa_status pa_copy_blocks(void* k_pool, void* v_pool, const int64_t* block_pairs, int32_t num_pairs,
                         int64_t block_bytes, void* stream) {
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs < 0");
  if (num_pairs > 65535) return fail(PA_ERR_UNSUPPORTED, "num_pairs > 65535");
  if (block_bytes <= 0 || block_bytes % 16)
    return fail(PA_ERR_INVALID_ARG, "block_bytes must be a positive multiple of 16");
  if (num_pairs == 0) return ok();
  if (!k_pool || !v_pool || !block_pairs) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(block_pairs, 8))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer");
  pa::CopyParams p{};
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.pairs = block_pairs;
  p.block_bytes = block_bytes;
  p.num_pairs = num_pairs;
  return hip_status(pa::launch_copy_blocks(p, static_cast<hipStream_t>(stream)), "copy launch");
}

pa_status pa_copy_blocks_partial(void* k_pool, void* v_pool, const int64_t* block_triples, int32_t num_pairs,
                                 int32_t num_kv_heads, int32_t block_size, int64_t row_bytes, void* stream) {
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs < 0");
  if (num_pairs > 65535) return fail(PA_ERR_UNSUPPORTED, "num_pairs > 65535");
  if (num_kv_heads <= 0 || block_size <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads and block_size must be > 0");
  if (row_bytes <= 0 || row_bytes % 16)
    return fail(PA_ERR_INVALID_ARG, "row_bytes must be a positive multiple of 16");
  if (num_pairs == 0) return ok();
  if (!k_pool || !v_pool || !block_triples) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(block_triples, 8))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer");
  pa::CopyRowsParams p{};
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.triples = block_triples;
  p.row_bytes = row_bytes;
  p.num_kv_heads = num_kv_heads;
  p.block_size = block_size;
  p.num_pairs = num_pairs;
  return hip_status(pa::launch_copy_rows(p, static_cast<hipStream_t>(stream)), "partial copy launch");
}

pa_status pa_copy_blocks_layers(void* const* k_pools, void* const* v_pools, int32_t num_layers,
                                const int64_t* block_pairs, int32_t num_pairs, int64_t block_bytes,
                                void* stream) {
  if (num_pairs < 0 || num_layers < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs or num_layers < 0");
  if (num_pairs > 65535 || num_layers > 65535) return fail(PA_ERR_UNSUPPORTED, "num_pairs or num_layers > 65535");
  if (block_bytes <= 0 || block_bytes % 16)
    return fail(PA_ERR_INVALID_ARG, "block_bytes must be a positive multiple of 16");
  if (num_pairs == 0 || num_layers == 0) return ok();
  if (!k_pools || !v_pools || !block_pairs) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(k_pools, 8) || !aligned(v_pools, 8) || !aligned(block_pairs, 8))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer");
  pa::CopyLayersParams p{};
  p.k_pools = k_pools;
  p.v_pools = v_pools;
  p.pairs = block_pairs;
  p.block_bytes = block_bytes;
  p.num_pairs = num_pairs;
  p.num_layers = num_layers;
  return hip_status(pa::launch_copy_layers(p, static_cast<hipStream_t>(stream)), "layer copy launch");
}

namespace {
// Address at which kernels reach `ptr`: device memory as it is, pinned host
// memory through its device mapping; pageable host memory is rejected.
bool device_address(const void* ptr, const void** out) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, ptr) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged || a.type == hipMemoryTypeUnified) {
    *out = ptr;
    return true;
  }
  if (a.type == hipMemoryTypeHost && a.devicePointer && a.hostPointer) {
    *out = static_cast<const char*>(a.devicePointer) +
           (static_cast<const char*>(ptr) - static_cast<const char*>(a.hostPointer));
    return true;
  }
  return false;
}
}  // namespace

pa_status pa_swap_blocks(void* dst_pool, const void* src_pool, const int64_t* block_pairs, int32_t num_pairs,
                         int64_t block_bytes, void* stream) {
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs < 0");
  if (num_pairs > 65535) return fail(PA_ERR_UNSUPPORTED, "num_pairs > 65535");
  if (block_bytes <= 0 || block_bytes % 16)
    return fail(PA_ERR_INVALID_ARG, "block_bytes must be a positive multiple of 16");
  if (num_pairs == 0) return ok();
  if (!dst_pool || !src_pool || !block_pairs) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(dst_pool, 16) || !aligned(src_pool, 16) || !aligned(block_pairs, 8))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer");
  const void *d = nullptr, *s = nullptr, *pr = nullptr;
  if (!device_address(dst_pool, &d) || !device_address(src_pool, &s) || !device_address(block_pairs, &pr))
    return fail(PA_ERR_INVALID_ARG, "pools and pairs must be device memory or pinned host memory");
  pa::SwapParams p{};
  p.dst = const_cast<void*>(d);
  p.src = s;
  p.pairs = static_cast<const int64_t*>(pr);
  p.block_bytes = block_bytes;
  p.num_pairs = num_pairs;
  return hip_status(pa::launch_swap_blocks(p, static_cast<hipStream_t>(stream)), "swap launch");
}

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                                 int32_t max_seq_len, int32_t partition_size) {
  (void)num_seqs;
  (void)num_kv_heads;
  if (max_seq_len <= 0 || (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64))
    return -1;
  if (!valid_request(partition_size, block_size)) return -1;
  if (partition_size == -1) return (max_seq_len + kUnit - 1) / kUnit * kUnit;
  return partition_size;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                                 int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len <= 0) return 0;
  if (!valid_request(partition_size, block_size)) return 0;
  Plan plan;
  fill_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition_size, &plan);
  return plan.workspace;
}

pa_status pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, const int32_t* seq_lens, float scale,
                    int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                    int32_t max_seq_len, pa_dtype q_dtype, pa_dtype cache_dtype, float k_scale,
                    float v_scale, int32_t partition_size, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return decode_impl(Stage::kBoth, out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                     block_size, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     max_blocks_per_seq, max_seq_len, q_dtype, cache_dtype, cache_dtype, k_scale,
                     v_scale, partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* seq_lens, float scale,
                            int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                            int32_t max_seq_len, pa_dtype q_dtype, pa_dtype cache_dtype,
                            float k_scale, float v_scale, int32_t partition_size, void* stream) {
  return decode_impl(Stage::kBoth, out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                     block_size, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     max_blocks_per_seq, max_seq_len, q_dtype, cache_dtype, cache_dtype, k_scale,
                     v_scale, partition_size, nullptr, 0, stream, nullptr, nullptr, nullptr,
                     nullptr, 0, 0, /*use_scratch=*/true);
}

size_t pa_decode_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

pa_status pa_decode_attention(void* out, const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens, float scale,
                              int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, pa_dtype q_dtype, pa_dtype cache_dtype,
                              float k_scale, float v_scale, int32_t partition_size,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(Stage::kAttention, out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                     block_size, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     max_blocks_per_seq, max_seq_len, q_dtype, cache_dtype, cache_dtype, k_scale,
                     v_scale, partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_decode_reduce(void* out, const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* seq_lens, float scale,
                           int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                           int32_t max_seq_len, pa_dtype q_dtype, pa_dtype cache_dtype,
                           float k_scale, float v_scale, int32_t partition_size, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return decode_impl(Stage::kReduce, out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                     block_size, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     max_blocks_per_seq, max_seq_len, q_dtype, cache_dtype, cache_dtype, k_scale,
                     v_scale, partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_decode_kv(void* out, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* seq_lens, float scale,
                       int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                       int32_t max_seq_len, pa_dtype q_dtype, pa_dtype k_cache_dtype,
                       pa_dtype v_cache_dtype, float k_scale, float v_scale,
                       int32_t partition_size, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return decode_impl(Stage::kBoth, out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                     block_size, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     max_blocks_per_seq, max_seq_len, q_dtype, k_cache_dtype, v_cache_dtype,
                     k_scale, v_scale, partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_decode_attention_kv(void* out, const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, const int32_t* seq_lens, float scale,
                                 int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                                 int32_t max_seq_len, pa_dtype q_dtype, pa_dtype k_cache_dtype,
                                 pa_dtype v_cache_dtype, float k_scale, float v_scale,
                                 int32_t partition_size, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return decode_impl(Stage::kAttention, out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                     block_size, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     max_blocks_per_seq, max_seq_len, q_dtype, k_cache_dtype, v_cache_dtype,
                     k_scale, v_scale, partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_decode_reduce_kv(void* out, const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens, float scale,
                              int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, pa_dtype q_dtype, pa_dtype k_cache_dtype,
                              pa_dtype v_cache_dtype, float k_scale, float v_scale,
                              int32_t partition_size, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return decode_impl(Stage::kReduce, out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                     block_size, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     max_blocks_per_seq, max_seq_len, q_dtype, k_cache_dtype, v_cache_dtype,
                     k_scale, v_scale, partition_size, workspace, workspace_bytes, stream);
}

#define PA_DECODE_INT8(NAME, STAGE)                                                           \
  pa_status NAME(void* out, const void* q, const void* k_pool, const void* v_pool,              \
                 const float* k_scales, const float* v_scales, const int32_t* block_tables,      \
                 const int32_t* seq_lens, float scale, int32_t block_size, int32_t num_seqs,     \
                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,                    \
                 int32_t max_blocks_per_seq, int32_t max_seq_len, pa_dtype q_dtype,              \
                 int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) { \
    return decode_impl(STAGE, out, q, k_pool, v_pool, block_tables, seq_lens, scale, block_size, \
                       num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,       \
                       max_seq_len, q_dtype, PA_DTYPE_INT8, PA_DTYPE_INT8, 1.0f, 1.0f,          \
                       partition_size, workspace, workspace_bytes, stream, k_scales, v_scales); \
  }
PA_DECODE_INT8(pa_decode_int8, Stage::kBoth)
PA_DECODE_INT8(pa_decode_attention_int8, Stage::kAttention)
PA_DECODE_INT8(pa_decode_reduce_int8, Stage::kReduce)
#undef PA_DECODE_INT8

#define PA_DECODE_APPEND(NAME, STAGE)                                                          \
  pa_status NAME(void* out, const void* q, const void* new_k, const void* new_v,                \
                 int64_t new_k_stride, int64_t new_v_stride, void* k_pool, void* v_pool,        \
                 const int32_t* block_tables, const int32_t* seq_lens, float scale,             \
                 int32_t block_size, int32_t num_seqs, int32_t num_q_heads,                     \
                 int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,            \
                 int32_t max_seq_len, pa_dtype q_dtype, pa_dtype cache_dtype, float k_scale,    \
                 float v_scale, int32_t partition_size, void* workspace,                        \
                 size_t workspace_bytes, void* stream) {                                        \
    if (!new_k || !new_v) return fail(PA_ERR_INVALID_ARG, "append needs new_k and new_v");     \
    return decode_impl(STAGE, out, q, k_pool, v_pool, block_tables, seq_lens, scale, block_size, \
                       num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,       \
                       max_seq_len, q_dtype, cache_dtype, cache_dtype, k_scale, v_scale,        \
                       partition_size, workspace, workspace_bytes, stream, nullptr, nullptr,    \
                       new_k, new_v, new_k_stride, new_v_stride);                               \
  }
PA_DECODE_APPEND(pa_decode_append, Stage::kBoth)
PA_DECODE_APPEND(pa_decode_attention_append, Stage::kAttention)
#undef PA_DECODE_APPEND

namespace {

// Checks a prefill call and fills its kernel parameters; *work is false when
// there is nothing to enqueue (no sequences or no query tokens).
pa_status prefill_setup(pa::PrefillParams* params, bool* work, void* out, const void* q,
                        const int32_t* query_start_loc, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, const int32_t* seq_lens, float scale,
                        int32_t block_size, int32_t num_seqs, int32_t total_q_tokens,
                        int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t max_blocks_per_seq, pa_dtype q_dtype,
                        pa_dtype cache_dtype, float k_scale, float v_scale,
                        const float* k_scales = nullptr, const float* v_scales = nullptr) {
  *work = false;
  if (num_seqs < 0 || total_q_tokens < 0 || max_q_len < 0)
    return fail(PA_ERR_INVALID_ARG, "negative size");
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "num_seqs > 65535");
  pa_status st = check_attention_shape(num_q_heads, num_kv_heads, head_dim, block_size,
                                       max_blocks_per_seq, q_dtype, cache_dtype, cache_dtype);
  if (st != PA_OK) return st;
  if (cache_dtype != q_dtype && cache_dtype != PA_DTYPE_FP8_E4M3 && cache_dtype != PA_DTYPE_INT8)
    return fail(PA_ERR_UNSUPPORTED,
                "prefill supports a cache of the query's type (f32, f16, bf16) or an fp8 or int8 cache "
                "beside bf16/f16 queries");
  if (cache_dtype == PA_DTYPE_INT8) {
    if (!k_scales || !v_scales)
      return fail(PA_ERR_INVALID_ARG, "an int8 cache needs its per-block scales (pa_prefill_chunk_int8)");
    if (!aligned(k_scales, 4) || !aligned(v_scales, 4))
      return fail(PA_ERR_INVALID_ARG, "misaligned per-block scales");
  }
  const int group = num_q_heads / num_kv_heads;
  if (q_dtype != PA_DTYPE_F32 && (group & (group - 1)))
    return fail(PA_ERR_UNSUPPORTED, "prefill over 16-bit or fp8 caches needs a power-of-two group");
  if (!std::isfinite(scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_INVALID_ARG, "scales must be finite");
  if ((long long)max_blocks_per_seq * block_size > (1 << 30))
    return fail(PA_ERR_UNSUPPORTED, "block table too wide");
  if (pa::prefill_smem_bytes(head_dim) > 160 * 1024)
    return fail(PA_ERR_UNSUPPORTED, "K/V tile stages do not fit in LDS");
  if (num_seqs == 0 || total_q_tokens == 0 || max_q_len == 0) return PA_OK;
  if (!out || !q || !query_start_loc || !k_pool || !v_pool || !block_tables || !seq_lens)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(query_start_loc, 4))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer");
  const int qpos = 128 / group;
  if ((max_q_len + qpos - 1) / qpos > 0x7FFFFFFF / 2) return fail(PA_ERR_UNSUPPORTED, "grid too large");
  pa::PrefillParams& p = *params;
  p = pa::PrefillParams{};
  p.out = out;
  p.q = q;
  p.query_start_loc = query_start_loc;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.qk_scale_log2 = scale * k_scale * 1.4426950408889634f;
  p.v_scale = v_scale;
  p.num_seqs = num_seqs;
  p.total_q = total_q_tokens;
  p.max_q_len = max_q_len;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks = max_blocks_per_seq;
  p.q_dtype = q_dtype;
  p.cache_dtype = cache_dtype;
  p.k_scales = k_scales;
  p.v_scales = v_scales;
  *work = true;
  return PA_OK;
}

}  // namespace

pa_status pa_prefill_chunk(void* out, const void* q, const int32_t* query_start_loc,
                           const void* k_pool, const void* v_pool, const int32_t* block_tables,
                           const int32_t* seq_lens, float scale, int32_t block_size,
                           int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t max_blocks_per_seq, pa_dtype q_dtype, pa_dtype cache_dtype,
                           float k_scale, float v_scale, void* stream) {
  pa::PrefillParams p;
  bool work = false;
  const pa_status st = prefill_setup(&p, &work, out, q, query_start_loc, k_pool, v_pool, block_tables,
                                     seq_lens, scale, block_size, num_seqs, total_q_tokens,
                                     max_q_len, num_q_heads, num_kv_heads, head_dim,
                                     max_blocks_per_seq, q_dtype, cache_dtype, k_scale, v_scale);
  if (st != PA_OK) return st;
  if (!work) return ok();
  return hip_status(pa::launch_prefill(p, static_cast<hipStream_t>(stream)), "prefill launch");
}

pa_status pa_prefill_chunk_int8(void* out, const void* q, const int32_t* query_start_loc,
                                const void* k_pool, const void* v_pool, const float* k_scales,
                                const float* v_scales, const int32_t* block_tables,
                                const int32_t* seq_lens, float scale, int32_t block_size,
                                int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_blocks_per_seq, pa_dtype q_dtype, void* stream) {
  if (q_dtype != PA_DTYPE_BF16 && q_dtype != PA_DTYPE_F16)
    return fail(PA_ERR_UNSUPPORTED, "an int8 cache takes bf16 or f16 queries");
  pa::PrefillParams p;
  bool work = false;
  const pa_status st = prefill_setup(&p, &work, out, q, query_start_loc, k_pool, v_pool, block_tables,
                                     seq_lens, scale, block_size, num_seqs, total_q_tokens,
                                     max_q_len, num_q_heads, num_kv_heads, head_dim,
                                     max_blocks_per_seq, q_dtype, PA_DTYPE_INT8, 1.0f, 1.0f, k_scales,
                                     v_scales);
  if (st != PA_OK) return st;
  if (!work) return ok();
  return hip_status(pa::launch_prefill(p, static_cast<hipStream_t>(stream)), "prefill launch");
}

static pa_status mixed_impl(void* prefill_out, const void* prefill_q, const int32_t* query_start_loc,
                            const int32_t* prefill_block_tables, const int32_t* prefill_seq_lens,
                            int32_t num_chunks, int32_t total_q_tokens, int32_t max_q_len,
                            int32_t prefill_max_blocks_per_seq, void* decode_out, const void* decode_q,
                            const int32_t* decode_block_tables, const int32_t* decode_seq_lens,
                            int32_t num_decodes, int32_t decode_max_blocks_per_seq, int32_t max_seq_len,
                            const void* k_pool, const void* v_pool, float scale, int32_t block_size,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, pa_dtype q_dtype,
                            pa_dtype cache_dtype, float k_scale, float v_scale, const float* k_scales,
                            const float* v_scales, int32_t partition_size, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if ((q_dtype != PA_DTYPE_BF16 && q_dtype != PA_DTYPE_F16) ||
      (cache_dtype != q_dtype && cache_dtype != PA_DTYPE_FP8_E4M3 && cache_dtype != PA_DTYPE_INT8))
    return fail(PA_ERR_UNSUPPORTED,
                "the mixed-step launch supports bf16/f16 queries over a cache of the same type, fp8 or "
                "int8");
  pa::PrefillParams pf{};
  bool pf_work = false;
  pa_status st = prefill_setup(&pf, &pf_work, prefill_out, prefill_q, query_start_loc, k_pool,
                               v_pool, prefill_block_tables, prefill_seq_lens, scale, block_size,
                               num_chunks, total_q_tokens, max_q_len, num_q_heads, num_kv_heads,
                               head_dim, prefill_max_blocks_per_seq, q_dtype, cache_dtype, k_scale,
                               v_scale, k_scales, v_scales);
  if (st != PA_OK) return st;
  pa::DecodeParams d{};
  bool d_work = false;
  st = decode_setup(&d, &d_work, decode_out, decode_q, k_pool, v_pool, decode_block_tables,
                    decode_seq_lens, scale, block_size, num_decodes, num_q_heads, num_kv_heads,
                    head_dim, decode_max_blocks_per_seq, max_seq_len, q_dtype, cache_dtype,
                    cache_dtype, k_scale, v_scale, partition_size, workspace, workspace_bytes,
                    k_scales, v_scales, nullptr, nullptr, 0, 0, false);
  if (st != PA_OK) return st;
  if (!pf_work) pf.num_seqs = 0;   // no query tokens: no prefill tiles
  if (!d_work) d.num_seqs = 0;
  if (!pf_work && !d_work) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = pa::launch_mixed(pf, d, s);
  if (e != hipSuccess) return hip_status(e, "mixed-step launch");
  if (d_work) {
    e = pa::launch_decode_reduce(d, s);
    if (e != hipSuccess) return hip_status(e, "decode reduce launch");
  }
  return ok();
}

pa_status pa_mixed_attention(void* prefill_out, const void* prefill_q,
                             const int32_t* query_start_loc, const int32_t* prefill_block_tables,
                             const int32_t* prefill_seq_lens, int32_t num_chunks,
                             int32_t total_q_tokens, int32_t max_q_len,
                             int32_t prefill_max_blocks_per_seq, void* decode_out,
                             const void* decode_q, const int32_t* decode_block_tables,
                             const int32_t* decode_seq_lens, int32_t num_decodes,
                             int32_t decode_max_blocks_per_seq, int32_t max_seq_len,
                             const void* k_pool, const void* v_pool, float scale,
                             int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, pa_dtype q_dtype, pa_dtype cache_dtype,
                             float k_scale, float v_scale, int32_t partition_size,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (cache_dtype == PA_DTYPE_INT8)
    return fail(PA_ERR_INVALID_ARG, "an int8 cache needs its per-block scales (pa_mixed_attention_int8)");
  return mixed_impl(prefill_out, prefill_q, query_start_loc, prefill_block_tables, prefill_seq_lens,
                    num_chunks, total_q_tokens, max_q_len, prefill_max_blocks_per_seq, decode_out, decode_q,
                    decode_block_tables, decode_seq_lens, num_decodes, decode_max_blocks_per_seq,
                    max_seq_len, k_pool, v_pool, scale, block_size, num_q_heads, num_kv_heads, head_dim,
                    q_dtype, cache_dtype, k_scale, v_scale, nullptr, nullptr, partition_size, workspace,
                    workspace_bytes, stream);
}

pa_status pa_mixed_attention_int8(void* prefill_out, const void* prefill_q,
                                  const int32_t* query_start_loc, const int32_t* prefill_block_tables,
                                  const int32_t* prefill_seq_lens, int32_t num_chunks,
                                  int32_t total_q_tokens, int32_t max_q_len,
                                  int32_t prefill_max_blocks_per_seq, void* decode_out,
                                  const void* decode_q, const int32_t* decode_block_tables,
                                  const int32_t* decode_seq_lens, int32_t num_decodes,
                                  int32_t decode_max_blocks_per_seq, int32_t max_seq_len,
                                  const void* k_pool, const void* v_pool, const float* k_scales,
                                  const float* v_scales, float scale, int32_t block_size,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  pa_dtype q_dtype, int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!k_scales || !v_scales) return fail(PA_ERR_INVALID_ARG, "an int8 cache needs its per-block scales");
  return mixed_impl(prefill_out, prefill_q, query_start_loc, prefill_block_tables, prefill_seq_lens,
                    num_chunks, total_q_tokens, max_q_len, prefill_max_blocks_per_seq, decode_out, decode_q,
                    decode_block_tables, decode_seq_lens, num_decodes, decode_max_blocks_per_seq,
                    max_seq_len, k_pool, v_pool, scale, block_size, num_q_heads, num_kv_heads, head_dim,
                    q_dtype, PA_DTYPE_INT8, 1.0f, 1.0f, k_scales, v_scales, partition_size, workspace,
                    workspace_bytes, stream);
}

pa_status pa_check_block_tables(const int32_t* block_tables, const int32_t* seq_lens,
                                const int32_t* query_start_loc, int32_t num_seqs,
                                int32_t total_q_tokens, int32_t max_blocks_per_seq,
                                int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                                int32_t* error, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks < 0 ||
      max_seq_len < 0 || total_q_tokens < 0)
    return fail(PA_ERR_INVALID_ARG, "negative size or non-positive table width / block size");
  if (!error || !aligned(error, 4)) return fail(PA_ERR_INVALID_ARG, "null or misaligned error word");
  if (num_seqs > 0 && (!block_tables || !seq_lens || !aligned(block_tables, 4) || !aligned(seq_lens, 4) ||
                       (query_start_loc && !aligned(query_start_loc, 4))))
    return fail(PA_ERR_INVALID_ARG, "null or misaligned pointer");
  pa::CheckParams p{};
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.query_start_loc = query_start_loc;
  p.err = error;
  p.num_items = num_seqs;
  p.max_blocks = max_blocks_per_seq;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  p.max_len = max_seq_len;
  p.total = total_q_tokens;
  return hip_status(pa::launch_check(p, static_cast<hipStream_t>(stream)), "check launch");
}

pa_status pa_check_slots(const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                         int32_t block_size, int32_t* error, void* stream) {
  if (num_tokens < 0 || num_blocks < 0 || block_size <= 0)
    return fail(PA_ERR_INVALID_ARG, "negative size or non-positive block size");
  if (!error || !aligned(error, 4)) return fail(PA_ERR_INVALID_ARG, "null or misaligned error word");
  if (num_tokens > 0 && (!slot_mapping || !aligned(slot_mapping, 8)))
    return fail(PA_ERR_INVALID_ARG, "null or misaligned slot mapping");
  pa::CheckParams p{};
  p.slots = num_tokens > 0 ? slot_mapping : reinterpret_cast<const int64_t*>(error);  // non-null: slots mode
  p.err = error;
  p.num_items = num_tokens;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  return hip_status(pa::launch_check(p, static_cast<hipStream_t>(stream)), "check launch");
}

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
    default: return "PA_ERR_UNKNOWN";
  }
}

const char* pa_last_error(void) { return g_last_error; }

pa_status pa_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink || bytes % 16 || !aligned(src, 16) || !aligned(sink, 16))
    return fail(PA_ERR_INVALID_ARG, "probe_read: null/misaligned pointer or size not /16");
  return hip_status(pa::launch_probe_read(src, bytes, sink, static_cast<hipStream_t>(stream)),
                    "probe launch");
}

pa_status pa_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 || !aligned(src, 16) || !aligned(dst, 16))
    return fail(PA_ERR_INVALID_ARG, "probe_copy: null/misaligned pointer or size not /16");
  return hip_status(pa::launch_probe_copy(dst, src, bytes, static_cast<hipStream_t>(stream)),
                    "probe launch");
}

}  // extern "C"
