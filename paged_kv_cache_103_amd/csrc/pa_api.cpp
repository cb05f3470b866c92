// C ABI of libpa: host-side validation, launch planning and error mapping.
// The operations are defined in include/pa.h; this file only checks the
// arguments that can be checked on the host, sizes the split-K plan from host
// scalars (never reading device memory), and enqueues the kernels.
#include "pa.h"
#include "pa_blocks.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_last_error.clear();
    return PA_OK;
  }
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A second stream per device for work that runs beside the caller's stream
// (the one-token rows of a mixed batch beside its chunks), with the events
// that fork it from and join it back to the caller's stream. Created on
// first use at the default priority; guarded, with the enqueue sequence
// that uses it, by g_side_mu.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[64];

hipError_t side_stream_of_current_device(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  SideStream& ss = g_side[dev];
  if (ss.stream == nullptr) {
    SideStream n;
    e = hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.stream) (void)hipStreamDestroy(n.stream);
      return e;
    }
    ss = n;
  }
  *out = &ss;
  return hipSuccess;
}

bool known_dtype(pa_dtype d) { return d == PA_F32 || d == PA_BF16 || d == PA_FP8_E4M3; }
const char* dtype_name(pa_dtype d) {
  switch (d) {
    case PA_F32: return "f32";
    case PA_BF16: return "bf16";
    case PA_FP8_E4M3: return "fp8_e4m3";
  }
  return "unknown";
}

// Checks shared by the two attention entry points.
pa_status check_attention_common(const void* out, const void* query, const void* k_cache,
                                 const void* v_cache, const float* k_scale, const float* v_scale,
                                 const int32_t* block_table, int32_t block_table_stride,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_size, int32_t block_size, int32_t num_blocks,
                                 pa_dtype q_dtype, pa_dtype cache_dtype, float scale,
                                 int32_t sliding_window) {
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (block_size != PA_BLOCK_SIZE)
    return fail(PA_ERR_UNSUPPORTED, "block_size must be %d (got %d)", PA_BLOCK_SIZE, block_size);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_size must be 64 or 128 (got %d)", head_size);
  if (num_heads <= 0 || num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_heads (%d) and num_kv_heads (%d) must be > 0",
                num_heads, num_kv_heads);
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_heads (%d) must be a multiple of num_kv_heads (%d)",
                num_heads, num_kv_heads);
  if (!known_dtype(q_dtype) || !known_dtype(cache_dtype))
    return fail(PA_ERR_INVALID_ARGUMENT, "unknown dtype (q %d, cache %d)", (int)q_dtype,
                (int)cache_dtype);
  if (q_dtype == PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "fp8 queries are not supported (cache only)");
  if (!(scale > 0.0f) || scale != scale)
    return fail(PA_ERR_INVALID_ARGUMENT, "scale must be a positive number");
  if (sliding_window < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "sliding_window must be >= 0 (got %d)", sliding_window);
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks must be > 0 (got %d)", num_blocks);
  if (num_seqs == 0) return PA_OK;
  if (max_context_len <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_context_len must be > 0 (got %d)", max_context_len);
  if (block_table_stride < (max_context_len + block_size - 1) / block_size)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "block_table_stride (%d) is smaller than ceil(max_context_len/block_size) (%d)",
                block_table_stride, (max_context_len + block_size - 1) / block_size);
  if (!out || !query || !k_cache || !v_cache || !block_table || !context_lens)
    return fail(PA_ERR_INVALID_ARGUMENT, "null device pointer");
  if (cache_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale))
    return fail(PA_ERR_INVALID_ARGUMENT, "fp8 cache needs k_scale and v_scale");
  const int group = num_heads / num_kv_heads;
  if (!pa::decode_supported((int)q_dtype, (int)cache_dtype, head_size, group))
    return fail(PA_ERR_UNSUPPORTED, "no decode kernel for q %s, cache %s, head_size %d, group %d",
                dtype_name(q_dtype), dtype_name(cache_dtype), head_size, group);
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                               const float* k_scale, const float* v_scale,
                               const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                               int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                               pa_dtype in_dtype, pa_dtype cache_dtype, pa_stream_t stream) {
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_tokens must be >= 0 (got %d)", num_tokens);
  if (block_size != PA_BLOCK_SIZE)
    return fail(PA_ERR_UNSUPPORTED, "block_size must be %d (got %d)", PA_BLOCK_SIZE, block_size);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_size must be 64 or 128 (got %d)", head_size);
  if (num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_kv_heads must be > 0 (got %d)", num_kv_heads);
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks must be > 0 (got %d)", num_blocks);
  if (!known_dtype(in_dtype) || !known_dtype(cache_dtype))
    return fail(PA_ERR_INVALID_ARGUMENT, "unknown dtype (in %d, cache %d)", (int)in_dtype, (int)cache_dtype);
  if (in_dtype != cache_dtype && cache_dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "write from %s into a %s cache is not supported",
                dtype_name(in_dtype), dtype_name(cache_dtype));
  if (in_dtype == PA_FP8_E4M3 && cache_dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "fp8 input needs an fp8 cache");
  const bool quantise = cache_dtype == PA_FP8_E4M3 && in_dtype != PA_FP8_E4M3;
  if (num_tokens == 0) {
    g_last_error.clear();
    return PA_OK;
  }
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARGUMENT, "null device pointer");
  if (quantise && (!k_scale || !v_scale))
    return fail(PA_ERR_INVALID_ARGUMENT, "quantising write needs k_scale and v_scale");
  hipError_t e = pa::launch_reshape_and_cache(key, value, k_cache, v_cache, k_scale, v_scale,
                                              slot_mapping, num_tokens, num_kv_heads, head_size,
                                              (int)in_dtype, (int)cache_dtype, (hipStream_t)stream);
  return hip_status(e, "reshape_and_cache launch");
}

static int elem_bytes(pa_dtype d) { return d == PA_F32 ? 4 : (d == PA_BF16 ? 2 : 1); }

// The supported (query, cache) pairs are (f32, f32), (bf16, bf16) and
// (bf16, fp8): the cache type decides the query type.
static pa::DecodePlan make_plan(int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_size, pa_dtype cache_dtype,
                                int32_t sliding_window, bool force_valu = false) {
  const int q_kind = cache_dtype == PA_F32 ? PA_F32 : PA_BF16;
  return pa::plan_decode(num_seqs, max_context_len, num_heads, num_kv_heads, head_size, q_kind,
                         (int)cache_dtype, sliding_window, force_valu);
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Points the decode arguments' summary buffers into the workspace.
static void bind_workspace(pa::DecodeArgs& a, const pa::DecodePlan& plan, void* workspace, int32_t num_seqs,
                           int32_t num_heads, int32_t num_kv_heads, int32_t head_size) {
  a.pb = plan.pb;
  a.max_parts = plan.max_parts;
  a.split_waves = plan.split_waves;
  a.one_per_stream = plan.one_per_stream;
  a.meta = nullptr;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.cu_groups = nullptr;
  a.group_prefix_len = nullptr;
  a.num_groups = 0;
  a.rec_cols = num_heads / num_kv_heads;
  if (workspace == nullptr) return;
  char* ws = static_cast<char*>(workspace);
  if (plan.split_waves > 0) {
    const int G = num_heads / num_kv_heads;
    const size_t slots = (size_t)plan.split_waves + (size_t)num_seqs * num_kv_heads;
    a.meta = reinterpret_cast<int*>(ws);
    ws += align256((size_t)(num_seqs + 2) * sizeof(int));
    a.part_o = reinterpret_cast<float*>(ws);
    ws += align256(slots * G * head_size * sizeof(float));
    a.part_ml = reinterpret_cast<float*>(ws);
  } else if (plan.max_parts > 1) {
    const size_t slots = (size_t)num_seqs * num_heads * plan.max_parts;
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float*>(ws) + slots * head_size;
  }
}

// Sequences per launch of pa_decode: batches the matrix-core kernel serves
// run as consecutive launches over groups of at most kMfmaMaxSeqs sequences
// (sequences are independent), each reusing the same workspace.
static int32_t decode_group_seqs(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, pa_dtype cache_dtype,
                                 bool force_valu) {
  const int q_kind = cache_dtype == PA_F32 ? PA_F32 : PA_BF16;
  const int G = std::max(1, num_heads / std::max(1, num_kv_heads));
  if (!force_valu && pa::decode_uses_mfma(q_kind, (int)cache_dtype, G)) return std::min(num_seqs, pa::kMfmaMaxSeqs);
  return num_seqs;
}

static size_t decode_ws_bytes(int32_t num_seqs, int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_size, pa_dtype cache_dtype, int32_t sliding_window, bool force_valu) {
  if (num_seqs <= 0 || max_context_len <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0)
    return 0;
  const int32_t n = decode_group_seqs(num_seqs, num_heads, num_kv_heads, cache_dtype, force_valu);
  const pa::DecodePlan plan = make_plan(n, max_context_len, num_heads, num_kv_heads, head_size, cache_dtype,
                                        sliding_window, force_valu);
  return pa::decode_workspace_bytes(plan, n, num_heads, num_kv_heads, head_size);
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_size, pa_dtype cache_dtype,
                                 int32_t sliding_window) {
  return decode_ws_bytes(num_seqs, max_context_len, num_heads, num_kv_heads, head_size, cache_dtype,
                         sliding_window, false);
}

size_t pa_decode_valu_workspace_bytes(int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_size, pa_dtype cache_dtype,
                                      int32_t sliding_window) {
  return decode_ws_bytes(num_seqs, max_context_len, num_heads, num_kv_heads, head_size, cache_dtype,
                         sliding_window, true);
}

size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_q_tokens, int32_t max_q_len,
                                  int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_size, pa_dtype cache_dtype, int32_t sliding_window) {
  // the prefill tiles need no scratch; one-token rows use the decode plan,
  // and there are none when every sequence has max_q_len > 1 tokens
  if (max_q_len > 1 && (long long)num_q_tokens == (long long)num_seqs * max_q_len) return 0;
  return pa_decode_workspace_bytes(num_seqs, max_context_len, num_heads, num_kv_heads, head_size,
                                   cache_dtype, sliding_window);
}

// pa_decode, pa_decode_partial when lse is given, pa_decode_valu with
// force_valu.
static pa_status decode_impl(void* out, float* lse, const void* query, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, const int32_t* block_table,
                             int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                             int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size, int32_t num_blocks, pa_dtype q_dtype,
                             pa_dtype cache_dtype, float scale, int32_t sliding_window, void* workspace,
                             size_t workspace_bytes, pa_stream_t stream, bool force_valu = false) {
  pa_status st = check_attention_common(out, query, k_cache, v_cache, k_scale, v_scale, block_table,
                                        block_table_stride, context_lens, num_seqs, max_context_len,
                                        num_heads, num_kv_heads, head_size, block_size, num_blocks,
                                        q_dtype, cache_dtype, scale, sliding_window);
  if (st != PA_OK) return st;
  if (num_seqs == 0) {
    g_last_error.clear();
    return PA_OK;
  }
  const int32_t group = decode_group_seqs(num_seqs, num_heads, num_kv_heads, cache_dtype, force_valu);
  const pa::DecodePlan plan = make_plan(group, max_context_len, num_heads, num_kv_heads, head_size,
                                        cache_dtype, sliding_window, force_valu);
  if (lse != nullptr && plan.split_waves <= 0)
    return fail(PA_ERR_UNSUPPORTED, "partial decode needs the matrix-core kernel (bf16 queries, bf16 or fp8 "
                "cache)");
  const size_t need = pa::decode_workspace_bytes(plan, group, num_heads, num_kv_heads, head_size);
  if (workspace_bytes < need || (need > 0 && workspace == nullptr))
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "decode needs %zu workspace bytes (got %zu)", need,
                workspace_bytes);
  const size_t row_bytes = (size_t)num_heads * head_size * elem_bytes(q_dtype);  // a query / output row
  for (int32_t s0 = 0; s0 < num_seqs; s0 += group) {
    const int32_t n = std::min(group, num_seqs - s0);
    pa::DecodeArgs a{};
    a.out = static_cast<char*>(out) + (size_t)s0 * row_bytes;
    a.query = static_cast<const char*>(query) + (size_t)s0 * row_bytes;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_table = block_table + (size_t)s0 * block_table_stride;
    a.context_lens = context_lens + s0;
    a.cu_seqlens = nullptr;
    bind_workspace(a, plan, need ? workspace : nullptr, n, num_heads, num_kv_heads, head_size);
    a.bt_stride = block_table_stride;
    a.num_seqs = n;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.window = sliding_window;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.lse = lse != nullptr ? lse + (size_t)s0 * num_heads : nullptr;
    hipError_t e = pa::launch_decode(a, (int)q_dtype, (int)cache_dtype, head_size, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "decode launch");
  }
  g_last_error.clear();
  return PA_OK;
}

pa_status pa_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
                    const float* k_scale, const float* v_scale, const int32_t* block_table,
                    int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                    int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_size, int32_t block_size, int32_t num_blocks, pa_dtype q_dtype,
                    pa_dtype cache_dtype, float scale, int32_t sliding_window, void* workspace,
                    size_t workspace_bytes, pa_stream_t stream) {
  return decode_impl(out, nullptr, query, k_cache, v_cache, k_scale, v_scale, block_table, block_table_stride,
                     context_lens, num_seqs, max_context_len, num_heads, num_kv_heads, head_size, block_size,
                     num_blocks, q_dtype, cache_dtype, scale, sliding_window, workspace, workspace_bytes, stream);
}

pa_status pa_decode_valu(void* out, const void* query, const void* k_cache, const void* v_cache,
                         const float* k_scale, const float* v_scale, const int32_t* block_table,
                         int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                         int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                         int32_t block_size, int32_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype,
                         float scale, int32_t sliding_window, void* workspace, size_t workspace_bytes,
                         pa_stream_t stream) {
  return decode_impl(out, nullptr, query, k_cache, v_cache, k_scale, v_scale, block_table, block_table_stride,
                     context_lens, num_seqs, max_context_len, num_heads, num_kv_heads, head_size, block_size,
                     num_blocks, q_dtype, cache_dtype, scale, sliding_window, workspace, workspace_bytes, stream,
                     true);
}

pa_status pa_decode_noalloc(void* out, const void* query, const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale, const int32_t* block_table,
                            int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                            int32_t block_size, int32_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype,
                            float scale, int32_t sliding_window, pa_stream_t stream) {
  // every argument check before the scratch array is looked up
  pa_status st = check_attention_common(out, query, k_cache, v_cache, k_scale, v_scale, block_table,
                                        block_table_stride, context_lens, num_seqs, max_context_len,
                                        num_heads, num_kv_heads, head_size, block_size, num_blocks,
                                        q_dtype, cache_dtype, scale, sliding_window);
  if (st != PA_OK) return st;
  if (num_seqs == 0) {
    g_last_error.clear();
    return PA_OK;
  }
  const size_t need = decode_ws_bytes(num_seqs, max_context_len, num_heads, num_kv_heads, head_size, cache_dtype,
                                      sliding_window, false);
  if (need > pa::kNoallocScratchBytes)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                "this decode needs %zu bytes of scratch; the no-allocation entry point holds %zu "
                "(use pa_decode with a workspace)",
                need, pa::kNoallocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = hipSuccess;
    ws = pa::noalloc_scratch(&e);
    if (ws == nullptr) return hip_status(e == hipSuccess ? hipErrorInvalidSymbol : e, "scratch lookup");
  }
  return decode_impl(out, nullptr, query, k_cache, v_cache, k_scale, v_scale, block_table, block_table_stride,
                     context_lens, num_seqs, max_context_len, num_heads, num_kv_heads, head_size, block_size,
                     num_blocks, q_dtype, cache_dtype, scale, sliding_window, ws, need, stream);
}

pa_status pa_decode_partial(void* out, float* lse, const void* query, const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale, const int32_t* block_table,
                            int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                            int32_t block_size, int32_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype,
                            float scale, void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  if (lse == nullptr && num_seqs > 0) return fail(PA_ERR_INVALID_ARGUMENT, "null device pointer (lse)");
  return decode_impl(out, lse, query, k_cache, v_cache, k_scale, v_scale, block_table, block_table_stride,
                     context_lens, num_seqs, max_context_len, num_heads, num_kv_heads, head_size, block_size,
                     num_blocks, q_dtype, cache_dtype, scale, 0, workspace, workspace_bytes, stream);
}

// Batches of more than mla_max_seqs() sequences run as consecutive launches
// over groups of that many sequences (sequences are independent), each
// reusing the same workspace.
size_t pa_mla_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads) {
  if (num_seqs <= 0 || num_heads <= 0) return 0;
  return pa::mla_workspace_bytes(std::min(num_seqs, pa::mla_max_seqs()), num_heads, pa::device_cu_count());
}

pa_status pa_mla_decode(void* out, const void* query, const void* latent_cache, const int32_t* block_table,
                        int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                        int32_t max_context_len, int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
                        int32_t block_size, int32_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype, float scale,
                        void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (block_size != PA_BLOCK_SIZE)
    return fail(PA_ERR_UNSUPPORTED, "block_size must be %d (got %d)", PA_BLOCK_SIZE, block_size);
  if (head_dim_v != 512) return fail(PA_ERR_UNSUPPORTED, "head_dim_v must be 512 (got %d)", head_dim_v);
  if (head_dim_k != 512 && head_dim_k != 576)
    return fail(PA_ERR_UNSUPPORTED, "head_dim_k must be 512 or 576 (got %d)", head_dim_k);
  if (num_heads != 16 && num_heads != 32 && num_heads != 64 && num_heads != 128)
    return fail(PA_ERR_UNSUPPORTED, "num_heads must be 16, 32, 64 or 128 (got %d)", num_heads);
  if (q_dtype != PA_BF16 || cache_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "latent decode takes bf16 queries and a bf16 cache");
  if (!(scale > 0.0f) || scale != scale) return fail(PA_ERR_INVALID_ARGUMENT, "scale must be a positive number");
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks must be > 0 (got %d)", num_blocks);
  if (num_seqs == 0) {
    g_last_error.clear();
    return PA_OK;
  }
  if (max_context_len <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_context_len must be > 0 (got %d)", max_context_len);
  if (block_table_stride < (max_context_len + 15) / 16)
    return fail(PA_ERR_INVALID_ARGUMENT, "block_table_stride (%d) is smaller than ceil(max_context_len/16) (%d)",
                block_table_stride, (max_context_len + 15) / 16);
  if (!out || !query || !latent_cache || !block_table || !context_lens)
    return fail(PA_ERR_INVALID_ARGUMENT, "null device pointer");
  const int grid = pa::device_cu_count();
  const int group = pa::mla_max_seqs();
  const size_t need = pa::mla_workspace_bytes(std::min(num_seqs, group), num_heads, grid);
  if (workspace_bytes < need || workspace == nullptr)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "latent decode needs %zu workspace bytes (got %zu)", need,
                workspace_bytes);
  for (int32_t s0 = 0; s0 < num_seqs; s0 += group) {  // (one launch pair per group of sequences)
    const int32_t n = std::min(group, num_seqs - s0);
    pa::MlaArgs a{};
    a.out = static_cast<uint16_t*>(out) + (size_t)s0 * num_heads * head_dim_v;
    a.query = static_cast<const uint16_t*>(query) + (size_t)s0 * num_heads * head_dim_k;
    a.cache = latent_cache;
    a.block_table = block_table + (size_t)s0 * block_table_stride;
    a.context_lens = context_lens + s0;
    pa::mla_bind_workspace(a, workspace, n, num_heads, grid);
    a.bt_stride = block_table_stride;
    a.num_seqs = n;
    a.num_heads = num_heads;
    a.scale_log2 = scale * 1.4426950408889634f;
    hipError_t e = pa::launch_mla_decode(a, head_dim_k, grid, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "latent decode launch");
  }
  g_last_error.clear();
  return PA_OK;
}

pa_status pa_merge_partials(void* out, float* lse_out, const void* parts, const float* parts_lse, int32_t num_parts,
                            int32_t num_rows, int32_t head_size, pa_dtype dtype, pa_stream_t stream) {
  if (num_parts < 1) return fail(PA_ERR_INVALID_ARGUMENT, "num_parts must be >= 1 (got %d)", num_parts);
  if (num_rows < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_rows must be >= 0 (got %d)", num_rows);
  if (head_size != 64 && head_size != 128 && head_size != 512)
    return fail(PA_ERR_UNSUPPORTED, "head_size must be 64, 128 or 512 (got %d)", head_size);
  if (dtype != PA_F32 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "merge dtype must be f32 or bf16 (got %d)", (int)dtype);
  if (num_rows == 0) {
    g_last_error.clear();
    return PA_OK;
  }
  if (!out || !parts || !parts_lse) return fail(PA_ERR_INVALID_ARGUMENT, "null device pointer");
  hipError_t e = pa::launch_merge_lse(out, lse_out, parts, parts_lse, num_parts, num_rows, head_size, (int)dtype,
                                      (hipStream_t)stream);
  return hip_status(e, "merge launch");
}

// Whether pa_decode_shared_prefix reads shared blocks once (else it serves
// the request as pa_decode).
static bool shared_prefix_applies(int32_t num_seqs, int32_t num_groups, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_size, pa_dtype cache_dtype, int32_t sliding_window) {
  if (num_groups <= 0 || num_seqs <= 0 || num_seqs > pa::kSharedPrefixMaxSeqs || sliding_window != 0) return false;
  if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return false;
  const pa::DecodePlan plan = make_plan(num_seqs, 1, num_heads, num_kv_heads, head_size, cache_dtype, 0);
  return plan.split_waves > 0;
}

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_groups, int32_t max_context_len,
                                               int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                               pa_dtype cache_dtype, int32_t sliding_window) {
  if (!shared_prefix_applies(num_seqs, num_groups, num_heads, num_kv_heads, head_size, cache_dtype,
                             sliding_window))
    return pa_decode_workspace_bytes(num_seqs, max_context_len, num_heads, num_kv_heads, head_size, cache_dtype,
                                     sliding_window);
  return pa::decode_shared_prefix_workspace_bytes(num_seqs, num_groups, num_heads, num_kv_heads, head_size);
}

pa_status pa_decode_shared_prefix(void* out, const void* query, const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale, const int32_t* block_table,
                                  int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                                  int32_t max_context_len, const int32_t* cu_groups,
                                  const int32_t* group_prefix_len, int32_t num_groups, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                  int32_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype, float scale,
                                  int32_t sliding_window, void* workspace, size_t workspace_bytes,
                                  pa_stream_t stream) {
  if (num_groups < 0 || num_groups > std::max(num_seqs, 0))
    return fail(PA_ERR_INVALID_ARGUMENT, "num_groups must be in [0, num_seqs] (got %d for %d sequences)",
                num_groups, num_seqs);
  if (num_groups > 0 && (!cu_groups || !group_prefix_len))
    return fail(PA_ERR_INVALID_ARGUMENT, "null device pointer (cu_groups / group_prefix_len)");
  pa_status st = check_attention_common(out, query, k_cache, v_cache, k_scale, v_scale, block_table,
                                        block_table_stride, context_lens, num_seqs, max_context_len,
                                        num_heads, num_kv_heads, head_size, block_size, num_blocks,
                                        q_dtype, cache_dtype, scale, sliding_window);
  if (st != PA_OK) return st;
  if (!shared_prefix_applies(num_seqs, num_groups, num_heads, num_kv_heads, head_size, cache_dtype,
                             sliding_window))
    return pa_decode(out, query, k_cache, v_cache, k_scale, v_scale, block_table, block_table_stride,
                     context_lens, num_seqs, max_context_len, num_heads, num_kv_heads, head_size, block_size,
                     num_blocks, q_dtype, cache_dtype, scale, sliding_window, workspace, workspace_bytes,
                     stream);
  const size_t need = pa::decode_shared_prefix_workspace_bytes(num_seqs, num_groups, num_heads, num_kv_heads,
                                                               head_size);
  if (workspace_bytes < need || workspace == nullptr)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "shared-prefix decode needs %zu workspace bytes (got %zu)", need,
                workspace_bytes);
  const pa::DecodePlan plan = make_plan(num_seqs, max_context_len, num_heads, num_kv_heads, head_size,
                                        cache_dtype, sliding_window);
  pa::DecodeArgs a{};
  a.out = out;
  a.query = query;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.cu_seqlens = nullptr;
  a.pb = plan.pb;
  a.max_parts = plan.max_parts;
  a.split_waves = plan.split_waves;
  char* ws = static_cast<char*>(workspace);
  const size_t slots = (size_t)plan.split_waves + (size_t)2 * num_seqs * num_kv_heads;
  a.meta = reinterpret_cast<int*>(ws);
  ws += align256((size_t)pa::shared_prefix_meta_ints(num_seqs, num_groups) * sizeof(int));
  a.part_o = reinterpret_cast<float*>(ws);
  ws += align256(slots * 16 * head_size * sizeof(float));
  a.part_ml = reinterpret_cast<float*>(ws);
  a.cu_groups = cu_groups;
  a.group_prefix_len = group_prefix_len;
  a.num_groups = num_groups;
  a.rec_cols = 16;
  a.bt_stride = block_table_stride;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.window = 0;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = pa::launch_decode(a, (int)q_dtype, (int)cache_dtype, head_size, (hipStream_t)stream);
  return hip_status(e, "shared-prefix decode launch");
}

// The selection's compacted tables and their key counts.
static size_t sparse_table_bytes(int32_t num_seqs, int32_t max_selected) {
  return align256((size_t)num_seqs * (size_t)(max_selected + 1) * sizeof(int)) +
         align256((size_t)num_seqs * sizeof(int));
}

size_t pa_decode_sparse_workspace_bytes(int32_t num_seqs, int32_t max_selected, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_size, pa_dtype cache_dtype) {
  if (num_seqs <= 0 || max_selected < 0 || max_selected > pa::kSparseMaxSelected || num_heads <= 0 ||
      num_kv_heads <= 0 || head_size <= 0)
    return 0;
  return sparse_table_bytes(num_seqs, max_selected) +
         pa_decode_workspace_bytes(num_seqs, 16 * (max_selected + 1), num_heads, num_kv_heads, head_size,
                                   cache_dtype, 0);
}

pa_status pa_decode_sparse(void* out, const void* query, const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale, const int32_t* block_table,
                           int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                           int32_t max_context_len, const int32_t* selected_blocks, int32_t selected_stride,
                           const int32_t* num_selected, int32_t max_selected, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_size, int32_t block_size, int32_t num_blocks,
                           pa_dtype q_dtype, pa_dtype cache_dtype, float scale, void* workspace,
                           size_t workspace_bytes, pa_stream_t stream) {
  if (max_selected < 0 || max_selected > pa::kSparseMaxSelected)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_selected must be in [0, %d] (got %d)", pa::kSparseMaxSelected,
                max_selected);
  if (max_selected > 0 && (!selected_blocks || !num_selected))
    return fail(PA_ERR_INVALID_ARGUMENT, "null device pointer (selected_blocks / num_selected)");
  if (max_selected > 0 && selected_stride < max_selected)
    return fail(PA_ERR_INVALID_ARGUMENT, "selected_stride (%d) is smaller than max_selected (%d)",
                selected_stride, max_selected);
  pa_status st = check_attention_common(out, query, k_cache, v_cache, k_scale, v_scale, block_table,
                                        block_table_stride, context_lens, num_seqs, max_context_len,
                                        num_heads, num_kv_heads, head_size, block_size, num_blocks,
                                        q_dtype, cache_dtype, scale, 0);
  if (st != PA_OK) return st;
  if (num_seqs == 0) {
    g_last_error.clear();
    return PA_OK;
  }
  if (pa::sparse_select_lds_bytes(max_context_len, pa::kSparseRankMax) > pa::kSparseMaxLds)
    return fail(PA_ERR_UNSUPPORTED, "max_context_len %d is beyond the sparse decode's block bitmap",
                max_context_len);
  const size_t need = pa_decode_sparse_workspace_bytes(num_seqs, max_selected, num_heads, num_kv_heads, head_size,
                                                       cache_dtype);
  if (workspace_bytes < need || workspace == nullptr)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "sparse decode needs %zu workspace bytes (got %zu)", need,
                workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  pa::SparseSelectArgs sa{};
  sa.block_table = block_table;
  sa.bt_stride = block_table_stride;
  sa.context_lens = context_lens;
  sa.selected = selected_blocks;
  sa.sel_stride = selected_stride;
  sa.num_selected = max_selected > 0 ? num_selected : nullptr;
  sa.max_selected = max_selected;
  sa.blocks_max = (max_context_len + 15) / 16;
  sa.words_max = (sa.blocks_max + 31) / 32;
  sa.cbt = reinterpret_cast<int*>(ws);
  sa.cbt_stride = max_selected + 1;
  sa.eff_ctx = reinterpret_cast<int*>(ws + align256((size_t)num_seqs * (size_t)(max_selected + 1) * sizeof(int)));
  sa.rank_list = pa::sparse_select_lds_bytes(max_context_len, max_selected) >
                 pa::sparse_select_lds_bytes(max_context_len, pa::kSparseRankMax);

  const int32_t eff_max = 16 * (max_selected + 1);
  const int32_t dgroup = decode_group_seqs(num_seqs, num_heads, num_kv_heads, cache_dtype, false);
  const pa::DecodePlan plan = make_plan(dgroup, eff_max, num_heads, num_kv_heads, head_size, cache_dtype, 0);
  pa::DecodeArgs a{};
  a.out = out;
  a.query = query;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.cu_seqlens = nullptr;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.window = 0;
  a.scale_log2 = scale * 1.4426950408889634f;
  // Two or more streams per CU and a short list on the matrix-core kernel:
  // one launch (a workgroup per stream selects, decodes and merges).
  if (plan.split_waves > 0 && (long long)num_seqs * num_kv_heads >= 2LL * pa::device_cu_count() &&
      pa::decode_sparse_fused_lds_bytes(sa.words_max, max_selected, num_heads / num_kv_heads, head_size) > 0) {
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.bt_stride = block_table_stride;
    bind_workspace(a, plan, nullptr, num_seqs, num_heads, num_kv_heads, head_size);
    hipError_t e = pa::launch_decode_sparse_fused(a, sa, (int)cache_dtype, head_size, (hipStream_t)stream);
    return hip_status(e, "sparse decode launch");
  }
  hipError_t e = pa::launch_sparse_select(sa, num_seqs, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "sparse block selection launch");
  // the decode over the compacted tables, in groups of sequences as pa_decode
  const size_t dec_need = pa::decode_workspace_bytes(plan, dgroup, num_heads, num_kv_heads, head_size);
  const size_t row_bytes = (size_t)num_heads * head_size * elem_bytes(q_dtype);
  for (int32_t s0 = 0; s0 < num_seqs; s0 += dgroup) {
    const int32_t n = std::min(dgroup, num_seqs - s0);
    a.out = static_cast<char*>(out) + (size_t)s0 * row_bytes;
    a.query = static_cast<const char*>(query) + (size_t)s0 * row_bytes;
    a.block_table = sa.cbt + (size_t)s0 * sa.cbt_stride;
    a.context_lens = sa.eff_ctx + s0;
    bind_workspace(a, plan, dec_need ? ws + sparse_table_bytes(num_seqs, max_selected) : nullptr, n, num_heads,
                   num_kv_heads, head_size);
    a.bt_stride = sa.cbt_stride;
    a.num_seqs = n;
    e = pa::launch_decode(a, (int)q_dtype, (int)cache_dtype, head_size, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "sparse decode launch");
  }
  g_last_error.clear();
  return PA_OK;
}

pa_status pa_prefill_chunk(void* out, const void* query, const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale, const int32_t* block_table,
                           int32_t block_table_stride, const int32_t* cu_seqlens,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_tokens,
                           int32_t max_q_len, int32_t max_context_len, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                           int32_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype, float scale,
                           int32_t sliding_window, void* workspace, size_t workspace_bytes,
                           pa_stream_t stream) {
  pa_status st = check_attention_common(out, query, k_cache, v_cache, k_scale, v_scale, block_table,
                                        block_table_stride, context_lens, num_seqs, max_context_len,
                                        num_heads, num_kv_heads, head_size, block_size, num_blocks,
                                        q_dtype, cache_dtype, scale, sliding_window);
  if (st != PA_OK) return st;
  if (num_seqs == 0) {
    g_last_error.clear();
    return PA_OK;
  }
  if (!cu_seqlens) return fail(PA_ERR_INVALID_ARGUMENT, "null cu_seqlens");
  if (num_q_tokens < num_seqs)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_q_tokens (%d) < num_seqs (%d): every sequence needs a query",
                num_q_tokens, num_seqs);
  if (max_q_len < 1 || max_q_len > num_q_tokens || max_q_len > max_context_len)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_q_len (%d) must be in [1, min(num_q_tokens, max_context_len)]",
                max_q_len);
  const int group = num_heads / num_kv_heads;
  const bool has_chunks = max_q_len > 1;
  if (has_chunks && !pa::prefill_supported((int)q_dtype, (int)cache_dtype, head_size, group))
    return fail(PA_ERR_UNSUPPORTED, "no prefill kernel for q %s, cache %s, head_size %d, group %d",
                dtype_name(q_dtype), dtype_name(cache_dtype), head_size, group);
  // Rows with one query token may exist unless every sequence provably has
  // max_q_len > 1 tokens (the only case the host scalars can prove).
  const bool any_single = !(has_chunks && (long long)num_q_tokens == (long long)num_seqs * max_q_len);
  // (one-token rows of more than kMfmaMaxSeqs sequences: groups, as pa_decode)
  const int32_t dgroup = decode_group_seqs(num_seqs, num_heads, num_kv_heads, cache_dtype, false);
  const pa::DecodePlan plan = make_plan(dgroup, max_context_len, num_heads, num_kv_heads, head_size,
                                        cache_dtype, sliding_window);
  const size_t need =
      any_single ? pa::decode_workspace_bytes(plan, dgroup, num_heads, num_kv_heads, head_size) : 0;
  if (workspace_bytes < need || (need > 0 && workspace == nullptr))
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "prefill needs %zu workspace bytes (got %zu)", need,
                workspace_bytes);
  const hipStream_t hs = (hipStream_t)stream;
  const float scale_log2 = scale * 1.4426950408889634f;

  // one-token rows: the decode kernel (skips rows of longer chunks; query
  // and output rows are addressed through cu_seqlens), for the sequences
  // [s0, s0 + n)
  auto decode_rows = [&](int32_t s0, int32_t n) {
    pa::DecodeArgs d{};
    d.out = out;
    d.query = query;
    d.k_cache = k_cache;
    d.v_cache = v_cache;
    d.k_scale = k_scale;
    d.v_scale = v_scale;
    d.block_table = block_table + (size_t)s0 * block_table_stride;
    d.context_lens = context_lens + s0;
    d.cu_seqlens = cu_seqlens + s0;
    bind_workspace(d, plan, need ? workspace : nullptr, n, num_heads, num_kv_heads, head_size);
    d.bt_stride = block_table_stride;
    d.num_seqs = n;
    d.num_heads = num_heads;
    d.num_kv_heads = num_kv_heads;
    d.window = sliding_window;
    d.scale_log2 = scale_log2;
    return d;
  };

  pa::PrefillArgs p{};
  if (has_chunks) {
    p.out = out;
    p.query = query;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.block_table = block_table;
    p.cu_seqlens = cu_seqlens;
    p.context_lens = context_lens;
    p.bt_stride = block_table_stride;
    p.num_seqs = num_seqs;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.window = sliding_window;
    p.scale_log2 = scale_log2;
    // bound on sum over sequences with q_len > 1 of ceil(q_len / TQ)
    const long long tq = pa::prefill_tokens_per_tile(group);
    const long long long_seqs = std::min<long long>(num_seqs, num_q_tokens / 2);
    const long long bound_a = long_seqs + (num_q_tokens + tq - 1) / tq;
    const long long bound_b = long_seqs * ((max_q_len + tq - 1) / tq);
    p.num_tiles = (int)std::min(bound_a, bound_b);
  }

  // A mixed batch: the chunks bound by the matrix cores, the one-token rows
  // by HBM ("从静态批处理到状态化推理集群", "Chunked prefill：在共置引擎里
  // 治理阶段干扰"). Where the shapes allow, the rows run on a second stream
  // beside the prefill kernel, one decode workgroup per CU next to each
  // prefill workgroup (both only read the cache and they write disjoint
  // rows of out); the caller's stream waits for both.
  bool beside = false;
  if (any_single && has_chunks && dgroup == num_seqs && plan.split_waves > 0 && !plan.one_per_stream &&
      pa::decode_side_supported((int)q_dtype, (int)cache_dtype, head_size, group)) {
    const size_t side = pa::decode_side_lds_bytes(num_seqs, group);
    const size_t pf = pa::prefill_lds_bytes((int)cache_dtype, head_size, group);
    const size_t cap = (size_t)pa::device_lds_per_cu();
    // more than half of a CU's LDS keeps a second decode workgroup off it
    beside = pf > 0 && 2 * side > cap && side + pf + 2048 <= cap &&
             plan.split_waves >= 4 * pa::device_cu_count();
  }
  if (beside) {
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream* ss = nullptr;
    hipError_t e = side_stream_of_current_device(&ss);
    if (e == hipSuccess) e = hipEventRecord(ss->fork, hs);
    if (e == hipSuccess) e = hipStreamWaitEvent(ss->stream, ss->fork, 0);
    if (e != hipSuccess) return hip_status(e, "side stream fork");
    p.nontemporal_kv = 1;
    e = pa::launch_prefill(p, (int)cache_dtype, head_size, hs);
    if (e != hipSuccess) return hip_status(e, "prefill launch");
    const hipError_t ed = pa::launch_decode_side(decode_rows(0, num_seqs), (int)cache_dtype, ss->stream);
    e = hipEventRecord(ss->join, ss->stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(hs, ss->join, 0);
    if (ed != hipSuccess) return hip_status(ed, "decode launch (one-token rows)");
    if (e != hipSuccess) return hip_status(e, "side stream join");
    g_last_error.clear();
    return PA_OK;
  }
  if (any_single) {
    for (int32_t s0 = 0; s0 < num_seqs; s0 += dgroup) {
      hipError_t e = pa::launch_decode(decode_rows(s0, std::min(dgroup, num_seqs - s0)), (int)q_dtype,
                                       (int)cache_dtype, head_size, hs);
      if (e != hipSuccess) return hip_status(e, "decode launch (one-token rows)");
    }
  }
  if (has_chunks) {
    hipError_t e = pa::launch_prefill(p, (int)cache_dtype, head_size, hs);
    if (e != hipSuccess) return hip_status(e, "prefill launch");
  }
  g_last_error.clear();
  return PA_OK;
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale, const int32_t* pairs,
                         int32_t num_pairs, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         int32_t head_size, pa_dtype cache_dtype, pa_stream_t stream) {
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_pairs must be >= 0 (got %d)", num_pairs);
  if (block_size != PA_BLOCK_SIZE)
    return fail(PA_ERR_UNSUPPORTED, "block_size must be %d (got %d)", PA_BLOCK_SIZE, block_size);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_size must be 64 or 128 (got %d)", head_size);
  if (num_kv_heads < 1 || num_blocks < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_kv_heads and num_blocks must be >= 1 (got %d, %d)", num_kv_heads,
                num_blocks);
  if (!known_dtype(cache_dtype)) return fail(PA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)cache_dtype);
  if (num_pairs == 0) {
    g_last_error.clear();
    return PA_OK;
  }
  if (!k_cache || !v_cache || !pairs) return fail(PA_ERR_INVALID_ARGUMENT, "null device pointer");
  if (cache_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale))
    return fail(PA_ERR_INVALID_ARGUMENT, "fp8 cache needs k_scale and v_scale");
  const size_t tile = (size_t)PA_BLOCK_SIZE * head_size * elem_bytes(cache_dtype);
  hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, cache_dtype == PA_FP8_E4M3 ? k_scale : nullptr,
                                        cache_dtype == PA_FP8_E4M3 ? v_scale : nullptr, pairs, num_pairs, tile,
                                        num_kv_heads, num_blocks, (hipStream_t)stream);
  return hip_status(e, "copy_blocks launch");
}

const char* pa_status_string(int32_t s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
  }
  return "PA_ERR_UNKNOWN";
}

const char* pa_last_error(void) { return g_last_error.c_str(); }


int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

}  // extern "C"

namespace pa {
pa_status set_error(pa_status st, const char* msg) {
  if (st == PA_OK) g_last_error.clear();
  else g_last_error = msg;
  return st;
}
}  // namespace pa
