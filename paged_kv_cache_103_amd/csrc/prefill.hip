// Host dispatch of the chunked-prefill kernel (prefill_bf16.hip serves bf16
// and fp8 caches alike): what the prefill entry point supports, the query
// tokens per workgroup tile, and the launch.
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

int prefill_tokens_per_tile(int cache_kind, int group) {
  (void)cache_kind;
  return prefill_bf16_tokens_per_tile(group);
}

bool prefill_supported(int q_kind, int cache_kind, int head_size, int group) {
  if (head_size != 64 && head_size != 128) return false;
  if (!(group == 1 || group == 2 || group == 4 || group == 8 || group == 16)) return false;
  return q_kind == KBF16 && (cache_kind == KBF16 || cache_kind == KFP8);
}

hipError_t launch_prefill(const PrefillArgs& a, int cache_kind, int head_size, hipStream_t stream) {
  return launch_prefill_bf16(a, cache_kind, head_size, stream);
}

}  // namespace pa
