// pa_check_batch (include/pa.h): the device-side preconditions of the
// attention and write calls, checked on host copies of a batch's metadata.
// The kernels never check them (a wrong block id reads the wrong block, or
// faults); a scheduler or a test can run this on every batch it builds.
//
// What is checked follows the paging rules the calls rely on: a sequence's
// logical block j lives in physical block block_table[s][j] and its slots
// are block * 16 + offset ("从静态批处理到状态化推理集群", "PagedAttention：
// 把逻辑连续与物理连续分开"; vLLM architecture summary, "第一部分：LLM 引擎核心",
// slot_mapping), and a block that more than one sequence maps is copied
// before it is written ("从静态批处理到状态化推理集群", "Prefix reuse：分页让
// 细粒度共享更便宜").
#include <stdint.h>

#include <algorithm>
#include <cstdio>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

pa_status bad(const char* fmt, long long a = 0, long long b = 0, long long c = 0, long long d = 0) {
  char buf[256];
  snprintf(buf, sizeof(buf), fmt, a, b, c, d);
  return pa::set_error(PA_ERR_INVALID_ARGUMENT, buf);
}

}  // namespace

extern "C" pa_status pa_check_batch(const int32_t* block_table, int32_t block_table_stride,
                                    const int32_t* context_lens, const int32_t* cu_seqlens, int32_t num_seqs,
                                    int32_t num_q_tokens, int32_t max_q_len, int32_t max_context_len,
                                    int32_t num_blocks, int32_t sliding_window, const int64_t* slot_mapping) {
  if (num_seqs < 0) return bad("num_seqs must be >= 0 (got %lld)", num_seqs);
  if (num_seqs == 0) return pa::set_error(PA_OK, "");
  if (!block_table || !context_lens) return bad("null host pointer (block_table / context_lens)");
  if (num_blocks <= 0) return bad("num_blocks must be > 0 (got %lld)", num_blocks);
  if (sliding_window < 0) return bad("sliding_window must be >= 0 (got %lld)", sliding_window);
  if (cu_seqlens == nullptr && num_q_tokens != num_seqs)
    return bad("a decode batch (no cu_seqlens) has one query per sequence: num_q_tokens %lld != num_seqs %lld",
               num_q_tokens, num_seqs);
  if (cu_seqlens != nullptr) {
    if (cu_seqlens[0] != 0) return bad("cu_seqlens[0] must be 0 (got %lld)", cu_seqlens[0]);
    if (cu_seqlens[num_seqs] != num_q_tokens)
      return bad("cu_seqlens[num_seqs] = %lld, num_q_tokens = %lld", cu_seqlens[num_seqs], num_q_tokens);
  }
  // references to each physical block among the blocks the batch reads
  std::vector<int32_t> refs((size_t)num_blocks, 0);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const long long ctx = context_lens[s];
    if (ctx < 1 || ctx > max_context_len)
      return bad("sequence %lld: context_lens %lld outside [1, max_context_len = %lld]", s, ctx, max_context_len);
    const long long nb = (ctx + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE;
    if (nb > block_table_stride)
      return bad("sequence %lld: %lld blocks > block_table_stride %lld", s, nb, block_table_stride);
    long long q_len = 1;
    if (cu_seqlens != nullptr) {
      q_len = (long long)cu_seqlens[s + 1] - cu_seqlens[s];
      if (q_len < 1 || q_len > ctx)
        return bad("sequence %lld: q_len %lld outside [1, context_lens = %lld]", s, q_len, ctx);
      if (q_len > max_q_len) return bad("sequence %lld: q_len %lld > max_q_len %lld", s, q_len, max_q_len);
    }
    // blocks read: from the first query's window start to the newest block
    long long lo = 0;
    if (sliding_window > 0) lo = std::max(0LL, ctx - q_len - sliding_window + 1);
    for (long long j = lo / PA_BLOCK_SIZE; j < nb; ++j) {
      const int32_t b = block_table[(size_t)s * block_table_stride + j];
      if (b < 0 || b >= num_blocks)
        return bad("sequence %lld, logical block %lld: block id %lld outside [0, num_blocks = %lld)", s, j, b,
                   num_blocks);
      ++refs[(size_t)b];
    }
  }
  if (slot_mapping != nullptr) {
    // every written slot is the token's own position in its sequence's
    // table, and its block is mapped by no other (sequence, logical block)
    std::vector<uint8_t> written((size_t)num_blocks * PA_BLOCK_SIZE, 0);
    for (int32_t s = 0; s < num_seqs; ++s) {
      const long long ctx = context_lens[s];
      const long long t0 = cu_seqlens ? cu_seqlens[s] : s;
      const long long q_len = cu_seqlens ? (long long)cu_seqlens[s + 1] - cu_seqlens[s] : 1;
      for (long long r = 0; r < q_len; ++r) {
        const int64_t slot = slot_mapping[t0 + r];
        if (slot < 0) continue;  // padding: skipped by the write
        const long long p = ctx - q_len + r;
        const long long want =
            (long long)block_table[(size_t)s * block_table_stride + p / PA_BLOCK_SIZE] * PA_BLOCK_SIZE +
            p % PA_BLOCK_SIZE;
        if (slot != want)
          return bad("token %lld (sequence %lld, position %lld): slot %lld is not the block table's", t0 + r, s, p,
                     slot);
        const long long b = slot / PA_BLOCK_SIZE;
        if (refs[(size_t)b] != 1)
          return bad("token %lld: slot %lld writes block %lld, which %lld (sequence, block) entries map "
                     "(copy it before writing)",
                     t0 + r, slot, b, refs[(size_t)b]);
        if (written[(size_t)slot]) return bad("token %lld: slot %lld written twice in one call", t0 + r, slot);
        written[(size_t)slot] = 1;
      }
    }
  }
  return pa::set_error(PA_OK, "");
}
