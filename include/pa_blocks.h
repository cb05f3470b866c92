/*
 * pa_blocks.h — host-side block manager of libpa and the copy-on-write block
 * copy, the producer of the block tables and slot mappings that pa.h's kernels
 * consume.
 *
 * What it keeps (page titles and sections as the sources):
 *  - a pool of fixed-size physical blocks allocated up front, each with a
 *    count of the requests using it; a request's logical blocks map to
 *    physical blocks through its block table ("大模型推理优化学习笔记",
 *    "逐出（LRU）"; "从静态批处理到状态化推理集群", "PagedAttention：把逻辑连续与物理
 *    连续分开");
 *  - allocation of the blocks a request's new tokens need (17 new tokens take
 *    ceil(17/16) = 2 blocks), taken from the head of a free queue and recorded
 *    in the request's table, failing without change when too few are free
 *    (vLLM architecture summary, "第一部分：LLM 引擎核心", allocate_slots);
 *  - prefix caching: every full block gets a hash of (the previous block's
 *    hash, its tokens, a salt); a new request takes over the longest run of
 *    cached blocks matching its prompt from the start; a block that is not
 *    full is never cached ("大模型推理优化学习笔记", "块哈希"; vLLM architecture
 *    summary, "第二部分：進階功能", Prefix Caching). A hit is confirmed on the
 *    block's exact tokens and salt and on the previous block's hash, not on
 *    its own hash alone;
 *  - release: a finished request's blocks whose count drops to zero go to the
 *    tail of the free queue with their contents and hash kept, so they can
 *    still be hit; allocation evicts from the head, least recently freed first
 *    ("大模型推理优化学习笔记", "逐出（LRU）");
 *  - sharing and copy-on-write: a fork shares all of a request's blocks (a
 *    subagent inheriting its parent's context, "宣稱省下 106 倍成本…", "vLLM 的
 *    解法：統一分頁 + 共用池"); a shared block that is not full is copied before
 *    either branch appends to it ("从静态批处理到状态化推理集群", "Prefix reuse"), and
 *    the copy is returned as a (source, destination) pair for pa_copy_blocks.
 *
 * The manager is host memory only and not thread-safe (one scheduler thread
 * owns it). Functions returning pa_status set pa_last_error() on failure.
 */
#ifndef PA_BLOCKS_H
#define PA_BLOCKS_H

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A pool of num_blocks blocks of block_size tokens (block_size 16 for the
 * kernels; any size >= 1 is managed). NULL if num_blocks < 1 or
 * block_size < 1. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* bm);

/* Blocks on the free queue (unused, cached or not). */
int32_t pa_bm_num_free_blocks(const pa_block_manager* bm);

/*
 * Admits request req_id (which must not exist) with its prompt tokens[n] and
 * cache salt: takes the longest run of cached full blocks matching the prompt
 * from its start (at most n - 1 tokens: the last prompt token is always
 * computed), and sets *num_cached_tokens to the tokens they hold. The rest
 * of the prompt is then appended with pa_bm_append_tokens.
 */
pa_status pa_bm_add_request(pa_block_manager* bm, int64_t req_id, const int32_t* tokens, int32_t n,
                            uint64_t salt, int32_t* num_cached_tokens);

/*
 * Appends k tokens (their ids, for the hashes of the blocks they fill) to
 * req_id: allocates the blocks they need and writes the cache slot of each
 * new token (block_id * block_size + offset) to slots[k]. If the request's
 * last block is not full and is shared, it is first replaced by a fresh copy:
 * the pair (source, destination) is written to cow_pairs[0..1] and
 * *num_cow = 1 (else 0); the caller runs pa_copy_blocks on it before writing
 * the new tokens' K/V. PA_ERR_OUT_OF_BLOCKS (nothing changed) if the free
 * queue holds too few blocks.
 */
pa_status pa_bm_append_tokens(pa_block_manager* bm, int64_t req_id, const int32_t* token_ids, int32_t k,
                              int64_t* slots, int32_t* cow_pairs, int32_t* num_cow);

/* child_id (which must not exist) shares every block of parent_id. */
pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id);

/* Releases req_id; its blocks' counts drop, from its last block to its
 * first, and blocks reaching zero join the free queue's tail (still
 * cached). */
pa_status pa_bm_free_request(pa_block_manager* bm, int64_t req_id);

/* Tokens held by req_id and its block table (physical ids in logical order):
 * writes min(count, max_blocks) ids to blocks and the count to *num_blocks. */
pa_status pa_bm_request_info(const pa_block_manager* bm, int64_t req_id, int32_t* num_tokens, int32_t* blocks,
                             int32_t max_blocks, int32_t* num_blocks);

/* Reference count of one physical block (-1 if out of range). */
int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block_id);

/*
 * GPU: copies whole physical blocks — every KV head's K and V tiles and, for
 * fp8 caches, the blocks' scales — from pairs[i][0] to pairs[i][1] (int32
 * [num_pairs][2], device; destinations distinct and not sources; a pair with
 * an id outside [0, num_blocks) is skipped). Layouts as in pa.h.
 * num_pairs == 0 enqueues nothing.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale, const int32_t* pairs,
                         int32_t num_pairs, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         int32_t head_size, pa_dtype cache_dtype, pa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H */
