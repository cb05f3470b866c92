/*
 * pa.h — C ABI of libpa: attention over a paged KV cache on MI355X (gfx950).
 *
 * What the calls compute (sources are the page titles and sections):
 *
 *  - pa_reshape_and_cache writes the new tokens' K and V into fixed-size
 *    physical blocks of 16 tokens through a per-token slot_mapping
 *    (vLLM architecture summary, "第一部分：LLM 引擎核心": the forward pass
 *    builds slot_mapping while preparing inputs; "大模型推理优化学习笔记",
 *    "KV Cache": K/V are written at prefill and appended at every decode step).
 *  - pa_decode computes, for one query token per sequence, softmax attention
 *    over that sequence's cached keys, reading K/V back through a per-sequence
 *    block table ("从静态批处理到状态化推理集群", "PagedAttention：把逻辑连续与物理
 *    连续分开": (sequence, logical block) -> physical block; the kernel reads
 *    K/V by block table). Long contexts are split into key ranges whose
 *    partial softmax summaries are merged exactly ("宣稱省下 106 倍成本…",
 *    the online-softmax Q&A of "中：Kimi K3 的 DCP 選擇與 DEP 轉折").
 *  - pa_decode_shared_prefix is pa_decode for batches whose sequences share
 *    prefix blocks, reading each shared block once per group of sequences.
 *  - pa_prefill_chunk does the same for a flattened variable-length batch of
 *    causal query chunks (cu_seqlens), e.g. decode tokens and one chunk of a
 *    long prompt scheduled together under a token budget
 *    ("大模型推理优化学习笔记", "Chunked Prefill"; "从静态批处理到状态化推理集群",
 *    "Chunked prefill：在共置引擎里治理阶段干扰").
 *
 * Semantics fixed by this library where the pages are silent:
 *  - the new tokens' K/V are written first and every query attends to itself:
 *    query row r of a sequence with q_len rows and context_len cached tokens
 *    (this call's tokens included) sits at position p = context_len - q_len + r
 *    and sees keys j <= p; with sliding_window W > 0 only j >= p - W + 1;
 *  - query head h reads KV head h / (num_heads / num_kv_heads);
 *  - softmax scale is the caller's `scale` (1/sqrt(head_size) in practice).
 *
 * Layouts (all tensors dense, row-major, device memory unless noted):
 *    k_cache  [num_blocks][num_kv_heads][block_size][head_size]
 *    v_cache  [num_blocks][num_kv_heads][head_size][block_size]   (V is stored
 *             transposed inside each block so that one block of one head is a
 *             contiguous tile whose rows run along keys)
 *    query/out [num_q_tokens][num_heads][head_size]
 *    key/value (new tokens) [num_tokens][num_kv_heads][head_size]
 *    block_table [num_seqs][block_table_stride] int32, physical block ids
 *    k_scale/v_scale [num_blocks] fp32, fp8 caches only (stored value =
 *             e4m3fn(byte) * scale[block]); NULL otherwise.
 *
 * Ownership and ordering: the caller allocates and frees every buffer,
 * including the workspace sized by the *_workspace_bytes queries. The library
 * never allocates, frees, synchronises or copies device-to-host; each call
 * only enqueues kernels on `stream` and returns.
 *
 * Errors: arguments checked on the host (sizes, dtypes, null pointers,
 * workspace size) return a non-PA_OK status, enqueue nothing and set a
 * thread-local message readable by pa_last_error(). A failed launch returns
 * PA_ERR_HIP. No C++ exception crosses this ABI.
 *
 * Device-side preconditions (the caller's; not checked on the device):
 *  1 <= context_lens[s] <= max_context_len; ceil(context_lens[s]/16) <=
 *  block_table_stride; every block id the sequence uses is in [0, num_blocks);
 *  1 <= q_len(s) <= context_lens[s] and cu_seqlens non-decreasing with
 *  cu_seqlens[0] = 0, cu_seqlens[num_seqs] = num_q_tokens, q_len(s) <= max_q_len;
 *  slots of one write call are unique and name blocks the writer owns
 *  exclusively (a shared non-full block is copied before it is written).
 *  pa_check_batch checks all of these on host copies of the metadata.
 *
 * Determinism: identical inputs and sizes give bitwise identical outputs.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t; NULL means the default stream. */
typedef struct ihipStream_t* pa_stream_t;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1,   /* bad size, null pointer, inconsistent sizes */
  PA_ERR_UNSUPPORTED = 2,        /* valid request this build has no kernel for */
  PA_ERR_WORKSPACE_TOO_SMALL = 3,
  PA_ERR_HIP = 4,                /* a HIP runtime call or launch failed */
  PA_ERR_OUT_OF_BLOCKS = 5       /* block manager: too few free blocks (pa_blocks.h) */
} pa_status;

enum {
  PA_F32 = 0,
  PA_BF16 = 1,
  PA_FP8_E4M3 = 2                /* OCP e4m3fn, KV cache only */
};
/* A dtype argument: one of the PA_F32 / PA_BF16 / PA_FP8_E4M3 codes. It is
   a plain int32_t, so that any other value reaches the library as it is and
   is rejected there (PA_ERR_INVALID_ARGUMENT) rather than being an
   out-of-range enum value. */
typedef int32_t pa_dtype;

#define PA_ABI_VERSION 1
#define PA_BLOCK_SIZE 16

/*
 * Write new K/V rows into the paged cache (one row per token and KV head).
 * key, value: [num_tokens][num_kv_heads][head_size] of in_dtype.
 * slot_mapping: int64 [num_tokens]; slot = physical_block * 16 + offset;
 *   a negative slot skips the token (padding).
 * cache_dtype == in_dtype: a bit-exact copy.
 * cache_dtype == PA_FP8_E4M3 with in_dtype F32 or BF16: quantising write,
 *   byte = e4m3fn(x / scale[block]) rounded to nearest even and saturated to
 *   +-448, the fp32 quotient correctly rounded; k_scale/v_scale are read,
 *   never written (the caller chose them).
 * num_tokens == 0 enqueues nothing and returns PA_OK.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                               const float* k_scale, const float* v_scale,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                               int32_t head_size, pa_dtype in_dtype, pa_dtype cache_dtype,
                               pa_stream_t stream);

/*
 * Decode attention: one query token per sequence.
 * out, query: [num_seqs][num_heads][head_size] of q_dtype (out has the query's
 *   type; results are rounded to nearest even from fp32).
 * context_lens: int32 [num_seqs]; max_context_len is a HOST scalar >= every
 *   context length (it sizes the grid without a device-to-host copy).
 * sliding_window: 0 = full attention, W > 0 = the last W positions.
 * workspace: device scratch of at least pa_decode_workspace_bytes(...) bytes,
 *   contents on entry irrelevant.
 * Supported: block_size 16; head_size 64 or 128; num_heads / num_kv_heads in
 *   {1, 2, 4, 8, 16}; (q, cache) dtypes (F32, F32), (BF16, BF16),
 *   (BF16, FP8_E4M3).
 * Batches of more than 16000 sequences over bf16/fp8 caches run as
 *   consecutive launches over groups of 16000 (the matrix-core kernel keeps
 *   per-sequence prefix sums in LDS), reusing one workspace; the workspace
 *   size is that of one group.
 */
pa_status pa_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
                    const float* k_scale, const float* v_scale, const int32_t* block_table,
                    int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                    int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_size, int32_t block_size, int32_t num_blocks, pa_dtype q_dtype,
                    pa_dtype cache_dtype, float scale, int32_t sliding_window, void* workspace,
                    size_t workspace_bytes, pa_stream_t stream);

/*
 * pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. The
 * arguments are pa_decode's without the workspace; the split-K summaries go
 * to a scratch array inside the library instead: PA_NOALLOC_SCRATCH_BYTES
 * (32 MiB) per GPU, part of the code object, held by each GPU the library
 * runs on until the process ends. The call allocates and frees nothing.
 * A request whose pa_decode_workspace_bytes(...) exceeds the array returns
 * PA_ERR_WORKSPACE_TOO_SMALL and enqueues nothing (about 14,000 (sequence,
 * KV head) streams at 4 query heads per KV head, head size 128). Every call
 * on one GPU shares that GPU's array and leaves its last contents there
 * (nothing in it needs clearing between calls): calls that can overlap on
 * one GPU (unordered streams) race, and must be ordered by the caller.
 * Results equal pa_decode's bit for bit.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pa_status pa_decode_noalloc(void* out, const void* query, const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale, const int32_t* block_table,
                            int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                            int32_t block_size, int32_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype,
                            float scale, int32_t sliding_window, pa_stream_t stream);

/*
 * pa_decode on the vector-ALU kernel, whatever the cache type: scores as
 * packed-bf16 dot products reduced across the wave with DPP row shuffles,
 * the online-softmax max and sum by the same shuffles, weights passed to the
 * value lanes through LDS, split-K partitions merged by log-sum-exp. This is
 * the design the grouped-query decode was first planned on; pa_decode serves
 * bf16 and fp8 caches on matrix cores instead (a grouped-query step is a
 * (group x head_size)(head_size x keys) product, so the dot products cost
 * no vector-ALU time there). Kept as an entry point of its own so that the
 * two can be measured side by side on the same batch; it computes the same
 * attention ("大模型推理优化学习笔记", "Decode": decode is memory-bound, each
 * step reading the whole KV cache). Arguments, layouts, support and errors
 * are pa_decode's; the workspace must hold
 * pa_decode_valu_workspace_bytes(...) bytes.
 */
pa_status pa_decode_valu(void* out, const void* query, const void* k_cache, const void* v_cache,
                         const float* k_scale, const float* v_scale, const int32_t* block_table,
                         int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                         int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                         int32_t block_size, int32_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype,
                         float scale, int32_t sliding_window, void* workspace, size_t workspace_bytes,
                         pa_stream_t stream);

/*
 * Decode attention where runs of consecutive sequences share the physical
 * blocks of a common prefix: a prefix cache points the block tables of
 * sequences with identical leading content at the same refcounted blocks
 * ("宣稱省下 106 倍成本…", "vLLM 的解法：統一分頁 + 共用池"), and agentic
 * subagents fork from their parent's context, so most of a decode batch's
 * keys can be shared ("Agentic Workload 為什麼難伺服：四個特徵與三個挑戰":
 * prefix reuse above 96%). The result is exactly pa_decode's (the same
 * attention, up to fp32 rounding order); what changes is that a group's
 * shared blocks are read once per 16 query heads of its members instead of
 * once per member, each member's own keys separately, and the partial softmax
 * summaries merged exactly (the online-softmax Q&A of "中：Kimi K3 的 DCP
 * 選擇與 DEP 轉折").
 * num_groups: host scalar in [0, num_seqs].
 * cu_groups: int32 [num_groups + 1], device: group k is the sequences
 *   cu_groups[k] .. cu_groups[k+1]-1 (disjoint runs, non-decreasing,
 *   cu_groups[num_groups] <= num_seqs); sequences outside every run, and
 *   runs whose usable prefix (below) is shorter than one block, share
 *   nothing. If the runs break these rules no group is used (checked on the
 *   device; the result is pa_decode's either way).
 * group_prefix_len: int32 [num_groups], device: tokens of group k's shared
 *   prefix; every member's block table holds the same physical blocks for
 *   logical blocks 0 .. group_prefix_len[k]/16 - 1 (the first member's table
 *   is the one read). The kernel uses the length rounded down to whole blocks
 *   and to at most every member's context length minus one (a member's own
 *   newest token is never shared), so any value is memory-safe; values that
 *   break the sharing precondition give wrong results, not faults.
 * Other arguments, layouts and the workspace rules are pa_decode's; the
 *   workspace must hold pa_decode_shared_prefix_workspace_bytes(...) bytes.
 * The shared-block reading applies to (BF16, BF16) and (BF16, FP8_E4M3) with
 *   sliding_window 0 and at most 3000 sequences; other requests (or
 *   num_groups == 0) are served as pa_decode would serve them.
 */
pa_status pa_decode_shared_prefix(void* out, const void* query, const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale, const int32_t* block_table,
                                  int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                                  int32_t max_context_len, const int32_t* cu_groups,
                                  const int32_t* group_prefix_len, int32_t num_groups, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                                  int32_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype, float scale,
                                  int32_t sliding_window, void* workspace, size_t workspace_bytes,
                                  pa_stream_t stream);

/*
 * Sparse decode: the newest token of each sequence attends only to the keys
 * of a chosen set of its logical blocks. Sparse attention looks at the top-k
 * history positions an indexer picks instead of all of them; the indexer
 * hands over one list per sequence for every head, and the work that remains
 * is fetching the chosen entries ("宣稱省下 106 倍成本…", "下：DeepSeek V4 的
 * 挑戰與 PCP/DEP 方案": "背景：什麼是稀疏注意力" and the three reasons that
 * follow), so the bytes read stop growing with the context (DeepSeek-V4.1
 * write-up, "三、第二招：把能合的内核全合成一个", sparse MQA logits). Candidates
 * here are whole 16-token blocks.
 * selected_blocks: int32 [num_seqs][selected_stride], device: logical block
 *   ids (position / 16) chosen for sequence s; its first num_selected[s]
 *   entries (clamped to [0, max_selected]) are read. Entries outside
 *   [0, newest block) are ignored, order and repeats do not matter, and the
 *   newest block (holding position context_lens[s] - 1) is always read, so
 *   the query always sees itself. Keys at positions >= context_lens[s] are
 *   never read.
 * num_selected: int32 [num_seqs], device. Both may be NULL when
 *   max_selected == 0 (every sequence reads its newest block only).
 * max_selected: host scalar in [0, 2^22]; selected_stride >= max_selected.
 * The result is pa_decode's over exactly those keys; choosing every block
 *   gives pa_decode's result. Other arguments and layouts are pa_decode's
 *   (no sliding window); max_context_len up to 8,257,536 (PA_ERR_UNSUPPORTED
 *   beyond: the block bitmap lives in 64 KiB of LDS). The workspace must
 *   hold pa_decode_sparse_workspace_bytes(...) bytes: it keeps the compacted
 *   block table ([num_seqs][max_selected + 1] int32) the decode then reads.
 * Launches: with bf16/fp8 caches, max_selected < 1024 and at least two
 *   (sequence, KV head) pairs per compute unit, one kernel selects, decodes
 *   and merges (a workgroup per pair; the workspace is then left untouched);
 *   otherwise a selection kernel writes the compacted tables and pa_decode's
 *   kernels follow. Either way the result is the one defined above (the
 *   rounding order of the merge differs between the two).
 */
pa_status pa_decode_sparse(void* out, const void* query, const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale, const int32_t* block_table,
                           int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                           int32_t max_context_len, const int32_t* selected_blocks, int32_t selected_stride,
                           const int32_t* num_selected, int32_t max_selected, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_size, int32_t block_size, int32_t num_blocks,
                           pa_dtype q_dtype, pa_dtype cache_dtype, float scale, void* workspace,
                           size_t workspace_bytes, pa_stream_t stream);

/*
 * One rank's share of decode context parallelism: the KV cache of every
 * sequence is split by position into contiguous ranges, one per GPU, each
 * GPU attends over its own range only, and the ranges' results are combined
 * with the online-softmax correction ("宣稱省下 106 倍成本…", "DCP 的切法：
 * 照「序列位置」切，不照「頭」切" and the online-softmax Q&A of "中：Kimi K3
 * 的 DCP 選擇與 DEP 轉折"). This call is pa_decode over the local range
 * (context_lens[s] = the tokens of sequence s this rank holds, which may be
 * 0; every one is visible to the query) that also writes
 *   lse: fp32 [num_seqs][num_heads], device: ln of the softmax denominator,
 *        ln sum_j exp(scale <q_h, K_j>) over the local keys (-inf, with a
 *        zero output row, when the range is empty).
 * The output is normalised over the local keys, in the query's type. No
 * sliding window. Needs the matrix-core decode (BF16 queries, BF16 or
 * FP8_E4M3 cache): PA_ERR_UNSUPPORTED otherwise. Workspace as pa_decode
 * (pa_decode_workspace_bytes with sliding_window 0).
 */
pa_status pa_decode_partial(void* out, float* lse, const void* query, const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale, const int32_t* block_table,
                            int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                            int32_t block_size, int32_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype,
                            float scale, void* workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * Combines num_parts results over disjoint key ranges of the same queries
 * (after the ranks' results are gathered onto one GPU):
 *   out[i] = sum_r e^(lse_r[i] - M) parts[r][i] / sum_r e^(lse_r[i] - M),
 *   M = max_r lse_r[i]; lse_out[i] = M + ln sum_r e^(lse_r[i] - M)
 * (same source as pa_decode_partial; the weighted-average example there).
 * parts: [num_parts][num_rows][head_size] in dtype (F32 or BF16), device;
 * parts_lse: fp32 [num_parts][num_rows], device; out: [num_rows][head_size]
 * in dtype; lse_out: fp32 [num_rows] or NULL. A row is one (token, head);
 * head_size 64, 128 or 512. Ranges with lse = -inf weigh nothing; a row with
 * every lse = -inf gets zeros and -inf.
 */
pa_status pa_merge_partials(void* out, float* lse_out, const void* parts, const float* parts_lse, int32_t num_parts,
                            int32_t num_rows, int32_t head_size, pa_dtype dtype, pa_stream_t stream);

/*
 * Decode over a paged latent (multi-head latent attention, MLA) cache: one
 * cached row per token shared by every head instead of a K and a V per head.
 * The heads' up-projections are folded into their queries (matrix
 * absorption), so head h scores its absorbed query directly against the rows
 * and takes the attention-weighted sum of the rows' first 512 elements (its
 * value up-projection is applied to that sum afterwards, outside this call)
 * ("宣稱省下 106 倍成本…", "MLA(Multi-head Latent Attention)是什麼、為什麼讓 TP
 * 沒效率" and its two Q&As):
 *   out[s][h][:] = sum_j softmax_j(scale <query[s][h], c_j>) c_j[0:512]
 * over the context_lens[s] rows c_j of sequence s (the newest included).
 * latent_cache: bf16 [num_blocks][16][head_dim_k]; row j of sequence s is
 *   latent_cache[block_table[s][j / 16]][j % 16]. head_dim_k is 512 (the
 *   latent alone, K = V = c) or 576 (512 latent elements and 64 more that
 *   take part in the scores only, such as a positional part).
 * query: bf16 [num_seqs][num_heads][head_dim_k]; out: bf16
 *   [num_seqs][num_heads][512]; head_dim_v must be 512.
 * num_heads: 16, 32, 64 or 128; context_lens[s] >= 1. Batches of more than
 *   2048 sequences run as consecutive launches over groups of 2048 (the
 *   kernels keep per-sequence prefix sums in LDS), reusing one workspace.
 * workspace: pa_mla_decode_workspace_bytes(num_seqs, num_heads) bytes (the
 *   size for min(num_seqs, 2048) sequences).
 * Numerics: scores on bf16 matrix cores with fp32 accumulation. With 16
 *   heads the weighted sum multiplies the bf16 rows by the weights split
 *   into bf16 hi + lo (16 significant bits). With more heads the rows'
 *   value part is converted to fp16 and the weights scaled by 2^7 into fp16
 *   (11 significant bits): exact for |c| in [2^-14, 65504]; a row whose
 *   values overflow fp16 comes out non-finite there and is then computed
 *   again in fp32 by the merge step. Any finite cached value gives a finite
 *   result as long as the fp32 sums stay in range.
 */
pa_status pa_mla_decode(void* out, const void* query, const void* latent_cache, const int32_t* block_table,
                        int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                        int32_t max_context_len, int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
                        int32_t block_size, int32_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype, float scale,
                        void* workspace, size_t workspace_bytes, pa_stream_t stream);

/* Workspace bytes pa_mla_decode needs (0 if arguments are out of range). */
size_t pa_mla_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads);

/*
 * Causal attention for a flattened variable-length batch.
 * Sequence s owns query rows cu_seqlens[s] .. cu_seqlens[s+1]-1 (int32
 * [num_seqs+1]); context_lens[s] counts its cached tokens including this
 * chunk, whose K/V must already be in the cache. Rows of sequences with one
 * query token take the decode kernel; longer chunks take the matrix-core
 * (MFMA) kernel. num_q_tokens, max_q_len and max_context_len are HOST
 * scalars bounding the device arrays.
 * Supported as pa_decode, except that chunks longer than one token need
 *   q_dtype BF16 (cache BF16 or FP8_E4M3).
 * Numerics of the chunks: scores on bf16 matrix cores (fp8 keys widened to
 *   bf16 exactly, the block scale applied to the fp32 score), fp32
 *   accumulation. The weighted sum of values runs on fp16 matrix cores: the
 *   values (bf16, or e4m3 times the block scale) rounded to fp16, the
 *   weights scaled by 2^7 into fp16 (11 significant bits). A tile of query
 *   rows whose values reach beyond fp16's range (|v| > 65504) is computed
 *   again with the values in bf16 (exact) against the weights split into
 *   bf16 hi + lo, so every finite cached value is in the domain; the fp32
 *   accumulator needs 2^15 * sum_j |v_j| below 3.4e38.
 * Streams: a batch holding both one-token rows and longer chunks, with bf16
 *   queries, a bf16 or fp8 e4m3 cache, head_size 128 and 1, 2, 4 or 8
 *   query heads per KV head (and a context long enough that the decode plan
 *   splits streams over waves),
 *   has its one-token rows decoded on a second stream that the library owns
 *   (one per device, default priority), next to the chunks' prefill kernel
 *   on `stream` ("从静态批处理到状态化推理集群", "Chunked prefill：在共置引擎
 *   里治理阶段干扰": decode rows and prefill chunks share a step). The second
 *   stream starts after the work already on `stream` and `stream` waits for
 *   it (events), so the call is ordered exactly like one on `stream` alone,
 *   also under HIP graph capture of `stream`. Calls that overlap in time
 *   from several host threads serialise their enqueueing on a lock.
 */
pa_status pa_prefill_chunk(void* out, const void* query, const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale, const int32_t* block_table,
                           int32_t block_table_stride, const int32_t* cu_seqlens,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_tokens,
                           int32_t max_q_len, int32_t max_context_len, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                           int32_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype, float scale,
                           int32_t sliding_window, void* workspace, size_t workspace_bytes,
                           pa_stream_t stream);

/* Workspace bytes pa_decode needs for these sizes and cache type: the
 * split-K summaries (per partition and query head, head_size + 2 floats) and
 * per-sequence block counts. 0 when no summaries are needed: one partition
 * (fp32 caches with short contexts), or bf16/fp8 caches whose (sequence, KV
 * head) streams are at most 16 blocks (max_context_len <= 256, or
 * sliding_window <= 240), which one wave each finishes in place. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_size, pa_dtype cache_dtype,
                                 int32_t sliding_window);

/* Workspace bytes pa_decode_valu needs for these sizes (0 if none). */
size_t pa_decode_valu_workspace_bytes(int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_size, pa_dtype cache_dtype,
                                      int32_t sliding_window);

/* Workspace bytes pa_decode_shared_prefix needs for these sizes (0 if none). */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_groups, int32_t max_context_len,
                                               int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                               pa_dtype cache_dtype, int32_t sliding_window);

/* Workspace bytes pa_decode_sparse needs for these sizes (0 if arguments are
 * out of range). */
size_t pa_decode_sparse_workspace_bytes(int32_t num_seqs, int32_t max_selected, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_size, pa_dtype cache_dtype);

/* Workspace bytes pa_prefill_chunk needs for these sizes (0 if none; the
 * one-token rows of a mixed batch use the decode plan). */
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_q_tokens, int32_t max_q_len,
                                  int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_size, pa_dtype cache_dtype, int32_t sliding_window);

/*
 * Checks a batch's metadata, on HOST copies, against the device-side
 * preconditions listed at the top of this header (which the kernels never
 * check): for each sequence 1 <= context_lens[s] <= max_context_len and
 * ceil(context_lens[s]/16) <= block_table_stride; every block id the
 * attention reads (from the first query's window start to the newest block)
 * in [0, num_blocks); with cu_seqlens (else a decode batch, num_q_tokens ==
 * num_seqs): cu_seqlens[0] = 0, cu_seqlens[num_seqs] = num_q_tokens and
 * 1 <= q_len(s) <= min(context_lens[s], max_q_len). With slot_mapping
 * ([num_q_tokens] int64; NULL skips the write checks): every non-negative
 * slot is its token's position in its own sequence's table (query row r
 * of sequence s at position context_lens[s] - q_len(s) + r), no slot twice,
 * and no written block mapped by any other (sequence, logical block) entry
 * of the batch: a block shared through a prefix is copied before it is
 * written ("从静态批处理到状态化推理集群", "Prefix reuse：分页让细粒度共享更便宜").
 * Returns PA_OK, or PA_ERR_INVALID_ARGUMENT with the first violation in
 * pa_last_error(). Touches no device memory; cost O(num_blocks + read
 * blocks + num_q_tokens).
 */
pa_status pa_check_batch(const int32_t* block_table, int32_t block_table_stride, const int32_t* context_lens,
                         const int32_t* cu_seqlens, int32_t num_seqs, int32_t num_q_tokens, int32_t max_q_len,
                         int32_t max_context_len, int32_t num_blocks, int32_t sliding_window,
                         const int64_t* slot_mapping);

/* Static name of a status code: any int (a pa_status value, or "PA_ERR_UNKNOWN"
   for one that is not; an int so that an unknown code is not an out-of-range
   enum value). */
const char* pa_status_string(int32_t status);

/* Detail of the calling thread's last non-OK status ("" if none). */
const char* pa_last_error(void);

/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
