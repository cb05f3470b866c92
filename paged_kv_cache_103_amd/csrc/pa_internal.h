// Internal interface between the C ABI layer (pa_api.cpp) and the kernel
// launchers. Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Sets (or, for PA_OK, clears) the thread's pa_last_error() text; returns st.
pa_status set_error(pa_status st, const char* msg);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale, const int32_t* pairs,
                              int num_pairs, size_t tile_bytes, int num_kv_heads, int num_blocks,
                              hipStream_t stream);

// e4m3fn saturation before the hardware conversion: finite values are clamped
// to +-448, NaN stays NaN.
__device__ __forceinline__ float sat_e4m3(float x) {
  return (x != x) ? x : fminf(fmaxf(x, -448.0f), 448.0f);
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int head_size, int in_kind, int cache_kind, hipStream_t stream);

// Split-K plan of the decode kernel: every sequence's key blocks are cut into
// partitions of `pb` blocks; `max_parts` bounds the partitions of any
// sequence. One partition means no partial results and no merge.
//
// The matrix-core kernel instead splits the concatenated (sequence, KV head)
// block streams evenly over a fixed number of waves (`split_waves` > 0); each
// wave writes one summary per stream segment it covers, in slot
// wave + stream (unique, since consecutive segments advance exactly one of
// the two).
// Longest (sequence, KV head) stream, in blocks, that the matrix-core decode
// serves with one wave per stream.
constexpr int kOnePerStreamMaxBlocks = 16;
struct DecodePlan {
  int pb;
  int max_parts;
  int split_waves;  // > 0: even split over this many waves (matrix-core kernel)
  int one_per_stream;  // matrix-core kernel, every stream short: a wave per (sequence, KV head), no merge
};
// force_valu: the VALU kernel whatever the cache type (pa_decode_valu).
DecodePlan plan_decode(int num_seqs, int max_context_len, int num_heads, int num_kv_heads, int head_size,
                       int q_kind, int cache_kind, int sliding_window, bool force_valu = false);
size_t decode_workspace_bytes(const DecodePlan& plan, int num_seqs, int num_heads, int num_kv_heads,
                              int head_size);
// Decode with groups of sequences sharing prefix blocks (matrix-core kernel
// only): workspace, the largest batch it serves, and the launch.
size_t decode_shared_prefix_workspace_bytes(int num_seqs, int num_groups, int num_heads, int num_kv_heads,
                                            int head_size);
constexpr int kSharedPrefixMaxSeqs = 3000;
int shared_prefix_meta_ints(int num_seqs, int num_groups);
bool decode_uses_mfma(int q_kind, int cache_kind, int group);
// Sequences one matrix-core decode launch takes (its per-sequence prefix sums
// live in LDS); pa_decode runs larger batches as groups of this many.
constexpr int kMfmaMaxSeqs = 16000;
int device_cu_count();
// LDS bytes one CU offers (shared by its resident workgroups).
int device_lds_per_cu();

struct DecodeArgs {
  void* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int* block_table;
  const int* context_lens;
  const int* cu_seqlens;  // null: pure decode (query row s); else rows with q_len == 1 only
  float* part_o;          // pb plan: [num_seqs][num_heads][max_parts][head_size]
                          // split plan: [slots][group][head_size]
  float* part_ml;         // running max (log2 units) and sum per summary
  int* meta;              // split plan: [0] = blocks per wave, [1 + s] = block prefix sums
                          // (with shared prefixes: then group of each sequence and chunk bases)
  const int* cu_groups;   // shared prefixes: group k = sequences [cu_groups[k], cu_groups[k+1])
  const int* group_prefix_len;  // shared prefixes: tokens of group k's shared blocks (multiple of 16)
  int num_groups;         // 0: no shared prefixes
  int rec_cols;           // query columns per summary record (group size G, or 16 with shared prefixes)
  int bt_stride;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int window;
  int pb;
  int max_parts;
  int split_waves;
  int one_per_stream;  // see DecodePlan
  float scale_log2;  // softmax scale * log2(e)
  float* lse;        // optional [rows][num_heads]: ln of the softmax denominator (matrix-core kernel)
};

// pa_decode_noalloc's per-GPU scratch array (noalloc.hip): its size and this
// device's address of it (null, with *err set, if the runtime lookup fails).
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
void* noalloc_scratch(hipError_t* err);

// q_kind / cache_kind: 0 = f32, 1 = bf16, 2 = fp8 e4m3fn.
hipError_t launch_decode(const DecodeArgs& args, int q_kind, int cache_kind, int head_size,
                         hipStream_t stream);
bool decode_supported(int q_kind, int cache_kind, int head_size, int group);

// Sparse decode: compaction of each sequence's chosen blocks into a block
// table of its own (cbt [num_seqs][cbt_stride]) and key counts (eff_ctx).
struct SparseSelectArgs {
  const int* block_table;
  int bt_stride;
  const int* context_lens;
  const int* selected;      // [num_seqs][sel_stride] logical block ids
  int sel_stride;
  const int* num_selected;  // [num_seqs]; null when max_selected == 0
  int max_selected;
  int blocks_max;           // ceil(max_context_len / 16)
  int words_max;            // ceil(blocks_max / 32): bitmap words in LDS
  int* cbt;
  int cbt_stride;           // max_selected + 1
  int* eff_ctx;
  int rank_list;            // compact by rank through an LDS list (short lists; see the kernel)
};
constexpr int kSparseMaxSelected = 1 << 22;
constexpr int kSparseRankMax = 1024;         // lists shorter than this are compacted by rank
constexpr size_t kSparseMaxLds = 64 * 1024;  // bitmap + scan (+ list): contexts up to ~8M tokens
// LDS of the selection kernel: the bitmap and scan, plus the rank list when
// max_selected < kSparseRankMax and it fits kSparseMaxLds (then it is used).
size_t sparse_select_lds_bytes(int max_context_len, int max_selected);
hipError_t launch_sparse_select(const SparseSelectArgs& a, int num_seqs, hipStream_t stream);
// Selection, decode and merge in one launch (matrix-core kernel, a workgroup
// per (sequence, KV head)): its LDS bytes, 0 when the shape is not served
// (lists of kSparseRankMax entries or more, more than 16 heads per KV head,
// or more than kSparseMaxLds).
size_t decode_sparse_fused_lds_bytes(int words_max, int max_selected, int group, int head_size);
// `a` carries the caller's block table and context lengths; no workspace.
hipError_t launch_decode_sparse_fused(const DecodeArgs& a, const SparseSelectArgs& sa, int cache_kind,
                                      int head_size, hipStream_t stream);

// Decode over a paged latent (MLA) cache: [num_blocks][16][head_dim_k] bf16
// rows shared by all heads; values are the rows' first 512 elements.
struct MlaArgs {
  void* out;            // bf16 [num_seqs][num_heads][512]
  const void* query;    // bf16 [num_seqs][num_heads][head_dim_k]
  const void* cache;
  const int* block_table;
  const int* context_lens;
  float* part_o;        // [grid + num_seqs][num_heads][512]
  float* part_ml;       // [grid + num_seqs][num_heads][2]
  int* meta;            // [0] = pairs per workgroup, [1 + s] = pair prefix sums
  int bt_stride;
  int num_seqs;
  int num_heads;
  float scale_log2;
};
size_t mla_workspace_bytes(int num_seqs, int num_heads, int grid);
void mla_bind_workspace(MlaArgs& a, void* workspace, int num_seqs, int num_heads, int grid);
int mla_max_seqs();
hipError_t launch_mla_decode(const MlaArgs& a, int head_dim_k, int grid, hipStream_t stream);

// Merge of per-range attention results (o_r, lse_r) into one.
hipError_t launch_merge_lse(void* out, float* lse_out, const void* parts, const float* parts_lse, int num_parts,
                            int num_rows, int head_size, int kind, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int* block_table;
  const int* cu_seqlens;
  const int* context_lens;
  int bt_stride;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int window;
  int num_tiles;  // grid bound on (sequence, query tile) pairs
  float scale_log2;
  int nontemporal_kv;  // K/V copies nontemporal (set when a decode kernel runs beside)
};
// The chunked-prefill kernel (prefill_bf16.hip: 32x32 MFMA, bf16 scores and
// fp16 values, direct global->LDS copies, 8 waves per workgroup) for bf16
// and fp8 caches: query tokens per workgroup tile, what it supports, launch.
int prefill_tokens_per_tile(int group);
bool prefill_supported(int q_kind, int cache_kind, int head_size, int group);
hipError_t launch_prefill(const PrefillArgs& args, int cache_kind, int head_size, hipStream_t stream);
// Static LDS bytes of one prefill workgroup (0 if unknown).
size_t prefill_lds_bytes(int cache_kind, int head_size, int group);

// Decode of a mixed batch's one-token rows beside the prefill kernel
// (decode_mfma.hip): one workgroup of four waves per CU, at most 64
// registers per wave, K/V streamed through LDS; bf16 or fp8 caches, head
// size 128, 1, 2, 4 or 8 query heads per KV head. Uses the split plan's
// workspace and merge; LDS bytes per workgroup for num_seqs sequences.
bool decode_side_supported(int q_kind, int cache_kind, int head_size, int group);
size_t decode_side_lds_bytes(int num_seqs, int group);
hipError_t launch_decode_side(const DecodeArgs& args, int cache_kind, hipStream_t stream);

}  // namespace pa
