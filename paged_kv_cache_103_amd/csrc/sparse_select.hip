// Sparse decode's selection kernel (pa_decode_sparse, include/pa.h), the
// first of three launches when the one-launch kernel does not serve the call:
// turns each sequence's list of chosen logical blocks into a compact block
// table of the physical blocks it will read, in ascending logical order with
// the newest block last, and the number of keys that leaves. The decode
// kernels then run on that table unchanged: positions are already encoded in
// Q and K, so only which keys are read matters, and every chosen key precedes
// the query. The bytes read stop growing with the context (DeepSeek-V4.1
// write-up, "三、第二招：把能合的内核全合成一个", sparse MQA logits).
//
// One workgroup per sequence; the marking and the ranking of short lists
// are sparse_pick.h's. Longer lists (kSparseRankMax entries or more) are
// compacted from the bitmap in ascending order by a workgroup scan of
// per-word popcounts.
#include <hip/hip_runtime.h>

#include "pa_internal.h"
#include "sparse_pick.h"

namespace pa {

__global__ __launch_bounds__(256) void sparse_select_kernel(SparseSelectArgs a) {
  extern __shared__ unsigned int lds_bits[];
  int* scan = reinterpret_cast<int*>(lds_bits + a.words_max);
  int* listed = scan + 256;  // short lists: the distinct chosen blocks, unordered
  __shared__ int nlisted;
  const int s = blockIdx.x, tid = threadIdx.x;
  const int ctx = a.context_lens[s];
  const int nbk = min(ctx > 0 ? (ctx + 15) >> 4 : 0, a.blocks_max);
  const int W = (nbk + 31) >> 5;
  const bool short_list = a.rank_list != 0;
  const int m = sparse_mark(a, s, nbk, lds_bits, short_list ? listed : nullptr, &nlisted);
  if (nbk == 0) {  // uniform over the workgroup
    if (tid == 0) a.eff_ctx[s] = 0;
    return;
  }
  const int* bt = a.block_table + (size_t)s * a.bt_stride;
  int* out = a.cbt + (size_t)s * a.cbt_stride;
  if (short_list) {
    sparse_rank(listed, m, bt, out);
    if (tid == 0) a.eff_ctx[s] = sparse_keys(m, ctx, nbk);
    return;
  }
  int base = 0;
  for (int w0 = 0; w0 < W; w0 += 256) {
    const int w = w0 + tid;
    const unsigned int v = w < W ? lds_bits[w] : 0u;
    const int c = __popc(v);
    scan[tid] = c;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int t = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += t;
      __syncthreads();
    }
    int pos = base + scan[tid] - c;
    for (unsigned int left = v; left != 0u; left &= left - 1u) out[pos++] = bt[w * 32 + __builtin_ctz(left)];
    base += scan[255];
    __syncthreads();
  }
  if (tid == 0) a.eff_ctx[s] = sparse_keys(base, ctx, nbk);
}

size_t sparse_select_lds_bytes(int max_context_len, int max_selected) {
  const int blocks = (max_context_len + 15) / 16;
  const size_t base = ((size_t)(blocks + 31) / 32 + 256) * sizeof(int);
  const size_t list = (size_t)(max_selected + 1) * sizeof(int);
  return max_selected < kSparseRankMax && base + list <= kSparseMaxLds ? base + list : base;
}

hipError_t launch_sparse_select(const SparseSelectArgs& a, int num_seqs, hipStream_t stream) {
  if (num_seqs == 0) return hipSuccess;
  const size_t lds = (size_t)(a.words_max + 256 + (a.rank_list ? a.max_selected + 1 : 0)) * sizeof(int);
  hipLaunchKernelGGL(sparse_select_kernel, dim3((unsigned)num_seqs), dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace pa
