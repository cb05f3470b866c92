// Sparse decode: the chosen blocks of one sequence, as one workgroup of 256
// threads computes them (the selection kernel and the one-launch decode).
// Sparse attention reads only the blocks an indexer ranks highest
// ("宣稱省下 106 倍成本…", "背景：什麼是稀疏注意力"): here the caller's list of
// logical block ids, in which order and repeats do not matter and ids
// outside [0, newest block) are dropped; the newest block is always read.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {

// Blocks of sequence s (at most blocks_max) and the keys its chosen blocks
// hold: 16 per block, the newest holding ctx - 16 * (blocks - 1).
__device__ __forceinline__ int sparse_keys(int chosen, int ctx, int nbk) {
  return chosen > 0 ? 16 * (chosen - 1) + min(16, ctx - 16 * (nbk - 1)) : 0;
}

// Sets, in the LDS bitmap `bits` (cleared here), one bit per distinct chosen
// block of sequence s, and with `list` (non-null: short lists) appends each
// block to it the first time its bit is set. Returns the number of listed
// blocks (the newest included; 0 for an empty context) when `list` is set,
// else 0. Ends with a barrier; all 256 threads must call it.
__device__ __forceinline__ int sparse_mark(const SparseSelectArgs& a, int s, int nbk, unsigned int* bits, int* list,
                                           int* nlisted) {
  const int tid = threadIdx.x;
  for (int w = tid; w < ((nbk + 31) >> 5); w += 256) bits[w] = 0u;
  if (tid == 0) *nlisted = 0;
  __syncthreads();
  // entry n stands for the newest block; an empty context marks nothing
  const int n = nbk > 0 ? min(max(a.num_selected != nullptr ? a.num_selected[s] : 0, 0), a.max_selected) : -1;
  const int* sel = a.selected + (size_t)s * a.sel_stride;
  for (int i = tid; i <= n; i += 256) {
    const int e = i < n ? sel[i] : nbk - 1;
    if (e >= 0 && (e < nbk - 1 || i == n)) {
      const unsigned int bit = 1u << (e & 31);
      const unsigned int old = atomicOr(&bits[e >> 5], bit);
      if (list != nullptr && !(old & bit)) list[atomicAdd(nlisted, 1)] = e;
    }
  }
  __syncthreads();
  return list != nullptr ? *nlisted : 0;
}

// Short lists: writes out[rank] = the physical id of each of the m listed
// blocks, rank = its place in ascending logical order (the newest last).
__device__ __forceinline__ void sparse_rank(const int* list, int m, const int* bt, int* out) {
  for (int j = threadIdx.x; j < m; j += 256) {
    const int v = list[j];
    int rank = 0;
    for (int k = 0; k < m; ++k) rank += list[k] < v;
    out[rank] = bt[v];
  }
}

}  // namespace pa
