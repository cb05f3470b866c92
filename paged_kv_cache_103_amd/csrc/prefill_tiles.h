// Work assignment shared by the chunked-prefill kernels: workgroup t (of a
// grid of num_tiles x num_kv_heads) owns one (sequence, query tile) pair of
// the flattened batch, found by a block-wide prefix scan over the sequences'
// tile counts. Only sequences with more than one query row have tiles; rows
// of one-token sequences go to the decode kernel.
#pragma once

#include <hip/hip_runtime.h>

namespace pa {

struct PrefillTile {
  int seq;   // -1: no tile for this workgroup
  int tile;  // query tile within the sequence, heaviest (last) first
};

// Requires blockDim.x == NT; sh_scan holds NT ints, sh_found 3.
template <int NT = 256>
__device__ inline PrefillTile find_prefill_tile(const int* cu_seqlens, int num_seqs, int tokens_per_tile, int t,
                                                int* sh_scan, int* sh_found) {
  const int tid = threadIdx.x;
  if (tid == 0) { sh_found[0] = -1; sh_found[1] = 0; sh_found[2] = 0; }
  __syncthreads();
  int running = 0;
  for (int base = 0; base < num_seqs; base += NT) {
    const int s = base + tid;
    int n = 0;
    if (s < num_seqs) {
      const int ql = cu_seqlens[s + 1] - cu_seqlens[s];
      n = ql > 1 ? (ql + tokens_per_tile - 1) / tokens_per_tile : 0;
    }
    sh_scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
      const int v = tid >= off ? sh_scan[tid - off] : 0;
      __syncthreads();
      sh_scan[tid] += v;
      __syncthreads();
    }
    const int incl = sh_scan[tid];
    if (n > 0 && t >= running + incl - n && t < running + incl) {
      sh_found[0] = s;
      sh_found[1] = t - (running + incl - n);
      sh_found[2] = n;
    }
    running += sh_scan[NT - 1];
    __syncthreads();
    if (sh_found[0] >= 0) break;
  }
  // the values are the same in every lane: make them scalar, so that what is
  // derived from them (block table, lengths) is read with scalar loads
  PrefillTile r;
  r.seq = __builtin_amdgcn_readfirstlane(sh_found[0]);
  r.tile = r.seq < 0 ? 0 : __builtin_amdgcn_readfirstlane(sh_found[2] - 1 - sh_found[1]);
  return r;
}

}  // namespace pa
