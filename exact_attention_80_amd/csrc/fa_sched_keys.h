// fa_sched_keys.h -- the pure functions behind the packed-batch work order:
// item counts, tile costs and the 64-bit sort keys of the scheduler kernel
// (fa_sched.hip).  Host-callable, so the ordering rules can be checked on the
// host against their definition.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_common.h"

namespace fa {
namespace sched {

__host__ __device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// chunks of sequence s's last query tile in the forward (0: not split)
__host__ __device__ __forceinline__ int fwd_split_chunks(bool causal, int lq, int lk, int tile, int fkv) {
  if (lq <= 0) return 0;
  const int last = (lq - 1) / tile;
  if (lq - last * tile > 32) return 0;
  const int end = causal ? imax(0, imin(lk, (last + 1) * tile + lk - lq)) : lk;
  const int nt = cdiv(end, fkv);
  const int ct = fwd_split_chunk_tiles(nt);
  const int n = cdiv(nt, ct);
  return n >= 2 ? n : 0;
}

// cost of one tile in units of the inner loop's tiles
__host__ __device__ __forceinline__ int tile_cost(int mode, bool causal, int lq, int lk, int tile, int idx,
                                        int fkv, int bq) {
  const int off = lk - lq;
  if (mode == 0) {
    const int end = causal ? imax(0, imin(lk, (idx + 1) * tile + off)) : lk;
    return cdiv(end, fkv);
  }
  const int nq = cdiv(lq, bq);
  return causal ? imax(0, nq - imax(0, idx * tile - off) / bq) : nq;
}

// cost of an item (a split chunk: its own key tiles)
__host__ __device__ __forceinline__ int item_cost(int mode, bool causal, int lq, int lk, int tile, int idx,
                                         int fkv, int bq) {
  if (mode == 0 && (idx & kSplitItem)) {
    const int last = (lq - 1) / tile;
    const int end = causal ? imax(0, imin(lk, (last + 1) * tile + lk - lq)) : lk;
    const int nt = cdiv(end, fkv);
    const int ct = fwd_split_chunk_tiles(nt);
    const int c = idx & 0xFFFFF;
    return imin(ct, nt - c * ct);
  }
  return tile_cost(mode, causal, lq, lk, tile, idx, fkv, bq);
}

// work items of sequence s: its query tiles (forward; a split last tile
// counts once per chunk) or its key tiles (backward)
__host__ __device__ __forceinline__ int seq_items(int mode, bool causal, const int* cu_q, const int* cu_k,
                                         int s, int tile, int fkv) {
  if (mode != 0) return cdiv(cu_k[s + 1] - cu_k[s], tile);
  const int lq = cu_q[s + 1] - cu_q[s], lk = cu_k[s + 1] - cu_k[s];
  const int n = fwd_split_chunks(causal, lq, lk, tile, fkv);
  return cdiv(lq, tile) + (n > 0 ? n - 1 : 0);
}

// item k (0-based, in natural order) of sequence s: its tile index, or for a
// chunk of a split forward tile kSplitItem | chunk
__host__ __device__ __forceinline__ int seq_item_index(int mode, bool causal, int lq, int lk, int tile,
                                              int fkv, int k) {
  if (mode != 0) return k;
  const int n = fwd_split_chunks(causal, lq, lk, tile, fkv);
  const int nq = cdiv(lq, tile);
  if (n == 0 || k < nq - 1) return k;
  return kSplitItem | (k - (nq - 1));
}

// sort keys hold an item index in 20 bits: a split chunk is bit 19 | chunk
__host__ __device__ __forceinline__ int key_idx(int idx) {
  return (idx & kSplitItem) ? ((1 << 19) | (idx & 0x7FFFF)) : idx;
}
__host__ __device__ __forceinline__ int unkey_idx(int k) {
  return (k & (1 << 19)) ? (kSplitItem | (k & 0x7FFFF)) : k;
}

// ascending keys give: modes 0 and 2 (cost = the sequence's largest tile
// cost) the sequences in descending order of it, each sequence's items
// together, mode 0 from the last query tile (split chunks first), mode 2
// from the last key tile; mode 1 (cost = the tile's own) every key tile in
// descending order of its cost
__host__ __device__ __forceinline__ unsigned long long sort_key(int mode, int cost, int seq, int idx) {
  const unsigned long long c = (unsigned long long)(unsigned)imin(cost, 0xFFFFFF);
  const unsigned long long s = (unsigned long long)(unsigned)seq & 0xFFFFFull;
  const unsigned long long t = (unsigned long long)(unsigned)key_idx(idx) & 0xFFFFFull;
  if (mode == 1) return ((0xFFFFFFull - c) << 40) | (s << 20) | t;
  return ((0xFFFFFFull - c) << 40) | (s << 20) | (0xFFFFFull - t);
}

__host__ __device__ __forceinline__ void decode_key(int mode, unsigned long long k, int& seq, int& idx) {
  seq = (int)((k >> 20) & 0xFFFFFull);
  if (mode == 1) idx = (int)(k & 0xFFFFFull);
  else idx = unkey_idx((int)(0xFFFFFull - (k & 0xFFFFFull)));
}

}  // namespace sched
}  // namespace fa
