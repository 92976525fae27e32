// fa_sched.hip -- on-device work ordering for packed variable-length batches.
//
// One workgroup reads cu_seqlens (never copied to the host), checks it, and
// writes the list of (sequence, tile) work items that the attention kernels
// walk, so the host never synchronises ([FA4B] 3.3.2: a preprocessing kernel
// orders the batches by their per-tile cost and emits the virtual -> actual
// index map the attention kernel then follows).
//   mode 0  forward query tiles, longest (most key tiles) first;
//   mode 1  backward key tiles, longest (most query tiles) first;
//   mode 2  backward key tiles for the deterministic reduction: sequences in
//           descending order of their largest tile cost ([FA4B] 3.3.2 sorts
//           the batches by per-tile time), the key tiles of a sequence kept
//           together and last first ([FA4B] 3.3.1: the cheapest causal tiles
//           first), so a key tile is always issued after every key tile it
//           waits for.  (A global cheapest-first order ran the longest
//           sequences' heaviest tiles last: 7.9 against 7.1 ms for the
//           natural order on a 65536-token batch.)
// The ordering only changes which work runs when, never any result.  Lists
// longer than the in-LDS sort capacity, or all lists when sorting is switched
// off (the tile-order ablation), are written in natural order (still
// last-tile-first within a sequence for mode 2).  Query and key offsets are
// separate arrays (the same one when every sequence has Lq == Lk); forward
// tiles split a sequence's queries, backward tiles its keys, and the cost of
// a tile counts the inner tiles its causal walk visits with the diagonal
// aligned bottom-right (offset Lk - Lq).
// Forward only: when a sequence's last query tile holds at most 32 queries
// (a decode step, or the tail of a chunk) and its keys span more than
// kSplitTiles key tiles, that tile becomes several items, each over its own
// chunk of key tiles, so one long row is spread over many workgroups; the
// chunks' partial results are merged exactly by the forward combine kernel.
// split_base[s] is the first partial slot of sequence s (split_base[nseq] is
// the total).  Every split decision is a pure function of the lengths, so the
// forward kernel recomputes it (fwd_split_chunk_tiles).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 1024;
constexpr int kSortCap = 8192;  // 64 KiB of 64-bit keys

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// chunks of sequence s's last query tile in the forward (0: not split)
__device__ __forceinline__ int fwd_split_chunks(bool causal, int lq, int lk, int tile, int fkv) {
  if (lq <= 0) return 0;
  const int last = (lq - 1) / tile;
  if (lq - last * tile > 32) return 0;
  const int end = causal ? max(0, min(lk, (last + 1) * tile + lk - lq)) : lk;
  const int nt = cdiv(end, fkv);
  const int ct = fwd_split_chunk_tiles(nt);
  const int n = cdiv(nt, ct);
  return n >= 2 ? n : 0;
}

// cost of one tile in units of the inner loop's tiles
__device__ __forceinline__ int tile_cost(int mode, bool causal, int lq, int lk, int tile, int idx,
                                        int fkv, int bq) {
  const int off = lk - lq;
  if (mode == 0) {
    const int end = causal ? max(0, min(lk, (idx + 1) * tile + off)) : lk;
    return cdiv(end, fkv);
  }
  const int nq = cdiv(lq, bq);
  return causal ? max(0, nq - max(0, idx * tile - off) / bq) : nq;
}

// cost of an item (a split chunk: its own key tiles)
__device__ __forceinline__ int item_cost(int mode, bool causal, int lq, int lk, int tile, int idx,
                                         int fkv, int bq) {
  if (mode == 0 && (idx & kSplitItem)) {
    const int last = (lq - 1) / tile;
    const int end = causal ? max(0, min(lk, (last + 1) * tile + lk - lq)) : lk;
    const int nt = cdiv(end, fkv);
    const int ct = fwd_split_chunk_tiles(nt);
    const int c = idx & 0xFFFFF;
    return min(ct, nt - c * ct);
  }
  return tile_cost(mode, causal, lq, lk, tile, idx, fkv, bq);
}

// work items of sequence s: its query tiles (forward; a split last tile
// counts once per chunk) or its key tiles (backward)
__device__ __forceinline__ int seq_items(int mode, bool causal, const int* cu_q, const int* cu_k,
                                         int s, int tile, int fkv) {
  if (mode != 0) return cdiv(cu_k[s + 1] - cu_k[s], tile);
  const int lq = cu_q[s + 1] - cu_q[s], lk = cu_k[s + 1] - cu_k[s];
  const int n = fwd_split_chunks(causal, lq, lk, tile, fkv);
  return cdiv(lq, tile) + (n > 0 ? n - 1 : 0);
}

// item k (0-based, in natural order) of sequence s: its tile index, or for a
// chunk of a split forward tile kSplitItem | chunk
__device__ __forceinline__ int seq_item_index(int mode, bool causal, int lq, int lk, int tile,
                                              int fkv, int k) {
  if (mode != 0) return k;
  const int n = fwd_split_chunks(causal, lq, lk, tile, fkv);
  const int nq = cdiv(lq, tile);
  if (n == 0 || k < nq - 1) return k;
  return kSplitItem | (k - (nq - 1));
}

// sort keys hold an item index in 20 bits: a split chunk is bit 19 | chunk
__device__ __forceinline__ int key_idx(int idx) {
  return (idx & kSplitItem) ? ((1 << 19) | (idx & 0x7FFFF)) : idx;
}
__device__ __forceinline__ int unkey_idx(int k) {
  return (k & (1 << 19)) ? (kSplitItem | (k & 0x7FFFF)) : k;
}

// ascending keys give: modes 0, 1 the most expensive item first; mode 2
// (cost = the sequence's largest tile cost) the most expensive sequence
// first, its key tiles together, last tile first
__device__ __forceinline__ unsigned long long sort_key(int mode, int cost, int seq, int idx) {
  const unsigned long long c = (unsigned long long)(unsigned)min(cost, 0xFFFFFF);
  const unsigned long long s = (unsigned long long)(unsigned)seq & 0xFFFFFull;
  const unsigned long long t = (unsigned long long)(unsigned)key_idx(idx) & 0xFFFFFull;
  if (mode == 2) return ((0xFFFFFFull - c) << 40) | (s << 20) | (0xFFFFFull - t);
  return ((0xFFFFFFull - c) << 40) | (s << 20) | t;
}

__device__ __forceinline__ void decode_key(int mode, unsigned long long k, int& seq, int& idx) {
  seq = (int)((k >> 20) & 0xFFFFFull);
  if (mode == 2) idx = (int)(0xFFFFFull - (k & 0xFFFFFull));
  else idx = unkey_idx((int)(k & 0xFFFFFull));
}

__global__ __launch_bounds__(kThreads) void sched_kernel(const int* cu_q, const int* cu_k,
                                                         int nseq, int total_q, int total_k,
                                                         int tile, int mode, int causal, int fkv,
                                                         int bq, int* tiles, int max_tiles,
                                                         int* split_base, int max_split,
                                                         uint32_t* hdr, int sorted) {
  __shared__ unsigned long long keys[kSortCap];
  __shared__ int scan[kThreads];
  __shared__ int scan2[kThreads];
  __shared__ int bad;
  const int tid = threadIdx.x;
  if (tid == 0) {
    bad = 0;
    hdr[kHdrErr] = 0u;  // the workspace may hold a previous call's word
  }
  __syncthreads();

  // ---- validation of both offset arrays: cu[0] == 0, cu[nseq] == total,
  // non-decreasing
  for (int s = tid; s < nseq; s += kThreads) {
    const int a = cu_q[s], b = cu_q[s + 1];
    if (b < a || (s == 0 && a != 0) || (s == nseq - 1 && b != total_q)) atomicOr(&bad, 1);
    const int c = cu_k[s], e = cu_k[s + 1];
    if (e < c || (s == 0 && c != 0) || (s == nseq - 1 && e != total_k)) atomicOr(&bad, 1);
  }
  __syncthreads();
  if (bad) {
    if (tid == 0) {
      atomicOr(&hdr[kHdrErr], kErrBadCu);
      hdr[kHdrCount] = 0u;
    }
    return;
  }

  // ---- tiles per thread-owned range of sequences, then an exclusive scan
  const int per = cdiv(nseq, kThreads);
  const int s_lo = min(nseq, tid * per), s_hi = min(nseq, s_lo + per);
  int mine = 0, mine_split = 0;
  for (int s = s_lo; s < s_hi; ++s) {
    mine += seq_items(mode, causal != 0, cu_q, cu_k, s, tile, fkv);
    if (mode == 0)
      mine_split += fwd_split_chunks(causal != 0, cu_q[s + 1] - cu_q[s], cu_k[s + 1] - cu_k[s],
                                     tile, fkv);
  }
  scan[tid] = mine;
  scan2[tid] = mine_split;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    const int v2 = tid >= off ? scan2[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    scan2[tid] += v2;
    __syncthreads();
  }
  const int count = scan[kThreads - 1];
  int pos = scan[tid] - mine;
  if (mode == 0 && split_base) {
    // first partial slot of every sequence of this thread's range
    int b = scan2[tid] - mine_split;
    for (int s = s_lo; s < s_hi; ++s) {
      split_base[s] = b;
      b += fwd_split_chunks(causal != 0, cu_q[s + 1] - cu_q[s], cu_k[s + 1] - cu_k[s], tile,
                            fkv);
    }
    if (tid == kThreads - 1) split_base[nseq] = scan2[kThreads - 1];
  }
  if (count > max_tiles || (mode == 0 && scan2[kThreads - 1] > max_split)) {
    if (tid == 0) {
      atomicOr(&hdr[kHdrErr], kErrTileOverflow);
      hdr[kHdrCount] = 0u;
    }
    return;
  }

  if (sorted && count <= kSortCap) {
    int n = 1;
    while (n < count) n <<= 1;
    for (int s = s_lo; s < s_hi; ++s) {
      const int lq = cu_q[s + 1] - cu_q[s], lk = cu_k[s + 1] - cu_k[s];
      const int nt = seq_items(mode, causal != 0, cu_q, cu_k, s, tile, fkv);
      int seq_cost = 0;  // mode 2: the sequence's largest tile cost
      if (mode == 2)
        for (int k = 0; k < nt; ++k)
          seq_cost = max(seq_cost, item_cost(mode, causal != 0, lq, lk, tile, k, fkv, bq));
      for (int k = 0; k < nt; ++k) {
        const int idx = seq_item_index(mode, causal != 0, lq, lk, tile, fkv, k);
        const int cost =
            mode == 2 ? seq_cost : item_cost(mode, causal != 0, lq, lk, tile, idx, fkv, bq);
        keys[pos++] = sort_key(mode, cost, s, idx);
      }
    }
    for (int x = count + tid; x < n; x += kThreads) keys[x] = ~0ull;
    __syncthreads();
    // bitonic sort, ascending
    for (int k = 2; k <= n; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int x = tid; x < n; x += kThreads) {
          const int y = x ^ j;
          if (y > x) {
            const unsigned long long a = keys[x], b = keys[y];
            const bool up = (x & k) == 0;
            if ((a > b) == up) {
              keys[x] = b;
              keys[y] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int x = tid; x < count; x += kThreads) {
      int seq, idx;
      decode_key(mode, keys[x], seq, idx);
      tiles[2 * x] = seq;
      tiles[2 * x + 1] = idx;
    }
  } else {
    for (int s = s_lo; s < s_hi; ++s) {
      const int lq = cu_q[s + 1] - cu_q[s], lk = cu_k[s + 1] - cu_k[s];
      const int nt = seq_items(mode, causal != 0, cu_q, cu_k, s, tile, fkv);
      for (int k = 0; k < nt; ++k) {
        tiles[2 * pos] = s;
        tiles[2 * pos + 1] =
            mode == 2 ? nt - 1 - k : seq_item_index(mode, causal != 0, lq, lk, tile, fkv, k);
        ++pos;
      }
    }
  }
  if (tid == 0) hdr[kHdrCount] = (uint32_t)count;
}

}  // namespace

hipError_t launch_sched(const int* cu_q, const int* cu_k, int nseq, int total_q, int total_k,
                        int tile, int mode, bool causal, int fwd_kv_tile, int bwd_q_tile,
                        int* tiles, int max_tiles, int* split_base, int max_split, uint32_t* hdr,
                        bool sorted, hipStream_t stream) {
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kThreads), 0, stream, cu_q, cu_k, nseq, total_q,
                     total_k, tile, mode, causal ? 1 : 0, fwd_kv_tile, bwd_q_tile, tiles,
                     max_tiles, split_base, max_split, hdr, sorted ? 1 : 0);
  return hipGetLastError();
}

}  // namespace fa
