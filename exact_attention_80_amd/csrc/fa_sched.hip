// fa_sched.hip -- on-device work ordering for packed variable-length batches.
//
// One workgroup reads cu_seqlens (never copied to the host), checks it, and
// writes the list of (sequence, tile) work items that the attention kernels
// walk, so the host never synchronises ([FA4B] 3.3.2: a preprocessing kernel
// orders the batches by their per-tile cost and emits the virtual -> actual
// index map the attention kernel then follows).
//   mode 0  forward query tiles: sequences in descending order of their
//           largest tile cost, a sequence's tiles together, last (most key
//           tiles when causal) first;
//   mode 1  backward key tiles: every tile in descending order of its cost;
//   mode 2  backward key tiles for the deterministic reduction: sequences as
//           in mode 0, a sequence's key tiles last first ([FA4B] 3.3.1: the
//           cheapest causal tiles first), so a key tile is always issued
//           after every key tile it waits for.
// Measured against one global order of all tiles by cost: on a 65536-token
// batch the forward takes 1.87 against 1.93 ms and the deterministic
// backward 7.1 against 7.9 ms; the fast backward keeps the global order,
// 2 % faster on a decode-shaped batch and 1 % slower on the 65536-token one.
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
#include "fa_sched_keys.h"

namespace fa {

namespace {

constexpr int kThreads = 1024;
constexpr int kSortCap = 8192;  // 64 KiB of 64-bit keys

using namespace sched;

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
      int seq_cost = 0;  // modes 0, 2: the sequence's largest tile cost
      if (mode != 1)
        for (int k = 0; k < nt; ++k)
          seq_cost = max(seq_cost,
                         item_cost(mode, causal != 0, lq, lk, tile,
                                   seq_item_index(mode, causal != 0, lq, lk, tile, fkv, k), fkv, bq));
      for (int k = 0; k < nt; ++k) {
        const int idx = seq_item_index(mode, causal != 0, lq, lk, tile, fkv, k);
        keys[pos++] = sort_key(
            mode, mode == 1 ? item_cost(mode, causal != 0, lq, lk, tile, idx, fkv, bq) : seq_cost,
            s, idx);
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
