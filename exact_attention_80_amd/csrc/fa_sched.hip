// fa_sched.hip -- on-device work ordering for packed variable-length batches.
//
// One workgroup reads cu_seqlens (never copied to the host), checks it, and
// writes the list of (sequence, tile) work items that the attention kernels
// walk, so the host never synchronises ([FA4B] 3.3.2: a preprocessing kernel
// orders the batches by their per-tile cost and emits the virtual -> actual
// index map the attention kernel then follows).
//   mode 0  forward query tiles, longest (most key tiles) first;
//   mode 1  backward key tiles, longest (most query tiles) first;
//   mode 2  backward key tiles for the deterministic reduction: cheapest first,
//           which within a sequence is last key tile first ([FA4B] 3.3.1), so a
//           key tile is always issued after every key tile it waits for.
// The ordering only changes which work runs when, never any result.  Lists
// longer than the in-LDS sort capacity are written in natural order (still
// last-tile-first within a sequence for mode 2).  Query and key offsets are
// separate arrays (the same one when every sequence has Lq == Lk); forward
// tiles split a sequence's queries, backward tiles its keys, and the cost of
// a tile counts the inner tiles its causal walk visits with the diagonal
// aligned bottom-right (offset Lk - Lq).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 1024;
constexpr int kSortCap = 8192;  // 64 KiB of 64-bit keys

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

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

// tiles of sequence s: its query rows (forward) or its keys (backward)
__device__ __forceinline__ int seq_tiles(int mode, const int* cu_q, const int* cu_k, int s,
                                         int tile) {
  const int* cu = mode == 0 ? cu_q : cu_k;
  return cdiv(cu[s + 1] - cu[s], tile);
}

__device__ __forceinline__ unsigned long long sort_key(int mode, int cost, int seq, int idx) {
  const unsigned long long c = (unsigned long long)(unsigned)cost & 0xFFFFFFull;
  const unsigned long long s = (unsigned long long)(unsigned)seq & 0xFFFFFull;
  const unsigned long long t = (unsigned long long)(unsigned)idx & 0xFFFFFull;
  if (mode == 2) return (c << 40) | ((0xFFFFFull - t) << 20) | s;
  return ((0xFFFFFFull - c) << 40) | (s << 20) | t;
}

__device__ __forceinline__ void decode_key(int mode, unsigned long long k, int& seq, int& idx) {
  if (mode == 2) {
    seq = (int)(k & 0xFFFFFull);
    idx = (int)(0xFFFFFull - ((k >> 20) & 0xFFFFFull));
  } else {
    idx = (int)(k & 0xFFFFFull);
    seq = (int)((k >> 20) & 0xFFFFFull);
  }
}

__global__ __launch_bounds__(kThreads) void sched_kernel(const int* cu_q, const int* cu_k,
                                                         int nseq, int total_q, int total_k,
                                                         int tile, int mode, int causal, int fkv,
                                                         int bq, int* tiles, int max_tiles,
                                                         uint32_t* hdr) {
  __shared__ unsigned long long keys[kSortCap];
  __shared__ int scan[kThreads];
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
  int mine = 0;
  for (int s = s_lo; s < s_hi; ++s) mine += seq_tiles(mode, cu_q, cu_k, s, tile);
  scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int count = scan[kThreads - 1];
  int pos = scan[tid] - mine;
  if (count > max_tiles) {
    if (tid == 0) {
      atomicOr(&hdr[kHdrErr], kErrTileOverflow);
      hdr[kHdrCount] = 0u;
    }
    return;
  }

  if (count <= kSortCap) {
    int n = 1;
    while (n < count) n <<= 1;
    for (int s = s_lo; s < s_hi; ++s) {
      const int lq = cu_q[s + 1] - cu_q[s], lk = cu_k[s + 1] - cu_k[s];
      const int nt = seq_tiles(mode, cu_q, cu_k, s, tile);
      for (int i = 0; i < nt; ++i)
        keys[pos++] = sort_key(mode, tile_cost(mode, causal != 0, lq, lk, tile, i, fkv, bq), s, i);
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
      const int nt = seq_tiles(mode, cu_q, cu_k, s, tile);
      for (int i = 0; i < nt; ++i) {
        tiles[2 * pos] = s;
        tiles[2 * pos + 1] = mode == 2 ? nt - 1 - i : i;
        ++pos;
      }
    }
  }
  if (tid == 0) hdr[kHdrCount] = (uint32_t)count;
}

}  // namespace

hipError_t launch_sched(const int* cu_q, const int* cu_k, int nseq, int total_q, int total_k,
                        int tile, int mode, bool causal, int fwd_kv_tile, int bwd_q_tile,
                        int* tiles, int max_tiles, uint32_t* hdr, hipStream_t stream) {
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kThreads), 0, stream, cu_q, cu_k, nseq, total_q,
                     total_k, tile, mode, causal ? 1 : 0, fwd_kv_tile, bwd_q_tile, tiles,
                     max_tiles, hdr);
  return hipGetLastError();
}

}  // namespace fa
