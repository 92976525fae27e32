// fa_launch.h -- host-side launch entry points of the kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "fa_common.h"

namespace fa {

constexpr int kFwdWaves = 8;   // forward workgroup: 8 waves, 256 query rows
constexpr int kFwdStages = 4;  // forward K/V copy ring depth (tiles)
// d = 256 also runs 8 waves (two per SIMD, rather than the one wave per SIMD
// that 512 registers would allow: 0.29 against 0.36 ms at B = 2, H = 16,
// N = 4096 causal even before the copy offsets moved to LDS) and a 2-deep
// ring of 70 KB K/V tiles
__host__ __device__ constexpr int fwd_waves(int) { return kFwdWaves; }
__host__ __device__ constexpr int fwd_stages(int d) { return d == 256 ? 2 : kFwdStages; }
constexpr int kBwdWaves = 8;   // backward workgroup (d <= 128): 8 waves, 256 keys
constexpr int kBwdBQ = 32;     // backward query tile
constexpr int kBwdBC = kBwdWaves * 32;
// d = 256: 4 waves of 32 keys (128 keys, one wave per SIMD with the whole
// register file for its dK, dV accumulators and V rows)
__host__ __device__ constexpr int bwd_waves(int d) { return d == 256 ? 4 : kBwdWaves; }
__host__ __device__ constexpr int bwd_tile_keys(int d) { return bwd_waves(d) * 32; }
// d = 256: two workgroups per key tile, one per half of the dK / dV / dQ
// columns (both recompute S and dP over the whole head dimension)
__host__ __device__ constexpr int bwd_col_halves(int d) { return d == 256 ? 2 : 1; }

// dQ reduction across key tiles
constexpr int kDqAtomic = 0;   // fp32 device atomics into dq_acc
constexpr int kDqOrdered = 1;  // semaphore-ordered adds into dq_acc (bit-reproducible)
constexpr int kDqPartial = 2;  // plain stores of every partial tile, summed by bwd_dq_reduce
constexpr int kDqFused = 3;    // partial tiles summed by the last workgroup to finish its own
constexpr int kDqFixed = 4;    // int32 fixed-point device atomics (bit-reproducible)

// Fixed-point dQ: row i of a query head accumulates round(x 2^e_i) in int32,
// where e_i = kDqFixedBits - (binary exponent of beta_i) and
// beta_i = |dO_i| max_j |V_j| max_jc |K_jc| bounds every element of the row's
// unscaled dQ and every partial sum of it, so the sum stays below
// 2^kDqFixedBits (2 bits of headroom in int32) and the integer adds are exact
// in any order.  kDqExpNonFinite marks a row whose bound is not finite.
constexpr int kDqFixedBits = 29;
constexpr int kDqExpNonFinite = 1 << 20;
constexpr int kKvBoundRows = 256;  // key rows per partial of the K/V magnitude scan

// e for a row whose bound is beta: beta < 2^k (frexp), e = kDqFixedBits - k,
// so every |x| <= beta has |x| 2^e < 2^kDqFixedBits, and 2^e is the largest
// power of two that guarantees it (beta 2^e >= 2^(kDqFixedBits - 1)); beta = 0
// gives kDqFixedBits, a non-finite beta kDqExpNonFinite.
__host__ __device__ inline int dq_fixed_exponent(float beta) {
  if (!(beta <= 3.40282347e38f)) return kDqExpNonFinite;
  int k = 0;
  (void)frexpf(beta, &k);
  return kDqFixedBits - k;
}

// Index of the partial dQ tile of (query tile i, key tile j) inside its
// (sequence, head): the query tiles' key-tile counts laid end to end (causal:
// query tile i meets key tiles 0 .. i / (kBwdBC / kBwdBQ)).
template <bool CAUSAL>
__host__ __device__ __forceinline__ long pair_index(int i, int j, int nkv) {
  constexpr int R = kBwdBC / kBwdBQ;
  if (CAUSAL) {
    const long a = i / R, r = i % R;
    return (a + 1) * (R / 2 * a + r) + j;
  }
  return (long)i * nkv + j;
}

int fwd_tile_rows(int d);
int fwd_tile_keys();

hipError_t launch_fwd(const FwdParams& p, int d, bool causal, bool varlen, int grid,
                      hipStream_t stream);

// Forward with fp8 (OCP e4m3) Q and K for the scores (p.q8, p.k8; p.c
// includes their descale factors) and bf16 V; d = 64 or 128.
hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, bool varlen, int grid,
                          hipStream_t stream);

// D = rowsum(dO o O) and LSE * log2(e) in the logsumexp layout; zeroes the
// fp32 dQ accumulator (when given), the semaphores and the workspace header.
// With kvb (fixed-point mode) it also writes each row's fixed-point exponent
// to dq_exp ([T, Hq]) from |dO_i| and kvb[h / G].
hipError_t launch_bwd_pre(const bf16* o, const bf16* dout, const float* lse, float* dvec,
                          float* lse2, float* dq_acc, int* sem, long sem_count, uint32_t* hdr,
                          int rows, int Hq, int d, bool varlen, int N, int T, const float* kvb,
                          int G, int* dq_exp, hipStream_t stream);

// Fixed-point mode, before the preprocess: kvb[g] = max_jc |K_jc| * max_j |V_j|
// over every key row j of key/value head g (Tk rows of [Tk, Hkv, d]); part
// holds Hkv * ceil(Tk / kKvBoundRows) pairs of partial maxima.  Non-finite
// values propagate.
hipError_t launch_bwd_kv_bound(const bf16* k, const bf16* v, float* part, float* kvb, long Tk,
                               int Hkv, int d, hipStream_t stream);

// mode: dQ reduction across key tiles (0 fp32 atomics, 1 semaphore-ordered
// adds, 2 partial tiles summed by launch_bwd_dq_reduce, 3 partial tiles summed
// inside the kernel by the last contributor of each query tile, 4 int32
// fixed-point atomics; 2 and 3 are dense-only)
hipError_t launch_bwd(const BwdParams& p, int d, bool causal, bool varlen, int mode, int grid,
                      hipStream_t stream);

// dQ = bf16(scale * sum of the partial tiles) for dense [B, N, Hq, d] (mode 2)
hipError_t launch_bwd_dq_reduce(const float* part, bf16* dq, int B, int N, int Hq, int d,
                                bool causal, int nq, int nkv, long head_pairs, float scale,
                                hipStream_t stream);

// partial dQ tiles per (batch, query head) in mode 2
long bwd_partial_pairs(int N, bool causal);

// whether this build offers the partial-tile dQ modes (2, 3) for head dim d
bool bwd_partial_modes(int d);

// dQ = bf16(scale * dQ_acc); when S > 1 also dK/dV = bf16(sum of the S partials).
// dq_elems counts query-side elements, kv_elems key-side ones.  With dq_exp
// (fixed-point mode) dQ_acc holds int32 values of row r (of d elements) in
// units of 2^-dq_exp[r].
hipError_t launch_bwd_post(const float* dq_acc, bf16* dq, long dq_elems, float scale,
                           const float* dk_part, const float* dv_part, bf16* dk, bf16* dv,
                           long kv_elems, int S, const int* dq_exp, int d, hipStream_t stream);

// Measurement aid (fa_probe_dq_reduction): the backward's atomic dQ reduction
// pattern alone (kind 0 fp32 adds, 2 int32 adds), or the same bytes as plain
// stores (kind 1).
hipError_t launch_probe_dq(float* buf, int rows, int row_floats, int blocks, int items, int kind,
                           hipStream_t stream);

// Variable-length scheduler: validates the query and key offsets (cu_q and
// cu_k may be the same array) and writes the ordered work list.
//   mode 0: forward query tiles, longest first
//   mode 1: backward key tiles, longest first
//   mode 2: backward key tiles, deterministic order (key tiles of a sequence last-first)
// With sorted == false the list keeps the natural order (sequence by sequence).
// Mode 0 also writes split_base (nseq + 1 ints, first partial slot per
// sequence) and flags an overflow when more than max_split chunks are needed.
hipError_t launch_sched(const int* cu_q, const int* cu_k, int nseq, int total_q, int total_k,
                        int tile, int mode, bool causal, int fwd_kv_tile, int bwd_q_tile,
                        int* tiles, int max_tiles, int* split_base, int max_split, uint32_t* hdr,
                        bool sorted, hipStream_t stream);

// Forward combine of split tiles: O = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c
// per row, in ascending chunk order; one workgroup per (sequence, query head).
hipError_t launch_fwd_combine(const FwdParams& p, int d, int nseq, hipStream_t stream);

}  // namespace fa
