/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (libfa_mi355x.so).
 *
 * The library computes exact scaled-dot-product attention, forward and backward,
 * with hand-written HIP kernels; it never approximates the softmax.  The method
 * follows the pages describing FlashAttention-2 and FlashAttention-4:
 *   [FA2]  "FlashAttention-2: Faster Attention with Better Parallelism and Work
 *          Partitioning (ICLR 2024)" (wiki summary), sections "Problem and
 *          motivation", "Core method" 1-4 and "Limitations and future work"
 *          (FP8 kernels);
 *   [FA4B] "FlashAttention-4 backward optimisation: 2-CTA mode and performance"
 *          (blog), sections 2.1 (global atomics for dQ), 3.2 (semaphore-ordered
 *          deterministic reduction), 3.3.1 (shortest-processing-time order for
 *          the causal deterministic backward), 3.3.2 (longest-processing-time
 *          order for variable-length batches), 5.2 (walk every query head of a
 *          key/value head together), 5.3 (bf16 operands, fp32 accumulation);
 *   [FA4N] "FlashAttention-4 wird offiziell veroeffentlicht" (news article),
 *          section on the co-design ideas (conditional softmax rescaling);
 *   [FA4C] "FlashAttention-4: memory and compute efficiency of GPU attention"
 *          (codechina article), section 5.1 (an FP8 compute mode for
 *          data-centre GPUs).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are caller-owned DEVICE memory (e.g. PyTorch allocations), dense,
 *    contiguous, 16-byte aligned.  Q, K, V, O, dO, dQ, dK, dV are bf16
 *    (fa_fwd_fp8 and fa_varlen_qk_fwd_fp8 take Q and K as one-byte e4m3
 *    values).
 *    The library never allocates or frees device memory.  Its only host state
 *    is a per-device property cache and the opt-in timing event pool below,
 *    so calls on different streams are independent as long as their buffers
 *    (including workspaces) differ.
 *  - Dense layout (token-major): Q/O/dO/dQ are [B, N, Hq, d]; K/V/dK/dV are
 *    [B, N, Hkv, d]; the logsumexp LSE is fp32 [B, Hq, N].
 *  - Packed variable-length layout: Q/O/dO/dQ are [T, Hq, d], K/V/dK/dV are
 *    [T, Hkv, d] and LSE is fp32 [Hq, T], where sequence s occupies tokens
 *    cu_seqlens[s] .. cu_seqlens[s+1]-1.  cu_seqlens is DEVICE int32 with
 *    nseq+1 entries; it is validated on the device (first 0, last T,
 *    non-decreasing) and a violation is reported through the workspace error
 *    word (fa_workspace_error), not by the return value.
 *  - d (head dimension) is 64, 128 or 256 (256: the fa_bwd partial-tile modes
 *    deterministic == 2, 3 are not offered, nor at d = 64 in a library built
 *    with 64 keys per backward wave (FA_BWD_KEY_BLOCKS=2); the fp8 forwards
 *    take 64 or 128).
 *    Hq must be a positive multiple of Hkv, and Hq * d below 2^24 (per-tile
 *    buffer ranges are 32-bit; larger shapes return FA_ERR_UNSUPPORTED);
 *    query head h uses key/value head h / (Hq/Hkv) ([FA2] "Core method" 4).
 *  - causal != 0 masks key j from query i when j > i ([FA2] "Core method" 2)
 *    when queries and keys have the same length.  The fa_varlen_qk_* calls
 *    take separate query and key lengths per sequence (Lq, Lk; the
 *    decode-shaped batches of [FA4B] 3.3.2): the queries are the last Lq
 *    positions of the Lk-token context, so the mask is aligned bottom-right,
 *    hiding key j from query i when j > i + Lk - Lq.  A query that sees no key
 *    (Lq > Lk, or Lk = 0) gets O = 0, LSE = -inf and dQ = 0.
 *  - softmax_scale multiplies q.k before the softmax (typically 1/sqrt(d)).
 *  - LSE_i = ln sum_j exp(softmax_scale * q_i.k_j)  ([FA2] "Core method" 1:
 *    the only statistic the backward needs), over the keys query i sees.
 *  - stream is a hipStream_t passed as void* (NULL = default stream).  Every
 *    call is asynchronous on that stream; argument errors are detected on the
 *    host and returned before anything is launched.
 *  - ws / ws_bytes: caller-owned device workspace of at least the size that the
 *    matching *_workspace_size query returns for the same arguments (ws may be
 *    NULL when that size is 0).  Its contents on entry do not matter.
 *  - Return value: an fa_status; fa_status_string() names it and
 *    fa_last_error() gives the detailed message of the calling thread's last
 *    failure.  No C++ exception ever crosses this interface.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,    /* null pointer, bad size, misalignment, bad flag */
  FA_ERR_UNSUPPORTED = 2,    /* valid but not implemented (e.g. d not in {64,128,256}) */
  FA_ERR_WORKSPACE = 3,      /* workspace missing or smaller than required */
  FA_ERR_HIP = 4,            /* a HIP runtime call or kernel launch failed */
  FA_ERR_DEVICE = 5,         /* current device is not a gfx950 GPU */
  FA_ERR_DEVICE_REPORTED = 6 /* a kernel flagged an error in the workspace */
} fa_status;

/* Bits of the device-side error word read by fa_workspace_error(). */
#define FA_DEVERR_BAD_CU_SEQLENS 1u  /* cu_seqlens not 0..T non-decreasing */
#define FA_DEVERR_WAIT_TIMEOUT 2u    /* deterministic dQ ordering wait expired */
#define FA_DEVERR_TILE_OVERFLOW 4u   /* more tiles than the workspace holds */

/* Version of this interface (incremented on any incompatible change). */
int fa_abi_version(void);

/* Static name of a status code. */
const char* fa_status_string(int status);

/* Detailed message of the calling thread's most recent non-FA_OK return. */
const char* fa_last_error(void);

/* ---- dense forward ------------------------------------------------------ */

/* Workspace bytes fa_fwd needs for these sizes (0: the dense forward needs none). */
size_t fa_fwd_workspace_size(int B, int N, int Hq, int Hkv, int d, int causal);

/*
 * Forward pass ([FA2] "Core method" 1-3, [FA4N] conditional rescaling):
 *   O = softmax(scale * Q K^T [causal mask]) V,   LSE as defined above.
 * q [B,N,Hq,d], k/v [B,N,Hkv,d] bf16 inputs; o [B,N,Hq,d] bf16 and
 * lse [B,Hq,N] fp32 outputs.  The result does not depend on the launch order
 * (every output element is written by exactly one workgroup).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int N, int Hq, int Hkv, int d, float softmax_scale, int causal,
           void* ws, size_t ws_bytes, void* stream);

/*
 * Forward pass with fp8 scores ([FA2] "Limitations and future work" names
 * FP8 kernels as the next step; [FA4C] 5.1):
 *   S = scale * (q_descale * Q8) (k_descale * K8)^T,
 *   O = softmax(S [causal mask]) V,   LSE_i = ln sum_j exp(S_ij).
 * q8 [B,N,Hq,d] and k8 [B,N,Hkv,d] hold one byte per element in the OCP
 * e4m3 format (the "fn" variant: no infinities, 0x7f / 0xff are NaN, largest
 * finite 448); q_descale and k_descale (positive, finite) are the per-tensor
 * factors that turn the stored values back into Q and K.  The product Q8 K8^T
 * is exact in the fp32 accumulator up to the order of the additions; P is
 * rounded to bf16 for the P V product as in fa_fwd.  v [B,N,Hkv,d] bf16, o
 * [B,N,Hq,d] bf16, lse [B,Hq,N] fp32 as in fa_fwd.  d = 64 or 128 (anything
 * else: FA_ERR_UNSUPPORTED); no workspace.  This call has no backward: the
 * fp8 inputs are meant for inference.
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v, void* o, float* lse,
               int B, int N, int Hq, int Hkv, int d, float softmax_scale,
               float q_descale, float k_descale, int causal, void* stream);

/* ---- dense backward ----------------------------------------------------- */

/* Workspace bytes fa_bwd needs (D = rowsum(dO o O), the fp32 dQ accumulator or,
 * for deterministic == 2 or 3, the fp32 partial dQ tiles (32 x d floats per
 * pair of a 32-row query tile and a 256-key tile that meet: about 2.2 GB for
 * causal B=2, Hq=16, N=8192, d=128), ordering semaphores or arrival counters,
 * split dK/dV partials; for deterministic == 4 an int32 accumulator, the K/V
 * maxima and one exponent per query row and head).  0 when the sizes or the
 * mode are invalid. */
size_t fa_bwd_workspace_size(int B, int N, int Hq, int Hkv, int d, int causal,
                             int deterministic);

/*
 * Backward pass: from Q, K, V, the forward's O and LSE, and dO, computes
 *   D = rowsum(dO o O), P = exp(scale Q K^T - LSE), dV = P^T dO,
 *   dP = dO V^T, dS = P o (dP - D), dQ = scale dS K, dK = scale dS^T Q,
 * with dK/dV summed over the query heads of each key/value head
 * ([FA2] "Core method" 2 and 4).  Work is split over key/value tiles; the
 * partial dQ of every tile is reduced in fp32 with device atomics when
 * deterministic == 0 ([FA4B] 2.1), or in a fixed order serialised by
 * semaphores when deterministic == 1 ([FA4B] 3.2, 3.3.1), or, when
 * deterministic == 2, stored as one fp32 tile per (query tile, key tile)
 * pair and summed in ascending key-tile order by a second kernel (no atomics;
 * dense layout only), or, when deterministic == 3, stored the same way
 * (coherent for the whole device) and summed in the same order inside the
 * main kernel by the last workgroup to contribute to each query tile, which
 * writes dQ itself (one counting atomic per tile; dense layout only), or,
 * when deterministic == 4, added with int32 device atomics in fixed point:
 * row i of query head h accumulates round(x 2^e) of every contribution x,
 * where 2^e is the largest power of two that keeps the bound
 * |dO_i| max_j |V_j| max |K| (K/V maxima over every key row of the key/value
 * head; a bound on every element of the row's unscaled dQ, see
 * fa_bwd.hip) below 2^29, so the integer sums are exact and do not depend
 * on the order of the adds.  A preprocessing pass reads K and V once for
 * those maxima.  The result differs from the fp32 sum by at most (number of
 * key tiles) / 2 + 32 steps of 2^-e per element before the final bf16
 * rounding (a row's dQ has about 29 significant bits relative to its bound);
 * a row whose bound is not finite (non-finite dO, K or V) gets dQ = NaN.
 * The step follows the bound, not the row's own dQ: one K or V row far
 * larger than the rest of its head (an outlier in any sequence) coarsens the
 * step of every row of that head by the same factor, which fp32 sums do not
 * suffer; with 100x outliers the step nears the bf16 rounding of dQ, so
 * modes 0 and 1 suit inputs with heavy-tailed K or V.
 * This is an MI355X-specific choice: int32 device atomics sustain about 1.7
 * TB/s against 1.35 TB/s for fp32 ones (fa_probe_dq_reduction).
 * Modes 1 to 4 make dQ/dK/dV bit-identical from run to run (and the
 * partial-tile modes 2 and 3 give the same dQ); mode 4 also across tile
 * orders.  dK/dV never use atomics.  Any other value: FA_ERR_INVALID_ARG.
 * Mode 1 bounds every semaphore wait (2 s, or FA_DET_SPIN_TICKS ticks of the
 * 100 MHz clock from the environment); a wait that expires sets
 * FA_DEVERR_WAIT_TIMEOUT in the workspace and the adds proceed unordered, so
 * the kernel always completes and dQ is still the correct sum, but not
 * bit-reproducible.  The return value cannot report this (the call is
 * asynchronous): a caller that relies on reproducibility must check
 * fa_workspace_error() after the call (the same holds for fa_varlen_bwd and
 * fa_varlen_qk_bwd with deterministic == 1).
 * Outputs dq [B,N,Hq,d], dk/dv [B,N,Hkv,d] bf16.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           int B, int N, int Hq, int Hkv, int d, float softmax_scale, int causal,
           int deterministic, void* ws, size_t ws_bytes, void* stream);

/* ---- packed variable-length forward / backward ---------------------------- */

/* max_seqlen: a hint (an upper bound on any sequence length, or 0 if unknown);
 * it must be >= 0 and is otherwise unused, since the scheduling kernel reads
 * the lengths from cu_seqlens itself.  total_tokens = T = cu_seqlens[nseq].
 * The forward workspace holds the header, the tile list and the partial
 * results of split query tiles: a sequence whose last query tile has at most
 * 32 queries and more than 32 key tiles of 64 keys has that tile split into
 * chunks of 32 key tiles that run as separate work items ([FA2] "Core
 * method" 2: parallelism over the sequence), merged exactly afterwards by a
 * second kernel.  0 for invalid sizes. */
size_t fa_varlen_fwd_workspace_size(int nseq, int total_tokens, int Hq, int Hkv, int d,
                                    int causal);

/*
 * Forward over a packed batch: every sequence attends only to itself.  A
 * one-workgroup scheduling kernel first reads cu_seqlens on the device and
 * orders the (sequence, query-tile) work items longest-first ([FA4B] 3.3.2),
 * so no host synchronisation is needed.  Shapes as in the packed layout above.
 */
int fa_varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens, int nseq, int total_tokens, int max_seqlen,
                  int Hq, int Hkv, int d, float softmax_scale, int causal,
                  void* ws, size_t ws_bytes, void* stream);

size_t fa_varlen_bwd_workspace_size(int nseq, int total_tokens, int Hq, int Hkv, int d,
                                    int causal, int deterministic);

/* Backward over a packed batch; semantics as fa_bwd, per sequence.
 * deterministic must be 0, 1 or 4 (2 or 3 returns FA_ERR_UNSUPPORTED); in
 * mode 4 the K/V maxima run over every key row of the batch. */
int fa_varlen_bwd(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  const int32_t* cu_seqlens, int nseq, int total_tokens, int max_seqlen,
                  int Hq, int Hkv, int d, float softmax_scale, int causal,
                  int deterministic, void* ws, size_t ws_bytes, void* stream);

/* ---- packed batches with separate query and key lengths ------------------
 * q/o/dout/dq [total_q, Hq, d] and lse [Hq, total_q]; k/v/dk/dv
 * [total_k, Hkv, d].  Sequence s has queries cu_seqlens_q[s] .. [s+1]-1 and
 * keys cu_seqlens_k[s] .. [s+1]-1; both arrays are DEVICE int32 with nseq+1
 * entries, validated on the device (first 0, last total_q / total_k,
 * non-decreasing; a violation sets FA_DEVERR_BAD_CU_SEQLENS).  A sequence may
 * have Lq = 0 or Lk = 0; total_q and total_k must be positive.  Causal masks
 * are bottom-right aligned (see the conventions above).  The scheduling kernel
 * orders the tiles by their cost under that mask, longest first ([FA4B]
 * 3.3.2).  max_seqlen_q / max_seqlen_k are hints (>= 0, 0 if unknown).  With
 * cu_seqlens_q == cu_seqlens_k these calls compute exactly what
 * fa_varlen_fwd / fa_varlen_bwd compute. */
size_t fa_varlen_qk_fwd_workspace_size(int nseq, int total_q, int total_k, int Hq, int Hkv,
                                       int d, int causal);

int fa_varlen_qk_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                     int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int Hq,
                     int Hkv, int d, float softmax_scale, int causal, void* ws, size_t ws_bytes,
                     void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid allocation): fa_varlen_qk_fwd
 * with no workspace argument.  The same kernels use instead one scratch array
 * of FA_NOALLOC_SCRATCH_BYTES per GPU, a static device array of the library
 * that the GPU holds until the process ends; its address is looked up once
 * per device on the first call there.  The caller still provides every input
 * and output.  A problem whose workspace (fa_varlen_qk_fwd_workspace_size)
 * exceeds FA_NOALLOC_SCRATCH_BYTES returns FA_ERR_WORKSPACE before any
 * launch.  Everything the kernels read from the scratch is written earlier
 * in the same call (the error word and tile list by the scheduling kernel,
 * the partial results of split tiles by the forward), so nothing carries
 * over from one call to the next; but every call on a GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (on different streams or
 * threads) race and must be serialised by the caller.  The device error word
 * of this call is not readable through fa_workspace_error.  Allocates
 * nothing, on the device or with any allocating library routine. */
#define FA_NOALLOC_SCRATCH_BYTES (64u << 20)
int fa_varlen_qk_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                             int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                             int Hq, int Hkv, int d, float softmax_scale, int causal,
                             void* stream);

/* fa_varlen_qk_fwd with fp8 scores, as in fa_fwd_fp8: q8 [total_q, Hq, d] and
 * k8 [total_k, Hkv, d] are OCP e4m3 bytes standing for q_descale * Q and
 * k_descale * K; v, o, lse, the offsets and the bottom-right causal mask as in
 * fa_varlen_qk_fwd; d = 64 or 128.  The workspace is sized by
 * fa_varlen_qk_fwd_workspace_size (the same layout).  The decode-shaped
 * batches of [FA4B] 3.3.2 with an fp8 key cache are the intended use. */
int fa_varlen_qk_fwd_fp8(const void* q8, const void* k8, const void* v, void* o, float* lse,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                         int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int Hq,
                         int Hkv, int d, float softmax_scale, float q_descale, float k_descale,
                         int causal, void* ws, size_t ws_bytes, void* stream);

/* deterministic must be 0, 1 or 4 (2 or 3 returns FA_ERR_UNSUPPORTED); the size
 * query returns 0 for invalid sizes or modes. */
size_t fa_varlen_qk_bwd_workspace_size(int nseq, int total_q, int total_k, int Hq, int Hkv,
                                       int d, int causal, int deterministic);

int fa_varlen_qk_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                     int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int Hq,
                     int Hkv, int d, float softmax_scale, int causal, int deterministic, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * Debug/test helper: synchronises `stream`, reads the device error word that
 * the last call using this workspace left, and returns FA_OK when it is clear
 * or FA_ERR_DEVICE_REPORTED (fa_last_error() then names the FA_DEVERR_* bits).
 * *bits (if not NULL) receives the raw word.  ws must be a workspace of a
 * varlen call or a backward call.
 */
int fa_workspace_error(const void* ws, size_t ws_bytes, void* stream, uint32_t* bits);

/* ---- measurement ----------------------------------------------------------
 * Opt-in kernel timing for benchmarks (not needed for correctness).  Between
 * fa_timing_begin() and fa_timing_end(), every forward / backward call made by
 * the calling thread records a pair of HIP events on its own stream around
 * each kernel it launches.  fa_timing_end() waits for the last event and
 * returns, per kernel kind, the number of launches and their summed duration
 * in milliseconds:
 *   kind 0: forward kernel;  kind 1: backward main kernel;
 *   kind 2: backward preprocess (D = rowsum(dO o O), zeroing);
 *   kind 3: backward post (dQ conversion or partial-tile sum, split dK/dV sum);
 *   kind 4: variable-length scheduler;
 *   kind 5: variable-length forward combine (merges the key chunks of split
 *           query tiles).
 * counts / ms must each point to FA_TIMING_KINDS elements (or be NULL).
 * Events are created lazily and reused; nothing is allocated on the device. */
/* Measurement aid: the dQ reduction traffic of the fast backward (d = 128)
 * without its products, to measure what the fp32 device atomics sustain
 * ([FA4B] 2.1: dQ is reduced across key tiles by global atomic adds).
 * `blocks` workgroups of 8 waves each take `items` 32-row x 128-column tiles
 * of buf [rows, row_floats] fp32 (device memory, rows a multiple of 32,
 * row_floats of 128) and add 1/1024 to every element of the tile with the
 * backward's buffer atomic instructions (32 x 16 columns per wave, 4 rows x
 * 16 columns per instruction), or, with store = 1, write the same bytes with
 * plain stores, or, with store = 2, add the int32 1 to every element with the
 * int32 atomic instructions of the fixed-point dQ mode (deterministic == 4;
 * buf then holds int32 values).  Moves blocks * items * 16 KiB; asynchronous
 * on `stream`; the caller times it. */
int fa_probe_dq_reduction(float* buf, int rows, int row_floats, int blocks, int items, int store,
                          void* stream);

#define FA_TIMING_KINDS 6
int fa_timing_begin(void);
int fa_timing_end(int* counts, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
