// fa_bwd.hip -- fused attention backward for gfx950.
//
// Method ([FA2] "Core method" 2 and 4; [FA4B] 2.1, 3.2, 3.3.1, 5.2, 5.3):
//  * preprocess: D = rowsum(dO o O) per query row (fp32), and the fp32 dQ
//    accumulator, the ordering semaphores and the workspace header are zeroed
//    (fixed-point mode: also each row's fixed-point exponent);
//  * main kernel: one workgroup per (sequence, key/value head, key tile of 256
//    keys -- 128 for d = 256, with one workgroup per half of the output
//    columns --, query-head subgroup).  Each of the 8 (d = 256: 4) waves owns
//    32 keys and keeps its
//    K and V rows and its dK, dV accumulators in registers for the whole
//    kernel.  The workgroup walks every query head of its key/value head
//    (subgroup) and, per head, the 32-row query tiles that see its keys
//    (causal: from the last one down to the diagonal, or from the diagonal
//    up in the ordered mode below) or all of them; per query tile:
//        S  = Q K^T,  P = exp2(S c - LSE log2 e)        (recomputed, masked)
//        dP = dO V^T, dS = P o (dP - D)
//        dV += P^T dO,  dK += dS^T Q                    (register accumulators)
//        dQ_tile += dS K                                (dS exchanged via LDS)
//    The dQ tile is reduced across key tiles either with fp32 device atomics
//    (fast) or, in deterministic mode, in a fixed order: for each dQ tile the
//    writers are applied in descending key-tile index, each waiting on a
//    per-tile semaphore until its rank comes up, adding, and releasing it
//    once its adds are known to be performed (two items later).
//    Workgroups take their work items from an atomic ticket in that same
//    descending order, so every workgroup a writer waits for already runs and
//    the causal walk (diagonal first) never stalls on its first write.
//    Two more deterministic ways need no atomic adds on dQ: every workgroup
//    stores its fp32 partial tile, and either a second kernel sums each
//    query tile's partial tiles in ascending key-tile order, or (fused) each
//    workgroup counts itself in with one atomic per tile once its stores are
//    complete and the last contributor of a query tile does that sum and
//    writes bf16 dQ itself.  The fixed-point mode adds with int32 device
//    atomics, which this GPU performs faster than fp32 ones: every
//    contribution to row i is rounded to a multiple of 2^-e_i, with e_i set
//    from a bound on the row's dQ (|dO_i| times the largest V row norm and
//    the largest |K| element of the key/value head, which a scan of K and V
//    before the preprocess finds) so that the int32 sums cannot overflow;
//    integer adds are exact, so the result does not depend on their order.
//  * post: dQ = bf16(scale * dQ_acc) (fixed point: scaled by 2^-e_i first);
//    split subgroups' dK/dV partials are summed in a fixed order.
// A packed sequence may have Lq queries and Lk keys (the decode-shaped
// batches of [FA4B] 3.3.2): the causal diagonal is then aligned bottom-right
// (query i sees key j iff j <= i + Lk - Lq), the walk of a key tile starts at
// the first query tile that sees it, and rows that see no key carry
// LSE = -inf, which the preprocess turns into P = 0.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int NW = kBwdWaves;
constexpr int NT = NW * 64;
constexpr int BQ = kBwdBQ;
constexpr int BC = kBwdBC;


// LDS plan.  K, Q and dO tiles are row-major SwzTiles (pitch 16 mod 64
// dwords) filled by direct global->LDS loads; Q/dO/LSE/D are double
// buffered.  dS^T is written by the waves with 8-byte stores into 64-byte rows
// whose 8-byte slots are permuted by the row's quad index (conflict-free for
// both the stores and the transposed reads); it is double buffered too, so
// that an item's dQ products can read it while the next item writes its own.
// d = 128: 81920 + 4 x 10240 + 512 + 16384 + 16384 bytes.
template <int D>
struct BwdLds {
  static constexpr int BCD = bwd_tile_keys(D);       // keys per workgroup
  static constexpr int CH = D / 8;
  // row pitch 16 (mod 64) dwords (320, 192 or 576 bytes); the d = 256 K tile
  // uses 544 bytes so that K, the double-buffered Q / dO and dS^T fit in LDS
  static constexpr int STRIDE = D == 256 ? 36 : (D == 128 ? 20 : 12);
  static constexpr int KSTRIDE = D == 256 ? 34 : STRIDE;
  using KT = SwzTile<BCD, CH, KSTRIDE>;              // K tile [BC][D]
  using QT = SwzTile<BQ, CH, STRIDE>;                // Q or dO tile [BQ][D]
  static constexpr int statBytes = 2 * BQ * 4;       // LSE[BQ] then D[BQ]
  static constexpr int dsPitch = BQ * 2;             // dS^T row: 32 bf16
  static constexpr int dsBytes = BCD * dsPitch;
};

// byte offset of the 8-byte slot holding dS^T[key][4s .. 4s+3].  The slot
// is permuted by f(k) = k ^ ((k & 2) << 1) of the row's quad index k = (key/4)
// mod 8: a bijection, so the stores of 32 consecutive keys to one slot hit 32
// different 2-bank pairs, and the quads k and k ^ 2 read together by the two
// 16-lane halves of a transposed read land in different 32-byte halves of
// their rows.
__device__ __forceinline__ int ds_off(int key, int s) {
  const int k = (key >> 2) & 7;
  return key * (BQ * 2) + ((s ^ k ^ ((k & 2) << 1)) << 3);
}

// Key blocks of 32 per wave in the backward: 1 by default (8 waves, two per
// SIMD).  A build with FA_BWD_KEY_BLOCKS=2 runs d = 64 with 4 waves of 64
// keys (one wave per SIMD with its 512 registers), so that every Q and dO
// operand read from LDS feeds the products of both key blocks; at d = 128
// the two blocks' accumulators and operands do not fit 512 registers (about
// 250 values spill), so d = 128 keeps one block.
#ifndef FA_BWD_KEY_BLOCKS
#define FA_BWD_KEY_BLOCKS 1
#endif
__host__ __device__ constexpr int bwd_key_blocks(int d) { return d == 64 ? FA_BWD_KEY_BLOCKS : 1; }
__host__ __device__ constexpr int bwd_threads(int d) { return bwd_waves(d) / bwd_key_blocks(d) * 64; }

template <int D, bool CAUSAL, bool VARLEN, int DQM>
__global__ __launch_bounds__(bwd_threads(D)) void bwd_kernel(BwdParams p) {
  constexpr int KB = bwd_key_blocks(D);   // 32-key blocks per wave
  constexpr int NW = bwd_waves(D) / KB;   // waves (shadows the d <= 128 defaults)
  constexpr int NT = NW * 64;
  constexpr int BC = NW * 32 * KB;
  // d = 256: each workgroup owns one half of the head dimension for dK, dV
  // and dQ (S and dP still use all of it), so its accumulators fit the
  // register file; two workgroups share a key tile
  constexpr int NHALF = bwd_col_halves(D);
  constexpr int DH = D / NHALF;     // output columns per workgroup
  constexpr bool DET = DQM == kDqOrdered;
  constexpr bool FUSED = DQM == kDqFused;
  constexpr bool FIXED = DQM == kDqFixed;
  constexpr bool PARTS = DQM == kDqPartial || FUSED;  // partial tiles in dq_part
  using L = BwdLds<D>;
  constexpr int ST = L::STRIDE;
  constexpr int KST = L::KSTRIDE;
  using KT = typename L::KT;
  using QT = typename L::QT;
  __shared__ __attribute__((aligned(16))) char k_s[KT::kBytes];
  __shared__ __attribute__((aligned(16))) char q_s0[QT::kBytes];
  __shared__ __attribute__((aligned(16))) char q_s1[QT::kBytes];
  __shared__ __attribute__((aligned(16))) char do_s0[QT::kBytes];
  __shared__ __attribute__((aligned(16))) char do_s1[QT::kBytes];
  __shared__ __attribute__((aligned(16))) char st_s0[L::statBytes];
  __shared__ __attribute__((aligned(16))) char st_s1[L::statBytes];
  __shared__ __attribute__((aligned(16))) char ds_s0[L::dsBytes];
  __shared__ __attribute__((aligned(16))) char ds_s1[L::dsBytes];
  __shared__ int sh_ticket;
  __shared__ int sh_last[4];  // fused mode: "this workgroup completes item t" (t mod 4)
  // fixed-point mode: the query tile's row exponents, item t in slot t mod 3
  // (copied with item t's rows, read by item t's dQ adds one item later,
  // while item t+2's copy goes to the third slot)
  __shared__ __attribute__((aligned(16))) int ex_s[FIXED ? 3 : 1][BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int g16 = lane >> 4;
  const int L16 = lane & 15;

  // ---------------- work item
  int r;
  if (DET) {
    if (tid == 0) sh_ticket = (int)atomicAdd(&p.hdr[kHdrTicket], 1u);
    __syncthreads();
    r = sh_ticket;
  } else {
    r = blockIdx.x;
  }
  const int chalf = NHALF > 1 ? (r % NHALF) : 0;  // output column half
  r /= NHALF;
  const int dh0 = chalf * DH;                     // first output column
  BwdItem it;
  const int HS = p.Hkv * p.S;
  if (VARLEN) {
    if (p.hdr[kHdrErr] & kErrBadCu) return;
    const int e = r / HS;
    const int u = r - e * HS;
    if (e >= (int)p.hdr[kHdrCount]) return;
    it.seq = p.tiles[2 * e];
    it.jt = p.tiles[2 * e + 1];
    it.hkv = u / p.S;
    it.split = u - it.hkv * p.S;
    it.q_start = p.cu_seqlens[it.seq];
    it.q_len = p.cu_seqlens[it.seq + 1] - it.q_start;
    it.k_start = p.cu_seqlens_k[it.seq];
    it.k_len = p.cu_seqlens_k[it.seq + 1] - it.k_start;
    it.off = it.k_len - it.q_len;
    it.nq = (it.q_len + BQ - 1) / BQ;
    it.nkv = (it.k_len + BC - 1) / BC;
  } else {
    const int U = p.B * HS;
    int u, jj;
    if (DET) {
      jj = r / U;
      u = r - jj * U;
      jj = p.nkv - 1 - jj;  // key tiles last-first (shortest work first when causal)
    } else if (p.sched == 0 && (U & 7) == 0) {
      const int x = r & 7, rr = r >> 3, ux = U >> 3;
      jj = rr / ux;
      u = x * ux + (rr - jj * ux);
    } else if (p.sched == 0) {
      jj = r / U;
      u = r - jj * U;
    } else {
      u = r / p.nkv;
      jj = r - u * p.nkv;
    }
    it.seq = u / HS;
    const int rest = u - it.seq * HS;
    it.hkv = rest / p.S;
    it.split = rest - it.hkv * p.S;
    it.jt = jj;
    it.q_start = it.seq * p.N;
    it.q_len = p.N;
    it.k_start = it.q_start;
    it.k_len = p.N;
    it.off = 0;
    it.nq = p.nq;
    it.nkv = p.nkv;
  }

  const int GS = p.G / p.S;
  const int h0 = it.hkv * p.G + it.split * GS;
  const long q_row = (long)p.Hq * D;
  const long kv_row = (long)p.Hkv * D;
  const int key0 = it.jt * BC;
  // block kb of this wave: keys wk0[kb] .. wk0[kb] + 31 (key rows of the
  // workgroup's tile from krow0[kb])
  int krow0[KB], wk0[KB], mykey[KB];
  bool key_ok[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    krow0[kb] = (wave * KB + kb) * 32;
    wk0[kb] = key0 + krow0[kb];
    mykey[kb] = wk0[kb] + l32;
    key_ok[kb] = mykey[kb] < it.k_len;
  }
  const int klast = it.k_len - 1;  // last key row (row clamp of the K copy)
  const int qlast = it.q_len - 1;  // last query row

  // ---------------- K tile -> LDS (direct), V rows of this wave -> registers
  const bf16* kseq = p.k + (long)it.k_start * kv_row + (long)it.hkv * D;
  const bf16* vseq = p.v + (long)it.k_start * kv_row + (long)it.hkv * D;
  dma_swz_tile<KT, KST, NW>(k_s, kseq, kv_row, key0, klast, wave, lane);
  bf16x8 vf[KB][D / 16];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      u32x4 b = {0u, 0u, 0u, 0u};
      if (key_ok[kb]) b = ld_global16(vseq + (long)mykey[kb] * kv_row + dc * 16 + half * 8);
      vf[kb][dc] = as_bf16x8(b);
    }
  wait_vmem();  // V rows and the K tile are in before the loop starts

  f32x16 dk_acc[KB][DH / 32], dv_acc[KB][DH / 32];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int x = 0; x < 16; ++x) { dk_acc[kb][db][x] = 0.f; dv_acc[kb][db][x] = 0.f; }

  // ---------------- walk over (head, query tile); causal: from the first
  // query tile holding a query that sees key0 (query >= key0 - off)
  const int i_start = CAUSAL ? max(0, key0 - it.off) / BQ : 0;
  const int nsteps = max(0, it.nq - i_start);
  const int nitems = GS * nsteps;
  // query tile of step u of a head's walk.  Causal, every mode but the
  // ordered one: from the last query tile down to the diagonal (measured
  // faster than the upward walk in the atomic and partial-tile modes; in the
  // fused mode the key tiles then reach a query tile at about the same step,
  // which spreads the last-contributor sums over the workgroups).  The
  // ordered mode walks from the diagonal upwards: a dQ tile's writers apply
  // in descending key-tile order, and a top-down walk would make every key
  // tile's first step wait for all higher ones.
  auto step_tile = [&](int u) { return (!DET && CAUSAL) ? it.nq - 1 - u : i_start + u; };

  // direct copy of one query tile's Q, dO rows (rows past the sequence end
  // read as zeros) and LSE, D values
  TileCopy<QT, NW> qcopy;
  qcopy.init(q_row * 2, ST, wave, lane, [](int row, int pc) { return QT::slot_chunk(row, pc); });
  auto issue_item = [&](int item, char* qd, char* dod, char* std_) {
    const int hh = item / nsteps;
    const int i = step_tile(item - hh * nsteps);
    const int h = h0 + hh;
    const int q0 = i * BQ;
    const long tok = (long)it.q_start + q0;
    const uint32_t range = tile_range(q0, it.q_len, q_row * 2, D * 2, BQ);
    qcopy.issue(qd, make_rsrc(p.q + tok * q_row + (long)h * D, range));
    qcopy.issue(dod, make_rsrc(p.dout + tok * q_row + (long)h * D, range));
    if (wave == NW - 1) {
      // lanes 0..31 copy the tile's LSE values, lanes 32..63 its D values;
      // both land at std_ + 4*lane, so the buffer holds LSE[BQ] then D[BQ]
      long base;
      if (VARLEN) base = (long)h * p.T + it.q_start;
      else base = ((long)it.seq * p.Hq + h) * p.N;
      const int q = min(q0 + l32, qlast);
      if (half == 0) dma4(p.lse + base + q, std_);
      else dma4(p.dvec + base + q, std_);
    }
    if (FIXED && wave == NW - 2 && half == 0) {
      const int q = min(q0 + l32, qlast);
      dma4(p.dq_exp + (tok - q0 + q) * p.Hq + h, ex_s[item % 3]);
    }
  };

  // dQ tile (BQ x D) of an item = dS (BQ x BC) K (BC x D) with 16x16x32
  // products: wave w owns NCB 16-column blocks of dQ, from dblk on, for NQB
  // 16-row blocks from qb0 on (d = 128: one column block, both row blocks;
  // d = 64: one of each; d = 256: four column blocks, both row blocks), over
  // all BC keys, so no partial sums are exchanged and every wave adds its own
  // blocks.
  constexpr int DB16 = DH / 16;              // 16-column blocks of dQ (this workgroup's)
  constexpr int UPW = (2 * DB16) / NW;       // (row block, column block) units per wave
  constexpr int NQB = UPW >= 2 ? 2 : 1;      // 16-row blocks per wave
  constexpr int NCB = UPW / NQB;             // 16-column blocks per wave
  static_assert(NQB * NCB * NW == 2 * DB16, "dQ work split");
  static_assert(NCB == 1 || !PARTS, "partial-tile modes use one column block per wave");
  constexpr int CG = DB16 / NCB;             // column groups
  const int dblk = (wave % CG) * NCB;
  const int qb0 = (wave / CG) * NQB;

  // Per-lane LDS byte offsets.  Every operand read below is one of these
  // bases plus a compile-time constant (the tile swizzle only permutes chunks
  // inside aligned groups of four, so it never mixes with the unrolled loop
  // indices).
  //   16-byte reads of chunk 2dc + half of row r:  base[dc & 1] + 64 (dc >> 1)
  const int q_rd[2] = {QT::off(l32, 8 * half), QT::off(l32, 16 + 8 * half)};
  int k_rd[KB][2];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    k_rd[kb][0] = KT::off(krow0[kb] + l32, 8 * half);
    k_rd[kb][1] = KT::off(krow0[kb] + l32, 16 + 8 * half);
  }
  //   transposed reads of Q/dO rows 16qc + 8ld + 4(g16/2) + L16/4, columns
  //   32db + 16(g16%2) + 4(L16%4):  base[ld] + 16 qc pitch + 64 db
  const int rq = 4 * (g16 >> 1) + (L16 >> 2);
  const int cq = 16 * (g16 & 1) + 4 * (L16 & 3);
  const int q_tr[2] = {QT::off(rq, cq), QT::off(rq + 8, cq)};
  //   dQ products, keys 32ks + 8 g16 + 4ld + L16/4 (ks = 0 .. BC/32-1):
  //   K columns 16 dblk + 4(L16%4):  k_tr[ld] + 32 ks pitch
  //   dS^T slots of queries 16qb + 4(L16%4):  ds_tr[qb][ld] + 2048 ks
  const int rk = 8 * g16 + (L16 >> 2);
  int k_tr[NCB][2];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    k_tr[c][0] = KT::off(rk, dh0 + 16 * (dblk + c) + 4 * (L16 & 3));
    k_tr[c][1] = KT::off(rk + 4, dh0 + 16 * (dblk + c) + 4 * (L16 & 3));
  }
  int ds_tr[NQB][2];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    ds_tr[qb][0] = ds_off(rk, 4 * (qb0 + qb) + (L16 & 3));
    ds_tr[qb][1] = ds_off(rk + 4, 4 * (qb0 + qb) + (L16 & 3));
  }

  // dQ of item `item` from its dS^T (all waves' rows), reduced into dq_acc
  // ordered mode: the semaphores of the dQ tiles whose adds this workgroup
  // issued one item ago (pend_old) and in the current item (pend_sem).  A
  // tile's semaphore is released only once its adds are known to be
  // performed: the wait at the top of item t covers every memory operation
  // issued before item t's copies, so it completes the adds issued two items
  // earlier, and the barrier after it makes that true for every wave.
  int* pend_sem = nullptr;
  int* pend_old = nullptr;
  auto release = [&](int*& sp) {
    if (DET && sp != nullptr) {
      if (tid == 0) __hip_atomic_fetch_add(sp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sp = nullptr;
    }
  };
  auto dq_item = [&](int item, const char* dss) {
    const int hh = item / nsteps;
    const int i = step_tile(item - hh * nsteps);
    const int h = h0 + hh;
    const int q0 = i * BQ;
    f32x4 acc[NCB * NQB];  // [c * NQB + qb]
#pragma unroll
    for (int u = 0; u < NCB * NQB; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    // operands of key step ks+1 are read while step ks's products run
    bf16x8 ob[2][NCB], oa[2][NQB];
    auto load_ks = [&](int ks, bf16x8 (&b)[NCB], bf16x8 (&a)[NQB]) {
      const int ko = 32 * ks * KT::kPitch;
#pragma unroll
      for (int c = 0; c < NCB; ++c)
        b[c] = cat8(ld_lds_tr8(k_s + k_tr[c][0] + ko), ld_lds_tr8(k_s + k_tr[c][1] + ko));
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        a[qb] = cat8(ld_lds_tr8(dss + ds_tr[qb][0] + 2048 * ks),
                     ld_lds_tr8(dss + ds_tr[qb][1] + 2048 * ks));
    };
    if constexpr (NCB == 1) {
      load_ks(0, ob[0], oa[0]);
#pragma unroll
      for (int ks = 0; ks < BC / 32; ++ks) {
        if (ks + 1 < BC / 32) load_ks(ks + 1, ob[(ks + 1) & 1], oa[(ks + 1) & 1]);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          acc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa[ks & 1][qb], ob[ks & 1][0],
                                                            acc[qb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // several column blocks (d = 256): one operand set at a time keeps the
      // register file for the dK, dV accumulators
#pragma unroll
      for (int ks = 0; ks < BC / 32; ++ks) {
        load_ks(ks, ob[0], oa[0]);
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            acc[c * NQB + qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                oa[0][qb], ob[0][c], acc[c * NQB + qb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // acc[c NQB + qb][r] = dQ[q = q0 + 16(qb0 + qb) + 4 g16 + r][d = 16 (dblk + c) + L16]
    if (DQM == kDqPartial) {
      // the tile in fragment order: 4 NQB floats per lane, NQB 16-byte stores
      const long slot = ((long)it.seq * p.Hq + h) * p.head_pairs + pair_index<CAUSAL>(i, it.jt, it.nkv);
      float* dst = p.dq_part + slot * (BQ * D) + ((wave * NQB) * 64 + lane) * 4;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) *reinterpret_cast<f32x4*>(dst + qb * 256) = acc[qb];
      return;
    }
    if (FUSED) {
      // the same tile, stored coherently for the whole device (sc1): another
      // workgroup, possibly on another XCD, sums it once the count says so
      const long slot = ((long)it.seq * p.Hq + h) * p.head_pairs + pair_index<CAUSAL>(i, it.jt, it.nkv);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          p.dq_part + slot * (BQ * D), (short)0, BQ * D * 4, 0x00020000);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        __builtin_amdgcn_raw_buffer_store_b128(as_u32x4(acc[qb]), rs,
                                               (((wave * NQB + qb) * 64 + lane) * 16), 0, kCoherent);
      return;
    }
    // exactly 4 NQB NCB atomic instructions per wave, so the next item can
    // wait for its copies alone: they go through a buffer descriptor whose
    // range ends at the tile's last valid row, and the hardware drops the ones
    // for rows past the sequence end (no traffic, and no pile-up of many
    // workgroups' adds on one clamped address when a sequence has a single
    // query).  Relaxed device-scope adds, performed where every XCD sees them.
    auto issue_atomics = [&]() {
      const int nvalid = min(BQ, it.q_len - q0);
      const float* tile0 = p.dq_acc + ((long)it.q_start + q0) * q_row + (long)h * D;
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(tile0), (short)0, (int)(((nvalid - 1) * q_row + D) * 4), 0x00020000);
      // byte offset of this lane's element in row 16 qb0 + 4 g16 of the tile;
      // rebuilt per item (the empty asm keeps the compiler from holding 4 NQB
      // offsets in registers across the whole loop)
      int vo = ((16 * qb0 + 4 * g16) * (int)q_row + dh0 + dblk * 16 + L16) * 4;
      asm volatile("" : "+v"(vo));
      const int row_bytes = (int)q_row * 4;
      if (FIXED) {
        // round(x 2^e) of row q, added as int32: exact, so the order of the
        // adds does not matter
        const int* ex = ex_s[item % 3];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const i32x4 ev = *reinterpret_cast<const i32x4*>(ex + 16 * (qb0 + qb) + 4 * g16);
#pragma unroll
          for (int c = 0; c < NCB; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              (void)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(
                  __float2int_rn(__builtin_amdgcn_ldexpf(acc[c * NQB + qb][r], ev[r])), rsrc,
                  vo + (16 * qb + r) * row_bytes + 64 * c, 0, 0);
        }
        return;
      }
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            (void)__builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                acc[c * NQB + qb][r], rsrc, vo + (16 * qb + r) * row_bytes + 64 * c, 0, 0);
    };
    if (!DET) {
      issue_atomics();
    } else {
      // ordered reduction: writers of a dQ tile apply in descending key-tile order
      const int jhi = CAUSAL ? min(it.nkv - 1, (q0 + BQ - 1 + it.off) / BC) : it.nkv - 1;
      const int rank = jhi - it.jt;
      long sidx;
      if (VARLEN) sidx = (long)h * p.sem_slots + it.q_start / BQ + it.seq + i;
      else sidx = ((long)it.seq * p.Hq + h) * p.nq + i;
      sidx = sidx * NHALF + chalf;  // each column half has its own order
      int* semp = p.sem + sidx;
      // Wait for our turn.  The semaphore and the dQ accumulator are only ever
      // touched by device-scope atomics, which are performed at the coherence
      // point, so no cache invalidation or write-back is needed: the spin uses
      // relaxed agent-scope loads and the adds below are issued after it.
      if (tid == 0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        uint32_t polls = 0;
        while (__hip_atomic_load(semp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != rank) {
          __builtin_amdgcn_s_sleep(2);
          if ((++polls & 63u) == 0) {
            const uint32_t err = __hip_atomic_load(&p.hdr[kHdrErr], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            if ((err & kErrWaitTimeout) ||
                __builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)p.spin_limit) {
              __hip_atomic_fetch_or(&p.hdr[kHdrErr], kErrWaitTimeout, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
          }
        }
      }
      __syncthreads();
      issue_atomics();
      // released two items later, once these adds are performed (see
      // pend_old).  Deferring cannot create a cycle: a writer only ever
      // waits for writers of higher key tiles, which never wait for it.
      pend_sem = semp;
    }
  };

  auto compute_item = [&](int item, const char* qs, const char* dos, const char* sts,
                          char* dsd) {
    const int hh = item / nsteps;
    const int i = step_tile(item - hh * nsteps);
    const int h = h0 + hh;
    const int q0 = i * BQ;

    if constexpr (KB == 1) {
      const int koff = VARLEN ? it.off : 0;  // causal diagonal offset Lk - Lq
      const bool active = wk0[0] < it.k_len && (!CAUSAL || q0 + BQ - 1 + koff >= wk0[0]);
      if (active) {
        f32x16 s, dp;
#pragma unroll
        for (int x = 0; x < 16; ++x) { s[x] = 0.f; dp[x] = 0.f; }
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
          const int qo = q_rd[dc & 1] + 64 * (dc >> 1);
          const bf16x8 aq = as_bf16x8(ld_lds16(qs + qo));
          const bf16x8 bk = as_bf16x8(ld_lds16(k_s + k_rd[0][dc & 1] + 64 * (dc >> 1)));
          const bf16x8 ado = as_bf16x8(ld_lds16(dos + qo));
          s = mfma32x32x16(aq, bk, s);
          dp = mfma32x32x16(ado, vf[0][dc], dp);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the phases apart: bounds register pressure
        // s[x] = S[q = q0 + 8(x/4) + 4 half + x%4][key = mykey]
        const float* lse_s = reinterpret_cast<const float*>(sts);
        const float* dv_s = lse_s + BQ;
        const bool need_mask = (CAUSAL && q0 + koff < wk0[0] + 31) || (wk0[0] + 32 > it.k_len) ||
                               (q0 + BQ > it.q_len);
        // P = exp2(S c - LSE log2 e), dS = P o (dP - D); with a causal mask the
        // masked copy runs on diagonal and ragged tiles only (a uniform branch)
        auto softmax_grad = [&](auto masked) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + 8 * g + 4 * half);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(dv_s + 8 * g + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int x = 4 * g + e;
              float pr = fast_exp2(fmaf(s[x], p.c, -l4[e]));
              if (decltype(masked)::value) {
                const int q = q0 + 8 * g + 4 * half + e;
                if (!key_ok[0] || q >= it.q_len || (CAUSAL && mykey[0] > q + koff)) pr = 0.f;
              }
              s[x] = pr;
              dp[x] = pr * (dp[x] - d4[e]);
            }
          }
        };
        if (CAUSAL && !need_mask) softmax_grad(std::false_type{});
        else softmax_grad(std::true_type{});
        bf16x8 pa[2], dsa[2];
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) {
          pa[qc] = frag_rows(s, qc);
          dsa[qc] = frag_rows(dp, qc);
        }
        // dV += P^T dO and dK += dS^T Q over two 16-query chunks; the B operands
        // are transposed reads of the row-major dO / Q tiles, rows
        // 16qc + 8ld + 4half + 0..3 matching the registers of P and dS
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) {
#pragma unroll
          for (int db = 0; db < DH / 32; ++db) {
            const int o0 = q_tr[0] + 16 * qc * QT::kPitch + 2 * dh0 + 64 * db;
            const int o1 = q_tr[1] + 16 * qc * QT::kPitch + 2 * dh0 + 64 * db;
            const bf16x8 bdo = cat8(ld_lds_tr8(dos + o0), ld_lds_tr8(dos + o1));
            const bf16x8 bq = cat8(ld_lds_tr8(qs + o0), ld_lds_tr8(qs + o1));
            dv_acc[0][db] = mfma32x32x16(pa[qc], bdo, dv_acc[0][db]);
            dk_acc[0][db] = mfma32x32x16(dsa[qc], bq, dk_acc[0][db]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // dS^T (bf16) rows of this wave's keys: the 4 consecutive queries of
        // register group g are words 2(g%2), 2(g%2)+1 of dsa[g/2]
        const int krow = wave * 32 + l32;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4 w4 = as_u32x4(dsa[g >> 1]);
          const u32x2 w = (g & 1) ? u32x2{w4[2], w4[3]} : u32x2{w4[0], w4[1]};
          st_lds8(dsd + ds_off(krow, 2 * g + half), w);
        }
      } else {
        const int krow = wave * 32 + l32;
        const u32x2 z = {0u, 0u};
#pragma unroll
        for (int g = 0; g < 4; ++g) st_lds8(dsd + ds_off(krow, 2 * g + half), z);
      }
    } else {
      const int koff = VARLEN ? it.off : 0;  // causal diagonal offset Lk - Lq
      // a block whose keys all lie past the sequence end or (causal) after
      // every query of the tile contributes nothing; with several blocks per
      // wave the products still run for all of them when any is active (the
      // mask then zeroes the inactive ones)
      bool active = false;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        active |= wk0[kb] < it.k_len && (!CAUSAL || q0 + BQ - 1 + koff >= wk0[kb]);
      if (active) {
        f32x16 s[KB], dp[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int x = 0; x < 16; ++x) { s[kb][x] = 0.f; dp[kb][x] = 0.f; }
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) {
          const int qo = q_rd[dc & 1] + 64 * (dc >> 1);
          const bf16x8 aq = as_bf16x8(ld_lds16(qs + qo));
          const bf16x8 ado = as_bf16x8(ld_lds16(dos + qo));
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const bf16x8 bk = as_bf16x8(ld_lds16(k_s + k_rd[kb][dc & 1] + 64 * (dc >> 1)));
            s[kb] = mfma32x32x16(aq, bk, s[kb]);
            dp[kb] = mfma32x32x16(ado, vf[kb][dc], dp[kb]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the phases apart: bounds register pressure
        // s[kb][x] = S[q = q0 + 8(x/4) + 4 half + x%4][key = mykey[kb]]
        const float* lse_s = reinterpret_cast<const float*>(sts);
        const float* dv_s = lse_s + BQ;
        // P = exp2(S c - LSE log2 e), dS = P o (dP - D); with a causal mask the
        // masked copy runs on diagonal and ragged tiles only (a uniform branch)
        auto softmax_grad = [&](auto masked, f32x16& sk, f32x16& dpk, int mk,
                                bool kok) __attribute__((always_inline)) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + 8 * g + 4 * half);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(dv_s + 8 * g + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int x = 4 * g + e;
              float pr = fast_exp2(fmaf(sk[x], p.c, -l4[e]));
              if (decltype(masked)::value) {
                const int q = q0 + 8 * g + 4 * half + e;
                if (!kok || q >= it.q_len || (CAUSAL && mk > q + koff)) pr = 0.f;
              }
              sk[x] = pr;
              dpk[x] = pr * (dpk[x] - d4[e]);
            }
          }
        };
        bf16x8 pa[KB][2], dsa[KB][2];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bool need_mask = (CAUSAL && q0 + koff < wk0[kb] + 31) || (wk0[kb] + 32 > it.k_len) ||
                                 (q0 + BQ > it.q_len);
          if (CAUSAL && !need_mask)
            softmax_grad(std::false_type{}, s[kb], dp[kb], mykey[kb], key_ok[kb]);
          else
            softmax_grad(std::true_type{}, s[kb], dp[kb], mykey[kb], key_ok[kb]);
#pragma unroll
          for (int qc = 0; qc < 2; ++qc) {
            pa[kb][qc] = frag_rows(s[kb], qc);
            dsa[kb][qc] = frag_rows(dp[kb], qc);
          }
        }
        // dV += P^T dO and dK += dS^T Q over two 16-query chunks; the B operands
        // are transposed reads of the row-major dO / Q tiles, rows
        // 16qc + 8ld + 4half + 0..3 matching the registers of P and dS, shared
        // by the key blocks
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) {
#pragma unroll
          for (int db = 0; db < DH / 32; ++db) {
            const int o0 = q_tr[0] + 16 * qc * QT::kPitch + 2 * dh0 + 64 * db;
            const int o1 = q_tr[1] + 16 * qc * QT::kPitch + 2 * dh0 + 64 * db;
            const bf16x8 bdo = cat8(ld_lds_tr8(dos + o0), ld_lds_tr8(dos + o1));
            const bf16x8 bq = cat8(ld_lds_tr8(qs + o0), ld_lds_tr8(qs + o1));
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              dv_acc[kb][db] = mfma32x32x16(pa[kb][qc], bdo, dv_acc[kb][db]);
              dk_acc[kb][db] = mfma32x32x16(dsa[kb][qc], bq, dk_acc[kb][db]);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // dS^T (bf16) rows of this wave's keys: the 4 consecutive queries of
        // register group g are words 2(g%2), 2(g%2)+1 of dsa[kb][g/2]
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int krow = krow0[kb] + l32;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const u32x4 w4 = as_u32x4(dsa[kb][g >> 1]);
            const u32x2 w = (g & 1) ? u32x2{w4[2], w4[3]} : u32x2{w4[0], w4[1]};
            st_lds8(dsd + ds_off(krow, 2 * g + half), w);
          }
        }
      } else {
        const u32x2 z = {0u, 0u};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int krow = krow0[kb] + l32;
#pragma unroll
          for (int g = 0; g < 4; ++g) st_lds8(dsd + ds_off(krow, 2 * g + half), z);
        }
      }
    }
  };

  // Fused mode.  count_item (thread 0): the partial tile of `item` is stored
  // by every wave; one relaxed device atomic counts it in, and the workgroup
  // that brings the count to the query tile's number of key tiles finishes
  // that tile.  reduce_item (all threads): sum of the partial tiles in
  // ascending key-tile order (coherent loads), times the scale, into bf16 dQ.
  auto count_item = [&](int item) {
    const int hh = item / nsteps;
    const int i = step_tile(item - hh * nsteps);
    const int h = h0 + hh;
    const int jn = CAUSAL ? min(it.nkv, (i * BQ + BQ - 1) / BC + 1) : it.nkv;
    const int old = __hip_atomic_fetch_add(p.sem + ((long)it.seq * p.Hq + h) * p.nq + i, 1,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_last[item & 3] = old == jn - 1;
  };
  auto reduce_item = [&](int item) {
    const int hh = item / nsteps;
    const int i = step_tile(item - hh * nsteps);
    const int h = h0 + hh;
    const int jn = CAUSAL ? min(it.nkv, (i * BQ + BQ - 1) / BC + 1) : it.nkv;
    constexpr int F = BQ * D;                  // floats per partial tile
    constexpr int V = F / (4 * NT);            // 16-byte pieces per thread per tile
    const long slot0 = ((long)it.seq * p.Hq + h) * p.head_pairs + pair_index<CAUSAL>(i, 0, it.nkv);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        p.dq_part + slot0 * F, (short)0, jn * F * 4, 0x00020000);
    f32x4 acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    int j = 0;
    for (; j + 4 <= jn; j += 4) {
      f32x4 x[4][V];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < V; ++v)
          x[u][v] = as_f32x4(__builtin_amdgcn_raw_buffer_load_b128(
              rs, ((j + u) * F + 4 * (tid + NT * v)) * 4, 0, kCoherent));
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] += x[u][v];
    }
    for (; j < jn; ++j)
#pragma unroll
      for (int v = 0; v < V; ++v)
        acc[v] += as_f32x4(__builtin_amdgcn_raw_buffer_load_b128(
            rs, (j * F + 4 * (tid + NT * v)) * 4, 0, kCoherent));
    // fragment order: float4 f4 = (w NQB + qb) 64 + lane holds rows
    // 16 ((w / DB16) NQB + qb) + 4 (lane / 16) + 0..3 of column 16 (w % DB16) + lane % 16
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int f4 = tid + NT * v;
      const int ln = f4 & 63, wq = f4 >> 6;
      const int w = wq / NQB, qb = wq - (wq / NQB) * NQB;
      const int row0 = 16 * ((w / DB16) * NQB + qb) + 4 * (ln >> 4);
      const int col = 16 * (w % DB16) + (ln & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = i * BQ + row0 + r;
        if (q < it.q_len)
          p.dq[((long)it.q_start + q) * q_row + (long)h * D + col] = (bf16)(acc[v][r] * p.scale);
      }
    }
  };

  // Per item: one barrier (the item's copies landed and the previous item's
  // dS^T is complete), then the previous item's dQ products and atomics,
  // then this item's S, dP, dV, dK and its dS^T (into the other buffer).
  // Before an item is computed its copies must have landed; only the atomics
  // or stores of the dQ issued in the previous item (4 NQB or NQB per wave)
  // were issued after them, so those stay in flight.
  auto wait_copies = [&](int item) {
    if ((DQM == kDqAtomic || DET || FIXED) && item >= 2) wait_vmem_leave<4 * NQB * NCB>();
    else if (PARTS && item >= 2) wait_vmem_leave<NQB>();
    else wait_vmem();
    lds_barrier();
  };
  // two-stage pipeline over the work items: item t+1's rows are copied into
  // the other buffer while item t is computed
  if (nitems > 0) issue_item(0, q_s0, do_s0, st_s0);
  for (int item = 0; item < nitems; ++item) {
    wait_copies(item);
    if (DET) {
      release(pend_old);  // its adds were issued before this item's copies
      pend_old = pend_sem;
      pend_sem = nullptr;
    }
    if (FUSED) {
      // the partial tile of item-3 is complete in every wave (its stores
      // were issued before copies this wait covered); item-4 was counted
      // before this barrier
      if (item >= 4 && sh_last[item & 3]) reduce_item(item - 4);
      if (item >= 3 && tid == 0) count_item(item - 3);
    }
    const bool odd = item & 1;
    char* qs = odd ? q_s1 : q_s0;
    char* dos = odd ? do_s1 : do_s0;
    char* sts = odd ? st_s1 : st_s0;
    if (item + 1 < nitems) issue_item(item + 1, odd ? q_s0 : q_s1, odd ? do_s0 : do_s1,
                                      odd ? st_s0 : st_s1);
    if (item >= 1) dq_item(item - 1, odd ? ds_s0 : ds_s1);
    __builtin_amdgcn_sched_barrier(0);
    compute_item(item, qs, dos, sts, odd ? ds_s1 : ds_s0);
  }
  if (nitems > 0) {
    if (DET) wait_vmem();  // every add issued so far is performed ...
    lds_barrier();         // ... in every wave; the last item's dS^T is complete
    release(pend_old);
    release(pend_sem);
    dq_item(nitems - 1, (nitems - 1) & 1 ? ds_s1 : ds_s0);
    if (DET) {
      wait_vmem();
      __syncthreads();
      release(pend_sem);
    }
  }
  if (FUSED && nitems > 0) {
    wait_vmem();    // every partial tile of this workgroup is stored
    lds_barrier();  // ... by every wave; item nitems-4 was counted
    const int t0 = max(0, nitems - 4);
    if (nitems >= 4 && sh_last[t0 & 3]) reduce_item(t0);
    __syncthreads();  // sh_last[t0 & 3] is reused below
    if (tid == 0)
      for (int t = max(0, nitems - 3); t < nitems; ++t) count_item(t);
    __syncthreads();
    for (int t = max(0, nitems - 3); t < nitems; ++t)
      if (sh_last[t & 3]) reduce_item(t);
  }

  // ---------------- dK = scale * sum dS^T Q, dV = sum P^T dO for this wave's keys
  // dk_acc[kb][db][x] = dK[key = wk0[kb] + 8(x/4) + 4 half + x%4][d = dh0 + 32 db + l32]
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int key = wk0[kb] + 8 * (x >> 2) + 4 * half + (x & 3);
        if (key < it.k_len) {
          const long off =
              ((long)it.k_start + key) * kv_row + (long)it.hkv * D + dh0 + db * 32 + l32;
          if (p.S == 1) {
            p.dk[off] = (bf16)(dk_acc[kb][db][x] * p.scale);
            p.dv[off] = (bf16)(dv_acc[kb][db][x]);
          } else {
            const long po = (long)it.split * p.Tk * kv_row + off;
            p.dk_part[po] = dk_acc[kb][db][x] * p.scale;
            p.dv_part[po] = dv_acc[kb][db][x];
          }
        }
      }
}

template <int D, bool CAUSAL, bool VARLEN, int DQM>
hipError_t launch_bwd_t(const BwdParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_kernel<D, CAUSAL, VARLEN, DQM>), dim3(grid), dim3(bwd_threads(D)), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_bwd_mode(const BwdParams& p, int mode, int grid, hipStream_t stream) {
  if (mode == kDqOrdered) return launch_bwd_t<D, CAUSAL, VARLEN, kDqOrdered>(p, grid, stream);
  if (mode == kDqFixed) return launch_bwd_t<D, CAUSAL, VARLEN, kDqFixed>(p, grid, stream);
  if constexpr (D != 256 && bwd_key_blocks(D) == 1) {  // partial tiles: 32 keys per wave
    if (mode == kDqPartial && !VARLEN)
      return launch_bwd_t<D, CAUSAL, false, kDqPartial>(p, grid, stream);
    if (mode == kDqFused && !VARLEN)
      return launch_bwd_t<D, CAUSAL, false, kDqFused>(p, grid, stream);
  }
  return launch_bwd_t<D, CAUSAL, VARLEN, kDqAtomic>(p, grid, stream);
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, bool causal, bool varlen, int mode, int grid,
                        hipStream_t stream) {
  if (causal) return varlen ? launch_bwd_mode<D, true, true>(p, mode, grid, stream)
                            : launch_bwd_mode<D, true, false>(p, mode, grid, stream);
  return varlen ? launch_bwd_mode<D, false, true>(p, mode, grid, stream)
                : launch_bwd_mode<D, false, false>(p, mode, grid, stream);
}

// ---------------------------------------------------------------------------
// preprocess: D = rowsum(dO o O); zero dQ_acc, semaphores, header

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* o, const bf16* dout,
                                                      const float* lse, float* dvec, float* lse2,
                                                      float* dq_acc, int* sem, long sem_count,
                                                      uint32_t* hdr, int rows, int Hq, bool varlen,
                                                      int N, int T, const float* kvb, int G,
                                                      int* dq_exp) {
  constexpr int EPT = D / 16;  // elements per thread (16 threads per row)
  // a block takes 16 consecutive tokens of one query head, so that its D
  // and LSE values are 16 consecutive floats of their [b, h, n] arrays
  const int h = blockIdx.x % Hq;
  const int tok = (blockIdx.x / Hq) * 16 + (threadIdx.x >> 4);
  const int row = tok * Hq + h;
  const int sub = threadIdx.x & 15;
  if (blockIdx.x == 0 && threadIdx.x < kHdrWords) hdr[threadIdx.x] = 0u;
  for (long s = (long)blockIdx.x * 256 + threadIdx.x; s < sem_count; s += (long)gridDim.x * 256)
    sem[s] = 0;
  if (tok >= rows / Hq) return;
  const long base = (long)row * D + sub * EPT;
  float acc = 0.f, nrm = 0.f;  // D and |dO|^2 of the row
  if (EPT == 8) {
    const u32x4 a = ld_global16(o + base), b = ld_global16(dout + base);
    const bf16x8 x = as_bf16x8(a), y = as_bf16x8(b);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc = fmaf((float)x[e], (float)y[e], acc);
      nrm = fmaf((float)y[e], (float)y[e], nrm);
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      acc = fmaf((float)o[base + e], (float)dout[base + e], acc);
      nrm = fmaf((float)dout[base + e], (float)dout[base + e], nrm);
    }
  }
  acc += __shfl_xor(acc, 8, 16);
  acc += __shfl_xor(acc, 4, 16);
  acc += __shfl_xor(acc, 2, 16);
  acc += __shfl_xor(acc, 1, 16);
  if (dq_exp) {
    nrm += __shfl_xor(nrm, 8, 16);
    nrm += __shfl_xor(nrm, 4, 16);
    nrm += __shfl_xor(nrm, 2, 16);
    nrm += __shfl_xor(nrm, 1, 16);
    // beta = |dO| max|K| max|V| bounds every element of the row's unscaled
    // dQ, and every partial sum of it over a subset of the keys:
    // |sum_j P_j (dP_j - D) K_jc| <= max|K| sum_j P_j |dP_j - D|, the mean
    // absolute deviation of dP_j = dO . V_j under the weights P_j around their
    // mean D, which is at most their standard deviation, which is at most half
    // their range (Popoviciu), <= |dO| max|V|.  beta < 2^k, so the sums stay
    // below 2^29 steps of 2^(k - 29), with 4x headroom in int32 for the
    // rounding of P, D and dS.
    const int ex = dq_fixed_exponent(sqrtf(nrm) * kvb[h / G]);
    if (sub == 0) dq_exp[row] = ex;
  }
  if (dq_acc) {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < EPT; e += 4) *reinterpret_cast<f32x4*>(dq_acc + base + e) = z;
  }
  if (sub == 0) {
    long idx;
    if (varlen) idx = (long)h * T + tok;
    else {
      const int b = tok / N, n = tok - b * N;
      idx = ((long)b * Hq + h) * N + n;
    }
    dvec[idx] = acc;
    // a row that saw no key (LSE = -inf) gets +inf, so P = exp2(S c - LSE2) = 0
    const float l = lse[idx];
    lse2[idx] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// fixed-point dQ: the K/V magnitudes of each key/value head.  Partial maxima
// per kKvBoundRows key rows (largest |K| element, largest squared V row norm),
// then one workgroup per head combines them.  NaN propagates through both
// maxima (a NaN input gives a non-finite bound, hence NaN dQ rows).
__device__ __forceinline__ float max_nan(float a, float b) { return (a > b || a != a) ? a : b; }

template <int D>
__global__ __launch_bounds__(256) void bwd_kv_bound_kernel(const bf16* k, const bf16* v,
                                                           float* part, long Tk, int Hkv,
                                                           int nchunk) {
  constexpr int TPR = D / 8;      // threads per key row, 8 elements each
  constexpr int RPP = 256 / TPR;  // rows per pass
  __shared__ float red[2][4];
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int sub = threadIdx.x % TPR;
  float km = 0.f, vm = 0.f;
  for (int r = threadIdx.x / TPR; r < kKvBoundRows; r += RPP) {
    const long row = (long)chunk * kKvBoundRows + r;
    float ss = 0.f;
    if (row < Tk) {
      const long base = (row * Hkv + g) * D + sub * 8;
      const bf16x8 a = as_bf16x8(ld_global16(k + base)), b = as_bf16x8(ld_global16(v + base));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        km = max_nan(fabsf((float)a[e]), km);
        ss = fmaf((float)b[e], (float)b[e], ss);
      }
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, TPR);
    vm = max_nan(ss, vm);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    km = max_nan(__shfl_xor(km, m), km);
    vm = max_nan(__shfl_xor(vm, m), vm);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = km;
    red[1][wave] = vm;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) {
      km = max_nan(red[0][w], km);
      vm = max_nan(red[1][w], vm);
    }
    part[2 * ((long)g * nchunk + chunk)] = km;
    part[2 * ((long)g * nchunk + chunk) + 1] = sqrtf(vm);
  }
}

__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(const float* part, float* kvb,
                                                            int nchunk) {
  __shared__ float red[2][4];
  const int g = blockIdx.x;
  float km = 0.f, vm = 0.f;
  for (int c = threadIdx.x; c < nchunk; c += 256) {
    km = max_nan(part[2 * ((long)g * nchunk + c)], km);
    vm = max_nan(part[2 * ((long)g * nchunk + c) + 1], vm);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    km = max_nan(__shfl_xor(km, m), km);
    vm = max_nan(__shfl_xor(vm, m), vm);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = km;
    red[1][wave] = vm;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) {
      km = max_nan(red[0][w], km);
      vm = max_nan(red[1][w], vm);
    }
    kvb[g] = km * vm;
  }
}

__global__ __launch_bounds__(256) void bwd_post_kernel(const float* dq_acc, bf16* dq, long dq_vec,
                                                       float scale, const float* dk_part,
                                                       const float* dv_part, bf16* dk, bf16* dv,
                                                       long kv_vec, int S, const int* dq_exp,
                                                       int row_vec_shift) {
  // every element handled in groups of 4 (all sizes are multiples of 64)
  const long stride = (long)gridDim.x * 256;
  for (long v = (long)blockIdx.x * 256 + threadIdx.x; v < dq_vec; v += stride) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(dq_acc + 4 * v);
    f32x4 a;
    if (dq_exp) {
      // int32 fixed point of row v / (d / 4), in units of 2^-e
      const int ex = dq_exp[v >> row_vec_shift];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        a[e] = ex == kDqExpNonFinite ? __builtin_nanf("")
                                     : __builtin_amdgcn_ldexpf((float)(int)raw[e], -ex);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = __uint_as_float(raw[e]);
    }
    u32x2 w;
    w[0] = pack2_bf16(a[0] * scale, a[1] * scale);
    w[1] = pack2_bf16(a[2] * scale, a[3] * scale);
    *reinterpret_cast<u32x2*>(dq + 4 * v) = w;
  }
  if (S > 1) {
    const long kv_elems = kv_vec * 4;
    for (long v = (long)blockIdx.x * 256 + threadIdx.x; v < kv_vec; v += stride) {
      f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < S; ++s) {  // fixed order: deterministic
        sk += *reinterpret_cast<const f32x4*>(dk_part + s * kv_elems + 4 * v);
        sv += *reinterpret_cast<const f32x4*>(dv_part + s * kv_elems + 4 * v);
      }
      u32x2 wk, wv;
      wk[0] = pack2_bf16(sk[0], sk[1]);
      wk[1] = pack2_bf16(sk[2], sk[3]);
      wv[0] = pack2_bf16(sv[0], sv[1]);
      wv[1] = pack2_bf16(sv[2], sv[3]);
      *reinterpret_cast<u32x2*>(dk + 4 * v) = wk;
      *reinterpret_cast<u32x2*>(dv + 4 * v) = wv;
    }
  }
}

// ---------------------------------------------------------------------------
// partial-sum mode: dQ tile (b, h, i) = scale * sum over its key tiles j of the
// partial tiles, added in ascending j (a fixed order), then stored as bf16.
// One workgroup per query tile; the partial tiles are in the fragment order
// of the dQ products (16x16 blocks: wave w owns columns 16 (w % (D/16)) ..
// and row blocks NQB (w / (D/16)) .. of the tile).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(const float* part, bf16* dq, int N,
                                                            int Hq, int nq, int nkv,
                                                            long head_pairs, float scale) {
  constexpr int F = BQ * D;       // floats per tile
  constexpr int V = F / 1024;     // float4 per thread
  constexpr int DB16 = D / 16;
  constexpr int NQB = (2 * DB16) / NW;
  constexpr int PITCH = D + 4;    // LDS row pitch in floats
  __shared__ float tile[BQ * PITCH];
  const int t = threadIdx.x;
  // heaviest query tiles (most key tiles) first, every head's at once
  const int nbh = gridDim.x / nq;
  const int i = CAUSAL ? nq - 1 - (int)(blockIdx.x / nbh) : (int)(blockIdx.x / nbh);
  const int bh = blockIdx.x % nbh;  // b * Hq + h
  const int jn = CAUSAL ? i / (BC / BQ) + 1 : nkv;
  const float* src = part + ((long)bh * head_pairs + pair_index<CAUSAL>(i, 0, nkv)) * F;
  f32x4 acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  // four partial tiles per step: 4 V independent 16-byte loads in flight
  // per thread, added in ascending j afterwards (the order never changes)
  int j = 0;
  for (; j + 4 <= jn; j += 4) {
    f32x4 x[4][V];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < V; ++v)
        x[u][v] = *reinterpret_cast<const f32x4*>(src + (long)(j + u) * F + 4 * (t + 256 * v));
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] += x[u][v];
  }
  for (; j < jn; ++j) {
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] += *reinterpret_cast<const f32x4*>(src + (long)j * F + 4 * (t + 256 * v));
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int f4 = t + 256 * v;          // (wave * NQB + qb) * 64 + lane
    const int lane = f4 & 63, wq = f4 >> 6;
    const int w = wq / NQB, qb = wq % NQB;
    const int row0 = 16 * ((w / DB16) * NQB + qb) + 4 * (lane >> 4);
    const int col = 16 * (w % DB16) + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) tile[(row0 + r) * PITCH + col] = acc[v][r];
  }
  __syncthreads();
  // thread t writes 16 consecutive elements (D = 128) or 8 (D = 64) of one row
  constexpr int EPT = F / 256;
  const int row = t / (D / EPT), c0 = (t % (D / EPT)) * EPT;
  const int b = bh / Hq, h = bh % Hq;
  const int q = i * BQ + row;
  if (q >= N) return;
  bf16* out = dq + (((long)b * N + q) * Hq + h) * D + c0;
#pragma unroll
  for (int e = 0; e < EPT; e += 8) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = pack2_bf16(tile[row * PITCH + c0 + e + 2 * k] * scale,
                        tile[row * PITCH + c0 + e + 2 * k + 1] * scale);
    *reinterpret_cast<u32x4*>(out + e) = w;
  }
}

// ---------------------------------------------------------------------------
// Measurement aid: the atomic dQ reduction of bwd_kernel (d = 128) without
// its products.  Workgroup w of 8 waves, at step t, takes the 32-row x 128-
// column tile ((w + t * gridDim.x) mod tiles) of a [rows, row_floats] fp32
// buffer; wave v adds its 32 x 16 column block with the 8 buffer atomic
// instructions (4 rows x 16 columns each) the backward issues per item, or
// (KIND 1) writes the same bytes with plain stores, or (KIND 2) adds the
// int32 1 with the fixed-point mode's int32 atomics.
template <int KIND>
__global__ __launch_bounds__(512) void probe_dq_kernel(float* buf, int rows, int row_floats,
                                                        int items) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int g16 = lane >> 4, L16 = lane & 15;
  const int heads = row_floats / 128;
  const long tiles = (long)(rows / 32) * heads;
  const float val = 1.0f / 1024.0f;
  for (int t = 0; t < items; ++t) {
    const long tile = ((long)blockIdx.x + (long)t * gridDim.x) % tiles;
    const int i = (int)(tile / heads), h = (int)(tile - (long)(tile / heads) * heads);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        buf + (long)i * 32 * row_floats + h * 128, (short)0, (31 * row_floats + 128) * 4,
        0x00020000);
    const int vo = ((4 * g16) * row_floats + wave * 16 + L16) * 4;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int off = vo + (16 * qb + r) * row_floats * 4;
        if (KIND == 1)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), rsrc, off, 0, 0);
        else if (KIND == 2)
          (void)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, rsrc, off, 0, 0);
        else
          (void)__builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(val, rsrc, off, 0, 0);
      }
  }
}

}  // namespace

hipError_t launch_probe_dq(float* buf, int rows, int row_floats, int blocks, int items, int kind,
                           hipStream_t stream) {
  if (kind == 1)
    hipLaunchKernelGGL(probe_dq_kernel<1>, dim3(blocks), dim3(512), 0, stream, buf, rows,
                       row_floats, items);
  else if (kind == 2)
    hipLaunchKernelGGL(probe_dq_kernel<2>, dim3(blocks), dim3(512), 0, stream, buf, rows,
                       row_floats, items);
  else
    hipLaunchKernelGGL(probe_dq_kernel<0>, dim3(blocks), dim3(512), 0, stream, buf, rows,
                       row_floats, items);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int d, bool causal, bool varlen, int mode, int grid,
                      hipStream_t stream) {
  if (d == 256) return launch_bwd_d<256>(p, causal, varlen, mode, grid, stream);
  if (d == 128) return launch_bwd_d<128>(p, causal, varlen, mode, grid, stream);
  return launch_bwd_d<64>(p, causal, varlen, mode, grid, stream);
}

template <int D, bool CAUSAL>
void launch_reduce_t(const float* part, bf16* dq, int N, int Hq, int nq, int nkv,
                     long head_pairs, float scale, long grid, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_dq_reduce_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0,
                     stream, part, dq, N, Hq, nq, nkv, head_pairs, scale);
}

hipError_t launch_bwd_dq_reduce(const float* part, bf16* dq, int B, int N, int Hq, int d,
                                bool causal, int nq, int nkv, long head_pairs, float scale,
                                hipStream_t stream) {
  const long grid = (long)B * Hq * nq;
  if (grid <= 0) return hipSuccess;
  if (d == 128) {
    if (causal) launch_reduce_t<128, true>(part, dq, N, Hq, nq, nkv, head_pairs, scale, grid, stream);
    else launch_reduce_t<128, false>(part, dq, N, Hq, nq, nkv, head_pairs, scale, grid, stream);
  } else {
    if (causal) launch_reduce_t<64, true>(part, dq, N, Hq, nq, nkv, head_pairs, scale, grid, stream);
    else launch_reduce_t<64, false>(part, dq, N, Hq, nq, nkv, head_pairs, scale, grid, stream);
  }
  return hipGetLastError();
}

bool bwd_partial_modes(int d) { return d != 256 && bwd_key_blocks(d) == 1; }

long bwd_partial_pairs(int N, bool causal) {
  const int nq = (N + kBwdBQ - 1) / kBwdBQ, nkv = (N + kBwdBC - 1) / kBwdBC;
  if (!causal) return (long)nq * nkv;
  const long a = nq / (kBwdBC / kBwdBQ), r = nq % (kBwdBC / kBwdBQ);
  return (a + 1) * ((kBwdBC / kBwdBQ) / 2 * a + r);
}

hipError_t launch_bwd_pre(const bf16* o, const bf16* dout, const float* lse, float* dvec,
                          float* lse2, float* dq_acc, int* sem, long sem_count, uint32_t* hdr,
                          int rows, int Hq, int d, bool varlen, int N, int T, const float* kvb,
                          int G, int* dq_exp, hipStream_t stream) {
  const int grid = max(1, Hq * ((rows / Hq + 15) / 16));
  if (d == 256)
    hipLaunchKernelGGL(bwd_pre_kernel<256>, dim3(grid), dim3(256), 0, stream, o, dout, lse, dvec,
                       lse2, dq_acc, sem, sem_count, hdr, rows, Hq, varlen, N, T, kvb, G, dq_exp);
  else if (d == 128)
    hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3(grid), dim3(256), 0, stream, o, dout, lse, dvec,
                       lse2, dq_acc, sem, sem_count, hdr, rows, Hq, varlen, N, T, kvb, G, dq_exp);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3(grid), dim3(256), 0, stream, o, dout, lse, dvec,
                       lse2, dq_acc, sem, sem_count, hdr, rows, Hq, varlen, N, T, kvb, G, dq_exp);
  return hipGetLastError();
}

hipError_t launch_bwd_kv_bound(const bf16* k, const bf16* v, float* part, float* kvb, long Tk,
                               int Hkv, int d, hipStream_t stream) {
  const int nchunk = (int)((Tk + kKvBoundRows - 1) / kKvBoundRows);
  if (nchunk > 0) {
    const dim3 grid(nchunk, Hkv);
    if (d == 256)
      hipLaunchKernelGGL(bwd_kv_bound_kernel<256>, grid, dim3(256), 0, stream, k, v, part, Tk,
                         Hkv, nchunk);
    else if (d == 128)
      hipLaunchKernelGGL(bwd_kv_bound_kernel<128>, grid, dim3(256), 0, stream, k, v, part, Tk,
                         Hkv, nchunk);
    else
      hipLaunchKernelGGL(bwd_kv_bound_kernel<64>, grid, dim3(256), 0, stream, k, v, part, Tk,
                         Hkv, nchunk);
  }
  hipLaunchKernelGGL(bwd_kv_reduce_kernel, dim3(Hkv), dim3(256), 0, stream, part, kvb, nchunk);
  return hipGetLastError();
}

hipError_t launch_bwd_post(const float* dq_acc, bf16* dq, long dq_elems, float scale,
                           const float* dk_part, const float* dv_part, bf16* dk, bf16* dv,
                           long kv_elems, int S, const int* dq_exp, int d, hipStream_t stream) {
  const long vec = dq_elems / 4;
  const long work = max(vec, S > 1 ? kv_elems / 4 : 0L);
  const long blocks = min(4096L, max(1L, (work + 255) / 256));
  const int row_vec_shift = d == 256 ? 6 : (d == 128 ? 5 : 4);  // log2(d / 4)
  hipLaunchKernelGGL(bwd_post_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dq_acc, dq,
                     vec, scale, dk_part, dv_part, dk, dv, kv_elems / 4, S, dq_exp,
                     row_vec_shift);
  return hipGetLastError();
}

}  // namespace fa
