// fa_fwd.hip -- fused attention forward for gfx950.
//
// Method ([FA2] "Core method" 1-3, [FA4N] co-design list):
//  * one workgroup per (sequence, query head, query tile of BR = 32*NW rows);
//    the tiles are independent, so the output never depends on launch order
//    (a split tile's key chunks are merged in a fixed order afterwards);
//  * split-Q: wave w owns query rows 32w..32w+31 of the tile and sees every
//    key/value tile, so no reduction between waves is ever needed;
//  * K and V tiles of 64 keys are copied global->LDS by direct loads (no
//    register staging) into padded tiles, through a ring of fwd_stages(D)
//    buffers (4; 2 for d = 256, whose tiles are twice as large): the next
//    tiles are in flight while tile j is computed; with 8 waves the first
//    four issue all copies: with the 4-deep ring after their own products
//    of a tile (they run ahead of their SIMD partners, which are the
//    critical path), with the 2-deep ring right after the barrier;
//  * a tile's K operands (and the first V^T operands) are read into
//    registers in one batch before its products;
//  * the score tile is computed transposed, S^T = K Q^T, so each lane holds one
//    query column: the row max and row sum are in-lane plus one exchange
//    between lane halves;
//  * online softmax in base 2 with conditional rescaling: a stale reference max
//    is kept and the accumulator is rescaled only when a row max grows by more
//    than kTau (log2 units), decided per wave; probabilities therefore stay
//    below 2^kTau and the result is unchanged;
//  * the unscaled output accumulator O^T += V^T P^T stays in registers (V^T is
//    read from the row-major V tile with transposed LDS reads, in the key
//    order the P fragment already has) and is divided by the row sum once at
//    the end; only LSE = ln(sum exp) is saved;
//  * causal: key tiles wholly above a wave's rows are skipped (as are all
//    tiles for a wave whose rows lie past the sequence end), the mask is
//    applied only on tiles that straddle the diagonal or the sequence end;
//    a packed sequence with Lq queries and Lk keys aligns the diagonal
//    bottom-right (query i sees key j iff j <= i + Lk - Lq, the decode-shaped
//    batches of [FA4B] 3.3.2), and a query that sees no key gets O = 0 and
//    LSE = -inf;
//  * fp8 scores (template flag FP8; [FA2] "Limitations and future
//    work", [FA4C] 5.1): Q and K arrive as OCP e4m3 bytes, the K tile is
//    copied as bytes, S^T takes d/64 fp8 32x32x64 products per 32 keys, and
//    the descale factors of Q and K are folded into the exponent scale c;
//    P, V and the P V product stay bf16.
#include "fa_common.h"
#include "fa_exp2.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kBC = 64;        // keys per K/V tile
// Rescale threshold in log2 units (probabilities stay <= 2^kTau).  The
// result does not depend on it; a build with FA_RESCALE_TAU=0 rescales on
// every growth of a row maximum, which the tests compare against.
#ifndef FA_RESCALE_TAU
#define FA_RESCALE_TAU 8.0f
#endif
constexpr float kTau = FA_RESCALE_TAU;
// Exponentials on the FMA units: with FA_EXP_POLY_EVERY = k > 0, one
// probability in k (register r of a lane's 16 with r % k == k - 1) comes
// from poly_exp2 instead of the exponential instruction.  Off by default: on
// this chip the instruction costs about two FMAs of issue time and the
// polynomial eight, and the forward is not bound by its exponentials.
#ifndef FA_EXP_POLY_EVERY
#define FA_EXP_POLY_EVERY 0
#endif
constexpr int kPolyEvery = FA_EXP_POLY_EVERY;

struct WorkItem {
  int seq_start;  // first query token of the sequence
  int seq_len;    // its query count
  int k_start;    // first key token
  int k_len;      // key count
  int off;        // causal offset k_len - seq_len
  int b;          // batch index (dense) or sequence index (varlen)
  int h;          // query head
  int qtile;
  bool valid;
  bool split;     // one chunk of a split query tile (varlen only)
  int chunk;
};

template <bool CAUSAL, bool VARLEN>
__device__ __forceinline__ WorkItem fwd_work_item(const FwdParams& p) {
  WorkItem w;
  const int t = blockIdx.x;
  if (VARLEN) {
    const int e = t / p.Hq;
    w.h = t - e * p.Hq;
    const int count = (int)p.hdr[kHdrCount];
    w.valid = e < count && (p.hdr[kHdrErr] & kErrBadCu) == 0;
    if (!w.valid) return w;
    w.b = p.tiles[2 * e];
    const int v = p.tiles[2 * e + 1];
    w.split = (v & kSplitItem) != 0;
    w.chunk = v & 0xFFFFF;
    w.qtile = w.split ? -1 : v;  // a split chunk belongs to the last query tile
    w.seq_start = p.cu_seqlens[w.b];
    w.seq_len = p.cu_seqlens[w.b + 1] - w.seq_start;
    w.k_start = p.cu_seqlens_k[w.b];
    w.k_len = p.cu_seqlens_k[w.b + 1] - w.k_start;
    w.off = w.k_len - w.seq_len;
  } else {
    const int BH = p.B * p.Hq;
    int i, bh;
    if (p.sched == 0 && (BH & 7) == 0) {
      // consecutive workgroups go to different XCDs (round robin over 8): give
      // each XCD a contiguous block of heads so the query heads of one
      // key/value head share that XCD's L2; inside it, most expensive first
      const int x = t & 7, r = t >> 3, hx = BH >> 3;
      const int ii = r / hx;
      bh = x * hx + (r - ii * hx);
      i = CAUSAL ? (p.nq - 1 - ii) : ii;
    } else if (p.sched == 0) {
      const int ii = t / BH;
      bh = t - ii * BH;
      i = CAUSAL ? (p.nq - 1 - ii) : ii;
    } else {
      bh = t / p.nq;
      i = t - bh * p.nq;
    }
    w.b = bh / p.Hq;
    w.h = bh - w.b * p.Hq;
    w.qtile = i;
    w.seq_start = w.b * p.N;
    w.seq_len = p.N;
    w.k_start = w.seq_start;
    w.k_len = p.N;
    w.off = 0;
    w.split = false;
    w.chunk = 0;
    w.valid = true;
  }
  return w;
}

template <int D, int NW, bool CAUSAL, bool VARLEN, bool FP8 = false>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(FwdParams p) {
  constexpr int BR = NW * 32;
  constexpr int EB = FP8 ? 1 : 2;                // bytes per Q / K element
  constexpr int CH = D / 8;                      // 16-byte chunks per bf16 row (V)
  constexpr int KCH = D * EB / 16;               // 16-byte chunks per K row
  using KT = PadTile<kBC, KCH, KCH + 1>;         // K: 16-byte operand reads
  // V: 8-byte transposed reads; row pitch 16 (mod 64) dwords where it fits
  using VT = SwzTile<kBC, CH, D == 256 ? 36 : (D == 128 ? 20 : 12)>;

  constexpr int STAGES = fwd_stages(D);          // K/V tiles in flight or in use
  // the K (bf16 or fp8) operands of a tile's products and its first V^T
  // operands are read in bulk ahead of them (d = 256 keeps interleaved reads)
  constexpr bool PREFETCH = D <= 128;
  static_assert(!FP8 || D <= 128, "fp8 scores take d = 64 or 128");
  __shared__ __attribute__((aligned(16))) char kv_s[STAGES][KT::kBytes + VT::kBytes];

  WorkItem wi = fwd_work_item<CAUSAL, VARLEN>(p);
  if (!wi.valid) return;
  if (VARLEN && wi.split) wi.qtile = (wi.seq_len - 1) / BR;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int g16 = lane >> 4;   // 16-lane group
  const int L16 = lane & 15;

  const int q0 = wi.qtile * BR;
  if (q0 >= wi.seq_len) return;
  const int hkv = wi.h / p.G;
  const long q_row = (long)p.Hq * D;   // elements between consecutive tokens
  const long kv_row = (long)p.Hkv * D;
  const char* qbase = reinterpret_cast<const char*>(FP8 ? (const void*)p.q8 : (const void*)p.q) +
                      ((long)wi.seq_start * q_row + (long)wi.h * D) * EB;
  const char* kbase = reinterpret_cast<const char*>(FP8 ? (const void*)p.k8 : (const void*)p.k) +
                      ((long)wi.k_start * kv_row + (long)hkv * D) * EB;
  const bf16* vbase = p.v + (long)wi.k_start * kv_row + (long)hkv * D;
  const int klen = wi.k_len;
  const int off = wi.off;

  // ---- this lane's query and its Q fragments (operand B of S^T = K Q^T)
  const int wq0 = q0 + wave * 32;
  const int qi = wq0 + l32;
  const bool q_ok = qi < wi.seq_len;
  // bf16: 8 values per lane per 16-wide step; fp8: 32 bytes per lane per
  // 64-wide step (head-dim elements 64t + 32 half .. +31)
  constexpr int NQF = FP8 ? D / 64 : D / 16;
  bf16x8 qf[FP8 ? 1 : D / 16];
  i32x8 qf8[FP8 ? D / 64 : 1];
#pragma unroll
  for (int dc = 0; dc < NQF; ++dc) {
    if (FP8) {
      u32x4 u0 = {0u, 0u, 0u, 0u}, u1 = {0u, 0u, 0u, 0u};
      if (q_ok) {
        const char* src = qbase + (long)qi * q_row + 64 * dc + 32 * half;
        u0 = ld_global16(src);
        u1 = ld_global16(src + 16);
      }
      qf8[dc] = i32x8{(int)u0[0], (int)u0[1], (int)u0[2], (int)u0[3],
                      (int)u1[0], (int)u1[1], (int)u1[2], (int)u1[3]};
    } else {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (q_ok) u = ld_global16(qbase + ((long)qi * q_row + dc * 16 + half * 8) * 2);
      qf[dc] = as_bf16x8(u);
    }
  }

  const int kv_end = CAUSAL ? max(0, min(klen, q0 + BR + off)) : klen;
  const int nt_all = (kv_end + kBC - 1) / kBC;
  // key tiles jb .. jb + nt - 1 (a split chunk covers its own range)
  const bool split = VARLEN && wi.split;
  const int ct = fwd_split_chunk_tiles(nt_all);
  const int jb = split ? wi.chunk * ct : 0;
  const int nt = split ? min(ct, nt_all - jb) : nt_all;

  // ---- direct global->LDS copy of one K and one V tile.  Rows past the
  // sequence end arrive as zeros (buffer range check); their scores are
  // masked.  With 8 waves only waves 0-3 copy, each the same number of
  // instructions per tile (kCopies), and they issue a tile's copies after
  // their own products of the previous tile: the two waves of a SIMD share
  // its matrix unit, the older one (waves 0-3) gets ahead and would otherwise
  // wait at the next barrier, so the copies cost the critical waves 4-7
  // nothing.  The 2-deep ring (d = 256) copies right after the barrier
  // instead, so each tile has a whole tile of products to arrive.
  constexpr int VST = D == 256 ? 36 : (D == 128 ? 20 : 12);
  constexpr int CW = NW == 8 ? NW / 2 : NW;      // waves that copy
  constexpr bool LATE = STAGES >= 3;             // copies after the products
  constexpr int kCopies = dma_count<KT, CW>() + dma_count<VT, CW>();
  const bool copier = wave < CW;
  const long kv_bytes = kv_row * 2;     // V row pitch (bf16)
  const long k_bytes = kv_row * EB;     // K row pitch
  // d = 256 holds the copy offsets in LDS: its products leave no register
  // free across the tile loop, and offsets spilled to scratch would be
  // reloaded with a wait that also drains the tile copies in flight
  constexpr bool OFF_LDS = D == 256;
  using KCopy = TileCopy<KT, CW, OFF_LDS>;
  using VCopy = TileCopy<VT, CW, OFF_LDS>;
  __shared__ uint32_t off_s[OFF_LDS ? KCopy::kStash + VCopy::kStash : 1];
  KCopy kcopy;
  VCopy vcopy;
  kcopy.init(k_bytes, KCH + 1, wave % CW, lane, [](int, int pc) { return pc < KCH ? pc : -1; },
             off_s, copier);
  vcopy.init(kv_bytes, VST, wave % CW, lane, [](int row, int pc) { return VT::slot_chunk(row, pc); },
             off_s + KCopy::kStash, copier);
  auto issue_tile = [&](int u) {  // the u-th tile of this item, key tile jb + u
    if (!copier) return;
    char* kt = kv_s[u % STAGES];
    const int j = jb + u;
    kcopy.issue(kt, make_rsrc(kbase + (long)j * kBC * k_bytes,
                              tile_range(j * kBC, klen, k_bytes, D * EB, kBC)));
    vcopy.issue(kt + KT::kBytes, make_rsrc(vbase + (long)j * kBC * kv_row,
                                           tile_range(j * kBC, klen, kv_bytes, D * 2, kBC)));
  };

  // ---- running softmax state (per lane = per query; both lane halves agree)
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_ref = -INFINITY;  // reference max in scaled log2 units
  float lsum = 0.f;         // this lane half's partial row sum

  // transposed reads of V rows 16kc + 8ld + 4(g16/2) + L16/4, columns
  // 32db + 16(g16%2) + 4(L16%4): v_tr[ld] + 16 kc pitch + 64 db
  const int v_tr[2] = {VT::off(4 * (g16 >> 1) + (L16 >> 2), 16 * (g16 & 1) + 4 * (L16 & 3)),
                       VT::off(8 + 4 * (g16 >> 1) + (L16 >> 2), 16 * (g16 & 1) + 4 * (L16 & 3))};

  // S^T = K Q^T for the two 32-key blocks of key tile j
  auto scores_tile = [&](const char* kt, f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
    if (FP8) {
      // every fp8 K operand of the tile is read before the first product
      i32x8 kf8[D / 64][2];
#pragma unroll
      for (int dc = 0; dc < D / 64; ++dc)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const char* src = kt + (kb * 32 + l32) * KT::kPitch + 64 * dc + 32 * half;
          const u32x4 a0 = ld_lds16(src), a1 = ld_lds16(src + 16);
          kf8[dc][kb] = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                              (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dc = 0; dc < D / 64; ++dc)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x64_fp8(kf8[dc][kb], qf8[dc], s[kb]);
    } else if (PREFETCH) {
      // every K operand of the tile is read before the first product, so the
      // products wait on one LDS latency instead of one per product pair
      bf16x8 kf[D / 16][2];
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          kf[dc][kb] = as_bf16x8(ld_lds16(kt + KT::off(kb * 32 + l32, 16 * dc + 8 * half)));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(kf[dc][kb], qf[dc], s[kb]);
    } else {
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = as_bf16x8(ld_lds16(kt + KT::off(kb * 32 + l32, 16 * dc + 8 * half)));
          s[kb] = mfma32x32x16(a, qf[dc], s[kb]);
        }
      }
    }
  };
  // masked online softmax and O^T += V^T P^T for key tile j
  auto finish_tile = [&](int j, const char* vt, f32x16 (&s)[2]) {
    const int key0 = j * kBC;
    // V^T operands of the first two 16-key chunks are read now, so their
    // latency hides behind the mask, the row max and the rescale
    bf16x8 vpre[2][D / 32];
    if (PREFETCH) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int vo = 16 * kc * VT::kPitch + 64 * db;
          vpre[kc][db] = cat8(ld_lds_tr8(vt + v_tr[0] + vo), ld_lds_tr8(vt + v_tr[1] + vo));
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    const bool need_mask = (CAUSAL && key0 + kBC - 1 > wq0 + off) || (key0 + kBC > klen);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool dead = key >= klen || (CAUSAL && key > qi + off);
          if (dead) s[kb][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = halves_max(mx) * p.c;
    const float m_new = fmaxf(m_ref, mx);
    const bool grow = m_new > m_ref + kTau;
    if (__ballot(grow) != 0ull) {
      // rescale the whole wave to the new reference (lanes whose max did not
      // move get alpha = 1); a row that has seen no key yet keeps -inf
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = fmaf(s[kb][r], p.c, -m_use);
        const float pv = (kPolyEvery > 0 && r % kPolyEvery == kPolyEvery - 1) ? poly_exp2(x)
                                                                               : fast_exp2(x);
        s[kb][r] = pv;
        lsum += pv;
      }
    // O^T += V^T P^T over four 16-key chunks; the transposed read of rows
    // 16kc + 8ld + 4half + 0..3 gives exactly the keys of P's registers
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const bf16x8 pb = frag_rows(s[kc >> 1], kc & 1);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        bf16x8 va;
        if (PREFETCH && kc < 2) {
          va = vpre[kc][db];
        } else {
          const int vo = 16 * kc * VT::kPitch + 64 * db;
          va = cat8(ld_lds_tr8(vt + v_tr[0] + vo), ld_lds_tr8(vt + v_tr[1] + vo));
        }
        oacc[db] = mfma32x32x16(va, pb, oacc[db]);
      }
    }
  };
  auto compute_tile = [&](int j, const char* kt, const char* vt) {
    f32x16 s[2];
    scores_tile(kt, s);
    finish_tile(j, vt, s);
  };

  // STAGES-deep copy ring: tiles j+1 .. j+STAGES-2 (and j+STAGES-1 once it is
  // issued) are in flight while tile j is computed.  Copies retire in issue
  // order, so waiting until at most (tiles issued after j) x kCopies copies
  // are outstanding means tile j is in (waves that do not copy pass at once;
  // the barrier makes the copiers' tiles visible to them).
  wait_vmem();  // Q fragments
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t)
    if (t < nt) issue_tile(t);
  for (int u = 0; u < nt; ++u) {
    const int j = jb + u;
    const int newer = min(nt - 1 - u, STAGES - 2);  // tiles issued after this one
    if (newer >= 2) wait_vmem_leave<2 * kCopies>();
    else if (newer == 1) wait_vmem_leave<kCopies>();
    else wait_vmem();
    lds_barrier();  // tile u landed for every wave; tile u-1's buffer is free
    if (!LATE && u + STAGES - 1 < nt) issue_tile(u + STAGES - 1);
    const char* kt = kv_s[u % STAGES];
    // a wave whose rows are all past the sequence end, or (causal) all above
    // this tile's first key, would only add exact zeros: it skips the tile
    // (it still copies and meets every barrier)
    const bool live = wq0 < wi.seq_len && (!CAUSAL || j * kBC <= wq0 + 31 + off);
    if (live) compute_tile(j, kt, kt + KT::kBytes);
    // (late) tile u+STAGES-1 goes into tile u-1's slot, which every wave left
    // before the barrier above
    if (LATE && u + STAGES - 1 < nt) issue_tile(u + STAGES - 1);
  }

  // ---- epilogue: O = O~ / l (single final rescale), LSE = (m + log2 l) ln 2;
  // a row that saw no key (l = 0) stores O = 0 and LSE = -inf
  const float ltot = halves_sum(lsum);
  if (!q_ok) return;
  if (split) {
    // a chunk of a split tile (only wave 0 holds live rows): the unscaled
    // O~, its reference max and row sum go to this chunk's partial slot
    const long slot = (long)p.split_base[wi.b] + wi.chunk;
    const long row = (slot * p.Hq + wi.h) * 32 + l32;
    float* po = p.part_o + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * half;
        *reinterpret_cast<f32x4*>(po + d0) = f32x4{oacc[db][4 * g + 0], oacc[db][4 * g + 1],
                                                   oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
      }
    if (half == 0) {
      p.part_ml[2 * row] = m_ref;
      p.part_ml[2 * row + 1] = ltot;
    }
    return;
  }
  const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
  bf16* orow = p.o + ((long)wi.seq_start + qi) * q_row + (long)wi.h * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + 8 * g + 4 * half;
      u32x2 w;
      w[0] = pack2_bf16(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
      w[1] = pack2_bf16(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + d0) = w;
    }
  if (half == 0) {
    const float lse = ltot > 0.f ? (m_ref + log2f(ltot)) * kLn2 : -INFINITY;
    long idx;
    if (VARLEN) idx = (long)wi.h * p.T + wi.seq_start + qi;
    else idx = ((long)wi.b * p.Hq + wi.h) * p.N + qi;
    p.lse[idx] = lse;
  }
}

// Merge of the chunks of split query tiles: per row, M = max_c m_c,
// l = sum_c 2^(m_c - M) l_c, O = sum_c 2^(m_c - M) O~_c / l, LSE =
// (M + log2 l) ln 2, with the chunks taken in ascending order (the same result
// on every run).  The chunks' m_c are reference maxima of the online softmax
// ([FA2] "Core method" 1): rescaling partial sums to a common maximum is the
// same step that merges key tiles inside one workgroup.
template <int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(FwdParams p, int br) {
  // nothing to merge when the scheduler rejected the offsets or the lists
  // overflowed (split_base may then be stale)
  if (p.hdr[kHdrErr] & (kErrBadCu | kErrTileOverflow)) return;
  const int s = blockIdx.x / p.Hq;
  const int h = blockIdx.x - s * p.Hq;
  const int base = p.split_base[s];
  const int n = p.split_base[s + 1] - base;
  if (n == 0) return;
  const int q_start = p.cu_seqlens[s];
  const int lq = p.cu_seqlens[s + 1] - q_start;
  const int q0 = ((lq - 1) / br) * br;  // first row of the split (last) tile
  const int live = lq - q0;             // at most 32
  constexpr int CPR = D / 8;            // 8-float chunks per row
  const int t = threadIdx.x;
  for (int w = t; w < 32 * CPR; w += 256) {
    const int r = w / CPR, c8 = (w - r * CPR) * 8;
    if (r >= live) continue;
    float M = -INFINITY;
    for (int c = 0; c < n; ++c)
      M = fmaxf(M, p.part_ml[2 * (((long)(base + c) * p.Hq + h) * 32 + r)]);
    float l = 0.f;
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < n; ++c) {
      const long row = ((long)(base + c) * p.Hq + h) * 32 + r;
      const float mc = p.part_ml[2 * row];
      if (mc == -INFINITY) continue;  // this chunk saw no key of the row
      const float wgt = fast_exp2(mc - M);
      l += wgt * p.part_ml[2 * row + 1];
      const f32x4* po = reinterpret_cast<const f32x4*>(p.part_o + row * D + c8);
      o0 += wgt * po[0];
      o1 += wgt * po[1];
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const long tok = (long)q_start + q0 + r;
    u32x4 w4;
    w4[0] = pack2_bf16(o0[0] * inv, o0[1] * inv);
    w4[1] = pack2_bf16(o0[2] * inv, o0[3] * inv);
    w4[2] = pack2_bf16(o1[0] * inv, o1[1] * inv);
    w4[3] = pack2_bf16(o1[2] * inv, o1[3] * inv);
    *reinterpret_cast<u32x4*>(p.o + tok * ((long)p.Hq * D) + (long)h * D + c8) = w4;
    if (c8 == 0) p.lse[(long)h * p.T + tok] = l > 0.f ? (M + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, int NW, bool CAUSAL, bool VARLEN, bool FP8 = false>
hipError_t launch_fwd_t(const FwdParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_kernel<D, NW, CAUSAL, VARLEN, FP8>), dim3(grid), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

int fwd_tile_rows(int d) { return fwd_waves(d) * 32; }

hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, bool varlen, int grid,
                          hipStream_t stream) {
  constexpr int NW = kFwdWaves;
  if (d == 128) {
    if (causal) return varlen ? launch_fwd_t<128, NW, true, true, true>(p, grid, stream)
                              : launch_fwd_t<128, NW, true, false, true>(p, grid, stream);
    return varlen ? launch_fwd_t<128, NW, false, true, true>(p, grid, stream)
                  : launch_fwd_t<128, NW, false, false, true>(p, grid, stream);
  }
  if (causal) return varlen ? launch_fwd_t<64, NW, true, true, true>(p, grid, stream)
                            : launch_fwd_t<64, NW, true, false, true>(p, grid, stream);
  return varlen ? launch_fwd_t<64, NW, false, true, true>(p, grid, stream)
                : launch_fwd_t<64, NW, false, false, true>(p, grid, stream);
}

hipError_t launch_fwd_combine(const FwdParams& p, int d, int nseq, hipStream_t stream) {
  const long grid = (long)nseq * p.Hq;
  if (grid <= 0) return hipSuccess;
  if (d == 256)
    hipLaunchKernelGGL(fwd_combine_kernel<256>, dim3((unsigned)grid), dim3(256), 0, stream, p,
                       fwd_tile_rows(256));
  else if (d == 128)
    hipLaunchKernelGGL(fwd_combine_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, p,
                       fwd_tile_rows(128));
  else
    hipLaunchKernelGGL(fwd_combine_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, p,
                       fwd_tile_rows(64));
  return hipGetLastError();
}
int fwd_tile_keys() { return kBC; }

hipError_t launch_fwd(const FwdParams& p, int d, bool causal, bool varlen, int grid,
                      hipStream_t stream) {
  constexpr int NW = kFwdWaves;
  if (d == 256) {
    if (causal) return varlen ? launch_fwd_t<256, NW, true, true>(p, grid, stream)
                              : launch_fwd_t<256, NW, true, false>(p, grid, stream);
    return varlen ? launch_fwd_t<256, NW, false, true>(p, grid, stream)
                  : launch_fwd_t<256, NW, false, false>(p, grid, stream);
  }
  if (d == 128) {
    if (causal) return varlen ? launch_fwd_t<128, NW, true, true>(p, grid, stream)
                              : launch_fwd_t<128, NW, true, false>(p, grid, stream);
    return varlen ? launch_fwd_t<128, NW, false, true>(p, grid, stream)
                  : launch_fwd_t<128, NW, false, false>(p, grid, stream);
  }
  if (causal) return varlen ? launch_fwd_t<64, NW, true, true>(p, grid, stream)
                            : launch_fwd_t<64, NW, true, false>(p, grid, stream);
  return varlen ? launch_fwd_t<64, NW, false, true>(p, grid, stream)
                : launch_fwd_t<64, NW, false, false>(p, grid, stream);
}

}  // namespace fa
