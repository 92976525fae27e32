// fa_bwd.hip -- fused attention backward for gfx950.
//
// Method ([FA2] "Core method" 2 and 4; [FA4B] 2.1, 3.2, 3.3.1, 5.2, 5.3):
//  * preprocess: D = rowsum(dO o O) per query row (fp32), and the fp32 dQ
//    accumulator, the ordering semaphores and the workspace header are zeroed;
//  * main kernel: one workgroup per (sequence, key/value head, key tile of 128
//    keys, query-head subgroup).  Each of the 4 waves owns 32 keys and keeps its
//    K and V rows and its dK, dV accumulators in registers for the whole
//    kernel.  The workgroup walks every query head of its key/value head
//    (subgroup) and, per head, the 32-row query tiles from the diagonal
//    upwards (causal) or all of them; per query tile:
//        S  = Q K^T,  P = exp2(S c - LSE log2 e)        (recomputed, masked)
//        dP = dO V^T, dS = P o (dP - D)
//        dV += P^T dO,  dK += dS^T Q                    (register accumulators)
//        dQ_tile += dS K                                (dS exchanged via LDS)
//    The dQ tile is reduced across key tiles either with fp32 device atomics
//    (fast) or, in deterministic mode, in a fixed order: for each dQ tile the
//    writers are applied in descending key-tile index, each waiting on a
//    per-tile semaphore until its rank comes up, adding, then releasing.
//    Workgroups take their work items from an atomic ticket in that same
//    descending order, so every workgroup a writer waits for already runs and
//    the causal walk (diagonal first) never stalls on its first write.
//  * post: dQ = bf16(scale * dQ_acc); split subgroups' dK/dV partials are
//    summed in a fixed order.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int NW = kBwdWaves;
constexpr int NT = NW * 64;
constexpr int BQ = kBwdBQ;
constexpr int BC = kBwdBC;

template <int D>
struct BwdLds {
  static constexpr int rowStride = D * 2 + 16;    // Q, dO row-major tiles
  static constexpr int tStride = BQ * 2 + 16;     // Q^T, dO^T (permuted query axis)
  static constexpr int sStride = BC * 2 + 16;     // dS [q][key]
  static constexpr int ktStride = BC * 2 + 16;    // K^T [d][key]
  static constexpr int qs = 0;
  static constexpr int dos = qs + BQ * rowStride;
  static constexpr int qt = dos + BQ * rowStride;
  static constexpr int dot = qt + D * tStride;
  static constexpr int lse = dot + D * tStride;
  static constexpr int dvec = lse + BQ * 4;
  static constexpr int ds = dvec + BQ * 4;
  static constexpr int kt = ds + BQ * sStride;
  static constexpr int misc = kt + D * ktStride;
  static constexpr int total = misc + 16;
};

struct BwdItem {
  int seq;        // batch index (dense) or sequence index (varlen)
  int seq_start;
  int seq_len;
  int hkv;
  int split;      // query-head subgroup
  int jt;         // key tile
  int nq;         // query tiles of this sequence
  int nkv;        // key tiles of this sequence
  bool valid;
};

template <int D, bool CAUSAL, bool VARLEN, bool DET>
__global__ __launch_bounds__(NT) void bwd_kernel(BwdParams p) {
  using L = BwdLds<D>;
  __shared__ __attribute__((aligned(16))) char smem[L::total];
  int* sh_int = reinterpret_cast<int*>(smem + L::misc);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // ---------------- work item
  int r;
  if (DET) {
    if (tid == 0) sh_int[0] = (int)atomicAdd(&p.hdr[kHdrTicket], 1u);
    __syncthreads();
    r = sh_int[0];
  } else {
    r = blockIdx.x;
  }
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
    it.seq_start = p.cu_seqlens[it.seq];
    it.seq_len = p.cu_seqlens[it.seq + 1] - it.seq_start;
    it.nq = (it.seq_len + BQ - 1) / BQ;
    it.nkv = (it.seq_len + BC - 1) / BC;
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
    it.seq_start = it.seq * p.N;
    it.seq_len = p.N;
    it.nq = p.nq;
    it.nkv = p.nkv;
  }

  const int GS = p.G / p.S;
  const int h0 = it.hkv * p.G + it.split * GS;
  const long q_row = (long)p.Hq * D;
  const long kv_row = (long)p.Hkv * D;
  const int key0 = it.jt * BC;
  const int wk0 = key0 + wave * 32;  // this wave's first key
  const int mykey = wk0 + l32;
  const bool key_ok = mykey < it.seq_len;

  // ---------------- K, V rows of this wave (operand B of S = Q K^T, dP = dO V^T)
  const bf16* kseq = p.k + (long)it.seq_start * kv_row + (long)it.hkv * D;
  const bf16* vseq = p.v + (long)it.seq_start * kv_row + (long)it.hkv * D;
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (key_ok) {
      a = ld_global16(kseq + (long)mykey * kv_row + dc * 16 + half * 8);
      b = ld_global16(vseq + (long)mykey * kv_row + dc * 16 + half * 8);
    }
    kf[dc] = as_bf16x8(a);
    vf[dc] = as_bf16x8(b);
  }
  // K^T of the whole key tile in LDS (operand B of dQ = dS K)
  {
    constexpr int KBL = (BC / 4) * (D / 8);
#pragma unroll
    for (int c = tid; c < KBL; c += NT) {
      const int a = c % (BC / 4), bcol = c / (BC / 4);
      u32x4 rows[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = key0 + 4 * a + e;
        u32x4 u = {0u, 0u, 0u, 0u};
        if (key < it.seq_len) u = ld_global16(kseq + (long)key * kv_row + bcol * 8);
        rows[e] = u;
      }
      store_transposed_4x8(smem + L::kt + (bcol * 8) * L::ktStride, L::ktStride, (4 * a) * 2,
                           rows[0], rows[1], rows[2], rows[3]);
    }
  }

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) { dk_acc[db][x] = 0.f; dv_acc[db][x] = 0.f; }

  // ---------------- walk over (head, query tile)
  const int i_start = CAUSAL ? (key0 / BQ) : 0;
  const int nsteps = max(0, it.nq - i_start);
  const int nitems = GS * nsteps;

  // staging of one query tile: Q and dO rows (row-major and transposed), LSE, D
  constexpr int QBL = (BQ / 4) * (D / 8);
  static_assert(2 * QBL <= NT, "one staging block per thread");
  u32x4 st[4];
  float st_f = 0.f;
  auto stage_load = [&](int item) {
    const int hh = item / nsteps;
    const int i = i_start + (item - hh * nsteps);
    const int h = h0 + hh;
    const int q0 = i * BQ;
    if (tid < 2 * QBL) {
      const bool is_do = tid >= QBL;
      const int c = is_do ? tid - QBL : tid;
      const int a = c % (BQ / 4), bcol = c / (BQ / 4);
      const bf16* src = (is_do ? p.dout : p.q) + (long)it.seq_start * q_row + (long)h * D;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int q = q0 + 4 * a + e;
        u32x4 u = {0u, 0u, 0u, 0u};
        if (q < it.seq_len) u = ld_global16(src + (long)q * q_row + bcol * 8);
        st[e] = u;
      }
    }
    if (tid < 2 * BQ) {
      const int c = tid;
      const bool is_d = c >= BQ;
      const int q = q0 + (is_d ? c - BQ : c);
      long idx;
      if (VARLEN) idx = (long)h * p.T + it.seq_start + q;
      else idx = ((long)it.seq * p.Hq + h) * p.N + q;
      if (q < it.seq_len) st_f = is_d ? p.dvec[idx] : p.lse[idx] * kLog2e;
      else st_f = is_d ? 0.f : INFINITY;  // padding rows: P = 0, dS = 0
    }
  };
  auto stage_store = [&]() {
    if (tid < 2 * QBL) {
      const bool is_do = tid >= QBL;
      const int c = is_do ? tid - QBL : tid;
      const int a = c % (BQ / 4), bcol = c / (BQ / 4);
      char* rm = smem + (is_do ? L::dos : L::qs);
      char* tr = smem + (is_do ? L::dot : L::qt);
#pragma unroll
      for (int e = 0; e < 4; ++e) st_lds16(rm + (4 * a + e) * L::rowStride + bcol * 16, st[e]);
      store_transposed_4x8(tr + (bcol * 8) * L::tStride, L::tStride, kperm16(4 * a) * 2,
                           st[0], st[1], st[2], st[3]);
    }
    if (tid < 2 * BQ) {
      const int c = tid;
      float* dst = reinterpret_cast<float*>(smem + (c >= BQ ? L::dvec : L::lse));
      dst[c >= BQ ? c - BQ : c] = st_f;
    }
  };

  if (nitems > 0) {
    stage_load(0);
    stage_store();
  }
  __syncthreads();

  for (int item = 0; item < nitems; ++item) {
    const int hh = item / nsteps;
    const int i = i_start + (item - hh * nsteps);
    const int h = h0 + hh;
    const int q0 = i * BQ;
    if (item + 1 < nitems) stage_load(item + 1);

    const bool active = key0 + wave * 32 < it.seq_len && (!CAUSAL || q0 + BQ - 1 >= wk0);
    short* ds_tile = reinterpret_cast<short*>(smem + L::ds);
    if (active) {
      f32x16 s, dp;
#pragma unroll
      for (int x = 0; x < 16; ++x) { s[x] = 0.f; dp[x] = 0.f; }
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        const bf16x8 aq = as_bf16x8(ld_lds16(smem + L::qs + l32 * L::rowStride + dc * 32 + half * 16));
        const bf16x8 ado = as_bf16x8(ld_lds16(smem + L::dos + l32 * L::rowStride + dc * 32 + half * 16));
        s = mfma32x32x16(aq, kf[dc], s);
        dp = mfma32x32x16(ado, vf[dc], dp);
      }
      // s[x] = S[q = q0 + 8(x/4) + 4 half + x%4][key = mykey]
      const float* lse_s = reinterpret_cast<const float*>(smem + L::lse);
      const float* dv_s = reinterpret_cast<const float*>(smem + L::dvec);
      const bool need_mask = (CAUSAL && q0 < wk0 + 31) || (wk0 + 32 > it.seq_len);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + 8 * g + 4 * half);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dv_s + 8 * g + 4 * half);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int x = 4 * g + e;
          float pr = fast_exp2(fmaf(s[x], p.c, -l4[e]));
          if (need_mask) {
            const int q = q0 + 8 * g + 4 * half + e;
            if (!key_ok || (CAUSAL && mykey > q)) pr = 0.f;
          }
          s[x] = pr;
          dp[x] = pr * (dp[x] - d4[e]);
        }
      }
      // dV += P^T dO and dK += dS^T Q over two 16-query chunks
#pragma unroll
      for (int qc = 0; qc < 2; ++qc) {
        const bf16x8 pa = frag_rows(s, qc);
        const bf16x8 dsa = frag_rows(dp, qc);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 bdo = as_bf16x8(ld_lds16(smem + L::dot + (db * 32 + l32) * L::tStride + qc * 32 + half * 16));
          const bf16x8 bq = as_bf16x8(ld_lds16(smem + L::qt + (db * 32 + l32) * L::tStride + qc * 32 + half * 16));
          dv_acc[db] = mfma32x32x16(pa, bdo, dv_acc[db]);
          dk_acc[db] = mfma32x32x16(dsa, bq, dk_acc[db]);
        }
      }
      // dS (bf16) to LDS as [q][key] for the workgroup-wide dQ product
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int q = 8 * (x >> 2) + 4 * half + (x & 3);
        ds_tile[q * (L::sStride / 2) + wave * 32 + l32] =
            (short)__builtin_bit_cast(unsigned short, (bf16)dp[x]);
      }
    } else {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int q = 8 * (x >> 2) + 4 * half + (x & 3);
        ds_tile[q * (L::sStride / 2) + wave * 32 + l32] = 0;
      }
    }
    __syncthreads();  // dS complete; Q/dO tiles no longer read
    if (item + 1 < nitems) stage_store();

    // ---------------- dQ_tile = dS K, reduced across key tiles
    constexpr int DQW = D / 32;  // waves that own a 32-column block of dQ
    f32x16 acc;
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[x] = 0.f;
    if (wave < DQW) {
#pragma unroll
      for (int kc = 0; kc < BC / 16; ++kc) {
        const bf16x8 a = as_bf16x8(ld_lds16(smem + L::ds + l32 * L::sStride + kc * 32 + half * 16));
        const bf16x8 b = as_bf16x8(ld_lds16(smem + L::kt + (wave * 32 + l32) * L::ktStride + kc * 32 + half * 16));
        acc = mfma32x32x16(a, b, acc);
      }
    }
    // acc[x] = dQ[q = q0 + 8(x/4) + 4 half + x%4][d = 32 wave + l32]
    float* dq_base = p.dq_acc + (long)it.seq_start * q_row + (long)h * D + wave * 32 + l32;
    if (!DET) {
      if (wave < DQW) {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int q = q0 + 8 * (x >> 2) + 4 * half + (x & 3);
          if (q < it.seq_len)
            __hip_atomic_fetch_add(dq_base + (long)q * q_row, acc[x], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    } else {
      // ordered reduction: writers of a dQ tile apply in descending key-tile order
      const int jhi = CAUSAL ? min(it.nkv - 1, (q0 + BQ - 1) / BC) : it.nkv - 1;
      const int rank = jhi - it.jt;
      long sidx;
      if (VARLEN) sidx = (long)h * p.sem_slots + it.seq_start / BQ + it.seq + i;
      else sidx = ((long)it.seq * p.Hq + h) * p.nq + i;
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
      if (wave < DQW) {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int q = q0 + 8 * (x >> 2) + 4 * half + (x & 3);
          if (q < it.seq_len)
            __hip_atomic_fetch_add(dq_base + (long)q * q_row, acc[x], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // every add of this workgroup has been performed before the release
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(semp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // dS reads done; next tile staged
  }

  // ---------------- dK = scale * sum dS^T Q, dV = sum P^T dO for this wave's keys
  // dk_acc[db][x] = dK[key = wk0 + 8(x/4) + 4 half + x%4][d = 32 db + l32]
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int key = wk0 + 8 * (x >> 2) + 4 * half + (x & 3);
      if (key < it.seq_len) {
        const long off = ((long)it.seq_start + key) * kv_row + (long)it.hkv * D + db * 32 + l32;
        if (p.S == 1) {
          p.dk[off] = (bf16)(dk_acc[db][x] * p.scale);
          p.dv[off] = (bf16)(dv_acc[db][x]);
        } else {
          const long po = (long)it.split * p.T * kv_row + off;
          p.dk_part[po] = dk_acc[db][x] * p.scale;
          p.dv_part[po] = dv_acc[db][x];
        }
      }
    }
}

template <int D, bool CAUSAL, bool VARLEN, bool DET>
hipError_t launch_bwd_t(const BwdParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_kernel<D, CAUSAL, VARLEN, DET>), dim3(grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_bwd_det(const BwdParams& p, bool det, int grid, hipStream_t stream) {
  return det ? launch_bwd_t<D, CAUSAL, VARLEN, true>(p, grid, stream)
             : launch_bwd_t<D, CAUSAL, VARLEN, false>(p, grid, stream);
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, bool causal, bool varlen, bool det, int grid,
                        hipStream_t stream) {
  if (causal) return varlen ? launch_bwd_det<D, true, true>(p, det, grid, stream)
                            : launch_bwd_det<D, true, false>(p, det, grid, stream);
  return varlen ? launch_bwd_det<D, false, true>(p, det, grid, stream)
                : launch_bwd_det<D, false, false>(p, det, grid, stream);
}

// ---------------------------------------------------------------------------
// preprocess: D = rowsum(dO o O); zero dQ_acc, semaphores, header

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* o, const bf16* dout, float* dvec,
                                                      float* dq_acc, int* sem, long sem_count,
                                                      uint32_t* hdr, int rows, int Hq, bool varlen,
                                                      int N, int T) {
  constexpr int EPT = D / 16;  // elements per thread (16 threads per row)
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (blockIdx.x == 0 && threadIdx.x < kHdrWords) hdr[threadIdx.x] = 0u;
  for (long s = (long)blockIdx.x * 256 + threadIdx.x; s < sem_count; s += (long)gridDim.x * 256)
    sem[s] = 0;
  if (row >= rows) return;
  const long base = (long)row * D + sub * EPT;
  float acc = 0.f;
  if (EPT == 8) {
    const u32x4 a = ld_global16(o + base), b = ld_global16(dout + base);
    const bf16x8 x = as_bf16x8(a), y = as_bf16x8(b);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc = fmaf((float)o[base + e], (float)dout[base + e], acc);
  }
  acc += __shfl_xor(acc, 8, 16);
  acc += __shfl_xor(acc, 4, 16);
  acc += __shfl_xor(acc, 2, 16);
  acc += __shfl_xor(acc, 1, 16);
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < EPT; e += 4) *reinterpret_cast<f32x4*>(dq_acc + base + e) = z;
  if (sub == 0) {
    const int tok = row / Hq, h = row - tok * Hq;
    long idx;
    if (varlen) idx = (long)h * T + tok;
    else {
      const int b = tok / N, n = tok - b * N;
      idx = ((long)b * Hq + h) * N + n;
    }
    dvec[idx] = acc;
  }
}

__global__ __launch_bounds__(256) void bwd_post_kernel(const float* dq_acc, bf16* dq, long dq_vec,
                                                       float scale, const float* dk_part,
                                                       const float* dv_part, bf16* dk, bf16* dv,
                                                       long kv_vec, int S) {
  // every element handled in groups of 4 (all sizes are multiples of 64)
  const long stride = (long)gridDim.x * 256;
  for (long v = (long)blockIdx.x * 256 + threadIdx.x; v < dq_vec; v += stride) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(dq_acc + 4 * v);
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

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int d, bool causal, bool varlen, bool det, int grid,
                      hipStream_t stream) {
  if (d == 128) return launch_bwd_d<128>(p, causal, varlen, det, grid, stream);
  return launch_bwd_d<64>(p, causal, varlen, det, grid, stream);
}

hipError_t launch_bwd_pre(const bf16* o, const bf16* dout, float* dvec, float* dq_acc, int* sem,
                          long sem_count, uint32_t* hdr, int rows, int Hq, int d, bool varlen,
                          int N, int T, hipStream_t stream) {
  const int grid = max(1, (rows + 15) / 16);
  if (d == 128)
    hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3(grid), dim3(256), 0, stream, o, dout, dvec,
                       dq_acc, sem, sem_count, hdr, rows, Hq, varlen, N, T);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3(grid), dim3(256), 0, stream, o, dout, dvec,
                       dq_acc, sem, sem_count, hdr, rows, Hq, varlen, N, T);
  return hipGetLastError();
}

hipError_t launch_bwd_post(const float* dq_acc, bf16* dq, long dq_elems, float scale,
                           const float* dk_part, const float* dv_part, bf16* dk, bf16* dv,
                           long kv_elems, int S, hipStream_t stream) {
  const long vec = dq_elems / 4;
  const long blocks = min(4096L, max(1L, (vec + 255) / 256));
  hipLaunchKernelGGL(bwd_post_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dq_acc, dq,
                     vec, scale, dk_part, dv_part, dk, dv, kv_elems / 4, S);
  return hipGetLastError();
}

}  // namespace fa
