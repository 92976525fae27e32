// fa_common.h -- device-side building blocks shared by the gfx950 attention kernels.
//
// Everything here is written for CDNA4 (gfx950) wave64 execution:
//  * v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] * B[16x32], bf16 in, fp32 out.
//    Operand A: lane l holds A[m = l%32][k = 8*(l/32) + j], j = 0..7 (8 bf16).
//    Operand B: lane l holds B[k = 8*(l/32) + j][n = l%32].
//    Result C : lane l holds C[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32], r = 0..15.
//  * A result fragment read along its rows therefore gives, per 16-row chunk c
//    (registers 8c..8c+7), exactly the 8 rows that the next product needs as
//    its k-slice in lane half l/32, in the order
//        row(c, half, j) = 16*(c%2) + 8*(j/4) + 4*half + j%4   (within 32 rows).
//    Every second operand that pairs with such a register fragment is stored in
//    LDS with its k axis permuted the same way (kperm16 below), so the
//    fragment is used in place with no cross-lane shuffle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Device error word bits (mirrors include/fa.h).
constexpr uint32_t kErrBadCu = 1u;
constexpr uint32_t kErrWaitTimeout = 2u;
constexpr uint32_t kErrTileOverflow = 4u;

// Workspace header (in 32-bit words) used by the varlen scheduler and the backward.
constexpr int kHdrErr = 0;       // error bits (atomic OR)
constexpr int kHdrTicket = 1;    // deterministic backward work-item ticket
constexpr int kHdrCount = 2;     // number of valid entries in the tile list
constexpr int kHdrWords = 64;    // 256 bytes

// Forward work items that are one chunk of a split query tile carry this bit
// (the low 20 bits are the chunk index).
constexpr int kSplitItem = 1 << 30;
// Key tiles per chunk of a split forward query tile with nt key tiles: 32,
// or more when a row has over 32768 key tiles (at most 1024 chunks).
__host__ __device__ __forceinline__ int fwd_split_chunk_tiles(int nt) {
  const int c = (nt + 1023) / 1024;
  return c > 32 ? c : 32;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32x32x64 product of fp8 (OCP e4m3) operands, fp32 accumulate.  Lane l
// supplies row l % 32 of A (column l % 32 of B) for 32 of the 64 reduction
// indices; A and B pair their bytes position by position, so any assignment
// of the reduction indices to (lane half, byte) works if both use it.
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 b) { return __builtin_bit_cast(u32x4, b); }
__device__ __forceinline__ u32x4 as_u32x4(f32x4 x) { return __builtin_bit_cast(u32x4, x); }
__device__ __forceinline__ f32x4 as_f32x4(u32x4 x) { return __builtin_bit_cast(f32x4, x); }

// cache-policy argument of the buffer load / store builtins that makes the
// access coherent across the whole device (the sc1 bit on gfx950): stores
// reach the level every XCD reads, loads read from it
constexpr int kCoherent = 16;

// Pack 8 fp32 values (round to nearest even) into one MFMA operand.
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3,
                                        float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
  r[4] = (bf16)a4; r[5] = (bf16)a5; r[6] = (bf16)a6; r[7] = (bf16)a7;
  return r;
}

// Two fp32 values rounded to bf16 (nearest even) packed into one 32-bit word.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const uint32_t lo = __builtin_bit_cast(unsigned short, (bf16)a);
  const uint32_t hi = __builtin_bit_cast(unsigned short, (bf16)b);
  return lo | (hi << 16);
}

// Registers 8c..8c+7 of a result fragment as one operand.
__device__ __forceinline__ bf16x8 frag_rows(const f32x16& x, int c) {
  return pack8(x[8 * c + 0], x[8 * c + 1], x[8 * c + 2], x[8 * c + 3],
               x[8 * c + 4], x[8 * c + 5], x[8 * c + 6], x[8 * c + 7]);
}

// Position, inside a 64-element row, at which element kk (0..63) of the permuted
// k axis is stored so that a 16-byte read at 16*c2 + 8*half returns the rows a
// result fragment holds in registers 8*(c2%2).. of lane half `half` (see top).
__device__ __forceinline__ int kperm16(int kk) {
  const int r16 = kk & 15;
  return (kk & ~15) + ((r16 >> 2) & 1) * 8 + (r16 >> 3) * 4 + (r16 & 3);
}

// Bitwise pack of two bf16 lanes of two 32-bit words (select low or high halves).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);  // {a.lo, b.lo}
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // {a.hi, b.hi}
}

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld_lds16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_lds16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st_lds8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Lanes l and l^32 hold the two halves of the same query row: combine them
// with one v_permlane32_swap (each lane ends up with its own value in one
// result and its partner's in the other).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// LDS tiles filled by direct global->LDS loads.
//
// A row-major tile of ROWS rows x CH 16-byte chunks is stored with a row pitch
// of STRIDE >= CH chunks.  A direct load writes 64 consecutive 16-byte slots
// per wave instruction, so slot s holds chunk s % STRIDE of row s / STRIDE; the
// STRIDE - CH padding slots of a row are filled with a copy of its chunk 0 and
// never read.  The padding staggers rows across the LDS banks while keeping
// every operand address a per-lane base plus a compile-time offset.
template <int ROWS, int CH, int STRIDE>
struct PadTile {
  static_assert(STRIDE >= CH, "row pitch");
  static constexpr int kPitch = STRIDE * 16;           // bytes per row
  static constexpr int kSlots = ROWS * STRIDE;
  static constexpr int kBytes = kSlots * 16;
  static constexpr int kInstr = (kSlots + 63) / 64;    // wave-wide loads per tile
  __device__ static constexpr int off(int row, int col) { return row * kPitch + col * 2; }
};

// Row-padded tile whose 16-byte chunks are also permuted within each group of
// four by the row's quad index: chunk c of row r sits at physical chunk
// c ^ ((r >> 2) & 3).  With a pitch of 16 (mod 64) dwords this keeps both
// 16-byte operand reads of 16 consecutive rows and 8-byte transposed reads of
// 4 consecutive rows x 64 bytes free of LDS bank conflicts, and every read
// address stays one of two per-lane bases plus compile-time offsets.
template <int ROWS, int CH, int STRIDE>
struct SwzTile {
  static_assert(CH % 4 == 0 && STRIDE >= CH, "tile geometry");
  static constexpr int kPitch = STRIDE * 16;
  static constexpr int kSlots = ROWS * STRIDE;
  static constexpr int kBytes = kSlots * 16;
  static constexpr int kInstr = (kSlots + 63) / 64;
  __device__ static constexpr int phys(int r, int c) { return c ^ ((r >> 2) & 3); }
  // byte offset of element `col` (a multiple of 4) of row r
  __device__ static constexpr int off(int r, int col) {
    return r * kPitch + (phys(r, col >> 3) << 4) + (col & 7) * 2;
  }
  // logical chunk stored in physical slot s (or -1 for a padding slot)
  __device__ static constexpr int slot_chunk(int r, int pc) { return pc < CH ? phys(r, pc) : -1; }
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// One wave-wide direct load: lane l copies 16 bytes from gsrc into
// lds_wave_base + 16*l (lds_wave_base must be the same for the whole wave).
// Issued as inline assembly so that the compiler does not guard every later
// LDS read with a wait for it: the kernels wait for these copies explicitly
// (wait_vmem*) before the barrier that publishes the tile.  A vector-memory
// instruction unknown to the compiler can only make its own waits stricter.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gsrc), "s"(m0) : "memory", "m0");
}
// Same with 4 bytes per lane (lds_wave_base + 4*l).
__device__ __forceinline__ void dma4(const void* gsrc, void* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(gsrc), "s"(m0) : "memory", "m0");
}

// Direct copy of a padded tile (see PadTile): row r of the tile comes from
// src + min(row0 + r, last) * src_row (rows past `last` repeat the last valid
// row).  Wave w of NW issues the tile's wave-wide loads w, w + NW, ...
template <class T, int CH, int STRIDE, int NW>
__device__ __forceinline__ void dma_tile(char* dst, const __bf16* src, long src_row, int row0,
                                         int last, int wave, int lane) {
#pragma unroll
  for (int k = 0; k < (T::kInstr + NW - 1) / NW; ++k) {
    const int kk = k * NW + wave;
    if (kk < T::kInstr) {
      const int s = kk * 64 + lane;
      if (s < T::kSlots) {
        const int row = s / STRIDE;
        int c = s - row * STRIDE;
        if (c >= CH) c = 0;
        dma16(src + (long)min(row0 + row, last) * src_row + c * 8, dst + kk * 1024);
      }
    }
  }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] << 14); the builtin form lets the compiler's own wait insertion
// know what has completed.
constexpr int kWaitVm0 = 0x0F70;   // vmcnt(0)
constexpr int kWaitVm16 = 0x4F70;  // vmcnt(16)
// ---------------------------------------------------------------------------
// Buffer-descriptor copies.  A raw buffer descriptor (base, byte range) lives
// in scalar registers; each lane supplies only a 32-bit byte offset, and
// lanes whose offset falls outside the range read zeros.  Tiles are copied
// with a descriptor whose base is the tile's first row and whose range ends
// after the sequence's last valid row, so rows past the end arrive as zeros
// without any clamping.
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);  // stride 0: raw byte addressing
  r[2] = (int)num_bytes;
  r[3] = 0x00020000;                            // gfx9 data format word
  return r;
}

// lane l copies 16 (or 4) bytes at byte `voff` of the buffer into
// lds_wave_base + 16*l (4*l).
__device__ __forceinline__ void dma16_buf(i32x4 rsrc, uint32_t voff, void* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m0), "v"(voff), "s"(rsrc) : "memory", "m0");
}
__device__ __forceinline__ void dma4_buf(i32x4 rsrc, uint32_t voff, void* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(m0), "v"(voff), "s"(rsrc) : "memory", "m0");
}

// Byte range of a tile of at most `tile_rows` rows that starts at row `row0`
// of a sequence of `len` rows of `row_bytes` pitch, `data_bytes` used per row
// (0 when the tile is empty).  The range ends with the tile's last valid row,
// so it never spans more than tile_rows rows and fits in 32 bits whenever
// tile_rows * row_bytes does (the host rejects shapes where it would not).
__host__ __device__ __forceinline__ uint32_t tile_range(int row0, int len, long row_bytes,
                                                        int data_bytes, int tile_rows) {
  if (row0 >= len) return 0u;
  const int rows = len - row0 < tile_rows ? len - row0 : tile_rows;
  return (uint32_t)((long)(rows - 1) * row_bytes + data_bytes);
}

// Per-lane offsets of the uniform-count copy of one tile (see dma_count):
// computed once, reused for every tile of the same geometry.  They are held
// in registers, or (IN_LDS, for kernels with no register to spare across the
// tile loop) in an LDS array of kStash dwords per lane, read back before each
// copy: the wave that writes a lane's offsets is the only one that reads them.
template <class T, int NW, bool IN_LDS = false>
struct TileCopy {
  static constexpr int kN = (T::kInstr + NW - 1) / NW;
  static constexpr int kLastLanes = T::kSlots - (T::kInstr - 1) * 64;  // lanes used by the last
  static constexpr int kStash = kN * NW * 64;  // dwords of the LDS array (IN_LDS)
  uint32_t voff[IN_LDS ? 1 : kN];
  uint32_t* stash_;  // IN_LDS: this lane's k-th offset at stash_[k * NW * 64]
  int wave_, lane_;
  // `stash` (IN_LDS): the kStash-dword LDS array; `writer`: this wave fills
  // its part of it (waves that never copy leave it alone)
  template <class ChunkOf>
  __device__ __forceinline__ void init(long row_bytes, int stride, int wave, int lane,
                                       ChunkOf chunk_of, uint32_t* stash = nullptr,
                                       bool writer = true) {
    wave_ = wave;
    lane_ = lane;
    stash_ = IN_LDS ? stash + wave * 64 + lane : nullptr;
#pragma unroll
    for (int k = 0; k < kN; ++k) {
      const int s = min(k * NW + wave, T::kInstr - 1) * 64 + lane;
      const int row = s / stride;
      int c = chunk_of(row, s - row * stride);
      if (c < 0) c = 0;
      const uint32_t o = (uint32_t)(row * row_bytes + c * 16);
      if (!IN_LDS) voff[k] = o;
      else if (writer) stash_[k * NW * 64] = o;
    }
  }
  __device__ __forceinline__ void issue(char* dst, i32x4 rsrc) const {
#pragma unroll
    for (int k = 0; k < kN; ++k) {
      const int kk = min(k * NW + wave_, T::kInstr - 1);  // wave-uniform
      const uint32_t o = IN_LDS ? stash_[k * NW * 64] : voff[k];
      if (kk < T::kInstr - 1 || lane_ < kLastLanes) dma16_buf(rsrc, o, dst + kk * 1024);
    }
  }
};

// Number of wave-wide copy instructions every wave issues for one tile when
// the uniform variants below are used (the last instruction is repeated by
// waves that have nothing left, rewriting identical bytes), so that a wave can
// wait for "all but the newest n tiles" with one s_waitcnt vmcnt(n * count).
template <class T, int NW>
constexpr int dma_count() { return (T::kInstr + NW - 1) / NW; }

template <class T, int NW, class ChunkOf>
__device__ __forceinline__ void dma_uniform(char* dst, const __bf16* src, long src_row, int row0,
                                            int last, int wave, int lane, int stride,
                                            ChunkOf chunk_of) {
#pragma unroll
  for (int k = 0; k < dma_count<T, NW>(); ++k) {
    const int kk = min(k * NW + wave, T::kInstr - 1);
    const int s = kk * 64 + lane;
    if (s < T::kSlots) {
      const int row = s / stride;
      int c = chunk_of(row, s - row * stride);
      if (c < 0) c = 0;
      dma16(src + (long)min(row0 + row, last) * src_row + c * 8, dst + kk * 1024);
    }
  }
}

// Direct copy of a SwzTile (rows as in dma_tile).
template <class T, int STRIDE, int NW>
__device__ __forceinline__ void dma_swz_tile(char* dst, const __bf16* src, long src_row, int row0,
                                             int last, int wave, int lane) {
#pragma unroll
  for (int k = 0; k < (T::kInstr + NW - 1) / NW; ++k) {
    const int kk = k * NW + wave;
    if (kk < T::kInstr) {
      const int s = kk * 64 + lane;
      if (s < T::kSlots) {
        const int row = s / STRIDE;
        int c = T::slot_chunk(row, s - row * STRIDE);
        if (c < 0) c = 0;
        dma16(src + (long)min(row0 + row, last) * src_row + c * 8, dst + kk * 1024);
      }
    }
  }
}

__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  asm volatile("" ::: "memory");
}
// Wait until at most 16 vector-memory instructions of this wave are
// outstanding (they retire in issue order, so everything older is complete).
template <int N>
__device__ __forceinline__ void wait_vmem_leave() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_vmem_leave16() {
  __builtin_amdgcn_s_waitcnt(kWaitVm16);
  asm volatile("" ::: "memory");
}
// Workgroup barrier for LDS traffic only: this wave's LDS accesses are
// complete, global memory operations may stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Transposed 8-byte LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element i%4 of the 8-byte rows that lanes i/4,
// i/4+4, i/4+8, i/4+12 of its group address.  If lane L of a group addresses
// row base + L/4 at column nbase + 4*(L%4), lane i gets column nbase + i of
// rows base .. base+3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 ld_lds_tr8(const void* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ bf16x8 cat8(u32x2 a, u32x2 b) {
  u32x4 u;
  u[0] = a[0]; u[1] = a[1]; u[2] = b[0]; u[3] = b[1];
  return as_bf16x8(u);
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposed 4x8 store: rows r0..r3 each hold 8 bf16 (a 16-byte chunk of a
// row-major tile, columns c..c+7).  Writes, for every column, the 4 values as
// one 8-byte word into a column-major tile at (column row stride `stride`
// bytes, byte offset `pos_bytes` inside each column row).
__device__ __forceinline__ void store_transposed_4x8(char* base, int stride, int pos_bytes,
                                                     const u32x4& r0, const u32x4& r1,
                                                     const u32x4& r2, const u32x4& r3) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    u32x2 lo, hi;
    lo[0] = pack_lo(r0[w], r1[w]);
    lo[1] = pack_lo(r2[w], r3[w]);
    hi[0] = pack_hi(r0[w], r1[w]);
    hi[1] = pack_hi(r2[w], r3[w]);
    st_lds8(base + (2 * w) * stride + pos_bytes, lo);
    st_lds8(base + (2 * w + 1) * stride + pos_bytes, hi);
  }
}

// ---------------------------------------------------------------------------
// Kernel parameter blocks (plain structs passed by value).

struct FwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  const uint8_t* q8;      // fp8 scores: Q and K as OCP e4m3 bytes (c then includes
  const uint8_t* k8;      // their descale factors)
  const int* cu_seqlens;  // varlen only: query offsets
  const int* cu_seqlens_k;  // varlen only: key offsets (the same array when Lq == Lk)
  const int* tiles;       // varlen only: (sequence, q-tile) pairs in schedule order
  const uint32_t* hdr;    // varlen only: workspace header (error word, tile count)
  const int* split_base;  // varlen only: first partial slot per sequence (nseq + 1)
  float* part_o;          // varlen only: [slot, Hq, 32, d] unnormalised partial outputs
  float* part_ml;         // varlen only: [slot, Hq, 32, 2] partial (reference max, row sum)
  int B, N, Hq, Hkv, G;   // dense: N is the sequence length
  int T;                  // total query tokens (varlen LSE layout [Hq, T])
  int nq;                 // dense: number of query tiles per sequence
  int sched;              // 0: longest-first, XCD-grouped; 1: natural order
  float c;                // softmax_scale * log2(e)
};

// One backward work item: a key tile of one (sequence, key/value head,
// query-head subgroup).
struct BwdItem {
  int seq;        // batch index (dense) or sequence index (varlen)
  int q_start;    // first query token, and the sequence's query count
  int q_len;
  int k_start;    // first key token, and the sequence's key count
  int k_len;
  int off;        // causal offset k_len - q_len: key j is visible to query i iff j <= i + off
  int hkv;
  int split;      // query-head subgroup
  int jt;         // key tile
  int nq;         // query tiles of this sequence
  int nkv;        // key tiles of this sequence
};

struct BwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* lse;       // LSE * log2(e), laid out like the forward's logsumexp
  const float* dvec;      // D = rowsum(dO o O), laid out like lse
  float* dq_acc;          // [T, Hq, d] fp32 (int32 fixed point in the fixed-point mode)
  const int* dq_exp;      // fixed-point mode: [T, Hq] exponent of each row's fixed-point scale
  bf16* dk;
  bf16* dv;
  float* dk_part;         // [S, Tk, Hkv, d] fp32 when S > 1
  float* dv_part;
  int* sem;               // dQ tile semaphores (ordered mode) or arrival counters (fused mode)
  float* dq_part;         // per-(query tile, key tile) dQ partial tiles (partial-sum modes)
  bf16* dq;               // dQ output (fused partial-sum mode writes it directly)
  long head_pairs;        // partial tiles per (sequence, query head)
  uint32_t* hdr;          // workspace header
  const int* cu_seqlens;  // varlen only: query offsets
  const int* cu_seqlens_k;  // varlen only: key offsets (the same array when Lq == Lk)
  const int* tiles;       // varlen only: (sequence, kv-tile) pairs in schedule order
  int B, N, Hq, Hkv, G, S;
  int T;                  // total query tokens
  int Tk;                 // total key tokens
  int nkv;                // dense: number of key tiles per sequence
  int nq;                 // dense: number of query tiles per sequence
  int sem_slots;          // varlen: semaphore slots per head
  int sched;
  float c;                // softmax_scale * log2(e)
  float scale;
  uint32_t spin_limit;    // deterministic wait bound (polls)
};

}  // namespace fa
