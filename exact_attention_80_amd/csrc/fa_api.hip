// fa_api.hip -- C ABI of the library: argument validation, workspace layout,
// device check and launch sequencing.  Declarations and the contract of every
// entry point are in include/fa.h.
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/fa.h"
#include "fa_launch.h"

// Scratch of fa_varlen_qk_fwd_noalloc (its size is FA_NOALLOC_SCRATCH_BYTES).
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

using fa::BwdParams;
using fa::FwdParams;

constexpr int kAbiVersion = 1;
constexpr size_t kAlign = 256;

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
long cdiv(long a, long b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// device check (gfx950 only), cached per device

struct DevInfo {
  bool gfx950 = false;
  int cus = 0;
  std::string arch;
};

std::mutex g_dev_mu;
std::unordered_map<int, DevInfo> g_dev;

int check_device(std::string* why) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *why = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return FA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  auto it = g_dev.find(dev);
  if (it == g_dev.end()) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      *why = std::string("hipGetDeviceProperties: ") + hipGetErrorString(e);
      return FA_ERR_HIP;
    }
    DevInfo info;
    info.arch = prop.gcnArchName;
    info.gfx950 = info.arch.rfind("gfx950", 0) == 0;
    info.cus = prop.multiProcessorCount;
    it = g_dev.emplace(dev, info).first;
  }
  if (!it->second.gfx950) {
    *why = "device " + std::to_string(dev) + " is " + it->second.arch + ", not gfx950";
    return FA_ERR_DEVICE;
  }
  return FA_OK;
}

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  return std::atoi(s);
}

// Ablation switch for the tile order: FA_SCHED=natural disables longest-first
// and XCD grouping in the dense grids and the cost sort of the packed-batch
// scheduler (read on every call; results never depend on it).
int sched_mode() {
  const char* s = std::getenv("FA_SCHED");
  return (s && std::strcmp(s, "natural") == 0) ? 1 : 0;
}

// Bound of a deterministic-mode wait, in ticks of the 100 MHz real-time clock.
uint32_t spin_limit() {
  const int v = env_int("FA_DET_SPIN_TICKS", 0);
  return v > 0 ? (uint32_t)v : 200000000u;  // 2 s
}

// ---------------------------------------------------------------------------
// opt-in per-thread kernel timing (fa_timing_begin / fa_timing_end)

struct Timing {
  bool on = false;
  std::vector<hipEvent_t> pool;  // reused across sessions
  size_t used = 0;
  std::vector<std::pair<int, size_t>> marks;  // (kind, index of the start event)
};
thread_local Timing g_timing;

hipEvent_t timing_event() {
  Timing& t = g_timing;
  if (t.used == t.pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    t.pool.push_back(e);
  }
  return t.pool[t.used++];
}

// Records a start event; returns a token for timing_stop (or -1 when off).
long timing_start(int kind, hipStream_t s) {
  Timing& t = g_timing;
  if (!t.on) return -1;
  const size_t idx = t.used;
  hipEvent_t a = timing_event();
  hipEvent_t b = timing_event();
  if (!a || !b) return -1;
  (void)hipEventRecord(a, s);
  t.marks.emplace_back(kind, idx);
  return (long)idx;
}

void timing_stop(long token, hipStream_t s) {
  if (token < 0) return;
  (void)hipEventRecord(g_timing.pool[(size_t)token + 1], s);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(FA_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned16(p)) return fail(FA_ERR_INVALID_ARG, std::string(name) + " is not 16-byte aligned");
  return FA_OK;
}

int check_dims(long tokens, int Hq, int Hkv, int d, int causal, float scale) {
  if (tokens <= 0) return fail(FA_ERR_INVALID_ARG, "sequence length / token count must be positive");
  if (Hq <= 0 || Hkv <= 0) return fail(FA_ERR_INVALID_ARG, "head counts must be positive");
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(FA_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
  if (d != 64 && d != 128 && d != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dimension must be 64, 128 or 256");
  if (tokens * (long)Hq * d >= (1L << 31) * 16L)
    return fail(FA_ERR_UNSUPPORTED, "tensor too large");
  if (tokens > (1L << 30)) return fail(FA_ERR_UNSUPPORTED, "too many tokens");
  // per-tile buffer ranges (at most 64 rows of one token's heads, fp32 for the
  // dQ accumulator) are 32-bit byte counts
  if ((long)Hq * d >= (1L << 24)) return fail(FA_ERR_UNSUPPORTED, "Hq * d must be below 2^24");
  return FA_OK;
}

// ---------------------------------------------------------------------------
// workspace layouts

struct FwdLayout {
  size_t hdr = 0, tiles = 0, split_base = 0, part_o = 0, part_ml = 0, total = 0;
  int max_tiles = 0;
  int max_split = 0;  // partial slots for the chunks of split query tiles
};

// T: query tokens, Tk: key tokens.  A split tile has at most
// ceil(key tiles / 32) chunks of 32 key tiles of 64 keys, so the chunks of
// all sequences number at most Tk / 2048 + 2 nseq.
FwdLayout fwd_layout(bool varlen, int nseq, long T, long Tk, int Hq, int d) {
  FwdLayout l;
  if (!varlen) return l;
  l.max_split = (int)(Tk / (fa::fwd_tile_keys() * 32) + 2L * nseq + 1);
  l.max_tiles = (int)(T / fa::fwd_tile_rows(d) + nseq + l.max_split);
  l.hdr = 0;
  size_t off = align_up(fa::kHdrWords * 4);
  l.tiles = off;
  off += align_up((size_t)l.max_tiles * 2 * 4);
  l.split_base = off;
  off += align_up((size_t)(nseq + 1) * 4);
  l.part_o = off;
  off += align_up((size_t)l.max_split * Hq * 32 * d * 4);
  l.part_ml = off;
  off += align_up((size_t)l.max_split * Hq * 32 * 2 * 4);
  l.total = off;
  return l;
}

// dQ modes whose partial tiles replace the accumulator (dense only)
bool partial_tile_mode(int m) { return m == fa::kDqPartial || m == fa::kDqFused; }

struct BwdLayout {
  size_t hdr = 0, dvec = 0, lse2 = 0, dq_acc = 0, dq_part = 0, sem = 0, tiles = 0, dk_part = 0,
         dv_part = 0, kv_part = 0, kvb = 0, dq_exp = 0, total = 0;
  long head_pairs = 0;  // mode 2: partial dQ tiles per (batch, query head)
  long sem_count = 0;
  int sem_slots = 0;  // varlen: per head
  int max_tiles = 0;
  int S = 1;
};

// Query-head subgroups per key/value head: split a group when there are too
// few (sequence, key/value head, key tile) work items to fill the GPU.  The
// choice depends only on the shapes, so it is the same for the size query and
// the call.
int choose_split(long units, int G) {
  const int env = env_int("FA_BWD_SPLIT", 0);
  if (env > 0 && G % env == 0) return env;
  for (int S = 1; S <= G; ++S)
    if (G % S == 0 && units * S >= 1024) return S;
  return G;
}

// T: query tokens, Tk: key tokens (equal for dense calls)
BwdLayout bwd_layout(bool varlen, int B, int N, int nseq, long T, long Tk, int Hq, int Hkv, int d,
                     int deterministic, bool causal) {
  BwdLayout l;
  const int G = Hq / Hkv;
  long units;
  if (varlen) {
    l.max_tiles = (int)(Tk / fa::bwd_tile_keys(d) + nseq);
    units = (long)Hkv * (Tk / fa::bwd_tile_keys(d) + 1);
  } else {
    units = (long)B * Hkv * cdiv(N, fa::bwd_tile_keys(d));
  }
  l.S = choose_split(units, G);
  size_t off = align_up(fa::kHdrWords * 4);
  l.dvec = off;
  off += align_up((size_t)T * Hq * 4);
  l.lse2 = off;
  off += align_up((size_t)T * Hq * 4);
  l.dq_acc = off;
  if (partial_tile_mode(deterministic)) {
    l.head_pairs = fa::bwd_partial_pairs(N, causal);
    l.dq_part = off;
    off += align_up((size_t)B * Hq * l.head_pairs * fa::kBwdBQ * d * 4);
  } else {
    off += align_up((size_t)T * Hq * d * 4);
  }
  if (deterministic == 1 || deterministic == 3) {  // semaphores, or arrival counters
    if (varlen) {
      l.sem_slots = (int)(T / fa::kBwdBQ + nseq + 1);
      l.sem_count = (long)Hq * l.sem_slots;
    } else {
      l.sem_count = (long)B * Hq * cdiv(N, fa::kBwdBQ);
    }
    l.sem_count *= fa::bwd_col_halves(d);  // one per column half of a dQ tile
  }
  l.sem = off;
  off += align_up((size_t)l.sem_count * 4);
  if (varlen) {
    l.tiles = off;
    off += align_up((size_t)l.max_tiles * 2 * 4);
  }
  if (l.S > 1) {
    l.dk_part = off;
    off += align_up((size_t)l.S * Tk * Hkv * d * 4);
    l.dv_part = off;
    off += align_up((size_t)l.S * Tk * Hkv * d * 4);
  }
  if (deterministic == fa::kDqFixed) {
    l.kv_part = off;
    off += align_up((size_t)Hkv * cdiv(Tk, fa::kKvBoundRows) * 2 * 4);
    l.kvb = off;
    off += align_up((size_t)Hkv * 4);
    l.dq_exp = off;
    off += align_up((size_t)T * Hq * 4);
  }
  l.total = off;
  return l;
}

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

int hip_fail(hipError_t e, const char* what) {
  return fail(FA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// scratch of the no-allocation entry point: one static device array per GPU
// (each device that loads the library holds its own copy).  Host code must
// never use the array's name as a device address: its address on the current
// device comes from hipGetSymbolAddress, looked up once per device.

constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;

std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch;

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(FA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                  (e != hipSuccess ? hipGetErrorString(e) : "null address"));
    it = g_scratch.emplace(dev, ptr).first;
  }
  *out = it->second;
  return FA_OK;
}

// ---------------------------------------------------------------------------
// shared implementations of dense and varlen calls

// Scores from fp8 inputs: q and k hold OCP e4m3 bytes standing for
// q_descale * Q and k_descale * K (fa_fwd_fp8, fa_varlen_qk_fwd_fp8).
struct Fp8Scores {
  bool on = false;
  float q_descale = 1.f, k_descale = 1.f;
};

// cu / T: query offsets and tokens; cu_k / Tk: key offsets and tokens
// (cu_k == cu and Tk == T for calls with equal lengths)
int run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, bool varlen, int B,
            int N, const int32_t* cu, const int32_t* cu_k, int nseq, long T, long Tk, int Hq,
            int Hkv, int d, float scale, int causal, void* ws, size_t ws_bytes, void* stream,
            Fp8Scores f8 = Fp8Scores{}) {
  int st;
  if ((st = check_ptr(q, f8.on ? "q8" : "q")) || (st = check_ptr(k, f8.on ? "k8" : "k")) ||
      (st = check_ptr(v, "v")) || (st = check_ptr(o, "o")) || (st = check_ptr(lse, "lse")))
    return st;
  if (varlen && ((st = check_ptr(cu, "cu_seqlens_q")) || (st = check_ptr(cu_k, "cu_seqlens_k"))))
    return st;
  if ((st = check_dims(T, Hq, Hkv, d, causal, scale))) return st;
  if ((st = check_dims(Tk, Hq, Hkv, d, causal, scale))) return st;
  float c = scale * fa::kLog2e;
  if (f8.on) {
    if (d != 64 && d != 128)
      return fail(FA_ERR_UNSUPPORTED, "fp8 scores support head dimension 64 or 128");
    if (!(f8.q_descale > 0.f) || !std::isfinite(f8.q_descale) || !(f8.k_descale > 0.f) ||
        !std::isfinite(f8.k_descale))
      return fail(FA_ERR_INVALID_ARG, "descale factors must be positive and finite");
    c = scale * f8.q_descale * f8.k_descale * fa::kLog2e;
    if (!std::isfinite(c) || !(c > 0.f))
      return fail(FA_ERR_INVALID_ARG, "softmax_scale * q_descale * k_descale out of range");
  }
  const FwdLayout lay = fwd_layout(varlen, nseq, T, Tk, Hq, d);
  if (ws_bytes < lay.total || (lay.total > 0 && !ws))
    return fail(FA_ERR_WORKSPACE, "workspace smaller than fa_*fwd_workspace_size()");
  if (lay.total > 0 && (st = check_ptr(ws, "ws"))) return st;
  std::string why;
  if ((st = check_device(&why))) return fail(st, why);

  hipStream_t s = static_cast<hipStream_t>(stream);
  FwdParams p{};
  if (f8.on) {
    p.q8 = static_cast<const uint8_t*>(q);
    p.k8 = static_cast<const uint8_t*>(k);
  } else {
    p.q = static_cast<const fa::bf16*>(q);
    p.k = static_cast<const fa::bf16*>(k);
  }
  p.v = static_cast<const fa::bf16*>(v);
  p.o = static_cast<fa::bf16*>(o);
  p.lse = lse;
  p.B = B;
  p.N = N;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.T = (int)T;
  p.sched = sched_mode();
  p.c = c;
  const int br = fa::fwd_tile_rows(d);
  long grid;
  hipError_t e;
  if (varlen) {
    uint32_t* hdr = reinterpret_cast<uint32_t*>(at(ws, lay.hdr));
    int* tiles = reinterpret_cast<int*>(at(ws, lay.tiles));
    const long tk = timing_start(4, s);
    int* split_base = reinterpret_cast<int*>(at(ws, lay.split_base));
    e = fa::launch_sched(cu, cu_k, nseq, (int)T, (int)Tk, br, 0, causal != 0, fa::fwd_tile_keys(),
                         fa::kBwdBQ, tiles, lay.max_tiles, split_base, lay.max_split, hdr,
                         p.sched == 0, s);
    timing_stop(tk, s);
    if (e != hipSuccess) return hip_fail(e, "scheduler launch");
    p.cu_seqlens = cu;
    p.cu_seqlens_k = cu_k;
    p.split_base = split_base;
    p.part_o = reinterpret_cast<float*>(at(ws, lay.part_o));
    p.part_ml = reinterpret_cast<float*>(at(ws, lay.part_ml));
    p.tiles = tiles;
    p.hdr = hdr;
    grid = (long)lay.max_tiles * Hq;
  } else {
    p.nq = (int)cdiv(N, br);
    grid = (long)p.nq * B * Hq;
  }
  if (grid <= 0) return FA_OK;
  if (grid > 0x7fffffffL) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  const long tk = timing_start(0, s);
  e = f8.on ? fa::launch_fwd_fp8(p, d, causal != 0, varlen, (int)grid, s)
            : fa::launch_fwd(p, d, causal != 0, varlen, (int)grid, s);
  timing_stop(tk, s);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  if (varlen) {
    const long tc = timing_start(5, s);
    e = fa::launch_fwd_combine(p, d, nseq, s);
    timing_stop(tc, s);
    if (e != hipSuccess) return hip_fail(e, "forward combine launch");
  }
  return FA_OK;
}

int run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
            const float* lse, void* dq, void* dk, void* dv, bool varlen, int B, int N,
            const int32_t* cu, const int32_t* cu_k, int nseq, long T, long Tk, int Hq, int Hkv,
            int d, float scale, int causal, int deterministic, void* ws, size_t ws_bytes,
            void* stream) {
  int st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")) || (st = check_ptr(dout, "dout")) || (st = check_ptr(lse, "lse")) ||
      (st = check_ptr(dq, "dq")) || (st = check_ptr(dk, "dk")) || (st = check_ptr(dv, "dv")))
    return st;
  if (varlen && ((st = check_ptr(cu, "cu_seqlens_q")) || (st = check_ptr(cu_k, "cu_seqlens_k"))))
    return st;
  if ((st = check_dims(T, Hq, Hkv, d, causal, scale))) return st;
  if ((st = check_dims(Tk, Hq, Hkv, d, causal, scale))) return st;
  if (deterministic < 0 || deterministic > 4)
    return fail(FA_ERR_INVALID_ARG, "deterministic must be 0, 1, 2, 3 or 4");
  if (varlen && partial_tile_mode(deterministic))
    return fail(FA_ERR_UNSUPPORTED, "deterministic == 2 or 3 (partial-tile dQ) is dense-only");
  if (partial_tile_mode(deterministic) && !fa::bwd_partial_modes(d))
    return fail(FA_ERR_UNSUPPORTED,
                "deterministic == 2 or 3 (partial-tile dQ) needs d <= 128 and 32 keys per wave");
  const BwdLayout lay =
      bwd_layout(varlen, B, N, nseq, T, Tk, Hq, Hkv, d, deterministic, causal != 0);
  if (!ws || ws_bytes < lay.total)
    return fail(FA_ERR_WORKSPACE, "workspace smaller than fa_*bwd_workspace_size()");
  if ((st = check_ptr(ws, "ws"))) return st;
  std::string why;
  if ((st = check_device(&why))) return fail(st, why);

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* hdr = reinterpret_cast<uint32_t*>(at(ws, 0));
  float* dvec = reinterpret_cast<float*>(at(ws, lay.dvec));
  float* dq_acc =
      partial_tile_mode(deterministic) ? nullptr : reinterpret_cast<float*>(at(ws, lay.dq_acc));
  int* sem = reinterpret_cast<int*>(at(ws, lay.sem));
  const bool fixed = deterministic == fa::kDqFixed;
  float* kvb = fixed ? reinterpret_cast<float*>(at(ws, lay.kvb)) : nullptr;
  int* dq_exp = fixed ? reinterpret_cast<int*>(at(ws, lay.dq_exp)) : nullptr;
  long tk = timing_start(2, s);
  hipError_t e = hipSuccess;
  if (fixed)
    e = fa::launch_bwd_kv_bound(static_cast<const fa::bf16*>(k), static_cast<const fa::bf16*>(v),
                                reinterpret_cast<float*>(at(ws, lay.kv_part)), kvb, Tk, Hkv, d, s);
  float* lse2 = reinterpret_cast<float*>(at(ws, lay.lse2));
  if (e == hipSuccess)
    e = fa::launch_bwd_pre(static_cast<const fa::bf16*>(o), static_cast<const fa::bf16*>(dout),
                           lse, dvec, lse2, dq_acc, sem, lay.sem_count, hdr, (int)(T * Hq), Hq, d,
                           varlen, N, (int)T, kvb, Hq / Hkv, dq_exp, s);
  timing_stop(tk, s);
  if (e != hipSuccess) return hip_fail(e, "backward preprocess launch");

  BwdParams p{};
  p.q = static_cast<const fa::bf16*>(q);
  p.k = static_cast<const fa::bf16*>(k);
  p.v = static_cast<const fa::bf16*>(v);
  p.dout = static_cast<const fa::bf16*>(dout);
  p.lse = lse2;  // LSE * log2(e), written by the preprocess
  p.dvec = dvec;
  p.dq_acc = dq_acc;
  p.dq_exp = dq_exp;
  p.dk = static_cast<fa::bf16*>(dk);
  p.dv = static_cast<fa::bf16*>(dv);
  p.dk_part = lay.S > 1 ? reinterpret_cast<float*>(at(ws, lay.dk_part)) : nullptr;
  p.dv_part = lay.S > 1 ? reinterpret_cast<float*>(at(ws, lay.dv_part)) : nullptr;
  p.sem = sem;
  p.dq_part =
      partial_tile_mode(deterministic) ? reinterpret_cast<float*>(at(ws, lay.dq_part)) : nullptr;
  p.dq = static_cast<fa::bf16*>(dq);
  p.head_pairs = lay.head_pairs;
  p.hdr = hdr;
  p.B = B;
  p.N = N;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.S = lay.S;
  p.T = (int)T;
  p.Tk = (int)Tk;
  p.sem_slots = lay.sem_slots;
  p.sched = sched_mode();
  p.c = scale * fa::kLog2e;
  p.scale = scale;
  p.spin_limit = spin_limit();
  long grid;
  if (varlen) {
    int* tiles = reinterpret_cast<int*>(at(ws, lay.tiles));
    tk = timing_start(4, s);
    e = fa::launch_sched(cu, cu_k, nseq, (int)T, (int)Tk, fa::bwd_tile_keys(d),
                         deterministic == fa::kDqOrdered ? 2 : 1,
                         causal != 0, fa::fwd_tile_keys(), fa::kBwdBQ, tiles, lay.max_tiles,
                         nullptr, 0, hdr, p.sched == 0, s);
    timing_stop(tk, s);
    if (e != hipSuccess) return hip_fail(e, "scheduler launch");
    p.cu_seqlens = cu;
    p.cu_seqlens_k = cu_k;
    p.tiles = tiles;
    grid = (long)lay.max_tiles * Hkv * lay.S;
  } else {
    p.nkv = (int)cdiv(N, fa::bwd_tile_keys(d));
    p.nq = (int)cdiv(N, fa::kBwdBQ);
    grid = (long)B * Hkv * lay.S * p.nkv;
  }
  grid *= fa::bwd_col_halves(d);  // d = 256: one workgroup per column half
  if (grid > 0x7fffffffL) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  if (grid > 0) {
    tk = timing_start(1, s);
    e = fa::launch_bwd(p, d, causal != 0, varlen, deterministic, (int)grid, s);
    timing_stop(tk, s);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
  }
  tk = timing_start(3, s);
  if (deterministic == 3) {
    // dQ is written by the main kernel; only split dK/dV partials remain
    if (lay.S > 1)
      e = fa::launch_bwd_post(nullptr, nullptr, 0, scale, p.dk_part, p.dv_part,
                              static_cast<fa::bf16*>(dk), static_cast<fa::bf16*>(dv),
                              Tk * Hkv * d, lay.S, nullptr, d, s);
  } else if (deterministic == 2) {
    e = fa::launch_bwd_dq_reduce(p.dq_part, static_cast<fa::bf16*>(dq), B, N, Hq, d, causal != 0,
                                 p.nq, p.nkv, lay.head_pairs, scale, s);
    if (e == hipSuccess && lay.S > 1)
      e = fa::launch_bwd_post(nullptr, nullptr, 0, scale, p.dk_part, p.dv_part,
                              static_cast<fa::bf16*>(dk), static_cast<fa::bf16*>(dv),
                              Tk * Hkv * d, lay.S, nullptr, d, s);
  } else {
    e = fa::launch_bwd_post(dq_acc, static_cast<fa::bf16*>(dq), T * Hq * d, scale, p.dk_part,
                            p.dv_part, static_cast<fa::bf16*>(dk), static_cast<fa::bf16*>(dv),
                            Tk * Hkv * d, lay.S, dq_exp, d, s);
  }
  timing_stop(tk, s);
  if (e != hipSuccess) return hip_fail(e, "backward post launch");
  return FA_OK;
}

bool dense_ok(int B, int N) { return B > 0 && N > 0; }

}  // namespace

extern "C" {

int fa_abi_version(void) { return kAbiVersion; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    case FA_ERR_DEVICE: return "FA_ERR_DEVICE";
    case FA_ERR_DEVICE_REPORTED: return "FA_ERR_DEVICE_REPORTED";
    default: return "FA_ERR_UNKNOWN";
  }
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

size_t fa_fwd_workspace_size(int B, int N, int Hq, int Hkv, int d, int causal) {
  (void)B; (void)N; (void)Hq; (void)Hkv; (void)d; (void)causal;
  return 0;
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int N, int Hq,
           int Hkv, int d, float softmax_scale, int causal, void* ws, size_t ws_bytes,
           void* stream) {
  if (!dense_ok(B, N)) return fail(FA_ERR_INVALID_ARG, "B and N must be positive");
  return run_fwd(q, k, v, o, lse, false, B, N, nullptr, nullptr, 0, (long)B * N, (long)B * N, Hq,
                 Hkv, d, softmax_scale, causal, ws, ws_bytes, stream);
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* v, void* o, float* lse, int B, int N,
               int Hq, int Hkv, int d, float softmax_scale, float q_descale, float k_descale,
               int causal, void* stream) {
  if (!dense_ok(B, N)) return fail(FA_ERR_INVALID_ARG, "B and N must be positive");
  return run_fwd(q8, k8, v, o, lse, false, B, N, nullptr, nullptr, 0, (long)B * N, (long)B * N,
                 Hq, Hkv, d, softmax_scale, causal, nullptr, 0, stream,
                 Fp8Scores{true, q_descale, k_descale});
}

size_t fa_bwd_workspace_size(int B, int N, int Hq, int Hkv, int d, int causal,
                             int deterministic) {
  if (!dense_ok(B, N) || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return 0;
  if (deterministic < 0 || deterministic > 4) return 0;
  if (partial_tile_mode(deterministic) && !fa::bwd_partial_modes(d)) return 0;
  return bwd_layout(false, B, N, 0, (long)B * N, (long)B * N, Hq, Hkv, d, deterministic,
                    causal != 0).total;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int N, int Hq, int Hkv, int d,
           float softmax_scale, int causal, int deterministic, void* ws, size_t ws_bytes,
           void* stream) {
  if (!dense_ok(B, N)) return fail(FA_ERR_INVALID_ARG, "B and N must be positive");
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, false, B, N, nullptr, nullptr, 0, (long)B * N,
                 (long)B * N, Hq, Hkv, d, softmax_scale, causal, deterministic, ws, ws_bytes,
                 stream);
}

size_t fa_varlen_fwd_workspace_size(int nseq, int total_tokens, int Hq, int Hkv, int d,
                                    int causal) {
  (void)Hkv; (void)causal;
  if (nseq <= 0 || total_tokens <= 0 || Hq <= 0 || (d != 64 && d != 128 && d != 256)) return 0;
  return fwd_layout(true, nseq, total_tokens, total_tokens, Hq, d).total;
}

int fa_varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens, int nseq, int total_tokens, int max_seqlen, int Hq,
                  int Hkv, int d, float softmax_scale, int causal, void* ws, size_t ws_bytes,
                  void* stream) {
  if (nseq <= 0) return fail(FA_ERR_INVALID_ARG, "nseq must be positive");
  if (max_seqlen < 0) return fail(FA_ERR_INVALID_ARG, "max_seqlen must be >= 0");
  return run_fwd(q, k, v, o, lse, true, 1, 0, cu_seqlens, cu_seqlens, nseq, total_tokens,
                 total_tokens, Hq, Hkv, d, softmax_scale, causal, ws, ws_bytes, stream);
}

size_t fa_varlen_bwd_workspace_size(int nseq, int total_tokens, int Hq, int Hkv, int d,
                                    int causal, int deterministic) {
  (void)causal;
  if (nseq <= 0 || total_tokens <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return 0;
  if (deterministic < 0 || deterministic > 4 || partial_tile_mode(deterministic)) return 0;
  return bwd_layout(true, 0, 0, nseq, total_tokens, total_tokens, Hq, Hkv, d, deterministic,
                    causal != 0).total;
}

int fa_varlen_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens,
                  int nseq, int total_tokens, int max_seqlen, int Hq, int Hkv, int d,
                  float softmax_scale, int causal, int deterministic, void* ws, size_t ws_bytes,
                  void* stream) {
  if (nseq <= 0) return fail(FA_ERR_INVALID_ARG, "nseq must be positive");
  if (max_seqlen < 0) return fail(FA_ERR_INVALID_ARG, "max_seqlen must be >= 0");
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, true, 1, 0, cu_seqlens, cu_seqlens, nseq,
                 total_tokens, total_tokens, Hq, Hkv, d, softmax_scale, causal, deterministic, ws,
                 ws_bytes, stream);
}

size_t fa_varlen_qk_fwd_workspace_size(int nseq, int total_q, int total_k, int Hq, int Hkv,
                                       int d, int causal) {
  (void)Hkv; (void)causal;
  if (nseq <= 0 || total_q <= 0 || total_k <= 0 || Hq <= 0 || (d != 64 && d != 128 && d != 256))
    return 0;
  return fwd_layout(true, nseq, total_q, total_k, Hq, d).total;
}

int fa_varlen_qk_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                     int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int Hq,
                     int Hkv, int d, float softmax_scale, int causal, void* ws, size_t ws_bytes,
                     void* stream) {
  if (nseq <= 0) return fail(FA_ERR_INVALID_ARG, "nseq must be positive");
  if (max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(FA_ERR_INVALID_ARG, "max_seqlen_q and max_seqlen_k must be >= 0");
  return run_fwd(q, k, v, o, lse, true, 1, 0, cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k,
                 Hq, Hkv, d, softmax_scale, causal, ws, ws_bytes, stream);
}

int fa_varlen_qk_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                             int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                             int Hq, int Hkv, int d, float softmax_scale, int causal,
                             void* stream) {
  if (nseq <= 0) return fail(FA_ERR_INVALID_ARG, "nseq must be positive");
  if (max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(FA_ERR_INVALID_ARG, "max_seqlen_q and max_seqlen_k must be >= 0");
  // the argument checks of run_fwd, made before the scratch is looked up
  int st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")) || (st = check_ptr(lse, "lse")) ||
      (st = check_ptr(cu_seqlens_q, "cu_seqlens_q")) ||
      (st = check_ptr(cu_seqlens_k, "cu_seqlens_k")))
    return st;
  if ((st = check_dims(total_q, Hq, Hkv, d, causal, softmax_scale))) return st;
  if ((st = check_dims(total_k, Hq, Hkv, d, causal, softmax_scale))) return st;
  const size_t need = fwd_layout(true, nseq, total_q, total_k, Hq, d).total;
  if (need > kScratchBytes)
    return fail(FA_ERR_WORKSPACE, "problem needs " + std::to_string(need) +
                                      " bytes of scratch, more than the no-allocation limit of " +
                                      std::to_string(kScratchBytes));
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return run_fwd(q, k, v, o, lse, true, 1, 0, cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k,
                 Hq, Hkv, d, softmax_scale, causal, ws, kScratchBytes, stream);
}

int fa_varlen_qk_fwd_fp8(const void* q8, const void* k8, const void* v, void* o, float* lse,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                         int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int Hq,
                         int Hkv, int d, float softmax_scale, float q_descale, float k_descale,
                         int causal, void* ws, size_t ws_bytes, void* stream) {
  if (nseq <= 0) return fail(FA_ERR_INVALID_ARG, "nseq must be positive");
  if (max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(FA_ERR_INVALID_ARG, "max_seqlen_q and max_seqlen_k must be >= 0");
  return run_fwd(q8, k8, v, o, lse, true, 1, 0, cu_seqlens_q, cu_seqlens_k, nseq, total_q,
                 total_k, Hq, Hkv, d, softmax_scale, causal, ws, ws_bytes, stream,
                 Fp8Scores{true, q_descale, k_descale});
}

size_t fa_varlen_qk_bwd_workspace_size(int nseq, int total_q, int total_k, int Hq, int Hkv,
                                       int d, int causal, int deterministic) {
  if (nseq <= 0 || total_q <= 0 || total_k <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return 0;
  if (deterministic < 0 || deterministic > 4 || partial_tile_mode(deterministic)) return 0;
  return bwd_layout(true, 0, 0, nseq, total_q, total_k, Hq, Hkv, d, deterministic, causal != 0)
      .total;
}

int fa_varlen_qk_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                     int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int Hq,
                     int Hkv, int d, float softmax_scale, int causal, int deterministic, void* ws,
                     size_t ws_bytes, void* stream) {
  if (nseq <= 0) return fail(FA_ERR_INVALID_ARG, "nseq must be positive");
  if (max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(FA_ERR_INVALID_ARG, "max_seqlen_q and max_seqlen_k must be >= 0");
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, true, 1, 0, cu_seqlens_q, cu_seqlens_k, nseq,
                 total_q, total_k, Hq, Hkv, d, softmax_scale, causal, deterministic, ws, ws_bytes,
                 stream);
}

int fa_probe_dq_reduction(float* buf, int rows, int row_floats, int blocks, int items, int store,
                          void* stream) {
  int st;
  if ((st = check_ptr(buf, "buf"))) return st;
  if (rows <= 0 || rows % 32 != 0) return fail(FA_ERR_INVALID_ARG, "rows must be a positive multiple of 32");
  if (row_floats <= 0 || row_floats % 128 != 0)
    return fail(FA_ERR_INVALID_ARG, "row_floats must be a positive multiple of 128");
  if ((long)row_floats * 32 * 4 >= (1L << 31)) return fail(FA_ERR_UNSUPPORTED, "rows too wide");
  if (blocks <= 0 || items <= 0) return fail(FA_ERR_INVALID_ARG, "blocks and items must be positive");
  if (store < 0 || store > 2) return fail(FA_ERR_INVALID_ARG, "store must be 0, 1 or 2");
  std::string why;
  if ((st = check_device(&why))) return fail(st, why);
  hipError_t e = fa::launch_probe_dq(buf, rows, row_floats, blocks, items, store,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return FA_OK;
}

int fa_timing_begin(void) {
  Timing& t = g_timing;
  t.on = true;
  t.used = 0;
  t.marks.clear();
  return FA_OK;
}

int fa_timing_end(int* counts, float* ms) {
  Timing& t = g_timing;
  t.on = false;
  if (counts)
    for (int i = 0; i < FA_TIMING_KINDS; ++i) counts[i] = 0;
  if (ms)
    for (int i = 0; i < FA_TIMING_KINDS; ++i) ms[i] = 0.f;
  for (const auto& m : t.marks) {
    hipEvent_t a = t.pool[m.second], b = t.pool[m.second + 1];
    hipError_t e = hipEventSynchronize(b);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float x = 0.f;
    e = hipEventElapsedTime(&x, a, b);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    if (counts) counts[m.first] += 1;
    if (ms) ms[m.first] += x;
  }
  t.marks.clear();
  t.used = 0;
  return FA_OK;
}

int fa_workspace_error(const void* ws, size_t ws_bytes, void* stream, uint32_t* bits) {
  if (!ws) return fail(FA_ERR_INVALID_ARG, "ws is NULL");
  if (ws_bytes < fa::kHdrWords * 4) return fail(FA_ERR_WORKSPACE, "workspace has no header");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  uint32_t w = 0;
  e = hipMemcpy(&w, ws, sizeof(w), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
  if (bits) *bits = w;
  if (w == 0) return FA_OK;
  std::string msg = "device reported:";
  if (w & FA_DEVERR_BAD_CU_SEQLENS) msg += " bad cu_seqlens;";
  if (w & FA_DEVERR_WAIT_TIMEOUT) msg += " deterministic wait timed out;";
  if (w & FA_DEVERR_TILE_OVERFLOW) msg += " tile list overflow;";
  return fail(FA_ERR_DEVICE_REPORTED, msg);
}

}  // extern "C"
