// gfx950 (MI355X) kernels of the per-decode-step sparse KV assembly path.
//
// One kvs_step of layer l runs, for the B units (b, l):
//   diff_lru   one workgroup per unit: slot lookup + validation, sparse diff
//              (misses compacted in Top-K order by a workgroup prefix sum),
//              hit touch, LRU victim choice from the unit's LRU order array,
//              eviction and map update; also the compacted hit list.
//   assemble   (default) the index copy and the attention in one grid: fetch
//              workgroups read miss rows from pinned host memory over PCIe
//              into the compute buffer and the victim slots and attend over
//              them; hit workgroups copy resident rows from the hot buffer to
//              the compute buffer and attend over them meanwhile.  Each
//              workgroup writes one attention partial
//              (v_mfma_f32_16x16x32_bf16 for Q.K^T and P.V, fp32 online
//              softmax).
//   combine    merges the partials, writes bf16 out and fp32 lse.
// With KVS_FLAG_SEPARATE_ATTENTION the copy and the attention are separate
// launches instead:
//   gather     the index copy (rows read in place: only the misses, into their
//              slots);
//   attention  split-K sparse MLA decode over the K gathered rows (or over
//              the hot buffer through row_slot); a single split writes out and
//              lse itself, more are merged by combine.
// Outside the step: init/reset kernels (pool creation, kvs_free_request), the
// append kernel (kvs_append) and the host-read probe (a measurement helper).
//
// Passages: index mapping / host pool / device cache / index-copy assembly
// ("Sparse Attention-Driven KVCache Management for Domestic AI Supernodes",
// abstract and agenda); Top-k LRU buffer, Sparse Diff Kernel and Top-k
// attention (SGLang/Tair hierarchical sparse attention summary, paragraphs
// 1-3).
#include <math.h>

#include <algorithm>
#include <mutex>

#include "kvs_internal.h"

// Per-step scratch of kvs_step_static, for callers that cannot allocate: one
// copy per GPU, created when the library's code object is loaded there and
// held until the process ends.  Host code never passes this name to a kernel
// (on the host it is only a stand-in for the symbol); it uses the device
// address from static_scratch_address().
static __device__ __align__(256) unsigned char scratch[KVS_STATIC_SCRATCH_BYTES];

namespace kvs {

hipError_t static_scratch_address(int device, void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  int current = -1;
  hipError_t e = hipGetDevice(&current);
  if (e != hipSuccess) return e;
  if (current != device) return hipErrorInvalidDevice;   // resolved with the device current
  std::lock_guard<std::mutex> lock(mu);
  if (addr[device] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *out = addr[device];
  return hipSuccess;
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte chunk
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;         // LDS-qualified

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;   // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Rows are streamed: each KV row a step moves is read once and written once
// (no reuse within a launch), so row loads and stores carry the nontemporal
// hint (`nt`).  On MI355X this lifts a random-row copy of 1152-byte rows from
// 4.4 to 6.5 TB/s (measured; a plain device-to-device copy reaches 5.4).
__device__ __forceinline__ u32x4 ld_row(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_row(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }
// The same hint for buffer-resource loads and stores (cache-policy bit `nt`).
constexpr int kNT = 2;

// A lane's value from another lane of its 16-lane DPP row (gfx9 DPP control).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                            0xf, 0xf, false));
}
// Max / sum over the 16 lanes of a DPP row.  Each step pairs lanes
// symmetrically (lane ^ 1, lane ^ 2 inside a quad, then the mirror inside 8
// and inside 16 lanes), so after each step the lanes of a group hold the same
// value, and the sum is the same bit pattern in all 16 lanes.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<0xb1>(x));    // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_f32<0x4e>(x));    // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, dpp_f32<0x141>(x));   // row_half_mirror
  return fmaxf(x, dpp_f32<0x140>(x));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xb1>(x);
  x += dpp_f32<0x4e>(x);
  x += dpp_f32<0x141>(x);
  return x + dpp_f32<0x140>(x);
}

// ------------------------------------------------------------------ device checks
// The checked build (libkvs_checked.so, KVS_DEVICE_CHECKS=1) compares every
// index a kernel takes from the Top-K, the maps, the LRU order or the step's
// lists with the extent of the array it addresses before the access.  In the
// normal build in_range() and in_bounds() are constant true and every check
// compiles away.
#ifndef KVS_DEVICE_CHECKS
#define KVS_DEVICE_CHECKS 0
#endif

// First failure wins: the status word takes KVS_EBOUNDS, words 1..3 the site
// (KVS_SITE_*) and the index (low, high 32 bits).
__device__ __noinline__ void latch_bounds(int32_t* status, int site, long long idx) {
  if (atomicCAS(status, 0, KVS_EBOUNDS) == 0) {
    status[1] = site;
    status[2] = (int32_t)(uint32_t)((unsigned long long)idx & 0xffffffffull);
    status[3] = (int32_t)(uint32_t)((unsigned long long)idx >> 32);
  }
}

// True when lo <= idx < hi; otherwise (checked build) latches the failure and
// returns false, and the caller skips the access.
__device__ __forceinline__ bool in_range(long long idx, long long lo, long long hi,
                                         int32_t* status, int site) {
  if constexpr (KVS_DEVICE_CHECKS) {
    if (idx >= lo && idx < hi) return true;
    latch_bounds(status, site, idx);
    return false;
  }
  return true;
}

__device__ __forceinline__ bool in_bounds(long long idx, long long n, int32_t* status, int site) {
  return in_range(idx, 0, n, status, site);
}

// ------------------------------------------------------------------ init
// Empties units [u0, u0 + count): maps -1, last_used -1, LRU order 0..S-1.
// The slot arrays hold Sp >= S entries per unit; the padding entries are
// never read as state (slot -1, order 0).
__global__ void init_units_kernel(int32_t* tok2slot, int32_t* slot2tok, int32_t* last_used,
                                  uint16_t* order, long long n_tok, long long n_slot, int S,
                                  int Sp) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long i0 = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  for (long long i = i0; i < n_tok; i += stride) tok2slot[i] = -1;
  for (long long i = i0; i < n_slot; i += stride) {
    const int s = (int)(i % Sp);
    slot2tok[i] = -1;
    last_used[i] = -1;
    order[i] = (uint16_t)(s < S ? s : 0);
  }
}

__global__ void reset_counters_kernel(int32_t* stepctr, long long* stats, int32_t* status,
                                      int units) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < units) {
    stepctr[i] = 0;
    stats[4 * i + 0] = 0;
    stats[4 * i + 1] = 0;
    stats[4 * i + 2] = 0;
    stats[4 * i + 3] = 0;
  }
  if (i < 4) status[i] = 0;
}

__global__ void clear_status_kernel(int32_t* status) {
  if (threadIdx.x < 4) status[threadIdx.x] = 0;
}

// ------------------------------------------------------------------ diff + LRU
// Word 3 of a raw (stride 0) buffer resource on gfx9-family parts: data format
// 32 bits, everything else zero.  Untyped loads ignore the format, but a zero
// format would mark the resource invalid.
constexpr int kBufRsrcWord3 = 0x00020000;

constexpr int kDiffThreads = 1024;
constexpr int kDiffWaves = kDiffThreads / 64;

struct DiffArgs {
  const int32_t* topk;     // [B][K]
  int32_t* tok2slot;       // [B*L][N]
  int32_t* slot2tok;       // [B*L][Sp]
  int32_t* last_used;      // [B*L][Sp]
  uint16_t* order;         // [B*L][Sp]
  int32_t* stepctr;        // [B*L]
  long long* stats;        // [B*L][4]
  int32_t* status;
  int32_t* slot_of;        // [B][K]
  int32_t* miss_pos;       // [B][K]
  int32_t* victims;        // [B][K]
  int32_t* evicted;        // [B][K]
  int32_t* counts;         // [B][4]
  int32_t* row_slot;       // [B][K]: slot of position i's row after the step, -1 empty
  int32_t* hit_pos;        // [B][K]: Top-K positions of the hits, in Top-K order
  int32_t* hit_slot;       // [B][K]: their slots
  int32_t* miss_tok;       // [B][K]: tokens of the misses, in Top-K order
  long long N;
  int S, K, L, layer, hash_bits;
  int Sp;                  // per-unit stride of slot2tok / last_used / order: S rounded up to 16
  int padded;              // 1: a Top-K entry of -1 is empty
};

// Inclusive prefix sum over the 64 lanes of a wave: within each row of 16
// lanes by DPP row shifts (a lane whose source lies outside its row reads 0),
// then the totals of rows 0..2 (read into scalars) added to the rows above.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  return x + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

// Exclusive prefix sum of `v` over the workgroup in thread order; `total`
// receives the workgroup sum.  Must be reached by every thread.  `wtot` holds
// the wave totals; each call site has its own, so one barrier suffices.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* wtot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kDiffWaves; ++w) {
    const int y = wtot[w];
    off += (w < wave) ? y : 0;
    tot += y;
  }
  total = tot;
  return off + x - v;
}

// Wide loads of a thread's run of W 32-bit words (16-byte aligned when W >= 4,
// 8-byte when W == 2): one memory instruction per 16 bytes instead of one per
// element.  Element-wise loads of the order and slot-token runs cost each CU
// about one address-unit clock per cache line per instruction; at 8192 slots
// they took 3.4 us of the diff kernel's start (measured).
template <int W>
__device__ __forceinline__ void load_words(const void* p, uint32_t (&w)[W]) {
  if constexpr (W >= 4) {
#pragma unroll
    for (int v = 0; v < W / 4; ++v) {
      const u32x4 x = reinterpret_cast<const u32x4*>(p)[v];
      w[4 * v + 0] = x[0];
      w[4 * v + 1] = x[1];
      w[4 * v + 2] = x[2];
      w[4 * v + 3] = x[3];
    }
  } else if constexpr (W == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x;
    w[1] = x.y;
  } else {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

// The matching wide stores of a thread's run of W 32-bit words.
template <int W>
__device__ __forceinline__ void store_words(void* p, const uint32_t (&w)[W]) {
  if constexpr (W >= 4) {
#pragma unroll
    for (int v = 0; v < W / 4; ++v)
      reinterpret_cast<u32x4*>(p)[v] = u32x4{w[4 * v], w[4 * v + 1], w[4 * v + 2], w[4 * v + 3]};
  } else if constexpr (W == 2) {
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  } else {
    *reinterpret_cast<uint32_t*>(p) = w[0];
  }
}

// The N uint16 order entries at p (aligned to 2N bytes), widened to int.
template <int N>
__device__ __forceinline__ void load_order(const uint16_t* p, int (&o)[N]) {
  if constexpr (N == 1) {
    o[0] = p[0];
  } else {
    uint32_t w[N / 2];
    load_words<N / 2>(p, w);
#pragma unroll
    for (int q = 0; q < N; ++q) o[q] = (int)((w[q >> 1] >> (16 * (q & 1))) & 0xffffu);
  }
}

// Bit k set when byte k of the N bytes at p (LDS, aligned to N) is non-zero.
template <int N>
__device__ __forceinline__ unsigned nonzero_bytes(const uint8_t* p) {
  unsigned mask = 0;
  if constexpr (N >= 4) {
#pragma unroll
    for (int v = 0; v < N / 4; ++v) {
      const uint32_t w = reinterpret_cast<const uint32_t*>(p)[v];
#pragma unroll
      for (int k = 0; k < 4; ++k) mask |= (((w >> (8 * k)) & 0xffu) != 0u ? 1u : 0u) << (4 * v + k);
    }
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) mask |= (p[k] != 0 ? 1u : 0u) << k;
  }
  return mask;
}

// Zero N bytes of LDS at p (aligned to min(N, 16)) with the widest stores.
template <int N>
__device__ __forceinline__ void zero_bytes(uint8_t* p) {
  if constexpr (N >= 16) {
#pragma unroll
    for (int v = 0; v < N / 16; ++v) reinterpret_cast<u32x4*>(p)[v] = u32x4{0u, 0u, 0u, 0u};
  } else if constexpr (N == 8) *reinterpret_cast<uint2*>(p) = make_uint2(0u, 0u);
  else if constexpr (N == 4) *reinterpret_cast<uint32_t*>(p) = 0u;
  else if constexpr (N == 2) *reinterpret_cast<uint16_t*>(p) = 0;
  else *p = 0;
}

// Thread t owns the contiguous Top-K entries [t*kpt, t*kpt + kpt) and the
// order positions / slots [t*SPT, t*SPT + SPT), so every order-preserving
// compaction is one local count, one workgroup scan and one local write-out.
// The slot arrays of a unit are Sp = S rounded up to 16 entries apart, so a
// thread's run of order entries and slot tokens is aligned for wide loads.
// Global loads are issued as early as their inputs allow: the Top-K entries,
// the LRU order, the slot tokens and the step counter at entry, then the
// token-to-slot lookups.  KPT / SPT: compile-time upper bounds of the Top-K
// entries and slots per thread (powers of two), so the per-thread loops carry
// no dead iterations.
template <int KPT, int SPT>
__global__ __launch_bounds__(kDiffThreads) void diff_lru_kernel(DiffArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int wtot[2][kDiffWaves];   // wave totals of the two workgroup scans
  __shared__ int err_bits;
  __shared__ int n_evict;

  // Every kernel argument is loaded at entry: the pointers used only after
  // the first barrier would otherwise be loaded late, and the barrier's wait
  // for LDS operations also waits for scalar loads (a memory round trip).
  asm volatile("" ::"s"(a.slot_of), "s"(a.miss_pos), "s"(a.victims), "s"(a.evicted),
               "s"(a.counts), "s"(a.row_slot), "s"(a.hit_pos), "s"(a.hit_slot));
  const int S = a.S, K = a.K, Sp = a.Sp;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const long long u = (long long)b * a.L + a.layer;
  const int H = 1 << a.hash_bits;
  const int kpt = (K + kDiffThreads - 1) / kDiffThreads;   // <= KPT
  const int i0 = tid * kpt;
  const int p0 = tid * SPT;
  const bool owns = p0 < Sp;          // the thread's run lies inside the (padded) slots
  const int pl = min(p0, Sp - SPT);   // run loaded (past the slots: the last one, unused)

  // LDS: per-slot flag [Sp] u8 (1 = hit, 2 = victim) | with S <= 8192 the
  //      token of every slot [Sp] i32 | the new LRU order [Sp] u16 | token
  //      hash set [H] i32, reused after validation as miss positions [K] +
  //      victims [K] + miss tokens [K] (the region holds max(H, 3K) words)
  constexpr bool kLdsTok = SPT <= 8;
  uint8_t* flag = smem;
  unsigned* flagw = reinterpret_cast<unsigned*>(smem);   // the same flags, 4 per word
  int32_t* s2t = reinterpret_cast<int32_t*>(smem + Sp);
  uint16_t* lorder = reinterpret_cast<uint16_t*>(smem + Sp + (kLdsTok ? 4 * Sp : 0));
  int32_t* hash = reinterpret_cast<int32_t*>(smem + 3 * Sp + (kLdsTok ? 4 * Sp : 0));
  int32_t* lmiss = hash;
  int32_t* lvict = hash + K;
  int32_t* lmtok = hash + 2 * K;

  int32_t* tok2slot = a.tok2slot + u * a.N;
  int32_t* slot2tok = a.slot2tok + u * Sp;
  int32_t* lu = a.last_used + u * Sp;
  uint16_t* gorder = a.order + u * Sp;
  const int32_t* topk = a.topk + (long long)b * K;
  const long long bk = (long long)b * K;

  // 0. independent loads first: Top-K entries, LRU order, slot tokens, step
  //    counter.  No load sits behind a branch: indices are clamped into range
  //    and the values of positions past K or S are never used (every later
  //    use is guarded).  With a branch per load the compiler's wait counting
  //    takes the path with no loads and drains every load before the next one
  //    is issued, which serialises the two independent chains below.
  int my_tok[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) my_tok[j] = topk[min(i0 + j, K - 1)];
  int my_ord[SPT];
  load_order<SPT>(gorder + pl, my_ord);
  // The step counter through a buffer load, a vector-memory load that travels
  // with the others (as a scalar load it was issued late and waited for before
  // the first barrier: a second round trip).
  const int t = (int)__builtin_amdgcn_raw_buffer_load_b32(
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.stepctr + u), (short)0, 4, kBufRsrcWord3), 0,
      0, 0);
  // The token each victim's slot held.  With S <= 8192 each thread reads the
  // tokens of its own slots (contiguous, not waiting for the order) into LDS
  // before the first scan; above that the LDS copy does not fit beside the
  // other arrays, and each thread reads the token of the slot at each of its
  // order positions (the order array is a permutation of the slots, so my_ord
  // is in range).
  int my_old[SPT];
  if constexpr (kLdsTok) {
    uint32_t w[SPT];
    load_words<SPT>(slot2tok + pl, w);
#pragma unroll
    for (int q = 0; q < SPT; ++q) my_old[q] = (int)w[q];
  } else {
#pragma unroll
    for (int q = 0; q < SPT; ++q)
      my_old[q] = slot2tok[KVS_DEVICE_CHECKS ? min(my_ord[q], S - 1) : my_ord[q]];
  }
  if (owns) {
    zero_bytes<SPT>(flag + p0);
    // positions past S keep slot 0; every position below S is written once below
    zero_bytes<2 * SPT>(reinterpret_cast<uint8_t*>(lorder + p0));
  }
  // 1a. slot lookup of every entry, issued before the first barrier and not
  //     used before it (an entry outside [0, N) reads token 0's slot; the
  //     validation after the barrier discards it)
  int my_slot[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int tok = my_tok[j];
    my_slot[j] = tok2slot[tok >= 0 && (long long)tok < a.N ? tok : 0];
  }
  // This thread's run of last_used, rewritten below with wide stores (the
  // touched slots stamped t): a store per touched slot scatters each wave's
  // stores over sixteen cache lines per instruction, about one address-unit
  // clock each.  Loaded after the lookups, which the next steps wait for
  // first.  Above 8 slots per thread the run does not fit the registers
  // beside the rest, and each touched slot is stamped on its own.
  constexpr bool kLuWide = SPT <= 8;
  uint32_t my_lu[kLuWide ? SPT : 1];
  if constexpr (kLuWide) load_words<SPT>(lu + pl, my_lu);
  for (int h = tid; h < H; h += kDiffThreads) hash[h] = -1;
  if (tid == 0) {
    err_bits = 0;
    n_evict = 0;
  }
  __syncthreads();

  // 1b. validation and hit flags.  my_slot: >= 0 hit slot, -1 miss, -2 empty
  //     entry of a padded Top-K; a looked-up slot outside [-1, S) means the
  //     map was corrupted.  A token given twice is resident in one slot
  //     (the second flag set of that slot reveals it) or in none (misses go
  //     through an LDS open-addressing set of tokens).
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = i0 + j;
    if (j < kpt && i < K) {
      const int tok = my_tok[j];
      if (a.padded && tok == -1) {
        my_slot[j] = -2;
      } else if (tok < 0 || (long long)tok >= a.N) {
        atomicOr(&err_bits, 1);
      } else if (my_slot[j] < -1 || my_slot[j] >= S) {
        atomicOr(&err_bits, 4);   // a map entry no step writes: corrupted state
      } else {
        if (my_slot[j] >= 0) {
          const unsigned bit = 1u << ((my_slot[j] & 3) * 8);   // flag byte := 1
          if (atomicOr(&flagw[my_slot[j] >> 2], bit) & bit) atomicOr(&err_bits, 2);
        } else {
          unsigned h = ((unsigned)tok * 2654435761u) >> (32 - a.hash_bits);
          while (true) {
            const int prev = atomicCAS(&hash[h], -1, tok);
            if (prev == -1) break;
            if (prev == tok) {
              atomicOr(&err_bits, 2);
              break;
            }
            h = (h + 1) & (unsigned)(H - 1);
          }
        }
      }
    }
  }
  if constexpr (KVS_DEVICE_CHECKS) {
    // the state the normal build trusts: the LRU order lists every slot once
    // (bit 7 of the slot's flag byte marks it seen; cleared below, before the
    // flags are read) and every slot's token lies in [-1, N)
#pragma unroll
    for (int q = 0; q < SPT; ++q) {
      const int p = p0 + q;
      if (p < S) {
        const int s = my_ord[q];
        if (!in_bounds(s, S, a.status, KVS_SITE_LRU_ORDER)) {
          atomicOr(&err_bits, 8);
        } else {
          const unsigned bit = 0x80u << ((s & 3) * 8);
          if (atomicOr(&flagw[s >> 2], bit) & bit) {
            latch_bounds(a.status, KVS_SITE_LRU_ORDER, s);
            atomicOr(&err_bits, 8);
          }
        }
        if (!in_range(my_old[q], -1, a.N, a.status, KVS_SITE_SLOT_TOKEN)) atomicOr(&err_bits, 8);
      }
    }
  }
  __syncthreads();
  if (err_bits) {   // invalid Top-K or map: leave the unit untouched, latch the error
    if (tid == 0) {
      a.counts[4 * b + 0] = 0;
      a.counts[4 * b + 1] = 0;
      a.counts[4 * b + 2] = 0;
      a.counts[4 * b + 3] = 0;
      atomicCAS(a.status, 0,
                (err_bits & 1)   ? KVS_ERANGE
                : (err_bits & 4) ? KVS_ECORRUPT
                : (err_bits & 2) ? KVS_EDUP
                                 : KVS_EBOUNDS);
    }
    return;
  }

  // 2 + 3. The two order-preserving compactions share one scan: misses in
  //    Top-K order (low 16 bits, m <= K <= 8192) and non-hit slots in LRU
  //    order (high 16 bits, at most S <= 16384).  The hit slots are distinct
  //    (a repeat was rejected above), so n_hit = S - non-hit slots.
  if constexpr (KVS_DEVICE_CHECKS) {   // each slot's flag byte belongs to its order position
#pragma unroll
    for (int q = 0; q < SPT; ++q)
      if (p0 + q < S) flag[my_ord[q]] &= 0x7f;
  }
  // 2. sparse diff: record slot_of, compact misses in Top-K order
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = i0 + j;
    if (j < kpt && i < K) {
      a.slot_of[bk + i] = my_slot[j];
      // a miss's row slot is its victim, written once in step 5
      if (my_slot[j] != -1) a.row_slot[bk + i] = my_slot[j] >= 0 ? my_slot[j] : -1;
      if (my_slot[j] == -1) ++cnt;
    }
  }
  // bit q: order position p0 + q holds a non-hit slot (each slot sits at one
  // order position, so no other thread writes these flags before the victims
  // below read the mask instead of the flags)
  // (the flag reads are unconditional, so they are issued together; the order
  // entries of positions past S are slot 0)
  unsigned nonhit = 0;
#pragma unroll
  for (int q = 0; q < SPT; ++q) {
    const bool free_slot = flag[min(my_ord[q], Sp - 1)] == 0;
    if (p0 + q < S && free_slot) {
      cnt += 1 << 16;
      nonhit |= 1u << q;
    }
  }
  if (kLdsTok && owns) {   // read after the scan's barrier
    if constexpr (SPT >= 4) {
#pragma unroll
      for (int v = 0; v < SPT / 4; ++v)
        reinterpret_cast<int4*>(s2t + p0)[v] =
            make_int4(my_old[4 * v], my_old[4 * v + 1], my_old[4 * v + 2], my_old[4 * v + 3]);
    } else {
#pragma unroll
      for (int q = 0; q < SPT; ++q) s2t[p0 + q] = my_old[q];
    }
  }
  int packed;
  const int ex = wg_exclusive_scan(cnt, wtot[0], packed);
  const int m = packed & 0xffff;
  const int n_hit = S - (packed >> 16);
  // the token of the slot at each of this thread's order positions, read
  // before any write below (victims use it).  The victims are the first m
  // non-hit entries of the order, in the first few threads: the others skip
  // these LDS reads (whole waves branch around them).
  int vold[SPT];
  if constexpr (kLdsTok) {
    if ((ex >> 16) < m) {
#pragma unroll
      for (int q = 0; q < SPT; ++q) vold[q] = s2t[min(my_ord[q], Sp - 1)];
    } else {
#pragma unroll
      for (int q = 0; q < SPT; ++q) vold[q] = -1;   // never read: no victim here
    }
  } else {
#pragma unroll
    for (int q = 0; q < SPT; ++q) vold[q] = my_old[q];
  }
  int r = ex & 0xffff;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = i0 + j;
    if (j < kpt && i < K && my_slot[j] == -1 &&
        in_bounds(r, K, a.status, KVS_SITE_DIFF_LIST)) {
      lmiss[r] = i;
      lmtok[r++] = my_tok[j];
    }
  }

  // 3. victims: the first m non-hit slots of the LRU order; the other
  //    non-hit slots keep their relative order at the front of the new order
  //    (built in LDS, written out below).  Each slot sits at one order
  //    position, so each flag byte below is written by one thread only.  The
  //    victims sit at the front of the order, in the first few threads: with
  //    the slot tokens in LDS their eviction stores wait for the map update,
  //    which spreads them over every thread.
  r = ex >> 16;
  int my_evict = 0;
#pragma unroll
  for (int q = 0; q < SPT; ++q) {
    if ((nonhit >> q) & 1u) {
      const int s = my_ord[q];
      if (r < m) {
        lvict[r] = s;
        flag[s] = 2;
        const int old = vold[q];
        if (old >= 0) ++my_evict;
        if constexpr (!kLdsTok) {
          a.evicted[bk + r] = old;
          if (old >= 0) tok2slot[old] = -1;   // evicted tokens are outside the Top-K set
        }
      } else if (in_bounds(r - m, S, a.status, KVS_SITE_DIFF_LIST)) {
        lorder[r - m] = (uint16_t)s;
      }
      ++r;
    }
  }
  // one LDS atomic per wave (the wave's sum sits in its last lane): an
  // atomic per thread on the one word serialises up to 1024 updates
  const int wave_evict = wave_inclusive_scan(my_evict);
  if ((tid & 63) == 63 && wave_evict != 0) atomicAdd(&n_evict, wave_evict);
  __syncthreads();

  // 4. the n_hit + m touched slots (hits and victims, all stamped t) close the
  //    order, ascending by slot.  The same scan counts the empty entries
  //    (high 16 bits), which places each thread's hits in the hit list.  The
  //    flags of slots past S are zero (cleared, never set).
  const unsigned touched = owns ? nonzero_bytes<SPT>(flag + p0) : 0u;
  cnt = __builtin_popcount(touched);
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (j < kpt && i0 + j < K && my_slot[j] == -2) cnt += 1 << 16;
  int n_touched;
  const int ex2 = wg_exclusive_scan(cnt, wtot[1], n_touched);
  // touched slots are stamped t here, from each thread's own contiguous
  // slots (where stamping each hit and victim through its slot index would
  // scatter the stores), in the run of last_used written back whole below
  r = S - (n_hit + m) + (ex2 & 0xffff);
#pragma unroll
  for (int q = 0; q < SPT; ++q) {
    if ((touched >> q) & 1u) {
      const int s = p0 + q;
      if constexpr (kLuWide) my_lu[q] = (uint32_t)t;
      else lu[s] = t;
      if (in_bounds(r, S, a.status, KVS_SITE_DIFF_LIST)) lorder[r++] = (uint16_t)s;
    }
  }
  if constexpr (kLuWide) {
    if (owns) store_words<SPT>(lu + p0, my_lu);
  }
  // hits in Top-K order: entries before this thread's, less its misses and empties
  r = i0 - (ex & 0xffff) - (ex2 >> 16);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = i0 + j;
    if (j < kpt && i < K && my_slot[j] >= 0 && in_bounds(r, K, a.status, KVS_SITE_DIFF_LIST)) {
      a.hit_pos[bk + r] = i;
      a.hit_slot[bk + r++] = my_slot[j];
    }
  }
  if (tid == 0) {   // n_evict is final after the barrier that follows the victims
    a.counts[4 * b + 0] = n_hit;
    a.counts[4 * b + 1] = m;
    a.counts[4 * b + 2] = n_evict;
    a.counts[4 * b + 3] = 1;
    unsigned long long* st = reinterpret_cast<unsigned long long*>(a.stats + 4 * u);
    atomicAdd(st + 0, 1ull);   // no return value is used: the adds do not stall
    atomicAdd(st + 1, (unsigned long long)n_hit);
    atomicAdd(st + 2, (unsigned long long)m);
    atomicAdd(st + 3, (unsigned long long)n_evict);
    a.stepctr[u] = t + 1;
  }

  __syncthreads();   // the new order is complete in LDS
  // each thread writes its run of the new order with one wide store
  if (owns) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(lorder + p0);
    uint8_t* dst = reinterpret_cast<uint8_t*>(gorder + p0);
    if constexpr (SPT >= 8) {
#pragma unroll
      for (int v = 0; v < SPT / 8; ++v)
        reinterpret_cast<u32x4*>(dst)[v] = reinterpret_cast<const u32x4*>(src)[v];
    } else if constexpr (SPT == 4) {
      *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
    } else if constexpr (SPT == 2) {
      *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
    } else {
      *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(src);
    }
  }

  // 5. map update: the j-th miss takes the j-th victim (and, with the slot
  //    tokens in LDS, the victim's old token leaves the map here)
  for (int j = tid; j < m; j += kDiffThreads) {
    const int i = lmiss[j];
    const int tok = lmtok[j];
    const int v = lvict[j];
    if (!in_bounds(v, S, a.status, KVS_SITE_DIFF_LIST)) continue;
    if constexpr (kLdsTok) {
      const int old = s2t[v];
      a.evicted[bk + j] = old;
      if (old >= 0) tok2slot[old] = -1;   // evicted tokens are outside the Top-K set
    }
    slot2tok[v] = tok;
    tok2slot[tok] = v;
    a.miss_pos[bk + j] = i;
    a.miss_tok[bk + j] = tok;
    a.victims[bk + j] = v;
    a.row_slot[bk + i] = v;
  }
}

// ------------------------------------------------------------------ gather
// LDS the gather launches reserve (and do not use): at most two workgroups of
// it fit a CU.  The index copy runs faster with two resident per CU than with
// the three its registers allow (70.5 % of the 8 TB/s peak instead of 69.2 %
// at 128K x 32, 151 MB per launch: fewer waves contend for the same HBM
// channels).
constexpr int kCopyLdsReserve = 64 << 10;
// Host reads in flight, at one per fetch thread, below which the separate
// gather issues all of a pass's reads at once (see its fetch role).
constexpr long long kDeepFetchBytes = 384ll << 10;
constexpr int kCopyThreads = 256;
constexpr int kCopyRows = 32;                                   // rows per block iteration
constexpr int kCopyItems = kRowChunks / 8;                      // 9 chunks / thread
static_assert(kCopyRows * 8 == kCopyThreads && kCopyItems * 8 == kRowChunks, "copy tiling");

struct GatherArgs {
  const u32x4* pool;       // host pool (pinned, GPU-mapped) [B][L][N] rows
  u32x4* hot;              // [B][L][S] rows
  u32x4* cbuf;             // [B][K] rows
  const int32_t* slot_of;  // [B][K]
  const int32_t* miss_pos; // [B][K]
  const int32_t* miss_tok; // [B][K]: tokens of the misses, in Top-K order
  const int32_t* victims;  // [B][K]
  const int32_t* counts;   // [B][4]
  long long N;
  int S, K, L, B, layer;
  int fetch_per_req;       // miss-role workgroups per request
  int fetch_wgs;           // fetch_per_req * B
  int hit_wgs;             // hit-role workgroups (each loops over 32-position groups)
  int hits_first;          // 0: fetch workgroups take the first grid indices; 1: hit ones do
  int write_cbuf;          // 0: rows are read in place from the hot buffer (no compute buffer)
  int deep_fetch;          // 1: a unit's pool rows span under 4 GiB (N * 1152 bytes)
  int32_t* status;         // checked build: bounds failures
};

// The index copy of one layer.  Workgroups [0, fetch_wgs) fetch misses: row =
// pool[b][l][tok_j] read straight from pinned host memory over PCIe, written to
// cbuf[b][miss_pos_j] and to the victim slot hot[b][l][v_j].  The remaining
// workgroups copy hits hot[b][l][slot_of_i] -> cbuf[b][i] within HBM.  One
// launch keeps both on one stream; the fetch workgroups come first so the host
// link starts as early as possible.  Hit slots and victim slots are disjoint,
// so the two roles never touch the same hot row.
__global__ __launch_bounds__(kCopyThreads) void gather_kernel(GatherArgs a) {
  const int K = a.K;
  const int id = a.hits_first ? ((int)blockIdx.x + a.fetch_wgs) % (a.fetch_wgs + a.hit_wgs)
                              : (int)blockIdx.x;
  if (id < a.fetch_wgs) {
    // fetch role: 32 rows per workgroup pass; chunk c = 256 j + thread of the
    // pass's 32 x 72 chunks, so each wave instruction reads 1 KB of
    // consecutive host memory (1-2 rows); the host link is measurably faster
    // with this order than with one row per 8 threads
    const int b = id / a.fetch_per_req;
    const int x = id - b * a.fetch_per_req;
    if (a.counts[4 * b + 3] == 0) return;
    const int n = a.counts[4 * b + 1];
    const long long u = (long long)b * a.L + a.layer;
    const long long bk = (long long)b * K;
    // Two ways to issue a pass's host reads.  Where the workgroups that have
    // misses hold kDeepFetchBytes or more with one read per thread, each
    // thread keeps one read in flight, the lists of a chunk loaded just before
    // its read: enough for the link, and more outstanding host reads
    // measurably slow it.  Below that the link idles on round trips, so the
    // pass's lists are loaded first and all its reads go out at once, through
    // a buffer resource over the unit's pool rows: chunks past the misses
    // read nothing, and no load sits under a branch (which would make the
    // compiler's in-order wait counts path-dependent, its waits for later
    // lists then draining the reads).  The resource needs the unit's rows
    // below 4 GiB.  The estimate takes every request's misses as this one's.
    const long long active =
        (long long)a.B * min(a.fetch_per_req, (n + kCopyRows - 1) / kCopyRows);
    const bool deep = a.deep_fetch && active * kCopyThreads * 16 < kDeepFetchBytes;
    const __amdgpu_buffer_rsrc_t psrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.pool + u * a.N * kRowChunks), (short)0,
        deep ? (int)(unsigned)(a.N * kRowBytes) : 0, kBufRsrcWord3);
    for (int j0 = x * kCopyRows; j0 < n; j0 += a.fetch_per_req * kCopyRows) {
      // per chunk only the Top-K position and the victim slot are kept (32-bit)
      // while the host loads are in flight; addresses are rebuilt for the stores
      u32x4 v[kCopyItems];
      int pos[kCopyItems], vic[kCopyItems];
      if (deep) {
        int tok[kCopyItems];
#pragma unroll
        for (int j = 0; j < kCopyItems; ++j) {
          const int jm = min(j0 + (j * kCopyThreads + (int)threadIdx.x) / kRowChunks, n - 1);
          tok[j] = a.miss_tok[bk + jm];
          pos[j] = a.miss_pos[bk + jm];
          vic[j] = a.victims[bk + jm];
        }
#pragma unroll
        for (int j = 0; j < kCopyItems; ++j) {
          const int c = j * kCopyThreads + threadIdx.x;
          const int r = c / kRowChunks;
          const int col = c - r * kRowChunks;
          const bool in = j0 + r < n && in_bounds(tok[j], a.N, a.status, KVS_SITE_MISS) &&
                          in_bounds(pos[j], K, a.status, KVS_SITE_MISS) &&
                          in_bounds(vic[j], a.S, a.status, KVS_SITE_MISS);
          if (!in) pos[j] = -1;
          const unsigned off = in ? (unsigned)tok[j] * kRowBytes + col * 16
                                  : (unsigned)(a.N * kRowBytes);   // out of range: zeros
          v[j] = __builtin_amdgcn_raw_buffer_load_b128(psrc, (int)off, 0, 0);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kCopyItems; ++j) {
          const int c = j * kCopyThreads + threadIdx.x;
          const int r = c / kRowChunks;
          const int col = c - r * kRowChunks;
          const int jj = j0 + r;
          pos[j] = -1;
          if (jj < n) {
            const int tok = a.miss_tok[bk + jj];
            const int i = a.miss_pos[bk + jj];
            const int vs = a.victims[bk + jj];
            if (!in_bounds(i, K, a.status, KVS_SITE_MISS) ||
                !in_bounds(tok, a.N, a.status, KVS_SITE_MISS) ||
                !in_bounds(vs, a.S, a.status, KVS_SITE_MISS))
              continue;
            v[j] = a.pool[(u * a.N + tok) * kRowChunks + col];
            pos[j] = i;
            vic[j] = vs;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kCopyItems; ++j) {
        if (pos[j] >= 0) {
          const int c = j * kCopyThreads + threadIdx.x;
          const int col = c - (c / kRowChunks) * kRowChunks;
          if (a.write_cbuf) st_row(a.cbuf + (bk + pos[j]) * kRowChunks + col, v[j]);
          st_row(a.hot + (u * a.S + vic[j]) * kRowChunks + col, v[j]);
        }
      }
    }
    return;
  }
  // hit role: 8 threads per row, 32 rows per pass; thread (row, sub) moves the
  // 16-byte chunks sub, sub + 8, ..., sub + 64 of its row, so each wave
  // instruction covers eight whole 128-byte lines
  const int rsub = threadIdx.x >> 3;
  const int sub = threadIdx.x & 7;
  // hit role: workgroup h copies 32-position groups h, h + hit_wgs, ... over all
  // requests' Top-K positions (request-major)
  const int groups_per_req = (K + kCopyRows - 1) / kCopyRows;
  const long long n_groups = (long long)groups_per_req * a.B;
  for (long long grp = id - a.fetch_wgs; grp < n_groups; grp += a.hit_wgs) {
    const int b = (int)(grp / groups_per_req);
    const int x = (int)(grp - (long long)b * groups_per_req);
    const int i = x * kCopyRows + rsub;
    // the request's valid flag and the slot are loaded together (the slot
    // index is clamped into the request's K entries and discarded below when
    // the position lies past K): one round trip before the row loads, not two
    const int valid = a.counts[4 * b + 3];
    const int s = a.slot_of[(long long)b * K + min(i, K - 1)];
    if (valid == 0 || i >= K) continue;
    if (s == -1) continue;   // a miss: the fetch role writes it
    if (!in_range(s, -2, a.S, a.status, KVS_SITE_HIT)) continue;
    u32x4* dst = a.cbuf + ((long long)b * K + i) * kRowChunks + sub;
    if (s < 0) {             // an empty entry of a padded Top-K gathers a zero row
#pragma unroll
      for (int j = 0; j < kCopyItems; ++j) st_row(dst + 8 * j, u32x4{0u, 0u, 0u, 0u});
      continue;
    }
    const long long u = (long long)b * a.L + a.layer;
    const u32x4* src = a.hot + (u * a.S + s) * kRowChunks + sub;
    u32x4 v[kCopyItems];
#pragma unroll
    for (int j = 0; j < kCopyItems; ++j) v[j] = ld_row(src + 8 * j);
#pragma unroll
    for (int j = 0; j < kCopyItems; ++j) st_row(dst + 8 * j, v[j]);
  }
}

// ------------------------------------------------------------------ attention
constexpr int kAttnThreads = 512;               // 8 waves
constexpr int kTile = 64;                       // tokens per LDS tile
constexpr int kLdsRow = kRowBytes;              // LDS row stride; chunks are XOR-swizzled
constexpr int kAttnItems = kRowChunks / 8;      // 9 chunks / thread, 8 threads per row
constexpr int kKSteps = kRowElems / 32;         // 18 MFMA k-steps over 576 dims
constexpr int kKHalf = kKSteps / 2;             // each Q.K^T wave takes half of them
constexpr int kPRow = kTile + 8;                // bf16 P row stride (144 B)
constexpr int kMaxParts = 256;   // attention partials per request merged by the combine
static_assert(kTile * 8 == kAttnThreads && kAttnItems * 8 == kRowChunks, "attention tiling");
static_assert(kKHalf * 2 == kKSteps, "k split");

// LDS placement of the 16-byte chunk c of tile row r: chunk c ^ sw(r) of the
// row (the XOR stays inside c's aligned group of 8 chunks).  With 1152-byte rows
// (288 dwords, so odd rows start half-way round the 64 banks) this spreads
//  - a wave's row stores (8 rows x 128 B) and the Q.K^T operand reads (16 rows
//    x 4 chunks) evenly over the banks, and
//  - the P.V operand reads (2-byte values of 4 rows 8 apart, 16 columns each)
//    over distinct banks.
__device__ __forceinline__ int lds_swz(int r) {
  return (((r >> 3) & 3) << 1) ^ (((r >> 1) & 1) << 2);
}

struct AttnArgs {
  const uint16_t* cbuf;     // [B][K][576]: assembled rows (direct == 0)
  const uint16_t* hot;      // [B*L][S][576]: hot buffer, rows read in place (direct == 1)
  const uint16_t* q;        // [B][16][576]
  const int32_t* slot_of;   // [B][K]: -2 marks an empty entry of a padded Top-K
  const int32_t* row_slot;  // [B][K]: slot of position i's row, -1 empty
  const int32_t* counts;    // [B][4]
  float* part_o;            // [B][parts][16][512]
  float* part_ml;           // [B][parts][16][2]
  int K, B, S, L, layer;
  int wgs;                  // workgroups sharing the B * ceil(K/64) tiles
  int parts;                // partials per request (the most workgroups one request spans)
  int padded;               // 1: mask the empty entries of a padded Top-K
  float scale_log2;         // softmax scale * log2(e): scores are kept in log2 units
  uint16_t* out;            // [B][16][512] bf16 when parts == 1 (no combine), else null
  float* lse;               // [B][16] or null; written here only when out is
  int32_t* status;          // checked build: bounds failures
};

// One 64-row tile in LDS: scores of the 16 heads against every row, the
// online softmax update and P.V.  Rows at or past n_valid, and rows whose mark
// equals pad_mark, score -inf.  Starts after the barrier that published the
// tile.  Two barriers inside: after the scores (sc complete; every wave is
// past the previous tile's P.V) and after the softmax (pb and alpha_s
// complete).  mid() runs in every thread between them, beside the softmax:
// work that must follow the previous tile's P.V and be published before the
// next tile's scores (the double-buffered attention stores the next tile
// there).  There is no barrier at the end: the caller keeps the tile, sc, pb
// and alpha_s unwritten until the next such barrier.
// MFMA operand layout used (v_mfma_f32_16x16x32_bf16): lane l supplies row
// (l % 16) of A and column (l % 16) of B with 8 consecutive k-values selected
// by l / 16; the result lane l holds rows 4*(l/16)+j, column l % 16.  Both
// operands of each product take their k-values through the same
// (l/16, j) -> k assignment, so the sum is over the intended k.
// Wave roles:
//   Q.K^T   wave w: tokens 16*(w % 4) .. +16, k-steps 9*(w / 4) .. +9 (two
//           partial score tiles per token block, summed in the softmax);
//   softmax waves 0..3: 16 lanes (one DPP row) per head, 4 tokens each;
//   P.V     wave w: value columns 64*w .. +64 (4 MFMA column tiles), the
//           value operand through transpose LDS reads.
// State per thread: qf (Q fragments, head r16, this wave's k-half), m_run /
// l_run (running max in log2 units and sum of its head, replicated over the
// head's 16 softmax threads), acc (O[h = 4g + j][e = 64w + 16nt + r16]).
template <class Mid>
__device__ __forceinline__ void attend_tile_mid(const unsigned char* kv, float* sc, uint16_t* pb,
                                                float* alpha_s, const int* vmark,
                                                const bf16x8 (&qf)[kKHalf], float& m_run,
                                                float& l_run, f32x4 (&acc)[4], int n_valid,
                                                int pad_mark, float scale_log2, Mid&& mid) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int tt = wave & 3, kh = wave >> 2;
  const bool sm_on = tid < kHeads * 16;
  const int c4 = (tid & 15) * 4;
  // partial scores of 16 tokens over half of the 576 dims
  {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    const int krow_i = tt * 16 + r16;
    const unsigned char* krow = kv + krow_i * kLdsRow;
    const int ksw = lds_swz(krow_i);
#pragma unroll
    for (int ks = 0; ks < kKHalf; ++ks) {
      const int chunk = (kh * kKHalf + ks) * 4 + g;   // dims chunk*8 .. +7
      const bf16x8 kf =
          as_bf16x8(*reinterpret_cast<const u32x4*>(krow + (chunk ^ ksw) * 16));
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], kf, s, 0, 0, 0);
    }
    float* sck = sc + kh * kHeads * kTile;
#pragma unroll
    for (int j = 0; j < 4; ++j) sck[(4 * g + j) * kTile + tt * 16 + r16] = s[j];
  }
  __syncthreads();

  // online softmax: head h = tid / 16 (threads 0..255, whole waves), tokens
  // c4 .. c4 + 3; rows past n_valid and empty entries score -inf.  The max and
  // the sum stay inside one 16-lane DPP row.
  if (sm_on) {
    const int h = tid >> 4;
    const float4 s0 = *reinterpret_cast<const float4*>(sc + h * kTile + c4);
    const float4 s1 = *reinterpret_cast<const float4*>(sc + kHeads * kTile + h * kTile + c4);
    const float z[4] = {s0.x + s1.x, s0.y + s1.y, s0.z + s1.z, s0.w + s1.w};
    const int4 mk = *reinterpret_cast<const int4*>(vmark + c4);
    const int mks[4] = {mk.x, mk.y, mk.z, mk.w};
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      x[k] = c4 + k < n_valid && mks[k] != pad_mark ? z[k] * scale_log2 : -INFINITY;
    const float m_new = fmaxf(m_run, row16_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]))));
    // no scored token yet (empty entries only): keep every weight at 0
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_ref);
    float p[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = exp2f(x[k] - m_ref);
    l_run = l_run * alpha + row16_sum((p[0] + p[1]) + (p[2] + p[3]));
    m_run = m_new;
    *reinterpret_cast<uint2*>(pb + h * kPRow + c4) =
        make_uint2((uint32_t)f32_to_bf16_rne(p[0]) | ((uint32_t)f32_to_bf16_rne(p[1]) << 16),
                   (uint32_t)f32_to_bf16_rne(p[2]) | ((uint32_t)f32_to_bf16_rne(p[3]) << 16));
    if ((tid & 15) == 0) alpha_s[h] = alpha;
  }
  mid();
  __syncthreads();

  // P.V: wave w owns value columns [64w, 64w + 64) as 4 MFMA column tiles
  {
    float al[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) al[j] = alpha_s[4 * g + j];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[nt][j] *= al[j];
    // B operand by transpose reads (ds_read_b64_tr_b16): within each
    // 16-lane block, lane c receives element c % 4 of the 8-byte row piece
    // addressed by lane 4j + c / 4, for j = 0..3.  Lane a = r16 of block g
    // therefore addresses V[row0 + a / 4][n0 + 4 (a % 4) .. +3], and lane
    // (g, r16) receives V[row0 + j][n0 + r16], j = 0..3: four consecutive
    // k-values of column n0 + r16.  Two reads (rows +0 and +4) give the 8
    // k-values 8g .. 8g + 7 of the MFMA's B operand.
    const int tr_row = g * 8 + (r16 >> 2);
    const int tr_sub = (r16 & 1) * 8;            // byte offset inside the 16-byte chunk
#pragma unroll
    for (int kk = 0; kk < kTile / 32; ++kk) {
      const bf16x8 pf =
          as_bf16x8(*reinterpret_cast<const u32x4*>(pb + r16 * kPRow + kk * 32 + g * 8));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int chunk = wave * 8 + nt * 2 + ((r16 & 3) >> 1);   // column (n0 + 4(a%4)) / 8
        const int r0 = kk * 32 + tr_row, r1 = r0 + 4;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(kv + r0 * kLdsRow + ((chunk ^ lds_swz(r0)) * 16) + tr_sub));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(kv + r1 * kLdsRow + ((chunk ^ lds_swz(r1)) * 16) + tr_sub));
        const u16x8 vv = {(uint16_t)lo[0], (uint16_t)lo[1], (uint16_t)lo[2], (uint16_t)lo[3],
                          (uint16_t)hi[0], (uint16_t)hi[1], (uint16_t)hi[2], (uint16_t)hi[3]};
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            pf, __builtin_bit_cast(bf16x8, vv), acc[nt], 0, 0, 0);
      }
    }
  }
}

// The tile routine with nothing between its barriers and a barrier at the
// end, after which the tile, sc, pb and alpha_s may be overwritten (one LDS
// tile: the assembling launch).
__device__ __forceinline__ void attend_tile(unsigned char* kv, float* sc, uint16_t* pb,
                                            float* alpha_s, const int* vmark,
                                            const bf16x8 (&qf)[kKHalf], float& m_run,
                                            float& l_run, f32x4 (&acc)[4], int n_valid,
                                            int pad_mark, float scale_log2) {
  attend_tile_mid(kv, sc, pb, alpha_s, vmark, qf, m_run, l_run, acc, n_valid, pad_mark,
                  scale_log2, [] {});
  __syncthreads();
}

// Workgroup w of `wgs` takes the tiles [w*G/wgs, (w+1)*G/wgs) of the G =
// B * ntiles tiles of every request's gathered rows in request-major order
// (an even share whatever B is: at 192 requests, 24 tiles each on 256
// workgroups instead of 32 on 192).  Its share is one or more segments, each
// the tiles [tb, te) of one request, through attend_tile; each segment writes
// one partial, the segment's index among the workgroups that share its
// request (part_slot).  With one partial per request (every request in one
// workgroup) the workgroup writes out and lse itself and no merge runs.
// DIRECT: rows read in place from the hot buffer at row_slot (a separate
// instantiation, so the assembled-buffer path carries no slot loads at all).
__device__ __forceinline__ int share_of(long long g, long long G, int wgs) {
  return (int)(((g + 1) * wgs - 1) / G);   // the workgroup whose share holds tile g
}

template <bool DIRECT>
__global__ __launch_bounds__(kAttnThreads) void attention_kernel(AttnArgs a) {
  // two LDS tiles (158.6 KB in all): one is attended while the next is stored
  __shared__ __attribute__((aligned(16))) unsigned char kv[2][kTile * kLdsRow];
  __shared__ float sc[2 * kHeads * kTile];
  __shared__ __attribute__((aligned(16))) uint16_t pb[kHeads * kPRow];
  __shared__ float alpha_s[kHeads];
  __shared__ __attribute__((aligned(16))) int vmark[2][kTile];   // each tile's empty-entry marks
  __shared__ float inv_l[kHeads];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int kh = wave >> 2;
  const int K = a.K;
  const int ntiles = (K + kTile - 1) / kTile;
  const long long G = (long long)a.B * ntiles;
  const int w = blockIdx.x;
  const long long g0 = (long long)w * G / a.wgs, g1 = (long long)(w + 1) * G / a.wgs;
  const int lrow = tid >> 3, lsub = tid & 7;
  const int lsw = lds_swz(lrow);
  const int pad_mark = DIRECT ? -1 : -2;
  // softmax: threads 0..255, 16 lanes per head (one DPP row)
  const bool sm_on = tid < kHeads * 16;

  for (long long gs = g0; gs < g1;) {
    const int b = (int)(gs / ntiles);
    const int tb = (int)(gs - (long long)b * ntiles);
    const int te = (int)min((long long)ntiles, g1 - (long long)b * ntiles);
    const int part_slot = w - share_of((long long)b * ntiles, G, a.wgs);
    gs = (long long)(b + 1) * ntiles;
    // invalid input, or no entry at all (padded): zero output, lse -inf
    // (written here with one partial per request, by the combine otherwise)
    if (a.counts[4 * b + 3] == 0 || a.counts[4 * b + 0] + a.counts[4 * b + 1] == 0) {
      if (a.out != nullptr) {
        u32x4* ob = reinterpret_cast<u32x4*>(a.out + (long long)b * kHeads * kVDim);
        for (int i = tid; i < kHeads * kVDim / 8; i += kAttnThreads) ob[i] = u32x4{0u, 0u, 0u, 0u};
        if (a.lse != nullptr && tid < kHeads) a.lse[b * kHeads + tid] = -INFINITY;
      }
      continue;
    }

    bf16x8 qf[kKHalf];
    float m_run = -INFINITY, l_run = 0.f;   // per head, replicated over its 16 softmax threads
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // two register buffers: the rows of the next two tiles are in flight while
    // a tile is consumed from LDS
    u32x4 ra[kAttnItems], rb[kAttnItems];
    int va, vb;   // empty-entry mark of this thread's tile row, stored to LDS with the rows
    // 8 threads per row: thread (row tid / 8, sub tid % 8) moves chunks sub + 8j.
    // The rows are read through a buffer resource that spans this request's K
    // rows: the hardware range check returns zeros for rows >= K and for the
    // out-of-range offset given for tiles past te.  So every load is issued
    // unconditionally, every path through the loop has the same number of
    // loads in flight, and the wait before a tile's LDS store covers only that
    // tile's own loads (a branch per load would make the count path-dependent
    // and the compiler would then drain everything before each use).
    // Rows: request b's K assembled rows in position order, or (direct) the
    // rows of unit (b, layer)'s hot buffer, indexed by row_slot.
    const uint16_t* base = DIRECT ? a.hot + ((long long)b * a.L + a.layer) * a.S * kRowElems
                                    : a.cbuf + (long long)b * K * kRowElems;
    const int rec_bytes = (DIRECT ? a.S : K) * kRowBytes;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, rec_bytes, kBufRsrcWord3);
    // row_slot of this thread's tile row, loaded one tile ahead of the rows
    // (DIRECT instantiation only)
    const __amdgpu_buffer_rsrc_t ssrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.row_slot + (long long)b * K), (short)0, DIRECT ? K * 4 : 0, kBufRsrcWord3);
    // The entry of each tile row that marks an empty position (slot_of -2, or
    // row_slot -1 when DIRECT) travels with the row and is stored beside it.
    // Without padding the resource is empty: the loads return 0 (valid) and
    // read nothing.
    const __amdgpu_buffer_rsrc_t vsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((DIRECT ? a.row_slot : a.slot_of) + (long long)b * K), (short)0,
        a.padded ? K * 4 : 0, kBufRsrcWord3);
    auto load_slot = [&](int tile) -> int {
      if (!DIRECT) return 0;
      return __builtin_amdgcn_raw_buffer_load_b32(
          ssrc, tile < te ? (tile * kTile + lrow) * 4 : K * 4, 0, 0);
    };
    auto load_tile = [&](u32x4 (&dst)[kAttnItems], int& dv, int tile, int slot) {
      const int tok = tile * kTile + lrow;
      const bool in = tile < te && tok < K;
      const bool ok = !DIRECT || !in || in_range(slot, -1, a.S, a.status, KVS_SITE_ROW_SLOT);
      const int off = !in || !ok ? rec_bytes
                      : DIRECT   ? (slot >= 0 ? slot * kRowBytes + lsub * 16 : rec_bytes)
                                 : tok * kRowBytes + lsub * 16;
#pragma unroll
      for (int j = 0; j < kAttnItems; ++j)
        dst[j] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + j * 128, 0, kNT);
      dv = __builtin_amdgcn_raw_buffer_load_b32(vsrc,
                                                tile < te ? (tile * kTile + lrow) * 4 : K * 4, 0,
                                                0);
    };
    auto store_tile = [&](const u32x4 (&src)[kAttnItems], int mark, int buf) {
      unsigned char* d = kv[buf] + lrow * kLdsRow + ((lsub ^ lsw) * 16);
#pragma unroll
      for (int j = 0; j < kAttnItems; ++j) *reinterpret_cast<u32x4*>(d + j * 128) = src[j];
      if (lsub == 0) vmark[buf][lrow] = mark;
    };

    // tile `tile` from LDS buffer buf: scores, online softmax, P.V, with
    // mid() between the tile routine's two barriers
    auto compute = [&](int tile, int buf, auto&& mid) {
      attend_tile_mid(kv[buf], sc, pb, alpha_s, vmark[buf], qf, m_run, l_run, acc,
                      K - tile * kTile, pad_mark, a.scale_log2, mid);
    };

    // Tiles two at a time so the buffers alternate without copies.  At the
    // top of each iteration LDS buffer 0 holds `tile` (published), rb holds
    // tile + 1 and ra tile + 2 (in flight).  While a tile is attended, the
    // register tile after it is stored to the other LDS buffer between the
    // tile routine's barriers (every wave is past that buffer's last P.V by
    // then, and the second barrier publishes it) and its register buffer is
    // reloaded at once, two tiles ahead: two barriers per tile, and each load
    // has two tiles of time before its store.
    {
      // the previous segment's last tile may still be read by slower waves
      __syncthreads();
      // Q as A-operand fragments: head r16, dims (kh*9 + ks)*32 + g*8 .. +7
      const u32x4* qh =
          reinterpret_cast<const u32x4*>(a.q + ((long long)b * kHeads + r16) * kRowElems);
#pragma unroll
      for (int ks = 0; ks < kKHalf; ++ks) qf[ks] = as_bf16x8(qh[(kh * kKHalf + ks) * 4 + g]);
      // every slot load is issued before the rows of the tile ahead of it, in
      // the prologue as in the loop, so the wait for a slot never covers rows
      int sa = load_slot(tb), sb = load_slot(tb + 1);
      load_tile(ra, va, tb, sa);
      sa = load_slot(tb + 2);
      load_tile(rb, vb, tb + 1, sb);
      sb = load_slot(tb + 3);
      store_tile(ra, va, 0);
      load_tile(ra, va, tb + 2, sa);
      sa = load_slot(tb + 4);
      __syncthreads();
      // full pairs; one exit, so the loads in flight are the same (rb's and
      // ra's) on the back edge and at the exit.  Loads of tiles past te read
      // the out-of-range offset: zeros that nothing attends.
      int tile = tb;
      for (; tile + 1 < te; tile += 2) {
        compute(tile, 0, [&] {
          store_tile(rb, vb, 1);
          load_tile(rb, vb, tile + 3, sb);
          sb = load_slot(tile + 5);
        });
        compute(tile + 1, 1, [&] {
          store_tile(ra, va, 0);
          load_tile(ra, va, tile + 4, sa);
          sa = load_slot(tile + 6);
        });
      }
      if (tile < te) compute(tile, 0, [] {});   // odd tile count: buffer 0 holds the last tile
    }

    // acc lane holds O[h = 4g + j][e = 64w + 16nt + r16]
    if (a.out != nullptr) {
      // one partial per request: this workgroup saw every token, so it
      // finishes the request with the combine's arithmetic (weight
      // 2^(m - m) = 1): out = O / l, lse = (m + log2 l) ln 2
      if (sm_on && (tid & 15) == 0) {
        const int h = tid >> 4;
        inv_l[h] = 1.f / l_run;
        if (a.lse != nullptr)
          a.lse[b * kHeads + h] = (m_run + log2f(l_run)) * 0.69314718055994531f;
      }
      __syncthreads();
      uint16_t* ob = a.out + (long long)b * kHeads * kVDim;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ob[(4 * g + j) * kVDim + wave * 64 + nt * 16 + r16] =
              f32_to_bf16_rne((0.f + acc[nt][j]) * inv_l[4 * g + j]);   // 0 + x: the
                                                                        // combine's zero sign
      continue;
    }
    // partial of this segment for the combine
    const long long part = (long long)b * a.parts + part_slot;
    float* po = a.part_o + part * kHeads * kVDim;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        po[(4 * g + j) * kVDim + wave * 64 + nt * 16 + r16] = acc[nt][j];
    if (sm_on && (tid & 15) == 0) {
      const int h = tid >> 4;
      a.part_ml[(part * kHeads + h) * 2 + 0] = m_run;
      a.part_ml[(part * kHeads + h) * 2 + 1] = l_run;
    }
  }
}

// ------------------------------------------------------------------ assemble + attend
// The index copy and the attention of one layer in one launch.  Two roles:
//  fetch  workgroup (b, x), x < fetch_per_req: the x-th of fetch_per_req equal
//         shares of request b's miss rows, in passes of up to 64: each row
//         read straight from pinned host memory over PCIe (each wave
//         instruction reads 1 KB of consecutive host memory), written to
//         cbuf[b][miss_pos_j] and to the victim slot hot[b][l][v_j], and
//         attended from LDS; partial hit_per_req + x.
//  hits   workgroup (b, x), x < hit_per_req: the x-th share of request b's hit
//         tiles (64 hits each, Top-K order), read from the hot buffer, written
//         to cbuf[b][hit_pos_j] and attended; partial x.  A request with no
//         miss spreads its hit tiles over its fetch workgroups too.
// Hit rows are resident before the step, so their attention runs while the
// host link delivers the misses; the combine merges every partial of a
// request.  Hit slots and victim slots are disjoint, so the roles never touch
// the same hot row.
struct AssembleArgs {
  const u32x4* pool;        // host pool (pinned, GPU-mapped) [B][L][N] rows
  uint16_t* hot;            // [B*L][S][576]
  uint16_t* cbuf;           // [B][K][576], or null when rows are read in place
  const uint16_t* q;        // [B][16][576]
  const int32_t* slot_of;   // [B][K]: -2 marks an empty entry of a padded Top-K
  const int32_t* hit_pos;   // [B][K]: Top-K positions of the hits, first n_hit valid
  const int32_t* hit_slot;  // [B][K]: their slots
  const int32_t* miss_pos;  // [B][K]: Top-K positions of the misses, first n_miss valid
  const int32_t* miss_tok;  // [B][K]: their tokens
  const int32_t* victims;   // [B][K]: their victim slots
  const int32_t* counts;    // [B][4]
  float* part_o;            // [B][parts][16][512]
  float* part_ml;           // [B][parts][16][2]
  long long N;
  int S, K, L, layer;
  int fetch_per_req, hit_per_req, parts;   // parts = hit_per_req + fetch_per_req
  int fetch_wgs;            // fetch_per_req * B
  int hits_first;           // 1: the hit workgroups take the first grid indices
  int padded;               // 1: zero the compute-buffer rows of empty entries
  float scale_log2;
  int32_t* status;          // checked build: bounds failures
};

__global__ __launch_bounds__(kAttnThreads) void assemble_kernel(AssembleArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char kv[kTile * kLdsRow];
  __shared__ float sc[2 * kHeads * kTile];
  __shared__ __attribute__((aligned(16))) uint16_t pb[kHeads * kPRow];
  __shared__ float alpha_s[kHeads];
  __shared__ __attribute__((aligned(16))) int vmark[kTile];   // all 0: every listed row is valid

  const int n_wgs = (int)gridDim.x;
  const int id = a.hits_first ? ((int)blockIdx.x + a.fetch_wgs) % n_wgs : (int)blockIdx.x;
  const bool fetch = id < a.fetch_wgs;
  int b, x;
  if (fetch) {
    b = id / a.fetch_per_req;
    x = id - b * a.fetch_per_req;
  } else {
    const int h = id - a.fetch_wgs;
    b = h / a.hit_per_req;
    x = h - b * a.hit_per_req;
  }
  if (a.counts[4 * b + 3] == 0) return;   // invalid Top-K: nothing to copy; the combine zeroes out
  const int n_hit = a.counts[4 * b + 0], n_miss = a.counts[4 * b + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15, kh = wave >> 2;
  const int K = a.K;
  const long long u = (long long)b * a.L + a.layer;
  const long long bk = (long long)b * K;

  bf16x8 qf[kKHalf];   // Q fragments: head r16, dims (kh*9 + ks)*32 + g*8 .. +7
  {
    const u32x4* qh =
        reinterpret_cast<const u32x4*>(a.q + ((long long)b * kHeads + r16) * kRowElems);
#pragma unroll
    for (int ks = 0; ks < kKHalf; ++ks) qf[ks] = as_bf16x8(qh[(kh * kKHalf + ks) * 4 + g]);
  }
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (tid < kTile) vmark[tid] = 0;

  // A request with no miss this step leaves its fetch workgroups nothing to
  // fetch: they take shares of its hit tiles beside the hit workgroups.  The
  // split depends only on the step's counts, so it is the same on every run.
  const bool all_hit = n_miss == 0;
  if (fetch && !all_hit) {
    // chunk c = 512 jj + tid of the pass's 64 x 72 chunks: row c / 72, column c % 72
    u32x4* hot = reinterpret_cast<u32x4*>(a.hot);
    u32x4* cbuf = reinterpret_cast<u32x4*>(a.cbuf);
    // this workgroup's share of the request's misses: rows [lo, hi), an equal
    // split by rows (not by 64-row passes), so the request's fetch workgroups
    // finish together
    const int lo = (int)((long long)x * n_miss / a.fetch_per_req);
    const int hi = (int)((long long)(x + 1) * n_miss / a.fetch_per_req);
    for (int j0 = lo; j0 < hi; j0 += kTile) {
      u32x4 v[kAttnItems];
      int pos[kAttnItems], vic[kAttnItems];
#pragma unroll
      for (int jj = 0; jj < kAttnItems; ++jj) {
        const int c = jj * kAttnThreads + tid;
        const int r = c / kRowChunks;
        const int col = c - r * kRowChunks;
        const int jm = j0 + r;
        v[jj] = u32x4{0u, 0u, 0u, 0u};   // rows past the share stay zero in LDS
        pos[jj] = -1;
        if (jm < hi) {
          const int tok = a.miss_tok[bk + jm];
          const int mp = a.miss_pos[bk + jm];
          const int vs = a.victims[bk + jm];
          if (!in_bounds(tok, a.N, a.status, KVS_SITE_MISS) ||
              !in_bounds(mp, K, a.status, KVS_SITE_MISS) ||
              !in_bounds(vs, a.S, a.status, KVS_SITE_MISS))
            continue;
          v[jj] = a.pool[(u * a.N + tok) * kRowChunks + col];
          pos[jj] = mp;
          vic[jj] = vs;
        }
      }
#pragma unroll
      for (int jj = 0; jj < kAttnItems; ++jj) {
        const int c = jj * kAttnThreads + tid;
        const int r = c / kRowChunks;
        const int col = c - r * kRowChunks;
        if (pos[jj] >= 0) {
          st_row(hot + (u * a.S + vic[jj]) * kRowChunks + col, v[jj]);
          if (cbuf != nullptr) st_row(cbuf + (bk + pos[jj]) * kRowChunks + col, v[jj]);
        }
        *reinterpret_cast<u32x4*>(kv + r * kLdsRow + ((col ^ lds_swz(r)) * 16)) = v[jj];
      }
      __syncthreads();
      attend_tile(kv, sc, pb, alpha_s, vmark, qf, m_run, l_run, acc, hi - j0, -1,
                  a.scale_log2);
    }
  } else {
    // this workgroup's share xh of nh: hit workgroups first, then (when the
    // request has no miss) its fetch workgroups
    const int nh = a.hit_per_req + (all_hit ? a.fetch_per_req : 0);
    const int xh = fetch ? a.hit_per_req + x : x;
    // compute-buffer rows of empty entries (padded Top-K) are zero: this
    // workgroup's share of the positions, 8 threads per row
    if (a.padded && a.cbuf != nullptr) {
      const int lo = (int)((long long)xh * K / nh);
      const int hi = (int)((long long)(xh + 1) * K / nh);
      u32x4* cb = reinterpret_cast<u32x4*>(a.cbuf) + bk * kRowChunks;
      for (int i = lo + (tid >> 3); i < hi; i += kAttnThreads / 8)
        if (a.slot_of[bk + i] == -2)
#pragma unroll
          for (int j = 0; j < kAttnItems; ++j)
            cb[(long long)i * kRowChunks + (tid & 7) + 8 * j] = u32x4{0u, 0u, 0u, 0u};
    }
    const int ntiles = (n_hit + kTile - 1) / kTile;
    const int tb = (int)((long long)xh * ntiles / nh);
    const int te = (int)((long long)(xh + 1) * ntiles / nh);
    // 8 threads per row: thread (row tid / 8, sub tid % 8) moves chunks sub + 8j.
    // Rows are read through a buffer resource over the unit's S hot rows and
    // written through one over request b's K compute-buffer rows (none when
    // rows are read in place): the hardware range check turns the loads of
    // rows past the hit list into zeros and drops the stores of rows that are
    // not there, so every load and store is issued unconditionally and each
    // path through the loop has the same memory operations in flight.
    const int lrow = tid >> 3, lsub = tid & 7;
    const int hot_bytes = a.S * kRowBytes;
    const int cb_bytes = a.cbuf != nullptr ? K * kRowBytes : 0;
    const __amdgpu_buffer_rsrc_t hsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.hot + u * a.S * kRowElems), (short)0, hot_bytes, kBufRsrcWord3);
    const __amdgpu_buffer_rsrc_t csrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.cbuf != nullptr ? a.cbuf + bk * kRowElems : a.hot), (short)0, cb_bytes,
        kBufRsrcWord3);
    const __amdgpu_buffer_rsrc_t ssrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.hit_slot + bk), (short)0, n_hit * 4, kBufRsrcWord3);
    const __amdgpu_buffer_rsrc_t psrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.hit_pos + bk), (short)0, n_hit * 4, kBufRsrcWord3);
    // slot and position of this thread's row of `tile`, loaded a tile ahead of the row
    auto load_meta = [&](int tile, int& slot, int& pos) {
      const int off = tile < te ? (tile * kTile + lrow) * 4 : n_hit * 4;
      slot = __builtin_amdgcn_raw_buffer_load_b32(ssrc, off, 0, 0);
      pos = __builtin_amdgcn_raw_buffer_load_b32(psrc, off, 0, 0);
    };
    auto load_tile = [&](u32x4 (&dst)[kAttnItems], int tile, int slot) {
      const bool in = tile < te && tile * kTile + lrow < n_hit &&
                      in_bounds(slot, a.S, a.status, KVS_SITE_HIT);
      const int off = in ? slot * kRowBytes + lsub * 16 : hot_bytes;
#pragma unroll
      for (int j = 0; j < kAttnItems; ++j)
        dst[j] = __builtin_amdgcn_raw_buffer_load_b128(hsrc, off + j * 128, 0, kNT);
    };
    const int lsw = lds_swz(lrow);
    auto store_tile = [&](const u32x4 (&src)[kAttnItems], int tile, int pos) {
      unsigned char* d = kv + lrow * kLdsRow + ((lsub ^ lsw) * 16);
      const bool in = tile < te && tile * kTile + lrow < n_hit &&
                      in_bounds(pos, K, a.status, KVS_SITE_HIT);
      const int coff = in ? pos * kRowBytes + lsub * 16 : cb_bytes;
#pragma unroll
      for (int j = 0; j < kAttnItems; ++j) {
        *reinterpret_cast<u32x4*>(d + j * 128) = src[j];
        __builtin_amdgcn_raw_buffer_store_b128(src[j], csrc, coff + j * 128, 0, kNT);
      }
    };
    auto compute = [&](int tile) {
      attend_tile(kv, sc, pb, alpha_s, vmark, qf, m_run, l_run, acc, n_hit - tile * kTile, -1,
                  a.scale_log2);
    };
    if (tb < te) {
      u32x4 ra[kAttnItems], rb[kAttnItems];
      int sa, sb, pa, pbv, pa2, pb2;
      load_meta(tb, sa, pa);
      load_meta(tb + 1, sb, pbv);
      load_tile(ra, tb, sa);
      load_meta(tb + 2, sa, pa2);
      load_tile(rb, tb + 1, sb);
      store_tile(ra, tb, pa);
      __syncthreads();
      // full pairs, as in the attention kernel: at the top of each iteration
      // LDS holds `tile`, rb holds tile + 1 (position pbv) and the metadata of
      // tile + 2 is in flight (sa, pa2)
      int tile = tb;
      for (; tile + 1 < te; tile += 2) {
        load_meta(tile + 3, sb, pb2);
        load_tile(ra, tile + 2, sa);
        compute(tile);
        store_tile(rb, tile + 1, pbv);
        __syncthreads();
        load_meta(tile + 4, sa, pa);
        load_tile(rb, tile + 3, sb);
        compute(tile + 1);
        store_tile(ra, tile + 2, pa2);
        __syncthreads();
        pa2 = pa;
        pbv = pb2;
      }
      if (tile < te) compute(tile);   // odd tile count: LDS holds the last tile
    }
  }

  // partial of this workgroup: hit partials first, then fetch partials
  const long long part = (long long)b * a.parts + (fetch ? a.hit_per_req + x : x);
  float* po = a.part_o + part * kHeads * kVDim;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int j = 0; j < 4; ++j) po[(4 * g + j) * kVDim + wave * 64 + nt * 16 + r16] = acc[nt][j];
  if (tid < kHeads * 16 && (tid & 15) == 0) {
    const int h = tid >> 4;
    a.part_ml[(part * kHeads + h) * 2 + 0] = m_run;
    a.part_ml[(part * kHeads + h) * 2 + 1] = l_run;
  }
}

// Merge of the attention partials of (request b, head h):
// out = sum_s 2^(m_s - M) O_s / L, L = sum_s 2^(m_s - M) l_s, lse = (M + log2 L) ln 2.
// A partial that saw no row has m_s = -inf and weight 0.  One workgroup of
// 128 threads per (h, b), 4 outputs per thread.
// stride = partial slots per request; with a work split over `wgs`
// workgroups (wgs > 0) request b has the partials of the workgroups its tiles
// span, the first ones of its slots.
// R > 0 (R >= every request's partial count, R <= 64): the request's counts,
// the partials' (max, sum) pairs (one per lane of the first wave) and this
// thread's four outputs of every partial are all loaded before any is used,
// one memory round trip; R == 0: any count, the pairs and then the outputs.
// The sums run in partial order either way.
template <int R>
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      const int32_t* __restrict__ counts,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse, int stride,
                                                      int wgs, int ntiles) {
  __shared__ float w[kMaxParts];
  __shared__ float inv_l, lse_h;
  const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  int splits = stride;
  if (wgs > 0) {
    const long long G = (long long)gridDim.y * ntiles;
    splits = share_of((long long)(b + 1) * ntiles - 1, G, wgs) -
             share_of((long long)b * ntiles, G, wgs) + 1;
  }
  const float* ml = part_ml + (long long)b * stride * kHeads * 2;
  const float* pob = part_o + (long long)b * stride * kHeads * kVDim + h * kVDim + tid * 4;
  // the counts through a buffer (vector-memory) load issued with the others:
  // as a scalar load the compiler waits for it before issuing them
  const u32x4 cnt = __builtin_amdgcn_raw_buffer_load_b128(
      __builtin_amdgcn_make_buffer_rsrc((void*)(counts + 4 * b), (short)0, 16, kBufRsrcWord3), 0,
      0, 0);
  float2 pair = make_float2(-INFINITY, 0.f);   // (max, sum) of partial tid (R > 0)
  float4 x[R > 0 ? R : 1];
  if constexpr (R > 0) {
    // unconditional loads at clamped indices (a partial past the request's
    // count repeats the last one and is never used)
    pair = *reinterpret_cast<const float2*>(ml + (min(tid, splits - 1) * kHeads + h) * 2);
#pragma unroll
    for (int s = 0; s < R; ++s)
      x[s] = *reinterpret_cast<const float4*>(pob + (long long)min(s, splits - 1) * kHeads * kVDim);
  }
  uint2* ob = reinterpret_cast<uint2*>(out + ((long long)b * kHeads + h) * kVDim);
  // An invalid Top-K, or no entry at all (padded), gives a zero output and
  // lse = -inf.  The merge below runs either way (on partials nobody wrote,
  // whose result is then discarded) and the counts are looked at only at the
  // end: otherwise the compiler issues the loads above after they arrive.
  if (tid < 64) {   // one wave: max and weighted sum over the partials
    float m = -INFINITY;
    if constexpr (R > 0) {
      if (tid < splits) m = pair.x;
    } else {
      for (int s = tid; s < splits; s += 64) m = fmaxf(m, ml[(s * kHeads + h) * 2]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float l = 0.f;
    if constexpr (R > 0) {
      if (tid < splits) {
        const float ws = exp2f(pair.x - m);
        w[tid] = ws;
        l = ws * pair.y;
      }
    } else {
      for (int s = tid; s < splits; s += 64) {
        const float ws = exp2f(ml[(s * kHeads + h) * 2] - m);
        w[s] = ws;
        l += ws * ml[(s * kHeads + h) * 2 + 1];
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
    if (tid == 0) {
      inv_l = 1.f / l;
      lse_h = (m + log2f(l)) * 0.69314718055994531f;
    }
  }
  __syncthreads();
  float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
  if constexpr (R > 0) {
#pragma unroll
    for (int s = 0; s < R; ++s) {
      if (s < splits) {
        const float ws = w[s];
        o0 += ws * x[s].x;
        o1 += ws * x[s].y;
        o2 += ws * x[s].z;
        o3 += ws * x[s].w;
      }
    }
  } else {
    for (int s = 0; s < splits; ++s) {
      const float ws = w[s];
      const float4 y = *reinterpret_cast<const float4*>(pob + (long long)s * kHeads * kVDim);
      o0 += ws * y.x;
      o1 += ws * y.y;
      o2 += ws * y.z;
      o3 += ws * y.w;
    }
  }
  const float il = inv_l;
  const bool empty = cnt[3] == 0 || cnt[0] + cnt[1] == 0;
  if (lse != nullptr && tid == 0) lse[b * kHeads + h] = empty ? -INFINITY : lse_h;
  ob[tid] = empty ? make_uint2(0u, 0u)
                  : make_uint2((uint32_t)f32_to_bf16_rne(o0 * il) |
                                   ((uint32_t)f32_to_bf16_rne(o1 * il) << 16),
                               (uint32_t)f32_to_bf16_rne(o2 * il) |
                                   ((uint32_t)f32_to_bf16_rne(o3 * il) << 16));
}

// ------------------------------------------------------------------ state check
// KVS_FLAG_CHECK: after the diff of `layer`, workgroup b verifies unit
// (b, layer): slot2tok and tok2slot are mutual inverses over all S slots and
// all N tokens, the LRU order holds every slot once in strictly ascending
// (last_used, slot) order (the order the victim choice relies on), and no
// victim of this step is a hit slot of it.  A violation latches KVS_ECORRUPT.
constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void check_state_kernel(
    const int32_t* __restrict__ tok2slot, const int32_t* __restrict__ slot2tok,
    const int32_t* __restrict__ last_used, const uint16_t* __restrict__ order,
    const int32_t* __restrict__ slot_of, const int32_t* __restrict__ victims,
    const int32_t* __restrict__ counts, int32_t* status, long long N, int S, int Sp, int K,
    int L, int layer) {
  extern __shared__ unsigned hitbits[];   // one bit per slot: hit slots of this step
  __shared__ int bad;
  const int b = blockIdx.x, tid = threadIdx.x;
  if (counts[4 * b + 3] == 0) return;     // invalid input: the unit was left untouched
  const long long u = (long long)b * L + layer;
  const int32_t* t2s = tok2slot + u * N;
  const int32_t* s2t = slot2tok + u * Sp;
  const int32_t* lu = last_used + u * Sp;
  const uint16_t* ord = order + u * Sp;
  const long long bk = (long long)b * K;
  for (int w = tid; w < (S + 31) / 32; w += kCheckThreads) hitbits[w] = 0u;
  if (tid == 0) bad = 0;
  __syncthreads();
  int err = 0;
  for (int s = tid; s < S; s += kCheckThreads) {          // slot -> token -> slot
    const int t = s2t[s];
    if (t < -1 || (t >= 0 && ((long long)t >= N || t2s[t] != s))) err = 1;
  }
  for (long long t = tid; t < N; t += kCheckThreads) {    // token -> slot -> token
    const int s = t2s[t];
    if (s < -1 || (s >= 0 && (s >= S || s2t[s] != (int)t))) err = 1;
  }
  for (int p = tid; p < S; p += kCheckThreads) {          // order: sorted permutation
    const int s = ord[p];
    if (s >= S) {
      err = 1;
    } else if (p + 1 < S) {
      const int s2 = ord[p + 1];
      if (s2 >= S) {
        err = 1;
      } else {
        const int a = lu[s], c = lu[s2];
        if (!(a < c || (a == c && s < s2))) err = 1;
      }
    }
  }
  for (int i = tid; i < K; i += kCheckThreads) {
    const int s = slot_of[bk + i];
    if (s >= 0 && s < S) atomicOr(&hitbits[s >> 5], 1u << (s & 31));
  }
  __syncthreads();
  const int m = counts[4 * b + 1];
  for (int j = tid; j < m; j += kCheckThreads) {           // victims are not hit slots
    const int v = victims[bk + j];
    if (v < 0 || v >= S || ((hitbits[v >> 5] >> (v & 31)) & 1u)) err = 1;
  }
  if (err) atomicOr(&bad, 1);
  __syncthreads();
  if (tid == 0 && bad) atomicCAS(status, 0, KVS_ECORRUPT);
}

// ------------------------------------------------------------------ append
// Lifecycle "publish" of one decode step's new rows: workgroup b writes row b
// of `rows` into the host pool at (b, layer, pos[b]) (PCIe writes to the
// mapped pinned pool) and, when that token is resident, over its hot slot, so
// the hot copy keeps equalling the pool.  pos[b] = -1: nothing to append.
constexpr int kAppendThreads = 128;   // 72 chunks of one row, one per thread
static_assert(kRowChunks <= kAppendThreads, "append tiling");

__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    const u32x4* __restrict__ rows, const long long* __restrict__ pos, u32x4* pool,
    u32x4* hot, const int32_t* __restrict__ tok2slot, int32_t* status, long long N, int S,
    int L, int layer) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const long long p = pos[b];
  if (p == -1) return;
  if (p < -1 || p >= N) {
    if (tid == 0) atomicCAS(status, 0, KVS_ERANGE);
    return;
  }
  const long long u = (long long)b * L + layer;
  const int s = tok2slot[u * N + p];
  if (!in_range(s, -1, S, status, KVS_SITE_APPEND)) return;   // the row is not appended
  if (tid < kRowChunks) {
    const u32x4 v = rows[(long long)b * kRowChunks + tid];
    pool[(u * N + p) * kRowChunks + tid] = v;
    if (s >= 0) hot[((long long)u * S + s) * kRowChunks + tid] = v;
  }
  // system-scope release: the pool row leaves this XCD's L2 for host memory,
  // where the host and every other XCD's fetches read it
  __threadfence_system();
}

// ------------------------------------------------------------------ host read probe
// Zero-copy read of pinned host memory with the fetch role's access pattern:
// each wave instruction reads 1 KB of consecutive host memory.  Every thread
// XOR-folds its chunks and stores one word, so no load can be dropped.
constexpr int kProbeBlocks = 256, kProbeThreads = 256;
static_assert(kProbeBlocks * kProbeThreads == KVS_PROBE_SINK_WORDS, "probe sink size");

__global__ __launch_bounds__(kProbeThreads) void host_read_probe_kernel(const u32x4* src,
                                                                         long long chunks,
                                                                         uint32_t* sink) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  long long c = t;
  // four chunks in flight per thread per pass
  for (; c + 3 * stride < chunks; c += 4 * stride) {
    const u32x4 v0 = src[c], v1 = src[c + stride], v2 = src[c + 2 * stride],
                v3 = src[c + 3 * stride];
    acc ^= v0 ^ v1 ^ v2 ^ v3;
  }
  for (; c < chunks; c += stride) acc ^= src[c];
  sink[t] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

// ------------------------------------------------------------------ launchers
size_t diff_lds_bytes(int S, int K) {
  int hb = 1;
  while ((1 << hb) < 2 * K) ++hb;
  const size_t words = (1u << hb) > 3u * K ? (1u << hb) : 3u * K;
  const size_t Sp = (size_t)((S + 15) & ~15);
  const size_t tok = S <= 8 * kDiffThreads ? 4 * Sp : 0;   // slot tokens
  return Sp + tok + 2 * Sp + 4 * words;                    // flags, tokens, new order, lists
}

static int hash_bits_for(int K) {
  int hb = 1;
  while ((1 << hb) < 2 * K) ++hb;
  return hb;
}

hipError_t launch_init_units(const Layout& lay, const DevPtrs& d, int unit_begin, int unit_count,
                             bool reset_counters, hipStream_t s) {
  const long long n_tok = (long long)unit_count * lay.N;
  const long long n_slot = (long long)unit_count * lay.Sp;
  const long long work = n_tok > n_slot ? n_tok : n_slot;
  long long blocks = (work + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(init_units_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     d.tok2slot + (long long)unit_begin * lay.N,
                     d.slot2tok + (long long)unit_begin * lay.Sp,
                     d.last_used + (long long)unit_begin * lay.Sp,
                     d.order + (long long)unit_begin * lay.Sp, n_tok, n_slot, lay.S, lay.Sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !reset_counters) return e;
  const int units = lay.B * lay.L;
  hipLaunchKernelGGL(reset_counters_kernel, dim3((units + 255) / 256), dim3(256), 0, s, d.stepctr,
                     d.stats, d.status, units);
  return hipGetLastError();
}

hipError_t launch_clear_status(const DevPtrs& d, hipStream_t s) {
  hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(64), 0, s, d.status);
  return hipGetLastError();
}

// The instantiation of diff_lru_kernel whose per-thread bounds cover K and S.
template <int KPT>
static const void* diff_kernel_spt(int spt) {
  if (spt <= 1) return reinterpret_cast<const void*>(diff_lru_kernel<KPT, 1>);
  if (spt <= 2) return reinterpret_cast<const void*>(diff_lru_kernel<KPT, 2>);
  if (spt <= 4) return reinterpret_cast<const void*>(diff_lru_kernel<KPT, 4>);
  if (spt <= 8) return reinterpret_cast<const void*>(diff_lru_kernel<KPT, 8>);
  return reinterpret_cast<const void*>(diff_lru_kernel<KPT, 16>);
}
static const void* diff_kernel_for(int K, int S) {
  const int kpt = (K + kDiffThreads - 1) / kDiffThreads;
  const int spt = (S + kDiffThreads - 1) / kDiffThreads;
  if (kpt <= 1) return diff_kernel_spt<1>(spt);
  if (kpt <= 2) return diff_kernel_spt<2>(spt);
  if (kpt <= 4) return diff_kernel_spt<4>(spt);
  return diff_kernel_spt<8>(spt);
}
static_assert(KVS_MAX_TOPK <= 8 * kDiffThreads && KVS_MAX_SLOTS <= 16 * kDiffThreads,
              "diff_lru instantiations cover the limits");

hipError_t prepare_kernels() {
  // the diff kernel's dynamic LDS can exceed the 64 KiB default (up to 152 KiB,
  // at 8192 slots with their tokens in LDS and the largest Top-K)
  const int max_lds = (int)std::max(diff_lds_bytes(8 * kDiffThreads, KVS_MAX_TOPK),
                                    diff_lds_bytes(KVS_MAX_SLOTS, KVS_MAX_TOPK));
  for (int kpt = 1; kpt <= 8; kpt *= 2)
    for (int spt = 1; spt <= 16; spt *= 2) {
      const hipError_t e = hipFuncSetAttribute(
          diff_kernel_for(kpt * kDiffThreads, spt * kDiffThreads),
          hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
      if (e != hipSuccess) return e;
    }
  return hipSuccess;
}

hipError_t launch_diff_lru(const Layout& lay, const DevPtrs& d, int layer, const int32_t* topk,
                           hipStream_t s) {
  const size_t lds = diff_lds_bytes(lay.S, lay.K);
  DiffArgs a;
  a.topk = topk;
  a.tok2slot = d.tok2slot;
  a.slot2tok = d.slot2tok;
  a.last_used = d.last_used;
  a.order = d.order;
  a.stepctr = d.stepctr;
  a.stats = d.stats;
  a.status = d.status;
  a.slot_of = d.slot_of;
  a.miss_pos = d.miss_pos;
  a.victims = d.victims;
  a.evicted = d.evicted;
  a.counts = d.counts;
  a.row_slot = d.row_slot;
  a.hit_pos = d.hit_pos;
  a.hit_slot = d.hit_slot;
  a.miss_tok = d.miss_tok;
  a.N = lay.N;
  a.S = lay.S;
  a.K = lay.K;
  a.L = lay.L;
  a.layer = layer;
  a.hash_bits = hash_bits_for(lay.K);
  a.Sp = lay.Sp;
  a.padded = (lay.flags & KVS_FLAG_PADDED_TOPK) != 0;
  const void* fn = diff_kernel_for(lay.K, lay.S);
  void* args[] = {&a};
  return hipLaunchKernel(fn, dim3(lay.B), dim3(kDiffThreads), args, lds, s);
}

hipError_t launch_gather(const Layout& lay, const DevPtrs& d, int layer, hipStream_t s) {
  GatherArgs a;
  a.pool = reinterpret_cast<const u32x4*>(d.pool);
  a.hot = reinterpret_cast<u32x4*>(d.hot);
  a.cbuf = reinterpret_cast<u32x4*>(d.cbuf);
  a.slot_of = d.slot_of;
  a.miss_tok = d.miss_tok;
  a.deep_fetch = lay.N * kRowBytes <= 0xffffffffll;
  a.miss_pos = d.miss_pos;
  a.victims = d.victims;
  a.counts = d.counts;
  a.N = lay.N;
  a.S = lay.S;
  a.K = lay.K;
  a.L = lay.L;
  a.layer = layer;
  a.B = lay.B;
  const int groups_per_req = (lay.K + kCopyRows - 1) / kCopyRows;
  int per_req = (lay.fetch_blocks + lay.B - 1) / lay.B;   // fetch workgroups spread over requests
  if (per_req > groups_per_req) per_req = groups_per_req;
  a.fetch_per_req = per_req;
  a.fetch_wgs = per_req * lay.B;
  const long long all_groups = (long long)groups_per_req * lay.B;
  a.hit_wgs = (int)(lay.hit_blocks > 0 && lay.hit_blocks < all_groups ? lay.hit_blocks : all_groups);
  a.hits_first = (lay.flags & KVS_FLAG_HITS_FIRST) != 0;
  a.write_cbuf = (lay.flags & KVS_FLAG_DIRECT_HOT) == 0;
  a.status = d.status;
  if (!a.write_cbuf) a.hit_wgs = 0;   // hits stay where they are
  const long long grid = (long long)a.fetch_wgs + (long long)a.hit_wgs;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)grid), dim3(kCopyThreads), kCopyLdsReserve, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_hit_copy(const Layout& lay, const DevPtrs& d, int layer, hipStream_t s) {
  GatherArgs a;
  a.pool = reinterpret_cast<const u32x4*>(d.pool);
  a.hot = reinterpret_cast<u32x4*>(d.hot);
  a.cbuf = reinterpret_cast<u32x4*>(d.cbuf);
  a.miss_tok = d.miss_tok;   // read by the fetch role only, which has no workgroup here
  a.deep_fetch = 0;
  a.slot_of = d.slot_of;
  a.miss_pos = d.miss_pos;
  a.victims = d.victims;
  a.counts = d.counts;
  a.N = lay.N;
  a.S = lay.S;
  a.K = lay.K;
  a.L = lay.L;
  a.layer = layer;
  a.B = lay.B;
  a.fetch_per_req = 1;
  a.fetch_wgs = 0;
  a.hit_wgs = (int)((long long)((lay.K + kCopyRows - 1) / kCopyRows) * lay.B);
  a.hits_first = 0;
  a.write_cbuf = 1;
  a.status = d.status;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)a.hit_wgs), dim3(kCopyThreads),
                     kCopyLdsReserve, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const Layout& lay, const DevPtrs& d, int layer, const uint16_t* q,
                            float scale, uint16_t* out, float* lse, hipStream_t s) {
  AttnArgs a;
  a.cbuf = d.cbuf;
  a.hot = d.hot;
  a.q = q;
  a.slot_of = d.slot_of;
  a.row_slot = d.row_slot;
  a.counts = d.counts;
  a.part_o = d.part_o;
  a.part_ml = d.part_ml;
  a.K = lay.K;
  a.B = lay.B;
  a.S = lay.S;
  a.L = lay.L;
  a.layer = layer;
  a.wgs = lay.attn_wgs;
  a.parts = lay.parts;
  a.padded = (lay.flags & KVS_FLAG_PADDED_TOPK) != 0;
  a.out = lay.parts == 1 ? out : nullptr;
  a.lse = lay.parts == 1 ? lse : nullptr;
  a.status = d.status;
  const bool direct = (lay.flags & KVS_FLAG_DIRECT_HOT) != 0;
  a.scale_log2 = scale * 1.4426950408889634f;
  if (direct)
    hipLaunchKernelGGL(attention_kernel<true>, dim3(lay.attn_wgs), dim3(kAttnThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attention_kernel<false>, dim3(lay.attn_wgs), dim3(kAttnThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_assemble(const Layout& lay, const DevPtrs& d, int layer, const uint16_t* q,
                           float scale, hipStream_t s) {
  AssembleArgs a;
  a.pool = reinterpret_cast<const u32x4*>(d.pool);
  a.hot = d.hot;
  a.cbuf = (lay.flags & KVS_FLAG_DIRECT_HOT) ? nullptr : d.cbuf;
  a.q = q;
  a.slot_of = d.slot_of;
  a.hit_pos = d.hit_pos;
  a.hit_slot = d.hit_slot;
  a.miss_pos = d.miss_pos;
  a.miss_tok = d.miss_tok;
  a.victims = d.victims;
  a.counts = d.counts;
  a.part_o = d.part_o;
  a.part_ml = d.part_ml;
  a.N = lay.N;
  a.S = lay.S;
  a.K = lay.K;
  a.L = lay.L;
  a.layer = layer;
  a.fetch_per_req = lay.fetch_per_req;
  a.hit_per_req = lay.splits;
  a.parts = lay.parts;
  a.fetch_wgs = lay.fetch_per_req * lay.B;
  a.hits_first = (lay.flags & KVS_FLAG_HITS_FIRST) != 0;
  a.padded = (lay.flags & KVS_FLAG_PADDED_TOPK) != 0;
  a.status = d.status;
  a.scale_log2 = scale * 1.4426950408889634f;
  const long long grid = (long long)(lay.fetch_per_req + lay.splits) * lay.B;
  hipLaunchKernelGGL(assemble_kernel, dim3((unsigned)grid), dim3(kAttnThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append(const Layout& lay, const DevPtrs& d, int layer, const uint16_t* rows,
                         const int64_t* pos, hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3(lay.B), dim3(kAppendThreads), 0, s,
                     reinterpret_cast<const u32x4*>(rows), reinterpret_cast<const long long*>(pos),
                     reinterpret_cast<u32x4*>(const_cast<uint16_t*>(d.pool)),
                     reinterpret_cast<u32x4*>(d.hot), d.tok2slot, d.status, (long long)lay.N,
                     lay.S, lay.L, layer);
  return hipGetLastError();
}

hipError_t launch_check_state(const Layout& lay, const DevPtrs& d, int layer, hipStream_t s) {
  const size_t lds = (size_t)((lay.S + 31) / 32) * 4;
  hipLaunchKernelGGL(check_state_kernel, dim3(lay.B), dim3(kCheckThreads), lds, s, d.tok2slot,
                     d.slot2tok, d.last_used, d.order, d.slot_of, d.victims, d.counts, d.status,
                     (long long)lay.N, lay.S, lay.Sp, lay.K, lay.L, layer);
  return hipGetLastError();
}

hipError_t launch_host_read_probe(const void* src, long long chunks, uint32_t* sink,
                                  hipStream_t s) {
  hipLaunchKernelGGL(host_read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, s,
                     reinterpret_cast<const u32x4*>(src), chunks, sink);
  return hipGetLastError();
}

hipError_t launch_combine(const Layout& lay, const DevPtrs& d, uint16_t* out, float* lse,
                          hipStream_t s) {
  // the separate attention's work split: its partials per request vary
  const bool split = (lay.flags & KVS_FLAG_SEPARATE_ATTENTION) != 0;
  // the smallest register count that holds every request's partials
  const int P = lay.parts;
  auto fn = P <= 4 ? combine_kernel<4> : P <= 8 ? combine_kernel<8> : P <= 16 ? combine_kernel<16>
          : P <= 32 ? combine_kernel<32> : combine_kernel<0>;
  hipLaunchKernelGGL(fn, dim3(kHeads, lay.B), dim3(128), 0, s, d.part_o, d.part_ml, d.counts,
                     out, lse, lay.parts, split ? lay.attn_wgs : 0, (lay.K + kTile - 1) / kTile);
  return hipGetLastError();
}

}  // namespace kvs
