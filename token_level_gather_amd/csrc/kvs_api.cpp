// Host runtime behind the C ABI in include/kvs.h: configuration and buffer
// validation, host-pool allocation, launch orchestration of one decode step
// (diff, the assembling launch and the merge of its partials on the caller's
// stream; or diff, gather, attention and the merge), status and statistics
// readback, and per-kernel event timing.
//
// The request lifecycle follows "XM-Sparse" (HiSparse integration section):
// publish = kvs_publish, fetch + write-back = kvs_step, free = kvs_free_request.
#include <math.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "kvs_internal.h"

namespace kvs {

static uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Attention workgroups resident at once: one per compute unit of an MI355X.
constexpr int kAttnWorkgroupsPerRound = 256;
// Assembling launch defaults, from sweeps at 4, 32, 64 and 192 requests:
// about two fetch workgroups (512 threads) per request, 64 to 128 in all
// (more outstanding PCIe reads lower the link's throughput and take CUs from
// the hit workgroups; fewer leave each request's misses to one workgroup's
// serial passes), and up to 8 hit workgroups per request, 128 in all.
constexpr int kAssembleFetchMin = 64, kAssembleFetchMax = 128;
constexpr int kAssembleHitBlocks = 128, kAssembleHitMaxPerReq = 8;

int make_layout(const kvs_config* c, Layout* lay) {
  if (c == nullptr || lay == nullptr) return KVS_EINVAL;
  if (c->batch < 1 || c->batch > 65535 || c->layers < 1) return KVS_EINVAL;
  if (c->topk < 1 || c->topk > KVS_MAX_TOPK) return KVS_EINVAL;
  if (c->slots < c->topk || c->slots > KVS_MAX_SLOTS) return KVS_EINVAL;
  if (c->context < c->topk || c->context > 0x7fffffffLL) return KVS_EINVAL;
  if (c->heads != KVS_HEADS || c->head_dim != KVS_HEAD_DIM || c->v_dim != KVS_V_DIM)
    return KVS_EINVAL;
  if (!(c->scale > 0.f) || !isfinite(c->scale)) return KVS_EINVAL;
  if (c->attn_splits < 0 || c->attn_splits > 64) return KVS_EINVAL;
  if (c->fetch_blocks < 0 || c->fetch_blocks > 65535) return KVS_EINVAL;
  if (c->hit_blocks < 0 || c->hit_blocks > 65535) return KVS_EINVAL;
  if ((c->flags & ~(KVS_FLAG_HITS_FIRST | KVS_FLAG_PADDED_TOPK | KVS_FLAG_DIRECT_HOT |
                    KVS_FLAG_CHECK | KVS_FLAG_SEPARATE_ATTENTION)) != 0)
    return KVS_EINVAL;
  if ((int64_t)c->batch * c->layers > 0x7fffffffLL) return KVS_EINVAL;

  const uint64_t B = c->batch, L = c->layers, N = c->context, K = c->topk;
  const uint64_t U = B * L;
  const int ntiles = (int)((K + 63) / 64);
  const bool separate = (c->flags & KVS_FLAG_SEPARATE_ATTENTION) != 0;
  int splits = c->attn_splits;
  int fetch_blocks, fetch_per_req = 0, parts;
  if (!separate) {
    // one assembling launch: fetch workgroups (one CU each for the whole
    // fetch) and hit workgroups (one CU each, several rounds); each writes
    // one attention partial
    if (c->fetch_blocks != 0) {
      fetch_blocks = c->fetch_blocks;
    } else {
      const uint64_t three_per_req = 3 * B;
      fetch_blocks = three_per_req < (uint64_t)kAssembleFetchMin   ? kAssembleFetchMin
                     : three_per_req > (uint64_t)kAssembleFetchMax ? kAssembleFetchMax
                                                                   : (int)three_per_req;
    }
    fetch_per_req = (int)((fetch_blocks + B - 1) / B);
    if (fetch_per_req > ntiles) fetch_per_req = ntiles;
    if (splits == 0) {
      splits = (int)((kAssembleHitBlocks + B - 1) / B);
      if (splits > kAssembleHitMaxPerReq) splits = kAssembleHitMaxPerReq;
      if (splits > ntiles) splits = ntiles;
    } else if (splits > ntiles) {
      return KVS_EINVAL;
    }
    parts = splits + fetch_per_req;
  } else if (splits > ntiles) {
    return KVS_EINVAL;
  }
  int attn_wgs = 0;
  if (separate) {
    // The attention's workgroups share the B * ntiles tiles evenly, request
    // after request (a workgroup's share may span requests).  An attention
    // workgroup holds one CU (its LDS tile), so at most 256 run at once, and
    // every workgroup first waits for its first two tiles: one round of the
    // fewest workgroups that reach the smallest share, ceil(G / 256) tiles.
    // With attn_splits = s the share of each request is s workgroups.
    const uint64_t G = B * (uint64_t)ntiles;
    uint64_t W;
    if (splits > 0) {
      W = B * (uint64_t)splits;
    } else {
      const uint64_t per = (G + kAttnWorkgroupsPerRound - 1) / kAttnWorkgroupsPerRound;
      W = (G + per - 1) / per;
    }
    if (W > 0x7fffffffu) return KVS_EINVAL;
    attn_wgs = (int)W;
    // partials per request: the most workgroups whose shares one request spans
    auto share_of = [&](uint64_t g) { return ((g + 1) * W - 1) / G; };
    parts = 1;
    for (uint64_t b = 0; b < B; ++b) {
      const int n = (int)(share_of((b + 1) * ntiles - 1) - share_of(b * ntiles) + 1);
      if (n > parts) parts = n;
    }
    if (parts > 256) return KVS_EINVAL;   // the merge takes at most 256 partials per request
    splits = parts;
    // 256 fetch workgroups (1 per CU) keep the host link saturated; more only
    // add outstanding PCIe reads, which slow the HBM traffic beside them
    fetch_blocks = c->fetch_blocks == 0 ? 256 : c->fetch_blocks;
  }

  lay->B = c->batch;
  lay->L = c->layers;
  lay->S = c->slots;
  // the slot arrays of a unit start 16 entries apart, so each diff thread's
  // run of order entries and slot tokens is aligned for wide loads
  lay->Sp = (c->slots + 15) & ~15;
  lay->K = c->topk;
  lay->N = c->context;
  lay->splits = splits;
  lay->parts = parts;
  lay->attn_wgs = attn_wgs;
  lay->fetch_blocks = fetch_blocks;
  lay->fetch_per_req = fetch_per_req;
  lay->hit_blocks = c->hit_blocks;
  lay->flags = c->flags;

  uint64_t o = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  lay->tok2slot = take(U * N * 4);
  const uint64_t Sp = (uint64_t)lay->Sp;
  lay->slot2tok = take(U * Sp * 4);
  lay->last_used = take(U * Sp * 4);
  lay->order = take(U * Sp * 2);
  lay->stepctr = take(U * 4);
  lay->stats = take(U * 4 * 8);
  lay->status = take(16);
  lay->meta_bytes = o;

  o = 0;
  lay->slot_of = take(B * K * 4);
  lay->miss_pos = take(B * K * 4);
  lay->victims = take(B * K * 4);
  lay->evicted = take(B * K * 4);
  lay->counts = take(B * 16);
  lay->row_slot = take(B * K * 4);
  lay->hit_pos = take(B * K * 4);
  lay->hit_slot = take(B * K * 4);
  lay->miss_tok = take(B * K * 4);
  lay->part_o = take(B * (uint64_t)parts * kHeads * kVDim * 4);
  lay->part_ml = take(B * (uint64_t)parts * kHeads * 2 * 4);
  lay->scratch_bytes = o;
  return KVS_OK;
}

}  // namespace kvs

using namespace kvs;

struct kvs_pool {
  kvs_config cfg;
  Layout lay;
  DevPtrs d;
  uint8_t* host_pool;       // host address of the pool (for kvs_publish)
  int device;
  // per-kernel timing: a pool of event pairs, one pair per recorded launch
  std::vector<hipEvent_t> prof_ev;
  std::vector<int> prof_kernel;
  int prof_cap;      // launches that can be recorded
  int prof_used;     // launches recorded
  int prof_steps;    // kvs_step calls recorded
  int prof_max_steps;
  uint32_t prof_mask;  // kernels recorded (1 << KVS_KERNEL_*)
  bool roctx;          // KVS_ROCTX=1 at creation: a named range around every kvs_step
  // the library's static scratch on this pool's device (kvs_step_static), or
  // null with the error that resolving its address gave
  void* static_scratch;
  hipError_t static_scratch_err;
  DevPtrs last_scratch;  // device pointers of the last step (its lists for kvs_debug_read_state)
  bool stepped;          // a step has been enqueued: last_scratch holds written lists
};

static int hip_err(hipError_t e) { return e == hipSuccess ? KVS_OK : KVS_EHIP_BASE - (int)e; }

#define KVS_TRY_HIP(expr)                       \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) return hip_err(e_);   \
  } while (0)

// Frees the pool's timing events and the pool itself.
static void destroy_pool(kvs_pool* p) {
  for (hipEvent_t ev : p->prof_ev) (void)hipEventDestroy(ev);
  delete p;
}

// The pool's buffers live on the device that was current at kvs_create_pool:
// work enqueued on a stream of another device would address them there.
static int check_device(const kvs_pool* p, hipStream_t s) {
  hipDevice_t dev = -1;
  if (hipStreamGetDevice(s, &dev) != hipSuccess) {
    (void)hipGetLastError();
    return KVS_EINVAL;
  }
  return dev == p->device ? KVS_OK : KVS_EINVAL;
}

#define KVS_TRY(expr)            \
  do {                           \
    const int rc_ = (expr);      \
    if (rc_ != KVS_OK) return rc_; \
  } while (0)

// Pointer arguments of one step: the kernels read q in 16-byte vectors, write
// out in 16-byte (empty request), 8-byte (merge) and 2-byte stores, and read
// topk and write lse as 4-byte words.  A misaligned pointer is rejected here
// instead of faulting the GPU.
static int check_step_args(const int32_t* topk, const void* q, const void* out,
                           const float* lse) {
  if (topk == nullptr || q == nullptr || out == nullptr) return KVS_EINVAL;
  if (((uintptr_t)q & 15) != 0 || ((uintptr_t)out & 15) != 0) return KVS_EINVAL;
  if (((uintptr_t)topk & 3) != 0 || ((uintptr_t)lse & 3) != 0) return KVS_EINVAL;
  return KVS_OK;
}

// `ptr` must be device memory of `device` with at least `bytes` from `ptr` to
// the end of its allocation.
static int check_device_buffer(const void* ptr, uint64_t bytes, int device) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, ptr) != hipSuccess) {
    (void)hipGetLastError();
    return KVS_EINVAL;
  }
  if (at.type != hipMemoryTypeDevice || at.device != device) return KVS_EINVAL;
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)ptr) != hipSuccess) {
    (void)hipGetLastError();
    return KVS_EINVAL;
  }
  const uintptr_t end = (uintptr_t)base + size;
  if ((uintptr_t)ptr < (uintptr_t)base || (uintptr_t)ptr + bytes > end) return KVS_ENOMEM;
  return KVS_OK;
}

// Points the per-step arrays of `d` into a scratch buffer laid out by `lay`.
static void bind_scratch(const Layout& lay, uint8_t* scr, DevPtrs* d) {
  d->slot_of = (int32_t*)(scr + lay.slot_of);
  d->miss_pos = (int32_t*)(scr + lay.miss_pos);
  d->victims = (int32_t*)(scr + lay.victims);
  d->evicted = (int32_t*)(scr + lay.evicted);
  d->counts = (int32_t*)(scr + lay.counts);
  d->row_slot = (int32_t*)(scr + lay.row_slot);
  d->hit_pos = (int32_t*)(scr + lay.hit_pos);
  d->hit_slot = (int32_t*)(scr + lay.hit_slot);
  d->miss_tok = (int32_t*)(scr + lay.miss_tok);
  d->part_o = (float*)(scr + lay.part_o);
  d->part_ml = (float*)(scr + lay.part_ml);
}

// Launch `fn` on `s`, bracketed by timing events when profiling.
template <typename F>
static hipError_t timed(kvs_pool* p, int kernel, hipStream_t s, F fn) {
  hipEvent_t* ev = nullptr;
  if (p->prof_steps < p->prof_max_steps && p->prof_used < p->prof_cap &&
      ((p->prof_mask >> kernel) & 1u)) {
    ev = &p->prof_ev[(size_t)p->prof_used * 2];
    p->prof_kernel[p->prof_used] = kernel;
    ++p->prof_used;
    hipError_t e = hipEventRecord(ev[0], s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = fn();
  if (e == hipSuccess && ev != nullptr) e = hipEventRecord(ev[1], s);
  return e;
}

extern "C" {

int kvs_query_sizes(const kvs_config* cfg, kvs_sizes* out) {
  if (out == nullptr) return KVS_EINVAL;
  Layout lay;
  const int rc = make_layout(cfg, &lay);
  if (rc != KVS_OK) return rc;
  const uint64_t B = cfg->batch, L = cfg->layers, N = cfg->context, S = cfg->slots,
                 K = cfg->topk;
  out->host_pool_bytes = B * L * N * kRowBytes;
  out->hot_bytes = B * L * S * kRowBytes;
  out->meta_bytes = lay.meta_bytes;
  out->cbuf_bytes = (cfg->flags & KVS_FLAG_DIRECT_HOT) ? 0 : B * K * kRowBytes;
  out->scratch_bytes = lay.scratch_bytes;
  out->attn_splits = lay.splits;
  out->fetch_blocks = lay.fetch_blocks;
  return KVS_OK;
}

int kvs_host_alloc(uint64_t bytes, void** out) {
  if (out == nullptr || bytes == 0) return KVS_EINVAL;
  *out = nullptr;
  // Pinned, mapped into the GPU's address space at the same address.  The
  // pool is read by GPU kernels over PCIe and written only by the host while
  // no step is in flight, so coarse-grained (non-coherent) memory suffices;
  // KVS_HOST_COHERENT=1 selects fine-grained memory instead.
  unsigned flags = hipHostMallocMapped | hipHostMallocPortable;
  const char* coh = getenv("KVS_HOST_COHERENT");
  flags |= (coh != nullptr && coh[0] == '1') ? hipHostMallocCoherent : hipHostMallocNonCoherent;
  void* p = nullptr;
  const hipError_t e = hipHostMalloc(&p, (size_t)bytes, flags);
  if (e != hipSuccess) return hip_err(e);
  *out = p;
  return KVS_OK;
}

int kvs_host_free(void* ptr) {
  if (ptr == nullptr) return KVS_EINVAL;
  return hip_err(hipHostFree(ptr));
}

int kvs_create_pool(const kvs_config* cfg, const kvs_buffers* bufs, void* stream,
                    kvs_pool** out) {
  if (out == nullptr || bufs == nullptr) return KVS_EINVAL;
  *out = nullptr;
  kvs_sizes need;
  int rc = kvs_query_sizes(cfg, &need);
  if (rc != KVS_OK) return rc;
  if (bufs->host_pool == nullptr || bufs->hot == nullptr || bufs->meta == nullptr ||
      (bufs->cbuf == nullptr && need.cbuf_bytes != 0) || bufs->scratch == nullptr)
    return KVS_EINVAL;
  if (bufs->host_pool_bytes < need.host_pool_bytes || bufs->hot_bytes < need.hot_bytes ||
      bufs->meta_bytes < need.meta_bytes || bufs->cbuf_bytes < need.cbuf_bytes ||
      bufs->scratch_bytes < need.scratch_bytes)
    return KVS_ENOMEM;
  const uintptr_t mis = (uintptr_t)bufs->host_pool | (uintptr_t)bufs->hot |
                        (uintptr_t)bufs->cbuf;
  if ((mis & 15) != 0 || ((uintptr_t)bufs->meta & 255) != 0 ||
      ((uintptr_t)bufs->scratch & 255) != 0)
    return KVS_EINVAL;

  // the pool must be pinned host memory the GPU can address
  void* pool_dev = nullptr;
  if (hipHostGetDevicePointer(&pool_dev, const_cast<void*>(bufs->host_pool), 0) != hipSuccess ||
      pool_dev == nullptr) {
    (void)hipGetLastError();
    return KVS_EINVAL;
  }
  // the device buffers must be device memory of the current device, each
  // allocation large enough for the capacity the caller states
  int device = -1;
  KVS_TRY_HIP(hipGetDevice(&device));
  KVS_TRY(check_device_buffer(bufs->hot, need.hot_bytes, device));
  KVS_TRY(check_device_buffer(bufs->meta, need.meta_bytes, device));
  KVS_TRY(check_device_buffer(bufs->scratch, need.scratch_bytes, device));
  if (need.cbuf_bytes != 0) KVS_TRY(check_device_buffer(bufs->cbuf, need.cbuf_bytes, device));

  kvs_pool* p = new (std::nothrow) kvs_pool();
  if (p == nullptr) return KVS_ENOMEM;
  p->cfg = *cfg;
  make_layout(cfg, &p->lay);
  p->prof_cap = 0;
  p->prof_used = 0;
  p->prof_steps = 0;
  p->prof_max_steps = 0;
  p->host_pool = (uint8_t*)const_cast<void*>(bufs->host_pool);
  const char* rx = getenv("KVS_ROCTX");
  p->roctx = rx != nullptr && rx[0] == '1';

  uint8_t* meta = (uint8_t*)bufs->meta;
  uint8_t* scr = (uint8_t*)bufs->scratch;
  const Layout& L = p->lay;
  DevPtrs& d = p->d;
  d.pool = (const uint16_t*)pool_dev;
  d.hot = (uint16_t*)bufs->hot;
  d.cbuf = (uint16_t*)bufs->cbuf;
  d.tok2slot = (int32_t*)(meta + L.tok2slot);
  d.slot2tok = (int32_t*)(meta + L.slot2tok);
  d.last_used = (int32_t*)(meta + L.last_used);
  d.order = (uint16_t*)(meta + L.order);
  d.stepctr = (int32_t*)(meta + L.stepctr);
  d.stats = (long long*)(meta + L.stats);
  d.status = (int32_t*)(meta + L.status);
  bind_scratch(L, scr, &d);
  p->last_scratch = d;
  p->stepped = false;

  p->device = device;
  p->static_scratch = nullptr;
  p->static_scratch_err = static_scratch_address(device, &p->static_scratch);
  hipError_t e = prepare_kernels();
  if (e == hipSuccess)
    e = launch_init_units(L, d, 0, L.B * L.L, /*reset_counters=*/true, (hipStream_t)stream);
  if (e != hipSuccess) {
    destroy_pool(p);
    return hip_err(e);
  }
  *out = p;
  return KVS_OK;
}

int kvs_publish(kvs_pool* p, int32_t req, int32_t layer, int64_t first_tok, int64_t n_tok,
                const void* rows) {
  if (p == nullptr || rows == nullptr) return KVS_EINVAL;
  if (req < 0 || req >= p->lay.B || layer < 0 || layer >= p->lay.L) return KVS_EINVAL;
  if (first_tok < 0 || n_tok < 0 || first_tok + n_tok > p->lay.N) return KVS_EINVAL;
  const uint64_t row0 = ((uint64_t)req * p->lay.L + layer) * (uint64_t)p->lay.N + first_tok;
  memcpy(p->host_pool + row0 * kRowBytes, rows, (size_t)n_tok * kRowBytes);
  return KVS_OK;
}

int kvs_publish_device(kvs_pool* p, int32_t req, int32_t layer, int64_t first_tok,
                       int64_t n_tok, const void* rows, void* stream) {
  if (p == nullptr || rows == nullptr) return KVS_EINVAL;
  if (req < 0 || req >= p->lay.B || layer < 0 || layer >= p->lay.L) return KVS_EINVAL;
  if (first_tok < 0 || n_tok < 0 || first_tok + n_tok > p->lay.N) return KVS_EINVAL;
  KVS_TRY(check_device(p, (hipStream_t)stream));
  if (n_tok == 0) return KVS_OK;
  const uint64_t row0 = ((uint64_t)req * p->lay.L + layer) * (uint64_t)p->lay.N + first_tok;
  return hip_err(hipMemcpyAsync(p->host_pool + row0 * kRowBytes, rows, (size_t)n_tok * kRowBytes,
                                hipMemcpyDeviceToHost, (hipStream_t)stream));
}

int kvs_append(kvs_pool* p, int32_t layer, const void* rows, const int64_t* pos, void* stream) {
  if (p == nullptr || rows == nullptr || pos == nullptr) return KVS_EINVAL;
  if (layer < 0 || layer >= p->lay.L) return KVS_EINVAL;
  if (((uintptr_t)rows & 15) != 0 || ((uintptr_t)pos & 7) != 0) return KVS_EINVAL;
  KVS_TRY(check_device(p, (hipStream_t)stream));
  return hip_err(launch_append(p->lay, p->d, layer, (const uint16_t*)rows, pos,
                               (hipStream_t)stream));
}

// Enqueues one layer step over the device pointers `d` (the pool's own
// scratch, or the library's static scratch for kvs_step_static).  `trace`
// allows the optional roctx range (kvs_step_static does without it: the
// tracer may allocate).
static int enqueue_step(kvs_pool* p, const DevPtrs& d, int32_t layer, const int32_t* topk,
                        const void* q, void* out, float* lse, hipStream_t s, bool trace) {
  const Layout& L = p->lay;
  // a host-side range for rocprofv3 --marker-trace (enqueue time, not GPU time)
  struct Range {
    bool on;
    Range(bool enable, int layer) : on(enable) {
      if (!on) return;
      char name[32];
      snprintf(name, sizeof(name), "kvs_step layer %d", layer);
      roctxRangePushA(name);
    }
    ~Range() {
      if (on) roctxRangePop();
    }
  } range(p->roctx && trace, layer);
  // lookup, sparse diff, LRU and map update for every request of the layer
  KVS_TRY_HIP(timed(p, KVS_KERNEL_DIFF_LRU, s, [&] { return launch_diff_lru(L, d, layer, topk, s); }));
  // optional verification of the updated state (not timed)
  if (L.flags & KVS_FLAG_CHECK) KVS_TRY_HIP(launch_check_state(L, d, layer, s));
  if (L.flags & KVS_FLAG_SEPARATE_ATTENTION) {
    // index copy: misses over PCIe (fetch + write-back) and hits within HBM
    KVS_TRY_HIP(timed(p, KVS_KERNEL_GATHER, s,
                      [&] { return launch_gather(L, d, layer, s); }));
    // Top-K sparse attention over the compute buffer
    KVS_TRY_HIP(timed(p, KVS_KERNEL_ATTENTION, s, [&] {
      return launch_attention(L, d, layer, (const uint16_t*)q, p->cfg.scale, (uint16_t*)out,
                              lse, s);
    }));
  } else {
    // index copy (misses over PCIe with write-back, hits within HBM) and the
    // attention over both, one partial per workgroup
    KVS_TRY_HIP(timed(p, KVS_KERNEL_ASSEMBLE, s, [&] {
      return launch_assemble(L, d, layer, (const uint16_t*)q, p->cfg.scale, s);
    }));
  }
  if (L.parts > 1 || !(L.flags & KVS_FLAG_SEPARATE_ATTENTION))
    KVS_TRY_HIP(timed(p, KVS_KERNEL_COMBINE, s,
                      [&] { return launch_combine(L, d, (uint16_t*)out, lse, s); }));
  if (p->prof_steps < p->prof_max_steps) ++p->prof_steps;
  p->last_scratch = d;
  p->stepped = true;
  return KVS_OK;
}

int kvs_step(kvs_pool* p, int32_t layer, const int32_t* topk, const void* q, void* out,
             float* lse, void* stream) {
  if (p == nullptr) return KVS_EINVAL;
  KVS_TRY(check_step_args(topk, q, out, lse));
  if (layer < 0 || layer >= p->lay.L) return KVS_EINVAL;
  const hipStream_t s = (hipStream_t)stream;
  KVS_TRY(check_device(p, s));
  return enqueue_step(p, p->d, layer, topk, q, out, lse, s, true);
}

int kvs_step_static(kvs_pool* p, int32_t layer, const int32_t* topk, const void* q, void* out,
                    float* lse, void* stream) {
  if (p == nullptr) return KVS_EINVAL;
  KVS_TRY(check_step_args(topk, q, out, lse));
  if (layer < 0 || layer >= p->lay.L) return KVS_EINVAL;
  if (p->lay.scratch_bytes > (uint64_t)KVS_STATIC_SCRATCH_BYTES) return KVS_ENOMEM;
  const hipStream_t s = (hipStream_t)stream;
  KVS_TRY(check_device(p, s));
  if (p->static_scratch == nullptr) return hip_err(p->static_scratch_err);
  // the same kernels, with every per-step list and partial in the static array
  DevPtrs d = p->d;
  bind_scratch(p->lay, (uint8_t*)p->static_scratch, &d);
  return enqueue_step(p, d, layer, topk, q, out, lse, s, false);
}

int kvs_free_request(kvs_pool* p, int32_t req, void* stream) {
  if (p == nullptr || req < 0 || req >= p->lay.B) return KVS_EINVAL;
  KVS_TRY(check_device(p, (hipStream_t)stream));
  return hip_err(launch_init_units(p->lay, p->d, req * p->lay.L, p->lay.L, false,
                                   (hipStream_t)stream));
}

int kvs_sync_status(kvs_pool* p, void* stream, kvs_step_stats* stats) {
  if (p == nullptr) return KVS_EINVAL;
  const hipStream_t s = (hipStream_t)stream;
  KVS_TRY_HIP(hipStreamSynchronize(s));
  int32_t status[4];
  KVS_TRY_HIP(hipMemcpyAsync(status, p->d.status, sizeof(status), hipMemcpyDeviceToHost, s));
  if (stats != nullptr) {
    const size_t units = (size_t)p->lay.B * p->lay.L;
    std::vector<long long> st(units * 4);
    KVS_TRY_HIP(hipMemcpyAsync(st.data(), p->d.stats, st.size() * sizeof(long long),
                               hipMemcpyDeviceToHost, s));
    KVS_TRY_HIP(hipStreamSynchronize(s));
    memset(stats, 0, sizeof(*stats));
    for (size_t u = 0; u < units; ++u) {
      stats->unit_steps += st[4 * u + 0];
      stats->hits += st[4 * u + 1];
      stats->misses += st[4 * u + 2];
      stats->evictions += st[4 * u + 3];
    }
    stats->host_bytes = stats->misses * kRowBytes;
    stats->status = status[0];
    if (status[0] == KVS_EBOUNDS) {   // the checked build's site and index, words 1..3
      stats->fault_site = status[1];
      stats->fault_index = (int64_t)(((uint64_t)(uint32_t)status[3] << 32) | (uint32_t)status[2]);
    }
  }
  KVS_TRY_HIP(hipStreamSynchronize(s));
  if (status[0] != 0) {
    KVS_TRY_HIP(launch_clear_status(p->d, s));
    KVS_TRY_HIP(hipStreamSynchronize(s));
  }
  return status[0];
}

int kvs_debug_read_state(kvs_pool* p, int32_t req, int32_t layer, void* stream,
                         kvs_unit_state* st) {
  if (p == nullptr || st == nullptr) return KVS_EINVAL;
  if (req < 0 || req >= p->lay.B || layer < 0 || layer >= p->lay.L) return KVS_EINVAL;
  const hipStream_t s = (hipStream_t)stream;
  const Layout& L = p->lay;
  const DevPtrs& d = p->d;
  const DevPtrs& ls = p->last_scratch;   // per-step lists of the last step
  const long long u = (long long)req * L.L + layer;
  auto get = [&](void* dst, const void* src, size_t bytes) -> hipError_t {
    if (dst == nullptr) return hipSuccess;
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, s);
  };
  KVS_TRY_HIP(get(st->tok2slot, d.tok2slot + u * L.N, (size_t)L.N * 4));
  KVS_TRY_HIP(get(st->slot2tok, d.slot2tok + u * L.Sp, (size_t)L.S * 4));
  KVS_TRY_HIP(get(st->last_used, d.last_used + u * L.Sp, (size_t)L.S * 4));
  KVS_TRY_HIP(get(st->slot_of, ls.slot_of + (long long)req * L.K, (size_t)L.K * 4));
  KVS_TRY_HIP(get(st->miss_pos, ls.miss_pos + (long long)req * L.K, (size_t)L.K * 4));
  KVS_TRY_HIP(get(st->victims, ls.victims + (long long)req * L.K, (size_t)L.K * 4));
  KVS_TRY_HIP(get(st->evicted, ls.evicted + (long long)req * L.K, (size_t)L.K * 4));
  KVS_TRY_HIP(get(st->counts, ls.counts + 4LL * req, 16));
  KVS_TRY_HIP(get(st->row_slot, ls.row_slot + (long long)req * L.K, (size_t)L.K * 4));
  std::vector<uint16_t> order(st->lru_order ? L.S : 0);
  KVS_TRY_HIP(get(st->lru_order ? order.data() : nullptr, d.order + u * L.Sp, (size_t)L.S * 2));
  int32_t step = 0;
  KVS_TRY_HIP(get(&step, d.stepctr + u, 4));
  KVS_TRY_HIP(hipStreamSynchronize(s));
  if (st->lru_order)
    for (int i = 0; i < L.S; ++i) st->lru_order[i] = order[i];
  st->step = step;
  return KVS_OK;
}

int kvs_profile_begin(kvs_pool* p, int32_t max_steps, uint32_t kernel_mask) {
  if (p == nullptr || max_steps < 0) return KVS_EINVAL;
  if ((kernel_mask >> KVS_NUM_KERNELS) != 0) return KVS_EINVAL;
  const size_t need = (size_t)max_steps * KVS_NUM_KERNELS;
  while (p->prof_ev.size() < need * 2) {
    // Timing only: no system-scope fence when the event is recorded.  With
    // the default fence every recorded event writes back and invalidates the
    // caches, which put about 5.5 us between a bracketed launch and its
    // neighbours (measured with rocprofv3 on MI355X).
    hipEvent_t e;
    KVS_TRY_HIP(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
    p->prof_ev.push_back(e);
  }
  p->prof_kernel.assign(need, 0);
  p->prof_cap = (int)need;
  p->prof_used = 0;
  p->prof_steps = 0;
  p->prof_max_steps = max_steps;
  p->prof_mask = kernel_mask;
  return KVS_OK;
}

int kvs_profile_end(kvs_pool* p, kvs_kernel_times* out) {
  if (p == nullptr || out == nullptr) return KVS_EINVAL;
  memset(out, 0, sizeof(*out));
  const int n = p->prof_used;
  for (int i = 0; i < n; ++i) {
    hipEvent_t* ev = &p->prof_ev[(size_t)i * 2];
    KVS_TRY_HIP(hipEventSynchronize(ev[1]));
    float ms = 0.f;
    KVS_TRY_HIP(hipEventElapsedTime(&ms, ev[0], ev[1]));
    out->ms_total[p->prof_kernel[i]] += ms;
    out->launches[p->prof_kernel[i]] += 1;
  }
  out->steps = p->prof_steps;
  p->prof_max_steps = 0;   // stop recording
  p->prof_used = 0;
  p->prof_steps = 0;
  return KVS_OK;
}

struct kvs_graph {
  hipGraphExec_t exec;
  int device;   // the pool's device: replays must go to a stream of it
};

int kvs_graph_capture(kvs_pool* p, int32_t layer, const int32_t* topk, const void* q, void* out,
                      float* lse, kvs_graph** out_graph) {
  if (out_graph == nullptr) return KVS_EINVAL;
  *out_graph = nullptr;
  if (p == nullptr) return KVS_EINVAL;
  KVS_TRY(check_step_args(topk, q, out, lse));
  if (layer < 0 || layer >= p->lay.L) return KVS_EINVAL;
  hipStream_t cs = nullptr;
  KVS_TRY_HIP(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  // no timing events inside the graph
  const int saved_max = p->prof_max_steps;
  p->prof_max_steps = 0;
  // a captured step runs only when the graph is launched: its lists are not
  // written yet (kvs_probe_hit_copy keeps refusing a pool that has run no step)
  const bool saved_stepped = p->stepped;
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  int rc = KVS_OK;
  hipGraph_t g = nullptr;
  if (e == hipSuccess) {
    rc = kvs_step(p, layer, topk, q, out, lse, cs);
    const hipError_t e2 = hipStreamEndCapture(cs, &g);   // always end the capture
    if (rc == KVS_OK && e2 != hipSuccess) rc = hip_err(e2);
  } else {
    rc = hip_err(e);
  }
  p->prof_max_steps = saved_max;
  p->stepped = saved_stepped;
  hipGraphExec_t exec = nullptr;
  if (rc == KVS_OK) {
    e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
    if (e != hipSuccess) rc = hip_err(e);
  }
  if (g != nullptr) (void)hipGraphDestroy(g);
  (void)hipStreamDestroy(cs);
  if (rc != KVS_OK) return rc;
  kvs_graph* kg = new (std::nothrow) kvs_graph();
  if (kg == nullptr) {
    (void)hipGraphExecDestroy(exec);
    return KVS_ENOMEM;
  }
  kg->exec = exec;
  kg->device = p->device;
  *out_graph = kg;
  return KVS_OK;
}

int kvs_graph_launch(kvs_graph* g, void* stream) {
  if (g == nullptr) return KVS_EINVAL;
  hipDevice_t dev = -1;
  if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess || dev != g->device) {
    (void)hipGetLastError();
    return KVS_EINVAL;
  }
  return hip_err(hipGraphLaunch(g->exec, (hipStream_t)stream));
}

int kvs_graph_destroy(kvs_graph* g) {
  if (g == nullptr) return KVS_EINVAL;
  const hipError_t e = hipGraphExecDestroy(g->exec);
  delete g;
  return hip_err(e);
}

int kvs_release(kvs_pool* p) {
  if (p == nullptr) return KVS_EINVAL;
  destroy_pool(p);
  return KVS_OK;
}

int kvs_probe_host_read(const void* host, uint64_t bytes, uint32_t* sink, void* stream) {
  if (host == nullptr || sink == nullptr || bytes == 0 || (bytes & 15) != 0) return KVS_EINVAL;
  if (((uintptr_t)host & 15) != 0 || ((uintptr_t)sink & 3) != 0) return KVS_EINVAL;
  void* dev = nullptr;
  if (hipHostGetDevicePointer(&dev, const_cast<void*>(host), 0) != hipSuccess || dev == nullptr) {
    (void)hipGetLastError();
    return KVS_EINVAL;
  }
  return hip_err(launch_host_read_probe(dev, (long long)(bytes / 16), sink, (hipStream_t)stream));
}

int kvs_probe_hit_copy(kvs_pool* p, int32_t layer, void* stream) {
  if (p == nullptr || layer < 0 || layer >= p->lay.L) return KVS_EINVAL;
  if ((p->lay.flags & KVS_FLAG_DIRECT_HOT) != 0 || !p->stepped) return KVS_EINVAL;
  const hipStream_t s = (hipStream_t)stream;
  KVS_TRY(check_device(p, s));
  return hip_err(launch_hit_copy(p->lay, p->last_scratch, layer, s));
}

const char* kvs_strerror(int code) {
  switch (code) {
    case KVS_OK: return "ok";
    case KVS_EINVAL: return "invalid argument or configuration";
    case KVS_ENOMEM: return "buffer smaller than kvs_query_sizes requires";
    case KVS_ERANGE: return "Top-K index or append position outside [0, context)";
    case KVS_EDUP: return "duplicate Top-K index within a request";
    case KVS_ECORRUPT: return "state check failed: maps, LRU order or victims break an invariant";
    case KVS_EBOUNDS: return "device-side bounds check failed (checked build)";
    default: break;
  }
  if (code <= KVS_EHIP_BASE) return "HIP runtime error (KVS_EHIP_BASE - hipError_t)";
  return "unknown error";
}

}  // extern "C"
