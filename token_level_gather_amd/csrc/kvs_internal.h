// Internal layout and launch interfaces shared by the host runtime and the
// gfx950 kernels of the sparse KV assembly library.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvs.h"

namespace kvs {

constexpr int kRowElems = KVS_HEAD_DIM;          // 576 bf16 per KV row
constexpr int kRowBytes = kRowElems * 2;         // 1152
constexpr int kRowChunks = kRowBytes / 16;       // 72 x 16-byte chunks per row
constexpr int kHeads = KVS_HEADS;                // 16
constexpr int kVDim = KVS_V_DIM;                 // 512

// Byte offsets of every array inside the caller's meta and scratch buffers.
struct Layout {
  int32_t B, L, S, K;
  int32_t splits;        // attention token splits per request: the hit splits of the
                         // assembling launch, or the splits of the separate attention
  int32_t parts;         // attention partials per request merged by the combine
  int32_t attn_wgs;      // separate attention: workgroups sharing the B * ceil(K/64) tiles
  int32_t fetch_blocks;  // miss-fetch workgroups of the gather launch
  int32_t fetch_per_req; // assembling launch: fetch workgroups per request
  int32_t hit_blocks;    // hit-copy workgroups of the gather launch (0 = one per 32 positions)
  int32_t flags;
  int32_t Sp;            // per-unit stride of slot2tok / last_used / order: S rounded up to 16
  int64_t N;
  // meta (persistent state)
  uint64_t tok2slot;   // int32 [B*L][N]
  uint64_t slot2tok;   // int32 [B*L][Sp]
  uint64_t last_used;  // int32 [B*L][Sp]
  uint64_t order;      // uint16 [B*L][Sp]: slots in ascending (last_used, slot)
  uint64_t stepctr;    // int32 [B*L]
  uint64_t stats;      // int64 [B*L][4]: steps, hits, misses, evictions
  uint64_t status;     // int32 [4]: sticky first error
  uint64_t meta_bytes;
  // scratch (per kvs_step call; request-indexed, reused across layers)
  uint64_t slot_of;    // int32 [B][K]
  uint64_t miss_pos;   // int32 [B][K]
  uint64_t victims;    // int32 [B][K]
  uint64_t evicted;    // int32 [B][K]
  uint64_t counts;     // int32 [B][4]: n_hit, n_miss, n_evict, valid
  uint64_t row_slot;   // int32 [B][K]: slot of position i's row after the step, -1 empty
  uint64_t hit_pos;    // int32 [B][K]: Top-K positions of the hits, Top-K order
  uint64_t hit_slot;   // int32 [B][K]: their slots
  uint64_t miss_tok;   // int32 [B][K]: tokens of the misses, Top-K order
  uint64_t part_o;     // float [B][parts][16][512]
  uint64_t part_ml;    // float [B][parts][16][2]: running max (log2 units), sum
  uint64_t scratch_bytes;
};

// Validates cfg and fills `lay`; returns KVS_OK or KVS_EINVAL.
int make_layout(const kvs_config* cfg, Layout* lay);

// Dynamic LDS bytes of the diff/LRU kernel for a layout.
size_t diff_lds_bytes(int S, int K);

// Device address of the library's static scratch (KVS_STATIC_SCRATCH_BYTES)
// on `device`, which must be the current device; resolved once per device.
hipError_t static_scratch_address(int device, void** out);

// Device pointers of one pool, resolved from the caller's buffers.
struct DevPtrs {
  const uint16_t* pool;  // host pool, device-visible address
  uint16_t* hot;
  uint16_t* cbuf;
  int32_t* tok2slot;
  int32_t* slot2tok;
  int32_t* last_used;
  uint16_t* order;
  int32_t* stepctr;
  long long* stats;
  int32_t* status;
  int32_t* slot_of;
  int32_t* miss_pos;
  int32_t* victims;
  int32_t* evicted;
  int32_t* counts;
  int32_t* row_slot;
  int32_t* hit_pos;
  int32_t* hit_slot;
  int32_t* miss_tok;
  float* part_o;
  float* part_ml;
};

// Kernel launchers (kvs_kernels.hip).  Each returns the launch's hipError_t.
// prepare_kernels sets per-kernel attributes on the current device (once per pool).
hipError_t prepare_kernels();
hipError_t launch_init_units(const Layout& lay, const DevPtrs& d, int unit_begin,
                             int unit_count, bool reset_counters, hipStream_t s);
hipError_t launch_diff_lru(const Layout& lay, const DevPtrs& d, int layer,
                           const int32_t* topk, hipStream_t s);
hipError_t launch_gather(const Layout& lay, const DevPtrs& d, int layer, hipStream_t s);
// With a single split the attention writes out / lse itself and no combine runs.
hipError_t launch_attention(const Layout& lay, const DevPtrs& d, int layer, const uint16_t* q,
                            float scale, uint16_t* out, float* lse, hipStream_t s);
hipError_t launch_combine(const Layout& lay, const DevPtrs& d, uint16_t* out, float* lse,
                          hipStream_t s);
// The index copy and the attention in one launch (default): fetch workgroups
// attend over the misses they fetch, hit workgroups over the resident hits.
hipError_t launch_assemble(const Layout& lay, const DevPtrs& d, int layer, const uint16_t* q,
                           float scale, hipStream_t s);
hipError_t launch_clear_status(const DevPtrs& d, hipStream_t s);
hipError_t launch_check_state(const Layout& lay, const DevPtrs& d, int layer, hipStream_t s);
// Measurement helper: the gather kernel's hit role alone (no fetch
// workgroups) over the lists in `d`, reading layer `layer`'s hot rows.
hipError_t launch_hit_copy(const Layout& lay, const DevPtrs& d, int layer, hipStream_t s);
hipError_t launch_host_read_probe(const void* src, long long chunks, uint32_t* sink,
                                  hipStream_t s);
hipError_t launch_append(const Layout& lay, const DevPtrs& d, int layer, const uint16_t* rows,
                         const int64_t* pos, hipStream_t s);

}  // namespace kvs
