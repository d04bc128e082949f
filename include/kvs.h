/*
 * kvs.h - C ABI of a per-decode-step sparse KV assembly library for AMD
 * Instinct MI355X (gfx950).
 *
 * What the library does, per decode step and per (request, layer) "unit":
 * it takes the Top-K token indices chosen by a sparse-attention selector,
 * looks them up in a device token-to-slot map of a fixed-size hot KV buffer in
 * HBM, splits them into hits and misses (the sparse diff), evicts by a
 * deterministic LRU rule, gathers hits from the hot buffer and misses from a
 * full-history KV pool in pinned host memory into a contiguous compute buffer
 * in Top-K order, writes the misses back into the hot buffer, and runs
 * MLA-style Top-K sparse decode attention over the gathered rows.
 *
 * Passages this follows:
 *  - "Sparse Attention-Driven KVCache Management for Domestic AI Supernodes"
 *    (abstract; agenda "Sparse-Driven System Design"): full history in a host
 *    memory pool, hot data cached on the device, an index mapping between them,
 *    Top-K indices driving token-level access, on-demand assembly by an
 *    index-based copy operator.
 *  - SGLang/Tair hierarchical sparse attention summary: a Top-k LRU buffer on
 *    the GPU (first paragraph), Top-k selection then attention over the
 *    selected tokens (second), incremental transfer of sparse changes through a
 *    "Sparse Diff Kernel" (third).
 *  - "XM-Sparse", HiSparse integration section: the request lifecycle
 *    publish -> fetch -> write-back -> free.
 *
 * Fixed by this library where the pages are silent:
 *  - A KV row is one token of an MLA layer: 576 bf16 values (512 latent +
 *    64 rope dims), 1152 bytes.  Attention uses all 576 dims for scores and
 *    dims 0..511 as values, 16 query heads, fp32 softmax and accumulation,
 *    bf16 output rounded to nearest-even.
 *  - LRU rule: the victims for the m misses of a step are the m slots that
 *    hold no token of the current Top-K set, taken in ascending
 *    (last_used_step, slot) order; an empty slot has last_used_step = -1.  The
 *    j-th miss in Top-K array order gets the j-th victim.  Hit slots and filled
 *    slots are stamped with the unit's step counter t, which counts the unit's
 *    valid steps (starting at 0).
 *
 * Conventions for every call:
 *  - Return value: KVS_OK (0) or a negative KVS_E* code; kvs_strerror names it.
 *  - "device" pointers are HIP device memory (for instance torch CUDA/HIP tensor
 *    storage); "host" pointers are ordinary host memory.  The library never
 *    allocates or frees device memory; the caller owns every buffer and keeps
 *    it alive until kvs_release.
 *  - A `stream` argument is a hipStream_t passed as void* (NULL = the default
 *    stream).  Calls only enqueue work on it, except where stated.
 *  - A pool is not thread-safe: calls on one pool must not overlap.
 *  - A pool's buffers live on the device current at kvs_create_pool; calls
 *    that enqueue work take a stream of that device (NULL = that device's
 *    default stream while it is current) and return KVS_EINVAL otherwise.
 *
 * Builds: libkvs.so, and libkvs_checked.so, the same library with device-side
 * bounds checks (a debugging aid, slower).  In the checked build every index
 * a kernel takes from the Top-K, the maps, the LRU order or the step's slot,
 * miss, victim and hit lists is compared with the extent of the array it
 * addresses before the access; a failure skips the access and latches
 * KVS_EBOUNDS, and kvs_step_stats.fault_site / fault_index name the access
 * (KVS_SITE_*) and the index.  State the normal build trusts (the LRU order is
 * a permutation of the slots, every slot-to-token entry lies in [-1, N)) is
 * verified before a step uses it; such a request is skipped untouched, like
 * an invalid Top-K.
 */
#ifndef KVS_H_
#define KVS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------ */
#define KVS_OK 0
#define KVS_EINVAL (-22)    /* bad argument or configuration */
#define KVS_ENOMEM (-12)    /* a caller buffer is smaller than kvs_query_sizes asks */
#define KVS_ERANGE (-34)    /* device saw a Top-K index outside [0, N) */
#define KVS_EDUP (-17)      /* device saw a repeated Top-K index within one request */
#define KVS_ECORRUPT (-74)  /* a unit's state breaks an invariant: a token-to-slot entry
                               outside [-1, S) seen by a step, or a KVS_FLAG_CHECK failure */
#define KVS_EBOUNDS (-14)   /* a device-side bounds check failed (libkvs_checked.so only) */
#define KVS_EHIP_BASE (-1000) /* KVS_EHIP_BASE - e: HIP runtime error e */

/* ---- limits ------------------------------------------------------------ */
#define KVS_HEADS 16
#define KVS_HEAD_DIM 576
#define KVS_V_DIM 512
#define KVS_MAX_SLOTS 16384
#define KVS_MAX_TOPK 8192

/* Indices of the per-kernel times in kvs_kernel_times.ms_total. */
#define KVS_KERNEL_DIFF_LRU 0   /* lookup + sparse diff + LRU + map update */
#define KVS_KERNEL_GATHER 1     /* index copy: misses host -> compute buffer + hot buffer
                                   (PCIe) and hits hot buffer -> compute buffer (HBM) */
#define KVS_KERNEL_ATTENTION 2  /* split-K sparse MLA decode (MFMA) */
#define KVS_KERNEL_COMBINE 3    /* merge of the attention partials */
#define KVS_KERNEL_ASSEMBLE 4   /* index copy and attention in one launch (default): misses
                                   over PCIe, hits within HBM, one partial per workgroup */
#define KVS_NUM_KERNELS 5

/* Accesses checked by libkvs_checked.so (kvs_step_stats.fault_site). */
#define KVS_SITE_LRU_ORDER 1   /* diff: an LRU order entry >= S, or a slot listed twice */
#define KVS_SITE_SLOT_TOKEN 2  /* diff: a slot-to-token entry outside [-1, N) */
#define KVS_SITE_DIFF_LIST 3   /* diff: a write position of the order, miss or hit lists */
#define KVS_SITE_MISS 4        /* copy: a miss's token, Top-K position or victim slot */
#define KVS_SITE_HIT 5         /* copy: a hit's slot or Top-K position */
#define KVS_SITE_ROW_SLOT 6    /* attention on rows in place: a row's slot */
#define KVS_SITE_APPEND 7      /* append: the slot of the appended token, outside [-1, S) */

/*
 * Shape of a pool.  B requests x L layers = B*L units; each unit has its own
 * host-pool slice, hot buffer, maps and step counter.
 */
typedef struct kvs_config {
  int32_t batch;        /* B >= 1 requests */
  int32_t layers;       /* L >= 1 layers */
  int64_t context;      /* N >= K tokens per unit in the host pool, N < 2^31 */
  int32_t slots;        /* S hot-buffer rows per unit, K <= S <= KVS_MAX_SLOTS */
  int32_t topk;         /* K Top-K indices per request per step, 1..KVS_MAX_TOPK */
  int32_t heads;        /* must be KVS_HEADS */
  int32_t head_dim;     /* must be KVS_HEAD_DIM */
  int32_t v_dim;        /* must be KVS_V_DIM */
  float scale;          /* softmax scale > 0, e.g. 1/sqrt(576) */
  int32_t attn_splits;  /* token splits per request in attention, 1..64 and at most ceil(K/64):
                           the hit workgroups per request of the assembling launch (each
                           attends over its share of the hits), or, with
                           KVS_FLAG_SEPARATE_ATTENTION, the attention's workgroups per
                           request (each takes an equal share of the request's 64-token
                           tiles); 0 = library's choice (separate attention: the
                           B*ceil(K/64) tiles shared evenly by at most 256 workgroups,
                           request after request, so one workgroup's share may span
                           requests) */
  int32_t fetch_blocks; /* workgroups that fetch misses over PCIe, 1..65535, spread evenly over
                           the requests (assembling launch: at most ceil(K/64) per request);
                           0 = library's choice */
  int32_t hit_blocks;   /* KVS_FLAG_SEPARATE_ATTENTION: workgroups that copy hits within HBM,
                           1..65535; 0 = library's choice.  Unused otherwise. */
  int32_t flags;        /* KVS_FLAG_* bits; 0 = default */
} kvs_config;

/* kvs_config.flags: give the hit-copy workgroups the first grid indices of the
 * gather launch (default: the PCIe fetch workgroups come first). */
#define KVS_FLAG_HITS_FIRST 1
/* kvs_config.flags: padded Top-K.  A selector may return fewer than K tokens
 * (a sequence shorter than K); a Top-K entry equal to -1 is then empty.  An
 * empty entry is neither a hit nor a miss: it reads no map, takes no slot,
 * does not shield any slot from eviction, gathers a zero row into cbuf and is
 * left out of the softmax.  A step whose entries are all empty still advances
 * the unit's step counter; its out row is zero and its lse -inf.  Without this
 * flag -1 is out of range (KVS_ERANGE).  The pages do not describe padding:
 * it completes the request lifecycle of "XM-Sparse", HiSparse integration
 * section, for requests shorter than K. */
#define KVS_FLAG_PADDED_TOPK 2
/* kvs_config.flags: attention reads each selected row in place from the hot
 * buffer (a hit at its slot, a miss at its victim slot after the write-back)
 * instead of from an assembled compute buffer.  The gather then only fetches
 * misses over PCIe into their victim slots; no hit row is copied and cbuf is
 * not used: kvs_query_sizes reports cbuf_bytes = 0 and kvs_buffers.cbuf may be
 * NULL.  Results are identical; the on-demand assembly of the pages (the
 * "Sparse Attention-Driven KVCache Management for Domestic AI Supernodes"
 * abstract: an index-based copy builds the step's data) becomes an indexed
 * read inside attention. */
#define KVS_FLAG_DIRECT_HOT 4
/* kvs_config.flags: after the diff of every step, verify each touched unit:
 * token-to-slot and slot-to-token maps are mutual inverses (all N tokens,
 * all S slots), the LRU order array holds every slot once in ascending
 * (last_used_step, slot) order, and no victim of the step is one of its hit
 * slots.  A violation latches KVS_ECORRUPT for kvs_sync_status.  One extra
 * launch per step that reads each unit's maps whole (4 B per token and
 * 10 B per slot): a debugging aid, not for timed runs. */
#define KVS_FLAG_CHECK 8
/* kvs_config.flags: run the index copy and the attention as separate launches
 * (gather, then attention over the complete compute buffer, then the merge of
 * its partials).  By default one assembling launch does both: workgroups
 * that fetch misses over PCIe attend over the rows they fetched, workgroups
 * that copy hits attend over the hits while the host link delivers the
 * misses, and a merge launch combines their partials.  Results are identical
 * within rounding; the compute buffer holds the same bytes either way. */
#define KVS_FLAG_SEPARATE_ATTENTION 16

/* Bytes each caller buffer must hold (see kvs_buffers). */
typedef struct kvs_sizes {
  uint64_t host_pool_bytes; /* B*L*N*576*2: the full-history pool, host */
  uint64_t hot_bytes;       /* B*L*S*576*2: hot KV buffer, device */
  uint64_t meta_bytes;      /* index maps, LRU state, counters, status, device */
  uint64_t cbuf_bytes;      /* B*K*576*2: compute buffer of one step, device (0 with
                               KVS_FLAG_DIRECT_HOT) */
  uint64_t scratch_bytes;   /* per-step lists and attention partials, device */
  int32_t attn_splits;      /* the resolved kvs_config.attn_splits these sizes assume
                               (KVS_FLAG_SEPARATE_ATTENTION: the attention partials per
                               request, the most workgroups one request's tiles span) */
  int32_t fetch_blocks;     /* resolved kvs_config.fetch_blocks */
} kvs_sizes;

/*
 * Buffers handed to kvs_create_pool.  Layouts (row = 576 bf16, row-major):
 *   host_pool [B][L][N] rows: token n of unit (b, l) at row (b*L + l)*N + n.
 *             Must come from kvs_host_alloc (pinned and mapped for the GPU).
 *   hot       [B][L][S] rows, device.
 *   cbuf      [B][K] rows, device; may be NULL with KVS_FLAG_DIRECT_HOT.
 *   meta, scratch: opaque device memory, 256-byte aligned.
 * The *_bytes fields state each buffer's capacity; a capacity below
 * kvs_query_sizes gives KVS_ENOMEM.  meta is initialised by kvs_create_pool.
 */
typedef struct kvs_buffers {
  const void* host_pool;
  void* hot;
  void* meta;
  void* cbuf;
  void* scratch;
  uint64_t host_pool_bytes;
  uint64_t hot_bytes;
  uint64_t meta_bytes;
  uint64_t cbuf_bytes;
  uint64_t scratch_bytes;
} kvs_buffers;

/* Totals over all units since kvs_create_pool (kvs_sync_status). */
typedef struct kvs_step_stats {
  int64_t unit_steps;   /* valid (request, layer) steps taken */
  int64_t hits;         /* Top-K entries found in the hot buffer */
  int64_t misses;       /* Top-K entries fetched from the host pool */
  int64_t evictions;    /* occupied slots overwritten */
  int64_t host_bytes;   /* bytes read from the host pool (misses * 1152) */
  int32_t status;       /* first device-detected error since the last sync, or KVS_OK */
  int32_t fault_site;   /* status KVS_EBOUNDS: the failed access (KVS_SITE_*), else 0 */
  int64_t fault_index;  /* status KVS_EBOUNDS: the index it was given, else 0 */
} kvs_step_stats;

/* Host copies of one unit's state, for tests (kvs_debug_read_state).  Each
 * pointer may be NULL; otherwise it must hold the stated count of int32. */
typedef struct kvs_unit_state {
  int32_t* tok2slot;    /* [N]: slot of token n, -1 if not resident */
  int32_t* slot2tok;    /* [S]: token in slot s, -1 if empty */
  int32_t* last_used;   /* [S]: step stamp of slot s, -1 if never used */
  int32_t* lru_order;   /* [S]: slots in ascending (last_used, slot) order */
  int32_t* slot_of;     /* [K]: last step of request b: slot of topk[i] before it, -1 = miss,
                           -2 = empty entry (KVS_FLAG_PADDED_TOPK) */
  int32_t* miss_pos;    /* [K]: Top-K positions of the misses, first n_miss valid */
  int32_t* victims;     /* [K]: slot given to the j-th miss, first n_miss valid */
  int32_t* evicted;     /* [K]: token that slot held, -1 if empty, first n_miss valid */
  int32_t* counts;      /* [4]: n_hit, n_miss, n_evicted, valid (1) / invalid input (0) */
  int32_t* row_slot;    /* [K]: slot holding topk[i]'s row after the step, -1 = empty entry */
  int32_t step;         /* out: the unit's step counter (steps taken) */
} kvs_unit_state;

/* Per-kernel device time summed over the launches recorded between
 * kvs_profile_begin and kvs_profile_end (HIP events on the launch streams). */
typedef struct kvs_kernel_times {
  int32_t steps;                      /* kvs_step calls recorded */
  int32_t launches[KVS_NUM_KERNELS];  /* launches recorded per kernel */
  float ms_total[KVS_NUM_KERNELS];    /* sum of launch durations, milliseconds */
} kvs_kernel_times;

typedef struct kvs_pool kvs_pool;

/* Validate `cfg` and report buffer sizes.  Pure host arithmetic, no GPU call.
 * KVS_EINVAL if the configuration is outside the limits above. */
int kvs_query_sizes(const kvs_config* cfg, kvs_sizes* out);

/* Allocate `bytes` of pinned host memory that GPU kernels can read directly
 * (same address on host and device).  *out receives the pointer; free it with
 * kvs_host_free after the last pool using it is released. */
int kvs_host_alloc(uint64_t bytes, void** out);
int kvs_host_free(void* ptr);

/* Create a pool over caller buffers and initialise its state on `stream`:
 * every unit empty (maps -1, last_used -1, LRU order 0..S-1), step counters,
 * stats and status 0.  Does not synchronise.
 * Checked first, with no GPU work: the configuration (KVS_EINVAL), NULL
 * buffers (KVS_EINVAL), stated capacities (KVS_ENOMEM) and alignment (hot and
 * cbuf 16 bytes, meta and scratch 256 bytes; KVS_EINVAL).  Then, through the
 * HIP runtime: host_pool must be pinned and GPU-mapped, and hot, meta, scratch
 * and cbuf must be device memory of the current device (KVS_EINVAL), each
 * allocation reaching at least kvs_query_sizes' bytes past the pointer
 * (KVS_ENOMEM). */
int kvs_create_pool(const kvs_config* cfg, const kvs_buffers* bufs, void* stream,
                    kvs_pool** out);

/* Lifecycle "publish": copy `n_tok` rows (host, 1152 B each) into the host pool
 * of unit (req, layer) starting at token `first_tok`.  Host memcpy; the caller
 * must not publish into a token that is resident in the hot buffer (free the
 * request first) nor while steps that read the pool are in flight. */
int kvs_publish(kvs_pool* pool, int32_t req, int32_t layer, int64_t first_tok,
                int64_t n_tok, const void* rows);

/* Lifecycle "publish" from device memory (a prefill's KV rows): enqueue on
 * `stream` a device-to-host copy of `n_tok` rows (device, [n_tok][576] bf16,
 * 1152 B each) into the host pool of unit (req, layer) from token `first_tok`.
 * The same rule as kvs_publish: the tokens must not be resident in the hot
 * buffer (use kvs_append for a token that may be).  KVS_EINVAL for bad
 * arguments; nothing is enqueued then. */
int kvs_publish_device(kvs_pool* pool, int32_t req, int32_t layer, int64_t first_tok,
                       int64_t n_tok, const void* rows, void* stream);

/* Lifecycle "publish" of one decode step's new KV rows, one per request
 * ("XM-Sparse", HiSparse integration section: publish -> fetch -> write-back
 * -> free; the new token of a decode step is published before later steps can
 * select it).  Enqueued on `stream`, one small kernel:
 *   rows [B][576] bf16, device: request b's new row for `layer`.
 *   pos  [B] int64, device: its token index in [0, N), or -1 for a request that
 *        appends nothing this step.
 * The row is written over PCIe into the host pool at (b, layer, pos[b]) and,
 * when that token is resident in the hot buffer, into its slot too, so hot
 * copies always equal the pool; no map or LRU state changes.  A position
 * outside [-1, N) skips that request and latches KVS_ERANGE for
 * kvs_sync_status.  Stream order makes the rows visible to later kvs_step
 * calls on the same stream and, after synchronisation, to the host. */
int kvs_append(kvs_pool* pool, int32_t layer, const void* rows, const int64_t* pos,
               void* stream);

/* Lifecycle "fetch + write-back" and the Top-K attention of one layer for all
 * B requests: kernel launches on `stream` only (diff, the assembling launch and
 * the merge of its partials; with KVS_FLAG_SEPARATE_ATTENTION diff, gather,
 * attention, and a merge when kvs_sizes.attn_splits > 1), no host
 * synchronisation, no device-to-host copy, no other stream.
 *   topk [B][K] int32, device, 4-byte aligned: request b's Top-K token indices,
 *        unique, in [0, N) (with KVS_FLAG_PADDED_TOPK also -1 = empty entry).
 *   q    [B][16][576] bf16, device, 16-byte aligned: queries.
 *   out  [B][16][512] bf16, device, 16-byte aligned: attention output.
 *   lse  [B][16] fp32, device, 4-byte aligned, or NULL: natural-log
 *        log-sum-exp of the scores.
 * KVS_EINVAL (nothing enqueued) for a NULL or misaligned pointer, a bad layer
 * or a stream of another device.
 * The compute buffer receives request b's rows at cbuf[b][i] = row of topk[b][i].
 * A request whose Top-K is invalid (KVS_ERANGE, KVS_EDUP), or whose map holds a
 * slot outside [-1, S) for one of its tokens (KVS_ECORRUPT), is skipped: its
 * state is unchanged, its out row is zero and its lse is -inf; the error is
 * latched for kvs_sync_status.  Other requests proceed.
 * Calls for one layer must be in decode order; cbuf is reused by every call. */
int kvs_step(kvs_pool* pool, int32_t layer, const int32_t* topk, const void* q,
             void* out, float* lse, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid allocation): kvs_step with
 * its per-step scratch (slot, miss and victim lists, counts and attention
 * partials) in a static device array of the library, KVS_STATIC_SCRATCH_BYTES
 * per GPU, instead of the pool's scratch buffer (which this call leaves
 * untouched).  The array exists once per GPU the library runs on, from the
 * first kvs_create_pool on that GPU until the process ends.  The call
 * allocates nothing, host or device.
 * Same arguments, results and errors as kvs_step, plus KVS_ENOMEM (nothing
 * enqueued) when the pool's kvs_sizes.scratch_bytes exceed
 * KVS_STATIC_SCRATCH_BYTES, and KVS_EHIP_* if the array's address could not
 * be resolved at kvs_create_pool.
 * Every call on one GPU, from any pool, shares that GPU's array and leaves
 * the last call's contents in it: calls that may run concurrently on one GPU
 * (different streams, or graphs replayed on them) race and must be ordered by
 * the caller.  kvs_debug_read_state reports the lists of a pool's last step
 * from the buffer that step used. */
#define KVS_STATIC_SCRATCH_BYTES (32u << 20)
int kvs_step_static(kvs_pool* pool, int32_t layer, const int32_t* topk, const void* q,
                    void* out, float* lse, void* stream);

/* Lifecycle "free": empty every layer of request `req` (maps -1, last_used -1,
 * LRU order 0..S-1).  Its step counters keep running.  Enqueued on `stream`. */
int kvs_free_request(kvs_pool* pool, int32_t req, void* stream);

/* Synchronise `stream`, then return the first device-detected error
 * (KVS_ERANGE / KVS_EDUP / KVS_ECORRUPT, and KVS_EBOUNDS in the checked
 * build) since the last call, or KVS_OK, and clear it.
 * `stats` (may be NULL) receives the running totals. */
int kvs_sync_status(kvs_pool* pool, void* stream, kvs_step_stats* stats);

/* Synchronising copy of unit (req, layer)'s state into host arrays (tests). */
int kvs_debug_read_state(kvs_pool* pool, int32_t req, int32_t layer, void* stream,
                         kvs_unit_state* st);

/* Record HIP-event times (one event pair around every launch of a kernel
 * whose bit (1 << KVS_KERNEL_*) is set in `kernel_mask`, on the stream it runs
 * on) for the next `max_steps` kvs_step calls.  The events are timing-only
 * (created without a system-scope fence, so recording them writes back no
 * cache); each pair still adds a little to the step, so timing runs bracket
 * only the kernels they need. */
int kvs_profile_begin(kvs_pool* pool, int32_t max_steps, uint32_t kernel_mask);
/* Synchronise and report the recorded times; stops recording. */
int kvs_profile_end(kvs_pool* pool, kvs_kernel_times* out);

/* A captured kvs_step (HIP graph), for callers that replay the decode step
 * with fixed buffers: the selector writes each step's Top-K into the same
 * `topk` buffer and the queries into the same `q` buffer, and the graph is
 * relaunched.  The graph holds no host synchronisation, no memset and no
 * host-side state: the step counters live in device memory, so every launch
 * is one more decode step of `layer` ("XM-Sparse", HiSparse integration: the
 * same path supports CUDA Graph on the pages' hardware). */
typedef struct kvs_graph kvs_graph;

/* Capture one kvs_step(pool, layer, topk, q, out, lse) into an executable
 * graph.  Nothing runs at capture time.  The buffers must stay valid while the
 * graph exists.  Errors as kvs_step, plus KVS_EHIP_* for graph API failures. */
int kvs_graph_capture(kvs_pool* pool, int32_t layer, const int32_t* topk, const void* q,
                      void* out, float* lse, kvs_graph** out_graph);
/* Enqueue one replay on `stream`. */
int kvs_graph_launch(kvs_graph* graph, void* stream);
int kvs_graph_destroy(kvs_graph* graph);

/* Destroy the pool's timing events and host-side state.  Caller buffers are untouched. */
int kvs_release(kvs_pool* pool);

/* ---- measurement helper (not a step of the path) ------------------------ */

/* The host link's zero-copy read ceiling, against which the miss fetch is
 * judged: read `bytes` of pinned host memory (from kvs_host_alloc; 16-byte
 * aligned, a multiple of 16 bytes) from the GPU with the fetch's own load
 * pattern (16 B per lane, consecutive lanes on consecutive 16-byte chunks,
 * 256 workgroups of 256 threads) and XOR-reduce it into `sink` (device,
 * KVS_PROBE_SINK_WORDS uint32, overwritten).  Enqueued on `stream`; the
 * caller times it with events on that stream.  KVS_EINVAL for a pointer the
 * GPU cannot address or a bad size or alignment. */
#define KVS_PROBE_SINK_WORDS 65536
int kvs_probe_host_read(const void* host, uint64_t bytes, uint32_t* sink, void* stream);

/* The hit index copy alone (the index copy of "Sparse Attention-Driven KVCache
 * Management for Domestic AI Supernodes", abstract: rows moved by index into a
 * contiguous compute buffer), for timing it apart from the attention it is
 * fused with in the default step: for every request whose last step was
 * valid, copy the rows at the hit slots of the pool's last step (its per-step
 * lists) from layer `layer`'s hot buffer to the compute buffer, within HBM,
 * with the copy kernel of KVS_FLAG_SEPARATE_ATTENTION steps (1152 B read and
 * 1152 B written per hit).  Miss rows are left alone; an empty entry of a
 * padded Top-K gets a zero row, as in a step.  Enqueued on `stream` (a stream
 * of the pool's device), nothing else changes; the caller times it with
 * events on that stream.  When `layer` is not the last
 * step's layer the compute buffer then holds rows of `layer` at the last
 * step's slots: a measurement, not a step result.  KVS_EINVAL for a NULL
 * pool, a layer outside [0, L), a pool without compute buffer
 * (KVS_FLAG_DIRECT_HOT), a pool that has run no step, or a stream of another
 * device. */
int kvs_probe_hit_copy(kvs_pool* pool, int32_t layer, void* stream);

/* Static description of a return code. */
const char* kvs_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* KVS_H_ */
