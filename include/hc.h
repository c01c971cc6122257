/*
 * hc.h -- C ABI of the HiCache host<->device KV page transfer library (libhc.so),
 * written for AMD Instinct MI355X (gfx950).
 *
 * The library moves KV-cache rows between a layer-first device pool (one buffer
 * per layer and sub-buffer, indexed by token slot) and a page-first pinned host
 * pool (indexed by host token = page * page_size + row), in both directions:
 *
 *   write-back (device -> host), all layers in one call, the staged
 *     layer-first -> page-first write-back of the hybrid-pool write-back page
 *     (prhub summary of sglang PR 28434: implementation breakdown and the
 *     host-pool / CPU-mock source excerpts);
 *   load-back (host -> device), one layer per call, each call recording a
 *     layer-done event so a forward pass can start layer l while later layers
 *     are still in flight (loader-thread page, sglang PR 38472: Motivation and
 *     Modifications; rank-sharded host tier page, sglang PR 41984);
 *   the per-layer exchange of a rank-sharded host tier (rank-sharded host tier
 *     page, Modifications): the owner of a layer packs the rows it loaded into a
 *     staging buffer, the other TP ranks unpack the broadcast bytes into the
 *     same slots (device memory only; the broadcast is the caller's).
 *
 * Host layouts:
 *   HC_LAYOUT_PAGE_FIRST      per sub-buffer [page][layer][row][elem_bytes]
 *                             (page_first_direct on the loader-thread page);
 *                             sub-buffer regions follow each other in order.
 *   HC_LAYOUT_KV_SPLIT_SHARD  [shard = page]{ sub 0 page | sub 1 page | ... | zero pad },
 *                             each sub page [layer][row][elem_bytes], shard size
 *                             rounded up to shard_align (CacheStore H2H page,
 *                             unified-cache-management PR 1292, section
 *                             "page_first_kv_split support"; Direct I/O uses 4096).
 *   HC_LAYOUT_PAGE_FIRST_TOKEN_MAJOR
 *                             per sub-buffer [page][row][layer][elem_bytes], i.e. host
 *                             token t = page * page_size + row holds its layers back to
 *                             back (the host-pool staging shape and the CPU mock
 *                             host[token, layer] of the hybrid-pool write-back page);
 *                             page blocks stay [page][layer].
 * A sub-buffer holds either token rows (HC_TOKEN_ROWS: elem_bytes per token per
 * layer) or page blocks (HC_PAGE_BLOCKS: elem_bytes per page per layer, e.g. the
 * DSA indexer-K page of 64 fp8 keys and 64 fp32 scales).  A page block moves
 * with the token at row 0 of its page, to/from device block slot / page_size.
 *
 * Payload bytes are never interpreted: bf16, fp8 and fp32 all move bit-exactly.
 *
 * Each write-back, load-back and graph launch call is a roctx range named after
 * the function, visible to rocprofv3 --marker-trace.
 *
 * Conventions for every call:
 *   - Return value: HC_OK (0) or a negative hc_status.  hc_last_error() returns
 *     a message for the calling thread's last failure.
 *   - Ownership: the caller owns every buffer, stream and event passed in and
 *     keeps them alive until the copy stream has drained.  The library owns only
 *     the pool handle and its small scratch (index plans, counters).
 *   - Threads: a pool's calls may come from several threads at once; the pool
 *     takes them one at a time (one lock per pool), so its copy stream sees them
 *     in the order they took the lock.  Handles must outlive every call on them.
 *   - Asynchrony: transfer calls enqueue on the pool's copy stream and return.
 *     Work on the copy stream runs in call order.  A caller whose index lists
 *     or device rows are produced on another stream must order that stream
 *     before the call (event record + hipStreamWaitEvent on the copy stream).
 *   - Indices are int64 token indices.  Device and host indices are each
 *     distinct and in range; with page-block sub-buffers every page named is
 *     named whole, as P consecutive list entries in row order (rows 0..P-1)
 *     that map onto one whole device page the same way, so the row-0 tokens sit
 *     at list positions k * P.  A host list
 *     read on the CPU is checked before anything is enqueued.  A list the kernels
 *     read must be device memory of the pool's device or pinned host memory and
 *     hold n entries inside its allocation; anything else (pageable host memory,
 *     a short buffer) is refused with HC_ERR_INVALID before any launch, and the
 *     write-back's host list must not be device memory.  Device-resident
 *     lists are read by the kernels, which range-check every index, skip an
 *     out-of-range row and report it as HC_ERR_DEVICE at the next
 *     hc_round_trip_check or hc_pool_sync; distinctness of device-resident lists
 *     is trusted.  Pools created with HC_FLAG_VALIDATE also check, on the device,
 *     that page-block rows form whole device pages (reported the same way).
 *   - Sizes: elem_bytes is a multiple of 16 (16-byte vectors, the element-size
 *     rule of the hybrid-pool write-back page) and at most 65536; every device
 *     layer pointer, the host pool and the staging buffer are 16-byte aligned.
 *   - Graph capture: hc_load_back_layer, hc_layer_pack and hc_layer_unpack may be
 *     recorded into a caller's HIP graph on the pool's stream; a replay reads the
 *     index lists and buffers as they are when it runs, and a pool created with
 *     HC_FLAG_PROFILE does not time the launches it records.  While the pool's
 *     stream is capturing, hc_write_back_all_layers (its plan is built on the CPU
 *     for each call, so a replay would reuse a stale plan), hc_pool_sync and
 *     hc_round_trip_check (both wait for the stream) return HC_ERR_UNSUPPORTED
 *     and enqueue nothing; so do hc_pool_create on a copy stream that is
 *     capturing (its set-up copies and waits) and hc_pool_destroy (it waits for
 *     the stream; nothing is freed, destroy the pool after the capture ends).
 */
#ifndef HC_H
#define HC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HC_MAX_SUBBUFS 4
#define HC_MAX_LAYERS 1024
#define HC_MAX_ELEM_BYTES 65536

typedef enum hc_status {
  HC_OK = 0,
  HC_ERR_INVALID = -1,     /* bad argument: null pointer, negative count, value out of range */
  HC_ERR_UNSUPPORTED = -2, /* well-formed but not handled: elem_bytes % 16, misalignment, mode */
  HC_ERR_HIP = -3,         /* a HIP runtime call failed (the message names it) */
  HC_ERR_NOMEM = -4,       /* the library could not allocate its own scratch */
  HC_ERR_DEVICE = -5,      /* a kernel flagged an index list: an out-of-range entry (always checked),
                              or page-block rows that are not one whole device page (HC_FLAG_VALIDATE) */
  HC_ERR_BUSY = -6         /* host-to-host queue capacity exhausted; nothing was submitted */
} hc_status;

enum { HC_TOKEN_ROWS = 0, HC_PAGE_BLOCKS = 1 };
enum { HC_LAYOUT_PAGE_FIRST = 0, HC_LAYOUT_KV_SPLIT_SHARD = 1, HC_LAYOUT_PAGE_FIRST_TOKEN_MAJOR = 2 };
/* Transfer modes.  STAGED: device kernels relayout through the device staging
 * buffer and the copy engines (hipMemcpyAsync) cross the host link.  ZEROCOPY:
 * kernels read or write the pinned host pool directly.  AUTO: write-back is staged
 * when the descriptor brings a staging buffer of at least one page image, else
 * zero-copy; load-back is zero-copy (hc_pool_mode reports the choice).
 * Measured on MI355X: zero-copy write-back reaches ~99 % of the host-link peak, but
 * while its kernel saturates the link, compute kernels on other streams slow down
 * until they barely overlap it; staged write-back runs ~12 % slower alone and leaves
 * concurrent compute almost untouched, because the copy engines carry its host
 * writes (which engine runs a copy is the runtime's choice: the library pads each
 * burst's plan upload to 256 KiB, after which the runtime sent the region copies to
 * the copy engines in every traced burst of 2 MB plans and in most small ones).  Zero-copy load-back overlaps compute well on its default grid.  Either way
 * the overlap needs the compute on a stream that does not share a hardware queue with
 * the copy stream: HIP maps a process's streams onto GPU_MAX_HW_QUEUES queues (4 by
 * default), and work on a shared queue runs in that queue's order (measured: with 4
 * queues one compute stream in five waited behind the whole burst; with 16, none). */
enum { HC_MODE_AUTO = 0, HC_MODE_STAGED = 1, HC_MODE_ZEROCOPY = 2 };
/* Pool flags. */
enum { HC_FLAG_VALIDATE = 1, HC_FLAG_PROFILE = 2 };

typedef struct hc_subbuf_desc {
  int32_t granularity;        /* HC_TOKEN_ROWS or HC_PAGE_BLOCKS */
  int32_t reserved;           /* must be 0 */
  int64_t elem_bytes;         /* bytes per token row (or per page block) per layer */
  void* const* device_layers; /* host array of num_layers device pointers; layer l holds
                                 device_slots rows (token rows) or device_slots/page_size
                                 blocks (page blocks) of elem_bytes each.  The array is
                                 read during hc_pool_create only. */
} hc_subbuf_desc;

/* Both directions at once: two pools over the same device and host buffers, each on
 * its own copy stream (their rows must not overlap).  Who issues the host accesses
 * decides how the link is shared (measured on MI355X, PCIe 5.0 x16): a staged
 * write-back pool (copy engines) beside a zero-copy load-back pool whose max_ctas is
 * HC_DUPLEX_LOAD_BACK_CTAS moves both directions near 45 GB/s each, ~0.9 of what
 * hipMemcpyAsync reaches in both directions at once; at the default 16 the load-back keeps
 * its full rate and the write-back backs off (load-back first, for a forward pass that
 * waits on it); a zero-copy write-back on 16 workgroups holds the link and starves
 * concurrent load-backs to ~30 GB/s. */
#define HC_DUPLEX_LOAD_BACK_CTAS 8

typedef struct hc_pool_desc {
  int32_t num_layers;   /* L, 1..HC_MAX_LAYERS */
  int32_t page_size;    /* P tokens per page, >= 1 */
  int32_t num_subbufs;  /* 1..HC_MAX_SUBBUFS */
  int32_t layout;       /* HC_LAYOUT_* */
  hc_subbuf_desc sub[HC_MAX_SUBBUFS];
  int64_t device_slots; /* S token slots per layer (a multiple of P when a sub-buffer holds page blocks) */
  int64_t host_pages;   /* H pages (shards) in the host pool.  0 makes a device-only pool: host_base
                           and staging are NULL, write-back and load-back are refused, and only the
                           layer exchange and the round-trip check run on it (a TP rank's view of
                           every layer of its replicated device pool, next to the pool of the host
                           layers it owns) */
  int64_t shard_align;  /* shard layout: power of two >= 16 (4096 for Direct I/O); ignored otherwise */
  void* host_base;      /* pinned host memory (hc_host_alloc or hipHostMalloc), >= hc_host_pool_bytes */
  int64_t host_bytes;   /* size of host_base */
  void* staging;        /* device memory for staged write-back (HC_MODE_STAGED, or HC_MODE_AUTO when it
                           holds at least one page image); NULL when no staged mode is used.  The
                           pool writes it during every staged write-back: pools whose transfers can
                           run at the same time (other streams) need their own staging buffers.
                           Pools used one after the other may share one: each staged burst rewrites
                           what it sends, shard pads included. */
  int64_t staging_bytes;/* size of staging; the chunk is staging_bytes / hc_staging_page_bytes pages,
                           capped so that one chunk fits the 256 MB Infinity Cache (at least 1 page) */
  void* copy_stream;    /* hipStream_t every transfer of this pool is enqueued on (NULL: null stream) */
  int32_t write_back_mode; /* HC_MODE_* */
  int32_t load_back_mode;  /* HC_MODE_* (load-back is always zero-copy in this version) */
  int32_t flags;           /* HC_FLAG_* */
  int32_t max_ctas;        /* cap on workgroups of the zero-copy kernels, 0..65536; 0 = library default (16:
                              the link saturates with 8, and idle CUs stay free for compute).  With a
                              write-back and a load-back running at once (two pools, two streams) the
                              caps decide how the link is shared: beside a staged write-back, a load-back
                              pool at 16 keeps its full rate, at 8 both directions move ~45 GB/s
                              (measured); a zero-copy write-back at 16 starves concurrent load-backs. */
} hc_pool_desc;

typedef struct hc_pool hc_pool; /* opaque, library-owned */

/* ---------------------------------------------------------------- layout queries (host only)
 * These run on the CPU and touch no GPU. */

/* Checks a descriptor's geometry, layout and sizes (not its pointers' memory kinds).
 * HC_ERR_INVALID / HC_ERR_UNSUPPORTED with a message, else HC_OK. */
int hc_desc_check(const hc_pool_desc* desc);

/* Bytes the host pool needs for desc's layout: H * (sum of sub-buffer pages) for
 * page-first, H * shard stride for the shard layout. */
int hc_host_pool_bytes(const hc_pool_desc* desc, int64_t* out_bytes);

/* Staging bytes per page of a chunk: the shard stride for the shard layout (each page
 * is staged as its whole shard image, pad included), the summed sub-buffer pages for the
 * page-first layouts (a chunk holds each sub-buffer's pages together, so that pages
 * adjacent in the host pool leave staging as one copy).  A chunk of C pages takes C times
 * this. */
int hc_staging_page_bytes(const hc_pool_desc* desc, int64_t* out_bytes);

/* Byte offset of (sub-buffer, page, layer, row) in the host pool.  For a page-block
 * sub-buffer the row is ignored.  HC_ERR_INVALID when any coordinate is out of range. */
int hc_host_offset(const hc_pool_desc* desc, int32_t sub, int64_t page, int32_t layer,
                   int32_t row, int64_t* out_offset);

/* ---------------------------------------------------------------- pinned host memory */

/* Page-locked host allocation through hipHostMalloc (device-mapped).  flags: 0 =
 * coherent, 1 = non-coherent.  The memory is zero-filled (through the device
 * mapping).  *out is 4096-aligned. */
int hc_host_alloc(int64_t bytes, int32_t flags, void** out);
int hc_host_free(void* ptr);

/* ---------------------------------------------------------------- pool lifetime */

/* Validates desc, copies the per-layer pointer tables to device memory, and
 * records the modes.  The descriptor follows the host-pool excerpt of the
 * hybrid-pool write-back page (prhub summary of sglang PR 28434, key source
 * excerpts): the host pool is page-first, the device staging buffer for the
 * staged write-back is allocated once, up front, and sized in pages (its chunk),
 * per-layer device pointers are kept in a table (as the pools' k_data_ptrs), and
 * the element size per token must be a multiple of 16 bytes.  The pool belongs to
 * the current HIP device: the layer
 * buffers, the staging buffer and copy_stream must be that device's
 * (HC_ERR_INVALID otherwise), and every later call makes it current.  Each device
 * layer, the used part of the staging buffer and (when HIP can look it up) the host
 * pool must fit inside their allocations, else HC_ERR_INVALID.  Refused
 * (HC_ERR_UNSUPPORTED) while copy_stream is capturing a graph: set-up copies the
 * layer tables on it and waits. */
int hc_pool_create(const hc_pool_desc* desc, hc_pool** out);

/* Waits for the pool's copy stream, then frees the handle and its scratch.  NULL is a no-op.
 * Refused (HC_ERR_INVALID, nothing freed) while a loader or a captured load-back graph
 * created on the pool still exists: destroy those first; and (HC_ERR_UNSUPPORTED,
 * nothing freed) while the copy stream is capturing a graph. */
int hc_pool_destroy(hc_pool* pool);

/* The mode write-back (which = 0) or load-back (which = 1) resolves to
 * (HC_MODE_STAGED or HC_MODE_ZEROCOPY). */
int hc_pool_mode(const hc_pool* pool, int32_t which, int32_t* out_mode);

/* Blocks until the copy stream has drained; reports HC_ERR_DEVICE when a kernel
 * flagged an index list since the last report (an out-of-range index, or with
 * HC_FLAG_VALIDATE page-block rows that do not form whole device pages).  The
 * message names the smallest list position (index i of the call's lists) flagged
 * by any call since then.  The report is cleared once returned. */
int hc_pool_sync(hc_pool* pool);

/* ---------------------------------------------------------------- transfers */

/* Write-back of all layers and sub-buffers (device -> host):
 *   host[sub b][page h/P][layer l][row h%P] <- device[sub b][layer l][slot d]
 * for every pair (d = device_idx[i], h = host_idx[i]), i < n; page blocks move
 * with the row-0 token of each page; in the shard layout the pad bytes of every
 * shard named become zero; nothing else in the host pool changes.
 *   device_idx: n int64 in device memory (or pinned host memory), read on the GPU.
 *   host_idx:   n int64 in host memory, read by the CPU during the call (the
 *               plan of host regions is built once per burst); may be freed
 *               when the call returns.
 *   done_event: hipEvent_t recorded on the copy stream after the last byte is
 *               enqueued, or NULL.
 * n must be below 2^31 (the plan numbers tokens in int32), else HC_ERR_INVALID.
 * Errors are reported before anything is enqueued; done_event is still
 * recorded on error when the pool is valid. */
int hc_write_back_all_layers(hc_pool* pool, const int64_t* device_idx, const int64_t* host_idx,
                             int64_t n, void* event);

/* Write-back that allocates nothing, for callers that cannot allocate device or
 * pinned memory in the middle of their work (tight serving loops, harnesses that
 * forbid hipMalloc): hc_write_back_all_layers grows its plan buffers with
 * hipHostMalloc / hipMalloc when a burst is larger than any before it (waiting
 * for the copy stream first); this variant never calls an allocator (device,
 * pinned or host heap: its host-side scratch is the pool's, sized at creation).  Its plan, a
 * device copy of host_idx, lives in a fixed array of HC_NOALLOC_MAX_TOKENS int64
 * entries (2 MiB) that every GPU the library runs on holds from the library's load
 * until the process ends.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (pools on different streams) race on it; calls on one
 * stream run in order.  The result is exactly hc_write_back_all_layers' on a
 * zero-copy pool: the same rows move with the same kernel, and shard pads of the
 * named pages become zero.
 *   pool:       its write-back mode must resolve to zero-copy (HC_ERR_UNSUPPORTED
 *               otherwise: the staged write-back plans copy-engine regions and a
 *               staging layout per burst).
 *   device_idx: n int64 in device memory (or pinned host memory), read on the GPU.
 *   host_idx:   n int64 in pinned host memory mapped at its host address
 *               (hc_host_alloc or hipHostMalloc), else HC_ERR_INVALID.  The CPU
 *               checks it during the call (range, distinctness, whole pages with
 *               page blocks) and the copy stream copies it into the array, so it
 *               must not change until the copy stream has passed this call.
 *   n:          0..HC_NOALLOC_MAX_TOKENS; larger is HC_ERR_INVALID, enqueueing
 *               nothing.
 *   event:      as for hc_write_back_all_layers (recorded on error too).
 * Refused while the pool's stream is capturing, like hc_write_back_all_layers.
 * Pools created with HC_FLAG_PROFILE do not time this call's kernels. */
#define HC_NOALLOC_MAX_TOKENS 262144
int hc_write_back_all_layers_noalloc(hc_pool* pool, const int64_t* device_idx, const int64_t* host_idx,
                                     int64_t n, void* event);

/* Load-back of one layer (host -> device):
 *   device[sub b][layer][slot d] <- host[sub b][page h/P][layer][row h%P]
 * for every pair (h = host_idx[i], d = device_idx[i]), i < n, every sub-buffer;
 * only layer `layer` of the device pool changes.
 *   host_idx, device_idx: n int64 each, in device memory (or pinned host
 *               memory), read on the GPU: no CPU-side descriptor is built.
 *   event:      hipEvent_t recorded on the copy stream once this layer's rows
 *               are enqueued (the layer-done event), or NULL.
 * The event is recorded even when the call fails (on the pool's copy stream,
 * or on the null stream when pool is NULL), so a consumer waiting on it never
 * hangs; the layer's rows are then stale. */
int hc_load_back_layer(hc_pool* pool, int32_t layer, const int64_t* host_idx,
                       const int64_t* device_idx, int64_t n, void* event);

/* Round-trip check.  The pages print no such call: its name and meaning are this
 * library's own, the check that a write-back followed by a load-back into other
 * slots restored every row (the accuracy claim of the rank-sharded tier page,
 * Accuracy Tests: pages come back bit-exactly).  It counts the (token,
 * sub-buffer, layer) units whose device
 * rows at slots idx_a[i] and idx_b[i] differ, over all layers and sub-buffers
 * (page blocks once per page, at tokens with idx_a[i] % P == 0).  Indices are
 * device-resident.  Synchronizes the copy stream and writes the count to
 * *mismatched_units (host memory). */
int hc_round_trip_check(hc_pool* pool, const int64_t* idx_a, const int64_t* idx_b, int64_t n,
                        int64_t* mismatched_units);

/* ---------------------------------------------------------------- layer exchange of a rank-sharded tier
 * A layer-owner sharded host tier (rank-sharded tier page, sglang PR 41984,
 * Modifications) gives each host layer one owner rank, round-robin over the TP
 * ranks; device pools and slot allocation stay replicated.  Write-back and
 * load-back of a rank then cover only its own layers: a pool over the device
 * buffers of the owned layers (the descriptor takes one pointer per layer) with a
 * host pool of those layers.  On load-back, once the owner has loaded layer l into
 * its device slots, it packs those rows into a staging buffer, the buffer is
 * broadcast to the other TP ranks (the caller's collective on its own
 * communicator; not part of this library), and each of them unpacks it into the
 * same slots.  Each rank's layer-done event follows its own exchange.  Pack and
 * unpack run on any pool, including a device-only one (host_pages = 0) over all
 * layers, which is how a rank addresses the layers it does not own.
 *
 * Staging bytes: sub-buffer after sub-buffer; inside sub-buffer b the token rows
 * of device_idx[0..n) in list order (n * elem_bytes), or for page blocks the block
 * of each page, taken at list positions 0, P, 2P, ... ((n / P) * elem_bytes).
 *   device_idx: n int64 slots in device memory (or pinned host memory), read on the
 *               GPU, distinct, the same list on every rank; with page blocks n is a
 *               multiple of P and every page is named whole in row order.
 *   dst / src:  device memory of the pool's device, 16-byte aligned, holding at
 *               least hc_layer_pack_bytes(n) bytes inside its allocation (dst_bytes /
 *               src_bytes give the caller's size; smaller is HC_ERR_INVALID).
 *   event:      hipEvent_t recorded on the copy stream after the kernel, or NULL;
 *               recorded on failure too (on the null stream when pool is NULL).
 * Out-of-range slots are skipped and reported as HC_ERR_DEVICE by the next
 * hc_pool_sync (a skipped slot leaves its staging row, or its device row, as it
 * was); with HC_FLAG_VALIDATE page-block slots are also checked to form whole
 * device pages.  Only layer `layer` of the device pool (unpack) or the staging
 * buffer (pack) changes.  Neither call touches the host link; hc_pool_stats does
 * not count them. */
int hc_layer_pack_bytes(const hc_pool* pool, int64_t n, int64_t* out_bytes);
int hc_layer_pack(hc_pool* pool, int32_t layer, const int64_t* device_idx, int64_t n, void* dst,
                  int64_t dst_bytes, void* event);
int hc_layer_unpack(hc_pool* pool, int32_t layer, const void* src, int64_t src_bytes,
                    const int64_t* device_idx, int64_t n, void* event);

/* ---------------------------------------------------------------- captured load-back bursts
 * The per-layer load-back chain of one burst, captured once into a HIP graph on
 * the pool's copy stream: L hc_load_back_layer calls, each with its layer-done
 * event record (loader-thread page, sglang PR 38472, Motivation: the per-layer
 * enqueue is launch overhead the forward pass waits behind).  A replay re-runs
 * all L layers with whatever the two index lists hold when it executes; the
 * lists' addresses, n and the events are fixed at capture.  One graph launch
 * replaces L kernel launches and L event records on the CPU.
 *
 * hc_load_back_graph_create: host_idx / device_idx are device-resident lists of n
 * entries that stay allocated while the graph lives; layer_events holds L
 * caller-owned events (entries may be NULL: no record for that layer).  Captures
 * in thread-local mode, so the pool's stream must not be capturing already and
 * nothing else may be enqueued on it from this thread meanwhile.  Pools created
 * with HC_FLAG_PROFILE are refused (HC_ERR_UNSUPPORTED): their per-launch timing is
 * not part of a graph.  On any failure nothing stays captured and *out is NULL.
 * hc_load_back_graph_launch enqueues one replay on the pool's copy stream (FIFO
 * with the pool's other calls).  hc_load_back_graph_destroy frees the graph (NULL
 * is a no-op); destroy graphs before their pool. */
typedef struct hc_lb_graph hc_lb_graph;
int hc_load_back_graph_create(hc_pool* pool, const int64_t* host_idx, const int64_t* device_idx, int64_t n,
                              void* const* layer_events, hc_lb_graph** out);
int hc_load_back_graph_launch(hc_lb_graph* graph);
int hc_load_back_graph_destroy(hc_lb_graph* graph);

/* ---------------------------------------------------------------- asynchronous load-back enqueue
 * A loader runs the per-layer load-back of whole bursts off the caller's thread
 * (loader-thread page, sglang PR 38472, Modifications): the caller hands over a
 * burst and returns at once; one FIFO worker thread makes the transfer stream
 * wait for the burst's start event, enqueues every layer in order and records
 * each layer's event.  Each layer also has a CPU-side "recorded" flag, because a
 * stream that waits on an event nobody has recorded yet does not wait at all:
 * hc_burst_wait_layer first blocks on the flag, then makes the consumer stream
 * wait on the device event.  Bursts complete in submission order.  If enqueueing
 * layer k fails, layers k..L-1 still get their events recorded and flags set, so
 * no consumer hangs, and the burst reports the error (its rows are stale); the
 * next burst is served normally.  A burst whose layer events are still held by an
 * earlier, not yet enqueued burst waits for that burst (event reuse backpressure).
 *
 * The device side goes through hc_loader_ops.  hc_loader_create with ops == NULL
 * binds the pool's own operations (hc_load_back_layer, hipStreamWaitEvent,
 * hipEventRecord, hipEventSynchronize on the pool's copy stream).  Other ops let
 * the ordering be observed without a GPU. */
typedef struct hc_loader hc_loader;
typedef struct hc_burst hc_burst;

typedef struct hc_loader_ops {
  void* ctx;
  /* enqueue one layer of a burst and record `event` after it; hc_status */
  int (*load_layer)(void* ctx, int32_t layer, const int64_t* host_idx, const int64_t* device_idx,
                    int64_t n, void* event);
  /* make the transfer stream wait for `event` (the burst's start event) */
  int (*wait_event)(void* ctx, void* event);
  /* record `event` on the transfer stream with no transfer before it (failure path) */
  int (*record_event)(void* ctx, void* event);
  /* block the calling thread until `event` has completed */
  int (*sync_event)(void* ctx, void* event);
  /* make `stream` wait for `event` */
  int (*stream_wait)(void* ctx, void* stream, void* event);
  /* enqueue one replay of a captured burst (hc_loader_submit_graph); may be NULL when
   * the loader never receives one */
  int (*launch_graph)(void* ctx, void* graph);
} hc_loader_ops;

/* async = 1: one worker thread; async = 0: hc_loader_submit runs the burst inline
 * on the caller's thread (same call sequence, no thread).  num_layers must equal
 * the pool's layer count when a pool is given.  ops may be NULL only with a pool. */
int hc_loader_create(hc_pool* pool, const hc_loader_ops* ops, int32_t num_layers, int32_t async,
                     hc_loader** out);
/* Queue one burst.  host_idx / device_idx / n are passed to load_layer unchanged
 * (device-resident lists for a pool); layer_events: num_layers caller-owned events,
 * all distinct; start_event: recorded by the producer at hand-over, or NULL.
 * Returns at once in async mode.  *out is released with hc_burst_release. */
int hc_loader_submit(hc_loader* loader, const int64_t* host_idx, const int64_t* device_idx, int64_t n,
                     void* const* layer_events, void* start_event, hc_burst** out);
/* Queue one replay of a captured load-back burst (hc_load_back_graph_create on the
 * loader's pool, or any graph the loader's launch_graph op accepts).  layer_events:
 * the num_layers events the graph was captured with, in layer order (the graph
 * records them; the loader needs them for its flags and for hc_burst_wait_layer).
 * The worker makes the transfer stream wait for start_event (if any), launches the
 * graph and flags every layer at once; on failure it records every layer event, as
 * hc_loader_submit does.  Bursts of both kinds share one FIFO and one event-reuse
 * rule.  HC_ERR_UNSUPPORTED when the loader's ops have no launch_graph.  A loader
 * created with the pool's own ops (ops NULL) checks at submit that the graph was
 * captured on its pool with exactly these events (so a graph captured with a NULL
 * layer event cannot be handed over) and refuses others with HC_ERR_INVALID. */
int hc_loader_submit_graph(hc_loader* loader, void* graph, void* const* layer_events, void* start_event,
                           hc_burst** out);
/* Block until layer `layer` of the burst is recorded, then make consumer_stream wait
 * on its event (consumer_stream NULL: block the calling thread until it completes). */
int hc_burst_wait_layer(hc_burst* burst, int32_t layer, void* consumer_stream);
/* Block until every layer is enqueued and the last layer's event has completed;
 * returns the burst's status (HC_OK or the error that stopped its enqueue). */
int hc_burst_wait(hc_burst* burst);
/* Non-blocking: layers enqueued so far and whether the burst is fully enqueued. */
int hc_burst_query(hc_burst* burst, int32_t* layers_enqueued, int32_t* enqueue_done);
/* Waits for the burst's enqueue to finish, then frees it. */
int hc_burst_release(hc_burst* burst);
/* Blocks until every submitted burst is enqueued. */
int hc_loader_drain(hc_loader* loader);
/* Number of bursts whose enqueue failed so far, and whether a worker thread runs. */
int hc_loader_info(hc_loader* loader, int64_t* failed_bursts, int32_t* worker_running);
/* Drains, joins the worker, frees.  NULL is a no-op.  Refused (HC_ERR_INVALID, nothing
 * freed) while a burst of the loader is not released.  Destroy a pool's loaders before
 * the pool. */
int hc_loader_destroy(hc_loader* loader);

/* ---------------------------------------------------------------- host-to-host shard copies
 * The storage side of the shard layout (CacheStore H2H page, unified-cache-management
 * PR 1292: Dump path, Load path, Queue backpressure, Failure handling,
 * page_first_kv_split support).  One page is one store shard: the page of every
 * tensor (sub-buffer) back to back, then zeros up to shard_bytes.  Each shard is one
 * job for a pool of CPU copy workers: one worker copies a shard's tensors in order,
 * different shards run concurrently.  Dump and load keep separate counts of
 * outstanding shards (queued + running); a request reserves capacity for all its
 * shards or is refused with HC_ERR_BUSY, never submitted in part.  A request with a
 * null address, a tensor-size mismatch or more shards than the queue depth (it could
 * never be admitted) is refused whole with HC_ERR_INVALID.
 * Every submitted job counts toward its request's completion.  The workers form an
 * unordered executor, not a FIFO stream: jobs (and requests) may finish in any
 * order, and a caller that needs ordering waits on the earlier request first. */
typedef struct hc_h2h hc_h2h;
typedef struct hc_h2h_request hc_h2h_request;
enum { HC_H2H_DUMP = 0, HC_H2H_LOAD = 1 };
#define HC_H2H_MAX_TENSORS 16

/* workers >= 1: that many copy threads; workers == 0: no threads, jobs run in the
 * thread that calls hc_h2h_wait (manual progress).  queue_depth: outstanding-shard
 * capacity per direction (>= 1). */
int hc_h2h_create(int32_t workers, int64_t queue_depth, hc_h2h** out);
/* Queue n shard jobs.  tensor_pages[i * tensors + t]: host address of tensor t's page
 * for shard i (tensor_bytes[t] contiguous bytes; in a page-first pool that is
 * hc_host_offset(sub t, page, 0, 0) from host_base).  shards[i]: the shard in the
 * store buffer, shard_bytes long, sum(tensor_bytes) <= shard_bytes.  Dump: shard <-
 * tensor pages, rest of the shard zeroed.  Load: tensor pages <- shard.  The arrays
 * are copied; the memory they point to must stay valid until hc_h2h_wait returns. */
int hc_h2h_submit(hc_h2h* h2h, int32_t direction, int32_t tensors, const int64_t* tensor_bytes,
                  void* const* tensor_pages, void* const* shards, int64_t shard_bytes, int64_t n,
                  hc_h2h_request** out);
/* Block until every job of the request has finished; returns the request's status. */
int hc_h2h_wait(hc_h2h_request* request);
/* Waits like hc_h2h_wait, then frees the request. */
int hc_h2h_release(hc_h2h_request* request);
int hc_h2h_outstanding(hc_h2h* h2h, int64_t* dump_shards, int64_t* load_shards);
/* Runs the remaining jobs, joins the workers, frees.  NULL is a no-op.  Refused
 * (HC_ERR_INVALID, nothing freed) while a request is not released. */
int hc_h2h_destroy(hc_h2h* h2h);

/* Cache identity (CacheStore H2H page, page_first_kv_split support: model, host layout,
 * page size, TP size and tensor sizes, so that incompatible layouts never share
 * cached data): 64-bit FNV-1a over the text
 *   "hicache-layout-v1;model=<model>;layout=<page_first|kv_split_shard|page_first_token_major>;
 *    layers=<L>;page_size=<P>;tp=<tp_size>;tensors=<g>:<bytes>,...;align=<shard_align or 0>"
 * (no spaces or line breaks; g is 'r' for token rows, 'b' for page blocks). */
int hc_cache_fingerprint(const hc_pool_desc* desc, const char* model, int32_t tp_size, uint64_t* out);

/* ---------------------------------------------------------------- measurement */

/* Running totals of a pool's transfer calls that were enqueued (refused calls are not
 * counted), for monitoring.  Bytes are the host-link bytes of the call: every named
 * token row of every layer moved, plus page blocks once per page. */
typedef struct hc_pool_stats {
  int64_t write_back_calls, write_back_tokens, write_back_bytes;
  int64_t load_back_calls, load_back_tokens, load_back_bytes;  /* one call = one layer */
  int64_t device_errors;  /* HC_ERR_DEVICE reports returned by hc_pool_sync */
} hc_pool_stats;
/* Copies the totals to *out (host memory); touches no GPU. */
int hc_pool_get_stats(hc_pool* pool, hc_pool_stats* out);

/* Per-kernel timing with HIP events on the copy stream (pools with HC_FLAG_PROFILE).
 * kind: 0 gather to staging, 1 zero-copy write-back, 2 zero-copy load-back,
 *       3 pad fill, 4 round-trip compare, 5 staged copy-engine transfers,
 *       6 layer pack, 7 layer unpack.
 * Returns the number of timed launches and their summed milliseconds since the
 * last reset (synchronizes the copy stream).  reset != 0 clears the counters. */
int hc_pool_kernel_time(hc_pool* pool, int32_t kind, int32_t reset, int64_t* launches,
                        double* total_ms);

const char* hc_last_error(void);
int hc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HC_H */
