// Internal declarations shared by the host-side API (hc_api.cpp) and the kernels
// (hc_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "hc.h"

namespace hc {

// Geometry of one sub-buffer as the kernels see it.  Every byte offset is int64.
struct SubGeom {
  const uint64_t* layers;  // device array [L] of layer base addresses
  int64_t elem;            // bytes per token row / page block
  uint32_t vecs;           // elem / 16
  int32_t gran;            // HC_TOKEN_ROWS or HC_PAGE_BLOCKS
  uint64_t vec_magic;      // ceil(2^40 / vecs): q = (u * magic) >> 40 == u / vecs for u < 2^20
  int64_t host_region;     // page-first: start of this sub-buffer's region; shard: offset inside a shard
  int64_t host_page_stride;// bytes from page p to page p+1 of this sub-buffer in the host pool
  int64_t layer_stride;    // bytes from layer l to l+1 inside one page
  int64_t row_stride;      // bytes from row r to r+1 inside one page and layer (0 for page blocks)
  int64_t img_off;         // staging: offset of this sub-buffer's slot-0 page image in a chunk
  int64_t stg_slot;        // staging: bytes from slot s to slot s+1 of this sub-buffer
};

struct Geom {
  SubGeom sub[HC_MAX_SUBBUFS];
  int32_t nsub;
  int32_t L;
  int32_t P;
  int32_t validate;        // HC_FLAG_VALIDATE: page-block rows checked to form whole device pages
  int64_t S;               // device token slots per layer
  int64_t host_tokens;     // H * P
  int64_t img_bytes;       // one staging page image (shard stride or summed sub pages)
  int64_t payload_bytes;   // summed sub-buffer pages
  int64_t pad_bytes;       // shard padding (0 for page-first)
};

// Host-side derived layout (pure arithmetic; no HIP calls).
struct Layout {
  int32_t L = 0, P = 0, nsub = 0, layout = 0;
  int32_t gran[HC_MAX_SUBBUFS] = {};
  int64_t elem[HC_MAX_SUBBUFS] = {};
  int64_t S = 0, H = 0, align = 0;
  int64_t subpage[HC_MAX_SUBBUFS] = {};   // one page of sub b over all layers
  int64_t payload = 0;                    // sum of subpage
  int64_t stride = 0;                     // shard stride / page image bytes
  int64_t host_region[HC_MAX_SUBBUFS] = {};
  int64_t host_page_stride[HC_MAX_SUBBUFS] = {};
  int64_t layer_stride[HC_MAX_SUBBUFS] = {};
  int64_t row_stride[HC_MAX_SUBBUFS] = {};
  int64_t img_off[HC_MAX_SUBBUFS] = {};
  int64_t host_bytes = 0;
  bool has_blocks = false;
};

// Fills *out from desc; on failure returns a negative hc_status and writes a message.
int layout_from_desc(const hc_pool_desc* desc, Layout* out, char* msg, size_t msg_len);

// Staging layout of one chunk of C page images.  Shard layout: whole shards back to back,
// so a shard leaves staging as one region with its zero pad.  Page-first layouts:
// sub-buffer-major, [sub-buffer][slot][one sub-buffer page], so the pages of one
// sub-buffer in consecutive slots form one contiguous range, which leaves staging as one
// region when their host pages are adjacent too.  Either way a chunk takes C * stride bytes.
inline int64_t staging_sub_base(const Layout& L, int b, int64_t C) {
  return L.layout == HC_LAYOUT_KV_SPLIT_SHARD ? L.img_off[b] : C * L.img_off[b];
}
inline int64_t staging_slot_stride(const Layout& L, int b) {
  return L.layout == HC_LAYOUT_KV_SPLIT_SHARD ? L.stride : L.subpage[b];
}
int64_t layout_host_offset(const Layout& lay, int b, int64_t page, int32_t layer, int32_t row);

// Thread-local error message of the C ABI (hc_last_error); returns `code`.
int set_error(int code, const char* fmt, ...);
// The pool's own device operations for an hc_loader, and its layer count.
void pool_loader_ops(hc_pool* pool, hc_loader_ops* ops);
int pool_layers(const hc_pool* pool);
bool pool_has_host(const hc_pool* pool);  // false for a device-only pool (no host pages)
// Loaders and captured graphs that hold a pool: hc_pool_destroy refuses while any do.
void pool_hold(hc_pool* pool);
void pool_release(hc_pool* pool);
// HC_OK when `graph` (an hc_lb_graph) was captured on `pool` and records exactly
// `events` (L entries, in layer order); else HC_ERR_INVALID with a message.
int graph_matches(const hc_pool* pool, const void* graph, void* const* events, int32_t L);

// Optional timing of one kernel launch: two timing events that the launch itself
// stamps with the kernel's start and end (hipExtLaunchKernel), so timing adds no
// marker packets to the stream.  Both null: untimed.
struct LaunchTimer {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Kernel launchers (hc_kernels.hip).  All enqueue on `stream` and return the launch status.
// Gather of staged tokens [t0, t0 + count) of a write-back plan: perm[k] is the list
// position of staged token k, srow[k] its row inside the chunk's staging images.
hipError_t launch_gather_stage(const Geom& g, const int64_t* dev_idx, const int64_t* host_idx,
                               const int32_t* perm, const int32_t* srow, int64_t t0, int64_t count,
                               uint8_t* staging, int32_t* err, int32_t num_cus, const LaunchTimer& t,
                               hipStream_t stream);
// The zero-copy launchers size their tiles on the host; wg_load is host scratch of at
// least max_ctas entries for that (the caller's, so a launch allocates nothing).
hipError_t launch_zc_write(const Geom& g, const int64_t* dev_idx, const int64_t* host_idx,
                           const int32_t* tok_list, int64_t count, uint8_t* host, int32_t* err,
                           int32_t max_ctas, int64_t* wg_load, const LaunchTimer& t, hipStream_t stream);
hipError_t launch_zc_read(const Geom& g, int32_t layer, const int64_t* host_idx, const int64_t* dev_idx,
                          int64_t n, const uint8_t* host, int32_t* err, int32_t max_ctas, int64_t* wg_load,
                          const LaunchTimer& t, hipStream_t stream);
hipError_t launch_zero_pads(uint8_t* base, const int64_t* pages, int64_t npages, int64_t stride,
                            int64_t off, int64_t bytes, const LaunchTimer& t, hipStream_t stream);
// Layer exchange of a layer-owner sharded tier (hc_exchange.hip): per sub-buffer the
// positions it moves (n token rows, or n / P page blocks), its offset in the staging
// buffer, its positions per unit and the running unit count.
struct XPlan {
  int64_t positions[HC_MAX_SUBBUFS];
  int64_t seg[HC_MAX_SUBBUFS];
  int64_t units_end[HC_MAX_SUBBUFS];
  int32_t tile[HC_MAX_SUBBUFS];
};
// Fills *x for n list entries; returns the staging bytes of one layer.
int64_t exchange_plan(const Geom& g, int64_t n, int32_t num_cus, XPlan* x);
// pack: staging <- rows of `layer` at dev_idx; else the rows <- staging.
hipError_t launch_layer_exchange(const Geom& g, bool pack, int32_t layer, const int64_t* dev_idx, int64_t n,
                                 uint8_t* staging, int32_t* err, int32_t num_cus, const LaunchTimer& t,
                                 hipStream_t stream);
// Shard pads of the pages a host token list names, found from the list itself: the
// position that starts each run of same-page entries zeroes [off, off + bytes) of its
// page (a page named in two runs is zeroed twice).  Tokens outside [0, host_pages * P)
// are skipped (the transfer kernel reports them).
hipError_t launch_zero_pads_runs(uint8_t* base, const int64_t* host_idx, int64_t n, int32_t P, int64_t host_pages,
                                 int64_t stride, int64_t off, int64_t bytes, hipStream_t stream);
// Device address of the no-allocation write-back's scratch on `device` (which must be
// current), HC_NOALLOC_MAX_TOKENS int64 entries; looked up once per device (hc_noalloc.hip).
int noalloc_scratch(int device, int64_t** out);
hipError_t launch_compare(const Geom& g, const int64_t* a, const int64_t* c, int64_t n,
                          unsigned long long* counter, int32_t* err, const LaunchTimer& t,
                          hipStream_t stream);

}  // namespace hc
