// Host-side layout arithmetic and descriptor checks.  Pure C++: no HIP calls, so
// these entry points work (and are tested) on machines without a GPU.
//
// Layouts (see hc.h): page-first [page][layer][row][elem] per sub-buffer, regions
// back to back (page_first_direct on the loader-thread page, sglang PR 38472,
// Motivation); token-major page-first [page][row][layer][elem] (hybrid-pool
// write-back page, host-pool and CPU-mock excerpts); shard = one page of every
// sub-buffer followed by zero padding to the alignment (CacheStore H2H page,
// unified-cache-management PR 1292, section "page_first_kv_split support").
// Every row sits at region + page*page_stride + layer*layer_stride + row*row_stride.
#include <stdio.h>
#include <string.h>

#include "hc_internal.h"

namespace hc {
namespace {

const int64_t kMaxBytes = (int64_t)1 << 62;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > kMaxBytes / a) return false;
  *out = a * b;
  return true;
}

bool add_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0 || a > kMaxBytes - b) return false;
  *out = a + b;
  return true;
}

int fail(char* msg, size_t len, int code, const char* text) {
  if (msg && len) snprintf(msg, len, "%s", text);
  return code;
}

}  // namespace

int layout_from_desc(const hc_pool_desc* d, Layout* out, char* msg, size_t len) {
  if (!d || !out) return fail(msg, len, HC_ERR_INVALID, "null descriptor");
  if (d->num_layers < 1 || d->num_layers > HC_MAX_LAYERS)
    return fail(msg, len, HC_ERR_INVALID, "num_layers must be in [1, HC_MAX_LAYERS]");
  if (d->page_size < 1 || d->page_size > (1 << 20))
    return fail(msg, len, HC_ERR_INVALID, "page_size must be in [1, 2^20]");
  if (d->num_subbufs < 1 || d->num_subbufs > HC_MAX_SUBBUFS)
    return fail(msg, len, HC_ERR_INVALID, "num_subbufs must be in [1, HC_MAX_SUBBUFS]");
  if (d->layout != HC_LAYOUT_PAGE_FIRST && d->layout != HC_LAYOUT_KV_SPLIT_SHARD &&
      d->layout != HC_LAYOUT_PAGE_FIRST_TOKEN_MAJOR)
    return fail(msg, len, HC_ERR_INVALID, "unknown layout");
  if (d->device_slots < 1) return fail(msg, len, HC_ERR_INVALID, "device_slots must be >= 1");
  if (d->host_pages < 0) return fail(msg, len, HC_ERR_INVALID, "host_pages must be >= 0 (0: a device-only pool)");
  Layout L;
  L.L = d->num_layers;
  L.P = d->page_size;
  L.nsub = d->num_subbufs;
  L.layout = d->layout;
  L.S = d->device_slots;
  L.H = d->host_pages;
  for (int b = 0; b < L.nsub; b++) {
    const hc_subbuf_desc& s = d->sub[b];
    if (s.granularity != HC_TOKEN_ROWS && s.granularity != HC_PAGE_BLOCKS)
      return fail(msg, len, HC_ERR_INVALID, "sub-buffer granularity must be HC_TOKEN_ROWS or HC_PAGE_BLOCKS");
    if (s.reserved != 0) return fail(msg, len, HC_ERR_INVALID, "sub-buffer reserved field must be 0");
    if (s.elem_bytes <= 0) return fail(msg, len, HC_ERR_INVALID, "elem_bytes must be > 0");
    if (s.elem_bytes % 16 != 0)
      return fail(msg, len, HC_ERR_UNSUPPORTED, "elem_bytes must be a multiple of 16 (16-byte vectors)");
    if (s.elem_bytes > HC_MAX_ELEM_BYTES)
      return fail(msg, len, HC_ERR_UNSUPPORTED, "elem_bytes above HC_MAX_ELEM_BYTES");
    L.gran[b] = s.granularity;
    L.elem[b] = s.elem_bytes;
    if (s.granularity == HC_PAGE_BLOCKS) L.has_blocks = true;
  }
  if (L.has_blocks && L.S % L.P != 0)
    return fail(msg, len, HC_ERR_INVALID, "device_slots must be a multiple of page_size with page-block sub-buffers");
  for (int b = 0; b < L.nsub; b++) {
    int64_t layer_bytes;  // one device layer: the extent hc_pool_create checks against its allocation
    if (!mul_ok(L.S, L.elem[b], &layer_bytes)) return fail(msg, len, HC_ERR_INVALID, "device layer size overflows");
  }
  int64_t tokens;
  if (!mul_ok(L.H, L.P, &tokens)) return fail(msg, len, HC_ERR_INVALID, "host_pages * page_size overflows");
  // one page of each sub-buffer over all layers
  int64_t payload = 0;
  for (int b = 0; b < L.nsub; b++) {
    int64_t per_layer, sp;
    if (L.gran[b] == HC_TOKEN_ROWS) {
      if (!mul_ok(L.P, L.elem[b], &per_layer)) return fail(msg, len, HC_ERR_INVALID, "page bytes overflow");
    } else {
      per_layer = L.elem[b];
    }
    if (!mul_ok(per_layer, L.L, &sp)) return fail(msg, len, HC_ERR_INVALID, "page bytes overflow");
    L.subpage[b] = sp;
    if (L.gran[b] == HC_PAGE_BLOCKS) {
      L.layer_stride[b] = L.elem[b];  // [page][layer]
      L.row_stride[b] = 0;
    } else if (L.layout == HC_LAYOUT_PAGE_FIRST_TOKEN_MAJOR) {
      L.layer_stride[b] = L.elem[b];  // [page][row][layer]
      L.row_stride[b] = (int64_t)L.L * L.elem[b];
    } else {
      L.layer_stride[b] = per_layer;  // [page][layer][row]
      L.row_stride[b] = L.elem[b];
    }
    L.img_off[b] = payload;
    if (!add_ok(payload, sp, &payload)) return fail(msg, len, HC_ERR_INVALID, "page bytes overflow");
  }
  L.payload = payload;
  if (L.layout == HC_LAYOUT_KV_SPLIT_SHARD) {
    const int64_t a = d->shard_align;
    if (a < 16 || (a & (a - 1)) != 0)
      return fail(msg, len, HC_ERR_INVALID, "shard_align must be a power of two >= 16");
    L.align = a;
    int64_t up;
    if (!add_ok(payload, a - 1, &up)) return fail(msg, len, HC_ERR_INVALID, "shard size overflows");
    L.stride = up / a * a;
    for (int b = 0; b < L.nsub; b++) {
      L.host_region[b] = L.img_off[b];
      L.host_page_stride[b] = L.stride;
    }
    if (!mul_ok(L.H, L.stride, &L.host_bytes)) return fail(msg, len, HC_ERR_INVALID, "host pool size overflows");
  } else {
    L.align = 0;
    L.stride = payload;
    int64_t region = 0;
    for (int b = 0; b < L.nsub; b++) {
      int64_t rb;
      L.host_region[b] = region;
      L.host_page_stride[b] = L.subpage[b];
      if (!mul_ok(L.H, L.subpage[b], &rb) || !add_ok(region, rb, &region))
        return fail(msg, len, HC_ERR_INVALID, "host pool size overflows");
    }
    L.host_bytes = region;
  }
  *out = L;
  return HC_OK;
}

int64_t layout_host_offset(const Layout& L, int b, int64_t page, int32_t layer, int32_t row) {
  return L.host_region[b] + page * L.host_page_stride[b] + (int64_t)layer * L.layer_stride[b] +
         (int64_t)row * L.row_stride[b];
}

}  // namespace hc
