/*
 * Oracle for the HiCache host<->device KV page transfer.  TEST INFRASTRUCTURE.
 *
 * Plain, slow, obviously correct CPU reference of what the transfer path
 * computes.  Only the test suite, __graft_entry__.smoke() and
 * the CPU-baseline leg of the benchmark may load, call or link this file.  The
 * product library never does, and this file shares no code with it.
 *
 * Sources (the pages, cited by title and section):
 *   [P1] "[HiCache] Run the host->device load-back enqueue on a loader thread
 *        (opt-in)" (sglang PR 38472): Motivation (per-layer load-back into
 *        device slots, page_first_direct host layout), Accuracy Tests (the
 *        change moves bytes, it must not alter them).
 *   [P2] "feat:add shard-level thread pool for parallel H2H transfers &&
 *        sglang integration" (unified-cache-management PR 1292), section
 *        "page_first_kv_split support": one page is one shard holding the
 *        K page, then the V page, then optional padding; with Direct I/O the
 *        shard size is a multiple of 4096 bytes.
 *   [P3] "[HiCache] Opt-in rank-sharded host tier for DSA under TP"
 *        (sglang PR 41984): Modifications (page_first_direct host pools for
 *        the MLA latent and the DSA indexer-K), Accuracy Tests (pages are
 *        restored bit-exactly), Modifications again for the per-layer
 *        exchange of a layer-owner sharded host tier: the owner of a layer
 *        gathers the rows it loaded into a staging buffer, broadcasts it, and
 *        every other rank scatters it into the same device slots (device slot
 *        allocation is replicated across the ranks).
 *   [P4] prhub summary of sglang PR 28434 (staged write-back JIT kernel for
 *        hybrid pools), key source excerpts: the CPU mock of the staged copy
 *        writes, for every layer, host[dst_index, layer] = device_layer[src_index]
 *        with int64 token indices; the host-pool excerpt sizes staging per
 *        token, per layer, per element.
 *
 * Readings taken where the pages leave a point open (all in the design notes):
 *   - Host page-first layout is [page][layer][row][element] per sub-buffer
 *     (the page_first_direct order of [P1]/[P3]); sub-buffer regions follow
 *     each other in one host allocation: region b starts after H pages of
 *     every earlier sub-buffer.
 *   - A sub-buffer is either TOKEN rows (E bytes per token per layer) or PAGE
 *     blocks (E bytes per page per layer, e.g. the DSA indexer page of 64
 *     fp8 keys followed by 64 fp32 scales).  A PAGE block moves with the
 *     token at row 0 of its page; the device block index is slot / P.
 *   - Token-major page-first ([P4] host-pool and CPU-mock excerpts: staging is
 *     (tokens, layers, elements) and the mock writes host[token, layer]): per
 *     sub-buffer the host rows are [page][row][layer][element], i.e. host token
 *     t = page * P + row holds all its layers back to back.  Page blocks keep
 *     [page][layer][element].
 *   - Shard layout ([P2]): shard p starts at p * stride; inside it the
 *     sub-buffers follow each other, each [layer][row][element]; stride is
 *     the summed sub-buffer page bytes rounded up to the alignment; the pad
 *     bytes of every shard the write-back touches are set to 0.
 *   - Indices are token-granular int64; host index h names page h / P,
 *     row h % P; device and host indices are each distinct and in range.
 *     Rows not named in the index list are left untouched.
 *   - Exchange staging bytes ([P3] leaves them open): sub-buffer after
 *     sub-buffer; inside sub-buffer b the rows of the listed device slots in
 *     list order, or for page blocks one block per page (the block of the
 *     slot at list positions 0, P, 2P, ...) in list order.  The list names
 *     whole device pages in row order when a sub-buffer holds page blocks.
 *
 * Payload bytes are opaque: nothing is interpreted as a number.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "hc_oracle.h"

/* Bytes one sub-buffer holds for one page over all layers. */
int64_t orc_sub_page_bytes(const orc_geom* g, int b) {
  if (g->gran[b] == ORC_PAGE_BLOCKS) return (int64_t)g->layers * g->bytes[b];
  return (int64_t)g->layers * g->page_size * g->bytes[b];
}

/* Payload bytes of one page over all sub-buffers (a shard without padding). */
int64_t orc_page_payload_bytes(const orc_geom* g) {
  int64_t s = 0;
  for (int b = 0; b < g->nsub; b++) s += orc_sub_page_bytes(g, b);
  return s;
}

/* [P2] page_first_kv_split: shard size rounded up to the Direct-I/O alignment. */
int64_t orc_shard_bytes(const orc_geom* g) {
  int64_t s = orc_page_payload_bytes(g);
  int64_t a = g->align;
  int64_t k = s / a;
  if (k * a < s) k = k + 1;
  return k * a;
}

int64_t orc_host_pool_bytes(const orc_geom* g) {
  if (g->layout == ORC_KV_SPLIT_SHARD) return g->host_pages * orc_shard_bytes(g);
  return g->host_pages * orc_page_payload_bytes(g);
}

/* Byte offset of (sub-buffer b, page p, layer l, row r) in the host pool.
 * For a PAGE sub-buffer the row is ignored: the block covers the page. */
int64_t orc_host_offset(const orc_geom* g, int b, int64_t p, int32_t l, int32_t r) {
  int64_t inner;
  if (g->gran[b] == ORC_PAGE_BLOCKS)
    inner = (int64_t)l * g->bytes[b];
  else if (g->layout == ORC_PAGE_FIRST_TOKEN_MAJOR)
    inner = ((int64_t)r * g->layers + l) * g->bytes[b];
  else
    inner = ((int64_t)l * g->page_size + r) * g->bytes[b];

  if (g->layout == ORC_KV_SPLIT_SHARD) {
    /* shard p, then the earlier sub-buffers' pages, then [layer][row] */
    int64_t before = 0;
    for (int c = 0; c < b; c++) before += orc_sub_page_bytes(g, c);
    return p * orc_shard_bytes(g) + before + inner;
  }
  /* region of sub-buffer b, then page p, then [layer][row] */
  int64_t region = 0;
  for (int c = 0; c < b; c++) region += g->host_pages * orc_sub_page_bytes(g, c);
  return region + p * orc_sub_page_bytes(g, b) + inner;
}

/* Byte offset of token slot s (or of the block holding it) in one device layer. */
int64_t orc_device_offset(const orc_geom* g, int b, int64_t s) {
  if (g->gran[b] == ORC_PAGE_BLOCKS) return (s / g->page_size) * g->bytes[b];
  return s * g->bytes[b];
}

static int has_page_blocks(const orc_geom* g) {
  for (int b = 0; b < g->nsub; b++)
    if (g->gran[b] == ORC_PAGE_BLOCKS) return 1;
  return 0;
}

int orc_check_geom(const orc_geom* g) {
  if (!g) return ORC_ERR_INVALID;
  if (g->layers <= 0 || g->page_size <= 0 || g->nsub <= 0 || g->nsub > ORC_MAX_SUB)
    return ORC_ERR_INVALID;
  if (g->host_pages <= 0 || g->device_slots <= 0) return ORC_ERR_INVALID;
  if (g->layout != ORC_PAGE_FIRST && g->layout != ORC_KV_SPLIT_SHARD && g->layout != ORC_PAGE_FIRST_TOKEN_MAJOR)
    return ORC_ERR_INVALID;
  if (g->layout == ORC_KV_SPLIT_SHARD && g->align <= 0) return ORC_ERR_INVALID;
  for (int b = 0; b < g->nsub; b++) {
    if (g->bytes[b] <= 0) return ORC_ERR_INVALID;
    if (g->gran[b] != ORC_TOKEN_ROWS && g->gran[b] != ORC_PAGE_BLOCKS) return ORC_ERR_INVALID;
  }
  if (has_page_blocks(g) && g->device_slots % g->page_size != 0) return ORC_ERR_INVALID;
  return ORC_OK;
}

/* Preconditions on an index list pair: every device index in [0, S), every
 * host index in [0, H*P), each list free of repeats.  With PAGE sub-buffers
 * every host page named is named whole (all P rows) and its rows map onto one
 * whole device page in order: the device slot of row r is d0 + r with d0 a
 * multiple of P. */
int orc_check_indices(const orc_geom* g, const int64_t* d, const int64_t* h, int64_t n) {
  if (orc_check_geom(g) != ORC_OK || n < 0) return ORC_ERR_INVALID;
  if (n > 0 && (!d || !h)) return ORC_ERR_INVALID;
  int64_t host_tokens = g->host_pages * g->page_size;
  unsigned char* seen_d = (unsigned char*)calloc((size_t)g->device_slots, 1);
  unsigned char* seen_h = (unsigned char*)calloc((size_t)host_tokens, 1);
  int rc = ORC_OK;
  if (!seen_d || !seen_h) rc = ORC_ERR_INVALID;
  for (int64_t i = 0; rc == ORC_OK && i < n; i++) {
    if (d[i] < 0 || d[i] >= g->device_slots || h[i] < 0 || h[i] >= host_tokens) {
      rc = ORC_ERR_INVALID;
      break;
    }
    if (seen_d[d[i]] || seen_h[h[i]]) {
      rc = ORC_ERR_INVALID;
      break;
    }
    seen_d[d[i]] = 1;
    seen_h[h[i]] = 1;
  }
  if (rc == ORC_OK && has_page_blocks(g)) {
    /* device slot of each named host token, -1 when not named */
    int64_t* dev_of = (int64_t*)malloc((size_t)host_tokens * sizeof(int64_t));
    if (!dev_of) rc = ORC_ERR_INVALID;
    for (int64_t t = 0; rc == ORC_OK && t < host_tokens; t++) dev_of[t] = -1;
    for (int64_t i = 0; rc == ORC_OK && i < n; i++) dev_of[h[i]] = d[i];
    for (int64_t i = 0; rc == ORC_OK && i < n; i++) {
      int64_t page = h[i] / g->page_size;
      int64_t first = dev_of[page * g->page_size];
      if (first < 0 || first % g->page_size != 0) { rc = ORC_ERR_INVALID; break; }
      for (int32_t r = 0; r < g->page_size; r++) {
        if (dev_of[page * g->page_size + r] != first + r) { rc = ORC_ERR_INVALID; break; }
      }
    }
    free(dev_of);
  }
  free(seen_d);
  free(seen_h);
  return rc;
}

/* Write-back, all layers ([P4] staged write-back semantics, [P2] shard padding).
 * dev[b * L + l] is the base of layer l of sub-buffer b.  For every token i,
 * every sub-buffer and every layer, the device row (or the page block at row 0)
 * is copied to its host position.  In the shard layout the padding bytes of
 * every shard named by the list are then set to zero. */
int orc_write_back(const orc_geom* g, uint8_t* const* dev, uint8_t* host,
                   const int64_t* d, const int64_t* h, int64_t n) {
  if (orc_check_indices(g, d, h, n) != ORC_OK || !dev || !host) return ORC_ERR_INVALID;
  const int L = g->layers, P = g->page_size;
  for (int64_t i = 0; i < n; i++) {
    int64_t page = h[i] / P;
    int32_t row = (int32_t)(h[i] % P);
    for (int b = 0; b < g->nsub; b++) {
      if (g->gran[b] == ORC_PAGE_BLOCKS && row != 0) continue;
      for (int l = 0; l < L; l++) {
        const uint8_t* src = dev[b * L + l] + orc_device_offset(g, b, d[i]);
        uint8_t* dst = host + orc_host_offset(g, b, page, l, row);
        memcpy(dst, src, (size_t)g->bytes[b]);
      }
    }
  }
  if (g->layout == ORC_KV_SPLIT_SHARD) {
    int64_t payload = orc_page_payload_bytes(g);
    int64_t stride = orc_shard_bytes(g);
    for (int64_t i = 0; i < n; i++) {
      int64_t page = h[i] / P;
      memset(host + page * stride + payload, 0, (size_t)(stride - payload));
    }
  }
  return ORC_OK;
}

/* Load-back of one layer ([P1] per-layer load-back): for every token i and
 * every sub-buffer, the host row (or page block at row 0) of layer l is
 * copied to device slot d[i] of layer l.  Nothing else changes. */
int orc_load_back_layer(const orc_geom* g, int32_t layer, uint8_t* const* dev,
                        const uint8_t* host, const int64_t* h, const int64_t* d, int64_t n) {
  if (orc_check_indices(g, d, h, n) != ORC_OK || !dev || !host) return ORC_ERR_INVALID;
  if (layer < 0 || layer >= g->layers) return ORC_ERR_INVALID;
  const int L = g->layers, P = g->page_size;
  for (int64_t i = 0; i < n; i++) {
    int64_t page = h[i] / P;
    int32_t row = (int32_t)(h[i] % P);
    for (int b = 0; b < g->nsub; b++) {
      if (g->gran[b] == ORC_PAGE_BLOCKS && row != 0) continue;
      const uint8_t* src = host + orc_host_offset(g, b, page, layer, row);
      uint8_t* dst = dev[b * L + layer] + orc_device_offset(g, b, d[i]);
      memcpy(dst, src, (size_t)g->bytes[b]);
    }
  }
  return ORC_OK;
}

/* Round-trip check: number of (token, sub-buffer, layer) units whose device
 * row at slot a[i] differs from the row at slot c[i].  A PAGE sub-buffer is
 * compared once per page, at the tokens with a[i] % P == 0, block a[i]/P
 * against block c[i]/P.  Returns the count, or -1 on bad arguments. */
int64_t orc_round_trip_check(const orc_geom* g, uint8_t* const* dev,
                             const int64_t* a, const int64_t* c, int64_t n) {
  if (orc_check_geom(g) != ORC_OK || !dev || n < 0) return -1;
  if (n > 0 && (!a || !c)) return -1;
  const int L = g->layers, P = g->page_size;
  int64_t bad = 0;
  for (int64_t i = 0; i < n; i++) {
    if (a[i] < 0 || a[i] >= g->device_slots || c[i] < 0 || c[i] >= g->device_slots) return -1;
    for (int b = 0; b < g->nsub; b++) {
      if (g->gran[b] == ORC_PAGE_BLOCKS && a[i] % P != 0) continue;
      for (int l = 0; l < L; l++) {
        const uint8_t* x = dev[b * L + l] + orc_device_offset(g, b, a[i]);
        const uint8_t* y = dev[b * L + l] + orc_device_offset(g, b, c[i]);
        if (memcmp(x, y, (size_t)g->bytes[b]) != 0) bad++;
      }
    }
  }
  return bad;
}

/* Host offsets of the rows named by h for one sub-buffer and layer:
 * out[i] = orc_host_offset(g, b, h[i] / P, layer, h[i] % P).  A plain loop, used
 * by the tests to locate rows of large pools without one call per row. */
int orc_host_offsets(const orc_geom* g, int b, int32_t layer, const int64_t* h, int64_t n, int64_t* out) {
  if (orc_check_geom(g) != ORC_OK || b < 0 || b >= g->nsub || layer < 0 || layer >= g->layers) return ORC_ERR_INVALID;
  if (n < 0 || (n > 0 && (!h || !out))) return ORC_ERR_INVALID;
  for (int64_t i = 0; i < n; i++) {
    if (h[i] < 0 || h[i] >= g->host_pages * g->page_size) return ORC_ERR_INVALID;
    out[i] = orc_host_offset(g, b, h[i] / g->page_size, layer, (int32_t)(h[i] % g->page_size));
  }
  return ORC_OK;
}

/* Host-to-host shard copy (CacheStore H2H page, Dump path / Load path and
 * "page_first_kv_split support"): one host page of a page-first pool is one store
 * shard laid out like the shard layout (sub-buffer pages back to back, then zero
 * pad).  Dump copies page src_pages[i] of the page-first pool `pf` into shard
 * dst_shards[i] of the shard pool `sh`, row by row, and zeroes the shard's pad;
 * load copies the rows back.  The two geometries must agree on everything but the
 * layout and the page count. */
static int same_rows(const orc_geom* pf, const orc_geom* sh) {
  if (orc_check_geom(pf) != ORC_OK || orc_check_geom(sh) != ORC_OK) return 0;
  if (pf->layout != ORC_PAGE_FIRST || sh->layout != ORC_KV_SPLIT_SHARD) return 0;
  if (pf->layers != sh->layers || pf->page_size != sh->page_size || pf->nsub != sh->nsub) return 0;
  for (int b = 0; b < pf->nsub; b++)
    if (pf->gran[b] != sh->gran[b] || pf->bytes[b] != sh->bytes[b]) return 0;
  return 1;
}

int orc_h2h_dump(const orc_geom* pf, const orc_geom* sh, const uint8_t* host, uint8_t* store,
                 const int64_t* src_pages, const int64_t* dst_shards, int64_t n) {
  if (!same_rows(pf, sh) || n < 0 || !host || !store) return ORC_ERR_INVALID;
  int64_t payload = orc_page_payload_bytes(sh), stride = orc_shard_bytes(sh);
  for (int64_t i = 0; i < n; i++) {
    if (src_pages[i] < 0 || src_pages[i] >= pf->host_pages || dst_shards[i] < 0 || dst_shards[i] >= sh->host_pages)
      return ORC_ERR_INVALID;
    for (int b = 0; b < pf->nsub; b++) {
      int32_t rows = pf->gran[b] == ORC_PAGE_BLOCKS ? 1 : pf->page_size;
      for (int32_t l = 0; l < pf->layers; l++)
        for (int32_t r = 0; r < rows; r++)
          memcpy(store + orc_host_offset(sh, b, dst_shards[i], l, r), host + orc_host_offset(pf, b, src_pages[i], l, r),
                 (size_t)pf->bytes[b]);
    }
    memset(store + dst_shards[i] * stride + payload, 0, (size_t)(stride - payload));
  }
  return ORC_OK;
}

int orc_h2h_load(const orc_geom* pf, const orc_geom* sh, uint8_t* host, const uint8_t* store,
                 const int64_t* src_shards, const int64_t* dst_pages, int64_t n) {
  if (!same_rows(pf, sh) || n < 0 || !host || !store) return ORC_ERR_INVALID;
  for (int64_t i = 0; i < n; i++) {
    if (dst_pages[i] < 0 || dst_pages[i] >= pf->host_pages || src_shards[i] < 0 || src_shards[i] >= sh->host_pages)
      return ORC_ERR_INVALID;
    for (int b = 0; b < pf->nsub; b++) {
      int32_t rows = pf->gran[b] == ORC_PAGE_BLOCKS ? 1 : pf->page_size;
      for (int32_t l = 0; l < pf->layers; l++)
        for (int32_t r = 0; r < rows; r++)
          memcpy(host + orc_host_offset(pf, b, dst_pages[i], l, r), store + orc_host_offset(sh, b, src_shards[i], l, r),
                 (size_t)pf->bytes[b]);
    }
  }
  return ORC_OK;
}

/* ---------------------------------------------------------------- layer exchange
 * [P3] Modifications (load-back of a rank-sharded tier): the owner of a layer
 * gathers the rows it loaded into a staging buffer; the other ranks scatter that
 * buffer into the same device slots.  The staging byte order is the reading
 * stated at the top of this file.  The list d holds n distinct device slots in
 * [0, S); with page blocks n is a multiple of P and positions kP..kP+P-1 hold
 * the slots d0..d0+P-1 of one whole device page (d0 % P == 0). */
static int check_exchange_list(const orc_geom* g, const int64_t* d, int64_t n) {
  if (orc_check_geom(g) != ORC_OK || n < 0 || (n > 0 && !d)) return ORC_ERR_INVALID;
  const int64_t P = g->page_size;
  unsigned char* seen = (unsigned char*)calloc((size_t)g->device_slots, 1);
  if (!seen) return ORC_ERR_INVALID;
  int rc = ORC_OK;
  for (int64_t i = 0; i < n; i++) {
    if (d[i] < 0 || d[i] >= g->device_slots || seen[d[i]]) { rc = ORC_ERR_INVALID; break; }
    seen[d[i]] = 1;
  }
  free(seen);
  if (rc == ORC_OK && has_page_blocks(g)) {
    if (n % P != 0) return ORC_ERR_INVALID;
    for (int64_t k = 0; k < n; k += P) {
      if (d[k] % P != 0) return ORC_ERR_INVALID;
      for (int64_t r = 1; r < P; r++)
        if (d[k + r] != d[k] + r) return ORC_ERR_INVALID;
    }
  }
  return rc;
}

/* Bytes of one layer's staging for n list entries, or -1 on bad arguments:
 * every token row once, every page block once per page. */
int64_t orc_layer_packed_bytes(const orc_geom* g, int64_t n) {
  if (orc_check_geom(g) != ORC_OK || n < 0) return -1;
  int64_t total = 0;
  for (int b = 0; b < g->nsub; b++) {
    if (g->gran[b] == ORC_PAGE_BLOCKS) {
      if (n % g->page_size != 0) return -1;
      total += (n / g->page_size) * g->bytes[b];
    } else {
      total += n * g->bytes[b];
    }
  }
  return total;
}

/* Owner side: out <- the rows of layer `layer` at the listed slots, in staging order. */
int orc_layer_pack(const orc_geom* g, int32_t layer, uint8_t* const* dev, const int64_t* d, int64_t n, uint8_t* out) {
  if (check_exchange_list(g, d, n) != ORC_OK || !dev || (n > 0 && !out)) return ORC_ERR_INVALID;
  if (layer < 0 || layer >= g->layers) return ORC_ERR_INVALID;
  const int L = g->layers;
  uint8_t* at = out;
  for (int b = 0; b < g->nsub; b++) {
    const int64_t step = g->gran[b] == ORC_PAGE_BLOCKS ? g->page_size : 1;
    for (int64_t i = 0; i < n; i += step) {
      memcpy(at, dev[b * L + layer] + orc_device_offset(g, b, d[i]), (size_t)g->bytes[b]);
      at += g->bytes[b];
    }
  }
  return ORC_OK;
}

/* Receiving side: the rows of layer `layer` at the listed slots <- in, read in
 * staging order.  Nothing else changes. */
int orc_layer_unpack(const orc_geom* g, int32_t layer, uint8_t* const* dev, const int64_t* d, int64_t n,
                     const uint8_t* in) {
  if (check_exchange_list(g, d, n) != ORC_OK || !dev || (n > 0 && !in)) return ORC_ERR_INVALID;
  if (layer < 0 || layer >= g->layers) return ORC_ERR_INVALID;
  const int L = g->layers;
  const uint8_t* at = in;
  for (int b = 0; b < g->nsub; b++) {
    const int64_t step = g->gran[b] == ORC_PAGE_BLOCKS ? g->page_size : 1;
    for (int64_t i = 0; i < n; i += step) {
      memcpy(dev[b * L + layer] + orc_device_offset(g, b, d[i]), at, (size_t)g->bytes[b]);
      at += g->bytes[b];
    }
  }
  return ORC_OK;
}
