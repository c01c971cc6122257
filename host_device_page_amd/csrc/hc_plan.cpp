// The write-back planner (see hc_plan.h).
#include "hc_plan.h"

#include <stdio.h>

#include <algorithm>

namespace hc {
namespace {

inline bool test_and_set(std::vector<uint64_t>& bits, int64_t k) {
  uint64_t& w = bits[(size_t)(k >> 6)];
  const uint64_t m = (uint64_t)1 << (k & 63);
  const bool was = (w & m) != 0;
  w |= m;
  return was;
}

inline void clear_bit(std::vector<uint64_t>& bits, int64_t k) { bits[(size_t)(k >> 6)] &= ~((uint64_t)1 << (k & 63)); }

}  // namespace

void Planner::reset(const Layout& lay) {
  lay_ = lay;
  page_slot_.assign((size_t)lay.H, -1);
  seen_.assign((size_t)((lay.H * lay.P + 63) / 64), 0);
  page_seen_.assign((size_t)((lay.H + 63) / 64), 0);
  page_rows_.assign((size_t)lay.H, 0);
}

int Planner::validate(const int64_t* h, int64_t n, char* msg, size_t msg_len) {
  const int64_t tokens = lay_.H * lay_.P;
  int64_t bad = -1;
  int64_t i = 0;
  for (; i < n; i++) {
    const int64_t x = h[i];
    if (x < 0 || x >= tokens || test_and_set(seen_, x)) {
      bad = i;
      break;
    }
  }
  for (int64_t j = 0; j < i; j++) clear_bit(seen_, h[j]);
  if (bad >= 0) {
    const int64_t x = h[bad];
    if (x < 0 || x >= tokens)
      snprintf(msg, msg_len, "host_idx[%lld] = %lld out of range [0, %lld)", (long long)bad, (long long)x,
               (long long)tokens);
    else
      snprintf(msg, msg_len, "host_idx[%lld] = %lld repeats an earlier entry", (long long)bad, (long long)x);
    return HC_ERR_INVALID;
  }
  if (lay_.has_blocks) {
    // every named page as P consecutive entries in row order (the kernels find a page's
    // block at the list position of its row 0, a multiple of P)
    for (int64_t j = 0; j < n; j++) {
      const bool ok = (j % lay_.P == 0) ? (h[j] % lay_.P == 0) : (h[j] == h[j - 1] + 1);
      if (!ok) {
        snprintf(msg, msg_len,
                 "host_idx[%lld] = %lld: with page-block sub-buffers the list names whole pages, each as %d "
                 "consecutive entries in row order",
                 (long long)j, (long long)h[j], lay_.P);
        return HC_ERR_INVALID;
      }
    }
    // every named page whole: count rows per page
    int rc = HC_OK;
    for (int64_t j = 0; j < n; j++) page_rows_[(size_t)(h[j] / lay_.P)]++;
    for (int64_t j = 0; j < n && rc == HC_OK; j++) {
      const int64_t page = h[j] / lay_.P;
      if (page_rows_[(size_t)page] != lay_.P) {
        snprintf(msg, msg_len, "page %lld is named partially; page-block sub-buffers need whole pages",
                 (long long)page);
        rc = HC_ERR_INVALID;
      }
    }
    for (int64_t j = 0; j < n; j++) page_rows_[(size_t)(h[j] / lay_.P)] = 0;
    return rc;
  }
  return HC_OK;
}

void Planner::emit_region(uint8_t* dst, const uint8_t* src, int64_t len) {
  // merge only inside the open chunk: a region of an earlier chunk is copied before
  // this chunk's gather fills its staging images
  if (regions.size() > chunk_first_region_) {
    Region& r = regions.back();
    if (r.dst + r.len == dst && r.src + r.len == src) {
      r.len += len;
      return;
    }
  }
  regions.push_back({dst, src, len});
}

void Planner::plan_staged(const int64_t* h, int64_t n, int64_t chunk_pages, uint8_t* host, const uint8_t* staging,
                          int32_t* perm, int32_t* srow, int32_t* ztok, int64_t* nz, int64_t* pads, int64_t* npads) {
  const Layout& L = lay_;
  const int64_t C = chunk_pages;
  regions.clear();
  chunks.clear();
  whole_.clear();
  *nz = 0;
  *npads = 0;
  max_slots_ = 0;
  // rows named per page; the wholly named pages, and the shard pages named in part
  for (int64_t i = 0; i < n; i++) page_rows_[(size_t)(h[i] / L.P)]++;
  const bool shard_pad = L.layout == HC_LAYOUT_KV_SPLIT_SHARD && L.stride > L.payload;
  for (int64_t i = 0; i < n; i++) {
    const int64_t page = h[i] / L.P;
    if (test_and_set(page_seen_, page)) continue;
    if (page_rows_[(size_t)page] == L.P) whole_.push_back(page);
    else if (shard_pad) pads[(*npads)++] = page;
  }
  std::sort(whole_.begin(), whole_.end());
  const int64_t nw = (int64_t)whole_.size();
  const int64_t nchunks = (nw + C - 1) / C;
  for (int64_t r = 0; r < nw; r++) page_slot_[(size_t)whole_[(size_t)r]] = (int32_t)r;
  // staged tokens per chunk, then their positions: chunk by chunk, list order inside
  chunk_fill_.assign((size_t)nchunks + 1, 0);
  for (int64_t i = 0; i < n; i++) {
    const int32_t rank = page_slot_[(size_t)(h[i] / L.P)];
    if (rank >= 0) chunk_fill_[(size_t)(rank / C) + 1]++;
  }
  for (int64_t c = 0; c < nchunks; c++) chunk_fill_[(size_t)c + 1] += chunk_fill_[(size_t)c];
  for (int64_t c = 0; c < nchunks; c++) chunks.push_back({chunk_fill_[(size_t)c], chunk_fill_[(size_t)c + 1], 0, 0});
  for (int64_t i = 0; i < n; i++) {
    const int64_t page = h[i] / L.P;
    const int32_t rank = page_slot_[(size_t)page];
    if (rank < 0) {
      ztok[(*nz)++] = (int32_t)i;
      continue;
    }
    const int64_t k = chunk_fill_[(size_t)(rank / C)]++;
    perm[k] = (int32_t)i;
    srow[k] = (int32_t)((rank % C) * L.P + (h[i] - page * L.P));
  }
  // the copy-engine regions of each chunk: slot s holds whole_[c * C + s]
  for (int64_t c = 0; c < nchunks; c++) {
    Chunk& ch = chunks[(size_t)c];
    ch.r0 = regions.size();
    chunk_first_region_ = ch.r0;
    const int64_t slots = std::min<int64_t>(C, nw - c * C);
    if (slots > max_slots_) max_slots_ = slots;
    if (L.layout == HC_LAYOUT_KV_SPLIT_SHARD) {
      for (int64_t s = 0; s < slots; s++) {
        const int64_t page = whole_[(size_t)(c * C + s)];
        emit_region(host + page * L.stride, staging + s * L.stride, L.stride);
      }
    } else {
      // sub-buffer-major staging: slot s of sub-buffer b is one sub-buffer page
      for (int b = 0; b < L.nsub; b++)
        for (int64_t s = 0; s < slots; s++) {
          const int64_t page = whole_[(size_t)(c * C + s)];
          emit_region(host + L.host_region[b] + page * L.subpage[b],
                      staging + staging_sub_base(L, b, C) + s * staging_slot_stride(L, b), L.subpage[b]);
        }
    }
    ch.r1 = regions.size();
  }
  // the per-page scratch back to its resting state
  for (int64_t i = 0; i < n; i++) {
    const int64_t page = h[i] / L.P;
    page_rows_[(size_t)page] = 0;
    page_slot_[(size_t)page] = -1;
    clear_bit(page_seen_, page);
  }
}

int64_t Planner::distinct_pages(const int64_t* h, int64_t n, int64_t* pages) {
  int64_t k = 0;
  for (int64_t i = 0; i < n; i++) {
    const int64_t page = h[i] / lay_.P;
    if (!test_and_set(page_seen_, page)) pages[k++] = page;
  }
  for (int64_t j = 0; j < k; j++) clear_bit(page_seen_, pages[j]);
  return k;
}

}  // namespace hc
