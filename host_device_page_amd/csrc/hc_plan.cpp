// The write-back planner (see hc_plan.h).
#include "hc_plan.h"

#include <stdio.h>

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
                          int32_t* srow, int32_t* ztok, int64_t* nz, int64_t* pads, int64_t* npads) {
  const Layout& L = lay_;
  const int64_t C = chunk_pages;
  regions.clear();
  chunks.clear();
  slot_page_.assign((size_t)C, -1);
  slot_rows_.assign((size_t)C, 0);
  int64_t nslots = 0, t0 = 0;
  *nz = 0;
  *npads = 0;
  max_slots_ = 0;
  auto close_chunk = [&](int64_t t1) {
    if (nslots > max_slots_) max_slots_ = nslots;
    const size_t r0 = regions.size();
    chunk_first_region_ = r0;
    for (int64_t s = 0; s < nslots; s++) {
      const int64_t page = slot_page_[(size_t)s];
      if (slot_rows_[(size_t)s] == L.P) {
        const uint8_t* img = staging + s * L.stride;
        if (L.layout == HC_LAYOUT_KV_SPLIT_SHARD) {
          emit_region(host + page * L.stride, img, L.stride);
        } else {
          for (int b = 0; b < L.nsub; b++)
            emit_region(host + L.host_region[b] + page * L.subpage[b], img + L.img_off[b], L.subpage[b]);
        }
      } else if (L.layout == HC_LAYOUT_KV_SPLIT_SHARD && L.stride > L.payload) {
        pads[(*npads)++] = page;
      }
      page_slot_[(size_t)page] = -1;
    }
    for (int64_t i = t0; i < t1; i++) {
      const int32_t s = srow[i] / L.P;
      if (slot_rows_[(size_t)s] != L.P) {
        srow[i] = -1;
        ztok[(*nz)++] = (int32_t)i;
      }
    }
    chunks.push_back({t0, t1, r0, regions.size()});
    t0 = t1;
    nslots = 0;
  };
  for (int64_t i = 0; i < n; i++) {
    const int64_t page = h[i] / L.P;
    const int32_t r = (int32_t)(h[i] - page * L.P);
    int32_t s = page_slot_[(size_t)page];
    if (s < 0) {
      if (nslots == C) close_chunk(i);
      s = (int32_t)nslots++;
      page_slot_[(size_t)page] = s;
      slot_page_[(size_t)s] = page;
      slot_rows_[(size_t)s] = 0;
    }
    slot_rows_[(size_t)s]++;
    srow[i] = s * L.P + r;
  }
  close_chunk(n);
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
