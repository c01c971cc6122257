// The write-back planner (hc_plan.cpp) on the CPU, under AddressSanitizer + UBSan.
// For random host-token lists on several layouts and chunk sizes, the plan is
// executed on host buffers by a model of the device side -- the gather fills each
// chunk's staging images, the region list is copied, split-page tokens are written
// row by row, listed shard pads are zeroed -- and the resulting host pool must hold
// exactly the named rows (and the named pages' blocks and pads) and nothing else.
// The structural rules are checked too: staged and split-page tokens cover the list
// once; a token goes through staging exactly when the list names its whole page;
// chunks partition the staged tokens, list order inside a chunk, at most chunk_pages
// pages each, pages ascending across slots and chunks; host pages adjacent in
// consecutive slots leave staging as one region.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "hc.h"
#include "hc_internal.h"
#include "hc_plan.h"

#define CHECK(cond)                                                                      \
  do {                                                                                   \
    if (!(cond)) {                                                                       \
      fprintf(stderr, "check failed at line %d (case %d): %s\n", __LINE__, g_case, #cond); \
      exit(1);                                                                           \
    }                                                                                    \
  } while (0)

static int g_case = 0;

static uint8_t truth(int64_t host_off) { return (uint8_t)((host_off * 2654435761u) >> 13 ^ 0x5a); }

struct Shape {
  int L, P, H, layout;
  std::vector<std::pair<int, int64_t>> subs;  // (granularity, elem bytes)
  int64_t align;
};

static hc::Layout layout_of(const Shape& sh) {
  hc_pool_desc d;
  memset(&d, 0, sizeof(d));
  d.num_layers = sh.L;
  d.page_size = sh.P;
  d.num_subbufs = (int32_t)sh.subs.size();
  d.layout = sh.layout;
  for (size_t b = 0; b < sh.subs.size(); b++) {
    d.sub[b].granularity = sh.subs[b].first;
    d.sub[b].elem_bytes = sh.subs[b].second;
  }
  d.device_slots = (int64_t)sh.H * sh.P;
  d.host_pages = sh.H;
  d.shard_align = sh.align;
  hc::Layout L;
  char msg[256];
  CHECK(hc::layout_from_desc(&d, &L, msg, sizeof(msg)) == HC_OK);
  return L;
}

// Writes the host bytes of token row (page, row) of every layer and sub-buffer (page
// blocks at row 0 only) from the truth function into `host`.
static void write_row(const hc::Layout& L, uint8_t* host, int64_t page, int row) {
  for (int b = 0; b < L.nsub; b++) {
    if (L.gran[b] == HC_PAGE_BLOCKS && row != 0) continue;
    for (int l = 0; l < L.L; l++) {
      const int64_t off = hc::layout_host_offset(L, b, page, l, L.gran[b] == HC_PAGE_BLOCKS ? 0 : row);
      for (int64_t k = 0; k < L.elem[b]; k++) host[off + k] = truth(off + k);
    }
  }
}

static void run_case(const Shape& sh, const std::vector<int64_t>& h, int64_t chunk_pages) {
  const hc::Layout L = layout_of(sh);
  hc::Planner pl;
  pl.reset(L);
  char msg[256];
  CHECK(pl.validate(h.data(), (int64_t)h.size(), msg, sizeof(msg)) == HC_OK);
  const int64_t n = (int64_t)h.size();
  const int64_t C = chunk_pages;
  std::vector<uint8_t> host((size_t)L.host_bytes, 0xAB), staging((size_t)(C * L.stride), 0);
  std::vector<int32_t> perm((size_t)std::max<int64_t>(n, 1)), srow((size_t)std::max<int64_t>(n, 1)),
      ztok((size_t)std::max<int64_t>(n, 1));
  std::vector<int64_t> pads((size_t)std::max<int64_t>(n, 1));
  int64_t nz = -1, npads = -1;
  pl.plan_staged(h.data(), n, C, host.data(), staging.data(), perm.data(), srow.data(), ztok.data(), &nz,
                 pads.data(), &npads);
  std::map<int64_t, int> rows;  // page -> rows the whole list names
  for (int64_t t : h) rows[t / L.P]++;
  const int64_t ns = n - nz;
  CHECK(nz >= 0 && ns >= 0);
  // staged tokens and split-page tokens: every list position exactly once
  std::vector<int> seen((size_t)std::max<int64_t>(n, 1), 0);
  for (int64_t k = 0; k < ns; k++) {
    CHECK(perm[(size_t)k] >= 0 && perm[(size_t)k] < n);
    CHECK(seen[(size_t)perm[(size_t)k]]++ == 0);
  }
  for (int64_t k = 0; k < nz; k++) {
    CHECK(ztok[(size_t)k] >= 0 && ztok[(size_t)k] < n);
    CHECK(seen[(size_t)ztok[(size_t)k]]++ == 0);
  }
  // split-page tokens: exactly those of pages the list names in part, in list order
  std::vector<int32_t> expect_z;
  std::set<int64_t> expect_pads;
  for (int64_t i = 0; i < n; i++) {
    const int64_t page = h[(size_t)i] / L.P;
    if (rows[page] != L.P) {
      expect_z.push_back((int32_t)i);
      if (L.layout == HC_LAYOUT_KV_SPLIT_SHARD && L.stride > L.payload) expect_pads.insert(page);
    }
  }
  CHECK(nz == (int64_t)expect_z.size());
  for (int64_t k = 0; k < nz; k++) CHECK(ztok[(size_t)k] == expect_z[(size_t)k]);
  // pads: each page named in part once
  std::set<int64_t> got_pads(pads.begin(), pads.begin() + npads);
  CHECK((int64_t)got_pads.size() == npads && got_pads == expect_pads);
  // chunks partition [0, ns) in order; regions likewise
  if (ns == 0) CHECK(pl.chunks.empty() && pl.regions.empty());
  if (ns > 0) {
    CHECK(pl.chunks.front().t0 == 0 && pl.chunks.back().t1 == ns);
    CHECK(pl.chunks.front().r0 == 0 && pl.chunks.back().r1 == pl.regions.size());
  }
  for (size_t c = 1; c < pl.chunks.size(); c++) {
    CHECK(pl.chunks[c].t0 == pl.chunks[c - 1].t1);
    CHECK(pl.chunks[c].r0 == pl.chunks[c - 1].r1);
  }
  int64_t prev_page = -1;
  for (const hc::Chunk& c : pl.chunks) {
    CHECK(c.t0 < c.t1 && c.r0 < c.r1);
    // model of the gather: each staged token's rows into its slot's page image
    std::map<int32_t, int64_t> slot_page;
    std::fill(staging.begin(), staging.end(), 0);
    for (int64_t k = c.t0; k < c.t1; k++) {
      if (k > c.t0) CHECK(perm[(size_t)k] > perm[(size_t)k - 1]);  // list order inside a chunk
      const int64_t i = perm[(size_t)k];
      const int64_t page = h[(size_t)i] / L.P;
      const int row = (int)(h[(size_t)i] % L.P);
      CHECK(rows[page] == L.P);
      CHECK(srow[(size_t)k] >= 0 && srow[(size_t)k] % L.P == row);
      const int32_t slot = srow[(size_t)k] / L.P;
      CHECK(slot < C);
      auto it = slot_page.find(slot);
      if (it == slot_page.end()) slot_page[slot] = page;
      else CHECK(it->second == page);
      for (int b = 0; b < L.nsub; b++) {
        if (L.gran[b] == HC_PAGE_BLOCKS && row != 0) continue;
        const int r = L.gran[b] == HC_PAGE_BLOCKS ? 0 : row;
        for (int l = 0; l < L.L; l++) {
          const int64_t src = hc::layout_host_offset(L, b, page, l, r);
          const int64_t img = hc::staging_sub_base(L, b, C) + (int64_t)slot * hc::staging_slot_stride(L, b) +
                              (int64_t)l * L.layer_stride[b] + (int64_t)r * L.row_stride[b];
          for (int64_t k2 = 0; k2 < L.elem[b]; k2++) staging[(size_t)(img + k2)] = truth(src + k2);
        }
      }
    }
    // slots 0..m-1, pages ascending with the slot, and above every earlier chunk's pages
    CHECK((int64_t)slot_page.size() <= C);
    int32_t expect_slot = 0;
    int64_t runs = 0;
    for (auto& kv : slot_page) {
      CHECK(kv.first == expect_slot++);
      CHECK(kv.second > prev_page);
      if (kv.second != prev_page + 1 || kv.first == 0) runs++;
      prev_page = kv.second;
    }
    // adjacent host pages in consecutive slots leave staging as one region: at most one
    // region per run of adjacent pages and sub-buffer, and no two consecutive regions that
    // could have been one copy
    const int64_t per_run = L.layout == HC_LAYOUT_KV_SPLIT_SHARD ? 1 : L.nsub;
    CHECK((int64_t)(c.r1 - c.r0) <= runs * per_run && (int64_t)(c.r1 - c.r0) >= runs);
    for (size_t r = c.r0 + 1; r < c.r1; r++) {
      const hc::Region& a = pl.regions[r - 1];
      const hc::Region& z = pl.regions[r];
      CHECK(!(a.dst + a.len == z.dst && a.src + a.len == z.src));
    }
    // the region list of this chunk, executed
    for (size_t r = c.r0; r < c.r1; r++) {
      const hc::Region& g = pl.regions[r];
      CHECK(g.len > 0);
      CHECK(g.src >= staging.data() && g.src + g.len <= staging.data() + staging.size());
      CHECK(g.dst >= host.data() && g.dst + g.len <= host.data() + host.size());
      memcpy(g.dst, g.src, (size_t)g.len);
    }
  }
  CHECK(pl.max_chunk_slots() <= C);
  for (int64_t k = 0; k < nz; k++) {
    const int64_t t = h[(size_t)ztok[(size_t)k]];
    write_row(L, host.data(), t / L.P, (int)(t % L.P));
  }
  for (int64_t k = 0; k < npads; k++)
    memset(host.data() + pads[(size_t)k] * L.stride + L.payload, 0, (size_t)(L.stride - L.payload));
  // the host pool now holds the named rows, pads of named shards, and nothing else
  std::vector<uint8_t> want((size_t)L.host_bytes, 0xAB);
  std::set<int64_t> named_pages;
  for (int64_t t : h) {
    write_row(L, want.data(), t / L.P, (int)(t % L.P));
    named_pages.insert(t / L.P);
  }
  if (L.layout == HC_LAYOUT_KV_SPLIT_SHARD)
    for (int64_t p : named_pages) memset(want.data() + p * L.stride + L.payload, 0, (size_t)(L.stride - L.payload));
  if (memcmp(host.data(), want.data(), want.size()) != 0) {
    for (size_t i = 0; i < want.size(); i++)
      if (host[i] != want[i]) {
        fprintf(stderr, "first differing host byte %zu (stride %lld payload %lld): got %d want %d\n", i,
                (long long)L.stride, (long long)L.payload, host[i], want[i]);
        break;
      }
  }
  CHECK(memcmp(host.data(), want.data(), want.size()) == 0);
  // distinct pages in first-use order
  std::vector<int64_t> dp((size_t)std::max<int64_t>(n, 1));
  const int64_t k = pl.distinct_pages(h.data(), n, dp.data());
  std::vector<int64_t> order;
  std::set<int64_t> seen_pages;
  for (int64_t t : h)
    if (seen_pages.insert(t / L.P).second) order.push_back(t / L.P);
  CHECK(k == (int64_t)order.size());
  for (int64_t i = 0; i < k; i++) CHECK(dp[(size_t)i] == order[(size_t)i]);
}

static std::vector<int64_t> random_list(std::mt19937& rng, const Shape& sh, bool whole_pages, bool interleave) {
  std::vector<int64_t> pages((size_t)sh.H);
  for (int i = 0; i < sh.H; i++) pages[(size_t)i] = i;
  std::shuffle(pages.begin(), pages.end(), rng);
  const int np = 1 + (int)(rng() % (unsigned)sh.H);
  std::vector<int64_t> h;
  for (int k = 0; k < np; k++) {
    const int64_t p = pages[(size_t)k];
    if (whole_pages || sh.P == 1 || rng() % 2) {
      for (int r = 0; r < sh.P; r++) h.push_back(p * sh.P + r);
    } else {
      std::vector<int> rows((size_t)sh.P);
      for (int r = 0; r < sh.P; r++) rows[(size_t)r] = r;
      std::shuffle(rows.begin(), rows.end(), rng);
      const int m = 1 + (int)(rng() % (unsigned)(sh.P - 1));
      for (int r = 0; r < m; r++) h.push_back(p * sh.P + rows[(size_t)r]);
    }
  }
  if (interleave) std::shuffle(h.begin(), h.end(), rng);
  return h;
}

static void validate_rejects() {
  Shape blocks{2, 4, 8, HC_LAYOUT_PAGE_FIRST, {{HC_TOKEN_ROWS, 32}, {HC_PAGE_BLOCKS, 48}}, 4096};
  hc::Planner pl;
  pl.reset(layout_of(blocks));
  char msg[256];
  std::vector<int64_t> h = {0, 1, 2, 3, 8, 9, 10, 11};
  CHECK(pl.validate(h.data(), (int64_t)h.size(), msg, sizeof(msg)) == HC_OK);
  h.back() = 32;  // out of range (8 pages x 4 rows)
  CHECK(pl.validate(h.data(), (int64_t)h.size(), msg, sizeof(msg)) == HC_ERR_INVALID && strstr(msg, "out of range"));
  h.back() = 9;  // repeat
  CHECK(pl.validate(h.data(), (int64_t)h.size(), msg, sizeof(msg)) == HC_ERR_INVALID && strstr(msg, "repeats"));
  h.pop_back();  // page 2 named in part
  CHECK(pl.validate(h.data(), (int64_t)h.size(), msg, sizeof(msg)) == HC_ERR_INVALID && strstr(msg, "partially"));
  h.push_back(11);  // and whole again: the scratch of the failed calls was cleared
  CHECK(pl.validate(h.data(), (int64_t)h.size(), msg, sizeof(msg)) == HC_OK);
  std::vector<int64_t> swapped = {0, 2, 1, 3, 8, 9, 10, 11};  // whole pages, rows out of order
  CHECK(pl.validate(swapped.data(), 8, msg, sizeof(msg)) == HC_ERR_INVALID && strstr(msg, "row order"));
  std::vector<int64_t> interleaved = {0, 1, 8, 9, 2, 3, 10, 11};  // whole pages, interleaved
  CHECK(pl.validate(interleaved.data(), 8, msg, sizeof(msg)) == HC_ERR_INVALID && strstr(msg, "row order"));
  std::vector<int64_t> neg = {-1};
  CHECK(pl.validate(neg.data(), 1, msg, sizeof(msg)) == HC_ERR_INVALID);
}

int main(int argc, char** argv) {
  // optional: random cases per (shape, chunk size); 40 by default
  const int trials = argc > 1 ? atoi(argv[1]) : 40;
  validate_rejects();
  const std::vector<Shape> shapes = {
      {3, 4, 24, HC_LAYOUT_PAGE_FIRST, {{HC_TOKEN_ROWS, 32}, {HC_TOKEN_ROWS, 16}}, 4096},
      {2, 8, 16, HC_LAYOUT_PAGE_FIRST_TOKEN_MAJOR, {{HC_TOKEN_ROWS, 48}, {HC_TOKEN_ROWS, 32}}, 4096},
      {3, 4, 20, HC_LAYOUT_KV_SPLIT_SHARD, {{HC_TOKEN_ROWS, 64}, {HC_TOKEN_ROWS, 16}}, 512},  // 960 B + 64 B pad
      {2, 4, 20, HC_LAYOUT_KV_SPLIT_SHARD, {{HC_TOKEN_ROWS, 64}, {HC_TOKEN_ROWS, 64}}, 256},  // no pad
      {2, 4, 16, HC_LAYOUT_PAGE_FIRST, {{HC_TOKEN_ROWS, 32}, {HC_PAGE_BLOCKS, 48}}, 4096},
      {2, 1, 32, HC_LAYOUT_PAGE_FIRST, {{HC_TOKEN_ROWS, 16}}, 4096},
  };
  std::mt19937 rng(11);
  int cases = 0;
  for (size_t s = 0; s < shapes.size(); s++) {
    const bool blocks = shapes[s].subs.back().first == HC_PAGE_BLOCKS;
    for (int64_t chunk : {1, 2, 3, 5, 64}) {
      for (int trial = 0; trial < trials; trial++) {
        g_case = (int)(s * 1000 + chunk * 100 + trial);
        const bool interleave = !blocks && trial % 3 == 2;
        run_case(shapes[s], random_list(rng, shapes[s], blocks || trial % 4 == 0, interleave), chunk);
        cases++;
      }
    }
    g_case = (int)s;
    run_case(shapes[s], {}, 3);  // empty list
  }
  printf("plan_host ok: %d cases\n", cases);
  return 0;
}
