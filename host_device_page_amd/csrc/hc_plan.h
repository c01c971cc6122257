// The write-back planner: the host-side part of a write-back burst, run once per
// burst on the CPU (hybrid-pool write-back page, implementation breakdown: the host
// index list stays on the CPU).  Pure C++ with no HIP calls, so it is built and
// tested on the CPU on its own.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "hc_internal.h"

namespace hc {

// One copy-engine transfer of the staged write-back: staging image bytes to host bytes.
struct Region {
  uint8_t* dst;
  const uint8_t* src;
  int64_t len;
};

// One staging chunk: staged tokens [t0, t1) of the plan's perm / srow arrays, its
// transfers regions[r0, r1).
struct Chunk {
  int64_t t0, t1;
  size_t r0, r1;
};

class Planner {
 public:
  // Sizes the scratch for a layout (once per pool).
  void reset(const Layout& lay);

  // Range and distinctness of the host token list, and, with page-block
  // sub-buffers, that the list is whole pages, each as P consecutive entries in row
  // order.  HC_OK, or HC_ERR_INVALID with a message in msg.
  int validate(const int64_t* host_idx, int64_t n, char* msg, size_t msg_len);

  // Staged plan.  The pages the list names whole (all P rows, anywhere in the list) go
  // through staging: sorted by host page and cut into chunks of at most chunk_pages
  // staging slots, so that pages adjacent in the host pool sit in adjacent slots of one
  // chunk and leave staging as one copy-engine region.  Their tokens are listed chunk by
  // chunk, in list order inside a chunk: perm[k] is the list position of staged token k
  // and srow[k] = slot * P + row its row inside the chunk's staging images; chunk c
  // covers k in [chunks[c].t0, chunks[c].t1).  Tokens of pages the list names only in
  // part go, in list order, to ztok[0, *nz) for the zero-copy kernel (rows the list does
  // not name must keep their bytes), and in the shard layout those pages go to
  // pads[0, *npads) (their pad is cleared separately).  Fills regions/chunks: every
  // staged page leaves staging as one region per sub-buffer (page-first layouts) or one
  // region per shard, adjacent regions of a chunk merged.  host and staging are base
  // addresses for the regions.  perm, srow and ztok hold n entries, pads n.
  void plan_staged(const int64_t* host_idx, int64_t n, int64_t chunk_pages, uint8_t* host, const uint8_t* staging,
                   int32_t* perm, int32_t* srow, int32_t* ztok, int64_t* nz, int64_t* pads, int64_t* npads);

  // Distinct pages named by the list, in order of first use; returns the count.
  int64_t distinct_pages(const int64_t* host_idx, int64_t n, int64_t* pages);

  std::vector<Region> regions;
  std::vector<Chunk> chunks;
  // Staging slots the fullest chunk of the last staged plan uses.
  int64_t max_chunk_slots() const { return max_slots_; }

 private:
  void emit_region(uint8_t* dst, const uint8_t* src, int64_t len);

  Layout lay_;
  size_t chunk_first_region_ = 0;    // regions before this index belong to closed chunks
  int64_t max_slots_ = 0;
  std::vector<int32_t> page_slot_;   // [H] rank of a staged page among the burst's staged pages, -1 otherwise
  std::vector<uint64_t> seen_;       // bitmap over host tokens (distinctness)
  std::vector<uint64_t> page_seen_;  // bitmap over host pages
  std::vector<int32_t> page_rows_;   // [H] rows named per page
  std::vector<int64_t> whole_;       // the burst's wholly named pages, sorted
  std::vector<int64_t> chunk_fill_;  // per chunk: next staged-token position
};

}  // namespace hc
