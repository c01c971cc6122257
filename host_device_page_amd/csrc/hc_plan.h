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

// One staging chunk: tokens [t0, t1) of the list, its transfers regions[r0, r1).
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

  // Staged plan: the list in order, cut into chunks of at most chunk_pages staging
  // slots (one slot per distinct host page).  Writes, per token, srow[i] = slot * P +
  // row inside the chunk's staging images, or -1 for tokens of pages the list names
  // only in part; those tokens' list positions go to ztok[0, *nz) for the zero-copy
  // kernel.  Fills regions/chunks: every wholly named page leaves staging as one
  // region per sub-buffer (page-first layouts) or one region per shard, adjacent
  // regions merged.  Shard pages named in part go to pads[0, *npads) (their pad is
  // cleared separately).  host and staging are base addresses for the regions.
  void plan_staged(const int64_t* host_idx, int64_t n, int64_t chunk_pages, uint8_t* host, const uint8_t* staging,
                   int32_t* srow, int32_t* ztok, int64_t* nz, int64_t* pads, int64_t* npads);

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
  std::vector<int32_t> page_slot_;   // [H] staging slot of a page in the open chunk, -1 otherwise
  std::vector<uint64_t> seen_;       // bitmap over host tokens (distinctness)
  std::vector<uint64_t> page_seen_;  // bitmap over host pages
  std::vector<int32_t> page_rows_;   // [H] rows named per page (page-block check)
  std::vector<int64_t> slot_page_;
  std::vector<int32_t> slot_rows_;
};

}  // namespace hc
