// HIP kernels of the KV page transfer, written for CDNA4 (gfx950, wave64).
//
// Every kernel moves opaque 16-byte vectors: rows of a layer-first device pool
// to/from a page-first host pool (directly over the host link, "zero-copy") or
// to a device staging buffer laid out as host page images (staged write-back:
// the layer-first -> page-first relayout of the hybrid-pool write-back page,
// sglang PR 28434 summary, implementation breakdown).
//
// Work is cut into units of (tile of 256 tokens, layer, sub-buffer).  A unit
// starts with an index intake: each of the 256 threads reads one token's
// device and host index, range-checks it, and computes the byte addresses of
// its source and destination row.  Rows that move are compacted into LDS with
// a wavefront ballot and a mbcnt prefix (page blocks keep only the row-0 token
// of each page; the staged write-back skips tokens of partial pages).  The copy
// loop then walks the unit's rows * (elem/16) vectors with all 256 lanes: lane
// u copies vector u % vecs of row u / vecs, so consecutive lanes touch
// consecutive 16-byte vectors of a row, and a run of slots that are adjacent
// on both sides is one contiguous stream of addresses.  Loads are issued in
// batches before their stores to keep enough bytes in flight (depth per kernel
// below).
//
// The zero-copy kernels shrink the tile to kTile >> tile_shift tokens for a
// small burst, so that it still spreads over enough workgroups to keep the host
// link busy (one workgroup alone reads only ~7 GB/s over it); the launcher picks
// the shift whose busiest workgroup carries the fewest bytes.  Each unit still
// moves whole rows, so a run of adjacent rows stays one contiguous stream on the
// link.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hc_internal.h"

namespace hc {
namespace {

// Build-time tuning knobs (hipcc -D...): loads in flight per thread, and whether
// row loads / stores carry the non-temporal hint (streamed data is not reused).
#ifndef HC_UNROLL
#define HC_UNROLL 8
#endif
// Non-temporal loads: every row is read once.  Measured on the Llama-3-8B burst, two
// rounds: the staged gather 6.19-6.22 TB/s against 5.91-5.92 without, the zero-copy
// write-back 56.5-56.6 GB/s against 55.7, the load-back unchanged.  Non-temporal stores
// cost the gather a sixth (4.9-5.1 TB/s): its staging images should stay in the Infinity
// Cache for the copy engines that read them next.
#ifndef HC_NT_LOAD
#define HC_NT_LOAD 1
#endif
#ifndef HC_NT_STORE
#define HC_NT_STORE 0
#endif
#ifndef HC_TILE
#define HC_TILE 256
#endif

constexpr int kThreads = 256;  // 4 waves of 64
// The load-back kernel reads over the host link: software-pipelined batches of 4
// (measured faster there; the HBM-bound kernels keep plain batches of kUnroll).
#ifndef HC_READ_PIPELINED
#define HC_READ_PIPELINED 1
#endif
#ifndef HC_READ_UNROLL
#define HC_READ_UNROLL 4
#endif
constexpr bool kReadPipelined = HC_READ_PIPELINED != 0;
constexpr int kReadUnroll = HC_READ_UNROLL;
// The write-back kernel reads HBM and writes over the host link, on a small grid: plain
// batches 16 deep (measured 38.46 ms per 2 GiB burst against 38.60 at 8, flat from 16 to
// 32; the pipelined loop is slower here, 39.1-40.2 ms).
#ifndef HC_WRITE_PIPELINED
#define HC_WRITE_PIPELINED 0
#endif
#ifndef HC_WRITE_UNROLL
#define HC_WRITE_UNROLL 16
#endif
constexpr bool kWritePipelined = HC_WRITE_PIPELINED != 0;
constexpr int kWriteUnroll = HC_WRITE_UNROLL;
constexpr int kTile = HC_TILE; // tokens per unit (<= kThreads): one per thread at intake
static_assert(kTile <= kThreads && kTile % 64 == 0, "tile must be whole waves of one block");
#ifndef HC_GATHER_TILE
#define HC_GATHER_TILE 128
#endif
#ifndef HC_GATHER_BLOCKS_PER_CU
#define HC_GATHER_BLOCKS_PER_CU 4
#endif
constexpr int kGatherTile = HC_GATHER_TILE;  // tokens per gather unit
static_assert(kGatherTile <= kThreads && kGatherTile % 64 == 0, "gather tile must be whole waves");
constexpr int kUnroll = HC_UNROLL;
constexpr int kWaves = kThreads / 64;

// 16-byte vector in global address space (global_load/store_dwordx4, not flat).
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const v4u* gload_t;
typedef __attribute__((address_space(1))) v4u* gstore_t;

__device__ __forceinline__ v4u ld16(uint64_t a) {
#if HC_NT_LOAD
  return __builtin_nontemporal_load(reinterpret_cast<gload_t>(a));
#else
  return *reinterpret_cast<gload_t>(a);
#endif
}
__device__ __forceinline__ void st16(uint64_t a, v4u v) {
#if HC_NT_STORE
  __builtin_nontemporal_store(v, reinterpret_cast<gstore_t>(a));
#else
  *reinterpret_cast<gstore_t>(a) = v;
#endif
}

// q = u / vecs for u < 2^20 and vecs <= 2^20 (magic = ceil(2^40 / vecs)).
__device__ __forceinline__ uint32_t div_vecs(uint32_t u, uint64_t magic) {
  return (uint32_t)(((uint64_t)u * magic) >> 40);
}

// Block-wide compaction of a per-thread predicate.  Each wave takes a 64-bit
// ballot; a lane's rank among its wave's kept lanes is mbcnt of the ballot;
// wave totals go through LDS for the block prefix.  Returns the thread's slot
// (meaningful when keep) and the block total in *total.
__device__ __forceinline__ int compact_slot(bool keep, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const unsigned long long m = __ballot(keep);
  const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  if (lane == 0) s_wave[wave] = __popcll(m);
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; w++) {
    const int c = s_wave[w];
    base += (w < wave) ? c : 0;
    all += c;
  }
  *total = all;
  return base + rank;
}

// Copies `rows` rows of `vecs` 16-byte vectors: row q from s_src[q] to s_dst[q].
// Each lane takes batches of U vectors, `kThreads` apart.  PIPELINED issues the loads
// of batch k+1 before the stores of batch k, so a lane keeps 2U loads in flight while
// its stores drain: the host-link read kernel gains from it, the HBM kernels lose
// occupancy to the extra registers and do not.
template <bool PIPELINED, int U>
__device__ __forceinline__ void copy_rows(const uint64_t* s_src, const uint64_t* s_dst, int rows,
                                          uint32_t vecs, uint64_t magic) {
  const uint32_t total = (uint32_t)rows * vecs;
  auto load_batch = [&](uint32_t u0, v4u* v, uint64_t* dst) {
#pragma unroll
    for (int k = 0; k < U; k++) {
      const uint32_t u = u0 + k * kThreads;
      if (u < total) {
        const uint32_t q = div_vecs(u, magic);
        const uint64_t off = (uint64_t)(u - q * vecs) * 16u;
        v[k] = ld16(s_src[q] + off);
        dst[k] = s_dst[q] + off;
      }
    }
  };
  auto store_batch = [&](uint32_t u0, const v4u* v, const uint64_t* dst) {
#pragma unroll
    for (int k = 0; k < U; k++) {
      const uint32_t u = u0 + k * kThreads;
      if (u < total) st16(dst[k], v[k]);
    }
  };
  constexpr uint32_t step = kThreads * U;
  if (!PIPELINED) {
    for (uint32_t u0 = threadIdx.x; u0 < total; u0 += step) {
      v4u v[U];
      uint64_t dst[U];
      load_batch(u0, v, dst);
      store_batch(u0, v, dst);
    }
    return;
  }
  v4u va[U], vb[U];
  uint64_t da[U], db[U];
  uint32_t u0 = threadIdx.x;
  if (u0 >= total) return;
  load_batch(u0, va, da);
  for (;;) {
    const uint32_t u1 = u0 + step;
    if (u1 < total) load_batch(u1, vb, db);
    store_batch(u0, va, da);
    if (u1 >= total) break;
    const uint32_t u2 = u1 + step;
    if (u2 < total) load_batch(u2, va, da);
    store_batch(u1, vb, db);
    if (u2 >= total) break;
    u0 = u2;
  }
}

__device__ __forceinline__ uint64_t layer_base(const SubGeom& s, int l) { return s.layers[l]; }

// Host byte offset of (sub s, page p, layer l, row r).
__device__ __forceinline__ int64_t host_off(const SubGeom& s, int64_t p, int l, int r) {
  return s.host_region + p * s.host_page_stride + (int64_t)l * s.layer_stride + (int64_t)r * s.row_stride;
}

// Device byte offset of slot d inside one layer.
__device__ __forceinline__ int64_t dev_off(const SubGeom& s, int64_t d, int P) {
  return (s.gran == HC_TOKEN_ROWS ? d : d / P) * s.elem;
}

// A bad index list: sets bit `bit` of the error word and keeps the smallest list position
// flagged since the last report in the uint64 that follows the word at byte 8.
__device__ __forceinline__ void flag_bad(int32_t* err, int bit, int64_t pos) {
  atomicOr(err, bit);
  atomicMin(reinterpret_cast<unsigned long long*>(err + 2), (unsigned long long)pos);
}

// HC_FLAG_VALIDATE for page-block sub-buffers: token i must either start a page on
// both sides (h % P == 0 with d % P == 0) or continue the previous token's run on both
// sides (d = d[i-1] + 1, h = h[i-1] + 1), so that every page moves as one whole device
// page.  Violations set bit 2 of the error word.
__device__ __forceinline__ void check_page_row(int64_t i, int64_t d, int64_t h, const int64_t* dev_idx,
                                               const int64_t* host_idx, int P, int32_t* err) {
  const bool ok = (h % P == 0) ? (d % P == 0) : (i > 0 && dev_idx[i - 1] + 1 == d && host_idx[i - 1] + 1 == h);
  if (!ok) flag_bad(err, 2, i);
}

// Zero-copy units.  A sub-buffer's units walk list positions j * stride: stride 1 for
// token rows; for page blocks, stride P when the list holds whole pages in row order
// (the row-0 token of every page then sits at a multiple of P), so a unit carries up
// to tile_n blocks instead of tile_n / P.  Units are sub-buffer-major (page blocks
// first, see unit_sub); `mult` counts
// the units per tile (the layer count for the all-layer write-back, 1 for a layer).
__host__ __device__ __forceinline__ int64_t sub_positions(const SubGeom& s, int64_t n, int blk_stride) {
  return s.gran == HC_PAGE_BLOCKS ? (n + blk_stride - 1) / blk_stride : n;
}

// Page blocks walked with the block stride take blk_tile blocks per unit, chosen by the
// launcher so that the blocks alone give about one unit per workgroup, at most
// kTile >> HC_BLOCK_TILE_SHIFT.  Measured on the 78-layer MLA + indexer load-back: at the
// full 1024-page burst a fixed 256 blocks per unit (2.1 MiB, 4 units per layer) gave
// 1.56 ms per layer, the token-strided walk 1.50 ms, 64 blocks 1.47 ms (99 % of the host
// link), 32 or 16 the same; but a fixed 64 left a 64-page burst's blocks in one unit that
// one workgroup read alone (147 us per layer against 101 us token-strided).
#ifndef HC_BLOCK_TILE_SHIFT
#define HC_BLOCK_TILE_SHIFT 2
#endif
#ifndef HC_BLOCK_STRIDE_ON
#define HC_BLOCK_STRIDE_ON 1
#endif
__host__ __device__ __forceinline__ int sub_tile(const SubGeom& s, int blk_stride, int tile_n, int blk_tile) {
  return (s.gran == HC_PAGE_BLOCKS && blk_stride > 1) ? blk_tile : tile_n;
}

__host__ __device__ __forceinline__ int64_t sub_units(const SubGeom& s, int64_t n, int blk_stride, int tile_n,
                                                      int blk_tile, int64_t mult) {
  const int t = sub_tile(s, blk_stride, tile_n, blk_tile);
  return (sub_positions(s, n, blk_stride) + t - 1) / t * mult;
}

// Sub-buffer of `unit`, and the unit's index inside that sub-buffer's units.  Page-block
// sub-buffers come first: with the block stride their units are the largest (a tile of
// whole-page blocks), and taken last they left a few workgroups running alone at the
// end of a layer.
__device__ __forceinline__ int unit_sub(const Geom& g, int64_t n, int blk_stride, int tile_n, int blk_tile,
                                        int64_t mult, int64_t unit, int64_t* rem) {
  int64_t acc = 0;
  for (int pass = 0; pass < 2; pass++) {
    for (int b = 0; b < g.nsub; b++) {
      if ((g.sub[b].gran == HC_PAGE_BLOCKS) != (pass == 0)) continue;
      const int64_t ub = sub_units(g.sub[b], n, blk_stride, tile_n, blk_tile, mult);
      if (unit < acc + ub) {
        *rem = unit - acc;
        return b;
      }
      acc += ub;
    }
  }
  // not reached for unit < units; a position past sub-buffer 0's last leaves every lane idle
  *rem = sub_units(g.sub[0], n, blk_stride, tile_n, blk_tile, mult);
  return 0;
}

// ---------------------------------------------------------------- staged write-back: gather
// Units of (sub-buffer, kGatherTile staged tokens of [t0, t0+count), layer), walked
// grid-stride by a grid of a few workgroups per CU: small units keep every CU streaming
// until the last unit, where one workgroup per (tile, layer, sub) left 2-3 rounds per CU
// and a thin tail.  Staged token k is list position perm[k]; srow[k] = slot * P + row
// inside the chunk's staging images (the planner lists a chunk's tokens together, so a
// chunk is a range of k), or -1 for a token that does not go through staging.
__global__ __launch_bounds__(kThreads) void k_gather_stage(Geom g, const int64_t* __restrict__ dev_idx,
                                                           const int64_t* __restrict__ host_idx,
                                                           const int32_t* __restrict__ perm,
                                                           const int32_t* __restrict__ srow, int64_t t0,
                                                           int64_t count, uint8_t* __restrict__ staging,
                                                           int32_t* __restrict__ err, int64_t units) {
  __shared__ uint64_t s_src[kGatherTile];
  __shared__ uint64_t s_dst[kGatherTile];
  __shared__ int s_wave[kWaves];
  // sub-buffer-major order: a workgroup's stride crosses sub-buffers of different row
  // sizes instead of staying on one of them
  const int64_t per_sub = units / g.nsub;
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int b = (int)(unit / per_sub);
    const int64_t rem = unit - (int64_t)b * per_sub;
    const int64_t tile = rem / g.L;
    const int l = (int)(rem - tile * g.L);
    const SubGeom& s = g.sub[b];
    const int64_t k = t0 + tile * kGatherTile + threadIdx.x;
    bool keep = false;
    uint64_t src = 0, dst = 0;
    if (threadIdx.x < kGatherTile && k < t0 + count) {
      const int64_t i = perm[k];
      const int32_t sr = srow[k];
      if (sr >= 0) {
        const int32_t slot = sr / g.P;
        const int32_t r = sr - slot * g.P;
        if (g.validate && s.gran == HC_PAGE_BLOCKS) check_page_row(i, dev_idx[i], host_idx[i], dev_idx, host_idx, g.P, err);
        if (s.gran == HC_TOKEN_ROWS || r == 0) {
          const int64_t d = dev_idx[i];
          if (d >= 0 && d < g.S) {
            src = layer_base(s, l) + (uint64_t)dev_off(s, d, g.P);
            dst = (uint64_t)staging + (uint64_t)((int64_t)slot * s.stg_slot + s.img_off +
                                                 (int64_t)l * s.layer_stride + (int64_t)r * s.row_stride);
            keep = true;
          } else {
            flag_bad(err, 1, i);
          }
        }
      }
    }
    int total;
    const int slot = compact_slot(keep, s_wave, &total);
    if (keep) {
      s_src[slot] = src;
      s_dst[slot] = dst;
    }
    __syncthreads();
    copy_rows<false, kUnroll>(s_src, s_dst, total, s.vecs, s.vec_magic);
    __syncthreads();  // LDS is rewritten by the next unit
  }
}

// ---------------------------------------------------------------- zero-copy write-back
// Device rows -> pinned host pool.  Tokens are [0, count) or tok_list[0, count).
// Units (sub, tile, layer) are walked grid-stride so a capped grid suffices.
// Tiles hold kTile >> tile_shift list positions (see sub_units for page blocks).
__global__ __launch_bounds__(kThreads) void k_zc_write(Geom g, const int64_t* __restrict__ dev_idx,
                                                       const int64_t* __restrict__ host_idx,
                                                       const int32_t* __restrict__ tok_list, int64_t count,
                                                       uint8_t* __restrict__ host, int32_t* __restrict__ err,
                                                       int64_t units, int tile_shift, int blk_stride,
                                                       int blk_tile) {
  __shared__ uint64_t s_src[kTile];
  __shared__ uint64_t s_dst[kTile];
  __shared__ int s_wave[kWaves];
  const int tile_n = kTile >> tile_shift;
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    int64_t rem;
    const int b = unit_sub(g, count, blk_stride, tile_n, blk_tile, g.L, unit, &rem);
    const int64_t tile = rem / g.L;
    const int l = (int)(rem - tile * g.L);
    const SubGeom& s = g.sub[b];
    const int st = sub_tile(s, blk_stride, tile_n, blk_tile);
    const int64_t j = tile * st + threadIdx.x;
    const int stride = s.gran == HC_PAGE_BLOCKS ? blk_stride : 1;
    bool keep = false;
    uint64_t src = 0, dst = 0;
    if ((int)threadIdx.x < st && j < sub_positions(s, count, blk_stride)) {
      const int64_t i = tok_list ? (int64_t)tok_list[j] : j * stride;
      const int64_t d = dev_idx[i];
      const int64_t h = host_idx[i];
      const int64_t p = h / g.P;
      const int r = (int)(h - p * g.P);
      if (g.validate && s.gran == HC_PAGE_BLOCKS) check_page_row(i, d, h, dev_idx, host_idx, g.P, err);
      if (s.gran == HC_TOKEN_ROWS || r == 0) {
        if (d >= 0 && d < g.S && h >= 0 && h < g.host_tokens) {
          src = layer_base(s, l) + (uint64_t)dev_off(s, d, g.P);
          dst = (uint64_t)host + (uint64_t)host_off(s, p, l, r);
          keep = true;
        } else {
          flag_bad(err, 1, i);
        }
      }
    }
    int total;
    const int slot = compact_slot(keep, s_wave, &total);
    if (keep) {
      s_src[slot] = src;
      s_dst[slot] = dst;
    }
    __syncthreads();
    copy_rows<kWritePipelined, kWriteUnroll>(s_src, s_dst, total, s.vecs, s.vec_magic);
    __syncthreads();  // LDS is rewritten by the next unit
  }
}

// ---------------------------------------------------------------- zero-copy load-back (one layer)
// Pinned host pool -> device rows of layer `layer`.  Indices are device-resident.
// Units (sub, tile) grid-stride.  With g.validate, page-block sub-buffers also check
// that each page's rows arrive as one run of P consecutive device slots starting on a
// page boundary (neighbour compare through a lane shuffle, LDS at wave edges).
// Tiles hold kTile >> tile_shift list positions, as in k_zc_write.
__global__ __launch_bounds__(kThreads) void k_zc_read(Geom g, int32_t layer, const int64_t* __restrict__ host_idx,
                                                      const int64_t* __restrict__ dev_idx, int64_t n,
                                                      const uint8_t* __restrict__ host, int32_t* __restrict__ err,
                                                      int64_t units, int tile_shift, int blk_stride,
                                                      int blk_tile) {
  __shared__ uint64_t s_src[kTile];
  __shared__ uint64_t s_dst[kTile];
  __shared__ int s_wave[kWaves];
  const int tile_n = kTile >> tile_shift;
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    int64_t tile;
    const int b = unit_sub(g, n, blk_stride, tile_n, blk_tile, 1, unit, &tile);
    const SubGeom& s = g.sub[b];
    const int st = sub_tile(s, blk_stride, tile_n, blk_tile);
    const int64_t j = tile * st + threadIdx.x;
    const int64_t i = j * (s.gran == HC_PAGE_BLOCKS ? blk_stride : 1);
    bool keep = false;
    uint64_t src = 0, dst = 0;
    int64_t d = 0, h = 0;
    const bool live = (int)threadIdx.x < st && j < sub_positions(s, n, blk_stride);
    if (live) {
      d = dev_idx[i];
      h = host_idx[i];
    }
    if (g.validate && s.gran == HC_PAGE_BLOCKS) {
      // previous token's indices: lane shuffle inside the wave, memory at the wave's first lane
      int64_t dp = __shfl_up(d, 1);
      int64_t hp = __shfl_up(h, 1);
      if ((threadIdx.x & 63) == 0 && live && i > 0) {
        dp = dev_idx[i - 1];
        hp = host_idx[i - 1];
      }
      if (live) {
        const bool first_row = (h % g.P) == 0;
        const bool ok = first_row ? (d % g.P == 0) : (i > 0 && dp + 1 == d && hp + 1 == h);
        if (!ok) flag_bad(err, 2, i);
      }
    }
    if (live) {
      const int64_t p = h / g.P;
      const int r = (int)(h - p * g.P);
      if (s.gran == HC_TOKEN_ROWS || r == 0) {
        if (d >= 0 && d < g.S && h >= 0 && h < g.host_tokens) {
          src = (uint64_t)host + (uint64_t)host_off(s, p, layer, r);
          dst = layer_base(s, layer) + (uint64_t)dev_off(s, d, g.P);
          keep = true;
        } else {
          flag_bad(err, 1, i);
        }
      }
    }
    int total;
    const int slot = compact_slot(keep, s_wave, &total);
    if (keep) {
      s_src[slot] = src;
      s_dst[slot] = dst;
    }
    __syncthreads();
    copy_rows<kReadPipelined, kReadUnroll>(s_src, s_dst, total, s.vecs, s.vec_magic);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- shard padding
// Zeroes [off, off + bytes) of page pages[k] (or page k when pages is null) for k < npages.
__global__ __launch_bounds__(kThreads) void k_zero_pads(uint8_t* __restrict__ base, const int64_t* __restrict__ pages,
                                                        int64_t npages, int64_t stride, int64_t off, uint32_t vecs) {
  const int64_t total = npages * (int64_t)vecs;
  const v4u z = {0u, 0u, 0u, 0u};
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total; u += (int64_t)gridDim.x * kThreads) {
    const int64_t k = u / vecs;
    const int64_t v = u - k * vecs;
    const int64_t p = pages ? pages[k] : k;
    st16((uint64_t)base + (uint64_t)(p * stride + off + v * 16), z);
  }
}

// Shard pads from the token list itself (no page list): position k zeroes vector v of its
// page's pad when it starts a run of same-page entries.  Used where no plan of distinct
// pages is uploaded (the write-back that allocates nothing).
__global__ __launch_bounds__(kThreads) void k_zero_pads_runs(uint8_t* __restrict__ base,
                                                             const int64_t* __restrict__ host_idx, int64_t n,
                                                             int32_t P, int64_t host_pages, int64_t stride,
                                                             int64_t off, uint32_t vecs) {
  const int64_t total = n * (int64_t)vecs;
  const v4u z = {0u, 0u, 0u, 0u};
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total; u += (int64_t)gridDim.x * kThreads) {
    const int64_t k = u / vecs;
    const int64_t v = u - k * vecs;
    const int64_t h = host_idx[k];
    if (h < 0 || h / P >= host_pages) continue;
    const int64_t p = h / P;
    if (k > 0) {
      const int64_t hp = host_idx[k - 1];
      if (hp >= 0 && hp / P == p) continue;  // not the first entry of its run
    }
    st16((uint64_t)base + (uint64_t)(p * stride + off + v * 16), z);
  }
}

// ---------------------------------------------------------------- round-trip compare
// grid = (tiles, L, nsub).  Counts rows (or page blocks at a[i] % P == 0) whose bytes
// at slot a[i] and slot c[i] differ.  One wave compares one row at a time; the row's
// result is the OR of the lanes' results (ballot).
__global__ __launch_bounds__(kThreads) void k_compare(Geom g, const int64_t* __restrict__ a,
                                                      const int64_t* __restrict__ c, int64_t n,
                                                      unsigned long long* __restrict__ counter,
                                                      int32_t* __restrict__ err) {
  __shared__ uint64_t s_x[kTile];
  __shared__ uint64_t s_y[kTile];
  __shared__ int s_wave[kWaves];
  const int b = blockIdx.z;
  const int l = blockIdx.y;
  const SubGeom& s = g.sub[b];
  const int64_t i = (int64_t)blockIdx.x * kTile + threadIdx.x;
  bool keep = false;
  uint64_t x = 0, y = 0;
  if (threadIdx.x < kTile && i < n) {
    const int64_t da = a[i], dc = c[i];
    if (da >= 0 && da < g.S && dc >= 0 && dc < g.S) {
      if (s.gran == HC_TOKEN_ROWS || da % g.P == 0) {
        x = layer_base(s, l) + (uint64_t)dev_off(s, da, g.P);
        y = layer_base(s, l) + (uint64_t)dev_off(s, dc, g.P);
        keep = true;
      }
    } else {
      flag_bad(err, 1, i);
    }
  }
  int total;
  const int slot = compact_slot(keep, s_wave, &total);
  if (keep) {
    s_x[slot] = x;
    s_y[slot] = y;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  unsigned long long bad = 0;
  for (int q = wave; q < total; q += kWaves) {
    bool diff = false;
    for (uint32_t v = lane; v < s.vecs; v += 64) {
      const v4u p0 = ld16(s_x[q] + (uint64_t)v * 16u);
      const v4u p1 = ld16(s_y[q] + (uint64_t)v * 16u);
      diff |= (p0.x != p1.x) | (p0.y != p1.y) | (p0.z != p1.z) | (p0.w != p1.w);
    }
    if (__ballot(diff) != 0ull) bad++;
  }
  if (lane == 0 && bad) atomicAdd(counter, bad);
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// One launch of kThreads-wide workgroups; timed through the launch itself when t holds events.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, const LaunchTimer& t, hipStream_t stream, Args... args) {
  (void)hipGetLastError();  // the status read below must be this launch's own
  if (t.start)
    hipExtLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, t.start, t.stop, 0, args...);
  else
    kernel<<<grid, kThreads, 0, stream>>>(args...);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_stage(const Geom& g, const int64_t* dev_idx, const int64_t* host_idx, const int32_t* perm,
                               const int32_t* srow, int64_t t0, int64_t count, uint8_t* staging, int32_t* err,
                               int32_t num_cus, const LaunchTimer& t, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const int64_t units = ceil_div(count, kGatherTile) * g.L * g.nsub;
  const int64_t cap = (int64_t)(num_cus > 0 ? num_cus : 256) * HC_GATHER_BLOCKS_PER_CU;
  const int64_t grid = units < cap ? units : cap;
  return launch(k_gather_stage, dim3((unsigned)grid), t, stream, g, dev_idx, host_idx, perm, srow, t0, count, staging,
                err, units);
}

// Units of a zero-copy launch over list positions [0, count): summed over sub-buffers.
static int64_t zc_units(const Geom& g, int64_t count, int blk_stride, int tile_n, int blk_tile, int64_t mult) {
  int64_t units = 0;
  for (int b = 0; b < g.nsub; b++) units += sub_units(g.sub[b], count, blk_stride, tile_n, blk_tile, mult);
  return units;
}

// Blocks per page-block unit under the block stride: enough units for the grid (blocks
// x mult / max_ctas, rounded up), at most kTile >> HC_BLOCK_TILE_SHIFT.
static int block_tile_for(int64_t count, int blk_stride, int64_t mult, int32_t max_ctas) {
  constexpr int64_t kMaxBlockTile = kTile >> HC_BLOCK_TILE_SHIFT;
  if (blk_stride <= 1) return (int)kMaxBlockTile;  // not used: blocks walk the token tiles
  const int64_t blocks = (count + blk_stride - 1) / blk_stride;
  const int64_t ctas = max_ctas > 0 ? max_ctas : 1;
  const int64_t t = (blocks * mult + ctas - 1) / ctas;
  return (int)(t < 1 ? 1 : (t > kMaxBlockTile ? kMaxBlockTile : t));
}
static_assert((kTile >> HC_BLOCK_TILE_SHIFT) >= 1 && (kTile >> HC_BLOCK_TILE_SHIFT) <= kTile,
              "a block unit fits the unit's LDS lists");

// Tile shift for a small burst.  Units go to workgroups round-robin (unit u to
// workgroup u % grid, in the kernels' order: page blocks first, then sub-buffer, tile,
// layer), and one workgroup moves only ~7 GB/s over the host link, so a launch lasts
// about as long as its busiest workgroup.  The shift (0 .. kMaxTileShift, tiles of
// kTile >> shift list positions) is the one whose busiest workgroup carries the fewest
// bytes, counting a fixed intake per unit.  Measured before this model, on the 78-layer
// MLA + indexer load-back: "shrink until the units fill the grid" left 17 units on 16
// workgroups for a 1-page burst (11.3 us per layer, 8.1 us when each workgroup takes one
// unit), and counting page-block units toward the grid left a 16-page burst's latent rows
// in 4 units of 256 tokens (44 us per layer against 32 us).
constexpr int kMaxTileShift = 6;
constexpr int64_t kUnitIntakeBytes = 8192;  // the intake's cost, in bytes of copying

static int64_t busiest_workgroup_bytes(const Geom& g, int64_t count, int bs, int tile_n, int bt, int64_t mult,
                                       int64_t grid, int64_t* load) {
  for (int64_t w = 0; w < grid; w++) load[w] = 0;
  int64_t u = 0;
  for (int pass = 0; pass < 2; pass++) {
    for (int b = 0; b < g.nsub; b++) {
      const SubGeom& s = g.sub[b];
      if ((s.gran == HC_PAGE_BLOCKS) != (pass == 0)) continue;
      const int t = sub_tile(s, bs, tile_n, bt);
      const int64_t pos = sub_positions(s, count, bs);
      for (int64_t j0 = 0; j0 < pos; j0 += t) {
        int64_t items = pos - j0 < t ? pos - j0 : t;
        if (s.gran == HC_PAGE_BLOCKS && bs <= 1) items = (items + g.P - 1) / g.P;  // one block per page
        const int64_t bytes = items * s.elem + kUnitIntakeBytes;
        for (int64_t l = 0; l < mult; l++) load[u++ % grid] += bytes;
      }
    }
  }
  int64_t most = 0;
  for (int64_t w = 0; w < grid; w++) most = load[w] > most ? load[w] : most;
  return most;
}

static int tile_shift_for(const Geom& g, int64_t count, int blk_stride, int blk_tile, int64_t mult,
                          int32_t max_ctas, int64_t* wg_load) {
  // under the block stride, page blocks have their own units (block_tile_for spreads them)
  auto row_units = [&](int tile_n) {
    int64_t n = 0;
    for (int b = 0; b < g.nsub; b++)
      if (blk_stride <= 1 || g.sub[b].gran != HC_PAGE_BLOCKS)
        n += sub_units(g.sub[b], count, blk_stride, tile_n, blk_tile, mult);
    return n;
  };
  const int64_t ctas = max_ctas > 0 ? max_ctas : 1;
  if (row_units(kTile) == 0 || row_units(kTile) >= 4 * ctas) return 0;  // no rows, or plenty of full tiles
  int best = 0;
  int64_t best_bytes = -1;
  for (int shift = 0; shift <= kMaxTileShift; shift++) {
    if (shift > 0 && row_units(kTile >> (shift - 1)) >= 4 * ctas) break;  // finer tiles only add intakes
    const int64_t units = zc_units(g, count, blk_stride, kTile >> shift, blk_tile, mult);
    const int64_t grid = units < ctas ? units : ctas;
    const int64_t most = busiest_workgroup_bytes(g, count, blk_stride, kTile >> shift, blk_tile, mult, grid, wg_load);
    if (best_bytes < 0 || most < best_bytes) {
      best = shift;
      best_bytes = most;
    }
  }
  return best;
}

// Page blocks take only the positions k * P when the list is known to hold whole pages
// in row order: always by contract without HC_FLAG_VALIDATE (with it, every position
// is visited so the order can be checked), never for a token sub-list.
static int block_stride(const Geom& g, bool full_list) {
  if (!HC_BLOCK_STRIDE_ON || g.validate || !full_list) return 1;
  for (int b = 0; b < g.nsub; b++)
    if (g.sub[b].gran == HC_PAGE_BLOCKS) return g.P;
  return 1;
}

hipError_t launch_zc_write(const Geom& g, const int64_t* dev_idx, const int64_t* host_idx, const int32_t* tok_list,
                           int64_t count, uint8_t* host, int32_t* err, int32_t max_ctas, int64_t* wg_load,
                           const LaunchTimer& t, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const int bs = block_stride(g, tok_list == nullptr);
  const int bt = block_tile_for(count, bs, g.L, max_ctas);
  const int shift = tile_shift_for(g, count, bs, bt, g.L, max_ctas, wg_load);
  const int64_t units = zc_units(g, count, bs, kTile >> shift, bt, g.L);
  const int64_t grid = units < max_ctas ? units : max_ctas;
  return launch(k_zc_write, dim3((unsigned)grid), t, stream, g, dev_idx, host_idx, tok_list, count, host, err, units,
                shift, bs, bt);
}

hipError_t launch_zc_read(const Geom& g, int32_t layer, const int64_t* host_idx, const int64_t* dev_idx, int64_t n,
                          const uint8_t* host, int32_t* err, int32_t max_ctas, int64_t* wg_load, const LaunchTimer& t,
                          hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int bs = block_stride(g, true);
  const int bt = block_tile_for(n, bs, 1, max_ctas);
  const int shift = tile_shift_for(g, n, bs, bt, 1, max_ctas, wg_load);
  const int64_t units = zc_units(g, n, bs, kTile >> shift, bt, 1);
  const int64_t grid = units < max_ctas ? units : max_ctas;
  return launch(k_zc_read, dim3((unsigned)grid), t, stream, g, layer, host_idx, dev_idx, n, host, err, units, shift,
                bs, bt);
}

hipError_t launch_zero_pads(uint8_t* base, const int64_t* pages, int64_t npages, int64_t stride, int64_t off,
                            int64_t bytes, const LaunchTimer& t, hipStream_t stream) {
  if (npages <= 0 || bytes <= 0) return hipSuccess;
  const uint32_t vecs = (uint32_t)(bytes / 16);
  const int64_t total = npages * (int64_t)vecs;
  int64_t grid = ceil_div(total, kThreads);
  if (grid > 4096) grid = 4096;
  return launch(k_zero_pads, dim3((unsigned)grid), t, stream, base, pages, npages, stride, off, vecs);
}

hipError_t launch_zero_pads_runs(uint8_t* base, const int64_t* host_idx, int64_t n, int32_t P, int64_t host_pages,
                                 int64_t stride, int64_t off, int64_t bytes, hipStream_t stream) {
  if (n <= 0 || bytes <= 0) return hipSuccess;
  const uint32_t vecs = (uint32_t)(bytes / 16);
  const int64_t total = n * (int64_t)vecs;
  int64_t grid = ceil_div(total, kThreads);
  if (grid > 4096) grid = 4096;
  return launch(k_zero_pads_runs, dim3((unsigned)grid), LaunchTimer{}, stream, base, host_idx, n, P, host_pages,
                stride, off, vecs);
}

hipError_t launch_compare(const Geom& g, const int64_t* a, const int64_t* c, int64_t n, unsigned long long* counter,
                          int32_t* err, const LaunchTimer& t, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t tiles = ceil_div(n, kTile);
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  return launch(k_compare, dim3((unsigned)tiles, (unsigned)g.L, (unsigned)g.nsub), t, stream, g, a, c, n, counter,
                err);
}

}  // namespace hc
