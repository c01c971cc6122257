// HIP kernels of the per-layer exchange of a layer-owner sharded host tier
// (rank-sharded tier page, sglang PR 41984, Modifications, load-back): each host
// layer has one owner rank; after the owner has loaded a layer into its device
// slots it gathers those rows into a staging buffer ("pack"), the buffer is
// broadcast to the other TP ranks, and each of them scatters it into the same
// device slots ("unpack"), since device slot allocation is replicated.
//
// Staging order: sub-buffer after sub-buffer; inside sub-buffer b the token rows of
// the listed slots in list order, or for page blocks one block per page (the block
// of the slot at list positions 0, P, 2P, ...).  Both directions are plain HBM
// gathers/scatters of 16-byte vectors, so they are written for HBM bandwidth:
//
// Work is cut into units of (sub-buffer, tile of list positions), sub-buffer-major,
// walked grid-stride.  The launcher sizes each sub-buffer's tile in bytes rather than
// rows, so a unit of 8448-byte indexer blocks carries about as many bytes as a unit of
// 1152-byte latent rows and no workgroup is left copying a few large units alone at
// the end.  A unit starts with an intake (one thread per position reads the slot,
// range-checks it and computes the device row address; the staging address follows
// from the position), then all 256 lanes walk rows * (elem/16) vectors, lane u taking
// vector u % vecs of row u / vecs, in batches of loads issued before their stores.
// These kernels live apart from the host-link kernels so that each file's measured
// code stays as it was measured.
//
// A flat split was tried and dropped: the layer's vectors cut into one contiguous, equal
// range per workgroup (2, 4 or 8 per CU), each walked in batches of up to 256 rows with an
// intake per batch.  It balances the work exactly but starts every workgroup on its intake
// at once and has no next unit to prefetch: over three interleaved rounds on the shard,
// 78-layer and Llama-3-8B layers it reached 5.11-5.23 TB/s for pack then unpack (4.53-4.65
// cold) against 5.47 (4.91) for the units below.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hc_internal.h"

namespace hc {
namespace {

constexpr int kXThreads = 256;  // 4 waves of 64
constexpr int kXMaxTile = 256;  // positions per unit at most (one per thread at intake)
#ifndef HC_XCHG_UNROLL
#define HC_XCHG_UNROLL 8
#endif
constexpr int kXUnroll = HC_XCHG_UNROLL;
// Bytes per unit: the launch's bytes spread over about HC_XCHG_UNITS_PER_CU units per
// CU, clamped to [kXMinUnitBytes, kXMaxUnitBytes], grown until the units fit that many
// (HC_XCHG_ROUND_FIT); a grid of HC_XCHG_BLOCKS_PER_CU workgroups per CU walks them, each
// loading its next unit's slots one unit ahead (HC_XCHG_PREFETCH).  Measured with the
// loads-only hint below, averaged over three interleaved rounds on the 48-layer shard,
// 78-layer MLA + indexer and Llama-3-8B layers (TB/s, pack then unpack on one staging
// buffer / each cold): 8 units and 4 workgroups per CU 5.51 / 4.94, 8 and 8 5.48 / 4.86,
// 16 and 8 5.38 / 4.82 (5.35 / 4.78 without the fit), 4 and 2 ~5.35.  An earlier sweep
// with both hints found 16 and 8 with the prefetch best (80-92 % of a plain copy of the
// same bytes), 4 and 4 without it 75-86 %, and 4 or 16 loads in flight per lane no better.
#ifndef HC_XCHG_UNITS_PER_CU
#define HC_XCHG_UNITS_PER_CU 8
#endif
constexpr int64_t kXMinUnitBytes = 16 << 10;
constexpr int64_t kXMaxUnitBytes = 256 << 10;
#ifndef HC_XCHG_PREFETCH
#define HC_XCHG_PREFETCH 1
#endif
#ifndef HC_XCHG_BLOCKS_PER_CU
#define HC_XCHG_BLOCKS_PER_CU 4
#endif
#ifndef HC_XCHG_ROUND_FIT
#define HC_XCHG_ROUND_FIT 1
#endif

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const v4u* gload_t;
typedef __attribute__((address_space(1))) v4u* gstore_t;

// Loads carry the non-temporal hint (bit 0), stores do not (bit 1 off): on the path the
// packed layer is read right after it is written (by the broadcast on the owner; by the
// unpack when a rank packs and unpacks in one place), so the staging bytes should stay in
// the Infinity Cache.  Measured on one GPU, pack then unpack of each layer on one staging
// buffer, three interleaved rounds (TB/s of the pair, read + write counted per call):
// 48-layer shard layer (237 MB) 5.72-5.89 with loads only against 4.92-5.23 with both
// hints; 78-layer MLA + indexer layer (84 MB) 5.24-5.33 against 5.05; Llama-3-8B layer
// (64 MiB) 4.93-5.20 against 4.89-4.92.  The unpack then reads staging at ~6 TB/s.  Each
// layer packed into its own staging buffer and unpacked later (everything cold) runs
// 3-8 % slower with loads only than with both hints, and 12-18 % slower with neither.
// Eight waves per SIMD (HC_XCHG_MIN_WAVES, which needs 4 loads in flight per lane to fit
// 64 registers) was slower with or without the hints.
#ifndef HC_XCHG_NT
#define HC_XCHG_NT 1
#endif
#ifndef HC_XCHG_MIN_WAVES
#define HC_XCHG_MIN_WAVES 1  // launch-bounds floor on waves per SIMD (caps registers)
#endif
__device__ __forceinline__ v4u xld16(uint64_t a) {
  if (HC_XCHG_NT & 1) return __builtin_nontemporal_load(reinterpret_cast<gload_t>(a));
  return *reinterpret_cast<gload_t>(a);
}
__device__ __forceinline__ void xst16(uint64_t a, v4u v) {
  if (HC_XCHG_NT & 2)
    __builtin_nontemporal_store(v, reinterpret_cast<gstore_t>(a));
  else
    *reinterpret_cast<gstore_t>(a) = v;
}

// The error word of the pool: bit `bit`, and the smallest flagged list position in the
// uint64 at byte 8 (the same report the transfer kernels make).
__device__ __forceinline__ void flag_position(int32_t* err, int bit, int64_t pos) {
  atomicOr(err, bit);
  atomicMin(reinterpret_cast<unsigned long long*>(err + 2), (unsigned long long)pos);
}

template <bool PACK>
__global__ __launch_bounds__(kXThreads, HC_XCHG_MIN_WAVES) void k_layer_exchange(Geom g, XPlan x, int32_t layer,
                                                              const int64_t* __restrict__ dev_idx,
                                                              uint8_t* __restrict__ staging,
                                                              int32_t* __restrict__ err) {
  __shared__ uint64_t s_dev[kXMaxTile];
  __shared__ uint64_t s_stg[kXMaxTile];
  const int64_t units = x.units_end[g.nsub - 1];
  // A unit's sub-buffer, first position and row count.
  auto locate = [&](int64_t unit, int* b, int64_t* j0, int* rows) {
    int c = 0;
    while (unit >= x.units_end[c]) c++;  // c < nsub because unit < units
    const int tile = x.tile[c];
    *b = c;
    *j0 = (unit - (c ? x.units_end[c - 1] : 0)) * tile;
    const int64_t left = x.positions[c] - *j0;
    *rows = left < tile ? (int)left : tile;
  };
  auto list_pos = [&](int b, int64_t j) { return g.sub[b].gran == HC_PAGE_BLOCKS ? j * g.P : j; };
  // This thread's slot of the workgroup's next unit, loaded one unit ahead so that the
  // index read overlaps the copy of the current unit instead of preceding it.
  int64_t d_next = 0;
  if (HC_XCHG_PREFETCH && (int64_t)blockIdx.x < units) {
    int b, rows;
    int64_t j0;
    locate(blockIdx.x, &b, &j0, &rows);
    if ((int)threadIdx.x < rows) d_next = dev_idx[list_pos(b, j0 + threadIdx.x)];
  }
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    int b, rows;
    int64_t j0;
    locate(unit, &b, &j0, &rows);
    int64_t d = 0;
    if (HC_XCHG_PREFETCH) {
      d = d_next;
      if (unit + gridDim.x < units) {
        int nb, nrows;
        int64_t nj0;
        locate(unit + gridDim.x, &nb, &nj0, &nrows);
        if ((int)threadIdx.x < nrows) d_next = dev_idx[list_pos(nb, nj0 + threadIdx.x)];
      }
    } else if ((int)threadIdx.x < rows) {
      d = dev_idx[list_pos(b, j0 + threadIdx.x)];
    }
    const SubGeom& s = g.sub[b];
    const bool blk = s.gran == HC_PAGE_BLOCKS;
    if ((int)threadIdx.x < rows) {
      const int64_t j = j0 + threadIdx.x;
      const int64_t pos = list_pos(b, j);
      uint64_t a = 0;
      if (d >= 0 && d < g.S) {
        if (blk && g.validate) {
          // whole device page in row order: pos holds a page start, pos + r holds d + r
          bool ok = d % g.P == 0;
          for (int r = 1; r < g.P && ok; r++) ok = dev_idx[pos + r] == d + r;
          if (!ok) flag_position(err, 2, pos);
        }
        a = s.layers[layer] + (uint64_t)((blk ? d / g.P : d) * s.elem);
      } else {
        flag_position(err, 1, pos);
      }
      s_dev[threadIdx.x] = a;
      s_stg[threadIdx.x] = (uint64_t)staging + (uint64_t)(x.seg[b] + j * s.elem);
    }
    __syncthreads();
    const uint32_t vecs = s.vecs;
    const uint32_t total = (uint32_t)rows * vecs;
    for (uint32_t u0 = threadIdx.x; u0 < total; u0 += kXThreads * kXUnroll) {
      v4u v[kXUnroll];
      uint64_t dst[kXUnroll];
#pragma unroll
      for (int k = 0; k < kXUnroll; k++) {
        const uint32_t u = u0 + k * kXThreads;
        dst[k] = 0;
        if (u < total) {
          const uint32_t q = (uint32_t)(((uint64_t)u * s.vec_magic) >> 40);  // u / vecs (u < 2^20)
          const uint64_t off = (uint64_t)(u - q * vecs) * 16u;
          const uint64_t dv = s_dev[q];
          if (dv) {
            const uint64_t sv = s_stg[q];
            v[k] = xld16((PACK ? dv : sv) + off);
            dst[k] = (PACK ? sv : dv) + off;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kXUnroll; k++)
        if (dst[k]) xst16(dst[k], v[k]);
    }
    __syncthreads();  // LDS is rewritten by the next unit
  }
}

}  // namespace

int64_t exchange_plan(const Geom& g, int64_t n, int32_t num_cus, XPlan* x) {
  int64_t bytes = 0;
  for (int b = 0; b < g.nsub; b++) {
    x->positions[b] = g.sub[b].gran == HC_PAGE_BLOCKS ? n / g.P : n;
    x->seg[b] = bytes;
    bytes += x->positions[b] * g.sub[b].elem;
  }
  const int64_t cus = num_cus > 0 ? num_cus : 1;
  const int64_t target = cus * HC_XCHG_UNITS_PER_CU;  // a whole number of rounds of the grid
  int64_t unit_bytes = (bytes + target - 1) / target;
  unit_bytes = unit_bytes < kXMinUnitBytes ? kXMinUnitBytes : (unit_bytes > kXMaxUnitBytes ? kXMaxUnitBytes : unit_bytes);
  int64_t units = 0;
  for (;;) {
    units = 0;
    bool capped = true;
    for (int b = 0; b < g.nsub; b++) {
      int64_t t = unit_bytes / g.sub[b].elem;
      t = t < 1 ? 1 : (t > kXMaxTile ? kXMaxTile : t);
      capped = capped && t == kXMaxTile;
      x->tile[b] = (int32_t)t;
      units += (x->positions[b] + t - 1) / t;
      x->units_end[b] = units;
    }
    // Whole rows per unit round each sub-buffer's count up, which can leave a few units
    // past the last full round of the grid, run by a few workgroups alone at the end (the
    // 48-layer shard layer made 4132 units for 2048 workgroups).  Units grow until they fit.
    if (!HC_XCHG_ROUND_FIT || units <= target || capped || unit_bytes >= kXMaxUnitBytes) break;
    unit_bytes += unit_bytes / 64 + 16;
  }
  for (int b = g.nsub; b < HC_MAX_SUBBUFS; b++) {
    x->positions[b] = 0;
    x->seg[b] = bytes;
    x->tile[b] = 1;
    x->units_end[b] = units;
  }
  return bytes;
}

hipError_t launch_layer_exchange(const Geom& g, bool pack, int32_t layer, const int64_t* dev_idx, int64_t n,
                                 uint8_t* staging, int32_t* err, int32_t num_cus, const LaunchTimer& t,
                                 hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  XPlan x;
  exchange_plan(g, n, num_cus, &x);
  const int64_t units = x.units_end[g.nsub - 1];
  if (units <= 0) return hipSuccess;
  const int64_t cap = (int64_t)(num_cus > 0 ? num_cus : 1) * HC_XCHG_BLOCKS_PER_CU;
  const int64_t grid = units < cap ? units : cap;
  void (*kernel)(Geom, XPlan, int32_t, const int64_t*, uint8_t*, int32_t*) =
      pack ? k_layer_exchange<true> : k_layer_exchange<false>;
  (void)hipGetLastError();  // the status read below must be this launch's own
  if (t.start)
    hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kXThreads), 0, stream, t.start, t.stop, 0, g, x, layer,
                          dev_idx, staging, err);
  else
    kernel<<<dim3((unsigned)grid), kXThreads, 0, stream>>>(g, x, layer, dev_idx, staging, err);
  return hipGetLastError();
}

}  // namespace hc
