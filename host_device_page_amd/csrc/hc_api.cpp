// C ABI of libhc.so: pool lifetime, the write-back planner, transfer orchestration
// on the copy stream, the layer-done event chain and measurement hooks.
//
// Write-back (hybrid-pool write-back page, sglang PR 28434 summary): the host
// index list stays on the CPU, as in the controller change that keeps host
// indices CPU-side; the CPU validates it once per burst and uploads a compact
// plan.  Zero-copy mode then runs one kernel over all tokens, layers and
// sub-buffers that writes straight into the pinned host pool.  Staged mode
// gathers chunks of wholly named host pages, sorted by host page, into the device
// staging buffer in their host byte order (one launch per chunk, all layers) and
// moves each run of adjacent pages with one copy-engine transfer; tokens of
// partially named pages go through the zero-copy kernel so rows the list does not
// name are never overwritten.
//
// Load-back (loader-thread page, sglang PR 38472, Motivation): one kernel per
// layer reads device-resident index lists, so the CPU builds no per-layer
// descriptor; the layer-done event is recorded right after it, and recorded even
// when the call fails so that a consumer waiting on it cannot hang (the same
// page, Modifications: loader failure still completes every layer event).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "hc_internal.h"
#include "hc_plan.h"

using hc::Geom;
using hc::Layout;

namespace {

thread_local std::string g_err;

int vset_err(int code, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof(buf), fmt, ap);
  g_err = buf;
  return code;
}

int set_err(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vset_err(code, fmt, ap);
  va_end(ap);
  return code;
}

#define HIP_TRY(call)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) return set_err(HC_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

constexpr int kKinds = 8;  // gather, zc write, zc read, pads, compare, copy engine, pack, unpack
// Zero-copy kernels wait on the host link, not on the CU: 8-16 workgroups already
// saturate it (measured 55 GB/s from 8 up to 1024), and every extra workgroup holds
// a slot on a CU that the forward pass could use.  With 16, a bf16 GEMM consumer on
// another stream overlaps 74 % of the per-layer load-back; with 256, 8 %.
constexpr int32_t kDefaultMaxCtas = 16;
// Staging chunks are capped at the MI355X Infinity Cache size (256 MB): the gather
// writes a chunk and the copy engines read it back right away, so a chunk that
// fits stays cache-resident between the two (measured: 32 x 8 MiB page images
// gather at 5.9 TB/s, 64 at 5.4 TB/s, 128 at 5.1 TB/s).
constexpr int64_t kStagingChunkTarget = (int64_t)256 << 20;
// Which engine runs a hipMemcpyAsync is the runtime's choice.  In rocprofv3 kernel +
// memory-copy traces on MI355X its device-to-host copies ran as copy kernels on the CUs on a
// stream whose last host-to-device copy was 16 KiB or smaller (or absent), and on the copy
// engines right after one of 64 KiB or more, a kernel in between or not; that is not the
// whole rule (a few small bursts still got copy kernels after a large upload).  A staged
// burst's plan upload is that copy, so it is padded to at least this size: unpadded, every
// region copy of a 512-token burst (a 14 KB plan) ran on the CUs; padded, most went to the
// copy engines, and every one of the 78-layer bursts (a ~2 MB plan) did either way.
constexpr int64_t kCopyEngineUploadBytes = (int64_t)256 << 10;

struct PlanBuf {
  uint8_t* h = nullptr;   // pinned
  uint8_t* d = nullptr;   // device
  int64_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};

struct TimedLaunch {
  int kind;
  hipEvent_t a, b;
};

}  // namespace

struct hc_pool {
  // Serializes the pool's entry points: a loader thread and the caller may use one
  // pool at the same time.  Recursive because hc_round_trip_check calls hc_pool_sync.
  std::recursive_mutex mu;
  std::atomic<int64_t> users{0};  // loaders and captured graphs that hold this pool
  Layout lay;
  Geom geom;
  int device = 0;
  hipStream_t stream = nullptr;
  int32_t wb_mode = HC_MODE_ZEROCOPY;
  int32_t lb_mode = HC_MODE_ZEROCOPY;
  int32_t flags = 0;
  int32_t max_ctas = kDefaultMaxCtas;
  bool capturing = false;       // hc_load_back_graph_create is recording this pool's stream
  int32_t num_cus = 0;          // compute units of the pool's device
  uint8_t* host = nullptr;      // host pool (host address == device address on ROCm)
  uint8_t* staging = nullptr;
  int64_t staging_bytes = 0;
  int64_t chunk_pages = 0;
  uint64_t* d_tables = nullptr; // [nsub][L] layer addresses
  int32_t* d_err = nullptr;
  unsigned long long* d_counter = nullptr;
  unsigned long long* h_counter = nullptr;  // pinned
  int32_t* h_err = nullptr;                 // pinned
  hc::Planner planner;  // write-back plan, once per burst on the CPU
  PlanBuf plan[2];
  int plan_cur = 0;
  // measurement
  std::vector<hipEvent_t> free_events;
  std::vector<TimedLaunch> pending_timed;
  int64_t kind_launches[kKinds] = {};
  double kind_ms[kKinds] = {};
  hc_pool_stats stats{};
  std::vector<int64_t> wg_load;       // [max_ctas] host scratch of the zero-copy launchers' tile sizing
  int64_t row_bytes_per_layer = 0;    // sum of token-row sub-buffers' elem_bytes
  int64_t block_bytes_per_layer = 0;  // sum of page-block sub-buffers' elem_bytes
};

namespace {

// Device memory of the pool's device (the kernels run there and take these addresses).
int check_device_ptr(const void* p, int device, const char* what) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_err(HC_ERR_INVALID, "%s is not memory known to HIP", what);
  }
  if (attr.type != hipMemoryTypeDevice)
    return set_err(HC_ERR_INVALID, "%s must be device memory", what);
  if (attr.device != device)
    return set_err(HC_ERR_INVALID, "%s is on device %d, the pool's (current) device is %d", what, attr.device, device);
  return HC_OK;
}

// An index list the kernels read: memory the pool's device can address (its device
// memory, or pinned host memory mapped at the same address) that holds n int64 entries
// inside one allocation.  Pageable host memory would fault the kernel, and a list
// shorter than n would be read past its end, so both are refused before any launch.
int check_device_list(const hc_pool* p, const int64_t* q, int64_t n, const char* what) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, q) != hipSuccess) {
    (void)hipGetLastError();
    return set_err(HC_ERR_INVALID, "%s is not memory known to HIP", what);
  }
  if (attr.type == hipMemoryTypeDevice) {
    if (attr.device != p->device)
      return set_err(HC_ERR_INVALID, "%s is on device %d, the pool's device is %d", what, attr.device, p->device);
  } else if (attr.type == hipMemoryTypeHost) {
    if (attr.devicePointer != (const void*)q)
      return set_err(HC_ERR_INVALID, "%s: pinned host memory not mapped at its host address", what);
  } else {
    return set_err(HC_ERR_INVALID,
                   "%s must be device memory (or pinned host memory): the kernels read it, and pageable host "
                   "memory would fault them",
                   what);
  }
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)q) != hipSuccess || !base) {
    (void)hipGetLastError();
    return set_err(HC_ERR_INVALID, "%s: its allocation could not be found", what);
  }
  const uint64_t end = (uint64_t)(uintptr_t)base + (uint64_t)size;
  const uint64_t need = (uint64_t)(uintptr_t)q + (uint64_t)n * sizeof(int64_t);
  if (need > end)
    return set_err(HC_ERR_INVALID, "%s holds fewer than n = %lld int64 entries (its allocation ends %llu bytes in)",
                   what, (long long)n, (unsigned long long)(end - (uint64_t)(uintptr_t)q));
  return HC_OK;
}

// [q, q + bytes) lies inside one allocation known to HIP.  `required`: an allocation
// that cannot be looked up is an error (else the extent is left unchecked).
int check_extent(const void* q, int64_t bytes, bool required, const char* what) {
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)q) != hipSuccess || !base) {
    (void)hipGetLastError();
    return required ? set_err(HC_ERR_INVALID, "%s: its allocation could not be found", what) : HC_OK;
  }
  const uint64_t end = (uint64_t)(uintptr_t)base + (uint64_t)size;
  if ((uint64_t)(uintptr_t)q + (uint64_t)bytes > end)
    return set_err(HC_ERR_INVALID, "%s: %lld bytes are needed, its allocation ends %llu bytes after it", what,
                   (long long)bytes, (unsigned long long)(end - (uint64_t)(uintptr_t)q));
  return HC_OK;
}

// A list in pinned host memory, mapped at its host address, holding n int64 entries inside
// its allocation: the CPU reads it and the copy engines copy it without staging.
int check_pinned_list(const int64_t* q, int64_t n, const char* what) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, q) != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return set_err(HC_ERR_INVALID, "%s must be pinned host memory (hc_host_alloc or hipHostMalloc)", what);
  }
  if (attr.devicePointer != (const void*)q)
    return set_err(HC_ERR_INVALID, "%s: pinned host memory not mapped at its host address", what);
  return check_extent(q, n * (int64_t)sizeof(int64_t), true, what);
}

// The write-back's host list is read by the CPU: device memory would crash it.
int check_host_list(const int64_t* q, const char* what) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, q) != hipSuccess) {
    (void)hipGetLastError();
    return HC_OK;  // not known to HIP: ordinary host memory
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeArray)
    return set_err(HC_ERR_INVALID, "%s must be in host memory: the CPU plans the write-back from it", what);
  return HC_OK;
}

// A roctx range over one entry point's enqueue, so a trace shows each burst and layer
// call next to the kernels and copies it launched (a no-op without a profiler).
struct TraceRange {
  explicit TraceRange(const char* name) { roctxRangePushA(name); }
  ~TraceRange() { roctxRangePop(); }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

// Host-link bytes of n named tokens in one layer: every token row, plus one block per
// page for page-block sub-buffers (their lists name whole pages).
int64_t layer_bytes(const hc_pool* p, int64_t n);

int use_device(hc_pool* p) {
  int cur = -1;
  HIP_TRY(hipGetDevice(&cur));
  if (cur != p->device) HIP_TRY(hipSetDevice(p->device));
  return HC_OK;
}

hipEvent_t take_event(hc_pool* p) {
  if (!p->free_events.empty()) {
    hipEvent_t e = p->free_events.back();
    p->free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Times one launch (or, for copy-engine work, one span of the stream) when the pool
// profiles.  Kernels get the events through hc::LaunchTimer and stamp them with their
// own start and end; copy-engine spans record them on the stream around the copies.
struct Timer {
  hc_pool* p;
  int kind;
  hc::LaunchTimer ev;
  // enabled = false: no timing for this launch (a launch recorded into a graph, whose
  // launch-stamped events and harvesting synchronizations would break the capture)
  Timer(hc_pool* pool, int k, bool enabled = true) : p(pool), kind(k) {
    if (enabled && (p->flags & HC_FLAG_PROFILE)) {
      ev.start = take_event(p);
      ev.stop = ev.start ? take_event(p) : nullptr;
      if (!ev.stop) {
        if (ev.start) p->free_events.push_back(ev.start);
        ev.start = nullptr;
      }
    }
  }
  void record_start() {
    if (ev.start) (void)hipEventRecord(ev.start, p->stream);
  }
  void record_stop() {
    if (ev.stop) (void)hipEventRecord(ev.stop, p->stream);
  }
  // launched: the work the events bracket was enqueued (else the events go back unused)
  void done(bool launched);
};

int harvest_timing(hc_pool* p) {
  if (p->pending_timed.empty()) return HC_OK;
  HIP_TRY(hipStreamSynchronize(p->stream));
  for (auto& t : p->pending_timed) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, t.a, t.b) == hipSuccess) {
      p->kind_launches[t.kind] += 1;
      p->kind_ms[t.kind] += ms;
    } else {
      (void)hipGetLastError();  // an unusable pair is skipped, not left as the thread's last error
    }
    p->free_events.push_back(t.a);
    p->free_events.push_back(t.b);
  }
  p->pending_timed.clear();
  return HC_OK;
}

// Timed launches are folded into the totals once this many are pending, so a pool
// that profiles for a long time keeps a bounded number of events.
constexpr size_t kMaxPendingTimed = 4096;

void Timer::done(bool launched) {
  if (!ev.start) return;
  if (launched) {
    p->pending_timed.push_back({kind, ev.start, ev.stop});
  } else {
    p->free_events.push_back(ev.start);
    p->free_events.push_back(ev.stop);
  }
  ev = hc::LaunchTimer{};
  if (p->pending_timed.size() >= kMaxPendingTimed) (void)harvest_timing(p);
}

uint64_t magic_for(uint32_t vecs) {
  // ceil(2^40 / vecs)
  const uint64_t one = (uint64_t)1 << 40;
  return (one + vecs - 1) / vecs;
}

void fill_geom(hc_pool* p) {
  const Layout& L = p->lay;
  Geom& g = p->geom;
  memset(&g, 0, sizeof(g));
  g.nsub = L.nsub;
  g.L = L.L;
  g.P = L.P;
  g.validate = (p->flags & HC_FLAG_VALIDATE) ? 1 : 0;
  g.S = L.S;
  g.host_tokens = L.H * L.P;
  g.img_bytes = L.stride;
  g.payload_bytes = L.payload;
  g.pad_bytes = L.stride - L.payload;
  for (int b = 0; b < L.nsub; b++) {
    hc::SubGeom& s = g.sub[b];
    s.layers = p->d_tables + (size_t)b * L.L;
    s.elem = L.elem[b];
    s.vecs = (uint32_t)(L.elem[b] / 16);
    s.gran = L.gran[b];
    s.vec_magic = magic_for(s.vecs);
    s.host_region = L.host_region[b];
    s.host_page_stride = L.host_page_stride[b];
    s.layer_stride = L.layer_stride[b];
    s.row_stride = L.row_stride[b];
    s.img_off = hc::staging_sub_base(L, b, p->chunk_pages);
    s.stg_slot = hc::staging_slot_stride(L, b);
  }
}

// Makes plan buffer `cur` hold at least `bytes` (pinned + device), waiting for its
// previous upload to finish before the CPU rewrites it.
int plan_reserve(hc_pool* p, int64_t bytes) {
  PlanBuf& pb = p->plan[p->plan_cur];
  if (pb.pending) {
    HIP_TRY(hipEventSynchronize(pb.ev));
    pb.pending = false;
  }
  if (pb.cap >= bytes) return HC_OK;
  // the device copy may still be read by queued kernels: drain before freeing
  HIP_TRY(hipStreamSynchronize(p->stream));
  if (pb.h) HIP_TRY(hipHostFree(pb.h));
  if (pb.d) HIP_TRY(hipFree(pb.d));
  pb.h = nullptr;
  pb.d = nullptr;
  pb.cap = 0;
  int64_t cap = std::max<int64_t>(bytes, 1 << 16);
  cap = (cap + 4095) / 4096 * 4096;
  HIP_TRY(hipHostMalloc((void**)&pb.h, (size_t)cap, hipHostMallocDefault));
  HIP_TRY(hipMalloc((void**)&pb.d, (size_t)cap));
  if (!pb.ev) HIP_TRY(hipEventCreateWithFlags(&pb.ev, hipEventDisableTiming));
  pb.cap = cap;
  return HC_OK;
}

int plan_upload(hc_pool* p, int64_t bytes) {
  PlanBuf& pb = p->plan[p->plan_cur];
  if (bytes > 0) {
    HIP_TRY(hipMemcpyAsync(pb.d, pb.h, (size_t)bytes, hipMemcpyHostToDevice, p->stream));
    HIP_TRY(hipEventRecord(pb.ev, p->stream));
    pb.pending = true;
  }
  return HC_OK;
}

inline int64_t align16(int64_t x) { return (x + 15) / 16 * 16; }

// Whether the pool's stream is recording a graph: the library's own capture of a load-back
// burst, or a caller's capture around library calls.
bool stream_capturing(const hc_pool* p) {
  if (p->capturing) return true;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(p->stream, &st) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return st != hipStreamCaptureStatusNone;
}

int refuse_capture(const char* what, const char* why) {
  return set_err(HC_ERR_UNSUPPORTED, "%s cannot run while the pool's stream is capturing a graph: %s", what, why);
}

int no_host_pool() {
  return set_err(HC_ERR_INVALID,
                 "the pool has no host pages (a device-only pool): only the layer exchange and the round-trip "
                 "check run on it");
}

int record_event(void* ev, hipStream_t s) {
  if (!ev) return HC_OK;
  hipError_t e = hipEventRecord((hipEvent_t)ev, s);
  if (e != hipSuccess) return set_err(HC_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
  return HC_OK;
}

}  // namespace

extern "C" {

int hc_version(void) { return 1; }

const char* hc_last_error(void) { return g_err.c_str(); }

int hc_desc_check(const hc_pool_desc* desc) {
  Layout L;
  char msg[256];
  int rc = hc::layout_from_desc(desc, &L, msg, sizeof(msg));
  if (rc != HC_OK) return set_err(rc, "%s", msg);
  if (desc->write_back_mode < HC_MODE_AUTO || desc->write_back_mode > HC_MODE_ZEROCOPY ||
      desc->load_back_mode < HC_MODE_AUTO || desc->load_back_mode > HC_MODE_ZEROCOPY)
    return set_err(HC_ERR_INVALID, "unknown transfer mode");
  if (desc->load_back_mode == HC_MODE_STAGED)
    return set_err(HC_ERR_UNSUPPORTED,
                   "staged load-back is not provided: per-(page, layer) copy-engine transfers run far below "
                   "the host-link rate, the zero-copy kernel does not");
  if (desc->flags & ~(HC_FLAG_VALIDATE | HC_FLAG_PROFILE)) return set_err(HC_ERR_INVALID, "unknown flags");
  if (desc->max_ctas < 0 || desc->max_ctas > 65536) return set_err(HC_ERR_INVALID, "max_ctas must be in [0, 65536]");
  if (L.H == 0) {
    // a device-only pool: the layer exchange and the round-trip check, no host transfers
    if (desc->host_base) return set_err(HC_ERR_INVALID, "a pool without host pages takes no host_base");
    if (desc->write_back_mode == HC_MODE_STAGED || desc->staging)
      return set_err(HC_ERR_INVALID, "a pool without host pages has no write-back: no staging, no HC_MODE_STAGED");
  } else {
    if (!desc->host_base) return set_err(HC_ERR_INVALID, "host_base is null");
    if (((uintptr_t)desc->host_base) % 16 != 0)
      return set_err(HC_ERR_UNSUPPORTED, "host_base must be 16-byte aligned");
    if (desc->host_bytes < L.host_bytes)
      return set_err(HC_ERR_INVALID, "host_bytes %lld below the layout's %lld", (long long)desc->host_bytes,
                     (long long)L.host_bytes);
  }
  for (int b = 0; b < L.nsub; b++) {
    if (!desc->sub[b].device_layers) return set_err(HC_ERR_INVALID, "sub-buffer %d: device_layers is null", b);
    for (int l = 0; l < L.L; l++) {
      const void* q = desc->sub[b].device_layers[l];
      if (!q) return set_err(HC_ERR_INVALID, "sub-buffer %d layer %d: null device pointer", b, l);
      if (((uintptr_t)q) % 16 != 0)
        return set_err(HC_ERR_UNSUPPORTED, "sub-buffer %d layer %d: device pointer not 16-byte aligned", b, l);
    }
  }
  if (desc->write_back_mode == HC_MODE_STAGED) {
    if (!desc->staging) return set_err(HC_ERR_INVALID, "staged write-back needs a staging buffer");
    if (((uintptr_t)desc->staging) % 16 != 0) return set_err(HC_ERR_UNSUPPORTED, "staging must be 16-byte aligned");
    if (desc->staging_bytes < L.stride)
      return set_err(HC_ERR_INVALID, "staging_bytes %lld below one page image (%lld bytes)",
                     (long long)desc->staging_bytes, (long long)L.stride);
  }
  return HC_OK;
}

int hc_host_pool_bytes(const hc_pool_desc* desc, int64_t* out_bytes) {
  if (!out_bytes) return set_err(HC_ERR_INVALID, "out_bytes is null");
  Layout L;
  char msg[256];
  int rc = hc::layout_from_desc(desc, &L, msg, sizeof(msg));
  if (rc != HC_OK) return set_err(rc, "%s", msg);
  *out_bytes = L.host_bytes;
  return HC_OK;
}

int hc_staging_page_bytes(const hc_pool_desc* desc, int64_t* out_bytes) {
  if (!out_bytes) return set_err(HC_ERR_INVALID, "out_bytes is null");
  Layout L;
  char msg[256];
  int rc = hc::layout_from_desc(desc, &L, msg, sizeof(msg));
  if (rc != HC_OK) return set_err(rc, "%s", msg);
  *out_bytes = L.stride;
  return HC_OK;
}

int hc_host_offset(const hc_pool_desc* desc, int32_t sub, int64_t page, int32_t layer, int32_t row,
                   int64_t* out_offset) {
  if (!out_offset) return set_err(HC_ERR_INVALID, "out_offset is null");
  Layout L;
  char msg[256];
  int rc = hc::layout_from_desc(desc, &L, msg, sizeof(msg));
  if (rc != HC_OK) return set_err(rc, "%s", msg);
  if (sub < 0 || sub >= L.nsub || page < 0 || page >= L.H || layer < 0 || layer >= L.L || row < 0 || row >= L.P)
    return set_err(HC_ERR_INVALID, "coordinate out of range");
  *out_offset = hc::layout_host_offset(L, sub, page, layer, row);
  return HC_OK;
}

int hc_host_alloc(int64_t bytes, int32_t flags, void** out) {
  if (!out || bytes <= 0) return set_err(HC_ERR_INVALID, "hc_host_alloc: bad size or null out");
  if (flags != 0 && flags != 1) return set_err(HC_ERR_INVALID, "hc_host_alloc: flags must be 0 or 1");
  void* p = nullptr;
  const unsigned hf = hipHostMallocMapped | (flags ? hipHostMallocNonCoherent : hipHostMallocCoherent);
  HIP_TRY(hipHostMalloc(&p, (size_t)bytes, hf));
  // zero through the device mapping (the host link is faster than CPU first touch)
  hipError_t e = hipMemset(p, 0, (size_t)bytes);
  if (e != hipSuccess) {
    (void)hipHostFree(p);
    return set_err(HC_ERR_HIP, "hipMemset of pinned memory failed: %s", hipGetErrorString(e));
  }
  *out = p;
  return HC_OK;
}

int hc_host_free(void* ptr) {
  if (!ptr) return HC_OK;
  HIP_TRY(hipHostFree(ptr));
  return HC_OK;
}

int hc_pool_create(const hc_pool_desc* desc, hc_pool** out) {
  if (!out) return set_err(HC_ERR_INVALID, "out is null");
  *out = nullptr;
  int rc = hc_desc_check(desc);
  if (rc != HC_OK) return rc;
  {
    // set-up copies the layer tables on the copy stream and waits for it: not inside a capture
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing((hipStream_t)desc->copy_stream, &st) != hipSuccess) {
      (void)hipGetLastError();  // an invalid stream is reported below
    } else if (st != hipStreamCaptureStatusNone) {
      return refuse_capture("hc_pool_create", "its set-up copies to the device and waits for the copy stream");
    }
  }
  hc_pool* p = new (std::nothrow) hc_pool();
  if (!p) return set_err(HC_ERR_NOMEM, "pool allocation failed");
  char msg[256];
  hc::layout_from_desc(desc, &p->lay, msg, sizeof(msg));
  const Layout& L = p->lay;
  auto bail = [&](int code) {
    hc_pool_destroy(p);
    return code;
  };
  if (hipGetDevice(&p->device) != hipSuccess) return bail(set_err(HC_ERR_HIP, "no HIP device"));
  if (hipDeviceGetAttribute(&p->num_cus, hipDeviceAttributeMultiprocessorCount, p->device) != hipSuccess)
    return bail(set_err(HC_ERR_HIP, "could not query the compute-unit count"));
  {
    // Set-up of the no-allocation write-back: the first lookup of its scratch on a device
    // makes the runtime load the code object that holds the array (device memory, once per
    // process and device), so that happens here and not inside that call.  A failure is
    // reported by the no-allocation write-back itself.
    int64_t* scratch = nullptr;
    if (hc::noalloc_scratch(p->device, &scratch) != HC_OK) g_err.clear();
  }
  p->stream = (hipStream_t)desc->copy_stream;
  if (p->stream) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(p->stream, &sd) != hipSuccess) {
      (void)hipGetLastError();
      return bail(set_err(HC_ERR_INVALID, "copy_stream is not a valid stream"));
    }
    if (sd != p->device)
      return bail(set_err(HC_ERR_INVALID, "copy_stream belongs to device %d, the pool's (current) device is %d", sd,
                          p->device));
  }
  p->flags = desc->flags;
  p->max_ctas = desc->max_ctas > 0 ? desc->max_ctas : kDefaultMaxCtas;
  try {
    p->wg_load.assign((size_t)p->max_ctas, 0);
  } catch (...) {
    return bail(set_err(HC_ERR_NOMEM, "host scratch allocation failed"));
  }
  // memory kinds
  if (L.H > 0) {
    void* dptr = nullptr;
    if (hipHostGetDevicePointer(&dptr, desc->host_base, 0) != hipSuccess || !dptr) {
      (void)hipGetLastError();
      return bail(set_err(HC_ERR_INVALID, "host_base is not pinned (page-locked) host memory"));
    }
    p->host = (uint8_t*)dptr;
    // every buffer the kernels address must hold what the layout puts in it
    rc = check_extent(desc->host_base, L.host_bytes, false, "host_base");
    if (rc != HC_OK) return bail(rc);
  }
  for (int b = 0; b < L.nsub; b++) {
    const int64_t units = L.gran[b] == HC_PAGE_BLOCKS ? L.S / L.P : L.S;
    for (int l = 0; l < L.L; l++) {
      char what[64];
      snprintf(what, sizeof(what), "sub-buffer %d layer %d", b, l);
      rc = check_device_ptr(desc->sub[b].device_layers[l], p->device, what);
      if (rc == HC_OK) rc = check_extent(desc->sub[b].device_layers[l], units * L.elem[b], true, what);
      if (rc != HC_OK) return bail(rc);
    }
  }
  // modes.  AUTO write-back is staged whenever the caller brings staging for it: a
  // zero-copy write-back that saturates the host link slows compute on other streams
  // until it barely overlaps, staged write-back leaves that compute alone (measured).
  const bool auto_staged = desc->write_back_mode == HC_MODE_AUTO && desc->staging &&
                           desc->staging_bytes >= L.stride && ((uintptr_t)desc->staging) % 16 == 0;
  p->wb_mode = (desc->write_back_mode == HC_MODE_STAGED || auto_staged) ? HC_MODE_STAGED : HC_MODE_ZEROCOPY;
  p->lb_mode = HC_MODE_ZEROCOPY;
  if (p->wb_mode == HC_MODE_STAGED) {
    rc = check_device_ptr(desc->staging, p->device, "staging");
    if (rc != HC_OK) return bail(rc);
    p->staging = (uint8_t*)desc->staging;
    p->staging_bytes = desc->staging_bytes;
    p->chunk_pages = std::min<int64_t>(desc->staging_bytes / L.stride, (int64_t)1 << 20);
    p->chunk_pages = std::min<int64_t>(p->chunk_pages, std::max<int64_t>(1, kStagingChunkTarget / L.stride));
    if (p->chunk_pages * L.P >= ((int64_t)1 << 31)) p->chunk_pages = (((int64_t)1 << 31) - 1) / L.P;
    rc = check_extent(desc->staging, p->chunk_pages * L.stride, true, "staging");
    if (rc != HC_OK) return bail(rc);
  }
  // device tables and scratch
  std::vector<uint64_t> tables((size_t)L.nsub * L.L);
  for (int b = 0; b < L.nsub; b++)
    for (int l = 0; l < L.L; l++) tables[(size_t)b * L.L + l] = (uint64_t)(uintptr_t)desc->sub[b].device_layers[l];
  if (hipMalloc((void**)&p->d_tables, tables.size() * sizeof(uint64_t)) != hipSuccess)
    return bail(set_err(HC_ERR_HIP, "hipMalloc of layer tables failed"));
  if (hipMalloc((void**)&p->d_err, 64) != hipSuccess) return bail(set_err(HC_ERR_HIP, "hipMalloc failed"));
  p->d_counter = (unsigned long long*)((uint8_t*)p->d_err + 32);
  if (hipHostMalloc((void**)&p->h_counter, 64, hipHostMallocDefault) != hipSuccess)
    return bail(set_err(HC_ERR_HIP, "hipHostMalloc failed"));
  p->h_err = (int32_t*)((uint8_t*)p->h_counter + 32);
  // d_err: [0, 4) error bits, [8, 16) smallest flagged list position (none: all ones), [32, 40) counter
  if (hipMemcpyAsync(p->d_tables, tables.data(), tables.size() * sizeof(uint64_t), hipMemcpyHostToDevice,
                     p->stream) != hipSuccess ||
      hipMemsetAsync(p->d_err, 0, 64, p->stream) != hipSuccess ||
      hipMemsetAsync((uint8_t*)p->d_err + 8, 0xFF, 8, p->stream) != hipSuccess)
    return bail(set_err(HC_ERR_HIP, "initial copies failed"));
  if (hipStreamSynchronize(p->stream) != hipSuccess) return bail(set_err(HC_ERR_HIP, "stream sync failed"));
  p->planner.reset(L);
  fill_geom(p);
  for (int b = 0; b < L.nsub; b++)
    (L.gran[b] == HC_PAGE_BLOCKS ? p->block_bytes_per_layer : p->row_bytes_per_layer) += L.elem[b];
  *out = p;
  return HC_OK;
}

int hc_pool_destroy(hc_pool* p) {
  if (!p) return HC_OK;
  if (p->users.load() > 0)
    return set_err(HC_ERR_INVALID, "%lld loader(s) or captured graph(s) still use the pool; destroy them first",
                   (long long)p->users.load());
  if (p->d_tables && stream_capturing(p))
    return refuse_capture("hc_pool_destroy", "it waits for the copy stream before freeing (nothing was freed)");
  int rc = HC_OK;
  if (p->stream || p->d_tables) {
    if (hipStreamSynchronize(p->stream) != hipSuccess) rc = set_err(HC_ERR_HIP, "stream sync failed in destroy");
  }
  for (auto& pb : p->plan) {
    if (pb.h) (void)hipHostFree(pb.h);
    if (pb.d) (void)hipFree(pb.d);
    if (pb.ev) (void)hipEventDestroy(pb.ev);
  }
  for (auto& t : p->pending_timed) {
    (void)hipEventDestroy(t.a);
    (void)hipEventDestroy(t.b);
  }
  for (auto e : p->free_events) (void)hipEventDestroy(e);
  if (p->d_tables) (void)hipFree(p->d_tables);
  if (p->d_err) (void)hipFree(p->d_err);
  if (p->h_counter) (void)hipHostFree(p->h_counter);
  delete p;
  return rc;
}

int hc_pool_mode(const hc_pool* p, int32_t which, int32_t* out_mode) {
  if (!p || !out_mode) return set_err(HC_ERR_INVALID, "null argument");
  if (which == 0) *out_mode = p->wb_mode;
  else if (which == 1) *out_mode = p->lb_mode;
  else return set_err(HC_ERR_INVALID, "which must be 0 (write-back) or 1 (load-back)");
  return HC_OK;
}

int hc_pool_sync(hc_pool* p) {
  if (!p) return set_err(HC_ERR_INVALID, "pool is null");
  std::lock_guard<std::recursive_mutex> lock(p->mu);
  int rc = use_device(p);
  if (rc != HC_OK) return rc;
  if (stream_capturing(p)) return refuse_capture("hc_pool_sync", "it waits for the stream");
  HIP_TRY(hipMemcpyAsync(p->h_err, p->d_err, 16, hipMemcpyDeviceToHost, p->stream));
  HIP_TRY(hipStreamSynchronize(p->stream));
  const int32_t e = *p->h_err;
  if (e) {
    uint64_t pos = 0;
    memcpy(&pos, (const uint8_t*)p->h_err + 8, sizeof(pos));
    HIP_TRY(hipMemsetAsync(p->d_err, 0, sizeof(int32_t), p->stream));
    HIP_TRY(hipMemsetAsync((uint8_t*)p->d_err + 8, 0xFF, 8, p->stream));
    HIP_TRY(hipStreamSynchronize(p->stream));
    p->stats.device_errors++;
    return set_err(HC_ERR_DEVICE,
                   "device-side check flagged an index list (code %d:%s%s first flagged list position %llu)", e,
                   (e & 1) ? " index out of range;" : "",
                   (e & 2) ? " page-block rows not one whole device page;" : "", (unsigned long long)pos);
  }
  return HC_OK;
}

int hc_write_back_all_layers(hc_pool* p, const int64_t* device_idx, const int64_t* host_idx, int64_t n,
                             void* event) {
  if (!p) return set_err(HC_ERR_INVALID, "pool is null");
  TraceRange range("hc_write_back_all_layers");
  std::lock_guard<std::recursive_mutex> lock(p->mu);
  int rc = use_device(p);
  if (rc != HC_OK) return rc;
  auto finish = [&](int code) {
    int r2 = record_event(event, p->stream);
    return code != HC_OK ? code : r2;
  };
  if (p->lay.H == 0) return finish(no_host_pool());
  if (stream_capturing(p))
    return finish(refuse_capture("hc_write_back_all_layers",
                                 "its plan is built on the CPU for each call, so a replay would reuse a stale "
                                 "plan"));
  if (n < 0) return finish(set_err(HC_ERR_INVALID, "n must be >= 0"));
  if (n == 0) return finish(HC_OK);
  if (!device_idx || !host_idx) return finish(set_err(HC_ERR_INVALID, "null index list"));
  if (n >= ((int64_t)1 << 31)) return finish(set_err(HC_ERR_INVALID, "n must be below 2^31"));
  rc = check_device_list(p, device_idx, n, "device_idx");
  if (rc == HC_OK) rc = check_host_list(host_idx, "host_idx");
  if (rc != HC_OK) return finish(rc);
  {
    char msg[256];
    rc = p->planner.validate(host_idx, n, msg, sizeof(msg));
    if (rc != HC_OK) return finish(set_err(rc, "%s", msg));
  }
  const Layout& L = p->lay;
  const bool staged = p->wb_mode == HC_MODE_STAGED;
  // plan buffer layout: hidx int64[n] | pads int64[n] | srow int32[n] | ztok int32[n] | perm int32[n]
  const int64_t o_hidx = 0;
  const int64_t o_pads = align16(o_hidx + 8 * n);
  const int64_t o_srow = align16(o_pads + 8 * n);
  const int64_t o_ztok = align16(o_srow + 4 * n);
  const int64_t o_perm = align16(o_ztok + 4 * n);
  const int64_t bytes = align16(o_perm + 4 * n);
  rc = plan_reserve(p, staged ? std::max(bytes, kCopyEngineUploadBytes) : bytes);
  if (rc != HC_OK) return finish(rc);
  PlanBuf& pb = p->plan[p->plan_cur];
  int64_t* hidx = (int64_t*)(pb.h + o_hidx);
  int64_t* pads = (int64_t*)(pb.h + o_pads);
  int32_t* srow = (int32_t*)(pb.h + o_srow);
  int32_t* ztok = (int32_t*)(pb.h + o_ztok);
  int32_t* perm = (int32_t*)(pb.h + o_perm);
  memcpy(hidx, host_idx, (size_t)(8 * n));
  int64_t nz = 0, npads = 0;
  if (staged) {
    p->planner.plan_staged(host_idx, n, p->chunk_pages, p->host, p->staging, perm, srow, ztok, &nz, pads, &npads);
  } else if (L.layout == HC_LAYOUT_KV_SPLIT_SHARD && L.stride > L.payload) {
    npads = p->planner.distinct_pages(host_idx, n, pads);
  }
  // staged: padded so the region copies below go to the copy engines (the padding is not read)
  const int64_t upload = staged ? std::max(bytes, kCopyEngineUploadBytes) : align16(o_pads + 8 * npads);
  rc = plan_upload(p, upload);
  if (rc != HC_OK) return finish(rc);
  const int64_t* d_hidx = (const int64_t*)(pb.d + o_hidx);
  const int64_t* d_pads = (const int64_t*)(pb.d + o_pads);
  const int32_t* d_srow = (const int32_t*)(pb.d + o_srow);
  const int32_t* d_ztok = (const int32_t*)(pb.d + o_ztok);
  const int32_t* d_perm = (const int32_t*)(pb.d + o_perm);
  p->plan_cur ^= 1;
  hipError_t e = hipSuccess;
  if (staged) {
    if (L.stride > L.payload && !p->planner.regions.empty()) {
      // Staging page images carry the shard's zero pad, and a whole page leaves staging with
      // it.  The gathers never write the pad, but another pool may have used this staging
      // buffer since the last burst, so the pads of the images this burst fills are cleared.
      // (untimed: a launch-stamped kernel ahead of the region copies turned them into blit kernels)
      e = hc::launch_zero_pads(p->staging, nullptr, p->planner.max_chunk_slots(), L.stride, L.payload,
                               L.stride - L.payload, hc::LaunchTimer{}, p->stream);
      if (e != hipSuccess) return finish(set_err(HC_ERR_HIP, "staging pad launch failed: %s", hipGetErrorString(e)));
    }
    for (const hc::Chunk& c : p->planner.chunks) {
      {
        // Recorded events, not launch-stamped ones: right after a launch-stamped kernel the
        // runtime ran the region copies below as blit kernels on the CUs instead of on the
        // copy engines (measured), which would take away the staged mode's point.
        Timer t(p, 0);
        t.record_start();
        e = hc::launch_gather_stage(p->geom, device_idx, d_hidx, d_perm, d_srow, c.t0, c.t1 - c.t0, p->staging,
                                    p->d_err, p->num_cus, hc::LaunchTimer{}, p->stream);
        t.record_stop();
        t.done(e == hipSuccess);
      }
      if (e != hipSuccess) return finish(set_err(HC_ERR_HIP, "gather launch failed: %s", hipGetErrorString(e)));
      if (c.r1 > c.r0) {
        Timer t(p, 5);
        t.record_start();
        for (size_t r = c.r0; r < c.r1 && e == hipSuccess; r++) {
          const hc::Region& g = p->planner.regions[r];
          e = hipMemcpyAsync(g.dst, g.src, (size_t)g.len, hipMemcpyDeviceToHost, p->stream);
        }
        t.record_stop();
        t.done(true);
        if (e != hipSuccess) return finish(set_err(HC_ERR_HIP, "hipMemcpyAsync failed: %s", hipGetErrorString(e)));
      }
    }
    if (nz > 0) {
      Timer t(p, 1);
      e = hc::launch_zc_write(p->geom, device_idx, d_hidx, d_ztok, nz, p->host, p->d_err, p->max_ctas,
                              p->wg_load.data(), t.ev, p->stream);
      t.done(e == hipSuccess);
      if (e != hipSuccess) return finish(set_err(HC_ERR_HIP, "zero-copy launch failed: %s", hipGetErrorString(e)));
    }
  } else {
    Timer t(p, 1);
    e = hc::launch_zc_write(p->geom, device_idx, d_hidx, nullptr, n, p->host, p->d_err, p->max_ctas,
                            p->wg_load.data(), t.ev, p->stream);
    t.done(e == hipSuccess);
    if (e != hipSuccess) return finish(set_err(HC_ERR_HIP, "zero-copy launch failed: %s", hipGetErrorString(e)));
  }
  if (npads > 0) {
    Timer t(p, 3);
    e = hc::launch_zero_pads(p->host, d_pads, npads, L.stride, L.payload, L.stride - L.payload, t.ev, p->stream);
    t.done(e == hipSuccess);
    if (e != hipSuccess) return finish(set_err(HC_ERR_HIP, "pad launch failed: %s", hipGetErrorString(e)));
  }
  p->stats.write_back_calls++;
  p->stats.write_back_tokens += n;
  p->stats.write_back_bytes += layer_bytes(p, n) * L.L;
  return finish(HC_OK);
}

int hc_write_back_all_layers_noalloc(hc_pool* p, const int64_t* device_idx, const int64_t* host_idx, int64_t n,
                                     void* event) {
  if (!p) return set_err(HC_ERR_INVALID, "pool is null");
  TraceRange range("hc_write_back_all_layers_noalloc");
  std::lock_guard<std::recursive_mutex> lock(p->mu);
  int rc = use_device(p);
  if (rc != HC_OK) return rc;
  auto finish = [&](int code) {
    int r2 = record_event(event, p->stream);
    return code != HC_OK ? code : r2;
  };
  if (p->lay.H == 0) return finish(no_host_pool());
  if (p->wb_mode != HC_MODE_ZEROCOPY)
    return finish(set_err(HC_ERR_UNSUPPORTED,
                          "the write-back without allocation runs on zero-copy pools only (this pool stages its "
                          "write-back)"));
  if (stream_capturing(p))
    return finish(refuse_capture("hc_write_back_all_layers_noalloc",
                                 "it checks the host list on the CPU for each call"));
  if (n < 0) return finish(set_err(HC_ERR_INVALID, "n must be >= 0"));
  if (n == 0) return finish(HC_OK);
  if (!device_idx || !host_idx) return finish(set_err(HC_ERR_INVALID, "null index list"));
  if (n > HC_NOALLOC_MAX_TOKENS)
    return finish(set_err(HC_ERR_INVALID, "n = %lld is above the %d tokens the write-back without allocation holds",
                          (long long)n, HC_NOALLOC_MAX_TOKENS));
  rc = check_device_list(p, device_idx, n, "device_idx");
  if (rc == HC_OK) rc = check_pinned_list(host_idx, n, "host_idx");
  if (rc != HC_OK) return finish(rc);
  {
    char msg[256];
    rc = p->planner.validate(host_idx, n, msg, sizeof(msg));
    if (rc != HC_OK) return finish(set_err(rc, "%s", msg));
  }
  int64_t* scratch = nullptr;
  rc = hc::noalloc_scratch(p->device, &scratch);
  if (rc != HC_OK) return finish(rc);
  const Layout& L = p->lay;
  hipError_t e = hipMemcpyAsync(scratch, host_idx, (size_t)n * sizeof(int64_t), hipMemcpyHostToDevice, p->stream);
  if (e != hipSuccess) return finish(set_err(HC_ERR_HIP, "host list copy failed: %s", hipGetErrorString(e)));
  e = hc::launch_zc_write(p->geom, device_idx, scratch, nullptr, n, p->host, p->d_err, p->max_ctas,
                          p->wg_load.data(), hc::LaunchTimer{}, p->stream);
  if (e != hipSuccess) return finish(set_err(HC_ERR_HIP, "zero-copy launch failed: %s", hipGetErrorString(e)));
  if (L.layout == HC_LAYOUT_KV_SPLIT_SHARD && L.stride > L.payload) {
    e = hc::launch_zero_pads_runs(p->host, scratch, n, L.P, L.H, L.stride, L.payload, L.stride - L.payload, p->stream);
    if (e != hipSuccess) return finish(set_err(HC_ERR_HIP, "pad launch failed: %s", hipGetErrorString(e)));
  }
  p->stats.write_back_calls++;
  p->stats.write_back_tokens += n;
  p->stats.write_back_bytes += layer_bytes(p, n) * L.L;
  return finish(HC_OK);
}

int hc_load_back_layer(hc_pool* p, int32_t layer, const int64_t* host_idx, const int64_t* device_idx, int64_t n,
                       void* event) {
  if (!p) {
    // still complete the layer event so a waiting consumer is released
    if (event) (void)hipEventRecord((hipEvent_t)event, nullptr);
    return set_err(HC_ERR_INVALID, "pool is null");
  }
  TraceRange range("hc_load_back_layer");
  std::lock_guard<std::recursive_mutex> lock(p->mu);
  int rc = use_device(p);
  auto finish = [&](int code) {
    int r2 = record_event(event, p->stream);
    return code != HC_OK ? code : r2;
  };
  if (rc != HC_OK) return finish(rc);
  if (p->lay.H == 0) return finish(no_host_pool());
  if (layer < 0 || layer >= p->lay.L)
    return finish(set_err(HC_ERR_INVALID, "layer %d out of range [0, %d)", layer, p->lay.L));
  if (n < 0) return finish(set_err(HC_ERR_INVALID, "n must be >= 0"));
  if (n == 0) return finish(HC_OK);
  if (!host_idx || !device_idx) return finish(set_err(HC_ERR_INVALID, "null index list"));
  if (p->lay.has_blocks && n % p->lay.P != 0)
    return finish(set_err(HC_ERR_INVALID, "page-block sub-buffers need whole pages (n %% page_size != 0)"));
  if (!p->capturing) {  // a capture checks its lists once, before it starts
    rc = check_device_list(p, host_idx, n, "host_idx");
    if (rc == HC_OK) rc = check_device_list(p, device_idx, n, "device_idx");
    if (rc != HC_OK) return finish(rc);
  }
  hipError_t e;
  {
    Timer t(p, 2, !stream_capturing(p));
    e = hc::launch_zc_read(p->geom, layer, host_idx, device_idx, n, p->host, p->d_err, p->max_ctas,
                           p->wg_load.data(), t.ev, p->stream);
    t.done(e == hipSuccess);
  }
  if (e != hipSuccess) return finish(set_err(HC_ERR_HIP, "load-back launch failed: %s", hipGetErrorString(e)));
  if (!p->capturing) {  // a captured call is counted when its graph replays
    p->stats.load_back_calls++;
    p->stats.load_back_tokens += n;
    p->stats.load_back_bytes += layer_bytes(p, n);
  }
  return finish(HC_OK);
}

int hc_round_trip_check(hc_pool* p, const int64_t* idx_a, const int64_t* idx_b, int64_t n,
                        int64_t* mismatched_units) {
  if (!p || !mismatched_units) return set_err(HC_ERR_INVALID, "null argument");
  std::lock_guard<std::recursive_mutex> lock(p->mu);
  int rc = use_device(p);
  if (rc != HC_OK) return rc;
  if (stream_capturing(p)) return refuse_capture("hc_round_trip_check", "it waits for the stream");
  if (n < 0) return set_err(HC_ERR_INVALID, "n must be >= 0");
  if (n > 0 && (!idx_a || !idx_b)) return set_err(HC_ERR_INVALID, "null index list");
  if (n > 0) {
    rc = check_device_list(p, idx_a, n, "idx_a");
    if (rc == HC_OK) rc = check_device_list(p, idx_b, n, "idx_b");
    if (rc != HC_OK) return rc;
  }
  HIP_TRY(hipMemsetAsync(p->d_counter, 0, sizeof(unsigned long long), p->stream));
  if (n > 0) {
    Timer t(p, 4);
    hipError_t e = hc::launch_compare(p->geom, idx_a, idx_b, n, p->d_counter, p->d_err, t.ev, p->stream);
    t.done(e == hipSuccess);
    if (e != hipSuccess) return set_err(HC_ERR_HIP, "compare launch failed: %s", hipGetErrorString(e));
  }
  HIP_TRY(hipMemcpyAsync(p->h_counter, p->d_counter, sizeof(unsigned long long), hipMemcpyDeviceToHost, p->stream));
  rc = hc_pool_sync(p);
  *mismatched_units = (int64_t)*p->h_counter;
  return rc;
}

int hc_layer_pack_bytes(const hc_pool* p, int64_t n, int64_t* out_bytes) {
  if (!p || !out_bytes) return set_err(HC_ERR_INVALID, "null argument");
  if (n < 0) return set_err(HC_ERR_INVALID, "n must be >= 0");
  if (p->lay.has_blocks && n % p->lay.P != 0)
    return set_err(HC_ERR_INVALID, "page-block sub-buffers need whole pages (n %% page_size != 0)");
  *out_bytes = layer_bytes(p, n);
  return HC_OK;
}

namespace {

// One side of the layer exchange; `staging` is dst (pack) or src (unpack).
int layer_exchange(hc_pool* p, bool pack, int32_t layer, const int64_t* device_idx, int64_t n, const void* staging,
                   int64_t staging_bytes, void* event) {
  std::lock_guard<std::recursive_mutex> lock(p->mu);
  int rc = use_device(p);
  auto finish = [&](int code) {
    int r2 = record_event(event, p->stream);
    return code != HC_OK ? code : r2;
  };
  if (rc != HC_OK) return finish(rc);
  if (layer < 0 || layer >= p->lay.L)
    return finish(set_err(HC_ERR_INVALID, "layer %d out of range [0, %d)", layer, p->lay.L));
  if (n < 0) return finish(set_err(HC_ERR_INVALID, "n must be >= 0"));
  if (n == 0) return finish(HC_OK);
  if (!device_idx || !staging) return finish(set_err(HC_ERR_INVALID, "null index list or staging buffer"));
  if (p->lay.has_blocks && n % p->lay.P != 0)
    return finish(set_err(HC_ERR_INVALID, "page-block sub-buffers need whole pages (n %% page_size != 0)"));
  const int64_t need = layer_bytes(p, n);
  if (staging_bytes < need)
    return finish(set_err(HC_ERR_INVALID, "staging_bytes %lld below the %lld bytes of %lld entries",
                          (long long)staging_bytes, (long long)need, (long long)n));
  if (((uintptr_t)staging) % 16 != 0) return finish(set_err(HC_ERR_UNSUPPORTED, "staging must be 16-byte aligned"));
  rc = check_device_list(p, device_idx, n, "device_idx");
  if (rc == HC_OK) rc = check_device_ptr(staging, p->device, "staging");
  if (rc == HC_OK) rc = check_extent(staging, need, true, "staging");
  if (rc != HC_OK) return finish(rc);
  hipError_t e;
  {
    Timer t(p, pack ? 6 : 7, !stream_capturing(p));
    e = hc::launch_layer_exchange(p->geom, pack, layer, device_idx, n, (uint8_t*)staging, p->d_err, p->num_cus,
                                  t.ev, p->stream);
    t.done(e == hipSuccess);
  }
  if (e != hipSuccess) return finish(set_err(HC_ERR_HIP, "exchange launch failed: %s", hipGetErrorString(e)));
  return finish(HC_OK);
}

}  // namespace

int hc_layer_pack(hc_pool* p, int32_t layer, const int64_t* device_idx, int64_t n, void* dst, int64_t dst_bytes,
                  void* event) {
  if (!p) {
    if (event) (void)hipEventRecord((hipEvent_t)event, nullptr);
    return set_err(HC_ERR_INVALID, "pool is null");
  }
  TraceRange range("hc_layer_pack");
  return layer_exchange(p, true, layer, device_idx, n, dst, dst_bytes, event);
}

int hc_layer_unpack(hc_pool* p, int32_t layer, const void* src, int64_t src_bytes, const int64_t* device_idx,
                    int64_t n, void* event) {
  if (!p) {
    if (event) (void)hipEventRecord((hipEvent_t)event, nullptr);
    return set_err(HC_ERR_INVALID, "pool is null");
  }
  TraceRange range("hc_layer_unpack");
  return layer_exchange(p, false, layer, device_idx, n, src, src_bytes, event);
}

}  // extern "C"

struct hc_lb_graph {
  hc_pool* pool = nullptr;
  bool held = false;  // counted in pool->users
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  std::vector<void*> events;  // the L layer events the replays record (NULL: none for that layer)
  int64_t n = 0;              // tokens per layer of every replay
};

extern "C" {

int hc_load_back_graph_destroy(hc_lb_graph* g) {
  if (!g) return HC_OK;
  int rc = HC_OK;
  if (g->exec && hipGraphExecDestroy(g->exec) != hipSuccess) rc = set_err(HC_ERR_HIP, "hipGraphExecDestroy failed");
  if (g->graph && hipGraphDestroy(g->graph) != hipSuccess) rc = set_err(HC_ERR_HIP, "hipGraphDestroy failed");
  if (g->held) hc::pool_release(g->pool);
  delete g;
  return rc;
}

int hc_load_back_graph_create(hc_pool* p, const int64_t* host_idx, const int64_t* device_idx, int64_t n,
                              void* const* layer_events, hc_lb_graph** out) {
  if (!out) return set_err(HC_ERR_INVALID, "out is null");
  *out = nullptr;
  if (!p || !layer_events) return set_err(HC_ERR_INVALID, "null argument");
  if (n < 0) return set_err(HC_ERR_INVALID, "n must be >= 0");
  if (n > 0 && (!host_idx || !device_idx)) return set_err(HC_ERR_INVALID, "null index list");
  std::lock_guard<std::recursive_mutex> lock(p->mu);
  if (p->lay.H == 0) return no_host_pool();
  if (p->flags & HC_FLAG_PROFILE)
    return set_err(HC_ERR_UNSUPPORTED, "a pool created with HC_FLAG_PROFILE cannot be captured");
  int rc = use_device(p);
  if (rc != HC_OK) return rc;
  hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
  HIP_TRY(hipStreamIsCapturing(p->stream, &status));
  if (status != hipStreamCaptureStatusNone) return set_err(HC_ERR_INVALID, "the pool's stream is already capturing");
  if (n > 0) {
    rc = check_device_list(p, host_idx, n, "host_idx");
    if (rc == HC_OK) rc = check_device_list(p, device_idx, n, "device_idx");
    if (rc != HC_OK) return rc;
  }
  hc_lb_graph* g = new (std::nothrow) hc_lb_graph();
  if (!g) return set_err(HC_ERR_NOMEM, "graph handle allocation failed");
  g->pool = p;
  g->n = n;
  try {
    g->events.assign(layer_events, layer_events + p->lay.L);
  } catch (...) {
    delete g;
    return set_err(HC_ERR_NOMEM, "graph handle allocation failed");
  }
  hipError_t e = hipStreamBeginCapture(p->stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    delete g;
    return set_err(HC_ERR_HIP, "hipStreamBeginCapture failed: %s", hipGetErrorString(e));
  }
  p->capturing = true;
  for (int32_t l = 0; l < p->lay.L && rc == HC_OK; l++)
    rc = hc_load_back_layer(p, l, host_idx, device_idx, n, layer_events[l]);
  p->capturing = false;
  const std::string layer_err = rc != HC_OK ? g_err : std::string();
  e = hipStreamEndCapture(p->stream, &g->graph);
  if (rc != HC_OK) {
    (void)hipGetLastError();
    hc_load_back_graph_destroy(g);
    return set_err(rc, "capture stopped: %s", layer_err.c_str());
  }
  if (e != hipSuccess || !g->graph) {
    (void)hipGetLastError();
    hc_load_back_graph_destroy(g);
    return set_err(HC_ERR_HIP, "hipStreamEndCapture failed: %s", hipGetErrorString(e));
  }
  e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    g->exec = nullptr;
    hc_load_back_graph_destroy(g);
    return set_err(HC_ERR_HIP, "hipGraphInstantiate failed: %s", hipGetErrorString(e));
  }
  hc::pool_hold(p);
  g->held = true;
  *out = g;
  return HC_OK;
}

int hc_load_back_graph_launch(hc_lb_graph* g) {
  if (!g) return set_err(HC_ERR_INVALID, "graph is null");
  TraceRange range("hc_load_back_graph_launch");
  hc_pool* p = g->pool;
  std::lock_guard<std::recursive_mutex> lock(p->mu);
  int rc = use_device(p);
  if (rc != HC_OK) return rc;
  HIP_TRY(hipGraphLaunch(g->exec, p->stream));
  if (g->n > 0) {
    p->stats.load_back_calls += p->lay.L;
    p->stats.load_back_tokens += g->n * p->lay.L;
    p->stats.load_back_bytes += layer_bytes(p, g->n) * p->lay.L;
  }
  return HC_OK;
}

int hc_pool_get_stats(hc_pool* p, hc_pool_stats* out) {
  if (!p || !out) return set_err(HC_ERR_INVALID, "null argument");
  std::lock_guard<std::recursive_mutex> lock(p->mu);
  *out = p->stats;
  return HC_OK;
}

int hc_pool_kernel_time(hc_pool* p, int32_t kind, int32_t reset, int64_t* launches, double* total_ms) {
  if (!p || !launches || !total_ms) return set_err(HC_ERR_INVALID, "null argument");
  std::lock_guard<std::recursive_mutex> lock(p->mu);
  if (kind < 0 || kind >= kKinds) return set_err(HC_ERR_INVALID, "kind out of range");
  int rc = use_device(p);
  if (rc != HC_OK) return rc;
  rc = harvest_timing(p);
  if (rc != HC_OK) return rc;
  *launches = p->kind_launches[kind];
  *total_ms = p->kind_ms[kind];
  if (reset) {
    for (int k = 0; k < kKinds; k++) {
      p->kind_launches[k] = 0;
      p->kind_ms[k] = 0.0;
    }
  }
  return HC_OK;
}

}  // extern "C"

namespace {

int op_load_layer(void* ctx, int32_t layer, const int64_t* h, const int64_t* d, int64_t n, void* ev) {
  return hc_load_back_layer((hc_pool*)ctx, layer, h, d, n, ev);
}

int op_wait_event(void* ctx, void* ev) {
  hc_pool* p = (hc_pool*)ctx;
  std::lock_guard<std::recursive_mutex> lock(p->mu);
  HIP_TRY(hipStreamWaitEvent(p->stream, (hipEvent_t)ev, 0));
  return HC_OK;
}

int op_record_event(void* ctx, void* ev) {
  hc_pool* p = (hc_pool*)ctx;
  std::lock_guard<std::recursive_mutex> lock(p->mu);
  HIP_TRY(hipEventRecord((hipEvent_t)ev, p->stream));
  return HC_OK;
}

int op_sync_event(void*, void* ev) {
  HIP_TRY(hipEventSynchronize((hipEvent_t)ev));
  return HC_OK;
}

int op_stream_wait(void*, void* stream, void* ev) {
  HIP_TRY(hipStreamWaitEvent((hipStream_t)stream, (hipEvent_t)ev, 0));
  return HC_OK;
}

int op_launch_graph(void* ctx, void* graph) {
  hc_lb_graph* g = (hc_lb_graph*)graph;
  if (g->pool != (hc_pool*)ctx) return set_err(HC_ERR_INVALID, "the graph was captured on another pool");
  return hc_load_back_graph_launch(g);
}

}  // namespace

namespace hc {

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vset_err(code, fmt, ap);
  va_end(ap);
  return code;
}

void pool_loader_ops(hc_pool* pool, hc_loader_ops* ops) {
  ops->ctx = pool;
  ops->load_layer = op_load_layer;
  ops->wait_event = op_wait_event;
  ops->record_event = op_record_event;
  ops->sync_event = op_sync_event;
  ops->stream_wait = op_stream_wait;
  ops->launch_graph = op_launch_graph;
}

int pool_layers(const hc_pool* pool) { return pool->lay.L; }

bool pool_has_host(const hc_pool* pool) { return pool->lay.H > 0; }

int graph_matches(const hc_pool* pool, const void* graph, void* const* events, int32_t L) {
  const hc_lb_graph* g = (const hc_lb_graph*)graph;
  if (g->pool != pool) return set_error(HC_ERR_INVALID, "the graph was captured on another pool");
  if ((int32_t)g->events.size() != L) return set_error(HC_ERR_INVALID, "the graph covers another layer count");
  for (int32_t l = 0; l < L; l++)
    if (g->events[(size_t)l] != events[l])
      return set_error(HC_ERR_INVALID,
                       "layer %d: the event differs from the one the graph was captured with (a replay records "
                       "only its own events)",
                       l);
  return HC_OK;
}

void pool_hold(hc_pool* pool) { pool->users.fetch_add(1); }

void pool_release(hc_pool* pool) { pool->users.fetch_sub(1); }

}  // namespace hc

namespace {

int64_t layer_bytes(const hc_pool* p, int64_t n) {
  return n * p->row_bytes_per_layer + (p->lay.has_blocks ? n / p->lay.P : 0) * p->block_bytes_per_layer;
}

}  // namespace
