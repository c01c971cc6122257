/* A write-back, a per-layer load-back, a captured load-back burst replayed into
 * new slots and a write-back that allocates nothing, through the C ABI from plain C
 * (HIP runtime for memory and streams, no Python), each checked byte for byte
 * against the C oracle.  Built by
 * tests/c/build.py, run by tests/test_c_programs.py on a GPU. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "hc.h"
#include "hc_oracle.h"

#define L 3
#define P 16
#define NSUB 2
#define S 1024
#define H 32
#define NPAGES 5

static const int64_t E[NSUB] = {256, 64};

#define HIPCK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "HIP %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 2;                                                               \
    }                                                                         \
  } while (0)
#define HCCK(x)                                                                      \
  do {                                                                               \
    int r_ = (x);                                                                    \
    if (r_ != HC_OK) {                                                               \
      fprintf(stderr, "hc status %d at line %d: %s\n", r_, __LINE__, hc_last_error()); \
      return 3;                                                                      \
    }                                                                                \
  } while (0)

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static uint64_t next(void) {  /* xorshift64 */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return rng;
}

int main(void) {
  HIPCK(hipSetDevice(0));
  void* dlayers[NSUB][L];
  uint8_t* hostcopy[NSUB * L];
  for (int b = 0; b < NSUB; b++)
    for (int l = 0; l < L; l++) {
      size_t n = (size_t)(S * E[b]);
      HIPCK(hipMalloc(&dlayers[b][l], n));
      uint8_t* buf = (uint8_t*)malloc(n);
      for (size_t i = 0; i < n; i++) buf[i] = (uint8_t)next();
      HIPCK(hipMemcpy(dlayers[b][l], buf, n, hipMemcpyHostToDevice));
      hostcopy[b * L + l] = buf;
    }
  hc_pool_desc d;
  memset(&d, 0, sizeof(d));
  d.num_layers = L;
  d.page_size = P;
  d.num_subbufs = NSUB;
  d.layout = HC_LAYOUT_PAGE_FIRST;
  for (int b = 0; b < NSUB; b++) {
    d.sub[b].granularity = HC_TOKEN_ROWS;
    d.sub[b].elem_bytes = E[b];
    d.sub[b].device_layers = dlayers[b];
  }
  d.device_slots = S;
  d.host_pages = H;
  int64_t host_bytes = 0;
  HCCK(hc_host_pool_bytes(&d, &host_bytes));
  void* host = NULL;
  HCCK(hc_host_alloc(host_bytes, 0, &host));
  d.host_base = host;
  d.host_bytes = host_bytes;
  hipStream_t stream;
  HIPCK(hipStreamCreate(&stream));
  d.copy_stream = stream;
  hc_pool* pool = NULL;
  HCCK(hc_pool_create(&d, &pool));

  /* burst: NPAGES random distinct host pages, whole pages; random distinct slots */
  int64_t n = NPAGES * P, hidx[NPAGES * P], didx[NPAGES * P], d2[NPAGES * P];
  int used_page[H] = {0}, used_slot[S] = {0};
  for (int k = 0; k < NPAGES; k++) {
    int p;
    do p = (int)(next() % H); while (used_page[p]);
    used_page[p] = 1;
    for (int r = 0; r < P; r++) hidx[k * P + r] = (int64_t)p * P + r;
  }
  for (int64_t i = 0; i < n; i++) {
    int s;
    do s = (int)(next() % S); while (used_slot[s]);
    used_slot[s] = 1;
    didx[i] = s;
  }
  for (int64_t i = 0; i < n; i++) {
    int s;
    do s = (int)(next() % S); while (used_slot[s]);
    used_slot[s] = 1;
    d2[i] = s;
  }
  int64_t *dd, *dh, *dd2;
  HIPCK(hipMalloc((void**)&dd, sizeof(didx)));
  HIPCK(hipMalloc((void**)&dh, sizeof(hidx)));
  HIPCK(hipMalloc((void**)&dd2, sizeof(d2)));
  HIPCK(hipMemcpy(dd, didx, sizeof(didx), hipMemcpyHostToDevice));
  HIPCK(hipMemcpy(dh, hidx, sizeof(hidx), hipMemcpyHostToDevice));
  HIPCK(hipMemcpy(dd2, d2, sizeof(d2), hipMemcpyHostToDevice));

  HCCK(hc_write_back_all_layers(pool, dd, hidx, n, NULL));
  HCCK(hc_pool_sync(pool));

  orc_geom g;
  memset(&g, 0, sizeof(g));
  g.layers = L;
  g.page_size = P;
  g.nsub = NSUB;
  g.layout = ORC_PAGE_FIRST;
  g.host_pages = H;
  g.device_slots = S;
  g.align = 4096;
  for (int b = 0; b < NSUB; b++) {
    g.gran[b] = ORC_TOKEN_ROWS;
    g.bytes[b] = E[b];
  }
  uint8_t* want = (uint8_t*)calloc((size_t)host_bytes, 1);
  if (orc_write_back(&g, hostcopy, want, didx, hidx, n) != ORC_OK) return 4;
  if (memcmp(want, host, (size_t)host_bytes) != 0) {
    fprintf(stderr, "write-back differs from the oracle\n");
    return 5;
  }
  hipEvent_t ev[L];
  for (int l = 0; l < L; l++) {
    HIPCK(hipEventCreateWithFlags(&ev[l], hipEventDisableTiming));
    HCCK(hc_load_back_layer(pool, l, dh, dd2, n, ev[l]));
  }
  for (int l = 0; l < L; l++) HIPCK(hipEventSynchronize(ev[l]));
  for (int l = 0; l < L; l++)
    if (orc_load_back_layer(&g, l, hostcopy, want, hidx, d2, n) != ORC_OK) return 6;
  for (int b = 0; b < NSUB; b++)
    for (int l = 0; l < L; l++) {
      size_t nb = (size_t)(S * E[b]);
      uint8_t* got = (uint8_t*)malloc(nb);
      HIPCK(hipMemcpy(got, dlayers[b][l], nb, hipMemcpyDeviceToHost));
      if (memcmp(got, hostcopy[b * L + l], nb) != 0) {
        fprintf(stderr, "load-back differs from the oracle (sub %d layer %d)\n", b, l);
        return 7;
      }
      free(got);
    }
  int64_t bad = -1;
  HCCK(hc_round_trip_check(pool, dd, dd2, n, &bad));
  if (bad != 0) return 8;

  /* the load-back captured once, then replayed after the slot list was rewritten in place */
  hc_lb_graph* graph = NULL;
  HCCK(hc_load_back_graph_create(pool, dh, dd2, n, (void* const*)ev, &graph));
  int64_t d3[NPAGES * P];
  for (int64_t i = 0; i < n; i++) {
    int s;
    do s = (int)(next() % S); while (used_slot[s]);
    used_slot[s] = 1;
    d3[i] = s;
  }
  HIPCK(hipMemcpy(dd2, d3, sizeof(d3), hipMemcpyHostToDevice));
  HCCK(hc_load_back_graph_launch(graph));
  for (int l = 0; l < L; l++) HIPCK(hipEventSynchronize(ev[l]));
  for (int l = 0; l < L; l++)
    if (orc_load_back_layer(&g, l, hostcopy, want, hidx, d3, n) != ORC_OK) return 9;
  for (int b = 0; b < NSUB; b++)
    for (int l = 0; l < L; l++) {
      size_t nb = (size_t)(S * E[b]);
      uint8_t* got = (uint8_t*)malloc(nb);
      HIPCK(hipMemcpy(got, dlayers[b][l], nb, hipMemcpyDeviceToHost));
      if (memcmp(got, hostcopy[b * L + l], nb) != 0) {
        fprintf(stderr, "captured load-back differs from the oracle (sub %d layer %d)\n", b, l);
        return 10;
      }
      free(got);
    }
  HCCK(hc_load_back_graph_destroy(graph));

  /* the write-back that allocates nothing: other host pages, from the slots just loaded;
   * its host list lives in pinned memory */
  int64_t* pinned = NULL;
  HCCK(hc_host_alloc((int64_t)sizeof(hidx), 0, (void**)&pinned));
  for (int k = 0; k < NPAGES; k++) {
    int p;
    do p = (int)(next() % H); while (used_page[p]);
    used_page[p] = 1;
    for (int r = 0; r < P; r++) pinned[k * P + r] = (int64_t)p * P + r;
  }
  HCCK(hc_write_back_all_layers_noalloc(pool, dd2, pinned, n, NULL));
  HCCK(hc_pool_sync(pool));
  if (orc_write_back(&g, hostcopy, want, d3, pinned, n) != ORC_OK) return 11;
  if (memcmp(want, host, (size_t)host_bytes) != 0) {
    fprintf(stderr, "write-back without allocation differs from the oracle\n");
    return 12;
  }
  HCCK(hc_host_free(pinned));
  HCCK(hc_pool_destroy(pool));
  HCCK(hc_host_free(host));
  printf("gpu_roundtrip ok: %lld tokens x %d layers x %d sub-buffers bit-exact, eager, captured and without allocation\n",
         (long long)n, L, NSUB);
  return 0;
}
