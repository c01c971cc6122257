// Host-only stress of the library's CPU-side machinery -- the load-back loader thread
// and the host-to-host shard worker pool -- built with ThreadSanitizer or with
// AddressSanitizer + UndefinedBehaviorSanitizer by tests/c/build.py.  No GPU: the
// loader drives recording callbacks through hc_loader_ops, the shard pool copies
// between host buffers.  The few library entry points these files use from the
// GPU-side translation unit are stubbed below.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

#include "hc.h"
#include "hc_internal.h"

namespace hc {
namespace {
thread_local char g_msg[256];
}
int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}
void pool_loader_ops(hc_pool*, hc_loader_ops*) { abort(); }  // every loader here brings its own ops
int pool_layers(const hc_pool*) { return 0; }
bool pool_has_host(const hc_pool*) { return true; }
void pool_hold(hc_pool*) {}
void pool_release(hc_pool*) {}
int graph_matches(const hc_pool*, const void*, void* const*, int32_t) { abort(); }  // pool ops only
}  // namespace hc

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      exit(1);                                                          \
    }                                                                   \
  } while (0)

// ------------------------------------------------------------------ loader
constexpr int kL = 8;
constexpr int kProducers = 4;
constexpr int kBursts = 150;

// Events are addresses into this array; host_idx carries (producer, burst) so a
// callback knows which burst it serves; burst b of every producer fails at layer 3
// when b % 7 == 3.
struct Recorder {
  std::atomic<int> records[kProducers][kL];  // layer events recorded (load or record op)
  std::atomic<int> loads{0}, waits{0}, stream_waits{0}, syncs{0};
  char events[kProducers][kL];
};

Recorder g_rec;

int producer_of(const void* ev) { return (int)(((const char*)ev - &g_rec.events[0][0]) / kL); }
int layer_of(const void* ev) { return (int)(((const char*)ev - &g_rec.events[0][0]) % kL); }

int op_load(void*, int32_t layer, const int64_t* h, const int64_t*, int64_t, void* ev) {
  const int64_t tag = (int64_t)(intptr_t)h;
  const int burst = (int)(tag % 1000);
  if (burst % 7 == 3 && layer == 3) return HC_ERR_HIP;
  if (burst % 5 == 0) std::this_thread::sleep_for(std::chrono::microseconds(50));
  CHECK(layer_of(ev) == layer);
  g_rec.records[producer_of(ev)][layer].fetch_add(1);
  g_rec.loads.fetch_add(1);
  return HC_OK;
}
int op_wait(void*, void*) {
  g_rec.waits.fetch_add(1);
  return HC_OK;
}
int op_record(void*, void* ev) {
  g_rec.records[producer_of(ev)][layer_of(ev)].fetch_add(1);
  return HC_OK;
}
int op_sync(void*, void*) {
  g_rec.syncs.fetch_add(1);
  return HC_OK;
}
int op_stream_wait(void*, void*, void*) {
  g_rec.stream_waits.fetch_add(1);
  return HC_OK;
}
// A captured burst: the graph handle is the address of its producer's event row; one
// launch records every layer event of that row.
int op_launch_graph(void*, void* graph) {
  const int p = producer_of(graph);
  for (int l = 0; l < kL; l++) g_rec.records[p][l].fetch_add(1);
  return HC_OK;
}

void loader_stress(int async) {
  for (auto& row : g_rec.records)
    for (auto& x : row) x.store(0);
  hc_loader_ops ops{};
  ops.load_layer = op_load;
  ops.wait_event = op_wait;
  ops.record_event = op_record;
  ops.sync_event = op_sync;
  ops.stream_wait = op_stream_wait;
  ops.launch_graph = op_launch_graph;
  hc_loader* ld = nullptr;
  CHECK(hc_loader_create(nullptr, &ops, kL, async, &ld) == HC_OK);
  std::atomic<int> failed{0};
  std::atomic<bool> done{false};
  std::thread observer([&] {  // queries from a third thread while bursts run
    while (!done.load()) {
      int64_t f = 0;
      int32_t running = 0;
      CHECK(hc_loader_info(ld, &f, &running) == HC_OK);
      std::this_thread::yield();
    }
  });
  std::vector<std::thread> producers;
  for (int p = 0; p < kProducers; p++) {
    producers.emplace_back([&, p] {
      void* evs[kL];
      for (int l = 0; l < kL; l++) evs[l] = &g_rec.events[p][l];
      for (int b = 0; b < kBursts; b++) {
        hc_burst* burst = nullptr;
        const int64_t tag = (int64_t)p * 1000 + b;
        // the same events for every burst of this producer: reuse waits for the previous one;
        // every third burst is a captured one
        if (b % 3 == 1) {
          CHECK(hc_loader_submit_graph(ld, evs[0], evs, nullptr, &burst) == HC_OK);
        } else {
          CHECK(hc_loader_submit(ld, (const int64_t*)(intptr_t)tag, nullptr, 1, evs, b % 2 ? evs[0] : nullptr,
                                 &burst) == HC_OK);
        }
        for (int l = 0; l < kL; l += 3) CHECK(hc_burst_wait_layer(burst, l, (void*)(intptr_t)(p + 1)) == HC_OK);
        int32_t enq = 0, fin = 0;
        CHECK(hc_burst_query(burst, &enq, &fin) == HC_OK);
        const int rc = hc_burst_wait(burst);
        if (b % 7 == 3 && b % 3 != 1) {
          CHECK(rc == HC_ERR_HIP);
          failed.fetch_add(1);
        } else {
          CHECK(rc == HC_OK);
        }
        CHECK(hc_burst_release(burst) == HC_OK);
      }
    });
  }
  for (auto& t : producers) t.join();
  CHECK(hc_loader_drain(ld) == HC_OK);
  done.store(true);
  observer.join();
  int64_t f = 0;
  int32_t running = 0;
  CHECK(hc_loader_info(ld, &f, &running) == HC_OK);
  CHECK(f == failed.load() && running == async);
  // every layer event of every burst recorded exactly once
  for (int p = 0; p < kProducers; p++)
    for (int l = 0; l < kL; l++) CHECK(g_rec.records[p][l].load() == kBursts);
  CHECK(hc_loader_destroy(ld) == HC_OK);
}

// ------------------------------------------------------------------ host-to-host shards
constexpr int kShards = 96;
constexpr int kTensors = 3;
const int64_t kSizes[kTensors] = {4096, 1024, 2048};
constexpr int64_t kShardBytes = 8192;  // 7168 payload + 1024 zero pad

void h2h_stress(int workers) {
  std::vector<uint8_t> pages((size_t)kShards * kTensors * 4096), back(pages.size(), 0);
  std::vector<uint8_t> store((size_t)kShards * kShardBytes, 0xEE);
  std::mt19937 rng(5);
  for (auto& x : pages) x = (uint8_t)rng();
  auto page_addr = [&](std::vector<uint8_t>& buf, int s, int t) { return (void*)&buf[((size_t)s * kTensors + t) * 4096]; };
  hc_h2h* e = nullptr;
  CHECK(hc_h2h_create(workers, 24, &e) == HC_OK);
  const int threads = workers ? 4 : 1;
  std::vector<std::thread> ts;
  std::atomic<int> busy{0};
  for (int k = 0; k < threads; k++) {
    ts.emplace_back([&, k] {
      const int per = kShards / threads;
      for (int dir = HC_H2H_DUMP; dir <= HC_H2H_LOAD; dir++) {
        for (int first = k * per; first < (k + 1) * per; first += 8) {
          std::vector<void*> tp, sh;
          for (int s = first; s < first + 8; s++) {
            for (int t = 0; t < kTensors; t++) tp.push_back(page_addr(dir == HC_H2H_DUMP ? pages : back, s, t));
            sh.push_back(&store[(size_t)s * kShardBytes]);
          }
          hc_h2h_request* r = nullptr;
          int rc;
          while ((rc = hc_h2h_submit(e, dir, kTensors, kSizes, tp.data(), sh.data(), kShardBytes, 8, &r)) ==
                 HC_ERR_BUSY) {
            busy.fetch_add(1);
            std::this_thread::yield();
          }
          CHECK(rc == HC_OK);
          int64_t dump = 0, load = 0;
          CHECK(hc_h2h_outstanding(e, &dump, &load) == HC_OK);
          CHECK(dump >= 0 && load >= 0 && dump <= 24 && load <= 24);
          CHECK(hc_h2h_release(r) == HC_OK);
        }
      }
    });
  }
  for (auto& t : ts) t.join();
  CHECK(hc_h2h_destroy(e) == HC_OK);
  for (int s = 0; s < kShards; s++) {
    const uint8_t* shard = &store[(size_t)s * kShardBytes];
    int64_t off = 0;
    for (int t = 0; t < kTensors; t++) {
      CHECK(memcmp(shard + off, page_addr(pages, s, t), (size_t)kSizes[t]) == 0);
      CHECK(memcmp(page_addr(back, s, t), page_addr(pages, s, t), (size_t)kSizes[t]) == 0);
      off += kSizes[t];
    }
    for (int64_t i = off; i < kShardBytes; i++) CHECK(shard[i] == 0);
  }
}

#if defined(__has_feature)
#if __has_feature(thread_sanitizer)
#define HC_SANITIZER "thread"
#elif __has_feature(address_sanitizer)
#define HC_SANITIZER "address"
#endif
#endif
#if !defined(HC_SANITIZER) && defined(__SANITIZE_THREAD__)
#define HC_SANITIZER "thread"
#endif
#if !defined(HC_SANITIZER) && defined(__SANITIZE_ADDRESS__)
#define HC_SANITIZER "address"
#endif
#ifndef HC_SANITIZER
#define HC_SANITIZER "none"
#endif

int main() {
  printf("sanitizer: %s\n", HC_SANITIZER);
  for (int round = 0; round < 3; round++) {
    loader_stress(1);
    loader_stress(0);
    h2h_stress(4);
    h2h_stress(0);
  }
  printf("sanitize_host ok\n");
  return 0;
}
