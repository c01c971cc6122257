// Asynchronous load-back enqueue (loader-thread page, sglang PR 38472: Motivation,
// Modifications).  The caller hands a burst over and returns; one FIFO worker
// thread makes the transfer stream wait for the burst's start event, enqueues the
// layers in order and records every layer event.  Per-layer CPU flags let a
// consumer block until a layer's event has actually been recorded: a stream that
// waits on an event nobody recorded yet does not wait.  On failure the remaining
// layer events are still recorded and flagged, so a consumer never hangs; the
// burst reports the error and the next burst is served.  All device work goes
// through hc_loader_ops, so the ordering rules are observable without a GPU.
#include <stdio.h>

#include <chrono>
#include <condition_variable>
#include <deque>
#include <mutex>
#include <new>
#include <thread>
#include <unordered_map>
#include <vector>

#include "hc_internal.h"

struct hc_burst {
  hc_loader* loader = nullptr;
  const int64_t* host_idx = nullptr;
  const int64_t* device_idx = nullptr;
  int64_t n = 0;
  std::vector<void*> events;
  void* start_event = nullptr;
  void* graph = nullptr;  // a captured burst to replay instead of per-layer enqueues
  // guarded by loader->mu
  int32_t flagged = 0;  // layers [0, flagged) have their event recorded
  bool done = false;    // every layer flagged (enqueue finished or failed)
  int status = HC_OK;
};

struct hc_loader {
  hc_loader_ops ops{};
  hc_pool* pool = nullptr;
  bool pool_ops = false;  // ops are the pool's own: graphs are hc_lb_graph handles
  int32_t L = 0;
  bool async = false;
  std::mutex mu;
  std::condition_variable cv;
  std::deque<hc_burst*> queue;
  std::unordered_map<void*, hc_burst*> held;  // layer event -> burst not yet fully enqueued
  bool stop = false;
  bool running = false;
  int64_t failed = 0;
  int64_t in_flight = 0;  // submitted, not yet done
  int64_t live = 0;       // submitted, not yet released (each holds a pointer to the loader)
  std::thread worker;
};

namespace {

int loader_err(int code, const char* msg) { return hc::set_error(code, "%s", msg); }

void flag_layers(hc_loader* ld, hc_burst* b, int32_t upto) {
  std::lock_guard<std::mutex> lk(ld->mu);
  b->flagged = upto;
  ld->cv.notify_all();
}

// The enqueue of one burst, on the worker thread (or inline on the caller's).
void run_burst(hc_loader* ld, hc_burst* b) {
  void* ctx = ld->ops.ctx;
  int st = HC_OK;
  if (b->start_event) st = ld->ops.wait_event(ctx, b->start_event);
  int32_t l = 0;
  if (b->graph) {
    // one replay enqueues and records every layer
    if (st == HC_OK) st = ld->ops.launch_graph(ctx, b->graph);
    if (st == HC_OK) {
      l = ld->L;
      flag_layers(ld, b, l);
    }
  }
  for (; !b->graph && st == HC_OK && l < ld->L; l++) {
    st = ld->ops.load_layer(ctx, l, b->host_idx, b->device_idx, b->n, b->events[(size_t)l]);
    if (st != HC_OK) break;
    flag_layers(ld, b, l + 1);
  }
  if (st != HC_OK) {
    // complete every layer from the failing one on, so waiting consumers are released
    for (int32_t k = l; k < ld->L; k++) (void)ld->ops.record_event(ctx, b->events[(size_t)k]);
    fprintf(stderr, "hc_loader: burst enqueue failed at layer %d (status %d); layers %d..%d completed without data\n",
            l, st, l, ld->L - 1);
  }
  std::lock_guard<std::mutex> lk(ld->mu);
  if (st != HC_OK) {
    b->status = st;
    ld->failed++;
  }
  b->flagged = ld->L;
  b->done = true;
  for (void* e : b->events) {
    auto it = ld->held.find(e);
    if (it != ld->held.end() && it->second == b) ld->held.erase(it);
  }
  ld->in_flight--;
  ld->cv.notify_all();
  // b is not touched after this point by the loader
}

void worker_main(hc_loader* ld) {
  for (;;) {
    hc_burst* b = nullptr;
    {
      std::unique_lock<std::mutex> lk(ld->mu);
      ld->cv.wait(lk, [&] { return ld->stop || !ld->queue.empty(); });
      if (ld->queue.empty()) return;  // stop requested and nothing left
      b = ld->queue.front();
      ld->queue.pop_front();
    }
    run_burst(ld, b);
  }
}

}  // namespace

extern "C" {

int hc_loader_create(hc_pool* pool, const hc_loader_ops* ops, int32_t num_layers, int32_t async,
                     hc_loader** out) {
  if (!out) return loader_err(HC_ERR_INVALID, "out is null");
  *out = nullptr;
  if (num_layers < 1 || num_layers > HC_MAX_LAYERS) return loader_err(HC_ERR_INVALID, "num_layers out of range");
  if (async != 0 && async != 1) return loader_err(HC_ERR_INVALID, "async must be 0 or 1");
  hc_loader_ops use{};
  if (ops) {
    use = *ops;
  } else {
    if (!pool) return loader_err(HC_ERR_INVALID, "a loader without ops needs a pool");
    if (!hc::pool_has_host(pool)) return loader_err(HC_ERR_INVALID, "the pool has no host pages to load from");
    hc::pool_loader_ops(pool, &use);
  }
  if (!use.load_layer || !use.wait_event || !use.record_event || !use.sync_event || !use.stream_wait)
    return loader_err(HC_ERR_INVALID, "every hc_loader_ops entry must be set");
  if (pool && hc::pool_layers(pool) != num_layers)
    return loader_err(HC_ERR_INVALID, "num_layers differs from the pool's layer count");
  hc_loader* ld = new (std::nothrow) hc_loader();
  if (!ld) return loader_err(HC_ERR_NOMEM, "loader allocation failed");
  ld->ops = use;
  ld->pool = pool;
  ld->pool_ops = !ops;
  ld->L = num_layers;
  ld->async = async == 1;
  if (ld->async) {
    try {
      ld->worker = std::thread(worker_main, ld);
    } catch (...) {
      delete ld;
      return loader_err(HC_ERR_NOMEM, "could not start the loader thread");
    }
    ld->running = true;
  }
  if (pool) hc::pool_hold(pool);
  *out = ld;
  return HC_OK;
}

namespace {

int submit_burst(hc_loader* ld, const int64_t* host_idx, const int64_t* device_idx, int64_t n, void* graph,
                 void* const* layer_events, void* start_event, hc_burst** out);

}  // namespace

int hc_loader_submit(hc_loader* ld, const int64_t* host_idx, const int64_t* device_idx, int64_t n,
                     void* const* layer_events, void* start_event, hc_burst** out) {
  if (!ld || !out || !layer_events) return loader_err(HC_ERR_INVALID, "null argument");
  *out = nullptr;
  if (n < 0) return loader_err(HC_ERR_INVALID, "n must be >= 0");
  return submit_burst(ld, host_idx, device_idx, n, nullptr, layer_events, start_event, out);
}

int hc_loader_submit_graph(hc_loader* ld, void* graph, void* const* layer_events, void* start_event,
                           hc_burst** out) {
  if (!ld || !out || !layer_events || !graph) return loader_err(HC_ERR_INVALID, "null argument");
  *out = nullptr;
  if (!ld->ops.launch_graph) return loader_err(HC_ERR_UNSUPPORTED, "the loader's ops cannot launch a graph");
  if (ld->pool_ops) {
    // a replay records only the events it was captured with; other ones would never be recorded
    const int rc = hc::graph_matches(ld->pool, graph, layer_events, ld->L);
    if (rc != HC_OK) return rc;
  }
  return submit_burst(ld, nullptr, nullptr, 0, graph, layer_events, start_event, out);
}

}  // extern "C"

namespace {

int submit_burst(hc_loader* ld, const int64_t* host_idx, const int64_t* device_idx, int64_t n, void* graph,
                 void* const* layer_events, void* start_event, hc_burst** out) {
  std::vector<void*> evs(layer_events, layer_events + ld->L);
  for (size_t i = 0; i < evs.size(); i++) {
    if (!evs[i]) return loader_err(HC_ERR_INVALID, "null layer event");
    for (size_t j = 0; j < i; j++)
      if (evs[j] == evs[i]) return loader_err(HC_ERR_INVALID, "layer events must be distinct");
  }
  hc_burst* b = new (std::nothrow) hc_burst();
  if (!b) return loader_err(HC_ERR_NOMEM, "burst allocation failed");
  b->loader = ld;
  b->host_idx = host_idx;
  b->device_idx = device_idx;
  b->n = n;
  b->graph = graph;
  b->events = std::move(evs);
  b->start_event = start_event;
  {
    std::unique_lock<std::mutex> lk(ld->mu);
    // an earlier burst that still has to record one of these events goes first
    ld->cv.wait(lk, [&] {
      for (void* e : b->events)
        if (ld->held.count(e)) return false;
      return true;
    });
    for (void* e : b->events) ld->held[e] = b;
    ld->in_flight++;
    ld->live++;
    if (ld->async) {
      ld->queue.push_back(b);
      ld->cv.notify_all();
    }
  }
  if (!ld->async) run_burst(ld, b);
  *out = b;
  return HC_OK;
}

}  // namespace

extern "C" {

int hc_burst_wait_layer(hc_burst* b, int32_t layer, void* consumer_stream) {
  if (!b) return loader_err(HC_ERR_INVALID, "burst is null");
  hc_loader* ld = b->loader;
  if (layer < 0 || layer >= ld->L) return loader_err(HC_ERR_INVALID, "layer out of range");
  {
    std::unique_lock<std::mutex> lk(ld->mu);
    auto t0 = std::chrono::steady_clock::now();
    while (b->flagged <= layer) {
      // a long wait is reported every 30 s (the burst may sit behind a slow one)
      if (ld->cv.wait_for(lk, std::chrono::seconds(30)) == std::cv_status::timeout && b->flagged <= layer) {
        const double s = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
        fprintf(stderr, "hc_loader: still waiting for layer %d to be recorded after %.0f s\n", layer, s);
      }
    }
  }
  void* ev = b->events[(size_t)layer];
  if (consumer_stream) return ld->ops.stream_wait(ld->ops.ctx, consumer_stream, ev);
  return ld->ops.sync_event(ld->ops.ctx, ev);
}

int hc_burst_wait(hc_burst* b) {
  if (!b) return loader_err(HC_ERR_INVALID, "burst is null");
  hc_loader* ld = b->loader;
  int status;
  {
    std::unique_lock<std::mutex> lk(ld->mu);
    ld->cv.wait(lk, [&] { return b->done; });
    status = b->status;
  }
  int rc = ld->ops.sync_event(ld->ops.ctx, b->events.back());
  if (status != HC_OK) return hc::set_error(status, "the burst's enqueue failed; its rows are stale");
  return rc;
}

int hc_burst_query(hc_burst* b, int32_t* layers_enqueued, int32_t* enqueue_done) {
  if (!b || !layers_enqueued || !enqueue_done) return loader_err(HC_ERR_INVALID, "null argument");
  std::lock_guard<std::mutex> lk(b->loader->mu);
  *layers_enqueued = b->flagged;
  *enqueue_done = b->done ? 1 : 0;
  return HC_OK;
}

int hc_burst_release(hc_burst* b) {
  if (!b) return HC_OK;
  hc_loader* ld = b->loader;
  {
    std::unique_lock<std::mutex> lk(ld->mu);
    ld->cv.wait(lk, [&] { return b->done; });
    ld->live--;
  }
  delete b;
  return HC_OK;
}

int hc_loader_drain(hc_loader* ld) {
  if (!ld) return loader_err(HC_ERR_INVALID, "loader is null");
  std::unique_lock<std::mutex> lk(ld->mu);
  ld->cv.wait(lk, [&] { return ld->in_flight == 0; });
  return HC_OK;
}

int hc_loader_info(hc_loader* ld, int64_t* failed_bursts, int32_t* worker_running) {
  if (!ld || !failed_bursts || !worker_running) return loader_err(HC_ERR_INVALID, "null argument");
  std::lock_guard<std::mutex> lk(ld->mu);
  *failed_bursts = ld->failed;
  *worker_running = ld->running ? 1 : 0;
  return HC_OK;
}

int hc_loader_destroy(hc_loader* ld) {
  if (!ld) return HC_OK;
  {
    std::lock_guard<std::mutex> lk(ld->mu);
    if (ld->live > 0)  // a later hc_burst_release would reach a freed loader
      return hc::set_error(HC_ERR_INVALID, "%lld burst(s) not released; release them first", (long long)ld->live);
    ld->stop = true;
    ld->cv.notify_all();
  }
  if (ld->worker.joinable()) ld->worker.join();  // the worker empties its queue first
  if (ld->pool) hc::pool_release(ld->pool);
  delete ld;
  return HC_OK;
}

}  // extern "C"
