// Host-to-host shard copies and the cache identity (CacheStore H2H page,
// unified-cache-management PR 1292: Dump path, Load path, Queue backpressure,
// Failure handling, page_first_kv_split support).  One page is one store shard
// (tensor pages back to back, then zeros); one shard is one job; a pool of CPU
// copy workers runs jobs concurrently, each shard's tensors in order by one worker.
// Dump and load count outstanding (queued + running) shards separately and reserve
// capacity for a whole request, or refuse it.
#include <stdio.h>
#include <string.h>

#include <condition_variable>
#include <deque>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "hc_internal.h"

struct hc_h2h_request {
  hc_h2h* eng = nullptr;
  int32_t dir = 0;
  int32_t tensors = 0;
  std::vector<int64_t> sizes;
  std::vector<void*> pages;   // [n][tensors]
  std::vector<void*> shards;  // [n]
  int64_t shard_bytes = 0;
  int64_t n = 0;
  int64_t remaining = 0;  // guarded by eng->mu
  int status = HC_OK;
};

struct hc_h2h {
  std::mutex mu;
  std::condition_variable cv_work, cv_done;
  std::deque<std::pair<hc_h2h_request*, int64_t>> queue;
  std::vector<std::thread> workers;
  bool stop = false;
  int64_t depth = 0;
  int64_t outstanding[2] = {0, 0};
  int64_t live = 0;  // requests submitted and not yet released (each holds a pointer to the engine)
};

namespace {

void copy_shard(const hc_h2h_request* r, int64_t i) {
  uint8_t* shard = (uint8_t*)r->shards[(size_t)i];
  int64_t off = 0;
  for (int32_t t = 0; t < r->tensors; t++) {
    uint8_t* page = (uint8_t*)r->pages[(size_t)(i * r->tensors + t)];
    const size_t len = (size_t)r->sizes[(size_t)t];
    if (r->dir == HC_H2H_DUMP) memcpy(shard + off, page, len);
    else memcpy(page, shard + off, len);
    off += r->sizes[(size_t)t];
  }
  if (r->dir == HC_H2H_DUMP && off < r->shard_bytes) memset(shard + off, 0, (size_t)(r->shard_bytes - off));
}

void finish_job(hc_h2h* e, hc_h2h_request* r) {
  std::lock_guard<std::mutex> lk(e->mu);
  r->remaining--;
  e->outstanding[r->dir]--;
  e->cv_done.notify_all();
}

void worker_main(hc_h2h* e) {
  for (;;) {
    std::pair<hc_h2h_request*, int64_t> job;
    {
      std::unique_lock<std::mutex> lk(e->mu);
      e->cv_work.wait(lk, [&] { return e->stop || !e->queue.empty(); });
      if (e->queue.empty()) return;
      job = e->queue.front();
      e->queue.pop_front();
    }
    copy_shard(job.first, job.second);
    finish_job(e, job.first);
  }
}

// Manual progress (no workers): run queued jobs of `r` (or of any request when r is
// null) on the calling thread.
void run_inline(hc_h2h* e, hc_h2h_request* r) {
  for (;;) {
    std::pair<hc_h2h_request*, int64_t> job{nullptr, 0};
    {
      std::lock_guard<std::mutex> lk(e->mu);
      for (auto it = e->queue.begin(); it != e->queue.end(); ++it) {
        if (!r || it->first == r) {
          job = *it;
          e->queue.erase(it);
          break;
        }
      }
    }
    if (!job.first) return;
    copy_shard(job.first, job.second);
    finish_job(e, job.first);
  }
}

uint64_t fnv1a64(const std::string& s) {
  uint64_t h = 0xcbf29ce484222325ull;  // FNV offset basis
  for (unsigned char c : s) {
    h ^= c;
    h *= 0x100000001b3ull;             // FNV prime
  }
  return h;
}

}  // namespace

extern "C" {

int hc_h2h_create(int32_t workers, int64_t queue_depth, hc_h2h** out) {
  if (!out) return hc::set_error(HC_ERR_INVALID, "out is null");
  *out = nullptr;
  if (workers < 0 || workers > 256) return hc::set_error(HC_ERR_INVALID, "workers must be in [0, 256]");
  if (queue_depth < 1) return hc::set_error(HC_ERR_INVALID, "queue_depth must be >= 1");
  hc_h2h* e = new (std::nothrow) hc_h2h();
  if (!e) return hc::set_error(HC_ERR_NOMEM, "allocation failed");
  e->depth = queue_depth;
  try {
    for (int32_t w = 0; w < workers; w++) e->workers.emplace_back(worker_main, e);
  } catch (...) {
    hc_h2h_destroy(e);
    return hc::set_error(HC_ERR_NOMEM, "could not start the copy workers");
  }
  *out = e;
  return HC_OK;
}

int hc_h2h_submit(hc_h2h* e, int32_t direction, int32_t tensors, const int64_t* tensor_bytes,
                  void* const* tensor_pages, void* const* shards, int64_t shard_bytes, int64_t n,
                  hc_h2h_request** out) {
  if (!e || !out) return hc::set_error(HC_ERR_INVALID, "null argument");
  *out = nullptr;
  if (direction != HC_H2H_DUMP && direction != HC_H2H_LOAD)
    return hc::set_error(HC_ERR_INVALID, "direction must be HC_H2H_DUMP or HC_H2H_LOAD");
  if (tensors < 1 || tensors > HC_H2H_MAX_TENSORS || !tensor_bytes)
    return hc::set_error(HC_ERR_INVALID, "tensor count must be in [1, HC_H2H_MAX_TENSORS]");
  if (n < 0) return hc::set_error(HC_ERR_INVALID, "n must be >= 0");
  if (n > 0 && (!tensor_pages || !shards)) return hc::set_error(HC_ERR_INVALID, "null address array");
  if (n > e->depth)  // could never be admitted: split it
    return hc::set_error(HC_ERR_INVALID, "%lld shards exceed the queue depth %lld", (long long)n,
                         (long long)e->depth);
  int64_t sum = 0;
  for (int32_t t = 0; t < tensors; t++) {
    if (tensor_bytes[t] <= 0) return hc::set_error(HC_ERR_INVALID, "tensor %d: size must be > 0", t);
    sum += tensor_bytes[t];
  }
  if (sum > shard_bytes)
    return hc::set_error(HC_ERR_INVALID, "tensor pages (%lld bytes) do not fit a %lld-byte shard", (long long)sum,
                         (long long)shard_bytes);
  for (int64_t i = 0; i < n; i++) {
    if (!shards[i]) return hc::set_error(HC_ERR_INVALID, "shard %lld: null address", (long long)i);
    for (int32_t t = 0; t < tensors; t++)
      if (!tensor_pages[i * tensors + t])
        return hc::set_error(HC_ERR_INVALID, "shard %lld tensor %d: null address", (long long)i, t);
  }
  hc_h2h_request* r = new (std::nothrow) hc_h2h_request();
  if (!r) return hc::set_error(HC_ERR_NOMEM, "allocation failed");
  r->eng = e;
  r->dir = direction;
  r->tensors = tensors;
  r->sizes.assign(tensor_bytes, tensor_bytes + tensors);
  r->pages.assign(tensor_pages, tensor_pages + n * tensors);
  r->shards.assign(shards, shards + n);
  r->shard_bytes = shard_bytes;
  r->n = n;
  {
    std::lock_guard<std::mutex> lk(e->mu);
    if (e->outstanding[direction] + n > e->depth) {
      delete r;
      return hc::set_error(HC_ERR_BUSY, "%lld shards requested, %lld of %lld outstanding: request refused whole",
                           (long long)n, (long long)e->outstanding[direction], (long long)e->depth);
    }
    e->outstanding[direction] += n;
    e->live++;
    r->remaining = n;
    for (int64_t i = 0; i < n; i++) e->queue.emplace_back(r, i);
    e->cv_work.notify_all();
  }
  *out = r;
  return HC_OK;
}

int hc_h2h_wait(hc_h2h_request* r) {
  if (!r) return hc::set_error(HC_ERR_INVALID, "request is null");
  hc_h2h* e = r->eng;
  if (e->workers.empty()) run_inline(e, r);
  std::unique_lock<std::mutex> lk(e->mu);
  e->cv_done.wait(lk, [&] { return r->remaining == 0; });
  return r->status;
}

int hc_h2h_release(hc_h2h_request* r) {
  if (!r) return HC_OK;
  int rc = hc_h2h_wait(r);
  {
    std::lock_guard<std::mutex> lk(r->eng->mu);
    r->eng->live--;
  }
  delete r;
  return rc;
}

int hc_h2h_outstanding(hc_h2h* e, int64_t* dump_shards, int64_t* load_shards) {
  if (!e || !dump_shards || !load_shards) return hc::set_error(HC_ERR_INVALID, "null argument");
  std::lock_guard<std::mutex> lk(e->mu);
  *dump_shards = e->outstanding[HC_H2H_DUMP];
  *load_shards = e->outstanding[HC_H2H_LOAD];
  return HC_OK;
}

int hc_h2h_destroy(hc_h2h* e) {
  if (!e) return HC_OK;
  {
    std::lock_guard<std::mutex> lk(e->mu);
    if (e->live > 0)  // a later hc_h2h_wait or release would reach a freed engine
      return hc::set_error(HC_ERR_INVALID, "%lld request(s) not released; release them first", (long long)e->live);
  }
  if (e->workers.empty()) run_inline(e, nullptr);
  {
    std::lock_guard<std::mutex> lk(e->mu);
    e->stop = true;
    e->cv_work.notify_all();
  }
  for (auto& t : e->workers)
    if (t.joinable()) t.join();
  delete e;
  return HC_OK;
}

int hc_cache_fingerprint(const hc_pool_desc* desc, const char* model, int32_t tp_size, uint64_t* out) {
  if (!out || !model) return hc::set_error(HC_ERR_INVALID, "null argument");
  if (tp_size < 1) return hc::set_error(HC_ERR_INVALID, "tp_size must be >= 1");
  hc::Layout L;
  char msg[256];
  int rc = hc::layout_from_desc(desc, &L, msg, sizeof(msg));
  if (rc != HC_OK) return hc::set_error(rc, "%s", msg);
  const char* layout = L.layout == HC_LAYOUT_KV_SPLIT_SHARD            ? "kv_split_shard"
                       : L.layout == HC_LAYOUT_PAGE_FIRST_TOKEN_MAJOR ? "page_first_token_major"
                                                                       : "page_first";
  std::string s = "hicache-layout-v1;model=";
  s += model;
  s += ";layout=";
  s += layout;
  s += ";layers=" + std::to_string(L.L) + ";page_size=" + std::to_string(L.P) + ";tp=" + std::to_string(tp_size);
  s += ";tensors=";
  for (int b = 0; b < L.nsub; b++) {
    if (b) s += ",";
    s += (L.gran[b] == HC_PAGE_BLOCKS ? "b:" : "r:") + std::to_string(L.elem[b]);
  }
  s += ";align=" + std::to_string(L.layout == HC_LAYOUT_KV_SPLIT_SHARD ? L.align : 0);
  *out = fnv1a64(s);
  return HC_OK;
}

}  // extern "C"
