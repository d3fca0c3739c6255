// dtd_sched.cpp -- continuous batching over the engine's public calls.
//
// The scheduling loop of the Qwen3-8B engine article (4.3.2): requests arrive at any time;
// each iteration takes the ready ones, runs one decode step for all of them together as one
// batch (a matrix product over every sequence instead of one small one each), and hands each
// its next token; nothing waits for the batch to fill.  Here a request is a prompt plus a
// token budget: it is admitted (prefilled) when the KV pool can hold its whole run, decodes in
// every later step alongside whatever else is running, and leaves (its KV blocks freed) when
// it has its tokens, so others join in its place.  The engine's paged KV pool (4.3.1) makes
// admission and release O(1) per block.
//
// A scheduler is a client of the C ABI only: prefill, decode_step, set_sampler, reset_seq
// and prefix_cache_add.  Engine calls are made by whichever thread runs a step (the caller's
// in dtd_sched_step, the scheduler's own after dtd_sched_start); submissions and result
// queries may come from any thread.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <thread>
#include <unordered_map>
#include <vector>

#include "../../include/dtd.h"

namespace {

struct Request {
  std::vector<int32_t> prompt;
  int32_t max_new = 0;
  int32_t stop = -1;
  dtd_sampler sampler{};
  std::vector<int32_t> out;   // generated tokens so far
  int32_t blocks = 0;         // KV blocks reserved for the whole run
  bool done = false;
  dtd_status status = DTD_OK;
};

bool sampler_ok(const dtd_sampler& s) {
  return std::isfinite(s.temperature) && s.temperature >= 0.f && s.top_k >= 0 && s.top_p > 0.f && s.top_p <= 1.f &&
         s.min_p >= 0.f && s.min_p <= 1.f;
}

}  // namespace

struct dtd_sched {
  dtd_engine* e = nullptr;
  dtd_config cfg{};
  hipStream_t st = nullptr;
  int budget = 0;             // prompt tokens admitted per step (at least one request)

  std::mutex mu;              // requests, queue, the stop flag
  std::condition_variable work, finished;
  std::unordered_map<int64_t, Request> reqs;
  std::deque<int64_t> queue;  // submitted, not admitted, in arrival order
  int64_t next_id = 0;
  std::string err;

  std::mutex step_mu;         // one step at a time; held across engine calls
  std::vector<int64_t> active;
  int32_t reserved = 0;       // KV blocks reserved by admitted requests
  int32_t* tok_dev = nullptr;
  int32_t* next_dev = nullptr;
  int32_t* prompt_dev = nullptr;
  size_t prompt_cap = 0;
  int32_t* tok_host = nullptr;   // pinned
  int32_t* next_host = nullptr;  // pinned

  std::thread th;
  bool running = false, stopping = false;
};

namespace {

int64_t seq_of(int64_t id) { return -(id + 1); }   // the scheduler's sequences have negative ids

int32_t blocks_for(const dtd_config& c, int64_t positions) {
  return (int32_t)((positions + c.kv_block_size - 1) / c.kv_block_size);
}

bool run_done(const Request& r) {
  return (int32_t)r.out.size() >= r.max_new || (r.stop >= 0 && !r.out.empty() && r.out.back() == r.stop);
}

// a finished request leaves: with the engine's prefix cache on, its prompt and tokens (all but
// the last, whose KV was never written) are recorded first, so a follow-up that repeats them
// skips their prefill
void retire(dtd_sched* s, int64_t id, Request& r) {
  std::vector<int32_t> all(r.prompt);
  if (r.out.size() > 1) all.insert(all.end(), r.out.begin(), r.out.end() - 1);
  if (r.status == DTD_OK) (void)dtd_prefix_cache_add(s->e, seq_of(id), all.data(), (int32_t)all.size());
  (void)dtd_reset_seq(s->e, seq_of(id));
  s->reserved -= r.blocks;
  std::lock_guard<std::mutex> g(s->mu);
  r.done = true;
  s->finished.notify_all();
}

dtd_status hip_fail(dtd_sched* s, hipError_t r, const char* what) {
  std::lock_guard<std::mutex> g(s->mu);
  s->err = std::string(what) + ": " + hipGetErrorString(r);
  return DTD_E_HIP;
}

// admits one request: prefill its prompt, first token out
dtd_status admit(dtd_sched* s, int64_t id, Request& r) {
  const size_t n = r.prompt.size();
  if (n > s->prompt_cap) {
    if (s->prompt_dev) (void)hipFree(s->prompt_dev);
    s->prompt_dev = nullptr;
    const hipError_t a = hipMalloc((void**)&s->prompt_dev, n * 4);
    if (a != hipSuccess) return hip_fail(s, a, "sched: prompt buffer");
    s->prompt_cap = n;
  }
  hipError_t h = hipMemcpyAsync(s->prompt_dev, r.prompt.data(), n * 4, hipMemcpyHostToDevice, s->st);
  if (h == hipSuccess) h = hipStreamSynchronize(s->st);   // the prompt is pageable host memory
  if (h != hipSuccess) return hip_fail(s, h, "sched: prompt copy");
  dtd_status st = dtd_set_sampler(s->e, seq_of(id), r.sampler.temperature > 0.f ? &r.sampler : nullptr);
  if (st == DTD_OK) st = dtd_prefill(s->e, seq_of(id), s->prompt_dev, (int32_t)n, s->next_dev, nullptr);
  if (st != DTD_OK) return st;
  h = hipMemcpyAsync(s->next_host, s->next_dev, 4, hipMemcpyDeviceToHost, s->st);
  if (h == hipSuccess) h = hipStreamSynchronize(s->st);
  if (h != hipSuccess) return hip_fail(s, h, "sched: token copy");
  std::lock_guard<std::mutex> g(s->mu);
  r.out.push_back(s->next_host[0]);
  return DTD_OK;
}

// Admission (arrival order; a request waits until the pool can hold its whole run and the
// batch has room), then one decode step for every running request, then departures.
dtd_status step_locked(dtd_sched* s, int32_t* pending) {
  const dtd_config& c = s->cfg;
  dtd_status first_err = DTD_OK;
  int admitted_tokens = 0;
  for (;;) {
    int64_t id;
    Request* r;
    {
      std::lock_guard<std::mutex> g(s->mu);
      if (s->queue.empty() || (int32_t)s->active.size() >= c.max_batch) break;
      id = s->queue.front();
      r = &s->reqs.at(id);
      if (s->reserved + r->blocks > c.kv_num_blocks || (int32_t)s->active.size() >= c.max_seqs) break;
      if (admitted_tokens > 0 && admitted_tokens + (int)r->prompt.size() > s->budget) break;
      s->queue.pop_front();
    }
    s->reserved += r->blocks;
    admitted_tokens += (int)r->prompt.size();
    const dtd_status st = admit(s, id, *r);
    if (st != DTD_OK) {
      r->status = st;
      if (first_err == DTD_OK) first_err = st;
      retire(s, id, *r);
      continue;
    }
    if (run_done(*r)) retire(s, id, *r);
    else s->active.push_back(id);
  }
  if (!s->active.empty()) {
    const int B = (int)s->active.size();
    std::vector<int64_t> seqs((size_t)B);
    {
      std::lock_guard<std::mutex> g(s->mu);
      for (int b = 0; b < B; b++) {
        seqs[(size_t)b] = seq_of(s->active[(size_t)b]);
        s->tok_host[b] = s->reqs.at(s->active[(size_t)b]).out.back();
      }
    }
    hipError_t h = hipMemcpyAsync(s->tok_dev, s->tok_host, (size_t)B * 4, hipMemcpyHostToDevice, s->st);
    if (h != hipSuccess) return hip_fail(s, h, "sched: token copy");
    dtd_status st = dtd_decode_step(s->e, B, seqs.data(), s->tok_dev, s->next_dev, nullptr);
    if (st == DTD_OK) {
      h = hipMemcpyAsync(s->next_host, s->next_dev, (size_t)B * 4, hipMemcpyDeviceToHost, s->st);
      if (h == hipSuccess) h = hipStreamSynchronize(s->st);
      if (h != hipSuccess) st = hip_fail(s, h, "sched: token copy");
    }
    std::vector<int64_t> still;
    for (int b = 0; b < B; b++) {
      const int64_t id = s->active[(size_t)b];
      Request& r = s->reqs.at(id);
      {
        std::lock_guard<std::mutex> g(s->mu);
        if (st == DTD_OK) r.out.push_back(s->next_host[b]);
        else r.status = st;
      }
      if (st != DTD_OK || run_done(r)) retire(s, id, r);
      else still.push_back(id);
    }
    s->active.swap(still);
    if (st != DTD_OK && first_err == DTD_OK) first_err = st;
  }
  std::lock_guard<std::mutex> g(s->mu);
  if (pending) *pending = (int32_t)(s->queue.size() + s->active.size());
  if (first_err != DTD_OK && s->err.empty()) s->err = dtd_last_error(s->e);
  return first_err;
}

void loop(dtd_sched* s) {
  for (;;) {
    {
      std::unique_lock<std::mutex> g(s->mu);
      s->work.wait(g, [&] { return s->stopping || !s->queue.empty() || !s->active.empty(); });
      if (s->stopping) return;
    }
    std::lock_guard<std::mutex> g(s->step_mu);
    (void)step_locked(s, nullptr);
  }
}

}  // namespace

extern "C" dtd_status dtd_sched_create(dtd_engine* e, int32_t prompt_budget, dtd_sched** out) {
  if (!out) return DTD_E_ARG;
  *out = nullptr;
  if (!e || prompt_budget < 0) return DTD_E_ARG;
  dtd_sched* s = new dtd_sched();
  s->e = e;
  dtd_status st = dtd_get_config(e, &s->cfg);
  if (st != DTD_OK) {
    delete s;
    return st;
  }
  s->st = (hipStream_t)dtd_get_stream(e);
  s->budget = prompt_budget > 0 ? prompt_budget : 4096;
  const size_t mb = (size_t)s->cfg.max_batch;
  if (hipMalloc((void**)&s->tok_dev, mb * 4) != hipSuccess || hipMalloc((void**)&s->next_dev, mb * 4) != hipSuccess ||
      hipHostMalloc((void**)&s->tok_host, mb * 4, 0) != hipSuccess ||
      hipHostMalloc((void**)&s->next_host, mb * 4, 0) != hipSuccess) {
    dtd_sched_destroy(s);
    return DTD_E_OOM;
  }
  *out = s;
  return DTD_OK;
}

extern "C" dtd_status dtd_sched_submit(dtd_sched* s, const int32_t* prompt_host, int32_t n, int32_t max_new_tokens,
                                       int32_t stop_token, const dtd_sampler* sampler, int64_t* id_out) {
  if (!s || !prompt_host || n < 1 || max_new_tokens < 1 || !id_out) return DTD_E_ARG;
  if (sampler && !sampler_ok(*sampler)) return DTD_E_ARG;
  for (int32_t i = 0; i < n; i++)
    if (prompt_host[i] < 0 || prompt_host[i] >= s->cfg.vocab) return DTD_E_ARG;
  // positions written: the prompt and every generated token but the last
  const int64_t positions = (int64_t)n + max_new_tokens - 1;
  if (positions > s->cfg.max_ctx) return DTD_E_CTX;
  const int32_t blocks = blocks_for(s->cfg, positions);
  if (blocks > s->cfg.kv_num_blocks) return DTD_E_KVFULL;
  Request r;
  r.prompt.assign(prompt_host, prompt_host + n);
  r.max_new = max_new_tokens;
  r.stop = stop_token;
  if (sampler) r.sampler = *sampler;
  r.blocks = blocks;
  std::lock_guard<std::mutex> g(s->mu);
  const int64_t id = s->next_id++;
  s->reqs.emplace(id, std::move(r));
  s->queue.push_back(id);
  *id_out = id;
  s->work.notify_all();
  return DTD_OK;
}

extern "C" dtd_status dtd_sched_step(dtd_sched* s, int32_t* pending) {
  if (!s) return DTD_E_ARG;
  {
    std::lock_guard<std::mutex> g(s->mu);
    if (s->running) return DTD_E_STATE;
  }
  std::lock_guard<std::mutex> g(s->step_mu);
  return step_locked(s, pending);
}

extern "C" int32_t dtd_sched_result(dtd_sched* s, int64_t id, int32_t* tokens_host, int32_t cap, int32_t* done) {
  if (!s || (cap > 0 && !tokens_host)) return DTD_E_ARG;
  std::lock_guard<std::mutex> g(s->mu);
  auto it = s->reqs.find(id);
  if (it == s->reqs.end()) return DTD_E_NOSEQ;
  const Request& r = it->second;
  const int32_t n = (int32_t)r.out.size();
  for (int32_t i = 0; i < std::min(n, cap); i++) tokens_host[i] = r.out[(size_t)i];
  if (done) *done = r.done ? 1 : 0;
  if (r.done && r.status != DTD_OK) return r.status;
  return n;
}

extern "C" dtd_status dtd_sched_release(dtd_sched* s, int64_t id) {
  if (!s) return DTD_E_ARG;
  std::lock_guard<std::mutex> g(s->mu);
  auto it = s->reqs.find(id);
  if (it == s->reqs.end()) return DTD_E_NOSEQ;
  if (!it->second.done) return DTD_E_STATE;
  s->reqs.erase(it);
  return DTD_OK;
}

extern "C" dtd_status dtd_sched_start(dtd_sched* s) {
  if (!s) return DTD_E_ARG;
  std::lock_guard<std::mutex> g(s->mu);
  if (s->running) return DTD_E_STATE;
  s->running = true;
  s->stopping = false;
  s->th = std::thread(loop, s);
  return DTD_OK;
}

extern "C" dtd_status dtd_sched_wait(dtd_sched* s, int64_t id, int32_t timeout_ms) {
  if (!s) return DTD_E_ARG;
  std::unique_lock<std::mutex> g(s->mu);
  auto it = s->reqs.find(id);
  if (it == s->reqs.end()) return DTD_E_NOSEQ;
  const Request& r = it->second;
  if (timeout_ms < 0) s->finished.wait(g, [&] { return r.done; });
  else if (!s->finished.wait_for(g, std::chrono::milliseconds(timeout_ms), [&] { return r.done; }))
    return DTD_E_STATE;
  return r.status;
}

extern "C" dtd_status dtd_sched_stop(dtd_sched* s) {
  if (!s) return DTD_E_ARG;
  {
    std::lock_guard<std::mutex> g(s->mu);
    if (!s->running) return DTD_OK;
    s->stopping = true;
    s->work.notify_all();
  }
  s->th.join();
  std::lock_guard<std::mutex> g(s->mu);
  s->running = false;
  return DTD_OK;
}

extern "C" const char* dtd_sched_last_error(const dtd_sched* s) {
  if (!s) return "null scheduler";
  return s->err.c_str();
}

extern "C" void dtd_sched_destroy(dtd_sched* s) {
  if (!s) return;
  (void)dtd_sched_stop(s);
  {
    std::lock_guard<std::mutex> g(s->step_mu);
    for (int64_t id : s->active) (void)dtd_reset_seq(s->e, seq_of(id));
    s->active.clear();
  }
  if (s->st) (void)hipStreamSynchronize(s->st);
  if (s->tok_dev) (void)hipFree(s->tok_dev);
  if (s->next_dev) (void)hipFree(s->next_dev);
  if (s->prompt_dev) (void)hipFree(s->prompt_dev);
  if (s->tok_host) (void)hipHostFree(s->tok_host);
  if (s->next_host) (void)hipHostFree(s->next_host);
  delete s;
}
