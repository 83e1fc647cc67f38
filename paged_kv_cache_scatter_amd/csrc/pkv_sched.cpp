// Host block manager and continuous-batching scheduler ("Build a Mini vLLM",
// sections 2, 5, 6 and 8). Decisions only: the caller runs the kernels.
#include "../../include/pkv_sched.h"

#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <deque>
#include <unordered_map>
#include <vector>

namespace pkv {
void set_error(const char* fmt, ...);
}

namespace {

struct Request {
  int32_t rid;
  int32_t prompt_len;   // grows by the generated tokens on preemption
  int32_t max_new;
  int32_t stop_after;
  int32_t generated = 0;   // tokens produced so far (kept across preemption)
  bool fresh = false;      // admitted in the current step
};

// Free list + tables ("The paged KV cache").
struct BlockManager {
  int32_t num_blocks, block_size;
  std::vector<int32_t> free;   // the end of the list is handed out first
  std::unordered_map<int32_t, std::vector<int32_t>> table;
  std::unordered_map<int32_t, int32_t> length;

  BlockManager(int32_t nb, int32_t bs) : num_blocks(nb), block_size(bs) {
    free.reserve(nb);
    for (int32_t i = 0; i < nb; ++i) free.push_back(i);
  }
  bool can_admit(int32_t n_tokens) const {
    return (int64_t)free.size() >= ((int64_t)n_tokens + 1 + block_size - 1) / block_size;
  }
  void start(int32_t sid) {
    table[sid].clear();
    length[sid] = 0;
  }
  // reserve the slot of the sequence's next token
  void append_slot(int32_t sid) {
    const int32_t pos = length[sid];
    if (pos % block_size == 0) {
      table[sid].push_back(free.back());
      free.pop_back();
    }
    length[sid] = pos + 1;
  }
  void release(int32_t sid) {
    auto& t = table[sid];
    free.insert(free.end(), t.begin(), t.end());
    table.erase(sid);
    length.erase(sid);
  }
  int64_t allocated_tokens() const {
    return (int64_t)(num_blocks - (int32_t)free.size()) * block_size;
  }
  int64_t used_tokens() const {
    int64_t u = 0;
    for (const auto& kv : length) u += kv.second;
    return u;
  }
};

struct Hist {
  int32_t running;
  int64_t naive, allocated, used;
};

}  // namespace

struct pkv_sched {
  BlockManager bm;
  int32_t max_batch;
  bool continuous;
  int32_t max_blocks;
  std::deque<Request> waiting;
  std::vector<Request> running;   // admission order; the back is the youngest
  std::unordered_map<int32_t, bool> known;
  pkv_sched_stats stats{};
  std::vector<Hist> history;

  pkv_sched(int32_t nb, int32_t bs, int32_t mb, bool cont, int32_t maxb)
      : bm(nb, bs), max_batch(mb), continuous(cont), max_blocks(maxb) {}

  void copy_table(int32_t sid, int32_t* row) const {
    std::fill(row, row + max_blocks, 0);
    const auto& t = bm.table.at(sid);
    std::copy(t.begin(), t.end(), row);
  }

  void admit() {
    while (!waiting.empty() && (int32_t)running.size() < max_batch &&
           bm.can_admit(waiting.front().prompt_len)) {
      Request r = waiting.front();
      waiting.pop_front();
      bm.start(r.rid);
      for (int32_t i = 0; i < r.prompt_len; ++i) bm.append_slot(r.rid);   // prefill writes
      r.generated += 1;   // the prefill's token
      r.fresh = true;
      running.push_back(r);
    }
  }

  void preempt_youngest() {
    Request r = running.back();
    running.pop_back();
    bm.release(r.rid);
    r.prompt_len += r.generated;   // generated tokens folded into the prompt
    r.fresh = false;
    waiting.push_front(r);
    stats.preemptions += 1;
  }
};

extern "C" {

pkv_sched* pkv_sched_create(int32_t num_blocks, int32_t block_size, int32_t max_batch,
                            int32_t continuous, int32_t max_blocks_per_seq) {
  if (num_blocks < 1 || block_size < 1 || max_batch < 1 || max_blocks_per_seq < 1) {
    pkv::set_error("bad sizes: num_blocks %d, block_size %d, max_batch %d, max_blocks %d",
                   num_blocks, block_size, max_batch, max_blocks_per_seq);
    return nullptr;
  }
  return new pkv_sched(num_blocks, block_size, max_batch, continuous != 0, max_blocks_per_seq);
}

void pkv_sched_destroy(pkv_sched* s) { delete s; }

pkv_status pkv_sched_submit(pkv_sched* s, int32_t rid, int32_t prompt_len, int32_t max_new,
                            int32_t stop_after) {
  if (!s) {
    pkv::set_error("scheduler is NULL");
    return PKV_ERR_NULL;
  }
  if (prompt_len < 1 || max_new < 1 || stop_after < 1 || s->known.count(rid)) {
    pkv::set_error("bad request %d: prompt %d, max_new %d, stop_after %d (or rid reused)", rid,
                   prompt_len, max_new, stop_after);
    return PKV_ERR_SHAPE;
  }
  const int64_t bs = s->bm.block_size;
  const int64_t need = ((int64_t)prompt_len + stop_after + bs - 1) / bs;
  if (need > s->max_blocks) {
    pkv::set_error("request %d needs up to %lld blocks, max_blocks_per_seq is %d", rid,
                   (long long)need, s->max_blocks);
    return PKV_ERR_CAPACITY;
  }
  Request r;
  r.rid = rid;
  r.prompt_len = prompt_len;
  r.max_new = max_new;
  r.stop_after = stop_after;
  s->waiting.push_back(r);
  s->known[rid] = true;
  return PKV_OK;
}

int32_t pkv_sched_pending(const pkv_sched* s) {
  return s ? (int32_t)(s->waiting.size() + s->running.size()) : 0;
}

pkv_status pkv_sched_step(pkv_sched* s, pkv_sched_step_out* out) {
  if (!s || !out) {
    pkv::set_error("scheduler or output is NULL");
    return PKV_ERR_NULL;
  }
  if (!out->prefill_rid || !out->prefill_len || !out->prefill_tables || !out->decode_rid ||
      !out->decode_pos || !out->decode_tables) {
    pkv::set_error("an output array of the step is NULL");
    return PKV_ERR_NULL;
  }
  out->num_prefill = out->num_decode = out->num_preempted = out->num_finished = 0;
  const int64_t pre0 = s->stats.preemptions;
  for (auto& r : s->running) r.fresh = false;
  if (s->continuous || s->running.empty()) s->admit();
  // every running request needs one slot this step; evict until that holds
  while (!s->running.empty()) {
    int64_t need = 0;
    for (const auto& r : s->running)
      if (s->bm.length.at(r.rid) % s->bm.block_size == 0) ++need;
    if (need <= (int64_t)s->bm.free.size()) break;
    s->preempt_youngest();
  }
  out->num_preempted = (int32_t)(s->stats.preemptions - pre0);
  if (s->running.empty()) {
    if (!s->waiting.empty()) {
      pkv::set_error("request %d (prompt %d tokens) can never be admitted into %d blocks",
                     s->waiting.front().rid, s->waiting.front().prompt_len, s->bm.num_blocks);
      return PKV_ERR_CAPACITY;
    }
    return PKV_OK;
  }
  // prefill rows: admitted this step and still running
  const int32_t mb = s->max_blocks;
  for (const auto& r : s->running) {
    if (!r.fresh) continue;
    const int32_t i = out->num_prefill++;
    out->prefill_rid[i] = r.rid;
    out->prefill_len[i] = r.prompt_len;
    s->copy_table(r.rid, out->prefill_tables + (size_t)i * mb);
  }
  // decode: one slot per running request, then one generated token each
  std::vector<Request> still;
  still.reserve(s->running.size());
  for (auto& r : s->running) {
    const int32_t pos = s->bm.length.at(r.rid);
    s->bm.append_slot(r.rid);
    const int32_t i = out->num_decode++;
    out->decode_rid[i] = r.rid;
    out->decode_pos[i] = pos;
    s->copy_table(r.rid, out->decode_tables + (size_t)i * mb);
    r.generated += 1;
  }
  for (auto& r : s->running) {
    if (r.generated >= r.stop_after) {
      s->bm.release(r.rid);
      s->stats.requests_done += 1;
      s->stats.tokens_generated += r.generated;
      out->num_finished += 1;
    } else {
      still.push_back(r);
    }
  }
  s->running.swap(still);
  Hist h;
  h.running = (int32_t)s->running.size();
  h.naive = 0;
  for (const auto& r : s->running) h.naive += (int64_t)r.prompt_len + r.max_new;
  h.allocated = s->bm.allocated_tokens();
  h.used = s->bm.used_tokens();
  s->history.push_back(h);
  s->stats.steps += 1;
  s->stats.sum_running += h.running;
  s->stats.sum_naive_tokens += h.naive;
  s->stats.sum_allocated_tokens += h.allocated;
  s->stats.sum_used_tokens += h.used;
  return PKV_OK;
}

pkv_status pkv_sched_get_stats(const pkv_sched* s, pkv_sched_stats* st) {
  if (!s || !st) {
    pkv::set_error("scheduler or stats is NULL");
    return PKV_ERR_NULL;
  }
  *st = s->stats;
  return PKV_OK;
}

int64_t pkv_sched_history(const pkv_sched* s, int32_t* running, int64_t* naive,
                          int64_t* allocated, int64_t* used, int64_t cap) {
  if (!s) return 0;
  const int64_t n = std::min<int64_t>(cap, (int64_t)s->history.size());
  for (int64_t i = 0; i < n; ++i) {
    const Hist& h = s->history[(size_t)i];
    if (running) running[i] = h.running;
    if (naive) naive[i] = h.naive;
    if (allocated) allocated[i] = h.allocated;
    if (used) used[i] = h.used;
  }
  return n;
}

}  // extern "C"
