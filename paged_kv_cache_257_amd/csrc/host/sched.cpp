// Iteration-level continuous-batching scheduler with preemption (see
// pkv_sched_* in pkv.h for the rules; "PagedAttention e continuous
// batching", 01 · Conceito, the scheduler and metrics paragraphs).
#include <algorithm>
#include <deque>
#include <string>
#include <unordered_map>
#include <vector>

#include "pool_internal.h"

using pkv::fail;

namespace {

struct Req {
  pkv_request r;
  pkv_request_state st;
  int32_t prefilled = 0;  // K/V tokens present in the current sequence
  int32_t target = 0;     // K/V tokens the current prefill must reach
};

}  // namespace

struct pkv_sched {
  pkv_pool* pool = nullptr;
  pkv_sched_config cfg{};
  std::vector<Req> reqs;
  std::vector<int32_t> arrival_order;  // request ids by (arrival, id)
  size_t next_arrival = 0;
  std::deque<int32_t> waiting;
  std::vector<int32_t> running;        // admission order
  std::vector<int32_t> retired;        // finished last step, freed at the next
  std::unordered_map<int32_t, int32_t> holder;  // prefix id -> request holding it
  int32_t t = 0;
  pkv_sched_stats_t stats{};
};

namespace {

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

int32_t free_blocks(const pkv_pool* p) { return int32_t(p->free_stack.size()); }

// Blocks an append of n tokens to `seq` takes (new blocks + a copy-on-write).
int64_t append_need(const pkv_pool* p, int32_t seq, int32_t n) {
  const pkv_seq_state* s = pkv::find_seq(p, seq);
  const int32_t bs = p->desc.block_size;
  int64_t need = blocks_for(int64_t(s->length) + n, bs) - int64_t(s->table.size());
  if (n > 0 && s->length % bs != 0 && p->rc[s->table.back()] > 1) need += 1;
  return need;
}

bool decoding(const Req& q) { return q.prefilled == q.target && q.st.generated < q.r.output_len; }

// A running request (other than `except`) whose sequence holds the prefix.
int32_t find_holder(const pkv_sched* s, int32_t prefix_id, int32_t except) {
  for (int32_t id : s->running) {
    const Req& q = s->reqs[id];
    if (id != except && q.r.prefix_id == prefix_id && q.prefilled >= q.r.prefix_len) return id;
  }
  return -1;
}

void drop_holder(pkv_sched* s, int32_t id) {
  const Req& q = s->reqs[id];
  if (q.r.prefix_id < 0) return;
  auto it = s->holder.find(q.r.prefix_id);
  if (it == s->holder.end() || it->second != id) return;
  const int32_t h = find_holder(s, q.r.prefix_id, id);
  if (h < 0)
    s->holder.erase(it);
  else
    it->second = h;
}

void note_progress(pkv_sched* s, int32_t id) {
  const Req& q = s->reqs[id];
  if (q.r.prefix_id >= 0 && q.r.prefix_len > 0 && q.prefilled >= q.r.prefix_len &&
      !s->holder.count(q.r.prefix_id))
    s->holder[q.r.prefix_id] = id;
}

// A prefill reached its target: the first token, unless it was generated
// before a preemption.
void prefill_done(pkv_sched* s, Req& q) {
  if (q.st.generated == 0) {
    q.st.generated = 1;
    q.st.first_token_at = s->t;
  }
}

}  // namespace

extern "C" {

pkv_status pkv_sched_create(pkv_pool* pool, const pkv_sched_config* cfg, const pkv_request* reqs,
                            int32_t n, pkv_sched** out) {
  if (!pool || !cfg || !out || n < 0 || (n > 0 && !reqs)) return fail(PKV_E_BAD_ARG, "null argument");
  if (cfg->max_batch_tokens < 1 || cfg->chunk_tokens < 1 || cfg->max_running < 1)
    return fail(PKV_E_BAD_ARG, "bad scheduler config");
  const int32_t bs = pool->desc.block_size;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_request& r = reqs[i];
    if (r.arrival < 0 || r.prompt_len < 1 || r.output_len < 1)
      return fail(PKV_E_BAD_ARG, "request " + std::to_string(i) + ": bad arrival / lengths");
    if (r.prefix_id >= 0 && (r.prefix_len < 0 || r.prefix_len % bs != 0 || r.prefix_len >= r.prompt_len))
      return fail(PKV_E_BAD_ARG, "request " + std::to_string(i) +
                                     ": prefix_len must be a multiple of block_size below prompt_len");
  }
  pkv_sched* s = new (std::nothrow) pkv_sched();
  if (!s) return fail(PKV_E_BAD_ARG, "out of host memory");
  s->pool = pool;
  s->cfg = *cfg;
  s->reqs.resize(n);
  for (int32_t i = 0; i < n; ++i) {
    Req& q = s->reqs[i];
    q.r = reqs[i];
    if (q.r.prefix_id < 0) q.r.prefix_len = 0;
    q.st = {PKV_REQ_PENDING, -1, -1, -1, -1, 0, 0, 0};
    s->arrival_order.push_back(i);
  }
  std::stable_sort(s->arrival_order.begin(), s->arrival_order.end(),
                   [s](int32_t a, int32_t b) { return s->reqs[a].r.arrival < s->reqs[b].r.arrival; });
  *out = s;
  return PKV_OK;
}

pkv_status pkv_sched_destroy(pkv_sched* s) {
  delete s;
  return PKV_OK;
}

pkv_status pkv_sched_step(pkv_sched* s, pkv_sched_item* items, int32_t cap, pkv_sched_step_info* info) {
  if (!s || !info || (cap > 0 && !items)) return fail(PKV_E_BAD_ARG, "null argument");
  if (cap < s->cfg.max_running) return fail(PKV_E_BAD_ARG, "items needs room for max_running entries");
  pkv_pool* p = s->pool;
  const int32_t bs = p->desc.block_size;
  pkv_sched_step_info ev{};
  ev.iteration = s->t;
  int32_t k = 0;
  auto emit = [&](int32_t id, int32_t kind, int32_t pos, int32_t n) {
    items[k++] = {id, s->reqs[id].st.seq, kind, pos, n};
  };

  // 0. sequences that finished in the previous iteration leave (their items
  //    were valid until now)
  for (int32_t id : s->retired) {
    Req& q = s->reqs[id];
    if (pkv_status st = pkv_seq_free(p, q.st.seq)) return st;
    q.st.seq = -1;
  }
  s->retired.clear();

  // 1. arrivals
  while (s->next_arrival < s->arrival_order.size() &&
         s->reqs[s->arrival_order[s->next_arrival]].r.arrival <= s->t) {
    const int32_t id = s->arrival_order[s->next_arrival++];
    s->reqs[id].st.state = PKV_REQ_WAITING;
    s->waiting.push_back(id);
  }

  // 2. room for one token per decoding sequence and for the next slice of
  //    the oldest running prefill, preempting the newest running sequences
  //    (never that prefill's own or older ones): the oldest running request
  //    always advances, so sliced prefills cannot hold every block while
  //    waiting on each other
  while (!s->running.empty()) {
    int64_t dec_need = 0, pf_need = 0, n_dec = 0;
    int32_t first_pf = -1;
    for (int32_t id : s->running) {
      const Req& q = s->reqs[id];
      if (decoding(q)) {
        dec_need += append_need(p, q.st.seq, 1);
        n_dec++;
      } else if (first_pf < 0 && q.prefilled < q.target) {
        first_pf = id;
      }
    }
    if (first_pf >= 0) {
      const Req& q = s->reqs[first_pf];
      const int64_t n = std::min<int64_t>({q.target - q.prefilled, s->cfg.chunk_tokens,
                                           int64_t(s->cfg.max_batch_tokens) - n_dec});
      if (n > 0) pf_need = append_need(p, q.st.seq, int32_t(n));
    }
    const int64_t free_now = free_blocks(p);
    // decodes come first (any newest sequence may go); the prefill's slice
    // only displaces sequences newer than it
    if (dec_need <= free_now && (dec_need + pf_need <= free_now || s->running.back() == first_pf)) break;
    const int32_t v = s->running.back();
    Req& q = s->reqs[v];
    drop_holder(s, v);
    if (pkv_status st = pkv_seq_free(p, q.st.seq)) return st;
    s->running.pop_back();
    q.st.seq = -1;
    q.st.state = PKV_REQ_WAITING;
    q.st.preemptions++;
    q.prefilled = 0;
    s->waiting.push_front(v);
    s->stats.preemptions++;
    ev.preempted++;
  }

  // 3. decode
  for (int32_t id : s->running) {
    Req& q = s->reqs[id];
    if (!decoding(q)) continue;
    const int32_t pos = q.prefilled;
    if (pkv_status st = pkv_seq_append(p, q.st.seq, 1, nullptr)) return st;
    q.prefilled++;
    q.target++;
    q.st.generated++;
    emit(id, PKV_ITEM_DECODE, pos, 1);
    ev.decode_tokens++;
  }
  int64_t budget = int64_t(s->cfg.max_batch_tokens) - ev.decode_tokens;

  // 4. prefills already running
  for (int32_t id : s->running) {
    if (budget <= 0) break;
    Req& q = s->reqs[id];
    if (q.prefilled >= q.target) continue;
    const int32_t n = int32_t(std::min<int64_t>({q.target - q.prefilled, s->cfg.chunk_tokens, budget}));
    if (append_need(p, q.st.seq, n) > free_blocks(p)) break;
    const int32_t pos = q.prefilled;
    if (pkv_status st = pkv_seq_append(p, q.st.seq, n, nullptr)) return st;
    q.prefilled += n;
    budget -= n;
    ev.prefill_tokens += n;
    emit(id, PKV_ITEM_PREFILL, pos, n);
    note_progress(s, id);
    if (q.prefilled == q.target) prefill_done(s, q);
  }

  // 5. admission, first come first served
  while (budget > 0 && !s->waiting.empty() && int32_t(s->running.size()) < s->cfg.max_running) {
    const int32_t id = s->waiting.front();
    Req& q = s->reqs[id];
    const int64_t final_blocks = blocks_for(int64_t(q.r.prompt_len) + q.r.output_len - 1, bs);
    if (final_blocks > p->desc.num_blocks || final_blocks > p->desc.max_blocks_per_seq) {
      s->waiting.pop_front();
      q.st.state = PKV_REQ_REJECTED;
      s->stats.rejected++;
      ev.rejected++;
      continue;
    }
    const int32_t target = q.r.prompt_len + std::max(q.st.generated - 1, 0);
    auto hit = q.r.prefix_id >= 0 && q.r.prefix_len > 0 ? s->holder.find(q.r.prefix_id) : s->holder.end();
    const int32_t start = hit != s->holder.end() ? q.r.prefix_len : 0;
    const int32_t n = int32_t(std::min<int64_t>({target - start, s->cfg.chunk_tokens, budget}));
    const int64_t need = blocks_for(int64_t(start) + n, bs) - blocks_for(start, bs);
    if (need > free_blocks(p)) break;
    int32_t seq = -1;
    if (start > 0) {
      if (pkv_status st = pkv_seq_fork_prefix(p, s->reqs[hit->second].st.seq, start, &seq)) return st;
      if (pkv_status st = pkv_seq_append(p, seq, n, nullptr)) return st;
    } else {
      if (pkv_status st = pkv_seq_alloc(p, n, &seq, nullptr)) return st;
    }
    s->waiting.pop_front();
    s->running.push_back(id);
    q.st.state = PKV_REQ_RUNNING;
    q.st.seq = seq;
    if (q.st.admitted_at < 0) q.st.admitted_at = s->t;
    q.st.prefix_hit_tokens += start;
    q.prefilled = start + n;
    q.target = target;
    s->stats.prompt_tokens_admitted += target;
    s->stats.prefix_hit_tokens += start;
    budget -= n;
    ev.prefill_tokens += n;
    ev.admitted++;
    emit(id, PKV_ITEM_PREFILL, start, n);
    note_progress(s, id);
    if (q.prefilled == q.target) prefill_done(s, q);
  }

  // 6. retire finished requests
  for (size_t i = 0; i < s->running.size();) {
    const int32_t id = s->running[i];
    Req& q = s->reqs[id];
    if (q.prefilled == q.target && q.st.generated >= q.r.output_len) {
      drop_holder(s, id);
      s->retired.push_back(id);
      q.st.state = PKV_REQ_FINISHED;
      q.st.finished_at = s->t;
      s->running.erase(s->running.begin() + i);
      s->stats.finished++;
      ev.finished++;
    } else {
      ++i;
    }
  }

  s->stats.prefill_tokens += ev.prefill_tokens;
  s->stats.decode_tokens += ev.decode_tokens;
  s->t++;
  s->stats.iterations = s->t;
  s->stats.waiting = int64_t(s->waiting.size());
  s->stats.running = int64_t(s->running.size());
  ev.n_items = k;
  *info = ev;
  return PKV_OK;
}

pkv_status pkv_sched_request(const pkv_sched* s, int32_t request, pkv_request_state* out) {
  if (!s || !out) return fail(PKV_E_BAD_ARG, "null argument");
  if (request < 0 || request >= int32_t(s->reqs.size())) return fail(PKV_E_BAD_ARG, "unknown request");
  *out = s->reqs[request].st;
  return PKV_OK;
}

pkv_status pkv_sched_stats(const pkv_sched* s, pkv_sched_stats_t* out) {
  if (!s || !out) return fail(PKV_E_BAD_ARG, "null argument");
  *out = s->stats;
  return PKV_OK;
}

}  // extern "C"
