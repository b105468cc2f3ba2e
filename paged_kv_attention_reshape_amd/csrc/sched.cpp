// Host-side continuous-batching scheduler and paged block allocator
// (declared in pa_sched.h, which states the behaviour and cites the pages).
//
// Data layout: requests live in a vector indexed by an internal slot, with a
// hash map from request id to slot; the running queue is a vector of slots in
// FCFS order, the waiting queue a deque; the free list a deque of physical
// block ids (reservations from the front, releases to the back).  Every
// request keeps its block list in logical order, committed blocks first and
// the pending plan's reservations last, so a rollback pops the tail.  A step
// touches only the running requests and the head of the waiting queue.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <deque>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa_sched.h"

namespace {

thread_local std::string g_err;

pa_status fail(pa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

enum Status : int8_t { kWaiting, kRunning, kFinished, kCancelled };

struct Req {
  int64_t id;
  int32_t prompt_len, output_len;
  int32_t generated = 0;
  int32_t num_computed = 0;
  int32_t reserved = 0;       // trailing blocks reserved by the pending plan
  int32_t pending_n = 0;      // tokens the pending plan schedules for it
  int32_t preemptions = 0;
  Status status = kWaiting;
  std::vector<int32_t> blocks;
  int64_t num_tokens() const { return (int64_t)prompt_len + generated; }
};

struct SchedEntry {
  int32_t slot;
  int32_t computed;
  int32_t n;
};

struct Preemption {
  int64_t id;
  int64_t held;
  int64_t released;
};

}  // namespace

struct pa_sched {
  int32_t B, capacity, max_seqs, budget, chunk;
  double hook_prob;
  int32_t hook_left;
  std::vector<double> hook_draws;
  size_t hook_next = 0;

  std::deque<int32_t> free_list;
  int64_t q_reserved = 0, q_committed = 0;
  std::vector<Req> reqs;
  std::unordered_map<int64_t, int32_t> slot_of;
  std::deque<int32_t> waiting;
  std::vector<int32_t> running;

  // pending plan
  bool pending = false;
  std::vector<SchedEntry> sched;
  std::vector<int32_t> new_running;
  std::vector<int32_t> admitted;
  std::vector<Preemption> preempted;

  pa_sched_metrics m{};

  // ---- pool -----------------------------------------------------------------
  void reserve(Req& r, int32_t k) {
    for (int32_t i = 0; i < k; ++i) {
      r.blocks.push_back(free_list.front());
      free_list.pop_front();
    }
    r.reserved += k;
    q_reserved += k;
    m.peak_used = std::max<int64_t>(m.peak_used, q_reserved + q_committed);
  }

  int64_t release_all(Req& r) {
    const int64_t n = (int64_t)r.blocks.size();
    free_list.insert(free_list.end(), r.blocks.begin(), r.blocks.end());
    q_reserved -= r.reserved;
    q_committed -= n - r.reserved;
    r.blocks.clear();
    r.reserved = 0;
    return n;
  }

  // Delta q: blocks covering num_computed + n positions minus blocks held
  int64_t blocks_needed(const Req& r, int64_t n) const {
    return ((int64_t)r.num_computed + n + B - 1) / B - (int64_t)r.blocks.size();
  }

  bool can_append(const Req& r, int64_t n) {
    if (hook_prob > 0 && hook_left > 0 && hook_next < hook_draws.size()) {
      const double u = hook_draws[hook_next++];
      if (u < hook_prob) {
        --hook_left;
        ++m.allocation_failures;
        return false;
      }
    }
    if (blocks_needed(r, n) <= (int64_t)free_list.size()) return true;
    ++m.allocation_failures;
    return false;
  }

  void preempt(int32_t slot) {
    Req& v = reqs[slot];
    const int64_t held = v.num_computed;
    const int64_t n = release_all(v);
    v.num_computed = 0;
    v.pending_n = 0;
    v.status = kWaiting;
    ++v.preemptions;
    waiting.push_front(slot);
    preempted.push_back({v.id, held, n});
    ++m.preemptions;
    m.recompute_tokens += held;
  }

  bool conserved() const {
    return (int64_t)free_list.size() + q_reserved + q_committed == capacity;
  }

  // ---- one step ---------------------------------------------------------------
  void plan() {
    int64_t left = budget;
    sched.clear();
    new_running.clear();
    admitted.clear();
    preempted.clear();
    std::vector<int32_t> queue(running);
    size_t i = 0;
    while (i < queue.size()) {
      Req& r = reqs[queue[i]];
      const int64_t n = std::min<int64_t>(std::min<int64_t>(r.num_tokens() - r.num_computed, chunk), left);
      if (n <= 0) {
        new_running.push_back(queue[i]);
        ++i;
        continue;
      }
      bool ok = true;
      while (!can_append(r, n)) {
        if (queue.size() - 1 > i) {          // someone behind r: preempt the tail
          const int32_t v = queue.back();
          queue.pop_back();
          preempt(v);
        } else {                             // r is the last: it preempts itself
          const int32_t self = queue[i];
          queue.erase(queue.begin() + (long)i);
          preempt(self);
          ok = false;
          break;
        }
      }
      if (!ok) continue;
      reserve(r, (int32_t)blocks_needed(r, n));
      r.pending_n = (int32_t)n;
      sched.push_back({queue[i], r.num_computed, (int32_t)n});
      left -= n;
      new_running.push_back(queue[i]);
      ++i;
    }
    if (preempted.empty()) {
      while (!waiting.empty() && (int64_t)new_running.size() < max_seqs && left > 0) {
        const int32_t slot = waiting.front();
        Req& r = reqs[slot];
        const int64_t n = std::min<int64_t>(std::min<int64_t>(r.num_tokens() - r.num_computed, chunk), left);
        const int64_t k = blocks_needed(r, n);
        if (k > (int64_t)free_list.size()) break;
        waiting.pop_front();
        reserve(r, (int32_t)k);
        r.status = kRunning;
        r.pending_n = (int32_t)n;
        sched.push_back({slot, r.num_computed, (int32_t)n});
        left -= n;
        new_running.push_back(slot);
        admitted.push_back(slot);
        ++m.admissions;
      }
    }
    running = new_running;
    pending = true;
  }

  void commit(std::vector<int64_t>& done) {
    q_committed += q_reserved;
    q_reserved = 0;
    std::vector<int32_t> next;
    next.reserve(new_running.size());
    for (const int32_t slot : new_running) {
      Req& r = reqs[slot];
      r.reserved = 0;
      if (r.pending_n > 0) {
        r.num_computed += r.pending_n;
        m.scheduled_tokens += r.pending_n;
        r.pending_n = 0;
        if (r.num_computed == r.num_tokens()) {
          ++r.generated;
          if (r.generated >= r.output_len) {
            r.status = kFinished;
            release_all(r);
            ++m.finished;
            done.push_back(r.id);
            continue;
          }
        }
      }
      next.push_back(slot);
    }
    running.swap(next);
    pending = false;
    ++m.steps;
  }

  void rollback() {
    for (const int32_t slot : new_running) {
      Req& r = reqs[slot];
      if (r.reserved > 0) {
        const size_t keep = r.blocks.size() - (size_t)r.reserved;
        free_list.insert(free_list.end(), r.blocks.begin() + (long)keep, r.blocks.end());
        r.blocks.resize(keep);
        q_reserved -= r.reserved;
        r.reserved = 0;
      }
      r.pending_n = 0;
    }
    for (auto it = admitted.rbegin(); it != admitted.rend(); ++it) {
      reqs[*it].status = kWaiting;
      waiting.push_front(*it);
    }
    std::vector<int32_t> next;
    for (const int32_t slot : new_running)
      if (std::find(admitted.begin(), admitted.end(), slot) == admitted.end()) next.push_back(slot);
    running.swap(next);
    pending = false;
    ++m.rollbacks;
  }
};

extern "C" {

const char* pa_sched_last_error(void) { return g_err.c_str(); }

pa_status pa_sched_create(const pa_sched_config* cfg, pa_sched** out) {
  g_err.clear();
  if (out == nullptr || cfg == nullptr) return fail(PA_ERR_NULL_PTR, "NULL argument");
  *out = nullptr;
  if (cfg->num_blocks <= 0 || cfg->block_size <= 0 || cfg->max_num_seqs <= 0 ||
      cfg->max_num_batched_tokens <= 0 || cfg->chunk <= 0)
    return fail(PA_ERR_BAD_SHAPE, "sizes must be positive");
  if (cfg->block_order == nullptr) return fail(PA_ERR_NULL_PTR, "block_order is NULL");
  if (!(cfg->hook_prob >= 0.0 && cfg->hook_prob <= 1.0) || cfg->hook_max < 0 || cfg->n_hook_draws < 0)
    return fail(PA_ERR_BAD_SHAPE, "hook_prob must be in [0, 1], hook_max and n_hook_draws >= 0");
  if (cfg->n_hook_draws > 0 && cfg->hook_draws == nullptr) return fail(PA_ERR_NULL_PTR, "hook_draws is NULL");
  std::vector<char> seen((size_t)cfg->num_blocks, 0);
  for (int32_t i = 0; i < cfg->num_blocks; ++i) {
    const int32_t b = cfg->block_order[i];
    if (b < 0 || b >= cfg->num_blocks || seen[(size_t)b])
      return fail(PA_ERR_OUT_OF_RANGE, "block_order is not a permutation (entry %d = %d)", i, b);
    seen[(size_t)b] = 1;
  }
  pa_sched* s = new (std::nothrow) pa_sched();
  if (s == nullptr) return fail(PA_ERR_BAD_SHAPE, "out of host memory");
  s->B = cfg->block_size;
  s->capacity = cfg->num_blocks;
  s->max_seqs = cfg->max_num_seqs;
  s->budget = cfg->max_num_batched_tokens;
  s->chunk = cfg->chunk;
  s->hook_prob = cfg->hook_prob;
  s->hook_left = cfg->hook_max;
  s->hook_draws.assign(cfg->hook_draws, cfg->hook_draws + cfg->n_hook_draws);
  s->free_list.assign(cfg->block_order, cfg->block_order + cfg->num_blocks);
  s->m.q_capacity = cfg->num_blocks;
  *out = s;
  return PA_OK;
}

void pa_sched_destroy(pa_sched* s) { delete s; }

pa_status pa_sched_add_request(pa_sched* s, int64_t request_id, int32_t prompt_len,
                               int32_t output_len) {
  g_err.clear();
  if (s == nullptr) return fail(PA_ERR_NULL_PTR, "NULL scheduler");
  if (prompt_len < 1 || output_len < 1)
    return fail(PA_ERR_BAD_SHAPE, "prompt_len %d and output_len %d must be >= 1", prompt_len, output_len);
  if (s->slot_of.count(request_id)) return fail(PA_ERR_BAD_SHAPE, "request %lld already added", (long long)request_id);
  if (s->reqs.size() >= (size_t)INT32_MAX) return fail(PA_ERR_BAD_SHAPE, "too many requests");
  Req r;
  r.id = request_id;
  r.prompt_len = prompt_len;
  r.output_len = output_len;
  const int32_t slot = (int32_t)s->reqs.size();
  s->reqs.push_back(std::move(r));
  s->slot_of.emplace(request_id, slot);
  s->waiting.push_back(slot);
  return PA_OK;
}

pa_status pa_sched_schedule(pa_sched* s, pa_sched_plan_info* info) {
  g_err.clear();
  if (s == nullptr) return fail(PA_ERR_NULL_PTR, "NULL scheduler");
  if (s->pending) return fail(PA_ERR_BAD_STATE, "a plan is pending: commit or roll it back first");
  s->plan();
  if (!s->conserved()) return fail(PA_ERR_BAD_STATE, "block conservation broken");  // cannot happen
  if (info != nullptr) {
    info->num_reqs = (int32_t)s->sched.size();
    info->num_preempted = (int32_t)s->preempted.size();
    int64_t toks = 0;
    int32_t mb = 0;
    for (const SchedEntry& e : s->sched) {
      toks += e.n;
      mb = std::max(mb, (int32_t)s->reqs[e.slot].blocks.size());
    }
    info->num_tokens = toks;
    info->max_blocks = mb;
    info->q_free = (int32_t)s->free_list.size();
    info->q_reserved = (int32_t)s->q_reserved;
    info->q_committed = (int32_t)s->q_committed;
  }
  return PA_OK;
}

pa_status pa_sched_plan_copy(const pa_sched* s, int64_t* request_ids, int32_t* num_computed,
                             int32_t* query_lens, int32_t cap_reqs, int32_t* block_table,
                             int32_t max_blocks_per_req, int64_t* preempted,
                             int32_t cap_preempted) {
  g_err.clear();
  if (s == nullptr) return fail(PA_ERR_NULL_PTR, "NULL scheduler");
  if (!s->pending) return fail(PA_ERR_BAD_STATE, "no pending plan");
  const size_t R = s->sched.size();
  if ((size_t)std::max(cap_reqs, 0) < R)
    return fail(PA_ERR_BAD_SHAPE, "cap_reqs %d < %zu scheduled requests", cap_reqs, R);
  if ((size_t)std::max(cap_preempted, 0) < s->preempted.size())
    return fail(PA_ERR_BAD_SHAPE, "cap_preempted %d < %zu preemptions", cap_preempted, s->preempted.size());
  for (const SchedEntry& e : s->sched)
    if ((int64_t)s->reqs[e.slot].blocks.size() > max_blocks_per_req)
      return fail(PA_ERR_BAD_SHAPE, "max_blocks_per_req %d too small", max_blocks_per_req);
  if (R > 0 && (!request_ids || !num_computed || !query_lens || !block_table))
    return fail(PA_ERR_NULL_PTR, "NULL output array");
  if (!s->preempted.empty() && preempted == nullptr) return fail(PA_ERR_NULL_PTR, "NULL preempted array");
  for (size_t i = 0; i < R; ++i) {
    const SchedEntry& e = s->sched[i];
    const Req& r = s->reqs[e.slot];
    request_ids[i] = r.id;
    num_computed[i] = e.computed;
    query_lens[i] = e.n;
    int32_t* row = block_table + i * (size_t)max_blocks_per_req;
    const size_t nb = r.blocks.size();
    std::copy(r.blocks.begin(), r.blocks.end(), row);
    std::fill(row + nb, row + max_blocks_per_req, -1);
  }
  for (size_t i = 0; i < s->preempted.size(); ++i) {
    preempted[3 * i] = s->preempted[i].id;
    preempted[3 * i + 1] = s->preempted[i].held;
    preempted[3 * i + 2] = s->preempted[i].released;
  }
  return PA_OK;
}

pa_status pa_sched_commit(pa_sched* s, int64_t* finished_ids, int32_t cap_finished,
                          int32_t* n_finished) {
  g_err.clear();
  if (s == nullptr) return fail(PA_ERR_NULL_PTR, "NULL scheduler");
  if (!s->pending) return fail(PA_ERR_BAD_STATE, "no pending plan to commit");
  // count the requests that will finish before changing anything
  int64_t will = 0;
  for (const int32_t slot : s->new_running) {
    const Req& r = s->reqs[slot];
    if (r.pending_n > 0 && r.num_computed + r.pending_n == r.num_tokens() && r.generated + 1 >= r.output_len) ++will;
  }
  if (will > std::max(cap_finished, 0) || (will > 0 && finished_ids == nullptr))
    return fail(PA_ERR_BAD_SHAPE, "%lld requests finish, cap_finished is %d", (long long)will, cap_finished);
  std::vector<int64_t> done;
  s->commit(done);
  for (size_t i = 0; i < done.size(); ++i) finished_ids[i] = done[i];
  if (n_finished != nullptr) *n_finished = (int32_t)done.size();
  return PA_OK;
}

pa_status pa_sched_rollback(pa_sched* s) {
  g_err.clear();
  if (s == nullptr) return fail(PA_ERR_NULL_PTR, "NULL scheduler");
  if (!s->pending) return fail(PA_ERR_BAD_STATE, "no pending plan to roll back");
  s->rollback();
  return PA_OK;
}

pa_status pa_sched_cancel(pa_sched* s, int64_t request_id) {
  g_err.clear();
  if (s == nullptr) return fail(PA_ERR_NULL_PTR, "NULL scheduler");
  auto it = s->slot_of.find(request_id);
  if (it == s->slot_of.end()) return fail(PA_ERR_OUT_OF_RANGE, "unknown request %lld", (long long)request_id);
  const int32_t slot = it->second;
  Req& r = s->reqs[slot];
  if (r.status == kFinished || r.status == kCancelled) return PA_OK;
  s->release_all(r);
  r.pending_n = 0;
  auto drop = [slot](std::vector<int32_t>& v) { v.erase(std::remove(v.begin(), v.end(), slot), v.end()); };
  drop(s->running);
  s->waiting.erase(std::remove(s->waiting.begin(), s->waiting.end(), slot), s->waiting.end());
  if (s->pending) {
    s->sched.erase(std::remove_if(s->sched.begin(), s->sched.end(),
                                  [slot](const SchedEntry& e) { return e.slot == slot; }),
                   s->sched.end());
    drop(s->new_running);
    drop(s->admitted);
  }
  r.status = kCancelled;
  ++s->m.cancelled;
  return PA_OK;
}

pa_status pa_sched_get_metrics(const pa_sched* s, pa_sched_metrics* m) {
  g_err.clear();
  if (s == nullptr || m == nullptr) return fail(PA_ERR_NULL_PTR, "NULL argument");
  *m = s->m;
  m->q_free = (int64_t)s->free_list.size();
  m->q_reserved = s->q_reserved;
  m->q_committed = s->q_committed;
  m->q_capacity = s->capacity;
  m->q_live = s->q_reserved + s->q_committed;
  int64_t tail = 0;
  for (const int32_t slot : s->running) {
    const Req& r = s->reqs[slot];
    if (!r.blocks.empty())
      tail += ((int64_t)r.blocks.size() - r.reserved) * s->B - r.num_computed;
  }
  m->tail_waste = tail;
  m->running = (int64_t)s->running.size();
  m->waiting = (int64_t)s->waiting.size();
  return PA_OK;
}

}  // extern "C"
