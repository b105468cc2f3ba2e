// Host-side continuous-batching scheduler and paged block allocator
// (declared in pa_sched.h, which states the behaviour and cites the pages).
//
// Data layout: requests live in a vector indexed by an internal slot, with a
// hash map from request id to slot; the running queue is a vector of slots in
// FCFS order, the waiting queue a deque.  Blocks: a free-list deque
// (reservations from the front, releases to the back) and per-block arrays of
// reference count, state (free / reserved by the pending plan / committed)
// and prefix key; the prefix index maps key -> block; cached blocks nobody
// references sit in an intrusive doubly linked list in release order (O(1)
// insert, unlink and evict).  A request keeps its block list in logical
// order; the pending plan's new blocks are its tail, a copy-on-write
// replacement and an attached cached prefix are remembered per request so
// rollback can undo them.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <deque>
#include <string>
#include <unordered_map>
#include <utility>
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
enum BlockState : int8_t { kFree, kReserved, kCommitted };

struct Req {
  int64_t id;
  int32_t prompt_len, output_len;
  int32_t generated = 0;
  int32_t num_computed = 0;
  int32_t registered = 0;     // leading key positions already offered to the index
  int32_t pend_new = 0;       // trailing blocks taken by the pending plan
  int32_t pend_cow_j = -1;    // block index replaced by copy-on-write in the pending plan
  int32_t pend_cow_old = -1;  // ... and the block it replaced
  int32_t pend_match = 0;     // leading blocks attached from the prefix index by the pending plan
  int32_t pending_n = 0;      // tokens the pending plan schedules for it
  int32_t preemptions = 0;
  Status status = kWaiting;
  std::vector<uint64_t> keys;
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
  std::vector<int32_t> ref;
  std::vector<int8_t> state;
  std::vector<uint64_t> key_of;
  std::vector<char> has_key;
  std::unordered_map<uint64_t, int32_t> index;
  // evictable list (release order): head -> oldest; links indexed by block, -1 = none
  std::vector<int32_t> lru_prev, lru_next;
  std::vector<char> in_lru;
  int32_t lru_head = -1, lru_tail = -1;
  int64_t n_evictable = 0;
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
  std::vector<int32_t> taken;
  std::vector<std::pair<int32_t, int32_t>> copies;
  std::vector<Preemption> preempted;

  pa_sched_metrics m{};

  // ---- evictable list ----------------------------------------------------------
  void lru_push_back(int32_t b) {
    lru_prev[b] = lru_tail;
    lru_next[b] = -1;
    if (lru_tail >= 0) lru_next[lru_tail] = b; else lru_head = b;
    lru_tail = b;
    in_lru[b] = 1;
    ++n_evictable;
  }
  void lru_unlink(int32_t b) {
    const int32_t p = lru_prev[b], n = lru_next[b];
    if (p >= 0) lru_next[p] = n; else lru_head = n;
    if (n >= 0) lru_prev[n] = p; else lru_tail = p;
    in_lru[b] = 0;
    --n_evictable;
  }

  // ---- pool ---------------------------------------------------------------------
  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    state[b] = kReserved;
    ref[b] = 1;
    ++q_reserved;
    taken.push_back(b);
    m.peak_used = std::max<int64_t>(m.peak_used, q_reserved + q_committed);
    return b;
  }

  void unref(int32_t b) {
    if (--ref[b] > 0) return;
    if (state[b] == kReserved) {
      state[b] = kFree;
      --q_reserved;
      free_list.push_back(b);
    } else if (has_key[b]) {
      lru_push_back(b);                        // cached: stays committed
    } else {
      state[b] = kFree;
      --q_committed;
      free_list.push_back(b);
    }
  }

  void make_free(int64_t k) {
    while ((int64_t)free_list.size() < k) {
      const int32_t b = lru_head;
      lru_unlink(b);
      index.erase(key_of[b]);
      has_key[b] = 0;
      state[b] = kFree;
      --q_committed;
      free_list.push_back(b);
      ++m.evictions;
    }
  }

  int64_t available() const { return (int64_t)free_list.size() + n_evictable; }

  bool cow_needed(const Req& r) const {
    const int64_t T = r.num_computed;
    const int64_t j = T / B;
    return T % B != 0 && j < (int64_t)r.blocks.size() && ref[r.blocks[(size_t)j]] > 1;
  }

  // Delta q: blocks covering num_computed + n positions minus blocks held,
  // plus one if the partly filled block being appended to is shared
  int64_t blocks_needed(const Req& r, int64_t n) const {
    return ((int64_t)r.num_computed + n + B - 1) / B - (int64_t)r.blocks.size() + (cow_needed(r) ? 1 : 0);
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
    if (blocks_needed(r, n) <= available()) return true;
    ++m.allocation_failures;
    return false;
  }

  void grow(Req& r, int64_t n) {
    make_free(blocks_needed(r, n));
    if (cow_needed(r)) {
      const int32_t j = r.num_computed / B;
      const int32_t old = r.blocks[(size_t)j];
      const int32_t nb = take();
      copies.emplace_back(old, nb);
      --ref[old];                              // still referenced by the others
      r.blocks[(size_t)j] = nb;
      r.pend_cow_j = j;
      r.pend_cow_old = old;
      ++m.cow_copies;
    }
    const int64_t k = ((int64_t)r.num_computed + n + B - 1) / B - (int64_t)r.blocks.size();
    for (int64_t i = 0; i < k; ++i) r.blocks.push_back(take());
    r.pend_new = (int32_t)k;
  }

  int64_t release_all(Req& r) {
    const int64_t n = (int64_t)r.blocks.size();
    for (const int32_t b : r.blocks) unref(b);
    r.blocks.clear();
    r.pend_new = 0;
    r.pend_cow_j = r.pend_cow_old = -1;
    r.pend_match = 0;
    return n;
  }

  // a finished or cancelled request keeps only its id and counters
  static void drop_storage(Req& r) {
    std::vector<uint64_t>().swap(r.keys);
    std::vector<int32_t>().swap(r.blocks);
  }

  void preempt(int32_t slot) {
    Req& v = reqs[(size_t)slot];
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

  // leading blocks of r found in the prefix index (not attached)
  void match(const Req& r, std::vector<int32_t>& out) const {
    out.clear();
    if (r.num_computed != 0 || !r.blocks.empty() || r.keys.empty()) return;
    const int64_t cap = std::min<int64_t>((r.num_tokens() - 1) / B, (int64_t)r.keys.size());
    for (int64_t j = 0; j < cap; ++j) {
      auto it = index.find(r.keys[(size_t)j]);
      if (it == index.end()) break;
      out.push_back(it->second);
    }
  }

  void register_blocks(Req& r) {
    const int32_t full = std::min<int32_t>((int32_t)r.keys.size(), r.num_computed / B);
    while (r.registered < full) {
      const int32_t j = r.registered;
      const int32_t b = r.blocks[(size_t)j];
      const uint64_t k = r.keys[(size_t)j];
      if (!has_key[b] && index.find(k) == index.end()) {
        index.emplace(k, b);
        key_of[b] = k;
        has_key[b] = 1;
      }
      ++r.registered;
    }
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
    taken.clear();
    copies.clear();
    preempted.clear();
    std::vector<int32_t> queue(running);
    size_t i = 0;
    while (i < queue.size()) {
      Req& r = reqs[(size_t)queue[i]];
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
      grow(r, n);
      r.pending_n = (int32_t)n;
      sched.push_back({queue[i], r.num_computed, (int32_t)n});
      left -= n;
      new_running.push_back(queue[i]);
      ++i;
    }
    if (preempted.empty()) {
      std::vector<int32_t> hit;
      while (!waiting.empty() && (int64_t)new_running.size() < max_seqs && left > 0) {
        const int32_t slot = waiting.front();
        Req& r = reqs[(size_t)slot];
        match(r, hit);
        const int64_t T0 = (int64_t)hit.size() * B;
        const int64_t n = std::min<int64_t>(std::min<int64_t>(r.num_tokens() - T0, chunk), left);
        const int64_t k = (T0 + n + B - 1) / B - (int64_t)hit.size();
        int64_t hit_evictable = 0;
        for (const int32_t b : hit) hit_evictable += in_lru[b] ? 1 : 0;
        if (k > available() - hit_evictable) break;
        waiting.pop_front();
        for (const int32_t b : hit) {        // attach the cached prefix
          if (in_lru[b]) lru_unlink(b);
          ++ref[b];
        }
        r.blocks.assign(hit.begin(), hit.end());
        r.num_computed = (int32_t)T0;
        r.pend_match = (int32_t)hit.size();
        m.prefix_hit_tokens += T0;
        grow(r, n);
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
    for (const int32_t b : taken)
      if (state[b] == kReserved) state[b] = kCommitted;
    q_committed += q_reserved;
    q_reserved = 0;
    std::vector<int32_t> next;
    next.reserve(new_running.size());
    for (const int32_t slot : new_running) {
      Req& r = reqs[(size_t)slot];
      r.pend_new = 0;
      r.pend_cow_j = r.pend_cow_old = -1;
      r.pend_match = 0;
      if (r.pending_n > 0) {
        r.num_computed += r.pending_n;
        m.scheduled_tokens += r.pending_n;
        r.pending_n = 0;
        register_blocks(r);
        if (r.num_computed == r.num_tokens()) {
          ++r.generated;
          if (r.generated >= r.output_len) {
            r.status = kFinished;
            release_all(r);
            drop_storage(r);
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
      Req& r = reqs[(size_t)slot];
      for (int32_t i = 0; i < r.pend_new; ++i) {
        const int32_t b = r.blocks.back();
        r.blocks.pop_back();
        unref(b);
      }
      r.pend_new = 0;
      if (r.pend_cow_j >= 0) {
        const int32_t nb = r.blocks[(size_t)r.pend_cow_j];
        r.blocks[(size_t)r.pend_cow_j] = r.pend_cow_old;
        ++ref[r.pend_cow_old];
        unref(nb);
        r.pend_cow_j = r.pend_cow_old = -1;
      }
      if (r.pend_match > 0) {
        for (int32_t i = 0; i < r.pend_match; ++i) unref(r.blocks[(size_t)i]);
        r.blocks.erase(r.blocks.begin(), r.blocks.begin() + r.pend_match);
        r.num_computed = 0;
        r.pend_match = 0;
      }
      r.pending_n = 0;
    }
    for (auto it = admitted.rbegin(); it != admitted.rend(); ++it) {
      reqs[(size_t)*it].status = kWaiting;
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
  const size_t N = (size_t)cfg->num_blocks;
  std::vector<char> seen(N, 0);
  for (size_t i = 0; i < N; ++i) {
    const int32_t b = cfg->block_order[i];
    if (b < 0 || b >= cfg->num_blocks || seen[(size_t)b])
      return fail(PA_ERR_OUT_OF_RANGE, "block_order is not a permutation (entry %zu = %d)", i, b);
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
  s->ref.assign(N, 0);
  s->state.assign(N, kFree);
  s->key_of.assign(N, 0);
  s->has_key.assign(N, 0);
  s->lru_prev.assign(N, -1);
  s->lru_next.assign(N, -1);
  s->in_lru.assign(N, 0);
  s->m.q_capacity = cfg->num_blocks;
  *out = s;
  return PA_OK;
}

void pa_sched_destroy(pa_sched* s) { delete s; }

pa_status pa_sched_add_request(pa_sched* s, int64_t request_id, int32_t prompt_len,
                               int32_t output_len, const uint64_t* block_keys, int32_t n_keys) {
  g_err.clear();
  if (s == nullptr) return fail(PA_ERR_NULL_PTR, "NULL scheduler");
  if (prompt_len < 1 || output_len < 1)
    return fail(PA_ERR_BAD_SHAPE, "prompt_len %d and output_len %d must be >= 1", prompt_len, output_len);
  if (n_keys < 0 || n_keys > prompt_len / s->B)
    return fail(PA_ERR_BAD_SHAPE, "n_keys %d not in [0, prompt_len / block_size = %d]", n_keys, prompt_len / s->B);
  if (n_keys > 0 && block_keys == nullptr) return fail(PA_ERR_NULL_PTR, "block_keys is NULL");
  if (s->slot_of.count(request_id)) return fail(PA_ERR_BAD_SHAPE, "request %lld already added", (long long)request_id);
  if (s->reqs.size() >= (size_t)INT32_MAX) return fail(PA_ERR_BAD_SHAPE, "too many requests");
  Req r;
  r.id = request_id;
  r.prompt_len = prompt_len;
  r.output_len = output_len;
  r.keys.assign(block_keys, block_keys + n_keys);
  const int32_t slot = (int32_t)s->reqs.size();
  s->reqs.push_back(std::move(r));
  s->slot_of.emplace(request_id, slot);
  s->waiting.push_back(slot);
  return PA_OK;
}

pa_status pa_sched_fork(pa_sched* s, int64_t parent_id, int64_t child_id, int32_t output_len) {
  g_err.clear();
  if (s == nullptr) return fail(PA_ERR_NULL_PTR, "NULL scheduler");
  if (s->pending) return fail(PA_ERR_BAD_STATE, "a plan is pending");
  auto it = s->slot_of.find(parent_id);
  if (it == s->slot_of.end()) return fail(PA_ERR_OUT_OF_RANGE, "unknown request %lld", (long long)parent_id);
  if (s->slot_of.count(child_id)) return fail(PA_ERR_BAD_SHAPE, "request %lld already added", (long long)child_id);
  const Req& p = s->reqs[(size_t)it->second];
  if (p.status != kRunning) return fail(PA_ERR_BAD_STATE, "request %lld is not running", (long long)parent_id);
  if (output_len <= p.generated)
    return fail(PA_ERR_BAD_SHAPE, "output_len %d must exceed the %d tokens generated", output_len, p.generated);
  Req c;
  c.id = child_id;
  c.prompt_len = p.prompt_len;
  c.output_len = output_len;
  c.keys = p.keys;
  c.registered = p.registered;
  c.generated = p.generated;
  c.num_computed = p.num_computed;
  c.status = kRunning;
  c.blocks = p.blocks;
  for (const int32_t b : c.blocks) ++s->ref[(size_t)b];
  const int32_t slot = (int32_t)s->reqs.size();
  s->reqs.push_back(std::move(c));
  s->slot_of.emplace(child_id, slot);
  s->running.push_back(slot);
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
    info->num_copies = (int32_t)s->copies.size();
    int64_t toks = 0;
    int32_t mb = 0;
    for (const SchedEntry& e : s->sched) {
      toks += e.n;
      mb = std::max(mb, (int32_t)s->reqs[(size_t)e.slot].blocks.size());
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
                             int32_t cap_preempted, int32_t* copies, int32_t cap_copies) {
  g_err.clear();
  if (s == nullptr) return fail(PA_ERR_NULL_PTR, "NULL scheduler");
  if (!s->pending) return fail(PA_ERR_BAD_STATE, "no pending plan");
  const size_t R = s->sched.size();
  if ((size_t)std::max(cap_reqs, 0) < R)
    return fail(PA_ERR_BAD_SHAPE, "cap_reqs %d < %zu scheduled requests", cap_reqs, R);
  if ((size_t)std::max(cap_preempted, 0) < s->preempted.size())
    return fail(PA_ERR_BAD_SHAPE, "cap_preempted %d < %zu preemptions", cap_preempted, s->preempted.size());
  if ((size_t)std::max(cap_copies, 0) < s->copies.size())
    return fail(PA_ERR_BAD_SHAPE, "cap_copies %d < %zu copies", cap_copies, s->copies.size());
  for (const SchedEntry& e : s->sched)
    if ((int64_t)s->reqs[(size_t)e.slot].blocks.size() > max_blocks_per_req)
      return fail(PA_ERR_BAD_SHAPE, "max_blocks_per_req %d too small", max_blocks_per_req);
  if (R > 0 && (!request_ids || !num_computed || !query_lens || !block_table))
    return fail(PA_ERR_NULL_PTR, "NULL output array");
  if (!s->preempted.empty() && preempted == nullptr) return fail(PA_ERR_NULL_PTR, "NULL preempted array");
  if (!s->copies.empty() && copies == nullptr) return fail(PA_ERR_NULL_PTR, "NULL copies array");
  for (size_t i = 0; i < R; ++i) {
    const SchedEntry& e = s->sched[i];
    const Req& r = s->reqs[(size_t)e.slot];
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
  for (size_t i = 0; i < s->copies.size(); ++i) {
    copies[2 * i] = s->copies[i].first;
    copies[2 * i + 1] = s->copies[i].second;
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
    const Req& r = s->reqs[(size_t)slot];
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
  Req& r = s->reqs[(size_t)slot];
  if (r.status == kFinished || r.status == kCancelled) return PA_OK;
  const int32_t cow_dst = r.pend_cow_j >= 0 ? r.blocks[(size_t)r.pend_cow_j] : -1;
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
    if (cow_dst >= 0)                          // its copy no longer has a reader
      s->copies.erase(std::remove_if(s->copies.begin(), s->copies.end(),
                                     [cow_dst](const std::pair<int32_t, int32_t>& c) { return c.second == cow_dst; }),
                      s->copies.end());
  }
  r.status = kCancelled;
  pa_sched::drop_storage(r);
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
  m->q_live = s->q_reserved + s->q_committed - s->n_evictable;
  int64_t tail = 0;
  for (const int32_t slot : s->running) {
    const Req& r = s->reqs[(size_t)slot];
    if (!r.blocks.empty())
      tail += ((int64_t)r.blocks.size() - r.pend_new) * s->B - r.num_computed;
  }
  m->tail_waste = tail;
  m->running = (int64_t)s->running.size();
  m->waiting = (int64_t)s->waiting.size();
  m->cached_blocks = (int64_t)s->index.size();
  m->evictable = s->n_evictable;
  return PA_OK;
}

}  // extern "C"
