"""Plain reference scheduler and block allocator (Python, host only).

TEST INFRASTRUCTURE ONLY.  Only the test suite may import this module; the
product scheduler (libpa_sched.so, include/pa_sched.h) shares no code with it.
Its decisions are integers, so the product must reproduce them exactly.

What it follows (pages as printed):
* "AI Infra入门干货总结：大模型是如何高效推理的", section "连续批处理": each
  request tracks num_computed_tokens and num_tokens (prompt + generated); a
  step schedules the difference within a token budget, a cap on running
  requests and the free KV blocks; section "附4": when blocks run out, the
  lowest-priority RUNNING request is preempted by recompute (all its blocks
  freed, num_computed reset to 0, back to the front of the waiting queue), and
  no waiting request is admitted in a step that preempted.
* "vLLM 抢占机制源码精读", sections "抢占的触发条件" / "Recompute 模式": the
  victim is taken from the tail of the running queue (FCFS order); a request
  that is the last one left preempts itself; generated tokens are kept and
  re-prefilled with the prompt; section "人工抢占测试": a test hook makes the
  free-block check fail with a given probability, a bounded number of times.
* "显存与调度" (ch. 32): "分配是词元计划的一部分" -- a plan needs
  Delta q_i = ceil((T_i + s_i)/B) - ceil(T_i/B) new blocks, their sum must fit
  q_free, blocks are reserved before execution, committed after it succeeds,
  and a failed or cancelled plan rolls back its uncommitted reservations;
  q_free + q_reserved + q_committed = q_capacity after every transition.
  "分块预填充共享每轮预算": the plan's tokens sum to at most the budget K.
  "同时验证分配器与调度器": the metrics of the pool (free, reserved,
  committed, live blocks, tail waste, allocation failures, peak use) and of
  scheduling (preemptions, recomputed tokens, admissions).

Readings where the pages leave a step open:
* the initial order of the free list is an input (physical placement);
  released blocks go to the back of the free list, reservations take from
  the front;
* a prefill chunk is at most `chunk` tokens of one request per step;
* when a request's computed tokens reach its known tokens it samples one
  token at the end of that step; it finishes when it has generated
  output_len tokens and then releases its blocks;
* the artificial-preemption hook consumes caller-provided uniform draws in
  order, one per free-block check while it is armed;
* rollback releases the plan's reservations and puts the requests the plan
  admitted back at the front of the waiting queue in their order; a
  preemption done while planning is not undone (its release already
  happened); cancel releases every block the request holds (reserved ones
  back as uncommitted, the rest as committed) and drops it from the plan.

Shared blocks ("显存与调度", "共享前缀会改变块的所有权" and figure 32.2):
* every physical block has a reference count; a request that stops using a
  block (finish, preemption, cancel, rollback) decrements it, and only a
  block whose count reaches 0 leaves the request state: back to the free
  list, or, if it is in the prefix index, into the evictable set (still
  committed: "cached state"), in least-recently-released order;
* q_live counts distinct referenced blocks; q_committed counts referenced
  committed blocks plus cached ones, so the conservation equation holds;
* prefix identity is an input: a request may carry one key per full prompt
  block, key j standing for the content of its first (j+1)*B prompt tokens
  (token ids, model, adapters, namespace -- the caller's hash).  When such a
  request is admitted with nothing computed, the longest run of leading keys
  present in the index is attached (reference counts up), at most
  floor((num_tokens - 1) / B) blocks so at least one token is computed and
  no write ever lands in a shared full block; num_computed starts after it.
  After a committed step a request registers each of its full prompt blocks
  whose key is not yet indexed;
* under memory pressure the least recently released cached blocks are
  evicted (index entry dropped, block freed) before any preemption;
* fork (parallel sampling) gives a new request every block of a running one
  (reference counts up) and its token state; when a request is about to
  write into a partly filled block that others also reference, it takes a
  fresh block, the plan lists the copy (old -> new) that must run before the
  write, and it drops its reference to the old block (copy-on-write).
"""
from __future__ import annotations

from collections import OrderedDict, deque
from typing import Dict, List, Optional, Sequence, Tuple

WAITING, RUNNING, FINISHED, CANCELLED = "WAITING", "RUNNING", "FINISHED", "CANCELLED"
FREE, RESERVED, COMMITTED = 0, 1, 2


class Req:
    def __init__(self, rid: int, prompt_len: int, output_len: int, keys: Sequence[int] = ()):
        self.rid = rid
        self.prompt_len = prompt_len
        self.output_len = output_len
        self.keys = tuple(int(k) for k in keys)
        self.registered = 0               # leading key positions already offered to the index
        self.generated = 0
        self.num_computed = 0
        self.status = WAITING
        self.blocks: List[int] = []       # logical order
        self.pend_new = 0                 # trailing blocks taken by the pending plan
        self.pend_cow = None              # (index, old block) of a copy-on-write in the pending plan
        self.pend_match = 0               # leading blocks attached from the index by the pending plan
        self.preemptions = 0

    @property
    def num_tokens(self) -> int:
        return self.prompt_len + self.generated


class Scheduler:
    def __init__(self, num_blocks: int, block_size: int, max_num_seqs: int,
                 max_num_batched_tokens: int, chunk: int, block_order: Sequence[int],
                 hook_prob: float = 0.0, hook_max: int = 0, hook_draws: Sequence[float] = ()):
        assert sorted(block_order) == list(range(num_blocks))
        self.B = block_size
        self.capacity = num_blocks
        self.max_num_seqs = max_num_seqs
        self.budget = max_num_batched_tokens
        self.chunk = chunk
        self.free = deque(block_order)
        self.ref = [0] * num_blocks
        self.state = [FREE] * num_blocks
        self.key_of: List[Optional[int]] = [None] * num_blocks
        self.index: Dict[int, int] = {}            # prefix key -> block
        self.evictable: "OrderedDict[int, None]" = OrderedDict()   # cached, unreferenced
        self.q_reserved = 0
        self.q_committed = 0
        self.reqs: Dict[int, Req] = {}
        self.waiting: deque = deque()
        self.running: List[Req] = []
        self.hook_prob = hook_prob
        self.hook_left = hook_max
        self.hook_draws = list(hook_draws)
        self.hook_next = 0
        self.pending = None   # (sched, new_running, admitted, taken, copies) between schedule and commit
        self.m = dict(steps=0, preemptions=0, recompute_tokens=0, admissions=0,
                      allocation_failures=0, finished=0, cancelled=0, rollbacks=0,
                      peak_used=0, scheduled_tokens=0, prefix_hit_tokens=0, evictions=0,
                      cow_copies=0)

    # ---- pool ---------------------------------------------------------------
    def check(self) -> None:
        assert len(self.free) + self.q_reserved + self.q_committed == self.capacity, "block conservation"

    def _take(self, taken: list) -> int:
        b = self.free.popleft()
        self.state[b] = RESERVED
        self.ref[b] = 1
        self.q_reserved += 1
        taken.append(b)
        self.m["peak_used"] = max(self.m["peak_used"], self.q_reserved + self.q_committed)
        return b

    def _unref(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] > 0:
            return
        if self.state[b] == RESERVED:
            self.state[b] = FREE
            self.q_reserved -= 1
            self.free.append(b)
        elif self.key_of[b] is not None:
            self.evictable[b] = None                  # cached: stays committed
        else:
            self.state[b] = FREE
            self.q_committed -= 1
            self.free.append(b)

    def _make_free(self, k: int) -> None:
        # evict least recently released cached blocks until k blocks are free
        while len(self.free) < k:
            b, _ = self.evictable.popitem(last=False)
            del self.index[self.key_of[b]]
            self.key_of[b] = None
            self.state[b] = FREE
            self.q_committed -= 1
            self.free.append(b)
            self.m["evictions"] += 1

    def _available(self) -> int:
        return len(self.free) + len(self.evictable)

    def _cow_needed(self, r: Req) -> bool:
        T = r.num_computed
        j = T // self.B
        return T % self.B != 0 and j < len(r.blocks) and self.ref[r.blocks[j]] > 1

    def _blocks_needed(self, r: Req, n: int) -> int:
        # Delta q = ceil((T + s) / B) - blocks already held, plus one block if
        # the partly filled block being appended to is shared
        return -(-(r.num_computed + n) // self.B) - len(r.blocks) + (1 if self._cow_needed(r) else 0)

    def _can_append(self, r: Req, n: int) -> bool:
        if self.hook_prob > 0 and self.hook_left > 0 and self.hook_next < len(self.hook_draws):
            u = self.hook_draws[self.hook_next]
            self.hook_next += 1
            if u < self.hook_prob:
                self.hook_left -= 1
                self.m["allocation_failures"] += 1
                return False
        if self._blocks_needed(r, n) <= self._available():
            return True
        self.m["allocation_failures"] += 1
        return False

    def _grow(self, r: Req, n: int, taken: list, copies: list) -> None:
        """Take the blocks the next n tokens of r need (after _can_append)."""
        self._make_free(self._blocks_needed(r, n))
        if self._cow_needed(r):
            j = r.num_computed // self.B
            old = r.blocks[j]
            nb = self._take(taken)
            copies.append((old, nb))
            self.ref[old] -= 1                        # still referenced by the others
            r.blocks[j] = nb
            r.pend_cow = (j, old)
            self.m["cow_copies"] += 1
        k = -(-(r.num_computed + n) // self.B) - len(r.blocks)
        for _ in range(k):
            r.blocks.append(self._take(taken))
        r.pend_new = k

    def _release_all(self, r: Req) -> int:
        n = len(r.blocks)
        for b in r.blocks:
            self._unref(b)
        r.blocks = []
        r.pend_new = 0
        r.pend_cow = None
        r.pend_match = 0
        return n

    def _preempt(self, v: Req, preempted: list) -> None:
        held = v.num_computed
        n = self._release_all(v)
        v.num_computed = 0
        v.status = WAITING
        v.preemptions += 1
        self.waiting.appendleft(v)
        preempted.append((v.rid, held, n))
        self.m["preemptions"] += 1
        self.m["recompute_tokens"] += held

    def _match(self, r: Req) -> List[int]:
        """Leading blocks of r found in the prefix index (not attached)."""
        if r.num_computed != 0 or r.blocks or not r.keys:
            return []
        cap = (r.num_tokens - 1) // self.B
        out = []
        for k in r.keys[:cap]:
            b = self.index.get(k)
            if b is None:
                break
            out.append(b)
        return out

    def _register(self, r: Req) -> None:
        """Offer r's full prompt blocks to the prefix index."""
        full = min(len(r.keys), r.num_computed // self.B)
        while r.registered < full:
            j = r.registered
            b = r.blocks[j]
            k = r.keys[j]
            if k not in self.index and self.key_of[b] is None:
                self.index[k] = b
                self.key_of[b] = k
            r.registered += 1

    # ---- API ----------------------------------------------------------------
    def add_request(self, rid: int, prompt_len: int, output_len: int,
                    keys: Sequence[int] = ()) -> None:
        assert rid not in self.reqs and prompt_len >= 1 and output_len >= 1
        assert len(keys) <= prompt_len // self.B
        r = Req(rid, prompt_len, output_len, keys)
        self.reqs[rid] = r
        self.waiting.append(r)

    def fork(self, parent: int, child: int, output_len: int) -> None:
        """Parallel sampling: child shares every block and the token state of
        the running request parent; it runs last in FCFS order."""
        assert self.pending is None and child not in self.reqs
        p = self.reqs[parent]
        assert p.status == RUNNING and output_len > p.generated
        c = Req(child, p.prompt_len, output_len, p.keys)
        c.registered = p.registered
        c.generated = p.generated
        c.num_computed = p.num_computed
        c.status = RUNNING
        c.blocks = list(p.blocks)
        for b in c.blocks:
            self.ref[b] += 1
        self.reqs[child] = c
        self.running.append(c)

    def schedule(self) -> dict:
        assert self.pending is None, "schedule() twice without commit/rollback"
        budget = self.budget
        sched: List[Tuple[int, int, int]] = []
        preempted: List[Tuple[int, int, int]] = []
        new_running: List[Req] = []
        admitted: List[Req] = []
        taken: List[int] = []
        copies: List[Tuple[int, int]] = []
        queue = list(self.running)
        i = 0
        while i < len(queue):
            r = queue[i]
            n = min(r.num_tokens - r.num_computed, self.chunk, budget)
            if n <= 0:
                new_running.append(r)
                i += 1
                continue
            ok = True
            while not self._can_append(r, n):
                if len(queue) - 1 > i:          # someone behind r: preempt the tail
                    self._preempt(queue.pop(), preempted)
                else:                           # r is the last: it preempts itself
                    self._preempt(r, preempted)
                    queue.pop(i)
                    ok = False
                    break
            if not ok:
                continue
            self._grow(r, n, taken, copies)
            sched.append((r.rid, r.num_computed, n))
            budget -= n
            new_running.append(r)
            i += 1
        if not preempted:
            while self.waiting and len(new_running) < self.max_num_seqs and budget > 0:
                r = self.waiting[0]
                match = self._match(r)
                T0 = len(match) * self.B
                n = min(r.num_tokens - T0, self.chunk, budget)
                k = -(-(T0 + n) // self.B) - len(match)
                if k > self._available() - sum(1 for b in match if b in self.evictable):
                    break
                self.waiting.popleft()
                for b in match:                     # attach the cached prefix
                    self.evictable.pop(b, None)
                    self.ref[b] += 1
                r.blocks = list(match)
                r.num_computed = T0
                r.pend_match = len(match)
                self.m["prefix_hit_tokens"] += T0
                self._grow(r, n, taken, copies)
                r.status = RUNNING
                sched.append((r.rid, r.num_computed, n))
                budget -= n
                new_running.append(r)
                admitted.append(r)
                self.m["admissions"] += 1
        self.check()
        self.pending = (sched, new_running, admitted, taken, copies)
        self.running = [r for r in new_running]
        return {
            "sched": list(sched),
            "blocks": {rid: list(self.reqs[rid].blocks) for rid, _, _ in sched},
            "preempted": list(preempted),
            "copies": list(copies),
            "q_free": len(self.free),
            "q_reserved": self.q_reserved,
            "q_committed": self.q_committed,
        }

    def commit(self) -> List[int]:
        """The step ran: commit reservations, advance, register full prompt
        blocks, sample, finish.  Returns the ids that finished."""
        assert self.pending is not None
        sched, new_running, _, taken, _ = self.pending
        n_of = {rid: n for rid, _, n in sched}
        for b in taken:
            if self.state[b] == RESERVED:
                self.state[b] = COMMITTED
        self.q_committed += self.q_reserved
        self.q_reserved = 0
        done = []
        running = []
        for r in new_running:
            r.pend_new = 0
            r.pend_cow = None
            r.pend_match = 0
            n = n_of.get(r.rid)
            if n is not None:
                r.num_computed += n
                self.m["scheduled_tokens"] += n
                self._register(r)
                if r.num_computed == r.num_tokens:
                    r.generated += 1
                    if r.generated >= r.output_len:
                        r.status = FINISHED
                        self._release_all(r)
                        self.m["finished"] += 1
                        done.append(r.rid)
                        continue
            running.append(r)
        self.running = running
        self.pending = None
        self.m["steps"] += 1
        self.check()
        return done

    def rollback(self) -> None:
        """The step failed: release its reservations and undo its copies and
        prefix attachments; requests it admitted go back to the front of the
        waiting queue in order."""
        assert self.pending is not None
        sched, new_running, admitted, _, _ = self.pending
        for r in new_running:
            for _ in range(r.pend_new):
                self._unref(r.blocks.pop())
            r.pend_new = 0
            if r.pend_cow is not None:
                j, old = r.pend_cow
                nb = r.blocks[j]
                r.blocks[j] = old
                self.ref[old] += 1
                self._unref(nb)
                r.pend_cow = None
            if r.pend_match:
                for b in r.blocks[:r.pend_match]:
                    self._unref(b)
                r.blocks = r.blocks[r.pend_match:]
                r.num_computed = 0
                r.pend_match = 0
        adm = {r.rid for r in admitted}
        for r in reversed(admitted):
            r.status = WAITING
            self.waiting.appendleft(r)
        self.running = [r for r in new_running if r.rid not in adm]
        self.pending = None
        self.m["rollbacks"] += 1
        self.check()

    def cancel(self, rid: int) -> None:
        r = self.reqs[rid]
        if r.status in (FINISHED, CANCELLED):
            return
        cow_dst = r.blocks[r.pend_cow[0]] if r.pend_cow is not None else None
        self._release_all(r)
        if r in self.running:
            self.running.remove(r)
        if r in self.waiting:
            self.waiting.remove(r)
        if self.pending is not None:
            sched, new_running, admitted, taken, copies = self.pending
            if cow_dst is not None:                   # its copy no longer has a reader
                copies = [c for c in copies if c[1] != cow_dst]
            self.pending = ([s for s in sched if s[0] != rid],
                            [x for x in new_running if x.rid != rid],
                            [x for x in admitted if x.rid != rid], taken, copies)
        r.status = CANCELLED
        self.m["cancelled"] += 1
        self.check()

    def metrics(self) -> dict:
        resident = [r for r in self.running if r.blocks]
        tail = sum((len(r.blocks) - r.pend_new) * self.B - r.num_computed for r in resident)
        out = dict(self.m)
        out.update(q_free=len(self.free), q_reserved=self.q_reserved,
                   q_committed=self.q_committed,
                   q_live=self.q_reserved + self.q_committed - len(self.evictable),
                   q_capacity=self.capacity, tail_waste=tail, running=len(self.running),
                   waiting=len(self.waiting), cached_blocks=len(self.index),
                   evictable=len(self.evictable))
        return out


def run_trace(sched: Scheduler, requests: Sequence[Tuple[int, int, int]], steps: int,
              fail_steps: Sequence[int] = ()) -> List[dict]:
    """Add every request (rid, prompt_len, output_len) at step 0, then plan
    `steps` steps; a step index in fail_steps is rolled back instead of
    committed.  Returns the plans (each with its metrics after the step)."""
    for rid, p, o in requests:
        sched.add_request(rid, p, o)
    fail = set(fail_steps)
    plans = []
    for k in range(steps):
        plan = sched.schedule()
        if k in fail:
            sched.rollback()
            plan["rolled_back"] = True
        else:
            plan["finished"] = sched.commit()
            plan["rolled_back"] = False
        plan["metrics"] = sched.metrics()
        plans.append(plan)
    return plans
