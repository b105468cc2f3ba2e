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
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List, Optional, Sequence, Tuple

WAITING, RUNNING, FINISHED, CANCELLED = "WAITING", "RUNNING", "FINISHED", "CANCELLED"


class Req:
    def __init__(self, rid: int, prompt_len: int, output_len: int):
        self.rid = rid
        self.prompt_len = prompt_len
        self.output_len = output_len
        self.generated = 0
        self.num_computed = 0
        self.status = WAITING
        self.blocks: List[int] = []       # committed first, then this plan's reservations
        self.reserved = 0                 # how many of the last blocks are reserved (uncommitted)
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
        self.q_reserved = 0
        self.q_committed = 0
        self.reqs: Dict[int, Req] = {}
        self.waiting: deque = deque()
        self.running: List[Req] = []
        self.hook_prob = hook_prob
        self.hook_left = hook_max
        self.hook_draws = list(hook_draws)
        self.hook_next = 0
        self.pending = None               # (sched, new_running, admitted) between schedule and commit
        self.m = dict(steps=0, preemptions=0, recompute_tokens=0, admissions=0,
                      allocation_failures=0, finished=0, cancelled=0, rollbacks=0,
                      peak_used=0, scheduled_tokens=0)

    # ---- pool ---------------------------------------------------------------
    def check(self) -> None:
        assert len(self.free) + self.q_reserved + self.q_committed == self.capacity, "block conservation"

    def _reserve(self, r: Req, k: int) -> None:
        assert 0 <= k <= len(self.free)
        for _ in range(k):
            r.blocks.append(self.free.popleft())
        r.reserved += k
        self.q_reserved += k
        self.m["peak_used"] = max(self.m["peak_used"], self.q_reserved + self.q_committed)

    def _release_all(self, r: Req) -> int:
        n = len(r.blocks)
        self.free.extend(r.blocks)
        self.q_reserved -= r.reserved
        self.q_committed -= n - r.reserved
        r.blocks = []
        r.reserved = 0
        return n

    def _blocks_needed(self, r: Req, n: int) -> int:
        # Delta q = ceil((T + s) / B) - blocks already held
        return -(-(r.num_computed + n) // self.B) - len(r.blocks)

    def _can_append(self, r: Req, n: int) -> bool:
        if self.hook_prob > 0 and self.hook_left > 0 and self.hook_next < len(self.hook_draws):
            u = self.hook_draws[self.hook_next]
            self.hook_next += 1
            if u < self.hook_prob:
                self.hook_left -= 1
                self.m["allocation_failures"] += 1
                return False
        if self._blocks_needed(r, n) <= len(self.free):
            return True
        self.m["allocation_failures"] += 1
        return False

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

    # ---- API ----------------------------------------------------------------
    def add_request(self, rid: int, prompt_len: int, output_len: int) -> None:
        assert rid not in self.reqs and prompt_len >= 1 and output_len >= 1
        r = Req(rid, prompt_len, output_len)
        self.reqs[rid] = r
        self.waiting.append(r)

    def schedule(self) -> dict:
        assert self.pending is None, "schedule() twice without commit/rollback"
        budget = self.budget
        sched: List[Tuple[int, int, int]] = []
        preempted: List[Tuple[int, int, int]] = []
        new_running: List[Req] = []
        admitted: List[Req] = []
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
            self._reserve(r, self._blocks_needed(r, n))
            sched.append((r.rid, r.num_computed, n))
            budget -= n
            new_running.append(r)
            i += 1
        if not preempted:
            while self.waiting and len(new_running) < self.max_num_seqs and budget > 0:
                r = self.waiting[0]
                n = min(r.num_tokens - r.num_computed, self.chunk, budget)
                k = self._blocks_needed(r, n)
                if k > len(self.free):
                    break
                self.waiting.popleft()
                self._reserve(r, k)
                r.status = RUNNING
                sched.append((r.rid, r.num_computed, n))
                budget -= n
                new_running.append(r)
                admitted.append(r)
                self.m["admissions"] += 1
        self.check()
        self.pending = (sched, new_running, admitted)
        self.running = [r for r in new_running]
        return {
            "sched": list(sched),
            "blocks": {rid: list(self.reqs[rid].blocks) for rid, _, _ in sched},
            "preempted": list(preempted),
            "q_free": len(self.free),
            "q_reserved": self.q_reserved,
            "q_committed": self.q_committed,
        }

    def commit(self) -> List[int]:
        """The step ran: commit reservations, advance, sample, finish.
        Returns the ids that finished."""
        assert self.pending is not None
        sched, new_running, _ = self.pending
        n_of = {rid: n for rid, _, n in sched}
        self.q_committed += self.q_reserved
        self.q_reserved = 0
        done = []
        running = []
        for r in new_running:
            r.reserved = 0
            n = n_of.get(r.rid)
            if n is not None:
                r.num_computed += n
                self.m["scheduled_tokens"] += n
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
        """The step failed: release its reservations; requests it admitted go
        back to the front of the waiting queue in order."""
        assert self.pending is not None
        sched, new_running, admitted = self.pending
        for r in new_running:
            if r.reserved:
                ids = r.blocks[len(r.blocks) - r.reserved:]
                del r.blocks[len(r.blocks) - r.reserved:]
                self.free.extend(ids)
                self.q_reserved -= r.reserved
                r.reserved = 0
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
        self._release_all(r)
        if r in self.running:
            self.running.remove(r)
        if r in self.waiting:
            self.waiting.remove(r)
        if self.pending is not None:
            sched, new_running, admitted = self.pending
            self.pending = ([s for s in sched if s[0] != rid],
                            [x for x in new_running if x.rid != rid],
                            [x for x in admitted if x.rid != rid])
        r.status = CANCELLED
        self.m["cancelled"] += 1
        self.check()

    def metrics(self) -> dict:
        live = self.q_reserved + self.q_committed
        resident = [r for r in self.running if r.blocks]
        tail = sum((len(r.blocks) - r.reserved) * self.B - r.num_computed for r in resident)
        out = dict(self.m)
        out.update(q_free=len(self.free), q_reserved=self.q_reserved,
                   q_committed=self.q_committed, q_live=live, q_capacity=self.capacity,
                   tail_waste=tail, running=len(self.running), waiting=len(self.waiting))
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
