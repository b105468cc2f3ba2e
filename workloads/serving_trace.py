"""Seeded serving trace: a continuous-batching scheduler over a paged block
pool, producing the step shapes of a 200-step trace (test harness; host only).

What it follows:
* "AI Infra入门干货总结：大模型是如何高效推理的", section "连续批处理": each
  request tracks num_computed_tokens and num_tokens (prompt + generated);
  a step schedules the difference, within a token budget, a cap on running
  requests, the model length and free KV blocks.
* same page, "附4": when blocks run out the scheduler preempts the lowest
  priority RUNNING request by recompute: all its blocks are freed,
  num_computed_tokens is reset to 0, it goes back to the front of the waiting
  queue, and no new waiting request is admitted in a step that preempted.
* "vLLM 抢占机制源码精读", sections "抢占的触发条件" and "Recompute 模式": the
  victim is popped from the tail of the running queue (FCFS order, lowest
  priority last); if the request being scheduled is the only one left it
  preempts itself; generated tokens are kept and re-prefilled with the prompt;
  section "人工抢占测试": a test hook makes the free-block check fail with a
  given probability, a bounded number of times.
* "显存与调度" (ch. 32), sections "分配是词元计划的一部分" and "分块预填充共享每轮预算":
  a step needs Delta q_i = ceil((T_i + s_i)/B) - ceil(T_i/B) new blocks,
  sum Delta q_i <= q_free, and q_free + q_reserved + q_committed = q_capacity
  at every transition; the step's tokens sum to at most the budget K.

Readings where the pages leave a step open (all recorded in the design notes):
* all requests arrive at step 0 in a FCFS waiting queue;
* a prefill chunk is at most `chunk` tokens of one request per step;
* when a request's computed tokens reach its known tokens it samples one new
  token at the end of that step (so its next step is a decode of 1 token);
  it finishes when it has generated its target output length;
* blocks are reserved when a request is scheduled and committed after the
  step ran (there is no failure path in this trace, so nothing rolls back).

The trace only decides shapes and block ownership; the K/V values of token
(request, layer, position) come from the counter-based generator, so a
request that is preempted and re-prefilled reproduces exactly the same K/V.
"""
from __future__ import annotations

import math
import random
from collections import deque
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

WAITING, RUNNING, FINISHED = "WAITING", "RUNNING", "FINISHED"


@dataclass
class TraceConfig:
    num_requests: int = 2048
    steps: int = 200
    max_num_seqs: int = 256
    max_num_batched_tokens: int = 8192
    chunk: int = 512
    block_size: int = 16
    num_blocks: int = 16384
    prompt_median: float = 1500.0
    prompt_sigma: float = 1.0
    prompt_max: int = 32768
    output_mean: float = 256.0
    max_model_len: int = 32768 + 4096
    seed: int = 5
    artificial_preempt_prob: float = 0.0   # test hook (0 disables)
    artificial_preempt_max: int = 500


@dataclass
class Request:
    rid: int
    prompt_len: int
    output_len: int
    generated: int = 0
    num_computed: int = 0
    status: str = WAITING
    blocks: List[int] = field(default_factory=list)
    preemptions: int = 0

    @property
    def num_tokens(self) -> int:
        return self.prompt_len + self.generated


@dataclass
class StepPlan:
    """One step: scheduled (rid, num_computed_before, n_tokens) in flattened
    order, each request's block list (covering num_computed_before + n),
    the preemptions that happened while planning it, and pool counters."""
    index: int
    sched: List[Tuple[int, int, int]]
    blocks: Dict[int, List[int]]
    preempted: List[Tuple[int, int, int]]   # (rid, tokens it held, blocks released)
    q_free: int
    q_reserved: int
    q_committed: int


class BlockPool:
    """Free list of physical block ids with reserve -> commit accounting."""

    def __init__(self, n: int, rng: random.Random):
        ids = list(range(n))
        rng.shuffle(ids)                 # scattered physical placement
        self.free = deque(ids)
        self.capacity = n
        self.reserved = 0
        self.committed = 0

    def reserve(self, k: int) -> List[int]:
        assert k <= len(self.free)
        out = [self.free.popleft() for _ in range(k)]
        self.reserved += k
        return out

    def commit_all(self) -> None:
        self.committed += self.reserved
        self.reserved = 0

    def release(self, ids: List[int], committed: bool = True) -> None:
        self.free.extend(ids)
        if committed:
            self.committed -= len(ids)
        else:
            self.reserved -= len(ids)

    def check(self) -> None:
        assert len(self.free) + self.reserved + self.committed == self.capacity, "block conservation"


def make_requests(cfg: TraceConfig) -> List[Request]:
    gen = np.random.default_rng(cfg.seed)
    prompts = np.rint(np.clip(gen.lognormal(math.log(cfg.prompt_median), cfg.prompt_sigma,
                                            cfg.num_requests), 1, cfg.prompt_max)).astype(int)
    outputs = gen.geometric(1.0 / cfg.output_mean, cfg.num_requests).astype(int)
    return [Request(i, int(p), int(o)) for i, (p, o) in enumerate(zip(prompts, outputs))]


def simulate(cfg: TraceConfig) -> Tuple[List[StepPlan], Dict[int, Request]]:
    """Run the scheduler for cfg.steps steps; returns the step plans and the
    final request states."""
    reqs = make_requests(cfg)
    by_id = {r.rid: r for r in reqs}
    pool = BlockPool(cfg.num_blocks, random.Random(cfg.seed))
    waiting: deque = deque(reqs)
    running: List[Request] = []
    hook_rng = random.Random(cfg.seed + 1)
    hook_left = cfg.artificial_preempt_max
    B = cfg.block_size
    plans: List[StepPlan] = []

    def blocks_needed(r: Request, n: int) -> int:
        return -(-(r.num_computed + n) // B) - len(r.blocks)

    def can_append(r: Request, n: int) -> bool:
        nonlocal hook_left
        if cfg.artificial_preempt_prob > 0 and hook_left > 0 and hook_rng.random() < cfg.artificial_preempt_prob:
            hook_left -= 1
            return False
        return blocks_needed(r, n) <= len(pool.free)

    def preempt(v: Request, preempted: list) -> None:
        held = v.num_computed
        nblk = len(v.blocks)
        pool.release(v.blocks, committed=True)
        v.blocks = []
        v.num_computed = 0
        v.status = WAITING
        v.preemptions += 1
        waiting.appendleft(v)
        preempted.append((v.rid, held, nblk))

    for step in range(cfg.steps):
        budget = cfg.max_num_batched_tokens
        sched: List[Tuple[int, int, int]] = []
        preempted: List[Tuple[int, int, int]] = []
        new_running: List[Request] = []
        queue = list(running)
        # ---- running requests, FCFS order; victims from the tail --------------
        i = 0
        while i < len(queue):
            r = queue[i]
            need = r.num_tokens - r.num_computed
            n = min(need, cfg.chunk, budget)
            if n <= 0:
                new_running.append(r)
                i += 1
                continue
            ok = True
            while not can_append(r, n):
                if len(queue) - 1 > i:          # someone behind r to preempt
                    v = queue.pop()
                    preempt(v, preempted)
                else:                           # r is the lowest priority: preempt itself
                    preempt(r, preempted)
                    queue.pop(i)
                    ok = False
                    break
            if not ok:
                continue
            k = blocks_needed(r, n)
            if k > 0:
                r.blocks.extend(pool.reserve(k))
            sched.append((r.rid, r.num_computed, n))
            budget -= n
            new_running.append(r)
            i += 1
        # ---- admit waiting requests, unless this step preempted ---------------
        if not preempted:
            while waiting and len(new_running) < cfg.max_num_seqs and budget > 0:
                r = waiting[0]
                n = min(r.num_tokens - r.num_computed, cfg.chunk, budget)
                k = blocks_needed(r, n)
                if k > len(pool.free):
                    break
                waiting.popleft()
                r.blocks.extend(pool.reserve(k))
                r.status = RUNNING
                sched.append((r.rid, r.num_computed, n))
                budget -= n
                new_running.append(r)
        pool.check()
        plans.append(StepPlan(step, sched, {rid: list(by_id[rid].blocks) for rid, _, _ in sched},
                              preempted, len(pool.free), pool.reserved, pool.committed))
        # ---- the step runs; commit, advance, sample, finish --------------------
        pool.commit_all()
        running = []
        for r in new_running:
            entry = [s for s in sched if s[0] == r.rid]
            if entry:
                r.num_computed += entry[0][2]
                if r.num_computed == r.num_tokens:
                    r.generated += 1
                    if r.generated >= r.output_len:
                        r.status = FINISHED
                        pool.release(r.blocks, committed=True)
                        r.blocks = []
                        continue
            running.append(r)
        pool.check()
    return plans, by_id


def token_row_keys(seed: int, tag: int, layer: int, rids, positions) -> np.ndarray:
    """Generator row keys of tokens (request, position) at one layer: the same
    token always gets the same K/V/Q values, also after a recompute."""
    from . import rng
    base = np.uint64(rng.key(seed, tag, layer))
    k = rng.derive(base, np.asarray(rids, dtype=np.uint64))
    return rng.derive(k, np.asarray(positions, dtype=np.uint64))


def step_arrays(plan: StepPlan, block_size: int):
    """Host arrays of one step: query lens, computed counts, block table
    [R, M] (-1 padded), request ids and token positions in flattened order."""
    R = len(plan.sched)
    qlens = np.array([n for _, _, n in plan.sched], dtype=np.int32)
    comp = np.array([c for _, c, _ in plan.sched], dtype=np.int32)
    M = max([len(plan.blocks[rid]) for rid, _, _ in plan.sched] + [1])
    bt = np.full((R, M), -1, dtype=np.int32)
    for i, (rid, _, _) in enumerate(plan.sched):
        b = plan.blocks[rid]
        bt[i, :len(b)] = b
    rids = np.concatenate([np.full(n, rid, np.int64) for rid, _, n in plan.sched]) if R else np.zeros(0, np.int64)
    pos = np.concatenate([np.arange(c, c + n) for _, c, n in plan.sched]) if R else np.zeros(0, np.int64)
    return qlens, comp, bt, rids, pos
