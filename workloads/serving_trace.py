"""Seeded serving trace: the inputs of a 200-step continuous-batching trace
(test harness; host only).

This module holds no scheduling logic.  It generates what a serving front end
would hand the scheduler -- the requests (prompt lengths lognormal, median
1500, clipped to [1, 32768]; output lengths geometric with mean 256), the
pool's initial free-list order (a seeded permutation: scattered physical
placement) and the uniform draws of the artificial-preemption test hook --
and drives any scheduler object with the interface of include/pa_sched.h
(add_request / schedule / commit / rollback / metrics): the product one in
paged_kv_attention_reshape_amd, or the reference one in the oracle.

Trace configuration readings (recorded in the design notes): 2048 requests
all arrive at step 0 in FCFS order; 16384 blocks of 16 tokens (small enough
that recompute preemption fires); at most 256 running requests, 8192 tokens
per step, 512 prefill tokens per request per step.

The K/V/Q values of token (request, layer, position) come from the
counter-based generator (token_row_keys), so a request that is preempted and
re-prefilled reproduces exactly the same K/V.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np


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
    seed: int = 5
    artificial_preempt_prob: float = 0.0   # test hook (0 disables)
    artificial_preempt_max: int = 500
    # shared system prompts: a request starts with one of `shared_prompts`
    # prompts of `shared_len` tokens with probability `shared_frac`
    shared_prompts: int = 0
    shared_len: int = 0
    shared_frac: float = 0.0


def requests(cfg: TraceConfig) -> List[Tuple[int, int, int]]:
    """(request id, prompt length, output length) of every request."""
    gen = np.random.default_rng(cfg.seed)
    prompts = np.rint(np.clip(gen.lognormal(math.log(cfg.prompt_median), cfg.prompt_sigma,
                                            cfg.num_requests), 1, cfg.prompt_max)).astype(int)
    outputs = gen.geometric(1.0 / cfg.output_mean, cfg.num_requests).astype(int)
    return [(i, int(p), int(o)) for i, (p, o) in enumerate(zip(prompts, outputs))]


def _mix(x: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser (Steele, Lea, Flood 2014) on uint64 arrays."""
    x = x.astype(np.uint64)
    with np.errstate(over="ignore"):
        x = (x ^ (x >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        x = (x ^ (x >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return x ^ (x >> np.uint64(31))


def block_keys(cfg: TraceConfig) -> dict:
    """Prefix keys of each request's full prompt blocks: a block lying wholly
    inside the request's shared system prompt gets the key of (prompt, block
    index) -- identical across requests -- any other block a key of (request,
    block index).  Requests without a shared prompt get no keys."""
    if cfg.shared_prompts <= 0 or cfg.shared_len <= 0:
        return {}
    gen = np.random.default_rng(cfg.seed + 3000)
    out = {}
    for rid, p, _ in requests(cfg):
        if gen.random() >= cfg.shared_frac:
            continue
        sp = int(gen.integers(cfg.shared_prompts))
        nfull = p // cfg.block_size
        j = np.arange(nfull, dtype=np.uint64)
        inside = (j + np.uint64(1)) * np.uint64(cfg.block_size) <= np.uint64(cfg.shared_len)
        with np.errstate(over="ignore"):
            shared = _mix(np.uint64(sp + 1) * np.uint64(0x9E3779B97F4A7C15) + j)
            own = _mix(np.uint64(rid + 1) * np.uint64(0xD1B54A32D192ED03) + j + np.uint64(1 << 40))
        out[rid] = np.where(inside, shared, own).tolist()
    return out


def block_order(cfg: TraceConfig) -> np.ndarray:
    """Initial free-list order of the pool: a seeded permutation."""
    return np.random.default_rng(cfg.seed + 1000).permutation(cfg.num_blocks).astype(np.int32)


def hook_draws(cfg: TraceConfig, n: int = 1 << 16) -> np.ndarray:
    """Uniform draws in [0, 1) the artificial-preemption hook consumes."""
    return np.random.default_rng(cfg.seed + 2000).random(n)


def scheduler_args(cfg: TraceConfig) -> dict:
    """Keyword arguments of a scheduler (product or reference) for cfg."""
    return dict(num_blocks=cfg.num_blocks, block_size=cfg.block_size,
                max_num_seqs=cfg.max_num_seqs, max_num_batched_tokens=cfg.max_num_batched_tokens,
                chunk=cfg.chunk, block_order=block_order(cfg).tolist(),
                hook_prob=cfg.artificial_preempt_prob, hook_max=cfg.artificial_preempt_max,
                hook_draws=hook_draws(cfg).tolist() if cfg.artificial_preempt_prob > 0 else [])


def drive(sched, cfg: TraceConfig, fail_steps: Sequence[int] = ()) -> List[dict]:
    """Queue every request at step 0, then plan cfg.steps steps with the given
    scheduler object; a step index in fail_steps is rolled back instead of
    committed.  Returns the plans (dicts: sched [(rid, num_computed, n)],
    blocks {rid: [block ids]}, preempted [(rid, held, released)], pool
    counters, index, rolled_back, finished, metrics)."""
    keys = block_keys(cfg)
    for rid, p, o in requests(cfg):
        sched.add_request(rid, p, o, keys.get(rid, ()))
    fail = set(fail_steps)
    plans = []
    for k in range(cfg.steps):
        plan = sched.schedule()
        plan["index"] = k
        if k in fail:
            sched.rollback()
            plan["rolled_back"], plan["finished"] = True, []
        else:
            plan["rolled_back"], plan["finished"] = False, sched.commit()
        plan["metrics"] = sched.metrics()
        plans.append(plan)
    return plans


def token_row_keys(seed: int, tag: int, layer: int, rids, positions) -> np.ndarray:
    """Generator row keys of tokens (request, position) at one layer: the same
    token always gets the same K/V/Q values, also after a recompute."""
    from . import rng
    base = np.uint64(rng.key(seed, tag, layer))
    k = rng.derive(base, np.asarray(rids, dtype=np.uint64))
    return rng.derive(k, np.asarray(positions, dtype=np.uint64))


def max_seq_len(cfg: TraceConfig) -> int:
    """Longest sequence any step of the trace can hold: a request's length is
    its prompt plus the tokens it has generated, at most one per step."""
    return int(cfg.prompt_max + cfg.steps)


def step_arrays(plan: dict, block_size: int):
    """Host arrays of one planned step: query lens, computed counts, block
    table [R, M] (-1 padded), request ids and token positions in flattened
    order."""
    sched = plan["sched"]
    R = len(sched)
    qlens = np.array([n for _, _, n in sched], dtype=np.int32)
    comp = np.array([c for _, c, _ in sched], dtype=np.int32)
    M = max([len(plan["blocks"][rid]) for rid, _, _ in sched] + [1])
    bt = np.full((R, M), -1, dtype=np.int32)
    for i, (rid, _, _) in enumerate(sched):
        b = plan["blocks"][rid]
        bt[i, :len(b)] = b
    rids = np.concatenate([np.full(n, rid, np.int64) for rid, _, n in sched]) if R else np.zeros(0, np.int64)
    pos = np.concatenate([np.arange(c, c + n) for _, c, n in sched]) if R else np.zeros(0, np.int64)
    return qlens, comp, bt, rids, pos
