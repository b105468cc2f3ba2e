"""CPU checks of the serving-trace scheduler that produces the 200-step
trace's step shapes (block conservation, budgets, recompute preemption)."""
import math

import numpy as np

import oracle
from workloads.serving_trace import TraceConfig, simulate, step_arrays


def _run(**kw):
    cfg = TraceConfig(**kw)
    plans, reqs = simulate(cfg)
    return cfg, plans, reqs


def test_trace_invariants_and_preemption_fires():
    cfg, plans, reqs = _run()
    assert len(plans) == cfg.steps
    n_pre = sum(len(p.preempted) for p in plans)
    assert n_pre >= 1, "the pool must be small enough for recompute preemption to fire"
    for p in plans:
        # conservation: free + reserved + committed = capacity
        assert p.q_free + p.q_reserved + p.q_committed == cfg.num_blocks
        toks = sum(n for _, _, n in p.sched)
        assert toks <= cfg.max_num_batched_tokens
        assert len(p.sched) <= cfg.max_num_seqs
        assert all(1 <= n <= cfg.chunk for _, _, n in p.sched)
        assert len({rid for rid, _, _ in p.sched}) == len(p.sched)
        for rid, c, n in p.sched:
            # each scheduled request holds exactly the blocks its tokens need
            assert len(p.blocks[rid]) == -(-(c + n) // cfg.block_size)
        # no block owned by two requests
        owned = [b for rid, _, _ in p.sched for b in p.blocks[rid]]
        assert len(owned) == len(set(owned))
        assert all(0 <= b < cfg.num_blocks for b in owned)


def test_no_admission_after_preemption_and_recompute_state():
    cfg, plans, reqs = _run()
    seen_prefix = {}
    for k, p in enumerate(plans):
        if p.preempted:
            # requests scheduled in a preempting step were all running before it
            prev = plans[k - 1] if k else None
            prev_ids = {rid for rid, _, _ in prev.sched} if prev else set()
            for rid, c, n in p.sched:
                assert rid in prev_ids, "a new request was admitted in a step that preempted"
        for rid, held, nblk in p.preempted:
            # released blocks are ceil(held tokens / B) (recompute accounting)
            assert nblk == oracle.preemption_accounting(held, cfg.block_size, 1, 1)["released_blocks"]
    # after a preemption a request restarts from position 0 with its output kept
    first_pre = {}
    for p in plans:
        for rid, held, _ in p.preempted:
            first_pre.setdefault(rid, (p.index, held))
    restarted = 0
    for rid, (k, held) in first_pre.items():
        for p in plans[k + 1:]:
            ent = [s for s in p.sched if s[0] == rid]
            if ent:
                assert ent[0][1] == 0, "a recomputed request must restart at position 0"
                restarted += 1
                break
    assert restarted >= 1


def test_step_arrays_match_plans():
    cfg, plans, _ = _run(steps=40)
    for p in plans[::7]:
        ql, cp, bt, rids, pos = step_arrays(p, cfg.block_size)
        assert ql.sum() == len(rids) == len(pos)
        slots = oracle.slot_mapping(bt, ql, cp, cfg.block_size)
        assert len(np.unique(slots)) == len(slots)


def test_artificial_preemption_hook_fires():
    cfg0, plans0, _ = _run(steps=30)
    cfg1, plans1, _ = _run(steps=30, artificial_preempt_prob=0.5, artificial_preempt_max=20)
    n0 = sum(len(p.preempted) for p in plans0)
    n1 = sum(len(p.preempted) for p in plans1)
    assert n1 > n0
    for p in plans1:
        assert p.q_free + p.q_reserved + p.q_committed == cfg1.num_blocks
