"""Pins for the reference scheduler / block allocator (oracle/sched_oracle.py):
the pages' worked preemption example, the allocator tests the memory chapter
lists (cancel between reserve and commit, rollback on failure, an exhausted
pool handled by explicit preemption / deferral), conservation after every
transition, the Delta q formula, the token budget, FCFS victims from the
tail and no admission in a step that preempted."""
import math
import random

import numpy as np
import pytest

import oracle
from oracle.sched_oracle import Scheduler, run_trace


def _sched(nb, B, seqs=8, budget=64, chunk=16, order=None, **kw):
    order = list(range(nb)) if order is None else order
    return Scheduler(nb, B, seqs, budget, chunk, order, **kw)


def test_preemption_worked_example():
    # "Chunked Prefill 与 Preemption": a request with 7 cached tokens and
    # block size 4 releases 2 blocks and later recomputes 7 tokens.
    s = _sched(3, 4, budget=64, chunk=64)
    s.add_request(0, 4, 5)      # B: 4-token prompt, admitted first
    s.add_request(1, 7, 5)      # A: 7-token prompt, behind B in FCFS order
    p0 = s.schedule()
    assert p0["sched"] == [(0, 0, 4), (1, 0, 7)]
    assert {k: len(v) for k, v in p0["blocks"].items()} == {0: 1, 1: 2}
    assert p0["q_free"] == 0
    s.commit()                  # both reach their known tokens: each samples one
    p1 = s.schedule()           # B's 5th token needs a second block: A (tail) is preempted
    want = oracle.preemption_accounting(7, 4, 1, 1)
    assert p1["preempted"] == [(1, 7, want["released_blocks"])] == [(1, 7, 2)]
    assert s.metrics()["recompute_tokens"] == want["recompute_tokens"] == 7
    assert p1["sched"] == [(0, 4, 1)]
    s.commit()
    # A restarts from position 0 with its sampled token kept: 8 tokens to recompute
    r = s.reqs[1]
    assert r.num_computed == 0 and r.num_tokens == 8 and s.waiting[0] is r


def test_delta_q_and_budget_by_hand():
    s = _sched(64, 16, budget=40, chunk=24)
    s.add_request(0, 37, 3)
    s.add_request(1, 81, 3)
    p = s.schedule()
    # request 0: 24 of 37 tokens (chunk), ceil(24/16) = 2 blocks; request 1
    # gets the remaining budget 16 -> 1 block
    assert p["sched"] == [(0, 0, 24), (1, 0, 16)]
    assert [len(p["blocks"][0]), len(p["blocks"][1])] == [2, 1]
    s.commit()
    p = s.schedule()
    # request 0 now at T=24: 13 more tokens -> ceil(37/16) - ceil(24/16) = 1 new block
    assert p["sched"][0] == (0, 24, 13)
    assert len(p["blocks"][0]) == 3
    assert sum(n for _, _, n in p["sched"]) <= 40
    s.commit()


def test_cancel_between_reserve_and_commit_returns_every_block():
    s = _sched(32, 16, budget=256, chunk=40)
    for i in range(3):
        s.add_request(i, 50 + 10 * i, 4)
    s.schedule(); s.commit()             # 40-token chunks: every request grows next step
    committed1 = len(s.reqs[1].blocks)
    p = s.schedule()                     # reserves the blocks of the next chunks
    reserved1 = s.reqs[1].pend_new
    assert reserved1 > 0 and any(rid == 1 for rid, _, _ in p["sched"])
    free_mid = s.metrics()["q_free"]
    s.cancel(1)                          # cancelled between reserve and commit
    m = s.metrics()
    assert m["q_free"] == free_mid + committed1 + reserved1
    assert m["q_free"] + m["q_reserved"] + m["q_committed"] == 32
    s.commit()                           # the rest of the plan still commits
    assert s.reqs[1].status == "CANCELLED" and s.reqs[1].blocks == []
    held = sum(len(s.reqs[i].blocks) for i in (0, 2))
    assert s.metrics()["q_free"] == 32 - held and s.metrics()["q_committed"] == held


def test_rollback_on_failure_keeps_committed_mappings():
    s = _sched(64, 16, budget=128, chunk=64)
    for i in range(4):
        s.add_request(i, 40 + 17 * i, 6)
    s.schedule(); s.commit()
    before = {rid: (list(r.blocks), r.num_computed, r.status) for rid, r in s.reqs.items()}
    m0 = s.metrics()
    s.schedule()                # plan reserves more blocks
    s.rollback()                # the step failed
    after = {rid: (list(r.blocks), r.num_computed, r.status) for rid, r in s.reqs.items()}
    assert after == before      # committed mappings and token state untouched
    m1 = s.metrics()
    assert (m1["q_free"], m1["q_reserved"], m1["q_committed"]) == (m0["q_free"], 0, m0["q_committed"])
    # the same plan can be retried and committed
    s.schedule(); s.commit()
    assert s.metrics()["steps"] == 2 and s.metrics()["rollbacks"] == 1


def test_rollback_returns_admitted_requests_to_the_front():
    s = _sched(64, 16, seqs=8, budget=64, chunk=32)
    for i in range(5):
        s.add_request(i, 20, 2)
    p = s.schedule()
    admitted = [rid for rid, _, _ in p["sched"]]
    s.rollback()
    assert [r.rid for r in list(s.waiting)[:len(admitted)]] == admitted
    assert all(s.reqs[i].status == "WAITING" for i in admitted)
    assert s.metrics()["q_free"] == 64


def test_exhausted_pool_self_preemption_then_deferral():
    # one request alone whose next token needs a block that does not exist:
    # it preempts itself (no retry loop), then is deferred while it cannot fit
    s = _sched(2, 4, budget=64, chunk=64)
    s.add_request(0, 8, 5)
    s.schedule(); s.commit()     # 8 tokens in 2 blocks, samples token 9
    p = s.schedule()             # token 9 needs a third block: the pool has 2
    assert p["preempted"] == [(0, 8, 2)] and p["sched"] == []
    s.commit()
    p = s.schedule()             # no admission in the preempting step; now 9 tokens > 2 blocks
    assert p["sched"] == [] and p["preempted"] == []
    s.commit()
    assert s.reqs[0].status == "WAITING" and s.metrics()["q_free"] == 2


def test_fcfs_victims_from_the_tail_and_no_admission_after_preemption():
    s = _sched(12, 4, seqs=8, budget=64, chunk=64)
    for i in range(4):
        s.add_request(i, 11, 40)     # 3 blocks each: the pool holds exactly 4
    s.add_request(9, 4, 2)           # waits behind them
    p = s.schedule(); s.commit()
    assert [rid for rid, _, _ in p["sched"]] == [0, 1, 2, 3]
    pre_all = []
    for _ in range(6):
        p = s.schedule()
        if p["preempted"]:
            # victims come from the tail: highest request ids first
            ids = [rid for rid, _, _ in p["preempted"]]
            assert ids == sorted(ids, reverse=True)
            assert 9 not in [rid for rid, _, _ in p["sched"]]
            pre_all += ids
        s.commit()
    assert pre_all and pre_all[0] == 3
    # preempted requests wait in FCFS order at the front
    w = [r.rid for r in s.waiting]
    assert w[:len(set(pre_all))] == sorted(w[:len(set(pre_all))])


@pytest.mark.parametrize("B", [1, 4, 16])
def test_random_trace_invariants(B):
    rng = random.Random(B)
    nb = 96 if B == 16 else 400
    order = list(range(nb)); rng.shuffle(order)
    draws = [rng.random() for _ in range(2000)]
    s = Scheduler(nb, B, 16, 96, 32, order, hook_prob=0.1, hook_max=50, hook_draws=draws)
    reqs = [(i, rng.randint(1, 300), rng.randint(1, 40)) for i in range(60)]
    fail = {5, 17, 18, 41}
    plans = run_trace(s, reqs, 80, fail_steps=fail)
    for k, p in enumerate(plans):
        assert p["q_free"] + p["q_reserved"] + p["q_committed"] == nb
        assert sum(n for _, _, n in p["sched"]) <= 96
        assert len(p["sched"]) <= 16
        owned = [b for rid, _, _ in p["sched"] for b in p["blocks"][rid]]
        assert len(owned) == len(set(owned))
        for rid, c, n in p["sched"]:
            assert 1 <= n <= 32
            assert len(p["blocks"][rid]) == -(-(c + n) // B)          # Delta q realised
        m = p["metrics"]
        assert m["q_reserved"] == 0                                    # after commit or rollback
        assert 0 <= m["tail_waste"] < B * max(1, m["running"])
    m = plans[-1]["metrics"]
    assert m["rollbacks"] == len(fail)
    assert m["preemptions"] > 0 and m["allocation_failures"] >= m["preemptions"]


# ----------------------------------------------------------------------------
# shared blocks: prefix index, reference counts, eviction, copy-on-write
# ----------------------------------------------------------------------------
def _keys(ns, n):
    """Keys of n full prompt blocks of a prompt in namespace ns."""
    return [hash((ns, j)) & 0x7FFFFFFFFFFF for j in range(n)]


def test_shared_prefix_reclaimed_only_after_the_last_reference():
    # "同时验证分配器与调度器": requests sharing a prefix finish in different
    # orders; shared blocks come back only when the last reference goes
    B = 4
    s = _sched(40, B, seqs=8, budget=64, chunk=64)
    pre = _keys("sys", 3)                          # 3 full blocks = 12 shared tokens
    s.add_request(0, 14, 1, keys=pre)              # A computes the prefix first
    s.schedule(); s.commit()
    assert s.metrics()["cached_blocks"] == 3 and s.reqs[0].status == "FINISHED"
    shared = [s.index[k] for k in pre]
    assert all(b in s.evictable for b in shared)   # cached, unreferenced, still committed
    m = s.metrics()
    assert m["q_live"] == m["q_committed"] - 3 == 0
    s.add_request(1, 13, 3, keys=pre)              # B: 12 cached + 1 own token
    s.add_request(2, 18, 1, keys=pre + _keys("x", 1))   # C: 12 cached + 6 own tokens
    p = s.schedule()
    assert p["sched"] == [(1, 12, 1), (2, 12, 6)]
    assert p["blocks"][1][:3] == shared == p["blocks"][2][:3]
    assert all(s.ref[b] == 2 for b in shared)
    m = s.metrics()
    assert m["prefix_hit_tokens"] == 24 and m["q_live"] == 3 + 1 + 2
    s.commit()                                      # C finishes first
    assert all(s.ref[b] == 1 for b in shared) and all(b not in s.evictable for b in shared)
    s.schedule(); s.commit()                        # B decodes once more
    s.schedule(); s.commit()                        # B finishes
    assert s.reqs[1].status == "FINISHED"
    assert all(s.ref[b] == 0 and b in s.evictable for b in shared)
    m = s.metrics()
    assert m["q_free"] + m["q_reserved"] + m["q_committed"] == 40 and m["q_live"] == 0


def test_prefix_match_leaves_one_token_and_namespaces_do_not_mix():
    B = 4
    s = _sched(40, B, budget=64, chunk=64)
    s.add_request(0, 8, 1, keys=_keys("m1", 2))
    s.schedule(); s.commit()
    s.add_request(1, 8, 1, keys=_keys("m1", 2))    # whole prompt cached: recompute the last token
    s.add_request(2, 8, 1, keys=_keys("m2", 2))    # another model version: no hit
    p = s.schedule()
    assert p["sched"] == [(1, 4, 4), (2, 0, 8)]
    assert s.metrics()["prefix_hit_tokens"] == 4
    s.commit()


def test_eviction_before_preemption_in_lru_order():
    B = 4
    s = _sched(6, B, seqs=4, budget=64, chunk=64)
    s.add_request(0, 8, 1, keys=_keys("a", 2))     # 2 blocks, cached after it finishes
    s.add_request(1, 4, 1, keys=_keys("b", 1))     # 1 block, cached after it finishes
    s.schedule(); s.commit()
    assert s.metrics()["evictable"] == 3 and s.metrics()["q_free"] == 3
    order = list(s.evictable)
    s.add_request(2, 20, 1)                        # needs 5 blocks: 3 free + 2 evicted
    p = s.schedule()
    assert p["preempted"] == [] and p["sched"] == [(2, 0, 20)]
    m = s.metrics()
    assert m["evictions"] == 2 and m["evictable"] == 1
    assert list(s.evictable) == order[2:]           # the least recently released went first
    s.commit()


def test_fork_copy_on_write_and_rollback():
    B = 4
    s = _sched(20, B, seqs=4, budget=64, chunk=64)
    s.add_request(0, 6, 5)                          # 6 tokens: block 1 half full
    s.schedule(); s.commit()                        # computes 6, samples the 7th
    s.fork(0, 1, 5)                                 # child shares both blocks
    b0, b1 = s.reqs[0].blocks
    assert s.ref[b0] == 2 and s.ref[b1] == 2
    p = s.schedule()                                # both write position 6 into the shared block 1
    # the parent copies first; the child is then the only owner of the old block
    assert len(p["copies"]) == 1 and p["copies"][0][0] == b1
    new = p["copies"][0][1]
    assert p["blocks"][0] == [b0, new] and p["blocks"][1] == [b0, b1]
    assert s.ref[b1] == 1 and s.ref[new] == 1 and s.ref[b0] == 2
    m = s.metrics()
    assert m["cow_copies"] == 1 and m["q_reserved"] == 1
    s.rollback()                                    # the failed step undoes the copy
    assert s.reqs[0].blocks == [b0, b1] and s.ref[b1] == 2
    assert s.metrics()["q_reserved"] == 0 and s.metrics()["q_free"] == 18
    p = s.schedule(); s.commit()
    assert len(p["copies"]) == 1
    m = s.metrics()
    assert m["q_live"] == 3 and m["q_free"] + m["q_committed"] == 20


def test_cancel_with_shared_blocks_drops_only_its_references():
    B = 4
    s = _sched(20, B, seqs=4, budget=64, chunk=64)
    s.add_request(0, 6, 9)
    s.schedule(); s.commit()
    s.fork(0, 1, 9)
    p = s.schedule()                                # parent copies the shared partial block
    s.cancel(0)                                     # between reserve and commit
    assert p["copies"] and s.pending[4] == []       # its copy has no reader any more
    b0 = s.reqs[1].blocks[0]
    assert s.ref[b0] == 1
    s.commit()
    m = s.metrics()
    assert m["q_free"] + m["q_reserved"] + m["q_committed"] == 20
    assert m["q_live"] == len(s.reqs[1].blocks) == 2
