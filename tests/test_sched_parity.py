"""Parity of the product scheduler / block allocator (libpa_sched.so, C++)
with the reference scheduler of the oracle: every plan (scheduled requests,
their computed counts and token counts, block tables, preemptions, pool
counters) and every metric after every step must be identical -- the
decisions are integers.  Also the C ABI's error paths and the serving trace's
invariants (conservation, budgets, ownership, recompute restarts)."""
import random

import numpy as np
import pytest

import oracle
from oracle.sched_oracle import Scheduler as RefScheduler
from workloads import serving_trace as st

pa = pytest.importorskip("paged_kv_attention_reshape_amd")


def _both(cfg):
    a = st.scheduler_args(cfg)
    return pa.Scheduler(**a), RefScheduler(**a)


def _same_plans(pp, pr):
    assert len(pp) == len(pr)
    for a, b in zip(pp, pr):
        for k in ("sched", "blocks", "preempted", "q_free", "q_reserved", "q_committed",
                  "rolled_back", "finished", "metrics"):
            assert a[k] == b[k], f"step {a['index']}: {k} differs"


def test_library_exports_every_header_symbol():
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    txt = open(os.path.join(root, "include", "pa_sched.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    syms = set(re.findall(r"\b(pa_sched_[a-z_0-9]+)\s*\(", txt))
    assert syms == set(pa.SCHED_EXPORTS)
    L = pa.sched_lib()
    for s in syms:
        assert hasattr(L, s), s


def test_serving_trace_200_steps_identical():
    cfg = st.TraceConfig()
    prod, ref = _both(cfg)
    pp = st.drive(prod, cfg)
    pr = st.drive(ref, cfg)
    _same_plans(pp, pr)
    m = pp[-1]["metrics"]
    assert m["preemptions"] >= 1 and m["steps"] == cfg.steps
    assert m["q_free"] + m["q_reserved"] + m["q_committed"] == cfg.num_blocks


def test_trace_with_hook_failures_and_cancels_identical():
    cfg = st.TraceConfig(num_requests=300, steps=120, num_blocks=2048, max_num_seqs=64,
                         max_num_batched_tokens=2048, chunk=256, artificial_preempt_prob=0.2,
                         artificial_preempt_max=40, seed=9)
    prod, ref = _both(cfg)
    rng = random.Random(3)
    fail = set(rng.sample(range(cfg.steps), 12))
    for s in (prod, ref):
        for rid, p, o in st.requests(cfg):
            s.add_request(rid, p, o)
    cancel_at = {k: rng.sample(range(cfg.num_requests), 3) for k in rng.sample(range(cfg.steps), 15)}
    for k in range(cfg.steps):
        a, b = prod.schedule(), ref.schedule()
        assert a == b, f"step {k}: plans differ"
        for rid in cancel_at.get(k, []):          # cancel between reserve and commit
            prod.cancel(rid)
            ref.cancel(rid)
            assert prod.metrics() == ref.metrics()
        if k in fail:
            prod.rollback(); ref.rollback()
        else:
            assert prod.commit() == ref.commit()
        assert prod.metrics() == ref.metrics(), f"step {k}: metrics differ"
    m = prod.metrics()
    assert m["rollbacks"] == len(fail) and m["cancelled"] > 0 and m["preemptions"] > 0


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_small_pools_identical(seed):
    rng = random.Random(seed)
    nb = rng.choice([3, 8, 40, 200])
    B = rng.choice([1, 2, 4, 16])
    order = list(range(nb)); rng.shuffle(order)
    draws = [rng.random() for _ in range(500)]
    args = dict(num_blocks=nb, block_size=B, max_num_seqs=rng.choice([1, 4, 32]),
                max_num_batched_tokens=rng.choice([8, 64, 512]), chunk=rng.choice([1, 7, 64]),
                block_order=order, hook_prob=rng.choice([0.0, 0.3]), hook_max=20, hook_draws=draws)
    prod, ref = pa.Scheduler(**args), RefScheduler(**args)
    for i in range(40):
        p, o = rng.randint(1, 120), rng.randint(1, 30)
        prod.add_request(i, p, o); ref.add_request(i, p, o)
    for k in range(150):
        assert prod.schedule() == ref.schedule()
        if rng.random() < 0.1:
            prod.rollback(); ref.rollback()
        else:
            assert prod.commit() == ref.commit()
        assert prod.metrics() == ref.metrics()


def test_trace_invariants_and_recompute_restart():
    cfg = st.TraceConfig()
    prod = pa.Scheduler(**st.scheduler_args(cfg))
    plans = st.drive(prod, cfg)
    B = cfg.block_size
    first_pre = {}
    for p in plans:
        assert p["q_free"] + p["q_reserved"] + p["q_committed"] == cfg.num_blocks
        assert sum(n for _, _, n in p["sched"]) <= cfg.max_num_batched_tokens
        assert len(p["sched"]) <= cfg.max_num_seqs
        owned = [b for rid, _, _ in p["sched"] for b in p["blocks"][rid]]
        assert len(owned) == len(set(owned)) and all(0 <= b < cfg.num_blocks for b in owned)
        for rid, c, n in p["sched"]:
            assert 1 <= n <= cfg.chunk and len(p["blocks"][rid]) == -(-(c + n) // B)
        if p["preempted"] and p["index"] > 0:           # no admission in a step that preempted
            assert p["metrics"]["admissions"] == plans[p["index"] - 1]["metrics"]["admissions"]
        for rid, held, nblk in p["preempted"]:
            assert nblk == oracle.preemption_accounting(held, B, 1, 1)["released_blocks"]
            first_pre.setdefault(rid, p["index"])
    restarted = 0
    for rid, k in first_pre.items():
        for p in plans[k + 1:]:
            ent = [s for s in p["sched"] if s[0] == rid]
            if ent:
                assert ent[0][1] == 0, "a recomputed request restarts at position 0"
                restarted += 1
                break
    assert restarted >= 1
    for p in plans[::17]:
        ql, cp, bt, rids, pos = st.step_arrays(p, B)
        slots = oracle.slot_mapping(bt, ql, cp, B)
        assert len(np.unique(slots)) == len(slots)


def test_c_abi_error_paths():
    args = dict(num_blocks=4, block_size=4, max_num_seqs=2, max_num_batched_tokens=16, chunk=8,
                block_order=[0, 1, 2, 3])
    with pytest.raises(pa.PAError, match="PA_ERR_OUT_OF_RANGE"):
        pa.Scheduler(**{**args, "block_order": [0, 1, 1, 3]})
    with pytest.raises(pa.PAError, match="PA_ERR_BAD_SHAPE"):
        pa.Scheduler(**{**args, "chunk": 0})
    with pytest.raises(pa.PAError, match="PA_ERR_BAD_SHAPE"):
        pa.Scheduler(**{**args, "hook_prob": 1.5})
    s = pa.Scheduler(**args)
    s.add_request(7, 5, 2)
    with pytest.raises(pa.PAError, match="PA_ERR_BAD_SHAPE"):
        s.add_request(7, 5, 2)                        # duplicate id
    with pytest.raises(pa.PAError, match="PA_ERR_BAD_SHAPE"):
        s.add_request(8, 0, 2)
    with pytest.raises(pa.PAError, match="PA_ERR_BAD_STATE"):
        s.commit()                                    # nothing planned
    with pytest.raises(pa.PAError, match="PA_ERR_BAD_STATE"):
        s.rollback()
    s.schedule()
    with pytest.raises(pa.PAError, match="PA_ERR_BAD_STATE"):
        s.schedule()                                  # plan pending
    with pytest.raises(pa.PAError, match="PA_ERR_OUT_OF_RANGE"):
        s.cancel(99)
    s.commit()
    s.cancel(7)
    s.cancel(7)                                       # idempotent
    assert s.metrics()["cancelled"] == 1 and s.metrics()["q_free"] == 4


def test_shared_prefix_trace_identical():
    cfg = st.TraceConfig(num_requests=600, steps=150, num_blocks=3000, max_num_seqs=96,
                         max_num_batched_tokens=4096, chunk=512, shared_prompts=4,
                         shared_len=700, shared_frac=0.8, seed=13)
    prod, ref = _both(cfg)
    pp = st.drive(prod, cfg, fail_steps=(7, 40, 41))
    pr = st.drive(ref, cfg, fail_steps=(7, 40, 41))
    _same_plans(pp, pr)
    m = pp[-1]["metrics"]
    assert m["prefix_hit_tokens"] > 0 and m["evictions"] > 0 and m["preemptions"] > 0
    assert m["q_live"] <= m["q_committed"]
    for p in pp:
        # shared blocks appear in several requests' tables: ownership is counted once
        owned = [b for rid, _, _ in p["sched"] for b in p["blocks"][rid]]
        assert len(set(owned)) <= len(owned)


@pytest.mark.parametrize("seed", [4, 5, 6, 7])
def test_forks_cow_cancels_rollbacks_identical(seed):
    rng = random.Random(seed)
    B = rng.choice([2, 4, 16])
    nb = rng.choice([24, 60, 300])
    order = list(range(nb)); rng.shuffle(order)
    args = dict(num_blocks=nb, block_size=B, max_num_seqs=rng.choice([4, 16]),
                max_num_batched_tokens=rng.choice([32, 256]), chunk=rng.choice([8, 64]),
                block_order=order)
    prod, ref = pa.Scheduler(**args), RefScheduler(**args)
    sysk = [[rng.getrandbits(60) for _ in range(6)] for _ in range(3)]
    nid = 0
    for i in range(30):
        p, o = rng.randint(1, 100), rng.randint(1, 25)
        keys = sysk[rng.randrange(3)][:min(6, p // B)] if rng.random() < 0.7 else []
        prod.add_request(nid, p, o, keys); ref.add_request(nid, p, o, keys)
        nid += 1
    for k in range(200):
        if rng.random() < 0.15:                    # parallel sampling of a running request
            running = [r.rid for r in ref.running]
            if running:
                par = rng.choice(running)
                out = ref.reqs[par].generated + rng.randint(1, 10)
                prod.fork(par, nid, out); ref.fork(par, nid, out)
                nid += 1
        a, b = prod.schedule(), ref.schedule()
        assert a == b, f"step {k}: plans differ"
        if rng.random() < 0.1:
            victim = rng.randrange(nid)
            prod.cancel(victim); ref.cancel(victim)
        if rng.random() < 0.12:
            prod.rollback(); ref.rollback()
        else:
            assert prod.commit() == ref.commit()
        assert prod.metrics() == ref.metrics(), f"step {k}: metrics differ"
        if rng.random() < 0.05:                    # new arrivals
            p, o = rng.randint(1, 100), rng.randint(1, 25)
            keys = sysk[rng.randrange(3)][:min(6, p // B)]
            prod.add_request(nid, p, o, keys); ref.add_request(nid, p, o, keys)
            nid += 1
    m = prod.metrics()
    assert m["q_free"] + m["q_reserved"] + m["q_committed"] == nb
