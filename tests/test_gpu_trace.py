"""Serving-trace parity: 200 consecutive steps of write_kv + attention over a
32-layer cache, with the steps the product scheduler / block allocator
(libpa_sched.so, recompute preemption) plans for the seeded request trace of
workloads.serving_trace, checked four ways:

* sampled (step, layer, request) triples against the fp64 oracle, which
  regenerates the request's whole history from the counter-based generator
  (outputs within the bf16 tolerance, the request's cache rows bit-exact);
* outputs of a preempted request after its re-prefill against the outputs the
  same (layer, position) had before the preemption (both GPU; the K/V are
  identical by construction, so only rounding may differ);
* every plan equals the reference scheduler's plan (also covered on the CPU by
  test_sched_parity.py, with the pool and scheduling invariants).
"""
import numpy as np
import pytest

import oracle
from helpers import assert_close, bits, say, storage_np
from workloads import rng
from oracle.sched_oracle import Scheduler as RefScheduler
from workloads import serving_trace as st
from workloads.serving_trace import TraceConfig, step_arrays, token_row_keys

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_attention_reshape_amd as pa  # noqa: E402
from workloads import _lib as wl  # noqa: E402

LAYERS = 32
HQ, HKV, D = 32, 8, 128
KEEP_LAYERS = (0, LAYERS - 1)


def _fill_rows(t, keys):
    wl.fill_rows(t, "bf16", row_keys=torch.from_numpy(keys.view(np.int64)).cuda())


def test_serving_trace_200_steps_32_layers():
    cfg = TraceConfig()
    plans = st.drive(pa.Scheduler(**st.scheduler_args(cfg)), cfg)
    ref = st.drive(RefScheduler(**st.scheduler_args(cfg)), cfg)
    assert [(p['sched'], p['blocks'], p['preempted']) for p in plans] == \
        [(p['sched'], p['blocks'], p['preempted']) for p in ref]
    B = cfg.block_size
    scale = 1.0 / np.sqrt(D)
    n_pre = sum(len(p['preempted']) for p in plans)
    say(f"trace: {len(plans)} steps, {n_pre} recompute preemptions, "
        f"{sum(sum(n for _, _, n in p['sched']) for p in plans)} scheduled tokens")
    assert n_pre >= 1

    # which (rid, pos) to remember for the re-prefill comparison: positions a
    # request computed before its first preemption (every 37th + the last)
    first_pre = {}
    for p in plans:
        for rid, held, _ in p['preempted']:
            first_pre.setdefault(rid, (p['index'], held))
    watch = {}
    for rid, (k, held) in first_pre.items():
        if held > 0:
            watch[rid] = set(range(0, held, 37)) | {held - 1}
    before = {}   # (layer, rid, pos) -> output row (uint16 [HQ, D])
    compared = 0

    # oracle samples: a few steps, layers 0 and 31, up to 3 requests per step
    g = np.random.default_rng(55)
    sample_steps = set(int(s) for s in g.choice(np.arange(20, len(plans)), 4, replace=False))
    sample_steps.add(len(plans) - 1)

    kc = torch.empty((LAYERS, cfg.num_blocks, B, HKV, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    kc.view(torch.int16).fill_(0x7FC0)   # NaN everywhere before the trace writes
    vc.view(torch.int16).fill_(0x7FC0)
    # one workspace for the whole trace, sized by the scheduler's limits
    ws = pa.alloc_workspace(pa.attention_workspace_bound(cfg.max_num_seqs, cfg.max_num_batched_tokens,
                                                         st.max_seq_len(cfg), HQ, HKV, D, B, pa.PA_BF16))
    worst = 0.0
    n_checked = 0
    for p in plans:
        if not p['sched']:
            continue
        ql, cp, bt, rids, pos = step_arrays(p, B)
        T = int(ql.sum())
        qsl, sl, sm = pa.build_step_metadata(ql, cp, bt, B, cfg.num_blocks)
        d_bt = torch.from_numpy(bt).cuda()
        d_qsl = torch.from_numpy(qsl).cuda()
        d_sl = torch.from_numpy(sl).cuda()
        d_nc = torch.from_numpy(cp).cuda()
        d_sm = torch.from_numpy(sm).cuda()
        q = torch.empty((T, HQ, D), dtype=torch.bfloat16, device="cuda")
        k = torch.empty((T, HKV, D), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        out = torch.empty_like(q)
        # the step is planned once; every layer runs with the same plan
        plan = pa.attention_plan(d_bt, d_qsl, d_sl, d_nc, qsl, sl, HQ, kc.shape[1:], pa.PA_BF16, ws)
        for layer in range(LAYERS):
            _fill_rows(q, token_row_keys(cfg.seed, rng.TAG_Q, layer, rids, pos))
            _fill_rows(k, token_row_keys(cfg.seed, rng.TAG_K, layer, rids, pos))
            _fill_rows(v, token_row_keys(cfg.seed, rng.TAG_V, layer, rids, pos))
            pa.write_kv(k, v, kc[layer], vc[layer], d_sm)
            pa.attention_run(plan, out, q, kc[layer], vc[layer], scale)
            if layer in KEEP_LAYERS:
                idx, keys = [], []
                for i, (rid, c, n) in enumerate(p['sched']):
                    if rid not in watch:
                        continue
                    for j in range(n):
                        if c + j in watch[rid]:
                            idx.append(int(qsl[i]) + j)
                            keys.append((layer, rid, c + j))
                if idx:
                    rows = storage_np(out.index_select(0, torch.tensor(idx, device="cuda")))
                    for row, key in zip(rows, keys):
                        if key in before:
                            got = oracle.as_f64(row, "bf16")
                            ref = oracle.as_f64(before[key], "bf16")
                            err = np.abs(got - ref)
                            assert np.all(err <= 2e-2 + 2e-2 * np.abs(ref)), \
                                f"re-prefill of request {key[1]} position {key[2]} layer {key[0]} differs (max {err.max():.3e})"
                            compared += 1
                        else:
                            before[key] = row.copy()
            if p['index'] in sample_steps and layer in KEEP_LAYERS:
                torch.cuda.synchronize()
                cand = [i for i, (_, _, n) in enumerate(p['sched']) if n == 1][:2] + \
                       [i for i, (_, _, n) in enumerate(p['sched']) if n > 1][:1]
                for i in cand:
                    rid, c, n = p['sched'][i]
                    L = c + n
                    allpos = np.arange(L)
                    kh = rng.row_values(token_row_keys(cfg.seed, rng.TAG_K, layer, np.full(L, rid), allpos),
                                        HKV * D, "bf16").reshape(L, HKV, D)
                    vh = rng.row_values(token_row_keys(cfg.seed, rng.TAG_V, layer, np.full(L, rid), allpos),
                                        HKV * D, "bf16").reshape(L, HKV, D)
                    rows = np.unique(np.clip(np.array([0, n // 2, n - 1]), 0, n - 1))
                    qh = rng.row_values(token_row_keys(cfg.seed, rng.TAG_Q, layer, np.full(len(rows), rid),
                                                       c + rows), HQ * D, "bf16").reshape(len(rows), HQ, D)
                    want, _ = oracle.attention_rows(qh, kh, vh, c + rows, scale, "bf16")
                    got = oracle.as_f64(storage_np(out[int(qsl[i]) + torch.from_numpy(rows).cuda()]), "bf16")
                    worst = max(worst, assert_close(got, want, "bf16", f"step {p['index']} layer {layer} req {rid}"))
                    # the request's cache rows 0..L-1, gathered through its blocks, bit-exact
                    blk = torch.from_numpy(np.asarray(p['blocks'][rid], np.int64)).cuda()
                    gk = oracle.gather_kv(storage_np(kc[layer].index_select(0, blk)),
                                          np.arange(len(p['blocks'][rid])), L, B)
                    gv = oracle.gather_kv(storage_np(vc[layer].index_select(0, blk)),
                                          np.arange(len(p['blocks'][rid])), L, B)
                    assert np.array_equal(bits(gk), bits(kh)), f"key cache of request {rid} differs"
                    assert np.array_equal(bits(gv), bits(vh)), f"value cache of request {rid} differs"
                    n_checked += 1
        if p['index'] % 40 == 0:
            torch.cuda.synchronize()
            say(f"step {p['index']}: R={len(p['sched'])} T={T} preempted={len(p['preempted'])}")
    torch.cuda.synchronize()
    say(f"oracle-checked {n_checked} (step, layer, request) samples, max err {worst:.2e}; "
        f"{compared} re-prefilled rows matched their pre-preemption outputs")
    assert n_checked >= 10
    assert compared >= 10
