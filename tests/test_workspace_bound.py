"""CPU checks of pa_attention_workspace_bound through the C ABI: the size it
returns for step limits (requests, query rows, longest sequence) covers the
exact workspace of every step within those limits -- the configurations, the
200 steps of the serving trace, seeded random steps over the support matrix
and the corner cases of the bound's derivation (all decodes at the longest
length, many short or deep chunks, one long prefill), with and without the
tuning overrides.  No kernel is launched."""
import numpy as np
import pytest

from workloads import configs, serving_trace as st

pa = pytest.importorskip("paged_kv_attention_reshape_amd")


def _mirrors(qlens, comp):
    ql = np.asarray(qlens, np.int64)
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    sl = (np.asarray(comp, np.int64) + ql).astype(np.int32)
    return qsl, sl


def _exact(qlens, comp, Hq, Hkv, D, B, dt):
    qsl, sl = _mirrors(qlens, comp)
    return pa.attention_workspace_size(qsl, sl, Hq, Hkv, D, B, dt)


def _bound(R, T, L, Hq, Hkv, D, B, dt):
    return pa.attention_workspace_bound(R, T, L, Hq, Hkv, D, B, dt)


def _dt(name):
    return pa.PA_BF16 if name == "bf16" else pa.PA_F32


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_bound_covers_the_configurations(name):
    spec = configs.BUILDERS[name]()
    dt = _dt(spec.dtype)
    exact = _exact(spec.query_lens, spec.num_computed, spec.Hq, spec.Hkv, spec.D, spec.B, dt)
    bound = _bound(spec.R, spec.T, int(spec.seq_lens.max()), spec.Hq, spec.Hkv, spec.D, spec.B, dt)
    assert bound >= exact > 0


def test_bound_covers_every_serving_trace_step():
    cfg = st.TraceConfig()
    plans = st.drive(pa.Scheduler(**st.scheduler_args(cfg)), cfg)
    Lmax = st.max_seq_len(cfg)
    bound = _bound(cfg.max_num_seqs, cfg.max_num_batched_tokens, Lmax, 32, 8, 128, cfg.block_size,
                   pa.PA_BF16)
    worst = 0
    for p in plans:
        if not p["sched"]:
            continue
        ql, cp, _, _, _ = st.step_arrays(p, cfg.block_size)
        assert int(ql.sum()) <= cfg.max_num_batched_tokens and len(ql) <= cfg.max_num_seqs
        assert int((ql + cp).max()) <= Lmax
        worst = max(worst, _exact(ql, cp, 32, 8, 128, cfg.block_size, pa.PA_BF16))
    assert bound >= worst > 0


def _corner_steps(R, T, L, TQ):
    """Steps at the corners of the derivation, within (R, T, L)."""
    n = min(R, T)
    yield [1] * n, [L - 1] * n                                   # every request a decode at L
    k = min(R, T // TQ)
    if k:
        yield [TQ] * k, [L - TQ] * k                             # full q-tiles deep in L
    k = min(R, T // (TQ + 1))
    if k:
        yield [TQ + 1] * k, [L - TQ - 1] * k                     # a partial tile per request
    k = min(R, T // 2)
    if k:
        yield [2] * k, [L - 2] * k                               # many two-token chunks
    q = min(T, L)
    yield [q], [L - q]                                           # one long prefill ending at L
    yield [q], [0] if q == L else [L - q]
    h = min(R // 2, T // 2)
    if h:
        qc = max(2, (T - h) // max(1, R - h))
        m = min(R - h, (T - h) // qc)
        yield [1] * h + [qc] * m, [L - 1] * h + [L - qc] * m     # half decodes, half chunks


GEOS = [("bf16", 32, 8, 128, 16), ("bf16", 64, 8, 128, 32), ("bf16", 8, 8, 64, 16),
        ("bf16", 16, 8, 128, 48), ("f32", 8, 2, 64, 16), ("f32", 32, 8, 128, 16)]
LIMITS = [(256, 8192, 32968), (64, 64, 4096), (515, 2048, 16384), (8, 300, 70000), (4, 245, 211)]
KNOBS = [{}, {"split_keys": 64}, {"split_keys": 1000}, {"chunk_segment": 512},
         {"chunk_segment": 1024}, {"split_rule": 1}, {"chunk_path": 1}]


@pytest.mark.parametrize("knobs", KNOBS, ids=[",".join(f"{k}={v}" for k, v in kn.items()) or "default"
                                              for kn in KNOBS])
def test_bound_covers_corner_and_random_steps(knobs):
    g = np.random.default_rng(len(str(knobs)))
    with pa.tuning(**knobs):
        for dtype, Hq, Hkv, D, B in GEOS:
            dt = _dt(dtype)
            TQ = 128 // (Hq // Hkv)
            for R, T, L in LIMITS:
                bound = _bound(R, T, L, Hq, Hkv, D, B, dt)
                steps = list(_corner_steps(R, T, L, TQ))
                for _ in range(12):          # random steps within the limits
                    r = int(g.integers(1, R + 1))
                    ql = np.ones(r, np.int64)
                    budget = T - r
                    for i in range(r):
                        if budget <= 0:
                            break
                        if g.random() < 0.4:
                            extra = int(g.integers(0, min(budget, L - 1) + 1))
                            ql[i] += extra
                            budget -= extra
                    comp = [int(g.integers(0, L - q + 1)) for q in ql]
                    steps.append((ql.tolist(), comp))
                for ql, comp in steps:
                    assert len(ql) <= R and sum(ql) <= T
                    assert max(q + c for q, c in zip(ql, comp)) <= L
                    exact = _exact(ql, comp, Hq, Hkv, D, B, dt)
                    assert bound >= exact, (dtype, Hq, Hkv, D, B, (R, T, L), knobs, exact, bound)


def test_bound_argument_checks():
    with pytest.raises(pa.PAError):
        _bound(-1, 8, 8, 32, 8, 128, 16, pa.PA_BF16)
    with pytest.raises(pa.PAError):
        _bound(4, 8, 8, 32, 8, 96, 16, pa.PA_BF16)
    assert _bound(0, 0, 0, 32, 8, 128, 16, pa.PA_BF16) >= 0


def test_tuning_knobs_set_get_restore():
    assert pa.get_tuning("split_keys") == 0
    with pa.tuning(split_keys=256, decode_kernel=2):
        assert pa.get_tuning("split_keys") == 256 and pa.get_tuning("decode_kernel") == 2
    assert pa.get_tuning("split_keys") == 0 and pa.get_tuning("decode_kernel") == 0
    with pytest.raises(pa.PAError):
        pa.set_tuning(99, 1)
    with pytest.raises(pa.PAError):
        pa.set_tuning("split_keys", -3)
    assert pa.lib().pa_get_tuning(99) == -1


def test_forced_partition_changes_the_exact_size():
    """The knobs reach the planner: 64-key partitions need more partial slots
    than the rule's choice for the same decodes."""
    spec = configs.c2()
    dt = pa.PA_BF16
    base = _exact(spec.query_lens, spec.num_computed, spec.Hq, spec.Hkv, spec.D, spec.B, dt)
    with pa.tuning(split_keys=64):
        fine = _exact(spec.query_lens, spec.num_computed, spec.Hq, spec.Hkv, spec.D, spec.B, dt)
    assert fine > base


def test_plan_and_run_host_checks():
    """pa_attention_run refuses a plan that pa_attention_plan did not fill, and
    pa_attention_plan refuses bad steps on the host (dummy device pointers,
    never dereferenced)."""
    import ctypes
    L = pa.lib()
    rec = pa._lib.StepPlanRecord()
    rc = L.pa_attention_run(ctypes.byref(rec), 4096, 4096, 4096, 4096, 0.125, None)
    assert pa.status_str(rc) == "PA_ERR_BAD_STATE"
    assert pa.status_str(L.pa_attention_run(None, 4096, 4096, 4096, 4096, 0.125, None)) == "PA_ERR_NULL_PTR"
    qsl = np.array([0, 1], np.int32)
    p32 = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))  # noqa: E731

    def plan(sl, wsb=1 << 20, D=64):
        return pa.status_str(L.pa_attention_plan(ctypes.byref(rec), 4096, 1, 4096, 4096, 4096, p32(qsl),
                                                 p32(np.array(sl, np.int32)), 1, 1, 8, 2, D, 4, 16, 1,
                                                 4096, wsb, None))
    assert plan([17]) == "PA_ERR_OUT_OF_RANGE"
    assert plan([0]) == "PA_ERR_INCONSISTENT_METADATA"
    assert plan([5], D=96) == "PA_ERR_UNSUPPORTED"
    assert plan([5], wsb=16) == "PA_ERR_WORKSPACE_TOO_SMALL"
    # a refused plan stays unusable
    rc = L.pa_attention_run(ctypes.byref(rec), 4096, 4096, 4096, 4096, 0.125, None)
    assert pa.status_str(rc) == "PA_ERR_BAD_STATE"
