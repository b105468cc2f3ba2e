"""GPU test of pa_attention_noalloc (the entry point for callers that cannot
allocate): through the C ABI, its outputs equal pa_attention's (which plans
into a caller workspace) bit for bit on two calls in a row, the second with
a smaller step, and a step that needs more than the static scratch is
refused before anything runs; C1-C4 and every step of the serving trace fit
in the static scratch."""
import numpy as np
import pytest

from helpers import assert_close, check_requests, say, storage_np
from workloads import configs

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_attention_reshape_amd as pa  # noqa: E402


def _prepare(spec):
    d = spec.device_inputs()
    qsl, sl, sm = pa.build_step_metadata(spec.query_lens, spec.num_computed, spec.block_table,
                                         spec.B, spec.num_blocks)
    pa.write_kv(d["key"], d["value"], d["key_cache"], d["value_cache"], torch.from_numpy(sm).cuda())
    return d, qsl, sl


def _both(spec):
    """(pa_attention output, pa_attention_noalloc output, inputs)."""
    d, qsl, sl = _prepare(spec)
    dt = pa.PA_BF16 if spec.dtype == "bf16" else pa.PA_F32
    ws = pa.alloc_workspace(pa.attention_workspace_size(qsl, sl, spec.Hq, spec.Hkv, spec.D, spec.B, dt))
    ref = torch.empty_like(d["query"])
    pa.attention(ref, d["query"], d["key_cache"], d["value_cache"], d["block_table"], d["query_start_loc"],
                 d["seq_lens"], d["num_computed"], qsl, sl, spec.scale, ws)
    out = torch.full_like(d["query"], float("nan"))
    pa.attention_noalloc(out, d["query"], d["key_cache"], d["value_cache"], d["block_table"],
                         d["query_start_loc"], d["seq_lens"], d["num_computed"], qsl, sl, spec.scale)
    torch.cuda.synchronize()
    return ref, out, d


def test_noalloc_matches_attention_on_two_calls_second_smaller():
    say("\n[gpu-test] noalloc: mixed step (C3), then a smaller mixed step")
    big = configs.c3()
    small = configs.custom("noalloc-small", "bf16", 32, 8, 128, 16, [1, 1, 90, 1], [4000, 30, 500, 64], 61)
    for spec in (big, small):
        ref, out, d = _both(spec)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{spec.name}: outputs differ"
        say(f"noalloc {spec.name}: T={spec.T} bitwise equal to pa_attention")
    # the smaller call's rows also meet the oracle (every request)
    err = check_requests(small, out, d["key_cache"], d["value_cache"], range(small.R), what="noalloc small")
    say(f"noalloc small vs oracle: max abs err {err:.2e}")


def test_noalloc_fp32_and_oversize_refused():
    say("\n[gpu-test] noalloc: fp32 step; oversize step refused")
    spec = configs.c1()
    ref, out, d = _both(spec)
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    # 64-key partitions over 512 decodes of 32768 keys: the plan needs far more
    # than the static scratch; refused on the host, nothing enqueued
    R, L = 512, 32768
    qsl = np.arange(R + 1, dtype=np.int32)
    sl = np.full(R, L, np.int32)
    with pa.tuning(split_keys=64):
        need = pa.attention_workspace_size(qsl, sl, 32, 8, 128, 16, pa.PA_BF16)
        assert need > pa.NOALLOC_SCRATCH_BYTES
        q = torch.zeros((R, 32, 128), dtype=torch.bfloat16, device="cuda")
        kc = torch.zeros((4, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
        bt = torch.zeros((R, L // 16), dtype=torch.int32, device="cuda")
        z = torch.zeros(R + 1, dtype=torch.int32, device="cuda")
        with pytest.raises(pa.PAError) as e:
            pa.attention_noalloc(q, q, kc, kc, bt, z, z[:R], z[:R], qsl, sl, 0.1)
        assert e.value.status_name == "PA_ERR_WORKSPACE_TOO_SMALL"
        assert "static scratch" in str(e.value)
    torch.cuda.synchronize()


def test_static_scratch_covers_the_configurations_and_the_serving_trace():
    """The exact workspace of C1-C4 and of every step of the 2048-request
    serving trace, sized on this device (its occupancy sets the partition
    lengths), fits in the static scratch, so those steps never need a
    caller workspace.  Host sizing only; nothing is launched."""
    import test_workspace_bound as wb
    from workloads import serving_trace as st
    torch.cuda.set_device(0)
    sizes = {}
    for name in ("c1", "c2", "c3", "c4"):
        s = configs.BUILDERS[name]()
        sizes[name] = wb._exact(s.query_lens, s.num_computed, s.Hq, s.Hkv, s.D, s.B, wb._dt(s.dtype))
    cfg = st.TraceConfig()
    worst = 0
    for p in st.drive(pa.Scheduler(**st.scheduler_args(cfg)), cfg):
        if p["sched"]:
            ql, cp, _, _, _ = st.step_arrays(p, cfg.block_size)
            worst = max(worst, wb._exact(ql, cp, 32, 8, 128, cfg.block_size, pa.PA_BF16))
    sizes["serving trace (worst step)"] = worst
    say("workspace MiB: " + ", ".join(f"{k} {v / 2**20:.1f}" for k, v in sizes.items()))
    assert all(0 < v <= pa.NOALLOC_SCRATCH_BYTES for v in sizes.values()), sizes
