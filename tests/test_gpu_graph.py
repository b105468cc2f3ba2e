"""GPU test: one whole step (device slot mapping, cache write, attention)
captured in a HIP graph and replayed.

The library allocates nothing, records no memset and never synchronises
inside a call, so a serving loop can capture a step whose sizes stay fixed
(the host mirrors of query_start_loc / seq_lens size the launches at capture
time) and replay it with new values in the same buffers.  Each replay runs
after unrelated eager work and a synchronisation, and must match an eager
step on the same inputs bit for bit."""
import numpy as np
import pytest

from helpers import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_attention_reshape_amd as pa  # noqa: E402
from workloads import configs  # noqa: E402


def _eager(spec, d, slots, kc, vc, out, ws):
    pa.compute_slot_mapping(slots, d["block_table"], d["query_start_loc"], d["num_computed"],
                            spec.num_blocks, spec.B)
    pa.write_kv(d["key"], d["value"], kc, vc, slots)
    pa.attention(out, d["query"], kc, vc, d["block_table"], d["query_start_loc"], d["seq_lens"],
                 d["num_computed"], spec.query_start_loc, spec.seq_lens, spec.scale, workspace=ws)


def test_step_graph_capture_and_replay():
    say("\n[gpu-test] step graph capture and replay")
    spec = configs.custom("graph", "bf16", 32, 8, 128, 16, [1, 1, 200, 1, 64, 1],
                          [3000, 17, 900, 700, 0, 1500], 21)
    dev = torch.device("cuda:0")
    d = spec.device_inputs(device=dev)
    kc0, vc0 = d["key_cache"].clone(), d["value_cache"].clone()   # pre-write pools
    slots = torch.empty((spec.T,), dtype=torch.int64, device=dev)
    # a workspace sized once from the step limits (as a serving loop would)
    ws = pa.alloc_workspace(pa.attention_workspace_bound(spec.R, spec.T, int(spec.seq_lens.max()), spec.Hq,
                                                         spec.Hkv, spec.D, spec.B, pa.PA_BF16), dev)
    assert ws.numel() >= pa.attention_workspace_size(spec.query_start_loc, spec.seq_lens, spec.Hq, spec.Hkv,
                                                     spec.D, spec.B, pa.PA_BF16)

    # eager reference on the original inputs
    kc, vc = kc0.clone(), vc0.clone()
    ref = torch.empty_like(d["query"])
    _eager(spec, d, slots, kc, vc, ref, ws)
    torch.cuda.synchronize()

    # capture the same step into a graph (on torch's capture stream)
    kc_g, vc_g = kc0.clone(), vc0.clone()
    out_g = torch.empty_like(d["query"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm-up outside the graph, as torch recommends
        _eager(spec, d, slots, kc_g, vc_g, out_g, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    out_g.fill_(float("nan"))
    with torch.cuda.graph(g):
        _eager(spec, d, slots, kc_g, vc_g, out_g, ws)
    torch.cuda.synchronize()

    scratch = torch.randn(1 << 20, device=dev)
    for rep in range(3):
        out_g.fill_(float("nan"))
        kc_g.copy_(kc0)
        vc_g.copy_(vc0)
        scratch.mul_(1.0001).add_(0.5)           # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), ref.view(torch.int16)), f"replay {rep}: output differs"
        assert torch.equal(kc_g.view(torch.int16), kc.view(torch.int16)), f"replay {rep}: key cache differs"
        assert torch.equal(vc_g.view(torch.int16), vc.view(torch.int16)), f"replay {rep}: value cache differs"

    # new query values in the same buffer: the replay reads them
    gen = torch.Generator(device="cpu").manual_seed(5)
    d["query"].copy_(torch.randn(d["query"].shape, generator=gen).to(dev, torch.bfloat16))
    kc, vc = kc0.clone(), vc0.clone()
    ref2 = torch.empty_like(d["query"])
    _eager(spec, d, slots, kc, vc, ref2, ws)
    kc_g.copy_(kc0)
    vc_g.copy_(vc0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out_g.view(torch.int16), ref2.view(torch.int16)), "replay after new inputs differs"
    assert not torch.equal(ref2.view(torch.int16), ref.view(torch.int16))
    say("graph replays match the eager step bit for bit")
