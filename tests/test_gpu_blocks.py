"""GPU tests of block movement: copy-on-write of shared blocks planned by the
product scheduler (forked sequences that share a partly filled block), and
swap-out / swap-in of blocks between the device cache and a pinned host pool
(pa_copy_blocks).  Copies are exact, so caches are compared bit for bit;
attention after the copies is compared with the fp64 oracle on each
sequence's own logical history (bf16 tolerance)."""
import numpy as np
import pytest

import oracle
from helpers import assert_close, bits, say, storage_np
from workloads import rng
from workloads.serving_trace import token_row_keys

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_attention_reshape_amd as pa  # noqa: E402
from workloads import _lib as wl  # noqa: E402

HQ, HKV, D, B = 32, 8, 128, 16
SEED = 31


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu-test] {request.node.name}")
    yield
    torch.cuda.synchronize()


def _keys(tag, owners, positions):
    return token_row_keys(SEED, tag, 0, owners, positions)


def _fill(t, keys):
    wl.fill_rows(t, "bf16", row_keys=torch.from_numpy(keys.view(np.int64)).cuda())


def test_fork_copy_on_write_then_attention():
    """Parent prefills 20 tokens (block 1 partly filled), two children fork
    from it; each then decodes its own tokens.  The plan's copy-on-write
    copies run before each step's cache write."""
    nb = 64
    order = np.random.default_rng(3).permutation(nb).astype(np.int32)
    s = pa.Scheduler(nb, B, 8, 256, 64, order)
    prompt = 20
    s.add_request(0, prompt, 6)
    kc = torch.empty((nb, B, HKV, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    kc.view(torch.int16).fill_(0x7FC0)
    vc.view(torch.int16).fill_(0x7FC0)
    ws = pa.alloc_workspace(pa.attention_workspace_bound(8, 256, nb * B, HQ, HKV, D, B, pa.PA_BF16))
    owner_of = {}          # (sequence, position) -> whose token values live there
    copies_seen = 0
    checked = 0
    for step in range(6):
        if step == 1:
            s.fork(0, 1, 6)
            s.fork(0, 2, 6)
            for child in (1, 2):          # the children share the parent's history
                for p in range(prompt):
                    owner_of[(child, p)] = owner_of[(0, p)]
        info, ids, comp, ql, bt, pre, cps = s.schedule_arrays()
        assert len(pre) == 0
        if len(cps):
            copies_seen += len(cps)
            pairs = torch.from_numpy(np.ascontiguousarray(cps)).cuda()
            pa.copy_blocks(kc, kc, pairs)
            pa.copy_blocks(vc, vc, pairs)
        # the step's tokens: each sequence's own values (positions < prompt
        # belong to the parent, later positions to the sequence itself)
        own, pos = [], []
        for rid, c, n in zip(ids, comp, ql):
            for p in range(c, c + n):
                o = 0 if p < prompt else int(rid)
                owner_of[(int(rid), p)] = o
                own.append(o)
                pos.append(p)
        own, pos = np.array(own), np.array(pos)
        T = len(pos)
        q = torch.empty((T, HQ, D), dtype=torch.bfloat16, device="cuda")
        k = torch.empty((T, HKV, D), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        _fill(q, _keys(rng.TAG_Q, own, pos))
        _fill(k, _keys(rng.TAG_K, own, pos))
        _fill(v, _keys(rng.TAG_V, own, pos))
        qsl, sl, sm = pa.build_step_metadata(ql, comp, bt, B, nb)
        pa.write_kv(k, v, kc, vc, torch.from_numpy(sm).cuda())
        out = torch.empty_like(q)
        pa.attention(out, q, kc, vc, torch.from_numpy(bt).cuda(), torch.from_numpy(qsl).cuda(),
                     torch.from_numpy(sl).cuda(), torch.from_numpy(comp).cuda(), qsl, sl,
                     1.0 / np.sqrt(D), workspace=ws)
        torch.cuda.synchronize()
        for i, (rid, c, n) in enumerate(zip(ids, comp, ql)):
            rid, L = int(rid), int(c + n)
            owners = np.array([owner_of[(rid, p)] for p in range(L)])
            kh = rng.row_values(_keys(rng.TAG_K, owners, np.arange(L)), HKV * D, "bf16").reshape(L, HKV, D)
            vh = rng.row_values(_keys(rng.TAG_V, owners, np.arange(L)), HKV * D, "bf16").reshape(L, HKV, D)
            blocks = bt[i][bt[i] >= 0]
            gk = oracle.gather_kv(storage_np(kc[torch.from_numpy(blocks.astype(np.int64)).cuda()]),
                                  np.arange(len(blocks)), L, B)
            gv = oracle.gather_kv(storage_np(vc[torch.from_numpy(blocks.astype(np.int64)).cuda()]),
                                  np.arange(len(blocks)), L, B)
            assert np.array_equal(bits(gk), bits(kh)), f"step {step} seq {rid}: key history differs"
            assert np.array_equal(bits(gv), bits(vh)), f"step {step} seq {rid}: value history differs"
            t0 = int(qsl[i])
            qh = storage_np(q[t0:t0 + int(n)])
            want, _ = oracle.attention_rows(qh, kh, vh, np.arange(int(c), L), 1.0 / np.sqrt(D), "bf16")
            got = oracle.as_f64(storage_np(out[t0:t0 + int(n)]), "bf16")
            assert_close(got, want, "bf16", f"step {step} seq {rid}")
            checked += 1
        s.commit()
    m = s.metrics()
    say(f"copy-on-write copies {copies_seen}, sequences checked {checked}, q_live {m['q_live']}")
    assert copies_seen == 2 and m["cow_copies"] == 2 and checked >= 13


def test_swap_out_and_in_round_trip_bit_exact():
    """Blocks of every layer's K and V pool go to a pinned host pool and come
    back into other device blocks unchanged."""
    layers, nb, hb = 8, 96, 40
    pools = torch.empty((2 * layers, nb, B, HKV, D), dtype=torch.bfloat16, device="cuda")
    keys = np.arange(2 * layers * nb * B, dtype=np.uint64) * np.uint64(2654435761) + np.uint64(17)
    flat = pools.view(2 * layers * nb * B, HKV, D)
    _fill(flat, keys)
    host = torch.empty((2 * layers, hb, B, HKV, D), dtype=torch.bfloat16, pin_memory=True)
    host.view(torch.int16).fill_(0x7FC0)
    g = np.random.default_rng(8)
    out_src = g.choice(nb, 24, replace=False).astype(np.int32)
    out_dst = g.choice(hb, 24, replace=False).astype(np.int32)
    before = storage_np(pools)
    pa.copy_blocks(pools, host, torch.from_numpy(np.stack([out_src, out_dst], 1)).cuda())
    torch.cuda.synchronize()
    hs = storage_np(host)
    assert np.array_equal(bits(hs[:, out_dst]), bits(before[:, out_src])), "swap-out copy differs"
    others = np.setdiff1d(np.arange(hb), out_dst)
    assert np.all(hs[:, others] == 0x7FC0), "host slots outside the mapping changed"
    # the device blocks are reused by others, then the request swaps back in elsewhere
    pools[:, torch.from_numpy(out_src.astype(np.int64)).cuda()] = 0
    in_dst = np.setdiff1d(np.arange(nb), out_src)[:24].astype(np.int32)
    pa.copy_blocks(host, pools, torch.from_numpy(np.stack([out_dst, in_dst], 1)).cuda())
    torch.cuda.synchronize()
    after = storage_np(pools)
    assert np.array_equal(bits(after[:, in_dst]), bits(before[:, out_src])), "swap-in copy differs"
    untouched = np.setdiff1d(np.arange(nb), np.concatenate([out_src, in_dst]))
    assert np.array_equal(bits(after[:, untouched]), bits(before[:, untouched]))


def test_swap_beside_a_step_on_a_second_stream():
    """A swap-out of blocks the step does not use (every layer's K and V block,
    to a pinned host pool, on the copy engines: pa_swap_blocks) on a second
    stream of default priority, ordered
    after the inputs with an event and joined afterwards, runs while a step
    (cache write + attention) runs on the current stream: the swapped bytes are
    exact, the step's outputs and caches equal the same step run alone bit for
    bit, and the swap-in onto other free blocks is exact."""
    from workloads import configs
    from helpers import run_step
    spec = configs.custom("swap-step", "bf16", HQ, HKV, D, B, [1, 1, 200, 1, 1], [3000, 900, 700, 4000, 60], 51,
                          pool_factor=1.6)
    used = np.unique(np.concatenate([spec.block_table[r, :-(-int(spec.seq_lens[r]) // B)]
                                     for r in range(spec.R)]))
    free = np.setdiff1d(np.arange(spec.num_blocks), used).astype(np.int32)
    assert len(free) >= 64
    swap_src, swap_back = free[:32], free[32:64]
    base = spec.device_inputs()
    # step alone
    alone = {k: (v.clone() if hasattr(v, "clone") else v) for k, v in base.items()}
    _, out_alone, _ = run_step(spec, pa, dev_inputs=alone)
    torch.cuda.synchronize()
    # more layers' pools beside layer 0, so the swap is long enough to overlap the step
    layers = 16
    extra = torch.empty((2 * layers, spec.num_blocks, B, HKV, D), dtype=torch.bfloat16, device="cuda")
    keys = np.arange(extra.numel() // (HKV * D), dtype=np.uint64) * np.uint64(0x9E3779B1) + np.uint64(5)
    _fill(extra.view(-1, HKV, D), keys)
    host = torch.empty((2 * layers, 64, B, HKV, D), dtype=torch.bfloat16, pin_memory=True)
    host.view(torch.int16).fill_(0x7FC0)
    before = storage_np(extra[:, torch.from_numpy(swap_src.astype(np.int64)).cuda()])
    pairs_out = np.stack([swap_src, np.arange(32, dtype=np.int32)], 1)
    d = {k: (v.clone() if hasattr(v, "clone") else v) for k, v in base.items()}
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()                 # default priority
    ready = torch.cuda.Event()
    ready.record(main)                         # inputs and pools are in place
    side.wait_event(ready)
    with torch.cuda.stream(side):
        for _ in range(4):                     # a few hundred MB over the host link, on the copy engines
            pa.swap_blocks(extra, host, pairs_out, stream=side)
    _, out, _ = run_step(spec, pa, dev_inputs=d)   # the step, on the current stream
    done = torch.cuda.Event()
    done.record(side)
    main.wait_event(done)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_alone.view(torch.int16)), "step output differs beside the swap"
    assert torch.equal(d["key_cache"].view(torch.int16), alone["key_cache"].view(torch.int16))
    assert torch.equal(d["value_cache"].view(torch.int16), alone["value_cache"].view(torch.int16))
    assert np.array_equal(bits(storage_np(host[:, :32])), bits(before)), "swapped-out blocks differ"
    # swap back in, onto other free blocks, beside another run of the step
    pairs_in = np.stack([np.arange(32, dtype=np.int32), swap_back], 1)
    ready.record(main)
    side.wait_event(ready)
    with torch.cuda.stream(side):
        pa.swap_blocks(host, extra, pairs_in, stream=side)
    d2 = {k: (v.clone() if hasattr(v, "clone") else v) for k, v in base.items()}
    _, out2, _ = run_step(spec, pa, dev_inputs=d2)
    done.record(side)
    main.wait_event(done)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out_alone.view(torch.int16))
    back = storage_np(extra[:, torch.from_numpy(swap_back.astype(np.int64)).cuda()])
    assert np.array_equal(bits(back), bits(before)), "swapped-in blocks differ"


def test_swap_blocks_copy_engines_round_trip():
    """pa_swap_blocks: runs of consecutive blocks (one 2-D copy each) and
    scattered blocks go out to a pinned host pool and come back exactly;
    nothing else changes."""
    layers, nb, hb = 6, 80, 48
    pools = torch.empty((2 * layers, nb, B, HKV, D), dtype=torch.bfloat16, device="cuda")
    keys = np.arange(2 * layers * nb * B, dtype=np.uint64) * np.uint64(0x2545F491) + np.uint64(3)
    _fill(pools.view(-1, HKV, D), keys)
    host = torch.empty((2 * layers, hb, B, HKV, D), dtype=torch.bfloat16, pin_memory=True)
    host.view(torch.int16).fill_(0x7FC0)
    g = np.random.default_rng(12)
    src = np.concatenate([np.arange(10, 20), g.choice(np.arange(30, nb), 14, replace=False)]).astype(np.int32)
    dst = np.concatenate([np.arange(5, 15), g.choice(np.arange(20, hb), 14, replace=False)]).astype(np.int32)
    before = storage_np(pools)
    pa.swap_blocks(pools, host, np.stack([src, dst], 1))
    torch.cuda.synchronize()
    hs = storage_np(host)
    assert np.array_equal(bits(hs[:, dst]), bits(before[:, src])), "swap-out differs"
    assert np.all(hs[:, np.setdiff1d(np.arange(hb), dst)] == 0x7FC0)
    back = np.setdiff1d(np.arange(nb), src)[:24].astype(np.int32)
    pa.swap_blocks(host, pools, np.stack([dst, back], 1))
    torch.cuda.synchronize()
    after = storage_np(pools)
    assert np.array_equal(bits(after[:, back]), bits(before[:, src])), "swap-in differs"
    rest = np.setdiff1d(np.arange(nb), back)
    assert np.array_equal(bits(after[:, rest]), bits(before[:, rest]))
