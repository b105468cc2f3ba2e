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
