"""Pins for the CPU oracle: values the pages print, closed forms, brute force
on tiny inputs, library special cases and structural invariants.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, the wrong GQA grouping, a mask off
by one, a wrong block lookup) fails at least one of them.
"""
import json
import math
import os
import random

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# slot mapping
# ----------------------------------------------------------------------------
def test_slot_worked_example():
    g = _golden("slot_example.json")
    bt = np.array([g["block_table_row"]], dtype=np.int32)
    # request 0 schedules one token at absolute position 25
    s = oracle.slot_mapping(bt, [1], [g["position"]], g["block_size"])
    assert s.dtype == np.int64
    assert int(s[0]) == g["slot"]
    assert int(s[0]) // g["block_size"] == g["physical_block"]
    assert int(s[0]) % g["block_size"] == g["offset"]


def _enumerated_slots(row, nblocks, B):
    """Independent formulation: list every slot of the request's blocks in
    logical order; position p is the p-th entry."""
    out = []
    for blk in row[:nblocks]:
        for off in range(B):
            out.append(int(blk) * B + off)
    return out


@pytest.mark.parametrize("B", [1, 2, 4, 16])
def test_slot_mapping_brute_force(B):
    rng = random.Random(11 + B)
    R = 5
    M = 12
    perm = list(range(R * M))
    rng.shuffle(perm)
    bt = np.array(perm, dtype=np.int32).reshape(R, M)
    qlens, comp = [], []
    for r in range(R):
        L = rng.randint(1, M * B)
        q = rng.randint(0, L)
        qlens.append(q)
        comp.append(L - q)
    got = oracle.slot_mapping(bt, qlens, comp, B)
    want = []
    for r in range(R):
        L = qlens[r] + comp[r]
        slots = _enumerated_slots(bt[r], -(-L // B), B)
        want.extend(slots[comp[r]:L])
    assert got.tolist() == want


def test_block_table_examples_map_positions():
    g = _golden("block_table_examples.json")
    # P5: pi = [7, 2, 9]; with B = 4 the request's positions 0..11 land in
    # blocks 7,7,7,7,2,2,2,2,9,9,9,9
    bt = np.array([g["p5_pi"]], dtype=np.int32)
    s = oracle.slot_mapping(bt, [12], [0], 4)
    assert (s // 4).tolist() == [7] * 4 + [2] * 4 + [9] * 4
    assert (s % 4).tolist() == [0, 1, 2, 3] * 3
    # P1: request 0 [5, 8, 12], request 1 [3, 7], B = 16, one decode token each
    t = g["p1_tables"]
    bt = np.array([t[0], t[1] + [-1]], dtype=np.int32)
    s = oracle.slot_mapping(bt, [1, 1], [40, 20], 16)
    assert s.tolist() == [12 * 16 + 8, 7 * 16 + 4]


# ----------------------------------------------------------------------------
# write / gather
# ----------------------------------------------------------------------------
def test_write_kv_bitexact_and_skip():
    rng = np.random.default_rng(3)
    nb, B, Hkv, D = 6, 4, 2, 8
    kc = rng.integers(0, 65535, size=(nb, B, Hkv, D), dtype=np.uint16)
    vc = kc.copy() ^ np.uint16(0x5555)
    k0, v0 = kc.copy(), vc.copy()
    key = rng.integers(0, 65535, size=(4, Hkv, D), dtype=np.uint16)
    val = rng.integers(0, 65535, size=(4, Hkv, D), dtype=np.uint16)
    slots = np.array([5, -1, 23, 0], dtype=np.int64)
    oracle.write_kv(kc, vc, key, val, slots, B)
    assert np.array_equal(kc[1, 1], key[0]) and np.array_equal(vc[1, 1], val[0])
    assert np.array_equal(kc[5, 3], key[2]) and np.array_equal(vc[5, 3], val[2])
    assert np.array_equal(kc[0, 0], key[3])
    touched = np.zeros((nb, B), dtype=bool)
    touched[1, 1] = touched[5, 3] = touched[0, 0] = True
    assert np.array_equal(kc[~touched], k0[~touched])
    assert np.array_equal(vc[~touched], v0[~touched])


def test_write_kv_rejects_duplicates_and_overflow():
    kc = np.zeros((2, 4, 1, 2), np.float32)
    vc = kc.copy()
    x = np.ones((2, 1, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.write_kv(kc, vc, x, x, np.array([3, 3]), 4)
    with pytest.raises(IndexError):
        oracle.write_kv(kc, vc, x[:1], x[:1], np.array([8]), 4)


def test_gather_brute_force():
    rng = np.random.default_rng(5)
    nb, B, Hkv, D = 9, 4, 2, 3
    cache = rng.standard_normal((nb, B, Hkv, D)).astype(np.float32)
    row = np.array([7, 2, 5, -1], dtype=np.int32)
    L = 10
    got = oracle.gather_kv(cache, row, L, B)
    slots = _enumerated_slots(row, 3, B)
    for p in range(L):
        blk, off = divmod(slots[p], B)
        assert np.array_equal(got[p], cache[blk, off])


# ----------------------------------------------------------------------------
# block accounting and preemption accounting
# ----------------------------------------------------------------------------
def _allocate_token_by_token(length, B):
    """Brute force: append tokens one at a time, opening a new block whenever
    the current one is full."""
    blocks, used_in_last = 0, B
    for _ in range(length):
        if used_in_last == B:
            blocks += 1
            used_in_last = 0
        used_in_last += 1
    return blocks


def test_tail_waste_table():
    g = _golden("tail_waste.json")
    lengths = g["lengths"]
    for row in g["rows"]:
        acc = oracle.block_accounting(lengths, row["block"])
        assert acc["entries"] == row["entries"]
        assert acc["allocated"] == row["allocated"]
        assert acc["waste"] == row["waste"]
        assert acc["blocks"] == [_allocate_token_by_token(t, row["block"]) for t in lengths]
        for w in acc["tail_waste"]:
            assert 0 <= w < row["block"]
    assert len(lengths) * g["declared_max"] == g["contiguous_max_reservation_slots"]


@pytest.mark.parametrize("B", [1, 3, 16, 32])
def test_block_accounting_brute_force(B):
    rng = random.Random(B)
    lengths = [rng.randint(1, 500) for _ in range(20)]
    acc = oracle.block_accounting(lengths, B)
    assert acc["blocks"] == [_allocate_token_by_token(t, B) for t in lengths]
    assert acc["allocated"] - sum(lengths) == acc["waste"]


def test_preemption_accounting_golden():
    g = _golden("preemption_accounting.json")
    a = oracle.preemption_accounting(g["cached_tokens"], g["block_size"],
                                     g["kv_bytes_per_token"], g["bandwidth_gbps"])
    assert a["released_blocks"] == g["released_blocks"]
    assert a["recompute_tokens"] == g["recompute_tokens"]
    assert round(a["swap_roundtrip_ms"], g["swap_roundtrip_ms_digits"]) == g["swap_roundtrip_ms_approx"]


def test_kv_bytes_per_token_matches_cache_layout():
    # one slot of the whole-model cache [layers, 2, blocks, block_size, Hkv, D]
    for L, Hkv, D, dt in [(32, 8, 128, np.uint16), (1, 2, 64, np.float32), (80, 8, 128, np.uint16)]:
        slot = np.zeros((L, 2, 1, 1, Hkv, D), dtype=dt)
        assert oracle.kv_bytes_per_token(L, Hkv, D, np.dtype(dt).itemsize) == slot.nbytes


# ----------------------------------------------------------------------------
# attention: brute force, library special cases, closed forms, invariants
# ----------------------------------------------------------------------------
def _random_step(rng, R, Hq, Hkv, D, B, maxlen, nb_extra=3, dtype="f32"):
    lens = [int(rng.integers(1, maxlen + 1)) for _ in range(R)]
    qlens = [int(rng.integers(1, L + 1)) for L in lens]
    comp = [L - q for L, q in zip(lens, qlens)]
    nblk = [-(-L // B) for L in lens]
    nb = sum(nblk) + nb_extra
    perm = rng.permutation(nb)
    M = max(nblk)
    bt = np.full((R, M), -1, dtype=np.int32)
    pos = 0
    for r in range(R):
        bt[r, :nblk[r]] = perm[pos:pos + nblk[r]]
        pos += nblk[r]
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1])
    if dtype == "f32":
        kc = rng.standard_normal((nb, B, Hkv, D)).astype(np.float32)
        vc = rng.standard_normal((nb, B, Hkv, D)).astype(np.float32)
        q = rng.standard_normal((T, Hq, D)).astype(np.float32)
    else:
        f = lambda shape: (rng.standard_normal(shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        kc, vc, q = f((nb, B, Hkv, D)), f((nb, B, Hkv, D)), f((T, Hq, D))
    return dict(lens=lens, qlens=qlens, comp=comp, bt=bt, qsl=qsl, kc=kc, vc=vc, q=q, nb=nb)


def _brute_attention(st, Hq, Hkv, D, B, scale, dtype):
    """Scalar loops: position p of request r is read from block
    bt[r][p // B] offset p % B; query head h uses kv head h // (Hq // Hkv)."""
    G = Hq // Hkv
    conv = (lambda x: float(x)) if dtype == "f32" else (
        lambda x: float(np.array([int(x) << 16], dtype=np.uint32).view(np.float32)[0]))
    T = int(st["qsl"][-1])
    out = np.zeros((T, Hq, D))
    for r in range(len(st["lens"])):
        a = int(st["qsl"][r])
        for i in range(st["qlens"][r]):
            t = a + i
            qpos = st["comp"][r] + i
            for h in range(Hq):
                g = h // G
                scores = []
                for j in range(qpos + 1):
                    blk = int(st["bt"][r][j // B])
                    off = j % B
                    s = 0.0
                    for d in range(D):
                        s += conv(st["q"][t, h, d]) * conv(st["kc"][blk, off, g, d])
                    scores.append(s * scale)
                mx = max(scores)
                ws = [math.exp(s - mx) for s in scores]
                tot = sum(ws)
                for d in range(D):
                    acc = 0.0
                    for j in range(qpos + 1):
                        blk = int(st["bt"][r][j // B])
                        acc += ws[j] * conv(st["vc"][blk, j % B, g, d])
                    out[t, h, d] = acc / tot
    return out


@pytest.mark.parametrize("B,dtype", [(1, "f32"), (2, "bf16"), (4, "f32"), (16, "bf16")])
def test_attention_brute_force(B, dtype):
    rng = np.random.default_rng(100 + B)
    Hq, Hkv, D = 4, 2, 5
    st = _random_step(rng, 3, Hq, Hkv, D, B, 40 if B > 1 else 20, dtype=dtype)
    scale = 1 / math.sqrt(D)
    got, _ = oracle.attention(st["q"], st["kc"], st["vc"], st["bt"], st["qsl"], st["lens"],
                              st["comp"], scale, B, dtype)
    want = _brute_attention(st, Hq, Hkv, D, B, scale, dtype)
    assert np.max(np.abs(got - want)) <= 1e-12


def _sdpa_reference(qf, kf, vf, c):
    """torch CPU fp64 scaled_dot_product_attention with a lower-right causal
    bias (query i of n at absolute position c + i sees keys 0..c+i) and torch's
    own GQA head grouping."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention.bias import causal_lower_right
    q = torch.from_numpy(qf).permute(1, 0, 2)[None]        # [1, Hq, n, D]
    k = torch.from_numpy(kf).permute(1, 0, 2)[None]
    v = torch.from_numpy(vf).permute(1, 0, 2)[None]
    n, L = qf.shape[0], kf.shape[0]
    assert L == c + n
    mask = causal_lower_right(n, L)
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (8, 1), (6, 3)])
def test_attention_matches_torch_sdpa(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    D, B = 16, 4
    st = _random_step(rng, 4, Hq, Hkv, D, B, 37)
    scale = 1 / math.sqrt(D)
    got, _ = oracle.attention(st["q"], st["kc"], st["vc"], st["bt"], st["qsl"], st["lens"],
                              st["comp"], scale, B, "f32")
    for r in range(4):
        a, b = st["qsl"][r], st["qsl"][r + 1]
        K = oracle.gather_kv(st["kc"], st["bt"][r], st["lens"][r], B).astype(np.float64)
        V = oracle.gather_kv(st["vc"], st["bt"][r], st["lens"][r], B).astype(np.float64)
        ref = _sdpa_reference(st["q"][a:b].astype(np.float64), K, V, st["comp"][r])
        assert np.allclose(got[a:b], ref, rtol=1e-12, atol=1e-12)


def test_chunked_trace_and_equivalence():
    g = _golden("chunk_trace.json")
    rng = np.random.default_rng(127)
    shape = tuple(g["shape"])
    q = rng.standard_normal(shape)
    k = rng.standard_normal(shape)
    v = rng.standard_normal(shape)
    scale = 1 / math.sqrt(shape[-1])
    full = oracle.dense_causal(q, k, v, scale)
    ch, trace = oracle.chunked_causal(q, k, v, g["chunk"], scale)
    assert [[a, b, list(shp)] for a, b, shp in trace] == g["trace"]
    assert np.allclose(ch, full, rtol=g["rtol"], atol=g["atol"])
    for chunk in [1, 2, 5, 7, 50]:
        ch, _ = oracle.chunked_causal(q, k, v, chunk, scale)
        assert np.max(np.abs(ch - full)) < 1e-13


def test_chunked_prefill_through_paged_cache_equals_full():
    """A prompt run as chunks (each chunk a step with num_computed = chunk
    start) through the paged cache equals the one-shot prefill."""
    rng = np.random.default_rng(9)
    Hq, Hkv, D, B, T = 4, 2, 8, 4, 23
    nb = 8
    perm = rng.permutation(nb)
    bt = perm[: -(-T // B)][None].astype(np.int32)
    kc = np.full((nb, B, Hkv, D), np.nan, np.float32)
    vc = kc.copy()
    q = rng.standard_normal((T, Hq, D)).astype(np.float32)
    k = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    scale = 0.3
    kc1, vc1 = kc.copy(), vc.copy()
    oracle.write_kv(kc1, vc1, k, v, oracle.slot_mapping(bt, [T], [0], B), B)
    full, _ = oracle.attention(q, kc1, vc1, bt, [0, T], [T], [0], scale, B, "f32")
    outs = []
    for a in range(0, T, 5):
        b = min(a + 5, T)
        oracle.write_kv(kc, vc, k[a:b], v[a:b], oracle.slot_mapping(bt, [b - a], [a], B), B)
        o, _ = oracle.attention(q[a:b], kc, vc, bt, [0, b - a], [b], [a], scale, B, "f32")
        outs.append(o)
    assert np.max(np.abs(np.concatenate(outs) - full)) < 1e-13


def test_special_cases_closed_form():
    rng = np.random.default_rng(4)
    Hq, Hkv, D, B = 4, 2, 6, 4
    # L = 1: the only visible key is position 0, softmax weight 1 -> out = v0
    kc = rng.standard_normal((3, B, Hkv, D)).astype(np.float32)
    vc = rng.standard_normal((3, B, Hkv, D)).astype(np.float32)
    bt = np.array([[2]], dtype=np.int32)
    q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    out, lse = oracle.attention(q, kc, vc, bt, [0, 1], [1], [0], 0.7, B, "f32")
    for h in range(Hq):
        assert np.array_equal(out[0, h], vc[2, 0, h // 2].astype(np.float64))
        s = 0.7 * float(q[0, h].astype(np.float64) @ kc[2, 0, h // 2].astype(np.float64))
        assert abs(lse[0, h] - s) < 1e-12
    # all keys equal -> uniform weights -> mean of the visible V rows
    kc[:] = kc[0, 0]
    out, lse = oracle.attention(q, kc, vc, np.array([[1, 0, 2]], np.int32), [0, 1], [10], [9],
                                1.0, B, "f32")
    vis = np.concatenate([vc[1], vc[0], vc[2]])[:10].astype(np.float64)
    for h in range(Hq):
        assert np.allclose(out[0, h], vis[:, h // 2].mean(axis=0), atol=1e-12)
    # GQA grouping: V of kv head g is the constant g -> query head h returns h // G
    vc2 = np.zeros_like(vc)
    for g in range(Hkv):
        vc2[:, :, g, :] = g
    out, _ = oracle.attention(q, kc, vc2, np.array([[1, 0, 2]], np.int32), [0, 1], [10], [9],
                              1.0, B, "f32")
    for h in range(Hq):
        assert np.all(out[0, h] == h // 2)
    # one dominant score -> output is (almost exactly) that key's V row
    kc3 = np.zeros_like(kc)
    qd = np.zeros((1, Hq, D), np.float32)
    qd[0, :, 0] = 1.0
    kc3[0, 2, :, 0] = 1000.0     # block 0 is logical block 1: position 4 + 2 = 6
    out, _ = oracle.attention(qd, kc3, vc, np.array([[1, 0, 2]], np.int32), [0, 1], [10], [9],
                              1.0, B, "f32")
    for h in range(Hq):
        assert np.allclose(out[0, h], vc[0, 2, h // 2], atol=1e-12)


def test_mask_is_causal_at_absolute_positions():
    """Changing a key beyond a query's absolute position leaves that query's
    output unchanged; changing one at or before it changes it."""
    rng = np.random.default_rng(8)
    Hq, Hkv, D, B = 2, 1, 4, 4
    st = _random_step(rng, 1, Hq, Hkv, D, B, 20, nb_extra=0)
    L, c = st["lens"][0], st["comp"][0]
    if st["qlens"][0] < 2:
        st["qlens"][0] = 2
        c = L - 2
        st["comp"][0] = c
        st["qsl"] = np.array([0, 2], np.int32)
        st["q"] = rng.standard_normal((2, Hq, D)).astype(np.float32)
    base, _ = oracle.attention(st["q"], st["kc"], st["vc"], st["bt"], st["qsl"], st["lens"],
                               st["comp"], 0.5, B, "f32")
    # key at position c + 1 is visible to row 1 only
    p = c + 1
    blk, off = int(st["bt"][0][p // B]), p % B
    kc = st["kc"].copy()
    kc[blk, off] += 3.0
    alt, _ = oracle.attention(st["q"], kc, st["vc"], st["bt"], st["qsl"], st["lens"],
                              st["comp"], 0.5, B, "f32")
    assert np.array_equal(alt[0], base[0])
    assert not np.allclose(alt[1], base[1])


def test_invariances_block_permutation_request_order_poison():
    rng = np.random.default_rng(21)
    Hq, Hkv, D, B = 4, 2, 8, 4
    st = _random_step(rng, 4, Hq, Hkv, D, B, 30, nb_extra=5)
    args = (0.35, B, "f32")
    base, _ = oracle.attention(st["q"], st["kc"], st["vc"], st["bt"], st["qsl"], st["lens"],
                               st["comp"], *args)
    # 1) relabel physical blocks, moving their data with them
    nb = st["nb"]
    perm = rng.permutation(nb)               # old id -> new id
    kc2 = np.empty_like(st["kc"])
    vc2 = np.empty_like(st["vc"])
    kc2[perm] = st["kc"]
    vc2[perm] = st["vc"]
    bt2 = np.where(st["bt"] >= 0, perm[np.maximum(st["bt"], 0)], -1).astype(np.int32)
    o2, _ = oracle.attention(st["q"], kc2, vc2, bt2, st["qsl"], st["lens"], st["comp"], *args)
    assert np.array_equal(o2, base)
    # 2) poison every slot no request may read (unused blocks, tail slots)
    kc3, vc3 = st["kc"].copy(), st["vc"].copy()
    readable = np.zeros((nb, B), dtype=bool)
    for r, L in enumerate(st["lens"]):
        for p in range(L):
            readable[st["bt"][r][p // B], p % B] = True
    kc3[~readable] = np.nan
    vc3[~readable] = np.nan
    o3, _ = oracle.attention(st["q"], kc3, vc3, st["bt"], st["qsl"], st["lens"], st["comp"], *args)
    assert np.array_equal(o3, base)
    # 3) reverse the request order in the flattened batch
    order = list(range(4))[::-1]
    q_parts = [st["q"][st["qsl"][r]:st["qsl"][r + 1]] for r in order]
    qsl4 = np.concatenate([[0], np.cumsum([st["qlens"][r] for r in order])]).astype(np.int32)
    o4, _ = oracle.attention(np.concatenate(q_parts), st["kc"], st["vc"], st["bt"][order], qsl4,
                             [st["lens"][r] for r in order], [st["comp"][r] for r in order], *args)
    for i, r in enumerate(order):
        assert np.array_equal(o4[qsl4[i]:qsl4[i + 1]], base[st["qsl"][r]:st["qsl"][r + 1]])


def test_merge_partials_equals_full_softmax():
    """Log-sum-exp merge of partial results over disjoint key ranges equals the
    softmax over all keys (scalar brute force for the partials)."""
    rng = np.random.default_rng(12)
    L, D = 37, 5
    s = rng.standard_normal(L) * 3
    v = rng.standard_normal((L, D))
    full = (np.exp(s - s.max())[:, None] * v).sum(0) / np.exp(s - s.max()).sum()
    for cuts in [[0, 37], [0, 10, 37], [0, 1, 2, 30, 37], list(range(0, 38, 4)) + [37]]:
        cuts = sorted(set(cuts))
        ms, ls, os_ = [], [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            m = max(s[a:b])
            ms.append(m)
            ls.append(sum(math.exp(x - m) for x in s[a:b]))
            os_.append(sum(math.exp(s[j] - m) * v[j] for j in range(a, b)))
        got = oracle.merge_partials(np.array(ms), np.array(ls), np.array(os_))
        assert np.allclose(got, full, atol=1e-13)


# ----------------------------------------------------------------------------
# attention_rows: the per-request checker of the large GPU parity cases
# ----------------------------------------------------------------------------
def _bf16_scalar(bits16):
    """One bf16 pattern -> Python float, by building the float32 word."""
    return float(np.array([int(bits16) << 16], dtype=np.uint32).view(np.float32)[0])


def _brute_rows(Q, K, V, qpos, scale, dtype, head_map):
    """Scalar loops over gathered rows: query row i at absolute position
    qpos[i] sees keys 0 .. qpos[i]; query head h reads kv head head_map(h)."""
    conv = _bf16_scalar if dtype == "bf16" else float
    n, Hq, D = Q.shape
    out = np.zeros((n, Hq, D))
    for i in range(n):
        for h in range(Hq):
            g = head_map(h)
            sc = []
            for j in range(int(qpos[i]) + 1):
                sc.append(scale * sum(conv(Q[i, h, d]) * conv(K[j, g, d]) for d in range(D)))
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            for d in range(D):
                out[i, h, d] = sum(w[j] * conv(V[j, g, d]) for j in range(len(w))) / tot
    return out


def _rows_case(rng, G, dtype, Hkv=2, D=6, L=33, n=5):
    Hq = G * Hkv
    if dtype == "f32":
        Q = rng.standard_normal((n, Hq, D)).astype(np.float32)
        K = rng.standard_normal((L, Hkv, D)).astype(np.float32)
        V = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    else:
        f = lambda shape: (rng.standard_normal(shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        Q, K, V = f((n, Hq, D)), f((L, Hkv, D)), f((L, Hkv, D))
    # rows at scattered absolute positions, the last key included; nonzero history
    qpos = np.sort(rng.choice(L, n, replace=False))
    qpos[-1] = L - 1
    return Q, K, V, qpos, 1 / math.sqrt(D)


def _rows_err(fn, G, dtype, seed):
    rng = np.random.default_rng(seed)
    Q, K, V, qpos, scale = _rows_case(rng, G, dtype)
    got, _ = fn(Q, K, V, qpos, scale, dtype)
    want = _brute_rows(Q, K, V, qpos, scale, dtype, lambda h: h // G)
    err = np.abs(np.asarray(got, np.float64) - want)
    return float(err.max()) if np.all(np.isfinite(err)) else math.inf


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_rows_brute_force(G, dtype):
    """Absolute query positions, contiguous GQA groups and the bf16 widening
    of attention_rows against scalar loops (independent bf16 conversion)."""
    assert _rows_err(oracle.attention_rows, G, dtype, 300 + G) <= 1e-12


def test_attention_rows_pin_catches_planted_slips():
    """The brute-force pin above fails for the plausible slips in
    attention_rows: a query position off by one, and the kv head taken as
    h % Hkv instead of h // G (the two maps differ once G, Hkv >= 2)."""
    from oracle import pa_oracle as po

    def shifted_qpos(Q, K, V, qpos, scale, dtype):
        return oracle.attention_rows(Q, K, V, np.asarray(qpos) - 1, scale, dtype)

    def modulo_heads(Q, K, V, qpos, scale, dtype):
        Qf, Kf, Vf = (oracle.as_f64(x, dtype) for x in (Q, K, V))
        out = np.empty(Qf.shape)
        Hkv = Kf.shape[1]
        for h in range(Qf.shape[1]):
            out[:, h], _ = po._softmax_attend(Qf[:, h], Kf[:, h % Hkv], Vf[:, h % Hkv],
                                              np.asarray(qpos), scale)
        return out, None

    for G in (2, 4):
        for dtype in ("f32", "bf16"):
            assert _rows_err(shifted_qpos, G, dtype, 300 + G) > 1e-3
            assert _rows_err(modulo_heads, G, dtype, 300 + G) > 1e-3


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_rows_equals_paged_attention(G, dtype):
    """attention_rows on a request's gathered history gives the rows that
    oracle.attention computes through the block table: decode rows, rows in
    the middle of a chunk and a chunk's last row."""
    rng = np.random.default_rng(400 + G)
    Hkv, D, B = 2, 8, 4
    Hq = G * Hkv
    st = _random_step(rng, 4, Hq, Hkv, D, B, 45, dtype=dtype)
    st["qlens"][0] = 1                    # one decode row at least
    st["comp"][0] = st["lens"][0] - 1
    st["qsl"] = np.concatenate([[0], np.cumsum(st["qlens"])]).astype(np.int32)
    T = int(st["qsl"][-1])
    if dtype == "f32":
        st["q"] = rng.standard_normal((T, Hq, D)).astype(np.float32)
    else:
        st["q"] = (rng.standard_normal((T, Hq, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    scale = 1 / math.sqrt(D)
    full, full_lse = oracle.attention(st["q"], st["kc"], st["vc"], st["bt"], st["qsl"], st["lens"],
                                      st["comp"], scale, B, dtype)
    checked = 0
    for r in range(4):
        a, q, L, c = int(st["qsl"][r]), st["qlens"][r], st["lens"][r], st["comp"][r]
        rows = np.unique([0, q // 2, q - 1])
        K = oracle.gather_kv(st["kc"], st["bt"][r], L, B)
        V = oracle.gather_kv(st["vc"], st["bt"][r], L, B)
        o, lse = oracle.attention_rows(st["q"][a + rows], K, V, c + rows, scale, dtype)
        assert np.allclose(o, full[a + rows], rtol=0, atol=1e-12)
        assert np.allclose(lse, full_lse[a + rows], rtol=0, atol=1e-12)
        checked += len(rows)
    assert checked >= 6


def test_bf16_widening_exact():
    # patterns of exactly representable values
    vals = np.array([1.0, -2.5, 0.0, 3.140625, -0.0078125, 65280.0], dtype=np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), vals.astype(np.float64))
    assert np.isnan(oracle.bf16_bits_to_f64(np.array([0x7FC0], np.uint16)))[0]


# ----------------------------------------------------------------------------
# rotary position embedding
# ----------------------------------------------------------------------------
def _angle_cache(max_pos, rotary_dim, base=10000.0):
    """cos/sin rows built from angles p * base^(-2i/rotary_dim) (the usual
    frequency ladder); cos in the first half of a row, sin in the second."""
    inv = base ** (-np.arange(0, rotary_dim, 2, dtype=np.float64) / rotary_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def _rope_complex(x, pos, cache, rotary_dim, neox):
    """Independent formulation: each rotated pair (a, b) is the complex number
    x_a + i x_b multiplied by e^{i theta} = cos + i sin, with Python complex
    arithmetic on scalars."""
    D = len(x)
    half = rotary_dim // 2
    out = [float(v) for v in x]
    for i in range(half):
        a, b = (i, i + half) if neox else (2 * i, 2 * i + 1)
        z = complex(float(x[a]), float(x[b])) * complex(float(cache[pos][i]), float(cache[pos][half + i]))
        out[a], out[b] = z.real, z.imag
    assert len(out) == D
    return out


def test_rope_quarter_turn_by_hand():
    # cos 0 / sin 1 on the first angle: the pair's first axis turns into the
    # second (counter-clockwise, the standard rotation sign)
    row = np.array([0.0, 1.0, 1.0, 0.0])            # rotary_dim 4: cos(th0, th1), sin(th0, th1)
    x = np.zeros((1, 1, 4))
    x[0, 0, 0] = 1.0
    got_gptj = oracle.rope(x, [0], row[None, :], 4, neox=False)[0, 0]
    got_neox = oracle.rope(x, [0], row[None, :], 4, neox=True)[0, 0]
    assert np.allclose(got_gptj, [0, 1, 0, 0])      # pair (0, 1)
    assert np.allclose(got_neox, [0, 0, 1, 0])      # pair (0, 2)
    # second angle is 0: its pair is untouched
    x2 = np.array([[[0.0, 3.0, 0.0, 5.0]]])
    assert np.allclose(oracle.rope(x2, [0], row[None, :], 4, neox=True)[0, 0], [0, 3, 0, 5])


@pytest.mark.parametrize("neox", [False, True])
@pytest.mark.parametrize("D,rd", [(8, 8), (16, 8), (64, 64), (128, 128)])
def test_rope_brute_force_complex(neox, D, rd):
    rng = np.random.default_rng(D + rd + neox)
    cache = _angle_cache(50, rd)
    x = rng.standard_normal((5, 2, D))
    pos = rng.integers(0, 50, 5)
    got = oracle.rope(x, pos, cache, rd, neox)
    for t in range(5):
        for h in range(2):
            want = _rope_complex(x[t, h], int(pos[t]), cache, rd, neox)
            assert np.max(np.abs(got[t, h] - np.array(want))) < 1e-12
    # dimensions at or past rotary_dim pass through unchanged
    assert np.array_equal(got[:, :, rd:], x[:, :, rd:])


@pytest.mark.parametrize("neox", [False, True])
def test_rope_rotation_invariants(neox):
    rng = np.random.default_rng(7)
    D = 64
    cache = _angle_cache(4096, D, base=500000.0)
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    # position 0 is the identity
    assert np.allclose(oracle.rope(q, [0], cache, D, neox), q, atol=0, rtol=0)
    # orthogonal: norms are kept
    for p in (1, 17, 4095):
        R = oracle.rope_matrix(cache[p], D, D, neox)
        assert np.allclose(R @ R.T, np.eye(D), atol=1e-13)
        assert abs(np.linalg.norm(oracle.rope(q, [p], cache, D, neox)) - np.linalg.norm(q)) < 1e-12
    # the score of rotated q (pos m) and k (pos n) depends only on m - n
    def score(m, n):
        return float(np.sum(oracle.rope(q, [m], cache, D, neox) * oracle.rope(k, [n], cache, D, neox)))
    for m, n, s in ((100, 40, 7), (5, 5, 300), (900, 12, 1000)):
        assert abs(score(m, n) - score(m + s, n + s)) < 1e-9
    # rotations compose: R(m) R(n) = R(m + n) for a cache built from angles
    Rm, Rn, Rmn = (oracle.rope_matrix(cache[p], D, D, neox) for p in (123, 456, 579))
    assert np.allclose(Rm @ Rn, Rmn, atol=1e-12)


def test_rope_styles_related_by_permutation():
    # the split-halves layout is the adjacent-pairs layout on permuted coordinates
    rng = np.random.default_rng(3)
    D = rd = 16
    cache = _angle_cache(10, rd)
    x = rng.standard_normal((3, 1, D))
    perm = np.empty(D, dtype=int)             # adjacent slot 2i <- i, 2i+1 <- i + rd/2
    perm[0::2] = np.arange(rd // 2)
    perm[1::2] = np.arange(rd // 2) + rd // 2
    pos = [0, 3, 9]
    neox = oracle.rope(x, pos, cache, rd, neox=True)
    gptj = oracle.rope(x[:, :, perm], pos, cache, rd, neox=False)
    assert np.allclose(neox[:, :, perm], gptj, atol=1e-14)


def test_rope_write_kv_order_and_skip():
    # rotated K lands at its slot, V unrotated, negative slots write nothing,
    # untouched slots keep their poison
    rng = np.random.default_rng(11)
    B, nb, H, D = 4, 3, 2, 8
    cache = _angle_cache(20, D)
    q = rng.standard_normal((3, 4, D))
    k = rng.standard_normal((3, H, D))
    v = rng.standard_normal((3, H, D))
    kc = np.full((nb, B, H, D), np.nan)
    vc = np.full((nb, B, H, D), np.nan)
    slots = np.array([5, -1, 8])
    pos = np.array([2, 3, 19])
    q_rot = oracle.rope_write_kv(q, k, v, kc, vc, slots, pos, cache, D, True, B)
    assert np.allclose(q_rot, oracle.rope(q, pos, cache, D, True))
    assert np.allclose(kc[1, 1], oracle.rope(k[0:1], pos[0:1], cache, D, True)[0])
    assert np.array_equal(vc[2, 0], v[2])
    assert np.isnan(kc[0]).all() and np.isnan(kc[1, [0, 2, 3]]).all() and np.isnan(vc[2, 1:]).all()
