"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Cache writes and slot mappings must match bit for bit; attention outputs
within atol = rtol = 1e-5 (fp32) or 1e-2 (bf16), elementwise.  Inputs are the
seeded synthetic steps of workloads.configs.  C1 is compared whole; C2, C3
and C4 row by row over every request (the oracle computes one request at a
time from the generator's pre-write pool blocks), with every written slot
bit-exact and every other slot of the pools unchanged.
"""
import math
import os

import numpy as np
import pytest

import oracle
from helpers import (assert_close, bits, check_full_step, check_requests, oracle_request, run_step,
                     sample_requests, say, storage_np)
from workloads import configs, rng

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_attention_reshape_amd as pa  # noqa: E402
from workloads import _lib as wl  # noqa: E402


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu-test] {request.node.name}")
    yield
    torch.cuda.synchronize()


def test_library_is_the_hip_build():
    assert os.path.exists(pa.LIB_PATH)
    assert pa.abi_version() == 1


def test_generator_device_matches_host_mirror():
    for dtype, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        t = torch.empty((37, 3, 64), dtype=tdt, device="cuda")
        keys = rng.base_row_keys(rng.key(5, 9), np.arange(37))
        wl.fill_rows(t, dtype, row_keys=torch.from_numpy(keys.view(np.int64)).cuda())
        want = rng.row_values(keys, 3 * 64, dtype).reshape(37, 3, 64)
        assert np.array_equal(bits(storage_np(t)), bits(want))
        pool = torch.empty((5, 16, 2, 64), dtype=tdt, device="cuda")
        valid = np.array([0, 16, 3, 9, 1], np.int32)
        wl.fill_pool(pool, dtype, 1234, torch.from_numpy(valid).cuda(), 16)
        rows = np.arange(5 * 16)
        hv = rng.row_values(rng.base_row_keys(1234, rows), 128, dtype).reshape(5, 16, 2, 64)
        bad = np.arange(16)[None, :] >= valid[:, None]
        hv[bad] = rng.storage_nan(dtype)
        assert np.array_equal(bits(storage_np(pool)), bits(hv))


def test_c1_tiny_mixed_fp32_full():
    spec = configs.c1()
    d, out, sm = run_step(spec, pa)
    torch.cuda.synchronize()
    # slot mapping: library (host C++) vs oracle, bit-exact
    want_sm = oracle.slot_mapping(spec.block_table, spec.query_lens, spec.num_computed, spec.B)
    assert np.array_equal(sm, want_sm)
    # whole pool after the write, bit-exact
    kp = spec.host_pool_blocks("k", np.arange(spec.num_blocks))
    vp = spec.host_pool_blocks("v", np.arange(spec.num_blocks))
    rows = np.arange(spec.T)
    oracle.write_kv(kp, vp, spec.host_rows("k", rows), spec.host_rows("v", rows), want_sm, spec.B)
    assert np.array_equal(bits(storage_np(d["key_cache"])), bits(kp))
    assert np.array_equal(bits(storage_np(d["value_cache"])), bits(vp))
    # every output row
    want, _ = oracle.attention(spec.host_rows("q", rows), kp, vp, spec.block_table,
                               spec.query_start_loc, spec.seq_lens, spec.num_computed,
                               spec.scale, spec.B, "f32")
    got = storage_np(out).astype(np.float64)
    err = assert_close(got, want, "f32", "c1")
    say(f"c1 max abs err {err:.2e}")


def _full(spec):
    """Run the step with the generator's pre-write pools kept aside, then check
    every row, every written slot and every untouched slot."""
    d = spec.device_inputs()
    pre_k, pre_v = d["key_cache"].clone(), d["value_cache"].clone()
    d, out, _ = run_step(spec, pa, dev_inputs=d)
    torch.cuda.synchronize()
    err, n_rows, n_slots = check_full_step(spec, pre_k, pre_v, out, d["key_cache"], d["value_cache"],
                                           what=spec.name)
    say(f"{spec.name}: all {n_rows} rows of {spec.R} requests within tolerance (max abs err {err:.2e}); "
        f"{n_slots} written slots bit-exact, every other slot unchanged")
    assert n_rows == spec.T


def test_c2_decode_bf16_full():
    _full(configs.c2())


def test_c3_mixed_chunked_bf16_full():
    _full(configs.c3())


def test_c4_long_decode_bf16_full():
    _full(configs.c4())


def test_determinism_bitwise():
    spec = configs.c2(R=16)
    d, out1, _ = run_step(spec, pa)
    _, out2, _ = run_step(spec, pa, dev_inputs=d)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def _small(dtype, Hq, Hkv, D, B, qlens, comp, seed=7, pool_factor=1.5):
    return configs.custom(f"s{seed}", dtype, Hq, Hkv, D, B, qlens, comp, seed, pool_factor)


def test_block_permutation_and_request_order_invariance():
    spec = _small("bf16", 16, 4, 128, 16, [1, 1, 37, 1, 5], [700, 33, 200, 0, 1000], seed=11)
    d, base, _ = run_step(spec, pa)
    torch.cuda.synchronize()
    # 1) relabel physical blocks (moving the data): outputs bitwise equal
    g = np.random.default_rng(3)
    perm = g.permutation(spec.num_blocks)
    kc = torch.empty_like(d["key_cache"])
    vc = torch.empty_like(d["value_cache"])
    pt = torch.from_numpy(perm).cuda()
    # pool before the write: regenerate, move, then run the step again
    fresh = spec.device_inputs()
    kc[pt] = fresh["key_cache"]
    vc[pt] = fresh["value_cache"]
    bt2 = np.where(spec.block_table >= 0, perm[np.maximum(spec.block_table, 0)], -1).astype(np.int32)
    spec2 = configs.StepSpec(**{**spec.__dict__, "block_table": bt2})
    fresh["key_cache"], fresh["value_cache"] = kc, vc
    fresh["block_table"] = torch.from_numpy(bt2).cuda()
    _, out2, _ = run_step(spec2, pa, dev_inputs=fresh)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), base.view(torch.int16))
    # 2) reverse request order: each request's rows bitwise unchanged
    order = list(range(spec.R))[::-1]
    qsl = spec.query_start_loc
    rows = np.concatenate([np.arange(qsl[r], qsl[r + 1]) for r in order])
    spec3 = configs.StepSpec(**{**spec.__dict__, "query_lens": spec.query_lens[order],
                                "num_computed": spec.num_computed[order],
                                "block_table": spec.block_table[order],
                                "q_row_keys": spec.row_keys("q", rows),
                                "k_row_keys": spec.row_keys("k", rows),
                                "v_row_keys": spec.row_keys("v", rows)})
    _, out3, _ = run_step(spec3, pa)
    torch.cuda.synchronize()
    q3 = spec3.query_start_loc
    for i, r in enumerate(order):
        assert torch.equal(out3[q3[i]:q3[i + 1]].view(torch.int16),
                           base[qsl[r]:qsl[r + 1]].view(torch.int16))


EDGE = [
    # dtype, Hq, Hkv, D, B, query lens, computed
    ("bf16", 8, 8, 128, 16, [1, 1, 1], [0, 15, 16]),          # G=1, L=1, 16, 17
    ("bf16", 16, 8, 64, 32, [1, 3, 1], [31, 40, 63]),         # G=2, D=64, B=32
    ("bf16", 64, 8, 128, 32, [1, 2, 1], [5000, 77, 1]),        # G=8
    ("f32", 32, 8, 128, 16, [1, 9, 1], [300, 50, 2]),          # fp32, D=128
    ("f32", 8, 1, 64, 48, [1, 20], [100, 13]),                 # G=8 fp32, B=48
    ("bf16", 32, 8, 128, 16, [0, 1, 0, 4], [10, 99, 0, 2]),    # requests with no rows
    ("bf16", 32, 8, 128, 64, [1, 1], [4095, 2047]),            # B=64
]


@pytest.mark.parametrize("idx", range(len(EDGE)), ids=[f"edge{i}" for i in range(len(EDGE))])
def test_edge_shapes(idx):
    case = EDGE[idx]
    dtype, Hq, Hkv, D, B, ql, cp = case
    spec = _small(dtype, Hq, Hkv, D, B, ql, cp, seed=100 + idx)
    d, out, _ = run_step(spec, pa)
    torch.cuda.synchronize()
    err = check_requests(spec, out, d["key_cache"], d["value_cache"], range(spec.R), what=str(case))
    say(f"{case} err {err:.2e}")


@pytest.mark.parametrize("split", [64, 128, 1024])
def test_forced_partition_sizes(split):
    spec = _small("bf16", 32, 8, 128, 16, [1, 1, 1, 7], [3000, 64, 63, 700], seed=split)
    with pa.tuning(split_keys=split):
        d, out, _ = run_step(spec, pa)
    torch.cuda.synchronize()
    err = check_requests(spec, out, d["key_cache"], d["value_cache"], range(spec.R), what=f"split{split}")
    say(f"split {split} err {err:.2e}")


@pytest.mark.parametrize("case", [
    # (query lens, computed counts, Hq, Hkv, D, B): long chunks that span many
    # key segments and q-tiles, beside short decodes
    ([16384, 1, 4096], [0, 9000, 12288], 32, 8, 128, 16),
    ([8192, 2048, 1], [8192, 0, 30000], 64, 8, 128, 32),
], ids=["16k-prompt+4k-after-12k", "g8-8k-after-8k"])
def test_long_chunks_sampled(case):
    """Chunks of thousands of tokens (many segments merged by log-sum-exp,
    long q-tile lists, large workspaces): 40 sampled rows of every request,
    including the first and last, against the oracle; caches bit-exact."""
    ql, comp, Hq, Hkv, D, B = case
    spec = _small("bf16", Hq, Hkv, D, B, ql, comp, seed=23 + len(ql), pool_factor=1.1)
    d, out, _ = run_step(spec, pa)
    torch.cuda.synchronize()
    err = check_requests(spec, out, d["key_cache"], d["value_cache"], range(spec.R), rows_per_req=40,
                         what=f"long {ql}")
    say(f"long chunks {ql} after {comp}: err {err:.2e}")


def test_fp32_prefill_rows_on_the_split_k_path():
    """fp32 chunk rows run on the split-K kernel (one row per wavefront and
    key partition, merged by log-sum-exp): a 700-token prompt, a 300-token
    chunk after 1500 tokens and decodes, every row against the oracle at the
    fp32 tolerance."""
    spec = _small("f32", 32, 8, 128, 16, [700, 1, 300, 1], [0, 2000, 1500, 33], seed=41)
    d, out, _ = run_step(spec, pa)
    torch.cuda.synchronize()
    err = check_requests(spec, out, d["key_cache"], d["value_cache"], range(spec.R), what="fp32 prefill")
    say(f"fp32 prefill rows err {err:.2e}")


def test_chunked_prefill_equals_full_prefill_on_gpu():
    """A 300-token prompt run as five chunks of 64 (each chunk a step that
    reads the cache the earlier chunks wrote) matches the one-shot prefill."""
    P, CH, Hq, Hkv, D, B = 300, 64, 32, 8, 128, 16
    seed = 21
    full = _small("bf16", Hq, Hkv, D, B, [P], [0], seed=seed)
    bt = full.block_table
    pos_keys = {w: rng.base_row_keys(rng.key(seed, tag, 0), np.arange(P))
                for w, tag in (("q", rng.TAG_Q), ("k", rng.TAG_K), ("v", rng.TAG_V))}
    full = configs.StepSpec(**{**full.__dict__, "q_row_keys": pos_keys["q"],
                               "k_row_keys": pos_keys["k"], "v_row_keys": pos_keys["v"]})
    d, out_full, _ = run_step(full, pa)
    pools = full.device_inputs()   # fresh NaN pool for the chunked run
    outs = []
    for a in range(0, P, CH):
        b = min(a + CH, P)
        st = configs.StepSpec(**{**full.__dict__, "query_lens": np.array([b - a], np.int32),
                                 "num_computed": np.array([a], np.int32),
                                 "q_row_keys": pos_keys["q"][a:b], "k_row_keys": pos_keys["k"][a:b],
                                 "v_row_keys": pos_keys["v"][a:b]})
        di = st.device_inputs(pools=False)
        di["key_cache"], di["value_cache"] = pools["key_cache"], pools["value_cache"]
        _, o, _ = run_step(st, pa, dev_inputs=di)
        outs.append(o)
    torch.cuda.synchronize()
    chunked = torch.cat(outs)
    g_full = oracle.as_f64(storage_np(out_full), "bf16")
    g_ch = oracle.as_f64(storage_np(chunked), "bf16")
    want, _, _, _, _, _ = oracle_request(full, 0)
    assert_close(g_full, want, "bf16", "full prefill")
    assert_close(g_ch, want, "bf16", "chunked prefill")
    assert np.max(np.abs(g_full - g_ch)) < 2e-2


def test_empty_and_noop_steps():
    kc = torch.zeros((4, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    e = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    pa.write_kv(e, e, kc, kc.clone(), torch.empty(0, dtype=torch.int64, device="cuda"))
    out = torch.empty((0, 8, 64), dtype=torch.bfloat16, device="cuda")
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa.attention(out, out, kc, kc, torch.zeros((1, 1), dtype=torch.int32, device="cuda"), z,
                 z[:0], z[:0], np.zeros(1, np.int32), np.zeros(0, np.int32), 0.125,
                 pa.alloc_workspace(256))


def test_write_kv_skips_negative_slots():
    spec = _small("bf16", 8, 2, 64, 16, [3, 2], [5, 0], seed=5)
    d = spec.device_inputs()
    before_k = storage_np(d["key_cache"]).copy()
    sm = torch.tensor([-1, 6 + int(spec.block_table[0, 0]) * 16, -1, -5, 1 + int(spec.block_table[1, 0]) * 16],
                      dtype=torch.int64, device="cuda")
    pa.write_kv(d["key"], d["value"], d["key_cache"], d["value_cache"], sm)
    torch.cuda.synchronize()
    after_k = storage_np(d["key_cache"])
    changed = np.argwhere(np.any(bits(after_k) != bits(before_k), axis=(2, 3)))
    b0, b1 = int(spec.block_table[0, 0]), int(spec.block_table[1, 0])
    assert sorted(map(tuple, changed.tolist())) == sorted([(b0, 6), (b1, 1)])
    kn = storage_np(d["key"])
    assert np.array_equal(bits(after_k[b0, 6]), bits(kn[1]))
    assert np.array_equal(bits(after_k[b1, 1]), bits(kn[4]))


CHUNK_CASES = [
    # Hq, Hkv, D, B, query lens, computed, forced key segment (0 = planner's choice)
    (32, 8, 128, 16, [100, 1, 300], [0, 500, 1000], 0),
    (32, 8, 128, 16, [100, 1, 300], [0, 500, 1000], 512),
    (8, 8, 64, 32, [77, 128], [33, 1000], 512),          # G=1, D=64
    (16, 8, 128, 48, [65, 3], [700, 2], 512),            # G=2, B=48
    (64, 8, 128, 32, [17, 40], [4000, 0], 1024),         # G=8
    (32, 8, 128, 64, [512], [2500], 512),                # B=64
    (32, 8, 64, 16, [2, 33, 64], [0, 31, 4095], 0),      # tiny chunks, D=64
]


@pytest.mark.parametrize("idx", range(len(CHUNK_CASES)), ids=[f"chunk{i}" for i in range(len(CHUNK_CASES))])
def test_chunk_kernel_shapes(idx):
    Hq, Hkv, D, B, ql, cp, seg = CHUNK_CASES[idx]
    spec = _small("bf16", Hq, Hkv, D, B, ql, cp, seed=300 + idx)
    with pa.tuning(chunk_segment=seg):
        d, out, _ = run_step(spec, pa)
    torch.cuda.synchronize()
    err = check_requests(spec, out, d["key_cache"], d["value_cache"], range(spec.R), what=f"chunk{idx}")
    say(f"chunk case {idx} err {err:.2e}")


def test_chunk_kernel_agrees_with_rowwise_path():
    spec = _small("bf16", 32, 8, 128, 16, [200, 1, 64], [300, 40, 0], seed=77)
    d, out_ck, _ = run_step(spec, pa)
    fresh = spec.device_inputs()
    with pa.tuning(chunk_path=1):
        _, out_rw, _ = run_step(spec, pa, dev_inputs=fresh)
    torch.cuda.synchronize()
    a = oracle.as_f64(storage_np(out_ck), "bf16")
    b = oracle.as_f64(storage_np(out_rw), "bf16")
    assert np.max(np.abs(a - b)) < 2e-2


def test_device_slot_mapping_matches_oracle():
    for spec in (configs.c1(), configs.c3()):
        d = spec.device_inputs(pools=False)
        sm = torch.full((spec.T,), -7, dtype=torch.int64, device="cuda")
        pa.compute_slot_mapping(sm, d["block_table"], d["query_start_loc"], d["num_computed"],
                                spec.num_blocks, spec.B)
        torch.cuda.synchronize()
        want = oracle.slot_mapping(spec.block_table, spec.query_lens, spec.num_computed, spec.B)
        assert np.array_equal(sm.cpu().numpy(), want)
    # an out-of-range block id gives slot -1 (nothing is written for that token)
    spec = _small("bf16", 8, 2, 64, 16, [2, 1], [15, 3], seed=9)   # request 0 spans 2 blocks
    bt = spec.block_table.copy()
    bt[0, 1] = spec.num_blocks + 5
    d = spec.device_inputs(pools=False)
    sm = torch.empty((spec.T,), dtype=torch.int64, device="cuda")
    pa.compute_slot_mapping(sm, torch.from_numpy(bt).cuda(), d["query_start_loc"], d["num_computed"],
                            spec.num_blocks, spec.B)
    torch.cuda.synchronize()
    got = sm.cpu().numpy()
    assert got[1] == -1 and got[0] == bt[0, 0] * 16 + 15 and got[2] == bt[1, 0] * 16 + 3


def test_profiling_events_bracket_the_kernels():
    spec = configs.c2(R=32)
    d = spec.device_inputs()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    pa.set_profiling_events(ev)
    try:
        run_step(spec, pa, dev_inputs=d)
    finally:
        pa.set_profiling_events(None)
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(4)]
    assert all(m >= 0 for m in ms) and ms[1] > 0
