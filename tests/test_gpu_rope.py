"""GPU parity of the fused rotary embedding + cache write (pa_rope_write_kv)
against the fp64 oracle.

The rotated query and the rotated K written to the cache are compared with
oracle.rope in fp64 from the exact stored inputs, to a tolerance derived from
the arithmetic: the kernel computes x' = fma(x, c, -(y s)) in fp32 (two
roundings, each at most 2^-24 relative to terms below 4 in magnitude for this
generator, so below 2^-21 absolute) and rounds once to the storage type
(2^-24 relative for fp32, 2^-8 for bf16).  Hence
    |got - want| <= ATOL + RTOL |want|,  ATOL = 2^-20,
    RTOL = 2^-23 (fp32) or 2^-8 + 2^-20 (bf16).
V rows, the pass-through dimensions of K and every cache slot the step does
not own must match bit for bit (a negative slot writes nothing).  An end to
end check runs attention on the rotated step and compares with the oracle's
rotate -> write -> attention.
"""
import numpy as np
import pytest

import oracle
from helpers import assert_close, bits, say, storage_np
from workloads import configs, rng

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_attention_reshape_amd as pa  # noqa: E402

RTOL = {"f32": 2.0 ** -23, "bf16": 2.0 ** -8 + 2.0 ** -20}
ATOL = 2.0 ** -20


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu-test] {request.node.name}")
    yield
    torch.cuda.synchronize()


def _close(got, want, dtype, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU values"
    err = np.abs(got - want)
    bad = err > ATOL + RTOL[dtype] * np.abs(want)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance, max err {err.max():.3e}"
    return float(err.max())


def _run(spec, rotary_dim, neox, slots=None, positions=None, max_position=None):
    """Device inputs of the step, the rope+write call, and host copies of the
    pools before the call.  Returns (dev dict, slots, positions, cache)."""
    d = spec.device_inputs()
    if slots is None:
        _, _, slots = pa.build_step_metadata(spec.query_lens, spec.num_computed, spec.block_table,
                                             spec.B, spec.num_blocks)
    if positions is None:
        positions = spec.positions()
    if max_position is None:
        max_position = int(max(spec.seq_lens.max(), 1))
    cache = configs.rope_cache(max_position, rotary_dim)
    d["slot_mapping"] = torch.from_numpy(np.asarray(slots, np.int64)).cuda()
    d["positions"] = torch.from_numpy(np.asarray(positions, np.int64)).cuda()
    d["cos_sin"] = torch.from_numpy(cache).cuda()
    # blocks whose bits are compared before/after: all of a small pool, else
    # every block the step writes plus 2048 others chosen at random
    slots_np = np.asarray(slots, np.int64)
    if spec.num_blocks <= 4096:
        watch = np.arange(spec.num_blocks)
    else:
        touched = np.unique(slots_np[slots_np >= 0] // spec.B)
        others = np.random.default_rng(5).choice(spec.num_blocks, 2048, replace=False)
        watch = np.union1d(touched, others)
    d["watch"] = watch
    idx = torch.from_numpy(watch).cuda()
    d["kc0"] = storage_np(d["key_cache"].index_select(0, idx))
    d["vc0"] = storage_np(d["value_cache"].index_select(0, idx))
    pa.rope_write_kv(d["query"], d["key"], d["value"], d["key_cache"], d["value_cache"],
                     d["slot_mapping"], d["positions"], d["cos_sin"], rotary_dim, neox)
    torch.cuda.synchronize()
    return d, np.asarray(slots, np.int64), np.asarray(positions, np.int64), cache


def _check(spec, d, slots, positions, cache, rotary_dim, neox, what):
    """Rotated Q everywhere, rotated K / copied V at every written slot,
    untouched slots unchanged."""
    dt = spec.dtype
    rows = np.arange(spec.T)
    pos = np.clip(positions, 0, cache.shape[0] - 1)
    q_in = oracle.as_f64(spec.host_rows("q", rows), dt)
    k_in = oracle.as_f64(spec.host_rows("k", rows), dt)
    v_st = spec.host_rows("v", rows)
    q_want = oracle.rope(q_in, pos, cache, rotary_dim, neox)
    k_want = oracle.rope(k_in, pos, cache, rotary_dim, neox)
    q_got = oracle.as_f64(storage_np(d["query"]), dt)
    eq = _close(q_got, q_want, dt, f"{what} query")
    assert np.array_equal(q_got[:, :, rotary_dim:], q_in[:, :, rotary_dim:]), f"{what}: query pass-through changed"
    B = spec.B
    watch = d["watch"]
    idx = torch.from_numpy(watch).cuda()
    kc = storage_np(d["key_cache"].index_select(0, idx))      # rows of `watch`
    vc = storage_np(d["value_cache"].index_select(0, idx))
    live = slots >= 0
    blk, off = np.searchsorted(watch, slots[live] // B), slots[live] % B
    assert np.array_equal(watch[blk], slots[live] // B)
    kg = oracle.as_f64(kc[blk, off], dt)
    ek = _close(kg, k_want[live], dt, f"{what} key cache")
    assert np.array_equal(kg[:, :, rotary_dim:], k_in[live][:, :, rotary_dim:]), f"{what}: K pass-through not exact"
    assert np.array_equal(bits(vc[blk, off]), bits(v_st[live])), f"{what}: value cache not bit-exact"
    # every slot the step does not write keeps its previous bits
    mask = np.ones(kc.shape[:2], bool)
    mask[blk, off] = False
    assert np.array_equal(bits(kc[mask]), bits(d["kc0"][mask])), f"{what}: foreign key slots changed"
    assert np.array_equal(bits(vc[mask]), bits(d["vc0"][mask])), f"{what}: foreign value slots changed"
    say(f"{what}: query err {eq:.2e}, key err {ek:.2e}")


def test_rope_write_c1_fp32_both_styles():
    spec = configs.c1()
    for neox in (True, False):
        d, s, p, c = _run(spec, 64, neox)
        _check(spec, d, s, p, c, 64, neox, f"c1 neox={neox}")


def test_rope_write_c3_bf16():
    spec = configs.c3()
    d, s, p, c = _run(spec, 128, True)
    _check(spec, d, s, p, c, 128, True, "c3")


@pytest.mark.parametrize("D,rd,neox", [(128, 64, True), (128, 64, False), (64, 64, False),
                                       (64, 32, True), (128, 16, False)])
def test_rope_write_partial_rotary_and_head_dims(D, rd, neox):
    spec = configs.custom("rope", "bf16", 16, 4, D, 32, [1, 1, 37, 80], [300, 12, 90, 0], 21)
    d, s, p, c = _run(spec, rd, neox)
    _check(spec, d, s, p, c, rd, neox, f"D={D} rd={rd} neox={neox}")


def test_rope_write_negative_slots_and_clamped_positions():
    spec = configs.custom("rope", "bf16", 8, 2, 128, 16, [3, 1, 20], [40, 7, 5], 22)
    _, _, slots = pa.build_step_metadata(spec.query_lens, spec.num_computed, spec.block_table,
                                         spec.B, spec.num_blocks)
    slots = slots.copy()
    slots[[0, 5, 17]] = -1                              # padding tokens: no write
    pos = spec.positions().copy()
    pos[2] = 10 ** 6                                    # past the table: clamped to its last row
    pos[9] = -5                                         # before it: clamped to row 0
    d, s, p, c = _run(spec, 128, True, slots=slots, positions=pos, max_position=64)
    _check(spec, d, s, p, c, 128, True, "negative slots")


def test_rope_then_attention_end_to_end():
    """rope_write_kv + attention on a mixed step against the oracle's
    rotate -> write -> attention (every row of every request)."""
    spec = configs.custom("rope-attn", "bf16", 32, 8, 128, 16, [1, 1, 64, 130, 1],
                          [700, 33, 200, 0, 2000], 23)
    rd, neox = 128, True
    d, slots, pos, cache = _run(spec, rd, neox)
    qsl, sl, _ = pa.build_step_metadata(spec.query_lens, spec.num_computed, spec.block_table,
                                        spec.B, spec.num_blocks)
    out = torch.empty_like(d["query"])
    ws = pa.alloc_workspace(pa.attention_workspace_size(qsl, sl, spec.Hq, spec.Hkv, spec.D, spec.B, pa.PA_BF16))
    pa.attention(out, d["query"], d["key_cache"], d["value_cache"], d["block_table"],
                 d["query_start_loc"], d["seq_lens"], d["num_computed"], qsl, sl, spec.scale, ws)
    torch.cuda.synchronize()
    # oracle: rotate the step's rows, store them as bf16 (the cache and the
    # query are bf16 tensors), write into the host pool, attend
    rows = np.arange(spec.T)

    def stored(x):
        return oracle.bf16_bits_to_f64(rng.f32_to_bf16_bits(x.astype(np.float32)))

    q_rot = stored(oracle.rope(oracle.as_f64(spec.host_rows("q", rows), "bf16"), pos, cache, rd, neox))
    k_rot = stored(oracle.rope(oracle.as_f64(spec.host_rows("k", rows), "bf16"), pos, cache, rd, neox))
    kp = oracle.as_f64(spec.host_pool_blocks("k", np.arange(spec.num_blocks)), "bf16")
    vp = oracle.as_f64(spec.host_pool_blocks("v", np.arange(spec.num_blocks)), "bf16")
    oracle.write_kv(kp, vp, k_rot, oracle.as_f64(spec.host_rows("v", rows), "bf16"), slots, spec.B)
    want, _ = oracle.attention(q_rot, kp, vp, spec.block_table, spec.query_start_loc, spec.seq_lens,
                               spec.num_computed, spec.scale, spec.B, "f32")
    got = oracle.as_f64(storage_np(out), "bf16")
    err = assert_close(got, want, "bf16", "rope + attention")
    say(f"rope + attention max err {err:.2e}")
