"""CPU-side checks of the C ABI: the library loads, exports every entry point
the header declares, and its host-only entry points (metadata builder,
validation, workspace sizing, argument checks) behave as documented.  No
kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from workloads import configs, rng

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pa = pytest.importorskip("paged_kv_attention_reshape_amd")


def _header_symbols():
    txt = open(os.path.join(ROOT, "include", "pa.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_header_symbol():
    L = pa.lib()
    syms = _header_symbols()
    assert set(syms) == set(pa.EXPORTS)
    for s in syms:
        assert hasattr(L, s), s
    assert pa.abi_version() == 1
    for code, name in pa._lib.STATUS.items():
        assert pa.status_str(code) == name
    assert pa.status_str(99) == "PA_UNKNOWN"


def test_workload_library_exports():
    from workloads import _lib as wl
    assert hasattr(wl.lib(), "wl_fill_rows")


def test_slot137_through_the_library():
    qsl, sl, sm = pa.build_step_metadata([1], [25], np.array([[5, 8, 12]]), 16, 64)
    assert sm.tolist() == [137] and qsl.tolist() == [0, 1] and sl.tolist() == [26]


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_metadata_builder_matches_oracle(name):
    spec = configs.BUILDERS[name]()
    qsl, sl, sm = pa.build_step_metadata(spec.query_lens, spec.num_computed, spec.block_table,
                                         spec.B, spec.num_blocks)
    assert np.array_equal(qsl, spec.query_start_loc)
    assert np.array_equal(sl, spec.seq_lens)
    want = oracle.slot_mapping(spec.block_table, spec.query_lens, spec.num_computed, spec.B)
    assert sm.dtype == np.int64 and np.array_equal(sm, want)
    pa.validate_metadata(qsl, sl, spec.num_computed, spec.block_table, sm, spec.num_blocks, spec.B)


def test_metadata_builder_random_brute_force():
    g = np.random.default_rng(0)
    for trial in range(30):
        R = int(g.integers(0, 7))
        B = int(g.choice([1, 4, 16, 32]))
        ql = g.integers(0, 40, size=R)
        nc = g.integers(0, 100, size=R)
        need = [-(-(int(a) + int(b)) // B) for a, b in zip(ql, nc)]
        M = max(need + [1])
        nb = sum(need) + 3
        perm = g.permutation(nb)
        bt = np.full((R, M), -1, np.int32)
        pos = 0
        for r in range(R):
            bt[r, :need[r]] = perm[pos:pos + need[r]]
            pos += need[r]
        qsl, sl, sm = pa.build_step_metadata(ql, nc, bt, B, nb)
        assert np.array_equal(sm, oracle.slot_mapping(bt, ql, nc, B))


def _valid_step():
    spec = configs.c1()
    qsl, sl, sm = pa.build_step_metadata(spec.query_lens, spec.num_computed, spec.block_table,
                                         spec.B, spec.num_blocks)
    return spec, qsl, sl, sm


def test_validate_metadata_error_paths():
    spec, qsl, sl, sm = _valid_step()
    nc, bt, nb, B = spec.num_computed, spec.block_table, spec.num_blocks, spec.B
    pa.validate_metadata(qsl, sl, nc, bt, sm, nb, B)

    def code(**kw):
        a = dict(query_start_loc=qsl, seq_lens=sl, num_computed=nc, block_table=bt,
                 slot_mapping=sm, num_blocks=nb, block_size=B)
        a.update(kw)
        with pytest.raises(pa.PAError) as e:
            pa.validate_metadata(**a)
        return e.value.status_name

    q2 = qsl.copy(); q2[0] = 1
    assert code(query_start_loc=q2) == "PA_ERR_INCONSISTENT_METADATA"
    s2 = sl.copy(); s2[1] += 1
    assert code(seq_lens=s2) == "PA_ERR_INCONSISTENT_METADATA"
    b2 = bt.copy(); b2[3, 0] = nb
    assert code(block_table=b2) == "PA_ERR_OUT_OF_RANGE"
    b3 = bt.copy(); b3[0, 2] = -1
    assert code(block_table=b3) == "PA_ERR_OUT_OF_RANGE"
    m2 = sm.copy(); m2[5] = nb * B
    assert code(slot_mapping=m2) == "PA_ERR_OUT_OF_RANGE"
    m3 = sm.copy(); m3[5] = m3[5] + 1 if (m3[5] + 1) % B else m3[5] - 1
    assert code(slot_mapping=m3) == "PA_ERR_INCONSISTENT_METADATA"
    # a duplicate that is also consistent: two requests sharing a block
    b4 = bt.copy(); b4[1, 5] = b4[0, 2]   # req1 pos 80 and req0 pos 36 -> both offset 0? make them collide
    spec2 = configs.custom("dup", "f32", 8, 2, 64, 16, [1, 1], [4, 4], 1, num_blocks=8)
    bt5 = spec2.block_table.copy(); bt5[1, 0] = bt5[0, 0]
    q5, s5, m5 = pa.build_step_metadata([1, 1], [4, 4], bt5, 16, 8)
    with pytest.raises(pa.PAError) as e:
        pa.validate_metadata(q5, s5, [4, 4], bt5, m5, 8, 16)
    assert e.value.status_name == "PA_ERR_DUPLICATE_SLOT"
    # negative slots are allowed (padding)
    m6 = sm.copy(); m6[3] = -1
    pa.validate_metadata(qsl, sl, nc, bt, m6, nb, B)


def test_build_metadata_errors():
    with pytest.raises(pa.PAError) as e:
        pa.build_step_metadata([3], [30], np.array([[1, 2]]), 16, 4)   # needs 3 blocks
    assert e.value.status_name == "PA_ERR_OUT_OF_RANGE"
    with pytest.raises(pa.PAError) as e:
        pa.build_step_metadata([1], [0], np.array([[9]]), 16, 4)
    assert e.value.status_name == "PA_ERR_OUT_OF_RANGE"
    with pytest.raises(pa.PAError):
        pa.build_step_metadata([-1], [0], np.array([[0]]), 16, 4)


def test_workspace_size_and_host_checks():
    spec = configs.c3()
    n = pa.attention_workspace_size(spec.query_start_loc, spec.seq_lens, 32, 8, 128, 16, pa.PA_BF16)
    assert n > 0 and n % 256 == 0
    # deterministic
    assert n == pa.attention_workspace_size(spec.query_start_loc, spec.seq_lens, 32, 8, 128, 16, pa.PA_BF16)
    # unsupported geometry / dtype are refused on the host
    L = pa.lib()
    qsl = spec.query_start_loc
    sl = spec.seq_lens
    assert L.pa_attention_workspace_size(qsl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                         sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                         spec.R, 32, 8, 96, 16, 1) == 0
    assert "head_dim" in pa.last_error()
    bad = sl.copy(); bad[0] = 0
    with pytest.raises(pa.PAError):
        pa.attention_workspace_size(qsl, bad, 32, 8, 128, 16, pa.PA_BF16)


def _call_attention(**over):
    """pa_attention with dummy (never dereferenced) pointers: every case below
    must be refused by the host checks before anything is launched."""
    L = pa.lib()
    qsl = np.array([0, 1], np.int32)
    sl = np.array([5], np.int32)
    a = dict(out=4096, query=4096, kc=4096, vc=4096, bt=4096, M=1, dqsl=4096, dsl=4096, dnc=4096,
             hqsl=qsl, hsl=sl, R=1, T=1, Hq=8, Hkv=2, D=64, N=4, B=16, scale=0.125, dtype=1,
             ws=4096, wsb=1 << 20)
    a.update(over)
    p32 = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    rc = L.pa_attention(a["out"], a["query"], a["kc"], a["vc"], a["bt"], a["M"], a["dqsl"],
                        a["dsl"], a["dnc"], p32(a["hqsl"]), p32(a["hsl"]), a["R"], a["T"], a["Hq"],
                        a["Hkv"], a["D"], a["N"], a["B"], a["scale"], a["dtype"], a["ws"], a["wsb"],
                        None)
    return pa.status_str(rc)


def test_attention_host_checks_refuse_bad_arguments():
    assert _call_attention(D=96) == "PA_ERR_UNSUPPORTED"
    assert _call_attention(Hq=12, Hkv=8) == "PA_ERR_UNSUPPORTED"
    assert _call_attention(Hq=48, Hkv=3) == "PA_ERR_UNSUPPORTED"      # G = 16
    assert _call_attention(B=24) == "PA_ERR_UNSUPPORTED"
    assert _call_attention(dtype=7) == "PA_ERR_BAD_DTYPE"
    assert _call_attention(T=2) == "PA_ERR_INCONSISTENT_METADATA"
    assert _call_attention(hsl=np.array([0], np.int32)) == "PA_ERR_INCONSISTENT_METADATA"
    assert _call_attention(hsl=np.array([17], np.int32)) == "PA_ERR_OUT_OF_RANGE"   # > M * B
    assert _call_attention(out=0) == "PA_ERR_NULL_PTR"
    assert _call_attention(ws=4096 + 16) == "PA_ERR_BAD_SHAPE"        # misaligned workspace
    assert _call_attention(wsb=16) == "PA_ERR_WORKSPACE_TOO_SMALL"
    assert _call_attention(scale=-1.0) == "PA_ERR_BAD_SHAPE"
    # a step with no query rows is a no-op (nothing to check, nothing launched)
    assert _call_attention(hqsl=np.array([0, 0], np.int32), T=0, out=0) == "PA_OK"


def test_write_kv_host_checks():
    L = pa.lib()
    def rc(**over):
        a = dict(k=4096, v=4096, kc=4096, vc=4096, sm=4096, T=3, N=4, B=16, Hkv=2, D=64, dt=1)
        a.update(over)
        return pa.status_str(L.pa_write_kv(a["k"], a["v"], a["kc"], a["vc"], a["sm"], a["T"], a["N"],
                                           a["B"], a["Hkv"], a["D"], a["dt"], None))
    assert rc(D=32) == "PA_ERR_UNSUPPORTED"
    assert rc(B=8) == "PA_ERR_UNSUPPORTED"
    assert rc(dt=3) == "PA_ERR_BAD_DTYPE"
    assert rc(sm=0) == "PA_ERR_NULL_PTR"
    assert rc(T=-1) == "PA_ERR_BAD_SHAPE"
    assert rc(k=4100) == "PA_ERR_BAD_SHAPE"
    assert rc(T=0, k=0) == "PA_OK"


def test_rope_write_kv_host_checks():
    L = pa.lib()
    def rc(**over):
        a = dict(q=4096, k=4096, v=4096, kc=4096, vc=4096, sm=4096, pos=4096, cs=4096, mp=100,
                 rd=64, nx=1, T=3, Hq=8, Hkv=2, D=64, N=4, B=16, dt=1)
        a.update(over)
        return pa.status_str(L.pa_rope_write_kv(a["q"], a["k"], a["v"], a["kc"], a["vc"], a["sm"],
                                                a["pos"], a["cs"], a["mp"], a["rd"], a["nx"], a["T"],
                                                a["Hq"], a["Hkv"], a["D"], a["N"], a["B"], a["dt"],
                                                None))
    assert rc(D=32) == "PA_ERR_UNSUPPORTED"
    assert rc(rd=0) == "PA_ERR_UNSUPPORTED"
    assert rc(rd=24) == "PA_ERR_UNSUPPORTED"          # not a multiple of 16
    assert rc(rd=128) == "PA_ERR_UNSUPPORTED"         # past head_dim
    assert rc(mp=0) == "PA_ERR_BAD_SHAPE"
    assert rc(nx=2) == "PA_ERR_BAD_SHAPE"
    assert rc(Hq=6) == "PA_ERR_UNSUPPORTED"           # GQA group 3
    assert rc(dt=3) == "PA_ERR_BAD_DTYPE"
    assert rc(pos=0) == "PA_ERR_NULL_PTR"
    assert rc(cs=0) == "PA_ERR_NULL_PTR"
    assert rc(q=4100) == "PA_ERR_BAD_SHAPE"
    assert rc(cs=4098) == "PA_ERR_BAD_SHAPE"
    assert rc(T=-1) == "PA_ERR_BAD_SHAPE"
    assert rc(T=0, q=0, pos=0) == "PA_OK"


def test_copy_blocks_host_checks():
    L = pa.lib()
    def rc(**over):
        a = dict(s=4096, d=4096, p=4096, n=3, P=2, ss=1 << 20, ds=1 << 20, ns=16, nd=16, bb=4096)
        a.update(over)
        return pa.status_str(L.pa_copy_blocks(a["s"], a["d"], a["p"], a["n"], a["P"], a["ss"], a["ds"],
                                              a["ns"], a["nd"], a["bb"], None))
    assert rc(n=-1) == "PA_ERR_BAD_SHAPE"
    assert rc(p=0) == "PA_ERR_NULL_PTR"
    assert rc(bb=100) == "PA_ERR_BAD_SHAPE"
    assert rc(ss=4096) == "PA_ERR_BAD_SHAPE"           # pools would overlap
    assert rc(s=4100) == "PA_ERR_BAD_SHAPE"
    assert rc(nd=0) == "PA_ERR_BAD_SHAPE"
    assert rc(P=70000) == "PA_ERR_BAD_SHAPE"
    assert rc(n=0, s=0) == "PA_OK"


def test_generator_host_mirror_properties():
    # deterministic, distinct streams, ~N(0,1), bf16 rounding to nearest even
    a = rng.row_values(rng.base_row_keys(rng.key(1, 2), np.arange(64)), 256, "f32")
    b = rng.row_values(rng.base_row_keys(rng.key(1, 2), np.arange(64)), 256, "f32")
    c = rng.row_values(rng.base_row_keys(rng.key(1, 3), np.arange(64)), 256, "f32")
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    big = rng.row_values(rng.base_row_keys(7, np.arange(4000)), 256, "f32")
    assert abs(big.mean()) < 0.01 and abs(big.std() - 1) < 0.01
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.5 - 2 ** -9], np.float32)
    hb = rng.f32_to_bf16_bits(x)
    back = oracle.bf16_bits_to_f64(hb)
    assert back.tolist() == [1.0, 1.0 + 4 * 2 ** -8, -1.5]   # ties to even


def test_noalloc_scratch_size_matches_header():
    txt = open(os.path.join(ROOT, "include", "pa.h")).read()
    m = re.search(r"#define PA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", txt)
    assert m and int(m.group(1)) << int(m.group(2)) == pa.NOALLOC_SCRATCH_BYTES


def test_swap_blocks_host_checks():
    """pa_swap_blocks checks its host-side block list before enqueueing
    anything (dummy pool pointers, never touched)."""
    L = pa.lib()

    def rc(pairs, n_src=8, n_dst=8, pools=4, bb=1024, sstride=8 * 1024, dstride=8 * 1024, src=4096, dst=8192):
        a = np.ascontiguousarray(np.asarray(pairs, np.int32).reshape(-1, 2))
        return pa.status_str(L.pa_swap_blocks(src, dst, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                              a.shape[0], pools, sstride, dstride, n_src, n_dst, bb, None))
    assert rc([[0, 1], [9, 2]]) == "PA_ERR_OUT_OF_RANGE"
    assert rc([[0, 1], [2, -1]]) == "PA_ERR_OUT_OF_RANGE"
    assert rc([[0, 3], [1, 3]]) == "PA_ERR_DUPLICATE_SLOT"
    assert rc([[0, 1]], sstride=1024) == "PA_ERR_BAD_SHAPE"
    assert rc([[0, 1]], bb=0) == "PA_ERR_BAD_SHAPE"
    assert rc([[0, 1]], src=0) == "PA_ERR_NULL_PTR"
    assert rc(np.zeros((0, 2))) == "PA_OK"
