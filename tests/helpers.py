"""Shared helpers for the GPU parity tests: run one step through the C ABI and
build the oracle's expected values for chosen requests from the host mirror of
the input generator."""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle

TOL = {"f32": (1e-5, 1e-5), "bf16": (1e-2, 1e-2)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def storage_np(t) -> np.ndarray:
    """Device/host torch tensor -> numpy storage array (bf16 as uint16)."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


def assert_close(got, want, dtype, what=""):
    """|got - want| <= atol + rtol * |want| elementwise (the assert_close form
    the chunked-prefill page uses), NaN nowhere."""
    atol, rtol = TOL[dtype]
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.all(np.isfinite(want)), f"{what}: oracle produced non-finite values"
    assert np.all(np.isfinite(got)), f"{what}: GPU produced non-finite values"
    err = np.abs(got - want)
    bad = err > atol + rtol * np.abs(want)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance, "
                           f"max err {err.max():.3e}")
    return float(err.max())


def run_step(spec, pa, dev_inputs=None, stream=None, workspace=None):
    """Write the step's new K/V and run attention through the C ABI.
    Returns (inputs dict, out tensor, host slot mapping)."""
    import torch
    d = dev_inputs if dev_inputs is not None else spec.device_inputs()
    qsl, sl, sm = pa.build_step_metadata(spec.query_lens, spec.num_computed, spec.block_table,
                                         spec.B, spec.num_blocks)
    d["slot_mapping"] = torch.from_numpy(sm).to(d["query"].device)
    pa.write_kv(d["key"], d["value"], d["key_cache"], d["value_cache"], d["slot_mapping"], stream=stream)
    out = torch.empty_like(d["query"])
    if workspace is None:
        workspace = pa.alloc_workspace(
            pa.attention_workspace_size(qsl, sl, spec.Hq, spec.Hkv, spec.D, spec.B,
                                        pa.PA_BF16 if spec.dtype == "bf16" else pa.PA_F32),
            d["query"].device)
    pa.attention(out, d["query"], d["key_cache"], d["value_cache"], d["block_table"],
                 d["query_start_loc"], d["seq_lens"], d["num_computed"], qsl, sl, spec.scale,
                 workspace=workspace, stream=stream)
    return d, out, sm


def oracle_request(spec, r, rows_local=None):
    """Oracle for request r: regenerate its blocks from the host mirror, apply
    the oracle's own slot mapping and write for the request's new tokens, then
    attention in fp64 for the chosen query rows (default: all).
    Returns (out [n, Hq, D], lse, kpool, vpool, block ids, rows_local)."""
    q = int(spec.query_lens[r])
    c = int(spec.num_computed[r])
    L = q + c
    B = spec.B
    nblk = -(-L // B)
    ids = spec.block_table[r, :nblk].astype(np.int64)
    kpool = spec.host_pool_blocks("k", ids)
    vpool = spec.host_pool_blocks("v", ids)
    t0 = int(spec.query_start_loc[r])
    mini = np.arange(nblk, dtype=np.int32)[None]
    if q:
        rows = np.arange(t0, t0 + q)
        slots = oracle.slot_mapping(mini, [q], [c], B)
        oracle.write_kv(kpool, vpool, spec.host_rows("k", rows), spec.host_rows("v", rows), slots, B)
    if rows_local is None:
        rows_local = np.arange(q)
    rows_local = np.asarray(rows_local, dtype=np.int64)
    K = oracle.gather_kv(kpool, mini[0], L, B)
    V = oracle.gather_kv(vpool, mini[0], L, B)
    Q = spec.host_rows("q", t0 + rows_local)
    out, lse = oracle.attention_rows(Q, K, V, c + rows_local, spec.scale, spec.dtype)
    return out, lse, kpool, vpool, ids, rows_local


def check_requests(spec, out_t, kc_t, vc_t, reqs, rows_per_req=None, what=""):
    """Compare GPU outputs (and the request's cache blocks, bit-exact) with the
    oracle for the listed requests."""
    import torch
    worst = 0.0
    for r in reqs:
        q = int(spec.query_lens[r])
        if q == 0:
            continue
        rows = None
        if rows_per_req is not None and q > rows_per_req:
            rng = np.random.default_rng(1000 + r)
            rows = np.unique(np.concatenate([[0, 1, q - 2, q - 1],
                                             rng.choice(q, rows_per_req - 4, replace=False)]))
        o, _, kp, vp, ids, rl = oracle_request(spec, r, rows)
        idx = torch.from_numpy(ids).to(kc_t.device)
        gk = storage_np(kc_t.index_select(0, idx))
        gv = storage_np(vc_t.index_select(0, idx))
        assert np.array_equal(bits(gk), bits(kp)), f"{what}: key cache blocks of request {r} differ"
        assert np.array_equal(bits(gv), bits(vp)), f"{what}: value cache blocks of request {r} differ"
        t0 = int(spec.query_start_loc[r])
        g = oracle.as_f64(storage_np(out_t[t0 + torch.from_numpy(rl).to(out_t.device)]), spec.dtype)
        worst = max(worst, assert_close(g, o, spec.dtype, f"{what} request {r}"))
    return worst


def sample_requests(spec, n, seed=0, must=()):
    rng = np.random.default_rng(seed)
    R = spec.R
    pick = set(int(x) for x in must)
    order = rng.permutation(R)
    for r in order:
        if len(pick) >= n:
            break
        pick.add(int(r))
    return sorted(pick)


def check_full_step(spec, pre_k, pre_v, out_t, kc_t, vc_t, what="", spot_blocks=16):
    """Whole-step parity.  pre_k / pre_v are device clones of the generator's
    pools taken before the step (the device generator equals its host mirror
    bit for bit; `spot_blocks` random blocks are re-checked against the host
    mirror here).  For every request: the oracle's own slot mapping and write
    on the request's pre-step blocks, then its attention for every query row;
    the GPU rows must be within the dtype's tolerance and the request's blocks
    after the step bit-exact.  Every slot outside the step's written slots
    must be unchanged (compared on the device, in slabs).
    Returns (worst abs err, rows checked, slots written)."""
    import torch
    dev = kc_t.device
    g = np.random.default_rng(spec.seed)
    spot = g.choice(spec.num_blocks, min(spot_blocks, spec.num_blocks), replace=False)
    for which, pre in (("k", pre_k), ("v", pre_v)):
        host = spec.host_pool_blocks(which, spot)
        got = storage_np(pre.index_select(0, torch.from_numpy(spot.astype(np.int64)).to(dev)))
        assert np.array_equal(bits(got), bits(host)), f"{what}: generator pool differs from its host mirror"
    T = spec.T
    rows = np.arange(T)
    q_all = spec.host_rows("q", rows)
    k_all = spec.host_rows("k", rows)
    v_all = spec.host_rows("v", rows)
    out_all = oracle.as_f64(storage_np(out_t), spec.dtype)
    worst, n_rows = 0.0, 0
    written = []
    for r in range(spec.R):
        q = int(spec.query_lens[r])
        if q == 0:
            continue
        c = int(spec.num_computed[r])
        L = q + c
        B = spec.B
        nblk = -(-L // B)
        ids = spec.block_table[r, :nblk].astype(np.int64)
        idx = torch.from_numpy(ids).to(dev)
        kp = storage_np(pre_k.index_select(0, idx)).copy()
        vp = storage_np(pre_v.index_select(0, idx)).copy()
        t0 = int(spec.query_start_loc[r])
        mini = np.arange(nblk, dtype=np.int32)[None]
        slots = oracle.slot_mapping(mini, [q], [c], B)
        oracle.write_kv(kp, vp, k_all[t0:t0 + q], v_all[t0:t0 + q], slots, B)
        written.append(ids[slots // B] * B + slots % B)
        assert np.array_equal(bits(storage_np(kc_t.index_select(0, idx))), bits(kp)), \
            f"{what}: key cache blocks of request {r} differ"
        assert np.array_equal(bits(storage_np(vc_t.index_select(0, idx))), bits(vp)), \
            f"{what}: value cache blocks of request {r} differ"
        K = oracle.gather_kv(kp, mini[0], L, B)
        V = oracle.gather_kv(vp, mini[0], L, B)
        want, _ = oracle.attention_rows(q_all[t0:t0 + q], K, V, c + np.arange(q), spec.scale, spec.dtype)
        worst = max(worst, assert_close(out_all[t0:t0 + q], want, spec.dtype, f"{what} request {r}"))
        n_rows += q
    written = np.sort(np.concatenate(written)) if written else np.zeros(0, np.int64)
    # every slot the step did not write keeps its pre-step bits
    slot_w = spec.Hkv * spec.D
    iv = torch.int16 if spec.dtype == "bf16" else torch.int32
    for post, pre in ((kc_t, pre_k), (vc_t, pre_v)):
        a = post.view(iv).reshape(-1, slot_w)
        b = pre.view(iv).reshape(-1, slot_w)
        changed = []
        step = 1 << 20
        for s0 in range(0, a.shape[0], step):
            ch = torch.nonzero((a[s0:s0 + step] != b[s0:s0 + step]).any(dim=1)).flatten() + s0
            changed.append(ch.cpu().numpy())
        changed = np.concatenate(changed)
        assert np.all(np.isin(changed, written)), f"{what}: slots outside the step's writes changed"
    return worst, n_rows, len(written)
