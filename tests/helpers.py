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
