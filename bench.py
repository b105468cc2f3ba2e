#!/usr/bin/env python3
"""Benchmark of the paged-KV attention step on one MI355X.

One step = the whole hot path over one synthetic batch, all on the device:
  slot mapping -> write_kv -> attention (plan, split-K decode rows, bf16 MFMA
  prefill chunks, log-sum-exp merge).
Default workload: the mixed chunked-prefill step (3 prefill chunks of 512
tokens at seeded offsets into 16384-token prompts + 512 decode requests with
lognormal contexts, median 2048; Llama-3-8B heads: 32 q, 8 kv, head_dim 128,
block 16, bf16), i.e. the configuration that exercises every part of the step.

Prints ONE JSON line.  `value` is the decode KV-read bandwidth (algorithmic
bytes of the decode rows / time of the split-K and merge kernels in the timed
steps); chunk TFLOP/s, per-kernel times, the roofline of the dominant kernel
and a CPU-oracle baseline ride along.  The fused rotary-embedding + cache-write
kernel (the step that precedes the write when Q/K still need their position
rotation) is timed on its own on the same tokens and reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode KV-read GB/s (% HBM peak) + prefill-chunk TFLOP/s (% MFMA) per step"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MALL_ROTATE_BYTES = 1 << 30      # footprint rotated through when a step's pools are small
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, published
KERNEL_SOURCES = {
    "rowwise": ["paged_kv_attention_reshape_amd/csrc/k_rowwise.hip",
                "paged_kv_attention_reshape_amd/csrc/k_rowwise_mfma.hip"],
    "chunk": ["paged_kv_attention_reshape_amd/csrc/k_chunk.hip"],
}


def decode_kernel_name(spec) -> str:
    """The split-K kernel the library runs for this geometry with the default
    tuning (its own rule, restated here as a label for the report)."""
    G = spec.Hq // spec.Hkv
    if spec.dtype == "bf16" and G == 8:
        if spec.D == 128 and spec.Hkv in (1, 2, 4, 8):
            return "rowwise_mfma_block_kernel (whole-block split-K decode on the matrix cores)"
        return "rowwise_mfma_kernel (split-K decode on the matrix cores)"
    if spec.dtype == "bf16" and spec.D == 128 and G in (1, 2, 4) and spec.Hkv in (1, 2, 4, 8):
        return "rowwise_block_kernel (whole-block split-K decode)"
    return "rowwise_kernel (per-head split-K decode)"


def source_hash(rels) -> str:
    """sha256 prefix over the concatenated source files (one path or a list)."""
    h = hashlib.sha256()
    for rel in ([rels] if isinstance(rels, str) else rels):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="c3", choices=["c2", "c3", "c4"])
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="budget of oracle work for the CPU baseline (0 disables it)")
    p.add_argument("--no-swap", dest="swap", action="store_false",
                   help="skip the swap-out / swap-in round-trip measurement")
    p.add_argument("--no-rope", dest="rope", action="store_false",
                   help="skip the separate timing of the fused rotary + cache-write kernel")
    p.add_argument("--no-serving", dest="serving", action="store_false",
                   help="skip the 32-layer serving-trace throughput measurement")
    p.add_argument("--no-extra", dest="extra", action="store_false",
                   help="skip the pure-decode and long-context decode configurations and their oracle timings")
    p.add_argument("--serving-only", action="store_true",
                   help="run only the serving-trace measurement (for profiling runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="instead of the step, run a plain 1 GiB device copy a few times "
                        "(reference for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def copy_calibration():
    """A plain device-to-device copy of exactly 1 GiB, three times: the HBM
    byte counters of a profiling run of this mode give the counter-to-bytes
    scale (2^30 bytes read and 2^30 bytes written per copy)."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)


def _host(t):
    import numpy as np
    import torch
    t = t.detach().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def oracle_request_seconds(spec, d, r) -> float:
    """Time the fp64 oracle on request r of a step: its slot mapping, cache
    write, gather and attention.  Inputs: the generator's pre-write pool
    blocks of the request and its query / new K/V rows, copied from the
    device before any step ran (not timed)."""
    import numpy as np
    import torch
    import oracle
    q = int(spec.query_lens[r])
    L = int(spec.seq_lens[r])
    c = L - q
    nblk = -(-L // spec.B)
    ids = torch.from_numpy(spec.block_table[r, :nblk].astype(np.int64)).to(d["key_cache"].device)
    kp = _host(d["key_cache"].index_select(0, ids))
    vp = _host(d["value_cache"].index_select(0, ids))
    t = int(spec.query_start_loc[r])
    qrows = _host(d["query"][t:t + q])
    knew = _host(d["key"][t:t + q])
    vnew = _host(d["value"][t:t + q])
    mini = np.arange(nblk, dtype=np.int32)[None]
    t0 = time.perf_counter()
    sm = oracle.slot_mapping(mini, [q], [c], spec.B)
    oracle.write_kv(kp, vp, knew, vnew, sm, spec.B)
    K = oracle.gather_kv(kp, mini[0], L, spec.B)
    V = oracle.gather_kv(vp, mini[0], L, spec.B)
    oracle.attention_rows(qrows, K, V, c + np.arange(q), spec.scale, spec.dtype)
    return time.perf_counter() - t0


def cpu_baseline(spec, d, budget_s):
    """Time the fp64 oracle on a bounded sample of the same step: every decode
    request in flattened order (until the time budget is spent), then the
    step's prefill chunks (all their rows).  The oracle gets the generator's
    pre-write pool blocks and the step's query / new K/V rows (copied from the
    device generator before any step ran) and does its own slot mapping,
    write, gather and attention.  `value` is the decode part in GB/s (the
    metric's unit); the chunk part is reported in GFLOP/s."""
    import numpy as np
    import torch
    import oracle
    from threadpoolctl import threadpool_info

    def run_request(r):
        return oracle_request_seconds(spec, d, r)

    dec = [r for r in range(spec.R) if spec.query_lens[r] == 1]
    chunks = [r for r in range(spec.R) if spec.query_lens[r] > 1]
    dec_s = 0.0
    dec_bytes = 0
    n = 0
    for r in dec:
        if dec_s >= budget_s:
            break
        dec_s += run_request(r)
        L = int(spec.seq_lens[r])
        dec_bytes += L * spec.Hkv * spec.D * 2 * spec.esize + 2 * spec.Hq * spec.D * spec.esize \
            + 4 * (-(-L // spec.B)) + 12
        n += 1
    ck_s = 0.0
    ck_flops = 0
    for r in chunks:
        ck_s += run_request(r)
        q, c = int(spec.query_lens[r]), int(spec.num_computed[r])
        ck_flops += 4 * spec.D * spec.Hq * (q * c + q * (q + 1) // 2)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": round(dec_bytes / dec_s / 1e9, 4) if dec_s > 0 else None,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n} of {len(dec)} decode requests ({dec_s:.1f} s) and all {len(chunks)} prefill chunks "
                  f"({ck_s:.1f} s) of the same step; fp64 numpy oracle: slot mapping, write, gather, attention",
        "chunk_gflops": round(ck_flops / ck_s / 1e9, 3) if ck_s > 0 else None,
        "scheduler_us_per_step": scheduler_timing(product=False)["us_per_step"],
        "scheduler_shared_prefix_us_per_step": scheduler_timing(product=False, shared=True)["us_per_step"],
        "host_cpus": len(os.sched_getaffinity(0)),
    }


SHARED_TRACE = dict(shared_prompts=8, shared_len=1024, shared_frac=0.8)


def scheduler_timing(product: bool, steps: int = 200, shared: bool = False):
    """Host time per planned step of the serving trace (2048 requests, 16384
    blocks of 16, budget 8192, chunk 512): schedule + copy of the step's
    arrays + commit.  shared=True gives 80 % of the requests one of 8 system
    prompts of 1024 tokens, with prefix keys, so admissions attach cached
    blocks.  product=False times the reference scheduler (only the
    CPU-baseline leg does that)."""
    from workloads import serving_trace as st
    cfg = st.TraceConfig(steps=steps, **(SHARED_TRACE if shared else {}))
    keys = st.block_keys(cfg)
    toks = 0
    if product:
        # the C ABI directly, with preallocated output arrays (what a serving
        # loop would do): plan, copy the step's metadata, commit
        import ctypes
        import numpy as np
        import paged_kv_attention_reshape_amd as pa
        from paged_kv_attention_reshape_amd import _sched
        s = pa.Scheduler(**st.scheduler_args(cfg))
        for rid, p, o in st.requests(cfg):
            s.add_request(rid, p, o, keys.get(rid, ()))
        L = pa.sched_lib()
        cap, M = cfg.max_num_seqs, -(-(cfg.prompt_max + 4096) // cfg.block_size)
        ids = np.zeros(cap, np.int64)
        comp = np.zeros(cap, np.int32)
        ql = np.zeros(cap, np.int32)
        bt = np.zeros((cap, M), np.int32)
        pre = np.zeros((cap, 3), np.int64)
        cps = np.zeros((cap, 2), np.int32)
        fin = np.zeros(cap, np.int64)
        info = _sched._PlanInfo()
        nfin = ctypes.c_int32()
        P = ctypes.POINTER
        a_ids, a_comp, a_ql = (x.ctypes.data_as(P(t)) for x, t in
                               ((ids, ctypes.c_int64), (comp, ctypes.c_int32), (ql, ctypes.c_int32)))
        a_bt = bt.ctypes.data_as(P(ctypes.c_int32))
        a_pre = pre.ctypes.data_as(P(ctypes.c_int64))
        a_cps = cps.ctypes.data_as(P(ctypes.c_int32))
        a_fin = fin.ctypes.data_as(P(ctypes.c_int64))
        t0 = time.perf_counter()
        for _ in range(cfg.steps):
            assert L.pa_sched_schedule(s._h, ctypes.byref(info)) == 0
            assert L.pa_sched_plan_copy(s._h, a_ids, a_comp, a_ql, cap, a_bt, info.max_blocks,
                                        a_pre, cap, a_cps, cap) == 0
            toks += info.num_tokens
            assert L.pa_sched_commit(s._h, a_fin, cap, ctypes.byref(nfin)) == 0
        dt = time.perf_counter() - t0
    else:
        from oracle.sched_oracle import Scheduler as RefScheduler
        s = RefScheduler(**st.scheduler_args(cfg))
        for rid, p, o in st.requests(cfg):
            s.add_request(rid, p, o, keys.get(rid, ()))
        t0 = time.perf_counter()
        for _ in range(cfg.steps):
            plan = s.schedule()
            toks += sum(n for _, _, n in plan["sched"])
            s.commit()
        dt = time.perf_counter() - t0
    m = s.metrics()
    out = {"us_per_step": round(dt / cfg.steps * 1e6, 1), "steps": cfg.steps,
           "scheduled_tokens": toks, "preemptions": m["preemptions"]}
    if shared:
        out.update({"prefix_hit_tokens": m["prefix_hit_tokens"], "evictions": m["evictions"],
                    "cow_copies": m["cow_copies"], "cached_blocks": m["cached_blocks"],
                    "trace": "as above, 80 % of requests start with one of 8 shared 1024-token system prompts"})
    return out


def serving_measurement(dev, first: int = 40, steps: int = 20, layers: int = 32):
    """GPU throughput on the serving trace: the steps the C++ scheduler plans
    for 2048 requests (prompts lognormal median 1500, chunk 512, budget 8192,
    recompute preemption), each run as write_kv + attention over every layer
    of a 32-layer, 16384-block cache (32 GiB, Llama-3-8B attention geometry).
    Each step is planned once (pa_attention_plan: the metadata has no layer
    dimension) and run per layer (pa_attention_run).  Steps first .. first +
    steps - 1 (past the ramp-up) are timed with HIP events around all their
    layers, then run again with the library's per-kernel events to split the
    time into plan, split-K decode, chunk and merge; inputs are device-resident
    and filled once per step (not timed)."""
    import numpy as np
    import torch
    import paged_kv_attention_reshape_amd as pa
    from workloads import serving_trace as st
    cfg = st.TraceConfig()
    plans = st.drive(pa.Scheduler(**st.scheduler_args(cfg)), cfg)
    sel = [p for p in plans[first:first + steps] if p["sched"]]
    HQ, HKV, D, B = 32, 8, 128, cfg.block_size
    kc = torch.zeros((layers, cfg.num_blocks, B, HKV, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    # one workspace for the whole trace, sized by the scheduler's limits
    ws_bytes = pa.attention_workspace_bound(cfg.max_num_seqs, cfg.max_num_batched_tokens, st.max_seq_len(cfg),
                                            HQ, HKV, D, B, pa.PA_BF16)
    ws = pa.alloc_workspace(ws_bytes, dev)
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device=dev).manual_seed(5)
    scale = 1.0 / np.sqrt(D)
    total_ms, total_tok, n_dec, n_chunk_tok = 0.0, 0, 0, 0
    host_plan_s = 0.0
    dec_bytes, chunk_flops = 0, 0
    acc = {"plan": 0.0, "write_kv": 0.0, "rowwise": 0.0, "chunk": 0.0, "merge": 0.0}
    per_step = []
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for p in sel:
        ql, cp, bt, _, _ = st.step_arrays(p, B)
        T = int(ql.sum())
        qsl, sl, sm = pa.build_step_metadata(ql, cp, bt, B, cfg.num_blocks)
        d = {k: torch.from_numpy(v).to(dev) for k, v in
             {"bt": bt, "qsl": qsl, "sl": sl, "nc": cp, "sm": sm}.items()}
        q = torch.randn((T, HQ, D), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((T, HKV, D), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((T, HKV, D), generator=gen, device=dev).to(torch.bfloat16)
        out = torch.empty_like(q)
        dl = (ql == 1)
        Ld = (ql + cp)[dl].astype(np.int64)
        dec_bytes += layers * int(np.sum(Ld) * HKV * D * 2 * 2 + dl.sum() * 2 * HQ * D * 2
                                  + 4 * np.sum(-(-Ld // B)) + 12 * dl.sum())
        cq, cc = ql[~dl].astype(np.int64), cp[~dl].astype(np.int64)
        chunk_flops += layers * int(np.sum(4 * D * HQ * (cq * cc + cq * (cq + 1) // 2)))
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        # planned once per step (the metadata has no layer dimension), run per layer
        h0 = time.perf_counter()
        plan = pa.attention_plan(d["bt"], d["qsl"], d["sl"], d["nc"], qsl, sl, HQ, kc.shape[1:], pa.PA_BF16, ws)
        host_plan_s += time.perf_counter() - h0
        for layer in range(layers):
            pa.write_kv(k, v, kc[layer], vc[layer], d["sm"])
            pa.attention_run(plan, out, q, kc[layer], vc[layer], scale)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        # the same step again with per-kernel events (the events add small gaps between kernels)
        pe = [ev() for _ in range(5)]
        lay = [[ev() for _ in range(5)] for _ in range(layers)]
        wk = [(ev(), ev()) for _ in range(layers)]
        pa.set_profiling_events(pe)
        plan = pa.attention_plan(d["bt"], d["qsl"], d["sl"], d["nc"], qsl, sl, HQ, kc.shape[1:], pa.PA_BF16, ws)
        for layer in range(layers):
            wk[layer][0].record(stream)
            pa.write_kv(k, v, kc[layer], vc[layer], d["sm"])
            wk[layer][1].record(stream)
            pa.set_profiling_events(lay[layer])
            pa.attention_run(plan, out, q, kc[layer], vc[layer], scale)
        pa.set_profiling_events(None)
        torch.cuda.synchronize()
        acc["plan"] += pe[0].elapsed_time(pe[1])
        for layer in range(layers):
            e = lay[layer]
            acc["write_kv"] += wk[layer][0].elapsed_time(wk[layer][1])
            acc["rowwise"] += e[1].elapsed_time(e[2])
            acc["chunk"] += e[2].elapsed_time(e[3])
            acc["merge"] += e[3].elapsed_time(e[4])
        total_ms += ms
        total_tok += T
        n_dec += int(dl.sum())
        n_chunk_tok += int(np.sum(ql[~dl]))
        per_step.append(round(ms, 3))
    del kc, vc
    torch.cuda.empty_cache()
    n = max(1, len(sel))
    us = {k: round(1e3 * v / n, 2) for k, v in acc.items()}
    dec_s = (acc["rowwise"] + acc["merge"]) * 1e-3
    rw_s = acc["rowwise"] * 1e-3
    ck_s = acc["chunk"] * 1e-3
    dec_gbs = dec_bytes / dec_s / 1e9 if dec_s > 0 else None
    rw_gbs = dec_bytes / rw_s / 1e9 if rw_s > 0 else None
    ck_tf = chunk_flops / ck_s / 1e12 if ck_s > 0 else None
    return {"steps": len(sel), "first_step": first, "layers": layers, "tokens": total_tok,
            "decode_rows": n_dec, "chunk_tokens": n_chunk_tok,
            "ms_per_step": round(total_ms / n, 3),
            "tokens_per_s": round(total_tok / (total_ms * 1e-3), 1) if total_ms > 0 else None,
            "step_ms_p10_p50_p90": [round(float(x), 3) for x in np.percentile(per_step, [10, 50, 90])],
            "kernel_us_per_step": us,
            "decode_bytes_per_step": dec_bytes // n, "chunk_flops_per_step": chunk_flops // n,
            "decode_gbs": round(dec_gbs, 1) if dec_gbs else None,
            "decode_frac_hbm": round(dec_gbs / HBM_PEAK_GBS, 4) if dec_gbs else None,
            "rowwise_gbs": round(rw_gbs, 1) if rw_gbs else None,
            "chunk_tflops": round(ck_tf, 1) if ck_tf else None,
            "chunk_frac_mfma": round(ck_tf / MFMA_BF16_PEAK_TFLOPS, 4) if ck_tf else None,
            "workspace_bytes": ws_bytes,
            "host_plan_us_per_step": round(1e6 * host_plan_s / n, 1),
            "trace": "2048 requests at step 0, prompts lognormal median 1500, outputs geometric mean 256, "
                     "chunk 512, budget 8192, 16384 blocks of 16; Hq 32, Hkv 8, D 128",
            "includes": "write_kv + attention (slot mapping built on the host) for every layer of the step; "
                        "one plan per step, one attention run per layer"}


def swap_measurement(dev, reps: int = 10):
    """Swap-out + swap-in of whole block columns (every layer's K and V
    block) between the device cache and a pinned host pool, in the geometry
    of the pages' worked swap example (512 KiB of K/V per token: 32 layers,
    32 kv heads, head_dim 128, bf16; block 16), on the copy engines
    (pa_swap_blocks, the swap path) and with the copy kernel (pa_copy_blocks)
    for comparison.  Returns the measured round trips and the pages' formula
    2 * payload / bandwidth beside them."""
    import numpy as np
    import torch
    import paged_kv_attention_reshape_amd as pa
    L, HKV, D, B = 32, 32, 128, 16
    kappa = 2 * L * HKV * D * 2                  # bytes of K/V per token (all layers)
    nb, hb = 96, 64
    pools = torch.zeros((2 * L, nb, B, HKV, D), dtype=torch.bfloat16, device=dev)
    host = torch.empty((2 * L, hb, B, HKV, D), dtype=torch.bfloat16, pin_memory=True)
    stream = torch.cuda.current_stream()
    res = {}
    for path in ("engines", "kernel"):
        out = {}
        for n in (1, 64):
            g = np.random.default_rng(n)
            src = g.choice(nb, n, replace=False).astype(np.int32)
            dst = g.choice(hb, n, replace=False).astype(np.int32)
            h_out, h_in = np.stack([src, dst], 1), np.stack([dst, src], 1)
            p_out, p_in = torch.from_numpy(h_out).to(dev), torch.from_numpy(h_in).to(dev)

            def go(direction):
                if path == "engines":
                    if direction == "out":
                        pa.swap_blocks(pools, host, h_out)
                    else:
                        pa.swap_blocks(host, pools, h_in)
                else:
                    if direction == "out":
                        pa.copy_blocks(pools, host, p_out)
                    else:
                        pa.copy_blocks(host, pools, p_in)
            for _ in range(2):
                go("out")
                go("in")
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            torch.cuda.synchronize()
            e[0].record(stream)
            for _ in range(reps):
                go("out")
            e[1].record(stream)
            for _ in range(reps):
                go("in")
            e[2].record(stream)
            torch.cuda.synchronize()
            t_out = e[0].elapsed_time(e[1]) / reps
            t_in = e[1].elapsed_time(e[2]) / reps
            payload = n * B * kappa
            out[f"{n}_block"] = {"bytes_each_way": payload, "out_ms": round(t_out, 4), "in_ms": round(t_in, 4),
                                 "roundtrip_ms": round(t_out + t_in, 4),
                                 "out_gbs": round(payload / t_out / 1e6, 1), "in_gbs": round(payload / t_in / 1e6, 1)}
        res[path] = out
    out = res["engines"]
    beta = 2 * out["64_block"]["bytes_each_way"] / (out["64_block"]["roundtrip_ms"] * 1e6)   # GB/s
    tokens = 7
    out["pages_example"] = {
        "tokens": tokens, "kv_bytes_per_token": kappa,
        "formula_ms_at_24_gbs": round(2 * tokens * kappa / 24e9 * 1e3, 4),
        "formula_ms_at_measured_bandwidth": round(2 * tokens * kappa / (beta * 1e9) * 1e3, 4),
        "measured_bandwidth_gbs": round(beta, 1),
        "measured_ms_one_block": out["1_block"]["roundtrip_ms"],
        "note": "the pool moves whole blocks: 7 tokens occupy one 16-token block column (16 * kappa bytes each way)",
    }
    out["path"] = "pa_swap_blocks: copy engines, one 2-D copy per run of consecutive block columns"
    out["copy_kernel"] = res["kernel"]
    del pools, host
    torch.cuda.empty_cache()
    return out


def pool_rotation(d, rotate_bytes=MALL_ROTATE_BYTES):
    """Pool copies so that consecutive steps touch >= rotate_bytes apart (the
    256 MB last-level cache must not serve a step's reads from the previous
    step); the first copy is the step's own pools."""
    pool_bytes = 2 * d["key_cache"].numel() * d["key_cache"].element_size()
    n = 1 if pool_bytes >= rotate_bytes else min(8, -(-rotate_bytes // pool_bytes))
    return [(d["key_cache"], d["value_cache"])] + \
        [(d["key_cache"].clone(), d["value_cache"].clone()) for _ in range(n - 1)]


def config_workload(name: str, dev, steps: int, warmup: int):
    """Another configuration (C1, C2, C4) timed like the main step: write_kv
    + attention per step over rotated pool copies, HIP events recorded by the
    library between its launches.  For the bf16 decode configurations (C2,
    C4): the split-K and merge times and the decode roofline (algorithmic
    bytes / time); C1 (fp32, a correctness configuration) reports its times
    only."""
    import numpy as np
    import torch
    import paged_kv_attention_reshape_amd as pa
    from workloads import configs
    spec = configs.BUILDERS[name]()
    d = spec.device_inputs(device=dev)
    pools = pool_rotation(d)
    out = torch.empty_like(d["query"])
    dt = pa.PA_BF16 if spec.dtype == "bf16" else pa.PA_F32
    ws = pa.alloc_workspace(pa.attention_workspace_size(spec.query_start_loc, spec.seq_lens, spec.Hq, spec.Hkv,
                                                        spec.D, spec.B, dt), dev)
    slots = torch.from_numpy(pa.build_step_metadata(spec.query_lens, spec.num_computed, spec.block_table,
                                                    spec.B, spec.num_blocks)[2]).to(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def one(i, events=None):
        kc, vc = pools[i % len(pools)]
        pa.write_kv(d["key"], d["value"], kc, vc, slots)
        if events is not None:
            pa.set_profiling_events(events)
        pa.attention(out, d["query"], kc, vc, d["block_table"], d["query_start_loc"], d["seq_lens"],
                     d["num_computed"], spec.query_start_loc, spec.seq_lens, spec.scale, ws)
        if events is not None:
            pa.set_profiling_events(None)

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        one(i)
    t1.record(stream)
    for i in range(steps):
        one(i, ev[i])
    torch.cuda.synchronize()
    rw = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
    ck = float(np.mean([e[2].elapsed_time(e[3]) for e in ev])) * 1e3
    mg = float(np.mean([e[3].elapsed_time(e[4]) for e in ev])) * 1e3
    pl = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    res = {"workload": configs.WORKLOADS[name], "requests": spec.R, "tokens": spec.T, "dtype": spec.dtype,
           "pool_copies": len(pools), "ms_per_step": round(t0.elapsed_time(t1) / steps, 4),
           "kernel_us": {"plan": round(pl, 2), "rowwise": round(rw, 2), "chunk": round(ck, 2), "merge": round(mg, 2)}}
    if spec.dtype != "bf16":
        res["note"] = "correctness configuration: times only, no roofline claim"
        return res
    db = spec.decode_bytes()
    rw_gbs = db / (rw * 1e-6) / 1e9
    val = db / ((rw + mg) * 1e-6) / 1e9
    res.update({"decode_bytes_per_step": db, "decode_gbs": round(val, 1), "decode_frac_hbm": round(val / HBM_PEAK_GBS, 4),
                "roofline": {"kernel": decode_kernel_name(spec), "bound": "hbm", "achieved": round(rw_gbs, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(rw_gbs / HBM_PEAK_GBS, 4)}})
    return res


def swap_beside_steps(dev, step, n_steps: int, stream, path: str = "engines"):
    """The step run n_steps times on the current stream, first alone and then
    while a swap-out (64 block columns: every layer's K and V block, 32 layers
    x 32 kv heads x 128 x bf16, 16 tokens a block; 512 MiB) runs repeatedly
    on a second stream of default priority, ordered after the inputs with an
    event.  path "engines": pa_swap_blocks (copy engines); "kernel":
    pa_copy_blocks (the copy kernel).  Reports the step time in both cases and
    the swap's bandwidth beside the steps and alone."""
    import numpy as np
    import torch
    import paged_kv_attention_reshape_amd as pa
    L, HKV, D, B = 32, 32, 128, 16
    nb, hb = 96, 64
    pools = torch.zeros((2 * L, nb, B, HKV, D), dtype=torch.bfloat16, device=dev)
    host = torch.empty((2 * L, hb, B, HKV, D), dtype=torch.bfloat16, pin_memory=True)
    g = np.random.default_rng(64)
    h_pairs = np.stack([g.choice(nb, 64, replace=False), np.arange(64)], 1).astype(np.int32)
    pairs = torch.from_numpy(h_pairs).to(dev)
    swap_bytes = 64 * 2 * L * B * HKV * D * 2
    side = torch.cuda.Stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def swap(s=None):
        if path == "engines":
            pa.swap_blocks(pools, host, h_pairs, stream=s)
        else:
            pa.copy_blocks(pools, host, pairs, stream=s)
    # swap alone (after two untimed ones)
    swap()
    swap()
    torch.cuda.synchronize()
    a0, a1 = ev(), ev()
    a0.record(stream)
    swap()
    a1.record(stream)
    torch.cuda.synchronize()
    swap_alone_ms = a0.elapsed_time(a1)
    # steps alone
    s0, s1 = ev(), ev()
    s0.record(stream)
    for _ in range(n_steps):
        step()
    s1.record(stream)
    torch.cuda.synchronize()
    alone_ms = s0.elapsed_time(s1) / n_steps
    reps = max(1, int(np.ceil(alone_ms * n_steps / swap_alone_ms)))
    # steps beside the swap
    ready = torch.cuda.Event()
    ready.record(stream)
    side.wait_event(ready)
    w0, w1 = ev(), ev()
    with torch.cuda.stream(side):
        w0.record(side)
        for _ in range(reps):
            swap(side)
        w1.record(side)
    b0, b1 = ev(), ev()
    b0.record(stream)
    for _ in range(n_steps):
        step()
    b1.record(stream)
    done = torch.cuda.Event()
    done.record(side)
    stream.wait_event(done)
    torch.cuda.synchronize()
    beside_ms = b0.elapsed_time(b1) / n_steps
    swap_ms = w0.elapsed_time(w1)
    del pools, host
    torch.cuda.empty_cache()
    return {"step_ms_alone": round(alone_ms, 4), "step_ms_beside_swap": round(beside_ms, 4),
            "step_slowdown": round(beside_ms / alone_ms, 4), "swap_bytes_each": swap_bytes, "swap_reps": reps,
            "swap_gbs_beside_steps": round(reps * swap_bytes / (swap_ms * 1e6), 1),
            "swap_gbs_alone": round(swap_bytes / (swap_alone_ms * 1e6), 1),
            "path": "pa_swap_blocks (copy engines, one 2-D copy per block column)" if path == "engines"
                    else "pa_copy_blocks (copy kernel, 64 workgroups)",
            "note": "swap-out of 64 block columns (512 MiB) repeated on a second default-priority stream, "
                    "event-ordered after the inputs, while the step runs on the current stream"}


def oracle_configs(dev, budget_s: float):
    """The fp64 oracle timed on the other configurations (bounded samples):
    C1 whole; every decode of C2 and of C4 (within budget_s each); a sample of
    the serving trace (the decode rows and one chunk of two planned steps, one
    layer).  Inputs are the generator's device-filled pools and rows copied to
    the host per request (C1, C2, C4), or host random values of the same
    shapes (C5 sample).  Returns per-configuration time and the metric's
    units."""
    import numpy as np
    import oracle
    from workloads import configs
    res = {}

    import torch
    for name in ("c1", "c2", "c4"):
        spec = configs.BUILDERS[name]()
        d = spec.device_inputs(device=dev)
        torch.cuda.synchronize()
        sec, n = 0.0, 0
        for r in range(spec.R):
            if sec > budget_s:
                break
            sec += oracle_request_seconds(spec, d, r)
            n += 1
        del d
        torch.cuda.empty_cache()
        done = np.zeros(spec.R, bool)
        done[:n] = True
        dec = (spec.query_lens == 1) & done
        L = spec.seq_lens[dec].astype(np.int64)
        dbytes = int(np.sum(L) * spec.Hkv * spec.D * 2 * spec.esize + 2 * dec.sum() * spec.Hq * spec.D * spec.esize
                     + 4 * np.sum(-(-L // spec.B)) + 12 * dec.sum())
        res[name] = {"sample": f"{n} of {spec.R} requests", "oracle_s": round(sec, 3),
                     "decode_gbs_equiv": round(dbytes / sec / 1e9, 4) if sec > 0 and dbytes else None}
        if name == "c1":
            res[name]["step_ms"] = round(sec * 1e3, 2)
    # serving-trace sample: two planned steps, one layer, every decode row and one chunk
    from workloads import serving_trace as st
    import paged_kv_attention_reshape_amd as pa
    cfg = st.TraceConfig()
    plans = st.drive(pa.Scheduler(**st.scheduler_args(cfg)), cfg)
    g = np.random.default_rng(9)
    HQ, HKV, D = 32, 8, 128
    sec, dbytes, flops, rows = 0.0, 0, 0, 0
    for p in (plans[45],):
        ql, cp, _, _, _ = st.step_arrays(p, cfg.block_size)
        idx = [i for i in range(len(ql)) if ql[i] == 1] + [i for i in range(len(ql)) if ql[i] > 1][:1]
        for i in idx:
            q, c = int(ql[i]), int(cp[i])
            L = q + c
            Q = g.standard_normal((q, HQ, D)).astype(np.float32)
            K = g.standard_normal((L, HKV, D)).astype(np.float32)
            V = g.standard_normal((L, HKV, D)).astype(np.float32)
            t0 = time.perf_counter()
            oracle.attention_rows(Q, K, V, c + np.arange(q), 1 / np.sqrt(D), "f32")
            sec += time.perf_counter() - t0
            rows += q
            if q == 1:
                dbytes += L * HKV * D * 2 * 2 + 2 * HQ * D * 2
            else:
                flops += 4 * D * HQ * (q * c + q * (q + 1) // 2)
    res["c5_sample"] = {"sample": f"step 45 of the serving trace, one layer: every decode row and the first "
                                  f"chunk ({rows} query rows)", "oracle_s": round(sec, 3),
                        "decode_gbs_equiv": round(dbytes / sec / 1e9, 4) if sec > 0 else None,
                        "chunk_flops": flops,
                        "note": "one (step, layer) sample of 200 steps x 32 layers; extrapolating this time to the "
                                "whole trace (x 6400) is an estimate, not a measurement"}
    return res


def load_traffic(kernel: str):
    """HBM traffic per launch measured by rocprofv3 counters (FETCH_SIZE,
    WRITE_SIZE), scaled by the copy-kernel calibration, if a summary exists for
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_c3_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        js = json.load(f)
    if js.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return js.get("traffic_bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the step shards by request or kv head with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.serving_only:
        import torch
        import paged_kv_attention_reshape_amd as pa
        torch.cuda.set_device(0)
        pa.lib()
        print(json.dumps({"serving_trace": serving_measurement(torch.device("cuda:0"))}), flush=True)
        return

    import numpy as np
    import torch

    import paged_kv_attention_reshape_amd as pa
    from workloads import configs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.lib()  # fail loudly if the HIP library is missing

    spec = configs.BUILDERS[args.workload]()
    d = spec.device_inputs(device=dev)
    torch.cuda.synchronize()

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(spec, d, args.cpu_seconds)
        if args.extra:
            cpu["configs"] = oracle_configs(dev, max(1.0, args.cpu_seconds / 4))

    # The 256 MB last-level (Infinity) cache must not serve a step's cache
    # reads from the previous step: when one layer's pools are small, steps
    # rotate over copies so that consecutive steps touch >= 1 GiB apart.
    pools = pool_rotation(d)
    n_copies = len(pools)
    torch.cuda.synchronize()

    qsl_h, sl_h = spec.query_start_loc, spec.seq_lens
    out = torch.empty_like(d["query"])
    slot_mapping = torch.empty((spec.T,), dtype=torch.int64, device=dev)
    ws = pa.alloc_workspace(pa.attention_workspace_size(qsl_h, sl_h, spec.Hq, spec.Hkv, spec.D, spec.B,
                                                        pa.PA_BF16 if spec.dtype == "bf16" else pa.PA_F32), dev)
    stream = torch.cuda.current_stream()

    step_no = [0]

    def step(events=None):
        kc, vc = pools[step_no[0] % n_copies]
        step_no[0] += 1
        if events is not None:
            events[0].record(stream)
        pa.compute_slot_mapping(slot_mapping, d["block_table"], d["query_start_loc"],
                                d["num_computed"], spec.num_blocks, spec.B)
        if events is not None:
            events[1].record(stream)
        pa.write_kv(d["key"], d["value"], kc, vc, slot_mapping)
        if events is not None:
            events[2].record(stream)
            pa.set_profiling_events(events[3:8])
        pa.attention(out, d["query"], kc, vc, d["block_table"],
                     d["query_start_loc"], d["seq_lens"], d["num_computed"], qsl_h, sl_h,
                     spec.scale, workspace=ws)
        if events is not None:
            pa.set_profiling_events(None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps back to back, no per-step instrumentation
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_begin.record(stream)
    for i in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_begin.elapsed_time(t_end)
    ms_step = total_ms / args.steps

    # the same step captured once in a HIP graph and replayed K times (the
    # library allocates, memsets and synchronises nothing, so a step of fixed
    # sizes captures whole); only when one pool copy is in use
    graph = None
    if n_copies == 1:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        for _ in range(2):
            g.replay()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        g0.record(stream)
        for _ in range(args.steps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph = {"ms_per_step": round(g0.elapsed_time(g1) / args.steps, 4),
                 "note": "the same step (slot mapping, write_kv, attention) captured once in a HIP graph "
                         "and replayed back to back"}

    # per-kernel breakdown: the same K steps again with events between the
    # launches (the events add a little time between kernels, not inside them)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()

    names = ["slot_mapping", "write_kv", "launch_gap", "plan", "rowwise", "chunk", "merge"]
    acc = {k: 0.0 for k in names}
    per_step = {k: [] for k in ("rowwise", "chunk", "merge", "step")}
    for e in ev:
        for k, (a, b) in zip(names, [(0, 1), (1, 2), (2, 3), (3, 4), (4, 5), (5, 6), (6, 7)]):
            t = e[a].elapsed_time(e[b])
            acc[k] += t
            if k in per_step:
                per_step[k].append(1e3 * t)
        per_step["step"].append(1e3 * e[0].elapsed_time(e[7]))
    us = {k: 1e3 * v / args.steps for k, v in acc.items()}
    us_pct = {k: [round(float(x), 2) for x in np.percentile(v, [10, 50, 90])]
              for k, v in per_step.items()}

    # fused rotary embedding + cache write on the same step's tokens (timed on
    # its own: Q rotated in place on a copy, K/V into the first pool copy)
    rope = None
    if args.rope:
        rd = spec.D
        cos_sin = torch.from_numpy(configs.rope_cache(int(spec.seq_lens.max()), rd)).to(dev)
        positions = torch.from_numpy(spec.positions()).to(dev)
        kc, vc = pools[0]
        # the step's Q/K/V (about 25 MB) would stay in the 256 MB last-level
        # cache across back-to-back calls: rotate over copies so consecutive
        # calls read >= 256 MB apart
        per_set = 3 * d["query"].numel() * d["query"].element_size()
        n_sets = max(2, min(64, -(-(256 << 20) // per_set) + 1))
        sets = [(d["query"].clone(), d["key"].clone(), d["value"].clone()) for _ in range(n_sets)]
        call_no = [0]

        def rope_call():
            q_i, k_i, v_i = sets[call_no[0] % n_sets]
            call_no[0] += 1
            pa.rope_write_kv(q_i, k_i, v_i, kc, vc, slot_mapping, positions, cos_sin, rd, True)

        for _ in range(args.warmup):
            rope_call()
        r0 = torch.cuda.Event(enable_timing=True)
        r1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        r0.record(stream)
        for _ in range(max(args.steps, 2 * n_sets)):
            rope_call()
        r1.record(stream)
        torch.cuda.synchronize()
        rope_us = 1e3 * r0.elapsed_time(r1) / max(args.steps, 2 * n_sets)
        rope_bytes = spec.rope_write_bytes(rd)
        rope_gbs = rope_bytes / (rope_us * 1e-6) / 1e9
        rope = {"kernel": "fused rotary embedding + cache write", "bound": "hbm",
                "tokens": spec.T, "rotary_dim": rd, "input_copies": n_sets, "us": round(rope_us, 2),
                "bytes_per_launch": rope_bytes, "achieved": round(rope_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(rope_gbs / HBM_PEAK_GBS, 4)}

    swap = swap_measurement(dev) if args.swap else None
    if swap is not None:
        swap["beside_step"] = swap_beside_steps(dev, step, args.steps, stream, "engines")
        swap["beside_step_copy_kernel"] = swap_beside_steps(dev, step, args.steps, stream, "kernel")
    serving = serving_measurement(dev) if args.serving else None
    extra = None
    if args.extra and args.workload == "c3":
        extra = {n: config_workload(n, dev, args.steps, args.warmup) for n in ("c1", "c2", "c4")}

    # host scheduler / block allocator (C++) on the serving trace
    sched_t = scheduler_timing(product=True)
    sched_t["trace"] = "2048 requests at step 0, 200 steps, 16384 blocks of 16, budget 8192, chunk 512"
    sched_t["includes"] = "pa_sched_schedule + pa_sched_plan_copy (block table rows at the step's own width) + pa_sched_commit, through ctypes"
    sched_t["shared_prefix"] = scheduler_timing(product=True, shared=True)

    dec_bytes = spec.decode_bytes()
    chunk_fl = spec.chunk_flops()
    dec_s = (us["rowwise"] + us["merge"]) * 1e-6
    value = dec_bytes / dec_s / 1e9 if dec_s > 0 else 0.0
    rw_gbs = dec_bytes / (us["rowwise"] * 1e-6) / 1e9 if us["rowwise"] > 0 else 0.0
    chunk_tf = chunk_fl / (us["chunk"] * 1e-6) / 1e12 if us["chunk"] > 0 and chunk_fl else 0.0
    traffic = load_traffic("rowwise")

    n_dec = int(np.sum(spec.query_lens == 1))
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {
            "workload": configs.WORKLOADS[args.workload],
            "requests": spec.R, "tokens": spec.T, "decode_rows": n_dec,
            "chunk_rows": int(spec.T - n_dec), "num_heads": spec.Hq, "num_kv_heads": spec.Hkv,
            "head_dim": spec.D, "block_size": spec.B, "num_blocks": spec.num_blocks,
            "seed": spec.seed, "pool_copies": n_copies,
        },
        "decode_frac_hbm": round(value / HBM_PEAK_GBS, 4),
        "chunk_tflops": round(chunk_tf, 2),
        "chunk_frac_mfma": round(chunk_tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "tokens_per_s": round(spec.T / (ms_step * 1e-3), 1),
        "kernel_us": {k: round(v, 2) for k, v in us.items()},
        "kernel_us_p10_p50_p90": us_pct,
        "decode_bytes_per_step": dec_bytes,
        "chunk_flops_per_step": chunk_fl,
        "write_kv_gbs": round(spec.write_bytes() / (us["write_kv"] * 1e-6) / 1e9, 1) if us["write_kv"] > 0 else None,
        "wall_s_timed": round(wall, 4),
        "roofline": {
            "kernel": decode_kernel_name(spec),
            "bound": "hbm",
            "achieved": round(rw_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(rw_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "chunk_roofline": {
            "kernel": "bf16 MFMA prefill chunk",
            "bound": "mfma",
            "achieved": round(chunk_tf, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(chunk_tf / MFMA_BF16_PEAK_TFLOPS, 4),
        },
        "graph_replay": graph,
        "rope_write_kv": rope,
        "scheduler": sched_t,
        "swap_roundtrip": swap,
        "serving_trace": serving,
        "other_configs": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
