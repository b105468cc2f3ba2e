"""Thin ctypes binding of libpa_sched.so (include/pa_sched.h): the host
scheduler and block allocator that produce the attention step's query
lengths, computed counts and block tables.  Argument marshalling only; raises
if the library is not built."""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Sequence

import numpy as np

from ._lib import STATUS, PAError

_HERE = os.path.dirname(os.path.abspath(__file__))
SCHED_LIB_PATH = os.path.join(_HERE, "libpa_sched.so")

SCHED_EXPORTS = [
    "pa_sched_create", "pa_sched_destroy", "pa_sched_add_request", "pa_sched_fork", "pa_sched_schedule",
    "pa_sched_plan_copy", "pa_sched_commit", "pa_sched_rollback", "pa_sched_cancel",
    "pa_sched_get_metrics", "pa_sched_last_error",
]


class _Config(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_num_seqs", ctypes.c_int32), ("max_num_batched_tokens", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("block_order", ctypes.POINTER(ctypes.c_int32)),
                ("hook_prob", ctypes.c_double), ("hook_max", ctypes.c_int32),
                ("hook_draws", ctypes.POINTER(ctypes.c_double)), ("n_hook_draws", ctypes.c_int32)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [("num_reqs", ctypes.c_int32), ("num_preempted", ctypes.c_int32),
                ("num_copies", ctypes.c_int32), ("num_tokens", ctypes.c_int64), ("max_blocks", ctypes.c_int32),
                ("q_free", ctypes.c_int32), ("q_reserved", ctypes.c_int32),
                ("q_committed", ctypes.c_int32)]


_METRIC_FIELDS = ["q_free", "q_reserved", "q_committed", "q_capacity", "q_live", "tail_waste",
                  "peak_used", "allocation_failures", "steps", "rollbacks", "admissions",
                  "preemptions", "recompute_tokens", "finished", "cancelled", "scheduled_tokens",
                  "running", "waiting", "prefix_hit_tokens", "evictions", "cow_copies",
                  "cached_blocks", "evictable"]


class _Metrics(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in _METRIC_FIELDS]


_lib = None


def sched_lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(SCHED_LIB_PATH):
        raise RuntimeError(f"{SCHED_LIB_PATH} is missing: build it with "
                           "`python -m paged_kv_attention_reshape_amd.build`")
    L = ctypes.CDLL(SCHED_LIB_PATH)
    vp = ctypes.c_void_p
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    L.pa_sched_last_error.restype = ctypes.c_char_p
    L.pa_sched_create.restype = ctypes.c_int
    L.pa_sched_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(vp)]
    L.pa_sched_destroy.restype = None
    L.pa_sched_destroy.argtypes = [vp]
    L.pa_sched_add_request.restype = ctypes.c_int
    L.pa_sched_add_request.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(ctypes.c_uint64), ctypes.c_int32]
    L.pa_sched_fork.restype = ctypes.c_int
    L.pa_sched_fork.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
    L.pa_sched_schedule.restype = ctypes.c_int
    L.pa_sched_schedule.argtypes = [vp, ctypes.POINTER(_PlanInfo)]
    L.pa_sched_plan_copy.restype = ctypes.c_int
    L.pa_sched_plan_copy.argtypes = [vp, i64p, i32p, i32p, ctypes.c_int32, i32p, ctypes.c_int32,
                                     i64p, ctypes.c_int32, i32p, ctypes.c_int32]
    L.pa_sched_commit.restype = ctypes.c_int
    L.pa_sched_commit.argtypes = [vp, i64p, ctypes.c_int32, i32p]
    L.pa_sched_rollback.restype = ctypes.c_int
    L.pa_sched_rollback.argtypes = [vp]
    L.pa_sched_cancel.restype = ctypes.c_int
    L.pa_sched_cancel.argtypes = [vp, ctypes.c_int64]
    L.pa_sched_get_metrics.restype = ctypes.c_int
    L.pa_sched_get_metrics.argtypes = [vp, ctypes.POINTER(_Metrics)]
    _lib = L
    return L


def _check(rc: int, where: str):
    if rc != 0:
        raise PAError(rc, where, sched_lib().pa_sched_last_error().decode())


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Scheduler:
    """Owns one pa_sched object; see include/pa_sched.h for the behaviour."""

    def __init__(self, num_blocks: int, block_size: int, max_num_seqs: int,
                 max_num_batched_tokens: int, chunk: int, block_order: Sequence[int],
                 hook_prob: float = 0.0, hook_max: int = 0, hook_draws: Sequence[float] = ()):
        L = sched_lib()
        self._order = np.ascontiguousarray(block_order, dtype=np.int32)
        self._draws = np.ascontiguousarray(hook_draws, dtype=np.float64)
        cfg = _Config(num_blocks, block_size, max_num_seqs, max_num_batched_tokens, chunk,
                      _ptr(self._order, ctypes.c_int32), float(hook_prob), int(hook_max),
                      _ptr(self._draws, ctypes.c_double) if len(self._draws) else None,
                      len(self._draws))
        h = ctypes.c_void_p()
        _check(L.pa_sched_create(ctypes.byref(cfg), ctypes.byref(h)), "pa_sched_create")
        self._h = h
        self.B = block_size

    def close(self):
        if getattr(self, "_h", None):
            sched_lib().pa_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add_request(self, rid: int, prompt_len: int, output_len: int, keys: Sequence[int] = ()) -> None:
        k = np.ascontiguousarray(np.asarray(keys, dtype=np.uint64))
        _check(sched_lib().pa_sched_add_request(self._h, rid, prompt_len, output_len,
                                                _ptr(k, ctypes.c_uint64) if len(k) else None, len(k)),
               "pa_sched_add_request")

    def fork(self, parent: int, child: int, output_len: int) -> None:
        _check(sched_lib().pa_sched_fork(self._h, parent, child, output_len), "pa_sched_fork")

    def schedule_arrays(self):
        """Plan a step; return (info, request_ids, num_computed, query_lens,
        block_table [R, M] -1 padded, preempted [P, 3], copies [C, 2])."""
        L = sched_lib()
        info = _PlanInfo()
        _check(L.pa_sched_schedule(self._h, ctypes.byref(info)), "pa_sched_schedule")
        R, P, C, M = info.num_reqs, info.num_preempted, info.num_copies, max(info.max_blocks, 1)
        ids = np.zeros(R, np.int64)
        comp = np.zeros(R, np.int32)
        ql = np.zeros(R, np.int32)
        bt = np.full((R, M), -1, np.int32)
        pre = np.zeros((P, 3), np.int64)
        cp = np.zeros((C, 2), np.int32)
        _check(L.pa_sched_plan_copy(self._h, _ptr(ids, ctypes.c_int64), _ptr(comp, ctypes.c_int32),
                                    _ptr(ql, ctypes.c_int32), R, _ptr(bt, ctypes.c_int32), M,
                                    _ptr(pre, ctypes.c_int64) if P else None, P,
                                    _ptr(cp, ctypes.c_int32) if C else None, C),
               "pa_sched_plan_copy")
        return info, ids, comp, ql, bt, pre, cp

    def schedule(self) -> dict:
        """The pending plan in the reference scheduler's format."""
        info, ids, comp, ql, bt, pre, cp = self.schedule_arrays()
        sched = [(int(i), int(c), int(n)) for i, c, n in zip(ids, comp, ql)]
        blocks = {int(i): row[row >= 0].tolist() for i, row in zip(ids, bt)}
        return {"sched": sched, "blocks": blocks,
                "preempted": [(int(a), int(b), int(c)) for a, b, c in pre],
                "copies": [(int(a), int(b)) for a, b in cp],
                "q_free": info.q_free, "q_reserved": info.q_reserved,
                "q_committed": info.q_committed}

    def commit(self) -> List[int]:
        cap = 4096
        buf = np.zeros(cap, np.int64)
        n = ctypes.c_int32()
        _check(sched_lib().pa_sched_commit(self._h, _ptr(buf, ctypes.c_int64), cap, ctypes.byref(n)),
               "pa_sched_commit")
        return [int(x) for x in buf[:n.value]]

    def rollback(self) -> None:
        _check(sched_lib().pa_sched_rollback(self._h), "pa_sched_rollback")

    def cancel(self, rid: int) -> None:
        _check(sched_lib().pa_sched_cancel(self._h, rid), "pa_sched_cancel")

    def metrics(self) -> Dict[str, int]:
        m = _Metrics()
        _check(sched_lib().pa_sched_get_metrics(self._h, ctypes.byref(m)), "pa_sched_get_metrics")
        return {f: int(getattr(m, f)) for f in _METRIC_FIELDS}
