"""ctypes loader for the device half of the input generator (libpa_workloads.so)."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import rng

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa_workloads.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.wl_fill_rows.restype = ctypes.c_int
        L.wl_fill_rows.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int32, ctypes.c_float, ctypes.c_void_p]
        _lib = L
    return _lib


def fill_rows(t, dtype: str, base_key: int = 0, row_keys=None, valid=None,
              rows_per_group: int = 1, stream=None):
    """Fill a contiguous device tensor viewed as [n_rows, row_len] where row_len
    is its last dimension times the product of all dims after the first.
    t: torch tensor (float32 or a uint16/int16/bfloat16 tensor for bf16)."""
    import torch
    assert t.is_cuda and t.is_contiguous()
    n_rows = t.shape[0] if t.dim() > 0 else 1
    row_len = t.numel() // max(n_rows, 1)
    if rows_per_group > 1 and valid is None:
        raise ValueError("rows_per_group needs valid")
    # pool tensors [N, B, Hkv, D] are filled with rows = N * B
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    rk = 0 if row_keys is None else row_keys.data_ptr()
    vp = 0 if valid is None else valid.data_ptr()
    rc = lib().wl_fill_rows(ctypes.c_void_p(t.data_ptr()), 1 if dtype == "bf16" else 0,
                            n_rows, row_len, ctypes.c_uint64(base_key), ctypes.c_void_p(rk),
                            ctypes.c_void_p(vp), rows_per_group, float(rng.NORM_SCALE),
                            ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"wl_fill_rows failed with code {rc}")


def fill_pool(t, dtype: str, base_key: int, valid_per_block, block_size: int):
    """Fill a cache pool [num_blocks, B, Hkv, D]: one generator row per slot
    (row = block * B + offset); slots at offsets >= valid_per_block[block] are
    NaN."""
    nb = t.shape[0]
    view = t.view(nb * block_size, -1)
    fill_rows(view, dtype, base_key=base_key, valid=valid_per_block, rows_per_group=block_size)


def host_rows(row_keys: np.ndarray, row_len: int, dtype: str) -> np.ndarray:
    return rng.row_values(row_keys, row_len, dtype)
