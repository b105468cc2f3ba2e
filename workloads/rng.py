"""Counter-based input values shared by the tests, the benchmark and the smoke
check (host mirror of workloads/csrc/wl_fill.hip).

Definition (both sides implement exactly this):

* mix64 is the SplitMix64 output function (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014; the finaliser
  constants are the ones java.util.SplittableRandom publishes):
      z ^= z >> 30; z *= 0xBF58476D1CE4E5B9
      z ^= z >> 27; z *= 0x94D049BB133111EB
      z ^= z >> 31
  with 64-bit wrap-around arithmetic.
* derive(k, n) = mix64(k + (n + 1) * GAMMA), GAMMA = 0x9E3779B97F4A7C15.
* A key is derive() folded over a tuple of non-negative integers, starting
  from mix64(seed).
* Element e of a row whose key is k draws u = derive(k, e) and maps it to an
  approximately standard normal value with the Irwin-Hall sum of its four
  16-bit lanes: S = sum(lanes) - 131070 (an exact integer), then
  x = float32(S) * NORM_SCALE in float32 (one correctly rounded multiply),
  where NORM_SCALE = float32(1 / sqrt((65536^2 - 1) / 3)) makes the variance 1.
* bf16 storage rounds x to nearest-even on the float32 bit pattern.
* Slots marked invalid hold a quiet NaN (bf16 0x7FC0, float32 0x7FC00000),
  so a stray read surfaces as NaN.

Everything is integer arithmetic plus one IEEE float32 multiply, so host and
device agree bit for bit.  This module holds none of the method's arithmetic.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
NORM_SCALE = np.float32(1.0 / np.sqrt((65536.0 ** 2 - 1.0) / 3.0))
BF16_NAN = np.uint16(0x7FC0)
F32_NAN_BITS = np.uint32(0x7FC00000)

# stream tags (first field of every key)
TAG_POOL_K = 1
TAG_POOL_V = 2
TAG_Q = 3
TAG_K = 4
TAG_V = 5


def mix64(z):
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = z ^ (z >> np.uint64(30))
        z = z * _M1
        z = z ^ (z >> np.uint64(27))
        z = z * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def derive(k, n):
    k = np.asarray(k, dtype=np.uint64)
    n = np.asarray(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(k + (n + np.uint64(1)) * GAMMA)


def key(seed: int, *fields: int) -> int:
    k = mix64(np.uint64(seed))
    for f in fields:
        k = derive(k, np.uint64(f))
    return int(k)


def normal_f32(u: np.ndarray) -> np.ndarray:
    u = np.asarray(u, dtype=np.uint64)
    m = np.uint64(0xFFFF)
    s = ((u & m) + ((u >> np.uint64(16)) & m) + ((u >> np.uint64(32)) & m)
         + (u >> np.uint64(48))).astype(np.int64) - 131070
    return s.astype(np.float32) * NORM_SCALE


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = b + np.uint32(0x7FFF) + lsb
    return (r >> np.uint32(16)).astype(np.uint16)


def row_values(row_keys: np.ndarray, row_len: int, dtype: str) -> np.ndarray:
    """[n, row_len] storage array: element e of row i is derived from
    row_keys[i] and e.  dtype 'bf16' returns uint16 bit patterns, 'f32'
    returns float32."""
    rk = np.asarray(row_keys, dtype=np.uint64).reshape(-1, 1)
    e = np.arange(row_len, dtype=np.uint64)[None, :]
    x = normal_f32(derive(rk, e))
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def base_row_keys(base_key: int, rows: np.ndarray) -> np.ndarray:
    """Row keys of a tensor generated from a single base key: row r -> derive(base, r)."""
    return derive(np.uint64(base_key), np.asarray(rows, dtype=np.uint64))


def storage_nan(dtype: str):
    return BF16_NAN if dtype == "bf16" else F32_NAN_BITS.view(np.float32)
