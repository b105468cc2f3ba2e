"""Seeded synthetic steps for the five workloads (shapes and distributions of
the pages' setting: Llama-3-8B attention heads, block size 16/32, mixed decode
and 512-token prefill chunks).

Each StepSpec holds only what a caller of the attention step would hold before
the step: per-request query lengths and computed-token counts, the block table
(physical blocks scattered over a pool by a seeded permutation), the pool
geometry and the keys of the counter-based value streams.  Flat slot indices
are NOT produced here: deriving them is part of the method, done by the library
under test and, separately, by the oracle.

Value streams (see workloads/rng.py):
  query rows      key(seed, TAG_Q, layer)      row = flattened token index
  new K / V rows  key(seed, TAG_K|TAG_V, layer)
  pool slots      key(seed, TAG_POOL_K|V, layer), row = block * B + offset;
                  slots past a request's retained history (positions >=
                  num_computed) and all unused blocks hold NaN.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from . import rng

WORKLOADS = {
    "c1": "tiny mixed step, fp32: 4 requests [37,81,130,211], 2 decodes, a 32-token chunk, a 211-token prefill; Hq 8, Hkv 2, D 64, B 16",
    "c2": "pure decode, bf16: 64 requests, context U[512,4096]; Hq 32, Hkv 8, D 128, B 16",
    "c3": "mixed chunked-prefill step, bf16: 3 chunks of 512 (16384-token prompts, offsets multiple of 512) + 512 decodes (lognormal median 2048, [128,16384]); Hq 32, Hkv 8, D 128, B 16",
    "c4": "long-context decode, bf16: 16 x 32768 + 240 lognormal (median 1024); Hq 64, Hkv 8, D 128, B 32",
}


@dataclass
class StepSpec:
    name: str
    dtype: str
    Hq: int
    Hkv: int
    D: int
    B: int
    num_blocks: int
    scale: float
    query_lens: np.ndarray
    num_computed: np.ndarray
    block_table: np.ndarray
    seed: int
    layer: int = 0
    pool_valid: Optional[np.ndarray] = None
    q_row_keys: Optional[np.ndarray] = None
    k_row_keys: Optional[np.ndarray] = None
    v_row_keys: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    # ---- derived host metadata -------------------------------------------
    @property
    def R(self) -> int:
        return int(len(self.query_lens))

    @property
    def T(self) -> int:
        return int(np.sum(self.query_lens))

    @property
    def seq_lens(self) -> np.ndarray:
        return (self.query_lens + self.num_computed).astype(np.int32)

    @property
    def query_start_loc(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.query_lens)]).astype(np.int32)

    @property
    def M(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def esize(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def key(self, tag: int) -> int:
        return rng.key(self.seed, tag, self.layer)

    def row_keys(self, which: str, rows=None) -> np.ndarray:
        explicit = {"q": self.q_row_keys, "k": self.k_row_keys, "v": self.v_row_keys}[which]
        if rows is None:
            rows = np.arange(self.T)
        rows = np.asarray(rows, dtype=np.int64)
        if explicit is not None:
            return np.asarray(explicit, dtype=np.uint64)[rows]
        tag = {"q": rng.TAG_Q, "k": rng.TAG_K, "v": rng.TAG_V}[which]
        return rng.base_row_keys(self.key(tag), rows)

    # ---- host mirror of the generated values --------------------------------
    def host_rows(self, which: str, rows) -> np.ndarray:
        """Storage values of query ('q') or new key/value ('k'/'v') rows."""
        width = (self.Hq if which == "q" else self.Hkv) * self.D
        vals = rng.row_values(self.row_keys(which, rows), width, self.dtype)
        heads = self.Hq if which == "q" else self.Hkv
        return vals.reshape(len(vals), heads, self.D)

    def host_pool_blocks(self, which: str, block_ids) -> np.ndarray:
        """Storage values of whole pool blocks before the step's write
        ([n, B, Hkv, D]); which is 'k' or 'v'."""
        block_ids = np.asarray(block_ids, dtype=np.int64)
        tag = rng.TAG_POOL_K if which == "k" else rng.TAG_POOL_V
        rows = (block_ids[:, None] * self.B + np.arange(self.B)[None, :]).reshape(-1)
        vals = rng.row_values(rng.base_row_keys(self.key(tag), rows), self.Hkv * self.D, self.dtype)
        vals = vals.reshape(len(block_ids), self.B, self.Hkv, self.D)
        valid = self.pool_valid if self.pool_valid is not None else np.zeros(self.num_blocks, np.int32)
        off = np.arange(self.B)[None, :]
        bad = off >= valid[block_ids][:, None]
        vals[bad] = rng.storage_nan(self.dtype)
        return vals

    # ---- device materialisation ---------------------------------------------
    def device_inputs(self, device="cuda", pools=True):
        """Allocate and fill the step's device tensors.  Returns a dict of torch
        tensors: query, key, value ([T, H, D]), key_cache, value_cache
        ([N, B, Hkv, D]), block_table, query_start_loc, seq_lens, num_computed
        (int32)."""
        import torch
        from . import _lib
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        out = {}
        T = self.T
        for which, H in (("q", self.Hq), ("k", self.Hkv), ("v", self.Hkv)):
            t = torch.empty((max(T, 1), H, self.D), dtype=tdt, device=device)[:T]
            if T:
                rk = torch.from_numpy(self.row_keys(which).view(np.int64)).to(device)
                _lib.fill_rows(t, self.dtype, row_keys=rk)
            out[{"q": "query", "k": "key", "v": "value"}[which]] = t
        if pools:
            valid = self.pool_valid if self.pool_valid is not None else np.zeros(self.num_blocks, np.int32)
            vd = torch.from_numpy(valid.astype(np.int32)).to(device)
            for which, tag in (("key_cache", rng.TAG_POOL_K), ("value_cache", rng.TAG_POOL_V)):
                t = torch.empty((self.num_blocks, self.B, self.Hkv, self.D), dtype=tdt, device=device)
                _lib.fill_pool(t, self.dtype, self.key(tag), vd, self.B)
                out[which] = t
        out["block_table"] = torch.from_numpy(np.ascontiguousarray(self.block_table, dtype=np.int32)).to(device)
        out["query_start_loc"] = torch.from_numpy(self.query_start_loc).to(device)
        out["seq_lens"] = torch.from_numpy(self.seq_lens).to(device)
        out["num_computed"] = torch.from_numpy(self.num_computed.astype(np.int32)).to(device)
        return out

    # ---- algorithmic work (for the roofline) ---------------------------------
    def decode_kv_bytes(self) -> int:
        """K and V bytes the decode rows must read once: sum over single-token
        requests of seq_len * Hkv * D * 2 * e."""
        L = self.seq_lens[self.query_lens == 1].astype(np.int64)
        return int(L.sum()) * self.Hkv * self.D * 2 * self.esize

    def decode_bytes(self) -> int:
        """Decode algorithmic bytes: K/V once per kv head, plus the query and
        output rows, the block-table entries and per-request metadata."""
        dec = self.query_lens == 1
        L = self.seq_lens[dec].astype(np.int64)
        n = int(dec.sum())
        return (self.decode_kv_bytes() + 2 * n * self.Hq * self.D * self.esize
                + 4 * int(np.sum(-(-L // self.B))) + 12 * n)

    def chunk_flops(self) -> int:
        """Causally visible (query, key) pairs of multi-token requests times
        4 * D * Hq (2 D for q.k, 2 D for p.v)."""
        tot = 0
        for q, c in zip(self.query_lens, self.num_computed):
            q, c = int(q), int(c)
            if q > 1:
                pairs = q * c + q * (q + 1) // 2
                tot += 4 * self.D * self.Hq * pairs
        return tot

    def positions(self) -> np.ndarray:
        """Absolute position of every scheduled token, flattened order
        (num_computed[r] + i): the rows the rotary table is indexed by."""
        return np.concatenate([np.arange(c, c + q, dtype=np.int64)
                               for q, c in zip(self.query_lens, self.num_computed)]
                              + [np.zeros(0, np.int64)])

    def rope_write_bytes(self, rotary_dim: int) -> int:
        """Bytes the fused rotary + cache write must move: Q read and written
        back, K and V read and written to the cache, one cos/sin row (fp32)
        and a slot and a position per token."""
        e = self.esize
        return (2 * self.T * self.D * e * (self.Hq + 2 * self.Hkv)
                + self.T * rotary_dim * 4 + 16 * self.T)

    def write_bytes(self) -> int:
        return 4 * self.T * self.Hkv * self.D * self.esize + 8 * self.T


# ----------------------------------------------------------------------------
# rotary table (model configuration, prepared once like the weights)
# ----------------------------------------------------------------------------
LLAMA3_ROPE_BASE = 500000.0


def rope_cache(max_position: int, rotary_dim: int, base: float = LLAMA3_ROPE_BASE) -> np.ndarray:
    """float32 [max_position, rotary_dim]: row p holds cos(p * f_i) for the
    rotary_dim/2 frequencies f_i = base^(-2i/rotary_dim), then sin(p * f_i).
    Computed in float64 and rounded once to float32."""
    inv = base ** (-np.arange(0, rotary_dim, 2, dtype=np.float64) / rotary_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


# ----------------------------------------------------------------------------
# builders
# ----------------------------------------------------------------------------
def _scatter_blocks(gen, seq_lens, B, pool_factor=1.25, num_blocks=None):
    need = [-(-int(L) // B) for L in seq_lens]
    total = int(sum(need))
    nb = num_blocks if num_blocks is not None else int(math.ceil(pool_factor * total))
    perm = gen.permutation(nb).astype(np.int32)
    M = max(need) if need else 1
    bt = np.full((len(seq_lens), max(M, 1)), -1, dtype=np.int32)
    pos = 0
    for r, n in enumerate(need):
        bt[r, :n] = perm[pos:pos + n]
        pos += n
    return bt, nb


def _history_valid(bt, num_computed, B, nb):
    """Slots holding retained history before the step: positions < c_r."""
    valid = np.zeros(nb, dtype=np.int32)
    for r, c in enumerate(num_computed):
        c = int(c)
        nfull = -(-c // B)
        for j in range(nfull):
            valid[bt[r, j]] = min(B, c - j * B)
    return valid


def _finish(name, dtype, Hq, Hkv, D, B, qlens, comp, gen, seed, pool_factor=1.25,
            num_blocks=None, order=None):
    qlens = np.asarray(qlens, dtype=np.int32)
    comp = np.asarray(comp, dtype=np.int32)
    if order is not None:
        qlens, comp = qlens[order], comp[order]
    seq = qlens + comp
    bt, nb = _scatter_blocks(gen, seq, B, pool_factor, num_blocks)
    valid = _history_valid(bt, comp, B, nb)
    return StepSpec(name=name, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, B=B, num_blocks=nb,
                    scale=1.0 / math.sqrt(D), query_lens=qlens, num_computed=comp,
                    block_table=bt, seed=seed, pool_valid=valid)


def c1() -> StepSpec:
    """Tiny mixed step (fp32): req0/req1 decode one token, req2 a 32-token chunk
    at positions 98..129, req3 a full 211-token prefill; 64-block pool whose
    block tables are consecutive slices of a seeded permutation."""
    gen = np.random.default_rng(1)
    lens = [37, 81, 130, 211]
    qlens = [1, 1, 32, 211]
    comp = [L - q for L, q in zip(lens, qlens)]
    return _finish("c1", "f32", 8, 2, 64, 16, qlens, comp, gen, 1, num_blocks=64)


def c2(R: int = 64) -> StepSpec:
    gen = np.random.default_rng(2)
    L = gen.integers(512, 4097, size=R)
    return _finish("c2", "bf16", 32, 8, 128, 16, np.ones(R, np.int32), L - 1, gen, 2)


def c3(n_decode: int = 512, n_chunks: int = 3, chunk: int = 512, prompt: int = 16384) -> StepSpec:
    gen = np.random.default_rng(3)
    offs = chunk * gen.choice(prompt // chunk, size=n_chunks, replace=False)
    Ld = np.rint(np.clip(gen.lognormal(mean=math.log(2048), sigma=1.0, size=n_decode),
                         128, 16384)).astype(np.int64)
    qlens = [chunk] * n_chunks + [1] * n_decode
    comp = [int(o) for o in offs] + [int(x) - 1 for x in Ld]
    order = gen.permutation(n_chunks + n_decode)
    return _finish("c3", "bf16", 32, 8, 128, 16, qlens, comp, gen, 3, order=order)


def c4(n_long: int = 16, n_short: int = 240) -> StepSpec:
    gen = np.random.default_rng(4)
    Ls = np.rint(np.clip(gen.lognormal(mean=math.log(1024), sigma=1.0, size=n_short),
                         16, 32768)).astype(np.int64)
    L = np.concatenate([np.full(n_long, 32768, np.int64), Ls])
    order = gen.permutation(len(L))
    return _finish("c4", "bf16", 64, 8, 128, 32, np.ones(len(L), np.int32), L - 1, gen, 4,
                   order=order)


def custom(name, dtype, Hq, Hkv, D, B, qlens, comp, seed, pool_factor=1.25, num_blocks=None) -> StepSpec:
    """A small step of any shape (for edge-case tests)."""
    gen = np.random.default_rng(seed)
    return _finish(name, dtype, Hq, Hkv, D, B, qlens, comp, gen, seed, pool_factor, num_blocks)


BUILDERS = {"c1": c1, "c2": c2, "c3": c3, "c4": c4}
