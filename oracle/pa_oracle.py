"""Plain CPU oracle for the paged-KV attention step (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the build entry
point and the CPU-baseline leg of the benchmark use it.  It shares no code with
the HIP library and imports nothing from it.

What it computes, and where the pages define it
-----------------------------------------------
* slot_mapping      -- "AI Infra入门干货总结：大模型是如何高效推理的", section
                       "Paged Attention": a token at absolute position p of a
                       request lives in logical block p // B, which the request's
                       block table maps to a physical block; the flat slot is
                       physical_block * B + p % B.
* write_kv          -- same page, "Paged Attention" and "Attention Module": the
                       new tokens' K/V are scattered into the per-layer cache
                       [num_blocks, block_size, num_kv_heads, head_dim] at the
                       slot the slot mapping names; block = slot // B,
                       offset = slot % B.  The copy is done on the raw storage
                       bits (bf16 as uint16), so it is exact.
* gather_kv         -- same page, "Attention Module": the kernel follows the
                       block table to assemble each request's history as a
                       logically contiguous [seq_len, num_kv_heads, head_dim]
                       sequence; "显存与调度" (ch. 32), section
                       "块表消除连续内存要求", gives the map pi_i from logical to
                       physical block.
* attention         -- softmax(scale * q k^T + M) v with the causal mask of
                       "Chunked Prefill 与 Preemption", section "Chunked
                       Prefill：改变调度粒度，不改变 causal 结果" (equation
                       M_{i,j}: 0 when key position j <= query position i,
                       -inf otherwise), taken at absolute positions: the query
                       row i of a request with num_computed_tokens c sits at
                       position c + i and sees keys 0 .. c + i.  Query heads
                       map to kv heads in contiguous groups (standard GQA,
                       "Attention Module (以标准GQA + RoPE为例)").  The method
                       (FlashAttention with online softmax) reaches this plain
                       definition exactly up to rounding order, so the oracle
                       is the definition itself, in fp64.
* chunked_causal    -- the same page's "可运行等价性与成本核算": a prompt processed
                       chunk by chunk with a growing cache; concatenated chunk
                       outputs equal the one-shot causal prefill.
* block_accounting  -- "显存与调度", section "从保留词元到物理块": q_i = ceil(T_i/B),
                       allocated slots q_i * B, tail waste w_i = q_i*B - T_i.
* preemption_accounting -- "Chunked Prefill 与 Preemption", section
                       "可运行等价性与成本核算": blocks released, tokens recomputed
                       and the swap round-trip bound 2 * payload / bandwidth.
* kv_bytes_per_token -- "显存与调度", equation kappa = 2 L n_kv d_head b_kv.
* rope              -- "AI Infra入门干货总结…", section "Attention Module
                       (以标准GQA + RoPE为例)": Q and K of a token are multiplied
                       by a block-diagonal rotation matrix whose angles come
                       from the row of a precomputed cos_sin_cache
                       [max_position, rotary_dim] selected by the token's
                       position; the kernel realises it elementwise with
                       sin/cos, the oracle builds the matrix and multiplies.
* rope_write_kv     -- same section, step order: rotate Q and K, then scatter
                       the rotated K (and V) into the paged cache by slot.

Every function here is pinned by tests against values and properties the pages
and the mathematics fix (worked examples, closed forms, brute force,
library special cases); see tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "as_f64",
    "slot_mapping",
    "write_kv",
    "gather_kv",
    "attention",
    "attention_rows",
    "dense_causal",
    "chunked_causal",
    "block_accounting",
    "preemption_accounting",
    "kv_bytes_per_token",
    "rope_matrix",
    "rope",
    "rope_write_kv",
]


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 storage (uint16 bit patterns) -> float64.

    bfloat16 is the upper half of an IEEE-754 binary32 word, so widening is a
    16-bit left shift of the pattern followed by an exact float32->float64
    conversion.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64.  dtype is 'f32' (float32 storage) or 'bf16'
    (uint16 bit patterns)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# step metadata: slot mapping
# ----------------------------------------------------------------------------
def slot_mapping(block_table: np.ndarray, query_lens: Sequence[int],
                 num_computed: Sequence[int], block_size: int) -> np.ndarray:
    """Flat cache slot of every scheduled token, in flattened batch order.

    Request r contributes query_lens[r] tokens at absolute positions
    num_computed[r] + i (i < query_lens[r]).  Position p maps to logical block
    p // B, physical block block_table[r, p // B], offset p % B, and slot
    physical * B + offset ("Paged Attention", worked example: block table
    [5, 8, 12], position 25, B = 16 -> slot 137).
    """
    bt = np.asarray(block_table, dtype=np.int64)
    out: List[int] = []
    for r, (q, c) in enumerate(zip(query_lens, num_computed)):
        for i in range(int(q)):
            p = int(c) + i
            logical = p // block_size
            phys = int(bt[r, logical])
            out.append(phys * block_size + p % block_size)
    return np.asarray(out, dtype=np.int64)


# ----------------------------------------------------------------------------
# write: scatter new K/V into the paged cache
# ----------------------------------------------------------------------------
def write_kv(key_cache: np.ndarray, value_cache: np.ndarray,
             key: np.ndarray, value: np.ndarray,
             slots: np.ndarray, block_size: int) -> None:
    """In place: cache[slot // B, slot % B] = new row, for every token whose
    slot is non-negative (a negative slot marks a token that writes nothing).

    Arrays keep their storage dtype, so the copy is bit-exact.  Two tokens
    naming the same slot is an invalid step; the oracle refuses it.
    """
    slots = np.asarray(slots, dtype=np.int64)
    live = slots[slots >= 0]
    if len(np.unique(live)) != len(live):
        raise ValueError("duplicate slot in one write")
    nb = key_cache.shape[0]
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        if blk >= nb:
            raise IndexError(f"slot {s} beyond the pool")
        key_cache[blk, off] = key[t]
        value_cache[blk, off] = value[t]


# ----------------------------------------------------------------------------
# gather: logical K/V sequence of one request
# ----------------------------------------------------------------------------
def gather_kv(cache: np.ndarray, block_table_row: np.ndarray,
              seq_len: int, block_size: int) -> np.ndarray:
    """[seq_len, num_kv_heads, head_dim] view of one request's history, in
    storage dtype: concatenate the physical blocks the block table lists, in
    logical order, and keep the first seq_len positions."""
    nblk = -(-int(seq_len) // block_size)
    ids = np.asarray(block_table_row[:nblk], dtype=np.int64)
    blocks = cache[ids]                                   # [nblk, B, Hkv, D]
    flat = blocks.reshape((nblk * block_size,) + cache.shape[2:])
    return flat[:seq_len]


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def _softmax_attend(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    qpos: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One request, one query head: q [n, D], k/v [L, D] (fp64); query row i is
    at absolute position qpos[i] and sees keys j <= qpos[i].
    Returns (out [n, D], lse [n]) with lse = max + log(sum exp)."""
    s = (q @ k.T) * scale                                 # [n, L]
    j = np.arange(k.shape[0])[None, :]
    s = np.where(j <= qpos[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ v) / l
    return out, (m + np.log(l))[:, 0]


def attention(query: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
              block_table: np.ndarray, query_start_loc: Sequence[int],
              seq_lens: Sequence[int], num_computed: Sequence[int],
              scale: float, block_size: int, dtype: str,
              requests: Sequence[int] | None = None):
    """GQA attention for a flattened, padding-free batch, reading history
    through the block table.

    query      [T, Hq, D] storage dtype
    key_cache, value_cache [num_blocks, B, Hkv, D] storage dtype
    returns (out [T, Hq, D] fp64, lse [T, Hq] fp64); rows of requests not
    listed in `requests` (when given) are left NaN.
    """
    T, Hq, D = query.shape
    Hkv = key_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    R = len(seq_lens)
    reqs = range(R) if requests is None else requests
    for r in reqs:
        a, b = int(query_start_loc[r]), int(query_start_loc[r + 1])
        if b == a:
            continue
        L = int(seq_lens[r])
        c = int(num_computed[r])
        K = as_f64(gather_kv(key_cache, block_table[r], L, block_size), dtype)
        V = as_f64(gather_kv(value_cache, block_table[r], L, block_size), dtype)
        Q = as_f64(query[a:b], dtype)
        qpos = c + np.arange(b - a)
        for h in range(Hq):
            g = h // G
            o, ls = _softmax_attend(Q[:, h, :], K[:, g, :], V[:, g, :], qpos, scale)
            out[a:b, h, :] = o
            lse[a:b, h] = ls
    return out, lse


def attention_rows(query_rows: np.ndarray, k_hist: np.ndarray, v_hist: np.ndarray,
                   qpos: Sequence[int], scale: float, dtype: str):
    """Attention for a few query rows of ONE request whose logical history
    k_hist/v_hist [L, Hkv, D] (storage dtype) is already gathered.
    query_rows [n, Hq, D]; row i at absolute position qpos[i].
    Used to check sampled outputs of large steps one by one."""
    Q = as_f64(query_rows, dtype)
    K = as_f64(k_hist, dtype)
    V = as_f64(v_hist, dtype)
    n, Hq, D = Q.shape
    G = Hq // K.shape[1]
    qpos = np.asarray(qpos, dtype=np.int64)
    out = np.empty((n, Hq, D))
    lse = np.empty((n, Hq))
    for h in range(Hq):
        o, ls = _softmax_attend(Q[:, h, :], K[:, h // G, :], V[:, h // G, :], qpos, scale)
        out[:, h, :] = o
        lse[:, h] = ls
    return out, lse


# ----------------------------------------------------------------------------
# dense references (no paging) and chunked prefill
# ----------------------------------------------------------------------------
def dense_causal(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """One-shot causal attention over [..., T, D] fp64 arrays (same T for q and
    k): the full-prefill side of the chunked-prefill equivalence."""
    T = q.shape[-2]
    s = (q @ np.swapaxes(k, -1, -2)) * scale
    mask = np.triu(np.ones((T, T), dtype=bool), 1)
    s = np.where(mask, -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=-1, keepdims=True)) @ v


def chunked_causal(q: np.ndarray, k: np.ndarray, v: np.ndarray, chunk: int,
                   scale: float):
    """Chunked prefill ("Chunked Prefill 与 Preemption", equation M_{i,j}):
    for each chunk [a, b) the cache holds keys 0:b and query i in [a, b) sees
    keys j <= i.  Returns (concatenated outputs, trace) where the trace lists
    (a, b, shape of the cache used for that chunk)."""
    T = q.shape[-2]
    outs = []
    trace = []
    for a in range(0, T, chunk):
        b = min(a + chunk, T)
        kc = k[..., :b, :]
        vc = v[..., :b, :]
        s = (q[..., a:b, :] @ np.swapaxes(kc, -1, -2)) * scale
        qi = np.arange(a, b)[:, None]
        kj = np.arange(b)[None, :]
        s = np.where(kj > qi, -np.inf, s)
        s = s - s.max(axis=-1, keepdims=True)
        e = np.exp(s)
        outs.append((e / e.sum(axis=-1, keepdims=True)) @ vc)
        trace.append((a, b, tuple(kc.shape)))
    return np.concatenate(outs, axis=-2), trace


# ----------------------------------------------------------------------------
# block accounting ("显存与调度", "从保留词元到物理块")
# ----------------------------------------------------------------------------
def block_accounting(lengths: Sequence[int], block_size: int) -> dict:
    """Per-request logical blocks q_i = ceil(T_i / B), allocated slots q_i * B
    and tail waste w_i = q_i * B - T_i, plus the totals."""
    q = [-(-int(t) // block_size) for t in lengths]
    w = [qi * block_size - int(t) for qi, t in zip(q, lengths)]
    return {
        "blocks": q,
        "tail_waste": w,
        "entries": sum(q),
        "allocated": sum(q) * block_size,
        "waste": sum(w),
    }


def preemption_accounting(cached_tokens: int, block_size: int,
                          kv_bytes_per_tok: int, bandwidth_gbps: float) -> dict:
    """Recompute preemption releases every block the request holds and later
    recomputes every cached token; a swap would move the payload out and back
    ("Chunked Prefill 与 Preemption", "可运行等价性与成本核算")."""
    blocks = -(-int(cached_tokens) // block_size)
    payload = int(cached_tokens) * int(kv_bytes_per_tok)
    return {
        "released_blocks": blocks,
        "recompute_tokens": int(cached_tokens),
        "swap_roundtrip_ms": 2.0 * payload / (bandwidth_gbps * 1e9) * 1e3,
    }


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       bytes_per_elem: int) -> int:
    """kappa = 2 * L * n_kv * d_head * b_kv ("显存与调度", equation kappa)."""
    return 2 * num_layers * num_kv_heads * head_dim * bytes_per_elem


def merge_partials(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Combine attention computed over disjoint key ranges: each part p gives a
    running max m_p, a sum l_p = sum exp(s - m_p) and an unnormalised output
    o_p = sum exp(s - m_p) v.  The exact combination rescales every part to
    the global max ("AI Infra入门干货总结…", section "总结": split-K partitions
    are normalised with log-sum-exp).  m, l: [P]; o: [P, D]."""
    M = np.max(m)
    w = np.exp(m - M)
    return (w[:, None] * o).sum(axis=0) / (w * l).sum()


__all__.append("merge_partials")


# ----------------------------------------------------------------------------
# rotary position embedding ("Attention Module (以标准GQA + RoPE为例)")
# ----------------------------------------------------------------------------
def _rope_pairs(rotary_dim: int, neox: bool) -> List[Tuple[int, int]]:
    """Coordinate pairs the 2x2 rotation blocks act on; pair i uses angle
    column i of the cache.  Adjacent pairs (2i, 2i+1) when neox is False;
    split halves (i, i + rotary_dim/2) when neox is True."""
    half = rotary_dim // 2
    if neox:
        return [(i, i + half) for i in range(half)]
    return [(2 * i, 2 * i + 1) for i in range(half)]


def rope_matrix(cos_sin_row: np.ndarray, head_dim: int, rotary_dim: int,
                neox: bool) -> np.ndarray:
    """[head_dim, head_dim] rotation for one position, fp64.

    cos_sin_row holds rotary_dim values: cos of the rotary_dim/2 angles, then
    their sin.  Pair (a, b) with angle column i gets the block
    [[cos_i, -sin_i], [sin_i, cos_i]]; dimensions at or past rotary_dim keep
    the identity.  A pure rotation: the matrix is orthogonal (pinned)."""
    row = np.asarray(cos_sin_row, dtype=np.float64)
    half = rotary_dim // 2
    R = np.eye(head_dim, dtype=np.float64)
    for i, (a, b) in enumerate(_rope_pairs(rotary_dim, neox)):
        c, s = row[i], row[half + i]
        R[a, a] = c
        R[a, b] = -s
        R[b, a] = s
        R[b, b] = c
    return R


def rope(x: np.ndarray, positions: np.ndarray, cos_sin_cache: np.ndarray,
         rotary_dim: int, neox: bool) -> np.ndarray:
    """Rotate x [T, H, head_dim] (fp64 values) token by token: row t of every
    head is multiplied by rope_matrix(cos_sin_cache[positions[t]])."""
    x = np.asarray(x, dtype=np.float64)
    T, H, D = x.shape
    out = np.empty_like(x)
    cache = np.asarray(cos_sin_cache, dtype=np.float64)
    for t in range(T):
        R = rope_matrix(cache[int(positions[t])], D, rotary_dim, neox)
        out[t] = x[t] @ R.T
    return out


def rope_write_kv(query: np.ndarray, key: np.ndarray, value: np.ndarray,
                  key_cache: np.ndarray, value_cache: np.ndarray, slots: np.ndarray,
                  positions: np.ndarray, cos_sin_cache: np.ndarray, rotary_dim: int,
                  neox: bool, block_size: int) -> np.ndarray:
    """The fused step in the pages' order: rotate Q and K, then write the
    rotated K and the unchanged V to the paged cache by slot.

    query / key / value are fp64 values; the caches must be float64 arrays
    (the rotated values are not representable in the storage dtype, so the
    comparison with a device cache is done to a tolerance).  Returns the
    rotated query."""
    q_rot = rope(query, positions, cos_sin_cache, rotary_dim, neox)
    k_rot = rope(key, positions, cos_sin_cache, rotary_dim, neox)
    write_kv(key_cache, value_cache, k_rot, np.asarray(value, dtype=np.float64), slots,
             block_size)
    return q_rot


def _self_check() -> None:  # pragma: no cover - manual sanity hook
    bt = np.array([[5, 8, 12]])
    assert slot_mapping(bt, [1], [25], 16)[0] == 137
    assert math.isclose(preemption_accounting(7, 4, 512 * 1024, 24)["swap_roundtrip_ms"],
                        0.30583466666666664)
