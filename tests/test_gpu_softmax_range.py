"""GPU tests of the online softmax over a wide dynamic range of scores.

Chunk rows go to the matrix-core kernel, whose running max is raised lazily
(only when a tile's max passes it by a slack) and whose scores leave the q.k
product already shifted by that max.  These cases make the max move a lot:

* rising   - key norms grow along the sequence and every query points along
             the keys' common direction, so each 64-key tile beats the
             running max and the rescale path runs over and over;
* falling  - the same keys with the queries reversed: the first tile holds the
             max and later probabilities underflow towards zero;
* wide     - random keys with queries 16x larger than N(0, 1): scores spread
             over hundreds of log2 units.

The caches are built directly on the device (every slot of every request
filled), attention runs through the C ABI, and each request is compared with
the fp64 oracle on the cache contents read back from the device (bf16
tolerance)."""
import numpy as np
import pytest

import oracle
from helpers import assert_close, say, storage_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_attention_reshape_amd as pa  # noqa: E402

# (history c, chunk length q) per request; all chunks (q > 1)
REQS = [(1500, 300), (0, 200), (700, 64), (130, 129)]

CASES = [
    ("rising", 32, 8, 128, 16),
    ("falling", 32, 8, 128, 16),
    ("wide", 32, 8, 128, 16),
    ("wide4", 32, 8, 128, 16),
    ("rising", 64, 8, 64, 32),
    ("wide", 16, 16, 128, 16),
]


def _build(pattern, Hq, Hkv, D, B, seed):
    g = np.random.default_rng(seed)
    R = len(REQS)
    L = np.array([c + q for c, q in REQS], np.int64)
    nblk = -(-L // B)
    num_blocks = int(nblk.sum()) + 7
    perm = g.permutation(num_blocks).astype(np.int32)
    M = int(nblk.max())
    bt = np.full((R, M), -1, np.int32)
    o = 0
    for r in range(R):
        bt[r, :nblk[r]] = perm[o:o + nblk[r]]
        o += nblk[r]
    kc = np.zeros((num_blocks, B, Hkv, D), np.float32)
    vc = g.standard_normal((num_blocks, B, Hkv, D)).astype(np.float32)
    u = g.standard_normal((Hkv, D)).astype(np.float32)       # common key direction per kv head
    qs = []
    for r, (c, q) in enumerate(REQS):
        pos = np.arange(L[r])
        if pattern.startswith("wide"):
            k = g.standard_normal((L[r], Hkv, D)).astype(np.float32)
        else:
            amp = (0.5 + 3.0 * pos / L[r]).astype(np.float32)
            k = amp[:, None, None] * u[None] + 0.3 * g.standard_normal((L[r], Hkv, D)).astype(np.float32)
        slots = bt[r, pos // B].astype(np.int64) * B + pos % B
        kc.reshape(-1, Hkv, D)[slots] = k
        G = Hq // Hkv
        if pattern.startswith("wide"):
            amp_q = 16.0 if pattern == "wide" else 4.0
            qq = amp_q * g.standard_normal((q, Hq, D)).astype(np.float32)
        else:
            sign = 1.0 if pattern == "rising" else -1.0
            qq = sign * 4.0 * np.repeat(u, G, axis=0)[None] + 0.3 * g.standard_normal((q, Hq, D)).astype(np.float32)
        qs.append(qq)
    query = np.concatenate(qs, axis=0)
    ql = np.array([q for _, q in REQS], np.int32)
    comp = np.array([c for c, _ in REQS], np.int32)
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    sl = (comp + ql).astype(np.int32)
    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    bf = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16).contiguous()  # noqa: E731
    return dict(q=bf(query), kc=bf(kc), vc=bf(vc), bt=to(bt), qsl=to(qsl), sl=to(sl), comp=to(comp),
                h_qsl=qsl, h_sl=sl, h_bt=bt, h_comp=comp, h_ql=ql)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-g{c[1] // c[2]}-d{c[3]}-b{c[4]}" for c in CASES])
def test_chunk_softmax_wide_dynamic_range(case):
    pattern, Hq, Hkv, D, B = case
    say(f"\n[gpu-test] softmax range {case}")
    x = _build(pattern, Hq, Hkv, D, B, seed=17 + CASES.index(case))
    scale = 1.0 / np.sqrt(D)
    out = torch.empty_like(x["q"])
    pa.attention(out, x["q"], x["kc"], x["vc"], x["bt"], x["qsl"], x["sl"], x["comp"],
                 x["h_qsl"], x["h_sl"], scale,
                 workspace=pa.alloc_workspace(pa.attention_workspace_size(x["h_qsl"], x["h_sl"], Hq, Hkv, D, B,
                                                                          pa.PA_BF16)))
    torch.cuda.synchronize()
    kc, vc, q_all, o_all = storage_np(x["kc"]), storage_np(x["vc"]), storage_np(x["q"]), storage_np(out)
    worst = 0.0
    for r, (c, q) in enumerate(REQS):
        L = c + q
        kh = oracle.gather_kv(kc, x["h_bt"][r], L, B)
        vh = oracle.gather_kv(vc, x["h_bt"][r], L, B)
        t0 = int(x["h_qsl"][r])
        want, _ = oracle.attention_rows(q_all[t0:t0 + q], kh, vh, np.arange(c, L), scale, "bf16")
        got = oracle.as_f64(o_all[t0:t0 + q], "bf16")
        worst = max(worst, assert_close(got, want, "bf16", f"{case} request {r}"))
    say(f"softmax range {case}: worst abs err {worst:.2e}")
