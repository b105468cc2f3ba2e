"""GPU parity over the support matrix and over very long contexts.

* A seeded sweep of random steps: dtype, GQA group, kv heads, head_dim and
  block size drawn from the supported set, a random mix of decode rows and
  chunks with random histories; every request is checked against the fp64
  oracle (caches bit-exact, outputs within the dtype's tolerance).
* A wider seeded sweep: up to 12 requests with histories up to 20 000 keys
  and chunks up to 700 tokens, with the decode kernel (matrix-core or
  vector), the vector kernel's staging (whole-block or per-head) and the
  partition length (64, 128 or 512 keys, or the automatic rule) drawn per
  case.
* Rows with more than 64 split-K partitions (the merge pass then makes
  several passes over the partitions): forced 64-key partitions over
  contexts of thousands of keys, and genuinely long contexts (70 000 keys)
  at the default partition length.
"""
import numpy as np
import pytest

from helpers import check_requests, run_step, say
from workloads import configs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_attention_reshape_amd as pa  # noqa: E402


def _random_case(i):
    g = np.random.default_rng(4000 + i)
    dtype = ["bf16", "f32"][int(g.integers(0, 2))]
    G = int(g.choice([1, 2, 4, 8]))
    Hkv = int(g.choice([1, 2, 4, 8]))
    D = int(g.choice([64, 128]))
    B = int(g.choice([16, 32, 48, 64]))
    R = int(g.integers(1, 9))
    qlens, comp = [], []
    for _ in range(R):
        if g.random() < 0.65:
            qlens.append(1)
        else:
            qlens.append(int(g.integers(2, 301)))
        comp.append(int(g.integers(0, 3001)))
    return dtype, G * Hkv, Hkv, D, B, qlens, comp


CASES = [_random_case(i) for i in range(16)]


@pytest.mark.parametrize("i", range(len(CASES)), ids=[f"rand{i}" for i in range(len(CASES))])
def test_random_steps_match_oracle(i):
    dtype, Hq, Hkv, D, B, qlens, comp = CASES[i]
    say(f"\n[gpu-test] random step {i}: {CASES[i]}")
    spec = configs.custom(f"rand{i}", dtype, Hq, Hkv, D, B, qlens, comp, seed=500 + i, pool_factor=1.4)
    d, out, _ = run_step(spec, pa)
    torch.cuda.synchronize()
    err = check_requests(spec, out, d["key_cache"], d["value_cache"], range(spec.R),
                         rows_per_req=24, what=f"random step {i}")
    say(f"random step {i}: worst abs err {err:.2e}")


def _wide_case(i):
    g = np.random.default_rng(10000 + i)
    dtype = ["bf16", "f32"][int(g.integers(0, 2))]
    G = int(g.choice([1, 2, 4, 8]))
    Hkv = int(g.choice([1, 2, 4, 8]))
    D = int(g.choice([64, 128]))
    B = int(g.choice([16, 32, 48, 64]))
    R = int(g.integers(1, 13))
    qlens, comp = [], []
    for _ in range(R):
        u = g.random()
        qlens.append(1 if u < 0.6 else int(g.integers(2, 40)) if u < 0.8 else int(g.integers(40, 700)))
        comp.append(int(g.choice([0, int(g.integers(0, 64)), int(g.integers(0, 5000)),
                                  int(g.integers(5000, 20000))], p=[0.1, 0.2, 0.5, 0.2])))
    mfma = ["0", "1", None][int(g.integers(0, 3))]
    split = [None, "64", "128", "512"][int(g.integers(0, 4))]
    staging = int(np.random.default_rng(30000 + i).integers(0, 2))   # 0 auto, 1 per-head
    return dtype, G * Hkv, Hkv, D, B, qlens, comp, mfma, split, staging


WIDE = [_wide_case(i) for i in range(64)]


@pytest.mark.parametrize("i", range(len(WIDE)), ids=[f"wide{i}" for i in range(len(WIDE))])
def test_wide_random_steps_match_oracle(i):
    dtype, Hq, Hkv, D, B, qlens, comp, mfma, split, staging = WIDE[i]
    say(f"\n[gpu-test] wide random step {i}: {WIDE[i]}")
    spec = configs.custom(f"wide{i}", dtype, Hq, Hkv, D, B, qlens, comp, seed=20000 + i, pool_factor=1.3)
    knobs = {"decode_kernel": None if mfma is None else (2 if mfma == "1" else 1),
             "split_keys": None if split is None else int(split),
             "decode_staging": staging or None}
    with pa.tuning(**knobs):
        d, out, _ = run_step(spec, pa)
    torch.cuda.synchronize()
    err = check_requests(spec, out, d["key_cache"], d["value_cache"], range(spec.R),
                         rows_per_req=6, what=f"wide random step {i}")
    say(f"wide random step {i}: worst abs err {err:.2e}")


_KERNELS = {"matrix": dict(decode_kernel=2), "matrix-per-head": dict(decode_kernel=2, decode_staging=1),
            "vector": dict(decode_kernel=1), "per-head": dict(decode_kernel=1, decode_staging=1)}


@pytest.mark.parametrize("kernel", list(_KERNELS))
@pytest.mark.parametrize("shape", [(32, 8, 128, 16), (64, 8, 128, 32), (16, 8, 64, 16)],
                         ids=["g4-d128-b16", "g8-d128-b32", "g2-d64-b16"])
def test_more_than_64_partitions_forced(kernel, shape):
    """64-key partitions over up to 9000 keys: up to 141 partials per row.
    (A setting without an instance for the shape runs the kernel that has
    one: with 2 q heads per kv head and head_dim 64, the per-head vector
    kernel.)"""
    Hq, Hkv, D, B = shape
    qlens = [1, 1, 1, 1]
    comp = [4095, 4096 + 63, 8999, 130]
    spec = configs.custom(f"p64-{kernel}-{Hq}", "bf16", Hq, Hkv, D, B, qlens, comp,
                          seed=71 + Hq, pool_factor=1.2)
    with pa.tuning(split_keys=64, **_KERNELS[kernel]):
        d, out, _ = run_step(spec, pa)
    torch.cuda.synchronize()
    err = check_requests(spec, out, d["key_cache"], d["value_cache"], range(spec.R),
                         what=f"{kernel} {shape} split 64")
    say(f"{kernel} {shape} split 64: worst abs err {err:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_seventy_thousand_key_contexts(dtype):
    """Decode rows over 70 000 keys at the default partition length (more
    than 64 partitions of 1024 keys), beside a short decode and a chunk."""
    spec = configs.custom(f"long70k-{dtype}", dtype, 8, 2, 128, 16, [1, 1, 1, 40],
                          [69999, 70500, 17, 900], seed=88, pool_factor=1.05)
    d, out, _ = run_step(spec, pa)
    torch.cuda.synchronize()
    err = check_requests(spec, out, d["key_cache"], d["value_cache"], range(spec.R),
                         rows_per_req=12, what=f"70k {dtype}")
    say(f"70k-key contexts {dtype}: worst abs err {err:.2e}")
