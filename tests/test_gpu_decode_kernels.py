"""GPU parity of the split-K decode kernels against the fp64 oracle.

bf16 caches with 8 query heads per kv head run a matrix-core kernel by
default, bf16 with up to 4 query heads per kv head a vector kernel; with
head_dim 128 both come in a whole-block form (one workgroup of Hkv waves per
item, slabs of all kv heads staged in LDS), the default, and a per-head form
(one wavefront per item and kv head); every other case runs the per-head
vector kernel.  The decode_kernel and decode_staging tuning knobs select
each of the four where it has an instance.  All are checked on context lengths around every tile and
partition edge (1, 15..17, 31..33, partition lengths +-1), with head_dim 64
and 128, 1, 2, 4 and 8 kv heads, block sizes 16, 32 and 48 (a size that is
not a power of two: 16-key halves of a 32-key tile fall in different
blocks), and several partition lengths (the merge pass combines their
partials); a 3-token chunk rides along in the same step.  Caches bit-exact,
outputs within the bf16 tolerance.
"""
import pytest

from helpers import check_requests, run_step, say
from workloads import configs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_attention_reshape_amd as pa  # noqa: E402

LENS = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1023, 1024, 1025, 2047, 3001]

SHAPES = [
    # Hq, Hkv, D, B
    (32, 8, 128, 16),
    (64, 8, 128, 32),
    (16, 4, 64, 16),
    (32, 4, 64, 48),
    (8, 2, 128, 48),
    (4, 1, 128, 16),
    (8, 4, 128, 32),
    (8, 8, 128, 16),
]

# kernel name -> tuning (whole-block where it has an instance, else per-head)
KERNELS = {"matrix": dict(decode_kernel=2), "matrix-per-head": dict(decode_kernel=2, decode_staging=1),
           "vector": dict(decode_kernel=1), "per-head": dict(decode_kernel=1, decode_staging=1)}


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("shape", SHAPES, ids=[f"g{s[0] // s[1]}-d{s[2]}-b{s[3]}" for s in SHAPES])
@pytest.mark.parametrize("split", [0, 64, 512])
def test_decode_kernel_matches_oracle(kernel, shape, split):
    Hq, Hkv, D, B = shape
    say(f"\n[gpu-test] decode {kernel} {shape} split {split or 'auto'}")
    qlens = [1] * len(LENS) + [3]
    comp = [L - 1 for L in LENS] + [700]
    spec = configs.custom(f"dec{Hq}-{Hkv}-{D}-{B}", "bf16", Hq, Hkv, D, B, qlens, comp,
                          seed=31 + B + D + Hq, pool_factor=1.3)
    with pa.tuning(split_keys=split, **KERNELS[kernel]):
        d, out, _ = run_step(spec, pa)
    torch.cuda.synchronize()
    err = check_requests(spec, out, d["key_cache"], d["value_cache"], range(spec.R),
                         what=f"{kernel} {shape} split {split}")
    say(f"decode {kernel} {shape} split {split}: worst abs err {err:.2e}")


def test_block_and_per_head_kernels_bitwise_equal():
    """The whole-block and per-head vector kernels run the same arithmetic in
    the same order (only where K/V bytes come from differs), so on a C3-like
    decode batch their outputs are identical bit for bit."""
    spec = configs.custom("dec-stage", "bf16", 32, 8, 128, 16, [1] * 40,
                          [16383, 9000, 4095] + [97 * i + 5 for i in range(37)], seed=78,
                          pool_factor=1.1)
    outs = []
    for staging in (0, 1):
        with pa.tuning(decode_staging=staging):
            _, out, _ = run_step(spec, pa)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).cpu())
    assert torch.equal(outs[0], outs[1])


def test_decode_kernels_close_to_each_other():
    """The matrix-core and vector kernels round differently (bf16
    probabilities in the matrix kernel, a lazily raised running max) but
    compute the same function: on a C4-like batch their outputs agree within
    the bf16 tolerance."""
    spec = configs.custom("dec-cmp", "bf16", 64, 8, 128, 32, [1] * 24,
                          [32767, 20000, 9000] + [100 * i + 7 for i in range(21)], seed=77,
                          pool_factor=1.1)
    outs = []
    for kernel in (2, 1):
        with pa.tuning(decode_kernel=kernel):
            _, out, _ = run_step(spec, pa)
        torch.cuda.synchronize()
        outs.append(out.float())
    diff = (outs[0] - outs[1]).abs()
    tol = 1e-2 + 1e-2 * outs[1].abs()
    assert bool((diff <= tol).all()), f"max diff {float(diff.max()):.3e}"
