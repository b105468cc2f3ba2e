"""GPU parity of the two split-K decode kernels against the fp64 oracle.

bf16 caches with 8 query heads per kv head run the matrix-core kernel by
default, every other case the vector-ALU kernel; the decode_kernel tuning knob selects
either kernel for groups of 4 and 8.  Both are checked on context lengths around every tile and partition
edge (1, 15..17, 31..33, partition lengths +-1), with head_dim 64 and 128,
block sizes 16, 32 and 48 (a size that is not a power of two: 16-key halves
of a 32-key tile fall in different blocks), and several partition lengths
(the merge pass combines their partials); a 3-token chunk rides along in the
same step.  Caches bit-exact, outputs within the bf16 tolerance.
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
]


@pytest.mark.parametrize("kernel", ["matrix", "vector"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"g{s[0] // s[1]}-d{s[2]}-b{s[3]}" for s in SHAPES])
@pytest.mark.parametrize("split", [0, 64, 512])
def test_decode_kernel_matches_oracle(kernel, shape, split):
    Hq, Hkv, D, B = shape
    say(f"\n[gpu-test] decode {kernel} {shape} split {split or 'auto'}")
    qlens = [1] * len(LENS) + [3]
    comp = [L - 1 for L in LENS] + [700]
    spec = configs.custom(f"dec{Hq}-{Hkv}-{D}-{B}", "bf16", Hq, Hkv, D, B, qlens, comp,
                          seed=31 + B + D + Hq, pool_factor=1.3)
    with pa.tuning(decode_kernel=2 if kernel == "matrix" else 1, split_keys=split):
        d, out, _ = run_step(spec, pa)
    torch.cuda.synchronize()
    err = check_requests(spec, out, d["key_cache"], d["value_cache"], range(spec.R),
                         what=f"{kernel} {shape} split {split}")
    say(f"decode {kernel} {shape} split {split}: worst abs err {err:.2e}")


def test_decode_kernels_close_to_each_other():
    """The two kernels round differently (bf16 probabilities in the matrix
    kernel, a lazily raised running max) but compute the same function: on a
    C4-like batch their outputs agree within the bf16 tolerance."""
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
