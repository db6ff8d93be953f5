"""GPU parity over seeded random shapes: every GEMM path against the CPU oracle
on shapes drawn across the tile table's boundaries (small-M, 128/192/256 tiles,
ragged M and N tails, K on and off the LDS-fetch kernel's rounds), with and
without bias, into an output with a padded row stride.  INT8 bit-exact,
FP8 / MX within 1e-2 * sum|a b| + 1 bf16 ulp and cosine >= 0.99999.
"""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from block_scaled_precision_02_amd import inputs  # noqa: E402
import block_scaled_precision_02_amd as q  # noqa: E402

from tests import parity  # noqa: E402

CASES = 10


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.force_tile(-1)
    yield
    q.force_tile(-1)


def _shape(rng, name):
    M = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 65)), int(rng.integers(65, 520))]))
    N = int(rng.integers(1, 520))
    if name in ("f8_block", "mxfp6", "mxfp6_e3m2"):
        K = 128 * int(rng.integers(1, 13))                 # these paths: K a multiple of 128
    else:
        # any multiple of 32 (K = 32 * odd: a last half stage, 16-byte
        # e2m1 row ends)
        K = 32 * int(rng.integers(1, 49))
    return M, N, K


def _make(name, M, N, K, bias, rng):
    d = inputs.make(name, M=M, N=N, K=K, bias=bias)
    if name == "mxfp8" and rng.random() < 0.5:
        # the 1x32 B-scale layout instead of the recipe's 32x32
        xb = rng.standard_normal((N, K)).astype(np.float32)
        d["B"], d["scale_b"] = inputs.mx_quantise(xb, "e4m3", 1)
        d["b_rows_per_scale"] = 1
    return d


NAMES = ["i8_small", "f8_ptpc", "mxfp8", "mxfp4", "f8_block", "mx_a8w4", "mx_a4w8", "mxfp6", "mxfp6_e3m2"]


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("case", range(CASES))
def test_random_shapes(name, case):
    rng = np.random.default_rng([2024, case, NAMES.index(name)])
    M, N, K = _shape(rng, name)
    bias = bool(rng.random() < 0.5)
    d = _make(name, M, N, K, bias, rng)
    _say(f"[sweep] {name} {M}x{N}x{K} bias={bias} brows={d['b_rows_per_scale']}")
    ldc = N + (-N) % 8 + 8 * int(rng.integers(0, 3))
    buf = torch.full((M + 2, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
    before = parity.bits(buf)
    parity.gpu_run(d, out=buf[:M, :N])
    torch.cuda.synchronize()
    after = parity.bits(buf)
    ref, absdot, _ = parity.oracle_run(d)
    parity.compare(d, after[:M, :N], ref, absdot, f"sweep {name} {M}x{N}x{K}")
    assert np.array_equal(after[:M, N:], before[:M, N:]), "wrote past N"
    assert np.array_equal(after[M:], before[M:]), "wrote past M"
