"""GPU parity of the e2m1 MX, 6-bit MX and blockscale FP8 LDS-fetch kernels on
grids of more than one round of tiles, where each workgroup, once its K loop
is done, loads the first lines of the A, B and scale rows of the tile that
starts after it on its XCD (a prefetch into L2 whose values are never used).

The cases put ragged M and N edges into the grid, so that some workgroups
prefetch for an edge tile, and cover plain and prepacked B, 1x32 and 32x32 B
scales, bias, and every LDS-fetch tile (256x256 on four and eight waves,
192x192, and 128x128, which holds two workgroups per CU).  The prefetch only
reads, through range-checked buffer loads; a wrong base or range could reach
memory it must not, and a wrong wait count could let a fetch land in the
output stash.  Every launch writes into a NaN-filled C: no output may stay
unwritten, and the first and last row of every tile band (all columns) must
match the oracle to the MX bar (1e-2 * sum|ab| + 1 bf16 ulp, cosine >=
0.99999)."""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from block_scaled_precision_02_amd import inputs  # noqa: E402
import block_scaled_precision_02_amd as q  # noqa: E402

from tests import parity  # noqa: E402


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


def _workload(M, N, K, brows, bias):
    """The MXFP4 recipe at M x N x K; with brows = 32 the B scales are every
    32nd row's (one ue8m0 row per 32 rows of B, the [N/32, K/32] layout)."""
    d = inputs.make("mxfp4", M=M, N=N, K=K, bias=bias)
    if brows == 32:
        d["scale_b"] = np.ascontiguousarray(d["scale_b"][::32])
        d["b_rows_per_scale"] = 32
    return d


def _run(d, packed, out):
    bias = None if d["bias"] is None else parity.dev(d["bias"].view(np.int16))
    A, sa, sb = parity.dev(d["A"]), parity.dev(d["scale_a"]), parity.dev(d["scale_b"])
    if packed:
        pb = q.qgemm_prepack_b(parity.dev(d["B"]))
        return q.qgemm_mx_prepacked(q.QGEMM_MX_E2M1, A, pb, sa, sb, d["b_rows_per_scale"], bias, out=out)
    return q.qgemm_mx(q.QGEMM_MX_E2M1, A, parity.dev(d["B"]), sa, sb, d["b_rows_per_scale"], bias, out=out)


# 4100 x 4600: 17 x 18 tiles of 256 (306, more than one round of 256), 22 x 24
# of 192 (528) and 33 x 36 of 128 (1188, more than the 512 that two
# workgroups per CU hold); the last tile row holds 4 rows, the last tile
# column 248, 184 or 120 columns.
SHAPE = (4100, 4600, 512)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("brows", [1, 32])
@pytest.mark.parametrize("tile", [4, 5, 6, 7])
def test_multi_round_ragged_grid(tile, brows, packed):
    M, N, K = SHAPE
    d = _workload(M, N, K, brows, False)
    _say(f"[successor] mxfp4 {M}x{N}x{K} tile={tile} brows={brows} packed={packed}")
    q.force_tile(tile)
    out = _run(d, packed, parity.nan_out(M, N))
    parity.check_full_grid(d, out, tile, f"successor tile={tile} brows={brows} packed={packed}")


@pytest.mark.parametrize("tile", [-1, 5])
@pytest.mark.parametrize("M,N,K", [(4100, 4600, 512), (8192, 4104, 256)])
def test_multi_round_bias_and_repeat(M, N, K, tile):
    """The table's tile (192x192 at these shapes) and the eight-wave 256x256
    one, with a bias, each launched twice into the same C (the second launch
    reads what the first one's prefetches touched): both launches equal to
    the oracle, and their outputs bit-identical."""
    d = _workload(M, N, K, 1, True)
    _say(f"[successor] mxfp4 {M}x{N}x{K} tile={tile} bias, twice")
    q.force_tile(tile)
    out = _run(d, False, parity.nan_out(M, N))
    parity.check_full_grid(d, out, tile, f"successor bias {M}x{N}x{K} tile={tile}")
    first = parity.bits(out)
    out.fill_(float("nan"))
    out = _run(d, False, out)
    parity.check_full_grid(d, out, tile, f"successor bias {M}x{N}x{K} tile={tile} (second launch)")
    assert np.array_equal(parity.bits(out), first), "two launches on the same inputs differ"


def _run_other(d, packed, out):
    bias = None if d["bias"] is None else parity.dev(d["bias"].view(np.int16))
    A, sa, sb = parity.dev(d["A"]), parity.dev(d["scale_a"]), parity.dev(d["scale_b"])
    if packed:
        pb = q.qgemm_prepack_b(parity.dev(d["B"]))
        return q.qgemm_f8_blockscale_prepacked(A, pb, sa, sb, bias, out=out)
    return parity.gpu_run(d, out=out)


# Blockscale FP8 (256x128 and 128x128 tiles) and both 6-bit MX formats
# (256x256 on four waves, 128x128) prefetch as well.
@pytest.mark.parametrize("name,tile,packed", [
    ("f8_block", -1, False), ("f8_block", 10, False), ("f8_block", 7, False), ("f8_block", 10, True),
    ("mxfp6", -1, False), ("mxfp6", 4, False), ("mxfp6", 7, False),
    ("mxfp6_e3m2", 4, False), ("mxfp6_e3m2", 7, False),
])
def test_multi_round_ragged_grid_other_paths(name, tile, packed):
    M, N, K = SHAPE
    d = inputs.make(name, M=M, N=N, K=K)
    _say(f"[successor] {name} {M}x{N}x{K} tile={tile} packed={packed}")
    q.force_tile(tile)
    out = _run_other(d, packed, parity.nan_out(M, N))
    parity.check_full_grid(d, out, tile, f"successor {name} tile={tile} packed={packed}")
