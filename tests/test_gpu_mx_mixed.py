"""GPU parity of the mixed-format MX GEMM (qgemm_mx_mixed: e4m3 A x e2m1 B,
and e2m1 A x e4m3 B) against the CPU oracle (orc_mx2) on the same seeded
inputs, through the C ABI.

Bar: per element |gpu - oracle| <= 1e-2 * sum_k |A~ B~| + 1 bf16 ulp, cosine
>= 0.99999.  Every LDS-fetch tile it runs on (4, 5, 7), both B-scale
layouts, ragged M / N tails, random scale codes (a scale paired with the wrong
K block or row leaves the bound), canaries around the output.
"""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from block_scaled_precision_02_amd import inputs  # noqa: E402
import block_scaled_precision_02_amd as q  # noqa: E402

from tests import parity  # noqa: E402

TILES = [4, 5, 7]


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


def _make(M, N, K, brows=1, bias=False, name="mx_a8w4"):
    d = inputs.make(name, M=M, N=N, K=K, bias=bias)
    if brows == 32:
        # 32x32 B scales: one code per 32 rows of B (the recipe's 1x32 codes of the group's first row)
        d["scale_b"] = np.ascontiguousarray(d["scale_b"][::32])
        d["b_rows_per_scale"] = 32
    return d


def _check(d, what, out=None):
    _say(f"[parity] {what} M={d['M']} N={d['N']} K={d['K']}")
    out = parity.gpu_run(d, out=out)
    torch.cuda.synchronize()
    ref, absdot, _ = parity.oracle_run(d)
    worst, cos = parity.compare(d, parity.bits(out), ref, absdot, what)
    _say(f"[parity] {what}: worst err/bound {worst:.3g} cos {cos:.8f}")
    return out


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("brows", [1, 32])
@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (33, 70, 512), (300, 520, 1024), (1, 1, 512), (257, 300, 1536),
                                   (300, 264, 256), (256, 512, 768), (130, 200, 1792),
                                   (300, 264, 192), (257, 300, 704), (64, 130, 64), (130, 257, 1216)])
def test_mx84_small(M, N, K, brows, tile):
    q.force_tile(tile)
    _check(_make(M, N, K, brows), f"mx84 brows={brows} tile={tile}")


@pytest.mark.parametrize("tile", TILES)
def test_mx84_bias_and_random_scales(tile):
    q.force_tile(tile)
    d = _make(320, 288, 2048, bias=True)
    rng = np.random.default_rng(9)
    d["scale_a"] = rng.integers(112, 142, d["scale_a"].shape, dtype=np.uint8)
    d["scale_b"] = rng.integers(112, 142, d["scale_b"].shape, dtype=np.uint8)
    _check(d, f"mx84 random scales tile={tile}")


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("M,N,K", [(17, 31, 512), (100, 200, 1024), (1000, 129, 2048)])
def test_mx84_edges_canaries(M, N, K, tile):
    q.force_tile(tile)
    d = _make(M, N, K, bias=True)
    ldc = N + (-N) % 8 + 8
    buf = torch.full((M + 3, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
    before = parity.bits(buf)
    _check(d, f"mx84 canaries tile={tile}", out=buf[:M, :N])
    after = parity.bits(buf)
    assert np.array_equal(after[:M, N:], before[:M, N:]), "wrote past N"
    assert np.array_equal(after[M:], before[M:]), "wrote past M"


def test_mx84_equal_formats_are_qgemm_mx():
    d = inputs.make("mxfp8", M=256, N=256, K=512)
    A, B = parity.dev(d["A"]), parity.dev(d["B"])
    sa, sb = parity.dev(d["scale_a"]), parity.dev(d["scale_b"])
    o1 = q.qgemm_mx(q.QGEMM_MX_E4M3, A, B, sa, sb, 32)
    o2 = q.qgemm_mx_mixed(q.QGEMM_MX_E4M3, q.QGEMM_MX_E4M3, A, B, sa, sb, 32)
    torch.cuda.synchronize()
    assert np.array_equal(parity.bits(o1), parity.bits(o2))


def test_mx84_rejects():
    A8 = torch.zeros((4, 528), dtype=torch.uint8, device="cuda")
    B4 = torch.zeros((4, 264), dtype=torch.uint8, device="cuda")
    s = torch.full((4, 16), 127, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):      # K = 528 is not a multiple of 32
        q.qgemm_mx_mixed(q.QGEMM_MX_E4M3, q.QGEMM_MX_E2M1, A8, B4, s, s, 1)
    with pytest.raises(ValueError):      # e2m1 A with e4m3 B, the same K
        q.qgemm_mx_mixed(q.QGEMM_MX_E2M1, q.QGEMM_MX_E4M3, B4, A8, s, s, 1)


def _sample_rows(M, n, rng):
    tail = np.arange(max(0, M - 8), M)
    head = np.arange(0, min(8, M))
    mid = rng.choice(M, size=max(0, n - len(head) - len(tail)), replace=False)
    return np.unique(np.concatenate([head, mid, tail]))


@pytest.mark.parametrize("tile", [-1, 7])
def test_mx84_full_workload_sampled(tile):
    """8192^3, launched as the benchmark launches it, into a NaN-filled C:
    every output written; the first and last row of every tile band and
    random rows against the oracle."""
    q.force_tile(tile)
    d = inputs.make("mx_a8w4")
    _say(f"[parity] full mx_a8w4 tile {tile}")
    out = parity.gpu_run(d, out=parity.nan_out(d["M"], d["N"]))
    worst, cos, _ = parity.check_full_grid(d, out, tile, "full mx_a8w4",
                                           _sample_rows(d["M"], 16, np.random.default_rng(2)))
    _say(f"[parity] full mx_a8w4: worst err/bound {worst:.3g} cos {cos:.8f}")


SMALL_M = [(1, 7168, 2048, 8), (5, 200, 256, 8), (16, 300, 1792, 8), (1, 1, 512, 8), (33, 130, 512, 9),
           (64, 264, 768, 9), (5, 200, 320, 8), (33, 130, 704, 9)]


@pytest.mark.parametrize("brows", [1, 32])
@pytest.mark.parametrize("M,N,K,tile", SMALL_M)
def test_mx84_small_m_kernel(M, N, K, tile, brows):
    """The small-M kernel: A e4m3 in its two-chunk map, B one 16-byte e2m1
    chunk per lane and step; ragged N, canaries, bias, random scale codes."""
    q.force_tile(tile)
    d = _make(M, N, K, brows, bias=(M % 2 == 1))
    rng = np.random.default_rng(M * 5 + N + brows)
    d["scale_a"] = rng.integers(112, 142, d["scale_a"].shape, dtype=np.uint8)
    d["scale_b"] = rng.integers(112, 142, d["scale_b"].shape, dtype=np.uint8)
    ldc = N + (-N) % 8 + 8
    buf = torch.full((M + 3, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
    before = parity.bits(buf)
    _check(d, f"mx84 small M tile {tile}", out=buf[:M, :N])
    after = parity.bits(buf)
    assert np.array_equal(after[:M, N:], before[:M, N:]), "wrote past N"
    assert np.array_equal(after[M:], before[M:]), "wrote past M"


# ---- e2m1 A x e4m3 B (the LDS-fetch tiles 4, 5, 7 at every M)

SHAPES = [(256, 256, 512), (33, 70, 512), (300, 520, 1024), (1, 1, 512), (257, 300, 1536), (300, 264, 256),
          (256, 512, 768), (130, 200, 1792), (16, 300, 640),
          # K % 128 == 64: scale rows off dword boundaries, a half-live last scale word
          (300, 264, 192), (257, 300, 704), (64, 130, 64), (130, 257, 1216)]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("brows", [1, 32])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_mx48_small(M, N, K, brows, tile):
    q.force_tile(tile)
    _check(_make(M, N, K, brows, name="mx_a4w8"), f"mx48 brows={brows} tile={tile}")


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("brows", [1, 32])
def test_mx48_bias_and_random_scales(tile, brows):
    q.force_tile(tile)
    d = _make(320, 288, 2048, brows, bias=True, name="mx_a4w8")
    rng = np.random.default_rng(11 + brows)
    d["scale_a"] = rng.integers(112, 142, d["scale_a"].shape, dtype=np.uint8)
    d["scale_b"] = rng.integers(112, 142, d["scale_b"].shape, dtype=np.uint8)
    _check(d, f"mx48 random scales brows={brows} tile={tile}")


@pytest.mark.parametrize("tile", TILES + [-1])
@pytest.mark.parametrize("M,N,K", [(17, 31, 512), (100, 200, 1024), (1000, 129, 2048), (5, 300, 384)])
def test_mx48_edges_canaries(M, N, K, tile):
    q.force_tile(tile)
    d = _make(M, N, K, bias=True, name="mx_a4w8")
    ldc = N + (-N) % 8 + 8
    buf = torch.full((M + 3, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
    before = parity.bits(buf)
    _check(d, f"mx48 canaries tile={tile}", out=buf[:M, :N])
    after = parity.bits(buf)
    assert np.array_equal(after[:M, N:], before[:M, N:]), "wrote past N"
    assert np.array_equal(after[M:], before[M:]), "wrote past M"


@pytest.mark.parametrize("tile", [-1, 5, 7])
def test_mx48_full_workload_sampled(tile):
    """8192^3 e2m1 A x e4m3 B, launched as the benchmark launches it, into a
    NaN-filled C: every output written; the first and last row of every tile
    band and random rows against the oracle."""
    q.force_tile(tile)
    d = inputs.make("mx_a4w8")
    _say(f"[parity] full mx_a4w8 tile {tile}")
    out = parity.gpu_run(d, out=parity.nan_out(d["M"], d["N"]))
    worst, cos, _ = parity.check_full_grid(d, out, tile, "full mx_a4w8",
                                           _sample_rows(d["M"], 16, np.random.default_rng(4)))
    _say(f"[parity] full mx_a4w8: worst err/bound {worst:.3g} cos {cos:.8f}")
