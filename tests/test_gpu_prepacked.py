"""GPU parity of the prepacked-B path: the prepacking kernel bit for bit
against the oracle's layout, and the ``_prepacked`` GEMMs against the oracle
GEMM on the unpacked B (INT8 bit-exact; FP8 / MX within the tolerance) and
bit for bit against the same tile reading the row-major B (the same bytes
reach LDS in the same order)."""
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


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


@pytest.mark.parametrize("N,row", [(1, 256), (17, 256), (300, 512), (2112, 7168)])
def test_prepack_bit_exact(orc, N, row):
    _say(f"[prepack] N={N} row={row}")
    rng = np.random.default_rng(N * 7 + row)
    B = rng.integers(0, 256, (N, row), dtype=np.uint8)
    Bd = torch.zeros((N, row + 64), dtype=torch.uint8, device="cuda")
    Bd[:, :row] = torch.from_numpy(B).cuda()
    nbytes = q.lib().qgemm_prepacked_b_bytes(N, row)
    buf = torch.full((nbytes + 256,), 0xA5, dtype=torch.uint8, device="cuda")
    pb = q.qgemm_prepack_b(Bd[:, :row], out=buf[:nbytes])
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.array_equal(got[:nbytes], orc.pack_b(B))
    assert (got[nbytes:] == 0xA5).all(), "wrote past Bp"
    assert pb.N == N and pb.row_bytes == row


def _run_packed(d, out=None):
    bias = None if d["bias"] is None else parity.dev(d["bias"].view(np.int16))
    B = parity.dev(d["B"])
    pb = q.qgemm_prepack_b(B)
    A, sa, sb = parity.dev(d["A"]), parity.dev(d["scale_a"]), parity.dev(d["scale_b"])
    if d["kind"] == "i8":
        return q.qgemm_i8_rowwise_prepacked(A, pb, sa, sb, bias, out=out)
    if d["kind"] == "f8":
        return q.qgemm_f8_pertoken_prepacked(A, pb, sa, sb, bias, out=out)
    if d["kind"] == "f8b":
        return q.qgemm_f8_blockscale_prepacked(A, pb, sa, sb, bias, out=out)
    fmt = q.QGEMM_MX_E4M3 if d["fmt"] == "e4m3" else q.QGEMM_MX_E2M1
    return q.qgemm_mx_prepacked(fmt, A, pb, sa, sb, d["b_rows_per_scale"], bias, out=out)


SHAPES = [(1, 1, 512), (17, 33, 512), (255, 257, 1024), (300, 520, 2048), (513, 64, 512), (64, 300, 1024)]


@pytest.mark.parametrize("tile", [-1, 4, 5, 6, 7, 8, 9])
@pytest.mark.parametrize("name", ["i8_small", "f8_ptpc", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_prepacked_gemm_edges(name, M, N, K, tile):
    """Ragged M / N, NaN-filled output with canaries past N and M; every
    LDS-fetch tile and the small-M tiles; bit for bit equal to the same tile
    on the row-major B."""
    kk = K if name != "mxfp4" else 2 * K      # e2m1: K elements are K/2 bytes
    d = inputs.make(name, M=M, N=N, K=kk, bias=(M % 2 == 1))
    _say(f"[prepacked] {name} {M}x{N}x{kk} tile {tile}")
    q.force_tile(tile)
    ldc = N + (-N) % 8 + 8
    buf = torch.full((M + 3, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
    before = parity.bits(buf)
    _run_packed(d, out=buf[:M, :N])
    after = parity.bits(buf)
    ref, absdot, _ = parity.oracle_run(d)
    parity.compare(d, after[:M, :N], ref, absdot, f"prepacked {name} {M}x{N}x{kk} tile {tile}")
    assert np.array_equal(after[:M, N:], before[:M, N:]), "wrote past N"
    assert np.array_equal(after[M:], before[M:]), "wrote past M"
    # the same tile on the row-major B: the same bytes in LDS, the same result
    q.force_tile(tile)
    plain = parity.bits(parity.gpu_run(d))
    assert np.array_equal(after[:M, :N], plain), "prepacked and row-major B differ"


@pytest.mark.parametrize("tile", [-1, 7, 10, 8, 9])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_prepacked_blockscale_edges(M, N, K, tile):
    """The blockscale GEMM on a prepacked B: every tile it runs on, ragged M /
    N, canaries; bit for bit equal to the same tile on the row-major B."""
    d = inputs.make("f8_block", M=M, N=N, K=K, bias=(M % 2 == 1))
    _say(f"[prepacked] f8_block {M}x{N}x{K} tile {tile}")
    q.force_tile(tile)
    ldc = N + (-N) % 8 + 8
    buf = torch.full((M + 3, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
    before = parity.bits(buf)
    _run_packed(d, out=buf[:M, :N])
    after = parity.bits(buf)
    ref, absdot, _ = parity.oracle_run(d)
    parity.compare(d, after[:M, :N], ref, absdot, f"prepacked f8_block {M}x{N}x{K} tile {tile}")
    assert np.array_equal(after[:M, N:], before[:M, N:]), "wrote past N"
    assert np.array_equal(after[M:], before[M:]), "wrote past M"
    q.force_tile(tile)
    plain = parity.bits(parity.gpu_run(d))
    assert np.array_equal(after[:M, :N], plain), "prepacked and row-major B differ"


@pytest.mark.parametrize("name", ["f8_ptpc", "mxfp8", "mxfp4", "i8_qkv", "f8_block"])
def test_prepacked_full_workload_sampled(name):
    """Each workload at its full size with a prepacked B, as the table
    launches it, into a NaN-filled C: every output written; the first and
    last row of every tile band and random rows against the oracle."""
    d = inputs.make(name)
    _say(f"[prepacked] full {name} M={d['M']} N={d['N']} K={d['K']}")
    q.force_tile(-1)
    out = _run_packed(d, out=parity.nan_out(d["M"], d["N"]))
    rng = np.random.default_rng(2)
    parity.check_full_grid(d, out, -1, f"prepacked full {name}", rng.choice(d["M"], 8, replace=False))


# ------------------------------------------ mixed MX: e2m1 B in 32-row groups

@pytest.mark.parametrize("N,row", [(1, 128), (33, 128), (300, 256), (7168, 1024)])
def test_prepack_b32_bit_exact(orc, N, row):
    B = np.random.default_rng(N + row).integers(0, 256, (N, row), dtype=np.uint8)
    pb = q.qgemm_prepack_b32(parity.dev(B))
    torch.cuda.synchronize()
    assert np.array_equal(pb.data.cpu().numpy(), orc.pack_b32(B))


def _run_mixed_packed(d, out=None):
    """e4m3 A with an e2m1 B from the 32-row packer, or e2m1 A with an e4m3 B
    from the 16-row one."""
    bias = None if d["bias"] is None else parity.dev(d["bias"].view(np.int16))
    a4 = d["fmt"] == "e2m1/e4m3"
    pb = q.qgemm_prepack_b(parity.dev(d["B"])) if a4 else q.qgemm_prepack_b32(parity.dev(d["B"]))
    fa, fb = (q.QGEMM_MX_E2M1, q.QGEMM_MX_E4M3) if a4 else (q.QGEMM_MX_E4M3, q.QGEMM_MX_E2M1)
    return q.qgemm_mx_mixed_prepacked(fa, fb, parity.dev(d["A"]), pb,
                                      parity.dev(d["scale_a"]), parity.dev(d["scale_b"]), d["b_rows_per_scale"],
                                      bias, out=out)


@pytest.mark.parametrize("tile", [-1, 4, 5, 7])
@pytest.mark.parametrize("name", ["mx_a8w4", "mx_a4w8"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (17, 33, 512), (255, 257, 1024), (300, 520, 2048), (64, 300, 768)])
def test_prepacked_mixed_edges(name, M, N, K, tile):
    """The mixed GEMMs on a prepacked B (e2m1 under e4m3 A, e4m3 under e2m1
    A): ragged M / N, canaries; bit for bit equal to the same tile on the
    row-major B (e4m3 A: M <= 16 runs the 128x128 tile)."""
    d = inputs.make(name, M=M, N=N, K=K, bias=(M % 2 == 1))
    _say(f"[prepacked] {name} {M}x{N}x{K} tile {tile}")
    q.force_tile(tile)
    ldc = N + (-N) % 8 + 8
    buf = torch.full((M + 3, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
    before = parity.bits(buf)
    _run_mixed_packed(d, out=buf[:M, :N])
    after = parity.bits(buf)
    ref, absdot, _ = parity.oracle_run(d)
    parity.compare(d, after[:M, :N], ref, absdot, f"prepacked {name} {M}x{N}x{K} tile {tile}")
    assert np.array_equal(after[:M, N:], before[:M, N:]), "wrote past N"
    assert np.array_equal(after[M:], before[M:]), "wrote past M"
    q.force_tile(7 if (tile == -1 and M <= 16 and name == "mx_a8w4") else tile)
    plain = parity.bits(parity.gpu_run(d))
    assert np.array_equal(after[:M, :N], plain), "prepacked and row-major B differ"


@pytest.mark.parametrize("name", ["mx_a8w4", "mx_a4w8"])
def test_prepacked_mixed_full_workload_sampled(name):
    d = inputs.make(name)
    q.force_tile(-1)
    _say(f"[prepacked] full {name}")
    out = _run_mixed_packed(d, out=parity.nan_out(d["M"], d["N"]))
    parity.check_full_grid(d, out, -1, f"prepacked full {name}",
                           np.random.default_rng(3).choice(d["M"], 8, replace=False))
