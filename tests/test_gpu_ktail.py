"""GPU parity of the LDS-fetch kernels when K is not a whole number of their
4-stage rounds (256 bytes of an operand row): the last round holds one to
three stages, and the stages past K must add nothing.

Each operand row is padded past K with poison (int8 127, e4m3 NaN, e2m1 6.0),
so a stage past K that read the row's own padding would change the result.
Every scale of the rows next to the ones checked is NaN (ue8m0 255) or
infinite (blockscale fp32): a kernel whose masked tail took any word of the
next scale row would turn a checked output into NaN.  Checked rows and
columns are compared with the CPU oracle: INT8 bit-exact, FP8 / MX within
1e-2 * sum|a b| + 1 bf16 ulp and cosine >= 0.99999.
"""
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


PAD = 64          # bytes of poison after each operand row


def _padded(x, poison):
    x = np.ascontiguousarray(x)
    buf = np.empty((x.shape[0], x.shape[1] + PAD), dtype=x.dtype)
    buf.view(np.uint8)[...] = poison
    buf[:, :x.shape[1]] = x
    return torch.from_numpy(buf).cuda()[:, :x.shape[1]]


def _poison_bytes(d):
    if d["kind"] == "i8":
        return 0x7F, 0x7F
    if d["kind"] in ("f8", "f8b"):
        return 0x7F, 0x7F                         # e4m3 NaN
    fa, fb = (d["fmt"].split("/") if "/" in d["fmt"] else (d["fmt"], d["fmt"]))
    code = {"e4m3": 0x7F, "e2m1": 0x77}
    return code[fa], code[fb]


def _run(d, At, Bt):
    dev = parity.dev
    bias = None if d["bias"] is None else dev(d["bias"].view(np.int16))
    sa, sb = dev(d["scale_a"]), dev(d["scale_b"])
    if d["kind"] == "i8":
        return q.qgemm_i8_rowwise(At, Bt, sa, sb, bias)
    if d["kind"] == "f8":
        return q.qgemm_f8_pertoken(At, Bt, sa, sb, bias)
    if d["kind"] == "f8b":
        return q.qgemm_f8_blockscale(At, Bt, sa, sb, bias)
    if "/" in d["fmt"]:
        fa, fb = (q.QGEMM_MX_E4M3 if f == "e4m3" else q.QGEMM_MX_E2M1 for f in d["fmt"].split("/"))
        return q.qgemm_mx_mixed(fa, fb, At, Bt, sa, sb, d["b_rows_per_scale"], bias)
    fmt = q.QGEMM_MX_E4M3 if d["fmt"] == "e4m3" else q.QGEMM_MX_E2M1
    return q.qgemm_mx(fmt, At, Bt, sa, sb, d["b_rows_per_scale"], bias)


def _poison_scales(d, keep=0):
    """Every scale of the A and B scale rows of parity 1 - keep is non-finite;
    returns the output rows and columns whose scales are all finite."""
    M, N = d["M"], d["N"]
    if d["kind"] in ("i8", "f8"):
        return np.arange(M), np.arange(N)        # scales applied per row in the epilogue
    sa, sb = d["scale_a"].copy(), d["scale_b"].copy()
    bad = np.float32(np.inf) if d["kind"] == "f8b" else np.uint8(255)
    sa[1 - keep::2, :] = bad  # every word of a neighbouring row, so each masked word position is checked
    sb[1 - keep::2, :] = bad
    d["scale_a"], d["scale_b"] = sa, sb
    group = 128 if d["kind"] == "f8b" else d["b_rows_per_scale"]
    cols = np.arange(N)
    return np.arange(keep, M, 2), cols[(cols // group) % 2 == keep]


def _check(name, M, N, K, tile, brows=None, bias=True, keep=0):
    q.force_tile(tile)
    d = inputs.make(name, M=M, N=N, K=K, bias=bias)
    if brows == 1 and d["kind"] == "mx" and d["b_rows_per_scale"] != 1:
        rng = np.random.default_rng(K + tile)
        xb = rng.standard_normal((N, K)).astype(np.float32)
        d["B"], d["scale_b"] = inputs.mx_quantise(xb, d["fmt"], 1)
        d["b_rows_per_scale"] = 1
    rows, cols = _poison_scales(d, keep)
    pa, pb = _poison_bytes(d)
    _say(f"[ktail] {name} {M}x{N}x{K} tile={tile} brows={d['b_rows_per_scale']}")
    out = _run(d, _padded(d["A"], pa), _padded(d["B"], pb))
    torch.cuda.synchronize()
    got = parity.bits(out)[rows][:, cols]
    ref, absdot, _ = parity.oracle_run(d, rows=rows)
    ref = ref[:, cols]
    absdot = None if absdot is None else absdot[:, cols]
    parity.compare(d, got, ref, absdot, f"ktail {name} {M}x{N}x{K} tile {tile}")


DMA_TILES = [4, 5, 6, 7]


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("name,K", [("i8_small", 64), ("i8_small", 192), ("i8_small", 320), ("i8_small", 1088),
                                    ("f8_ptpc", 128), ("f8_ptpc", 448)])
def test_partial_round_i8_f8(name, K, tile):
    _check(name, 200, 300, K, tile)


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("brows", [1, 32])
@pytest.mark.parametrize("K", [128, 384, 1152])
def test_partial_round_mxfp8(K, brows, tile):
    _check("mxfp8", 200, 300, K, tile, brows=brows)


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("K", [128, 384, 640])
def test_partial_round_mxfp4(K, tile):
    _check("mxfp4", 200, 300, K, tile)


@pytest.mark.parametrize("tile", [7, 10])
@pytest.mark.parametrize("K", [128, 384, 1152])
def test_partial_round_blockscale(K, tile):
    _check("f8_block", 280, 300, K, tile)


@pytest.mark.parametrize("tile", [4, 5, 7])
@pytest.mark.parametrize("K", [128, 384, 640])
def test_partial_round_mixed(K, tile):
    _check("mx_a8w4", 200, 300, K, tile)


@pytest.mark.parametrize("tile", [4, 5, 7])
@pytest.mark.parametrize("K", [128, 384, 640])
def test_partial_round_mixed_e2m1_a(K, tile):
    _check("mx_a4w8", 200, 300, K, tile)


# K % 128 == 64 on the e4m3-staged MX paths: scale rows of K/32 = 4n + 2
# bytes (every other row starts 2 bytes into a dword), a last round of one or
# three stages whose last scale word is half past K.  Both row parities are
# checked against poisoned neighbours.
@pytest.mark.parametrize("keep", [0, 1])
@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("brows", [1, 32])
@pytest.mark.parametrize("K", [64, 192, 320, 1216])
@pytest.mark.parametrize("M,N", [(200, 300), (201, 289)])   # odd: the last scale row ends mid-dword
def test_k64_mxfp8(M, N, K, brows, tile, keep):
    _check("mxfp8", M, N, K, tile, brows=brows, keep=keep)


@pytest.mark.parametrize("keep", [0, 1])
@pytest.mark.parametrize("tile", [4, 5, 7])
@pytest.mark.parametrize("name", ["mx_a8w4", "mx_a4w8"])
@pytest.mark.parametrize("K", [64, 192, 704])
@pytest.mark.parametrize("M,N", [(200, 300), (201, 289)])
def test_k64_mixed(name, M, N, K, tile, keep):
    _check(name, M, N, K, tile, keep=keep)


@pytest.mark.parametrize("keep", [0, 1])
@pytest.mark.parametrize("tile", [4, 5, 7])
@pytest.mark.parametrize("K", [64, 192, 320, 1216])
@pytest.mark.parametrize("M,N", [(200, 300), (201, 289)])
def test_k64_mxfp4(M, N, K, tile, keep):
    """e2m1 at K % 128 == 64: both operands in 64-element stages (32-byte rows,
    the row's last 32 bytes a stage of their own)."""
    _check("mxfp4", M, N, K, tile, keep=keep)


def test_k64_full_size_mxfp4():
    """8192 x 8192 x 8256 e2m1 (129 stages of 64 elements) in the table's
    launch, into a NaN-filled C, on the band rows and sampled rows."""
    d = inputs.make("mxfp4", K=8256)
    assert q.select_tile(3, d["M"], d["N"], d["K"]) == 5
    _say(f"[ktail] full mxfp4 {d['M']}x{d['N']}x{d['K']}")
    out = parity.gpu_run(d, out=parity.nan_out(d["M"], d["N"]))
    rng = np.random.default_rng(6)
    parity.check_full_grid(d, out, -1, "k64 full mxfp4", rng.choice(d["M"], 8, replace=False))


def test_k64_full_size_mxfp8():
    """16384 x 7168 x 2112 (K/32 = 66, 33 stages) in the launch the benchmark
    uses for MXFP8, into a NaN-filled C, on sampled whole rows of both
    parities."""
    d = inputs.make("mxfp8", K=2112)
    assert q.select_tile(2, d["M"], d["N"], d["K"]) == 5
    _say(f"[ktail] full mxfp8 {d['M']}x{d['N']}x{d['K']}")
    out = parity.gpu_run(d, out=parity.nan_out(d["M"], d["N"]))
    rng = np.random.default_rng(5)
    parity.check_full_grid(d, out, -1, "k64 full mxfp8", rng.choice(d["M"], 16, replace=False))


# K % 64 == 32 (K/32 odd) on the e4m3-staged MX paths and e2m1: the last
# stage holds 32 K elements (its other chunks are fetched as zeros), scale
# rows start 1-3 bytes into a dword and the last live scale word ends one or
# three bytes into the row's end; against poisoned operand padding and
# poisoned neighbouring scale rows.
@pytest.mark.parametrize("keep", [0, 1])
@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("brows", [1, 32])
@pytest.mark.parametrize("K", [32, 96, 224, 288, 1120])
@pytest.mark.parametrize("M,N", [(200, 300), (201, 289)])
def test_k32_mxfp8(M, N, K, brows, tile, keep):
    _check("mxfp8", M, N, K, tile, brows=brows, keep=keep)


@pytest.mark.parametrize("keep", [0, 1])
@pytest.mark.parametrize("tile", [4, 5, 7])
@pytest.mark.parametrize("name", ["mx_a8w4", "mx_a4w8"])
@pytest.mark.parametrize("K", [32, 96, 224, 736])
@pytest.mark.parametrize("M,N", [(200, 300), (201, 289)])
def test_k32_mixed(name, M, N, K, tile, keep):
    _check(name, M, N, K, tile, keep=keep)


@pytest.mark.parametrize("tile", [8, 9])
@pytest.mark.parametrize("K", [32, 96, 224, 736])
@pytest.mark.parametrize("M", [1, 13])
def test_k32_mixed_small_m(M, K, tile):
    """e4m3 x e2m1 at K % 64 == 32 in the small-M kernel (16-byte e2m1 row
    ends fetched as zeros past K)."""
    _check("mx_a8w4", M, 300, K, tile)


@pytest.mark.parametrize("keep", [0, 1])
@pytest.mark.parametrize("tile", [4, 5, 7])
@pytest.mark.parametrize("K", [32, 96, 160, 224, 1184])
@pytest.mark.parametrize("M,N", [(200, 300), (201, 289)])
def test_k32_mxfp4(M, N, K, tile, keep):
    """e2m1 at K % 128 == 32 or 96: 64-element stages, the last one 16 bytes
    of each row."""
    _check("mxfp4", M, N, K, tile, keep=keep)


def test_k32_full_size_mxfp8():
    """16384 x 7168 x 2080 (K/32 = 65: 32.5 stages) in the launch the
    benchmark uses for MXFP8, into a NaN-filled C, on the band rows and
    sampled rows."""
    d = inputs.make("mxfp8", K=2080)
    assert q.select_tile(2, d["M"], d["N"], d["K"]) == 5
    _say(f"[ktail] full mxfp8 {d['M']}x{d['N']}x{d['K']}")
    out = parity.gpu_run(d, out=parity.nan_out(d["M"], d["N"]))
    rng = np.random.default_rng(7)
    parity.check_full_grid(d, out, -1, "k32 full mxfp8", rng.choice(d["M"], 16, replace=False))


def test_k32_full_size_mxfp4():
    """8192 x 8192 x 8224 e2m1 (128.5 stages of 64 elements) in the table's
    launch, into a NaN-filled C, on the band rows and sampled rows."""
    d = inputs.make("mxfp4", K=8224)
    assert q.select_tile(3, d["M"], d["N"], d["K"]) == 5
    _say(f"[ktail] full mxfp4 {d['M']}x{d['N']}x{d['K']}")
    out = parity.gpu_run(d, out=parity.nan_out(d["M"], d["N"]))
    rng = np.random.default_rng(8)
    parity.check_full_grid(d, out, -1, "k32 full mxfp4", rng.choice(d["M"], 8, replace=False))


def test_partial_round_full_size_mxfp8():
    """16384 x 7168 x 2176 (K/32 = 68: a last round of two stages) in the
    launch the benchmark uses for MXFP8, on sampled whole rows."""
    d = inputs.make("mxfp8", K=2176)
    assert q.select_tile(2, d["M"], d["N"], d["K"]) == 5
    _say(f"[ktail] full mxfp8 {d['M']}x{d['N']}x{d['K']}")
    out = parity.gpu_run(d, out=parity.nan_out(d["M"], d["N"]))
    rng = np.random.default_rng(3)
    parity.check_full_grid(d, out, -1, "ktail full mxfp8", rng.choice(d["M"], 16, replace=False))


@pytest.mark.parametrize("name,tile", [("f8_block", 8), ("f8_block", 9), ("mx_a8w4", 8), ("mxfp8", 8),
                                       ("mxfp4", 8), ("i8_small", 9), ("f8_ptpc", 8)])
@pytest.mark.parametrize("K", [128, 384])
def test_small_m_kernel_k_not_multiple_of_256(name, tile, K):
    """The small-M kernel (eight waves splitting K) at K that the LDS-fetch
    kernels take as a partial round: same poisoned padding and scales."""
    M = 12 if tile == 8 else 40
    _check(name, M, 300, K, tile)


@pytest.mark.parametrize("name,shape,path,tile", [("f8_block", (16384, 7168, 2176), 4, 10),
                                                  ("i8_qkv", (30000, 21504, 5440), 0, 5)])
def test_partial_round_full_size(name, shape, path, tile):
    """Blockscale 16384 x 7168 x 2176 (17 blocks: a last round of one block)
    and INT8 30000 x 21504 x 5440 (85 stages: a last round of one stage), in
    the launch the benchmark uses, into a NaN-filled C; the first and last
    row of every tile band and random rows."""
    M, N, K = shape
    assert q.select_tile(path, M, N, K) == tile
    d = inputs.make(name, M=M, N=N, K=K)
    _say(f"[ktail] full {name} {M}x{N}x{K}")
    out = parity.gpu_run(d, out=parity.nan_out(M, N))
    rng = np.random.default_rng(4)
    parity.check_full_grid(d, out, tile, f"ktail full {name}", rng.choice(M, 12, replace=False))
