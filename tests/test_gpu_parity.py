"""GPU parity: the HIP library against the CPU oracle on the same seeded
inputs, through the C ABI (the ctypes binding).

INT8 bit-exact (bf16 output and int32 accumulator); FP8 / MX within
1e-2 * sum|a b| + 1 bf16 ulp per element with cosine >= 0.99999.
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


def _full_check(d, what, tile=None):
    _say(f"[parity] {what} M={d['M']} N={d['N']} K={d['K']} tile={tile}")
    if tile is not None:
        q.force_tile(tile)
    out = parity.gpu_run(d)
    torch.cuda.synchronize()
    got = parity.bits(out)
    ref, absdot, _ = parity.oracle_run(d)
    return parity.compare(d, got, ref, absdot, what)


# ------------------------------------------------------------------ INT8

@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5, 6, 7])
def test_i8_small_workload(bias, tile):
    d = inputs.make("i8_small", bias=bias)
    _full_check(d, f"i8_small bias={bias}", tile)


def test_i8_accumulator_exact():
    d = inputs.make("i8_small")
    A, B = parity.dev(d["A"]), parity.dev(d["B"])
    for tile in (0, 1, 2, 3, 4, 5, 6, 7):
        q.force_tile(tile)
        acc = q.qgemm_i8_acc_i32(A, B)
        torch.cuda.synchronize()
        _, _, ref = parity.oracle_run(d)
        assert np.array_equal(acc.cpu().numpy(), ref), f"tile {tile}"
    # extreme values: all -128 x -128 over a deep K
    K = 8192
    A = torch.full((3, K), -128, dtype=torch.int8, device="cuda")
    acc = q.qgemm_i8_acc_i32(A, A)
    assert (acc.cpu().numpy() == K * 16384).all()


def test_i8_signed_zero_and_subnormals():
    """No-bias epilogue keeps -0 (comfy-kitchen PR #174, Summary) and fp32
    subnormals; the same rows with a +0 bias give +0."""
    d = inputs.make("i8_small", bias=False)
    A, sa, sb = d["A"].copy(), d["scale_a"].copy(), d["scale_b"].copy()
    A[0:8] = 0
    sa[0:8] = -np.abs(sa[0:8])
    # rows 8..15: acc = -1 exactly in column 0, scales push it below fp32's range
    A[8:16] = 0
    A[8:16, 0] = -1
    B = d["B"].copy()
    B[0] = 0
    B[0, 0] = 1
    sa[8:16] = np.float32(2.0 ** -100)
    sb[0] = np.float32(2.0 ** -50)
    # row 16: acc = +1 in column 1 with 2^-100 * 2^-30 = 2^-130 (fp32 subnormal)
    A[16] = 0
    A[16, 1] = 1
    B[1] = 0
    B[1, 1] = 1
    sa[16] = np.float32(2.0 ** -100)
    sb[1] = np.float32(2.0 ** -30)
    d2 = dict(d, A=A, B=B, scale_a=sa, scale_b=sb)
    out = parity.bits(parity.gpu_run(d2))
    ref, _, _ = parity.oracle_run(d2)
    assert np.array_equal(out, ref)
    assert (out[0:8] == 0x8000).all()
    assert (out[8:16, 0] == 0x8000).all()
    assert out[16, 1] == 0x0008
    d3 = dict(d2, bias=np.zeros(d["N"], np.uint16))
    out3 = parity.bits(parity.gpu_run(d3))
    assert (out3[0:8] == 0).all() and (out3[8:16, 0] == 0).all()


EDGE_SHAPES = [(1, 1, 32), (17, 31, 64), (48, 33, 96), (100, 2112, 256), (255, 256, 512),
               (256, 255, 640), (257, 300, 1280), (1000, 129, 2048)]


@pytest.mark.parametrize("M,N,K", EDGE_SHAPES)
def test_i8_edges_canaries(M, N, K):
    """Ragged shapes, NaN-filled output with canary columns (ldc > N) and a
    canary row block: nothing outside [0,M) x [0,N) may change."""
    d = inputs.make("i8_small", M=M, N=N, K=K)
    ldc = N + (-N) % 8 + 8
    buf = torch.full((M + 3, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
    before = parity.bits(buf)
    out = buf[:M, :N]
    parity.gpu_run(d, out=out)
    after = parity.bits(buf)
    ref, _, _ = parity.oracle_run(d)
    parity.compare(d, after[:M, :N], ref, None, f"i8 {M}x{N}x{K}")
    assert np.array_equal(after[:M, N:], before[:M, N:]), "wrote past N"
    assert np.array_equal(after[M:], before[M:]), "wrote past M"


def test_i8_empty_is_noop():
    A = torch.zeros((0, 64), dtype=torch.int8, device="cuda")
    B = torch.zeros((5, 64), dtype=torch.int8, device="cuda")
    out = q.qgemm_i8_rowwise(A, B, torch.zeros(0, device="cuda"), torch.ones(5, device="cuda"))
    assert out.shape == (0, 5)


# ------------------------------------------------------------------ FP8

@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (17, 33, 96), (300, 2112, 1024)])
@pytest.mark.parametrize("bias", [False, True])
def test_f8_small(M, N, K, bias):
    d = inputs.make("f8_ptpc", M=M, N=N, K=K, bias=bias)
    _full_check(d, f"f8 {M}x{N}x{K} bias={bias}")


# ------------------------------------------------------------------ MX

@pytest.mark.parametrize("name", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (33, 70, 96), (300, 520, 1024),
                                   (129, 64, 160)])
@pytest.mark.parametrize("bias", [False, True])
def test_mx_small(name, M, N, K, bias):
    d = inputs.make(name, M=M, N=N, K=K, bias=bias)
    _full_check(d, f"{name} {M}x{N}x{K} bias={bias}")


@pytest.mark.parametrize("name", ["mxfp8", "mxfp4"])
def test_mx_other_b_layout(name):
    """mxfp8 with 1x32 B scales and mxfp4 with 32x32 B scales."""
    rng = np.random.default_rng(77)
    d = inputs.make(name, M=130, N=96, K=512)
    fmt = d["fmt"]
    brows = 1 if d["b_rows_per_scale"] == 32 else 32
    xb = rng.standard_normal((96, 512)).astype(np.float32)
    cb, sb = inputs.mx_quantise(xb, fmt, brows)
    if fmt == "e2m1":
        cb = inputs.pack_e2m1(cb)
    d2 = dict(d, B=cb, scale_b=sb, b_rows_per_scale=brows)
    _full_check(d2, f"{name} B-scale rows {brows}")


@pytest.mark.parametrize("name", ["mxfp8", "mxfp4"])
def test_mx_random_scales_repeated(name):
    """Random per-block scales (a stale or misrouted scale shows at once),
    output NaN-filled before each of 12 launches; every launch must match the
    oracle and equal the first bit for bit."""
    rng = np.random.default_rng(5)
    d = inputs.make(name, M=512, N=512, K=1280)
    d = dict(d, scale_a=rng.integers(118, 136, d["scale_a"].shape, dtype=np.uint8),
             scale_b=rng.integers(118, 136, d["scale_b"].shape, dtype=np.uint8))
    ref, absdot, _ = parity.oracle_run(d)
    first = None
    out = torch.empty((512, 512), dtype=torch.bfloat16, device="cuda")
    for it in range(12):
        out.fill_(float("nan"))
        parity.gpu_run(d, out=out)
        got = parity.bits(out)
        if first is None:
            parity.compare(d, got, ref, absdot, f"{name} launch 0")
            first = got
        else:
            assert np.array_equal(got, first), f"launch {it} differs"


# ------------------------------------------------------------------ variants

@pytest.mark.parametrize("name", ["i8_small", "f8_ptpc", "mxfp8", "mxfp4"])
def test_tile_variants_identical(name):
    """Tiles 0-3 run each output's accumulation as the same sequence of MFMAs,
    so they agree bit for bit; the LDS-fetch kernels (tiles 4-7) group K
    blocks into MFMAs differently, so they are bit-identical for INT8 and
    within the tolerance for FP8 / MX (and identical to each other: their
    per-output MFMA sequences match)."""
    d = inputs.make(name, M=300, N=280, K=512)
    outs = []
    for tile in (0, 1, 2, 3, 4, 5, 6, 7):
        q.force_tile(tile)
        outs.append(parity.bits(parity.gpu_run(d)))
    for t in (1, 2, 3):
        assert np.array_equal(outs[0], outs[t]), f"tile {t}"
    for t in (5, 6, 7):
        assert np.array_equal(outs[4], outs[t]), f"tiles 4 and {t}"
    if d["kind"] == "i8":
        assert np.array_equal(outs[0], outs[4])
    else:
        ref, absdot, _ = parity.oracle_run(d)
        parity.compare(d, outs[4], ref, absdot, f"{name} tile 4")


DMA_SHAPES = [(1, 1, 256), (17, 33, 512), (255, 257, 1024), (300, 520, 2048), (513, 64, 256)]


@pytest.mark.parametrize("tile", [4, 5, 6, 7])
@pytest.mark.parametrize("name", ["i8_small", "f8_ptpc", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("M,N,K", DMA_SHAPES)
def test_dma_kernel_edges(name, M, N, K, tile):
    """The LDS-fetch kernels on ragged M / N, NaN-filled output with canaries
    beyond N and M (K a whole number of their stages)."""
    kk = K if name != "mxfp4" else 2 * K      # e2m1: K elements are K/2 bytes
    d = inputs.make(name, M=M, N=N, K=kk, bias=(M % 2 == 1))
    q.force_tile(tile)
    ldc = N + (-N) % 8 + 8
    buf = torch.full((M + 3, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
    before = parity.bits(buf)
    parity.gpu_run(d, out=buf[:M, :N])
    after = parity.bits(buf)
    ref, absdot, _ = parity.oracle_run(d)
    parity.compare(d, after[:M, :N], ref, absdot, f"dma {name} {M}x{N}x{kk}")
    assert np.array_equal(after[:M, N:], before[:M, N:]), "wrote past N"
    assert np.array_equal(after[M:], before[M:]), "wrote past M"


@pytest.mark.parametrize("tile", [4, 5, 6, 7])
@pytest.mark.parametrize("name", ["mxfp8", "mxfp4"])
def test_dma_kernel_other_b_layout_and_random_scales(name, tile):
    rng = np.random.default_rng(78)
    d = inputs.make(name, M=260, N=300, K=1024)
    fmt = d["fmt"]
    brows = 1 if d["b_rows_per_scale"] == 32 else 32
    cb, sb = inputs.mx_quantise(rng.standard_normal((300, 1024)).astype(np.float32), fmt, brows)
    if fmt == "e2m1":
        cb = inputs.pack_e2m1(cb)
    d = dict(d, B=cb, scale_b=sb, b_rows_per_scale=brows,
             scale_a=rng.integers(118, 136, d["scale_a"].shape, dtype=np.uint8))
    q.force_tile(tile)
    ref, absdot, _ = parity.oracle_run(d)
    first = None
    for it in range(6):
        got = parity.bits(parity.gpu_run(d))
        if first is None:
            parity.compare(d, got, ref, absdot, f"dma {name} B rows {brows}")
            first = got
        else:
            assert np.array_equal(got, first), f"launch {it} differs"


@pytest.mark.parametrize("tile", [-1, 4, 5, 7])
@pytest.mark.parametrize("brows", [1, 32])
@pytest.mark.parametrize("K", [1088, 2880])
def test_mx4_k64_stages_random_scales(K, brows, tile):
    """e2m1 at K % 128 == 64 (64-element stages, scale rows of K/32 = 4n + 2
    bytes): both B-scale layouts, random scale codes, bias, repeated launches
    bit-identical."""
    rng = np.random.default_rng(K + brows)
    d = inputs.make("mxfp4", M=300, N=264, K=K, bias=True)
    if brows == 32:
        cb, sb = inputs.mx_quantise(rng.standard_normal((264, K)).astype(np.float32), "e2m1", 32)
        d = dict(d, B=inputs.pack_e2m1(cb), scale_b=sb, b_rows_per_scale=32)
    d["scale_a"] = rng.integers(118, 136, d["scale_a"].shape, dtype=np.uint8)
    q.force_tile(tile)
    _say(f"[parity] mx4 K={K} brows={brows} tile={tile}")
    ref, absdot, _ = parity.oracle_run(d)
    first = None
    for it in range(3):
        got = parity.bits(parity.gpu_run(d))
        if first is None:
            parity.compare(d, got, ref, absdot, f"mx4 K={K} brows={brows} tile={tile}")
            first = got
        else:
            assert np.array_equal(got, first), f"launch {it} differs"


@pytest.mark.parametrize("tile", [4, 5, 6, 7])
def test_dma_tile_falls_back_when_k_does_not_fit(tile):
    d = inputs.make("i8_small", M=100, N=70, K=96)
    q.force_tile(tile)
    ref, _, _ = parity.oracle_run(d)
    parity.compare(d, parity.bits(parity.gpu_run(d)), ref, None, f"tile {tile} fallback K=96")


SKINNY_SHAPES = [(1, 1, 32), (1, 300, 512), (5, 33, 96), (16, 16, 1024), (17, 70, 224), (64, 129, 544),
                 (33, 2112, 7168)]


@pytest.mark.parametrize("tile", [8, 9])
@pytest.mark.parametrize("name", ["i8_small", "f8_ptpc", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("M,N,K", SKINNY_SHAPES)
def test_skinny_kernel_edges(name, M, N, K, tile):
    """The small-M kernel (eight waves splitting K, partial sums added in
    LDS) on ragged M / N / K, NaN-filled output with canaries beyond N and M;
    INT8 also bit for bit against the 256x256 register-staged tile.  MX: the
    32x32 B-scale recipe for e4m3 (a 16-column workgroup meets one or two
    scale rows), 1x32 for e2m1."""
    d = inputs.make(name, M=M, N=N, K=K, bias=(M % 2 == 1))
    q.force_tile(tile)
    ldc = N + (-N) % 8 + 8
    buf = torch.full((M + 3, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
    before = parity.bits(buf)
    parity.gpu_run(d, out=buf[:M, :N])
    after = parity.bits(buf)
    ref, absdot, _ = parity.oracle_run(d)
    parity.compare(d, after[:M, :N], ref, absdot, f"skinny {name} {M}x{N}x{K} tile {tile}")
    assert np.array_equal(after[:M, N:], before[:M, N:]), "wrote past N"
    assert np.array_equal(after[M:], before[M:]), "wrote past M"
    if d["kind"] == "i8":
        q.force_tile(0)
        assert np.array_equal(after[:M, :N], parity.bits(parity.gpu_run(d)))


@pytest.mark.parametrize("name,path", [("f8_ptpc", 1), ("mxfp8", 2), ("mxfp4", 3)])
@pytest.mark.parametrize("M", [1, 16, 64])
def test_skinny_table_choice_full_width(name, path, M):
    """M = 1, 16, 64 over each workload's full weight (FP8 2112 x 7168, MXFP8
    7168 x 2048, MXFP4 8192 x 8192), as the table launches it (the small-M
    kernel, for MX up to 16 rows), every output row checked."""
    d = inputs.make(name, M=M)
    q.force_tile(-1)
    if path >= 2 and M > 16:
        assert q.select_tile(path, M, d["N"], d["K"]) not in (8, 9)   # MX: 16-row form only
    else:
        assert q.select_tile(path, M, d["N"], d["K"]) in (8, 9)
    ref, absdot, _ = parity.oracle_run(d)
    parity.compare(d, parity.bits(parity.gpu_run(d)), ref, absdot, f"skinny {name} M={M}")


def test_non_default_stream():
    d = inputs.make("mxfp4", M=256, N=512, K=512)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = parity.gpu_run(d, stream=s)
    s.synchronize()
    ref, absdot, _ = parity.oracle_run(d)
    parity.compare(d, parity.bits(out), ref, absdot, "side stream")


# ------------------------------------------------------------------ full sizes

def _sample_rows(M, n, rng):
    tail = np.arange(max(0, M - 8), M)
    head = np.arange(0, min(8, M))
    mid = rng.choice(M, size=max(0, n - len(head) - len(tail)), replace=False)
    return np.unique(np.concatenate([head, mid, tail]))


@pytest.mark.parametrize("tile", [-1, 4, 5, 6])
@pytest.mark.parametrize("name", ["f8_ptpc", "mxfp8", "mxfp4", "i8_qkv"])
def test_full_workload_sampled(name, tile):
    """The workload at its full size, launched as the benchmark launches it
    (and on each LDS-fetch tile), into a NaN-filled C: every output written,
    and the first and last row of every tile band plus random rows (all
    columns) against the oracle."""
    d = inputs.make(name)
    _say(f"[parity] full {name} M={d['M']} N={d['N']} K={d['K']} tile {tile}")
    q.force_tile(tile)
    out = parity.gpu_run(d, out=parity.nan_out(d["M"], d["N"]))
    extra = _sample_rows(d["M"], 24, np.random.default_rng(1))
    worst, cos, n = parity.check_full_grid(d, out, tile, f"full {name} tile {tile}", extra)
    _say(f"[parity] full {name}: {n} rows, worst err/bound {worst:.3g} cos {cos:.8f}")


@pytest.mark.parametrize("tile", [4, 5, 6, 7])
@pytest.mark.parametrize("M,N,K", [(300, 520, 768), (257, 256, 1792), (64, 96, 256)])
def test_mx8_dma_kernel_scale_rows_of_8_byte_words(M, N, K, tile):
    """e4m3 MX on the LDS-fetch kernels with K a multiple of 256 but not of 512:
    each 4-stage round reads the first 8 bytes of a 16-byte scale chunk that
    may run past the row (into the next row, or past the range at the last
    one); random scale codes so that a misplaced scale leaves the bound."""
    d = inputs.make("mxfp8", M=M, N=N, K=K, bias=True)
    rng = np.random.default_rng(M + N + K)
    d["scale_a"] = rng.integers(112, 142, d["scale_a"].shape, dtype=np.uint8)
    d["scale_b"] = rng.integers(112, 142, d["scale_b"].shape, dtype=np.uint8)
    q.force_tile(tile)
    _say(f"[parity] mx8 K%512!=0 {M}x{N}x{K} tile {tile}")
    out = parity.gpu_run(d)
    torch.cuda.synchronize()
    ref, absdot, _ = parity.oracle_run(d)
    parity.compare(d, parity.bits(out), ref, absdot, f"mx8 {M}x{N}x{K} tile {tile}")


def test_mx8_pages_shape_sampled():
    """MXFP8 at 32768 x 7168 x 1792 (the MI355X MXFP8 shape of ROCm/mori PR
    #806's measurements), launched with the table's tile; sampled rows."""
    d = inputs.make("mxfp8", M=32768, N=7168, K=1792)
    assert q.select_tile(2, 32768, 7168, 1792) == 5
    _say("[parity] full mxfp8 32768x7168x1792")
    out = parity.gpu_run(d, out=parity.nan_out(d["M"], d["N"]))
    worst, cos, _ = parity.check_full_grid(d, out, -1, "full mxfp8 32768x7168x1792",
                                           _sample_rows(d["M"], 16, np.random.default_rng(4)))
    _say(f"[parity] full mxfp8 32768x7168x1792: worst err/bound {worst:.3g} cos {cos:.8f}")


@pytest.mark.parametrize("tile,K", [(-1, 131040), (0, 131040), (5, 130816)])
def test_i8_largest_k(tile, K):
    """The largest K the int32 accumulator admits (K * 128^2 < 2^31, K a
    multiple of 32; 130816 for the LDS-fetch tile, a multiple of 256), with
    every product at the extreme: A = -128, B = -128 gives acc = K * 16384
    exactly, 2.1e9, and the bf16 output bit-exact against the oracle."""
    M, N = 3, 40
    d = inputs.make("i8_small", M=M, N=N, K=K)
    d["A"] = np.full((M, K), -128, np.int8)
    d["B"] = np.full((N, K), -128, np.int8)
    d["B"][1::2, ::2] = 127          # odd rows of B: alternating -128 / 127
    q.force_tile(tile)
    _say(f"[parity] i8 largest K={K} tile {tile}")
    acc = q.qgemm_i8_acc_i32(parity.dev(d["A"]), parity.dev(d["B"]))
    out = parity.gpu_run(d)
    torch.cuda.synchronize()
    ref, _, ref_acc = parity.oracle_run(d)
    assert acc[0, 0].item() == K * 16384
    assert np.array_equal(acc.cpu().numpy(), ref_acc)
    parity.compare(d, parity.bits(out), ref, None, f"i8 K={K} tile {tile}")
