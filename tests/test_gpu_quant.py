"""GPU parity of the activation quantisers: codes and scales bit for bit
against the CPU oracle on the same seeded bf16 inputs, through the C ABI;
nothing outside the outputs' [M, K] is written; the quantised operands feed
the GEMMs (the GEMM then within its own tolerance of the oracle GEMM on the
oracle's operands, which are the same bytes)."""
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


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


def _bf16(x):
    return inputs.bf16_bits(np.asarray(x, np.float32))


def _special_rows(K):
    """Rows that reach the edge cases: zeros and signed zeros, bf16
    subnormals, the top of the bf16 range, exact e4m3 midpoints at scale 1
    (a row whose amax is 448), e2m1 midpoints, and values that round to zero
    with a negative sign."""
    rows = []
    z = np.zeros(K, np.float32)
    z[1::2] = -0.0
    rows.append(z)
    rng = np.random.default_rng(7)
    rows.append((rng.standard_normal(K) * 2.0 ** -128).astype(np.float32))          # subnormal
    rows.append((rng.standard_normal(K) * 1e37).astype(np.float32))                 # near the top
    mid = np.array([1.0625, 1.1875, -1.0625, 0.0146484375, 0.0009765625, 0.0029296875, 455.0, 448.0],
                   np.float32)
    rows.append(np.resize(mid, K))
    e2 = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.75, -5.0], np.float32)
    rows.append(np.resize(e2, K))
    t = (rng.standard_normal(K) * 1e-3).astype(np.float32)
    t[0] = 1000.0
    rows.append(t)                                                                  # many round to +-0
    return _bf16(np.stack(rows))


def _inputs(M, K, seed):
    X = inputs.make_activations(M, K, seed=seed)
    sp = _special_rows(K)
    n = min(M, len(sp))
    X[:n] = sp[:n]
    return X


def _dev(X, ld=None):
    M, K = X.shape
    ld = ld or K
    buf = torch.zeros((M, ld), dtype=torch.int16, device="cuda")
    buf[:, :K] = torch.from_numpy(X.view(np.int16)).cuda()
    return buf[:, :K]


QUANT_SHAPES = [(1, 32), (3, 64), (6, 96), (17, 7168), (5, 8192), (7, 10240), (64, 256), (300, 544), (1, 65536)]


@pytest.mark.parametrize("M,K", QUANT_SHAPES)
def test_quant_f8_pertoken_bit_exact(orc, M, K):
    _say(f"[quant] f8 pertoken M={M} K={K}")
    X = _inputs(M, K, seed=M * 131 + K)
    ldq = K + 32
    qbuf = torch.full((M + 2, ldq), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((M + 4,), float("nan"), dtype=torch.float32, device="cuda")
    Qv, sv = q.qgemm_quant_f8_pertoken(_dev(X, ld=K + 64), out=qbuf[:M, :K], scale=sbuf[:M])
    torch.cuda.synchronize()
    Qr, sr = orc.quant_f8_pertoken(X)
    got_q = qbuf.cpu().numpy()
    got_s = sbuf.cpu().numpy()
    assert np.array_equal(got_q[:M, :K], Qr), f"{np.count_nonzero(got_q[:M, :K] != Qr)} codes differ"
    assert np.array_equal(got_s[:M].view(np.uint32), sr.view(np.uint32))
    assert (got_q[:M, K:] == 0xA5).all() and (got_q[M:] == 0xA5).all(), "wrote outside Q"
    assert np.isnan(got_s[M:]).all(), "wrote outside scale"


@pytest.mark.parametrize("fmt", [q.QGEMM_MX_E4M3, q.QGEMM_MX_E2M1])
@pytest.mark.parametrize("M,K", QUANT_SHAPES)
def test_quant_mx_bit_exact(orc, fmt, M, K):
    _say(f"[quant] mx fmt={fmt} M={M} K={K}")
    X = _inputs(M, K, seed=M * 137 + K + fmt)
    row = K if fmt == q.QGEMM_MX_E4M3 else K // 2
    ldq = row + (-row) % 16 + 16
    qbuf = torch.full((M + 2, ldq), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((M + 2, K // 32 + 3), 0x5A, dtype=torch.uint8, device="cuda")
    q.qgemm_quant_mx(fmt, _dev(X, ld=K + 8), out=qbuf[:M, :row], scales=sbuf[:M, :K // 32])
    torch.cuda.synchronize()
    Qr, Sr = orc.quant_mx(fmt, X)
    got_q = qbuf.cpu().numpy()
    got_s = sbuf.cpu().numpy()
    assert np.array_equal(got_q[:M, :row], Qr), f"{np.count_nonzero(got_q[:M, :row] != Qr)} codes differ"
    assert np.array_equal(got_s[:M, :K // 32], Sr)
    assert (got_q[:M, row:] == 0xA5).all() and (got_q[M:] == 0xA5).all(), "wrote outside Q"
    assert (got_s[:M, K // 32:] == 0x5A).all() and (got_s[M:] == 0x5A).all(), "wrote outside S"


BLOCK_SHAPES = [(3, 128), (17, 7168), (5, 8192), (64, 256), (300, 640), (1, 65536)]


@pytest.mark.parametrize("M,K", BLOCK_SHAPES)
def test_quant_f8_block_bit_exact(orc, M, K):
    _say(f"[quant] f8 block M={M} K={K}")
    X = _inputs(M, K, seed=M * 139 + K)
    qbuf = torch.full((M + 2, K + 32), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((M + 2, K // 128 + 3), float("nan"), dtype=torch.float32, device="cuda")
    q.qgemm_quant_f8_block(_dev(X, ld=K + 64), out=qbuf[:M, :K], scales=sbuf[:M, :K // 128])
    torch.cuda.synchronize()
    Qr, Sr = orc.quant_f8_block(X)
    got_q = qbuf.cpu().numpy()
    got_s = sbuf.cpu().numpy()
    assert np.array_equal(got_q[:M, :K], Qr), f"{np.count_nonzero(got_q[:M, :K] != Qr)} codes differ"
    assert np.array_equal(got_s[:M, :K // 128].view(np.uint32), Sr.view(np.uint32))
    assert (got_q[:M, K:] == 0xA5).all() and (got_q[M:] == 0xA5).all(), "wrote outside Q"
    assert np.isnan(got_s[:M, K // 128:]).all() and np.isnan(got_s[M:]).all(), "wrote outside S"


@pytest.mark.parametrize("which", ["f8", "mxfp8", "mxfp4", "f8_block"])
def test_quant_full_workload_shape(orc, which):
    """The activation shape of each GEMM workload, as the benchmark times it;
    every code and scale compared."""
    _, M, K = inputs.QUANT_SHAPES[which]
    _say(f"[quant] full {which} M={M} K={K}")
    X = inputs.make_activations(M, K)
    Xd = torch.from_numpy(X.view(np.int16)).cuda()
    if which == "f8":
        Qd, sd = q.qgemm_quant_f8_pertoken(Xd)
        Qr, sr = orc.quant_f8_pertoken(X)
        assert np.array_equal(sd.cpu().numpy().view(np.uint32), sr.view(np.uint32))
    elif which == "f8_block":
        Qd, sd = q.qgemm_quant_f8_block(Xd)
        Qr, sr = orc.quant_f8_block(X)
        assert np.array_equal(sd.cpu().numpy().view(np.uint32), sr.view(np.uint32))
    else:
        fmt = q.QGEMM_MX_E4M3 if which == "mxfp8" else q.QGEMM_MX_E2M1
        Qd, sd = q.qgemm_quant_mx(fmt, Xd)
        Qr, sr = orc.quant_mx(fmt, X)
        assert np.array_equal(sd.cpu().numpy(), sr)
    assert np.array_equal(Qd.cpu().numpy(), Qr)


def test_quantised_operands_feed_the_gemms(orc):
    """Quantise activations and weights on the GPU, multiply on the GPU, and
    compare with the oracle GEMM on the oracle's quantisation of the same
    bf16 values (FP8 per-token x per-channel, MXFP8 and MXFP4 with 1x32 B
    scales)."""
    M, N, K = 200, 96, 512
    Xa = inputs.make_activations(M, K, seed=41)
    Xb = inputs.make_activations(N, K, seed=42)
    Ad, Bd = (torch.from_numpy(v.view(np.int16)).cuda() for v in (Xa, Xb))
    qa, sa = q.qgemm_quant_f8_pertoken(Ad)
    qb, sb = q.qgemm_quant_f8_pertoken(Bd)
    C = parity.bits(q.qgemm_f8_pertoken(qa, qb, sa, sb))
    (QA, SA), (QB, SB) = orc.quant_f8_pertoken(Xa), orc.quant_f8_pertoken(Xb)
    ref, _, absdot = orc.f8_pertoken(QA, QB, SA, SB)
    d = dict(kind="f8", M=M, N=N, K=K)
    parity.compare(d, C, ref, absdot, "quantised f8")
    for fmt in (q.QGEMM_MX_E4M3, q.QGEMM_MX_E2M1):
        qa, sa = q.qgemm_quant_mx(fmt, Ad)
        qb, sb = q.qgemm_quant_mx(fmt, Bd)
        C = parity.bits(q.qgemm_mx(fmt, qa, qb, sa, sb, q.QGEMM_MX_BSCALE_1x32))
        (QA, SA), (QB, SB) = orc.quant_mx(fmt, Xa), orc.quant_mx(fmt, Xb)
        ref, _, absdot = orc.mx(fmt, QA, QB, SA, SB, 1, K)
        parity.compare(dict(kind="mx", M=M, N=N, K=K), C, ref, absdot, f"quantised mx {fmt}")


def test_quantised_blockscale_operand_feeds_the_gemm(orc):
    """Activations quantised per 1x128 block on the GPU feed the blockscale
    GEMM (weights in 128x128 blocks from the input recipe); compared with the
    oracle GEMM on the oracle's quantisation of the same bf16 values."""
    M, N, K = 200, 300, 1024
    Xa = inputs.make_activations(M, K, seed=43)
    qa, sa = q.qgemm_quant_f8_block(torch.from_numpy(Xa.view(np.int16)).cuda())
    xb = np.random.default_rng(44).standard_normal((N, K)).astype(np.float32)
    B, sb = inputs.block_quantise_e4m3(xb, 128)
    C = parity.bits(q.qgemm_f8_blockscale(qa, parity.dev(B), sa, parity.dev(sb)))
    QA, SA = orc.quant_f8_block(Xa)
    assert np.array_equal(qa.cpu().numpy(), QA)
    ref, _, absdot = orc.f8_blockscale(QA, B, SA, sb)
    parity.compare(dict(kind="f8b", M=M, N=N, K=K), C, ref, absdot, "quantised blockscale")


def _near_midpoint_rows(n_scales=6000, seed=12):
    """Rows of 128 bf16 values: element 0 is the row's amax (so the scale is
    s = fp32(amax / 448), an inexact quotient), the rest are bf16 values x
    whose binary32 quotient x / s lies within 16 units in the last place of
    an e4m3 rounding midpoint (found by search), or of the e4m3 subnormal
    boundary; filler below amax elsewhere.  Returns (rows, hits)."""
    rng = np.random.default_rng(seed)
    # every positive bf16 value from 2^-14 up to 2^7
    allv = (np.arange(0x3880, 0x4300, dtype=np.uint32) << 16).view(np.float32)
    rows, hits = [], 0
    for amax in (rng.uniform(0.5, 100.0, n_scales)).astype(np.float32):
        amax = (np.array([amax]).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)[0]
        s = np.float32(amax) / np.float32(448.0)
        cand = allv[(allv <= amax) & (allv >= s * np.float32(2.0 ** -6))]
        qv = (cand / s).astype(np.float32)
        low = qv.view(np.uint32) & 0xFFFFF
        sel = cand[np.abs(low.astype(np.int64) - 0x80000) <= 16]
        if len(sel) == 0:
            continue
        hits += len(sel)
        row = (rng.uniform(-1, 1, 128) * amax).astype(np.float32)
        row[0] = amax
        k = min(len(sel), 127)
        row[1:1 + k] = sel[:k] * np.where(rng.random(k) < 0.5, -1.0, 1.0).astype(np.float32)
        rows.append(row)
    return _bf16(np.stack(rows)), hits


def test_quant_quotients_near_e4m3_midpoints(orc):
    """The per-token and blockscale quantisers reach the code of the IEEE
    quotient without dividing every element; quotients near a rounding
    midpoint take the division.  Rows built so that every element's quotient
    sits within 16 units of a midpoint: codes bit-exact against the oracle."""
    X, hits = _near_midpoint_rows()
    assert hits >= 50, hits
    _say(f"[quant] near-midpoint quotients: {hits} in {X.shape[0]} rows")
    Xd = torch.from_numpy(X.view(np.int16)).cuda()
    Qd, sd = q.qgemm_quant_f8_pertoken(Xd)
    Qr, sr = orc.quant_f8_pertoken(X)
    assert np.array_equal(sd.cpu().numpy().view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(Qd.cpu().numpy(), Qr), f"{np.count_nonzero(Qd.cpu().numpy() != Qr)} codes differ"
    Qd, sd = q.qgemm_quant_f8_block(Xd)
    Qr, sr = orc.quant_f8_block(X)
    assert np.array_equal(sd.cpu().numpy().view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(Qd.cpu().numpy(), Qr), f"{np.count_nonzero(Qd.cpu().numpy() != Qr)} codes differ"
