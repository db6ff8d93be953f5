"""Pins of the CPU oracle's two-format MX GEMM (orc_mx2: e4m3 activations x
e2m1 weights, or the reverse) against facts that do not come from that
function.

The MX rule of ROCm/mori PR #806 "perf(gemm-ar): mxfp8 with row-major scales
staged through LDS" (What) and ROCm/FlyDSL PR #990 "[fp4_gemm_4wave] MXFP4 GEMM
perf optimize" applies per operand; pairing an e4m3 operand with an e2m1 one is
the reading this function adds.  Pinned by:
  * every e2m1 value is exactly an e4m3 value, so re-encoding the e2m1 operand's
    nibbles as e4m3 codes (through torch's own float8_e4m3fn cast of the
    hand-written e2m1 table) must give the single-format oracle's result, bit
    for bit, for either operand and both B-scale layouts;
  * with equal formats it is the single-format oracle;
  * exact rational brute force on tiny shapes;
  * the nibble order: a lone nonzero element at odd k sits in a high nibble.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_values():
    vals = {}
    for line in open(os.path.join(GOLDEN, "e2m1_codes.txt")):
        line = line.split("#", 1)[0].strip()
        if line:
            c, v = line.split()
            vals[int(c)] = float(v)
    return np.array([vals[c] for c in range(16)])


def _e2m1_to_e4m3_codes(packed, K):
    """[R, K/2] packed e2m1 -> [R, K] e4m3fn codes of the same values."""
    lo, hi = packed & 15, packed >> 4
    nib = np.empty((packed.shape[0], K), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = lo, hi
    v = torch.from_numpy(_e2m1_values()[nib]).to(torch.float8_e4m3fn)
    return v.view(torch.uint8).numpy()


def _e4m3(rng, shape):
    x = rng.integers(0, 256, shape, dtype=np.uint8)
    x[(x & 0x7F) == 0x7F] = 0x7E        # no NaN codes
    return x


def _scales(rng, rows, K):
    return rng.integers(118, 136, (rows, K // 32), dtype=np.uint8)


@pytest.mark.parametrize("brows", [1, 32])
@pytest.mark.parametrize("M,N,K", [(7, 40, 64), (33, 65, 256)])
def test_e2m1_weights_equal_their_e4m3_reencoding(orc, brows, M, N, K):
    rng = np.random.default_rng(M * N + K + brows)
    A = _e4m3(rng, (M, K))
    B4 = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa, sb = _scales(rng, M, K), _scales(rng, -(-N // brows), K)
    bias = rng.integers(0, 1 << 16, N, dtype=np.uint16) & 0xBFFF   # finite bf16
    C2, acc2, abs2 = orc.mx2(orc.MX_E4M3, orc.MX_E2M1, A, B4, sa, sb, brows, K, bias)
    B8 = _e2m1_to_e4m3_codes(B4, K)
    C1, acc1, abs1 = orc.mx(orc.MX_E4M3, A, B8, sa, sb, brows, K, bias)
    np.testing.assert_array_equal(acc2, acc1)
    np.testing.assert_array_equal(abs2, abs1)
    np.testing.assert_array_equal(C2, C1)


def test_e2m1_activations_equal_their_e4m3_reencoding(orc):
    rng = np.random.default_rng(3)
    M, N, K = 20, 24, 128
    A4 = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    B = _e4m3(rng, (N, K))
    sa, sb = _scales(rng, M, K), _scales(rng, N, K)
    C2, acc2, _ = orc.mx2(orc.MX_E2M1, orc.MX_E4M3, A4, B, sa, sb, 1, K)
    C1, acc1, _ = orc.mx(orc.MX_E4M3, _e2m1_to_e4m3_codes(A4, K), B, sa, sb, 1, K)
    np.testing.assert_array_equal(acc2, acc1)
    np.testing.assert_array_equal(C2, C1)


@pytest.mark.parametrize("fmt", [0, 1])
def test_equal_formats_are_the_single_format_oracle(orc, fmt):
    rng = np.random.default_rng(10 + fmt)
    M, N, K = 9, 35, 96
    row = K if fmt == 0 else K // 2
    A = _e4m3(rng, (M, row)) if fmt == 0 else rng.integers(0, 256, (M, row), dtype=np.uint8)
    B = _e4m3(rng, (N, row)) if fmt == 0 else rng.integers(0, 256, (N, row), dtype=np.uint8)
    sa, sb = _scales(rng, M, K), _scales(rng, -(-N // 32), K)
    r2 = orc.mx2(fmt, fmt, A, B, sa, sb, 32, K)
    r1 = orc.mx(fmt, A, B, sa, sb, 32, K)
    for x, y in zip(r2, r1):
        np.testing.assert_array_equal(x, y)


_E2M1 = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]


def _e4m3_fraction(c):
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    v = Fraction(m, 512) if e == 0 else Fraction(8 + m) * Fraction(2) ** (e - 10)
    return -v if s else v


def test_mx2_brute_force(orc):
    rng = np.random.default_rng(5)
    M, N, K = 3, 33, 64
    A = _e4m3(rng, (M, K))
    B = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa, sb = _scales(rng, M, K), _scales(rng, 2, K)
    C, acc, absdot = orc.mx2(orc.MX_E4M3, orc.MX_E2M1, A, B, sa, sb, 32, K)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                a = _e4m3_fraction(int(A[m, k])) * Fraction(2) ** (int(sa[m, k // 32]) - 127)
                byte = int(B[n, k // 2])
                nib = (byte >> 4) if (k & 1) else (byte & 15)
                b = _E2M1[nib & 7] * (-1 if nib & 8 else 1) * Fraction(2) ** (int(sb[n // 32, k // 32]) - 127)
                tot += a * b
                mag += abs(a * b)
            assert Fraction(acc[m, n]) == tot
            assert Fraction(absdot[m, n]) == mag
            f = torch.tensor([float(tot)], dtype=torch.float64).to(torch.float32).to(torch.bfloat16)
            assert C[m, n] == f.view(torch.int16).numpy().view(np.uint16)[0]


def test_mx2_nibble_order(orc):
    K = 64
    A = np.zeros((1, K), np.uint8)
    B = np.zeros((1, K // 2), np.uint8)
    A[0, 37] = 0x38                       # 1.0 at k = 37 (odd)
    B[0, 18] = 0x70 | 0x01                # high nibble (k = 37) = 6.0, low nibble (k = 36) = 0.5
    s = np.full((1, 2), 127, np.uint8)
    _, acc, _ = orc.mx2(orc.MX_E4M3, orc.MX_E2M1, A, B, s, s, 1, K)
    assert acc[0, 0] == 6.0
    A[0, 37], A[0, 36] = 0, 0x38
    _, acc, _ = orc.mx2(orc.MX_E4M3, orc.MX_E2M1, A, B, s, s, 1, K)
    assert acc[0, 0] == 0.5
