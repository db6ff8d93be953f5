"""Pins of the CPU oracle's FP8 blockscale GEMM against facts that do not come
from that function.

The variant is named, with its measured shape, in ROCm/mori PR #806 "perf(gemm-ar):
mxfp8 with row-major scales staged through LDS" (commit message table); the
block sizes (1x128 for A, 128x128 for B, fp32) are the reading stated in the
oracle.  The pages print no output values, so the function is pinned by:
  * exact rational brute force on tiny ragged shapes (distinct scales per row,
    per K block and per 128-row group of B, so a wrong scale index fails);
  * reduction to the per-token FP8 oracle (itself pinned) when every scale is
    a power of two and constant along K;
  * a one-hot closed form per K block;
  * a recomputation from torch's float8_e4m3fn decode and numpy matmul;
  * invariants: doubling one block's scale adds exactly that block's
    contribution; permuting K blocks together with their scales changes
    nothing; a zero scale removes a block.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from block_scaled_precision_02_amd import inputs


def _bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _dec(codes):
    """e4m3fn codes -> float64 through torch's own cast (a library decoder)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _case(M, N, K, seed, pow2=False):
    r = np.random.default_rng(seed)
    A = r.integers(0, 256, size=(M, K), dtype=np.uint8)
    B = r.integers(0, 256, size=(N, K), dtype=np.uint8)
    # no NaN codes (S.1111.111)
    A[(A & 0x7F) == 0x7F] = 0x7E
    B[(B & 0x7F) == 0x7F] = 0x7E
    KB, NB = K // 128, (N + 127) // 128
    if pow2:
        sa = np.ldexp(1.0, r.integers(-12, -4, size=(M, KB))).astype(np.float32)
        sb = np.ldexp(1.0, r.integers(-12, -4, size=(NB, KB))).astype(np.float32)
    else:
        sa = r.uniform(1e-3, 1e-2, size=(M, KB)).astype(np.float32)
        sb = r.uniform(1e-3, 1e-2, size=(NB, KB)).astype(np.float32)
        sa[0, 0] = -sa[0, 0]            # a negative scale
    return A, B, sa, sb


@pytest.mark.parametrize("M,N,K,with_bias", [(3, 130, 256, False), (2, 131, 384, True), (1, 1, 128, False)])
def test_blockscale_brute_force(orc, M, N, K, with_bias):
    A, B, sa, sb = _case(M, N, K, seed=M * 1000 + N + K)
    bias = _bf16(np.random.default_rng(7).standard_normal(N)) if with_bias else None
    C, acc, absdot = orc.f8_blockscale(A, B, sa, sb, bias)
    da, db = _dec(A), _dec(B)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                w = Fraction(float(sa[m, k // 128])) * Fraction(float(sb[n // 128, k // 128]))
                p = w * Fraction(da[m, k]) * Fraction(db[n, k])
                exact += p
                mag += abs(p)
            assert abs(Fraction(acc[m, n]) - exact) <= Fraction(K // 128 + 1, 2 ** 53) * mag + Fraction(1, 2 ** 1000)
            assert absdot[m, n] == pytest.approx(float(mag), rel=1e-12, abs=1e-300)
            f = np.float32(float(exact))
            if bias is not None:
                f = np.float32(f + (np.uint32(bias[n]) << np.uint32(16)).view(np.float32))
            assert C[m, n] == _bf16(np.array([f]))[0], (m, n)


def test_blockscale_reduces_to_pertoken_with_pow2_scales(orc):
    # sa[m, kb] = 2^ea[m] and sb[nb, kb] = 2^eb for every kb: the block sum is
    # sa * sb * sum_k a b exactly, and the per-token epilogue's multiplications
    # by powers of two are exact, so both give the same bits.
    M, N, K = 9, 200, 512
    A, B, _, _ = _case(M, N, K, seed=11)
    r = np.random.default_rng(12)
    ea = r.integers(-10, -3, size=M)
    eb = r.integers(-10, -3, size=(N + 127) // 128)
    sa = np.repeat(np.ldexp(1.0, ea)[:, None], K // 128, axis=1).astype(np.float32)
    sb = np.repeat(np.ldexp(1.0, eb)[:, None], K // 128, axis=1).astype(np.float32)
    C, acc, _ = orc.f8_blockscale(A, B, sa, sb)
    Cp, accp, _ = orc.f8_pertoken(A, B, sa[:, 0], np.repeat(sb[:, 0], 128)[:N])
    np.testing.assert_array_equal(C, Cp)
    scale = np.ldexp(1.0, ea)[:, None] * np.repeat(np.ldexp(1.0, eb), 128)[None, :N]
    np.testing.assert_array_equal(acc, accp * scale)


def test_blockscale_one_hot_closed_form(orc):
    # A row m and B row n each hold one nonzero element, at the same k: the
    # output is sa[m, k/128] * sb[n/128, k/128] * a * b, rounded once to fp32.
    M, N, K = 4, 260, 512
    _, _, sa, sb = _case(M, N, K, seed=21)
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    ks = [5, 130, 300, 511]
    codes_a = [0x38, 0xB9, 0x7E, 0x01]        # 1, -1.125, 448, 2^-9
    for m in range(M):
        A[m, ks[m]] = codes_a[m]
    for n in range(N):
        B[n, ks[n % M]] = 0x40 + (n % 7)       # 2 .. 3.75
    C, acc, _ = orc.f8_blockscale(A, B, sa, sb)
    da, db = _dec(A), _dec(B)
    for m in range(M):
        for n in range(N):
            if n % M != m:
                assert acc[m, n] == 0.0
                continue
            k = ks[m]
            v = Fraction(float(sa[m, k // 128])) * Fraction(float(sb[n // 128, k // 128])) \
                * Fraction(da[m, k]) * Fraction(db[n, k])
            assert acc[m, n] == float(v)
            assert C[m, n] == _bf16(np.array([np.float32(float(v))]))[0]


def test_blockscale_matches_library_matmul(orc):
    d = inputs.make("f8_block", M=192, N=300, K=1024)
    C, acc, absdot = orc.f8_blockscale(d["A"], d["B"], d["scale_a"], d["scale_b"])
    da, db = _dec(d["A"]), _dec(d["B"])
    ref = np.zeros((192, 300))
    sbr = np.repeat(d["scale_b"], 128, axis=0)[:300]
    for kb in range(1024 // 128):
        sl = slice(128 * kb, 128 * kb + 128)
        part = da[:, sl] @ db[:, sl].T
        ref += part * d["scale_a"][:, kb].astype(np.float64)[:, None] * sbr[:, kb].astype(np.float64)[None, :]
    assert np.all(np.abs(acc - ref) <= 1e-13 * absdot + 1e-300)
    assert np.all(absdot > 0)


def test_blockscale_invariants(orc):
    M, N, K = 6, 140, 768
    A, B, sa, sb = _case(M, N, K, seed=31, pow2=True)
    # power-of-two scales and at most 6 blocks: every sum below is exact
    _, acc, _ = orc.f8_blockscale(A, B, sa, sb)
    # doubling sa[:, 2] adds exactly block 2's contribution once more
    sa2 = sa.copy()
    sa2[:, 2] *= 2
    _, acc2, _ = orc.f8_blockscale(A, B, sa2, sb)
    z = sa.copy()
    z[:, [0, 1, 3, 4, 5]] = 0
    _, blk2, _ = orc.f8_blockscale(A, B, z, sb)
    np.testing.assert_array_equal(acc2, acc + blk2)
    # a zero scale removes its block: the blocks' parts add up to the whole
    total = np.zeros_like(acc)
    for kb in range(K // 128):
        zz = np.zeros_like(sa)
        zz[:, kb] = sa[:, kb]
        total += orc.f8_blockscale(A, B, zz, sb)[1]
    np.testing.assert_array_equal(total, acc)
    # permuting whole K blocks together with their scales changes nothing
    perm = np.array([4, 0, 5, 2, 1, 3])
    cols = np.concatenate([np.arange(128 * p, 128 * p + 128) for p in perm])
    _, accp, _ = orc.f8_blockscale(A[:, cols], B[:, cols], sa[:, perm], sb[:, perm])
    np.testing.assert_array_equal(accp, acc)


def test_blockscale_k_must_be_whole_blocks(orc):
    A = np.zeros((2, 96), np.uint8)
    with pytest.raises(AssertionError):
        orc.f8_blockscale(A, A, np.ones((2, 1), np.float32), np.ones((1, 1), np.float32))


def test_block_quantise_recipe():
    # the input recipe: every block's largest magnitude lands on +-448 and
    # the scale is amax/448 in fp32
    x = np.random.default_rng(5).standard_normal((130, 256)).astype(np.float32)
    codes, s = inputs.block_quantise_e4m3(x, 128)
    assert s.shape == (2, 2)
    dq = _dec(codes)
    for rb in range(2):
        for kb in range(2):
            blk = dq[128 * rb:128 * rb + 128, 128 * kb:128 * kb + 128]
            assert np.abs(blk).max() == 448.0
            xb = x[128 * rb:128 * rb + 128, 128 * kb:128 * kb + 128]
            assert s[rb, kb] == np.float32(np.abs(xb).max() / np.float32(448.0))
