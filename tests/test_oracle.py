"""Pins of the CPU oracle against facts that do not come from the oracle.

The pages print no GEMM output values, so the oracle is pinned by:
  * library decoders (torch's float8_e4m3fn / float8_e8m0fnu casts) and the
    hand-written tables under tests/golden/;
  * brute force over Python integers / fractions on tiny shapes, with the
    epilogue redone in numpy binary32 and torch's bf16 cast;
  * closed forms (identity, one-hot, constant rows, cancelling rows);
  * MX invariants (a scale step doubles one block; permuting K blocks with
    their scales; zero blocks; swapping A and B transposes C);
  * an exact integer recomputation of the fp64 accumulators;
  * the epilogue cases of tests/golden/epilogue_cases.txt (association
    (acc*sa)*sb, no FMA, signed zero without bias, subnormals kept, ties).
Each would fail on a plausible slip in the oracle: a dropped term, a sign or
index error, transposed operands, a wrong scale row, a wrong nibble, an FMA,
a reassociated scale product, a flush to zero.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out


def _pow(s):
    return 2.0 ** int(s[2:]) if s.startswith("2^") else float(s)


def bf16_torch(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ decoders

def test_e4m3_spot_values(orc):
    for code, val in _rows("e4m3_spot.txt"):
        got = orc.dec_e4m3(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), code


def test_e4m3_exhaustive_vs_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.dec_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(ours), np.signbit(ref))
    assert np.nanmax(np.abs(ours)) == 448.0


def test_e2m1_table(orc):
    rows = _rows("e2m1_codes.txt")
    got = orc.dec_e2m1(np.array([int(c) for c, _ in rows], np.uint8))
    exp = np.array([float(v) for _, v in rows])
    assert np.array_equal(got, exp) and np.array_equal(np.signbit(got), np.signbit(exp))


def test_ue8m0(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.dec_ue8m0(codes)
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127
    assert np.isnan(got[255])
    if hasattr(torch, "float8_e8m0fnu"):
        ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
        assert np.array_equal(got[:255], ref[:255]) and np.isnan(ref[255])


def test_bf16_rne_vs_torch(orc):
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
        rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0x3F808000, 0x3F818000, 0x00008000, 0x80018000, 0x7F7FFFFF, 0x7F800000,
                  0xFF800000, 0x7FC00001, 0xFFA00000, 0x00000001], np.uint32).view(np.float32),
    ])
    ours = orc.bf16_rne(x)
    ref = bf16_torch(x)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.isnan(bf16_to_f32(ours[nan])).all()                # NaN stays NaN
    # the two documented ties: 1.00390625 -> 1.0 (even), 1.01171875 -> 1.015625
    assert orc.bf16_rne(np.array([0x3F808000], np.uint32).view(np.float32))[0] == 0x3F80
    assert orc.bf16_rne(np.array([0x3F818000], np.uint32).view(np.float32))[0] == 0x3F82


# ------------------------------------------------------------------ INT8

def _epilogue_ref(acc_f32, sa, sb, bias_bits):
    """binary32 epilogue redone in numpy (each op RNE), bf16 via torch."""
    f = np.asarray(acc_f32, np.float32) * np.asarray(sa, np.float32)[:, None]
    f = f * np.asarray(sb, np.float32)[None, :]
    if bias_bits is not None:
        f = f + bf16_to_f32(bias_bits)[None, :]
    return bf16_torch(f)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (3, 5, 64), (8, 7, 96), (5, 8, 32)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_i8_brute_force(orc, M, N, K, with_bias):
    rng = np.random.default_rng([M, N, K, with_bias])
    A = rng.integers(-128, 128, (M, K), dtype=np.int8)
    B = rng.integers(-128, 128, (N, K), dtype=np.int8)
    sa = rng.uniform(-1e-2, 1e-2, M).astype(np.float32)
    sb = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    bias = bf16_torch(rng.standard_normal(N)) if with_bias else None
    C, acc = orc.i8_rowwise(A, B, sa, sb, bias)
    ref = np.array([[sum(int(A[m, k]) * int(B[n, k]) for k in range(K)) for n in range(N)]
                    for m in range(M)], dtype=np.int64)
    assert np.array_equal(acc, ref)
    assert np.array_equal(C, _epilogue_ref(ref.astype(np.float32), sa, sb, bias))


def test_i8_closed_forms(orc):
    K = N = 64
    rng = np.random.default_rng(3)
    A = rng.integers(-127, 128, (16, K), dtype=np.int8)
    ones = np.ones(N, np.float32)
    # B = c * I  =>  acc = c * A
    for c in (1, -3, 127):
        B = (np.eye(N, K, dtype=np.int64) * c).astype(np.int8)
        _, acc = orc.i8_rowwise(A, B, np.ones(16, np.float32), ones)
        assert np.array_equal(acc, A.astype(np.int64) * c)
    # one-hot rows: a single product survives
    Ao = np.zeros((4, K), np.int8)
    Bo = np.zeros((4, K), np.int8)
    for i, (ka, va, vb) in enumerate([(0, 5, -7), (63, -128, -128), (17, 127, 1), (40, -1, 99)]):
        Ao[i, ka] = va
        Bo[:, ka] = 0
        Bo[i, ka] = vb
    _, acc = orc.i8_rowwise(Ao, Bo, np.ones(4, np.float32), np.ones(4, np.float32))
    assert np.array_equal(np.diag(acc), [-35, 16384, 127, -99])
    assert (acc - np.diag(np.diag(acc)) == 0).all()
    # all +127 x +127 => K * 16129;  alternating +-127 rows against all-ones => 0
    K2 = 5376
    P = np.full((2, K2), 127, np.int8)
    _, acc = orc.i8_rowwise(P, P, np.ones(2, np.float32), np.ones(2, np.float32))
    assert (acc == K2 * 16129).all()
    alt = np.tile(np.array([127, -127], np.int8), K2 // 2)[None, :]
    _, acc = orc.i8_rowwise(alt, np.ones((3, K2), np.int8), np.ones(1, np.float32),
                            np.ones(3, np.float32))
    assert (acc == 0).all()


def test_i8_overflow_guard(orc):
    # 131072 * (-128)^2 = 2^31 does not fit int32: the oracle refuses it.
    K = 131072
    A = np.full((1, K), -128, np.int8)
    with pytest.raises(OverflowError):
        orc.i8_rowwise(A, A, np.ones(1, np.float32), np.ones(1, np.float32))


def _one_row_pair(acc):
    """int8 rows a, b (K a multiple of 32) with sum_k a[k]*b[k] == acc exactly:
    q products 127*127, then (r//127)*127 and (r%127)*1."""
    q, r = divmod(abs(acc), 16129)
    K = ((q + 2 + 31) // 32) * 32
    a = np.zeros((1, K), np.int8)
    b = np.zeros((1, K), np.int8)
    s = -1 if acc < 0 else 1
    a[0, :q] = 127 * s
    b[0, :q] = 127
    a[0, q], b[0, q] = s * (r // 127), 127
    a[0, q + 1], b[0, q + 1] = s * (r % 127), 1
    return a, b


def test_epilogue_golden_cases(orc):
    """Drive each case through the oracle with one-hot rows that make acc
    exactly the listed integer."""
    for acc_s, sa_s, sb_s, bias_s, expect_s in (r[:5] for r in _rows("epilogue_cases.txt")):
        acc = int(acc_s)
        a, b = _one_row_pair(acc)
        sa = np.array([_pow(sa_s)], np.float32)
        sb = np.array([_pow(sb_s)], np.float32)
        bias = None if bias_s == "none" else np.array([int(bias_s, 16)], np.uint16)
        C, accv = orc.i8_rowwise(a, b, sa, sb, bias)
        assert accv[0, 0] == acc
        assert C[0, 0] == int(expect_s, 16), (acc_s, sa_s, sb_s, bias_s, hex(C[0, 0]))


def test_association_is_acc_sa_then_sb(orc):
    """Triples where bf16((acc*sa)*sb) != bf16(acc*(sa*sb)) exist; the oracle
    gives the former (comfy-kitchen PR #174, Update "rebased onto v0.2.40")."""
    rng = np.random.default_rng(11)
    acc = rng.integers(-2 ** 26, 2 ** 26, 200000).astype(np.float32)
    sa = rng.uniform(1e-3, 1e-2, 200000).astype(np.float32)
    sb = rng.uniform(1e-3, 1e-2, 200000).astype(np.float32)
    left = bf16_torch((acc * sa) * sb)
    right = bf16_torch(acc * (sa * sb))
    idx = np.nonzero(left != right)[0][:40]
    assert len(idx) > 0
    for i in idx:
        a = int(acc[i])
        av, bv = _one_row_pair(a)
        C, accv = orc.i8_rowwise(av, bv, sa[i:i + 1], sb[i:i + 1])
        assert accv[0, 0] == a
        assert C[0, 0] == left[i] and C[0, 0] != right[i]


def test_no_fma_in_bias_add(orc):
    """Cases where an FMA (x*sb + bias rounded once) differs from the two
    rounded steps after bf16; the oracle must give the two-step result."""
    rng = np.random.default_rng(12)
    n = 1000000
    acc = rng.integers(-2000, 2000, n).astype(np.float32)   # x*sb near -bias: cancellation
    sa = np.ones(n, np.float32)
    sb = rng.uniform(1e-3, 1e-2, n).astype(np.float32)
    bias_bits = bf16_torch(rng.standard_normal(n))
    bias = bf16_to_f32(bias_bits)
    two_step = bf16_torch((acc * sb) + bias)
    fused = bf16_torch((acc.astype(np.float64) * sb.astype(np.float64) +
                        bias.astype(np.float64)).astype(np.float32))
    idx = np.nonzero(two_step != fused)[0][:30]
    assert len(idx) > 0
    for i in idx:
        av, bv = _one_row_pair(int(acc[i]))
        C, _ = orc.i8_rowwise(av, bv, sa[i:i + 1], sb[i:i + 1], bias_bits[i:i + 1])
        assert C[0, 0] == two_step[i] and C[0, 0] != fused[i]


# ------------------------------------------------------------------ FP8

def _e4m3_fraction(code):
    v = torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()
    return Fraction(v)


def _finite_e4m3(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (4, 3, 64), (8, 8, 96)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_f8_brute_force(orc, M, N, K, with_bias):
    rng = np.random.default_rng([M, N, K, 8])
    A = _finite_e4m3(rng, (M, K))
    B = _finite_e4m3(rng, (N, K))
    sa = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    sb = rng.uniform(-1e-1, 1e-1, N).astype(np.float32)
    bias = bf16_torch(rng.standard_normal(N)) if with_bias else None
    C, acc, absdot = orc.f8_pertoken(A, B, sa, sb, bias)
    fa = [[_e4m3_fraction(int(x)) for x in row] for row in A]
    fb = [[_e4m3_fraction(int(x)) for x in row] for row in B]
    for m in range(M):
        for n in range(N):
            exact = sum(fa[m][k] * fb[n][k] for k in range(K))
            assert Fraction(acc[m, n]) == exact
            tot = sum(abs(fa[m][k] * fb[n][k]) for k in range(K))
            assert absdot[m, n] == pytest.approx(float(tot) * abs(float(sa[m]) * float(sb[n])),
                                                 rel=1e-15)
    ref = _epilogue_ref(acc.astype(np.float32), sa, sb, bias)
    assert np.array_equal(C, ref)


def test_f8_exact_integer_recomputation(orc):
    """Each e4m3 value is an integer times 2^-9; int64 sums of the integer
    products must equal the fp64 accumulator bit for bit (exactness)."""
    rng = np.random.default_rng(5)
    M, N, K = 6, 40, 7168
    A = _finite_e4m3(rng, (M, K))
    B = _finite_e4m3(rng, (N, K))
    _, acc, _ = orc.f8_pertoken(A, B, np.ones(M, np.float32), np.ones(N, np.float32))
    lut = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ia = np.rint(lut[A] * 512).astype(np.int64)
    ib = np.rint(lut[B] * 512).astype(np.int64)
    exact = ia @ ib.T                                  # integer units of 2^-18
    assert np.abs(exact).max() < 2 ** 53
    assert np.array_equal(acc, exact.astype(np.float64) * 2.0 ** -18)


def test_f8_matches_library_matmul(orc):
    rng = np.random.default_rng(6)
    A = _finite_e4m3(rng, (33, 256))
    B = _finite_e4m3(rng, (17, 256))
    _, acc, _ = orc.f8_pertoken(A, B, np.ones(33, np.float32), np.ones(17, np.float32))
    lut = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_allclose(acc, lut[A] @ lut[B].T, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------ MX

def _mx_inputs(rng, fmt, M, N, K, brows, lo=120, hi=134):
    if fmt == 0:
        A = _finite_e4m3(rng, (M, K))
        B = _finite_e4m3(rng, (N, K))
    else:
        A = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
        B = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = rng.integers(lo, hi, (M, K // 32), dtype=np.uint8)
    sb = rng.integers(lo, hi, (-(-N // brows), K // 32), dtype=np.uint8)
    return A, B, sa, sb


_E2M1 = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]


def _elem_fraction(fmt, row, k):
    if fmt == 0:
        return _e4m3_fraction(int(row[k]))
    byte = int(row[k // 2])
    nib = (byte >> 4) if (k & 1) else (byte & 15)
    v = _E2M1[nib & 7]
    return -v if nib & 8 else v


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("brows", [1, 32])
@pytest.mark.parametrize("M,N,K", [(2, 3, 32), (5, 33, 96), (3, 40, 64)])
def test_mx_brute_force(orc, fmt, brows, M, N, K):
    rng = np.random.default_rng([fmt, brows, M, N, K])
    A, B, sa, sb = _mx_inputs(rng, fmt, M, N, K, brows)
    bias = bf16_torch(rng.standard_normal(N))
    C, acc, absdot = orc.mx(fmt, A, B, sa, sb, brows, K, bias)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            tot = Fraction(0)
            for k in range(K):
                ea = Fraction(2) ** (int(sa[m, k // 32]) - 127)
                eb = Fraction(2) ** (int(sb[n // brows, k // 32]) - 127)
                p = _elem_fraction(fmt, A[m], k) * ea * _elem_fraction(fmt, B[n], k) * eb
                exact += p
                tot += abs(p)
            # double summation: exact when the terms' span fits 53 bits,
            # otherwise within K * 2^-53 * sum|p| of the exact sum.
            assert abs(Fraction(acc[m, n]) - exact) <= Fraction(K, 2 ** 53) * tot, (m, n)
            assert abs(Fraction(absdot[m, n]) - tot) <= Fraction(K, 2 ** 53) * tot
    f = acc.astype(np.float32) + bf16_to_f32(bias)[None, :]
    assert np.array_equal(C, bf16_torch(f))


@pytest.mark.parametrize("fmt", [0, 1])
def test_mx_exact_on_workload_inputs(orc, fmt):
    """On inputs built by the workload recipe (N(0,1) data, shared exponent
    per block) the double accumulator is the exact sum: recompute a few rows
    with Python integers on a common power-of-two grid."""
    from block_scaled_precision_02_amd import inputs
    name = "mxfp8" if fmt == 0 else "mxfp4"
    d = inputs.make(name, M=4, N=64, K=2048)
    brows = d["b_rows_per_scale"]
    _, acc, _ = orc.mx(fmt, d["A"], d["B"], d["scale_a"], d["scale_b"], brows, 2048)
    K = 2048

    def ints(X, S, rows_per):
        # element value = integer * 2^-9 (e4m3) or * 2^-1 (e2m1)
        if fmt == 0:
            lut = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
            v = np.rint(lut[X] * 512).astype(np.int64)
        else:
            lo, hi = X & 15, X >> 4
            codes = np.stack([lo, hi], axis=-1).reshape(X.shape[0], -1)
            tab = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)
            v = tab[codes]
        e = np.repeat(np.repeat(S.astype(np.int64), rows_per, axis=0)[:X.shape[0]], 32, axis=1)
        return v, e

    va, ea = ints(d["A"], d["scale_a"], 1)
    vb, eb = ints(d["B"], d["scale_b"], brows)
    unit = 9 if fmt == 0 else 1
    for m in range(4):
        for n in range(0, 64, 7):
            ex = ea[m] + eb[n]
            lo = int(ex.min())
            total = sum(int(va[m, k]) * int(vb[n, k]) << int(ex[k] - lo) for k in range(K))
            exact = Fraction(total) * Fraction(2) ** (lo - 254 - 2 * unit)
            assert Fraction(acc[m, n]) == exact, (m, n)


@pytest.mark.parametrize("fmt", [0, 1])
def test_mx_invariants(orc, fmt):
    # workload-recipe inputs keep every sum exact, so the identities hold bitwise
    from block_scaled_precision_02_amd import inputs
    rng = np.random.default_rng(40 + fmt)
    M, N, K = 6, 10, 256
    d = inputs.make("mxfp8" if fmt == 0 else "mxfp4", M=M, N=N, K=K, seed=40 + fmt)
    A, B, sa = d["A"], d["B"], d["scale_a"]
    sb = inputs.mx_quantise(rng.standard_normal((N, K)), "e4m3" if fmt == 0 else "e2m1", 1)[1]
    _, acc, _ = orc.mx(fmt, A, B, sa, sb, 1, K)
    # (1) one more on one A scale code doubles that block's contribution
    kb = 3
    sa2 = sa.copy()
    sa2[:, kb] += 1
    _, acc2, _ = orc.mx(fmt, A, B, sa2, sb, 1, K)
    Ablk = np.zeros_like(A)
    w = 32 if fmt == 0 else 16
    Ablk[:, kb * w:(kb + 1) * w] = A[:, kb * w:(kb + 1) * w]
    _, part, _ = orc.mx(fmt, Ablk, B, sa, sb, 1, K)
    assert np.array_equal(acc2, acc + part)
    # (2) permuting whole K blocks together with their scales changes nothing
    perm = rng.permutation(K // 32)
    cols = np.concatenate([np.arange(p * w, (p + 1) * w) for p in perm])
    _, acc3, _ = orc.mx(fmt, A[:, cols], B[:, cols], sa[:, perm], sb[:, perm], 1, K)
    assert np.array_equal(acc3, acc)
    # (3) appending zero K blocks (any scale) changes nothing
    zA = np.concatenate([A, np.zeros((M, 2 * w), np.uint8)], axis=1)
    zB = np.concatenate([B, np.zeros((N, 2 * w), np.uint8)], axis=1)
    zsa = np.concatenate([sa, np.full((M, 2), 200, np.uint8)], axis=1)
    zsb = np.concatenate([sb, np.full((N, 2), 90, np.uint8)], axis=1)
    _, acc4, _ = orc.mx(fmt, zA, zB, zsa, zsb, 1, K + 64)
    assert np.array_equal(acc4, acc)
    # (4) swapping A and B (with their scales) transposes the result
    _, acc5, _ = orc.mx(fmt, B, A, sb, sa, 1, K)
    assert np.array_equal(acc5, acc.T)


def test_mx_32x32_scale_rows(orc):
    """With 32x32 B scales, B row n uses scale row n//32: equal to the 1x32
    call with each scale row repeated for its 32 rows of B."""
    rng = np.random.default_rng(9)
    M, N, K = 4, 70, 128
    A, B, sa, sb = _mx_inputs(rng, 0, M, N, K, 32)
    _, acc32, _ = orc.mx(0, A, B, sa, sb, 32, K)
    sb_full = np.repeat(sb, 32, axis=0)[:N]
    _, acc1, _ = orc.mx(0, A, B, sa, sb_full, 1, K)
    assert np.array_equal(acc32, acc1)


def test_mx_matches_library_matmul(orc):
    rng = np.random.default_rng(10)
    M, N, K = 20, 30, 512
    A, B, sa, sb = _mx_inputs(rng, 1, M, N, K, 1)
    _, acc, _ = orc.mx(1, A, B, sa, sb, 1, K)

    def deq(X, S):
        lo = X & 15
        hi = X >> 4
        codes = np.stack([lo, hi], axis=-1).reshape(X.shape[0], -1)
        vals = np.array([float(v) for v in _E2M1] + [-float(v) for v in _E2M1])[codes]
        return vals * np.repeat(2.0 ** (S.astype(np.float64) - 127), 32, axis=1)

    np.testing.assert_allclose(acc, deq(A, sa) @ deq(B, sb).T, rtol=1e-13, atol=1e-30)


def test_mx_e2m1_nibble_order(orc):
    """Element k even sits in the low nibble: a single low-nibble code 2 (1.0)
    in byte 0 meets B's element 0 only."""
    K = 32
    A = np.zeros((1, 16), np.uint8)
    B = np.zeros((2, 16), np.uint8)
    A[0, 0] = 0x02          # a[0] = 1.0, a[1] = 0
    B[0, 0] = 0x04          # b[0] = 2.0
    B[1, 0] = 0x40          # b[1] = 2.0, b[0] = 0
    s = np.full((1, 1), 127, np.uint8)
    _, acc, _ = orc.mx(1, A, B, s, np.full((2, 1), 127, np.uint8), 1, K)
    assert acc[0, 0] == 2.0 and acc[0, 1] == 0.0


def test_mx_scale_255_is_nan(orc):
    A = np.full((1, 32), 0x38, np.uint8)
    B = np.full((1, 32), 0x38, np.uint8)
    C, acc, _ = orc.mx(0, A, B, np.full((1, 1), 255, np.uint8), np.full((1, 1), 127, np.uint8), 1, 32)
    assert np.isnan(acc[0, 0]) and (C[0, 0] & 0x7FFF) > 0x7F80
