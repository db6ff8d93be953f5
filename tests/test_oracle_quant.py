"""Pins of the oracle's activation quantisers (per-token e4m3, MX e4m3 / e2m1)
against facts that do not come from the oracle:

  * the hand-worked rounding cases of tests/golden/quant_round_cases.txt
    (midpoints, saturation, subnormals, signed zero);
  * torch's float32 -> float8_e4m3fn cast, a library routine, on every
    midpoint of the e4m3 grid and on random values;
  * exhaustive round trips through the decoders;
  * worked rows and blocks whose scales and codes follow by hand from the
    readings (per-token scale amax/448; OCP MX shared exponent
    floor(log2 amax) - emax, clamped to the ue8m0 range);
  * invariants: scaling a row by 2 (a block by 2^j) leaves the codes and
    moves the scale exactly; negation flips only the sign bits; the amax
    element lands on the largest magnitude (per-token) or in
    [2^emax, 2^(emax+1)) before saturation (MX); every code is a nearest one.
A slip in the oracle -- max instead of max-abs, a wrong emax or bias, an off
by one in the exponent, ties away from zero, no saturation, a swapped nibble
-- fails one of these.
"""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

E4M3_FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


def bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def _cases():
    out = []
    with open(os.path.join(GOLDEN, "quant_round_cases.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                fmt, v, c = line.split()[:3]
                out.append((fmt, float(v), int(c, 16)))
    return out


# ---------------------------------------------------------------- element codes

@pytest.mark.parametrize("fmt,value,code", _cases())
def test_golden_rounding_cases(orc, fmt, value, code):
    enc = orc.enc_e4m3 if fmt == "e4m3" else orc.enc_e2m1
    assert enc(np.array([value]))[0] == code


def test_round_trip_every_finite_code(orc):
    codes = np.array(E4M3_FINITE, np.uint8)
    assert np.array_equal(orc.enc_e4m3(orc.dec_e4m3(codes)), codes)
    nib = np.arange(16, dtype=np.uint8)
    assert np.array_equal(orc.enc_e2m1(orc.dec_e2m1(nib)), nib)


def _torch_e4m3(x32):
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_matches_torch_cast_on_every_midpoint(orc):
    """Midpoints between neighbouring magnitudes (ties), and values just
    either side of them, for both signs (torch's cast rounds to nearest even;
    below 464 it never saturates differently from the reading)."""
    mags = orc.dec_e4m3(np.arange(127, dtype=np.uint8))
    mid = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)      # exact in fp32
    up = np.nextafter(mid, np.float32(np.inf))
    down = np.nextafter(mid, np.float32(0))
    x = np.concatenate([mid, up, down, mags.astype(np.float32)])
    x = np.concatenate([x, -x])
    assert np.array_equal(orc.enc_e4m3(x.astype(np.float64)), _torch_e4m3(x))


def test_e4m3_matches_torch_cast_on_random_values(orc):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-14, 9, 200000))).astype(np.float32)
    x = x[np.abs(x) < 448]
    assert np.array_equal(orc.enc_e4m3(x.astype(np.float64)), _torch_e4m3(x))


# ---------------------------------------------------------------- per-token e4m3

def test_pertoken_worked_row(orc):
    """Row [1, -2, 0.5, 0, -0]: amax 2, scale fp32(2/448) = fp32(1/224); the
    quotients are 224, -448, 112 up to one fp32 rounding, whose codes sit in
    the middle of their e4m3 steps (spacing 16, 32, 8): 0x76, 0xFE, 0x6E."""
    X = bf16(np.array([[1.0, -2.0, 0.5, 0.0, -0.0]], np.float32))
    Q, s = orc.quant_f8_pertoken(X)
    assert s[0] == np.float32(1.0) / np.float32(224.0)
    assert list(Q[0]) == [0x76, 0xFE, 0x6E, 0x00, 0x80]


def test_pertoken_zero_row_and_signs(orc):
    X = bf16(np.array([[0.0, -0.0, 0.0, -0.0]], np.float32))
    Q, s = orc.quant_f8_pertoken(X)
    assert s[0] == 0.0 and list(Q[0]) == [0x00, 0x80, 0x00, 0x80]


def _rows(M=16, K=256, seed=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp2(rng.integers(-8, 8, (M, 1)))
    return bf16(x)


def test_pertoken_invariants(orc):
    X = _rows()
    Q, s = orc.quant_f8_pertoken(X)
    x = f32(X)
    # the amax element of each row lands on the largest magnitude
    i = np.argmax(np.abs(x), axis=1)
    assert np.all((Q[np.arange(len(i)), i] & 0x7F) == 0x7E)
    # scaling by 2 (exact in bf16) doubles the scale and keeps every code
    Q2, s2 = orc.quant_f8_pertoken(bf16(2 * x))
    assert np.array_equal(Q2, Q) and np.array_equal(s2, 2 * s)
    # negation flips the sign bits only
    Qn, sn = orc.quant_f8_pertoken(bf16(-x))
    assert np.array_equal(Qn, Q ^ 0x80) and np.array_equal(sn, s)


def test_pertoken_codes_are_nearest(orc):
    X = _rows(seed=4)
    Q, s = orc.quant_f8_pertoken(X)
    y = (f32(X) / s[:, None]).astype(np.float64)               # fp32 quotient
    v = orc.dec_e4m3(Q)
    mag = Q & 0x7F
    lo = orc.dec_e4m3(np.maximum(mag, 1) - 1)
    hi = orc.dec_e4m3(np.minimum(mag, 125) + 1)
    ay = np.abs(y)
    assert np.all(np.abs(np.abs(v) - ay) <= np.abs(lo - ay))
    assert np.all(np.abs(np.abs(v) - ay) <= np.abs(hi - ay) + (mag == 126) * 1e9)
    assert np.all(np.signbit(v) == np.signbit(y))


# ---------------------------------------------------------------- MX

def test_mx_worked_blocks(orc):
    """One e4m3 block and one e2m1 block with amax 1: X = 0 - emax, so the
    scale codes are 127 - 8 = 119 and 127 - 2 = 125 and the elements are
    multiplied by 2^8 and 2^2 before rounding."""
    row = np.zeros(32, np.float32)
    row[:5] = [1.0, 0.5, -0.75, 0.1, -1.0]
    X = bf16(row[None, :])
    Q, S = orc.quant_mx(orc.MX_E4M3, X)
    assert S[0, 0] == 119
    # 256 -> 0x78, 128 -> 0x70, -192 -> 0xF4, bf16(0.1)*256 = 25.6 -> 26 (step 2) = 1.625*2^4 -> 0x5D,
    # -256 -> 0xF8
    assert list(Q[0, :5]) == [0x78, 0x70, 0xF4, 0x5D, 0xF8]
    assert np.all(Q[0, 5:] == 0)
    Q4, S4 = orc.quant_mx(orc.MX_E2M1, X)
    assert S4[0, 0] == 125
    # 4 -> 6, 2 -> 4, -3 -> 0xD, 0.4 -> 0.5 = 1, -4 -> 0xE; pairs packed low nibble first
    assert list(Q4[0, :3]) == [0x6 | (0x4 << 4), 0xD | (0x1 << 4), 0xE]
    assert np.all(Q4[0, 3:] == 0)


def test_mx_block_at_the_format_max_keeps_the_elements(orc):
    """amax = 448 = 1.75 * 2^8: X = 8 - 8 = 0, scale code 127, and every
    element is encoded as it is."""
    rng = np.random.default_rng(9)
    row = (rng.standard_normal(32) * 50).astype(np.float32)
    row[7] = 448.0
    X = bf16(row[None, :])
    Q, S = orc.quant_mx(orc.MX_E4M3, X)
    assert S[0, 0] == 127
    assert np.array_equal(Q[0], orc.enc_e4m3(f32(X[0]).astype(np.float64)))


def test_mx_tiny_block_clamps_the_scale(orc):
    """amax = 2^-130 (a bf16 subnormal): X = -130 - 8 = -138 is below the
    ue8m0 range, code 0 (2^-127); the element becomes 2^-130 * 2^127 = 2^-3,
    code 0x20."""
    row = np.zeros(32, np.float32)
    row[0] = 2.0 ** -130
    Q, S = orc.quant_mx(orc.MX_E4M3, bf16(row[None, :]))
    assert S[0, 0] == 0 and Q[0, 0] == 0x20


def test_mx_zero_block(orc):
    row = np.zeros(64, np.float32)
    row[32:] = 1.0
    row[3] = -0.0
    Q, S = orc.quant_mx(orc.MX_E4M3, bf16(row[None, :]))
    assert S[0, 0] == 0 and Q[0, 3] == 0x80 and np.all(np.delete(Q[0, :32], 3) == 0)
    assert S[0, 1] == 119


@pytest.mark.parametrize("fmt", [0, 1])
def test_mx_invariants(orc, fmt):
    rng = np.random.default_rng(11 + fmt)
    x = (rng.standard_normal((8, 256)) * np.exp2(rng.integers(-20, 20, (8, 1)))).astype(np.float32)
    X = bf16(x)
    xf = f32(X)
    Q, S = orc.quant_mx(fmt, X)
    emax = 8 if fmt == 0 else 2
    # power-of-two scaling: the same codes, every scale code moved by j
    for j in (1, -3, 5):
        Qj, Sj = orc.quant_mx(fmt, bf16(xf * np.float32(2.0 ** j)))
        assert np.array_equal(Qj, Q) and np.array_equal(Sj.astype(int), S.astype(int) + j)
    # negation flips the sign bits only
    Qn, Sn = orc.quant_mx(fmt, bf16(-xf))
    flip = 0x80 if fmt == 0 else 0x88
    assert np.array_equal(Qn, Q ^ flip) and np.array_equal(Sn, S)
    # the block's amax, scaled, lies in [2^emax, 2^(emax+1))
    amax = np.abs(xf).reshape(8, 8, 32).max(axis=2).astype(np.float64)
    y = amax * np.exp2(127.0 - S)
    assert np.all((y >= 2.0 ** emax) & (y < 2.0 ** (emax + 1)))
    # every element code is a nearest one to x * 2^(127 - S)
    codes = Q if fmt == 0 else np.stack([Q & 15, Q >> 4], axis=2).reshape(8, 256)
    dec = orc.dec_e4m3 if fmt == 0 else orc.dec_e2m1
    top = 126 if fmt == 0 else 7
    ye = xf.astype(np.float64) * np.exp2(127.0 - np.repeat(S, 32, axis=1))
    mag = codes & (0x7F if fmt == 0 else 7)
    v = np.abs(dec(mag))
    lo = np.abs(dec(np.maximum(mag, 1) - 1))
    hi = np.abs(dec(np.minimum(mag, top - 1) + 1))
    ay = np.abs(ye)
    assert np.all(np.abs(v - ay) <= np.abs(lo - ay))
    assert np.all((np.abs(v - ay) <= np.abs(hi - ay)) | (mag == top))


def test_mx_agrees_with_the_input_generator_away_from_signed_zero(orc):
    """The seeded input generator has its own MX quantiser (numpy grid search,
    written separately); it maps a negative value that rounds to zero to +0,
    which is its only intended difference."""
    from block_scaled_precision_02_amd import inputs
    rng = np.random.default_rng(21)
    x = f32(bf16(rng.standard_normal((16, 512)).astype(np.float32)))
    for fmt, name in ((0, "e4m3"), (1, "e2m1")):
        Q, S = orc.quant_mx(fmt, bf16(x))
        codes, scales = inputs.mx_quantise(x.astype(np.float64), name, 1)
        assert np.array_equal(S, scales)
        mine = Q if fmt == 0 else np.stack([Q & 15, Q >> 4], axis=2).reshape(16, 512)
        zero_mag = (mine & (0x7F if fmt == 0 else 7)) == 0
        assert np.array_equal(np.where(zero_mag, 0, mine), np.where(zero_mag, 0, codes))


# ------------------------------------------------------------ blockscale e4m3

def test_f8_block_on_one_block_is_the_pertoken_quantiser(orc):
    """K = 128: one block per row, so the blockscale quantiser is the
    per-token one (pinned above), bit for bit."""
    X = _rows(M=24, K=128, seed=9)
    Q, S = orc.quant_f8_block(X)
    Qp, Sp = orc.quant_f8_pertoken(X)
    np.testing.assert_array_equal(Q, Qp)
    np.testing.assert_array_equal(S[:, 0].view(np.uint32), Sp.view(np.uint32))


def test_f8_block_is_the_pertoken_quantiser_per_block(orc):
    """Each 128-column slice of a row is quantised as the per-token quantiser
    quantises that slice alone; all-zero blocks keep their signed zeros."""
    X = _rows(M=12, K=640, seed=10)
    X[3, 128:256] = 0
    X[3, 129:256:2] = 0x8000
    Q, S = orc.quant_f8_block(X)
    for b in range(5):
        Qp, Sp = orc.quant_f8_pertoken(np.ascontiguousarray(X[:, 128 * b:128 * b + 128]))
        np.testing.assert_array_equal(Q[:, 128 * b:128 * b + 128], Qp)
        np.testing.assert_array_equal(S[:, b].view(np.uint32), Sp.view(np.uint32))
    assert S[3, 1] == 0 and (Q[3, 129:256:2] == 0x80).all() and (Q[3, 128:256:2] == 0).all()


def test_f8_block_agrees_with_the_input_generator_away_from_signed_zero(orc):
    """The blockscale workload's input recipe (its own quantiser, numpy and
    torch's e4m3 grid) gives the same codes and scales, except that it writes
    +0 where a negative value rounds to zero."""
    from block_scaled_precision_02_amd import inputs
    x = np.random.default_rng(11).standard_normal((9, 384)).astype(np.float32)
    X = inputs.bf16_bits(x)
    xb = (X.astype(np.uint32) << 16).view(np.float32)
    codes, s = inputs.block_quantise_e4m3(xb, 1)
    Q, S = orc.quant_f8_block(X)
    np.testing.assert_array_equal(S.view(np.uint32), s.view(np.uint32))
    diff = Q != codes
    assert np.all((Q[diff] == 0x80) & (codes[diff] == 0))
