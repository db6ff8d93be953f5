"""The seeded generators: determinism and the stated recipes."""
import numpy as np

from block_scaled_precision_02_amd import inputs


def test_deterministic_and_seeded():
    a = inputs.make("i8_small")
    b = inputs.make("i8_small")
    assert inputs.digest(a) == inputs.digest(b)
    c = inputs.make("i8_small", rot=1)
    assert inputs.digest(a) != inputs.digest(c)


def test_i8_ranges():
    d = inputs.make("i8_small")
    assert d["A"].dtype == np.int8 and d["A"].min() >= -127
    assert (d["scale_a"] >= 1e-3).all() and (d["scale_a"] <= 1e-2).all()
    assert d["bias"] is not None and d["bias"].dtype == np.uint16


def test_f8_rows_hit_448(orc):
    d = inputs.make("f8_ptpc", M=64, N=32, K=512)
    vals = orc.dec_e4m3(d["A"])
    assert (np.abs(vals).max(axis=1) == 448.0).all()
    x = inputs.rng(d["seed"], 0).standard_normal(size=(64, 512), dtype=np.float32)
    np.testing.assert_allclose(d["scale_a"], np.abs(x).max(axis=1) / 448, rtol=1e-6)
    # dequantised values are within half an e4m3 step (relative 2^-4) of the draw
    deq = vals * d["scale_a"][:, None]
    assert (np.abs(deq - x) <= np.abs(x) * 2.0 ** -4 + d["scale_a"][:, None] * 2.0 ** -10).all()


def test_mx_shared_exponent_rule(orc):
    for name, emax in (("mxfp8", 8), ("mxfp4", 2)):
        d = inputs.make(name, M=32, N=64, K=256)
        x = inputs.rng(d["seed"], 0).standard_normal(size=(32, 256), dtype=np.float32)
        amax = np.abs(x).reshape(32, 8, 32).max(axis=2)
        expect = np.floor(np.log2(amax)).astype(int) - emax + 127
        assert np.array_equal(d["scale_a"].astype(int), expect)
    d = inputs.make("mxfp8", M=32, N=64, K=256)
    assert d["scale_b"].shape == (2, 8)


def test_e2m1_packing_matches_oracle(orc):
    d = inputs.make("mxfp4", M=8, N=8, K=64)
    x = inputs.rng(d["seed"], 0).standard_normal(size=(8, 64), dtype=np.float32)
    lo, hi = d["A"] & 15, d["A"] >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(8, 64)
    deq = orc.dec_e2m1(codes) * np.repeat(orc.dec_ue8m0(d["scale_a"]), 32, axis=1)
    # nearest e2m1 value of x * 2^-X; saturation at 6 (|x * 2^-X| < 8) costs at most 2
    assert (np.abs(deq - x) <= np.repeat(orc.dec_ue8m0(d["scale_a"]), 32, axis=1) * 2.0 + 1e-12).all()
    assert np.corrcoef(deq.ravel(), x.ravel())[0, 1] > 0.95
