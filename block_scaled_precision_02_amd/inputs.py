"""Seeded synthetic inputs for the scaled low-precision GEMM.

This module is shared by the tests (which hand the same arrays to the CPU
oracle and to the HIP library) and by the benchmark.  It draws random
numbers and quantises them into the input formats; it holds none of the
GEMM's own arithmetic (no decode-and-accumulate, no epilogue).

Recipe per workload (seed = 101..105 for the five workloads; every tensor
draws from ``numpy.random.default_rng([seed, tensor_id, rot])`` with
tensor_id A=0, B=1, scale_A=2, scale_B=3, bias=4 and ``rot`` the index of a
rotating input set):

  i8_small   INT8 M=256 N=256 K=512: A, B uniform integers in [-127, 127];
             scale_A, scale_B uniform in [1e-3, 1e-2] (fp32); bias bf16 of N(0,1).
  f8_ptpc    FP8 e4m3 M=4096 N=2112 K=7168: A, B ~ N(0,1) (fp32); per row
             s = amax/448 (fp32), codes = e4m3(x/s) rounded to nearest even;
             no bias.
  mxfp8      MX e4m3 M=16384 N=7168 K=2048: A, B ~ N(0,1); shared exponent
             X = floor(log2(block amax)) - 8 per 1x32 block of A and per 32x32
             block of B (scales [M,K/32] and [N/32,K/32]); codes e4m3(x*2^-X)
             rounded to nearest even and saturated at 448; no bias.
  mxfp4      MX e2m1 M=N=K=8192: as mxfp8 with X = floor(log2(amax)) - 2,
             1x32 blocks for A and B (scales [M,K/32] and [N,K/32]); two codes
             per byte, even k in the low nibble; no bias.
  i8_qkv     INT8 M=30000 N=21504 K=5376 with bias, values as i8_small.
  mx_a8w4    MX with e4m3 A (activations) and e2m1 B (weights), M=N=K=8192
             (seed 107): A as mxfp8's A, B as mxfp4's B, 1x32 scales on both
             ([M,K/32], [N,K/32]); no bias.
  mx_a4w8    the same pairing the other way round (seed 110): e2m1 A as
             mxfp4's A, e4m3 B as mxfp8's with 1x32 scales.
  mxfp6      MX e2m3 (OCP FP6) M=N=K=8192 (seed 108): as mxfp4 with the
             6-bit E2M3 element (emax 2: X = floor(log2(amax)) - 2), four
             codes per three bytes (element k in bits 6k..6k+5 of the row,
             lowest bits first), 1x32 scales on both operands; no bias.
  mxfp6_e3m2 the same with the E3M2 element (emax 4), seed 109.
  f8_block   FP8 e4m3 with block scales, M=16384 N=7168 K=2048 (seed 106):
             A, B ~ N(0,1) (fp32); s = amax/448 (fp32) per 1x128 block of A
             (scale_A [M, K/128]) and per 128x128 block of B (scale_B
             [ceil(N/128), K/128]), codes = e4m3(x/s) rounded to nearest
             even; no bias.  (ROCm/mori PR #806 measures its "blockscale"
             GEMM at this shape; the block sizes are a reading.)

The recipes follow the workloads named for this GEMM (INT8 rowwise as in
comfy-kitchen PR #174's 30000x21504x5376 projection; per-token FP8 and MXFP8
as in ROCm/mori PR #806; MXFP4 8192^3 as in ROCm/FlyDSL PR #990).  All
inputs are synthetic.
"""
import hashlib

import numpy as np

# name -> (kind, M, N, K, seed, has_bias, fmt, b_rows_per_scale)
WORKLOADS = {
    "i8_small": ("i8", 256, 256, 512, 101, True, None, None),
    "f8_ptpc": ("f8", 4096, 2112, 7168, 102, False, None, None),
    "mxfp8": ("mx", 16384, 7168, 2048, 103, False, "e4m3", 32),
    "mxfp4": ("mx", 8192, 8192, 8192, 104, False, "e2m1", 1),
    "i8_qkv": ("i8", 30000, 21504, 5376, 105, True, None, None),
    "f8_block": ("f8b", 16384, 7168, 2048, 106, False, None, 128),
    "mx_a8w4": ("mx", 8192, 8192, 8192, 107, False, "e4m3/e2m1", 1),
    "mx_a4w8": ("mx", 8192, 8192, 8192, 110, False, "e2m1/e4m3", 1),
    "mxfp6": ("mx", 8192, 8192, 8192, 108, False, "e2m3", 1),
    "mxfp6_e3m2": ("mx", 8192, 8192, 8192, 109, False, "e3m2", 1),
}
ORDER = ["i8_small", "f8_ptpc", "mxfp8", "mxfp4", "i8_qkv"]

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def rng(seed, tensor_id, rot=0):
    return np.random.default_rng([seed, tensor_id, rot])


# ------------------------------------------------------------ quantisers

def _e4m3_grid():
    """Non-negative finite e4m3fn magnitudes, indexed by code 0..126, as
    torch decodes them (a library cast, not this project's decoder)."""
    import torch
    codes = torch.arange(127, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


# OCP MX v1.0 FP4 E2M1 magnitudes in code order 0..7.
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
# OCP MX v1.0 FP6 magnitudes in code order 0..31: E2M3 (exponent bias 1, three
# mantissa bits) and E3M2 (bias 3, two mantissa bits); exponent 0 subnormal.
_E2M3_GRID = np.array([m / 8 for m in range(8)] + [(1 + m / 8) * 2.0 ** (e - 1) for e in (1, 2, 3) for m in range(8)])
_E3M2_GRID = np.array([m / 16 for m in range(4)] + [(1 + m / 4) * 2.0 ** (e - 3) for e in range(1, 8) for m in range(4)])
_GRIDS = {"e2m1": _E2M1_GRID, "e2m3": _E2M3_GRID, "e3m2": _E3M2_GRID}
# largest exponent of each element type (the MX shared-exponent rule)
EMAX = {"e4m3": 8, "e2m1": 2, "e2m3": 2, "e3m2": 4}
SIGN_BIT = {"e4m3": 0x80, "e2m1": 0x8, "e2m3": 0x20, "e3m2": 0x20}
_grid_cache = {}


def _grid(fmt):
    if fmt not in _grid_cache:
        _grid_cache[fmt] = _e4m3_grid() if fmt == "e4m3" else _GRIDS[fmt]
    return _grid_cache[fmt]


def quantise(x, fmt):
    """Round x to the nearest representable value of fmt (ties to the even
    code), saturating at the largest finite magnitude.  Returns codes (uint8;
    for e2m1 one 4-bit code per element, not yet packed)."""
    grid = _grid(fmt)
    x = np.asarray(x, dtype=np.float64)
    ax = np.minimum(np.abs(x), grid[-1])
    hi = np.searchsorted(grid, ax, side="left")          # grid[hi] >= ax
    hi = np.minimum(hi, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = ax - grid[lo]
    dhi = grid[hi] - ax
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign_bit = SIGN_BIT[fmt]
    neg = np.signbit(x) & (code != 0)
    return np.where(neg, code | sign_bit, code).astype(np.uint8)


def pack_e2m1(codes):
    """[R, K] 4-bit codes -> [R, K/2] bytes, element k even in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] & 15) | ((codes[:, 1::2] & 15) << 4)


def pack_fp6(codes):
    """[R, K] 6-bit codes (K % 4 == 0) -> [R, 3K/4] bytes: element k in bits
    6k..6k+5 of the row, the row's bit b being bit b % 8 of byte b / 8."""
    c = np.asarray(codes, dtype=np.uint8).reshape(codes.shape[0], -1, 4) & 63
    c0, c1, c2, c3 = (c[..., i] for i in range(4))
    out = np.stack([c0 | (c1 << 6), (c1 >> 2) | (c2 << 4), (c2 >> 4) | (c3 << 2)], axis=-1)
    return out.reshape(codes.shape[0], -1).astype(np.uint8)


def row_bytes(fmt, K):
    return K if fmt == "e4m3" else K // 2 if fmt == "e2m1" else 3 * K // 4


def pack(codes, fmt):
    return pack_e2m1(codes) if fmt == "e2m1" else pack_fp6(codes) if fmt in ("e2m3", "e3m2") else codes


def floor_log2(x):
    """floor(log2(x)) for x > 0, exact (from frexp, not a float log)."""
    _, e = np.frexp(np.asarray(x, dtype=np.float64))
    return e.astype(np.int64) - 1


def _by_rows(fn, R, step, *outs):
    """Run fn(r0, r1) over row ranges [r0, r1) of `step` rows (a multiple of
    every block height involved, so each range holds whole blocks) on a small
    thread pool; numpy releases the GIL inside its loops, and ranges keep
    the float64 temporaries small.  The result does not depend on the split."""
    import concurrent.futures
    import os
    spans = [(r0, min(R, r0 + step)) for r0 in range(0, R, step)]
    if len(spans) <= 1:
        for a, b in spans:
            fn(a, b)
        return
    with concurrent.futures.ThreadPoolExecutor(min(16, os.cpu_count() or 4, len(spans))) as ex:
        list(ex.map(lambda ab: fn(*ab), spans))


def mx_quantise(x, fmt, block_rows):
    """MX-quantise x [R, K] (K % 32 == 0) with one ue8m0 scale per
    block_rows x 32 block.  Returns (codes [R, K] uint8, scales
    [ceil(R/block_rows), K/32] uint8)."""
    emax = EMAX[fmt]
    R, K = x.shape
    Rb = -(-R // block_rows)
    codes = np.empty((R, K), np.uint8)
    scales = np.empty((Rb, K // 32), np.uint8)

    def part(r0, r1):
        xs = x[r0:r1]
        n = r1 - r0
        nb = -(-n // block_rows)
        pad = nb * block_rows - n
        xp = np.pad(np.abs(xs), ((0, pad), (0, 0))) if pad else np.abs(xs)
        amax = xp.reshape(nb, block_rows, K // 32, 32).max(axis=(1, 3))
        X = np.where(amax > 0, floor_log2(np.where(amax > 0, amax, 1.0)) - emax, -127)
        code = np.clip(X + 127, 0, 254).astype(np.uint8)
        scales[r0 // block_rows:r0 // block_rows + nb] = code
        Xe = code.astype(np.int64) - 127
        Xfull = np.repeat(np.repeat(Xe, block_rows, axis=0)[:n], 32, axis=1)
        codes[r0:r1] = quantise(np.ldexp(np.asarray(xs, dtype=np.float64), -Xfull), fmt)

    _by_rows(part, R, 256 if block_rows <= 256 else block_rows)
    return codes, scales


def block_quantise_e4m3(x, block_rows):
    """e4m3 with one fp32 scale s = amax/448 per block_rows x 128 block of
    x [R, K] (K % 128 == 0; an all-zero block gets s = 1).  Returns
    (codes [R, K] uint8, scales [ceil(R/block_rows), K/128] float32)."""
    R, K = x.shape
    Rb = -(-R // block_rows)
    codes = np.empty((R, K), np.uint8)
    scales = np.empty((Rb, K // 128), np.float32)

    def part(r0, r1):
        xs = x[r0:r1]
        n = r1 - r0
        nb = -(-n // block_rows)
        pad = nb * block_rows - n
        xp = np.pad(np.abs(xs), ((0, pad), (0, 0))) if pad else np.abs(xs)
        amax = xp.reshape(nb, block_rows, K // 128, 128).max(axis=(1, 3)).astype(np.float32)
        s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
        s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
        scales[r0 // block_rows:r0 // block_rows + nb] = s
        sfull = np.repeat(np.repeat(s, block_rows, axis=0)[:n], 128, axis=1)
        codes[r0:r1] = quantise(np.asarray(xs, np.float32) / sfull, "e4m3")

    _by_rows(part, R, 256 if block_rows <= 256 else block_rows)
    return codes, scales


def rowwise_quantise_e4m3(x):
    """Per-row e4m3: s = amax/448 (fp32; an all-zero row gets s = 1), codes =
    e4m3(x/s).  Returns (codes [R, K] uint8, s [R] float32)."""
    R, K = x.shape
    codes = np.empty((R, K), np.uint8)
    scales = np.empty(R, np.float32)

    def part(r0, r1):
        xs = x[r0:r1]
        amax = np.abs(xs).max(axis=1)
        s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
        s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
        scales[r0:r1] = s
        codes[r0:r1] = quantise(xs / s[:, None], "e4m3")

    _by_rows(part, R, 256)
    return codes, scales


def bf16_bits(x):
    """float values -> bfloat16 bit patterns via torch's own cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------ activations

# Activation shapes of the quantisers: the A operand of each GEMM workload.
QUANT_SHAPES = {"f8": ("f8_ptpc", 4096, 7168), "mxfp8": ("mxfp8", 16384, 2048), "mxfp4": ("mxfp4", 8192, 8192),
                "f8_block": ("f8_block", 16384, 2048)}


def make_activations(M, K, seed=300, rot=0, outlier_cols=8):
    """bf16 activations [M, K] as bit patterns (uint16): standard normal
    values, each row scaled by 2^u (u uniform in [-6, 6]) so that rows differ
    in range, plus a few columns of 16x outliers (the heavy channels that make
    per-token and per-block scales matter).  Seeded by (seed, rot)."""
    r = rng(seed, 0, rot)
    x = r.standard_normal((M, K)).astype(np.float32)
    x *= np.exp2(r.uniform(-6, 6, (M, 1))).astype(np.float32)
    if outlier_cols and K:
        cols = r.choice(K, size=min(outlier_cols, K), replace=False)
        x[:, cols] *= np.float32(16.0)
    return bf16_bits(x)


# ------------------------------------------------------------ workloads

def make(name, rot=0, M=None, N=None, K=None, bias=None, seed=None):
    """Build one workload's inputs (numpy, host memory).  Shape overrides keep
    the recipe and seed.  Returns a dict with kind, fmt, M, N, K, A, B,
    scale_a, scale_b, bias (uint16 bf16 bits or None), b_rows_per_scale."""
    kind, M0, N0, K0, seed0, bias0, fmt, brows = WORKLOADS[name]
    M = M0 if M is None else M
    N = N0 if N is None else N
    K = K0 if K is None else K
    seed = seed0 if seed is None else seed
    has_bias = bias0 if bias is None else bias
    d = dict(name=name, kind=kind, fmt=fmt, M=M, N=N, K=K, b_rows_per_scale=brows,
             seed=seed, rot=rot)
    if kind == "i8":
        d["A"] = rng(seed, 0, rot).integers(-127, 128, size=(M, K), dtype=np.int8)
        d["B"] = rng(seed, 1, rot).integers(-127, 128, size=(N, K), dtype=np.int8)
        d["scale_a"] = rng(seed, 2, rot).uniform(1e-3, 1e-2, size=M).astype(np.float32)
        d["scale_b"] = rng(seed, 3, rot).uniform(1e-3, 1e-2, size=N).astype(np.float32)
    elif kind == "f8":
        for tid, rows, key in ((0, M, "A"), (1, N, "B")):
            x = rng(seed, tid, rot).standard_normal(size=(rows, K), dtype=np.float32)
            d[key], d["scale_a" if key == "A" else "scale_b"] = rowwise_quantise_e4m3(x)
    elif kind == "f8b":
        for tid, rows, br, key in ((0, M, 1, "A"), (1, N, 128, "B")):
            x = rng(seed, tid, rot).standard_normal(size=(rows, K), dtype=np.float32)
            codes, s = block_quantise_e4m3(x, br)
            d[key] = codes
            d["scale_a" if key == "A" else "scale_b"] = s
    elif kind == "mx":
        fa, fb = fmt.split("/") if "/" in fmt else (fmt, fmt)
        xa = rng(seed, 0, rot).standard_normal(size=(M, K), dtype=np.float32)
        ca, sa = mx_quantise(xa, fa, 1)
        del xa
        xb = rng(seed, 1, rot).standard_normal(size=(N, K), dtype=np.float32)
        cb, sb = mx_quantise(xb, fb, brows)
        del xb
        d.update(A=pack(ca, fa), B=pack(cb, fb), scale_a=sa, scale_b=sb)
    else:
        raise ValueError(name)
    d["bias"] = (bf16_bits(rng(seed, 4, rot).standard_normal(size=N).astype(np.float32))
                 if has_bias else None)
    return d


def digest(d):
    """sha256 over the input bytes, for the benchmark report."""
    h = hashlib.sha256()
    for key in ("A", "B", "scale_a", "scale_b", "bias"):
        if d.get(key) is not None:
            h.update(np.ascontiguousarray(d[key]).tobytes())
    return h.hexdigest()
