"""CPU oracle for the scaled low-precision GEMM (test infrastructure only).

Loads ``liboracle.so`` built from ``qgemm_oracle.c`` (plain C, OpenMP, fp64
accumulation, fixed-order binary32 epilogue).  Only the tests, the smoke
check and the benchmark's CPU-baseline leg import this package; the product
library never does.  It shares no code with the HIP path: inputs arrive as
numpy arrays and results leave as numpy arrays.

Functions follow the definitions in ``qgemm_oracle.c``:
  i8_rowwise   -- INT8, rowwise fp32 scales (comfy-kitchen PR #174 "Optimize
                  HIP WMMA INT8 GEMM ...": Summary, Validation).
  f8_pertoken  -- FP8 e4m3 per-token / per-channel (ROCm/mori PR #806,
                  Measured: "ptpc").
  mx           -- MX e4m3 / e2m1 with ue8m0 per 32 K elements (ROCm/mori PR
                  #806, What; ROCm/FlyDSL PR #990).
  mx2          -- MX with its own element format per operand (e.g. e4m3
                  activations x e2m1 weights); the same scale rule.
  mxf          -- MX with any of e4m3, e2m1 and the 6-bit e2m3 / e3m2
                  (OCP Microscaling v1.0's FP6) per operand; the same rule.
  f8_blockscale
               -- FP8 e4m3 with fp32 scales per 128-element K block: A per
                  row, B per 128 rows (ROCm/mori PR #806, commit message
                  table: "blockscale"; the block sizes are a reading, stated
                  in ``qgemm_oracle.c``).
  pack_b       -- the prepacked weight layout of the ``_prepacked`` GEMM entry
                  points (defined in ``qgemm_oracle.c``).
  pack_b32     -- the prepacked layout of an e2m1 B under e4m3 A (32-row
                  groups of 32-byte pieces; ``qgemm_mx_mixed_prepacked``).
  quant_f8_pertoken, quant_f8_block, quant_mx
               -- the activation quantisers producing those operands from
                  bf16 (ROCm/mori PR #806, What: the quantiser's [M, K/32]
                  uint8 scales; the scale rules are readings, stated in
                  ``qgemm_oracle.c``).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "qgemm_oracle.c")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64

MX_E4M3 = 0
MX_E2M1 = 1
MX_E2M3 = 2
MX_E3M2 = 3


def build(force=True):
    """Compile liboracle.so with gcc (no fast-math, no FP contraction)."""
    import subprocess
    cmd = ["gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    if force or not os.path.exists(_LIB_PATH):
        subprocess.check_call(cmd)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_dec_e4m3.restype = ctypes.c_double
    lib.orc_dec_e4m3.argtypes = [ctypes.c_uint8]
    lib.orc_dec_e2m1.restype = ctypes.c_double
    lib.orc_dec_e2m1.argtypes = [ctypes.c_uint8]
    lib.orc_dec_ue8m0.restype = ctypes.c_double
    lib.orc_dec_ue8m0.argtypes = [ctypes.c_uint8]
    lib.orc_bf16_rne.restype = ctypes.c_uint16
    lib.orc_bf16_rne.argtypes = [ctypes.c_float]
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_dec_e2m3.restype = ctypes.c_double
    lib.orc_dec_e2m3.argtypes = [ctypes.c_uint8]
    lib.orc_dec_e3m2.restype = ctypes.c_double
    lib.orc_dec_e3m2.argtypes = [ctypes.c_uint8]
    lib.orc_mx_codes.restype = None
    lib.orc_mx_codes.argtypes = [ctypes.c_int, _P, _I64, _P]
    lib.orc_mx_row_bytes.restype = _I64
    lib.orc_mx_row_bytes.argtypes = [ctypes.c_int, _I64]
    lib.orc_mxf.restype = ctypes.c_int
    lib.orc_mxf.argtypes = [ctypes.c_int, ctypes.c_int, _P, _I64, _P, _I64, _P, _P, ctypes.c_int, _P,
                            _P, _I64, _P, _P, _I64, _I64, _I64]
    for name in ("orc_dec_e4m3_array", "orc_dec_e2m1_array", "orc_dec_ue8m0_array",
                 "orc_bf16_rne_array", "orc_dec_e2m3_array", "orc_dec_e3m2_array"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [_P, _P, _I64]
    for name in ("orc_enc_e4m3_array", "orc_enc_e2m1_array"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [_P, _P, _I64]
    lib.orc_quant_f8_pertoken.restype = None
    lib.orc_quant_f8_pertoken.argtypes = [_P, _I64, _P, _I64, _P, _I64, _I64]
    lib.orc_quant_f8_block.restype = ctypes.c_int
    lib.orc_quant_f8_block.argtypes = [_P, _I64, _P, _I64, _P, _I64, _I64, _I64]
    lib.orc_quant_mx.restype = ctypes.c_int
    lib.orc_quant_mx.argtypes = [ctypes.c_int, _P, _I64, _P, _I64, _P, _I64, _I64, _I64]
    lib.orc_pack_b32.restype = None
    lib.orc_pack_b32.argtypes = [_P, _I64, _I64, _I64, _P]
    lib.orc_pack_b.restype = None
    lib.orc_pack_b.argtypes = [_P, _I64, _I64, _I64, _P]
    lib.orc_i8_rowwise.restype = ctypes.c_int
    lib.orc_i8_rowwise.argtypes = [_P, _I64, _P, _I64, _P, _P, _P, _P, _I64, _P,
                                   _I64, _I64, _I64]
    lib.orc_f8_pertoken.restype = None
    lib.orc_f8_pertoken.argtypes = [_P, _I64, _P, _I64, _P, _P, _P, _P, _I64, _P, _P,
                                    _I64, _I64, _I64]
    lib.orc_mx2.restype = ctypes.c_int
    lib.orc_mx2.argtypes = [ctypes.c_int, ctypes.c_int, _P, _I64, _P, _I64, _P, _P, ctypes.c_int, _P,
                            _P, _I64, _P, _P, _I64, _I64, _I64]
    lib.orc_f8_blockscale.restype = ctypes.c_int
    lib.orc_f8_blockscale.argtypes = [_P, _I64, _P, _I64, _P, _P, _P, _P, _I64, _P, _P,
                                      _I64, _I64, _I64]
    lib.orc_mx.restype = ctypes.c_int
    lib.orc_mx.argtypes = [ctypes.c_int, _P, _I64, _P, _I64, _P, _P, ctypes.c_int, _P,
                           _P, _I64, _P, _P, _I64, _I64, _I64]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def num_threads():
    return _load().orc_num_threads()


def dec_e4m3(codes):
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float64)
    _load().orc_dec_e4m3_array(_ptr(codes), _ptr(out), codes.size)
    return out


def dec_e2m1(nibbles):
    nibbles = _c(nibbles, np.uint8)
    out = np.empty(nibbles.shape, np.float64)
    _load().orc_dec_e2m1_array(_ptr(nibbles), _ptr(out), nibbles.size)
    return out


def dec_ue8m0(codes):
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float64)
    _load().orc_dec_ue8m0_array(_ptr(codes), _ptr(out), codes.size)
    return out


def bf16_rne(x):
    """binary32 values -> bfloat16 bit patterns (uint16), round-nearest-even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().orc_bf16_rne_array(_ptr(x), _ptr(out), x.size)
    return out


def i8_rowwise(A, B, scale_a, scale_b, bias=None):
    """INT8 rowwise GEMM.  A [M,K] int8, B [N,K] int8, scale_a [M] / scale_b [N]
    float32, bias [N] bf16 bits (uint16) or None.
    Returns (C bf16 bits uint16 [M,N], acc int32 [M,N])."""
    A = _c(A, np.int8)
    B = _c(B, np.int8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    sa = _c(scale_a, np.float32)
    sb = _c(scale_b, np.float32)
    bias = _c(bias, np.uint16)
    assert sa.shape == (M,) and sb.shape == (N,)
    C = np.empty((M, N), np.uint16)
    acc = np.empty((M, N), np.int32)
    rc = _load().orc_i8_rowwise(_ptr(A), K, _ptr(B), K, _ptr(sa), _ptr(sb), _ptr(bias),
                                _ptr(C), N, _ptr(acc), M, N, K)
    if rc != 0:
        raise OverflowError("int32 accumulator out of range")
    return C, acc


def f8_pertoken(A, B, scale_a, scale_b, bias=None):
    """FP8 e4m3 per-token/per-channel GEMM.  A [M,K], B [N,K] uint8 e4m3 codes.
    Returns (C uint16 [M,N], acc float64 [M,N], absdot float64 [M,N])."""
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    sa = _c(scale_a, np.float32)
    sb = _c(scale_b, np.float32)
    bias = _c(bias, np.uint16)
    assert sa.shape == (M,) and sb.shape == (N,)
    C = np.empty((M, N), np.uint16)
    acc = np.empty((M, N), np.float64)
    absdot = np.empty((M, N), np.float64)
    _load().orc_f8_pertoken(_ptr(A), K, _ptr(B), K, _ptr(sa), _ptr(sb), _ptr(bias),
                            _ptr(C), N, _ptr(acc), _ptr(absdot), M, N, K)
    return C, acc, absdot


def mx(fmt, A, B, scale_a, scale_b, b_rows_per_scale, K, bias=None):
    """MX GEMM.  fmt MX_E4M3 (A [M,K], B [N,K] bytes) or MX_E2M1 (A [M,K/2],
    B [N,K/2] bytes, element k in the low nibble when k is even).  scale_a
    [M,K/32] ue8m0, scale_b [N or ceil(N/32), K/32] ue8m0.
    Returns (C uint16 [M,N], acc float64 [M,N], absdot float64 [M,N])."""
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    M, N = A.shape[0], B.shape[0]
    row_bytes = K if fmt == MX_E4M3 else K // 2
    assert A.shape[1] == row_bytes and B.shape[1] == row_bytes and K % 32 == 0
    sa = _c(scale_a, np.uint8)
    sb = _c(scale_b, np.uint8)
    assert sa.shape == (M, K // 32)
    assert sb.shape == ((N + b_rows_per_scale - 1) // b_rows_per_scale, K // 32)
    bias = _c(bias, np.uint16)
    C = np.empty((M, N), np.uint16)
    acc = np.empty((M, N), np.float64)
    absdot = np.empty((M, N), np.float64)
    rc = _load().orc_mx(fmt, _ptr(A), row_bytes, _ptr(B), row_bytes, _ptr(sa), _ptr(sb),
                        b_rows_per_scale, _ptr(bias), _ptr(C), N, _ptr(acc), _ptr(absdot),
                        M, N, K)
    if rc != 0:
        raise ValueError("bad MX format or B-scale layout")
    return C, acc, absdot


def mx2(fmt_a, fmt_b, A, B, scale_a, scale_b, b_rows_per_scale, K, bias=None):
    """MX GEMM with a format per operand (MX_E4M3: [rows, K] bytes; MX_E2M1:
    [rows, K/2] bytes, element k even in the low nibble).  Scales as for mx.
    Returns (C uint16 [M,N], acc float64 [M,N], absdot float64 [M,N])."""
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    M, N = A.shape[0], B.shape[0]
    row_a = K if fmt_a == MX_E4M3 else K // 2
    row_b = K if fmt_b == MX_E4M3 else K // 2
    assert A.shape[1] == row_a and B.shape[1] == row_b and K % 32 == 0
    sa = _c(scale_a, np.uint8)
    sb = _c(scale_b, np.uint8)
    assert sa.shape == (M, K // 32)
    assert sb.shape == ((N + b_rows_per_scale - 1) // b_rows_per_scale, K // 32)
    bias = _c(bias, np.uint16)
    C = np.empty((M, N), np.uint16)
    acc = np.empty((M, N), np.float64)
    absdot = np.empty((M, N), np.float64)
    rc = _load().orc_mx2(fmt_a, fmt_b, _ptr(A), row_a, _ptr(B), row_b, _ptr(sa), _ptr(sb),
                         b_rows_per_scale, _ptr(bias), _ptr(C), N, _ptr(acc), _ptr(absdot), M, N, K)
    if rc != 0:
        raise ValueError("bad MX format or B-scale layout")
    return C, acc, absdot


def dec_e2m3(codes):
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_dec_e2m3_array(_ptr(c), _ptr(out), c.size)
    return out


def dec_e3m2(codes):
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_dec_e3m2_array(_ptr(c), _ptr(out), c.size)
    return out


def mx_row_bytes(fmt, K):
    return int(_load().orc_mx_row_bytes(fmt, K))


def mx_codes(fmt, row, K):
    """Element codes 0..K-1 of one packed MX operand row (the element layout
    the oracle reads)."""
    r = _c(row, np.uint8)
    assert r.size >= mx_row_bytes(fmt, K)
    out = np.empty(K, np.uint8)
    _load().orc_mx_codes(fmt, _ptr(r), K, _ptr(out))
    return out


def mxf(fmt_a, fmt_b, A, B, scale_a, scale_b, b_rows_per_scale, K, bias=None):
    """MX GEMM with any of MX_E4M3, MX_E2M1, MX_E2M3, MX_E3M2 per operand
    (rows of K, K/2, 3K/4 and 3K/4 bytes; 6-bit elements packed lowest bits
    first, four in three bytes).  Scales as for mx.
    Returns (C uint16 [M,N], acc float64 [M,N], absdot float64 [M,N])."""
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    M, N = A.shape[0], B.shape[0]
    row_a, row_b = mx_row_bytes(fmt_a, K), mx_row_bytes(fmt_b, K)
    assert A.shape[1] == row_a and B.shape[1] == row_b and K % 32 == 0
    sa = _c(scale_a, np.uint8)
    sb = _c(scale_b, np.uint8)
    assert sa.shape == (M, K // 32)
    assert sb.shape == ((N + b_rows_per_scale - 1) // b_rows_per_scale, K // 32)
    bias = _c(bias, np.uint16)
    C = np.empty((M, N), np.uint16)
    acc = np.empty((M, N), np.float64)
    absdot = np.empty((M, N), np.float64)
    rc = _load().orc_mxf(fmt_a, fmt_b, _ptr(A), row_a, _ptr(B), row_b, _ptr(sa), _ptr(sb),
                         b_rows_per_scale, _ptr(bias), _ptr(C), N, _ptr(acc), _ptr(absdot), M, N, K)
    if rc != 0:
        raise ValueError("bad MX format, B-scale layout or K")
    return C, acc, absdot


def f8_blockscale(A, B, scale_a, scale_b, bias=None):
    """FP8 e4m3 GEMM with block scales.  A [M,K], B [N,K] uint8 e4m3 codes,
    K % 128 == 0; scale_a float32 [M, K/128]; scale_b float32
    [ceil(N/128), K/128].
    Returns (C uint16 [M,N], acc float64 [M,N], absdot float64 [M,N])."""
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K and K % 128 == 0
    sa = _c(scale_a, np.float32)
    sb = _c(scale_b, np.float32)
    assert sa.shape == (M, K // 128) and sb.shape == ((N + 127) // 128, K // 128)
    bias = _c(bias, np.uint16)
    C = np.empty((M, N), np.uint16)
    acc = np.empty((M, N), np.float64)
    absdot = np.empty((M, N), np.float64)
    rc = _load().orc_f8_blockscale(_ptr(A), K, _ptr(B), K, _ptr(sa), _ptr(sb), _ptr(bias),
                                   _ptr(C), N, _ptr(acc), _ptr(absdot), M, N, K)
    if rc != 0:
        raise ValueError("K must be a multiple of 128")
    return C, acc, absdot


def enc_e4m3(y):
    """float64 values -> e4m3fn codes (nearest, ties to even, saturating, sign kept)."""
    y = _c(y, np.float64)
    out = np.empty(y.shape, np.uint8)
    _load().orc_enc_e4m3_array(_ptr(y), _ptr(out), y.size)
    return out


def enc_e2m1(y):
    """float64 values -> e2m1 codes, one per byte (0..15)."""
    y = _c(y, np.float64)
    out = np.empty(y.shape, np.uint8)
    _load().orc_enc_e2m1_array(_ptr(y), _ptr(out), y.size)
    return out


def quant_f8_pertoken(X):
    """Per-token e4m3 quantiser.  X [M,K] bf16 bits (uint16).
    Returns (Q uint8 [M,K] e4m3 codes, scale float32 [M])."""
    X = _c(X, np.uint16)
    M, K = X.shape
    Q = np.empty((M, K), np.uint8)
    s = np.empty(M, np.float32)
    _load().orc_quant_f8_pertoken(_ptr(X), K, _ptr(Q), K, _ptr(s), M, K)
    return Q, s


def quant_f8_block(X):
    """Blockscale e4m3 quantiser, one fp32 scale per 128 elements of a row.
    X [M,K] bf16 bits (uint16), K % 128 == 0.
    Returns (Q uint8 [M,K] e4m3 codes, S float32 [M, K/128])."""
    X = _c(X, np.uint16)
    M, K = X.shape
    assert K % 128 == 0
    Q = np.empty((M, K), np.uint8)
    S = np.empty((M, K // 128), np.float32)
    if _load().orc_quant_f8_block(_ptr(X), K, _ptr(Q), K, _ptr(S), K // 128, M, K) != 0:
        raise ValueError("K must be a multiple of 128")
    return Q, S


def quant_mx(fmt, X):
    """MX quantiser, one ue8m0 scale per 32 elements of a row.  X [M,K] bf16
    bits (uint16), K % 32 == 0.  Returns (Q uint8 [M,K] (e4m3) or [M,K/2]
    (e2m1, element k even in the low nibble), S uint8 [M,K/32])."""
    X = _c(X, np.uint16)
    M, K = X.shape
    assert K % 32 == 0
    row = K if fmt == MX_E4M3 else K // 2
    Q = np.zeros((M, row), np.uint8)
    S = np.empty((M, K // 32), np.uint8)
    rc = _load().orc_quant_mx(fmt, _ptr(X), K, _ptr(Q), row, _ptr(S), K // 32, M, K)
    if rc != 0:
        raise ValueError("bad MX format")
    return Q, S


def pack_b(B):
    """B [N, row_bytes] bytes (row_bytes % 64 == 0) -> the prepacked layout,
    uint8 [ceil(N/16) * 16 * row_bytes]."""
    B = _c(B, np.uint8)
    N, row = B.shape
    assert row % 64 == 0
    out = np.empty(((N + 15) // 16) * 16 * row, np.uint8)
    _load().orc_pack_b(_ptr(B), row, N, row, _ptr(out))
    return out


def pack_b32(B):
    """B [N, row_bytes] bytes (row_bytes % 32 == 0) -> the prepacked layout of
    an e2m1 B under e4m3 A, uint8 [ceil(N/32) * 32 * row_bytes]."""
    B = _c(B, np.uint8)
    N, row = B.shape
    assert row % 32 == 0
    out = np.empty(((N + 31) // 32) * 32 * row, np.uint8)
    _load().orc_pack_b32(_ptr(B), row, N, row, _ptr(out))
    return out
