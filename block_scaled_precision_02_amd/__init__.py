"""Python binding of libqgemm, the gfx950 scaled low-precision GEMM.

    C = bf16( scale_A (.) scale_B (.) (A . B^T) + bias )

The functions carry the names of the C ABI in ``include/qgemm.h`` and only
marshal arguments: torch tensors supply device memory and the stream, every
step of the computation runs in the library's HIP kernels.  There is no
fallback: if ``libqgemm.so`` is missing, or the device is not gfx950, the
call raises.

    qgemm_i8_rowwise(A, B, scale_a, scale_b, bias=None, out=None)
    qgemm_i8_acc_i32(A, B, out=None)
    qgemm_f8_pertoken(A, B, scale_a, scale_b, bias=None, out=None)
    qgemm_f8_blockscale(A, B, scale_a, scale_b, bias=None, out=None)
    qgemm_mx(fmt, A, B, scale_a, scale_b, b_layout, bias=None, out=None, K=None)
    qgemm_mx_mixed(fmt_a, fmt_b, A, B, scale_a, scale_b, b_layout, bias=None, out=None)
    qgemm_prepack_b(B, row_bytes=None, out=None)          -> PackedB
    qgemm_i8_rowwise_prepacked(A, Bp, scale_a, scale_b, bias=None, out=None)
    qgemm_f8_pertoken_prepacked(A, Bp, scale_a, scale_b, bias=None, out=None)
    qgemm_f8_blockscale_prepacked(A, Bp, scale_a, scale_b, bias=None, out=None)
    qgemm_mx_prepacked(fmt, A, Bp, scale_a, scale_b, b_layout, bias=None, out=None)
    qgemm_prepack_b32(B, out=None)                        -> PackedB (the mixed GEMM's e2m1 B)
    qgemm_mx_mixed_prepacked(fmt_a, fmt_b, A, Bp, scale_a, scale_b, b_layout, bias=None, out=None)
    qgemm_quant_f8_pertoken(X, out=None, scale=None)      -> (Q, scale)
    qgemm_quant_f8_block(X, out=None, scales=None)        -> (Q, S)
    qgemm_quant_mx(fmt, X, out=None, scales=None)         -> (Q, S)

Operands are [rows, K] with unit stride along K (row stride may exceed the
row; it is passed as lda).  ``out`` may be a view of a wider buffer (row
stride = ldc).  Errors in arguments raise ValueError; a device or HIP
failure raises RuntimeError.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemm.so")

QGEMM_OK = 0
QGEMM_ERR_NULL_POINTER = 1
QGEMM_ERR_BAD_SHAPE = 2
QGEMM_ERR_BAD_LAYOUT = 3
QGEMM_ERR_BAD_FORMAT = 4
QGEMM_ERR_UNSUPPORTED_DEVICE = 5
QGEMM_ERR_HIP = 6

QGEMM_MX_E4M3 = 0
QGEMM_MX_E2M1 = 1
QGEMM_MX_E2M3 = 2
QGEMM_MX_E3M2 = 3
QGEMM_MX_BSCALE_1x32 = 1
QGEMM_MX_BSCALE_32x32 = 32

# Every symbol include/qgemm.h declares.
EXPORTS = ("qgemm_i8_rowwise", "qgemm_i8_acc_i32", "qgemm_f8_pertoken", "qgemm_f8_blockscale", "qgemm_mx", "qgemm_mx_mixed",
           "qgemm_prepacked_b32_bytes", "qgemm_prepack_b32", "qgemm_mx_mixed_prepacked",
           "qgemm_prepacked_b_bytes", "qgemm_prepack_b", "qgemm_i8_rowwise_prepacked",
           "qgemm_f8_pertoken_prepacked", "qgemm_f8_blockscale_prepacked", "qgemm_mx_prepacked",
           "qgemm_quant_f8_pertoken", "qgemm_quant_f8_block", "qgemm_quant_mx",
           "qgemm_last_error", "qgemm_status_string", "qgemm_select_tile",
           "qgemm_tile_rows", "qgemm_force_tile")

_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def lib():
    """The loaded C library (ctypes), with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m block_scaled_precision_02_amd.build`")
    _lib = declare(ctypes.CDLL(LIB_PATH))
    return _lib


def declare(L):
    """Declare the argument and return types of every exported function on a
    loaded copy of the library (libqgemm.so, or the conservative-sync twin
    built from the same sources) and return it."""
    st = ctypes.c_int
    L.qgemm_i8_rowwise.restype = st
    L.qgemm_i8_rowwise.argtypes = [_P, _I64, _P, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
    L.qgemm_i8_acc_i32.restype = st
    L.qgemm_i8_acc_i32.argtypes = [_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _P]
    L.qgemm_f8_pertoken.restype = st
    L.qgemm_f8_pertoken.argtypes = [_P, _I64, _P, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
    L.qgemm_f8_blockscale.restype = st
    L.qgemm_f8_blockscale.argtypes = [_P, _I64, _P, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
    L.qgemm_mx.restype = st
    L.qgemm_mx.argtypes = [ctypes.c_int, _P, _I64, _P, _I64, _P, _P, ctypes.c_int, _P, _P, _I64,
                           _I64, _I64, _I64, _P]
    L.qgemm_mx_mixed.restype = st
    L.qgemm_mx_mixed.argtypes = [ctypes.c_int, ctypes.c_int, _P, _I64, _P, _I64, _P, _P, ctypes.c_int, _P, _P,
                                 _I64, _I64, _I64, _I64, _P]
    L.qgemm_prepacked_b32_bytes.restype = _I64
    L.qgemm_prepacked_b32_bytes.argtypes = [_I64, _I64]
    L.qgemm_prepack_b32.restype = st
    L.qgemm_prepack_b32.argtypes = [_P, _I64, _I64, _I64, _P, _P]
    L.qgemm_mx_mixed_prepacked.restype = st
    L.qgemm_mx_mixed_prepacked.argtypes = [ctypes.c_int, ctypes.c_int, _P, _I64, _P, _P, _P, ctypes.c_int, _P, _P,
                                           _I64, _I64, _I64, _I64, _P]
    L.qgemm_prepacked_b_bytes.restype = _I64
    L.qgemm_prepacked_b_bytes.argtypes = [_I64, _I64]
    L.qgemm_prepack_b.restype = st
    L.qgemm_prepack_b.argtypes = [_P, _I64, _I64, _I64, _P, _P]
    L.qgemm_i8_rowwise_prepacked.restype = st
    L.qgemm_i8_rowwise_prepacked.argtypes = [_P, _I64, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
    L.qgemm_f8_pertoken_prepacked.restype = st
    L.qgemm_f8_pertoken_prepacked.argtypes = [_P, _I64, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
    L.qgemm_f8_blockscale_prepacked.restype = st
    L.qgemm_f8_blockscale_prepacked.argtypes = [_P, _I64, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
    L.qgemm_mx_prepacked.restype = st
    L.qgemm_mx_prepacked.argtypes = [ctypes.c_int, _P, _I64, _P, _P, _P, ctypes.c_int, _P, _P, _I64, _I64, _I64,
                                     _I64, _P]
    L.qgemm_quant_f8_pertoken.restype = st
    L.qgemm_quant_f8_pertoken.argtypes = [_P, _I64, _P, _I64, _P, _I64, _I64, _P]
    L.qgemm_quant_f8_block.restype = st
    L.qgemm_quant_f8_block.argtypes = [_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _P]
    L.qgemm_quant_mx.restype = st
    L.qgemm_quant_mx.argtypes = [ctypes.c_int, _P, _I64, _P, _I64, _P, _I64, _I64, _I64, _P]
    L.qgemm_last_error.restype = ctypes.c_char_p
    L.qgemm_last_error.argtypes = []
    L.qgemm_status_string.restype = ctypes.c_char_p
    L.qgemm_status_string.argtypes = [ctypes.c_int]
    L.qgemm_select_tile.restype = ctypes.c_int
    L.qgemm_select_tile.argtypes = [ctypes.c_int, _I64, _I64, _I64]
    L.qgemm_tile_rows.restype = ctypes.c_int
    L.qgemm_tile_rows.argtypes = [ctypes.c_int]
    L.qgemm_force_tile.restype = ctypes.c_int
    L.qgemm_force_tile.argtypes = [ctypes.c_int]
    return L


class QGemmError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


class QGemmArgError(QGemmError, ValueError):
    pass


def _check(status):
    if status == QGEMM_OK:
        return
    msg = lib().qgemm_last_error().decode()
    if status in (QGEMM_ERR_NULL_POINTER, QGEMM_ERR_BAD_SHAPE, QGEMM_ERR_BAD_LAYOUT,
                  QGEMM_ERR_BAD_FORMAT):
        raise QGemmArgError(status, msg)
    raise QGemmError(status, msg)


def select_tile(path, M, N, K):
    return lib().qgemm_select_tile(path, M, N, K)


def tile_rows(tile):
    return lib().qgemm_tile_rows(tile)


def force_tile(tile):
    """Force a tile id on this thread (-1 restores the table); returns the previous one."""
    prev = lib().qgemm_force_tile(tile)
    if prev == -2:
        raise ValueError(f"unknown tile id {tile}")
    return prev


# ------------------------------------------------------------ marshalling

def _torch():
    import torch
    return torch


def _operand(t, name, dtypes, row_bytes_per_elem=1):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} dtype must be one of {dtypes}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along K")
    ld = t.stride(0) * t.element_size() if t.shape[0] > 1 else t.shape[1] * t.element_size()
    return ld


def _vector(t, name, n, dtypes):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.dtype not in dtypes:
        raise ValueError(f"{name} must be a tensor of {dtypes}")
    if t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous with {n} elements, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    return t


def _out(out, M, N, device, dtype):
    torch = _torch()
    if out is None:
        # Rows padded to a multiple of 8 elements (the library's ldc rule).
        return torch.empty((M, N + (-N) % 8), dtype=dtype, device=device)[:, :N]
    if out.shape != (M, N) or out.dtype != dtype or out.device != device:
        raise ValueError(f"out must be shape {(M, N)}, dtype {dtype}, device {device}; got "
                         f"shape {tuple(out.shape)}, dtype {out.dtype}, device {out.device}")
    if N > 1 and out.stride(1) != 1:
        raise ValueError("out must have unit stride along N")
    return out


def _ldc(out, N):
    return out.stride(0) if out.shape[0] > 1 else max(N + (-N) % 8, 8)


def _same_device(device, *ts):
    for t in ts:
        if t is not None and t.device != device:
            raise ValueError(f"all tensors must be on {device}, found one on {t.device}")


def _stream(device, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _bias(bias, N):
    torch = _torch()
    return _vector(bias, "bias", N, (torch.bfloat16, torch.int16, torch.uint16))


def qgemm_i8_rowwise(A, B, scale_a, scale_b, bias=None, out=None, stream=None):
    """INT8 rowwise GEMM -> bf16 [M, N]."""
    torch = _torch()
    lda = _operand(A, "A", (torch.int8,))
    ldb = _operand(B, "B", (torch.int8,))
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError(f"A is [M, K={K}] but B is {tuple(B.shape)}")
    sa = _vector(scale_a, "scale_a", M, (torch.float32,))
    sb = _vector(scale_b, "scale_b", N, (torch.float32,))
    bias = _bias(bias, N)
    _same_device(A.device, B, sa, sb, bias)
    out = _out(out, M, N, A.device, torch.bfloat16)
    with torch.cuda.device(A.device):
        _check(lib().qgemm_i8_rowwise(_ptr(A), lda, _ptr(B), ldb, _ptr(sa), _ptr(sb), _ptr(bias),
                                      _ptr(out), _ldc(out, N), M, N, K, _stream(A.device, stream)))
    return out


def qgemm_i8_acc_i32(A, B, out=None, stream=None):
    """The INT8 product alone, int32 [M, N]."""
    torch = _torch()
    lda = _operand(A, "A", (torch.int8,))
    ldb = _operand(B, "B", (torch.int8,))
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError(f"A is [M, K={K}] but B is {tuple(B.shape)}")
    _same_device(A.device, B)
    out = _out(out, M, N, A.device, torch.int32)
    with torch.cuda.device(A.device):
        _check(lib().qgemm_i8_acc_i32(_ptr(A), lda, _ptr(B), ldb, _ptr(out), _ldc(out, N), M, N, K,
                                      _stream(A.device, stream)))
    return out


def _fp8_dtypes():
    torch = _torch()
    return (torch.uint8, torch.float8_e4m3fn)


def qgemm_f8_pertoken(A, B, scale_a, scale_b, bias=None, out=None, stream=None):
    """FP8 e4m3 per-token / per-channel GEMM -> bf16 [M, N]."""
    torch = _torch()
    lda = _operand(A, "A", _fp8_dtypes())
    ldb = _operand(B, "B", _fp8_dtypes())
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError(f"A is [M, K={K}] but B is {tuple(B.shape)}")
    sa = _vector(scale_a, "scale_a", M, (torch.float32,))
    sb = _vector(scale_b, "scale_b", N, (torch.float32,))
    bias = _bias(bias, N)
    _same_device(A.device, B, sa, sb, bias)
    out = _out(out, M, N, A.device, torch.bfloat16)
    with torch.cuda.device(A.device):
        _check(lib().qgemm_f8_pertoken(_ptr(A), lda, _ptr(B), ldb, _ptr(sa), _ptr(sb), _ptr(bias),
                                       _ptr(out), _ldc(out, N), M, N, K, _stream(A.device, stream)))
    return out


def _matrix(t, name, shape, dtypes):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype not in dtypes:
        raise ValueError(f"{name} must be a tensor of {dtypes}")
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous with shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    return t


def qgemm_f8_blockscale(A, B, scale_a, scale_b, bias=None, out=None, stream=None):
    """FP8 e4m3 GEMM with fp32 scales per 128-element K block -> bf16 [M, N].
    scale_a [M, K/128], scale_b [ceil(N/128), K/128], both contiguous."""
    torch = _torch()
    lda = _operand(A, "A", _fp8_dtypes())
    ldb = _operand(B, "B", _fp8_dtypes())
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError(f"A is [M, K={K}] but B is {tuple(B.shape)}")
    if K % 128:
        raise ValueError(f"K={K} is not a multiple of 128")
    sa = _matrix(scale_a, "scale_a", (M, K // 128), (torch.float32,))
    sb = _matrix(scale_b, "scale_b", ((N + 127) // 128, K // 128), (torch.float32,))
    bias = _bias(bias, N)
    _same_device(A.device, B, sa, sb, bias)
    out = _out(out, M, N, A.device, torch.bfloat16)
    with torch.cuda.device(A.device):
        _check(lib().qgemm_f8_blockscale(_ptr(A), lda, _ptr(B), ldb, _ptr(sa), _ptr(sb), _ptr(bias),
                                         _ptr(out), _ldc(out, N), M, N, K, _stream(A.device, stream)))
    return out


def qgemm_mx(fmt, A, B, scale_a, scale_b, b_layout, bias=None, out=None, stream=None):
    """MX GEMM -> bf16 [M, N].  fmt QGEMM_MX_E4M3 (A [M,K] bytes),
    QGEMM_MX_E2M1 (A [M,K/2] bytes, two codes per byte) or the 6-bit
    QGEMM_MX_E2M3 / QGEMM_MX_E3M2 (A [M,3K/4] bytes, four codes per three
    bytes); scale_a [M, K/32] and scale_b [N, K/32] (b_layout 1) or
    [ceil(N/32), K/32] (b_layout 32), ue8m0 codes as uint8."""
    torch = _torch()
    dts = (torch.uint8, torch.float8_e4m3fn) if fmt == QGEMM_MX_E4M3 else (torch.uint8,)
    lda = _operand(A, "A", dts)
    ldb = _operand(B, "B", dts)
    M, row = A.shape
    N = B.shape[0]
    if B.shape[1] != row:
        raise ValueError(f"A is [M, {row}] but B is {tuple(B.shape)}")
    if fmt in (QGEMM_MX_E2M3, QGEMM_MX_E3M2):
        if row % 3:
            raise ValueError(f"6-bit MX rows are 3K/4 bytes: {row} is not a multiple of 3")
        K = row // 3 * 4
    else:
        K = row if fmt == QGEMM_MX_E4M3 else 2 * row
    sdt = (torch.uint8,) + ((torch.float8_e8m0fnu,) if hasattr(torch, "float8_e8m0fnu") else ())
    brows = -(-N // b_layout) if b_layout in (1, 32) else N
    if scale_a is None or tuple(scale_a.shape) != (M, K // 32):
        raise ValueError(f"scale_a must be [{M}, {K // 32}]")
    if scale_b is None or tuple(scale_b.shape) != (brows, K // 32):
        raise ValueError(f"scale_b must be [{brows}, {K // 32}]")
    sa = _vector(scale_a.reshape(-1) if scale_a.is_contiguous() else scale_a, "scale_a",
                 M * (K // 32), sdt)
    sb = _vector(scale_b.reshape(-1) if scale_b.is_contiguous() else scale_b, "scale_b",
                 brows * (K // 32), sdt)
    bias = _bias(bias, N)
    _same_device(A.device, B, sa, sb, bias)
    out = _out(out, M, N, A.device, torch.bfloat16)
    with torch.cuda.device(A.device):
        _check(lib().qgemm_mx(fmt, _ptr(A), lda, _ptr(B), ldb, _ptr(sa), _ptr(sb), b_layout,
                              _ptr(bias), _ptr(out), _ldc(out, N), M, N, K,
                              _stream(A.device, stream)))
    return out


def qgemm_mx_mixed(fmt_a, fmt_b, A, B, scale_a, scale_b, b_layout, bias=None, out=None, stream=None):
    """MX GEMM with a format per operand -> bf16 [M, N] (e4m3 A with e2m1 B,
    e2m1 A with e4m3 B, or equal formats).  A [M, K] (e4m3) or [M, K/2]
    (e2m1) bytes, B likewise; scales as for qgemm_mx."""
    torch = _torch()

    def dts(fmt):
        return (torch.uint8, torch.float8_e4m3fn) if fmt == QGEMM_MX_E4M3 else (torch.uint8,)
    lda = _operand(A, "A", dts(fmt_a))
    ldb = _operand(B, "B", dts(fmt_b))
    M, N = A.shape[0], B.shape[0]
    K = A.shape[1] if fmt_a == QGEMM_MX_E4M3 else 2 * A.shape[1]
    kb = B.shape[1] if fmt_b == QGEMM_MX_E4M3 else 2 * B.shape[1]
    if kb != K:
        raise ValueError(f"A holds K={K} elements per row but B holds {kb}")
    sdt = (torch.uint8,) + ((torch.float8_e8m0fnu,) if hasattr(torch, "float8_e8m0fnu") else ())
    brows = -(-N // b_layout) if b_layout in (1, 32) else N
    if scale_a is None or tuple(scale_a.shape) != (M, K // 32):
        raise ValueError(f"scale_a must be [{M}, {K // 32}]")
    if scale_b is None or tuple(scale_b.shape) != (brows, K // 32):
        raise ValueError(f"scale_b must be [{brows}, {K // 32}]")
    sa = _vector(scale_a.reshape(-1) if scale_a.is_contiguous() else scale_a, "scale_a",
                 M * (K // 32), sdt)
    sb = _vector(scale_b.reshape(-1) if scale_b.is_contiguous() else scale_b, "scale_b",
                 brows * (K // 32), sdt)
    bias = _bias(bias, N)
    _same_device(A.device, B, sa, sb, bias)
    out = _out(out, M, N, A.device, torch.bfloat16)
    with torch.cuda.device(A.device):
        _check(lib().qgemm_mx_mixed(fmt_a, fmt_b, _ptr(A), lda, _ptr(B), ldb, _ptr(sa), _ptr(sb), b_layout,
                                    _ptr(bias), _ptr(out), _ldc(out, N), M, N, K,
                                    _stream(A.device, stream)))
    return out


# ------------------------------------------------------------ quantisers

def _activations(X):
    torch = _torch()
    ld = _operand(X, "X", (torch.bfloat16, torch.int16, torch.uint16))
    return ld // 2


def _codes_out(out, shape, device, name):
    torch = _torch()
    M, row = shape
    if out is None:
        # rows padded to a multiple of 16 bytes (the library's ldq rule)
        return torch.empty((M, row + (-row) % 16), dtype=torch.uint8, device=device)[:, :row]
    if tuple(out.shape) != shape or out.dtype not in (torch.uint8, torch.float8_e4m3fn) or out.device != device:
        raise ValueError(f"{name} must be uint8 {shape} on {device}")
    if row > 1 and out.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along K")
    return out


def _ld_bytes(t, row):
    return t.stride(0) * t.element_size() if t.shape[0] > 1 else row + (-row) % 16


def qgemm_quant_f8_pertoken(X, out=None, scale=None, stream=None):
    """Per-token e4m3 quantiser: bf16 X [M, K] -> (Q uint8 e4m3fn codes [M, K],
    scale fp32 [M]), the A operand and scale_a of qgemm_f8_pertoken."""
    torch = _torch()
    ldx = _activations(X)
    M, K = X.shape
    out = _codes_out(out, (M, K), X.device, "out")
    if scale is None:
        scale = torch.empty(M, dtype=torch.float32, device=X.device)
    _vector(scale, "scale", M, (torch.float32,))
    _same_device(X.device, out, scale)
    with torch.cuda.device(X.device):
        _check(lib().qgemm_quant_f8_pertoken(_ptr(X), ldx, _ptr(out), _ld_bytes(out, K), _ptr(scale), M, K,
                                             _stream(X.device, stream)))
    return out, scale


def qgemm_quant_f8_block(X, out=None, scales=None, stream=None):
    """Blockscale e4m3 quantiser: X [M, K] bf16 (K % 128 == 0) -> (Q uint8
    [M, K] e4m3 codes, S fp32 [M, K/128]), the A operand and scale_a of
    qgemm_f8_blockscale."""
    torch = _torch()
    ldx = _activations(X)
    M, K = X.shape
    if K % 128:
        raise ValueError(f"K={K} is not a multiple of 128")
    out = _codes_out(out, (M, K), X.device, "out")
    if scales is None:
        scales = torch.empty((M, K // 128), dtype=torch.float32, device=X.device)
    if (scales.dtype != torch.float32 or tuple(scales.shape) != (M, K // 128) or scales.device != X.device
            or (M > 1 and scales.stride(1) != 1)):
        raise ValueError(f"scales must be float32 [{M}, {K // 128}] with unit stride along K/128 on {X.device}")
    lds = scales.stride(0) if M > 1 else K // 128
    with torch.cuda.device(X.device):
        _check(lib().qgemm_quant_f8_block(_ptr(X), ldx, _ptr(out), _ld_bytes(out, K), _ptr(scales), lds, M, K,
                                          _stream(X.device, stream)))
    return out, scales


def qgemm_quant_mx(fmt, X, out=None, scales=None, stream=None):
    """MX quantiser: bf16 X [M, K] -> (Q uint8 [M, K] (e4m3) or [M, K/2] (e2m1,
    two codes per byte), S uint8 ue8m0 [M, K/32]), the A operand and scale_a
    of qgemm_mx."""
    torch = _torch()
    if fmt not in (QGEMM_MX_E4M3, QGEMM_MX_E2M1):
        raise ValueError(f"unknown MX format {fmt}")
    ldx = _activations(X)
    M, K = X.shape
    row = K if fmt == QGEMM_MX_E4M3 else K // 2
    out = _codes_out(out, (M, row), X.device, "out")
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=X.device)
    if tuple(scales.shape) != (M, K // 32) or scales.dtype != torch.uint8 or scales.device != X.device:
        raise ValueError(f"scales must be uint8 [{M}, {K // 32}] on {X.device}")
    if K // 32 > 1 and scales.stride(1) != 1:
        raise ValueError("scales must have unit stride along K/32")
    lds = scales.stride(0) if M > 1 else K // 32
    _same_device(X.device, out, scales)
    with torch.cuda.device(X.device):
        _check(lib().qgemm_quant_mx(fmt, _ptr(X), ldx, _ptr(out), _ld_bytes(out, row), _ptr(scales), lds, M, K,
                                    _stream(X.device, stream)))
    return out, scales


# ------------------------------------------------------------ prepacked B

class PackedB:
    """A B operand in the prepacked layout: ``data`` (uint8 device tensor of
    qgemm_prepacked_b_bytes(N, row_bytes) bytes), the row count N and the
    row length in bytes of the B it was made from."""

    def __init__(self, data, N, row_bytes, group_rows=16):
        self.data, self.N, self.row_bytes, self.group_rows = data, N, row_bytes, group_rows


def qgemm_prepack_b(B, out=None, stream=None):
    """B [N, row_bytes] (int8, e4m3 or e2m1 bytes; row_bytes a multiple of
    256) -> PackedB, for the ``_prepacked`` GEMMs."""
    torch = _torch()
    ldb = _operand(B, "B", (torch.int8, torch.uint8, torch.float8_e4m3fn))
    N, row = B.shape[0], B.shape[1] * B.element_size()
    nbytes = lib().qgemm_prepacked_b_bytes(N, row)
    if nbytes < 0:
        raise ValueError(f"B rows of {row} bytes cannot be prepacked (need a multiple of 256)")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=B.device)
    if out.numel() * out.element_size() != nbytes or not out.is_contiguous() or out.device != B.device:
        raise ValueError(f"out must be a contiguous buffer of {nbytes} bytes on {B.device}")
    with torch.cuda.device(B.device):
        _check(lib().qgemm_prepack_b(_ptr(B), ldb, N, row, _ptr(out), _stream(B.device, stream)))
    return PackedB(out, N, row)


def qgemm_prepack_b32(B, out=None, stream=None):
    """The mixed GEMM's e2m1 B [N, K/2] bytes (K/2 a multiple of 128) ->
    PackedB in 32-row groups of 32-byte pieces, for qgemm_mx_mixed_prepacked."""
    torch = _torch()
    ldb = _operand(B, "B", (torch.uint8,))
    N, row = B.shape
    nbytes = lib().qgemm_prepacked_b32_bytes(N, row)
    if nbytes < 0:
        raise ValueError(f"B rows of {row} bytes cannot be prepacked (need a multiple of 128)")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=B.device)
    if out.numel() * out.element_size() != nbytes or not out.is_contiguous() or out.device != B.device:
        raise ValueError(f"out must be a contiguous buffer of {nbytes} bytes on {B.device}")
    with torch.cuda.device(B.device):
        _check(lib().qgemm_prepack_b32(_ptr(B), ldb, N, row, _ptr(out), _stream(B.device, stream)))
    return PackedB(out, N, row, group_rows=32)


def qgemm_mx_mixed_prepacked(fmt_a, fmt_b, A, Bp, scale_a, scale_b, b_layout, bias=None, out=None, stream=None):
    """The mixed MX GEMM with a prepacked B -> bf16 [M, N]: e4m3 A [M, K] with
    an e2m1 B from qgemm_prepack_b32, or e2m1 A [M, K/2] with an e4m3 B from
    qgemm_prepack_b."""
    torch = _torch()
    if (fmt_a, fmt_b) == (QGEMM_MX_E4M3, QGEMM_MX_E2M1):
        lda = _operand(A, "A", (torch.uint8, torch.float8_e4m3fn))
        M, K = A.shape
        if not isinstance(Bp, PackedB) or Bp.group_rows != 32:
            raise ValueError("Bp must be a PackedB from qgemm_prepack_b32")
        if Bp.row_bytes != K // 2:
            raise ValueError(f"Bp was packed from rows of {Bp.row_bytes} bytes; K/2 = {K // 2}")
    elif (fmt_a, fmt_b) == (QGEMM_MX_E2M1, QGEMM_MX_E4M3):
        lda = _operand(A, "A", (torch.uint8,))
        M, K = A.shape[0], 2 * A.shape[1]
        if not isinstance(Bp, PackedB) or Bp.group_rows != 16:
            raise ValueError("Bp must be a PackedB from qgemm_prepack_b")
        if Bp.row_bytes != K:
            raise ValueError(f"Bp was packed from rows of {Bp.row_bytes} bytes; K = {K}")
    else:
        raise ValueError("the prepacked mixed GEMM takes e4m3 A with e2m1 B or e2m1 A with e4m3 B")
    N = Bp.N
    sdt = (torch.uint8,) + ((torch.float8_e8m0fnu,) if hasattr(torch, "float8_e8m0fnu") else ())
    brows = -(-N // b_layout) if b_layout in (1, 32) else N
    if scale_a is None or tuple(scale_a.shape) != (M, K // 32):
        raise ValueError(f"scale_a must be [{M}, {K // 32}]")
    if scale_b is None or tuple(scale_b.shape) != (brows, K // 32):
        raise ValueError(f"scale_b must be [{brows}, {K // 32}]")
    sa = _vector(scale_a.reshape(-1) if scale_a.is_contiguous() else scale_a, "scale_a", M * (K // 32), sdt)
    sb = _vector(scale_b.reshape(-1) if scale_b.is_contiguous() else scale_b, "scale_b", brows * (K // 32), sdt)
    bias = _bias(bias, N)
    _same_device(A.device, Bp.data, sa, sb, bias)
    out = _out(out, M, N, A.device, torch.bfloat16)
    with torch.cuda.device(A.device):
        _check(lib().qgemm_mx_mixed_prepacked(fmt_a, fmt_b, _ptr(A), lda, _ptr(Bp.data), _ptr(sa), _ptr(sb),
                                              b_layout, _ptr(bias), _ptr(out), _ldc(out, N), M, N, K,
                                              _stream(A.device, stream)))
    return out


def _packed(Bp, row):
    if not isinstance(Bp, PackedB) or Bp.group_rows != 16:
        raise ValueError("Bp must be a PackedB from qgemm_prepack_b")
    if Bp.row_bytes != row:
        raise ValueError(f"Bp was packed from rows of {Bp.row_bytes} bytes; A's rows are {row} bytes")
    return Bp


def qgemm_i8_rowwise_prepacked(A, Bp, scale_a, scale_b, bias=None, out=None, stream=None):
    """INT8 rowwise GEMM with a prepacked B -> bf16 [M, N]."""
    torch = _torch()
    lda = _operand(A, "A", (torch.int8,))
    M, K = A.shape
    Bp = _packed(Bp, K)
    N = Bp.N
    sa = _vector(scale_a, "scale_a", M, (torch.float32,))
    sb = _vector(scale_b, "scale_b", N, (torch.float32,))
    bias = _bias(bias, N)
    _same_device(A.device, Bp.data, sa, sb, bias)
    out = _out(out, M, N, A.device, torch.bfloat16)
    with torch.cuda.device(A.device):
        _check(lib().qgemm_i8_rowwise_prepacked(_ptr(A), lda, _ptr(Bp.data), _ptr(sa), _ptr(sb), _ptr(bias),
                                                _ptr(out), _ldc(out, N), M, N, K, _stream(A.device, stream)))
    return out


def qgemm_f8_pertoken_prepacked(A, Bp, scale_a, scale_b, bias=None, out=None, stream=None):
    """FP8 per-token / per-channel GEMM with a prepacked B -> bf16 [M, N]."""
    torch = _torch()
    lda = _operand(A, "A", _fp8_dtypes())
    M, K = A.shape
    Bp = _packed(Bp, K)
    N = Bp.N
    sa = _vector(scale_a, "scale_a", M, (torch.float32,))
    sb = _vector(scale_b, "scale_b", N, (torch.float32,))
    bias = _bias(bias, N)
    _same_device(A.device, Bp.data, sa, sb, bias)
    out = _out(out, M, N, A.device, torch.bfloat16)
    with torch.cuda.device(A.device):
        _check(lib().qgemm_f8_pertoken_prepacked(_ptr(A), lda, _ptr(Bp.data), _ptr(sa), _ptr(sb), _ptr(bias),
                                                 _ptr(out), _ldc(out, N), M, N, K, _stream(A.device, stream)))
    return out


def qgemm_f8_blockscale_prepacked(A, Bp, scale_a, scale_b, bias=None, out=None, stream=None):
    """FP8 blockscale GEMM with a prepacked B -> bf16 [M, N]; scale_a
    [M, K/128], scale_b [ceil(N/128), K/128] fp32, contiguous."""
    torch = _torch()
    lda = _operand(A, "A", _fp8_dtypes())
    M, K = A.shape
    Bp = _packed(Bp, K)
    N = Bp.N
    if K % 128:
        raise ValueError(f"K={K} is not a multiple of 128")
    sa = _matrix(scale_a, "scale_a", (M, K // 128), (torch.float32,))
    sb = _matrix(scale_b, "scale_b", ((N + 127) // 128, K // 128), (torch.float32,))
    bias = _bias(bias, N)
    _same_device(A.device, Bp.data, sa, sb, bias)
    out = _out(out, M, N, A.device, torch.bfloat16)
    with torch.cuda.device(A.device):
        _check(lib().qgemm_f8_blockscale_prepacked(_ptr(A), lda, _ptr(Bp.data), _ptr(sa), _ptr(sb), _ptr(bias),
                                                   _ptr(out), _ldc(out, N), M, N, K, _stream(A.device, stream)))
    return out


def qgemm_mx_prepacked(fmt, A, Bp, scale_a, scale_b, b_layout, bias=None, out=None, stream=None):
    """MX GEMM with a prepacked B -> bf16 [M, N] (scales as for qgemm_mx)."""
    torch = _torch()
    dts = (torch.uint8, torch.float8_e4m3fn) if fmt == QGEMM_MX_E4M3 else (torch.uint8,)
    lda = _operand(A, "A", dts)
    M, row = A.shape
    Bp = _packed(Bp, row)
    N = Bp.N
    K = row if fmt == QGEMM_MX_E4M3 else 2 * row
    brows = -(-N // b_layout) if b_layout in (1, 32) else N
    if scale_a is None or tuple(scale_a.shape) != (M, K // 32):
        raise ValueError(f"scale_a must be [{M}, {K // 32}]")
    if scale_b is None or tuple(scale_b.shape) != (brows, K // 32):
        raise ValueError(f"scale_b must be [{brows}, {K // 32}]")
    sa = _vector(scale_a.reshape(-1) if scale_a.is_contiguous() else scale_a, "scale_a", M * (K // 32),
                 (torch.uint8,))
    sb = _vector(scale_b.reshape(-1) if scale_b.is_contiguous() else scale_b, "scale_b", brows * (K // 32),
                 (torch.uint8,))
    bias = _bias(bias, N)
    _same_device(A.device, Bp.data, sa, sb, bias)
    out = _out(out, M, N, A.device, torch.bfloat16)
    with torch.cuda.device(A.device):
        _check(lib().qgemm_mx_prepacked(fmt, _ptr(A), lda, _ptr(Bp.data), _ptr(sa), _ptr(sb), b_layout,
                                        _ptr(bias), _ptr(out), _ldc(out, N), M, N, K, _stream(A.device, stream)))
    return out
