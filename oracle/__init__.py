"""CPU oracle for the Q4_K, Q4_0, Q6_K and ternary matrix-vector products.

TEST INFRASTRUCTURE ONLY: this package may be imported by tests/, by the
package smoke check and by bench.py's CPU-baseline leg, nothing else.  It
loads oracle/libq4k_oracle.so (plain scalar C, see q4k_oracle.c) through
ctypes and takes/returns numpy arrays.  It shares no code with the GPU
library.

Every function here follows a passage of the pages (cited in q4k_oracle.c)
and is pinned by tests/test_oracle_pins.py.
"""
import ctypes
import os

import numpy as np

from ._build import LIB as _LIB_PATH

_lib = None

OK = 0
EINVAL_DIM = -1
ENULL = -2


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"oracle library {_LIB_PATH} is not built; run "
            "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_f16_to_f32_array.argtypes = [P, P, I64]
    lib.oracle_f16_to_f32_array.restype = None
    lib.oracle_q4k_unpack_scales.argtypes = [P, P, P]
    lib.oracle_q4k_unpack_scales.restype = None
    lib.oracle_q4k_dequant_block.argtypes = [P, P]
    lib.oracle_q4k_dequant_block.restype = None
    for name in ("oracle_q4k_gemv", "oracle_q4k_gemv_lazy"):
        f = getattr(lib, name)
        f.argtypes = [P, P, I64, I64, P]
        f.restype = ctypes.c_int
    lib.oracle_q4k_matmul.argtypes = [P, P, I64, I64, I64, P]
    lib.oracle_q4k_matmul.restype = ctypes.c_int
    lib.oracle_q4k_matmul_part.argtypes = [P, P, I64, I64, I64, I64, I64,
                                           I64, I64, P]
    lib.oracle_q4k_matmul_part.restype = ctypes.c_int
    lib.oracle_q4_0_dequant_block.argtypes = [P, P]
    lib.oracle_q4_0_dequant_block.restype = None
    lib.oracle_q4_0_gemv.argtypes = [P, P, I64, I64, P]
    lib.oracle_q4_0_gemv.restype = ctypes.c_int
    lib.oracle_q6k_dequant_block.argtypes = [P, P]
    lib.oracle_q6k_dequant_block.restype = None
    lib.oracle_q6k_gemv.argtypes = [P, P, I64, I64, P]
    lib.oracle_q6k_gemv.restype = ctypes.c_int
    lib.oracle_q4k_relayout_tiled.argtypes = [P, I64, I64, P]
    lib.oracle_q4k_relayout_tiled.restype = ctypes.c_int
    lib.oracle_ternary_decode_byte.argtypes = [ctypes.c_uint8, P]
    lib.oracle_ternary_decode_byte.restype = None
    lib.oracle_ternary_gemv_codes.argtypes = [P, P, I64, I64, P]
    lib.oracle_ternary_gemv_codes.restype = ctypes.c_int
    lib.oracle_ternary_gemv.argtypes = [P, P, ctypes.c_float, I64, I64, P]
    lib.oracle_ternary_gemv.restype = ctypes.c_int
    lib.oracle_ternary_matmul.argtypes = [P, P, ctypes.c_float, I64, I64, I64, P]
    lib.oracle_ternary_matmul.restype = ctypes.c_int
    _lib = lib
    return lib


class OracleError(ValueError):
    def __init__(self, code):
        super().__init__(f"oracle rejected the call (code {code})")
        self.code = code


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != OK:
        raise OracleError(rc)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _u8(a):
    return np.ascontiguousarray(a, dtype=np.uint8)


def f16_to_f32(bits):
    """binary16 bit patterns (uint16 array) -> float32 values."""
    h = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    _load().oracle_f16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


def q4k_unpack_scales(s12):
    """12 packed bytes -> (sc[8], m[8]) as uint8 arrays."""
    s = _u8(s12)
    assert s.size == 12
    sc = np.zeros(8, np.uint8)
    m = np.zeros(8, np.uint8)
    _load().oracle_q4k_unpack_scales(_ptr(s), _ptr(sc), _ptr(m))
    return sc, m


def q4k_dequant_block(block):
    """One 144-byte block -> 256 fp32 weights."""
    b = _u8(block)
    assert b.size == 144
    w = np.empty(256, np.float32)
    _load().oracle_q4k_dequant_block(_ptr(b), _ptr(w))
    return w


def q4k_gemv(x, w_blocks, input_dim, output_dim):
    """y = W x in float64 (dequantize to fp32, then a double dot)."""
    xx, ww = _f32(x), _u8(w_blocks)
    y = np.empty(max(int(output_dim), 0), np.float64)
    _check(_load().oracle_q4k_gemv(_ptr(xx), _ptr(ww), input_dim, output_dim,
                                   _ptr(y)))
    return y


def q4k_gemv_lazy(x, w_blocks, input_dim, output_dim):
    """y = W x evaluated in the lazy-dmin form, float64."""
    xx, ww = _f32(x), _u8(w_blocks)
    y = np.empty(max(int(output_dim), 0), np.float64)
    _check(_load().oracle_q4k_gemv_lazy(_ptr(xx), _ptr(ww), input_dim,
                                        output_dim, _ptr(y)))
    return y


def q4k_matmul(X, w_blocks, n_tokens, input_dim, output_dim):
    """Y[M, N] = X[M, K] W^T in float64."""
    xx, ww = _f32(X), _u8(w_blocks)
    Y = np.empty((max(int(n_tokens), 0), max(int(output_dim), 0)), np.float64)
    _check(_load().oracle_q4k_matmul(_ptr(xx), _ptr(ww), n_tokens, input_dim,
                                     output_dim, _ptr(Y)))
    return Y


def q4k_matmul_part(X, w_blocks, n_tokens, input_dim, output_dim, tokens,
                    rows):
    """Entries Y[t, o] for t in range(*tokens), o in range(*rows); the rest of
    the returned [M, N] array is NaN."""
    xx, ww = _f32(X), _u8(w_blocks)
    Y = np.full((int(n_tokens), int(output_dim)), np.nan, np.float64)
    _check(_load().oracle_q4k_matmul_part(
        _ptr(xx), _ptr(ww), n_tokens, input_dim, output_dim, tokens[0],
        tokens[1], rows[0], rows[1], _ptr(Y)))
    return Y


def q4k_tiled_size(input_dim, output_dim):
    """Bytes of a Q4_K matrix in the tiled block order (row groups of 16)."""
    return ((int(output_dim) + 15) // 16) * (int(input_dim) // 256) * 2304


def q4k_relayout_tiled(w_blocks, input_dim, output_dim):
    """The canonical Q4_K matrix moved into the tiled block order (uint8)."""
    ww = _u8(w_blocks)
    size = max(q4k_tiled_size(input_dim, output_dim), 0) if output_dim > 0 else 0
    out = np.zeros(max(size, 1), np.uint8)
    _check(_load().oracle_q4k_relayout_tiled(_ptr(ww), input_dim, output_dim,
                                             _ptr(out)))
    return out[:size]


def q4_0_dequant_block(block):
    """One 18-byte Q4_0 block -> 32 fp32 weights."""
    b = _u8(block)
    assert b.size == 18
    w = np.empty(32, np.float32)
    _load().oracle_q4_0_dequant_block(_ptr(b), _ptr(w))
    return w


def q4_0_gemv(x, w_blocks, input_dim, output_dim):
    """y = W x for a Q4_0 matrix, float64 (dequantize, then a double dot)."""
    xx, ww = _f32(x), _u8(w_blocks)
    y = np.empty(max(int(output_dim), 0), np.float64)
    _check(_load().oracle_q4_0_gemv(_ptr(xx), _ptr(ww), input_dim, output_dim,
                                    _ptr(y)))
    return y


def q6k_dequant_block(block):
    """One 210-byte Q6_K block -> 256 fp32 weights."""
    b = _u8(block)
    assert b.size == 210
    w = np.empty(256, np.float32)
    _load().oracle_q6k_dequant_block(_ptr(b), _ptr(w))
    return w


def q6k_gemv(x, w_blocks, input_dim, output_dim):
    """y = W x for a Q6_K matrix, float64 (dequantize, then a double dot)."""
    xx, ww = _f32(x), _u8(w_blocks)
    y = np.empty(max(int(output_dim), 0), np.float64)
    _check(_load().oracle_q6k_gemv(_ptr(xx), _ptr(ww), input_dim, output_dim,
                                   _ptr(y)))
    return y


def ternary_decode_byte(byte):
    c = np.zeros(4, np.int32)
    _load().oracle_ternary_decode_byte(int(byte), _ptr(c))
    return c


def ternary_gemv_codes(x, codes, input_dim, output_dim):
    """t = codes-dot (scale not applied), float64."""
    xx, cc = _f32(x), _u8(codes)
    t = np.empty(max(int(output_dim), 0), np.float64)
    _check(_load().oracle_ternary_gemv_codes(_ptr(xx), _ptr(cc), input_dim,
                                             output_dim, _ptr(t)))
    return t


def ternary_gemv(x, codes, scale, input_dim, output_dim):
    """y = scale * codes-dot, float64."""
    xx, cc = _f32(x), _u8(codes)
    y = np.empty(max(int(output_dim), 0), np.float64)
    _check(_load().oracle_ternary_gemv(_ptr(xx), _ptr(cc), float(scale),
                                       input_dim, output_dim, _ptr(y)))
    return y


def ternary_matmul(X, codes, scale, n_tokens, input_dim, output_dim):
    """Y[r] = scale * codes-dot(X[r]) for each token row, float64 [M, N]."""
    XX, cc = _f32(X), _u8(codes)
    Y = np.empty((max(int(n_tokens), 0), max(int(output_dim), 0)), np.float64)
    _check(_load().oracle_ternary_matmul(_ptr(XX), _ptr(cc), np.float32(scale), n_tokens,
                                         input_dim, output_dim, _ptr(Y)))
    return Y
