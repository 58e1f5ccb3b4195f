"""Thin ctypes binding over libq4k.so (include/q4k.h, include/q4k_bench.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their data pointers, sizes and the current torch
stream to the C entry point of the same name, and raises on a non-zero
return code.  There is no fallback: if libq4k.so is missing the first call
raises.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq4k.so")

Q4K_OK = 0
Q4K_EINVAL_DIM = -1
Q4K_ENULL = -2
Q4K_EALIGN = -3
Q4K_EHIP = -4
Q4K_ESCRATCH = -5

EXPORTED = (
    "q4k_gemv", "q4k_matmul", "ternary_gemv_codes", "ternary_gemv", "ternary_matmul",
    "q4k_gemv_shaped", "q4k_gemv_walk_shaped", "q4_0_gemv", "q4_0_gemv_shaped", "q6k_gemv",
    "q6k_gemv_shaped",
    "q4k_tiled_size", "q4k_relayout_tiled", "q4k_gemv_tiled", "q4k_gemv_tiled_shaped",
    "q4k_matmul_tiled", "q4k_matmul_shaped", "q4k_matmul_tiled_shaped", "ternary_matmul_shaped",
    "q4k_matmul_noalloc",
    "q4k_strerror",
    "q4k_bench_empty", "q4k_bench_delay", "q4k_bench_stream_read", "q4k_bench_copy",
)

_lib = None


class Q4KError(ValueError):
    """A non-zero return code from libq4k.so."""

    def __init__(self, code, func):
        msg = lib().q4k_strerror(code).decode()
        super().__init__(f"{func}: {msg} (code {code})")
        self.code = code


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built: run `python -m q4_packed_weight_amd.build` "
            "(there is no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    sig = {
        "q4k_gemv": [P, P, I64, I64, P, P],
        "q4k_matmul": [P, P, I64, I64, I64, P, P],
        "q4k_matmul_noalloc": [P, P, I64, I64, I64, P, P],
        "ternary_gemv_codes": [P, P, I64, I64, P, P],
        "ternary_gemv": [P, P, F, I64, I64, P, P],
        "ternary_matmul": [P, P, F, I64, I64, I64, P, P],
        "ternary_matmul_shaped": [P, P, F, I64, I64, I64, P, P, I],
        "q4k_gemv_shaped": [P, P, I64, I64, P, P, I, I, I],
        "q4_0_gemv": [P, P, I64, I64, P, P],
        "q4_0_gemv_shaped": [P, P, I64, I64, P, P, I, I, I],
        "q6k_gemv": [P, P, I64, I64, P, P],
        "q6k_gemv_shaped": [P, P, I64, I64, P, P, I, I, I],
        "q4k_relayout_tiled": [P, I64, I64, P, P],
        "q4k_gemv_tiled": [P, P, I64, I64, P, P],
        "q4k_gemv_tiled_shaped": [P, P, I64, I64, P, P, I, I, I],
        "q4k_gemv_walk_shaped": [P, P, I64, I64, P, P, I, I, I],
        "q4k_matmul_tiled": [P, P, I64, I64, I64, P, P],
        "q4k_matmul_shaped": [P, P, I64, I64, I64, P, P, I],
        "q4k_matmul_tiled_shaped": [P, P, I64, I64, I64, P, P, I],
        "q4k_bench_empty": [P],
        "q4k_bench_delay": [I64, P],
        "q4k_bench_stream_read": [P, I64, P, I64, P],
        "q4k_bench_copy": [P, P, I64, P],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = I
    L.q4k_tiled_size.argtypes = [I64, I64]
    L.q4k_tiled_size.restype = I64
    L.q4k_strerror.argtypes = [I]
    L.q4k_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else ctypes.c_void_p(t.data_ptr() or 0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc, func):
    if rc != Q4K_OK:
        raise Q4KError(rc, func)


def _expect(t, dtype, name, need=0):
    """Type/layout/size marshalling check; `need` is the element count the
    dimensions imply (0 = not checked here, the C side validates dims)."""
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if need > 0 and t.numel() < need:
        raise ValueError(f"{name} has {t.numel()} elements, the dimensions need {need}")


def _q4k_need(K, N):
    return N * (K // 256) * 144 if (K > 0 and N > 0 and K % 256 == 0) else 0


def _pos(*v):
    return all(int(a) > 0 for a in v)


def q4k_gemv(x, w_blocks, input_dim, output_dim, y, stream=None):
    K, N = int(input_dim), int(output_dim)
    _expect(x, torch.float32, "x", K if _pos(K, N) else 0)
    _expect(w_blocks, torch.uint8, "w_blocks", _q4k_need(K, N))
    _expect(y, torch.float32, "y", N if _pos(K, N) else 0)
    _check(lib().q4k_gemv(_ptr(x), _ptr(w_blocks), int(input_dim), int(output_dim),
                          _ptr(y), _stream(stream)), "q4k_gemv")
    return y


def q4k_gemv_shaped(x, w_blocks, input_dim, output_dim, y, rows_per_lane=0,
                    k_waves=0, workgroup_waves=0, stream=None):
    K, N = int(input_dim), int(output_dim)
    _expect(x, torch.float32, "x", K if _pos(K, N) else 0)
    _expect(w_blocks, torch.uint8, "w_blocks", _q4k_need(K, N))
    _expect(y, torch.float32, "y", N if _pos(K, N) else 0)
    _check(lib().q4k_gemv_shaped(_ptr(x), _ptr(w_blocks), int(input_dim),
                                 int(output_dim), _ptr(y), _stream(stream),
                                 int(rows_per_lane), int(k_waves), int(workgroup_waves)),
           "q4k_gemv_shaped")
    return y


def q4k_matmul(X, w_blocks, n_tokens, input_dim, output_dim, Y, stream=None):
    M, K, N = int(n_tokens), int(input_dim), int(output_dim)
    ok = _pos(M, K, N)
    _expect(X, torch.float32, "X", M * K if ok else 0)
    _expect(w_blocks, torch.uint8, "w_blocks", _q4k_need(K, N) if ok else 0)
    _expect(Y, torch.float32, "Y", M * N if ok else 0)
    _check(lib().q4k_matmul(_ptr(X), _ptr(w_blocks), int(n_tokens), int(input_dim),
                            int(output_dim), _ptr(Y), _stream(stream)), "q4k_matmul")
    return Y


def q4k_matmul_noalloc(X, w_blocks, n_tokens, input_dim, output_dim, Y, stream=None):
    M, K, N = int(n_tokens), int(input_dim), int(output_dim)
    ok = _pos(M, K, N)
    _expect(X, torch.float32, "X", M * K if ok else 0)
    _expect(w_blocks, torch.uint8, "w_blocks", _q4k_need(K, N) if ok else 0)
    _expect(Y, torch.float32, "Y", M * N if ok else 0)
    _check(lib().q4k_matmul_noalloc(_ptr(X), _ptr(w_blocks), M, K, N, _ptr(Y), _stream(stream)),
           "q4k_matmul_noalloc")
    return Y


def _q4_0_need(K, N):
    return N * (K // 32) * 18 if (K > 0 and N > 0 and K % 32 == 0) else 0


def q4_0_gemv(x, w_blocks, input_dim, output_dim, y, stream=None):
    K, N = int(input_dim), int(output_dim)
    _expect(x, torch.float32, "x", K if _pos(K, N) else 0)
    _expect(w_blocks, torch.uint8, "w_blocks", _q4_0_need(K, N))
    _expect(y, torch.float32, "y", N if _pos(K, N) else 0)
    _check(lib().q4_0_gemv(_ptr(x), _ptr(w_blocks), K, N, _ptr(y), _stream(stream)),
           "q4_0_gemv")
    return y


def q4_0_gemv_shaped(x, w_blocks, input_dim, output_dim, y, rows_per_lane=0,
                     k_waves=0, workgroup_waves=0, stream=None):
    K, N = int(input_dim), int(output_dim)
    _expect(x, torch.float32, "x", K if _pos(K, N) else 0)
    _expect(w_blocks, torch.uint8, "w_blocks", _q4_0_need(K, N))
    _expect(y, torch.float32, "y", N if _pos(K, N) else 0)
    _check(lib().q4_0_gemv_shaped(_ptr(x), _ptr(w_blocks), K, N, _ptr(y), _stream(stream),
                                  int(rows_per_lane), int(k_waves), int(workgroup_waves)),
           "q4_0_gemv_shaped")
    return y


def q4k_tiled_size(input_dim, output_dim):
    """Bytes of the tiled order (raises on invalid dimensions)."""
    n = lib().q4k_tiled_size(int(input_dim), int(output_dim))
    _check(n if n < 0 else Q4K_OK, "q4k_tiled_size")
    return n


def _tiled_need(K, N):
    return ((N + 15) // 16) * (K // 256) * 2304 if (K > 0 and N > 0 and K % 256 == 0) else 0


def q4k_relayout_tiled(w_blocks, input_dim, output_dim, w_tiled, stream=None):
    K, N = int(input_dim), int(output_dim)
    _expect(w_blocks, torch.uint8, "w_blocks", _q4k_need(K, N))
    _expect(w_tiled, torch.uint8, "w_tiled", _tiled_need(K, N))
    _check(lib().q4k_relayout_tiled(_ptr(w_blocks), K, N, _ptr(w_tiled), _stream(stream)),
           "q4k_relayout_tiled")
    return w_tiled


def q4k_gemv_tiled(x, w_tiled, input_dim, output_dim, y, stream=None):
    K, N = int(input_dim), int(output_dim)
    _expect(x, torch.float32, "x", K if _pos(K, N) else 0)
    _expect(w_tiled, torch.uint8, "w_tiled", _tiled_need(K, N))
    _expect(y, torch.float32, "y", N if _pos(K, N) else 0)
    _check(lib().q4k_gemv_tiled(_ptr(x), _ptr(w_tiled), K, N, _ptr(y), _stream(stream)),
           "q4k_gemv_tiled")
    return y


def q4k_matmul_shaped(X, w_blocks, n_tokens, input_dim, output_dim, Y, form=0, stream=None):
    M, K, N = int(n_tokens), int(input_dim), int(output_dim)
    _expect(X, torch.float32, "X", M * K if _pos(M, K, N) else 0)
    _expect(w_blocks, torch.uint8, "w_blocks", _q4k_need(K, N))
    _expect(Y, torch.float32, "Y", M * N if _pos(M, K, N) else 0)
    _check(lib().q4k_matmul_shaped(_ptr(X), _ptr(w_blocks), M, K, N, _ptr(Y), _stream(stream),
                                   int(form)), "q4k_matmul_shaped")
    return Y


def q4k_matmul_tiled(X, w_tiled, n_tokens, input_dim, output_dim, Y, stream=None):
    M, K, N = int(n_tokens), int(input_dim), int(output_dim)
    _expect(X, torch.float32, "X", M * K if _pos(M, K, N) else 0)
    _expect(w_tiled, torch.uint8, "w_tiled", _tiled_need(K, N))
    _expect(Y, torch.float32, "Y", M * N if _pos(M, K, N) else 0)
    _check(lib().q4k_matmul_tiled(_ptr(X), _ptr(w_tiled), M, K, N, _ptr(Y), _stream(stream)),
           "q4k_matmul_tiled")
    return Y


def q4k_matmul_tiled_shaped(X, w_tiled, n_tokens, input_dim, output_dim, Y, form=0,
                            stream=None):
    M, K, N = int(n_tokens), int(input_dim), int(output_dim)
    _expect(X, torch.float32, "X", M * K if _pos(M, K, N) else 0)
    _expect(w_tiled, torch.uint8, "w_tiled", _tiled_need(K, N))
    _expect(Y, torch.float32, "Y", M * N if _pos(M, K, N) else 0)
    _check(lib().q4k_matmul_tiled_shaped(_ptr(X), _ptr(w_tiled), M, K, N, _ptr(Y),
                                         _stream(stream), int(form)),
           "q4k_matmul_tiled_shaped")
    return Y


def q4k_gemv_walk_shaped(x, w_blocks, input_dim, output_dim, y, waves=0, row_groups=0,
                         depth=0, stream=None):
    K, N = int(input_dim), int(output_dim)
    _expect(x, torch.float32, "x", K if _pos(K, N) else 0)
    _expect(w_blocks, torch.uint8, "w_blocks", _q4k_need(K, N))
    _expect(y, torch.float32, "y", N if _pos(K, N) else 0)
    _check(lib().q4k_gemv_walk_shaped(_ptr(x), _ptr(w_blocks), K, N, _ptr(y), _stream(stream),
                                      int(waves), int(row_groups), int(depth)),
           "q4k_gemv_walk_shaped")
    return y


def q4k_gemv_tiled_shaped(x, w_tiled, input_dim, output_dim, y, waves=0, row_groups=0,
                          depth=0, stream=None):
    K, N = int(input_dim), int(output_dim)
    _expect(x, torch.float32, "x", K if _pos(K, N) else 0)
    _expect(w_tiled, torch.uint8, "w_tiled", _tiled_need(K, N))
    _expect(y, torch.float32, "y", N if _pos(K, N) else 0)
    _check(lib().q4k_gemv_tiled_shaped(_ptr(x), _ptr(w_tiled), K, N, _ptr(y), _stream(stream),
                                       int(waves), int(row_groups), int(depth)),
           "q4k_gemv_tiled_shaped")
    return y


def _q6k_need(K, N):
    return N * (K // 256) * 210 if (K > 0 and N > 0 and K % 256 == 0) else 0


def q6k_gemv(x, w_blocks, input_dim, output_dim, y, stream=None):
    K, N = int(input_dim), int(output_dim)
    _expect(x, torch.float32, "x", K if _pos(K, N) else 0)
    _expect(w_blocks, torch.uint8, "w_blocks", _q6k_need(K, N))
    _expect(y, torch.float32, "y", N if _pos(K, N) else 0)
    _check(lib().q6k_gemv(_ptr(x), _ptr(w_blocks), K, N, _ptr(y), _stream(stream)),
           "q6k_gemv")
    return y


def q6k_gemv_shaped(x, w_blocks, input_dim, output_dim, y, rows_per_lane=0,
                    k_waves=0, workgroup_waves=0, stream=None):
    K, N = int(input_dim), int(output_dim)
    _expect(x, torch.float32, "x", K if _pos(K, N) else 0)
    _expect(w_blocks, torch.uint8, "w_blocks", _q6k_need(K, N))
    _expect(y, torch.float32, "y", N if _pos(K, N) else 0)
    _check(lib().q6k_gemv_shaped(_ptr(x), _ptr(w_blocks), K, N, _ptr(y), _stream(stream),
                                 int(rows_per_lane), int(k_waves), int(workgroup_waves)),
           "q6k_gemv_shaped")
    return y


def _ternary_need(K, N):
    return N * (K // 4) if (K > 0 and N > 0 and K % 4 == 0) else 0


def ternary_gemv_codes(x, codes, input_dim, output_dim, y, stream=None):
    K, N = int(input_dim), int(output_dim)
    _expect(x, torch.float32, "x", K if _ternary_need(K, N) else 0)
    _expect(codes, torch.uint8, "codes", _ternary_need(K, N))
    _expect(y, torch.float32, "y", N if _ternary_need(K, N) else 0)
    _check(lib().ternary_gemv_codes(_ptr(x), _ptr(codes), int(input_dim),
                                    int(output_dim), _ptr(y), _stream(stream)),
           "ternary_gemv_codes")
    return y


def ternary_gemv(x, codes, scale, input_dim, output_dim, y, stream=None):
    K, N = int(input_dim), int(output_dim)
    _expect(x, torch.float32, "x", K if _ternary_need(K, N) else 0)
    _expect(codes, torch.uint8, "codes", _ternary_need(K, N))
    _expect(y, torch.float32, "y", N if _ternary_need(K, N) else 0)
    _check(lib().ternary_gemv(_ptr(x), _ptr(codes), float(scale), int(input_dim),
                              int(output_dim), _ptr(y), _stream(stream)), "ternary_gemv")
    return y


def ternary_matmul(X, codes, scale, n_tokens, input_dim, output_dim, Y, stream=None):
    M, K, N = int(n_tokens), int(input_dim), int(output_dim)
    ok = M > 0 and _ternary_need(K, N) > 0
    _expect(X, torch.float32, "X", M * K if ok else 0)
    _expect(codes, torch.uint8, "codes", _ternary_need(K, N))
    _expect(Y, torch.float32, "Y", M * N if ok else 0)
    _check(lib().ternary_matmul(_ptr(X), _ptr(codes), float(scale), M, K, N, _ptr(Y),
                                _stream(stream)), "ternary_matmul")
    return Y


def ternary_matmul_shaped(X, codes, scale, n_tokens, input_dim, output_dim, Y, form=0,
                          stream=None):
    M, K, N = int(n_tokens), int(input_dim), int(output_dim)
    ok = M > 0 and _ternary_need(K, N) > 0
    _expect(X, torch.float32, "X", M * K if ok else 0)
    _expect(codes, torch.uint8, "codes", _ternary_need(K, N))
    _expect(Y, torch.float32, "Y", M * N if ok else 0)
    _check(lib().ternary_matmul_shaped(_ptr(X), _ptr(codes), float(scale), M, K, N, _ptr(Y),
                                       _stream(stream), int(form)), "ternary_matmul_shaped")
    return Y


def bench_empty(stream=None):
    _check(lib().q4k_bench_empty(_stream(stream)), "q4k_bench_empty")


def bench_delay(ns, stream=None):
    _check(lib().q4k_bench_delay(int(ns), _stream(stream)), "q4k_bench_delay")


def bench_stream_read(src, sink, stream=None):
    _expect(sink, torch.int32, "sink")
    _check(lib().q4k_bench_stream_read(_ptr(src), src.numel() * src.element_size(),
                                       _ptr(sink), sink.numel(), _stream(stream)),
           "q4k_bench_stream_read")


def bench_copy(src, dst, stream=None):
    n = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= n
    _check(lib().q4k_bench_copy(_ptr(src), _ptr(dst), n, _stream(stream)),
           "q4k_bench_copy")
