"""C-ABI checks that need no GPU: the library loads, exports every function
include/*.h declares, and rejects bad arguments before launching anything
(the Q4_K page's test plan: inputDim not a multiple of 256 is rejected).

The rejection calls pass fake, never-dereferenced pointers: validation runs
before any HIP call, so these return without touching a device.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(inc, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return names


@pytest.fixture(scope="module")
def lib():
    from q4_packed_weight_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from q4_packed_weight_amd import build
        build.build()
    return binding.lib()


def test_headers_declare_the_boundary():
    names = set(_declared_functions())
    for n in ("q4k_gemv", "q4k_matmul", "ternary_gemv_codes", "ternary_gemv",
              "q4k_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_binding_covers_every_export(lib):
    from q4_packed_weight_amd import binding
    assert set(_declared_functions()) == set(binding.EXPORTED)


P = ctypes.c_void_p
GOOD = P(0x10000)       # 16-byte aligned fake device addresses
GOOD2 = P(0x20000)
GOOD3 = P(0x30000)
ODD = P(0x10004)


@pytest.mark.parametrize("K", [255, 257, 4000, 0, -256, 1 << 31, (1 << 24) + 256])
def test_q4k_rejects_bad_input_dim(lib, K):
    assert lib.q4k_gemv(GOOD, GOOD2, K, 16, GOOD3, None) == -1
    assert lib.q4k_matmul(GOOD, GOOD2, 4, K, 16, GOOD3, None) == -1
    assert lib.q4k_gemv_shaped(GOOD, GOOD2, K, 16, GOOD3, None, 0, 0, 0) == -1


@pytest.mark.parametrize("N", [0, -1])
def test_q4k_rejects_bad_output_dim(lib, N):
    assert lib.q4k_gemv(GOOD, GOOD2, 256, N, GOOD3, None) == -1
    assert lib.q4k_matmul(GOOD, GOOD2, 2, 256, N, GOOD3, None) == -1


@pytest.mark.parametrize("M", [0, -3])
def test_q4k_matmul_rejects_bad_tokens(lib, M):
    assert lib.q4k_matmul(GOOD, GOOD2, M, 256, 8, GOOD3, None) == -1


def test_q4k_rejects_null_pointers(lib):
    assert lib.q4k_gemv(None, GOOD2, 256, 8, GOOD3, None) == -2
    assert lib.q4k_gemv(GOOD, None, 256, 8, GOOD3, None) == -2
    assert lib.q4k_gemv(GOOD, GOOD2, 256, 8, None, None) == -2
    assert lib.q4k_matmul(GOOD, None, 3, 256, 8, GOOD3, None) == -2


def test_q4k_rejects_misaligned(lib):
    assert lib.q4k_gemv(ODD, GOOD2, 256, 8, GOOD3, None) == -3
    assert lib.q4k_gemv(GOOD, ODD, 256, 8, GOOD3, None) == -3
    assert lib.q4k_matmul(GOOD, ODD, 3, 256, 8, GOOD3, None) == -3


def test_dimension_error_takes_precedence(lib):
    assert lib.q4k_gemv(None, ODD, 100, 8, None, None) == -1


@pytest.mark.parametrize("rpl,kw,wg", [(3, 0, 0), (16, 1, 0), (0, 3, 0), (1, 8, 0),
                                       (-1, 0, 0), (1, 1, 3), (1, 4, 2), (2, 2, 1),
                                       (1, 1, 16), (8, 1, 8), (1, 4, 8), (4, 0, 16),
                                       (0, 2, 16), (0, 0, 32)])
def test_shaped_rejects_bad_launch_shape(lib, rpl, kw, wg):
    assert lib.q4k_gemv_shaped(GOOD, GOOD2, 256, 8, GOOD3, None, rpl, kw, wg) == -1


@pytest.mark.parametrize("waves,rg,depth", [(3, 0, 0), (32, 0, 0), (2, 0, 0), (0, 5, 0),
                                             (0, -1, 0), (0, 0, 3), (0, 0, 1), (4, 0, 2),
                                             (16, 0, 4), (4, 1, 2), (-8, 0, 0)])
def test_walk_shaped_rejects_bad_shape(lib, waves, rg, depth):
    assert lib.q4k_gemv_walk_shaped(GOOD, GOOD2, 256, 8, GOOD3, None, waves, rg, depth) == -1


def test_walk_shaped_validates_like_gemv(lib):
    assert lib.q4k_gemv_walk_shaped(GOOD, GOOD2, 300, 8, GOOD3, None, 0, 0, 0) == -1
    assert lib.q4k_gemv_walk_shaped(None, GOOD2, 256, 8, GOOD3, None, 0, 0, 0) == -2
    assert lib.q4k_gemv_walk_shaped(GOOD, ODD, 256, 8, GOOD3, None, 0, 0, 0) == -3


@pytest.mark.parametrize("K", [32, 96, 288, 4000, 0, -256, 1 << 31, (1 << 24) + 256])
def test_q4_0_rejects_bad_input_dim(lib, K):
    """Multiples of 32 that are not whole 144-byte groups are rejected too."""
    assert lib.q4_0_gemv(GOOD, GOOD2, K, 16, GOOD3, None) == -1
    assert lib.q4_0_gemv_shaped(GOOD, GOOD2, K, 16, GOOD3, None, 0, 0, 0) == -1


def test_q4_0_rejects_null_misaligned_and_bad_shape(lib):
    assert lib.q4_0_gemv(GOOD, GOOD2, 256, 0, GOOD3, None) == -1
    assert lib.q4_0_gemv(None, GOOD2, 256, 8, GOOD3, None) == -2
    assert lib.q4_0_gemv(GOOD, None, 256, 8, GOOD3, None) == -2
    assert lib.q4_0_gemv(GOOD, GOOD2, 256, 8, None, None) == -2
    assert lib.q4_0_gemv(ODD, GOOD2, 256, 8, GOOD3, None) == -3
    assert lib.q4_0_gemv(GOOD, ODD, 256, 8, GOOD3, None) == -3
    for rpl, kw, wg in [(3, 0, 0), (1, 8, 0), (8, 1, 8), (1, 0, 16), (0, 1, 16), (0, 0, 32)]:
        assert lib.q4_0_gemv_shaped(GOOD, GOOD2, 256, 8, GOOD3, None, rpl, kw, wg) == -1
    # the matrix-core form takes rows of at most 256 groups of eight blocks
    assert lib.q4_0_gemv_shaped(GOOD, GOOD2, 257 * 256, 8, GOOD3, None, 0, 0, 16) == -1


@pytest.mark.parametrize("K", [32, 255, 257, 4000, 0, -256, 1 << 31, (1 << 24) + 256])
def test_q6k_rejects_bad_input_dim(lib, K):
    assert lib.q6k_gemv(GOOD, GOOD2, K, 16, GOOD3, None) == -1
    assert lib.q6k_gemv_shaped(GOOD, GOOD2, K, 16, GOOD3, None, 0, 0, 0) == -1


def test_q6k_rejects_null_misaligned_and_bad_shape(lib):
    assert lib.q6k_gemv(GOOD, GOOD2, 256, 0, GOOD3, None) == -1
    assert lib.q6k_gemv(None, GOOD2, 256, 8, GOOD3, None) == -2
    assert lib.q6k_gemv(GOOD, None, 256, 8, GOOD3, None) == -2
    assert lib.q6k_gemv(GOOD, GOOD2, 256, 8, None, None) == -2
    assert lib.q6k_gemv(ODD, GOOD2, 256, 8, GOOD3, None) == -3
    assert lib.q6k_gemv(GOOD, ODD, 256, 8, GOOD3, None) == -3
    for rpl, kw, wg in [(3, 0, 0), (1, 8, 0), (8, 1, 8), (0, 0, 16)]:
        assert lib.q6k_gemv_shaped(GOOD, GOOD2, 256, 8, GOOD3, None, rpl, kw, wg) == -1
    # 64 lanes (input_dim > 2048), 8 rows per lane, a 4-way split: LDS too small
    assert lib.q6k_gemv_shaped(GOOD, GOOD2, 4096, 8, GOOD3, None, 8, 4, 4) == -1


def test_ternary_matmul_shaped_rejects_bad_forms(lib):
    F = ctypes.c_float
    for form in (2, 8, 48, 128, -16):
        assert lib.ternary_matmul_shaped(GOOD, GOOD2, F(1.0), 16, 256, 8, GOOD3, None, form) == -1
    assert lib.ternary_matmul_shaped(GOOD, GOOD2, F(1.0), 16, 100, 8, GOOD3, None, 16) == -1
    assert lib.ternary_matmul_shaped(ODD, GOOD2, F(1.0), 16, 256, 8, GOOD3, None, 32) == -3
    assert lib.ternary_matmul_shaped(GOOD, GOOD2, F(1.0), 0, 256, 8, GOOD3, None, 16) == -1


def test_ternary_matmul_rejects_bad_args(lib):
    F = ctypes.c_float
    assert lib.ternary_matmul(GOOD, GOOD2, F(1.0), 0, 64, 8, GOOD3, None) == -1
    assert lib.ternary_matmul(GOOD, GOOD2, F(1.0), -2, 64, 8, GOOD3, None) == -1
    assert lib.ternary_matmul(GOOD, GOOD2, F(1.0), 3, 66, 8, GOOD3, None) == -1
    assert lib.ternary_matmul(GOOD, GOOD2, F(1.0), 3, 64, 0, GOOD3, None) == -1
    assert lib.ternary_matmul(None, GOOD2, F(1.0), 3, 64, 8, GOOD3, None) == -2
    assert lib.ternary_matmul(GOOD, None, F(1.0), 3, 64, 8, GOOD3, None) == -2
    assert lib.ternary_matmul(GOOD, GOOD2, F(1.0), 3, 64, 8, None, None) == -2


def test_matmul_shaped_rejects_bad_forms(lib):
    for form in (2, 8, 48, 137, -16):
        assert lib.q4k_matmul_shaped(GOOD, GOOD2, 16, 256, 64, GOOD3, None, form) == -1
    assert lib.q4k_matmul_shaped(GOOD, GOOD2, 9, 256, 64, GOOD3, None, 1) == -1  # > 8 tokens
    assert lib.q4k_matmul_tiled_shaped(GOOD, GOOD2, 9, 256, 64, GOOD3, None, 1) == -1
    assert lib.q4k_matmul_shaped(GOOD, GOOD2, 16, 255, 64, GOOD3, None, 16) == -1
    assert lib.q4k_matmul_shaped(None, GOOD2, 16, 256, 64, GOOD3, None, 16) == -2
    assert lib.q4k_matmul_shaped(ODD, GOOD2, 16, 256, 64, GOOD3, None, 16) == -3
    for form in (2, 8, 48, 65, 128, 131, -16):
        assert lib.q4k_matmul_tiled_shaped(GOOD, GOOD2, 16, 256, 64, GOOD3, None, form) == -1
    assert lib.q4k_matmul_tiled_shaped(GOOD, ODD, 16, 256, 64, GOOD3, None, 32) == -3


def test_tiled_size_is_host_only_arithmetic(lib):
    assert lib.q4k_tiled_size(4096, 4096) == 256 * 16 * 2304
    assert lib.q4k_tiled_size(256, 1) == 2304
    assert lib.q4k_tiled_size(512, 17) == 2 * 2 * 2304
    for K, N in ((255, 1), (0, 1), (256, 0), (-256, 4), ((1 << 24) + 256, 1)):
        assert lib.q4k_tiled_size(K, N) == -1


@pytest.mark.parametrize("K", [255, 257, 0, -256, (1 << 24) + 256])
def test_tiled_entry_points_reject_bad_input_dim(lib, K):
    assert lib.q4k_relayout_tiled(GOOD, K, 16, GOOD2, None) == -1
    assert lib.q4k_gemv_tiled(GOOD, GOOD2, K, 16, GOOD3, None) == -1
    assert lib.q4k_gemv_tiled_shaped(GOOD, GOOD2, K, 16, GOOD3, None, 0, 0, 0) == -1


def test_tiled_entry_points_reject_null_misaligned_and_bad_shape(lib):
    assert lib.q4k_relayout_tiled(GOOD, 256, 0, GOOD2, None) == -1
    assert lib.q4k_relayout_tiled(None, 256, 16, GOOD2, None) == -2
    assert lib.q4k_relayout_tiled(GOOD, 256, 16, None, None) == -2
    assert lib.q4k_relayout_tiled(ODD, 256, 16, GOOD2, None) == -3
    assert lib.q4k_relayout_tiled(GOOD, 256, 16, ODD, None) == -3
    assert lib.q4k_gemv_tiled(None, GOOD2, 256, 16, GOOD3, None) == -2
    assert lib.q4k_gemv_tiled(GOOD, None, 256, 16, GOOD3, None) == -2
    assert lib.q4k_gemv_tiled(GOOD, GOOD2, 256, 16, None, None) == -2
    assert lib.q4k_gemv_tiled(ODD, GOOD2, 256, 16, GOOD3, None) == -3
    assert lib.q4k_gemv_tiled(GOOD, ODD, 256, 16, GOOD3, None) == -3
    for M in (0, -1):
        assert lib.q4k_matmul_tiled(GOOD, GOOD2, M, 256, 16, GOOD3, None) == -1
    assert lib.q4k_matmul_tiled(GOOD, GOOD2, 4, 255, 16, GOOD3, None) == -1
    assert lib.q4k_matmul_tiled(None, GOOD2, 4, 256, 16, GOOD3, None) == -2
    assert lib.q4k_matmul_tiled(GOOD, GOOD2, 4, 256, 16, None, None) == -2
    assert lib.q4k_matmul_tiled(ODD, GOOD2, 4, 256, 16, GOOD3, None) == -3
    assert lib.q4k_matmul_tiled(GOOD, ODD, 4, 256, 16, GOOD3, None) == -3
    for waves, rg, depth in ((2, 0, 0), (32, 0, 0), (8, 5, 0), (8, -1, 0), (8, 0, 3),
                             (16, 0, 4), (8, 0, 1)):
        assert lib.q4k_gemv_tiled_shaped(GOOD, GOOD2, 4096, 16, GOOD3, None,
                                         waves, rg, depth) == -1, (waves, rg, depth)


@pytest.mark.parametrize("K", [3, 5, 4098, 0, -4])
def test_ternary_rejects_bad_input_dim(lib, K):
    assert lib.ternary_gemv_codes(GOOD, GOOD2, K, 8, GOOD3, None) == -1
    assert lib.ternary_gemv(GOOD, GOOD2, 1.0, K, 8, GOOD3, None) == -1


def test_ternary_rejects_null(lib):
    assert lib.ternary_gemv_codes(GOOD, None, 64, 8, GOOD3, None) == -2
    assert lib.ternary_gemv(None, GOOD2, 2.0, 64, 8, GOOD3, None) == -2


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, 7):
        s = lib.q4k_strerror(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert b"256" in lib.q4k_strerror(-1)


def test_binding_raises_value_error_on_bad_dim(lib):
    """The Python layer turns Q4K_EINVAL_DIM into ValueError, mirroring the
    page's IllegalArgumentException."""
    from q4_packed_weight_amd import binding
    rc = lib.q4k_gemv(GOOD, GOOD2, 300, 1, GOOD3, None)
    with pytest.raises(ValueError) as e:
        binding._check(rc, "q4k_gemv")
    assert e.value.code == binding.Q4K_EINVAL_DIM


def test_bench_helpers_validate(lib):
    assert lib.q4k_bench_stream_read(GOOD, 100, GOOD2, 4, None) == -1
    assert lib.q4k_bench_stream_read(ODD, 160, GOOD2, 4, None) == -3
    assert lib.q4k_bench_copy(GOOD, None, 160, None) == -2
    assert lib.q4k_bench_delay(-1, None) == -1
    assert lib.q4k_bench_delay(200000000, None) == -1


def test_matmul_noalloc_rejects_bad_arguments_before_launching(lib):
    """The no-allocation form validates like q4k_matmul, before any HIP call."""
    assert lib.q4k_matmul_noalloc(GOOD, GOOD2, 16, 255, 64, GOOD3, None) == -1
    assert lib.q4k_matmul_noalloc(GOOD, GOOD2, 0, 256, 64, GOOD3, None) == -1
    assert lib.q4k_matmul_noalloc(None, GOOD2, 16, 256, 64, GOOD3, None) == -2
    assert lib.q4k_matmul_noalloc(ODD, GOOD2, 16, 256, 64, GOOD3, None) == -3
    assert b"scratch" in lib.q4k_strerror(-5)
