"""Every path at the largest input_dim the C ABI accepts (2^24 activations:
9.4 MB Q4_K rows, a 64 MB activation vector), against the oracle, through
the C ABI.  These sizes put the kernels' buffer offsets at their largest
(up to about 2^30 bytes for 16 token rows of X), so they check the offset
arithmetic that small shapes never reach.  Parity bar as everywhere
(tests/tolerance.py); batched products are checked on sampled token rows.
"""
import numpy as np
import pytest
import torch

from q4_packed_weight_amd import binding, synth
from gpu_util import DEV, canary_intact, dev, host, out_with_canary
from tolerance import assert_parity

pytestmark = pytest.mark.gpu

KMAX = 1 << 24


@pytest.fixture(scope="module")
def x_max():
    return synth.activations(KMAX, config=60)


def gemv(fn, x, w, N, *extra):
    buf, y = out_with_canary(N)
    fn(dev(x), w if isinstance(w, torch.Tensor) else dev(w), KMAX, N, y, *extra)
    out = host(y)
    assert canary_intact(buf, N)
    return out


def test_q4k_gemv_max_input_dim(oracle_lib, x_max):
    N = 3
    w = synth.q4k_weights(N, KMAX, config=60)
    ref = oracle_lib.q4k_gemv(x_max, w, KMAX, N)
    assert_parity(gemv(binding.q4k_gemv, x_max, w, N), ref, what="vector form")
    assert_parity(gemv(binding.q4k_gemv_shaped, x_max, w, N, 0, 0, 16), ref, what="matrix-core form")
    # the walk q4k_gemv takes for such rows from output_dim 3072 on (one
    # workgroup here, 8192 units per wave)
    assert_parity(gemv(binding.q4k_gemv_walk_shaped, x_max, w, N, 0, 0, 0), ref, what="walk")


def test_q4k_gemv_tiled_max_input_dim(oracle_lib, x_max):
    N = 3
    w = synth.q4k_weights(N, KMAX, config=61)
    wt = torch.empty(binding.q4k_tiled_size(KMAX, N), dtype=torch.uint8, device=DEV)
    binding.q4k_relayout_tiled(dev(w), KMAX, N, wt)
    assert_parity(gemv(binding.q4k_gemv_tiled, x_max, wt, N), oracle_lib.q4k_gemv(x_max, w, KMAX, N))


def test_q4_0_and_q6k_gemv_max_input_dim(oracle_lib, x_max):
    N = 3
    w0 = synth.q4_0_weights(N, KMAX, config=62)
    assert_parity(gemv(binding.q4_0_gemv, x_max, w0, N), oracle_lib.q4_0_gemv(x_max, w0, KMAX, N),
                  what="Q4_0")
    w6 = synth.q6k_weights(N, KMAX, config=62)
    assert_parity(gemv(binding.q6k_gemv, x_max, w6, N), oracle_lib.q6k_gemv(x_max, w6, KMAX, N),
                  what="Q6_K")


def test_ternary_gemv_max_input_dim(oracle_lib, x_max):
    N = 3
    codes, _ = synth.ternary_codes(N, KMAX, copy=60)
    buf, y = out_with_canary(N)
    binding.ternary_gemv(dev(x_max), dev(codes), 1.5, KMAX, N, y)
    out = host(y)
    assert canary_intact(buf, N)
    assert_parity(out, oracle_lib.ternary_gemv(x_max, codes, 1.5, KMAX, N))


@pytest.mark.parametrize("M,form", [(3, 1), (17, 16), (17, 64)])
def test_q4k_matmul_max_input_dim(oracle_lib, M, form):
    """The batched kernel (form 1) and the prefill tiles at two heights;
    token rows 0 and M - 1 against the oracle."""
    N = 20
    w = synth.q4k_weights(N, KMAX, config=63)
    X = synth.activations(KMAX, n_tokens=M, config=63)
    buf, Y = out_with_canary(N, rows=M)
    binding.q4k_matmul_shaped(dev(X), dev(w), M, KMAX, N, Y, form)
    out = host(Y)
    assert canary_intact(buf, M * N)
    for t in (0, M - 1):
        ref = oracle_lib.q4k_matmul_part(X, w, M, KMAX, N, (t, t + 1), (0, N))[t]
        assert_parity(out[t], ref, what=f"form {form} token {t}")


def test_ternary_matmul_max_input_dim(oracle_lib):
    M, N = 17, 20
    codes, _ = synth.ternary_codes(N, KMAX, copy=64)
    X = synth.activations(KMAX, n_tokens=M, config=synth.C5_TERNARY, copy=64)
    buf, Y = out_with_canary(N, rows=M)
    binding.ternary_matmul_shaped(dev(X), dev(codes), 1.0, M, KMAX, N, Y, 16)
    out = host(Y)
    assert canary_intact(buf, M * N)
    for t in (0, M - 1):
        assert_parity(out[t], oracle_lib.ternary_gemv(X[t], codes, 1.0, KMAX, N), what=f"token {t}")


# Rows of more than 256 super-blocks take exact normal code operands in the
# matrix-core GEMV kernels (shorter rows keep the cheaper subnormal codes);
# 257 super-blocks is the first length on that side, checked in full.
K257 = 257 * 256


def test_normal_code_forms_just_past_the_threshold(oracle_lib):
    N, M = 40, 5
    w = synth.q4k_weights(N, K257, config=65)
    x = synth.activations(K257, config=65)
    X = synth.activations(K257, n_tokens=M, config=66)
    ref = oracle_lib.q4k_gemv(x, w, K257, N)
    refM = oracle_lib.q4k_matmul(X, w, M, K257, N)
    buf, y = out_with_canary(N)
    binding.q4k_gemv_shaped(dev(x), dev(w), K257, N, y, 0, 0, 16)
    assert_parity(host(y), ref, what="matrix-core GEMV")
    wt = torch.empty(binding.q4k_tiled_size(K257, N), dtype=torch.uint8, device=DEV)
    binding.q4k_relayout_tiled(dev(w), K257, N, wt)
    binding.q4k_gemv_tiled(dev(x), wt, K257, N, y)
    assert_parity(host(y), ref, what="tiled GEMV")
    assert canary_intact(buf, N)
    bufM, Y = out_with_canary(N, rows=M)
    binding.q4k_matmul_shaped(dev(X), dev(w), M, K257, N, Y, 1)
    assert_parity(host(Y), refM, rowwise=True, what="batched")
    binding.q4k_matmul_tiled_shaped(dev(X), wt, M, K257, N, Y, 1)
    assert_parity(host(Y), refM, rowwise=True, what="tiled batched")
    assert canary_intact(bufM, M * N)


def test_normal_code_forms_integer_bit_exact(oracle_lib):
    """Integer weights and activations past the threshold: exact."""
    N, M = 24, 3
    w = synth.q4k_integer_weights(N, K257, config=67)
    X = synth.integer_activations(K257, n_tokens=M, config=67)
    refM = oracle_lib.q4k_matmul(X, w, M, K257, N)
    buf, y = out_with_canary(N)
    binding.q4k_gemv_shaped(dev(X[0]), dev(w), K257, N, y, 0, 0, 16)
    assert np.array_equal(host(y).astype(np.float64), refM[0])
    bufM, Y = out_with_canary(N, rows=M)
    binding.q4k_matmul_shaped(dev(X), dev(w), M, K257, N, Y, 1)
    assert np.array_equal(host(Y).astype(np.float64), refM)
