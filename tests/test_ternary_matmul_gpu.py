"""Batched ternary product on the GPU against the CPU oracle (the ternary
page's prefill row loop), through the C ABI.  Parity bar as for Q4_K
(tests/tolerance.py), per token row; bit-exact on integer activations.
"""
import numpy as np
import pytest
import torch

from q4_packed_weight_amd import binding, synth
from gpu_util import DEV, dev, host, out_with_canary, canary_intact
from tolerance import assert_parity

pytestmark = pytest.mark.gpu


def run(X, codes, scale, M, K, N, x_offset=0):
    if x_offset:
        buf = torch.zeros(M * K + x_offset, dtype=torch.float32, device=DEV)
        buf[x_offset:] = torch.from_numpy(np.ascontiguousarray(X).reshape(-1)).to(DEV)
        Xd = buf[x_offset:]
    else:
        Xd = dev(X)
    ybuf, Y = out_with_canary(N, rows=M)
    binding.ternary_matmul(Xd, dev(codes), scale, M, K, N, Y)
    out = host(Y)
    assert canary_intact(ybuf, M * N), "write past the end of Y"
    return out


# token tiles (3..100, ragged), stages (input_dim 64 .. 14336, ragged last
# stage when input_dim % 1024 != 0), row tiles (ragged N); 2 tokens (and 3
# with input_dim > 8192) take the row loop
SHAPES = [(2, 64, 1), (3, 64, 5), (3, 1024, 64), (16, 4096, 64), (17, 1088, 130),
          (5, 11008, 300), (4, 11008, 40), (33, 2048, 1000), (64, 4096, 4096),
          (64, 14336, 128), (8, 256, 4097), (100, 512, 70)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_ternary_matmul_parity(oracle_lib, M, K, N):
    codes, _ = synth.ternary_codes(N, K, copy=M + K + N)
    X = synth.activations(K, n_tokens=M, config=synth.C5_TERNARY, copy=M + K + N)
    scale = synth.ternary_scale(copy=M)
    Y = run(X, codes, scale, M, K, N)
    assert_parity(Y, oracle_lib.ternary_matmul(X, codes, scale, M, K, N), rowwise=True,
                  what=f"M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N,off", [(4, 100, 33, 0), (6, 36, 7, 0), (5, 1024, 64, 1), (3, 4096, 100, 3)])
def test_ternary_matmul_row_loop_fallback(oracle_lib, M, K, N, off):
    """input_dim not a multiple of 64, or X not 16-byte aligned: one
    ternary_gemv launch per token row."""
    codes, _ = synth.ternary_codes(N, K, copy=7)
    X = synth.activations(K, n_tokens=M, config=synth.C5_TERNARY, copy=7)
    Y = run(X, codes, 0.75, M, K, N, x_offset=off)
    assert_parity(Y, oracle_lib.ternary_matmul(X, codes, 0.75, M, K, N), rowwise=True)


@pytest.mark.parametrize("M,K,N", [(16, 4096, 256), (37, 1088, 70), (64, 14336, 64)])
def test_ternary_matmul_integer_bit_exact(oracle_lib, M, K, N):
    """Integer activations in [-8, 8] and all four field values (3 decodes
    to +2): every product and partial sum is an exact fp32 integer, so the
    GPU equals the oracle bit for bit (scale 1)."""
    codes, _ = synth.ternary_codes(N, K, copy=11, allow_code3=True)
    X = synth.integer_activations(K, lo=-8, hi=8, n_tokens=M, config=synth.C5_TERNARY, copy=11)
    Y = run(X, codes, 1.0, M, K, N)
    ref = oracle_lib.ternary_matmul(X, codes, 1.0, M, K, N)
    assert np.all(ref == np.round(ref))
    assert np.array_equal(Y.astype(np.float64), ref)


def test_ternary_matmul_one_token_is_gemv():
    K, N = 4096, 512
    codes, _ = synth.ternary_codes(N, K, copy=12)
    x = synth.activations(K, config=synth.C5_TERNARY, copy=12)
    Y = run(x.reshape(1, K), codes, 1.5, 1, K, N)
    y = torch.empty(N, dtype=torch.float32, device=DEV)
    binding.ternary_gemv(dev(x), dev(codes), 1.5, K, N, y)
    assert np.array_equal(Y[0].view(np.uint32), host(y).view(np.uint32))


def test_ternary_matmul_wide_range_activations(oracle_lib):
    """Token rows at magnitudes 2^-30 .. 2^40 (far outside fp16), the
    256-position blocks of a row a further 2^-10 .. 2^10 apart, and a zero
    row: each block is rescaled before its fp16 split, so every row stays
    within the bar."""
    M, K, N = 16, 2048, 300
    codes, _ = synth.ternary_codes(N, K, copy=13)
    X = synth.activations(K, n_tokens=M, config=synth.C5_TERNARY, copy=13)
    X *= np.exp2(np.linspace(-30, 40, M)).astype(np.float32)[:, None]
    g = np.random.default_rng(13)
    blk = np.exp2(g.integers(-10, 11, (M, K // 256))).astype(np.float32)
    X = (X.reshape(M, K // 256, 256) * blk[:, :, None]).reshape(M, K)
    X[5] = 0.0
    Y = run(X, codes, 1.0, M, K, N)
    ref = oracle_lib.ternary_matmul(X, codes, 1.0, M, K, N)
    assert np.all(Y[5] == 0.0)
    assert_parity(np.delete(Y, 5, 0), np.delete(ref, 5, 0), rowwise=True)


def test_ternary_matmul_deterministic():
    M, K, N = 64, 4096, 1024
    codes, _ = synth.ternary_codes(N, K, copy=14)
    X = synth.activations(K, n_tokens=M, config=synth.C5_TERNARY, copy=14)
    a = run(X, codes, 1.0, M, K, N)
    b = run(X, codes, 1.0, M, K, N)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("M,K", [(0, 64), (-1, 64), (4, 66), (4, 0)])
def test_ternary_matmul_rejects_bad_dims(M, K):
    Xd = dev(np.zeros(max(M, 1) * max(K, 1), np.float32))
    cd = dev(np.zeros(64, np.uint8))
    ybuf, Y = out_with_canary(4, rows=max(M, 1))
    with pytest.raises(ValueError) as e:
        binding.ternary_matmul(Xd, cd, 1.0, M, K, 4, Y)
    assert getattr(e.value, "code", binding.Q4K_EINVAL_DIM) == binding.Q4K_EINVAL_DIM
    assert np.all(np.isnan(host(ybuf)))


# --- the matrix-core tiles at every workgroup height (ternary_matmul_shaped) --

def run_form(X, codes, scale, M, K, N, form):
    ybuf, Y = out_with_canary(N, rows=M)
    binding.ternary_matmul_shaped(dev(X), dev(codes), scale, M, K, N, Y, form)
    out = host(Y)
    assert canary_intact(ybuf, M * N), "write past the end of Y"
    return out


@pytest.mark.parametrize("rows", [16, 32, 64])
@pytest.mark.parametrize("M,K,N", [(3, 64, 5), (16, 4096, 64), (17, 1088, 130), (33, 2048, 100),
                                   (2, 14336, 40), (9, 256, 4097)])
def test_ternary_matmul_every_height(oracle_lib, M, K, N, rows):
    """Ragged rows, token tiles and stages; 16 rows splits each block's
    steps between two waves."""
    codes, _ = synth.ternary_codes(N, K, copy=M + K + rows)
    X = synth.activations(K, n_tokens=M, config=synth.C5_TERNARY, copy=M + K + rows)
    Y = run_form(X, codes, 0.8, M, K, N, rows)
    assert_parity(Y, oracle_lib.ternary_matmul(X, codes, 0.8, M, K, N), rowwise=True,
                  what=f"M={M} K={K} N={N} rows {rows}")


@pytest.mark.parametrize("rows", [16, 32, 64])
def test_ternary_matmul_every_height_integer_bit_exact(oracle_lib, rows):
    M, K, N = 24, 4096, 96
    codes, _ = synth.ternary_codes(N, K, copy=15, allow_code3=True)
    X = synth.integer_activations(K, lo=-8, hi=8, n_tokens=M, config=synth.C5_TERNARY, copy=15)
    Y = run_form(X, codes, 1.0, M, K, N, rows)
    assert np.array_equal(Y.astype(np.float64), oracle_lib.ternary_matmul(X, codes, 1.0, M, K, N))


def test_ternary_matmul_forced_row_loop(oracle_lib):
    M, K, N = 20, 1024, 70
    codes, _ = synth.ternary_codes(N, K, copy=16)
    X = synth.activations(K, n_tokens=M, config=synth.C5_TERNARY, copy=16)
    Y = run_form(X, codes, 1.25, M, K, N, 1)
    assert_parity(Y, oracle_lib.ternary_matmul(X, codes, 1.25, M, K, N), rowwise=True)


@pytest.mark.parametrize("rows", [16, 32])
def test_ternary_matmul_narrow_wide_range(oracle_lib, rows):
    """Per-(token, block) scaling at the narrow heights (shared exponent
    table, two waves per block at 16 rows)."""
    M, K, N = 16, 2048, 300
    codes, _ = synth.ternary_codes(N, K, copy=17)
    X = synth.activations(K, n_tokens=M, config=synth.C5_TERNARY, copy=17)
    X *= np.exp2(np.linspace(-30, 40, M)).astype(np.float32)[:, None]
    Y = run_form(X, codes, 1.0, M, K, N, rows)
    assert_parity(Y, oracle_lib.ternary_matmul(X, codes, 1.0, M, K, N), rowwise=True)

