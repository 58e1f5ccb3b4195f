"""The tiled block order on the GPU: the one-time relayout against the
oracle's (bit-exact byte moves), and the GEMV that streams it against the
oracle's product on the canonical matrix, through the C ABI.

SKaiNET docs, "Eager execution: backends and kernels": a packed weight
declares its block order and a canonical weight is relayouted into it once.
Parity bar for the product as for Q4_K (tests/tolerance.py); bit-exact where
every product and partial sum is exact.
"""
import numpy as np
import pytest
import torch

from q4_packed_weight_amd import binding, synth
from gpu_util import DEV, canary_intact, dev, host, out_with_canary
from tolerance import assert_parity

pytestmark = pytest.mark.gpu

PAD = 64  # canary bytes after the tiled buffer


def relayout(w, K, N):
    """GPU relayout of canonical bytes; returns (tiled view, full buffer)."""
    size = binding.q4k_tiled_size(K, N)
    buf = torch.full((size + PAD,), 0xA5, dtype=torch.uint8, device=DEV)
    binding.q4k_relayout_tiled(dev(w), K, N, buf[:size])
    return buf[:size], buf


def gemv_tiled(x, wt, K, N, shape=None):
    buf, y = out_with_canary(N)
    if shape is None:
        binding.q4k_gemv_tiled(dev(x), wt, K, N, y)
    else:
        binding.q4k_gemv_tiled_shaped(dev(x), wt, K, N, y, *shape)
    out = host(y)
    assert canary_intact(buf, N), "write past the end of y"
    return out


RELAYOUT_SHAPES = [(256, 1), (256, 15), (512, 17), (768, 33), (4096, 64), (2304, 129),
                   (4096, 4096), (1280, 1000)]


@pytest.mark.parametrize("K,N", RELAYOUT_SHAPES)
def test_relayout_bit_exact(oracle_lib, K, N):
    w = synth.q4k_weights(N, K, config=30, copy=K + N)
    wt, buf = relayout(w, K, N)
    got = host(buf)
    assert np.array_equal(got[:-PAD], oracle_lib.q4k_relayout_tiled(w, K, N))
    assert np.all(got[-PAD:] == 0xA5), "write past the end of the tiled buffer"


@pytest.mark.parametrize("K,N", [(4096, 14336), (14336, 4096)])
def test_relayout_full_ffn_matrices_bit_exact(oracle_lib, K, N):
    w = synth.q4k_weights(N, K, config=synth.C3_FFN, extra=int(K > N))
    wt, _ = relayout(w, K, N)
    assert np.array_equal(host(wt), oracle_lib.q4k_relayout_tiled(w, K, N))


# single block, ragged row groups (N % 16 != 0), chunked input_dim (more than
# 64 super-blocks: 20480 and 65536), every workgroup-count regime
SHAPES = [(256, 1), (512, 1), (256, 7), (4096, 64), (768, 37), (1280, 5), (2304, 129),
          (3840, 333), (4352, 1000), (14336, 100), (1024, 1024), (8192, 17), (256, 4097),
          (20480, 50), (16384, 48), (4096, 4096), (2560, 4090)]


@pytest.mark.parametrize("K,N", SHAPES)
def test_gemv_tiled_parity(oracle_lib, K, N):
    w = synth.q4k_weights(N, K, config=31, copy=K + N)
    x = synth.activations(K, config=31, copy=K + N)
    wt, _ = relayout(w, K, N)
    y = gemv_tiled(x, wt, K, N)
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what=f"K={K} N={N}")


@pytest.mark.parametrize("K,N,name", [(1024, 1024, "c1"), (4096, 4096, "c2"),
                                      (4096, 14336, "c3-up"), (14336, 4096, "c3-down")])
def test_gemv_tiled_parity_full_configs(oracle_lib, K, N, name):
    cfg = {"c1": synth.C1_Q4K_1K, "c2": synth.C2_Q4K_4K}.get(name, synth.C3_FFN)
    extra = 1 if name == "c3-down" else 0
    w = synth.q4k_weights(N, K, config=cfg, extra=extra)
    x = synth.activations(K, config=cfg, extra=extra)
    wt, _ = relayout(w, K, N)
    y = gemv_tiled(x, wt, K, N)
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what=name)


@pytest.mark.parametrize("waves,depth", [(4, 2), (4, 4), (8, 2), (8, 4), (16, 2)])
@pytest.mark.parametrize("rg", [1, 2, 3, 4])
@pytest.mark.parametrize("K,N", [(4096, 333), (14336, 67), (1024, 129), (256, 50),
                                 (20480, 40)])
def test_gemv_tiled_every_launch_shape(oracle_lib, K, N, waves, depth, rg):
    w = synth.q4k_weights(N, K, config=32, copy=K)
    x = synth.activations(K, config=32, copy=K)
    wt, _ = relayout(w, K, N)
    y = gemv_tiled(x, wt, K, N, shape=(waves, rg, depth))
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what=f"shape {waves},{rg},{depth}")


def test_gemv_tiled_reads_oracle_tiled_bytes(oracle_lib):
    """The product of bytes laid out by the oracle's relayout (not the
    GPU's) equals the product of the GPU's relayout bit for bit."""
    K, N = 4096, 300
    w = synth.q4k_weights(N, K, config=33)
    x = synth.activations(K, config=33)
    y_oracle_bytes = gemv_tiled(x, dev(oracle_lib.q4k_relayout_tiled(w, K, N)), K, N)
    wt, _ = relayout(w, K, N)
    assert np.array_equal(y_oracle_bytes.view(np.uint32), gemv_tiled(x, wt, K, N).view(np.uint32))
    assert_parity(y_oracle_bytes, oracle_lib.q4k_gemv(x, w, K, N))


@pytest.mark.parametrize("N", [4096, 333, 16])
def test_sixteen_waves_equal_canonical_matrix_core_form(N):
    """With 16 super-blocks per row and 16 waves, a wave of the tiled kernel
    does exactly what a wave of the canonical matrix-core form does, in the
    same order: the two forms agree bit for bit (the relayout changes where
    the bytes are read, not the arithmetic)."""
    K = 4096
    w = synth.q4k_weights(N, K, config=34, copy=N)
    x = synth.activations(K, config=34, copy=N)
    wt, _ = relayout(w, K, N)
    y_t = gemv_tiled(x, wt, K, N, shape=(16, 1, 2))
    buf, y = out_with_canary(N)
    binding.q4k_gemv_shaped(dev(x), dev(w), K, N, y, 0, 0, 16)
    assert np.array_equal(y_t.view(np.uint32), host(y).view(np.uint32))


@pytest.mark.parametrize("K,N", [(4096, 4096), (14336, 64), (768, 100), (20480, 33)])
def test_gemv_tiled_integer_bit_exact(oracle_lib, K, N):
    """d = dmin = 1 and small integer activations: every product and partial
    sum is an exact integer, so the GPU equals the oracle exactly."""
    w = synth.q4k_integer_weights(N, K, config=35)
    x = synth.integer_activations(K, config=35)
    wt, _ = relayout(w, K, N)
    y = gemv_tiled(x, wt, K, N)
    ref = oracle_lib.q4k_gemv(x, w, K, N)
    assert np.all(ref == np.round(ref))
    assert np.array_equal(y.astype(np.float64), ref)


def test_gemv_tiled_one_hot_bit_exact_all_positions(oracle_lib):
    """x = e_k: y[o] is the oracle's fp32 weight W[o,k], for every k of a
    block and 17 rows (two row groups, the second padded)."""
    K, N = 256, 17
    w = synth.q4k_weights(N, K, config=36)
    wt, _ = relayout(w, K, N)
    buf, y = out_with_canary(N)
    X = np.eye(K, dtype=np.float32)
    for k in range(K):
        binding.q4k_gemv_tiled(dev(X[k]), wt, K, N, y)
        got = host(y)
        ref = oracle_lib.q4k_gemv(X[k], w, K, N).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), k
    assert canary_intact(buf, N)


@pytest.mark.parametrize("K,N,lo,hi", [(4096, 4096, -40, 40), (2560, 300, -40, 40),
                                       (4096, 256, -60, 92), (14336, 200, -60, 92)])
def test_gemv_tiled_wide_range_activations(oracle_lib, K, N, lo, hi):
    """Sub-blocks at scales 2^lo .. 2^hi and some all zero (each 32-element
    sub-block is rescaled by a power of two before its fp16 split)."""
    w = synth.q4k_weights(N, K, config=37, copy=K + N)
    x = synth.activations(K, config=37, copy=K + N)
    g = np.random.default_rng(37)
    scale = np.exp2(g.integers(lo, hi + 1, K // 32)).astype(np.float32)
    scale[g.choice(K // 32, 3, replace=False)] = 0.0
    x = (x.reshape(-1, 32) * scale[:, None]).reshape(-1)
    wt, _ = relayout(w, K, N)
    assert_parity(gemv_tiled(x, wt, K, N), oracle_lib.q4k_gemv(x, w, K, N), what="wide range")


def test_gemv_tiled_zero_activation_and_determinism():
    K, N = 4096, 1024
    w = synth.q4k_weights(N, K, config=38)
    wt, _ = relayout(w, K, N)
    assert np.all(gemv_tiled(np.zeros(K, np.float32), wt, K, N) == 0.0)
    x = synth.activations(K, config=38)
    a, b = gemv_tiled(x, wt, K, N), gemv_tiled(x, wt, K, N)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_gemv_tiled_many_rows_sampled(oracle_lib):
    """2^20 rows of one block (151 MB tiled): sampled rows against the
    oracle run on just those rows."""
    K, N = 256, 1 << 20
    w = synth.q4k_weights(N, K, config=39)
    x = synth.activations(K, config=39)
    wt, _ = relayout(w, K, N)
    y = gemv_tiled(x, wt, K, N)
    rows = np.concatenate([np.random.default_rng(39).choice(N, 2000, replace=False), [0, N - 1]])
    assert_parity(y[rows], oracle_lib.q4k_gemv(x, w[rows], K, len(rows)), what="sampled rows")


def test_gemv_tiled_long_rows(oracle_lib):
    K, N = 65536, 40
    w = synth.q4k_weights(N, K, config=40)
    x = synth.activations(K, config=40)
    wt, _ = relayout(w, K, N)
    assert_parity(gemv_tiled(x, wt, K, N), oracle_lib.q4k_gemv(x, w, K, N), what="K=65536")


def test_tiled_rejects_bad_args_and_leaves_outputs_untouched():
    x = torch.zeros(4096, dtype=torch.float32, device=DEV)
    wt = torch.zeros(2304 * 16, dtype=torch.uint8, device=DEV)
    buf, y = out_with_canary(8)
    for K in (255, 257, 4000):
        with pytest.raises(ValueError):
            binding.q4k_gemv_tiled(x, wt, K, 8, y)
    with pytest.raises(ValueError):
        binding.q4k_gemv_tiled(x, wt[4:], 256, 8, y)
    with pytest.raises(ValueError):
        binding.q4k_gemv_tiled_shaped(x, wt, 256, 8, y, 8, 5, 0)
    assert bool(torch.all(torch.isnan(buf)))
    w = torch.zeros(144 * 16, dtype=torch.uint8, device=DEV)
    out = torch.full((2304 + 16,), 0xA5, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        binding.q4k_relayout_tiled(w, 255, 16, out)
    with pytest.raises(ValueError):
        binding.q4k_relayout_tiled(w, 256, 16, out[4:])
    with pytest.raises(ValueError):
        binding.q4k_relayout_tiled(w[8:], 256, 8, out)
    assert np.all(host(out) == 0xA5)


# --- batched and prefill products on tiled weights (q4k_matmul_tiled) ------

def matmul_tiled(X, wt, M, K, N):
    buf, Y = out_with_canary(N, rows=M)
    binding.q4k_matmul_tiled(dev(X), wt, M, K, N, Y)
    out = host(Y)
    assert canary_intact(buf, M * N), "write past the end of Y"
    return out


def matmul_tiled_form(X, wt, M, K, N, form):
    buf, Y = out_with_canary(N, rows=M)
    binding.q4k_matmul_tiled_shaped(dev(X), wt, M, K, N, Y, form)
    out = host(Y)
    assert canary_intact(buf, M * N), "write past the end of Y"
    return out


def matmul_canonical(X, w, M, K, N, form=0):
    buf, Y = out_with_canary(N, rows=M)
    binding.q4k_matmul_shaped(dev(X), dev(w), M, K, N, Y, form)
    return host(Y)


# few tokens take the batched kernel (2 .. 4 at input_dim 1024), more the
# prefill tiles (5 .. 130: ragged token tiles)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 9, 16, 17, 63, 64, 65, 130])
def test_matmul_tiled_token_counts(oracle_lib, M):
    K, N = 1024, 200
    w = synth.q4k_weights(N, K, config=41, copy=M)
    X = synth.activations(K, n_tokens=M, config=41, copy=M)
    wt, _ = relayout(w, K, N)
    Y = matmul_tiled(X, wt, M, K, N)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what=f"M={M}")


# ragged stages (input_dim/256 not a multiple of 4), ragged row groups and
# row-group quartets, long rows, the batched kernel at several N regimes
# (5 to 8 tokens with input_dim >= 4096 and up to 4 at any shape)
@pytest.mark.parametrize("M,K,N", [(64, 256, 16), (64, 4096, 64), (5, 14336, 33), (64, 768, 1000),
                                   (48, 2304, 129), (64, 512, 4097), (16, 256, 64), (17, 768, 65),
                                   (33, 1280, 130), (8, 256, 1), (4, 512, 17), (6, 1280, 129),
                                   (8, 14336, 64), (2, 4096, 12000), (3, 20480, 40), (7, 4096, 8000),
                                   (4, 4096, 14336)])
def test_matmul_tiled_shapes(oracle_lib, M, K, N):
    w = synth.q4k_weights(N, K, config=42, copy=K + N)
    X = synth.activations(K, n_tokens=M, config=42, copy=K + N)
    wt, _ = relayout(w, K, N)
    Y = matmul_tiled(X, wt, M, K, N)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what=f"{M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(64, 4096, 512), (17, 768, 65), (33, 1280, 130), (16, 14336, 64),
                                   (40, 8448, 130), (64, 8192, 64)])
def test_prefill_tiled_equals_canonical_prefill(M, K, N):
    """The tiled prefill does the canonical 64-row prefill's arithmetic in
    the same order (only where the weight bytes come from differs): bit for
    bit.  From input_dim 8192 on the 64-row tiles are staged through LDS
    (33 super-blocks: a ragged last stage), below it loaded into registers."""
    w = synth.q4k_weights(N, K, config=43, copy=M)
    X = synth.activations(K, n_tokens=M, config=43, copy=M)
    wt, _ = relayout(w, K, N)
    a = matmul_tiled_form(X, wt, M, K, N, 64)
    b = matmul_canonical(X, w, M, K, N, form=64)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("rows", [16, 32, 64])
@pytest.mark.parametrize("M,K,N", [(16, 256, 16), (17, 768, 65), (33, 1280, 130), (2, 1024, 100),
                                   (9, 14336, 40), (16, 512, 4097)])
def test_prefill_tiled_every_height_equals_canonical(M, K, N, rows):
    """At every workgroup height the tiled prefill does the canonical
    prefill's arithmetic in the same order: bit for bit (and both pass the
    oracle's bar in tests/test_matmul_gpu.py)."""
    w = synth.q4k_weights(N, K, config=51, copy=K + N)
    X = synth.activations(K, n_tokens=M, config=51, copy=K + N)
    wt, _ = relayout(w, K, N)
    a = matmul_tiled_form(X, wt, M, K, N, rows)
    b = matmul_canonical(X, w, M, K, N, form=rows)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("rows,M,K,N", [(64, 20, 8448, 70), (64, 64, 16384, 33)])
def test_prefill_tiled_staged_64_rows_parity(oracle_lib, rows, M, K, N):
    """The 64-row tiles staged through LDS (input_dim >= 8192) against the
    oracle: ragged rows, tokens and stages."""
    w = synth.q4k_weights(N, K, config=54, copy=M)
    X = synth.activations(K, n_tokens=M, config=54, copy=M)
    wt, _ = relayout(w, K, N)
    assert_parity(matmul_tiled_form(X, wt, M, K, N, rows), oracle_lib.q4k_matmul(X, w, M, K, N),
                  rowwise=True, what=f"{M}x{K}x{N} rows {rows}")


@pytest.mark.parametrize("rows", [16, 32])
def test_prefill_tiled_narrow_parity(oracle_lib, rows):
    M, K, N = 24, 4096, 300
    w = synth.q4k_weights(N, K, config=52)
    X = synth.activations(K, n_tokens=M, config=52)
    wt, _ = relayout(w, K, N)
    assert_parity(matmul_tiled_form(X, wt, M, K, N, rows), oracle_lib.q4k_matmul(X, w, M, K, N),
                  rowwise=True, what=f"rows {rows}")


@pytest.mark.parametrize("M", [2, 3, 4, 5, 8])
def test_batch_tiled_equals_canonical_batch_one_block_per_wave(M):
    """With 8 super-blocks per row each of the 8 waves owns one super-block
    in both batched forms: the tiled one equals the canonical one bit for
    bit."""
    K, N = 2048, 300
    w = synth.q4k_weights(N, K, config=44, copy=M)
    X = synth.activations(K, n_tokens=M, config=44, copy=M)
    wt, _ = relayout(w, K, N)
    a = matmul_tiled_form(X, wt, M, K, N, 1)
    b = matmul_canonical(X, w, M, K, N, form=1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_matmul_tiled_full_config_sampled_tokens(oracle_lib):
    """64 x 4096 x 4096: every output of 8 sampled token rows."""
    M, K, N = 64, 4096, 4096
    w = synth.q4k_weights(N, K, config=synth.C4_PREFILL)
    X = synth.activations(K, n_tokens=M, config=synth.C4_PREFILL)
    wt, _ = relayout(w, K, N)
    Y = matmul_tiled(X, wt, M, K, N)
    for t in (0, 7, 21, 33, 40, 52, 62, 63):
        ref = oracle_lib.q4k_matmul_part(X, w, M, K, N, (t, t + 1), (0, N))[t]
        assert_parity(Y[t], ref, what=f"token {t}")


def test_batch_tiled_full_size(oracle_lib):
    M, K, N = 8, 4096, 4096
    w = synth.q4k_weights(N, K, config=synth.C2_Q4K_4K)
    X = synth.activations(K, n_tokens=M, config=synth.C2_Q4K_4K)
    wt, _ = relayout(w, K, N)
    assert_parity(matmul_tiled(X, wt, M, K, N), oracle_lib.q4k_matmul(X, w, M, K, N),
                  rowwise=True, what="8x4096x4096")


@pytest.mark.parametrize("M", [2, 8, 13, 64])
def test_matmul_tiled_integer_bit_exact(oracle_lib, M):
    K, N = 4096, 256
    w = synth.q4k_integer_weights(N, K, config=45)
    X = synth.integer_activations(K, n_tokens=M, config=45)
    wt, _ = relayout(w, K, N)
    Y = matmul_tiled(X, wt, M, K, N)
    assert np.array_equal(Y.astype(np.float64), oracle_lib.q4k_matmul(X, w, M, K, N))


def test_batch_tiled_wide_range_tokens(oracle_lib):
    """Tokens at 2^-30 .. 2^60 (one all zero), sub-blocks at 2^-20 .. 2^20:
    each token's super-block is rescaled before its fp16 split (the
    batched kernel, forced)."""
    M, K, N = 8, 2048, 200
    w = synth.q4k_weights(N, K, config=46)
    X = synth.activations(K, n_tokens=M, config=46)
    g = np.random.default_rng(46)
    sub = np.exp2(g.integers(-20, 21, (M, K // 32))).astype(np.float32)
    tok = np.exp2(np.array([-30, 0, 10, 30, 50, 60, -10, 0], np.float64)).astype(np.float32)
    X = (X.reshape(M, -1, 32) * sub[:, :, None] * tok[:, None, None]).reshape(M, K)
    X[6] = 0.0
    wt, _ = relayout(w, K, N)
    Y = matmul_tiled_form(X, wt, M, K, N, 1)
    assert np.all(Y[6] == 0.0)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what="wide-range tokens")


def test_matmul_tiled_deterministic_and_rejects():
    M, K, N = 64, 1024, 256
    w = synth.q4k_weights(N, K, config=47)
    X = synth.activations(K, n_tokens=M, config=47)
    wt, _ = relayout(w, K, N)
    a, b = matmul_tiled(X, wt, M, K, N), matmul_tiled(X, wt, M, K, N)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    buf, Y = out_with_canary(N, rows=M)
    for bad_k in (255, 1000):
        with pytest.raises(ValueError):
            binding.q4k_matmul_tiled(dev(X), wt, M, bad_k, N, Y)
    assert bool(torch.all(torch.isnan(buf)))


@pytest.mark.parametrize("rows,K", [(16, 2048), (32, 2048), (64, 2048), (64, 8448)])
def test_prefill_tiled_wide_range(oracle_lib, rows, K):
    """The prefill tiles on tiled weights (64 rows below input_dim 8192 load
    tiles into registers, the rest stage them through LDS) with sub-blocks
    from 2^-40 to 2^40, zero sub-blocks, and whole token rows at 1e-5, 3e5,
    2^-60 and 2^60: each token's super-block is scaled by a power of two
    before its fp16 split."""
    M, N = 40, 130
    w = synth.q4k_weights(N, K, config=57, copy=rows)
    X = synth.activations(K, n_tokens=M, config=57, copy=rows)
    g = np.random.default_rng(57 + rows)
    sub = np.exp2(g.integers(-40, 41, (M, K // 32))).astype(np.float32)
    sub[g.random((M, K // 32)) < 0.1] = 0.0
    X = (X.reshape(M, -1, 32) * sub[:, :, None]).reshape(M, K)
    X[:8] = synth.activations(K, n_tokens=8, config=58) * np.float32(
        [1e-5, 1e-5, 3e5, 3e5, 2.0 ** -60, 2.0 ** -60, 2.0 ** 60, 2.0 ** 60])[:, None]
    wt, _ = relayout(w, K, N)
    Y = matmul_tiled_form(X, wt, M, K, N, rows)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True,
                  what=f"{M}x{K}x{N} rows {rows}")
