"""Batched (prefill) Q4_K product on the GPU against the CPU oracle."""
import numpy as np
import pytest
import torch

from q4_packed_weight_amd import binding, synth
from gpu_util import DEV, canary_intact, dev, host, out_with_canary
from tolerance import assert_parity

pytestmark = pytest.mark.gpu


def run(X, w, M, K, N):
    buf, Y = out_with_canary(N, rows=M)
    binding.q4k_matmul(dev(X), dev(w), M, K, N, Y)
    out = host(Y)
    assert canary_intact(buf, M * N)
    return out


@pytest.mark.parametrize("M", [1, 2, 3, 17, 63, 64, 65, 130])
def test_matmul_parity_token_counts(oracle_lib, M):
    K, N = 1024, 200
    w = synth.q4k_weights(N, K, config=30, copy=M)
    X = synth.activations(K, n_tokens=M, config=30, copy=M)
    Y = run(X, w, M, K, N)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what=f"M={M}")


@pytest.mark.parametrize("M,K,N", [(64, 256, 16), (64, 4096, 64), (5, 14336, 33),
                                   (64, 768, 1000), (48, 2304, 129), (64, 512, 4097)])
def test_matmul_parity_shapes(oracle_lib, M, K, N):
    w = synth.q4k_weights(N, K, config=31, copy=K + N)
    X = synth.activations(K, n_tokens=M, config=31, copy=K + N)
    Y = run(X, w, M, K, N)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what=f"{M}x{K}x{N}")


def test_matmul_full_config_all_tokens(oracle_lib):
    """64 x 4096 x 4096 (the prefill workload): every output of every token
    row."""
    M, K, N = 64, 4096, 4096
    w = synth.q4k_weights(N, K, config=synth.C4_PREFILL)
    X = synth.activations(K, n_tokens=M, config=synth.C4_PREFILL)
    Y = run(X, w, M, K, N)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what="64x4096x4096")


def test_matmul_rows_match_gemv_on_integer_inputs(oracle_lib):
    """Integer-exact inputs: every token row equals the oracle bit for bit."""
    M, K, N = 64, 4096, 256
    w = synth.q4k_integer_weights(N, K, config=32)
    X = synth.integer_activations(K, n_tokens=M, config=32)
    Y = run(X, w, M, K, N)
    ref = oracle_lib.q4k_matmul(X, w, M, K, N)
    assert np.array_equal(Y.astype(np.float64), ref)


def test_matmul_deterministic():
    """Every output has one writer: repeated calls agree bit for bit."""
    M, K, N = 64, 4096, 512
    w = dev(synth.q4k_weights(N, K, config=34))
    X = dev(synth.activations(K, n_tokens=M, config=34))
    Y = torch.empty(M, N, dtype=torch.float32, device=DEV)
    outs = []
    for _ in range(3):
        binding.q4k_matmul(X, w, M, K, N, Y)
        outs.append(host(Y).copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("M,K,N", [(16, 256, 64), (17, 768, 65), (33, 1280, 130)])
def test_matmul_ragged_stage_and_tile_edges(oracle_lib, M, K, N):
    """input_dim not a multiple of the 4-block stage, and partial row and
    token tiles."""
    w = synth.q4k_weights(N, K, config=35, copy=K + N)
    X = synth.activations(K, n_tokens=M, config=35, copy=K + N)
    Y = run(X, w, M, K, N)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what=f"{M}x{K}x{N}")


def test_matmul_zero_activation():
    M, K, N = 64, 1024, 256
    w = synth.q4k_weights(N, K, config=33)
    Y = run(np.zeros((M, K), np.float32), w, M, K, N)
    assert np.all(Y == 0.0)


def test_matmul_rejects_bad_input_dim():
    X = torch.zeros(4, 300, dtype=torch.float32, device=DEV)
    w = torch.zeros(144 * 8, dtype=torch.uint8, device=DEV)
    buf, Y = out_with_canary(8, rows=4)
    with pytest.raises(ValueError):
        binding.q4k_matmul(X, w, 4, 300, 8, Y)
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(buf)))


# ---- a few tokens: the batched matrix-core GEMV (forced with form 1; the
#      automatic choice is checked by the token-count tests)

def run_batch(X, w, M, K, N):
    buf, Y = out_with_canary(N, rows=M)
    binding.q4k_matmul_shaped(dev(X), dev(w), M, K, N, Y, 1)
    out = host(Y)
    assert canary_intact(buf, M * N)
    return out


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 7, 8])
def test_batch_token_counts(oracle_lib, M):
    """Every token count of the batched form (2, 4 and 8-token kernels with
    tokens past M zero)."""
    K, N = 4096, 300
    w = synth.q4k_weights(N, K, config=36, copy=M)
    X = synth.activations(K, n_tokens=M, config=36, copy=M)
    Y = run_batch(X, w, M, K, N)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what=f"M={M}")


@pytest.mark.parametrize("M", [2, 3, 4, 5, 7, 8, 9, 12, 15, 16, 17, 24, 32, 33])
def test_automatic_choice_token_counts(oracle_lib, M):
    """The automatic choice around the hand-overs between the batched form,
    the prefill tiles and the split tiles (output_dim above 4096 and
    input_dim from 8192 move the last hand-over)."""
    for K, N in ((4096, 300), (14336, 64), (2048, 4200), (8192, 130)):
        w = synth.q4k_weights(N, K, config=53, copy=M)
        X = synth.activations(K, n_tokens=M, config=53, copy=M)
        Y = run(X, w, M, K, N)
        assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what=f"{M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(8, 256, 1), (4, 512, 17), (6, 1280, 129), (8, 14336, 64),
                                   (3, 768, 4097), (8, 2304, 1000), (2, 65536, 40), (7, 1792, 16),
                                   (2, 1024, 14341), (4, 4352, 100), (2, 8448, 33),
                                   (3, 66048, 20)])
def test_batch_shapes(oracle_lib, M, K, N):
    """One super-block (7 of 8 waves without work), ragged super-block counts
    per wave, ragged row tiles, long rows; 16-wave workgroups (up to 4
    tokens, at most 256 workgroups, 16+ super-blocks a row) with 17, 33 and
    258 super-blocks, the last with exact normal code operands."""
    w = synth.q4k_weights(N, K, config=37, copy=K + N)
    X = synth.activations(K, n_tokens=M, config=37, copy=K + N)
    Y = run_batch(X, w, M, K, N)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what=f"{M}x{K}x{N}")


@pytest.mark.parametrize("M", [2, 4, 8])
def test_batch_full_size(oracle_lib, M):
    """M tokens x 4096 -> 4096, every output (16-wave workgroups for 2 and
    4 tokens, 8 waves for 8)."""
    K, N = 4096, 4096
    w = synth.q4k_weights(N, K, config=synth.C2_Q4K_4K)
    X = synth.activations(K, n_tokens=M, config=synth.C2_Q4K_4K)
    Y = run_batch(X, w, M, K, N)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what=f"{M}x4096x4096")


@pytest.mark.parametrize("M", [2, 5, 8])
def test_batch_integer_bit_exact(oracle_lib, M):
    """d = dmin = 1, x in {-1, 0, 1}: every partial sum is an exact integer,
    so the batched form equals the oracle bit for bit."""
    K, N = 4096, 256
    w = synth.q4k_integer_weights(N, K, config=38)
    X = synth.integer_activations(K, n_tokens=M, config=38)
    Y = run_batch(X, w, M, K, N)
    assert np.array_equal(Y.astype(np.float64), oracle_lib.q4k_matmul(X, w, M, K, N))


def test_batch_wide_range_tokens(oracle_lib):
    """Tokens at very different scales (2^-30 .. 2^60, one all zero), and
    sub-blocks within a token at scales 2^-20 .. 2^20: each token's
    activations are rescaled per super-block before their fp16 split."""
    M, K, N = 8, 2048, 200
    w = synth.q4k_weights(N, K, config=39)
    X = synth.activations(K, n_tokens=M, config=39)
    g = np.random.default_rng(39)
    sub = np.exp2(g.integers(-20, 21, (M, K // 32))).astype(np.float32)
    tok = np.exp2(np.array([-30, 0, 10, 30, 50, 60, -10, 0], np.float64)).astype(np.float32)
    X = (X.reshape(M, -1, 32) * sub[:, :, None] * tok[:, None, None]).reshape(M, K)
    X[6] = 0.0
    Y = run_batch(X, w, M, K, N)
    ref = oracle_lib.q4k_matmul(X, w, M, K, N)
    assert np.all(Y[6] == 0.0)
    assert_parity(Y, ref, rowwise=True, what="wide-range tokens")


# --- the prefill tiles at every workgroup height (q4k_matmul_shaped) -------

def run_rows(X, w, M, K, N, rows):
    buf, Y = out_with_canary(N, rows=M)
    binding.q4k_matmul_shaped(dev(X), dev(w), M, K, N, Y, rows)
    out = host(Y)
    assert canary_intact(buf, M * N)
    return out


# 65: the 64-row tiles whose waves own whole super-blocks (activations
# loaded straight into MFMA operand registers); 128: the 128-row x 32-token
# tiles with input_dim split across workgroups (the shapes below give 1 to 8
# ranges, odd range lengths, a single super-block and ragged rows and tokens)
PREFILL_FORMS = [16, 32, 64, 65, 128]


@pytest.mark.parametrize("rows", PREFILL_FORMS)
@pytest.mark.parametrize("M,K,N", [(16, 256, 16), (17, 768, 65), (33, 1280, 130), (2, 1024, 100),
                                   (64, 4096, 64), (9, 14336, 40), (48, 2304, 129), (16, 512, 4097)])
def test_prefill_every_workgroup_height(oracle_lib, M, K, N, rows):
    """Ragged rows (N not a multiple of the height), ragged token tiles and
    stages; 16 rows splits each block's sub-blocks between two waves."""
    w = synth.q4k_weights(N, K, config=48, copy=K + N)
    X = synth.activations(K, n_tokens=M, config=48, copy=K + N)
    Y = run_rows(X, w, M, K, N, rows)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what=f"{M}x{K}x{N} rows {rows}")


@pytest.mark.parametrize("rows", PREFILL_FORMS)
def test_prefill_every_height_integer_bit_exact(oracle_lib, rows):
    M, K, N = 24, 4096, 96
    w = synth.q4k_integer_weights(N, K, config=49)
    X = synth.integer_activations(K, n_tokens=M, config=49)
    Y = run_rows(X, w, M, K, N, rows)
    assert np.array_equal(Y.astype(np.float64), oracle_lib.q4k_matmul(X, w, M, K, N))


@pytest.mark.parametrize("M,N", [(16, 4096), (32, 4096), (16, 14336)])
def test_prefill_narrow_full_size_sampled(oracle_lib, M, N):
    """The token counts that narrow the workgroups (automatic choice), at
    full size: every output of sampled token rows."""
    K = 4096
    w = synth.q4k_weights(N, K, config=50, copy=M)
    X = synth.activations(K, n_tokens=M, config=50, copy=M)
    Y = run(X, w, M, K, N)
    for t in (0, M // 2, M - 1):
        ref = oracle_lib.q4k_matmul_part(X, w, M, K, N, (t, t + 1), (0, N))[t]
        assert_parity(Y[t], ref, what=f"token {t}")



def wide_range_subblocks(M, K, config):
    """N(0,1) activations with every 32-element sub-block scaled by its own
    power of two in 2^-40 .. 2^40 and about one in ten sub-blocks zero."""
    X = synth.activations(K, n_tokens=M, config=config)
    g = np.random.default_rng(config)
    sub = np.exp2(g.integers(-40, 41, (M, K // 32))).astype(np.float32)
    sub[g.random((M, K // 32)) < 0.1] = 0.0
    return (X.reshape(M, -1, 32) * sub[:, :, None]).reshape(M, K)


def wide_range_tokens(M, K, config):
    """Whole token rows at very different magnitudes: 1e-5, 3e5 (above the
    fp16 range), 2^-60, 2^60, one all-zero row, the rest N(0,1)."""
    X = synth.activations(K, n_tokens=M, config=config)
    scale = np.ones(M, np.float32)
    scale[0:M // 5] = 1e-5
    scale[M // 5:2 * M // 5] = 3e5
    scale[2 * M // 5:3 * M // 5] = 2.0 ** -60
    scale[3 * M // 5:4 * M // 5] = 2.0 ** 60
    scale[M - 1] = 0.0
    return X * scale[:, None]


@pytest.mark.parametrize("rows", PREFILL_FORMS)
@pytest.mark.parametrize("M,K,N", [(24, 2048, 200), (40, 4096, 130)])
def test_prefill_wide_range_subblocks_every_height(oracle_lib, M, K, N, rows):
    """Sub-blocks from 2^-40 to 2^40 and zero sub-blocks: each token's
    super-block is scaled by a power of two before its fp16 split, so the
    prefill tiles stay within the bar at every height."""
    w = synth.q4k_weights(N, K, config=54, copy=rows)
    X = wide_range_subblocks(M, K, 54 + rows)
    Y = run_rows(X, w, M, K, N, rows)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True,
                  what=f"{M}x{K}x{N} rows {rows}")


@pytest.mark.parametrize("rows", PREFILL_FORMS)
def test_prefill_wide_range_tokens_every_height(oracle_lib, rows):
    """Token rows at 1e-5, 3e5 (|x| above 65504), 2^-60 and 2^60, and a zero
    row, at every workgroup height."""
    M, K, N = 40, 2048, 200
    w = synth.q4k_weights(N, K, config=55, copy=rows)
    X = wide_range_tokens(M, K, 55 + rows)
    Y = run_rows(X, w, M, K, N, rows)
    ref = oracle_lib.q4k_matmul(X, w, M, K, N)
    assert np.all(Y[M - 1] == 0.0)
    assert_parity(Y[:M - 1], ref[:M - 1], rowwise=True, what=f"rows {rows}")


def test_matmul_wide_range_full_config(oracle_lib):
    """The automatic choice at the prefill workload's shape with wide-range
    sub-blocks: every output of every token row."""
    M, K, N = 64, 4096, 4096
    w = synth.q4k_weights(N, K, config=synth.C4_PREFILL)
    X = wide_range_subblocks(M, K, 56)
    Y = run(X, w, M, K, N)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what="64x4096x4096")


@pytest.mark.parametrize("rows", [64, 65, 128])
def test_prefill_full_config_every_form(oracle_lib, rows):
    """64 x 4096 x 4096 on each 64-row prefill kernel, every output."""
    M, K, N = 64, 4096, 4096
    w = synth.q4k_weights(N, K, config=synth.C4_PREFILL)
    X = synth.activations(K, n_tokens=M, config=synth.C4_PREFILL)
    Y = run_rows(X, w, M, K, N, rows)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what=f"form {rows}")


def test_split_input_dim_same_bits_and_growing_workspace(oracle_lib):
    """Form 128 adds the ranges' partial tiles in range order whichever
    workgroup arrives last, so repeated calls give the same bits; shapes
    that need more workspace than the last one (the library grows it
    between calls) and smaller ones after them stay correct."""
    shapes = [(33, 1280, 130), (64, 4096, 4096), (9, 14336, 40), (64, 4096, 64), (48, 2304, 129)]
    for M, K, N in shapes:
        w = synth.q4k_weights(N, K, config=57, copy=M)
        X = synth.activations(K, n_tokens=M, config=57, copy=N)
        Y1 = run_rows(X, w, M, K, N, 128)
        Y2 = run_rows(X, w, M, K, N, 128)
        assert np.array_equal(Y1, Y2), f"{M}x{K}x{N}"
        if M * K * N <= 64 * 4096 * 64:
            assert_parity(Y1, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True,
                          what=f"{M}x{K}x{N}")
        else:
            for t in (0, M - 1):
                ref = oracle_lib.q4k_matmul_part(X, w, M, K, N, (t, t + 1), (0, N))[t]
                assert_parity(Y1[t], ref, what=f"{M}x{K}x{N} token {t}")


@pytest.mark.parametrize("S", range(1, 9))
def test_split_every_range_count(oracle_lib, S):
    """Forms 129 .. 136 fix the number of input_dim ranges (16 super-blocks:
    ranges of 2 to 16, some of odd length)."""
    M, K, N = 40, 4096, 200
    w = synth.q4k_weights(N, K, config=58, copy=S)
    X = synth.activations(K, n_tokens=M, config=58, copy=S)
    Y = run_rows(X, w, M, K, N, 128 + S)
    assert_parity(Y, oracle_lib.q4k_matmul(X, w, M, K, N), rowwise=True, what=f"S={S}")
