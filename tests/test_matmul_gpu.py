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


def test_matmul_full_config_sampled_tokens(oracle_lib):
    """64 x 4096 x 4096: every output of 8 sampled token rows."""
    M, K, N = 64, 4096, 4096
    w = synth.q4k_weights(N, K, config=synth.C4_PREFILL)
    X = synth.activations(K, n_tokens=M, config=synth.C4_PREFILL)
    Y = run(X, w, M, K, N)
    for t in (0, 7, 21, 33, 40, 52, 62, 63):
        ref = oracle_lib.q4k_matmul_part(X, w, M, K, N, (t, t + 1), (0, N))[t]
        assert_parity(Y[t], ref, what=f"token {t}")


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
