"""Every entry point captured into a HIP graph and replayed several times,
with eager work and synchronisation between replays; each replay must match
the eager result (the benchmark times graph replays of these calls)."""
import numpy as np
import pytest
import torch

from q4_packed_weight_amd import binding, synth
from gpu_util import DEV, dev, host
from tolerance import assert_parity

pytestmark = pytest.mark.gpu


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s), torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _replays_match(fn, out, eager, exact=True):
    g = _capture(fn)
    for i in range(4):
        out.fill_(float("nan"))              # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        got = host(out)
        if exact:
            assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), i
        else:
            assert_parity(got, eager.astype(np.float64), rowwise=got.ndim == 2, what=f"replay {i}")


@pytest.mark.parametrize("K,N", [(4096, 1000), (14336, 4096), (4096, 14336)],
                         ids=["vector", "walk-per-wave", "walk-4-groups"])
def test_gemv_graph_replays(K, N):
    w = dev(synth.q4k_weights(N, K, config=40))
    x = dev(synth.activations(K, config=40))
    y = torch.empty(N, dtype=torch.float32, device=DEV)
    binding.q4k_gemv(x, w, K, N, y)
    eager = host(y).copy()
    _replays_match(lambda: binding.q4k_gemv(x, w, K, N, y), y, eager)


def test_ternary_graph_replays():
    K, N = 4096, 700
    c = dev(synth.ternary_codes(N, K, config=41)[0])
    x = dev(synth.activations(K, config=41))
    y = torch.empty(N, dtype=torch.float32, device=DEV)
    binding.ternary_gemv(x, c, 1.25, K, N, y)
    eager = host(y).copy()
    _replays_match(lambda: binding.ternary_gemv(x, c, 1.25, K, N, y), y, eager)


def test_matmul_graph_replays():
    """The batched path: replays match the eager result bit for bit, on
    float and on integer inputs."""
    M, K, N = 64, 2048, 384
    w = dev(synth.q4k_weights(N, K, config=42))
    X = dev(synth.activations(K, n_tokens=M, config=42))
    Y = torch.empty(M, N, dtype=torch.float32, device=DEV)
    binding.q4k_matmul(X, w, M, K, N, Y)
    eager = host(Y).copy()
    _replays_match(lambda: binding.q4k_matmul(X, w, M, K, N, Y), Y, eager, exact=True)
    wi = dev(synth.q4k_integer_weights(N, K, config=43))
    Xi = dev(synth.integer_activations(K, n_tokens=M, config=43))
    binding.q4k_matmul(Xi, wi, M, K, N, Y)
    eager = host(Y).copy()
    _replays_match(lambda: binding.q4k_matmul(Xi, wi, M, K, N, Y), Y, eager, exact=True)


@pytest.mark.parametrize("M", [2, 5, 8])
def test_matmul_few_tokens_graph_replays(M):
    """The few-token path (the batched matrix-core GEMV): replays match the
    eager result bit for bit."""
    K, N = 4096, 512
    w = dev(synth.q4k_weights(N, K, config=44))
    X = dev(synth.activations(K, n_tokens=M, config=44))
    Y = torch.empty(M, N, dtype=torch.float32, device=DEV)
    binding.q4k_matmul(X, w, M, K, N, Y)
    eager = host(Y).copy()
    _replays_match(lambda: binding.q4k_matmul(X, w, M, K, N, Y), Y, eager, exact=True)


@pytest.mark.parametrize("form", [128, 136])
def test_matmul_split_graph_replays(form):
    """The split tiles (input_dim ranges added through the library's
    workspace, arrival counters left at zero by every call): replays match
    the eager result bit for bit."""
    M, K, N = 48, 4096, 640
    w = dev(synth.q4k_weights(N, K, config=45))
    X = dev(synth.activations(K, n_tokens=M, config=45))
    Y = torch.empty(M, N, dtype=torch.float32, device=DEV)
    binding.q4k_matmul_shaped(X, w, M, K, N, Y, form)
    eager = host(Y).copy()
    _replays_match(lambda: binding.q4k_matmul_shaped(X, w, M, K, N, Y, form), Y, eager, exact=True)
