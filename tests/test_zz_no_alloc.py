"""q4k_matmul_noalloc (for callers that cannot allocate: its split tiles use
a fixed scratch array that comes with the library) against q4k_matmul, on
two calls in a row, the second smaller, and once more on a shape that takes
no scratch."""
import numpy as np
import pytest

from q4_packed_weight_amd import binding, synth
from gpu_util import canary_intact, dev, host, out_with_canary
from tolerance import assert_parity

pytestmark = pytest.mark.gpu


def test_noalloc_matches_matmul_on_consecutive_calls():
    # 64x4096x4096: 64 tiles x 4 ranges (the whole 4 MiB of partial tiles);
    # 40x2048x200: 4 tiles x 4 ranges; 4 tokens: the batched GEMV, no scratch
    for M, K, N in ((64, 4096, 4096), (40, 2048, 200), (4, 1024, 96)):
        w = dev(synth.q4k_weights(N, K, config=59, copy=M))
        X = dev(synth.activations(K, n_tokens=M, config=59, copy=N))
        buf, Y = out_with_canary(N, rows=M)
        binding.q4k_matmul_noalloc(X, w, M, K, N, Y)
        got = host(Y)
        assert canary_intact(buf, M * N)
        _, R = out_with_canary(N, rows=M)
        binding.q4k_matmul(X, w, M, K, N, R)
        ref = host(R)
        assert_parity(got, ref.astype(np.float64), rowwise=True, what=f"{M}x{K}x{N}")
        # same kernel, same ranges, same order of additions
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{M}x{K}x{N}"
