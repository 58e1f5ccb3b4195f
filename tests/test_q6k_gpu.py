"""Q6_K GEMV on the GPU against the CPU oracle, through the C ABI.

Q6_K is the Q4_K page's second follow-up format (section "Out of scope": ql
and qh, four codes' high bits per qh byte).  Its 210-byte blocks put rows
at any even byte offset, so the shapes below include input_dim values whose
rows are not 16-byte aligned.  Parity bar as for Q4_K (tests/tolerance.py);
bit-exact where every product and partial sum is exact.
"""
import numpy as np
import pytest

from q4_packed_weight_amd import binding, synth
from gpu_util import VECTOR_SHAPES, canary_intact, dev, host, out_with_canary
from tolerance import assert_parity

pytestmark = pytest.mark.gpu


def run(x, w, K, N, shape=None):
    xd, wd = dev(x), dev(w)
    buf, y = out_with_canary(N)
    if shape is None:
        binding.q6k_gemv(xd, wd, K, N, y)
    else:
        binding.q6k_gemv_shaped(xd, wd, K, N, y, *shape)
    out = host(y)
    assert canary_intact(buf, N), "write past the end of y"
    return out


# aligned rows (input_dim a multiple of 2048) and rows at every even offset
# (input_dim/256 odd or not a multiple of 8); 32- and 64-lane steps; ragged
# row counts; the persistent walk; the FFN shapes
SHAPES = [(256, 1), (256, 9), (768, 37), (1280, 5), (2304, 129), (4096, 64),
          (3840, 333), (4352, 1000), (11008, 100), (14336, 100), (1024, 1024),
          (4096, 4096), (2048, 33000), (4096, 14336), (14336, 4096), (256, 4097)]


@pytest.mark.parametrize("K,N", SHAPES)
def test_q6k_parity(oracle_lib, K, N):
    w = synth.q6k_weights(N, K, copy=K + N)
    x = synth.activations(K, config=synth.Q6K_4K, copy=K + N)
    y = run(x, w, K, N)
    assert_parity(y, oracle_lib.q6k_gemv(x, w, K, N), what=f"K={K} N={N}")


@pytest.mark.parametrize("rpl,kw,wg", VECTOR_SHAPES)
@pytest.mark.parametrize("K,N", [(4096, 333), (14336, 67), (1024, 129), (768, 50)])
def test_q6k_every_launch_shape(oracle_lib, K, N, rpl, kw, wg):
    w = synth.q6k_weights(N, K, copy=5 * K)
    x = synth.activations(K, config=synth.Q6K_4K, copy=5 * K)
    if rpl == 8 and kw == 4 and 4 * (K // 256) > 32:
        # 64 lanes per row: the tiles of this shape exceed the LDS
        with pytest.raises(ValueError) as e:
            run(x, w, K, N, shape=(rpl, kw, wg))
        assert e.value.code == binding.Q4K_EINVAL_DIM
        return
    y = run(x, w, K, N, shape=(rpl, kw, wg))
    assert_parity(y, oracle_lib.q6k_gemv(x, w, K, N), what=f"shape {rpl},{kw},{wg}")


def test_q6k_one_hot_bit_exact_all_positions(oracle_lib):
    """x = e_k: y[o] is the oracle's fp32 weight d*scale*(q-32) exactly, for
    every position of a block; nine one-block rows start at every even byte
    offset mod 16, so this also pins the realignment of misaligned rows."""
    K, N = 256, 9
    w = synth.q6k_weights(N, K, copy=1)
    wd = dev(w)
    buf, y = out_with_canary(N)
    X = np.eye(K, dtype=np.float32)
    for k in range(K):
        binding.q6k_gemv(dev(X[k]), wd, K, N, y)
        got = host(y)
        ref = oracle_lib.q6k_gemv(X[k], w, K, N).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), k
    assert canary_intact(buf, N)


@pytest.mark.parametrize("K,N", [(4096, 300), (11008, 40)])
def test_q6k_one_hot_bit_exact_sampled_large(oracle_lib, K, N):
    w = synth.q6k_weights(N, K, copy=2)
    wd = dev(w)
    for k in np.random.default_rng(61).choice(K, 40, replace=False):
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        buf, yd = out_with_canary(N)
        binding.q6k_gemv(dev(x), wd, K, N, yd)
        got = host(yd)
        ref = oracle_lib.q6k_gemv(x, w, K, N).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), k


@pytest.mark.parametrize("K,N", [(4096, 512), (14336, 64), (768, 100), (11008, 33), (4096, 14336)])
def test_q6k_integer_inputs_bit_exact(oracle_lib, K, N):
    """d = 1, scales +-1, x in {-1, 0, 1}: every partial sum is an integer
    below 2^24, so the GPU equals the oracle exactly."""
    w = synth.q6k_integer_weights(N, K, config=74)
    x = synth.integer_activations(K, config=74)
    y = run(x, w, K, N)
    ref = oracle_lib.q6k_gemv(x, w, K, N)
    assert np.all(ref == np.round(ref))
    assert np.array_equal(y.astype(np.float64), ref)


def test_q6k_wide_range_activations(oracle_lib):
    K, N = 4096, 512
    w = synth.q6k_weights(N, K, copy=5)
    x = synth.activations(K, config=synth.Q6K_4K, copy=5)
    g = np.random.default_rng(75)
    scale = np.exp2(g.integers(-40, 41, K // 16)).astype(np.float32)
    scale[g.choice(K // 16, 3, replace=False)] = 0.0
    x = (x.reshape(-1, 16) * scale[:, None]).reshape(-1)
    assert_parity(run(x, w, K, N), oracle_lib.q6k_gemv(x, w, K, N), what="wide range")


def test_q6k_extreme_scales_and_subnormal_d(oracle_lib):
    K, N = 2304, 64
    w = synth.q6k_weights(N, K, copy=7).reshape(-1, 210).copy()
    g = np.random.default_rng(76)
    w[:, 192:208] = np.where(g.random((w.shape[0], 16)) < 0.5, -128, 127).astype(np.int8).view(np.uint8)
    w[::3, 208:210] = g.integers(1, 1024, len(w[::3])).astype(np.uint16).view(np.uint8).reshape(-1, 2)
    w = w.reshape(N, -1)
    x = synth.activations(K, config=synth.Q6K_4K, copy=7)
    assert_parity(run(x, w, K, N), oracle_lib.q6k_gemv(x, w, K, N), what="extreme scales")


def test_q6k_zero_activation_and_determinism(oracle_lib):
    K, N = 4096, 1024
    w = synth.q6k_weights(N, K, copy=6)
    assert np.all(run(np.zeros(K, np.float32), w, K, N) == 0.0)
    x = synth.activations(K, config=synth.Q6K_4K, copy=6)
    a, b = run(x, w, K, N), run(x, w, K, N)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("K", [32, 255, 257, 0, -256])
def test_q6k_rejects_input_dim_not_multiple_of_256(K):
    xd = dev(np.zeros(max(K, 1), np.float32))
    wd = dev(np.zeros(210 * 2, np.uint8))
    buf, y = out_with_canary(1)
    with pytest.raises(ValueError) as e:
        binding.q6k_gemv(xd, wd, K, 1, y)
    assert getattr(e.value, "code", binding.Q4K_EINVAL_DIM) == binding.Q4K_EINVAL_DIM
    assert np.all(np.isnan(host(buf)))


def test_q6k_rejects_misaligned_weights():
    K, N = 256, 2
    xd = dev(np.zeros(K, np.float32))
    wd = dev(np.zeros(N * 210 + 16, np.uint8))[2:]
    buf, y = out_with_canary(N)
    with pytest.raises(ValueError) as e:
        binding.q6k_gemv(xd, wd, K, N, y)
    assert e.value.code == binding.Q4K_EALIGN
    assert np.all(np.isnan(host(buf)))
