"""Q4_0 GEMV on the GPU against the CPU oracle, through the C ABI.

Q4_0 is the Q4_K page's follow-up format (section "Out of scope": the same
algorithm on a block of 32 weights in 18 bytes).  Parity bar as for Q4_K
(tests/tolerance.py); bit-exact where every product and partial sum is exact
(one-hot and integer inputs).
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
        binding.q4_0_gemv(xd, wd, K, N, y)
    else:
        binding.q4_0_gemv_shaped(xd, wd, K, N, y, *shape)
    out = host(y)
    assert canary_intact(buf, N), "write past the end of y"
    return out


# one 144-byte group, several, ragged group counts (K/256 not a multiple of
# 16), ragged row counts, the persistent walk (one step per row, many rows)
SHAPES = [(256, 1), (256, 7), (512, 64), (768, 37), (2304, 129), (3840, 333),
          (4352, 1000), (14336, 100), (1024, 1024), (4096, 4096), (256, 4097),
          (4096, 14336), (14336, 4096), (2048, 33000)]


@pytest.mark.parametrize("K,N", SHAPES)
def test_q4_0_parity(oracle_lib, K, N):
    w = synth.q4_0_weights(N, K, copy=K + N)
    x = synth.activations(K, config=synth.Q40_4K, copy=K + N)
    y = run(x, w, K, N)
    assert_parity(y, oracle_lib.q4_0_gemv(x, w, K, N), what=f"K={K} N={N}")


@pytest.mark.parametrize("rpl,kw,wg", VECTOR_SHAPES)
@pytest.mark.parametrize("K,N", [(4096, 333), (14336, 67), (1024, 129), (256, 50)])
def test_q4_0_every_launch_shape(oracle_lib, K, N, rpl, kw, wg):
    w = synth.q4_0_weights(N, K, copy=3 * K)
    x = synth.activations(K, config=synth.Q40_4K, copy=3 * K)
    y = run(x, w, K, N, shape=(rpl, kw, wg))
    assert_parity(y, oracle_lib.q4_0_gemv(x, w, K, N), what=f"shape {rpl},{kw},{wg}")


# the matrix-core form: one group, fewer groups than waves, ragged rows, the
# shapes the automatic choice gives it, and the longest rows it takes
MFMA_SHAPES = [(256, 1), (256, 7), (768, 37), (2304, 129), (3072, 3072), (4096, 4096),
               (4096, 333), (14336, 100), (65536, 20)]
MFMA = (0, 0, 16)


@pytest.mark.parametrize("K,N", MFMA_SHAPES)
def test_q4_0_matrix_core_form_parity(oracle_lib, K, N):
    w = synth.q4_0_weights(N, K, copy=K + 2 * N)
    x = synth.activations(K, config=synth.Q40_4K, copy=K + 2 * N)
    y = run(x, w, K, N, shape=MFMA)
    assert_parity(y, oracle_lib.q4_0_gemv(x, w, K, N), what=f"mfma K={K} N={N}")


def test_q4_0_matrix_core_form_one_hot_bit_exact(oracle_lib):
    """x = e_k through the matrix-core form: every position of a group of
    eight blocks (block order, nibble-to-element mapping, the realigned
    code bytes of the odd blocks, the lane groups' A rows) gives d*(q-8)
    exactly, for 17 rows (two row tiles, the second ragged)."""
    K, N = 256, 17
    w = synth.q4_0_weights(N, K, copy=11)
    wd = dev(w)
    buf, y = out_with_canary(N)
    X = np.eye(K, dtype=np.float32)
    for k in range(K):
        binding.q4_0_gemv_shaped(dev(X[k]), wd, K, N, y, *MFMA)
        got = host(y)
        ref = oracle_lib.q4_0_gemv(X[k], w, K, N).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), k
    assert canary_intact(buf, N)


@pytest.mark.parametrize("K,N", [(4096, 512), (3072, 3072), (65536, 16)])
def test_q4_0_matrix_core_form_integer_bit_exact(oracle_lib, K, N):
    w = synth.q4_0_integer_weights(N, K, config=74)
    x = synth.integer_activations(K, config=74)
    y = run(x, w, K, N, shape=MFMA)
    assert np.array_equal(y.astype(np.float64), oracle_lib.q4_0_gemv(x, w, K, N))


def test_q4_0_matrix_core_form_wide_range_and_subnormal_d(oracle_lib):
    """Blocks of activations 2^-40 .. 2^40 apart (some zero, some near the
    largest finite fp32 the split takes) and binary16 subnormal d."""
    K, N = 4096, 300
    w = synth.q4_0_weights(N, K, copy=12).reshape(-1, 18).copy()
    g = np.random.default_rng(75)
    sub = g.choice(w.shape[0], w.shape[0] // 3, replace=False)
    w[sub, 0:2] = g.integers(1, 1024, sub.size).astype(np.uint16).view(np.uint8).reshape(-1, 2)
    w = w.reshape(N, -1)
    x = synth.activations(K, config=synth.Q40_4K, copy=12)
    scale = np.exp2(g.integers(-40, 41, K // 32)).astype(np.float32)
    scale[g.choice(K // 32, 3, replace=False)] = 0.0
    scale[5] = np.float32(2.0 ** 90)
    x = (x.reshape(-1, 32) * scale[:, None]).reshape(-1)
    y = run(x, w, K, N, shape=MFMA)
    assert_parity(y, oracle_lib.q4_0_gemv(x, w, K, N), what="mfma wide range")
    a, b = run(x, w, K, N, shape=MFMA), run(x, w, K, N, shape=MFMA)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("K,N,mfma", [(4096, 4096, True), (3072, 3072, True), (6144, 3072, True),
                                      (2048, 4096, False), (4096, 2048, False),
                                      (6400, 4096, False), (4096, 8192, False)])
def test_q4_0_automatic_choice(oracle_lib, K, N, mfma):
    """q4_0_gemv equals, bit for bit, the form it is documented to take."""
    w = synth.q4_0_weights(N, K, copy=13)
    x = synth.activations(K, config=synth.Q40_4K, copy=13)
    y = run(x, w, K, N)
    y2 = run(x, w, K, N, shape=MFMA if mfma else (0, 0, 0))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_q4_0_one_hot_bit_exact_all_positions(oracle_lib):
    """x = e_k: y[o] is the oracle's fp32 weight d*(q-8) exactly, for every
    position of a 256-weight group (eight blocks) -- pins the block order,
    the nibble-to-element mapping and the realignment of odd blocks."""
    K, N = 256, 9
    w = synth.q4_0_weights(N, K, copy=1)
    wd = dev(w)
    buf, y = out_with_canary(N)
    X = np.eye(K, dtype=np.float32)
    for k in range(K):
        binding.q4_0_gemv(dev(X[k]), wd, K, N, y)
        got = host(y)
        ref = oracle_lib.q4_0_gemv(X[k], w, K, N).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), k
    assert canary_intact(buf, N)


def test_q4_0_one_hot_bit_exact_sampled_large(oracle_lib):
    K, N = 4096, 300
    w = synth.q4_0_weights(N, K, copy=2)
    wd = dev(w)
    for k in np.random.default_rng(6).choice(K, 48, replace=False):
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        buf, yd = out_with_canary(N)
        binding.q4_0_gemv(dev(x), wd, K, N, yd)
        got = host(yd)
        ref = oracle_lib.q4_0_gemv(x, w, K, N).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), k


@pytest.mark.parametrize("K,N", [(4096, 512), (14336, 64), (768, 100), (4096, 14336)])
def test_q4_0_integer_inputs_bit_exact(oracle_lib, K, N):
    """d = 1, x in {-1, 0, 1}: every partial sum is an integer far below
    2^24, so any summation order is exact and the GPU equals the oracle."""
    w = synth.q4_0_integer_weights(N, K, config=71)
    x = synth.integer_activations(K, config=71)
    y = run(x, w, K, N)
    ref = oracle_lib.q4_0_gemv(x, w, K, N)
    assert np.all(ref == np.round(ref))
    assert np.array_equal(y.astype(np.float64), ref)


def test_q4_0_wide_range_activations(oracle_lib):
    """Activations at 2^-40 .. 2^40 per 32-element block, some blocks zero."""
    K, N = 4096, 512
    w = synth.q4_0_weights(N, K, copy=5)
    x = synth.activations(K, config=synth.Q40_4K, copy=5)
    g = np.random.default_rng(72)
    scale = np.exp2(g.integers(-40, 41, K // 32)).astype(np.float32)
    scale[g.choice(K // 32, 3, replace=False)] = 0.0
    x = (x.reshape(-1, 32) * scale[:, None]).reshape(-1)
    y = run(x, w, K, N)
    assert_parity(y, oracle_lib.q4_0_gemv(x, w, K, N), what="wide range")


def test_q4_0_zero_activation_and_determinism(oracle_lib):
    K, N = 4096, 1024
    w = synth.q4_0_weights(N, K, copy=6)
    assert np.all(run(np.zeros(K, np.float32), w, K, N) == 0.0)
    x = synth.activations(K, config=synth.Q40_4K, copy=6)
    a, b = run(x, w, K, N), run(x, w, K, N)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_q4_0_subnormal_scales(oracle_lib):
    """binary16 subnormal d in every block still decodes exactly."""
    K, N = 1024, 64
    w = synth.q4_0_weights(N, K, copy=7).reshape(-1, 18).copy()
    g = np.random.default_rng(73)
    w[:, 0:2] = g.integers(1, 1024, w.shape[0]).astype(np.uint16).view(np.uint8).reshape(-1, 2)
    w = w.reshape(N, -1)
    x = synth.activations(K, config=synth.Q40_4K, copy=7)
    assert_parity(run(x, w, K, N), oracle_lib.q4_0_gemv(x, w, K, N), what="subnormal d")


@pytest.mark.parametrize("K", [32, 96, 288, 0, -256])
def test_q4_0_rejects_input_dim_not_multiple_of_256(K):
    """The format allows any multiple of 32; this kernel takes whole
    144-byte groups only and must reject the rest before launching."""
    xd = dev(np.zeros(max(K, 1), np.float32))
    wd = dev(np.zeros(18 * max(K // 32, 1), np.uint8))
    buf, y = out_with_canary(1)
    with pytest.raises(ValueError) as e:
        binding.q4_0_gemv(xd, wd, K, 1, y)
    assert getattr(e.value, "code", binding.Q4K_EINVAL_DIM) == binding.Q4K_EINVAL_DIM
    assert np.all(np.isnan(host(buf)))


def test_q4_0_rejects_misaligned_weights():
    K, N = 256, 2
    xd = dev(np.zeros(K, np.float32))
    wd = dev(np.zeros(N * 8 * 18 + 16, np.uint8))[2:]
    buf, y = out_with_canary(N)
    with pytest.raises(ValueError) as e:
        binding.q4_0_gemv(xd, wd, K, N, y)
    assert e.value.code == binding.Q4K_EALIGN
    assert np.all(np.isnan(host(buf)))
