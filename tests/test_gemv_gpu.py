"""Q4_K GEMV on the GPU against the CPU oracle, through the C ABI.

Parity bar: |y - ref| <= 1e-4*|ref| + 1e-4*rms(ref) elementwise (the Q4_K
page's "within 1e-4 relative", read as in tests/tolerance.py); bit-exact
where every product and partial sum is exact (one-hot and integer inputs).
"""
import numpy as np
import pytest
import torch

from q4_packed_weight_amd import binding, synth
from gpu_util import VECTOR_SHAPES, canary_intact, dev, host, out_with_canary
from tolerance import assert_parity

pytestmark = pytest.mark.gpu


def run_gemv(x, w, K, N, shape=None, walk=None):
    xd, wd = dev(x), dev(w)
    buf, y = out_with_canary(N)
    if walk is not None:
        binding.q4k_gemv_walk_shaped(xd, wd, K, N, y, *walk)
    elif shape is None:
        binding.q4k_gemv(xd, wd, K, N, y)
    else:
        binding.q4k_gemv_shaped(xd, wd, K, N, y, *shape)
    out = host(y)
    assert canary_intact(buf, N), "write past the end of y"
    return out


# (K, N): single block, multi-block, multi-row, the page's 4096x64, ragged
# slab counts (K/256 not a multiple of 16) and ragged row counts.
SHAPES = [(256, 1), (512, 1), (256, 7), (4096, 64), (768, 37), (1280, 5),
          (2304, 129), (3840, 333), (4352, 1000), (14336, 100), (1024, 1024),
          (8192, 17), (256, 4097)]


@pytest.mark.parametrize("K,N", SHAPES)
def test_gemv_parity(oracle_lib, K, N):
    w = synth.q4k_weights(N, K, config=10, copy=K + N)
    x = synth.activations(K, config=10, copy=K + N)
    y = run_gemv(x, w, K, N)
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what=f"K={K} N={N}")


@pytest.mark.parametrize("K,N,name", [(1024, 1024, "c1"), (4096, 4096, "c2"),
                                      (4096, 14336, "c3-up"), (14336, 4096, "c3-down")])
def test_gemv_parity_full_configs(oracle_lib, K, N, name):
    cfg = {"c1": synth.C1_Q4K_1K, "c2": synth.C2_Q4K_4K}.get(name, synth.C3_FFN)
    extra = 1 if name == "c3-down" else 0
    w = synth.q4k_weights(N, K, config=cfg, extra=extra)
    x = synth.activations(K, config=cfg, extra=extra)
    y = run_gemv(x, w, K, N)
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what=name)


@pytest.mark.parametrize("K,N", SHAPES + [(4096, 4096), (14336, 300), (2560, 4090)])
def test_matrix_core_form_parity(oracle_lib, K, N):
    """workgroup_waves = 16: the MFMA form at every shape (single block,
    ragged rows and super-block counts, waves without blocks, long rows)."""
    w = synth.q4k_weights(N, K, config=20, copy=K + N)
    x = synth.activations(K, config=20, copy=K + N)
    y = run_gemv(x, w, K, N, shape=(0, 0, 16))
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what=f"mfma K={K} N={N}")


@pytest.mark.parametrize("K,N", [(4096, 4096), (14336, 64), (768, 100)])
def test_matrix_core_form_integer_bit_exact(oracle_lib, K, N):
    """Integer weights and activations: the MFMA form is exact too (the
    codes and the hi/lo activation halves are exact fp16 operands)."""
    w = synth.q4k_integer_weights(N, K, config=21)
    x = synth.integer_activations(K, config=21)
    y = run_gemv(x, w, K, N, shape=(0, 0, 16))
    assert np.array_equal(y.astype(np.float64), oracle_lib.q4k_gemv(x, w, K, N))


@pytest.mark.parametrize("form", [None, (0, 0, 16), "walk"], ids=["auto", "mfma", "walk"])
@pytest.mark.parametrize("K,N,lo,hi", [(4096, 4096, -40, 40), (2560, 300, -40, 40),
                                       (4096, 256, -60, 92), (18432, 100, -60, 92)])
def test_wide_range_activations(oracle_lib, K, N, lo, hi, form):
    """Activations far outside fp16's range, with every 32-element sub-block
    at its own scale 2^lo .. 2^hi (up to just below the documented 2^96
    bound of the matrix-core form) and some sub-blocks all zero: both forms
    stay within the bar (the matrix-core form rescales each sub-block by a
    power of two before its fp16 split)."""
    w = synth.q4k_weights(N, K, config=22, copy=K + N)
    x = synth.activations(K, config=22, copy=K + N)
    g = np.random.default_rng(22)
    scale = np.exp2(g.integers(lo, hi + 1, K // 32)).astype(np.float32)
    scale[g.choice(K // 32, 3, replace=False)] = 0.0
    x = (x.reshape(-1, 32) * scale[:, None]).reshape(-1)
    assert np.abs(x).max() > 1e9
    if form == "walk":
        y = run_gemv(x, w, K, N, walk=(8, 0, 2))
    else:
        y = run_gemv(x, w, K, N, shape=form)
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what=f"wide K={K} N={N}")


# The persistent matrix-core walk: (waves, row groups per workgroup, units
# ahead); 0 lets the library choose.
WALK_SHAPES = [(8, 0, 2), (8, 0, 4), (4, 0, 4), (16, 0, 2), (8, 1, 2), (8, 2, 2), (8, 3, 4),
               (4, 4, 4), (16, 4, 2)]


@pytest.mark.parametrize("wf", WALK_SHAPES)
@pytest.mark.parametrize("K,N", [(256, 7), (2048, 333), (4096, 1000), (5120, 64), (14336, 100),
                                 (18432, 37), (65792, 20)])
def test_walk_every_shape(oracle_lib, K, N, wf):
    """Every launch shape of the walk over: one super-block and fewer rows
    than a group (waves without units), fewer super-blocks than waves,
    16 super-blocks (activations staged for the whole workgroup), 20 and 56
    (staged per wave where each wave keeps its super-blocks, by the
    workgroup otherwise), 72 (two chunks of activations) and 257 (exact
    normal code operands, five chunks); ragged row groups and row-group
    counts not a multiple of the workgroup's."""
    w = synth.q4k_weights(N, K, config=23, copy=K + N)
    x = synth.activations(K, config=23, copy=K + N)
    y = run_gemv(x, w, K, N, walk=wf)
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what=f"walk {wf} K={K} N={N}")


@pytest.mark.parametrize("wf", [(8, 0, 2), (4, 0, 4), (16, 0, 2)])
@pytest.mark.parametrize("K,N", [(14336, 64), (4096, 512), (18432, 48), (65792, 16)])
def test_walk_integer_bit_exact(oracle_lib, K, N, wf):
    """Integer weights and activations: the walk is exact (exact fp16
    operands, integer partial sums below 2^24), including the normal-code
    instantiation for rows of more than 256 super-blocks."""
    w = synth.q4k_integer_weights(N, K, config=24)
    x = synth.integer_activations(K, config=24)
    y = run_gemv(x, w, K, N, walk=wf)
    assert np.array_equal(y.astype(np.float64), oracle_lib.q4k_gemv(x, w, K, N))


# (K, N, form q4k_gemv takes): each side of the measured boundaries between
# the vector form, the matrix-core form and the walk.
AUTO_CHOICES = [(2048, 4096, "vector"), (3072, 3072, "mfma"), (3072, 4096, "mfma"),
                (4096, 2048, "vector"), (4096, 4096, "mfma"), (4096, 8192, "vector"),
                (4864, 3072, "mfma"), (5120, 3072, "walk"), (6144, 4096, "walk"),
                (8192, 2048, "vector"), (5120, 5120, "walk")]


@pytest.mark.parametrize("K,N,form", AUTO_CHOICES)
def test_automatic_choice_is_the_measured_form(oracle_lib, K, N, form):
    """q4k_gemv equals, bit for bit, the form it is documented to take at
    this shape, and matches the oracle."""
    w = synth.q4k_weights(N, K, config=26, copy=K + N)
    x = synth.activations(K, config=26, copy=K + N)
    y = run_gemv(x, w, K, N)
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what=f"auto K={K} N={N}")
    if form == "walk":
        y2 = run_gemv(x, w, K, N, walk=(0, 0, 0))
    else:
        y2 = run_gemv(x, w, K, N, shape=(0, 0, 16 if form == "mfma" else 0))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), form


@pytest.mark.parametrize("K,N", [(4096, 14341), (8192, 4096), (11008, 4096)])
def test_walk_automatic_choice(oracle_lib, K, N):
    """Shapes q4k_gemv hands to the walk: four row groups per workgroup with
    a ragged last group and a last workgroup of one group; one row group
    per workgroup with per-wave staging (32 and 43 super-blocks)."""
    w = synth.q4k_weights(N, K, config=25, copy=K + N)
    x = synth.activations(K, config=25, copy=K + N)
    y = run_gemv(x, w, K, N)
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what=f"auto walk K={K} N={N}")
    y2 = run_gemv(x, w, K, N, walk=(0, 0, 0))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_walk_many_rows_sampled(oracle_lib):
    """2^17 rows of 16 super-blocks (302 MB of weights, 8192 workgroups of
    four row groups): sampled rows against the oracle run on just those
    rows, the first and last included."""
    K, N = 4096, 1 << 17
    w = synth.q4k_weights(N, K, config=27)
    x = synth.activations(K, config=27)
    y = run_gemv(x, w, K, N)
    rows = np.random.default_rng(27).choice(N, 1500, replace=False)
    rows = np.concatenate([rows, [0, N - 1]])
    assert_parity(y[rows], oracle_lib.q4k_gemv(x, w[rows], K, len(rows)), what="sampled rows")


def test_walk_deterministic():
    """One writer per output and a fixed summation order: repeated calls
    agree bit for bit."""
    K, N = 14336, 512
    w = synth.q4k_weights(N, K, config=26)
    x = synth.activations(K, config=26)
    a = run_gemv(x, w, K, N, walk=(8, 0, 2))
    b = run_gemv(x, w, K, N, walk=(8, 0, 2))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_matrix_core_form_rejects_shape_fields():
    xd = dev(np.zeros(256, np.float32))
    wd = dev(np.zeros(144, np.uint8))
    buf, y = out_with_canary(1)
    with pytest.raises(ValueError):
        binding.q4k_gemv_shaped(xd, wd, 256, 1, y, 4, 0, 16)


@pytest.mark.parametrize("rpl,kw,wg", VECTOR_SHAPES)
@pytest.mark.parametrize("K,N", [(4096, 333), (14336, 67), (1024, 129), (256, 50)])
def test_every_launch_shape(oracle_lib, K, N, rpl, kw, wg):
    w = synth.q4k_weights(N, K, config=11, copy=K)
    x = synth.activations(K, config=11, copy=K)
    y = run_gemv(x, w, K, N, shape=(rpl, kw, wg))
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what=f"shape {rpl},{kw},{wg}")


def test_one_hot_bit_exact_all_positions(oracle_lib):
    """x = e_k: y[o] is the oracle's fp32 weight W[o,k] exactly (every other
    term is an exact zero), for every k of a block -- pins the nibble and
    sub-block mapping and the scale unpacking on the GPU."""
    K, N = 256, 9
    w = synth.q4k_weights(N, K, config=12)
    wd = dev(w)
    buf, y = out_with_canary(N)
    X = np.eye(K, dtype=np.float32)
    for k in range(K):
        binding.q4k_gemv(dev(X[k]), wd, K, N, y)
        got = host(y)
        ref = oracle_lib.q4k_gemv(X[k], w, K, N).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), k
    assert canary_intact(buf, N)


def test_one_hot_bit_exact_sampled_large(oracle_lib):
    K, N = 4096, 300
    w = synth.q4k_weights(N, K, config=13)
    wd = dev(w)
    g = np.random.default_rng(3)
    for k in g.choice(K, 48, replace=False):
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        buf, yd = out_with_canary(N)
        binding.q4k_gemv(dev(x), wd, K, N, yd)
        got = host(yd)
        ref = oracle_lib.q4k_gemv(x, w, K, N).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), k


@pytest.mark.parametrize("K,N", [(4096, 512), (14336, 64), (768, 100), (4096, 8200)])
def test_integer_inputs_bit_exact(oracle_lib, K, N):
    """d = dmin = 1, x in {-1, 0, 1}: all partial sums are integers below
    2^24, so any summation order is exact and the GPU equals the oracle."""
    w = synth.q4k_integer_weights(N, K, config=14)
    x = synth.integer_activations(K, config=14)
    y = run_gemv(x, w, K, N)
    ref = oracle_lib.q4k_gemv(x, w, K, N)
    assert np.all(ref == np.round(ref))
    assert np.array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("K,N", [(4096, 8200), (4096, 14341), (512, 70001), (2048, 33000)])
def test_persistent_walk(oracle_lib, K, N):
    """More row groups than resident workgroups: each workgroup walks several
    units with the next unit's tile prefetched (ragged last unit, one
    workgroup with a shorter walk, exact and uneven unit counts)."""
    w = synth.q4k_weights(N, K, config=19, copy=K + N)
    x = synth.activations(K, config=19, copy=K + N)
    y = run_gemv(x, w, K, N)
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what=f"K={K} N={N}")


def test_zero_activation_exact_zero():
    K, N = 4096, 256
    w = synth.q4k_weights(N, K, config=15)
    y = run_gemv(np.zeros(K, np.float32), w, K, N)
    assert np.all(y == 0.0)


def test_deterministic():
    K, N = 4096, 1024
    w = synth.q4k_weights(N, K, config=16)
    x = synth.activations(K, config=16)
    a = run_gemv(x, w, K, N)
    b = run_gemv(x, w, K, N)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_many_rows_sampled(oracle_lib):
    """2^20 rows of one block (151 MB of weights): sampled rows against the
    oracle run on just those rows."""
    K, N = 256, 1 << 20
    w = synth.q4k_weights(N, K, config=17)
    x = synth.activations(K, config=17)
    y = run_gemv(x, w, K, N)
    rows = np.random.default_rng(4).choice(N, 2000, replace=False)
    rows = np.concatenate([rows, [0, N - 1]])
    ref = oracle_lib.q4k_gemv(x, w[rows], K, len(rows))
    assert_parity(y[rows], ref, what="sampled rows")


def test_long_rows(oracle_lib):
    """input_dim = 65536 (256 blocks per row)."""
    K, N = 65536, 40
    w = synth.q4k_weights(N, K, config=18)
    x = synth.activations(K, config=18)
    y = run_gemv(x, w, K, N)
    assert_parity(y, oracle_lib.q4k_gemv(x, w, K, N), what="K=65536")


def test_rejects_bad_input_dim_and_leaves_y_untouched():
    x = torch.zeros(4000, dtype=torch.float32, device="cuda:0")
    w = torch.zeros(144 * 16, dtype=torch.uint8, device="cuda:0")
    buf, y = out_with_canary(8)
    for K in (255, 257, 4000):
        with pytest.raises(ValueError):
            binding.q4k_gemv(x, w, K, 8, y)
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(buf)))


def test_rejects_misaligned_weights():
    x = torch.zeros(256, dtype=torch.float32, device="cuda:0")
    w = torch.zeros(144 * 4 + 4, dtype=torch.uint8, device="cuda:0")
    buf, y = out_with_canary(4)
    with pytest.raises(ValueError):
        binding.q4k_gemv(x, w[4:], 256, 4, y)
