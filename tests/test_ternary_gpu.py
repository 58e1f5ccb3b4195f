"""Ternary (BitNet b1.58) GEMV on the GPU against the CPU oracle.

The ternary page's test asks for exact equality on the codes-dot and a
tolerance only for summation order: integer-valued and one-hot activations
must give bit-equal codes-dots; N(0,1) activations meet the 1e-4 bar.
"""
import numpy as np
import pytest
import torch

from q4_packed_weight_amd import binding, synth
from gpu_util import DEV, canary_intact, dev, host, out_with_canary
from tolerance import assert_parity

pytestmark = pytest.mark.gpu


def run(x, codes, K, N, scale=None, x_offset=0):
    xd = dev(np.concatenate([np.zeros(x_offset, np.float32), x]))[x_offset:] if x_offset else dev(x)
    cd = dev(codes)
    buf, y = out_with_canary(N)
    if scale is None:
        binding.ternary_gemv_codes(xd, cd, K, N, y)
    else:
        binding.ternary_gemv(xd, cd, scale, K, N, y)
    out = host(y)
    assert canary_intact(buf, N)
    return out


# fast path (K % 64 == 0) and generic path (K % 64 != 0), ragged rows; the
# fast path's 1, 2 and 4 rows per lane (output_dim below 4096, from 4096,
# from 12288 or from 8192 with input_dim from 12288)
SHAPES = [(64, 1), (128, 5), (1024, 333), (4096, 4096), (4160, 77), (4100, 7),
          (4, 3), (12, 65), (14336, 100), (65536, 9), (2048, 4100), (1024, 12300),
          (12352, 8195), (4096, 2050)]


@pytest.mark.parametrize("K,N", SHAPES)
def test_codes_dot_parity(oracle_lib, K, N):
    codes, _ = synth.ternary_codes(N, K, config=20, copy=K)
    x = synth.activations(K, config=20, copy=K)
    t = run(x, codes, K, N)
    assert_parity(t, oracle_lib.ternary_gemv_codes(x, codes, K, N), what=f"K={K} N={N}")


def test_full_config_with_scale(oracle_lib):
    K = N = 4096
    codes, _ = synth.ternary_codes(N, K)
    x = synth.activations(K, config=synth.C5_TERNARY)
    scale = synth.ternary_scale()
    y = run(x, codes, K, N, scale=scale)
    assert_parity(y, oracle_lib.ternary_gemv(x, codes, scale, K, N), what="c5")


@pytest.mark.parametrize("K,N", [(4096, 300), (4100, 50), (1024, 64)])
@pytest.mark.parametrize("code3", [False, True])
def test_codes_dot_exact_on_integer_activations(oracle_lib, K, N, code3):
    codes, u = synth.ternary_codes(N, K, config=21, copy=K, allow_code3=code3)
    x = synth.integer_activations(K, lo=-8, hi=8, config=21, copy=K)
    t = run(x, codes, K, N)
    ref = oracle_lib.ternary_gemv_codes(x, codes, K, N)
    assert np.array_equal(t.astype(np.float64), ref)


def test_codes_dot_one_hot_exact():
    K, N = 256, 12
    codes, u = synth.ternary_codes(N, K, config=22, allow_code3=True)
    cd = dev(codes)
    buf, y = out_with_canary(N)
    for k in range(K):
        x = torch.zeros(K, dtype=torch.float32, device=DEV)
        x[k] = 1.0
        binding.ternary_gemv_codes(x, cd, K, N, y)
        assert np.array_equal(host(y), u[:, k].astype(np.float32) - 1.0), k


def test_scale_is_applied_after_the_dot():
    K, N = 4096, 512
    codes, _ = synth.ternary_codes(N, K, config=23)
    x = synth.activations(K, config=23)
    scale = np.float32(1.7384)
    t = run(x, codes, K, N)
    y = run(x, codes, K, N, scale=float(scale))
    assert np.array_equal(y, (scale * t).astype(np.float32))
    y1 = run(x, codes, K, N, scale=1.0)
    assert np.array_equal(y1, t)


def test_unaligned_activations_use_generic_path(oracle_lib):
    K, N = 4096, 100
    codes, _ = synth.ternary_codes(N, K, config=24)
    x = synth.activations(K, config=24)
    t = run(x, codes, K, N, x_offset=1)
    assert_parity(t, oracle_lib.ternary_gemv_codes(x, codes, K, N), what="unaligned x")


def test_rejects_bad_input_dim():
    x = torch.zeros(16, dtype=torch.float32, device=DEV)
    c = torch.zeros(64, dtype=torch.uint8, device=DEV)
    buf, y = out_with_canary(4)
    for K in (3, 5, 6):
        with pytest.raises(ValueError):
            binding.ternary_gemv_codes(x, c, K, 4, y)
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(buf)))
