"""Seeded synthetic inputs for the Q4_K, Q4_0, Q6_K and ternary products.

This module only draws random numbers and lays them out in the input
formats; it holds none of the products' arithmetic.  Both the GPU path's
tests/benchmark and the CPU oracle's tests take their inputs from here.

Recipe (one numpy Generator per (config, copy, role); role 0 = weights,
role 1 = activations):

Q4_K matrix with R = rows * (K / 256) super-blocks, drawn in this order:
  1. d    = float16(|standard_normal(R)| / 64)       (round-to-nearest-even)
  2. dmin = float16(|standard_normal(R)| / 64)
  3. the 12 packed scale bytes: integers(0, 256, (R, 12)) -- uniform bytes
     are uniform independent 6-bit scales and mins, since the packing uses
     each of the 96 bits exactly once
  4. qs: integers(0, 256, (R, 128)) -- uniform nibbles
and each block is d | dmin | scales | qs (144 bytes), blocks row-major.
Activations: standard_normal(K) as float32 (or (M, K) for a token batch).

Q4_0 matrix with R = rows * (K / 32) blocks: d = float16(|standard_normal(R)|
/ 64), then qs = integers(0, 256, (R, 16)); each block is d | qs (18 bytes),
blocks row-major.

Q6_K matrix with R = rows * (K / 256) blocks: d = float16(|standard_normal(R)|
/ 64), then ql = integers(0, 256, (R, 128)), qh = integers(0, 256, (R, 64))
(uniform 6-bit codes), scales = integers(-128, 128, (R, 16)) as int8; each
block is ql | qh | scales | d (210 bytes), blocks row-major.

Ternary matrix: codes u = integers(0, 3, (N, K)) (so u - 1 is uniform over
{-1, 0, 1}), four per byte as u0 | u1<<2 | u2<<4 | u3<<6, rows of K/4 bytes;
one float32 per-tensor scale uniform(0.5, 2).

These shapes and distributions are the workloads the Q4_K page benchmarks
("LLM-typical" inputDim x outputDim, batch 1) and the configurations built
on them; no dataset is involved.
"""
import numpy as np

SEED = 2026
BLOCK_BYTES = 144
QK = 256

Q40_BLOCK_BYTES = 18
Q40_QK = 32
Q6K_BLOCK_BYTES = 210

# Configuration ids used in seeds.
C1_Q4K_1K, C2_Q4K_4K, C3_FFN, C4_PREFILL, C5_TERNARY = 1, 2, 3, 4, 5
Q40_4K = 6
Q6K_4K = 7
ROLE_W, ROLE_X = 0, 1


def rng(config, copy=0, role=ROLE_W, extra=0):
    return np.random.default_rng((SEED, int(config), int(copy), int(role),
                                  int(extra)))


def q4k_blocks_from_fields(d_f16, dmin_f16, scales12, qs128):
    """Assemble [R, 144] block bytes from already-drawn fields."""
    R = d_f16.shape[0]
    out = np.empty((R, BLOCK_BYTES), np.uint8)
    out[:, 0:2] = np.ascontiguousarray(d_f16, np.float16).view(np.uint8).reshape(R, 2)
    out[:, 2:4] = np.ascontiguousarray(dmin_f16, np.float16).view(np.uint8).reshape(R, 2)
    out[:, 4:16] = scales12
    out[:, 16:144] = qs128
    return out


def q4k_weights(n_rows, input_dim, config=C2_Q4K_4K, copy=0, extra=0):
    """Random Q4_K matrix as uint8 [n_rows, (input_dim/256)*144]."""
    assert input_dim % QK == 0
    nb = input_dim // QK
    R = n_rows * nb
    g = rng(config, copy, ROLE_W, extra)
    d = (np.abs(g.standard_normal(R)) / 64).astype(np.float16)
    dmin = (np.abs(g.standard_normal(R)) / 64).astype(np.float16)
    scales = g.integers(0, 256, (R, 12), dtype=np.uint8)
    qs = g.integers(0, 256, (R, 128), dtype=np.uint8)
    return q4k_blocks_from_fields(d, dmin, scales, qs).reshape(n_rows, nb * BLOCK_BYTES)


def q4_0_blocks_from_fields(d_f16, qs16):
    """Assemble [R, 18] Q4_0 block bytes from already-drawn fields."""
    R = d_f16.shape[0]
    out = np.empty((R, Q40_BLOCK_BYTES), np.uint8)
    out[:, 0:2] = np.ascontiguousarray(d_f16, np.float16).view(np.uint8).reshape(R, 2)
    out[:, 2:18] = qs16
    return out


def q4_0_weights(n_rows, input_dim, config=Q40_4K, copy=0, extra=0):
    """Random Q4_0 matrix as uint8 [n_rows, (input_dim/32)*18]."""
    assert input_dim % Q40_QK == 0
    nb = input_dim // Q40_QK
    R = n_rows * nb
    g = rng(config, copy, ROLE_W, extra)
    d = (np.abs(g.standard_normal(R)) / 64).astype(np.float16)
    qs = g.integers(0, 256, (R, 16), dtype=np.uint8)
    return q4_0_blocks_from_fields(d, qs).reshape(n_rows, nb * Q40_BLOCK_BYTES)


def q6k_blocks_from_fields(ql128, qh64, scales16, d_f16):
    """Assemble [R, 210] Q6_K block bytes from already-drawn fields."""
    R = ql128.shape[0]
    out = np.empty((R, Q6K_BLOCK_BYTES), np.uint8)
    out[:, 0:128] = ql128
    out[:, 128:192] = qh64
    out[:, 192:208] = np.ascontiguousarray(scales16, np.int8).view(np.uint8)
    out[:, 208:210] = np.ascontiguousarray(d_f16, np.float16).view(np.uint8).reshape(R, 2)
    return out


def q6k_weights(n_rows, input_dim, config=Q6K_4K, copy=0, extra=0):
    """Random Q6_K matrix as uint8 [n_rows, (input_dim/256)*210]."""
    assert input_dim % QK == 0
    nb = input_dim // QK
    R = n_rows * nb
    g = rng(config, copy, ROLE_W, extra)
    d = (np.abs(g.standard_normal(R)) / 64).astype(np.float16)
    ql = g.integers(0, 256, (R, 128), dtype=np.uint8)
    qh = g.integers(0, 256, (R, 64), dtype=np.uint8)
    sc = g.integers(-128, 128, (R, 16)).astype(np.int8)
    return q6k_blocks_from_fields(ql, qh, sc, d).reshape(n_rows, nb * Q6K_BLOCK_BYTES)


def activations(input_dim, n_tokens=None, config=C2_Q4K_4K, copy=0, extra=0):
    """standard_normal float32 of shape [input_dim] or [n_tokens, input_dim]."""
    g = rng(config, copy, ROLE_X, extra)
    shape = (input_dim,) if n_tokens is None else (n_tokens, input_dim)
    return g.standard_normal(shape, dtype=np.float32)


def ternary_codes(n_rows, input_dim, config=C5_TERNARY, copy=0, extra=0,
                  allow_code3=False):
    """Packed ternary matrix uint8 [n_rows, input_dim/4] and the unpacked
    field values u (0..2, or 0..3 if allow_code3) for test bookkeeping."""
    assert input_dim % 4 == 0
    g = rng(config, copy, ROLE_W, extra)
    hi = 4 if allow_code3 else 3
    u = g.integers(0, hi, (n_rows, input_dim), dtype=np.uint8)
    return pack_2bit(u), u


def pack_2bit(u):
    """Four 2-bit fields per byte, field i of a group of four at bits 2i."""
    n, k = u.shape
    g = u.reshape(n, k // 4, 4).astype(np.uint8)
    return (g[:, :, 0] | (g[:, :, 1] << 2) | (g[:, :, 2] << 4) |
            (g[:, :, 3] << 6)).astype(np.uint8)


def ternary_scale(config=C5_TERNARY, copy=0, extra=0):
    g = rng(config, copy, ROLE_W, 1000 + extra)
    return np.float32(g.uniform(0.5, 2.0))


# ---------------------------------------------------------------------------
# Structured inputs for exactness checks.

def q4k_integer_weights(n_rows, input_dim, config=C2_Q4K_4K, copy=0, extra=0):
    """Blocks with d = dmin = 1.0 and random scales/mins/codes: every weight
    is an integer in [-63, 945]."""
    nb = input_dim // QK
    R = n_rows * nb
    g = rng(config, copy, ROLE_W, 500 + extra)
    one = np.ones(R, np.float16)
    scales = g.integers(0, 256, (R, 12), dtype=np.uint8)
    qs = g.integers(0, 256, (R, 128), dtype=np.uint8)
    return q4k_blocks_from_fields(one, one, scales, qs).reshape(n_rows, nb * BLOCK_BYTES)


def q4_0_integer_weights(n_rows, input_dim, config=Q40_4K, copy=0, extra=0):
    """Q4_0 blocks with d = 1.0 and random codes: every weight is an integer
    in [-8, 7]."""
    nb = input_dim // Q40_QK
    R = n_rows * nb
    g = rng(config, copy, ROLE_W, 500 + extra)
    qs = g.integers(0, 256, (R, 16), dtype=np.uint8)
    return q4_0_blocks_from_fields(np.ones(R, np.float16), qs).reshape(
        n_rows, nb * Q40_BLOCK_BYTES)


def q6k_integer_weights(n_rows, input_dim, config=Q6K_4K, copy=0, extra=0):
    """Q6_K blocks with d = 1.0, scales in {-1, 1} and random codes: every
    weight is an integer in [-32, 32]."""
    nb = input_dim // QK
    R = n_rows * nb
    g = rng(config, copy, ROLE_W, 500 + extra)
    ql = g.integers(0, 256, (R, 128), dtype=np.uint8)
    qh = g.integers(0, 256, (R, 64), dtype=np.uint8)
    sc = (2 * g.integers(0, 2, (R, 16)) - 1).astype(np.int8)
    return q6k_blocks_from_fields(ql, qh, sc, np.ones(R, np.float16)).reshape(
        n_rows, nb * Q6K_BLOCK_BYTES)


def integer_activations(input_dim, lo=-1, hi=1, n_tokens=None, config=C2_Q4K_4K,
                        copy=0, extra=0):
    g = rng(config, copy, ROLE_X, 500 + extra)
    shape = (input_dim,) if n_tokens is None else (n_tokens, input_dim)
    return g.integers(lo, hi + 1, shape).astype(np.float32)
