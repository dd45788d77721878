"""Seeded synthetic inputs for the MXFP8 cast and the blocked scale layout.

This module only draws numbers and rounds them to bf16; it holds none of the
cast's arithmetic, so the CPU oracle and the GPU library can both be fed from
it.  bf16 tensors are returned as numpy uint16 bit patterns (row-major), scale
tensors as uint8.

The workloads follow the shapes on the pages:
  * square matrices with M, K, N from 1024 to 16384 ("triton kernel to cast to
    mx across dim0 and dim1", Summary);
  * MoE activations (16640, 5120) split into 4 groups along M and expert
    weights (G, 8192, 5120) ("[mxfp8 moe training] add compile support",
    microbenchmark table and perf analysis);
  * e8m0 scale tensors (5120, 512), (8192, 4096), (2048, 4096) with groups
    along K ("... scale blocked format kernel for groups along K", Benchmarks).
No dataset is involved; every value is drawn from numpy's PCG64 generator.
"""
from __future__ import annotations

import numpy as np

CHUNK_ROWS = 1024


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, rounded to nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(shape, seed, std=1.0) -> np.ndarray:
    """N(0, std^2) bf16 bits, drawn in row chunks to bound host memory."""
    rng = np.random.default_rng(seed)
    out = np.empty(shape, np.uint16)
    flat = out.reshape(-1, shape[-1])
    for r0 in range(0, flat.shape[0], CHUNK_ROWS):
        r1 = min(r0 + CHUNK_ROWS, flat.shape[0])
        a = rng.standard_normal((r1 - r0, shape[-1]), dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        flat[r0:r1] = bf16_bits(a)
    return out


# --------------------------------------------------------------------------
# 1024 x 1024 with special tiles (correctness case the oracle finishes fast)
# --------------------------------------------------------------------------
ZERO_TILE = (64, 128)        # (row, col) of a 32x32 all-zero tile
DENORMAL_TILE = (320, 512)   # 32x32 tile whose blocks all have amax 2^-130
OUTLIER_TILE = (704, 800)    # 32x32 tile with +-1e4 on its diagonal


def square_with_special_tiles(n: int = 1024, seed: int = 1) -> np.ndarray:
    """N(0,1) (n, n) plus three 32x32 tiles aligned to block boundaries, so
    that both the row blocks and the column blocks through them see the same
    kind of block: all zeros; bf16 denormals with amax exactly 2^-130 (the
    diagonal holds +-2^-130, the rest is clip(z/4, -1, 1) * 2^-130); N(0,1)
    with alternating +-1e4 outliers on the diagonal."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, n), dtype=np.float32)
    r, c = ZERO_TILE
    x[r:r + 32, c:c + 32] = 0.0
    r, c = DENORMAL_TILE
    t = np.clip(rng.standard_normal((32, 32), dtype=np.float32) / 4, -1, 1) * np.float32(2.0 ** -130)
    idx = np.arange(32)
    t[idx, idx] = np.where(idx % 2 == 0, 1.0, -1.0).astype(np.float32) * np.float32(2.0 ** -130)
    x[r:r + 32, c:c + 32] = t
    r, c = OUTLIER_TILE
    o = rng.standard_normal((32, 32), dtype=np.float32)
    o[idx, idx] = np.where(idx % 2 == 0, 1e4, -1e4).astype(np.float32)
    x[r:r + 32, c:c + 32] = o
    return bf16_bits(x)


# --------------------------------------------------------------------------
# 16384 x 16384 heavy-tailed rows (the headline cast workload)
# --------------------------------------------------------------------------
def heavy_tailed_rows(rows: int = 16384, cols: int = 16384, seed: int = 2,
                      log_std: float = 2.0) -> np.ndarray:
    """X[r, :] = N(0,1) * exp(z_r), z_r ~ N(0, log_std^2) per row, so that
    column blocks mix rows of very different magnitude."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(rows).astype(np.float32) * np.float32(log_std)
    row_scale = np.exp(z).astype(np.float32)
    out = np.empty((rows, cols), np.uint16)
    for r0 in range(0, rows, CHUNK_ROWS):
        r1 = min(r0 + CHUNK_ROWS, rows)
        a = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        a *= row_scale[r0:r1, None]
        out[r0:r1] = bf16_bits(a)
    return out


# --------------------------------------------------------------------------
# MoE activations with 4 groups along M
# --------------------------------------------------------------------------
def group_ends(total: int, groups: int, unit: int, rng) -> np.ndarray:
    """Cumulative END offsets of `groups` groups whose sizes are positive
    multiples of `unit` summing to `total` (groups - 1 distinct cut points)."""
    slots = total // unit
    cuts = np.sort(rng.choice(np.arange(1, slots), size=groups - 1, replace=False))
    return np.concatenate([cuts * unit, [total]]).astype(np.int32)


def moe_activations(rows: int = 16640, cols: int = 5120, groups: int = 4, seed: int = 3):
    """(bf16 bits (rows, cols) N(0,1), int32 group END offsets along M).
    Group sizes are multiples of 32 rows."""
    rng = np.random.default_rng(seed)
    ends = group_ends(rows, groups, 32, rng)
    x = normal_bf16((rows, cols), seed=[seed, 1])
    return x, ends


# --------------------------------------------------------------------------
# e8m0 scale tensors with K groups
# --------------------------------------------------------------------------
K_GROUP_SHAPES = ((5120, 512), (8192, 4096), (2048, 4096))


def k_group_scales(shape, groups: int = 4, seed: int = 4):
    """(uint8 scales uniform in [100, 140], int32 END offsets in scale
    columns; groups are multiples of 4 columns)."""
    r, c = shape
    rng = np.random.default_rng([seed, r, c])
    s = rng.integers(100, 141, size=(r, c), dtype=np.uint8)
    ends = group_ends(c, groups, 4, rng)
    return s, ends


# --------------------------------------------------------------------------
# 3D expert weights
# --------------------------------------------------------------------------
def expert_weight(e: int, n: int = 8192, k: int = 5120, seed: int = 5) -> np.ndarray:
    """Expert e's (n, k) weights: N(0, 0.02^2), with a seeded 1% of the
    elements multiplied by 100.  Each expert has its own stream, so experts
    can be drawn one at a time."""
    rng = np.random.default_rng([seed, e])
    out = np.empty((n, k), np.uint16)
    for r0 in range(0, n, CHUNK_ROWS):
        r1 = min(r0 + CHUNK_ROWS, n)
        a = rng.standard_normal((r1 - r0, k), dtype=np.float32) * np.float32(0.02)
        mask = rng.random((r1 - r0, k), dtype=np.float32) < np.float32(0.01)
        a[mask] *= np.float32(100.0)
        out[r0:r1] = bf16_bits(a)
    return out


def expert_weights(experts: int = 16, n: int = 8192, k: int = 5120, seed: int = 5) -> np.ndarray:
    out = np.empty((experts, n, k), np.uint16)
    for e in range(experts):
        out[e] = expert_weight(e, n, k, seed)
    return out


# --------------------------------------------------------------------------
# Small mixed inputs for edge cases
# --------------------------------------------------------------------------
def special_values_bf16(shape, seed: int, p_special: float = 0.02) -> np.ndarray:
    """N(0,1) with exponents spread over the whole bf16 range, and a fraction
    p_special of entries replaced by one of: +-0, +-Inf, NaN (either sign),
    bf16 denormals, the largest finite bf16."""
    if shape[-1] % 32:
        raise ValueError("the last dimension must be a multiple of 32")
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32)
    block_exp = rng.integers(-140, 120, size=tuple(shape[:-1]) + (shape[-1] // 32,))
    e = np.repeat(block_exp, 32, axis=-1)
    a = (a.astype(np.float64) * np.exp2(e.astype(np.float64))).astype(np.float32)
    bits = bf16_bits(np.nan_to_num(a, nan=0.0, posinf=0.0, neginf=0.0))
    specials = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x8005,
                         0x007F, 0x7F7F, 0xFF7F], dtype=np.uint16)
    pick = rng.random(shape) < p_special
    bits[pick] = specials[rng.integers(0, specials.size, size=int(pick.sum()))]
    return bits
