"""Pins of the oracle's MX-scaled GEMM: a hand-worked case, the dequantised
operands multiplied by numpy (decoded with torch's own float8 decoders, not
the oracle's), the grouped form against the dense one per group, and scale
equivariance."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_gemm_worked.json")


def _expand(rows):
    out = []
    for r in rows:
        vals = []
        for i in range(0, len(r), 2):
            vals += [int(r[i], 16)] * r[i + 1]
        out.append(vals)
    return np.array(out, np.uint8)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_worked(case):
    c, _ = oracle.mx_gemm(_expand(case["qa"]), np.array(case["sa"], np.uint8), _expand(case["qb"]),
                          np.array(case["sb"], np.uint8))
    assert np.array_equal(c, np.array(case["c"])), case["derivation"]


def _dequant_torch(q, s):
    v = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sc = torch.from_numpy(s).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    return v * np.repeat(sc, 32, axis=1)


def _random_operands(rows, k, seed, nan_free=True):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(rows, k), dtype=np.uint8)
    if nan_free:
        q[(q & 0x7F) == 0x7F] = 0x7E
    s = rng.integers(110, 145, size=(rows, k // 32), dtype=np.uint8)
    return q, s


@pytest.mark.parametrize("m,n,k", [(7, 5, 32), (33, 17, 96), (64, 48, 256)])
def test_matches_numpy_matmul_of_torch_dequantised(m, n, k):
    qa, sa = _random_operands(m, k, 1)
    qb, sb = _random_operands(n, k, 2)
    c, absum = oracle.mx_gemm(qa, sa, qb, sb)
    a = _dequant_torch(qa, sa)
    b = _dequant_torch(qb, sb)
    want = a @ b.T
    assert np.allclose(c, want, rtol=1e-12, atol=1e-12 * (np.abs(a) @ np.abs(b).T).max())
    assert np.allclose(absum, np.abs(a) @ np.abs(b).T, rtol=1e-12)


def test_grouped_is_dense_per_group_and_clamps():
    k, n = 64, 24
    qa, sa = _random_operands(100, k, 3)
    qb = np.stack([_random_operands(n, k, 10 + g)[0] for g in range(3)])
    sb = np.stack([_random_operands(n, k, 10 + g)[1] for g in range(3)])
    for ends in ([30, 30, 100], [50, 40, 90], [-3, 60, 200]):
        c, _ = oracle.mx_gemm_grouped(qa, sa, qb, sb, np.array(ends, np.int32))
        lo = 0
        for g, e in enumerate(ends):
            hi = min(max(e, lo), 100)
            ref, _ = oracle.mx_gemm(qa[lo:hi], sa[lo:hi], qb[g], sb[g])
            assert np.array_equal(c[lo:hi], ref)
            lo = hi
        assert np.all(np.isnan(c[lo:]))


def test_scale_equivariance_and_nan():
    qa, sa = _random_operands(16, 128, 4)
    qb, sb = _random_operands(8, 128, 5)
    c, _ = oracle.mx_gemm(qa, sa, qb, sb)
    sa2 = sa.copy()
    sa2[3] += 1                      # every block of row 3 doubled
    c2, _ = oracle.mx_gemm(qa, sa2, qb, sb)
    assert np.array_equal(c2[3], 2 * c[3]) and np.array_equal(np.delete(c2, 3, 0), np.delete(c, 3, 0))
    sb2 = sb.copy()
    sb2[2, 1] = 0xFF                 # a NaN scale poisons column 2
    c3, _ = oracle.mx_gemm(qa, sa, qb, sb2)
    assert np.all(np.isnan(c3[:, 2])) and not np.any(np.isnan(np.delete(c3, 2, 1)))
