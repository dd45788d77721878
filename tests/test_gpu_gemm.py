"""GPU parity of the MX-scaled GEMM (dense and grouped along M) with the
oracle's fp64 definition.  Operands are MX casts made by the ORACLE from
seeded bf16 data (or seeded random codes and scales), uploaded as they are.

Tolerance, from the arithmetic: the block-scaled MFMA sums the 64 products
of a K step with less than binary32 precision -- an in-bounds probe on
MI355X measured at most 3.4e-4 of the step's largest product and 1.7e-4 of
the sum of the step's |products| -- and the steps accumulate in binary32.
So |C - C_exact| <= 2^-10 * sum_k |A(m,k) B(n,k)| (about 6x the measured
worst case), plus half a bf16 ulp of |C| when C is stored as bf16."""
import numpy as np
import pytest
import torch

import fp8_precision_quantization_amd as mx
from fp8_precision_quantization_amd import workloads
from tests.gpu_util import device, to_dev_u8

pytestmark = pytest.mark.gpu

REL_SUM = 2.0 ** -10


def _codes_scales(rows, k, seed, lo=118, hi=136):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(rows, k), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E
    s = rng.integers(lo, hi, size=(rows, k // 32), dtype=np.uint8)
    return q, s


def _cast_operand(oracle_mod, rows, k, seed):
    return oracle_mod.cast_dim0(workloads.heavy_tailed_rows(rows, k, seed=seed))


def _check(got, want, absum, bf16, what):
    got = got.float().cpu().numpy().astype(np.float64)
    tol = REL_SUM * absum + (np.abs(want) * 2.0 ** -8 if bf16 else 0.0) + 1e-30
    err = np.abs(got - want)
    bad = err > tol
    assert not bad.any(), "%s: %d of %d outside tolerance, worst err/tol %.3g" % (
        what, int(bad.sum()), bad.size, float((err / tol).max()))
    return float((err / (absum + 1e-300)).max())


@pytest.mark.parametrize("m,n,k", [(128, 128, 64), (256, 384, 128), (200, 136, 96), (1, 1, 32),
                                   (300, 260, 5120), (64, 1000, 2080)])
@pytest.mark.parametrize("bf16", [False, True])
def test_gemm_random_operands(oracle_mod, m, n, k, bf16):
    dev = device()
    qa, sa = _codes_scales(m, k, m + k)
    qb, sb = _codes_scales(n, k, n + 2 * k)
    want, absum = oracle_mod.mx_gemm(qa, sa, qb, sb)
    got = mx.mx_gemm_mxfp8(to_dev_u8(qa, dev), to_dev_u8(sa, dev), to_dev_u8(qb, dev), to_dev_u8(sb, dev),
                           out_dtype=torch.bfloat16 if bf16 else torch.float32)
    _check(got, want, absum, bf16, "gemm %dx%dx%d" % (m, n, k))


def test_gemm_of_casts(oracle_mod):
    """Operands as the dim0 cast makes them from bf16 data (heavy-tailed rows:
    scales over many binades, zero and denormal-free)."""
    dev = device()
    qa, sa = _cast_operand(oracle_mod, 384, 1024, 3)
    qb, sb = _cast_operand(oracle_mod, 256, 1024, 4)
    want, absum = oracle_mod.mx_gemm(qa, sa, qb, sb)
    got = mx.mx_gemm_mxfp8(to_dev_u8(qa, dev), to_dev_u8(sa, dev), to_dev_u8(qb, dev), to_dev_u8(sb, dev),
                           out_dtype=torch.float32)
    worst = _check(got, want, absum, False, "gemm of casts")
    assert worst < 2.0 ** -11


def test_gemm_zero_k_and_empty():
    dev = device()
    z = torch.empty((0,), dtype=torch.uint8, device=dev)
    c = torch.full((4, 3), 7.0, device=dev)
    mx.mx_gemm_mxfp8(z.view(4, 0), z.view(4, 0), z.view(3, 0), z.view(3, 0), out_dtype=torch.float32, out=c)
    torch.cuda.synchronize(dev)
    assert torch.all(c == 0)
    e = mx.mx_gemm_mxfp8(z.view(0, 0), z.view(0, 0), z.view(3, 0), z.view(3, 0))
    assert tuple(e.shape) == (0, 3)


GROUP_CASES = [("one", 500, [500]), ("four", 1000, [100, 100, 613, 1000]), ("ragged", 777, [1, 130, 700, 777]),
               ("malformed", 600, [300, 200, 900, 600]), ("short", 600, [128, 300])]


@pytest.mark.parametrize("name,m,ends", GROUP_CASES, ids=[c[0] for c in GROUP_CASES])
def test_grouped_gemm(oracle_mod, name, m, ends):
    dev = device()
    n, k, g = 192, 256, len(ends)
    qa, sa = _codes_scales(m, k, 7)
    qb = np.stack([_codes_scales(n, k, 20 + i)[0] for i in range(g)])
    sb = np.stack([_codes_scales(n, k, 20 + i)[1] for i in range(g)])
    want, absum = oracle_mod.mx_gemm_grouped(qa, sa, qb, sb, np.asarray(ends, np.int32))
    out = torch.full((m, n), 12345.0, device=dev)
    mx.mx_grouped_gemm_mxfp8(to_dev_u8(qa, dev), to_dev_u8(sa, dev), to_dev_u8(qb, dev), to_dev_u8(sb, dev),
                             torch.tensor(ends, dtype=torch.int32, device=dev), out_dtype=torch.float32, out=out)
    torch.cuda.synchronize(dev)
    rows = ~np.isnan(want[:, 0])
    _check(out[torch.from_numpy(rows).to(dev)], want[rows], absum[rows], False, "grouped " + name)
    # rows past the last (clamped) end are left as they were
    assert torch.all(out[torch.from_numpy(~rows).to(dev)] == 12345.0)


def test_gemm_full_size_sampled(oracle_mod):
    """The benchmark's dense shape, M = 16640, N = 8192, K = 5120, in its launch
    configuration; 24 sampled rows compared against the oracle in full."""
    dev = device()
    m, n, k = 16640, 8192, 5120
    qa, sa = _codes_scales(m, k, 101)
    qb, sb = _codes_scales(n, k, 102)
    got = mx.mx_gemm_mxfp8(to_dev_u8(qa, dev), to_dev_u8(sa, dev), to_dev_u8(qb, dev), to_dev_u8(sb, dev))
    rows = np.sort(np.random.default_rng(5).choice(m, 24, replace=False))
    want, absum = oracle_mod.mx_gemm(qa[rows], sa[rows], qb, sb)
    _check(got[torch.from_numpy(rows).to(dev)], want, absum, True, "16640x8192x5120 sampled")
