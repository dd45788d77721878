"""GPU parity of the dense MX GEMM on seeded random shapes: M and N any size
from 1 to 700 (ragged 256-row and 256-column tiles, rows of C that are whole
16-byte chunks and rows that are not, which take the per-element stores),
K any multiple of 32 up to 1536, bf16 and binary32 output.  Same operands and
tolerance as the fixed-shape GEMM tests."""
import numpy as np
import pytest
import torch

import fp8_precision_quantization_amd as mx
from tests.gpu_util import device, to_dev_u8
from tests.test_gpu_gemm import _blocked, _check, _codes_scales

pytestmark = pytest.mark.gpu


def _case(i):
    rng = np.random.default_rng([311, i])
    m = int(rng.integers(1, 701))
    n = int(rng.integers(1, 701))
    if i % 3 == 0:
        n = -(-n // 8) * 8   # whole 16-byte bf16 rows: the staged epilogue
    k = 32 * int(rng.integers(1, 49))
    return m, n, k, i % 2 == 0


@pytest.mark.parametrize("i", list(range(12)))
def test_gemm_random_shape(oracle_mod, i):
    m, n, k, bf16 = _case(i)
    dev = device()
    qa, sa = _codes_scales(m, k, [312, i])
    qb, sb = _codes_scales(n, k, [313, i])
    want, absum = oracle_mod.mx_gemm(qa, sa, qb, sb)
    got = mx.mx_gemm_mxfp8(to_dev_u8(qa, dev), _blocked(oracle_mod, sa, dev), to_dev_u8(qb, dev),
                           _blocked(oracle_mod, sb, dev), out_dtype=torch.bfloat16 if bf16 else torch.float32)
    _check(got, want, absum, bf16, "case %d: gemm %dx%dx%d bf16=%s" % (i, m, n, k, bf16))
