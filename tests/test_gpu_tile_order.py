"""GPU parity of the casts at shapes whose XCD pieces start a multiple of
4 KiB apart in the col-major output (32768 rows: 256 row tiles; with one or
two column tiles a piece is 32 or 64 whole row tiles), where the host has
each XCD start its piece at a point of its own.  Every output byte of the
blocked-scale, plain, M-grouped and both-grouped casts against the oracle."""
import numpy as np
import pytest
import torch

import fp8_precision_quantization_amd as mx
from fp8_precision_quantization_amd import workloads
from tests import test_gpu_grouped_blocked as gb_t
from tests import test_gpu_mgrouped as mg_t
from tests.gpu_util import assert_bytes_equal, device, host, to_dev_bf16

pytestmark = pytest.mark.gpu

SHAPES = [(32768, 256), (32768, 512)]


def _input(shape):
    return workloads.special_values_bf16(shape, seed=[71, shape[0], shape[1]], p_special=0.0005)


@pytest.mark.parametrize("shape", SHAPES, ids=["%dx%d" % s for s in SHAPES])
def test_rotated_blocked_and_plain(oracle_mod, shape):
    dev = device()
    bits = _input(shape)
    x = to_dev_bf16(bits, dev)
    r_q0, r_s0 = oracle_mod.cast_dim0(bits)
    r_q1, r_s1 = oracle_mod.cast_dim1(bits)
    q0, b0, q1, b1 = mx.mx_cast_dim0_dim1_blocked(x, raw=True)
    p0, s0, p1, s1 = mx.mx_cast_dim0_dim1(x, raw=True)
    torch.cuda.synchronize(dev)
    what = "%dx%d" % shape
    assert_bytes_equal(host(q0), r_q0, what + " blocked q_row")
    assert_bytes_equal(host(q1), r_q1, what + " blocked q_col")
    assert_bytes_equal(host(b0).reshape(-1), oracle_mod.to_blocked(r_s0), what + " blocked s_row")
    assert_bytes_equal(host(b1).reshape(-1), oracle_mod.to_blocked(r_s1), what + " blocked s_col")
    assert_bytes_equal(host(p0), r_q0, what + " plain q_row")
    assert_bytes_equal(host(s0), r_s0, what + " plain s_row")
    assert_bytes_equal(host(p1), r_q1, what + " plain q_col")
    assert_bytes_equal(host(s1), r_s1, what + " plain s_col")


@pytest.mark.parametrize("shape", SHAPES, ids=["%dx%d" % s for s in SHAPES])
def test_rotated_grouped(oracle_mod, shape):
    dev = device()
    bits = _input(shape)
    ends = [1440, 9984, 9984, 30016, 32768]
    mg_t.check(oracle_mod, bits, ends, dev, "M-grouped %dx%d" % shape)
    gb_t.check(oracle_mod, bits, ends, dev, "both grouped %dx%d" % shape)
