"""GPU parity of the MX casts: the HIP library (through the C ABI) against the
CPU oracle on the same seeded inputs, byte for byte (tolerance 0)."""
import numpy as np
import pytest
import torch

import fp8_precision_quantization_amd as mx
from fp8_precision_quantization_amd import workloads
from tests import sweep_blocks as sb
from tests.gpu_util import assert_bytes_equal, device, host, sentinel, to_dev_bf16

pytestmark = pytest.mark.gpu


def gpu_cast(bits, dev, dim0=True, dim1=True, fill=0xCD):
    r, c = bits.shape
    out = (sentinel((r, c), dev, fill) if dim0 else None,
           sentinel((r, c // 32), dev, fill) if dim0 else None,
           sentinel((c, r), dev, fill) if dim1 else None,
           sentinel((c, r // 32), dev, fill) if dim1 else None)
    res = mx.mx_cast_dim0_dim1(to_dev_bf16(bits, dev), dim0=dim0, dim1=dim1, out=out, raw=True)
    torch.cuda.synchronize(dev)
    return [None if t is None else host(t) for t in res]


def check_cast(oracle_mod, bits, dev, what, dim0=True, dim1=True):
    q0, s0, q1, s1 = gpu_cast(bits, dev, dim0, dim1)
    if dim0:
        r_q0, r_s0 = oracle_mod.cast_dim0(bits)
        assert_bytes_equal(q0, r_q0, what + " q_row")
        assert_bytes_equal(s0, r_s0, what + " s_row")
    if dim1:
        r_q1, r_s1 = oracle_mod.cast_dim1(bits)
        assert_bytes_equal(q1, r_q1, what + " q_col")
        assert_bytes_equal(s1, r_s1, what + " s_col")


def test_square_with_special_tiles(oracle_mod):
    """1024 x 1024 N(0,1) with all-zero, denormal (amax 2^-130) and 1e4
    outlier tiles, both directions, every output byte."""
    dev = device()
    check_cast(oracle_mod, workloads.square_with_special_tiles(1024, seed=1), dev, "1024^2")


SHAPES = [(32, 32), (32, 256), (64, 96), (96, 288), (128, 256), (160, 544), (256, 800),
          (416, 1056), (1024, 32), (32, 2080), (1568, 1056), (544, 3104), (2048, 64)]


@pytest.mark.parametrize("shape", SHAPES)
def test_shapes_finite(oracle_mod, shape):
    """Ragged row tiles (rows % 128 != 0) and column tiles (cols % 256 != 0),
    exponents spread over the whole bf16 range, no Inf/NaN."""
    dev = device()
    bits = workloads.special_values_bf16(shape, seed=shape[0] * 7 + shape[1], p_special=0.0)
    check_cast(oracle_mod, bits, dev, "finite %s" % (shape,))


@pytest.mark.parametrize("p_special", [0.0005, 0.01, 0.2])
def test_special_values(oracle_mod, p_special):
    """+-0, +-Inf, NaN of either sign, denormals and the largest finite bf16
    mixed in at several densities (waves with and without them)."""
    dev = device()
    bits = workloads.special_values_bf16((320, 544), seed=int(p_special * 1e4), p_special=p_special)
    check_cast(oracle_mod, bits, dev, "special p=%g" % p_special)


@pytest.mark.parametrize("dim0,dim1", [(True, False), (False, True)])
def test_single_direction(oracle_mod, dim0, dim1):
    dev = device()
    bits = workloads.special_values_bf16((192, 800), seed=11, p_special=0.002)
    check_cast(oracle_mod, bits, dev, "single", dim0=dim0, dim1=dim1)


# Rows a multiple of 16384 and cols a multiple of 8192, or exactly 16384 x
# 4096, at most 1024 scale columns in each scale matrix present: the scales
# are written in the blocked layout and converted back to rows in place, one
# 128-row band per workgroup (16384 x 16384 is covered by the full-size
# configuration test, 32768 x 8192 below).  16384 x 4096 and 16384 x 8192
# take that path; 16512 x 4096, 16384 x 3968, 16384 x 4224 and 16384 x 5120
# sit next to it and take the direct kernel.
VIA_BLOCKED = [(16384, 4096), (16384, 8192), (16512, 4096), (16384, 3968), (16384, 4224), (16384, 5120)]


@pytest.mark.parametrize("dim0,dim1", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("shape", VIA_BLOCKED)
def test_scales_through_blocked_layout(oracle_mod, shape, dim0, dim1):
    dev = device()
    bits = workloads.special_values_bf16(shape, seed=[23, shape[0], shape[1]], p_special=0.001)
    check_cast(oracle_mod, bits, dev, "%s dim0=%s dim1=%s" % (shape, dim0, dim1), dim0=dim0, dim1=dim1)


def test_scales_through_blocked_layout_widest(oracle_mod):
    """32768 x 8192: dim1 scale rows of 1024 bytes, the widest band the
    in-place conversion takes (256 tiles, its whole LDS)."""
    dev = device()
    shape = (32768, 8192)
    bits = workloads.special_values_bf16(shape, seed=[31, shape[0], shape[1]], p_special=0.0005)
    check_cast(oracle_mod, bits, dev, "%s widest band" % (shape,))


def test_scales_off_16_byte_alignment(oracle_mod):
    """Scale buffers 4 bytes past a 16-byte boundary at a shape that would
    otherwise go through the blocked layout: the direct kernel writes them
    (the plain scales carry no alignment requirement), and the bytes before
    each buffer stay untouched."""
    dev = device()
    r, c = 16384, 4096
    bits = workloads.special_values_bf16((r, c), seed=[29, r, c], p_special=0.001)
    bufs = [sentinel((n + 4,), dev) for n in (r * (c // 32), c * (r // 32))]
    s0 = bufs[0][4:].view(r, c // 32)
    s1 = bufs[1][4:].view(c, r // 32)
    assert s0.data_ptr() % 16 == 4 and s1.data_ptr() % 16 == 4
    q0, q1 = sentinel((r, c), dev), sentinel((c, r), dev)
    mx.mx_cast_dim0_dim1(to_dev_bf16(bits, dev), out=(q0, s0, q1, s1), raw=True)
    torch.cuda.synchronize(dev)
    r_q0, r_s0 = oracle_mod.cast_dim0(bits)
    r_q1, r_s1 = oracle_mod.cast_dim1(bits)
    assert_bytes_equal(host(q0), r_q0, "off-alignment q_row")
    assert_bytes_equal(host(s0), r_s0, "off-alignment s_row")
    assert_bytes_equal(host(q1), r_q1, "off-alignment q_col")
    assert_bytes_equal(host(s1), r_s1, "off-alignment s_col")
    for b in bufs:
        assert np.all(host(b[:4]) == 0xCD), "bytes before a scale buffer written"


def reachable_pairs(cols=1024):
    """Blocks that put every bf16 pattern against every finite scale byte it
    can meet (sweep_blocks.finite_pair_blocks), with no +-Inf or NaN, so that
    every wave takes the kernels' finite path."""
    return sb.blocks_to_matrix(sb.finite_pair_blocks(), cols)


def test_exhaustive_reachable_pairs(oracle_mod):
    """Every (bf16 pattern, scale byte) pair a finite block can produce, cast
    through the dim0 path, and through the dim1 path on the transpose."""
    dev = device()
    bits = reachable_pairs()
    q0, s0, _, _ = gpu_cast(bits, dev, dim1=False)
    r_q0, r_s0 = oracle_mod.cast_dim0(bits)
    assert_bytes_equal(s0, r_s0, "pairs s_row")
    assert_bytes_equal(q0, r_q0, "pairs q_row")
    assert set(np.unique(s0).tolist()) == set(range(247))
    t = np.ascontiguousarray(bits.T)
    _, _, q1, s1 = gpu_cast(t, dev, dim0=False)
    assert_bytes_equal(q1, r_q0, "pairs q_col of transpose")
    assert_bytes_equal(s1, r_s0, "pairs s_col of transpose")


def test_repeatable_and_fully_written(oracle_mod):
    """Two runs into outputs pre-filled with different sentinels agree."""
    dev = device()
    bits = workloads.special_values_bf16((288, 544), seed=5, p_special=0.001)
    a = gpu_cast(bits, dev, fill=0xCD)
    b = gpu_cast(bits, dev, fill=0x33)
    for x, y, n in zip(a, b, ("q_row", "s_row", "q_col", "s_col")):
        assert_bytes_equal(x, y, "rerun " + n)


def test_empty_inputs():
    dev = device()
    for shape in [(0, 64), (64, 0), (0, 0)]:
        x = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        q0, s0, q1, s1 = mx.mx_cast_dim0_dim1(x, raw=True)
        assert q0.shape == shape and q1.shape == shape[::-1]
        assert s0.shape == (shape[0], shape[1] // 32) and s1.shape == (shape[1], shape[0] // 32)


def test_rejects_bad_shapes():
    dev = device()
    for shape in [(33, 64), (64, 48)]:
        x = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
        with pytest.raises(mx.MxError) as e:
            mx.mx_cast_dim0_dim1(x)
        assert e.value.status == 2


@pytest.mark.parametrize("e,n,k", [(3, 64, 96), (2, 160, 288), (4, 256, 512), (1, 32, 32),
                                   (3, 544, 64), (2, 1024, 1056), (5, 96, 2080)])
def test_dim1_3d(oracle_mod, e, n, k):
    dev = device()
    w = workloads.special_values_bf16((e * n, k), seed=e * 100 + n, p_special=0.001).reshape(e, n, k)
    q = sentinel((e, k, n), dev)
    s = sentinel((e, k, n // 32), dev)
    mx.mx_cast_dim1_3d(to_dev_bf16(w, dev), out=(q, s), raw=True)
    torch.cuda.synchronize(dev)
    r_q, r_s = oracle_mod.cast_dim1_3d(w)
    assert_bytes_equal(host(q), r_q, "3d q")
    assert_bytes_equal(host(s), r_s, "3d s")
