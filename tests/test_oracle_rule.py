"""Pins of the oracle's element and scale rule against things other than the
oracle itself: hand-worked blocks, torch's own fp8/e8m0 codecs, closed forms
of the scale, exhaustive sweeps of every bf16 pattern."""
import json
import math
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _f64(bits):
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_worked_blocks(oracle_mod):
    fx = json.load(open(os.path.join(HERE, "golden", "worked_blocks.json")))
    assert len(fx["blocks"]) >= 10
    for b in fx["blocks"]:
        lead = [int(h, 16) for h in b["in"]]
        x = np.array(lead + [int(b["rest_in"], 16)] * (32 - len(lead)), dtype=np.uint16)
        q, s = oracle_mod.quantize_block(x)
        want_q = [int(h, 16) for h in b["q"]]
        want_q += [int(b["rest_q"], 16)] * (32 - len(want_q))
        assert s == b["scale"], b["name"]
        assert q.tolist() == want_q, b["name"]


def test_e4m3_codebook_matches_torch(oracle_mod):
    # torch's float8_e4m3fn decoder is an independent definition of the format.
    codes = torch.arange(0, 127, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle_mod.e4m3_value(c) for c in range(127)])
    np.testing.assert_array_equal(got, ref)
    assert oracle_mod.e4m3_value(0x7E) == 448.0
    assert oracle_mod.e4m3_value(0x01) == 2.0 ** -9


def test_e8m0_matches_torch(oracle_mod):
    b = torch.arange(0, 255, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle_mod.e8m0_value(i) for i in range(255)])
    np.testing.assert_array_equal(got, ref)
    assert math.isnan(oracle_mod.e8m0_value(255))


def test_scale_byte_exhaustive(oracle_mod):
    """Every non-negative bf16 amax: the oracle (frexp) against numpy's log2
    and against the exponent-field closed form max(E - 8, 0)."""
    mags = np.arange(0x0000, 0x8000, dtype=np.uint32).astype(np.uint16)
    vals = _f64(mags)
    got = np.array([oracle_mod.scale_byte(v) for v in vals])
    finite = np.isfinite(vals)
    pos = finite & (vals > 0)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(pos, vals, 1.0))) - 8
    want = np.where(pos, np.clip(e, -127, 127) + 127, 0)
    want = np.where(vals == np.inf, 254, want)
    want = np.where(np.isnan(vals), 255, want)
    np.testing.assert_array_equal(got, want.astype(np.int64))
    # closed form from the exponent field for finite amax
    ef = (mags.astype(np.int64) >> 7) & 0xFF
    closed = np.maximum(ef - 8, 0)
    np.testing.assert_array_equal(got[finite], closed[finite])
    assert got[0x7F7F] == 246 and got[0x7F80] == 254 and got[0x7FC0] == 255


@pytest.mark.parametrize("chunk", range(5))
def test_element_rule_exhaustive_vs_torch(oracle_mod, chunk):
    """All 65536 bf16 patterns under every finite scale byte (split into five
    parametrised chunks): oracle == torch's float8_e4m3fn cast of the exactly
    scaled value clamped to +-448 (torch rounds to nearest-even but does not
    saturate, hence the clamp)."""
    x64 = _f64(ALL_BF16)
    finite = ~np.isnan(x64)
    xt = torch.from_numpy(x64)
    for s in range(chunk * 51, chunk * 51 + 51):
        got = oracle_mod.quantize_elements(ALL_BF16, s)
        v = torch.clamp(xt * 2.0 ** (127 - s), -448.0, 448.0)
        ref = v.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        bad = np.nonzero((got != ref) & finite)[0]
        assert bad.size == 0, (s, [hex(int(b)) for b in bad[:5]])
        # NaN inputs become NaN with their own sign
        nan_bits = ALL_BF16[~finite]
        assert np.all(got[~finite] == (0x7F | ((nan_bits >> 8) & 0x80)))


def test_element_rule_nan_scale(oracle_mod):
    got = oracle_mod.quantize_elements(ALL_BF16, 255)
    np.testing.assert_array_equal(got, (0x7F | ((ALL_BF16 >> 8) & 0x80)).astype(np.uint8))


def test_representable_values_round_trip(oracle_mod):
    """Every e4m3 value times 2^e is quantized back to its own code."""
    for s in (0, 1, 60, 119, 127, 200, 246):
        e = s - 127
        for c in range(127):
            v = oracle_mod.e4m3_value(c) * 2.0 ** e
            if v == 0 or not (2.0 ** -133 <= v < 2.0 ** 128):
                continue
            # only values exactly representable in bf16 are possible inputs
            if float(np.float32(v)) != v:
                continue
            b = (np.array([v], np.float32).view(np.uint32) >> 16).astype(np.uint16)
            if _f64(b)[0] != v:
                continue
            assert oracle_mod.quantize_element(v, s) == c
            assert oracle_mod.quantize_element(-v, s) == c | 0x80


def test_page_shapes(oracle_mod):
    """(16640, 5120) activations carry (16640, 160) dim0 scales in the compile
    support page's error trace: one scale per 32 elements of the last axis."""
    x = np.zeros((32, 5120), np.uint16)
    q, s = oracle_mod.cast_dim0(x)
    assert q.shape == (32, 5120) and s.shape == (32, 160)
    assert oracle_mod.blocked_grouped_size(16640, 160, 4, 0) == (16640 + 4 * 128) * 160
