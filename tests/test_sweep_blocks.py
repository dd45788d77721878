"""The exhaustive block sweeps the GPU parity tests run (tests/sweep_blocks.py)
cover what they claim: every pattern in every block family, and a +-Inf or
NaN in every wave of the special-path layout."""
import numpy as np

from tests import sweep_blocks as sb


def test_finite_pairs_cover_every_pair():
    blk = sb.finite_pair_blocks()
    mags = blk & 0x7FFF
    assert mags.max() == 0x7F7F
    amax = mags.max(axis=1)
    # the scale byte of each block from its amax exponent field
    byte = np.maximum((amax >> 7).astype(np.int64) - 8, 0)
    for b in (0, 1, 100, 246):
        sel = blk[byte == b]
        vals = np.unique(sel)
        anchor = ((b + 8) << 7) | 0x7F
        want = np.concatenate([np.arange(anchor + 1), np.arange(anchor + 1) | 0x8000])
        assert np.array_equal(vals, np.unique(want)), b
    assert set(np.unique(byte).tolist()) == set(range(247))


def test_inf_blocks_hold_every_finite_pattern():
    blk = sb.inf_blocks()
    assert np.all(((blk & 0x7FFF) == 0x7F80).any(axis=1))
    assert not np.any(((blk & 0x7FFF) > 0x7F80))
    vals = np.unique(blk)
    want = np.concatenate([np.arange(0x7F81), np.arange(0x8000, 0xFF81)])
    assert np.array_equal(vals, want)
    # both anchor signs and every anchor slot
    pos = np.argmax((blk & 0x7FFF) == 0x7F80, axis=1)
    assert set(pos.tolist()) == set(range(32))
    assert {int(v) for v in blk[np.arange(blk.shape[0]), pos]} == {0x7F80, 0xFF80}


def test_nan_blocks_hold_every_pattern():
    blk = sb.nan_blocks()
    assert np.all(((blk & 0x7FFF) > 0x7F80).any(axis=1))
    assert np.array_equal(np.unique(blk), np.arange(65536))
    # 31 swept values per block: the sweep needs ceil(65536 / 31) blocks
    assert blk.shape[0] == -(-65536 // 31)


def test_special_wave_layout():
    fin = sb.finite_pair_blocks(max_byte=40)
    spec = np.concatenate([sb.inf_blocks(), sb.nan_blocks()])
    m = sb.special_wave_layout(fin, spec)
    assert m.shape[1] == 256 and m.shape[0] % 256 == 0
    assert sb.every_wave_special(m)
    blocks = m.reshape(-1, 32)
    # every input block is present (as a row of the block list)
    have = {bytes(b) for b in blocks}
    assert all(bytes(b) in have for b in fin[::97])
    assert all(bytes(b) in have for b in spec)
    # and the finite-only matrix has no special value at all
    f = sb.blocks_to_matrix(fin, 1024)
    assert not np.any((f & 0x7FFF) >= 0x7F80)
