"""Pins of the oracle's 128x4 blocked layout and its grouped forms against
independent constructions: a numpy reshape/transpose statement of the tile
order, permutation checks, and slice-convert-concatenate assembly of groups."""
import numpy as np
import pytest


def blocked_by_reshape(s):
    """Blocked layout as a reshape: pad to (128a, 4b); split rows into
    (row block, 32-row sub-block, row-in-sub-block) and columns into (column
    block, column-in-block); emit in order row block, column block,
    row-in-sub-block, sub-block, column-in-block."""
    r, c = s.shape
    rp, cp = -(-r // 128) * 128, -(-c // 4) * 4
    p = np.zeros((rp, cp), np.uint8)
    p[:r, :c] = s
    t = p.reshape(rp // 128, 4, 32, cp // 4, 4)
    return t.transpose(0, 3, 2, 1, 4).reshape(-1)


def test_blocked_matches_reshape_all_small_shapes(oracle_mod):
    rng = np.random.default_rng(0)
    for r in range(1, 261):
        for c in range(1, 13):
            s = rng.integers(0, 256, (r, c), dtype=np.uint8)
            got = oracle_mod.to_blocked(s)
            np.testing.assert_array_equal(got, blocked_by_reshape(s), err_msg=f"{r}x{c}")


def test_blocked_is_a_permutation(oracle_mod):
    r, c = 256, 12
    ids = np.arange(r * c, dtype=np.uint16).reshape(r, c)
    lo = oracle_mod.to_blocked((ids & 0xFF).astype(np.uint8))
    hi = oracle_mod.to_blocked((ids >> 8).astype(np.uint8))
    back = lo.astype(np.int64) | (hi.astype(np.int64) << 8)
    np.testing.assert_array_equal(np.sort(back), np.arange(r * c))
    # tile 0 begins with rows 0, 32, 64, 96 of columns 0..3
    assert back[:16].tolist() == [ids[32 * j, k] for j in range(4) for k in range(4)]


def test_batched_is_concatenation(oracle_mod):
    rng = np.random.default_rng(1)
    s = rng.integers(0, 256, (3, 130, 7), dtype=np.uint8)
    got = oracle_mod.to_blocked(s)
    want = np.concatenate([blocked_by_reshape(s[i]) for i in range(3)])
    np.testing.assert_array_equal(got, want)


def test_3d_weight_scales_equal_2d_reshape(oracle_mod):
    """Per-expert blocked scales equal the blocked form of the stacked
    (E*K, N/32) matrix when K is a multiple of 128."""
    rng = np.random.default_rng(2)
    s = rng.integers(0, 256, (4, 256, 8), dtype=np.uint8)
    np.testing.assert_array_equal(oracle_mod.to_blocked(s), oracle_mod.to_blocked(s.reshape(-1, 8)))


def _expected_grouped(s, ends, axis):
    r, c = s.shape
    g = len(ends)
    rp, cp = -(-r // 128) * 128, -(-c // 4) * 4
    size = (r + 128 * g) * cp if axis == 0 else rp * (cp + 4 * g)
    out = np.zeros(size, np.uint8)
    starts = [0]
    lo = 0
    extent = r if axis == 0 else c
    for e in ends:
        hi = min(max(int(e), lo), extent)
        part = s[lo:hi, :] if axis == 0 else s[:, lo:hi]
        blk = blocked_by_reshape(part) if part.size else np.zeros(0, np.uint8)
        if axis == 0:
            off = starts[-1] * cp
            out[off:off + blk.size] = blk
            starts.append(starts[-1] + -(-(hi - lo) // 128) * 128)
        else:
            off = rp * starts[-1]
            out[off:off + blk.size] = blk
            starts.append(starts[-1] + -(-(hi - lo) // 4) * 4)
        lo = hi
    return out, np.array(starts, np.int64)


@pytest.mark.parametrize("axis", [0, 1])
def test_grouped_single_group_is_ungrouped(oracle_mod, axis):
    rng = np.random.default_rng(3)
    s = rng.integers(0, 256, (200, 10), dtype=np.uint8)
    ext = s.shape[axis]
    out, starts = oracle_mod.to_blocked_grouped(s, np.array([ext]), axis)
    flat = oracle_mod.to_blocked(s)
    np.testing.assert_array_equal(out[:flat.size], flat)
    assert np.all(out[flat.size:] == 0)
    pad = 128 if axis == 0 else 4
    assert starts.tolist() == [0, -(-ext // pad) * pad]


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("seed", range(6))
def test_grouped_is_slice_convert_concatenate(oracle_mod, axis, seed):
    rng = np.random.default_rng(10 + seed)
    r, c = int(rng.integers(1, 400)), int(rng.integers(1, 40))
    s = rng.integers(0, 256, (r, c), dtype=np.uint8)
    g = int(rng.integers(1, 6))
    ext = s.shape[axis]
    cuts = np.sort(rng.integers(0, ext + 1, g - 1))   # empty groups allowed
    ends = np.concatenate([cuts, [ext]]).astype(np.int32)
    out, starts = oracle_mod.to_blocked_grouped(s, ends, axis)
    want, want_starts = _expected_grouped(s, ends, axis)
    np.testing.assert_array_equal(out, want)
    np.testing.assert_array_equal(starts, want_starts)


@pytest.mark.parametrize("axis", [0, 1])
def test_grouped_malformed_offsets_are_clamped(oracle_mod, axis):
    rng = np.random.default_rng(20)
    s = rng.integers(0, 256, (300, 24), dtype=np.uint8)
    ext = s.shape[axis]
    ends = np.array([ext // 2, ext // 4, -5, ext + 1000, 3], np.int32)   # decreasing, negative, too big
    out, starts = oracle_mod.to_blocked_grouped(s, ends, axis)
    want, want_starts = _expected_grouped(s, ends, axis)
    np.testing.assert_array_equal(out, want)
    np.testing.assert_array_equal(starts, want_starts)


def test_grouped_sizes(oracle_mod):
    # rows + 128 per group (axis 0), 4 extra scale columns per group (axis 1)
    assert oracle_mod.blocked_grouped_size(16640, 160, 4, 0) == 17152 * 160
    assert oracle_mod.blocked_grouped_size(5120, 512, 4, 1) == 5120 * 528
    assert oracle_mod.blocked_grouped_size(100, 5, 2, 1) == 128 * 16
    assert oracle_mod.blocked_grouped_size(100, 5, 0, 1) == -1
    assert oracle_mod.blocked_grouped_size(100, 5, 1, 2) == -1
