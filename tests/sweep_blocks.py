"""Exhaustive sweeps of 32-element blocks for the GPU parity tests.

Three families of blocks, each a (n, 32) array of bf16 bit patterns:
  * finite_pair_blocks: every (bf16 pattern, finite scale byte) pair a block
    with a finite amax can produce.  For scale byte b the block's largest
    magnitude is ((b + 8) << 7) | 0x7F (the largest bf16 with that byte), and
    the other 31 slots run through every magnitude up to it, both signs.
  * inf_blocks: blocks whose amax is +Inf (scale byte 254): a +Inf or -Inf
    anchor and every finite bf16 pattern, both signs, and +-Inf themselves.
  * nan_blocks: blocks holding a NaN (scale byte 0xFF): a NaN anchor (several
    encodings, both signs) and every one of the 65536 bf16 patterns.
The anchor's slot rotates over the 32 positions.

special_wave_layout places such blocks in a matrix so that every wave of the
cast kernels (32 rows x 256 columns of the input, both for the dim0 cast of
the matrix and for the dim1 cast of its transpose) holds at least one block
with a +-Inf or NaN, which sends the whole wave down the kernels' general
path: finite blocks are then cast by that path too.
"""
from __future__ import annotations

import numpy as np

POS_INF, NEG_INF = 0x7F80, 0xFF80
NAN_PATTERNS = (0x7FC0, 0xFFC0, 0x7F81, 0xFFFF, 0x7FFF, 0xFF81, 0x7FA5, 0xFFD3)
# largest finite magnitude pattern of bf16 (0x7F7F); 0x7F80 is +Inf
FINITE_MAGS = np.arange(0x7F80, dtype=np.uint32)


def _with_anchor(vals: np.ndarray, anchors) -> np.ndarray:
    """Blocks of 31 values from `vals` (zero-padded) plus one anchor each,
    anchors cycling over `anchors`, the anchor's slot rotating 0..31."""
    vals = np.asarray(vals, np.uint16)
    nb = -(-vals.size // 31)
    vals = np.concatenate([vals, np.zeros(nb * 31 - vals.size, np.uint16)]).reshape(nb, 31)
    anchor = np.asarray(anchors, np.uint16)[np.arange(nb) % len(anchors)]
    blk = np.empty((nb, 32), np.uint16)
    pos = np.arange(nb) % 32
    for p in range(32):
        sel = pos == p
        blk[sel, :p] = vals[sel, :p]
        blk[sel, p] = anchor[sel]
        blk[sel, p + 1:] = vals[sel, p:]
    return blk


def finite_pair_blocks(max_byte: int = 246) -> np.ndarray:
    out = []
    for b in range(0, max_byte + 1):
        anchor = ((b + 8) << 7) | 0x7F
        mags = np.arange(anchor + 1, dtype=np.uint32)
        vals = np.concatenate([mags, mags | 0x8000])
        out.append(_with_anchor(vals, [anchor]))
    return np.concatenate(out)


def inf_blocks() -> np.ndarray:
    vals = np.concatenate([FINITE_MAGS, FINITE_MAGS | 0x8000, [POS_INF, NEG_INF]])
    return _with_anchor(vals, [POS_INF, NEG_INF])


def nan_blocks() -> np.ndarray:
    return _with_anchor(np.arange(65536, dtype=np.uint32), NAN_PATTERNS)


def blocks_to_matrix(blocks: np.ndarray, cols: int) -> np.ndarray:
    """Row-major matrix of the blocks (zero blocks pad the last rows to a
    multiple of 32)."""
    per = cols // 32
    rows = -(-blocks.shape[0] // per)
    rows = -(-rows // 32) * 32
    flat = np.zeros((rows * per, 32), np.uint16)
    flat[:blocks.shape[0]] = blocks
    return flat.reshape(rows, cols)


def special_wave_layout(finite: np.ndarray, special: np.ndarray) -> np.ndarray:
    """(R, 256) matrix holding every block of `finite` and `special` once
    (special blocks repeated where more poison slots than special blocks are
    needed).  Block (r, j), r a multiple of 32, j = (r / 32) % 8, is always a
    special block: every 32-row wave of the dim0 cast (rows 32g .. 32g + 31,
    all 256 columns) holds one, and so does every wave of the dim1 cast of the
    transpose (block column j over rows 256m .. 256m + 255)."""
    per_row = 8
    nblocks = finite.shape[0] + special.shape[0]
    groups = -(-nblocks // (32 * per_row))
    groups = -(-groups // 8) * 8
    slots = np.zeros((groups * 32, per_row, 32), np.uint16)
    g = np.arange(groups)
    poison = np.zeros((groups * 32, per_row), bool)
    poison[32 * g, g % per_row] = True
    npoison = groups
    # poison slots: special blocks, cycling if there are fewer of them
    slots[poison] = special[np.arange(npoison) % special.shape[0]]
    rest = np.concatenate([special[npoison:], finite]) if special.shape[0] > npoison else finite
    free = ~poison
    fill = np.zeros((int(free.sum()), 32), np.uint16)
    fill[:rest.shape[0]] = rest
    slots[free] = fill
    return slots.reshape(groups * 32, per_row * 32)


def every_wave_special(m: np.ndarray) -> bool:
    """True when every 32 x 256 wave region of the dim0 cast of m and of the
    dim1 cast of m's transpose holds a +-Inf or NaN (checked on the bits)."""
    special = (m & 0x7FFF) >= POS_INF
    r, c = m.shape
    for r0 in range(0, r, 32):
        for c0 in range(0, c, 256):
            if not special[r0:r0 + 32, c0:c0 + 256].any():
                return False
    # transpose: 32 of m's columns x 256 of m's rows
    for c0 in range(0, c, 32):
        for r0 in range(0, r, 256):
            if not special[r0:r0 + 256, c0:c0 + 32].any():
                return False
    return True
