// bf16 -> MXFP8 cast along dim0 and dim1 from one read of the input
// (pytorch/ao page "triton kernel to cast to mx across dim0 and dim1",
// Summary), and the dim1-only cast of 3D expert weights ("[mxfp8 moe
// training] add compile support", Perf analysis item 4).
//
// Work decomposition (gfx950, wave64):
//   workgroup = 4 waves stacked along rows = a 128-row x 256-column tile;
//   wave      = 32 rows x 256 columns: exactly one dim1 block height;
//   lane      = 32 rows x 4 columns, loaded as 32 x 8-byte row segments.
// Each row segment of a wave is 512 contiguous bytes, so every load is fully
// coalesced.  A dim0 block (32 columns of one row) spans eight lanes and is
// reduced with three DPP moves; a dim1 block (32 rows of one column) lives in
// one lane, so its amax is a tree of packed 16-bit maxes.
//
// Stores are shaped for the memory system rather than for the lanes that
// produce them.  dim0 codes leave each wave as 256-byte row segments.  The
// dim1 codes of a column (32 bytes per wave) are staged in LDS, and once the
// four waves are done the workgroup writes each column's 128 rows as one full
// 128-byte line, eight lanes x 16 bytes per line; dim1 scale bytes are staged
// the same way and leave as one 4-byte run per column.  Workgroups are
// numbered so that the 32 tiles of one column range that share the lines of
// the dim1 scale matrix run back to back on the same XCD (workgroups are
// dispatched round-robin over the 8 XCDs), where that XCD's L2 merges them.
#include "mx_device.h"
#include "mxcast.h"
#include "mx_launch.h"

namespace mx {

constexpr int kWaveRows = 32;
constexpr int kWaves = 4;
constexpr int kTileRows = kWaves * kWaveRows;   // 128
constexpr int kLaneCols = 4;
constexpr int kTileCols = 64 * kLaneCols;       // 256
constexpr int kXcds = 8;
constexpr int kRowGroup = 32;                   // row tiles sharing one dim1 scale line
constexpr int kSlots = kTileRows / 16;          // 16-byte slots per staged column (8)

__device__ __forceinline__ uint32_t half_of(const uint2& v, int k) { return k == 0 ? v.x : v.y; }

// Column maxima of the tile's magnitudes for columns (2k, 2k+1), k = 0, 1,
// by a balanced tree of independent maxes.
__device__ __forceinline__ void column_max(const uint2 (&d)[kWaveRows], uint32_t (&cm)[2]) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    uint32_t t[kWaveRows / 2];
#pragma unroll
    for (int i = 0; i < kWaveRows / 2; ++i)
      t[i] = max2(mag2(half_of(d[2 * i], k)), mag2(half_of(d[2 * i + 1], k)));
#pragma unroll
    for (int w = kWaveRows / 4; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i)
        t[i] = max2(t[i], t[i + w]);
    cm[k] = t[0];
  }
}

// LDS slot of 16 dim1 codes: column col (0..255), rows 16 * slot .. +15 of
// the tile.  The slot index is XOR-swizzled with bits of the column so that
// the eight lanes of a 128-byte LDS access hit eight different bank groups
// both when the producing lanes (consecutive columns) write and when the
// storing lanes (one column, eight slots) read.
__device__ __forceinline__ int q1_slot(int col, int slot) { return col * kSlots + (slot ^ ((col >> 2) & 7)); }

// dim0 of a wave's 32 rows: per row pair, the block amax over 8 lanes, then 4
// codes per lane (one 256-byte row segment per wave) and one scale byte per
// 8 lanes.
template <bool SPECIAL>
__device__ __forceinline__ void dim0_rows(const uint2 (&d)[kWaveRows], int lane, uint8_t* __restrict__ q0,
                                          uint8_t* __restrict__ s0, int64_t cols, int64_t sb_cols) {
#pragma unroll
  for (int i = 0; i < kWaveRows; i += 2) {
    uint32_t ma = max2(mag2(d[i].x), mag2(d[i].y));
    uint32_t mb = max2(mag2(d[i + 1].x), mag2(d[i + 1].y));
    uint32_t m = max2(__builtin_amdgcn_perm(mb, ma, 0x05040100u),   // [ma.lo, mb.lo]
                      __builtin_amdgcn_perm(mb, ma, 0x07060302u));  // [ma.hi, mb.hi]
    m = max2(m, quad_swap1(m));
    m = max2(m, quad_swap2(m));
    m = max2(m, half_row_mirror(m));
    BlockParams pa = block_params<SPECIAL>(m & 0xFFFFu);
    BlockParams pb = block_params<SPECIAL>(m >> 16);
    *reinterpret_cast<uint32_t*>(q0 + (int64_t)i * cols) = quant4<SPECIAL>(d[i].x, d[i].y, pa);
    *reinterpret_cast<uint32_t*>(q0 + (int64_t)(i + 1) * cols) = quant4<SPECIAL>(d[i + 1].x, d[i + 1].y, pb);
    if ((lane & 7) == 0) {
      s0[(int64_t)i * sb_cols] = (uint8_t)pa.byte;
      s0[(int64_t)(i + 1) * sb_cols] = (uint8_t)pb.byte;
    }
  }
}

// dim1 of a wave's 32 rows: for each of the lane's 4 columns, 32 codes into
// two LDS slots and the scale byte into the column's scale word.
template <bool SPECIAL>
__device__ __forceinline__ void dim1_rows(const uint2 (&d)[kWaveRows], const uint32_t (&cm)[2], int lane,
                                          int wave, uint4* q1_lds, uint8_t* s1_lds) {
#pragma unroll
  for (int j = 0; j < kLaneCols; ++j) {
    const int k = j >> 1;
    const bool hi = j & 1;
    BlockParams p = block_params<SPECIAL>(hi ? (cm[k] >> 16) : (cm[k] & 0xFFFFu));
    const uint32_t sel = hi ? 0x07060302u : 0x05040100u;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < kWaveRows; i += 4) {
      // Column j of rows (i, i+1) and (i+2, i+3) as bf16 pairs.
      uint32_t p01 = __builtin_amdgcn_perm(half_of(d[i + 1], k), half_of(d[i], k), sel);
      uint32_t p23 = __builtin_amdgcn_perm(half_of(d[i + 3], k), half_of(d[i + 2], k), sel);
      w[i / 4] = quant4<SPECIAL>(p01, p23, p);
    }
    const int col = lane * kLaneCols + j;
    q1_lds[q1_slot(col, 2 * wave)] = make_uint4(w[0], w[1], w[2], w[3]);
    q1_lds[q1_slot(col, 2 * wave + 1)] = make_uint4(w[4], w[5], w[6], w[7]);
    s1_lds[col * kWaves + wave] = (uint8_t)p.byte;
  }
}

// Tile order: groups of kRowGroup row tiles; inside a group, column tiles
// outermost; each XCD takes a contiguous run of this order.
__device__ __forceinline__ bool tile_of(uint32_t bid, uint32_t row_tiles, uint32_t col_tiles,
                                        uint32_t per_xcd, uint32_t& rt, uint32_t& ct) {
  const uint32_t id = (bid % kXcds) * per_xcd + bid / kXcds;
  if (id >= row_tiles * col_tiles)
    return false;
  const uint32_t group_tiles = kRowGroup * col_tiles;
  const uint32_t g = id / group_tiles;
  const uint32_t within = id - g * group_tiles;
  const uint32_t gs = min((uint32_t)kRowGroup, row_tiles - g * kRowGroup);
  ct = within / gs;
  rt = g * kRowGroup + (within - ct * gs);
  return true;
}

// rows_per_seg: the rows of x form consecutive segments of this many rows
// (3D weights: one per expert; 2D: one segment).  Segment e's dim1 output is
// a (cols, rows_per_seg) matrix at e * cols * rows_per_seg, its scales a
// (cols, rows_per_seg / 32) matrix at e * cols * rows_per_seg / 32.
template <bool DIM0, bool DIM1>
__global__ __launch_bounds__(256) void cast_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                   int64_t cols, int64_t rows_per_seg,
                                                   uint32_t row_tiles, uint32_t col_tiles,
                                                   uint32_t per_xcd, uint8_t* __restrict__ q0,
                                                   uint8_t* __restrict__ s0,
                                                   uint8_t* __restrict__ q1,
                                                   uint8_t* __restrict__ s1) {
  __shared__ uint4 q1_lds[DIM1 ? kTileCols * kSlots : 1];
  __shared__ uint8_t s1_lds[DIM1 ? kTileCols * kWaves : 1];

  uint32_t rt, ct;
  if (!tile_of(blockIdx.x, row_tiles, col_tiles, per_xcd, rt, ct))
    return;  // uniform over the workgroup
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t tile_r = (int64_t)rt * kTileRows;
  const int64_t tile_c = (int64_t)ct * kTileCols;
  const int64_t r0 = tile_r + wave * kWaveRows;
  const int64_t c = tile_c + lane * kLaneCols;
  // rows, cols are multiples of 32: a wave is fully in or out, and the 8
  // lanes of a dim0 block agree.
  const bool on = r0 < rows && c < cols;

  if (on) {
    uint2 d[kWaveRows];
    const uint16_t* src = x + r0 * cols + c;
#pragma unroll
    for (int i = 0; i < kWaveRows; ++i)
      d[i] = *reinterpret_cast<const uint2*>(src + (int64_t)i * cols);

    uint32_t cm[2];
    column_max(d, cm);
    const uint32_t all = max2(cm[0], cm[1]);
    const bool special = (all & 0xFFFFu) >= kInfBits || (all >> 16) >= kInfBits;
    // Any +-Inf or NaN among the wave's active lanes sends the wave down the
    // general path (uniform branch); finite data never pays for it.
    const bool any_special = __any(special);
    if (DIM1) {
      if (any_special)
        dim1_rows<true>(d, cm, lane, wave, q1_lds, s1_lds);
      else
        dim1_rows<false>(d, cm, lane, wave, q1_lds, s1_lds);
    }
    if (DIM0) {
      uint8_t* q0_row = q0 + r0 * cols + c;
      uint8_t* s0_row = s0 + r0 * (cols / 32) + c / 32;
      if (any_special)
        dim0_rows<true>(d, lane, q0_row, s0_row, cols, cols / 32);
      else
        dim0_rows<false>(d, lane, q0_row, s0_row, cols, cols / 32);
    }
  }

  if (DIM1) {
    __syncthreads();
    const int valid_rows = (int)min((int64_t)kTileRows, rows - tile_r);   // multiple of 32
    const int valid_cols = (int)min((int64_t)kTileCols, cols - tile_c);
    // Segment of the tile's first row; the tile crosses at most a few
    // segment ends (segments are multiples of 32 rows).
    const int64_t seg0 = tile_r / rows_per_seg;
    const int64_t off0 = tile_r - seg0 * rows_per_seg;
    const bool one_seg = off0 + valid_rows <= rows_per_seg;
    const int64_t seg_blocks = rows_per_seg / 32;

    // Codes: 8 lanes per column, 16 bytes each; a wave covers 8 columns per pass.
    const int slot = threadIdx.x & 7;
#pragma unroll 4
    for (int pass = 0; pass < kTileCols / 32; ++pass) {
      const int col = pass * 32 + (threadIdx.x >> 3);
      if (col < valid_cols && slot * 16 < valid_rows) {
        int64_t seg = seg0, off = off0 + slot * 16;
        while (off >= rows_per_seg) {
          off -= rows_per_seg;
          ++seg;
        }
        uint8_t* dst = q1 + (seg * cols + tile_c + col) * rows_per_seg + off;
        *reinterpret_cast<uint4*>(dst) = q1_lds[q1_slot(col, slot)];
      }
    }
    // Scales: one thread per column, the four 32-row blocks of the tile.
    const int col = threadIdx.x;
    if (col < valid_cols) {
      const uint32_t v = reinterpret_cast<const uint32_t*>(s1_lds)[col];
      const int nblk = valid_rows / 32;
      uint8_t* dst = s1 + (seg0 * cols + tile_c + col) * seg_blocks + off0 / 32;
      if (one_seg && nblk == kWaves && ((uintptr_t)dst % 4) == 0) {
        *reinterpret_cast<uint32_t*>(dst) = v;
      } else {
        for (int b = 0; b < nblk; ++b) {
          int64_t seg = seg0, off = off0 + 32 * b;
          while (off >= rows_per_seg) {
            off -= rows_per_seg;
            ++seg;
          }
          s1[(seg * cols + tile_c + col) * seg_blocks + off / 32] = (uint8_t)(v >> (8 * b));
        }
      }
    }
  }
}

struct CastGrid {
  uint32_t row_tiles, col_tiles, per_xcd;
  int64_t blocks;
};

static CastGrid cast_grid(int64_t rows, int64_t cols) {
  CastGrid g;
  const int64_t rt = (rows + kTileRows - 1) / kTileRows;
  const int64_t ct = (cols + kTileCols - 1) / kTileCols;
  const int64_t per = (rt * ct + kXcds - 1) / kXcds;
  g.row_tiles = (uint32_t)rt;
  g.col_tiles = (uint32_t)ct;
  g.per_xcd = (uint32_t)per;
  g.blocks = per * kXcds;
  return g;
}

int64_t cast_grid_blocks(int64_t rows, int64_t cols) { return cast_grid(rows, cols).blocks; }

template <bool DIM0, bool DIM1>
static hipError_t launch_cast(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_seg,
                              uint8_t* q0, uint8_t* s0, uint8_t* q1, uint8_t* s1,
                              hipStream_t stream) {
  const CastGrid g = cast_grid(rows, cols);
  hipLaunchKernelGGL((cast_kernel<DIM0, DIM1>), dim3((unsigned)g.blocks), dim3(kWaves * 64), 0, stream,
                     x, rows, cols, rows_per_seg, g.row_tiles, g.col_tiles, g.per_xcd, q0, s0, q1, s1);
  return hipGetLastError();
}

hipError_t launch_cast_any(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_seg,
                           uint8_t* q0, uint8_t* s0, uint8_t* q1, uint8_t* s1,
                           hipStream_t stream) {
  const bool d0 = q0 != nullptr, d1 = q1 != nullptr;
  if (d0 && d1)
    return launch_cast<true, true>(x, rows, cols, rows_per_seg, q0, s0, q1, s1, stream);
  if (d0)
    return launch_cast<true, false>(x, rows, cols, rows_per_seg, q0, s0, q1, s1, stream);
  return launch_cast<false, true>(x, rows, cols, rows_per_seg, q0, s0, q1, s1, stream);
}

}  // namespace mx
