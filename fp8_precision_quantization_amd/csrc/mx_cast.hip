// bf16 -> MXFP8 cast along dim0 and dim1 from one read of the input
// (pytorch/ao page "triton kernel to cast to mx across dim0 and dim1",
// Summary), and the dim1-only cast of 3D expert weights ("[mxfp8 moe
// training] add compile support", Perf analysis item 4).
//
// Work decomposition (gfx950, wave64):
//   workgroup = 4 waves stacked along rows = 128 rows x 256 columns;
//   wave      = 32 rows x 256 columns: exactly one dim1 block height;
//   lane      = 32 rows x 4 columns, loaded as 32 x 8-byte row segments.
// Each row segment of a wave is 512 contiguous bytes, so every load is fully
// coalesced.  A dim0 block (32 columns of one row) spans eight lanes and is
// reduced with three DPP moves; a dim1 block (32 rows of one column) lives
// entirely in one lane, so its amax is a chain of packed 16-bit maxes with no
// data exchange.  The dim1 codes leave the lane as 32 consecutive bytes of
// one output row (two 16-byte stores); the four waves of a workgroup fill
// each 128-byte line of the col-major output from one XCD's L2.
//
// No LDS is used: the transpose that the col-major output needs happens on
// the 1-byte codes (bytes of four consecutive rows of one column are packed
// into one register by the converts), not on the bf16 inputs.
#include "mx_device.h"
#include "mxcast.h"
#include "mx_launch.h"

namespace mx {

constexpr int kWaveRows = 32;
constexpr int kWavesPerGroup = 4;
constexpr int kGroupRows = kWaveRows * kWavesPerGroup;  // 128
constexpr int kLaneCols = 4;
constexpr int kGroupCols = 64 * kLaneCols;              // 256

__device__ __forceinline__ uint32_t half_of(const uint2& v, int k) { return k == 0 ? v.x : v.y; }

// One wave's 32 x 256 tile, already in registers.  rows_per_seg: the rows of
// x form consecutive segments of this many rows (3D weights: one per expert;
// 2D: a single segment); segment e's dim1 output is a (cols, rows_per_seg)
// matrix at e * cols * rows_per_seg.
template <bool DIM0, bool DIM1, bool SPECIAL>
__device__ __forceinline__ void cast_wave_tile(const uint2 (&d)[kWaveRows], bool active, int lane,
                                               int64_t r0, int64_t c, int64_t cols,
                                               int64_t rows_per_seg, uint8_t* __restrict__ q0,
                                               uint8_t* __restrict__ s0, uint8_t* __restrict__ q1,
                                               uint8_t* __restrict__ s1) {
  if (DIM0) {
    const int64_t sb_cols = cols / 32;
#pragma unroll
    for (int i = 0; i < kWaveRows; i += 2) {
      // Lane maxima of rows i and i+1 packed as [row i, row i+1], then the
      // max over the eight lanes of each 32-column block.
      uint32_t ma = max2(mag2(d[i].x), mag2(d[i].y));
      uint32_t mb = max2(mag2(d[i + 1].x), mag2(d[i + 1].y));
      uint32_t m = max2(__builtin_amdgcn_perm(mb, ma, 0x05040100u),   // [ma.lo, mb.lo]
                        __builtin_amdgcn_perm(mb, ma, 0x07060302u));  // [ma.hi, mb.hi]
      m = max2(m, quad_swap1(m));
      m = max2(m, quad_swap2(m));
      m = max2(m, half_row_mirror(m));
      BlockParams pa = block_params<SPECIAL>(m & 0xFFFFu);
      BlockParams pb = block_params<SPECIAL>(m >> 16);
      if (active) {
        *reinterpret_cast<uint32_t*>(q0 + (r0 + i) * cols + c) = quant4<SPECIAL>(d[i].x, d[i].y, pa);
        *reinterpret_cast<uint32_t*>(q0 + (r0 + i + 1) * cols + c) =
            quant4<SPECIAL>(d[i + 1].x, d[i + 1].y, pb);
        if ((lane & 7) == 0) {
          s0[(r0 + i) * sb_cols + c / 32] = (uint8_t)pa.byte;
          s0[(r0 + i + 1) * sb_cols + c / 32] = (uint8_t)pb.byte;
        }
      }
    }
  }
  if (DIM1) {
    if (!active)
      return;
    const int64_t seg = r0 / rows_per_seg;
    const int64_t n0 = r0 - seg * rows_per_seg;
    uint8_t* q1_seg = q1 + seg * cols * rows_per_seg;
    uint8_t* s1_seg = s1 + seg * cols * (rows_per_seg / 32);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      // Column maxima over the wave's 32 rows for columns 2k, 2k+1.
      uint32_t cm = mag2(half_of(d[0], k));
#pragma unroll
      for (int i = 1; i < kWaveRows; ++i)
        cm = max2(cm, mag2(half_of(d[i], k)));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = 2 * k + h;
        BlockParams p = block_params<SPECIAL>(h ? (cm >> 16) : (cm & 0xFFFFu));
        const uint32_t sel = h ? 0x07060302u : 0x05040100u;
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < kWaveRows; i += 4) {
          // Column j of rows (i, i+1) and (i+2, i+3) as bf16 pairs.
          uint32_t p01 = __builtin_amdgcn_perm(half_of(d[i + 1], k), half_of(d[i], k), sel);
          uint32_t p23 = __builtin_amdgcn_perm(half_of(d[i + 3], k), half_of(d[i + 2], k), sel);
          w[i / 4] = quant4<SPECIAL>(p01, p23, p);
        }
        uint8_t* dst = q1_seg + (c + j) * rows_per_seg + n0;
        reinterpret_cast<uint4*>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
        reinterpret_cast<uint4*>(dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
        s1_seg[(c + j) * (rows_per_seg / 32) + n0 / 32] = (uint8_t)p.byte;
      }
    }
  }
}

template <bool DIM0, bool DIM1>
__global__ __launch_bounds__(256) void cast_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                   int64_t cols, int64_t rows_per_seg,
                                                   int64_t col_tiles, uint8_t* __restrict__ q0,
                                                   uint8_t* __restrict__ s0,
                                                   uint8_t* __restrict__ q1,
                                                   uint8_t* __restrict__ s1) {
  const int64_t tile = blockIdx.x;
  const int64_t row_tile = tile / col_tiles;
  const int64_t col_tile = tile - row_tile * col_tiles;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t r0 = row_tile * kGroupRows + (int64_t)wave * kWaveRows;
  if (r0 >= rows)
    return;  // rows is a multiple of 32: a wave is either fully in or out
  const int64_t c = col_tile * kGroupCols + (int64_t)lane * kLaneCols;
  const bool active = c < cols;  // cols is a multiple of 32: the 8 lanes of a block agree

  uint2 d[kWaveRows];
  const uint16_t* src = x + r0 * cols + (active ? c : 0);
#pragma unroll
  for (int i = 0; i < kWaveRows; ++i)
    d[i] = active ? *reinterpret_cast<const uint2*>(src + (int64_t)i * cols) : make_uint2(0, 0);

  // Any +-Inf or NaN in this wave's tile sends the whole wave down the
  // general path (uniform branch); finite data never pays for it.
  uint32_t all = 0;
#pragma unroll
  for (int i = 0; i < kWaveRows; ++i)
    all = max2(all, max2(mag2(d[i].x), mag2(d[i].y)));
  const bool special = (all & 0xFFFFu) >= kInfBits || (all >> 16) >= kInfBits;
  if (__builtin_expect(__any(special), 0))
    cast_wave_tile<DIM0, DIM1, true>(d, active, lane, r0, c, cols, rows_per_seg, q0, s0, q1, s1);
  else
    cast_wave_tile<DIM0, DIM1, false>(d, active, lane, r0, c, cols, rows_per_seg, q0, s0, q1, s1);
}

template <bool DIM0, bool DIM1>
static hipError_t launch_cast(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_seg,
                              uint8_t* q0, uint8_t* s0, uint8_t* q1, uint8_t* s1,
                              hipStream_t stream) {
  const int64_t col_tiles = (cols + kGroupCols - 1) / kGroupCols;
  hipLaunchKernelGGL((cast_kernel<DIM0, DIM1>), dim3((unsigned)cast_grid_blocks(rows, cols)),
                     dim3(256), 0, stream, x, rows, cols, rows_per_seg, col_tiles, q0, s0, q1, s1);
  return hipGetLastError();
}

int64_t cast_grid_blocks(int64_t rows, int64_t cols) {
  return ((rows + kGroupRows - 1) / kGroupRows) * ((cols + kGroupCols - 1) / kGroupCols);
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
