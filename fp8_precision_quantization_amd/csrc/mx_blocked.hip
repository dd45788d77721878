// e8m0 scales -> 128x4 blocked layout, plain / batched / grouped along M /
// grouped along K, with group offsets read only on the device.
//
// Pages: "[mxfp8 moe training] parallelize along col blocks in scale blocked
// format kernel for groups along K" (Changes: a 128x4 granularity, and
// parallelism over both row and column blocks) and "[mxfp8 moe training] add
// compile support" (change list: no host read of the offsets, output rows
// bounded by rows + num_groups * 128; Perf analysis item 2: M-group, K-group
// and per-expert 3D variants).
//
// One workgroup (256 threads) owns one 128-row block and up to 16 or 32
// consecutive output tiles (column blocks of 4; 32 where the grid still has
// 512 workgroups).  It stages the strip in LDS with 64- or 128-byte
// contiguous reads per source row, all of a thread's loads in flight at
// once, then writes the tiles: each store instruction of a wave writes two
// whole 512-byte tiles, non-temporal (the lines are complete, so nothing is
// gained by keeping them in the L2).  Workgroups are numbered so that each
// XCD (workgroups are dispatched round-robin over the 8 XCDs) takes
// consecutive strips: strips that read parts of the same source lines then
// share its L2.  The source reads stay ordinary loads: a 16-tile strip
// covers half a line.  Chosen by timing on MI355X against 8-tile strips,
// plain numbering, ordinary stores and non-temporal loads (e.g. the (16,
// 5120, 256) per-expert layout: 12.0 -> 6.6 us, K groups of (8192, 4096):
// 22.9 -> 18.7 us), then 32-tile strips and all loads in flight at once
// (5.1 and 12.0 us).  The
// grouped forms rebuild the group table (clamped ends, padded starts) in LDS
// in every workgroup with one wave-wide scan, so the whole conversion is a
// single launch with no host round trip.
//
// unblock_kernel (end of file) is the inverse map, in place, behind the
// plain-scale cast.
#include <type_traits>

#include "mx_device.h"
#include "mx_groups.h"
#include "mxcast.h"
#include "mx_launch.h"

namespace mx {

constexpr int kBlkThreads = 256;
constexpr int kXcdCount = 8;
constexpr int kTileRows = 128;
constexpr int kTileBytes = 512;

enum : int { kModeBatched = 0, kModeMGroups = 1, kModeKGroups = 2 };

struct Slot {
  int64_t src_col;   // first source column of this tile
  int32_t ncols;     // valid source columns (0..4); 0 -> zero tile
  int64_t out_off;   // output byte offset of the tile; < 0 -> no tile
};

struct Args {
  const uint8_t* s;
  int64_t rows, cols;
  int64_t batch;
  const int32_t* ends;
  int32_t groups;
  uint8_t* out;
  int64_t out_bytes;
  int64_t* out_starts;
  int64_t row_blocks;   // output row blocks in the grid
  int64_t col_chunks;   // strips (of STRIP tiles) per row block in the grid
  int64_t blocks;       // workgroups doing work (the grid rounds up to 8 XCDs)
  int64_t per_xcd;      // consecutive work items per XCD
};

template <int MODE, int STRIP>
__global__ __launch_bounds__(kBlkThreads) void blocked_kernel(Args a) {
  static_assert(STRIP % 8 == 0 && kBlkThreads % STRIP == 0, "a strip is whole store passes and load rows");
  constexpr int kLdsStride = STRIP + 1;  // dwords per staged row (+1 against bank conflicts)
  __shared__ uint32_t strip[kTileRows * kLdsStride];
  __shared__ std::conditional_t<MODE == kModeBatched, NoTable, GroupTable> table;

  const int tid = threadIdx.x;
  const int64_t cols_pad = (a.cols + 3) / 4 * 4;
  const int64_t rows_pad = (a.rows + kTileRows - 1) / kTileRows * kTileRows;
  const int64_t ncb = cols_pad / 4;

  // XCD-aware numbering: XCD x = blockIdx % 8 takes items [x * per_xcd, ...).
  int64_t bid = (int64_t)(blockIdx.x % kXcdCount) * a.per_xcd + blockIdx.x / kXcdCount;
  if (bid >= a.blocks)
    return;  // uniform over the workgroup, before any barrier; item 0 always runs
  const int64_t chunk = bid % a.col_chunks;
  bid /= a.col_chunks;
  const int64_t orb = bid % a.row_blocks;  // output row block (within a batch entry)
  const int64_t b = bid / a.row_blocks;

  if constexpr (MODE != kModeBatched) {
    if (tid < 64) {
      const int32_t extent = (int32_t)(MODE == kModeMGroups ? a.rows : a.cols);
      const int32_t unit = MODE == kModeMGroups ? kTileRows : 4;
      if (a.groups <= kScalarTableGroups)
        build_group_table_scalar(a.ends, a.groups, extent, unit, table);
      else
        build_group_table(a.ends, a.groups, extent, unit, table);
    }
    __syncthreads();
    if (bid == 0 && a.out_starts != nullptr) {
      for (int g = tid; g <= a.groups; g += kBlkThreads)
        a.out_starts[g] = table.start[g];
    }
  }

  // Source rows of this workgroup.
  const uint8_t* src = a.s + b * a.rows * a.cols;
  int64_t row0 = orb * kTileRows;
  int64_t nrows = min((int64_t)kTileRows, a.rows - row0);
  if constexpr (MODE == kModeMGroups) {
    int g = find_group(table, a.groups, (int32_t)(orb * kTileRows));
    if (g < 0) {
      nrows = 0;
      row0 = 0;
    } else {
      row0 = table.lo[g] + (orb * kTileRows - table.start[g]);
      nrows = min((int64_t)kTileRows, (int64_t)table.hi[g] - row0);
    }
  }
  if (nrows < 0)
    nrows = 0;

  auto slot_of = [&](int k) -> Slot {
    Slot sl;
    const int64_t cb = chunk * STRIP + k;
    if constexpr (MODE == kModeKGroups) {
      const int64_t tcb = ncb + a.groups;
      if (cb >= tcb) {
        sl.src_col = 0;
        sl.ncols = 0;
        sl.out_off = -1;
        return sl;
      }
      int g = find_group(table, a.groups, (int32_t)(cb * 4));
      if (g < 0) {  // slack after the last group: zero tiles, one column block each
        sl.src_col = 0;
        sl.ncols = 0;
        sl.out_off = rows_pad * 4 * cb + orb * kTileBytes;
        return sl;
      }
      const int64_t local_cb = cb - table.start[g] / 4;
      const int64_t width_pad = (table.hi[g] - table.lo[g] + 3) / 4 * 4;
      sl.src_col = table.lo[g] + 4 * local_cb;
      sl.ncols = (int32_t)min((int64_t)4, (int64_t)table.hi[g] - sl.src_col);
      sl.out_off = rows_pad * table.start[g] + (orb * (width_pad / 4) + local_cb) * kTileBytes;
      return sl;
    }
    if (cb >= ncb) {
      sl.src_col = 0;
      sl.ncols = 0;
      sl.out_off = -1;
      return sl;
    }
    sl.src_col = 4 * cb;
    sl.ncols = (int32_t)min((int64_t)4, a.cols - 4 * cb);
    sl.out_off = ((b * a.row_blocks + orb) * ncb + cb) * kTileBytes;
    return sl;
  };

  // Stage: row i, tile k -> one dword (4 scale bytes, column order = byte order).
  // A thread keeps one tile k and takes every (256 / STRIP)-th row; when its
  // tile's 4 source columns are a whole aligned dword, all of its loads are
  // issued at once as buffer loads ranged to the block's valid rows (rows
  // past them read zero), else it assembles the bytes one by one.
  {
    constexpr int kRowsPerPass = kBlkThreads / STRIP;
    constexpr int kPasses = kTileRows / kRowsPerPass;
    const int k = tid % STRIP;
    const int i0 = tid / STRIP;
    const Slot sl = slot_of(k);
    const bool aligned = sl.ncols == 4 && (a.cols % 4) == 0 && (sl.src_col % 4) == 0 &&
                         ((uintptr_t)src % 4) == 0 && a.cols < (1 << 23);
    if (aligned && nrows > 0) {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src + row0 * a.cols, (uint32_t)(nrows * a.cols));
      uint32_t v[kPasses];
#pragma unroll
      for (int p = 0; p < kPasses; ++p)
        v[p] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)((i0 + p * kRowsPerPass) * a.cols + sl.src_col), 0, 0);
#pragma unroll
      for (int p = 0; p < kPasses; ++p)
        strip[(i0 + p * kRowsPerPass) * kLdsStride + k] = v[p];
    } else {
      for (int p = 0; p < kPasses; ++p) {
        const int i = i0 + p * kRowsPerPass;
        uint32_t v = 0;
        if (i < nrows && sl.ncols > 0) {
          const uint8_t* sp = src + (row0 + i) * a.cols + sl.src_col;
          for (int j = 0; j < sl.ncols; ++j)
            v |= (uint32_t)sp[j] << (8 * j);
        }
        strip[i * kLdsStride + k] = v;
      }
    }
  }
  __syncthreads();

  // Write: in pass h, lanes 0-31 of wave w write tile k = 8 h + 2 w and
  // lanes 32-63 tile k + 1; lane i (mod 32) writes tile row i, the 16 bytes
  // of the four 32-row sub-blocks of that row, 4 columns each.  One store
  // instruction thus writes two whole tiles.
  {
    const int wave = tid >> 6;
    const int i = tid & 31;
#pragma unroll
    for (int h = 0; h < STRIP / 8; ++h) {
      const int k = 8 * h + 2 * wave + ((tid >> 5) & 1);
      const Slot sl = slot_of(k);
      if (sl.out_off >= 0) {
        uint4 o = make_uint4(strip[i * kLdsStride + k], strip[(32 + i) * kLdsStride + k],
                             strip[(64 + i) * kLdsStride + k], strip[(96 + i) * kLdsStride + k]);
        const int64_t off = sl.out_off + i * 16;
        if (off + 16 <= a.out_bytes) {
          store_line_nt(a.out + off, o);
        } else if (off < a.out_bytes) {
          const uint32_t w[4] = {o.x, o.y, o.z, o.w};
          for (int j = 0; off + j < a.out_bytes; ++j)
            a.out[off + j] = (uint8_t)(w[j / 4] >> (8 * (j % 4)));
        }
      }
    }
  }
}

// Work items of a launch (row blocks x strips of `strip` tiles), 0 when
// there is nothing to do.
static int64_t plan_blocked(int mode, Args& a, int strip) {
  const int64_t ncb = (a.cols + 3) / 4;
  const int64_t rb = (a.rows + kTileRows - 1) / kTileRows;
  if (mode == kModeBatched) {
    a.row_blocks = rb;
    a.col_chunks = (ncb + strip - 1) / strip;
    return a.batch * a.row_blocks * a.col_chunks;
  }
  // Grouped forms always launch at least one workgroup: the padded starts
  // are written even when the scale matrix is empty.
  if (mode == kModeMGroups) {
    a.row_blocks = (a.rows + (int64_t)kTileRows * a.groups + kTileRows - 1) / kTileRows;
    a.col_chunks = (ncb + strip - 1) / strip;
  } else {
    a.row_blocks = rb;
    a.col_chunks = (ncb + a.groups + strip - 1) / strip;
  }
  a.row_blocks = a.row_blocks > 0 ? a.row_blocks : 1;
  a.col_chunks = a.col_chunks > 0 ? a.col_chunks : 1;
  a.batch = 1;
  return a.row_blocks * a.col_chunks;
}

// Strip width: 32 tiles (128 source bytes per row) where that still gives
// the launch kBlkWideMin workgroups, else 16.  Timed on MI355X (back to back,
// 300 launches): K groups of (8192, 4096) 13.3 us with 16-tile strips, 12.0
// with 32, 13.9 with 64; the (16, 5120, 256) per-expert layout 5.2 / 5.1 /
// 5.4 us; the small grids (M groups of (16640, 160): 268 workgroups of 32
// tiles) 4.1 us with 16 against 4.9 with 32.
constexpr int64_t kBlkWideMin = 512;
static int strip_of(int mode, const Args& a0) {
  Args a = a0;
  return plan_blocked(mode, a, 32) >= kBlkWideMin ? 32 : 16;
}

int64_t blocked_grid_blocks(int32_t mode, int64_t batch, int64_t rows, int64_t cols, int32_t groups) {
  Args a = {};
  a.batch = batch;
  a.rows = rows;
  a.cols = cols;
  a.groups = groups;
  // the narrowest strip gives the largest grid
  const int64_t items = plan_blocked(mode, a, 16);
  return (items + kXcdCount - 1) / kXcdCount * kXcdCount;
}

template <int MODE>
static void launch_mode(const Args& a, int strip, dim3 grid, hipStream_t stream) {
  if (strip == 32)
    hipLaunchKernelGGL((blocked_kernel<MODE, 32>), grid, dim3(kBlkThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((blocked_kernel<MODE, 16>), grid, dim3(kBlkThreads), 0, stream, a);
}

static hipError_t launch_blocked(int mode, const Args& a0, hipStream_t stream) {
  Args a = a0;
  const int strip = strip_of(mode, a0);
  a.blocks = plan_blocked(mode, a, strip);
  if (a.blocks == 0)
    return hipSuccess;
  a.per_xcd = (a.blocks + kXcdCount - 1) / kXcdCount;
  const dim3 grid((unsigned)(a.per_xcd * kXcdCount));
  if (mode == kModeBatched)
    launch_mode<kModeBatched>(a, strip, grid, stream);
  else if (mode == kModeMGroups)
    launch_mode<kModeMGroups>(a, strip, grid, stream);
  else
    launch_mode<kModeKGroups>(a, strip, grid, stream);
  return hipGetLastError();
}

hipError_t launch_blocked_batched(const uint8_t* s, int64_t batch, int64_t rows, int64_t cols,
                                  uint8_t* out, hipStream_t stream) {
  Args a = {};
  a.s = s;
  a.rows = rows;
  a.cols = cols;
  a.batch = batch;
  a.out = out;
  a.out_bytes = batch * ((rows + 127) / 128 * 128) * ((cols + 3) / 4 * 4);
  return launch_blocked(kModeBatched, a, stream);
}

hipError_t launch_blocked_grouped(const uint8_t* s, int64_t rows, int64_t cols, const int32_t* ends,
                                  int32_t groups, int32_t axis, uint8_t* out, int64_t out_bytes,
                                  int64_t* out_starts, hipStream_t stream) {
  Args a = {};
  a.s = s;
  a.rows = rows;
  a.cols = cols;
  a.batch = 1;
  a.ends = ends;
  a.groups = groups;
  a.out = out;
  a.out_bytes = out_bytes;
  a.out_starts = out_starts;
  return launch_blocked(axis == 0 ? kModeMGroups : kModeKGroups, a, stream);
}

// The inverse map, in place: e8m0 scale matrices of R x C bytes (R % 128 ==
// 0, C % 16 == 0, C <= kUnblockMaxCols) from the 128x4 blocked layout to the
// plain row-major one.  A 128-row band occupies the same 128 * C bytes in
// both layouts (in the blocked one as its C / 4 tiles, one after another), so
// one workgroup per band reads the whole band with contiguous 16-byte loads,
// regroups it in LDS and writes it back as contiguous rows of 16-byte chunks.
// Dword j of chunk i of tile k is row i + 32 j, scale columns 4 k .. 4 k + 3.
// Every load of a band has returned (its value is in LDS) before the
// barrier, and only after it does any thread of the workgroup store into the
// band.
//
// The band loads are non-temporal: cached loads took ~4 us longer at 16384 x
// 16384 (172 -> 168 us for the whole plain-scale call; 32768 x 8192 184 ->
// 175 us; smaller inputs even), although a kernel that reads the plain
// scales right after then takes longer (the two layout launches of both
// 16384 x 512 matrices ~5 us more); the whole-line 16-byte stores are
// non-temporal too (0.2 us).
constexpr int kUnblockTiles = kUnblockMaxCols / 4;     // tiles per band, at most
constexpr int kUnblockPitch = kUnblockTiles + 1;       // dwords per staged row (odd: no bank conflicts)
constexpr int kUnblockThreads = 1024;                  // 16 waves share a band's latency
constexpr int kUnblockChunks = kUnblockTiles * 32 / kUnblockThreads;   // 16-byte chunks per thread, at most

__global__ __launch_bounds__(kUnblockThreads) void unblock_kernel(uint8_t* m0, int64_t c0, int64_t bands0,
                                                                  uint8_t* m1, int64_t c1) {
  __shared__ uint32_t staged[kTileRows * kUnblockPitch];
  int64_t band = blockIdx.x;
  uint8_t* m = m0;
  int64_t c = c0;
  if (band >= bands0) {
    band -= bands0;
    m = m1;
    c = c1;
  }
  const int tiles = (int)(c / 4);
  const int chunks = tiles * 32;   // 16-byte chunks of the band, in either layout
  uint8_t* base = m + band * kTileRows * c;
  const int t = threadIdx.x;
  uint4 v[kUnblockChunks];
#pragma unroll
  for (int n = 0; n < kUnblockChunks; ++n) {
    const int q = t + kUnblockThreads * n;
    if (q < chunks) {
      const u32x4 l = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + 16 * (int64_t)q));
      v[n] = make_uint4(l[0], l[1], l[2], l[3]);
    }
  }
#pragma unroll
  for (int n = 0; n < kUnblockChunks; ++n) {
    const int q = t + kUnblockThreads * n;
    if (q < chunks) {
      const int k = q >> 5, i = q & 31;
      staged[i * kUnblockPitch + k] = v[n].x;
      staged[(i + 32) * kUnblockPitch + k] = v[n].y;
      staged[(i + 64) * kUnblockPitch + k] = v[n].z;
      staged[(i + 96) * kUnblockPitch + k] = v[n].w;
    }
  }
  __syncthreads();
  // Plain chunk e = r * (tiles / 4) + j holds dwords 4 j .. 4 j + 3 of row r,
  // for e = t, t + 1024, ...  All LDS reads first, then the stores.
  const int per_row = tiles / 4;
  uint4 w[kUnblockChunks];
#pragma unroll
  for (int n = 0; n < kUnblockChunks; ++n) {
    const int e = t + kUnblockThreads * n;
    if (e < chunks) {
      const int r = e / per_row, j = e - r * per_row;
      const uint32_t* src = &staged[r * kUnblockPitch + 4 * j];
      w[n] = make_uint4(src[0], src[1], src[2], src[3]);
    }
  }
#pragma unroll
  for (int n = 0; n < kUnblockChunks; ++n) {
    const int e = t + kUnblockThreads * n;
    if (e < chunks)
      store_line_nt(base + 16 * (int64_t)e, w[n]);
  }
}

hipError_t launch_unblock_inplace(uint8_t* m0, int64_t r0, int64_t c0, uint8_t* m1, int64_t r1, int64_t c1,
                                  hipStream_t stream) {
  const auto fits = [](const uint8_t* m, int64_t r, int64_t c) {
    return m == nullptr || (r % kTileRows == 0 && c % 16 == 0 && c > 0 && c <= kUnblockMaxCols &&
                            ((uintptr_t)m % 16) == 0);
  };
  if (!fits(m0, r0, c0) || !fits(m1, r1, c1))
    return hipErrorInvalidValue;
  const int64_t b0 = m0 != nullptr ? r0 / kTileRows : 0;
  const int64_t b1 = m1 != nullptr ? r1 / kTileRows : 0;
  if (b0 + b1 == 0)
    return hipSuccess;
  hipLaunchKernelGGL(unblock_kernel, dim3((unsigned)(b0 + b1)), dim3(kUnblockThreads), 0, stream, m0, c0, b0, m1, c1);
  return hipGetLastError();
}

}  // namespace mx
