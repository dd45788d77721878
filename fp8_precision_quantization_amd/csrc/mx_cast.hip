// bf16 -> MXFP8 cast along dim0 and dim1 from one read of the input
// (pytorch/ao page "triton kernel to cast to mx across dim0 and dim1",
// Summary), and the dim1-only cast of 3D expert weights ("[mxfp8 moe
// training] add compile support", Perf analysis item 4).
//
// Work decomposition (gfx950, wave64):
//   workgroup = 4 waves stacked along rows = a 128-row x 256-column tile;
//   wave      = 32 rows x 256 columns, one dim1 block height: lanes 0-31 hold
//               rows 0-15 and lanes 32-63 rows 16-31 of the same columns;
//   lane      = 16 rows x 8 columns, loaded as 16 x 16-byte row segments.
// Each load instruction of a wave reads two 512-byte row segments; loads and
// row-major stores are buffer instructions whose row offset sits in a scalar
// register, and the input loads are non-temporal.  A dim0 block (32 columns
// of one row) spans a quad of lanes and is reduced with two DPP moves; a dim1
// block (32 rows of one column) is split between lanes l and l + 32: an
// in-lane tree of packed 16-bit maxes, then one permlane32 swap.  The
// magnitudes are formed once for both.
//
// Stores are shaped for the memory system rather than for the lanes that
// produce them.  dim0 codes leave each wave as 256-byte row segments.  The
// dim1 codes of a column (16 bytes per lane) are staged in LDS, and once the
// four waves are done the workgroup writes each column's 128 rows as one full
// 128-byte line, eight lanes x 16 bytes per line; dim1 scale bytes are staged
// the same way and leave as one 4-byte run per column.  The barrier between
// the two orders LDS only: __syncthreads() would also wait for global memory.
//
// Cache policy of the stores, by timing on MI355X (outputs unchanged):
// - the stores that write whole 128-byte lines -- the staged dim1 codes and
//   the blocked scale chunks -- are non-temporal while the col-major output
//   is larger than 128 MiB (16384 x 16384, blocked scales: 215 -> 163 us
//   against ordinary stores), and written through to memory (sc0 sc1) up to
//   that size, where that is faster again (16640 x 5120 M-grouped: 63.1 ->
//   60.8 us; at 16384 x 16384 it would be 160.6 -> 201 us): 30 shapes from
//   4096 x 2048 to 32768 x 16384 split cleanly at that size, which is where
//   the two code matrices stop fitting the 256 MB memory-side cache (timed
//   on the dim0+dim1 casts; the dim1-only cast takes the same rule, and its
//   (16, 8192, 5120) workload, 640 MiB of codes, stays non-temporal: written
//   through it took 345 against 338 us);
// - the dim0 row segments, whose lines neighbouring lanes complete, are
//   written through (sc0 sc1: 16384 x 16384 161.0 -> 160.6 us, 16640 x 5120
//   63.5 -> 63.1 us; non-temporal there cost time);
// - the plain scale runs, whose lines neighbouring workgroups complete in
//   the L2, stay ordinary (written through they cost 1 us at 16640 x 5120).
//
// With BLK the scales come out directly in the 128x4 blocked layout that
// grouped GEMMs read ("[mxfp8 moe training] parallelize along col blocks in
// scale blocked format kernel for groups along K", Changes: 128x4 is the
// granularity of the swizzle), as the first page lists among its future
// improvements (swizzled scales written by the cast): a tile of 128 rows
// and 256 columns owns two 512-byte blocks of dim0 scales (128 rows x 4
// scale columns each) and two of dim1 scales (128 columns x 4 row blocks),
// so each is assembled in LDS and stored as whole 16-byte chunks, the
// padding bytes of a ragged edge written as zero by the tile that owns them.
//
// Workgroups are numbered so that each XCD (workgroups are dispatched
// round-robin over the 8 XCDs) works on a compact region of the matrix:
// row_group row tiles side by side, column tiles outermost.  Its L2 then
// merges the partial lines of the plain scale matrices, and the region's
// shape sets how long the contiguous runs of reads and stores are.  The
// shapes (per output form, see cast_args) and the non-temporal loads were
// chosen by timing on MI355X.
#include <type_traits>

#include "mx_device.h"
#include "mx_groups.h"
#include "mxcast.h"
#include "mx_launch.h"

namespace mx {

constexpr int kLaneRows = 16;
constexpr int kWaveRows = 32;
constexpr int kWaves = 4;
constexpr int kTileRows = kWaves * kWaveRows;   // 128
constexpr int kLaneCols = 8;
constexpr int kTileCols = 32 * kLaneCols;       // 256
constexpr int kXcds = 8;
constexpr int kSlots = kTileRows / 16;          // 16-byte slots per staged column (8)
constexpr int kLoadNT = 2;                      // cache-policy bits of the input loads: nt
constexpr int kStoreWT = 17;                    // ... of stores written through: sc0 sc1
constexpr int64_t kWriteThroughMax = 128 << 20; // largest col-major output whose lines are written through
constexpr uint32_t kRowGroupBlocked = 2;        // see cast_args
constexpr uint32_t kRowGroupPlain = 8;
constexpr uint32_t kRowGroupDim1 = 1024;

// 16 bytes that, across the lanes of one instruction, make up whole 128-byte
// lines, written through, at byte offset off of buffer rs.  (The
// non-temporal form is store_line_nt: as a buffer store it was ~1% slower at
// 16384 x 16384 and (16, 8192, 5120).)
__device__ __forceinline__ void store_line_wt(__amdgpu_buffer_rsrc_t rs, uint32_t off, const uint4& v) {
  __builtin_amdgcn_raw_buffer_store_b128((u32x4){v.x, v.y, v.z, v.w}, rs, off, 0, kStoreWT);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// LDS slot of 16 dim1 codes: column col (0..255), rows 16 * slot .. +15 of
// the tile.  The slot index is XOR-swizzled with bits of the column so that
// the eight lanes of a 128-byte LDS access hit eight different bank groups
// both when the producing lanes (columns 8 apart) write and when the storing
// lanes (one column, eight slots) read.
__device__ __forceinline__ int q1_slot(int col, int slot) { return col * kSlots + (slot ^ ((col >> 3) & 7)); }

// Finite-path parameters of two blocks at once: m holds two 15-bit amax
// patterns [a, b].  For each: byte = max(E - 8, 0) (E = exponent field), the
// clamp limit ((byte + 8) << 7) | 0x60 = bf16 pattern of 448 * 2^e, and the
// convert's scale operand.  The convert reads only the exponent field of
// that operand, so the limit shifted into place minus 8 << 23 is the scale.
struct PairParams {
  uint32_t t2_a, t2n_a, t2_b, t2n_b;
  float scale_a, scale_b;
};
__device__ __forceinline__ PairParams pair_params(uint32_t m) {
  PairParams p;
  const uint32_t t = max2(m & 0x7F807F80u, 0x04000400u) | 0x00600060u;
  p.t2_a = __builtin_amdgcn_perm(t, t, 0x01000100u);
  p.t2_b = __builtin_amdgcn_perm(t, t, 0x03020302u);
  p.t2n_a = p.t2_a | 0x80008000u;
  p.t2n_b = p.t2_b | 0x80008000u;
  p.scale_a = __uint_as_float((t << 16) - 0x04000000u);
  p.scale_b = __uint_as_float((t & 0xFFFF0000u) - 0x04000000u);
  return p;
}

__device__ __forceinline__ uint32_t fast_quant4(uint32_t x01, uint32_t x23, uint32_t t2, uint32_t t2n,
                                                float scale) {
  return cvt4_e4m3(clamp_mag2(x01, t2, t2n), clamp_mag2(x23, t2, t2n), scale);
}

// dim0 of a lane's 16 rows.  rm[i/2] = [row max of row i, row i+1] over the
// lane's 8 columns; after two DPP moves, the quad's block amax.  Codes: 8 per
// lane per row (one 256-byte segment per half-wave).  Scale bytes (one per
// quad): straight to the plain scale matrix (IMG = 0), or into an LDS image
// of the tile's scales, row i at s0_lds + img_off + i * IMG: the image of the
// tile's two 128x4 blocked tiles (IMG = 16) or a plain 128 x 8 image (8).
template <bool SPECIAL, int IMG>
__device__ __forceinline__ void dim0_rows(const uint4 (&d)[kLaneRows], const uint32_t (&rm)[kLaneRows / 2],
                                          bool quad_leader, __amdgpu_buffer_rsrc_t q0, int q0_off,
                                          __amdgpu_buffer_rsrc_t s0, int s0_off, uint32_t cols,
                                          uint32_t sb_cols, uint8_t* s0_lds, int img_off) {
#pragma unroll
  for (int i = 0; i < kLaneRows; i += 2) {
    uint32_t m = rm[i / 2];
    m = max2(m, quad_swap1(m));
    m = max2(m, quad_swap2(m));
    uint32_t qa0, qa1, qb0, qb1, ba, bb;
    if (SPECIAL) {
      BlockParams pa = block_params<true>(m & 0xFFFFu);
      BlockParams pb = block_params<true>(m >> 16);
      qa0 = quant4<true>(d[i].x, d[i].y, pa);
      qa1 = quant4<true>(d[i].z, d[i].w, pa);
      qb0 = quant4<true>(d[i + 1].x, d[i + 1].y, pb);
      qb1 = quant4<true>(d[i + 1].z, d[i + 1].w, pb);
      ba = pa.byte;
      bb = pb.byte;
    } else {
      const PairParams p = pair_params(m);
      qa0 = fast_quant4(d[i].x, d[i].y, p.t2_a, p.t2n_a, p.scale_a);
      qa1 = fast_quant4(d[i].z, d[i].w, p.t2_a, p.t2n_a, p.scale_a);
      qb0 = fast_quant4(d[i + 1].x, d[i + 1].y, p.t2_b, p.t2n_b, p.scale_b);
      qb1 = fast_quant4(d[i + 1].z, d[i + 1].w, p.t2_b, p.t2n_b, p.scale_b);
      ba = __float_as_uint(p.scale_a) >> 23;
      bb = __float_as_uint(p.scale_b) >> 23;
    }
    __builtin_amdgcn_raw_buffer_store_b64((u32x2){qa0, qa1}, q0, q0_off, (int)(i * cols), kStoreWT);
    __builtin_amdgcn_raw_buffer_store_b64((u32x2){qb0, qb1}, q0, q0_off, (int)((i + 1) * cols), kStoreWT);
    if (quad_leader) {
      if (IMG != 0) {
        // rows i, i+1 of the lane are consecutive rows of the tile
        s0_lds[img_off + i * IMG] = (uint8_t)ba;
        s0_lds[img_off + (i + 1) * IMG] = (uint8_t)bb;
      } else {
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)ba, s0, s0_off, (int)(i * sb_cols), 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)bb, s0, s0_off, (int)((i + 1) * sb_cols), 0);
      }
    }
  }
}

// One 16-byte chunk of a 128x4 blocked tile: tile row i (0..31) holds rows
// i, 32+i, 64+i, 96+i (4 bytes each, columns 0..3).  Bytes of rows at or past
// valid_blocks * 32 and of columns at or past valid_cols become 0.
__device__ __forceinline__ uint4 mask_chunk(uint4 v, int valid_blocks, int valid_cols) {
  const uint32_t cmask = valid_cols >= 4 ? 0xFFFFFFFFu : valid_cols <= 0 ? 0u : (1u << (8 * valid_cols)) - 1u;
  v.x = valid_blocks > 0 ? v.x & cmask : 0u;
  v.y = valid_blocks > 1 ? v.y & cmask : 0u;
  v.z = valid_blocks > 2 ? v.z & cmask : 0u;
  v.w = valid_blocks > 3 ? v.w & cmask : 0u;
  return v;
}

// dim1 of a lane's 16 rows: for each of its 8 columns, 16 codes into one LDS
// slot; the lower half-wave also records the column's scale byte.
template <bool SPECIAL>
__device__ __forceinline__ void dim1_cols(const uint4 (&d)[kLaneRows], const uint32_t (&cm)[4], int lc,
                                          int slot, bool lower, uint4* q1_lds, uint8_t* s1_lds, int wave) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t t2[2], t2n[2], bytes[2];
    float scale[2];
    BlockParams bp[2];
    if (SPECIAL) {
      bp[0] = block_params<true>(cm[k] & 0xFFFFu);
      bp[1] = block_params<true>(cm[k] >> 16);
      bytes[0] = bp[0].byte;
      bytes[1] = bp[1].byte;
    } else {
      const PairParams p = pair_params(cm[k]);
      t2[0] = p.t2_a;
      t2n[0] = p.t2n_a;
      scale[0] = p.scale_a;
      t2[1] = p.t2_b;
      t2n[1] = p.t2n_b;
      scale[1] = p.scale_b;
      bytes[0] = __float_as_uint(p.scale_a) >> 23;
      bytes[1] = __float_as_uint(p.scale_b) >> 23;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t sel = h ? 0x07060302u : 0x05040100u;
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < kLaneRows; i += 4) {
        // Column 2k+h of rows (i, i+1) and (i+2, i+3) as bf16 pairs.
        uint32_t p01 = __builtin_amdgcn_perm(word(d[i + 1], k), word(d[i], k), sel);
        uint32_t p23 = __builtin_amdgcn_perm(word(d[i + 3], k), word(d[i + 2], k), sel);
        w[i / 4] = SPECIAL ? quant4<true>(p01, p23, bp[h]) : fast_quant4(p01, p23, t2[h], t2n[h], scale[h]);
      }
      const int col = lc * kLaneCols + 2 * k + h;
      q1_lds[q1_slot(col, slot)] = make_uint4(w[0], w[1], w[2], w[3]);
      if (lower)
        s1_lds[col * kWaves + wave] = (uint8_t)bytes[h];
    }
  }
}

struct CastArgs {
  const uint16_t* x;
  int64_t rows, cols, rows_per_seg;
  uint32_t row_tiles, col_tiles, per_xcd;
  uint32_t row_group;  // row bands that run side by side on one XCD
  uint32_t rotate;     // XCD pieces start at points of their own (tile_of)
  uint32_t wt;         // whole-line stores written through, else non-temporal
  // Blocked scale outputs: column blocks of the dim0 scale matrix, of one
  // segment's dim1 scale matrix, and that matrix's size in bytes.
  int64_t ncb0, ncb1, seg_blk_bytes;
  uint8_t *q0, *s0, *q1, *s1;
  // M-grouped dim0 scales: group END offsets (device), their count, the
  // padded starts to write (device, may be null), the output's size in bytes.
  const int32_t* ends;
  int32_t groups;
  int64_t* out_starts;
  int64_t s0_bytes;
  // K-grouped dim1 scales (the same groups of rows, in 32-row blocks): the
  // padded column starts to write (device, may be null), the output's size.
  int64_t* s1_starts;
  int64_t s1_bytes;
};


struct Stage {
  uint4 q1[kTileCols * kSlots];   // dim1 codes, 128 rows x 256 columns
  uint32_t s1[kTileCols];         // dim1 scale bytes, 4 blocks per column
};
struct NoStage {};  // dim0-only casts stage nothing

// Work order: groups of row_group row tiles; inside a group, column tiles
// outermost; each XCD takes a contiguous run of this order, starting at a
// point of its own within the run.
__device__ __forceinline__ bool tile_of(uint32_t bid, uint32_t row_tiles, uint32_t col_tiles,
                                        uint32_t per_xcd, uint32_t row_group, bool rotate, uint32_t& rt,
                                        uint32_t& ct) {
  // rotate: XCD x starts its piece x quarters of a piece in, wrapping round
  // (when it pays; see cast_args).
  const uint32_t x = bid % kXcds, p = bid / kXcds;
  const uint32_t id = x * per_xcd + (rotate ? (p + x * (per_xcd / 4)) % per_xcd : p);
  if (id >= row_tiles * col_tiles)
    return false;
  const uint32_t group_items = row_group * col_tiles;
  const uint32_t g = id / group_items;
  const uint32_t within = id - g * group_items;
  const uint32_t gs = min(row_group, row_tiles - g * row_group);
  ct = within / gs;
  rt = g * row_group + (within - ct * gs);
  return true;
}

// 4 bytes of dim0 scales (scale columns 4 cb .. 4 cb + 3) of output row o of
// an M-grouped blocked matrix with ncb column blocks.
__device__ __forceinline__ void put_row_block(uint8_t* s0, int64_t ncb, int64_t o, int64_t cb, uint32_t v) {
  const int64_t idx = ((o >> 7) * ncb + cb) * 512 + (o & 31) * 16 + ((o & 127) >> 5) * 4;
  *reinterpret_cast<uint32_t*>(s0 + idx) = v;
}

// Store phase of the M-grouped dim0 scales of tile (rt, ct); img holds the
// tile's scales as 128 rows x 8 bytes.
__device__ __forceinline__ void mgrouped_scales(const CastArgs& a, const GroupTable& table, const uint8_t* img,
                                                uint32_t rt, uint32_t ct, int64_t tile_r, int valid_rows) {
  const int t = threadIdx.x;
  const int64_t nsc = a.cols / 32;
  const int64_t cb0 = 2 * (int64_t)ct, cb1 = cb0 + 1;
  const bool has1 = cb1 < a.ncb0;
  // scale columns past the matrix are padding: 0
  const int64_t v0 = min((int64_t)4, nsc - 4 * cb0), v1 = min((int64_t)4, nsc - 4 * cb1);
  const uint32_t m0 = v0 >= 4 ? 0xFFFFFFFFu : (1u << (8 * v0)) - 1u;
  const uint32_t m1 = v1 >= 4 ? 0xFFFFFFFFu : v1 <= 0 ? 0u : (1u << (8 * v1)) - 1u;
  // rows of the tile that belong to a group
  if (t < valid_rows) {
    const int64_t r = tile_r + t;
    const int g = find_source_group(table, a.groups, (int32_t)r);
    if (g >= 0) {
      const int64_t o = table.start[g] + (r - table.lo[g]);
      const uint2 w = reinterpret_cast<const uint2*>(img)[t];
      put_row_block(a.s0, a.ncb0, o, cb0, w.x & m0);
      if (has1)
        put_row_block(a.s0, a.ncb0, o, cb1, w.y & m1);
    }
  }
  // padding rows of the groups whose last row lies in this tile
  for (int g = find_source_group(table, a.groups, (int32_t)tile_r);
       g >= 0 && g < a.groups && table.hi[g] <= tile_r + valid_rows; ++g) {
    if (table.hi[g] == table.lo[g])
      continue;  // an empty group has no rows and no padding
    const int64_t o1 = table.start[g + 1];
    for (int64_t o = table.start[g] + (table.hi[g] - table.lo[g]) + t; o < o1; o += kWaves * 64) {
      put_row_block(a.s0, a.ncb0, o, cb0, 0u);
      if (has1)
        put_row_block(a.s0, a.ncb0, o, cb1, 0u);
    }
  }
  // bytes past the padded total (whole tiles end there): zero, split over
  // the workgroups of the last row of tiles
  if (rt == a.row_tiles - 1) {
    const int64_t lo = (int64_t)table.start[a.groups] * a.ncb0 * 4;   // multiple of 512
    const int64_t chunk = ((a.s0_bytes - lo + a.col_tiles - 1) / a.col_tiles + 15) / 16 * 16;
    const int64_t b0 = lo + (int64_t)ct * chunk, b1 = min(a.s0_bytes, b0 + chunk);
    for (int64_t b = b0 + 16 * t; b < b1; b += 16 * kWaves * 64) {
      if (b + 16 <= b1) {
        *reinterpret_cast<uint4*>(a.s0 + b) = make_uint4(0, 0, 0, 0);
      } else {
        for (int64_t j = b; j < b1; j += 4)
          *reinterpret_cast<uint32_t*>(a.s0 + j) = 0u;
      }
    }
  }
  if (blockIdx.x == 0 && a.out_starts != nullptr) {
    for (int g = t; g <= a.groups; g += kWaves * 64)
      a.out_starts[g] = table.start[g];
  }
}

// Group of scale column (32-row block) b under the K-group reading: the g
// with lo_g / 32 <= b < hi_g / 32, or -1 past the last group.
__device__ __forceinline__ int kgroup_of(const GroupTable& t, int groups, int64_t b) {
  if (groups <= 0 || b >= t.hi[groups - 1] / 32)
    return -1;
  int lo = 0, hi = groups - 1;  // smallest g with hi[g] / 32 > b lies in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (t.hi[mid] / 32 > b)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// Byte (c, p) of group g's blocked matrix in the K-grouped layout: the
// group's matrix (ceil128(C) rows x its padded width wp columns) starts at
// ceil128(C) * kstart[g].
__device__ __forceinline__ int64_t kgroup_index(int64_t cpad, int64_t kstart, int64_t wp, int64_t c, int64_t p) {
  return cpad * kstart + ((c >> 7) * (wp >> 2) + (p >> 2)) * 512 + (c & 31) * 16 + ((c & 127) >> 5) * 4 + (p & 3);
}

// Store phase of the K-grouped dim1 scales of tile (rt, ct): s1img[col] holds
// the four block scales (blocks 4 rt .. 4 rt + 3) of x column tc + col.
// - Each column's bytes go to their groups' matrices: one 4-byte store when
//   the tile's four blocks open a 4-column block of one group, else byte by
//   byte.
// - The padding columns of a group whose last block is in this row of
//   tiles are zeroed for this tile's columns.
// - The last column of tiles also zeroes the padding rows (x columns C ..
//   ceil128(C) - 1) of this row of tiles' blocks and of those padding
//   columns.
// - Bytes past the padded total are zeroed, split over the workgroups of
//   the last row of tiles.
__device__ inline void kgrouped_scales(const CastArgs& a, const GroupTable& table, const KStarts& ks,
                                       const uint32_t* s1img, uint32_t rt, uint32_t ct, int valid_rows,
                                       int valid_cols) {
  const int t = threadIdx.x;
  const int64_t C = a.cols;
  const int64_t cpad = (C + 127) / 128 * 128;
  const int64_t tc = (int64_t)ct * kTileCols;
  const int nblk = valid_rows / 32;
  const int64_t b0 = 4 * (int64_t)rt;
  // the tile's blocks: group, local column, padded width (uniform)
  int bg[kWaves];
  int64_t bp[kWaves], bw[kWaves];
#pragma unroll
  for (int j = 0; j < kWaves; ++j) {
    bg[j] = j < nblk ? kgroup_of(table, a.groups, b0 + j) : -1;
    bp[j] = bg[j] >= 0 ? b0 + j - table.lo[bg[j]] / 32 : 0;
    bw[j] = bg[j] >= 0 ? (table.hi[bg[j]] / 32 - table.lo[bg[j]] / 32 + 3) / 4 * 4 : 0;
  }
  const bool whole = nblk == kWaves && bg[0] >= 0 && bg[0] == bg[kWaves - 1] && (bp[0] & 3) == 0;
  if (t < valid_cols) {
    const int64_t c = tc + t;
    const uint32_t v = s1img[t];
    if (whole) {
      *reinterpret_cast<uint32_t*>(a.s1 + kgroup_index(cpad, ks.start[bg[0]], bw[0], c, bp[0])) = v;
    } else {
#pragma unroll
      for (int j = 0; j < kWaves; ++j)
        if (bg[j] >= 0)
          a.s1[kgroup_index(cpad, ks.start[bg[j]], bw[j], c, bp[j])] = (uint8_t)(v >> (8 * j));
    }
  }
  // groups whose last block lies in this row of tiles: their padding columns
  const bool last_ct = ct == a.col_tiles - 1;
  for (int g = max(0, kgroup_of(table, a.groups, b0)); g >= 0 && g < a.groups; ++g) {
    const int64_t klo = table.lo[g] / 32, khi = table.hi[g] / 32;
    if (khi > b0 + nblk)
      break;  // this group (and every later one) ends further down
    if (khi <= b0 || khi == klo)
      continue;  // ends above this row of tiles, or has no blocks
    const int64_t w = khi - klo, wp = (w + 3) / 4 * 4;
    // padding columns w .. wp - 1, this tile's columns (and, from the last
    // column of tiles, the padding rows)
    const int64_t c_end = last_ct ? cpad : tc + valid_cols;
    for (int64_t c = tc + t; c < c_end; c += kWaves * 64)
      for (int64_t p = w; p < wp; ++p)
        a.s1[kgroup_index(cpad, ks.start[g], wp, c, p)] = 0;
  }
  // padding rows of this row of tiles' blocks
  if (last_ct && cpad > C) {
    for (int64_t c = C + t; c < cpad; c += kWaves * 64)
#pragma unroll
      for (int j = 0; j < kWaves; ++j)
        if (bg[j] >= 0)
          a.s1[kgroup_index(cpad, ks.start[bg[j]], bw[j], c, bp[j])] = 0;
  }
  // bytes past the padded total (whole 512-byte tiles from there on)
  if (rt == a.row_tiles - 1) {
    const int64_t lo = cpad * ks.start[a.groups];
    const int64_t chunk = ((a.s1_bytes - lo + a.col_tiles - 1) / a.col_tiles + 15) / 16 * 16;
    const int64_t e0 = lo + (int64_t)ct * chunk, e1 = min(a.s1_bytes, e0 + chunk);
    for (int64_t e = e0 + 16 * t; e < e1; e += 16 * kWaves * 64) {
      if (e + 16 <= e1) {
        *reinterpret_cast<uint4*>(a.s1 + e) = make_uint4(0, 0, 0, 0);
      } else {
        for (int64_t j = e; j < e1; ++j)
          a.s1[j] = 0;
      }
    }
  }
  if (blockIdx.x == 0 && a.s1_starts != nullptr) {
    for (int g = t; g <= a.groups; g += kWaves * 64)
      a.s1_starts[g] = ks.start[g];
  }
}

// rows_per_seg: the rows of x form consecutive segments of this many rows
// (3D weights: one per expert; 2D: one segment).  Segment e's dim1 output is
// a (cols, rows_per_seg) matrix at e * cols * rows_per_seg, its scales a
// (cols, rows_per_seg / 32) matrix at e * cols * rows_per_seg / 32.
// BLK: the scale outputs are written in the 128x4 blocked layout instead of
// plain row-major matrices.  A tile's dim0 scales are exactly two whole
// blocked tiles (its 128 rows x 8 scale columns) and its dim1 scales two more
// (256 matrix rows x 4 scale columns), so every blocked tile, padding
// included, is written by exactly one workgroup.
// MGRP (dim0 + plain dim1 only): the dim0 scales are written in the M-grouped
// blocked layout (the blocked layout of each group of rows, each group
// padded to a multiple of 128 rows and placed at its padded start; the group
// table is rebuilt from the device offsets in every workgroup).  Each row's
// 8 scale bytes of a tile go to its output row as two 4-byte stores; the
// workgroup holding a group's last row zeroes the group's padding rows, and
// the last row of tiles zeroes the bytes past the padded total.
// KGRP (with MGRP and DIM1): the dim1 scales are written in the K-grouped
// blocked layout of the same groups counted in 32-row blocks (kgrouped_scales).
template <bool DIM0, bool DIM1, bool BLK, bool MGRP, bool KGRP = false>
__global__ __launch_bounds__(256) void cast_kernel(CastArgs a) {
  static_assert(!KGRP || (MGRP && DIM1 && !BLK), "K-grouped dim1 scales come with the M-grouped cast");
  __shared__ std::conditional_t<DIM1, Stage, NoStage> stage;
  // the tile's dim0 scales: two blocked tiles (BLK) or a plain image (MGRP)
  // read back as 16- and 8-byte words
  __shared__ __attribute__((aligned(16))) uint8_t s0_blk[(DIM0 && (BLK || MGRP)) ? 2 * 512 : 1];
  __shared__ std::conditional_t<MGRP, GroupTable, NoTable> table;
  __shared__ std::conditional_t<KGRP, KStarts, NoKStarts> kstarts;

  uint32_t rt, ct;
  if (!tile_of(blockIdx.x, a.row_tiles, a.col_tiles, a.per_xcd, a.row_group, a.rotate != 0, rt, ct))
    return;  // uniform over the workgroup
  // The wave index is uniform; saying so keeps the buffer descriptors built
  // from it in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;      // which 16 rows of the wave's 32
  const int lc = lane & 31;        // which 8 columns of the tile
  const int64_t cols = a.cols;
  const int64_t tile_r = (int64_t)rt * kTileRows;
  const int64_t r0 = tile_r + wave * kWaveRows;
  const int64_t tc = (int64_t)ct * kTileCols;
  // rows and cols are multiples of 32: a wave is fully in or out, and the 4
  // lanes of a dim0 block agree.
  const bool wave_on = r0 < a.rows;
  const bool on = wave_on && tc + lc * kLaneCols < cols;

  if (wave_on) {
    // Row i of this lane is row r0 + 16 * half + i; lanes past the last
    // column reread the first column of their rows (never stored).
    const uint32_t row_bytes = (uint32_t)(cols * 2);
    const int x_off = (int)(half * kLaneRows * row_bytes) + (on ? lc * 16 : 0);
    const __amdgpu_buffer_rsrc_t xs = buffer_rsrc(a.x + r0 * cols + tc, 0xFFFFFFFFu);
    uint4 d[kLaneRows];
#pragma unroll
    for (int i = 0; i < kLaneRows; ++i) {
      // non-temporal: the input is read once
      auto v = __builtin_amdgcn_raw_buffer_load_b128(xs, x_off, (int)(i * row_bytes), kLoadNT);
      d[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    if constexpr (MGRP) {
      // A few groups: wave 0 (always on) reads the ends with scalar loads
      // while its input loads are in flight, before its first store.  Read
      // with vector loads after the stores, they would wait for every one of
      // them: the vector memory counter counts stores too.
      if (wave == 0 && a.groups <= kScalarTableGroups)
        build_group_table_scalar(a.ends, a.groups, (int32_t)a.rows, kTileRows, table);
    }
    {
      // Magnitudes once; row maxima of row pairs and column maxima from them.
      uint32_t rm[kLaneRows / 2];
      uint32_t cm[4];
      {
        uint32_t mg[kLaneRows][4];
#pragma unroll
        for (int i = 0; i < kLaneRows; ++i) {
          mg[i][0] = mag2(d[i].x);
          mg[i][1] = mag2(d[i].y);
          mg[i][2] = mag2(d[i].z);
          mg[i][3] = mag2(d[i].w);
        }
#pragma unroll
        for (int i = 0; i < kLaneRows; i += 2) {
          const uint32_t ma = max2(max2(mg[i][0], mg[i][1]), max2(mg[i][2], mg[i][3]));
          const uint32_t mb = max2(max2(mg[i + 1][0], mg[i + 1][1]), max2(mg[i + 1][2], mg[i + 1][3]));
          rm[i / 2] = max2(__builtin_amdgcn_perm(mb, ma, 0x05040100u),   // [ma.lo, mb.lo]
                           __builtin_amdgcn_perm(mb, ma, 0x07060302u));  // [ma.hi, mb.hi]
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t t[kLaneRows / 2];
#pragma unroll
          for (int i = 0; i < kLaneRows / 2; ++i)
            t[i] = max2(mg[2 * i][k], mg[2 * i + 1][k]);
#pragma unroll
          for (int w = kLaneRows / 4; w >= 1; w >>= 1)
#pragma unroll
            for (int i = 0; i < w; ++i)
              t[i] = max2(t[i], t[i + w]);
          // combine with the partner lane holding the other 16 rows
          auto sw = __builtin_amdgcn_permlane32_swap(t[0], t[0], false, false);
          cm[k] = max2(sw[0], sw[1]);
        }
      }
      const uint32_t all = max2(max2(cm[0], cm[1]), max2(cm[2], cm[3]));
      const bool special = on && ((all & 0xFFFFu) >= kInfBits || (all >> 16) >= kInfBits);
      // Any +-Inf or NaN among the wave's lanes sends the wave down the
      // general path (uniform branch); finite data never pays for it.
      const bool any_special = __any(special);
      if (on) {
        if constexpr (DIM1) {
          const int slot = 2 * wave + half;
          uint8_t* s1b = reinterpret_cast<uint8_t*>(stage.s1);
          if (any_special)
            dim1_cols<true>(d, cm, lc, slot, half == 0, stage.q1, s1b, wave);
          else
            dim1_cols<false>(d, cm, lc, slot, half == 0, stage.q1, s1b, wave);
        }
        if constexpr (DIM0) {
          const uint32_t sb = (uint32_t)(cols / 32);
          const __amdgpu_buffer_rsrc_t q0 = buffer_rsrc(a.q0 + r0 * cols + tc, 0xFFFFFFFFu);
          const __amdgpu_buffer_rsrc_t s0 = buffer_rsrc(a.s0 + r0 * (cols / 32) + tc / 32, 0xFFFFFFFFu);
          const int q0_off = (int)(half * kLaneRows * (uint32_t)cols) + lc * kLaneCols;
          const int s0_off = (int)(half * kLaneRows * sb) + (lc >> 2);
          const bool leader = (lc & 3) == 0;
          // blocked image: tile (lc >> 4), row 16 * half + i of sub-block
          // `wave`, column (lc >> 2) & 3; plain image: row 32 * wave + 16 *
          // half + i, column lc >> 2
          constexpr int kImg = BLK ? 16 : MGRP ? 8 : 0;
          const int img_off = BLK ? (lc >> 4) * 512 + half * 256 + wave * 4 + ((lc >> 2) & 3)
                                  : (wave * kWaveRows + half * kLaneRows) * 8 + (lc >> 2);
          if (any_special)
            dim0_rows<true, kImg>(d, rm, leader, q0, q0_off, s0, s0_off, (uint32_t)cols, sb, s0_blk, img_off);
          else
            dim0_rows<false, kImg>(d, rm, leader, q0, q0_off, s0, s0_off, (uint32_t)cols, sb, s0_blk, img_off);
        }
      }
    }
  }

  if constexpr (MGRP) {
    if (wave == 0) {
      if (a.groups > kScalarTableGroups)
        build_group_table(a.ends, a.groups, (int32_t)a.rows, kTileRows, table);
      if constexpr (KGRP)
        build_kstarts(table, a.groups, kstarts);
    }
  }
  if constexpr (DIM1 || (DIM0 && (BLK || MGRP))) {
    // Every wave reaches the barrier; it orders LDS only (no wait on
    // global memory).
    lds_barrier();
  }
  const int valid_rows = (int)min((int64_t)kTileRows, a.rows - tile_r);   // multiple of 32
  const int valid_cols = (int)min((int64_t)kTileCols, cols - tc);
  if constexpr (DIM0 && BLK) {
    // Two blocked tiles (scale columns 8 ct .. 8 ct + 7), 32 chunks each.
    if (wave == 0) {
      const int t = lane >> 5, i = lane & 31;
      const int64_t cb = 2 * (int64_t)ct + t;
      if (cb < a.ncb0) {
        uint4 v = reinterpret_cast<const uint4*>(s0_blk)[t * 32 + i];
        v = mask_chunk(v, valid_rows / 32, (int)min((int64_t)4, cols / 32 - 4 * cb));
        if (a.wt != 0) {
          // The workgroup's two blocked tiles are 1024 consecutive bytes.
          const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.s0 + ((int64_t)rt * a.ncb0 + 2 * (int64_t)ct) * 512, 1024);
          store_line_wt(rs, lane * 16, v);
        } else {
          store_line_nt(a.s0 + ((int64_t)rt * a.ncb0 + cb) * 512 + i * 16, v);
        }
      }
    }
  }
  if constexpr (DIM0 && MGRP)
    mgrouped_scales(a, table, s0_blk, rt, ct, tile_r, valid_rows);
  if constexpr (DIM1) {
    const Stage& st = stage;
    const int64_t rps = a.rows_per_seg;
    // Segment of the band's first row; the band crosses at most a few
    // segment ends (segments are multiples of 32 rows).
    const int64_t seg0 = tile_r / rps;
    const int64_t off0 = tile_r - seg0 * rps;
    const bool one_seg = off0 + valid_rows <= rps;
    const int64_t seg_blocks = rps / 32;
    // Codes: 8 lanes per column, 16 bytes each; a wave covers 8 columns per pass.
    const int slot = threadIdx.x & 7;
    // Written through: within one segment the tile's columns are output rows
    // tc .. tc + 255 of that segment, rps bytes apart, which one buffer
    // covers while they span less than 2 GiB (else non-temporal).  The loop
    // is written once per policy, the choice taken outside it.
    const bool wt = a.wt != 0 && one_seg && (int64_t)kTileCols * rps < (1ll << 31);
    const auto put_codes = [&](auto wt_tag) {
      constexpr bool WT = decltype(wt_tag)::value;
      const __amdgpu_buffer_rsrc_t q1rs = buffer_rsrc(a.q1 + (seg0 * cols + tc) * rps, WT ? (uint32_t)(kTileCols * rps) : 0u);
#pragma unroll 4
      for (int pass = 0; pass < kTileCols / 32; ++pass) {
        const int col = pass * 32 + (threadIdx.x >> 3);
        if (col < valid_cols && slot * 16 < valid_rows) {
          const uint4 w = st.q1[q1_slot(col, slot)];
          if constexpr (WT) {
            store_line_wt(q1rs, (uint32_t)(col * rps + off0 + slot * 16), w);
          } else {
            int64_t seg = seg0, off = off0 + slot * 16;
            while (off >= rps) {
              off -= rps;
              ++seg;
            }
            store_line_nt(a.q1 + (seg * cols + tc + col) * rps + off, w);
          }
        }
      }
    };
    if (wt)
      put_codes(std::true_type{});
    else
      put_codes(std::false_type{});
    if constexpr (BLK) {
      // Two blocked tiles of the segment's dim1 scale matrix: matrix rows
      // (x columns) tc .. tc + 255, scale column block off0 / 128 (the host
      // guarantees that a tile never crosses a segment end here).  Chunk i of
      // tile t holds columns 128 t + 32 s + i, s = 0..3, 4 row blocks each.
      if (wave == 1) {
        const int t = lane >> 5, i = lane & 31;
        const int64_t rb = 2 * (int64_t)ct + t;
        if (rb * 128 < cols) {
          uint4 v = make_uint4(st.s1[128 * t + i], st.s1[128 * t + 32 + i], st.s1[128 * t + 64 + i],
                               st.s1[128 * t + 96 + i]);
          const int64_t left = cols - (tc + 128 * t + i);   // columns from this one on
          const int valid_s = (int)min((int64_t)4, max((int64_t)0, (left + 31) / 32));
          v = mask_chunk(v, valid_s, valid_rows / 32);
          uint8_t* pair = a.s1 + seg0 * a.seg_blk_bytes + (2 * (int64_t)ct * a.ncb1 + off0 / 128) * 512;
          if (a.wt != 0 && (a.ncb1 + 1) * 512 < (1ll << 31)) {
            // Tile t of the pair starts ncb1 blocked tiles after tile 0.
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(pair, (uint32_t)((a.ncb1 + 1) * 512));
            store_line_wt(rs, (uint32_t)(t * a.ncb1 * 512 + i * 16), v);
          } else {
            store_line_nt(pair + t * a.ncb1 * 512 + i * 16, v);
          }
        }
      }
    } else if constexpr (KGRP) {
      kgrouped_scales(a, table, kstarts, st.s1, rt, ct, valid_rows, valid_cols);
    } else {
      // Plain scales: one thread per column, the four 32-row blocks of the band.
      const int col = threadIdx.x;
      if (col < valid_cols) {
        const uint32_t v = st.s1[col];
        const int nblk = valid_rows / 32;
        uint8_t* dst = a.s1 + (seg0 * cols + tc + col) * seg_blocks + off0 / 32;
        if (one_seg && nblk == kWaves && ((uintptr_t)dst % 4) == 0) {
          *reinterpret_cast<uint32_t*>(dst) = v;
        } else {
          for (int b = 0; b < nblk; ++b) {
            int64_t seg = seg0, off = off0 + 32 * b;
            while (off >= rps) {
              off -= rps;
              ++seg;
            }
            a.s1[(seg * cols + tc + col) * seg_blocks + off / 32] = (uint8_t)(v >> (8 * b));
          }
        }
      }
    }
  }
}

static CastArgs cast_args(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_seg,
                          uint8_t* q0, uint8_t* s0, uint8_t* q1, uint8_t* s1, bool blocked, int64_t* blocks) {
  CastArgs a;
  a.x = x;
  a.rows = rows;
  a.cols = cols;
  a.rows_per_seg = rows_per_seg;
  a.q0 = q0;
  a.s0 = s0;
  a.q1 = q1;
  a.s1 = s1;
  const int64_t rt = (rows + kTileRows - 1) / kTileRows;
  const int64_t ct = (cols + kTileCols - 1) / kTileCols;
  const int64_t per = (rt * ct + kXcds - 1) / kXcds;
  a.row_tiles = (uint32_t)rt;
  a.col_tiles = (uint32_t)ct;
  a.per_xcd = (uint32_t)per;
  // Row tiles per XCD group, chosen by timing on MI355X at 16384 x 16384
  // and (16 * 8192) x 5120: the dim0+dim1 cast with blocked scales favours
  // the widest groups, with plain scales somewhat taller ones (the tiles
  // that share a plain scale line then run together on one XCD), the
  // dim1-only cast one segment's height (all of its stores are col-major: an
  // XCD walking a segment's whole column strip writes each of its output rows
  // from end to end, 128 bytes per tile; at (16 * 8192) x 5120, 64 row tiles
  // 345 us against 352 with 32, 355 with 128, 353 with 1024 and 384 with 16).
  a.row_group = q0 != nullptr ? (blocked ? kRowGroupBlocked : kRowGroupPlain)
                              : (uint32_t)std::min<int64_t>(kRowGroupDim1,
                                                            std::max<int64_t>(1, rows_per_seg / kTileRows));
  // With every XCD at the start of its piece, XCDs whose pieces begin a
  // multiple of 4 KiB apart in the col-major output (pieces of whole row
  // bands, per / ct row tiles of 128 bytes there, a multiple of 32) write it
  // at addresses that far apart at the same moment, which cost up to a fifth
  // of the time; starting each XCD at a point of its own removes that
  // (32768 x 8192, blocked scales: 199 -> 163 us; 65536 x 5120, plain or
  // grouped scales: 292-297 -> 263 us).  Casts whose stores all write whole
  // lines (blocked scales, dim1 only) are as fast or faster rotated at every
  // shape timed (16384 x 2048: 29.8 -> 28.0 us; 16384 x 16384 unchanged);
  // the plain and grouped ones, whose partial scale lines merge in the L2 of
  // the XCD running the neighbouring tiles, are slower rotated elsewhere
  // (16384 x 16384: 185 against 193 us).
  a.rotate = q0 == nullptr || blocked || (per % ct == 0 && (per / ct) % 32 == 0) ? 1u : 0u;
  a.wt = q1 != nullptr && rows * cols <= kWriteThroughMax ? 1u : 0u;
  a.ends = nullptr;
  a.groups = 0;
  a.out_starts = nullptr;
  a.s0_bytes = 0;
  a.s1_starts = nullptr;
  a.s1_bytes = 0;
  a.ncb0 = (cols / 32 + 3) / 4;
  a.ncb1 = (rows_per_seg / 32 + 3) / 4;
  a.seg_blk_bytes = (cols + 127) / 128 * 128 * (a.ncb1 * 4);
  *blocks = per * kXcds;
  return a;
}

int64_t cast_grid_blocks(int64_t rows, int64_t cols) {
  int64_t blocks;
  cast_args(nullptr, rows, cols, rows, nullptr, nullptr, nullptr, nullptr, false, &blocks);
  return blocks;
}

// The dim1-only casts (3D expert weights) run faster with 2 workgroups per
// CU than with the 4 their registers allow: each launch reserves this much
// LDS beyond what the kernel uses, so that only two fit a CU's 160 KiB.
// Timed on MI355X at (16, 8192, 5120), A/B/A/B: with blocked scales 345.8
// -> 340.9 us, with plain scales 359.7 -> 345.1 us (3 per CU: 344.6 and
// 356.3 us).  The dim0+dim1 casts are slower with fewer than 3 (16384^2:
// 160.9 -> 164.2 us at 2 per CU).
constexpr size_t kDim1OnlyExtraLds = 20 * 1024;

template <bool DIM0, bool DIM1, bool BLK, bool MGRP = false, bool KGRP = false>
static hipError_t launch_cast(const CastArgs& a, int64_t blocks, hipStream_t stream) {
  const size_t extra_lds = (!DIM0 && DIM1) ? kDim1OnlyExtraLds : 0;
  hipLaunchKernelGGL((cast_kernel<DIM0, DIM1, BLK, MGRP, KGRP>), dim3((unsigned)blocks), dim3(kWaves * 64),
                     extra_lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_cast_any(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_seg,
                           uint8_t* q0, uint8_t* s0, uint8_t* q1, uint8_t* s1, bool blocked,
                           hipStream_t stream) {
  int64_t blocks;
  const CastArgs a = cast_args(x, rows, cols, rows_per_seg, q0, s0, q1, s1, blocked, &blocks);
  const bool d0 = q0 != nullptr, d1 = q1 != nullptr;
  if (blocked) {
    if (d0 && d1)
      return launch_cast<true, true, true>(a, blocks, stream);
    if (d0)
      return launch_cast<true, false, true>(a, blocks, stream);
    return launch_cast<false, true, true>(a, blocks, stream);
  }
  if (d0 && d1)
    return launch_cast<true, true, false>(a, blocks, stream);
  if (d0)
    return launch_cast<true, false, false>(a, blocks, stream);
  return launch_cast<false, true, false>(a, blocks, stream);
}

hipError_t launch_cast_mgrouped(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* ends,
                                int32_t groups, uint8_t* q0, uint8_t* s0_grouped, int64_t s0_bytes,
                                int64_t* out_starts, uint8_t* q1, uint8_t* s1, hipStream_t stream) {
  int64_t blocks;
  CastArgs a = cast_args(x, rows, cols, rows, q0, s0_grouped, q1, s1, false, &blocks);
  a.ends = ends;
  a.groups = groups;
  a.out_starts = out_starts;
  a.s0_bytes = s0_bytes;
  if (q1 != nullptr)
    return launch_cast<true, true, false, true>(a, blocks, stream);
  return launch_cast<true, false, false, true>(a, blocks, stream);
}

hipError_t launch_cast_grouped_blocked(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* ends,
                                       int32_t groups, uint8_t* q0, uint8_t* s0_grouped, int64_t s0_bytes,
                                       int64_t* row_starts, uint8_t* q1, uint8_t* s1_grouped, int64_t s1_bytes,
                                       int64_t* col_starts, hipStream_t stream) {
  int64_t blocks;
  CastArgs a = cast_args(x, rows, cols, rows, q0, s0_grouped, q1, s1_grouped, false, &blocks);
  a.ends = ends;
  a.groups = groups;
  a.out_starts = row_starts;
  a.s0_bytes = s0_bytes;
  a.s1_starts = col_starts;
  a.s1_bytes = s1_bytes;
  return launch_cast<true, true, false, true, true>(a, blocks, stream);
}

}  // namespace mx
