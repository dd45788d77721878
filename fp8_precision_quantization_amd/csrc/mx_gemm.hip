// MX-scaled GEMM on gfx950's block-scaled MFMA: the consumer of the dim0
// casts ("[mxfp8 moe training] add compile support", Perf analysis item 1:
// MXFP8 grouped GEMMs of the (16640, 5120) activations, grouped along M,
// against per-group (8192, 5120) weights).
//
//   C[m][n] = sum over k of A(m, k) * B(n, k),  A(m, k) = e4m3(qa[m][k]) *
//   2^(S_A(m, k / 32) - 127), B likewise: both operands K-major, as the dim0
//   cast writes them (codes (rows, K)), the scales S in the 128 x 4 blocked
//   layout the casts can write directly.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies a 32 x 64 slab of A by a
// 64 x 32 slab of B and applies one e8m0 scale per row and 32-element block
// of K to each operand.  Its lane layout, measured on MI355X with an
// in-bounds probe of random operands: lane l holds row (or column) l % 32;
// its bytes 0-15 are K 16 (l / 32) .. +15 of the step's first 32-block and
// bytes 16-31 the same of the second block; the scale of block h of row r
// comes from lane r + 32 h (byte 0 of its scale register); result register
// v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.  The
// instruction sums a step's 64 products with less than binary32 precision
// (measured: within 3.4e-4 of the largest product of the step); the fp32
// accumulator carries the sum across steps.
//
// Work decomposition: a 256-thread workgroup owns a 256 x 256 tile of C;
// wave w its (w / 2, w % 2) 128 x 128 quarter = 4 x 4 MFMA blocks, whose
// 256 accumulators live in the accumulation registers.  K advances in
// stages of 128 bytes.  Every load instruction of a wave brings 8 whole
// 128-byte rows of A or B straight from memory into LDS (buffer loads to
// LDS, 16 bytes per lane in lane order), one stage (32 KiB of A, 32 KiB of
// B) into one half of a double-buffered area while the MFMAs work on the
// other.  Each wave reads its MFMA operands from LDS with 16-byte reads.
// In LDS a row's eight 16-byte chunks are permuted by an XOR of the row
// index (f below), applied through the loads' per-lane source offsets, so
// that the 16 lanes of one LDS read phase, which read one chunk of 16
// consecutive rows, hit distinct banks.  Scales come from the blocked
// layout: a wave's 128 rows of A (or B) are one row of 128 x 4 tiles, and
// one 16-byte load per lane and stage gives the lane its row's four block
// scales for each of its four row slabs.
//
// Buffer ranges end at the tile's last row, so rows past M or N read as
// zero; chunks past K load zero and their blocks' scales are the layout's
// zero padding.  Tiles are ordered in bands of 8 tile rows, column by
// column, and the ordered list is cut into 8 contiguous pieces, one per XCD
// (workgroups are dealt to the XCDs round-robin), so that each XCD's L2
// sees a compact region of A rows and B columns.  The output tile leaves
// through LDS as whole rows of 16-byte stores (the epilogue below).
//
// Grouped along M: the tiles of group g cover its rows [lo_g, hi_g) in
// 256-row steps (the group table of the blocked layouts, rebuilt from the
// device offsets in each workgroup); A's scales are the M-grouped blocked
// layout (groups padded to 128 rows), B and its scales are group g's (N, K)
// slice.  Rows past the last end are not written.
//
// Grouped along K (the weight gradient): one (M, N) output per group, over
// the group's K range; the scales are the K-grouped blocked layouts.
//
// Grouped either way, each group's ordered tiles are cut into 8 pieces, one
// per XCD, and an XCD runs its pieces group after group, so that the chip
// streams one group's operands at a time.
#include "mx_device.h"
#include "mx_groups.h"
#include "mxcast.h"
#include "mx_launch.h"

#include <type_traits>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kGemmThreads = 256;
constexpr int kGemmTile = 256;                 // rows and columns of C per workgroup
constexpr int kGemmTK = 128;                   // K bytes per LDS stage
constexpr int kGemmWaveBlocks = 4;             // 32 x 32 MFMA blocks per wave along M and along N
constexpr int kGemmLoadRows = kGemmThreads * 16 / kGemmTK;   // rows per load instruction (32)
constexpr int kGemmLoads = kGemmTile / kGemmLoadRows;        // load instructions per operand and stage (8)
constexpr int kGemmStageBytes = kGemmTile * kGemmTK;         // one operand's stage (32 KiB)
constexpr int kGemmBand = 8;                   // tile rows per band of the tile order
constexpr int kGemmOrderMax = 64;              // grouped along K: groups ordered by K length up to this count

struct GemmArgs {
  const uint8_t *qa, *sa, *qb, *sb;
  int64_t m, n, k;
  void* c;
  const int32_t* ends;
  int32_t groups;
  int64_t sb_bytes;            // bytes of one group's blocked B scales
  uint32_t tiles_m, tiles_n;   // tile grid (tiles_m includes one spare tile per group when grouped)
  uint32_t per_xcd;            // tiles per XCD
};

// Position of 16-byte chunk c of a stage row in LDS (bytes from the
// operand's stage base).  The XOR keeps a read of one chunk by 16
// consecutive rows, and a write of a row's 8 chunks by 8 lanes, on
// distinct banks.
__device__ __forceinline__ int lds_chunk(int row, int c) {
  return row * kGemmTK + 16 * (c ^ ((row & 7) ^ ((row >> 3) & 1)));
}

__device__ __forceinline__ int32_t wave_sum(int32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1)
    v += __shfl_xor(v, d);
  return v;
}

// Two binary32 values -> their bf16 bits, nearest-even, packed with the
// first in the low half: gfx950's v_cvt_pk_bf16_f32, one instruction for
// both.  Checked on MI355X against a software nearest-even rounding over
// every binary32 bit pattern: identical for all non-NaN inputs (subnormal
// results and overflow to Inf included); NaN stays NaN.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
// One value, for the per-element stores of outputs whose rows are not whole
// 16-byte chunks (the same rounding; NaN -> 0x7FC0).  With this path the
// bf16 kernels keep 12 accumulators in scratch between the main loop and the
// epilogue (12 dword stores per lane and tile, reloaded only on this path);
// converting this path in pairs with pack_bf16 as well removes them but
// changes the register allocation of the main loop, which then ran 8%
// slower (dense 611 -> 662 us).
__device__ __forceinline__ uint16_t to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u)
    return 0x7FC0u;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

enum : int { kGemmDense = 0, kGemmGroupsM = 1, kGemmGroupsK = 2 };

template <int MODE, bool BF16>
__global__ __launch_bounds__(kGemmThreads) void mx_gemm_kernel(GemmArgs a) {
  constexpr bool GROUPED = MODE == kGemmGroupsM;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kGemmStageBytes];   // [stage][A, B]

  // tile order: XCD x owns ordered tiles [x * per_xcd, (x + 1) * per_xcd).
  // Grouped along K there is one grid of tiles per group and each group's
  // ordered tiles are cut into 8 pieces of per_xcd, one per XCD; an XCD
  // runs its piece of every group, one group after the other, the group
  // with the longest K range first (the groups' K lengths differ widely,
  // and short tiles last keep the CUs' finishing times close together).
  // Grouped along M the same holds: each group's tiles are cut into 8
  // pieces and the XCDs run the groups one after another, so that the
  // chip works on one group's weights at a time (all groups' weights at
  // once would not fit the memory-side cache next to A).
  const uint32_t tiles = a.tiles_m * a.tiles_n;
  uint32_t id = (blockIdx.x % 8) * a.per_xcd + blockIdx.x / 8;
  uint32_t kslot = 0;   // grouped along K: this tile's place in the group order
  if constexpr (MODE == kGemmGroupsK) {
    kslot = (blockIdx.x / 8) / a.per_xcd;
    id = (blockIdx.x % 8) * a.per_xcd + (blockIdx.x / 8) % a.per_xcd;
    if (kslot >= (uint32_t)a.groups)
      return;  // uniform, before any barrier
  }
  if (MODE != kGemmGroupsM && id >= tiles)
    return;  // uniform, before any barrier
  // band order over a grid of tile rows: bands of 8 tile rows, column by column
  auto band_tile = [&](uint32_t i, uint32_t rows_of_tiles, uint32_t& m_t, uint32_t& n_t) {
    const uint32_t band = i / (kGemmBand * a.tiles_n);
    const uint32_t band_rows = min((uint32_t)kGemmBand, rows_of_tiles - band * kGemmBand);
    const uint32_t within = i - band * kGemmBand * a.tiles_n;
    m_t = band * kGemmBand + within % band_rows;
    n_t = within / band_rows;
  };
  uint32_t tm = 0, tn = 0;
  if constexpr (MODE != kGemmGroupsM)
    band_tile(id, a.tiles_m, tm, tn);

  // k: the reduction length of this tile; ld: the operands' row length
  int64_t k = a.k;
  const int64_t ld = a.k;
  const uint8_t* qa = a.qa;
  const uint8_t* qb = a.qb;
  const uint8_t* sa = a.sa;
  const uint8_t* sb = a.sb;
  void* c = a.c;
  int64_t strip_blocks = (k / 32 + 3) / 4;   // 128 x 4 tiles along a row of the scale layouts
  int64_t row0, rows_valid, srow0;
  // Grouped along K, stages stay on 128-byte boundaries of the operand rows
  // (a stage that straddles two cache lines per row costs about a third
  // more): the group's first stage starts kofs = 32 d bytes before its first
  // block, d = (first block) % 4, and its chunks outside the group load zero.
  int kofs = 0;
  if constexpr (MODE == kGemmGroupsK) {
    // Group kg's K range: 32-row (here 32-column) blocks [lo / 32, hi / 32)
    // of its clamped token range; its scales are its own blocked matrices in
    // the K-grouped layouts of A and B, at ceil128(rows) * kstart[kg].  The
    // tables borrow the B half of LDS stage 1 until the first stages load.
    static_assert(sizeof(GroupTable) + sizeof(KStarts) + kGemmOrderMax * sizeof(int32_t) <= kGemmStageBytes,
                  "group tables fit a stage half");
    GroupTable& table = *reinterpret_cast<GroupTable*>(lds[1][1]);
    KStarts& kst = *reinterpret_cast<KStarts*>(lds[1][1] + sizeof(GroupTable));
    int32_t* order = reinterpret_cast<int32_t*>(lds[1][1] + sizeof(GroupTable) + sizeof(KStarts));
    if (threadIdx.x < 64) {
      if (a.groups <= kScalarTableGroups)
        build_group_table_scalar(a.ends, a.groups, (int32_t)a.k, 32, table);
      else
        build_group_table(a.ends, a.groups, (int32_t)a.k, 32, table);
      build_kstarts(table, a.groups, kst);
      // up to 64 groups: longest block count first, ties by index (lane g
      // counts the groups that go before it)
      if (a.groups <= kGemmOrderMax) {
        const int g = threadIdx.x;
        const int32_t len = g < a.groups ? table.hi[g] / 32 - table.lo[g] / 32 : -1;
        int rank = 0;
        for (int q = 0; q < a.groups; ++q) {
          const int32_t lq = __shfl(len, q);
          rank += (lq > len) || (lq == len && q < g);
        }
        if (g < a.groups)
          order[rank] = g;
      }
    }
    lds_barrier();
    const int kg = a.groups <= kGemmOrderMax ? __builtin_amdgcn_readfirstlane(order[kslot]) : (int)kslot;
    const int32_t klo = __builtin_amdgcn_readfirstlane(table.lo[kg]) / 32;
    const int32_t khi = __builtin_amdgcn_readfirstlane(table.hi[kg]) / 32;
    const int32_t ks = __builtin_amdgcn_readfirstlane(kst.start[kg]);
    lds_barrier();   // every wave is done with the tables
    k = 32 * (int64_t)(khi - klo);
    strip_blocks = (khi - klo + 3) / 4;
    kofs = 32 * (klo % 4);
    qa += 32 * (int64_t)klo - kofs;
    qb += 32 * (int64_t)klo - kofs;
    sa += (a.m + 127) / 128 * 128 * (int64_t)ks;
    sb += (a.n + 127) / 128 * 128 * (int64_t)ks;
    c = static_cast<uint8_t*>(c) + (int64_t)kg * a.m * a.n * (BF16 ? 2 : 4);
    row0 = (int64_t)tm * kGemmTile;
    rows_valid = min((int64_t)kGemmTile, a.m - row0);
    srow0 = row0;
  } else if constexpr (GROUPED) {
    // The group table and the XCD piece starts borrow the B half of LDS
    // stage 1 until the first stages are loaded.  (One LDS object keeps the
    // compiler able to tell the loads into one stage from the reads of the
    // other.)
    static_assert(sizeof(GroupTable) + (MX_MAX_GROUPS + 1) * sizeof(int32_t) <= kGemmStageBytes,
                  "group tables fit a stage half");
    GroupTable& table = *reinterpret_cast<GroupTable*>(lds[1][1]);
    int32_t* xs = reinterpret_cast<int32_t*>(lds[1][1] + sizeof(GroupTable));
    if (threadIdx.x < 64) {
      if (a.groups <= kScalarTableGroups)
        build_group_table_scalar(a.ends, a.groups, (int32_t)a.m, kGemmTile, table);
      else
        build_group_table(a.ends, a.groups, (int32_t)a.m, kGemmTile, table);
      build_piece_starts(table, a.groups, kGemmTile, a.tiles_n, xs);
    }
    lds_barrier();
    // Values read from LDS are per-lane to the compiler; readfirstlane
    // makes them scalar (they are the same in every lane), so that the
    // buffer descriptors built from them stay in scalar registers.
    // XCD x's p-th tile: piece p - xs[g] of group g, the last g with
    // xs[g] <= p (xs[G] = the pieces per XCD in all).
    const int32_t p = (int32_t)(blockIdx.x / 8), x = (int32_t)(blockIdx.x % 8);
    if (p >= __builtin_amdgcn_readfirstlane(xs[a.groups]))
      return;  // uniform; no barrier follows
    int glo = 0, ghi = a.groups;   // xs[glo] <= p < xs[ghi]
    while (ghi - glo > 1) {
      const int mid = (glo + ghi) >> 1;
      if (xs[mid] <= p)
        glo = mid;
      else
        ghi = mid;
    }
    const int g = __builtin_amdgcn_readfirstlane(glo);
    const int32_t lo = __builtin_amdgcn_readfirstlane(table.lo[g]);
    const int32_t hi = __builtin_amdgcn_readfirstlane(table.hi[g]);
    const uint32_t trows = (uint32_t)(__builtin_amdgcn_readfirstlane(table.start[g + 1]) -
                                      __builtin_amdgcn_readfirstlane(table.start[g])) / kGemmTile;
    const uint32_t tg = trows * a.tiles_n, pg = (tg + 7) / 8;
    const uint32_t idx = (uint32_t)x * pg + (uint32_t)(p - __builtin_amdgcn_readfirstlane(xs[g]));
    if (idx >= tg)
      return;  // uniform; no barrier follows
    band_tile(idx, trows, tm, tn);
    const int32_t r0 = lo + (int32_t)tm * kGemmTile;
    row0 = r0;
    rows_valid = min(kGemmTile, hi - r0);
    // the tile's first row in A's M-grouped blocked scales: group g starts
    // there at the sum of the earlier groups' sizes rounded up to 128 rows
    int32_t part = 0;
    for (int q = threadIdx.x & 63; q < g; q += 64)
      part += (table.hi[q] - table.lo[q] + 127) / 128 * 128;
    srow0 = __builtin_amdgcn_readfirstlane(wave_sum(part)) + (r0 - lo);
    lds_barrier();   // every wave is done with the tables
    qb += (int64_t)g * a.n * ld;
    sb += (int64_t)g * a.sb_bytes;
  } else {
    row0 = (int64_t)tm * kGemmTile;
    rows_valid = min((int64_t)kGemmTile, a.m - row0);
    srow0 = row0;
  }
  const int64_t col0 = (int64_t)tn * kGemmTile;
  const int64_t cols_valid = min((int64_t)kGemmTile, a.n - col0);

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // ranges over the tile's rows of A and of B, ending with the last row's
  // k bytes (rows past them read zero; loads never reach past k in a row)
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(qa + row0 * ld, (uint32_t)((rows_valid - 1) * ld + kofs + k));
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(qb + col0 * ld, (uint32_t)((cols_valid - 1) * ld + kofs + k));
  // Scales: the wave's 128 rows of A (and of B) are one row of 128 x 4
  // tiles of the blocked layout, a strip of 512 bytes per stage; a wave
  // whose rows all lie past the tile's end reads zero scales.
  const int64_t strip = strip_blocks * 512;
  const bool a_on = rows_valid > wm * 128, b_on = cols_valid > wn * 128;
  const __amdgpu_buffer_rsrc_t rsa =
      buffer_rsrc(sa + (a_on ? (srow0 + wm * 128) / 128 * strip : 0), a_on ? (uint32_t)strip : 0u);
  const __amdgpu_buffer_rsrc_t rsb =
      buffer_rsrc(sb + (b_on ? (col0 + wn * 128) / 128 * strip : 0), b_on ? (uint32_t)strip : 0u);
  // Loader role: load instruction u of wave w fills stage rows 32 u + 8 w ..
  // + 7 (1 KiB of LDS, 16 bytes per lane in lane order); lane l writes row
  // position l % 8 of row 32 u + 8 w + l / 8, which holds chunk
  // (l % 8) ^ f(row).  f(row) depends on row % 16 only, so the chunk and the
  // row's offset are the same for every u but for 32 u rows.
  const int lrow = 8 * wave + lane / 8;
  const int lchunk = (lane % 8) ^ ((lrow & 7) ^ ((lrow >> 3) & 1));
  const int g_off = lrow * (int)ld + 16 * lchunk;         // + 32 u ld (< 2^31 for ld <= 2^23)
  // MFMA role
  const int r = lane & 31, h = lane >> 5;
  const int fr = (r & 7) ^ ((r >> 3) & 1);
  const int a_base = (wm * 128 + r) * kGemmTK, b_base = (wn * 128 + r) * kGemmTK;

  v16f acc[kGemmWaveBlocks][kGemmWaveBlocks];
#pragma unroll
  for (int i = 0; i < kGemmWaveBlocks; ++i)
#pragma unroll
    for (int j = 0; j < kGemmWaveBlocks; ++j)
      acc[i][j] = (v16f){};

  const int stages = (int)((kofs + k + kGemmTK - 1) / kGemmTK);
  // a stage's scale words per operand: the stage's tile, and grouped along
  // K also the tile before it (combined when the scales are used, so that
  // no wait for the scale loads stands before the MFMAs that follow them)
  constexpr int kSW = MODE == kGemmGroupsK ? 2 * kGemmWaveBlocks : kGemmWaveBlocks;
  uint32_t s0a[kSW], s0b[kSW], s1a[kSW] = {}, s1b[kSW] = {};

  // Load u (0 .. 15) of a stage: load instruction u / 2 of operand u % 2,
  // from memory straight into LDS half st.  Chunks outside [kofs, kofs + K)
  // (all of them when kt >= kofs + K) get an offset past the buffer's range
  // and load zero.
  auto load_one = [&](auto st_c, int kt, int u) {
    constexpr int st = decltype(st_c)::value;
    const int off = (uint32_t)(kt + 16 * lchunk - kofs) < (uint32_t)k ? g_off : (int)0x80000000;
    const int row = (u / 2) * kGemmLoadRows + 8 * wave;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(u % 2 ? rb : ra,
                                             (__attribute__((address_space(3))) void*)(lds[st][u % 2] + row * kGemmTK),
                                             16, off + (u / 2) * kGemmLoadRows * (int)ld, kt, 0, 0);
  };
  // The stage's scales: lane r + 32 h reads bytes 16 r .. + 15 of the
  // stage's 512-byte tile, whose dword i holds the four block scales of row
  // 32 i + r.  Blocks past K are the layout's zero padding (their data is
  // zero too); a stage past K reads zero.  With kofs = 32 d the stage's
  // blocks are the group's blocks 4 j - d .. 4 j - d + 3: the last d bytes
  // of tile j - 1 and the first 4 - d of tile j.  Tile j - 1 is the previous
  // stage's tile, still in registers (prev; zero before the first stage,
  // as the data of blocks before the group's first is): a copy, so that the
  // stage issues no more loads than a dense one (the loads into LDS, not
  // the MFMAs, bound these kernels).
  auto load_scales = [&](int kt, uint32_t (&s_a)[kSW], uint32_t (&s_b)[kSW], const uint32_t (&prev_a)[kSW],
                         const uint32_t (&prev_b)[kSW]) {
    if constexpr (MODE == kGemmGroupsK) {
#pragma unroll
      for (int i = 0; i < kGemmWaveBlocks; ++i) {
        s_a[kGemmWaveBlocks + i] = prev_a[i];
        s_b[kGemmWaveBlocks + i] = prev_b[i];
      }
    }
    const u32x4 va = __builtin_amdgcn_raw_buffer_load_b128(rsa, 16 * r, kt / kGemmTK * 512, 0);
    const u32x4 vb = __builtin_amdgcn_raw_buffer_load_b128(rsb, 16 * r, kt / kGemmTK * 512, 0);
#pragma unroll
    for (int i = 0; i < kGemmWaveBlocks; ++i) {
      s_a[i] = va[i];
      s_b[i] = vb[i];
    }
  };
  // MFMA operands of one step as 16-byte halves: [slab][0] = chunk 4 s + h
  // (first 32-block of the step), [slab][1] = chunk 4 s + 2 + h (second).
  typedef u32x4 Half[kGemmWaveBlocks][2];
  // Read q (0 .. 15) of a step's operands from LDS half st, in the order
  // the MFMAs consume them: A slab 0, B slabs 0 .. 3, A slabs 1 .. 3, each
  // as its two halves.
  auto read_one = [&](auto st_c, int s, int q, Half& fa, Half& fb) {
    constexpr int st = decltype(st_c)::value;
    const int slab = q / 2, half = q % 2;   // 0: A0, 1-4: B0-B3, 5-7: A1-A3
    const bool is_b = slab >= 1 && slab <= 4;
    const int i = slab == 0 ? 0 : is_b ? slab - 1 : slab - 4;
    const uint8_t* base = is_b ? lds[st][1] + b_base : lds[st][0] + a_base;
    const u32x4 v = *reinterpret_cast<const u32x4*>(base + i * 32 * kGemmTK + 16 * ((4 * s + 2 * half + h) ^ fr));
    (is_b ? fb : fa)[i][half] = v;
  };
  auto mfma = [&](int i, int j, const Half& fa, const Half& fb, int xa, int xb) {
    const v8i va = (v8i){(int)fa[i][0][0], (int)fa[i][0][1], (int)fa[i][0][2], (int)fa[i][0][3],
                         (int)fa[i][1][0], (int)fa[i][1][1], (int)fa[i][1][2], (int)fa[i][1][3]};
    const v8i vb = (v8i){(int)fb[j][0][0], (int)fb[j][0][1], (int)fb[j][0][2], (int)fb[j][0][3],
                         (int)fb[j][1][0], (int)fb[j][1][1], (int)fb[j][1][2], (int)fb[j][1][3]};
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc[i][j], 0, 0, 0, xa, 0, xb);
  };
  // this lane's scale bytes for step s: stage block 2 s + h (grouped along
  // K: byte 2 s + h of the last d bytes of the previous tile followed by the
  // first 4 - d of the stage's tile)
  auto step_scales = [&](int s, const uint32_t (&sc)[kSW], int (&x)[kGemmWaveBlocks]) {
#pragma unroll
    for (int i = 0; i < kGemmWaveBlocks; ++i) {
      if constexpr (MODE == kGemmGroupsK) {
        const uint64_t pair = ((uint64_t)sc[i] << 32) | sc[kGemmWaveBlocks + i];
        x[i] = (int)((pair >> (32 - 8 * (kofs / 32) + 16 * s + 8 * h)) & 0xFFu);
      } else {
        x[i] = (int)((sc[i] >> (16 * s + 8 * h)) & 0xFFu);
      }
    }
  };

  // Stage t (LDS half st = t % 2, K offset kt) runs in two halves.
  // First half, entered with the first step's operands f0 read (or in
  // flight) and the stage's scales in cur: the scales of stage t + 1 are
  // loaded into nxt, and each MFMA of the first step is followed by one LDS
  // read of the second step's operands f1.  Second half: once this wave's
  // loads of stage t + 1 have landed and every wave is past its reads of
  // half st, a barrier; then each MFMA of the second step is followed by one
  // load of stage t + 2 into half st and one LDS read of stage t + 1's
  // first-step operands from the other half.  A stage's loads thus have
  // about a stage of MFMA time to arrive, and no barrier stands between the
  // last MFMA of a stage and the first of the next.  Stages past K load
  // zero.  sched_barrier keeps the compiler to this instruction order.
  auto first_half = [&](auto st_c, int kt, const Half& f0a, const Half& f0b,
                        const uint32_t (&cur_a)[kSW], const uint32_t (&cur_b)[kSW],
                        uint32_t (&nxt_a)[kSW], uint32_t (&nxt_b)[kSW], Half& f1a,
                        Half& f1b) {
    load_scales(kt + kGemmTK, nxt_a, nxt_b, cur_a, cur_b);
    int xa[kGemmWaveBlocks], xb[kGemmWaveBlocks];
    step_scales(0, cur_a, xa);
    step_scales(0, cur_b, xb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < kGemmWaveBlocks * kGemmWaveBlocks; ++q) {
      mfma(q / kGemmWaveBlocks, q % kGemmWaveBlocks, f0a, f0b, xa[q / kGemmWaveBlocks], xb[q % kGemmWaveBlocks]);
      read_one(st_c, 1, q, f1a, f1b);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto second_half = [&](auto st_c, int kt, const Half& f1a, const Half& f1b,
                         const uint32_t (&cur_a)[kSW], const uint32_t (&cur_b)[kSW],
                         Half& f0a, Half& f0b) {
    constexpr int st = decltype(st_c)::value;
    int xa[kGemmWaveBlocks], xb[kGemmWaveBlocks];
    step_scales(1, cur_a, xa);
    step_scales(1, cur_b, xb);
    __builtin_amdgcn_sched_barrier(0);
    // all but the two scale loads of stage t + 1: this wave's loads of
    // stage t + 1 (vmcnt), then every wave's
    __builtin_amdgcn_s_waitcnt(0x0F70 | 2);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < kGemmWaveBlocks * kGemmWaveBlocks; ++q) {
      mfma(q / kGemmWaveBlocks, q % kGemmWaveBlocks, f1a, f1b, xa[q / kGemmWaveBlocks], xb[q % kGemmWaveBlocks]);
      load_one(st_c, kt + 2 * kGemmTK, q);
      read_one(std::integral_constant<int, st ^ 1>(), 0, q, f0a, f0b);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  static_assert(2 * kGemmLoads == kGemmWaveBlocks * kGemmWaveBlocks, "one load per second-step MFMA");

  // Stages alternate between LDS halves 0 and 1 and scale registers s0 /
  // s1.  A trip of the loop starts with a second half, whose barrier comes
  // before its first MFMA (so the compiler's conservative waits at the loop
  // head cost nothing), and runs two stages; the loop ends with the first
  // half of the stage after the last (an odd count: of two), past K, whose
  // data and scales load as zero and add nothing.
  if (stages > 0) {
#pragma unroll
    for (int u = 0; u < 2 * kGemmLoads; ++u) {
      load_one(S0(), 0, u);
      load_one(S1(), kGemmTK, u);
    }
    // (s1 is zero here: the tile before the first stage's)
    load_scales(0, s0a, s0b, s1a, s1b);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    lds_barrier();
    Half f0a, f0b, f1a, f1b;
#pragma unroll
    for (int q = 0; q < 2 * kGemmLoads; ++q)
      read_one(S0(), 0, q, f0a, f0b);
    first_half(S0(), 0, f0a, f0b, s0a, s0b, s1a, s1b, f1a, f1b);
    for (int st = 0; st < stages; st += 2) {
      second_half(S0(), st * kGemmTK, f1a, f1b, s0a, s0b, f0a, f0b);
      first_half(S1(), (st + 1) * kGemmTK, f0a, f0b, s1a, s1b, s0a, s0b, f1a, f1b);
      second_half(S1(), (st + 1) * kGemmTK, f1a, f1b, s1a, s1b, f0a, f0b);
      first_half(S0(), (st + 2) * kGemmTK, f0a, f0b, s0a, s0b, s1a, s1b, f1a, f1b);
    }
    // the last trip's loads (past K) must land before the workgroup's LDS
    // is released
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }

  // Epilogue.  Register v of lane l holds row 8 (v / 4) + 4 h + v % 4,
  // column r of its 32 x 32 block.  bf16 output with rows of whole 16-byte
  // chunks (n % 8 == 0, c 16-byte aligned): the tile goes through LDS (the
  // operand stages are free now; 256 x 256 bf16 is exactly their 128 KiB)
  // and leaves as 512-byte rows of 16-byte stores -- written straight from
  // the registers it would take 2-byte stores, 1024 instructions per
  // workgroup, and measured a fifth of the GEMM's time.  In LDS, dword d of
  // row R (columns 2 d, 2 d + 1) sits at d ^ swz(R), swz(R) = 16 (2 ((R >> 2)
  // & 1) + (R & 1)): the two rows one write instruction touches (R and R + 4,
  // 16 dwords each) land on different 16-bank groups, and a 16-byte chunk
  // stays whole.
  if constexpr (BF16) {
    if ((a.n & 7) == 0 && (reinterpret_cast<uintptr_t>(c) & 15) == 0) {
      uint32_t* ldsw = reinterpret_cast<uint32_t*>(&lds[0][0][0]);
      auto swz = [](int row) { return 16 * (2 * ((row >> 2) & 1) + (row & 1)); };
      lds_barrier();   // every wave is done reading operands from LDS
      // Rows R and R + 1 of column r (accumulators v and v + 1) are converted
      // together and written as the two 2-byte halves of their dwords (the
      // lanes of columns r and r ^ 1 fill one dword).  With R = wm 128 + 32 i
      // + 8 (v / 4) + 4 h + v % 4 (v even), bit 2 of R is h and bit 0 is 0,
      // so swz(R) = 32 h and swz(R + 1) = 32 h + 16: the byte address of
      // column r of row R is 4 (128 R + wn 64 + 16 (j ^ 2 h) + r / 2) + 2 (r &
      // 1), a per-lane base for each j plus a constant.  (Trading values
      // with the neighbouring lane so that each lane writes whole dwords cost
      // more VALU time than the second LDS write: dense 609 against 599 us.)
      uint8_t* ldsb = &lds[0][0][0];
      const int lane_b = 512 * (wm * 128 + 4 * h) + 4 * (wn * 64 + (r >> 1)) + 2 * (r & 1);
      int base_r[kGemmWaveBlocks], base_r1[kGemmWaveBlocks];
#pragma unroll
      for (int j = 0; j < kGemmWaveBlocks; ++j) {
        base_r[j] = lane_b + 64 * (j ^ (2 * h));
        base_r1[j] = lane_b + 512 + 64 * (j ^ (2 * h) ^ 1);
      }
#pragma unroll
      for (int i = 0; i < kGemmWaveBlocks; ++i)
#pragma unroll
        for (int j = 0; j < kGemmWaveBlocks; ++j)
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            const uint32_t pair = pack_bf16(acc[i][j][v], acc[i][j][v + 1]);
            const int off = 512 * (32 * i + 8 * (v / 4) + (v % 4));
            *reinterpret_cast<uint16_t*>(ldsb + base_r[j] + off) = (uint16_t)pair;
            *reinterpret_cast<uint16_t*>(ldsb + base_r1[j] + off) = (uint16_t)(pair >> 16);
          }
      lds_barrier();
      // thread t: 16-byte chunk t % 32 of rows t / 32 + 8 p
      const int chunk = threadIdx.x & 31;
      const bool col_on = 8 * chunk < cols_valid;
      uint8_t* cb = static_cast<uint8_t*>(c) + ((row0 * a.n + col0) * 2 + 16 * chunk);
#pragma unroll 8
      for (int p = 0; p < kGemmTile / 8; ++p) {
        const int row = (threadIdx.x >> 5) + 8 * p;
        if (row < rows_valid && col_on) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(&ldsw[row * 128 + ((4 * chunk) ^ swz(row))]);
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(cb + (int64_t)row * a.n * 2));
        }
      }
      return;
    }
  } else {
    // fp32 output, rows of whole 16-byte chunks (n % 4 == 0): the same in two
    // passes of 128 rows (the waves with wm = pass write their quadrants),
    // dword d of row R at d ^ (32 ((R >> 2) & 1)) so that rows R and R + 4
    // of one write instruction use different banks.
    if ((a.n & 3) == 0 && (reinterpret_cast<uintptr_t>(c) & 15) == 0) {
      uint32_t* ldsw = reinterpret_cast<uint32_t*>(&lds[0][0][0]);
      auto swz = [](int row) { return 32 * ((row >> 2) & 1); };
      const int chunk = threadIdx.x & 63;
      const bool col_on = 4 * chunk < cols_valid;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        lds_barrier();   // operands (pass 0) or the previous pass (pass 1) are read
        if (wm == pass) {
#pragma unroll
          for (int i = 0; i < kGemmWaveBlocks; ++i)
#pragma unroll
            for (int j = 0; j < kGemmWaveBlocks; ++j)
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int row = 32 * i + 8 * (v / 4) + 4 * h + (v % 4);   // within the pass
                const int d = wn * 128 + 32 * j + r;
                ldsw[row * 256 + (d ^ swz(row))] = __float_as_uint(acc[i][j][v]);
              }
        }
        lds_barrier();
        // thread t: 16-byte chunk t % 64 of rows t / 64 + 4 p of the pass
        uint8_t* cb = static_cast<uint8_t*>(c) + (((row0 + 128 * pass) * a.n + col0) * 4 + 16 * chunk);
#pragma unroll 8
        for (int p = 0; p < 32; ++p) {
          const int row = (threadIdx.x >> 6) + 4 * p;
          if (128 * pass + row < rows_valid && col_on) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(&ldsw[row * 256 + ((4 * chunk) ^ swz(row))]);
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(cb + (int64_t)row * a.n * 4));
          }
        }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < kGemmWaveBlocks; ++i)
#pragma unroll
    for (int j = 0; j < kGemmWaveBlocks; ++j) {
      const int64_t lc = wn * 128 + 32 * j + r;   // column within the tile
      if (lc >= cols_valid)
        continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t lr = wm * 128 + 32 * i + 8 * (v / 4) + 4 * h + (v % 4);   // row within the tile
        if (lr < rows_valid) {
          const int64_t idx = (row0 + lr) * a.n + col0 + lc;
          if (BF16)
            static_cast<uint16_t*>(c)[idx] = to_bf16(acc[i][j][v]);
          else
            static_cast<float*>(c)[idx] = acc[i][j][v];
        }
      }
    }
}

// mode: kGemmDense, kGemmGroupsM or kGemmGroupsK
static GemmArgs gemm_args(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t m,
                          int64_t n, int64_t k, void* c, int mode, const int32_t* ends, int32_t groups,
                          int64_t* blocks) {
  GemmArgs a;
  a.qa = qa;
  a.sa = sa;
  a.qb = qb;
  a.sb = sb;
  a.m = m;
  a.n = n;
  a.k = k;
  a.c = c;
  a.ends = ends;
  a.groups = groups;
  a.sb_bytes = (n + 127) / 128 * 128 * ((k / 32 + 3) / 4 * 4);
  // grouped along M: every group may end with a partial tile -> one spare
  // tile each; grouped along K: one grid of tiles per group, each cut into
  // 8 pieces of per_xcd tiles, one per XCD
  const int64_t tm = (m + kGemmTile - 1) / kGemmTile + (mode == kGemmGroupsM ? groups : 0);
  const int64_t tn = (n + kGemmTile - 1) / kGemmTile;
  a.tiles_m = (uint32_t)tm;
  a.tiles_n = (uint32_t)tn;
  // grouped along M each group's tiles are cut into 8 pieces of ceil(T_g /
  // 8): in all at most ceil(tm * tn / 8) + groups per XCD
  const int64_t per = (tm * tn + 7) / 8 + (mode == kGemmGroupsM ? groups : 0);
  a.per_xcd = (uint32_t)per;
  *blocks = per * 8 * (mode == kGemmGroupsK ? groups : 1);
  return a;
}

int64_t gemm_grid_blocks(int64_t m, int64_t n, int mode, int32_t groups) {
  int64_t blocks;
  gemm_args(nullptr, nullptr, nullptr, nullptr, m, n, 64, nullptr, mode, nullptr, groups, &blocks);
  return blocks;
}

template <int MODE>
static void launch_gemm_mode(const GemmArgs& a, bool bf16, dim3 grid, hipStream_t stream) {
  if (bf16)
    hipLaunchKernelGGL((mx_gemm_kernel<MODE, true>), grid, dim3(kGemmThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<MODE, false>), grid, dim3(kGemmThreads), 0, stream, a);
}

hipError_t launch_mx_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t m,
                          int64_t n, int64_t k, void* c, bool bf16, int mode, const int32_t* ends, int32_t groups,
                          hipStream_t stream) {
  int64_t blocks;
  const GemmArgs a = gemm_args(qa, sa, qb, sb, m, n, k, c, mode, ends, groups, &blocks);
  const dim3 grid((unsigned)blocks);
  if (mode == kGemmGroupsK)
    launch_gemm_mode<kGemmGroupsK>(a, bf16, grid, stream);
  else if (mode == kGemmGroupsM)
    launch_gemm_mode<kGemmGroupsM>(a, bf16, grid, stream);
  else
    launch_gemm_mode<kGemmDense>(a, bf16, grid, stream);
  return hipGetLastError();
}

}  // namespace mx
