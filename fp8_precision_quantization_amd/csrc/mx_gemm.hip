// MX-scaled GEMM on gfx950's block-scaled MFMA: the consumer of the dim0
// casts ("[mxfp8 moe training] add compile support", Perf analysis item 1:
// MXFP8 grouped GEMMs of the (16640, 5120) activations, grouped along M,
// against per-group (8192, 5120) weights).
//
//   C[m][n] = sum over k of A(m, k) * B(n, k),  A(m, k) = e4m3(qa[m][k]) *
//   2^(sa[m][k / 32] - 127), B likewise: both operands K-major, as the dim0
//   cast writes them (codes (rows, K), plain scales (rows, K / 32)).
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
// stages of 128 bytes: the workgroup loads the stage's 256 rows of A and of
// B (32 KiB each; every load instruction reads 32 whole 128-byte rows) into
// registers while the MFMAs work on the previous stage, then writes them to
// the other half of a double-buffered LDS area.  Each wave reads its MFMA
// operands from LDS with 16-byte reads.  In LDS a row's eight 16-byte chunks
// are permuted by an XOR of the row index (f below), so that the 16 lanes
// of one LDS read phase, which read one chunk of 16 consecutive rows, hit
// distinct banks, as do the writes.  Scales go straight to registers: one
// dword (the row's four blocks of the stage) per row slab and lane.
//
// Buffer ranges end at the tile's last row, so rows past M or N read as
// zero; chunks past K are not loaded (zero), and their blocks take scale 1.
// Tiles are ordered in bands of 8 tile rows, column by column, and the
// ordered list is cut into 8 contiguous pieces, one per XCD (workgroups are
// dealt to the XCDs round-robin), so that each XCD's L2 sees a compact
// region of A rows and B columns.
//
// Grouped along M (GROUPED): the tiles of group g cover its rows [lo_g,
// hi_g) in 256-row steps from the group's padded start (the group table of
// the blocked layouts, rebuilt from the device offsets in each workgroup);
// B and its scales are group g's (N, K) slice.  Rows past the last end are
// not written.
#include "mx_device.h"
#include "mx_groups.h"
#include "mxcast.h"
#include "mx_launch.h"

#include <type_traits>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kGemmTile = 256;                 // rows and columns of C per workgroup
constexpr int kGemmTK = 128;                   // K bytes per LDS stage
constexpr int kGemmWaveBlocks = 4;             // 32 x 32 MFMA blocks per wave along M and along N
constexpr int kGemmLoadRows = kGemmThreads * 16 / kGemmTK;   // rows per load instruction (32)
constexpr int kGemmLoads = kGemmTile / kGemmLoadRows;        // load instructions per operand and stage (8)
constexpr int kGemmStageBytes = kGemmTile * kGemmTK;         // one operand's stage (32 KiB)
constexpr int kGemmBand = 8;                   // tile rows per band of the tile order
constexpr uint32_t kE8m0One = 127;             // e8m0 byte of 2^0

struct GemmArgs {
  const uint8_t *qa, *sa, *qb, *sb;
  int64_t m, n, k;
  void* c;
  const int32_t* ends;
  int32_t groups;
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

// binary32 -> bf16 bits, nearest-even; NaN -> 0x7FC0.
__device__ __forceinline__ uint16_t to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u)
    return 0x7FC0u;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// The four block scales (bytes) of the stage at K offset kt for the row
// whose scales start at row_off (bytes) in rs.  DW: the row's scales are
// dword-aligned (K % 128 == 0).
template <bool DW>
__device__ __forceinline__ uint32_t stage_scales(__amdgpu_buffer_rsrc_t rs, int row_off, int kt, int64_t kb) {
  if (DW)   // a stage past K reads zero (its data is zero too)
    return __builtin_amdgcn_raw_buffer_load_b32(rs, kt / 32 < kb ? row_off : (int)0x80000000, kt / 32, 0);
  uint32_t w = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int blk = kt / 32 + b;
    const uint32_t v = blk < kb ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, row_off, blk, 0) : kE8m0One;
    w |= v << (8 * b);
  }
  return w;
}

template <bool GROUPED, bool BF16, bool DW>
__global__ __launch_bounds__(kGemmThreads) void mx_gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kGemmStageBytes];   // [stage][A, B]
  __shared__ std::conditional_t<GROUPED, GroupTable, NoTable> table;

  // tile order: XCD x owns ordered tiles [x * per_xcd, (x + 1) * per_xcd)
  const uint32_t tiles = a.tiles_m * a.tiles_n;
  const uint32_t id = (blockIdx.x % 8) * a.per_xcd + blockIdx.x / 8;
  if (id >= tiles)
    return;  // uniform, before any barrier
  const uint32_t band = id / (kGemmBand * a.tiles_n);
  const uint32_t band_rows = min((uint32_t)kGemmBand, a.tiles_m - band * kGemmBand);
  const uint32_t within = id - band * kGemmBand * a.tiles_n;
  const uint32_t tm = band * kGemmBand + within % band_rows;
  const uint32_t tn = within / band_rows;

  const int64_t k = a.k;
  const int64_t kb = k / 32;
  const uint8_t* qb = a.qb;
  const uint8_t* sb = a.sb;
  int64_t row0, rows_valid;
  if constexpr (GROUPED) {
    if (threadIdx.x < 64)
      build_group_table(a.ends, a.groups, (int32_t)a.m, kGemmTile, table);
    lds_barrier();
    const int32_t pos = (int32_t)tm * kGemmTile;
    const int g = find_group(table, a.groups, pos);
    if (g < 0)
      return;  // uniform; no barrier follows
    row0 = table.lo[g] + (pos - table.start[g]);
    rows_valid = min((int64_t)kGemmTile, (int64_t)table.hi[g] - row0);
    qb += (int64_t)g * a.n * k;
    sb += (int64_t)g * a.n * kb;
  } else {
    row0 = (int64_t)tm * kGemmTile;
    rows_valid = min((int64_t)kGemmTile, a.m - row0);
  }
  const int64_t col0 = (int64_t)tn * kGemmTile;
  const int64_t cols_valid = min((int64_t)kGemmTile, a.n - col0);

  // ranges over the tile's rows of A and of B (rows past them read zero)
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a.qa + row0 * k, (uint32_t)(rows_valid * k));
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(qb + col0 * k, (uint32_t)(cols_valid * k));
  const __amdgpu_buffer_rsrc_t rsa = buffer_rsrc(a.sa + row0 * kb, (uint32_t)(rows_valid * kb));
  const __amdgpu_buffer_rsrc_t rsb = buffer_rsrc(sb + col0 * kb, (uint32_t)(cols_valid * kb));

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  // Loader role: load instruction u of wave w fills stage rows 32 u + 8 w ..
  // + 7 (1 KiB of LDS, 16 bytes per lane in lane order); lane l writes row
  // position l % 8 of row 32 u + 8 w + l / 8, which holds chunk
  // (l % 8) ^ f(row).  f(row) depends on row % 16 only, so the chunk and the
  // row's offset are the same for every u but for 32 u rows.
  const int lrow = 8 * wave + lane / 8;
  const int lchunk = (lane % 8) ^ ((lrow & 7) ^ ((lrow >> 3) & 1));
  const int g_off = lrow * (int)k + 16 * lchunk;          // + 32 u k (< 2^31 for k <= 2^23)
  // MFMA role
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, h = lane >> 5;
  const int fr = (r & 7) ^ ((r >> 3) & 1);
  const int a_base = (wm * 128 + r) * kGemmTK, b_base = (wn * 128 + r) * kGemmTK;
  int sa_off[kGemmWaveBlocks], sb_off[kGemmWaveBlocks];
#pragma unroll
  for (int i = 0; i < kGemmWaveBlocks; ++i) {
    sa_off[i] = (wm * 128 + 32 * i + r) * (int)kb;
    sb_off[i] = (wn * 128 + 32 * i + r) * (int)kb;
  }

  v16f acc[kGemmWaveBlocks][kGemmWaveBlocks];
#pragma unroll
  for (int i = 0; i < kGemmWaveBlocks; ++i)
#pragma unroll
    for (int j = 0; j < kGemmWaveBlocks; ++j)
      acc[i][j] = (v16f){};

  const int stages = (int)((k + kGemmTK - 1) / kGemmTK);
  uint32_t s0a[kGemmWaveBlocks], s0b[kGemmWaveBlocks], s1a[kGemmWaveBlocks], s1b[kGemmWaveBlocks];

  // The stage at K offset kt, from memory straight into LDS stage st.
  // Chunks past K (all of them when kt >= K) get an offset past the
  // buffer's range and load zero.
  auto load_stage = [&](auto st_c, int kt) {
    constexpr int st = decltype(st_c)::value;
    const int off = kt + (DW ? 0 : 16 * lchunk) < k ? g_off : (int)0x80000000;
#pragma unroll
    for (int u = 0; u < kGemmLoads; ++u) {
      const int row = u * kGemmLoadRows + 8 * wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(lds[st][0] + row * kGemmTK),
                                               16, off + u * kGemmLoadRows * (int)k, kt, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void*)(lds[st][1] + row * kGemmTK),
                                               16, off + u * kGemmLoadRows * (int)k, kt, 0, 0);
    }
  };
  auto load_scales = [&](int kt, uint32_t (&s_a)[kGemmWaveBlocks], uint32_t (&s_b)[kGemmWaveBlocks]) {
#pragma unroll
    for (int i = 0; i < kGemmWaveBlocks; ++i) {
      s_a[i] = stage_scales<DW>(rsa, sa_off[i], kt, kb);
      s_b[i] = stage_scales<DW>(rsb, sb_off[i], kt, kb);
    }
  };
  // operand of slab i for MFMA step s: chunks 4 s + h and 4 s + 2 + h
  auto read_slab = [&](const uint8_t* base, int i, int s) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + i * 32 * kGemmTK + 16 * ((4 * s + h) ^ fr));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + i * 32 * kGemmTK + 16 * ((4 * s + 2 + h) ^ fr));
    return (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto read_step = [&](auto st_c, int s, v8i (&fa)[kGemmWaveBlocks], v8i (&fb)[kGemmWaveBlocks]) {
    constexpr int st = decltype(st_c)::value;
#pragma unroll
    for (int i = 0; i < kGemmWaveBlocks; ++i) {
      fa[i] = read_slab(lds[st][0] + a_base, i, s);
      fb[i] = read_slab(lds[st][1] + b_base, i, s);
    }
  };
  auto mma = [&](int s, const v8i (&fa)[kGemmWaveBlocks], const v8i (&fb)[kGemmWaveBlocks],
                 const uint32_t (&sc_a)[kGemmWaveBlocks], const uint32_t (&sc_b)[kGemmWaveBlocks]) {
    // this lane's block of step s is stage block 2 s + h
    int xa[kGemmWaveBlocks], xb[kGemmWaveBlocks];
#pragma unroll
    for (int i = 0; i < kGemmWaveBlocks; ++i) {
      xa[i] = (int)((sc_a[i] >> (16 * s + 8 * h)) & 0xFFu);
      xb[i] = (int)((sc_b[i] >> (16 * s + 8 * h)) & 0xFFu);
    }
#pragma unroll
    for (int i = 0; i < kGemmWaveBlocks; ++i)
#pragma unroll
      for (int j = 0; j < kGemmWaveBlocks; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, xa[i], 0,
                                                                    xb[j]);
  };
  // one LDS read after each MFMA, so that the reads of the next step's
  // operands trickle in behind the MFMAs
  auto interleave = [&]() {
#pragma unroll
    for (int q = 0; q < 2 * kGemmWaveBlocks; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kGemmWaveBlocks * kGemmWaveBlocks - 2 * kGemmWaveBlocks, 0);
  };
  // Stage t (LDS half st = t % 2, K offset kt), entered with its first
  // step's operands f0 read (or in flight) and its scales in cur:
  //   - the scales of stage t + 1 are loaded into nxt;
  //   - the second step's operands are read while the first step multiplies;
  //   - once this wave's loads of stage t + 1 have landed and every wave is
  //     past its reads of half st (barrier), stage t + 2 is loaded into
  //     half st and the first-step operands of stage t + 1 are read from
  //     the other half while the second step multiplies.
  // A stage's loads thus have about a stage of MFMA time to arrive, and no
  // barrier stands between the last MFMA of a stage and the first of the
  // next.  Stages past K load zero.
  auto stage = [&](auto st_c, int kt, v8i (&f0a)[kGemmWaveBlocks], v8i (&f0b)[kGemmWaveBlocks],
                   const uint32_t (&cur_a)[kGemmWaveBlocks], const uint32_t (&cur_b)[kGemmWaveBlocks],
                   uint32_t (&nxt_a)[kGemmWaveBlocks], uint32_t (&nxt_b)[kGemmWaveBlocks]) {
    constexpr int st = decltype(st_c)::value;
    // (sched_barrier: the compiler keeps these phases in this order)
    load_scales(kt + kGemmTK, nxt_a, nxt_b);
    __builtin_amdgcn_sched_barrier(0);
    v8i f1a[kGemmWaveBlocks], f1b[kGemmWaveBlocks];
    read_step(st_c, 1, f1a, f1b);
    mma(0, f0a, f0b, cur_a, cur_b);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    // all but the scale loads just issued: the loads of stage t + 1 (vmcnt)
    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kGemmWaveBlocks * (DW ? 1 : 4)));
    lds_barrier();
    load_stage(st_c, kt + 2 * kGemmTK);
    __builtin_amdgcn_sched_barrier(0);
    read_step(std::integral_constant<int, st ^ 1>(), 0, f0a, f0b);
    mma(1, f1a, f1b, cur_a, cur_b);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  // Stages alternate between LDS halves 0 and 1 and scale registers s0 /
  // s1, two per trip; an odd count ends with one stage past K, whose data
  // and scales load as zero and add nothing.
  if (stages > 0) {
    load_stage(S0(), 0);
    load_stage(S1(), kGemmTK);
    load_scales(0, s0a, s0b);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    lds_barrier();
    v8i f0a[kGemmWaveBlocks], f0b[kGemmWaveBlocks];
    read_step(S0(), 0, f0a, f0b);
    for (int st = 0; st < stages; st += 2) {
      stage(S0(), st * kGemmTK, f0a, f0b, s0a, s0b, s1a, s1b);
      stage(S1(), (st + 1) * kGemmTK, f0a, f0b, s1a, s1b, s0a, s0b);
    }
    // the last trip's loads (past K) must land before the workgroup's LDS
    // is released
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }

  // epilogue: register v of lane l is row 8 (v / 4) + 4 h + v % 4, column r
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
            static_cast<uint16_t*>(a.c)[idx] = to_bf16(acc[i][j][v]);
          else
            static_cast<float*>(a.c)[idx] = acc[i][j][v];
        }
      }
    }
}

static GemmArgs gemm_args(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t m,
                          int64_t n, int64_t k, void* c, bool grouped, const int32_t* ends, int32_t groups,
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
  // grouped: every group may end with a partial tile -> one spare tile each
  const int64_t tm = (m + kGemmTile - 1) / kGemmTile + (grouped ? groups : 0);
  const int64_t tn = (n + kGemmTile - 1) / kGemmTile;
  a.tiles_m = (uint32_t)tm;
  a.tiles_n = (uint32_t)tn;
  const int64_t per = (tm * tn + 7) / 8;
  a.per_xcd = (uint32_t)per;
  *blocks = per * 8;
  return a;
}

int64_t gemm_grid_blocks(int64_t m, int64_t n, bool grouped, int32_t groups) {
  int64_t blocks;
  gemm_args(nullptr, nullptr, nullptr, nullptr, m, n, 64, nullptr, grouped, nullptr, groups, &blocks);
  return blocks;
}

template <bool DW>
static void launch_gemm_dw(const GemmArgs& a, bool grouped, bool bf16, dim3 grid, hipStream_t stream) {
  const dim3 block(kGemmThreads);
  if (grouped) {
    if (bf16)
      hipLaunchKernelGGL((mx_gemm_kernel<true, true, DW>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((mx_gemm_kernel<true, false, DW>), grid, block, 0, stream, a);
  } else {
    if (bf16)
      hipLaunchKernelGGL((mx_gemm_kernel<false, true, DW>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((mx_gemm_kernel<false, false, DW>), grid, block, 0, stream, a);
  }
}

hipError_t launch_mx_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t m,
                          int64_t n, int64_t k, void* c, bool bf16, const int32_t* ends, int32_t groups,
                          hipStream_t stream) {
  int64_t blocks;
  const GemmArgs a = gemm_args(qa, sa, qb, sb, m, n, k, c, ends != nullptr, ends, groups, &blocks);
  const dim3 grid((unsigned)blocks);
  if (k % kGemmTK == 0)
    launch_gemm_dw<true>(a, ends != nullptr, bf16, grid, stream);
  else
    launch_gemm_dw<false>(a, ends != nullptr, bf16, grid, stream);
  return hipGetLastError();
}

}  // namespace mx
