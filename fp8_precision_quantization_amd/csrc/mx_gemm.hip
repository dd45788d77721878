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
// Work decomposition: a 256-thread workgroup owns a 128 x 128 tile of C;
// wave w its (w / 2, w % 2) 64 x 64 quadrant = 2 x 2 MFMA blocks.  Operands
// go straight from memory to registers in the MFMA layout (two 16-byte
// buffer loads per 32-row slab per lane), double-buffered so that the loads
// of the next K step are in flight while the current one multiplies.  Buffer
// ranges end at the tile's last row, so rows past M or N read as zero.
// Workgroups are numbered so that each XCD works on a compact block of
// tiles, whose A rows and B columns then stay in its L2.
//
// Grouped along M (GROUPED): the tiles of group g cover its rows [lo_g,
// hi_g) in 128-row steps from the group's padded start (the group table of
// the blocked layouts, rebuilt from the device offsets in each workgroup);
// B and its scales are group g's (N, K) slice.  Rows past the last end are
// not written.
#include "mx_device.h"
#include "mx_groups.h"
#include "mxcast.h"
#include "mx_launch.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kGemmTile = 128;      // rows and columns of C per workgroup
constexpr int kGemmStep = 64;       // K per MFMA
constexpr int kGemmXcdBlock = 8;    // tiles per side of an XCD's block of C
constexpr uint32_t kE8m0One = 127;  // e8m0 byte of 2^0

struct GemmArgs {
  const uint8_t *qa, *sa, *qb, *sb;
  int64_t m, n, k;
  void* c;
  const int32_t* ends;
  int32_t groups;
  uint32_t tiles_m, tiles_n;   // tile grid (tiles_m includes one spare tile per group when grouped)
  uint32_t items;              // work items: whole kGemmXcdBlock^2 blocks of tiles
  uint32_t per_xcd;            // work items per XCD
};

struct Operands {
  v8i a[2], b[2];
  int sa[2], sb[2];
};

// One 32-row slab of an operand for K step k0: the lane's row at row_off
// (bytes, within the tile), bytes 16 (l / 32) .. + 15 of both 32-blocks.
// A step past K (the half block of a K that is 32 mod 64) reads as zero.
__device__ __forceinline__ v8i load_slab(__amdgpu_buffer_rsrc_t rs, int row_off, int k0, bool second_ok) {
  const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rs, row_off, k0, 0);
  u32x4 hi = {0, 0, 0, 0};
  if (second_ok)
    hi = __builtin_amdgcn_raw_buffer_load_b128(rs, row_off, k0 + 32, 0);
  return (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__device__ __forceinline__ void load_step(Operands& o, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rsa,
                                          __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rsb,
                                          const int (&a_off)[2], const int (&b_off)[2], const int (&sa_off)[2],
                                          const int (&sb_off)[2], int k0, bool second_ok, bool my_block_ok) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    o.a[i] = load_slab(ra, a_off[i], k0, second_ok);
    o.b[i] = load_slab(rb, b_off[i], k0, second_ok);
    // this lane's scale: block (l / 32) of the step; a block past K gets
    // scale 1 (its data is zero)
    o.sa[i] = my_block_ok ? (int)__builtin_amdgcn_raw_buffer_load_b8(rsa, sa_off[i], k0 / 32, 0) : (int)kE8m0One;
    o.sb[i] = my_block_ok ? (int)__builtin_amdgcn_raw_buffer_load_b8(rsb, sb_off[i], k0 / 32, 0) : (int)kE8m0One;
  }
}

__device__ __forceinline__ void mma_step(v16f (&acc)[2][2], const Operands& o) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.a[i], o.b[j], acc[i][j], 0, 0, 0, o.sa[i], 0,
                                                                  o.sb[j]);
}

// binary32 -> bf16 bits, nearest-even; NaN -> 0x7FC0.
__device__ __forceinline__ uint16_t to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u)
    return 0x7FC0u;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <bool GROUPED, bool BF16>
__global__ __launch_bounds__(kGemmThreads) void mx_gemm_kernel(GemmArgs a) {
  __shared__ std::conditional_t<GROUPED, GroupTable, NoTable> table;
  // XCD-aware order: XCD x takes items [x * per_xcd, ...); items run over
  // blocks of kGemmXcdBlock x kGemmXcdBlock tiles, row-major inside a block.
  const uint32_t id = (blockIdx.x % 8) * a.per_xcd + blockIdx.x / 8;
  if (id >= a.items)
    return;  // uniform, before any barrier
  const uint32_t bn = (a.tiles_n + kGemmXcdBlock - 1) / kGemmXcdBlock;
  const uint32_t blk = id / (kGemmXcdBlock * kGemmXcdBlock), in = id % (kGemmXcdBlock * kGemmXcdBlock);
  const uint32_t bm_i = blk / bn, bn_i = blk % bn;
  const uint32_t rows_here = min((uint32_t)kGemmXcdBlock, a.tiles_m - bm_i * kGemmXcdBlock);
  const uint32_t cols_here = min((uint32_t)kGemmXcdBlock, a.tiles_n - bn_i * kGemmXcdBlock);
  if (in >= rows_here * cols_here)
    return;
  const uint32_t tm = bm_i * kGemmXcdBlock + in / cols_here;
  const uint32_t tn = bn_i * kGemmXcdBlock + in % cols_here;

  const int64_t k = a.k;
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
    sb += (int64_t)g * a.n * (k / 32);
  } else {
    row0 = (int64_t)tm * kGemmTile;
    rows_valid = min((int64_t)kGemmTile, a.m - row0);
  }
  const int64_t col0 = (int64_t)tn * kGemmTile;
  const int64_t cols_valid = min((int64_t)kGemmTile, a.n - col0);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, h = lane >> 5;
  // the wave's 64 rows of A and 64 rows of B (columns of C)
  const int64_t ar0 = row0 + wm * 64, br0 = col0 + wn * 64;
  const int64_t a_rows = max((int64_t)0, min((int64_t)64, rows_valid - wm * 64));
  const int64_t b_rows = max((int64_t)0, min((int64_t)64, cols_valid - wn * 64));
  const int64_t kb = k / 32;
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a.qa + (a_rows ? ar0 : 0) * k, (uint32_t)(a_rows * k));
  const __amdgpu_buffer_rsrc_t rsa = buffer_rsrc(a.sa + (a_rows ? ar0 : 0) * kb, (uint32_t)(a_rows * kb));
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(qb + (b_rows ? br0 : 0) * k, (uint32_t)(b_rows * k));
  const __amdgpu_buffer_rsrc_t rsb = buffer_rsrc(sb + (b_rows ? br0 : 0) * kb, (uint32_t)(b_rows * kb));
  int a_off[2], b_off[2], sa_off[2], sb_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a_off[i] = (int)((32 * i + r) * k) + 16 * h;
    b_off[i] = a_off[i];
    sa_off[i] = (int)((32 * i + r) * kb) + h;
    sb_off[i] = sa_off[i];
  }

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = (v16f){};
  const int steps = (int)((k + kGemmStep - 1) / kGemmStep);
  Operands cur, nxt;
  load_step(cur, ra, rsa, rb, rsb, a_off, b_off, sa_off, sb_off, 0, 32 < k, h == 0 || 32 < k);
  for (int s = 0; s < steps; ++s) {
    if (s + 1 < steps) {
      const int k1 = (s + 1) * kGemmStep;
      load_step(nxt, ra, rsa, rb, rsb, a_off, b_off, sa_off, sb_off, k1, k1 + 32 < k, h == 0 || k1 + 32 < k);
    }
    mma_step(acc, cur);
    cur = nxt;
  }

  // epilogue: register v of lane l is row 8 (v / 4) + 4 h + v % 4, column r
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = br0 + 32 * j + r;
      if (col - col0 >= cols_valid)
        continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t lr = wm * 64 + 32 * i + 8 * (v / 4) + 4 * h + (v % 4);   // row within the tile
        if (lr < rows_valid) {
          const int64_t idx = (row0 + lr) * a.n + col;
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
  // items: whole kGemmXcdBlock^2 blocks, so that the block arithmetic holds
  const int64_t bm = (tm + kGemmXcdBlock - 1) / kGemmXcdBlock, bn = (tn + kGemmXcdBlock - 1) / kGemmXcdBlock;
  const int64_t items = bm * bn * kGemmXcdBlock * kGemmXcdBlock;
  a.items = (uint32_t)items;
  const int64_t per = (items + 7) / 8;
  a.per_xcd = (uint32_t)per;
  *blocks = per * 8;
  return a;
}

int64_t gemm_grid_blocks(int64_t m, int64_t n, bool grouped, int32_t groups) {
  int64_t blocks;
  gemm_args(nullptr, nullptr, nullptr, nullptr, m, n, 64, nullptr, grouped, nullptr, groups, &blocks);
  return blocks;
}

hipError_t launch_mx_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t m,
                          int64_t n, int64_t k, void* c, bool bf16, const int32_t* ends, int32_t groups,
                          hipStream_t stream) {
  int64_t blocks;
  const GemmArgs a = gemm_args(qa, sa, qb, sb, m, n, k, c, ends != nullptr, ends, groups, &blocks);
  const dim3 grid((unsigned)blocks), block(kGemmThreads);
  if (ends != nullptr) {
    if (bf16)
      hipLaunchKernelGGL((mx_gemm_kernel<true, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((mx_gemm_kernel<true, false>), grid, block, 0, stream, a);
  } else {
    if (bf16)
      hipLaunchKernelGGL((mx_gemm_kernel<false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((mx_gemm_kernel<false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mx
