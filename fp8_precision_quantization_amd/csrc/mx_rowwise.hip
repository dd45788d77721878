// Row-wise fp8 cast: one bf16 scale per row of a bf16 matrix (gist "FP8
// linear triton with row-wise scaling", quantize_fp8_rowwise).  Per row:
// amax of |x| (bf16); scale = amax / 448 formed in binary32 and rounded to
// bf16; codes = binary32(x) / scale converted to e4m3fn (nearest-even, no
// saturation: magnitudes above 464 and +-Inf become NaN).  The sign bit of
// every code is the sign bit of x, and a NaN scale is written as 0x7FC0.
//
// Work decomposition (gfx950, wave64).  A row of up to 32768 columns stays in
// registers between its amax and its quantisation, so the input is read
// once: a lane holds K 16-byte chunks, and a row is owned by WPR waves of a
// 256-thread workgroup (WPR = 1: four rows per workgroup, a wave per row and
// no barrier; WPR = 4: the workgroup per row, wave maxima combined in LDS).
// Chunk j of a row sits in lane j % 64 of wave (j / 64) % WPR, so each load
// instruction of a wave reads 1 KiB and each store writes 512 contiguous
// bytes.  Loads and stores are buffer instructions whose range is the row:
// chunks past the row's end load as zero (neutral for the amax) and are not
// stored.  Longer rows, and rows whose length or base is not a whole number
// of 16-byte chunks, go to a two-pass kernel that streams the row twice
// (the second pass mostly hits the cache).
//
// The scale and the element quotient are mx_fp8.h's; rows whose scale is
// zero, subnormal, Inf or NaN are uniform per row and take its general path.
#include "mx_fp8.h"
#include "mxcast.h"
#include "mx_launch.h"

namespace mx {

constexpr int kRowThreads = 256;
constexpr int kLoadNTRow = 2;             // cache-policy bits of the input loads: nt
// ... of the code stores: written through (sc0 sc1); 16384 x 16384 118.5 ->
// 116.0 us against ordinary stores, 125.3 us non-temporal (MI355X).
constexpr int kStoreWTRow = 17;

template <int WPR, int K>
__global__ __launch_bounds__(kRowThreads) void rowwise_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                              int64_t cols, uint8_t* __restrict__ q,
                                                              uint16_t* __restrict__ scale) {
  static_assert(WPR == 1 || WPR == 2 || WPR == 4, "waves per row");
  constexpr int kRowsPerGroup = 4 / WPR;
  __shared__ uint32_t wave_amax[4];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wr = wave % WPR;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerGroup + wave / WPR;
  const bool row_on = row < rows;
  // Range of the row; an absent row has range 0, so its loads read zeros
  // and its stores are dropped.
  const uint32_t row_bytes = row_on ? (uint32_t)(cols * 2) : 0u;
  const __amdgpu_buffer_rsrc_t xs = buffer_rsrc(x + (row_on ? row : 0) * cols, row_bytes);
  const __amdgpu_buffer_rsrc_t qs = buffer_rsrc(q + (row_on ? row : 0) * cols, row_bytes / 2);

  uint4 d[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    auto v = __builtin_amdgcn_raw_buffer_load_b128(xs, lane * 16, (k * WPR + wr) * 1024, kLoadNTRow);
    d[k] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < K; ++k)
    m = max2(m, chunk_amax(d[k]));
  m = wave_max(max(m & 0xFFFFu, m >> 16));
  if constexpr (WPR > 1) {
    if (lane == 0)
      wave_amax[wave] = m;
    lds_barrier();
    const int first = wave - wr;
#pragma unroll
    for (int i = 0; i < WPR; ++i)
      m = max(m, wave_amax[first + i]);
  }
  const Fp8Scale p = fp8_scale(m);
  if (row_on && wr == 0 && lane == 0)
    scale[row] = (uint16_t)p.bits;
  if (p.fast) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint2 c = quant8<true>(d[k], p);
      __builtin_amdgcn_raw_buffer_store_b64((u32x2){c.x, c.y}, qs, lane * 8, (k * WPR + wr) * 512, kStoreWTRow);
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint2 c = quant8<false>(d[k], p);
      __builtin_amdgcn_raw_buffer_store_b64((u32x2){c.x, c.y}, qs, lane * 8, (k * WPR + wr) * 512, kStoreWTRow);
    }
  }
}

// Any row length: one workgroup per row, the row read twice.  VEC: the row
// is a whole number of 16-byte chunks at 16-byte aligned addresses (and its
// codes at 8-byte aligned ones); otherwise element by element.
template <bool VEC>
__global__ __launch_bounds__(kRowThreads) void rowwise_stream_kernel(const uint16_t* __restrict__ x,
                                                                     int64_t cols, uint8_t* __restrict__ q,
                                                                     uint16_t* __restrict__ scale) {
  __shared__ uint32_t wave_amax[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * cols;
  uint8_t* qr = q + row * cols;
  const int t = threadIdx.x;
  uint32_t m = 0;
  if (VEC) {
    const uint4* x16 = reinterpret_cast<const uint4*>(xr);
    for (int64_t j = t; j < cols / 8; j += kRowThreads)
      m = max2(m, chunk_amax(x16[j]));
    m = max(m & 0xFFFFu, m >> 16);
  } else {
    for (int64_t i = t; i < cols; i += kRowThreads)
      m = max(m, (uint32_t)xr[i] & 0x7FFFu);
  }
  m = wave_max(m);
  const int wave = t >> 6;
  if ((t & 63) == 0)
    wave_amax[wave] = m;
  lds_barrier();
  m = max(max(wave_amax[0], wave_amax[1]), max(wave_amax[2], wave_amax[3]));
  const Fp8Scale p = fp8_scale(m);
  if (t == 0)
    scale[row] = (uint16_t)p.bits;
  if (VEC) {
    const uint4* x16 = reinterpret_cast<const uint4*>(xr);
    uint2* q8 = reinterpret_cast<uint2*>(qr);
    if (p.fast) {
      for (int64_t j = t; j < cols / 8; j += kRowThreads)
        q8[j] = quant8<true>(x16[j], p);
    } else {
      for (int64_t j = t; j < cols / 8; j += kRowThreads)
        q8[j] = quant8<false>(x16[j], p);
    }
  } else {
    for (int64_t i = t; i < cols; i += kRowThreads)
      qr[i] = (uint8_t)quant1(xr[i], p);
  }
}

constexpr int64_t kRegCols = 32768;   // longest row kept in registers

// Launch shape for a row length: waves per row and chunks per lane, or
// {0, 0} for the streaming kernel.
struct RowShape {
  int wpr, k;
};
static RowShape row_shape(int64_t cols) {
  const int64_t chunks = (cols + 7) / 8;
  if (chunks <= 64 * 8) {
    int k = 1;
    while (64 * k < chunks)
      k *= 2;
    return {1, k};
  }
  if (cols <= kRegCols) {
    int k = 4;   // more than 512 chunks: at least 4 per lane of the workgroup
    while (4 * 64 * k < chunks)
      k *= 2;
    return {4, k};
  }
  return {0, 0};
}

int64_t rowwise_grid_blocks(int64_t rows, int64_t cols, bool vec) {
  const RowShape sh = vec ? row_shape(cols) : RowShape{0, 0};
  if (sh.wpr == 0)
    return rows;
  const int per = 4 / sh.wpr;
  return (rows + per - 1) / per;
}

template <int WPR, int K>
static hipError_t launch_rows(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint16_t* s,
                              hipStream_t stream) {
  const int64_t blocks = (rows + 4 / WPR - 1) / (4 / WPR);
  hipLaunchKernelGGL((rowwise_kernel<WPR, K>), dim3((unsigned)blocks), dim3(kRowThreads), 0, stream, x, rows,
                     cols, q, s);
  return hipGetLastError();
}

hipError_t launch_rowwise(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint16_t* s, bool vec,
                          hipStream_t stream) {
  const RowShape sh = vec ? row_shape(cols) : RowShape{0, 0};
  if (sh.wpr == 1) {
    switch (sh.k) {
      case 1: return launch_rows<1, 1>(x, rows, cols, q, s, stream);
      case 2: return launch_rows<1, 2>(x, rows, cols, q, s, stream);
      case 4: return launch_rows<1, 4>(x, rows, cols, q, s, stream);
      default: return launch_rows<1, 8>(x, rows, cols, q, s, stream);
    }
  }
  if (sh.wpr == 4) {
    switch (sh.k) {
      case 4: return launch_rows<4, 4>(x, rows, cols, q, s, stream);
      case 8: return launch_rows<4, 8>(x, rows, cols, q, s, stream);
      default: return launch_rows<4, 16>(x, rows, cols, q, s, stream);
    }
  }
  if (vec)
    hipLaunchKernelGGL((rowwise_stream_kernel<true>), dim3((unsigned)rows), dim3(kRowThreads), 0, stream, x, cols,
                       q, s);
  else
    hipLaunchKernelGGL((rowwise_stream_kernel<false>), dim3((unsigned)rows), dim3(kRowThreads), 0, stream, x,
                       cols, q, s);
  return hipGetLastError();
}

}  // namespace mx
