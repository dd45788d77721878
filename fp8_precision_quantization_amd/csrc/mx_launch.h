// Internal launchers behind the C ABI (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// Cast kernel: rows x cols bf16; q0/s0 (dim0) and/or q1/s1 (dim1) non-null.
// rows_per_seg splits the rows into segments whose dim1 outputs are stored
// one after another (3D expert weights); pass rows for a plain 2D cast.
// blocked: scales in the 128x4 blocked layout (dim1 segments must then be
// multiples of 128 rows, or the whole matrix).
hipError_t launch_cast_any(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_per_seg,
                           uint8_t* q0, uint8_t* s0, uint8_t* q1, uint8_t* s1, bool blocked,
                           hipStream_t stream);
int64_t cast_grid_blocks(int64_t rows, int64_t cols);
// dim0 + (optional) plain dim1 cast with the dim0 scales in the M-grouped
// blocked layout (s0_bytes = the grouped output's size).
hipError_t launch_cast_mgrouped(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* ends,
                                int32_t groups, uint8_t* q0, uint8_t* s0_grouped, int64_t s0_bytes,
                                int64_t* out_starts, uint8_t* q1, uint8_t* s1, hipStream_t stream);
hipError_t launch_cast_grouped_blocked(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* ends,
                                       int32_t groups, uint8_t* q0, uint8_t* s0_grouped, int64_t s0_bytes,
                                       int64_t* row_starts, uint8_t* q1, uint8_t* s1_grouped, int64_t s1_bytes,
                                       int64_t* col_starts, hipStream_t stream);

hipError_t launch_blocked_batched(const uint8_t* s, int64_t batch, int64_t rows, int64_t cols,
                                  uint8_t* out, hipStream_t stream);
// Grid of a blocked-layout launch; mode 0 batched, 1 M groups, 2 K groups.
int64_t blocked_grid_blocks(int32_t mode, int64_t batch, int64_t rows, int64_t cols, int32_t groups);
hipError_t launch_blocked_grouped(const uint8_t* s, int64_t rows, int64_t cols, const int32_t* ends,
                                  int32_t groups, int32_t axis, uint8_t* out, int64_t out_bytes,
                                  int64_t* out_starts, hipStream_t stream);

// In place, blocked -> plain: scale matrices m0 (r0 x c0 bytes) and m1 (r1 x
// c1), either may be null; rows multiples of 128, columns multiples of 16 (a
// plain row is whole 16-byte chunks) and at most kUnblockMaxCols (a 128-row
// band then fills 128 KiB of LDS), 16-byte aligned.
constexpr int64_t kUnblockMaxCols = 1024;
hipError_t launch_unblock_inplace(uint8_t* m0, int64_t r0, int64_t c0, uint8_t* m1, int64_t r1, int64_t c1,
                                  hipStream_t stream);

// Row-wise fp8 cast.  vec: cols % 8 == 0, x 16-byte and q 8-byte aligned.
hipError_t launch_rowwise(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint16_t* s, bool vec,
                          hipStream_t stream);
int64_t rowwise_grid_blocks(int64_t rows, int64_t cols, bool vec);

// Tensor-wise fp8 cast (three launches); partial holds tensorwise_partials(n)
// words.  vec: x 16-byte and q 8-byte aligned.
hipError_t launch_tensorwise(const uint16_t* x, int64_t n, uint8_t* q, uint16_t* scale, uint32_t* partial,
                             bool vec, hipStream_t stream);
int64_t tensorwise_partials(int64_t n);
// The allocation-free variant's per-device scratch (the device address of a
// static __device__ array, looked up on the current device) and its size.
hipError_t tensorwise_scratch(uint32_t** out);
int64_t tensorwise_scratch_bytes();
int64_t tensorwise_cast_blocks(int64_t n, bool vec);

// MX-scaled GEMM, c fp32 or bf16; modes: 0 dense, 1 grouped along M, 2 grouped
// along K (ends non-null for 1 and 2)
hipError_t launch_mx_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t m,
                          int64_t n, int64_t k, void* c, bool bf16, int mode, const int32_t* ends, int32_t groups,
                          hipStream_t stream);
int64_t gemm_grid_blocks(int64_t m, int64_t n, int mode, int32_t groups);

}  // namespace mx
