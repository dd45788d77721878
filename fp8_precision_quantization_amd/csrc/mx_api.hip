// C ABI of libmxcast: argument validation on the host, then the launches
// (one per call, three for the tensor-wise cast).  Every check runs before
// any HIP call, so a rejected call enqueues nothing and the checks can be
// exercised on a machine without a GPU.
#include <limits.h>

#include "mx_launch.h"
#include "mxcast.h"

namespace {

constexpr int64_t kMaxExtent = (int64_t)1 << 40;  // per-dimension bound, keeps products in int64
// The cast kernels address 32 rows of a row-major matrix from one scalar base
// with 32-bit row offsets: 32 * cols * 2 bytes must stay below 2^31.
constexpr int64_t kMaxCastCols = (int64_t)1 << 25;
// The dispatch packet holds the grid size in work-items as a 32-bit field, and
// every launch checked against this bound has 256 threads per workgroup.
constexpr int64_t kMaxGridBlocks = (int64_t)UINT32_MAX / 256;
constexpr int64_t kMaxRowwiseCols = (int64_t)1 << 30;
// The GEMM addresses a wave's 64 operand rows from one base with 32-bit
// offsets: 64 * k bytes must stay below 2^31.
constexpr int64_t kMaxGemmK = (int64_t)1 << 23;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

mx_status from_hip(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

mx_status check_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t m,
                     int64_t n, int64_t k, const void* c, int32_t c_bf16) {
  if (m < 0 || n < 0 || k < 0 || k % MX_BLOCK != 0 || m >= INT_MAX || n >= INT_MAX || k > kMaxGemmK)
    return MX_ERR_SHAPE;
  if (c_bf16 != 0 && c_bf16 != 1)
    return MX_ERR_SHAPE;
  if (m == 0 || n == 0)
    return MX_OK;
  if (c == nullptr || (k > 0 && (qa == nullptr || sa == nullptr || qb == nullptr || sb == nullptr)))
    return MX_ERR_NULL;
  if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(sa, 16) || !aligned(sb, 16) ||
      !aligned(c, c_bf16 ? 2 : 4))
    return MX_ERR_ALIGN;
  return MX_OK;
}

}  // namespace

extern "C" {

const char* mx_status_string(int status) {
  switch (status) {
    case MX_OK: return "ok";
    case MX_ERR_NULL: return "a required pointer is NULL";
    case MX_ERR_SHAPE: return "unsupported shape (negative, not a multiple of the block, or too large)";
    case MX_ERR_GROUPS: return "num_groups or group_axis out of range";
    case MX_ERR_HIP: return "the HIP runtime rejected the launch";
    case MX_ERR_ALIGN: return "a pointer is not aligned as required";
    case MX_ERR_WORKSPACE: return "the workspace is smaller than required";
  }
  return "unknown status";
}

mx_status mx_cast_dim0_dim1(const void* x, int64_t rows, int64_t cols, uint8_t* q_row,
                            uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, hipStream_t stream) {
  if (rows < 0 || cols < 0 || rows % MX_BLOCK != 0 || cols % MX_BLOCK != 0 || rows > kMaxExtent ||
      cols > kMaxCastCols)
    return MX_ERR_SHAPE;
  if (rows == 0 || cols == 0)
    return MX_OK;  // nothing to read or write; the pointers may be NULL
  const bool d0 = q_row != nullptr || s_row != nullptr;
  const bool d1 = q_col != nullptr || s_col != nullptr;
  if (x == nullptr || (!d0 && !d1))
    return MX_ERR_NULL;
  if ((d0 && (q_row == nullptr || s_row == nullptr)) || (d1 && (q_col == nullptr || s_col == nullptr)))
    return MX_ERR_NULL;
  if (mx::cast_grid_blocks(rows, cols) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  if (!aligned(x, 16) || (d0 && !aligned(q_row, 8)) || (d1 && !aligned(q_col, 16)))
    return MX_ERR_ALIGN;
  // On some large inputs whose 128-row scale bands all fit one workgroup's
  // LDS, the scales are written in the blocked layout, whose stores are whole
  // lines, and then turned into the plain one in place (the same bytes).
  // Timed on MI355X against the direct kernel's partial 1- and 4-byte scale
  // runs (both directions, 150 calls after 40, us via blocked / direct):
  // 16384 x 16384 169.0 / 182.7, 16384 x 4096 49.8 / 58.4, 32768 x 8192
  // 175.2 / 190.6, 32768 x 16384 421 / 438, 16384 x 8192 91.6 / 92.0; the
  // direct kernel wins at 16384 x 5120 (56.8 / 60.7), 16640 x 8192 (89.7 /
  // 95.5), 32768 x 4096 (88.2 / 93.4), 16640 x 5120, 12288 x 8192,
  // 8192 x 16384, 4096 x 16384 and smaller inputs.  The direct kernel is at
  // its slowest where both sizes are powers of two (its partial scale lines
  // then collide), hence the rule.  Every band is then whole 16-byte chunks.
  const bool big = (rows % 16384 == 0 && cols % 8192 == 0) || (rows == 16384 && cols == 4096);
  const bool via_blocked = big &&
                           (!d0 || (cols / MX_BLOCK <= mx::kUnblockMaxCols && aligned(s_row, 16))) &&
                           (!d1 || (rows / MX_BLOCK <= mx::kUnblockMaxCols && aligned(s_col, 16)));
  if (via_blocked) {
    hipError_t e = mx::launch_cast_any(static_cast<const uint16_t*>(x), rows, cols, rows, d0 ? q_row : nullptr,
                                       d0 ? s_row : nullptr, d1 ? q_col : nullptr, d1 ? s_col : nullptr, true,
                                       stream);
    if (e == hipSuccess)
      e = mx::launch_unblock_inplace(d0 ? s_row : nullptr, rows, cols / MX_BLOCK, d1 ? s_col : nullptr, cols,
                                     rows / MX_BLOCK, stream);
    return from_hip(e);
  }
  return from_hip(mx::launch_cast_any(static_cast<const uint16_t*>(x), rows, cols, rows,
                                      d0 ? q_row : nullptr, d0 ? s_row : nullptr,
                                      d1 ? q_col : nullptr, d1 ? s_col : nullptr, false, stream));
}

mx_status mx_cast_dim0_dim1_blocked(const void* x, int64_t rows, int64_t cols, uint8_t* q_row,
                                    uint8_t* s_row_blocked, uint8_t* q_col, uint8_t* s_col_blocked,
                                    hipStream_t stream) {
  if (rows < 0 || cols < 0 || rows % MX_BLOCK != 0 || cols % MX_BLOCK != 0 || rows > kMaxExtent ||
      cols > kMaxCastCols)
    return MX_ERR_SHAPE;
  if (rows == 0 || cols == 0)
    return MX_OK;  // nothing to read or write; the pointers may be NULL
  const bool d0 = q_row != nullptr || s_row_blocked != nullptr;
  const bool d1 = q_col != nullptr || s_col_blocked != nullptr;
  if (x == nullptr || (!d0 && !d1))
    return MX_ERR_NULL;
  if ((d0 && (q_row == nullptr || s_row_blocked == nullptr)) ||
      (d1 && (q_col == nullptr || s_col_blocked == nullptr)))
    return MX_ERR_NULL;
  if (mx::cast_grid_blocks(rows, cols) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  if (!aligned(x, 16) || (d0 && (!aligned(q_row, 8) || !aligned(s_row_blocked, 16))) ||
      (d1 && (!aligned(q_col, 16) || !aligned(s_col_blocked, 16))))
    return MX_ERR_ALIGN;
  return from_hip(mx::launch_cast_any(static_cast<const uint16_t*>(x), rows, cols, rows,
                                      d0 ? q_row : nullptr, d0 ? s_row_blocked : nullptr,
                                      d1 ? q_col : nullptr, d1 ? s_col_blocked : nullptr, true,
                                      stream));
}

mx_status mx_cast_dim0_dim1_mgrouped(const void* x, int64_t rows, int64_t cols,
                                     const int32_t* group_end_offsets, int32_t num_groups, uint8_t* q_row,
                                     uint8_t* s_row_grouped, int64_t* out_group_starts, uint8_t* q_col,
                                     uint8_t* s_col, hipStream_t stream) {
  if (rows < 0 || cols < 0 || rows % MX_BLOCK != 0 || cols % MX_BLOCK != 0 || rows > kMaxExtent ||
      cols > kMaxCastCols)
    return MX_ERR_SHAPE;
  if (num_groups < 1 || num_groups > MX_MAX_GROUPS)
    return MX_ERR_GROUPS;
  if (rows + 128 * (int64_t)num_groups >= INT_MAX)
    return MX_ERR_SHAPE;
  const int64_t bytes = mx_blocked_grouped_bytes(rows, cols / MX_BLOCK, num_groups, 0);
  if (group_end_offsets == nullptr || (bytes > 0 && s_row_grouped == nullptr))
    return MX_ERR_NULL;
  if (!aligned(group_end_offsets, 4) || (s_row_grouped != nullptr && !aligned(s_row_grouped, 16)) ||
      (out_group_starts != nullptr && !aligned(out_group_starts, 8)))
    return MX_ERR_ALIGN;
  if (rows == 0 || cols == 0) {
    // no codes: the grouped scale buffer is all padding (and the starts)
    return from_hip(mx::launch_blocked_grouped(nullptr, rows, cols / MX_BLOCK, group_end_offsets, num_groups,
                                               0, s_row_grouped, bytes, out_group_starts, stream));
  }
  const bool d1 = q_col != nullptr || s_col != nullptr;
  if (x == nullptr || q_row == nullptr || (d1 && (q_col == nullptr || s_col == nullptr)))
    return MX_ERR_NULL;
  if (mx::cast_grid_blocks(rows, cols) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q_row, 8) || (d1 && !aligned(q_col, 16)))
    return MX_ERR_ALIGN;
  return from_hip(mx::launch_cast_mgrouped(static_cast<const uint16_t*>(x), rows, cols, group_end_offsets,
                                           num_groups, q_row, s_row_grouped, bytes, out_group_starts,
                                           d1 ? q_col : nullptr, d1 ? s_col : nullptr, stream));
}

mx_status mx_cast_dim0_dim1_grouped_blocked(const void* x, int64_t rows, int64_t cols,
                                            const int32_t* group_end_offsets, int32_t num_groups, uint8_t* q_row,
                                            uint8_t* s_row_grouped, int64_t* row_group_starts, uint8_t* q_col,
                                            uint8_t* s_col_grouped, int64_t* col_group_starts,
                                            hipStream_t stream) {
  if (rows < 0 || cols < 0 || rows % MX_BLOCK != 0 || cols % MX_BLOCK != 0 || rows > kMaxExtent ||
      cols > kMaxCastCols || (cols == 0 && rows > 0))
    return MX_ERR_SHAPE;
  if (num_groups < 1 || num_groups > MX_MAX_GROUPS)
    return MX_ERR_GROUPS;
  if (rows + 128 * (int64_t)num_groups >= INT_MAX || cols + 128 >= INT_MAX)
    return MX_ERR_SHAPE;
  const int64_t bytes0 = mx_blocked_grouped_bytes(rows, cols / MX_BLOCK, num_groups, 0);
  const int64_t bytes1 = mx_blocked_grouped_bytes(cols, rows / MX_BLOCK, num_groups, 1);
  if (group_end_offsets == nullptr || (bytes0 > 0 && s_row_grouped == nullptr) ||
      (bytes1 > 0 && s_col_grouped == nullptr))
    return MX_ERR_NULL;
  if (!aligned(group_end_offsets, 4) || (s_row_grouped != nullptr && !aligned(s_row_grouped, 16)) ||
      (s_col_grouped != nullptr && !aligned(s_col_grouped, 16)) ||
      (row_group_starts != nullptr && !aligned(row_group_starts, 8)) ||
      (col_group_starts != nullptr && !aligned(col_group_starts, 8)))
    return MX_ERR_ALIGN;
  if (rows == 0) {
    // no codes and every group empty: both grouped buffers are all padding
    hipError_t e = mx::launch_blocked_grouped(nullptr, rows, cols / MX_BLOCK, group_end_offsets, num_groups, 0,
                                              s_row_grouped, bytes0, row_group_starts, stream);
    if (e == hipSuccess)
      e = mx::launch_blocked_grouped(nullptr, cols, rows / MX_BLOCK, group_end_offsets, num_groups, 1,
                                     s_col_grouped, bytes1, col_group_starts, stream);
    return from_hip(e);
  }
  if (x == nullptr || q_row == nullptr || q_col == nullptr)
    return MX_ERR_NULL;
  if (mx::cast_grid_blocks(rows, cols) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q_row, 8) || !aligned(q_col, 16))
    return MX_ERR_ALIGN;
  return from_hip(mx::launch_cast_grouped_blocked(static_cast<const uint16_t*>(x), rows, cols, group_end_offsets,
                                                  num_groups, q_row, s_row_grouped, bytes0, row_group_starts,
                                                  q_col, s_col_grouped, bytes1, col_group_starts, stream));
}

mx_status mx_cast_dim1_3d(const void* w, int64_t experts, int64_t n, int64_t k, uint8_t* q,
                          uint8_t* s, hipStream_t stream) {
  if (experts < 0 || n < 0 || k < 0 || n % MX_BLOCK != 0 || k % MX_BLOCK != 0 ||
      experts > kMaxExtent || n > kMaxExtent || k > kMaxCastCols ||
      (n > 0 && experts > kMaxExtent / n))
    return MX_ERR_SHAPE;
  if (experts == 0 || n == 0 || k == 0)
    return MX_OK;  // nothing to read or write; the pointers may be NULL
  if (w == nullptr || q == nullptr || s == nullptr)
    return MX_ERR_NULL;
  if (mx::cast_grid_blocks(experts * n, k) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(q, 16))
    return MX_ERR_ALIGN;
  return from_hip(mx::launch_cast_any(static_cast<const uint16_t*>(w), experts * n, k, n, nullptr,
                                      nullptr, q, s, false, stream));
}

mx_status mx_cast_dim1_3d_blocked(const void* w, int64_t experts, int64_t n, int64_t k, uint8_t* q,
                                  uint8_t* s_blocked, hipStream_t stream) {
  if (experts < 0 || n < 0 || k < 0 || n % 128 != 0 || k % MX_BLOCK != 0 ||
      experts > kMaxExtent || n > kMaxExtent || k > kMaxCastCols ||
      (n > 0 && experts > kMaxExtent / n))
    return MX_ERR_SHAPE;
  if (experts == 0 || n == 0 || k == 0)
    return MX_OK;  // nothing to read or write; the pointers may be NULL
  if (w == nullptr || q == nullptr || s_blocked == nullptr)
    return MX_ERR_NULL;
  if (mx::cast_grid_blocks(experts * n, k) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(s_blocked, 16))
    return MX_ERR_ALIGN;
  return from_hip(mx::launch_cast_any(static_cast<const uint16_t*>(w), experts * n, k, n, nullptr,
                                      nullptr, q, s_blocked, true, stream));
}

int64_t mx_blocked_bytes(int64_t batch, int64_t rows, int64_t cols) {
  if (batch < 0 || rows < 0 || cols < 0 || batch > kMaxExtent || rows > kMaxExtent ||
      cols > kMaxExtent)
    return -1;
  const int64_t r = round_up(rows, 128), c = round_up(cols, 4);
  if (c > 0 && r > INT64_MAX / c)
    return -1;
  const int64_t per = r * c;
  if (per > 0 && batch > INT64_MAX / per)
    return -1;
  return batch * per;
}

mx_status mx_scales_to_blocked(const uint8_t* s, int64_t batch, int64_t rows, int64_t cols,
                               uint8_t* out, hipStream_t stream) {
  const int64_t bytes = mx_blocked_bytes(batch, rows, cols);
  if (bytes < 0)
    return MX_ERR_SHAPE;
  if (bytes == 0)
    return MX_OK;
  if (out == nullptr || (s == nullptr && rows * cols > 0))
    return MX_ERR_NULL;
  if (mx::blocked_grid_blocks(0, batch, rows, cols, 1) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  if (!aligned(out, 16))
    return MX_ERR_ALIGN;
  return from_hip(mx::launch_blocked_batched(s, batch, rows, cols, out, stream));
}

int64_t mx_blocked_grouped_bytes(int64_t rows, int64_t cols, int32_t num_groups,
                                 int32_t group_axis) {
  if (rows < 0 || cols < 0 || num_groups < 1 || num_groups > MX_MAX_GROUPS ||
      (group_axis != 0 && group_axis != 1))
    return -1;
  if (rows >= INT_MAX || cols >= INT_MAX || rows + 128 * (int64_t)num_groups >= INT_MAX ||
      cols + 4 * (int64_t)num_groups >= INT_MAX)
    return -1;
  if (group_axis == 0)
    return (rows + 128 * (int64_t)num_groups) * round_up(cols, 4);
  return round_up(rows, 128) * (round_up(cols, 4) + 4 * (int64_t)num_groups);
}

mx_status mx_scales_to_blocked_grouped(const uint8_t* s, int64_t rows, int64_t cols,
                                       const int32_t* group_end_offsets, int32_t num_groups,
                                       int32_t group_axis, uint8_t* out,
                                       int64_t* out_group_starts, hipStream_t stream) {
  if (num_groups < 1 || num_groups > MX_MAX_GROUPS || (group_axis != 0 && group_axis != 1))
    return MX_ERR_GROUPS;
  if (rows < 0 || cols < 0 || rows >= INT_MAX || cols >= INT_MAX || rows + 128 * (int64_t)num_groups >= INT_MAX ||
      cols + 4 * (int64_t)num_groups >= INT_MAX)
    return MX_ERR_SHAPE;
  const int64_t bytes = mx_blocked_grouped_bytes(rows, cols, num_groups, group_axis);
  if (group_end_offsets == nullptr || (out == nullptr && bytes > 0) ||
      (s == nullptr && rows * cols > 0))
    return MX_ERR_NULL;
  if (mx::blocked_grid_blocks(group_axis == 0 ? 1 : 2, 1, rows, cols, num_groups) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  if (out != nullptr && !aligned(out, 16))
    return MX_ERR_ALIGN;
  if (out_group_starts != nullptr && !aligned(out_group_starts, 8))
    return MX_ERR_ALIGN;
  if (!aligned(group_end_offsets, 4))
    return MX_ERR_ALIGN;
  return from_hip(mx::launch_blocked_grouped(s, rows, cols, group_end_offsets, num_groups,
                                             group_axis, out, bytes, out_group_starts, stream));
}

mx_status mx_quantize_fp8_rowwise(const void* x, int64_t rows, int64_t cols, uint8_t* q,
                                  uint16_t* scale, hipStream_t stream) {
  if (rows < 0 || cols < 0 || rows > kMaxExtent || cols > kMaxRowwiseCols)
    return MX_ERR_SHAPE;
  if (rows == 0 || cols == 0)
    return MX_OK;  // nothing to read or write; the pointers may be NULL
  if (x == nullptr || q == nullptr || scale == nullptr)
    return MX_ERR_NULL;
  if (!aligned(x, 2) || !aligned(scale, 2))
    return MX_ERR_ALIGN;
  const bool vec = cols % 8 == 0 && aligned(x, 16) && aligned(q, 8);
  if (mx::rowwise_grid_blocks(rows, cols, vec) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  return from_hip(mx::launch_rowwise(static_cast<const uint16_t*>(x), rows, cols, q, scale, vec, stream));
}

int64_t mx_tensorwise_workspace_bytes(int64_t n) {
  if (n < 0 || n > kMaxExtent)
    return -1;
  return 4 * mx::tensorwise_partials(n);
}

mx_status mx_quantize_fp8_tensorwise(const void* x, int64_t n, uint8_t* q, uint16_t* scale, void* workspace,
                                     int64_t workspace_bytes, hipStream_t stream) {
  if (n < 0 || n > kMaxExtent)
    return MX_ERR_SHAPE;
  if (n == 0)
    return MX_OK;  // nothing to read or write; the pointers may be NULL
  if (x == nullptr || q == nullptr || scale == nullptr || workspace == nullptr)
    return MX_ERR_NULL;
  if (workspace_bytes < mx_tensorwise_workspace_bytes(n))
    return MX_ERR_WORKSPACE;
  if (!aligned(x, 2) || !aligned(scale, 2) || !aligned(workspace, 4))
    return MX_ERR_ALIGN;
  const bool vec = aligned(x, 16) && aligned(q, 8);
  if (mx::tensorwise_cast_blocks(n, vec) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  return from_hip(mx::launch_tensorwise(static_cast<const uint16_t*>(x), n, q, scale,
                                        static_cast<uint32_t*>(workspace), vec, stream));
}

mx_status mx_quantize_fp8_tensorwise_noalloc(const void* x, int64_t n, uint8_t* q, uint16_t* scale,
                                             hipStream_t stream) {
  if (n < 0 || n > kMaxExtent)
    return MX_ERR_SHAPE;
  if (n == 0)
    return MX_OK;  // nothing to read or write; the pointers may be NULL
  if (x == nullptr || q == nullptr || scale == nullptr)
    return MX_ERR_NULL;
  if (mx_tensorwise_workspace_bytes(n) > mx::tensorwise_scratch_bytes())
    return MX_ERR_WORKSPACE;
  if (!aligned(x, 2) || !aligned(scale, 2))
    return MX_ERR_ALIGN;
  const bool vec = aligned(x, 16) && aligned(q, 8);
  if (mx::tensorwise_cast_blocks(n, vec) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  uint32_t* partial = nullptr;
  if (mx::tensorwise_scratch(&partial) != hipSuccess)
    return MX_ERR_HIP;
  return from_hip(mx::launch_tensorwise(static_cast<const uint16_t*>(x), n, q, scale, partial, vec, stream));
}

mx_status mx_gemm_mxfp8(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t m,
                        int64_t n, int64_t k, void* c, int32_t c_bf16, hipStream_t stream) {
  const mx_status st = check_gemm(qa, sa, qb, sb, m, n, k, c, c_bf16);
  if (st != MX_OK || m == 0 || n == 0)
    return st;
  if (mx::gemm_grid_blocks(m, n, 0, 0) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  return from_hip(mx::launch_mx_gemm(qa, sa, qb, sb, m, n, k, c, c_bf16 != 0, 0, nullptr, 0, stream));
}

mx_status mx_grouped_gemm_mxfp8(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
                                const int32_t* group_end_offsets, int32_t num_groups, int64_t m, int64_t n,
                                int64_t k, void* c, int32_t c_bf16, hipStream_t stream) {
  if (num_groups < 1 || num_groups > MX_MAX_GROUPS)
    return MX_ERR_GROUPS;
  const mx_status st = check_gemm(qa, sa, qb, sb, m, n, k, c, c_bf16);
  if (st != MX_OK || m == 0 || n == 0)
    return st;
  if (m + 256 * (int64_t)num_groups >= INT_MAX)
    return MX_ERR_SHAPE;
  if (group_end_offsets == nullptr)
    return MX_ERR_NULL;
  if (!aligned(group_end_offsets, 4))
    return MX_ERR_ALIGN;
  if (mx::gemm_grid_blocks(m, n, 1, num_groups) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  return from_hip(
      mx::launch_mx_gemm(qa, sa, qb, sb, m, n, k, c, c_bf16 != 0, 1, group_end_offsets, num_groups, stream));
}

mx_status mx_kgrouped_gemm_mxfp8(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
                                 const int32_t* group_end_offsets, int32_t num_groups, int64_t m, int64_t n,
                                 int64_t k, void* c, int32_t c_bf16, hipStream_t stream) {
  if (num_groups < 1 || num_groups > MX_MAX_GROUPS)
    return MX_ERR_GROUPS;
  const mx_status st = check_gemm(qa, sa, qb, sb, m, n, k, c, c_bf16);
  if (st != MX_OK || m == 0 || n == 0)
    return st;
  if (k + 4 * 32 * (int64_t)num_groups >= INT_MAX || m + 128 >= INT_MAX || n + 128 >= INT_MAX)
    return MX_ERR_SHAPE;
  if (group_end_offsets == nullptr)
    return MX_ERR_NULL;
  if (!aligned(group_end_offsets, 4))
    return MX_ERR_ALIGN;
  if (mx::gemm_grid_blocks(m, n, 2, num_groups) > kMaxGridBlocks)
    return MX_ERR_SHAPE;
  return from_hip(
      mx::launch_mx_gemm(qa, sa, qb, sb, m, n, k, c, c_bf16 != 0, 2, group_end_offsets, num_groups, stream));
}

}  // extern "C"
