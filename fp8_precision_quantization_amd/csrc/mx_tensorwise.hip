// Tensor-wise fp8 cast: one bf16 scale for a whole bf16 tensor.  The
// structure is the one the "[float8nocompile]: Triton kernels for conversion
// to float8 dtypes for forward pass of Float8LinearNoCompile" review thread
// settles on: amaxes of blocks of the tensor computed in parallel into a
// buffer, then one global amax from them, then the conversion.  The scale and
// element rule are the row-wise cast's (mx_fp8.h) applied to that amax.
//
// Three launches over the flattened tensor:
//   1. tw_amax_kernel: at most 2048 workgroups (all resident at once), each
//      the amax of one span of consecutive 16-byte chunks (15-bit magnitude
//      pattern; NaN > Inf > finite) into partial[span];
//   2. tw_scale_kernel: one workgroup reduces the partials and writes the
//      scale's bf16 bits to the output;
//   3. tw_cast_kernel: short workgroups of 1024 chunks each read the scale
//      and convert, loads all issued before the first conversion.
// The thread weighs a separate scale step against every conversion block
// reducing the block amaxes itself.  Timed on MI355X at 16384 x 16384, the
// separate step with short conversion workgroups (123 us for steps 2 + 3)
// beat 2048 long-span workgroups that each reduce the 8 KiB of partials
// (128 us): the short workgroups keep more loads in flight.  Re-reading each
// span from its end, in the hope that the memory-side cache still held the
// end the first pass read last, gained nothing and was dropped.
//
// Loads of x are non-temporal buffer loads ranged to the workgroup's chunks
// (chunks past the end read as zero, which is neutral for the amax); on
// MI355X this took the amax pass from 122 us to ~78 us.  A tensor whose base
// or codes are not 16- / 8-byte aligned is handled element by element with
// the same three steps.  A tail of n % 8 elements after the last whole chunk
// belongs to workgroup 0 of steps 1 and 3.
#include <mutex>

#include "mx_fp8.h"
#include "mxcast.h"
#include "mx_launch.h"

namespace mx {

constexpr int kTwThreads = 256;
constexpr int kTwAmaxUnroll = 8;                   // chunks in flight per thread, step 1
constexpr int kTwCastUnroll = 4;                   // chunks per thread, step 3
constexpr int64_t kTwElemsPerSpan = 32768;         // smallest span of step 1, in elements
constexpr int64_t kTwMaxSpans = 2048;
constexpr int kTwLoadNT = 2;                       // cache-policy bits of the loads of x: nt
// ... of the code stores of step 3: written through (sc0 sc1); 16384 x 16384
// 197.2 -> 191.2 us for the three steps against ordinary stores, 202.8 us
// non-temporal (MI355X).
constexpr int kTwStoreWT = 17;
constexpr int64_t kTwScalarPerGroup = 4096;        // elements per step-3 workgroup, unaligned path

struct TwPlan {
  int64_t spans;  // workgroups of step 1 (= partials)
  int64_t span;   // units (chunks, or elements when !vec) per step-1 workgroup
};

static TwPlan tw_plan(int64_t n, bool vec) {
  TwPlan p;
  p.spans = (n + kTwElemsPerSpan - 1) / kTwElemsPerSpan;
  p.spans = p.spans < 1 ? 1 : p.spans > kTwMaxSpans ? kTwMaxSpans : p.spans;
  const int64_t units = vec ? n / 8 : n;
  const int64_t step = vec ? (int64_t)kTwThreads * kTwAmaxUnroll : kTwThreads;
  const int64_t per = (units + p.spans - 1) / p.spans;
  p.span = (per + step - 1) / step * step;
  if (p.span == 0)
    p.span = step;
  return p;
}

int64_t tensorwise_partials(int64_t n) { return tw_plan(n, false).spans; }

// Block amaxes of the allocation-free entry point: one array per GPU for the
// life of the process, big enough for the largest plan (kTwMaxSpans words).
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not the device address): tensorwise_scratch looks the address
// up once per device, with that device current, and hands that out.
static __device__ __align__(256) uint32_t scratch[kTwMaxSpans];

constexpr int kScratchDevices = 64;
static std::mutex g_scratch_mu;
static uint32_t* g_scratch_ptr[kScratchDevices];

int64_t tensorwise_scratch_bytes() { return (int64_t)sizeof(scratch); }

hipError_t tensorwise_scratch(uint32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return e;
  if (dev < 0 || dev >= kScratchDevices)
    return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
      return e;
    g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Max over the 256 threads of a workgroup (every thread gets it).
__device__ __forceinline__ uint32_t group_max(uint32_t m, uint32_t* lds4) {
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0)
    lds4[threadIdx.x >> 6] = m;
  lds_barrier();
  return max(max(lds4[0], lds4[1]), max(lds4[2], lds4[3]));
}

template <bool VEC>
__global__ __launch_bounds__(kTwThreads) void tw_amax_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                             int64_t span, uint32_t* __restrict__ partial) {
  __shared__ uint32_t lds4[4];
  const int t = threadIdx.x;
  const int64_t units = VEC ? n / 8 : n;
  const int64_t lo = (int64_t)blockIdx.x * span;
  const int64_t hi = min(units, lo + span);
  uint32_t m = 0;
  if (VEC) {
    // a span is at most 2^40 / 8 / 2048 chunks = 1 GiB: 32-bit offsets
    const uint32_t bytes = hi > lo ? (uint32_t)((hi - lo) * 16) : 0u;
    const __amdgpu_buffer_rsrc_t xs = buffer_rsrc(x + (hi > lo ? lo * 8 : 0), bytes);
    constexpr uint32_t kStep = kTwThreads * 16 * kTwAmaxUnroll;
    for (uint32_t off = 0; off < bytes; off += kStep) {
      u32x4 d[kTwAmaxUnroll];
#pragma unroll
      for (int u = 0; u < kTwAmaxUnroll; ++u)
        d[u] = __builtin_amdgcn_raw_buffer_load_b128(xs, t * 16, off + u * kTwThreads * 16, kTwLoadNT);
#pragma unroll
      for (int u = 0; u < kTwAmaxUnroll; ++u)
        m = max2(m, max2(max2(mag2(d[u][0]), mag2(d[u][1])), max2(mag2(d[u][2]), mag2(d[u][3]))));
    }
    m = max(m & 0xFFFFu, m >> 16);
    if (blockIdx.x == 0 && t < n % 8)
      m = max(m, (uint32_t)x[n / 8 * 8 + t] & 0x7FFFu);
  } else {
    for (int64_t i = lo + t; i < hi; i += kTwThreads)
      m = max(m, (uint32_t)x[i] & 0x7FFFu);
  }
  m = group_max(m, lds4);
  if (t == 0)
    partial[blockIdx.x] = m;
}

__global__ __launch_bounds__(kTwThreads) void tw_scale_kernel(const uint32_t* __restrict__ partial, int32_t spans,
                                                              uint16_t* __restrict__ scale) {
  __shared__ uint32_t lds4[4];
  // all of a thread's loads issued at once (this kernel is pure latency);
  // the range of the buffer makes the ones past the last partial read 0
  constexpr int kPerThread = (int)(kTwMaxSpans / kTwThreads);
  const __amdgpu_buffer_rsrc_t ps = buffer_rsrc(partial, (uint32_t)spans * 4u);
  uint32_t v[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k)
    v[k] = __builtin_amdgcn_raw_buffer_load_b32(ps, threadIdx.x * 4, k * kTwThreads * 4, 0);
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k)
    m = max(m, v[k]);
  m = group_max(m, lds4);
  if (threadIdx.x == 0)
    *scale = (uint16_t)fp8_scale_bits(m);
}

template <bool FAST>
__device__ __forceinline__ void tw_cast_chunks(const u32x4 (&d)[kTwCastUnroll], __amdgpu_buffer_rsrc_t qs,
                                               const Fp8Scale& p) {
#pragma unroll
  for (int u = 0; u < kTwCastUnroll; ++u) {
    const uint2 c = quant8<FAST>(make_uint4(d[u][0], d[u][1], d[u][2], d[u][3]), p);
    __builtin_amdgcn_raw_buffer_store_b64((u32x2){c.x, c.y}, qs, threadIdx.x * 8, u * kTwThreads * 8, kTwStoreWT);
  }
}

template <bool VEC>
__global__ __launch_bounds__(kTwThreads) void tw_cast_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                             const uint16_t* __restrict__ scale,
                                                             uint8_t* __restrict__ q) {
  const int t = threadIdx.x;
  const Fp8Scale p = fp8_scale_of_bits(*scale);
  if (VEC) {
    constexpr int64_t kPer = (int64_t)kTwThreads * kTwCastUnroll;
    const int64_t units = n / 8;
    const int64_t lo = (int64_t)blockIdx.x * kPer;
    const int64_t hi = min(units, lo + kPer);
    const uint32_t bytes = hi > lo ? (uint32_t)((hi - lo) * 16) : 0u;
    const __amdgpu_buffer_rsrc_t xs = buffer_rsrc(x + (hi > lo ? lo * 8 : 0), bytes);
    const __amdgpu_buffer_rsrc_t qs = buffer_rsrc(q + (hi > lo ? lo * 8 : 0), bytes / 2);
    u32x4 d[kTwCastUnroll];
#pragma unroll
    for (int u = 0; u < kTwCastUnroll; ++u)
      d[u] = __builtin_amdgcn_raw_buffer_load_b128(xs, t * 16, u * kTwThreads * 16, kTwLoadNT);
    if (p.fast)
      tw_cast_chunks<true>(d, qs, p);
    else
      tw_cast_chunks<false>(d, qs, p);
    if (blockIdx.x == 0 && t < n % 8) {
      const int64_t i = n / 8 * 8 + t;
      q[i] = (uint8_t)quant1(x[i], p);
    }
  } else {
    const int64_t lo = (int64_t)blockIdx.x * kTwScalarPerGroup;
    const int64_t hi = min(n, lo + kTwScalarPerGroup);
    for (int64_t i = lo + t; i < hi; i += kTwThreads)
      q[i] = (uint8_t)quant1(x[i], p);
  }
}

int64_t tensorwise_cast_blocks(int64_t n, bool vec) {
  const int64_t per = vec ? (int64_t)kTwThreads * kTwCastUnroll * 8 : kTwScalarPerGroup;
  const int64_t b = (n + per - 1) / per;
  return b < 1 ? 1 : b;
}

hipError_t launch_tensorwise(const uint16_t* x, int64_t n, uint8_t* q, uint16_t* scale, uint32_t* partial,
                             bool vec, hipStream_t stream) {
  const TwPlan p = tw_plan(n, vec);
  const dim3 block(kTwThreads);
  const dim3 cast_grid((unsigned)tensorwise_cast_blocks(n, vec));
  if (vec)
    hipLaunchKernelGGL((tw_amax_kernel<true>), dim3((unsigned)p.spans), block, 0, stream, x, n, p.span, partial);
  else
    hipLaunchKernelGGL((tw_amax_kernel<false>), dim3((unsigned)p.spans), block, 0, stream, x, n, p.span, partial);
  hipLaunchKernelGGL(tw_scale_kernel, dim3(1), block, 0, stream, partial, (int32_t)p.spans, scale);
  if (vec)
    hipLaunchKernelGGL((tw_cast_kernel<true>), cast_grid, block, 0, stream, x, n, scale, q);
  else
    hipLaunchKernelGGL((tw_cast_kernel<false>), cast_grid, block, 0, stream, x, n, scale, q);
  return hipGetLastError();
}

}  // namespace mx
