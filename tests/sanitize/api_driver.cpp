// Driver for the AddressSanitizer + UndefinedBehaviorSanitizer build of the
// library's host code (argument validation and size helpers in mx_api.hip,
// the plan and grid helpers behind them), run by tests/test_sanitizers.py on
// a machine without a GPU.  Every entry point is called with sizes, group
// counts and pointers drawn from extreme sets (negative, odd, 2^40 and past,
// INT64_MAX / INT64_MIN, INT32 extremes, NULL and misaligned pointers), each
// call holding at least one argument the header rejects, so that no call
// reaches a launch (one that did would report MX_ERR_HIP, counted here as a
// failure).  Any overflow or out-of-bounds access in the host arithmetic
// stops the run.  Exit status 0: clean.
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "mxcast.h"

namespace {

int failures = 0;
long calls = 0;

void expect_rejected(mx_status st, const char* what, int64_t a, int64_t b, int64_t c) {
  ++calls;
  if (st == MX_OK || st == MX_ERR_HIP || st < MX_OK || st > MX_ERR_WORKSPACE) {
    fprintf(stderr, "%s(%lld, %lld, %lld) -> %d (expected a rejection)\n", what, (long long)a, (long long)b,
            (long long)c, (int)st);
    ++failures;
  }
}

const std::vector<int64_t> kBad = {-1, -32, 33, 48, ((int64_t)1 << 40) + 32, ((int64_t)1 << 41), INT64_MAX,
                                   INT64_MIN, INT64_MAX - 127, (int64_t)1 << 62, -((int64_t)1 << 62)};
const std::vector<int64_t> kGood = {32, 128, 4096};
// sizes the layouts reject (they accept any non-negative extent below 2^31)
const std::vector<int64_t> kBadLayout = {-1, -32, ((int64_t)1 << 40) + 32, ((int64_t)1 << 41), INT64_MAX,
                                         INT64_MIN, INT64_MAX - 127, (int64_t)1 << 62, -((int64_t)1 << 62)};
const std::vector<int32_t> kBadGroups = {-1, 0, 1025, INT32_MAX, INT32_MIN};

void* const P = reinterpret_cast<void*>(0x10000);    // aligned, never dereferenced
void* const ODD = reinterpret_cast<void*>(0x10001);
uint8_t* const PU = static_cast<uint8_t*>(P);
const int32_t* const PI = static_cast<const int32_t*>(P);
int64_t* const PL = static_cast<int64_t*>(P);

// every (a, b) pair with at least one of them bad
template <class F>
void pairs(F f) {
  std::vector<int64_t> all(kBad);
  all.insert(all.end(), kGood.begin(), kGood.end());
  for (int64_t a : all)
    for (int64_t b : all) {
      bool bad_a = false, bad_b = false;
      for (int64_t v : kBad) {
        bad_a |= a == v;
        bad_b |= b == v;
      }
      if (bad_a || bad_b)
        f(a, b);
    }
}

}  // namespace

int main() {
  for (int s = -3; s < 12; ++s)
    (void)mx_status_string(s);

  pairs([](int64_t r, int64_t c) {
    expect_rejected(mx_cast_dim0_dim1(P, r, c, PU, PU, PU, PU, nullptr), "mx_cast_dim0_dim1", r, c, 0);
    expect_rejected(mx_cast_dim0_dim1_blocked(P, r, c, PU, PU, PU, PU, nullptr), "mx_cast_dim0_dim1_blocked", r,
                    c, 0);
    expect_rejected(mx_cast_dim0_dim1_mgrouped(P, r, c, PI, 4, PU, PU, PL, PU, PU, nullptr),
                    "mx_cast_dim0_dim1_mgrouped", r, c, 4);
    expect_rejected(mx_cast_dim0_dim1_grouped_blocked(P, r, c, PI, 4, PU, PU, PL, PU, PU, PL, nullptr),
                    "mx_cast_dim0_dim1_grouped_blocked", r, c, 4);
    expect_rejected(mx_quantize_fp8_rowwise(P, r, c < 0 || c > (1 << 30) ? c : ((int64_t)1 << 30) + 1,
                                            PU, static_cast<uint16_t*>(P), nullptr),
                    "mx_quantize_fp8_rowwise", r, c, 0);
    for (int64_t e : {(int64_t)1, (int64_t)16, INT64_MAX, (int64_t)-1}) {
      expect_rejected(mx_cast_dim1_3d(P, e, r, c, PU, PU, nullptr), "mx_cast_dim1_3d", e, r, c);
      expect_rejected(mx_cast_dim1_3d_blocked(P, e, r, c, PU, PU, nullptr), "mx_cast_dim1_3d_blocked", e, r, c);
    }
    for (int64_t k : {(int64_t)64, (int64_t)-32, INT64_MAX}) {
      expect_rejected(mx_gemm_mxfp8(PU, PU, PU, PU, r, c, k == 64 ? -32 : k, P, 1, nullptr), "mx_gemm_mxfp8", r,
                      c, k);
      expect_rejected(mx_grouped_gemm_mxfp8(PU, PU, PU, PU, PI, 4, r, c, k == 64 ? 33 : k, P, 1, nullptr),
                      "mx_grouped_gemm_mxfp8", r, c, k);
      expect_rejected(mx_kgrouped_gemm_mxfp8(PU, PU, PU, PU, PI, 4, r, c, k == 64 ? 33 : k, P, 1, nullptr),
                      "mx_kgrouped_gemm_mxfp8", r, c, k);
    }
    // size helpers take any value
    for (int64_t b : {(int64_t)1, (int64_t)3, INT64_MAX, INT64_MIN})
      (void)mx_blocked_bytes(b, r, c);
    for (int32_t g : {1, 4, 1024, 1025, -1, INT32_MAX, INT32_MIN})
      for (int32_t axis : {0, 1, 2, -1})
        (void)mx_blocked_grouped_bytes(r, c, g, axis);
    (void)mx_tensorwise_workspace_bytes(r);
    expect_rejected(mx_quantize_fp8_tensorwise(P, r < 0 || r > ((int64_t)1 << 40) ? r : -r, PU,
                                               static_cast<uint16_t*>(P), P, INT64_MAX, nullptr),
                    "mx_quantize_fp8_tensorwise", r, 0, 0);
    expect_rejected(mx_quantize_fp8_tensorwise_noalloc(P, r < 0 || r > ((int64_t)1 << 40) ? r : -r, PU,
                                                       static_cast<uint16_t*>(P), nullptr),
                    "mx_quantize_fp8_tensorwise_noalloc", r, 0, 0);
  });

  // layouts: sizes past every bound, and bad group counts / axes with good sizes
  for (int64_t r : kBadLayout)
    for (int64_t c : kBadLayout) {
      expect_rejected(mx_scales_to_blocked(PU, 1, r, c, PU, nullptr), "mx_scales_to_blocked", r, c, 1);
      expect_rejected(mx_scales_to_blocked(PU, INT64_MAX, r, c, PU, nullptr), "mx_scales_to_blocked", r, c,
                      INT64_MAX);
      for (int32_t axis : {0, 1})
        expect_rejected(mx_scales_to_blocked_grouped(PU, r, c, PI, 4, axis, PU, PL, nullptr),
                        "mx_scales_to_blocked_grouped", r, c, axis);
    }
  for (int64_t r : kGood)
    for (int32_t g : kBadGroups)
      for (int32_t axis : {0, 1, 2, -1}) {
        expect_rejected(mx_scales_to_blocked_grouped(PU, r, r, PI, g, axis, PU, PL, nullptr),
                        "mx_scales_to_blocked_grouped", r, g, axis);
        expect_rejected(mx_cast_dim0_dim1_mgrouped(P, r, r, PI, g, PU, PU, PL, PU, PU, nullptr),
                        "mx_cast_dim0_dim1_mgrouped", r, g, 0);
        expect_rejected(mx_grouped_gemm_mxfp8(PU, PU, PU, PU, PI, g, r, r, r, P, 1, nullptr),
                        "mx_grouped_gemm_mxfp8", r, g, 0);
      }
  // misaligned and NULL pointers with good sizes
  expect_rejected(mx_cast_dim0_dim1(ODD, 32, 32, PU, PU, PU, PU, nullptr), "mx_cast_dim0_dim1 odd", 32, 32, 0);
  expect_rejected(mx_cast_dim0_dim1(nullptr, 32, 32, PU, PU, PU, PU, nullptr), "mx_cast_dim0_dim1 null", 32, 32,
                  0);
  expect_rejected(mx_quantize_fp8_tensorwise(P, 64, PU, static_cast<uint16_t*>(P), P, 3, nullptr),
                  "mx_quantize_fp8_tensorwise small workspace", 64, 3, 0);

  if (failures) {
    fprintf(stderr, "%d of %ld calls not rejected\n", failures, calls);
    return 1;
  }
  printf("api sanitizer run clean (%ld calls)\n", calls);
  return 0;
}
