// Host-side driver for the sanitizer test (tests/test_abi_sanitize.py).
//
// Built with g++ -fsanitize=address,undefined together with the library's C
// ABI source (gla_abi.cpp) and a stub of the kernel-launch layer, so that
// AddressSanitizer and UndefinedBehaviorSanitizer watch every validation path
// of the entry points on the host.  No GPU code is compiled or run: the
// pointers are fake, never-dereferenced addresses, and the one valid call is
// made only when the HIP runtime reports no device (it must then return
// GLA_ERR_HIP).  Exit status 0 when every call returned its expected status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include <hip/hip_runtime_api.h>

#include "gla.h"
#include "gla_internal.h"
#include "../gated_bidirectional_linear_amd/csrc/gla_launch.h"

// The launch layer is replaced: nothing here may reach a device.
namespace gla {
hipError_t launch_operator(const LaunchArgs&, Timer&) { return hipErrorInvalidValue; }
}  // namespace gla

namespace {

int failures = 0;

void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    std::printf("FAIL line %d: %s returned %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

const uintptr_t A = uintptr_t(1) << 40;
void* P[10];

struct Args {
  void* p[10];
  int batch = 1, T = 2, H = 4, W = 4, heads = 2, d = 32;
  float eps = 1e-6f;
  int dtype = GLA_DTYPE_BF16;
  int F = 1, t_offset = 0, include_self = 1;
  Args() {
    for (int i = 0; i < 10; ++i) p[i] = P[i];
  }
};

int fwd(const Args& a) {
  return gla_forward(a.p[0], a.p[1], a.p[2], a.p[3], a.p[4], (const float*)a.p[5], a.T, a.H, a.W, a.heads, a.d,
                     a.eps, a.p[6], nullptr, a.dtype);
}
int fwd_b(const Args& a) {
  return gla_forward_batch(a.p[0], a.p[1], a.p[2], a.p[3], a.p[4], (const float*)a.p[5], a.batch, a.T, a.H, a.W,
                           a.heads, a.d, a.eps, a.p[6], nullptr, a.dtype);
}
int bc(const Args& a) {
  return gla_block_causal_forward(a.p[0], a.p[1], a.p[2], a.p[3], a.p[4], (const float*)a.p[5], a.T, a.H, a.W,
                                  a.heads, a.d, a.eps, a.p[6], nullptr, (float*)a.p[7], (float*)a.p[8], a.F,
                                  a.dtype);
}
int bc_at(const Args& a) {
  return gla_block_causal_forward_at(a.p[0], a.p[1], a.p[2], a.p[3], a.p[4], (const float*)a.p[5], a.T, a.H, a.W,
                                     a.heads, a.d, a.eps, a.p[6], nullptr, (float*)a.p[7], (float*)a.p[8], a.F,
                                     a.t_offset, a.dtype);
}
int bc_b(const Args& a) {
  return gla_block_causal_forward_batch(a.p[0], a.p[1], a.p[2], a.p[3], a.p[4], (const float*)a.p[5], a.batch, a.T,
                                        a.H, a.W, a.heads, a.d, a.eps, a.p[6], nullptr, (float*)a.p[7],
                                        (float*)a.p[8], a.F, a.t_offset, a.dtype);
}
int tc(const Args& a) {
  return gla_token_causal_forward(a.p[0], a.p[1], a.p[2], a.p[3], a.p[4], (const float*)a.p[5], a.T, a.H, a.W,
                                  a.heads, a.d, a.eps, a.p[6], nullptr, (float*)a.p[7], (float*)a.p[8],
                                  a.include_self, a.t_offset, a.dtype);
}
int tc_b(const Args& a) {
  return gla_token_causal_forward_batch(a.p[0], a.p[1], a.p[2], a.p[3], a.p[4], (const float*)a.p[5], a.batch, a.T,
                                        a.H, a.W, a.heads, a.d, a.eps, a.p[6], nullptr, (float*)a.p[7],
                                        (float*)a.p[8], a.include_self, a.t_offset, a.dtype);
}

typedef int (*Entry)(const Args&);
const Entry kAll[] = {fwd, fwd_b, bc, bc_at, bc_b, tc, tc_b};

}  // namespace

int main() {
  for (int i = 0; i < 10; ++i) P[i] = reinterpret_cast<void*>(A + uintptr_t(i) * (uintptr_t(1) << 36));

  for (Entry e : kAll) {
    Args a;
    // dtype and head dim
    for (int dt : {-1, 4, 7}) { a = Args(); a.dtype = dt; EXPECT(e(a), GLA_ERR_DTYPE); }
    for (int d : {0, 16, 48, 96, 256}) { a = Args(); a.d = d; EXPECT(e(a), GLA_ERR_UNSUPPORTED_D); }
    // shapes, eps and size limits
    a = Args(); a.T = -1; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.W = -3; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.heads = 0; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.heads = std::numeric_limits<int>::min(); EXPECT(e(a), GLA_ERR_SHAPE);
    for (float eps : {0.0f, -1e-6f, std::nanf(""), INFINITY, 1e-40f}) { a = Args(); a.eps = eps; EXPECT(e(a), GLA_ERR_SHAPE); }
    a = Args(); a.T = 2000; a.H = 2000; a.W = 2000; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.T = a.H = a.W = std::numeric_limits<int>::max(); EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.T = 1000; a.H = 1000; a.W = 1000; a.heads = 64; a.d = 128; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.T = a.H = a.W = 1; a.heads = 1 << 18; a.d = 128; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.T = a.H = a.W = 1; a.heads = std::numeric_limits<int>::max(); a.d = 128; EXPECT(e(a), GLA_ERR_SHAPE);
    // null, alignment, aliasing
    for (int i = 0; i < 7; ++i) { a = Args(); a.p[i] = nullptr; EXPECT(e(a), GLA_ERR_NULL); }
    for (int i = 0; i < 7; ++i) { a = Args(); a.p[i] = static_cast<char*>(P[i]) + 8; EXPECT(e(a), GLA_ERR_ALIGN); }
    for (int i = 0; i < 6; ++i) { a = Args(); a.p[6] = a.p[i]; EXPECT(e(a), GLA_ERR_ALIAS); }
    // empty grid: nothing to do, pointers may be null
    a = Args(); a.T = 0; for (auto& p : a.p) p = nullptr; EXPECT(e(a), GLA_OK);
  }
  for (Entry e : {bc, bc_at, bc_b, tc, tc_b}) {
    Args a;
    for (int i : {7, 8}) { a = Args(); a.p[i] = nullptr; EXPECT(e(a), GLA_ERR_NULL); }
    a = Args(); a.p[7] = a.p[6]; EXPECT(e(a), GLA_ERR_ALIAS);
    a = Args(); a.p[8] = static_cast<char*>(P[7]) + 16; EXPECT(e(a), GLA_ERR_ALIAS);
  }
  for (Entry e : {bc, bc_at, bc_b}) {
    Args a;
    a = Args(); a.F = 0; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.F = std::numeric_limits<int>::min(); EXPECT(e(a), GLA_ERR_SHAPE);
  }
  for (Entry e : {bc_at, bc_b}) {
    Args a;
    a = Args(); a.F = 3; a.t_offset = 4; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.F = 2; a.t_offset = -2; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.t_offset = std::numeric_limits<int>::max() - 1; a.T = 5; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.t_offset = std::numeric_limits<int>::max(); EXPECT(e(a), GLA_ERR_SHAPE);
  }
  for (Entry e : {tc, tc_b}) {
    Args a;
    a = Args(); a.include_self = 2; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.include_self = -1; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.t_offset = -1; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.t_offset = std::numeric_limits<int>::max(); a.T = 5; EXPECT(e(a), GLA_ERR_SHAPE);
  }
  for (Entry e : {fwd_b, bc_b, tc_b}) {
    Args a;
    a = Args(); a.batch = 0; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.batch = std::numeric_limits<int>::min(); EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.batch = 1 << 20; a.T = 1 << 11; a.H = a.W = 1; EXPECT(e(a), GLA_ERR_SHAPE);
    a = Args(); a.batch = std::numeric_limits<int>::max(); a.T = std::numeric_limits<int>::max(); EXPECT(e(a), GLA_ERR_SHAPE);
  }

  // status strings, version, timing and plan knobs
  for (int st = -20; st <= 5; ++st)
    if (gla_status_string(st) == nullptr) { std::printf("FAIL: null status string %d\n", st); ++failures; }
  EXPECT(gla_version() >> 16, 1);
  for (int id = -3; id < 8; ++id)
    if (gla_kernel_name(id) == nullptr) { std::printf("FAIL: null kernel name %d\n", id); ++failures; }
  double ms[GLA_NUM_KERNELS + 2];
  long long n[GLA_NUM_KERNELS + 2];
  EXPECT(gla_timing_read(ms, n, GLA_NUM_KERNELS + 2), GLA_OK);
  EXPECT(gla_timing_read(nullptr, nullptr, 0), GLA_OK);
  EXPECT(gla_plan_override(-1, 1), GLA_ERR_SHAPE);
  EXPECT(gla_plan_override(GLA_PLAN_NUM_KNOBS, 1), GLA_ERR_SHAPE);
  EXPECT(gla_plan_override(0, -1), GLA_ERR_SHAPE);
  for (int k = 0; k < GLA_PLAN_NUM_KNOBS; ++k) EXPECT(gla_plan_override(k, 7), GLA_OK);
  for (int k = 0; k < GLA_PLAN_NUM_KNOBS; ++k) EXPECT(gla_plan_override(k, 0), GLA_OK);

  // a fixed scratch buffer too small for the call: rejected before any device work
  {
    const gla::FixedScratch tiny{[](int) -> void* { return nullptr; }, 1024};
    Args a;
    EXPECT(gla::forward_fixed_scratch(a.p[0], a.p[1], a.p[2], a.p[3], a.p[4], (const float*)a.p[5], a.T, a.H, a.W,
                                      a.heads, a.d, a.eps, a.p[6], nullptr, a.dtype, tiny),
           GLA_ERR_TOO_LARGE);
    a.dtype = 9;
    EXPECT(gla::forward_fixed_scratch(a.p[0], a.p[1], a.p[2], a.p[3], a.p[4], (const float*)a.p[5], a.T, a.H, a.W,
                                      a.heads, a.d, a.eps, a.p[6], nullptr, a.dtype, tiny),
           GLA_ERR_DTYPE);
  }

  // a valid call with no device: GLA_ERR_HIP, nothing launched
  int count = 0;
  const bool device = hipGetDeviceCount(&count) == hipSuccess && count > 0;
  if (!device) {
    for (Entry e : kAll) {
      Args a;
      a.batch = 2;
      EXPECT(e(a), GLA_ERR_HIP);
    }
  } else {
    std::printf("note: a device is visible; the no-device calls were skipped\n");
  }

  std::printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
