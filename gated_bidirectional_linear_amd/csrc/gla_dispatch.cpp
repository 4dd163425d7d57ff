// Launch sequence of one operator call: RoPE table (only when pass 1 cannot
// hold a chunk's RoPE rows in LDS; otherwise pass 1 computes the table), state
// partials, reduce/prefix, fused output (or the token-causal walk), each
// bracketed by the optional timer.
#include "gla_launch.h"

namespace gla {

typedef unsigned short bf16_t;
typedef unsigned char fp8_t;
enum class bf8_t : unsigned char {};

template <int D> hipError_t launch_rope_table(const LaunchArgs& a);
template <int D> hipError_t launch_state_reduce(const LaunchArgs& a);
template <int D, typename E> hipError_t launch_state_partial(const LaunchArgs& a);
template <int D, typename E> hipError_t launch_output(const LaunchArgs& a);
template <int D, typename E> hipError_t launch_token_causal(const LaunchArgs& a);

template <int D, typename E>
static hipError_t launch_all(const LaunchArgs& a, Timer& tm) {
  hipError_t e;
  if (!a.geo.rope_lds1) {   // otherwise pass 1 computes the RoPE table
    tm.begin(0, a.stream);
    e = launch_rope_table<D>(a);
    tm.end(0, a.stream);
    if (e != hipSuccess) return e;
  }
  tm.begin(1, a.stream);
  e = launch_state_partial<D, E>(a);
  tm.end(1, a.stream);
  if (e != hipSuccess) return e;
  tm.begin(2, a.stream);
  e = launch_state_reduce<D>(a);
  tm.end(2, a.stream);
  if (e != hipSuccess) return e;
  tm.begin(3, a.stream);
  e = a.geo.token_causal ? launch_token_causal<D, E>(a) : launch_output<D, E>(a);
  tm.end(3, a.stream);
  return e;
}

hipError_t launch_operator(const LaunchArgs& a, Timer& tm) {
  // dtype codes of include/gla.h: 0 fp32, 1 bf16, 2 fp8 e4m3, 3 fp8 e5m2
  if (a.dtype == 1) {
    switch (a.geo.d) {
      case 32: return launch_all<32, bf16_t>(a, tm);
      case 64: return launch_all<64, bf16_t>(a, tm);
      case 128: return launch_all<128, bf16_t>(a, tm);
    }
  } else if (a.dtype == 2) {
    switch (a.geo.d) {
      case 32: return launch_all<32, fp8_t>(a, tm);
      case 64: return launch_all<64, fp8_t>(a, tm);
      case 128: return launch_all<128, fp8_t>(a, tm);
    }
  } else if (a.dtype == 3) {
    switch (a.geo.d) {
      case 32: return launch_all<32, bf8_t>(a, tm);
      case 64: return launch_all<64, bf8_t>(a, tm);
      case 128: return launch_all<128, bf8_t>(a, tm);
    }
  } else if (a.dtype == 0) {
    switch (a.geo.d) {
      case 32: return launch_all<32, float>(a, tm);
      case 64: return launch_all<64, float>(a, tm);
      case 128: return launch_all<128, float>(a, tm);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace gla
