// RoPE table generation and the fixed-order reduction / block prefix of the
// per-chunk state partials.
#include "gla_common.h"

namespace gla {

// ===========================================================================
// 1. RoPE tables
// ===========================================================================
template <int D>
// Frame row t (of all T frames of the batch) holds item frame t % T_item, at
// absolute frame t_offset + t % T_item (streaming across calls); rows and
// columns always start at 0.  The pass-1 kernels compute the same entries
// (Rope::compute) when their rows fit in LDS; this kernel runs only when they
// do not.
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ tab, int T, int H, int W, int t_offset,
                                                         int T_item) {
  using R = Rope<D>;
  const long total = (long)T * R::PT + (long)H * R::PY + (long)W * R::PX;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  long pos;
  int p;   // pair of the head dim
  if (idx < (long)T * R::PT) {
    pos = (idx / R::PT) % T_item + t_offset; p = (int)(idx % R::PT);
  } else if (idx < (long)T * R::PT + (long)H * R::PY) {
    const long r = idx - (long)T * R::PT;
    pos = r / R::PY; p = R::PT + (int)(r % R::PY);
  } else {
    const long r = idx - (long)T * R::PT - (long)H * R::PY;
    pos = r / R::PX; p = R::PT + R::PY + (int)(r % R::PX);
  }
  tab[idx] = R::cos_sin((double)pos * R::freq_of(p));
}

// ===========================================================================
// 3. Reduce chunk partials per segment (pairwise tree of fixed shape), then
//    prefix over the segments of a batch item on top of its carried state:
//    inclusive of the segment (bidirectional and block-causal forms) or
//    exclusive (the token-causal form, whose segments are walked token by
//    token).  One thread per (state element, head, item).  When sbf is given,
//    each segment's S is also written rounded to bf16 (the operand the
//    four-head output kernel loads as MFMA fragments).  P: the chunk count
//    rounded up to a power of two (1: one partial per segment), so that the
//    tree's loads and adds are unrolled for exactly the levels in use.
// ===========================================================================
template <int D, int P>
__global__ __launch_bounds__(256) void state_reduce_kernel(const float* __restrict__ partial,
                                                           const float* S_in, const float* z_in,
                                                           float* __restrict__ states, float* S_out,
                                                           float* z_out, bf16_t* __restrict__ sbf, Geometry G) {
  constexpr int SZ = D * D + D;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;   // batch item
  if (e >= SZ) return;
  const size_t hb = (size_t)b * G.heads + h;   // (item, head) of the carried state
  float running = 0.f;
  if (S_in != nullptr) running = (e < D * D) ? S_in[hb * D * D + e] : z_in[hb * D + (e - D * D)];
  const int sfirst = b * G.segs_item;   // this item's first segment
  const float* src = partial + ((size_t)h * G.nseg + sfirst) * G.cps1 * SZ + e;
  if constexpr (P == 1) {
    // one partial per segment: the tree is the partial itself; the loads of
    // 8 segments are issued together
    constexpr int kBatch = 8;
    for (int s0 = 0; s0 < G.segs_item; s0 += kBatch) {
      float x[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) x[i] = (s0 + i < G.segs_item) ? src[(size_t)(s0 + i) * SZ] : 0.f;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (s0 + i >= G.segs_item) break;
        const float before = running;
        running += x[i];
        const float sv = G.states_exclusive ? before : running;
        states[((size_t)(sfirst + s0 + i) * G.heads + h) * SZ + e] = sv;
        if (sbf != nullptr && e < D * D) sbf[((size_t)(sfirst + s0 + i) * G.heads + h) * (D * D) + e] = f2bf(sv);
      }
    }
  } else {
    // levels of the 64-leaf tree at or above the chunk count add only zeros
    // (exactly), so they are skipped: the same sums in the same order
    static_assert(P <= kMaxChunks, "tree size");
    for (int s = 0; s < G.segs_item; ++s) {
      float v[P];
#pragma unroll
      for (int i = 0; i < P; ++i) v[i] = (i < G.cps1) ? src[(size_t)(s * G.cps1 + i) * SZ] : 0.f;
#pragma unroll
      for (int w = P / 2; w >= 1; w >>= 1) {
#pragma unroll
        for (int i = 0; i < w; ++i) v[i] += v[i + w];
      }
      const float before = running;
      running += v[0];
      const float sv = G.states_exclusive ? before : running;
      states[((size_t)(sfirst + s) * G.heads + h) * SZ + e] = sv;
      if (sbf != nullptr && e < D * D) sbf[((size_t)(sfirst + s) * G.heads + h) * (D * D) + e] = f2bf(sv);
    }
  }
  if (S_out != nullptr) {
    if (e < D * D) S_out[hb * D * D + e] = running;
    else z_out[hb * D + (e - D * D)] = running;
  }
}

template <int D>
hipError_t launch_rope_table(const LaunchArgs& a) {
  const Geometry& G = a.geo;
  const long total = (long)G.T * (D / 8) + (long)G.H * (3 * D / 16) + (long)G.W * (3 * D / 16);
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL((rope_table_kernel<D>), dim3(blocks), dim3(256), 0, a.stream, a.rope, G.T, G.H, G.W, G.t_offset,
                     G.T_item);
  return hipGetLastError();
}

template <int D, int P>
static void launch_reduce_p(const LaunchArgs& a) {
  const Geometry& G = a.geo;
  constexpr int SZ = D * D + D;
  dim3 grid((SZ + 255) / 256, G.heads, G.batch);
  hipLaunchKernelGGL((state_reduce_kernel<D, P>), grid, dim3(256), 0, a.stream, (const float*)a.partial, a.S_in,
                     a.z_in, a.states, a.S_out, a.z_out, (bf16_t*)a.states_bf16, G);
}

template <int D>
hipError_t launch_state_reduce(const LaunchArgs& a) {
  const int c = a.geo.cps1;   // 1 .. kMaxChunks (the planner's bound)
  if (c <= 1) launch_reduce_p<D, 1>(a);
  else if (c <= 2) launch_reduce_p<D, 2>(a);
  else if (c <= 4) launch_reduce_p<D, 4>(a);
  else if (c <= 8) launch_reduce_p<D, 8>(a);
  else if (c <= 16) launch_reduce_p<D, 16>(a);
  else if (c <= 32) launch_reduce_p<D, 32>(a);
  else if (c <= kMaxChunks) launch_reduce_p<D, kMaxChunks>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template hipError_t launch_rope_table<32>(const LaunchArgs&);
template hipError_t launch_rope_table<64>(const LaunchArgs&);
template hipError_t launch_rope_table<128>(const LaunchArgs&);
template hipError_t launch_state_reduce<32>(const LaunchArgs&);
template hipError_t launch_state_reduce<64>(const LaunchArgs&);
template hipError_t launch_state_reduce<128>(const LaunchArgs&);

}  // namespace gla
