// Device code shared by the operator's kernels: chunk geometry, batched row
// loads and the RoPE table view.
#pragma once
#include "gla_device.h"
#include "gla_launch.h"

namespace gla {

// ===========================================================================
// Chunk geometry shared by the kernels (all integer arithmetic, no tables)
// ===========================================================================
struct Chunk {
  long begin, end;  // token range [begin, end)
  int head, seg, index;
};

// Chunk-major order: consecutive workgroup ids take the same chunk of
// consecutive heads, so (after the XCD swizzle) all heads of a token range run
// on one XCD at the same time: their rows share DRAM pages and the beta rows
// (one cache line holds every head of a token) are fetched into one L2.
// Token range [s0, s1) of segment `seg`: within its batch item, whose last
// segment may be shorter.
__device__ __forceinline__ void seg_bounds(const Geometry& G, int seg, long& s0, long& s1) {
  const int item = seg / G.segs_item;
  const long base = (long)item * G.n_item;
  s0 = base + (long)(seg - item * G.segs_item) * G.seg_len;
  s1 = min(s0 + (long)G.seg_len, base + (long)G.n_item);
}

__device__ __forceinline__ Chunk chunk_of(int lin, const Geometry& G, int cps, int chunk_len) {
  Chunk c;
  const int ci = lin / G.heads;          // chunk index within a head, over all segments
  c.head = lin - ci * G.heads;
  c.seg = ci / cps;
  c.index = ci;
  const int j = ci - c.seg * cps;
  long s0, s1;
  seg_bounds(G, c.seg, s0, s1);
  c.begin = min(s0 + (long)j * chunk_len, s1);
  c.end = min(c.begin + (long)chunk_len, s1);
  return c;
}

// Issue the loads of 8 channels of TPT consecutive tokens of one head.  Rows
// at or past `end` are clamped to the last valid row (end > n0 is guaranteed
// by the callers) so every load is unconditional and all of them are in
// flight together; the clamped rows are zeroed when unpacked.
template <int D, typename E, int TPT>
__device__ __forceinline__ void issue_rows(const E* __restrict__ base, long n0, long end, int heads, int head,
                                           int cg, typename Elem<E>::Raw (&r)[TPT]) {
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const long n = min(n0 + i, end - 1);
    r[i] = Elem<E>::load_raw(base + ((size_t)n * heads + head) * D + 8 * cg);
  }
}

template <typename E, int TPT>
__device__ __forceinline__ void unpack_rows(const typename Elem<E>::Raw (&r)[TPT], long n0, long end,
                                            float (&x)[TPT][8]) {
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    Elem<E>::unpack(r[i], x[i]);
    if (n0 + i >= end) {
#pragma unroll
      for (int c = 0; c < 8; ++c) x[i][c] = 0.f;
    }
  }
}

// Write TPT consecutive-token values of one channel into a transposed LDS row.
template <typename E, int TPT>
__device__ __forceinline__ void store_tcol(E* dst, const float (&x)[TPT][8], int c) {
  if constexpr (Elem<E>::is_bf16) {
    if constexpr (TPT == 4) {
      uint2 u;
      u.x = pack2bf(x[0][c], x[1][c]);
      u.y = pack2bf(x[2][c], x[3][c]);
      *reinterpret_cast<uint2*>(dst) = u;
    } else if constexpr (TPT == 2) {
      *reinterpret_cast<uint32_t*>(dst) = pack2bf(x[0][c], x[1][c]);
    } else {
      *dst = f2bf(x[0][c]);
    }
  } else {
    if constexpr (TPT == 4) {
      *reinterpret_cast<float4*>(dst) = make_float4(x[0][c], x[1][c], x[2][c], x[3][c]);
    } else if constexpr (TPT == 2) {
      *reinterpret_cast<float2*>(dst) = make_float2(x[0][c], x[1][c]);
    } else {
      *dst = x[0][c];
    }
  }
}

// Stage the RoPE rows of the frames a chunk spans (or use the global table).
template <int D, bool LDSR, int kMaxEntries = kRopeLdsEntries>
__device__ __forceinline__ typename Rope<D>::View rope_view(float2* lds, const float2* __restrict__ rope,
                                                            const Geometry& G, long begin, long end) {
  if constexpr (LDSR) {
    const int HW = G.H * G.W;
    const int t_lo = begin < end ? (int)(begin / HW) : 0;
    const int nt = begin < end ? (int)((end - 1) / HW) - t_lo + 1 : 0;
    return Rope<D>::template stage<kMaxEntries>(lds, rope, G.T, G.H, G.W, t_lo, nt);
  } else {
    return typename Rope<D>::View{rope, 0, G.T, G.H};
  }
}

}  // namespace gla
