// Device helpers for the gfx950 kernels: element loads/stores, bf16 packing,
// 64-wide wavefront DPP reductions, MFMA wrappers and the RoPE table lookup.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short bf16_t;  // bf16 storage

constexpr int kTile = 64;       // tokens per staged tile
constexpr int kThreads = 256;   // 4 waves of 64

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint16_t f2bf(float f) {   // round to nearest even
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// ---------------------------------------------------------------------------
// 8 consecutive channels of one token: load as fp32, store from fp32
// ---------------------------------------------------------------------------
template <typename E> struct Elem;

template <> struct Elem<float> {
  static constexpr bool is_bf16 = false;
  __device__ __forceinline__ static void load8(const float* p, float (&x)[8]) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ __forceinline__ static void store8(float* p, const float (&x)[8]) {
    const f32x4 a = {x[0], x[1], x[2], x[3]};
    const f32x4 b = {x[4], x[5], x[6], x[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p) + 1);
  }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
};

template <> struct Elem<bf16_t> {
  static constexpr bool is_bf16 = true;
  __device__ __forceinline__ static void load8(const bf16_t* p, float (&x)[8]) {
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    x[0] = bf16lo(u.x); x[1] = bf16hi(u.x); x[2] = bf16lo(u.y); x[3] = bf16hi(u.y);
    x[4] = bf16lo(u.z); x[5] = bf16hi(u.z); x[6] = bf16lo(u.w); x[7] = bf16hi(u.w);
  }
  __device__ __forceinline__ static void store8(bf16_t* p, const float (&x)[8]) {
    const u32x4 u = {pack2bf(x[0], x[1]), pack2bf(x[2], x[3]), pack2bf(x[4], x[5]), pack2bf(x[6], x[7])};
    __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(p));
  }
  __device__ __forceinline__ static float load1(const bf16_t* p) {
    return __uint_as_float(((uint32_t)*p) << 16);
  }
};

// ---------------------------------------------------------------------------
// Sum over groups of L consecutive lanes (L = 4, 8 or 16), result in every lane
// of the group.  quad_perm xor-1 / xor-2, then row_half_mirror (8) and
// row_mirror (16): after each step every lane of the group-so-far holds the
// same partial, so a mirror adds exactly the other half.
// ---------------------------------------------------------------------------
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(L == 4 || L == 8 || L == 16, "group size");
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  if constexpr (L >= 8)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  if constexpr (L >= 16)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// ---------------------------------------------------------------------------
// MFMA 32x32 with fp32 accumulation.  Operand fragments per lane l:
//   A[m = l%32][k = KPL*(l/32) + j],  B[k = KPL*(l/32) + j][n = l%32]
//   C[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32],  r = 0..15
// bf16: KPL = 8, one instruction covers K = 16.  fp32: KPL = 1, K = 2.
// ---------------------------------------------------------------------------
template <typename E> struct Mfma;

template <> struct Mfma<bf16_t> {
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 16;
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // 8 consecutive bf16 from LDS (16-byte aligned)
  __device__ __forceinline__ static frag lds_frag(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
  }
  __device__ __forceinline__ static frag from_f32(const float* x) {  // 8 values
    uint4 u;
    u.x = pack2bf(x[0], x[1]); u.y = pack2bf(x[2], x[3]);
    u.z = pack2bf(x[4], x[5]); u.w = pack2bf(x[6], x[7]);
    return __builtin_bit_cast(bf16x8, u);
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 2;
  typedef float frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag lds_frag(const float* p) { return *p; }
  __device__ __forceinline__ static frag from_f32(const float* x) { return x[0]; }
};

// ---------------------------------------------------------------------------
// 3D RoPE table: float2 (cos, sin) entries, three per-axis blocks
//   [T][d/8], then [H][3d/16], then [W][3d/16].
// Pair p (channels 2p, 2p+1) of the head dim belongs to axis t for p < d/8,
// y for p < d/8 + 3d/16, x otherwise.
// ---------------------------------------------------------------------------
template <int D>
struct Rope {
  static constexpr int PT = D / 8;        // pairs on the t axis
  static constexpr int PY = 3 * D / 16;   // pairs on the y axis
  static constexpr int PX = 3 * D / 16;   // pairs on the x axis
  // rotate the 4 pairs held by a thread (channels 8cg..8cg+7) of token (t,y,x)
  __device__ __forceinline__ static void rotate(float (&x)[8], int cg, int t, int y, int xx,
                                                const float2* __restrict__ tab, int T, int H) {
    const float2* tab_t = tab;
    const float2* tab_y = tab + (size_t)T * PT;
    const float2* tab_x = tab_y + (size_t)H * PY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = 4 * cg + j;
      const float2* e;
      if (p < PT) e = tab_t + t * PT + p;
      else if (p < PT + PY) e = tab_y + y * PY + (p - PT);
      else e = tab_x + xx * PX + (p - PT - PY);
      const float2 cs = *e;
      const float u = x[2 * j], w = x[2 * j + 1];
      x[2 * j] = u * cs.x - w * cs.y;
      x[2 * j + 1] = u * cs.y + w * cs.x;
    }
  }
};

// Map a linear workgroup id so that ids dispatched to the same XCD (ids are
// dealt round-robin over the 8 XCDs) get consecutive logical ids, i.e. the
// same head and neighbouring chunks share an L2.
__device__ __forceinline__ int xcd_swizzle(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int per = nblocks / kXcd;
  const int rem = nblocks % kXcd;
  const int xcd = bid % kXcd;
  const int local = bid / kXcd;
  // xcds [0, rem) hold per+1 blocks, the rest hold per
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + local;
}

}  // namespace gla
