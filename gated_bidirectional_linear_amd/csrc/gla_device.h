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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short bf16_t;  // bf16 storage
typedef unsigned char fp8_t;    // OCP FP8 E4M3 (e4m3fn) storage
enum class bf8_t : unsigned char {};   // OCP FP8 E5M2 storage (a distinct one-byte type)

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
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {   // one v_cvt_pk_bf16_f32
  typedef float f2v __attribute__((ext_vector_type(2)));
  typedef __bf16 b2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, b2v));
}

// ---------------------------------------------------------------------------
// 8 consecutive channels of one token: load as fp32, store from fp32
// ---------------------------------------------------------------------------
template <typename E> struct Elem;

template <> struct Elem<float> {
  static constexpr bool is_bf16 = false;
  static constexpr bool is_f8 = false;
  typedef float Lds;   // LDS staging / MFMA operand type
  struct Raw { f32x4 a, b; };  // 8 channels as loaded
  __device__ __forceinline__ static Raw load_raw(const float* p) {
    Raw r;
    r.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    r.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
    return r;
  }
  __device__ __forceinline__ static void unpack(const Raw& r, float (&x)[8]) {
    x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w; x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
  }
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
  __device__ __forceinline__ static Raw pack(const float (&x)[8]) {
    Raw r;
    r.a = (f32x4){x[0], x[1], x[2], x[3]};
    r.b = (f32x4){x[4], x[5], x[6], x[7]};
    return r;
  }
  __device__ __forceinline__ static void store_raw(float* p, const Raw& r) {
    __builtin_nontemporal_store(r.a, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(r.b, reinterpret_cast<f32x4*>(p) + 1);
  }
};

template <> struct Elem<bf16_t> {
  static constexpr bool is_bf16 = true;
  static constexpr bool is_f8 = false;
  typedef bf16_t Lds;
  typedef u32x4 Raw;  // 8 channels as loaded
  __device__ __forceinline__ static Raw load_raw(const bf16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ static void unpack(const Raw& u, float (&x)[8]) {
    x[0] = bf16lo(u.x); x[1] = bf16hi(u.x); x[2] = bf16lo(u.y); x[3] = bf16hi(u.y);
    x[4] = bf16lo(u.z); x[5] = bf16hi(u.z); x[6] = bf16lo(u.w); x[7] = bf16hi(u.w);
  }
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
  __device__ __forceinline__ static Raw pack(const float (&x)[8]) {
    return (u32x4){pack2bf(x[0], x[1]), pack2bf(x[2], x[3]), pack2bf(x[4], x[5]), pack2bf(x[6], x[7])};
  }
  __device__ __forceinline__ static void store_raw(bf16_t* p, const Raw& r) {
    __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(p));
  }
};

// FP8 E4M3 (OCP e4m3fn: bias 7, no infinities, max 448).  gfx950's
// v_cvt_pk_f32_fp8 / v_cvt_pk_fp8_f32 convert this format exactly and round
// to nearest even (values at or past 480 become NaN; the operator's inputs and
// outputs stay far below that).  Every e4m3 value is exact in bf16, so the
// kernels stage fp8 operands as bf16 for the MFMA.
template <> struct Elem<fp8_t> {
  static constexpr bool is_bf16 = false;
  static constexpr bool is_f8 = true;
  typedef bf16_t Lds;
  typedef u32x2 Raw;  // 8 channels as loaded
  __device__ __forceinline__ static Raw load_raw(const fp8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  }
  __device__ __forceinline__ static void unpack(const Raw& u, float (&x)[8]) {
    typedef float f2v __attribute__((ext_vector_type(2)));
    const f2v a = __builtin_amdgcn_cvt_pk_f32_fp8((int)u.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)u.x, true);
    const f2v c = __builtin_amdgcn_cvt_pk_f32_fp8((int)u.y, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)u.y, true);
    x[0] = a.x; x[1] = a.y; x[2] = b.x; x[3] = b.y; x[4] = c.x; x[5] = c.y; x[6] = d.x; x[7] = d.y;
  }
  __device__ __forceinline__ static void load8(const fp8_t* p, float (&x)[8]) { unpack(load_raw(p), x); }
  __device__ __forceinline__ static Raw pack(const float (&x)[8]) {
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], w1, true);
    return (u32x2){(uint32_t)w0, (uint32_t)w1};
  }
  __device__ __forceinline__ static void store8(fp8_t* p, const float (&x)[8]) {
    __builtin_nontemporal_store(pack(x), reinterpret_cast<u32x2*>(p));
  }
  __device__ __forceinline__ static void store_raw(fp8_t* p, const Raw& r) {
    __builtin_nontemporal_store(r, reinterpret_cast<u32x2*>(p));
  }
  __device__ __forceinline__ static float load1(const fp8_t* p) { return __builtin_amdgcn_cvt_f32_fp8((int)*p, 0); }
  // bytes 2 SEL .. 2 SEL + 1 of w as a bf16 pair (v_cvt_scalef32_pk_bf16_fp8 with scale 1: exact)
  template <bool SEL>
  __device__ __forceinline__ static uint32_t bf16_pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, SEL));
  }
  __device__ __forceinline__ static float code_to_f32(int code) { return __builtin_amdgcn_cvt_f32_fp8(code, 0); }
};

// FP8 E5M2 (OCP: bias 15, max 57344, with infinities and NaN).  gfx950's
// v_cvt_pk_f32_bf8 / v_cvt_pk_bf8_f32 convert it, rounding to nearest even;
// every e5m2 value is exact in bf16 (and in fp32), so the kernels treat it as
// the e4m3 rows above with the other conversion instructions.
template <> struct Elem<bf8_t> {
  static constexpr bool is_bf16 = false;
  static constexpr bool is_f8 = true;
  typedef bf16_t Lds;
  typedef u32x2 Raw;  // 8 channels as loaded
  __device__ __forceinline__ static Raw load_raw(const bf8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  }
  __device__ __forceinline__ static void unpack(const Raw& u, float (&x)[8]) {
    typedef float f2v __attribute__((ext_vector_type(2)));
    const f2v a = __builtin_amdgcn_cvt_pk_f32_bf8((int)u.x, false), b = __builtin_amdgcn_cvt_pk_f32_bf8((int)u.x, true);
    const f2v c = __builtin_amdgcn_cvt_pk_f32_bf8((int)u.y, false), d = __builtin_amdgcn_cvt_pk_f32_bf8((int)u.y, true);
    x[0] = a.x; x[1] = a.y; x[2] = b.x; x[3] = b.y; x[4] = c.x; x[5] = c.y; x[6] = d.x; x[7] = d.y;
  }
  __device__ __forceinline__ static void load8(const bf8_t* p, float (&x)[8]) { unpack(load_raw(p), x); }
  __device__ __forceinline__ static Raw pack(const float (&x)[8]) {
    int w0 = __builtin_amdgcn_cvt_pk_bf8_f32(x[0], x[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_bf8_f32(x[2], x[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_bf8_f32(x[4], x[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_bf8_f32(x[6], x[7], w1, true);
    return (u32x2){(uint32_t)w0, (uint32_t)w1};
  }
  __device__ __forceinline__ static void store8(bf8_t* p, const float (&x)[8]) {
    __builtin_nontemporal_store(pack(x), reinterpret_cast<u32x2*>(p));
  }
  __device__ __forceinline__ static void store_raw(bf8_t* p, const Raw& r) {
    __builtin_nontemporal_store(r, reinterpret_cast<u32x2*>(p));
  }
  __device__ __forceinline__ static float load1(const bf8_t* p) {
    return __builtin_amdgcn_cvt_f32_bf8((int)static_cast<unsigned char>(*p), 0);
  }
  template <bool SEL>
  __device__ __forceinline__ static uint32_t bf16_pair(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w, 1.0f, SEL));
  }
  __device__ __forceinline__ static float code_to_f32(int code) { return __builtin_amdgcn_cvt_f32_bf8(code, 0); }
};

// ---------------------------------------------------------------------------
// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes every wave wait for its outstanding global loads (the
// prefetched next tile) at each barrier.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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

// x[l] + x[l ^ 16]: v_permlane16_swap hands each lane both rows of its pair
__device__ __forceinline__ float pair_rows_sum(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
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
  // Every thread holds channels 8cg..8cg+7 = pairs 4cg..4cg+3.  When the axis
  // boundaries are multiples of 4 pairs (d = 64, 128) those 4 pairs share an
  // axis and sit next to each other in its table: two 16-byte reads.
  static constexpr bool kGrouped = (PT % 4 == 0) && (PY % 4 == 0);

  // A view of the table: frames [t_lo, t_lo + nt) of the t block, then the
  // whole y block [H][PY] and x block [W][PX].  The global table is the view
  // with t_lo = 0, nt = T; the LDS copy holds only the frames a chunk spans.
  struct View {
    const float2* tab;
    int t_lo, nt, H;
    // float2 offset of pair p of a token at (t, y, x)
    __device__ __forceinline__ int offset(int p, int t, int y, int x) const {
      const int axis = (p < PT) ? 0 : ((p < PT + PY) ? 1 : 2);
      const int pos = axis == 0 ? (t - t_lo) : (axis == 1 ? y : x);
      const int base = axis == 0 ? p : (axis == 1 ? nt * PT + (p - PT) : nt * PT + H * PY + (p - PT - PY));
      const int stride = axis == 0 ? PT : (axis == 1 ? PY : PX);
      return base + pos * stride;
    }
  };

  struct CS { float c[4], s[4]; };

  __device__ __forceinline__ static CS fetch(const View& v, int cg, int t, int y, int x) {
    CS r;
    if constexpr (kGrouped) {
      const f32x4* e = reinterpret_cast<const f32x4*>(v.tab + v.offset(4 * cg, t, y, x));
      const f32x4 a = e[0], b = e[1];
      r.c[0] = a.x; r.s[0] = a.y; r.c[1] = a.z; r.s[1] = a.w;
      r.c[2] = b.x; r.s[2] = b.y; r.c[3] = b.z; r.s[3] = b.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float2 cs = v.tab[v.offset(4 * cg + j, t, y, x)];
        r.c[j] = cs.x;
        r.s[j] = cs.y;
      }
    }
    return r;
  }

  // (u, w) -> (u cos - w sin, u sin + w cos) on each of the 4 pairs
  __device__ __forceinline__ static void apply(float (&x)[8], const CS& cs) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float u = x[2 * j], w = x[2 * j + 1];
      x[2 * j] = u * cs.c[j] - w * cs.s[j];
      x[2 * j + 1] = u * cs.s[j] + w * cs.c[j];
    }
  }

  // Frequency of pair p of the head dim: pair i of an axis of width da turns
  // by pos * 10000^(-2i/da).
  __device__ __forceinline__ static double freq_of(int p) {
    const int i = p < PT ? p : (p < PT + PY ? p - PT : p - PT - PY);
    const int da = p < PT ? D / 4 : 3 * D / 8;
    return pow(10000.0, -2.0 * (double)i / (double)da);
  }

  // (cos a, sin a): the angle in fp64, reduced to [-pi, pi] in fp64 (2 pi as
  // a two-term sum), then sine and cosine of the reduced angle in fp32 (the
  // table stores fp32).  Exact to the last bits of fp32 for positions up to
  // 2^31.
  __device__ __forceinline__ static float2 cos_sin(double a) {
    const double k = rint(a * 0.15915494309189535);
    double r = fma(-k, 6.283185307179586, a);
    r = fma(-k, 2.4492935982947064e-16, r);
    float s, c;
    sincosf((float)r, &s, &c);
    return make_float2(c, s);
  }

  // Position and pair of entry e of a table laid out as frames [t_lo, t_lo +
  // nt) ([nt][PT]), then [H][PY], then [W][PX].  Frame row t (of the batch's
  // frame rows) holds item frame t % T_item at absolute frame t_offset + that.
  __device__ __forceinline__ static void entry_pos(int e, int t_lo, int nt, int H, int T_item, int t_offset,
                                                   long& pos, int& p) {
    const int n_t = nt * PT;
    if (e < n_t) {
      pos = (long)((t_lo + e / PT) % T_item) + t_offset;
      p = e % PT;
    } else if (e < n_t + H * PY) {
      const int r = e - n_t;
      pos = r / PY;
      p = PT + r % PY;
    } else {
      const int r = e - n_t - H * PY;
      pos = r / PX;
      p = PT + PY + r % PX;
    }
  }

  // Compute the frames [t_lo, t_lo + nt) and the y/x blocks of the table into
  // LDS as put(index, (cos, sin)), and write them to the global table `tab`
  // ([T][PT], [H][PY], [W][PX]) for the later kernels: the frame rows always
  // (workgroups whose chunks share a frame write the same bits), the y/x blocks
  // when write_yx.  freq: LDS space for D/2 doubles.  All NT threads take
  // part; the caller synchronises before the LDS entries are read.
  template <int kMaxEntries, int NT, typename Put>
  __device__ __forceinline__ static void compute(Put put, double* freq, float2* __restrict__ tab, int T, int H, int W,
                                                 int T_item, int t_offset, int t_lo, int nt, bool write_yx) {
    const int tid = (int)threadIdx.x;
    if (tid < D / 2) freq[tid] = freq_of(tid);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    const int n_t = nt * PT;
    const int total = n_t + H * PY + W * PX;
    for (int e = tid; e < total && e < kMaxEntries; e += NT) {
      long pos;
      int p;
      entry_pos(e, t_lo, nt, H, T_item, t_offset, pos, p);
      const float2 cs = cos_sin((double)pos * freq[p]);
      put(e, cs);
      if (e < n_t) tab[(long)t_lo * PT + e] = cs;
      else if (write_yx) tab[(long)T * PT + (e - n_t)] = cs;
    }
  }

  // Copy the frames [t_lo, t_lo + nt) and the y/x blocks of the global table
  // into LDS (all kThreads threads take part; caller synchronises).  At most
  // kMaxEntries entries, in rounds of 8 per thread: every thread issues a
  // round's loads together (indices past the end are clamped to entry 0 and
  // not stored).
  template <int kMaxEntries>
  __device__ __forceinline__ static View stage(float2* lds, const float2* __restrict__ tab, int T, int H, int W,
                                               int t_lo, int nt) {
    constexpr int PER = 8;
    const int n_t = nt * PT;
    const int total = n_t + H * PY + W * PX;
    const int lim = total < kMaxEntries ? total : kMaxEntries;
    for (int base = 0; base < lim; base += PER * kThreads) {
      float2 tmp[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = base + (int)threadIdx.x + j * kThreads;
        const int src = (i < n_t) ? t_lo * PT + i : T * PT + (i - n_t);
        tmp[j] = tab[i < lim ? src : 0];
      }
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = base + (int)threadIdx.x + j * kThreads;
        if (i < lim) lds[i] = tmp[j];
      }
    }
    return View{lds, t_lo, nt, H};
  }
};

// ---------------------------------------------------------------------------
// Raw buffer access.  A buffer resource (gfx9 descriptor word 3 = 0x00020000,
// stride 0) over `bytes` bytes from `p`: loads past the range return zero and
// stores past it are dropped.  Offsets are a per-lane VGPR plus a
// wave-uniform SGPR, so streaming loops need no per-lane 64-bit addresses.
//
// Token rows are read once and written once, so the row accessors carry
// streaming cache policies (the cache-policy operand: bit 0 sc0, bit 1 nt,
// bit 4 sc1): loads are nontemporal, stores nontemporal at device scope, which
// writes them through the XCD's L2 instead of leaving dirty lines there.  At
// 720p/60s in the full step this measured 722 us against 760 us for the
// paired-head output kernel and 1369 us against 1390 us for the token-causal
// walk; in isolation neither hint helped alone (nt loads only: +0.5%, nt
// stores only: -2%, both: -9%).
// ---------------------------------------------------------------------------
constexpr int kLoadStream = 2;         // nt
constexpr int kStoreStream = 16 | 2;   // sc1 (device scope) | nt
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kLoadStream));
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)voff, (int)soff, kStoreStream);
}
// 8 channels of one row: 16 bytes (bf16) or 32 bytes (fp32)
template <typename E> struct BufRow;
template <> struct BufRow<bf16_t> {
  typedef u32x4 Raw;
  __device__ __forceinline__ static Raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return buf_load16(r, voff, soff);
  }
  __device__ __forceinline__ static void store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, const Raw& v) {
    buf_store16(r, voff, soff, v);
  }
};
template <typename E> struct BufRow8 {   // 8 channels of one-byte elements: 8 bytes
  typedef u32x2 Raw;
  __device__ __forceinline__ static Raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kLoadStream));
  }
  __device__ __forceinline__ static void store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, const Raw& v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)voff, (int)soff, kStoreStream);
  }
};
template <> struct BufRow<bf8_t> : BufRow8<bf8_t> {};
template <> struct BufRow<fp8_t> {
  typedef u32x2 Raw;
  __device__ __forceinline__ static Raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kLoadStream));
  }
  __device__ __forceinline__ static void store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, const Raw& v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)voff, (int)soff, kStoreStream);
  }
};
template <> struct BufRow<float> {
  typedef Elem<float>::Raw Raw;
  __device__ __forceinline__ static Raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    Raw x;
    x.a = __builtin_bit_cast(f32x4, buf_load16(r, voff, soff));
    x.b = __builtin_bit_cast(f32x4, buf_load16(r, voff + 16, soff));
    return x;
  }
  __device__ __forceinline__ static void store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, const Raw& v) {
    buf_store16(r, voff, soff, __builtin_bit_cast(u32x4, v.a));
    buf_store16(r, voff + 16, soff, __builtin_bit_cast(u32x4, v.b));
  }
};

// bf16 helpers working on packed pairs
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
// sum of squares of the two bf16 values in u, added to acc (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2sq(uint32_t u, float acc) {
  const bf16x2 v = __builtin_bit_cast(bf16x2, u);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}
// Gates read as fp8 (e4m3 or e5m2) take sigmoid(g) from a table of all 256
// codes in LDS: one read per element in place of a decode, an exp and a
// reciprocal.  The entries use the per-element formula, so the results are the
// same.
template <typename E>
__device__ __forceinline__ void fill_sigmoid_fp8(float* tab, int tid, int nthreads) {
  for (int i = tid; i < 256; i += nthreads)
    tab[i] = __builtin_amdgcn_rcpf(1.0f + __expf(-Elem<E>::code_to_f32(i)));
}
// sigmoid of code `byte` (0..3) of the packed word w
__device__ __forceinline__ float sigmoid_fp8(const float* tab, uint32_t w, int byte) {
  return tab[(w >> (8 * byte)) & 0xffu];
}

// sum of the two bf16 products a.lo*b.lo + a.hi*b.hi, accumulated in fp32
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}
// ReLU of both bf16 values: the sign bit of bf16 is the int16 sign bit, and
// int16 order matches value order on the non-negative side (v_pk_max_i16)
__device__ __forceinline__ uint32_t relu2(uint32_t u) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, u), (s16x2){0, 0}));
}

// Output RMSNorm scale of x = y / den for a row whose gated numerator y has
// mean square ms and whose denominator is den > 0:
//   x / sqrt(mean(x^2) + eps) = y / sqrt(ms + eps * den^2).
// No 1/den is formed, so a zero row (y = 0, den as small as eps^1.5) cannot
// turn into inf * 0.  The floor at FLT_MIN keeps the reciprocal square root
// finite when ms + eps * den^2 underflows (then y = 0 and the result is 0).
__device__ __forceinline__ float out_scale(float ms, float den, float eps) {
  return __builtin_amdgcn_rsqf(fmaxf(ms + eps * den * den, 1.17549435e-38f));
}

// Position (t, y, x) of a token on the latent grid, advanced without division.
struct GridPos {
  int t, y, x;
  __device__ __forceinline__ void set(int n, int H, int W) {
    const int HW = H * W;
    t = n / HW;
    const int rem = n - t * HW;
    y = rem / W;
    x = rem - y * W;
  }
  // n + (dt*H*W + dy*W + dx) with dx < W, dy < H
  __device__ __forceinline__ void advance(int dt, int dy, int dx, int H, int W) {
    x += dx;
    const bool cy = x >= W;
    x = cy ? x - W : x;
    y += dy + (cy ? 1 : 0);
    const bool ct = y >= H;
    y = ct ? y - H : y;
    t += dt + (ct ? 1 : 0);
  }
  __device__ __forceinline__ void next(int H, int W) {   // n + 1
    ++x;
    const bool cy = x == W;
    x = cy ? 0 : x;
    y += cy ? 1 : 0;
    const bool ct = y == H;
    y = ct ? 0 : y;
    t += ct ? 1 : 0;
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
