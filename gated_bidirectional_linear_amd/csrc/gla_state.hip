// Pass 1: per-chunk partial states S_p = V_p^T (beta R phi K^)_p and key sums.
#include "gla_common.h"

namespace gla {

// ===========================================================================
// 2. State partials: S_p = V_p^T (beta R phi K^)_p and z_p = sum phi K^
// ===========================================================================
// E is the tensor element type; operands are staged in LDS and fed to the
// MFMA as Elem<E>::Lds (fp32 for fp32, bf16 for bf16 and fp8).
template <int D, typename E>
struct PartialCfg {
  typedef typename Elem<E>::Lds L;
  static constexpr int CG = D / 8;                 // threads per token (8 channels each)
  static constexpr int TG = kThreads / CG;         // token groups
  static constexpr int TPT = kTile / TG;           // tokens per thread per tile
  static constexpr int MT = D / 32;                // 32-row MFMA tiles per dim
  static constexpr bool KSPLIT = MT * MT < 4;      // too few output tiles: waves split K
  static constexpr int TPW = KSPLIT ? 1 : MT * MT / 4;   // output tiles per wave
  static constexpr int PITCH = kTile + (Elem<L>::is_bf16 ? 8 : 2);  // LDS row pitch (elements)
  static constexpr int STAGE_BYTES = 2 * D * PITCH * (int)sizeof(L);
  static constexpr int ZRED_BYTES = TG * D * 4;
  static constexpr int KRED_BYTES = KSPLIT ? 4 * 64 * 16 * 4 : 0;
  static constexpr int SMEM = STAGE_BYTES > ZRED_BYTES ? (STAGE_BYTES > KRED_BYTES ? STAGE_BYTES : KRED_BYTES)
                                                       : (ZRED_BYTES > KRED_BYTES ? ZRED_BYTES : KRED_BYTES);
};

// LDSR: the chunk's RoPE rows fit in LDS; the kernel then computes them there
// and writes them to the global table for the later kernels (no table
// kernel runs).  Otherwise it reads the table the table kernel wrote.
template <int D, typename E, bool LDSR>
__global__ __launch_bounds__(kThreads) void state_partial_kernel(
    const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ beta,
    float2* __restrict__ rope, float* __restrict__ partial, Geometry G) {
  using C = PartialCfg<D, E>;
  using L = typename C::L;
  using M = Mfma<L>;
  constexpr int ROPE_BYTES = LDSR ? kRopeLdsEntries * 8 : 0;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM + ROPE_BYTES];
  L* rkT = reinterpret_cast<L*>(smem);          // [D][PITCH]  (k channel, token)
  L* vT = rkT + D * C::PITCH;                   // [D][PITCH]  (v channel, token)

  const int lin = xcd_swizzle(blockIdx.x, gridDim.x);
  const Chunk ch = chunk_of(lin, G, G.cps1, G.chunk1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cg = tid % C::CG;
  const int tg = tid / C::CG;
  const int HW = G.H * G.W;

  float zacc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) zacc[c] = 0.f;
  f32x16 acc[C::TPW];
#pragma unroll
  for (int u = 0; u < C::TPW; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;

  typename Elem<E>::Raw kr[C::TPT], vr[C::TPT];
  E br[C::TPT];   // raw: converted only when the tile is consumed
  auto issue = [&](long t0) {
    const long n0 = t0 + (long)tg * C::TPT;
    issue_rows<D, E, C::TPT>(k, n0, ch.end, G.heads, ch.head, cg, kr);
    issue_rows<D, E, C::TPT>(v, n0, ch.end, G.heads, ch.head, cg, vr);
#pragma unroll
    for (int i = 0; i < C::TPT; ++i)
      br[i] = beta[(size_t)min(n0 + i, ch.end - 1) * G.heads + ch.head];
  };
  if (ch.begin < ch.end) issue(ch.begin);
  typename Rope<D>::View rv;
  if constexpr (LDSR) {
    // the frequency scratch sits in the tile region, unused until the loop
    float2* tab = reinterpret_cast<float2*>(smem + C::SMEM);
    const int t_lo = ch.begin < ch.end ? (int)(ch.begin / HW) : 0;
    const int nt = ch.begin < ch.end ? (int)((ch.end - 1) / HW) - t_lo + 1 : 0;
    Rope<D>::template compute<kRopeLdsEntries, kThreads>([&](int e, float2 cs) { tab[e] = cs; },
                                                         reinterpret_cast<double*>(smem), rope, G.T, G.H, G.W,
                                                         G.T_item, G.t_offset, t_lo, nt, lin == 0);
    rv = typename Rope<D>::View{tab, t_lo, nt, G.H};
    lds_barrier();
  } else {
    rv = typename Rope<D>::View{rope, 0, G.T, G.H};
  }

  for (long t0 = ch.begin; t0 < ch.end; t0 += kTile) {
    const long n0 = t0 + (long)tg * C::TPT;
    float kx[C::TPT][8], vx[C::TPT][8];
    float bt[C::TPT];
    unpack_rows<E, C::TPT>(kr, n0, ch.end, kx);
    unpack_rows<E, C::TPT>(vr, n0, ch.end, vx);
#pragma unroll
    for (int i = 0; i < C::TPT; ++i) bt[i] = (n0 + i < ch.end) ? Elem<E>::load1(&br[i]) : 0.f;
    // RoPE entries of this tile are requested before the next tile's rows so
    // that waiting for them (in-order counter) does not wait for the prefetch.
    typename Rope<D>::CS cs[C::TPT];
#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
      const int n = (int)min(n0 + i, (long)G.N - 1);
      const int t = n / HW;
      const int rem = n - t * HW;
      const int y = rem / G.W;
      cs[i] = Rope<D>::fetch(rv, cg, t, y, rem - y * G.W);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (t0 + kTile < ch.end) issue(t0 + kTile);   // prefetch the next tile
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss += kx[i][c] * kx[i][c];
      ss = group_sum<C::CG>(ss);
      const float inv = rsqrtf(ss * (1.0f / D) + G.eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float p = fmaxf(kx[i][c] * inv, 0.f);
        kx[i][c] = p;
        zacc[c] += p;
      }
      Rope<D>::apply(kx[i], cs[i]);
#pragma unroll
      for (int c = 0; c < 8; ++c) kx[i][c] *= bt[i];
    }

    const int col = tg * C::TPT;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      store_tcol<L, C::TPT>(rkT + (8 * cg + c) * C::PITCH + col, kx, c);
      store_tcol<L, C::TPT>(vT + (8 * cg + c) * C::PITCH + col, vx, c);
    }
    lds_barrier();

    const int lrow = lane & 31;
    const int lk = M::KPL * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kTile / M::KSTEP; ++ks) {
      if constexpr (C::KSPLIT) {
        if ((ks & 3) != wave) continue;
        const typename M::frag a = M::lds_frag(vT + lrow * C::PITCH + ks * M::KSTEP + lk);
        const typename M::frag b = M::lds_frag(rkT + lrow * C::PITCH + ks * M::KSTEP + lk);
        acc[0] = M::mma(a, b, acc[0]);
      } else if constexpr (C::TPW >= C::MT) {
        // wave owns one v-channel tile row and MT k-channel tiles (TPW == MT)
        const int dvt = wave;
        const typename M::frag a = M::lds_frag(vT + (32 * dvt + lrow) * C::PITCH + ks * M::KSTEP + lk);
#pragma unroll
        for (int u = 0; u < C::TPW; ++u) {
          const typename M::frag b = M::lds_frag(rkT + (32 * u + lrow) * C::PITCH + ks * M::KSTEP + lk);
          acc[u] = M::mma(a, b, acc[u]);
        }
      } else {
        const int ti = wave;  // TPW == 1
        const int dvt = ti / C::MT, dkt = ti % C::MT;
        const typename M::frag a = M::lds_frag(vT + (32 * dvt + lrow) * C::PITCH + ks * M::KSTEP + lk);
        const typename M::frag b = M::lds_frag(rkT + (32 * dkt + lrow) * C::PITCH + ks * M::KSTEP + lk);
        acc[0] = M::mma(a, b, acc[0]);
      }
    }
    lds_barrier();
  }

  float* dst = partial + ((size_t)ch.head * G.nseg * G.cps1 + ch.index) * (size_t)(D * D + D);

  // key-sum partial: fixed-order sum over the token groups
  float* zred = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int c = 0; c < 8; ++c) zred[tg * D + 8 * cg + c] = zacc[c];
  lds_barrier();
  if (tid < D) {
    float s = 0.f;
    for (int gi = 0; gi < C::TG; ++gi) s += zred[gi * D + tid];
    dst[D * D + tid] = s;
  }
  lds_barrier();

  const int l32 = lane & 31;
  const int hi = lane >> 5;
  if constexpr (C::KSPLIT) {
    float* kred = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int r = 0; r < 16; ++r) kred[(wave * 16 + r) * 64 + lane] = acc[0][r];
    lds_barrier();
    if (wave == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float s = ((kred[(0 * 16 + r) * 64 + lane] + kred[(1 * 16 + r) * 64 + lane]) +
                         (kred[(2 * 16 + r) * 64 + lane] + kred[(3 * 16 + r) * 64 + lane]));
        const int row = 8 * (r >> 2) + 4 * hi + (r & 3);
        dst[row * D + l32] = s;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < C::TPW; ++u) {
      int dvt, dkt;
      if constexpr (C::TPW >= C::MT) { dvt = wave; dkt = u; }
      else { dvt = wave / C::MT; dkt = wave % C::MT; }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * dvt + 8 * (r >> 2) + 4 * hi + (r & 3);
        dst[row * D + 32 * dkt + l32] = acc[u][r];
      }
    }
  }
}


// ===========================================================================
// Pass 1 for bf16, d = 128: MFMA operand fragments built in registers.
//
// A wave works in 16-token steps.  Lane l owns channels 4m..4m+3 (m = l % 32)
// of 8 tokens; lanes 0-31 and 32-63 (h = l / 32) take the two halves of the
// step.  Every row load is 8 bytes per lane and 32 lanes cover a whole
// 256-byte token row (two full rows per load instruction).  Channel 4m + c is
// row/column m of MFMA slot c, so the 32x32x16 operand fragments come straight
// from registers: the k-side fragment of slot c packs channel c of the lane's
// 8 tokens with v_cvt_pk_bf16_f32, the v-side fragment selects the same 16-bit
// halves of the raw rows with v_perm_b32.  Output tile (a, c) of the state is
// S[4i + a][4j + c] (i, j = 0..31), the product of v-side slot a and k-side
// slot c.
//
// Per-step work is kept off the vector ALU where it can be:
//  * each step's loads go through buffer resources that end at the chunk's
//    last row, so rows past it read as zero (k = 0, v = 0, beta = 0) and add
//    nothing: no per-token masks;
//  * lane l walks the grid position of its own token 8h + (l % 8) of the step
//    and packs the three RoPE table row offsets of that token into one word;
//    DPP row broadcasts hand a token's word and beta to the lanes of its half,
//    which keep the table field of their own axis;
//  * the RMS sum over a token's 32 lanes uses DPP within 16-lane rows and
//    v_permlane16_swap across the two rows: no LDS round trips;
//  * the LDS RoPE table holds, per pair, the bf16 words (cos, -sin) and
//    (sin, cos), so each rotated channel is one v_dot2_f32_bf16 of the ReLU'd
//    bf16 pair with fp32 accumulation;
//  * the key sum takes two tokens per v_dot2_f32_bf16: (phi k_a, phi k_b) of
//    one channel against their RMS factors (bf16).
//
// state_partial_acc_kernel: every wave keeps the whole 128 x 128 state of its
// tokens in accumulation registers (16 tiles, 256 registers; one wave per
// SIMD, one workgroup per CU) and runs the 16 MFMAs of each step on its own
// fragments, 4 at a time between the token pairs of the next step (a wave
// issues in order).  No LDS traffic or barriers in the loop; rows are fetched
// three steps ahead.  The four waves' states are summed through LDS at the
// end.
// ===========================================================================
namespace frag1 {
constexpr int D = 128;
constexpr int kStep = 16;    // tokens per step (one MFMA K)
// Packed table row offsets (16-byte units) of a token, one word for its three
// axes.  A table of at most kNarrowEntries entries takes 10-bit fields (frame,
// y and x rows at bits 0, 10 and 20); a wide one (up to kRopeLdsEntries) 11-bit
// y and x fields at bits 10 and 21 beside the 10-bit frame field (a chunk spans
// at most kRegRopeMaxFrames frames).  The kernel is instantiated for both.
constexpr int kNarrowEntries = 2048;
template <bool WIDE> struct Pack {
  static constexpr int TB = 10, YB = WIDE ? 11 : 10, XB = WIDE ? 11 : 10;
  static constexpr int kEntries = WIDE ? kRopeLdsEntries : kNarrowEntries;
};
constexpr int kRotBytes = kRopeLdsEntries * 8; // LDS rotation table
using R = Rope<D>;

// Every row is read once: streaming loads carry kLoadStream (nontemporal).
// The tensor element type seen by the bf16 code: 4 channels of one token as
// two bf16 words.  fp8 rows are loaded as 4 bytes and widened right before
// use (every e4m3 value is exact in bf16).
template <typename E> struct Io;
template <> struct Io<bf16_t> {
  static constexpr uint32_t ES = 2;   // bytes per element
  typedef u32x2 Word;                 // 4 channels as loaded
  __device__ __forceinline__ static Word load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, kLoadStream));
  }
  __device__ __forceinline__ static u32x2 bf16x4(Word w) { return w; }
  __device__ __forceinline__ static uint32_t load_beta(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, 0, 0);
  }
  __device__ __forceinline__ static int beta_f32_bits(uint32_t b) { return (int)(b << 16); }
};
template <> struct Io<bf8_t> {
  static constexpr uint32_t ES = 1;
  typedef uint32_t Word;
  __device__ __forceinline__ static Word load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, kLoadStream);
  }
  __device__ __forceinline__ static u32x2 bf16x4(Word w) {
    return (u32x2){Elem<bf8_t>::bf16_pair<false>(w), Elem<bf8_t>::bf16_pair<true>(w)};
  }
  __device__ __forceinline__ static uint32_t load_beta(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, 0, 0);
  }
  __device__ __forceinline__ static int beta_f32_bits(uint32_t b) {
    return __float_as_int(__builtin_amdgcn_cvt_f32_bf8((int)b, 0));
  }
};
template <> struct Io<fp8_t> {
  static constexpr uint32_t ES = 1;
  typedef uint32_t Word;
  __device__ __forceinline__ static Word load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, kLoadStream);
  }
  __device__ __forceinline__ static u32x2 bf16x4(Word w) {
    return (u32x2){Elem<fp8_t>::bf16_pair<false>(w), Elem<fp8_t>::bf16_pair<true>(w)};
  }
  __device__ __forceinline__ static uint32_t load_beta(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, 0, 0);
  }
  __device__ __forceinline__ static int beta_f32_bits(uint32_t b) {
    return __float_as_int(__builtin_amdgcn_cvt_f32_fp8((int)b, 0));
  }
};

template <typename E>
struct Rows {
  typename Io<E>::Word k[8], v[8];
  uint32_t b;               // beta (raw bits) of this lane's own token
};

// Per-lane constants of a chunk.
struct Lane {
  int lane, m, h;
  uint32_t lane_off;        // byte offset of this lane's 4 channels in a step's row 8h
  uint32_t beta_off;        // byte offset of beta of token (lane % 16) / 2 of this lane's half in a step
  uint32_t ROW;             // bytes between tokens
  uint32_t lane_rel;        // this lane's pair offset inside a table row (16-byte units)
  uint32_t ashift;          // bit offset of this lane's axis in the packed row offsets
  uint32_t awidth;          // and its width (wide tables)
  int t_lo, t_last, nt;     // frames the chunk spans
};

template <typename E, bool WIDE>
__device__ __forceinline__ Lane make_lane(const Geometry& G, const Chunk& ch) {
  using P = Pack<WIDE>;
  constexpr uint32_t ES = Io<E>::ES;
  Lane L;
  L.lane = threadIdx.x & 63;
  L.m = L.lane & 31;
  L.h = L.lane >> 5;
  L.ROW = (uint32_t)G.heads * D * ES;
  L.lane_off = (uint32_t)(8 * L.h) * L.ROW + (uint32_t)ch.head * D * ES + 4u * ES * L.m;
  L.beta_off = ((uint32_t)(8 * L.h + ((L.lane & 15) >> 1)) * (uint32_t)G.heads + (uint32_t)ch.head) * ES;
  // pairs 2m and 2m+1 share an axis
  const int axis = (2 * L.m < R::PT) ? 0 : ((2 * L.m < R::PT + R::PY) ? 1 : 2);
  const int first = axis == 0 ? 0 : (axis == 1 ? R::PT : R::PT + R::PY);
  L.lane_rel = (uint32_t)(2 * L.m - first) / 2;
  if constexpr (WIDE) {
    L.ashift = axis == 0 ? 0u : (axis == 1 ? (uint32_t)P::TB : (uint32_t)(P::TB + P::YB));
    L.awidth = axis == 0 ? (uint32_t)P::TB : (uint32_t)P::YB;
  } else {
    L.ashift = (uint32_t)axis * P::TB;
    L.awidth = (uint32_t)P::TB;
  }
  const int HW = G.H * G.W;
  L.t_lo = ch.begin < ch.end ? (int)(ch.begin / HW) : 0;
  L.t_last = ch.begin < ch.end ? (int)((ch.end - 1) / HW) : 0;
  L.nt = L.t_last - L.t_lo + 1;
  return L;
}

// RoPE rows of the frames the chunk spans, the y block and the x block,
// computed into LDS as per-pair bf16 words (cos, -sin), (sin, cos), and
// written in fp32 to the global table for the later kernels (the y/x blocks
// by one workgroup).  All threads take part; the caller synchronises.
template <bool WIDE>
__device__ __forceinline__ void compute_rotations(unsigned char* rtab, double* freq, float2* __restrict__ rope,
                                                  const Geometry& G, const Lane& L, bool write_yx) {
  R::template compute<Pack<WIDE>::kEntries, kThreads>(
      [&](int e, float2 cs) {
        *reinterpret_cast<u32x2*>(rtab + 8 * e) = (u32x2){pack2bf(cs.x, -cs.y), pack2bf(cs.y, cs.x)};
      },
      freq, rope, G.T, G.H, G.W, G.T_item, G.t_offset, L.t_lo, L.nt, write_yx);
}

// bf16 pair (lo: token a, hi: token b) of channel c from two raw 4-channel rows
__device__ __forceinline__ uint32_t sel_channel(u32x2 ra, u32x2 rb, int c) {
  const uint32_t wa = (c < 2) ? ra.x : ra.y;
  const uint32_t wb = (c < 2) ? rb.x : rb.y;
  // v_perm_b32 dst = bytes of {wb:wa} picked by the selector (byte 0-3 = wa)
  return (c & 1) ? __builtin_amdgcn_perm(wb, wa, 0x07060302u) : __builtin_amdgcn_perm(wb, wa, 0x05040100u);
}


// Rows [base, base + 16) of a step; rows at or past `end` read as zero.
template <typename E>
__device__ __forceinline__ void issue(Rows<E>& r, const E* __restrict__ k, const E* __restrict__ v,
                                      const E* __restrict__ beta, long base, long end, int heads,
                                      const Lane& L) {
  const long left = end - base;
  const uint32_t nvalid = left <= 0 ? 0u : (left >= kStep ? (uint32_t)kStep : (uint32_t)left);
  const size_t row0 = (size_t)base * heads * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + row0, nvalid * L.ROW);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + row0, nvalid * L.ROW);
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(beta + (size_t)base * heads, nvalid * (uint32_t)heads * Io<E>::ES);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    r.k[i] = Io<E>::load(krs, L.lane_off + (uint32_t)i * L.ROW);
    r.v[i] = Io<E>::load(vrs, L.lane_off + (uint32_t)i * L.ROW);
  }
  r.b = Io<E>::load_beta(brs, L.beta_off);
}

// Table row offsets (16-byte units) of the token at `gp` on the three axes.
template <bool WIDE>
__device__ __forceinline__ uint32_t table_rows(const GridPos& gp, const Lane& L, int H) {
  using P = Pack<WIDE>;
  const int tc = gp.t < L.t_last ? gp.t : L.t_last;
  return (uint32_t)((tc - L.t_lo) * R::PT / 2) |
         ((uint32_t)((L.nt * R::PT + gp.y * R::PY) / 2) << P::TB) |
         ((uint32_t)((L.nt * R::PT + H * R::PY + gp.x * R::PX) / 2) << (P::TB + P::YB));
}
static_assert(Pack<true>::TB + Pack<true>::YB + Pack<true>::XB == 32, "three fields in one word");
static_assert(Pack<false>::kEntries / 2 <= (1 << Pack<false>::XB), "narrow: rows fit 10-bit fields");
static_assert(Pack<true>::kEntries / 2 <= (1 << Pack<true>::XB), "wide: y and x rows fit 11-bit fields");
static_assert((kRegRopeMaxFrames - 1) * R::PT / 2 < (1 << Pack<true>::TB), "frame rows fit their field");

// Lane l "owns" token 8h + (l & 7) of a step: every 16-lane row holds the 8
// tokens of its half, so DPP row_newbcast:i hands token i of the lane's half
// to all lanes of a row without going through LDS.
__device__ __forceinline__ int own_token(int lane) { return 8 * (lane >> 5) + (lane & 7); }
template <int I>
__device__ __forceinline__ int row_bcast(int x) {
  return __builtin_amdgcn_mov_dpp(x, 0x150 + I, 0xF, 0xF, false);
}

// The 8 operand fragments of a step: kf[c] (k side) and vf[c] (v side).
// `offs` holds the packed table rows of this lane's own token.  The k-side
// RMS scale rides on the per-token factor: with
// inv = 1/sqrt(mean(k^2) + eps), phi(k inv) = inv phi(k), so
// rk = (beta inv) R phi(k) and the key sum adds inv phi(k).
// `between(ip)` runs after token pair ip (0..3): a caller can put work of its
// own (the previous step's MFMAs) between the vector instructions.
struct NoWork {
  __device__ __forceinline__ void operator()(int) const {}
};
template <typename E, bool WIDE, typename Between = NoWork>
__device__ __forceinline__ void build_step(const Rows<E>& raw, uint32_t offs, const unsigned char* rtab, const Lane& L,
                                           float eps, float (&zacc)[4], u32x4 (&kf)[4], u32x4 (&vf)[4],
                                           Between between = Between()) {
  // 4 channels of each of the 8 tokens as bf16 words
  struct { u32x2 k[8], v[8]; } r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    r.k[i] = Io<E>::bf16x4(raw.k[i]);
    r.v[i] = Io<E>::bf16x4(raw.v[i]);
  }
  // rotation words of the 8 tokens: all table reads issued together
  u32x4 cs[8];
#define GLA_FETCH(I)                                                                                 \
  {                                                                                                  \
    const uint32_t o = (uint32_t)row_bcast<I>((int)offs);                                            \
    cs[I] = *reinterpret_cast<const u32x4*>(rtab + 16 * (__builtin_amdgcn_ubfe(o, L.ashift, WIDE ? L.awidth : (uint32_t)Pack<false>::TB) + L.lane_rel)); \
  }
  GLA_FETCH(0) GLA_FETCH(1) GLA_FETCH(2) GLA_FETCH(3) GLA_FETCH(4) GLA_FETCH(5) GLA_FETCH(6) GLA_FETCH(7)
#undef GLA_FETCH
  // RMS factors.  Every lane holds 4 channels of each of its half's 8 tokens.
  // A butterfly over the 16 lanes of a row halves the tokens a lane carries at
  // every step (row_mirror pairs lane i with 15 - i, row_half_mirror i with
  // 7 - i, quad_perm [3,2,1,0] i with i ^ 3, then [1,0,3,2] i with i ^ 1), so
  // that lanes 2t and 2t + 1 of a row end with token t's sum over the row; the
  // other row of the half is added, and each lane takes one reciprocal square
  // root, of token t = (lane % 16) / 2, whose beta it also loaded.
  float sq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sq[i] = dot2bf(r.k[i].x, r.k[i].x, dot2bf(r.k[i].y, r.k[i].y, 0.f));
  const int lr = L.lane & 15;
  float s4[4], s2[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float keep = lr >= 8 ? sq[j + 4] : sq[j], send = lr >= 8 ? sq[j] : sq[j + 4];
    s4[j] = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0x140, 0xF, 0xF, false));
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float keep = (lr & 4) ? s4[j + 2] : s4[j], send = (lr & 4) ? s4[j] : s4[j + 2];
    s2[j] = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0x141, 0xF, 0xF, false));
  }
  float s1;
  {
    const float keep = (lr & 2) ? s2[1] : s2[0], send = (lr & 2) ? s2[0] : s2[1];
    s1 = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0x1B, 0xF, 0xF, false));
  }
  s1 += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s1), 0xB1, 0xF, 0xF, false));
  const float inv_own = __builtin_amdgcn_rsqf(pair_rows_sum(s1) * (1.0f / D) + eps);
  const float sc_own = __int_as_float(Io<E>::beta_f32_bits(raw.b)) * inv_own;   // beta / rms
  // the key sum's factors of token pair p as a bf16 pair, at lanes 4p, 4p + 1 of a row
  const uint32_t ip_own =
      pack2bf(inv_own, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(inv_own), 0x4E, 0xF, 0xF, false)));
  // every token's scale, and every token pair's key-sum factors, from their lanes
  float scs[8];
  uint32_t ips[4];
#define GLA_BCAST(I) scs[I] = __int_as_float(row_bcast<2 * I>(__float_as_int(sc_own)));
  GLA_BCAST(0) GLA_BCAST(1) GLA_BCAST(2) GLA_BCAST(3) GLA_BCAST(4) GLA_BCAST(5) GLA_BCAST(6) GLA_BCAST(7)
#undef GLA_BCAST
#define GLA_BCAST(P) ips[P] = (uint32_t)row_bcast<4 * P>((int)ip_own);
  GLA_BCAST(0) GLA_BCAST(1) GLA_BCAST(2) GLA_BCAST(3)
#undef GLA_BCAST
  uint32_t kp[4][4];   // [channel slot c][token pair]
#pragma unroll
  for (int ip = 0; ip < 4; ++ip) {
    float rk2[2][4];
    uint32_t ph2[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = 2 * ip + j;
      const float sc = scs[i];
      const uint32_t p01 = relu2(r.k[i].x), p23 = relu2(r.k[i].y);
      rk2[j][0] = sc * dot2bf(p01, cs[i].x, 0.f);
      rk2[j][1] = sc * dot2bf(p01, cs[i].y, 0.f);
      rk2[j][2] = sc * dot2bf(p23, cs[i].z, 0.f);
      rk2[j][3] = sc * dot2bf(p23, cs[i].w, 0.f);
      ph2[j][0] = p01;
      ph2[j][1] = p23;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) kp[c][ip] = pack2bf(rk2[0][c], rk2[1][c]);
    // key sum: channel c of the token pair against (inv_a, inv_b)
    const uint32_t ip2 = ips[ip];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t pa = ph2[0][c >> 1], pb = ph2[1][c >> 1];
      const uint32_t pr = (c & 1) ? __builtin_amdgcn_perm(pb, pa, 0x07060302u) : __builtin_amdgcn_perm(pb, pa, 0x05040100u);
      zacc[c] = dot2bf(pr, ip2, zacc[c]);
    }
    between(ip);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    kf[c] = (u32x4){kp[c][0], kp[c][1], kp[c][2], kp[c][3]};
    vf[c] = (u32x4){sel_channel(r.v[0], r.v[1], c), sel_channel(r.v[2], r.v[3], c),
                    sel_channel(r.v[4], r.v[5], c), sel_channel(r.v[6], r.v[7], c)};
  }
}

// Key sums of a workgroup: lanes m and m + 32 hold the same channels, then
// across the 4 waves through `zred` (LDS, 2 KB); wave 0 writes them.
__device__ __forceinline__ void write_key_sum(float (&zacc)[4], float* zred, float* dst, const Lane& L, int wave) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    zacc[c] += __int_as_float(__builtin_amdgcn_ds_bpermute((L.lane ^ 32) * 4, __float_as_int(zacc[c])));
  if (L.h == 0) *reinterpret_cast<f32x4*>(zred + wave * 128 + 4 * L.m) = (f32x4){zacc[0], zacc[1], zacc[2], zacc[3]};
  lds_barrier();
  if (wave == 0 && L.lane < 32) {
    f32x4 zz = *reinterpret_cast<const f32x4*>(zred + 4 * L.m);
#pragma unroll
    for (int wv = 1; wv < 4; ++wv) {
      const f32x4 o = *reinterpret_cast<const f32x4*>(zred + wv * 128 + 4 * L.m);
      zz.x += o.x; zz.y += o.y; zz.z += o.z; zz.w += o.w;
    }
    *reinterpret_cast<f32x4*>(dst + D * D + 4 * L.m) = zz;
  }
}
}  // namespace frag1

namespace acc1 {
constexpr int kHalfBytes = 32 * 1024;        // half of one wave's state (v-side slots 2R, 2R + 1)
constexpr int kSumBytes = 4 * kHalfBytes;    // the 4 waves' halves during the final sum
static_assert(frag1::kRotBytes <= kSumBytes, "the rotation table lies inside the final-sum space");
#ifndef GLA_ACC_DEPTH
#define GLA_ACC_DEPTH 3
#endif
constexpr int kDepth = GLA_ACC_DEPTH;        // steps of rows in flight per wave
}  // namespace acc1

template <typename E, bool WIDE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void state_partial_acc_kernel(
    const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ beta,
    float2* __restrict__ rope, float* __restrict__ partial, Geometry G) {
  using namespace frag1;
  using namespace acc1;
  // the RoPE table and the final sum share LDS (the table is dead by then)
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSumBytes + 2048];
  unsigned char* const rtab = smem;
  float* const zred = reinterpret_cast<float*>(smem + kSumBytes);

  const int lin = xcd_swizzle(blockIdx.x, gridDim.x);
  const Chunk ch = chunk_of(lin, G, G.cps1, G.chunk1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const Lane L = make_lane<E, WIDE>(G, ch);
  const int HW = G.H * G.W;
  // the first rows are requested before the RoPE rows are computed
  Rows<E> rr[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) issue(rr[d], k, v, beta, ch.begin + d * kTile + wave * kStep, ch.end, G.heads, L);
  compute_rotations<WIDE>(rtab, reinterpret_cast<double*>(zred), rope, G, L, lin == 0);

  // grid position of this lane's own token; a wave's steps are 64 apart
  GridPos gp;
  gp.set((int)(ch.begin + wave * kStep + own_token(L.lane)), G.H, G.W);
  const int adt = kTile / HW, ady = (kTile % HW) / G.W, adx = (kTile % HW) % G.W;

  f32x16 acc[4][4];   // [v-side slot a][k-side slot c]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;
  float zacc[4] = {0.f, 0.f, 0.f, 0.f};

  lds_barrier();   // RoPE rows staged

  // The MFMAs of a step run while the next step is built: one wave per SIMD
  // issues in order, so the 16 MFMAs of step s go out 4 at a time between
  // the token pairs of step s + 1 (fragments pk, pv; zero before the first).
  u32x4 pk[4], pv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) pk[c] = pv[c] = (u32x4){0u, 0u, 0u, 0u};
  auto mfma_row = [&](int a) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pv[a]),
                                                          __builtin_bit_cast(bf16x8, pk[c]), acc[a][c], 0, 0, 0);
  };

  // Wave w takes the steps at t0 + 16 w of every 64-token tile.  Every step
  // refills its rows and the loop body runs all kDepth steps, also past the
  // chunk end (those rows read as zero and add nothing): with the same loads
  // on every path the compiler waits for exactly the rows a step uses.
  auto step = [&](Rows<E>& rows, long t0) {
    u32x4 kf[4], vf[4];
    build_step<E, WIDE>(rows, table_rows<WIDE>(gp, L, G.H), rtab, L, G.eps, zacc, kf, vf, mfma_row);
    gp.advance(adt, ady, adx, G.H, G.W);
    issue(rows, k, v, beta, t0 + kDepth * kTile + wave * kStep, ch.end, G.heads, L);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      pk[c] = kf[c];
      pv[c] = vf[c];
    }
  };

  for (long t0 = ch.begin; t0 < ch.end; t0 += kDepth * kTile) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) step(rr[d], t0 + d * kTile);
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) mfma_row(a);   // the last step's MFMAs

  // Sum the 4 waves' states in two rounds of two v-side slots: every wave
  // stores its half as [a'][r][lane][c] (the 4 k-side slots of one output row
  // next to each other), then every thread adds the 4 copies in wave order
  // (the same result on every run) and writes rows of the partial.
  float* dst = partial + ((size_t)ch.head * G.nseg * G.cps1 + ch.index) * (size_t)(D * D + D);
  write_key_sum(zacc, zred, dst, L, wave);   // its barrier also retires the table
#pragma unroll
  for (int R = 0; R < 2; ++R) {
    if (R == 1) lds_barrier();   // round 0 read out
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        *reinterpret_cast<f32x4*>(smem + wave * kHalfBytes + ((a2 * 16 + r) * 64 + L.lane) * 16) =
            (f32x4){acc[2 * R + a2][0][r], acc[2 * R + a2][1][r], acc[2 * R + a2][2][r], acc[2 * R + a2][3][r]};
    lds_barrier();
    // S[4 mr + a][4 n + c] with mr = 8(r/4) + 4h + r%4, n = lane % 32
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = (int)threadIdx.x + j * kThreads;   // (a' * 16 + r) * 64 + lane
      const int ln = e & 63, r = (e >> 6) & 15, a = 2 * R + (e >> 10);
      const int mr = 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
      f32x4 sum = *reinterpret_cast<const f32x4*>(smem + e * 16);
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(smem + w * kHalfBytes + e * 16);
        sum.x += o.x; sum.y += o.y; sum.z += o.z; sum.w += o.w;
      }
      *reinterpret_cast<f32x4*>(dst + (4 * mr + a) * D + 4 * (ln & 31)) = sum;
    }
  }
}

template <int D, typename E>
hipError_t launch_state_partial(const LaunchArgs& a) {
  const Geometry& G = a.geo;
  const int blocks = G.heads * G.nseg * G.cps1;
  if constexpr (D == 128 && Elem<typename Elem<E>::Lds>::is_bf16) {   // bf16 and fp8 rows
    if (G.pass1_reg) {   // the planner sets it only with the RoPE rows in LDS
      // entries of the table a chunk stages: the y and x blocks and the frames it spans
      const long HW = (long)G.H * G.W;
      long frames = (G.chunk1 + HW - 2) / HW + 1;
      if (frames > G.T_item) frames = G.T_item;
      const long entries = (long)(G.H + G.W) * (3 * D / 16) + frames * (D / 8);
      if (entries > frag1::kNarrowEntries)
        hipLaunchKernelGGL((state_partial_acc_kernel<E, true>), dim3(blocks), dim3(kThreads), 0, a.stream,
                           (const E*)a.k, (const E*)a.v, (const E*)a.beta, a.rope, a.partial, G);
      else
        hipLaunchKernelGGL((state_partial_acc_kernel<E, false>), dim3(blocks), dim3(kThreads), 0, a.stream,
                           (const E*)a.k, (const E*)a.v, (const E*)a.beta, a.rope, a.partial, G);
      return hipGetLastError();
    }
  }
  if (G.rope_lds1)
    hipLaunchKernelGGL((state_partial_kernel<D, E, true>), dim3(blocks), dim3(kThreads), 0, a.stream,
                       (const E*)a.k, (const E*)a.v, (const E*)a.beta, a.rope, a.partial, G);
  else
    hipLaunchKernelGGL((state_partial_kernel<D, E, false>), dim3(blocks), dim3(kThreads), 0, a.stream,
                       (const E*)a.k, (const E*)a.v, (const E*)a.beta, a.rope, a.partial, G);
  return hipGetLastError();
}

template hipError_t launch_state_partial<32, float>(const LaunchArgs&);
template hipError_t launch_state_partial<64, float>(const LaunchArgs&);
template hipError_t launch_state_partial<128, float>(const LaunchArgs&);
template hipError_t launch_state_partial<32, bf16_t>(const LaunchArgs&);
template hipError_t launch_state_partial<64, bf16_t>(const LaunchArgs&);
template hipError_t launch_state_partial<128, bf16_t>(const LaunchArgs&);
template hipError_t launch_state_partial<32, fp8_t>(const LaunchArgs&);
template hipError_t launch_state_partial<64, fp8_t>(const LaunchArgs&);
template hipError_t launch_state_partial<128, fp8_t>(const LaunchArgs&);
template hipError_t launch_state_partial<32, bf8_t>(const LaunchArgs&);
template hipError_t launch_state_partial<64, bf8_t>(const LaunchArgs&);
template hipError_t launch_state_partial<128, bf8_t>(const LaunchArgs&);

}  // namespace gla
