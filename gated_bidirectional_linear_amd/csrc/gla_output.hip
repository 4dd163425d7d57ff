// Pass 2: the fused output kernel.
#include "gla_common.h"

namespace gla {

// ===========================================================================
// 4. Fused output
// ===========================================================================
// E is the tensor element type; the rotated queries go to LDS and into the
// MFMA as Elem<E>::Lds (fp32 for fp32, bf16 for bf16 and fp8).
template <int D, typename E>
struct OutputCfg {
  typedef typename Elem<E>::Lds L;
  static constexpr int CG = D / 8;
  static constexpr int TG = kThreads / CG;
  // 32-token tiles where every thread still has a whole token (d >= 64):
  // half the LDS and prefetch registers of 64-token tiles, so more
  // workgroups fit on a CU
  static constexpr int TILE = TG > 32 ? TG : 32;
  static constexpr int TPT = TILE / TG;
  static constexpr int MT = D / 32;                 // v-channel tiles
  static constexpr int NTK = TILE / 32;             // token tiles
  static constexpr int PAIRS = MT * NTK;
  static constexpr int PPW = PAIRS >= 4 ? PAIRS / 4 : 1;   // (v tile, token tile) pairs per wave
  static constexpr int ACTIVE = PAIRS >= 4 ? 4 : PAIRS;    // waves with MFMA work
  static constexpr int RQ_PITCH = D + (Elem<L>::is_bf16 ? 8 : 4);  // elements
  static constexpr int NUM_PITCH = D + 4;                           // floats
  static constexpr int RQ_BYTES = TILE * RQ_PITCH * (int)sizeof(L);
  static constexpr int NUM_BYTES = TILE * NUM_PITCH * 4;
  static constexpr int SMEM = RQ_BYTES + NUM_BYTES;   // separate regions: two barriers per tile
};

// The q-side RMS scale is folded out of the per-element work: with
// r = sqrt(mean(q^2) + eps), phi(q/r) = phi(q)/r, so
//   sigmoid(g) * S R phi(q^) / (phi(q^) . z + eps)
//     = sigmoid(g) * S R phi(q) / (phi(q) . z + eps * r).
// The MFMA therefore takes the rotated raw features, and the output RMSNorm
// of x = y / den (y = sigmoid(g) * num, den > 0) is w * y times the per-token
// scale 1 / sqrt(mean(y^2) + eps * den^2) (out_scale), which needs no 1 / den.
template <int D, typename E, bool LDSR>
__global__ __launch_bounds__(kThreads) void output_kernel(
    const E* __restrict__ q, const E* __restrict__ g, const float* __restrict__ states,
    const float* __restrict__ rms_w, const float2* __restrict__ rope, E* __restrict__ out, Geometry G) {
  using C = OutputCfg<D, E>;
  using L = typename C::L;
  using M = Mfma<L>;
  using R = Rope<D>;
  using BR = BufRow<E>;
  typedef typename BR::Raw Raw;
  constexpr int KSTEPS = D / M::KSTEP;
  constexpr int SZ = D * D + D;
  constexpr int ROPE_BYTES = LDSR ? kRopeLdsEntries * 8 : 0;
  constexpr bool kBf16 = Elem<E>::is_bf16;
  constexpr bool kFp8 = Elem<E>::is_f8;
  constexpr int SIG_BYTES = kFp8 ? 256 * 4 : 0;   // sigmoid of every fp8 gate code
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM + ROPE_BYTES + SIG_BYTES];
  constexpr int kT = C::TILE;
  L* rqs = reinterpret_cast<L*>(smem);                          // [kT][RQ_PITCH]  (token, k channel)
  float* nums = reinterpret_cast<float*>(smem + C::RQ_BYTES);   // [kT][NUM_PITCH] (token, v channel)

  const int lin = xcd_swizzle(blockIdx.x, gridDim.x);
  const Chunk ch = chunk_of(lin, G, G.cps2, G.chunk2);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int cg = tid % C::CG;
  const int tg = tid / C::CG;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  // read first in a tile's epilogue, after that tile's two barriers
  float* sig_tab = reinterpret_cast<float*>(smem + C::SMEM + ROPE_BYTES);
  if constexpr (kFp8) fill_sigmoid_fp8<E>(sig_tab, tid, kThreads);

  // Every tile's loads and stores go through buffer resources based at the
  // tile's first row and this head and ending at the chunk's last row: rows
  // past it read as zero and stores to them are dropped, so no path needs a
  // mask and every path issues the same memory operations (the compiler's
  // waits then cover exactly the rows in use).
  const uint32_t ROW = (uint32_t)G.heads * D * sizeof(E);
  const uint32_t head_off = (uint32_t)ch.head * D * sizeof(E);
  auto tile_rsrc = [&](const void* p, long t0) {
    const long left = ch.end - t0;
    const uint32_t rows = left <= 0 ? 0u : (left >= kT ? (uint32_t)kT : (uint32_t)left);
    const uint32_t bytes = rows == 0 ? 0u : rows * ROW - head_off;   // the last row ends at this head's D channels
    return make_rsrc(reinterpret_cast<const char*>(p) + (size_t)t0 * ROW + head_off, bytes);
  };
  uint32_t voff[C::TPT];
#pragma unroll
  for (int i = 0; i < C::TPT; ++i) voff[i] = (uint32_t)(tg * C::TPT + i) * ROW + 8u * cg * sizeof(E);

  const float* Sst = states + ((size_t)ch.seg * G.heads + ch.head) * SZ;
  // This wave's v-channel tile of S as MFMA A-fragments: A[m = v ch][k = k ch].
  const int dvt = (wave * C::PPW) / C::NTK;
  typename M::frag sfrag[KSTEPS];
  if (wave < C::ACTIVE) {
    const float* srow = Sst + (size_t)(32 * dvt + l32) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      float tmp[M::KPL];
#pragma unroll
      for (int j = 0; j < M::KPL; ++j) tmp[j] = srow[ks * M::KSTEP + M::KPL * hi + j];
      sfrag[ks] = M::from_f32(tmp);
    }
  }
  float zc[8], wc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    zc[c] = Sst[D * D + 8 * cg + c];
    wc[c] = rms_w[8 * cg + c];
  }

  const typename R::View rv = rope_view<D, LDSR>(reinterpret_cast<float2*>(smem + C::SMEM), rope, G, ch.begin, ch.end);
  // RoPE rows of this thread's 4 pairs: one axis when they share it
  const int p0 = 4 * cg;
  const int axis = (p0 < R::PT) ? 0 : ((p0 < R::PT + R::PY) ? 1 : 2);
  const int rbase = axis == 0 ? p0 - rv.t_lo * R::PT
                  : (axis == 1 ? rv.nt * R::PT + (p0 - R::PT) : rv.nt * R::PT + rv.H * R::PY + (p0 - R::PT - R::PY));
  const int rstride = axis == 0 ? R::PT : (axis == 1 ? R::PY : R::PX);
  // grid position of this thread's first token, advanced by kT per tile
  GridPos pos;
  pos.set((int)min(ch.begin + (long)tg * C::TPT, (long)G.N - 1), G.H, G.W);
  const int HW = G.H * G.W;
  const int adt = kT / HW, ady = (kT % HW) / G.W, adx = kT % G.W;

  // Two tiles of q/g rows in flight: buffers A and B alternate.
  Raw qa[C::TPT], ga[C::TPT], qb[C::TPT], gb[C::TPT];
  auto issue = [&](Raw (&qr)[C::TPT], Raw (&gr)[C::TPT], long t0) {
    const __amdgpu_buffer_rsrc_t qrs = tile_rsrc(q, t0), grs = tile_rsrc(g, t0);
#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
      qr[i] = BR::load(qrs, voff[i], 0);
      gr[i] = BR::load(grs, voff[i], 0);
    }
  };
  issue(qa, ga, ch.begin);
  issue(qb, gb, ch.begin + kT);
  if constexpr (LDSR) lds_barrier();

  auto tile = [&](Raw (&qr)[C::TPT], Raw (&gr)[C::TPT], long t0) {
    // RoPE entries of this tile's tokens
    typename R::CS cs[C::TPT];
    GridPos pp = pos;
#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
      if constexpr (R::kGrouped) {
        const int ps = axis == 0 ? pp.t : (axis == 1 ? pp.y : pp.x);
        const f32x4* e = reinterpret_cast<const f32x4*>(rv.tab + rbase + ps * rstride);
        const f32x4 a = e[0], b = e[1];
        cs[i].c[0] = a.x; cs[i].s[0] = a.y; cs[i].c[1] = a.z; cs[i].s[1] = a.w;
        cs[i].c[2] = b.x; cs[i].s[2] = b.y; cs[i].c[3] = b.z; cs[i].s[3] = b.w;
      } else {
        cs[i] = R::fetch(rv, cg, pp.t, pp.y, pp.x);
      }
      pp.next(G.H, G.W);
    }
    pos.advance(adt, ady, adx, G.H, G.W);

    float den[C::TPT];
#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
      float ph[8];
      float ss = 0.f;
      if constexpr (kBf16) {
        const u32x4 u = qr[i];
        ss = dot2sq(u.x, ss); ss = dot2sq(u.y, ss); ss = dot2sq(u.z, ss); ss = dot2sq(u.w, ss);
        const u32x4 rl = {relu2(u.x), relu2(u.y), relu2(u.z), relu2(u.w)};
        Elem<E>::unpack(rl, ph);
      } else {
        Elem<E>::unpack(qr[i], ph);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          ss += ph[c] * ph[c];
          // ReLU as one v_max_i32 on the bits (fmaxf adds a canonicalising max):
          // every negative value, -0 included, has the sign bit set
          const int b = __float_as_int(ph[c]);
          ph[c] = __int_as_float(b > 0 ? b : 0);
        }
      }
      float dp = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) dp += ph[c] * zc[c];
      ss = group_sum<C::CG>(ss);
      dp = group_sum<C::CG>(dp);
      const float ms = ss * (1.0f / D) + G.eps;
      const float r = ms * __builtin_amdgcn_rsqf(ms);   // sqrt(ms) without the IEEE sqrt sequence
      den[i] = dp + G.eps * r;
      R::apply(ph, cs[i]);
      L* dst = rqs + (tg * C::TPT + i) * C::RQ_PITCH + 8 * cg;
      if constexpr (Elem<L>::is_bf16) {
        *reinterpret_cast<u32x4*>(dst) = Elem<bf16_t>::pack(ph);
      } else {
        *reinterpret_cast<f32x4*>(dst) = (f32x4){ph[0], ph[1], ph[2], ph[3]};
        *reinterpret_cast<f32x4*>(dst + 4) = (f32x4){ph[4], ph[5], ph[6], ph[7]};
      }
    }
    // q rows consumed: refill with the rows two tiles ahead
    {
      const __amdgpu_buffer_rsrc_t qrs = tile_rsrc(q, t0 + 2 * kT);
#pragma unroll
      for (int i = 0; i < C::TPT; ++i) qr[i] = BR::load(qrs, voff[i], 0);
    }
    // rq tile complete; every wave has also finished reading the previous
    // tile's nums, so they may be overwritten below
    lds_barrier();

    if (wave < C::ACTIVE) {
#pragma unroll
      for (int u = 0; u < C::PPW; ++u) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const int ntt = (wave * C::PPW + u) % C::NTK;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const typename M::frag b = M::lds_frag(rqs + (32 * ntt + l32) * C::RQ_PITCH + ks * M::KSTEP + M::KPL * hi);
          acc = M::mma(sfrag[ks], b, acc);
        }
        float* row = nums + (32 * ntt + l32) * C::NUM_PITCH + 32 * dvt + 4 * hi;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          *reinterpret_cast<f32x4*>(row + 8 * rb) = (f32x4){acc[4 * rb], acc[4 * rb + 1], acc[4 * rb + 2], acc[4 * rb + 3]};
      }
    }
    // nums complete; every wave has also finished reading rq
    lds_barrier();

    const __amdgpu_buffer_rsrc_t ors = tile_rsrc(out, t0);
#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
      const float* src = nums + (tg * C::TPT + i) * C::NUM_PITCH + 8 * cg;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
      float y[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      float ss = 0.f;
      if constexpr (kFp8) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          y[c] *= sigmoid_fp8(sig_tab, c < 4 ? gr[i].x : gr[i].y, c & 3);   // sigmoid(g) * num
          ss += y[c] * y[c];
        }
      } else {
        float gv[8];
        Elem<E>::unpack(gr[i], gv);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          y[c] *= __builtin_amdgcn_rcpf(1.0f + __expf(-gv[c]));   // sigmoid(g) * num
          ss += y[c] * y[c];
        }
      }
      ss = group_sum<C::CG>(ss);
      const float scale = out_scale(ss * (1.0f / D), den[i], G.eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = wc[c] * y[c] * scale;
      BR::store(ors, voff[i], 0, Elem<E>::pack(y));   // rows past the chunk are dropped
    }
    // g rows consumed: refill with the rows two tiles ahead
    {
      const __amdgpu_buffer_rsrc_t grs = tile_rsrc(g, t0 + 2 * kT);
#pragma unroll
      for (int i = 0; i < C::TPT; ++i) gr[i] = BR::load(grs, voff[i], 0);
    }
  };

  // Both tiles of the body run also past the chunk end (their rows read as
  // zero and their stores are dropped).
  for (long t0 = ch.begin; t0 < ch.end; t0 += 2 * kT) {
    tile(qa, ga, t0);
    tile(qb, gb, t0 + kT);
  }
}

// ===========================================================================
// Fused output for bf16, d = 128, HP heads per workgroup (2 or 4).
//
// Taking heads in pairs gives each workgroup 512-byte token row segments and
// measured faster than one head per workgroup (~770 against ~800 us at
// 720p/60s).  128 HP threads (two waves per head): lane group cg = tid % (16 HP)
// holds 8 channels (head cg / 16, channels 8 (cg % 16)..+7) of token
// tg = tid / (16 HP) + 8 i (i = 0..3) of each 32-token tile; rows are fetched
// two tiles ahead through buffer resources that end at the chunk (rows past it
// read as zero, stores to them are dropped).  Two workgroups share a CU, so
// one's MFMAs overlap the other's vector work.  Wave w multiplies head w / 2's
// rotated queries by two 32-row tiles of its state (16 A-fragments in
// registers).  The per-token math is the same as in output_kernel.
// ===========================================================================
namespace pair2 {
// 8 channels of one token as the kernel reads and writes them (bf16 rows of
// 16 bytes).
template <typename E> struct Row8;
template <> struct Row8<bf16_t> {
  static constexpr uint32_t ES = 2;
  typedef u32x4 Raw;
  __device__ __forceinline__ static Raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff) { return buf_load16(r, voff, 0); }
  __device__ __forceinline__ static u32x4 bf16x8(const Raw& u) { return u; }
  __device__ __forceinline__ static void store(__amdgpu_buffer_rsrc_t r, uint32_t voff, const float (&y)[8]) {
    buf_store16(r, voff, 0, Elem<bf16_t>::pack(y));
  }
};

constexpr int D = 128;
constexpr int TILE = 32;              // tokens per tile
constexpr int DEPTH = 2;              // tiles of rows in flight
constexpr int RQ_PITCH = D + 8;       // bf16 elements per (token, head) row
constexpr int NUM_PITCH = D + 4;      // floats per (token, head) row
constexpr int KSTEPS = D / 16;
template <int HP>
struct Cfg {
  static constexpr int THREADS = 128 * HP;                 // two waves per head
  static constexpr int LPT = HP * D / 8;                   // lanes per token row segment
  static constexpr int TPI = THREADS / LPT;                // tokens per load instruction round (8)
  static constexpr int TPT = TILE / TPI;                   // tokens per thread per tile (4)
  static constexpr int RQ_BYTES = TILE * HP * RQ_PITCH * 2;
  static constexpr int NUM_BYTES = TILE * HP * NUM_PITCH * 4;
};
}  // namespace pair2

template <typename E, int HP>
__global__ __launch_bounds__(pair2::Cfg<HP>::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void output_pair_kernel(
    const E* __restrict__ q, const E* __restrict__ g, const float* __restrict__ states,
    const float* __restrict__ rms_w, const float2* __restrict__ rope, E* __restrict__ out, Geometry G) {
  using namespace pair2;
  using CF = Cfg<HP>;
  constexpr int TPI = CF::TPI, TPT = CF::TPT, RQ_BYTES = CF::RQ_BYTES, NUM_BYTES = CF::NUM_BYTES;
  using IO = Row8<E>;
  constexpr uint32_t ES = IO::ES;
  using R = Rope<D>;
  using M = Mfma<bf16_t>;
  constexpr int SZ = D * D + D;
  __shared__ __attribute__((aligned(16))) unsigned char smem[RQ_BYTES + NUM_BYTES + kRopeLdsEntries * 8];
  bf16_t* rqs = reinterpret_cast<bf16_t*>(smem);                 // [TILE][HP][RQ_PITCH]
  float* nums = reinterpret_cast<float*>(smem + RQ_BYTES);       // [TILE][HP][NUM_PITCH]

  // chunk-major over head groups: consecutive ids take the same token range
  const int npairs = G.heads / HP;
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x);
  const int ci = lin / npairs;
  const int pair = lin - ci * npairs;
  const int seg = ci / G.cps2;
  long s0, s1;
  seg_bounds(G, seg, s0, s1);
  const long cbeg = min(s0 + (long)(ci - seg * G.cps2) * G.chunk2, s1);
  const long cend = min(cbeg + (long)G.chunk2, s1);
  const int h0 = HP * pair;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int cg = tid % CF::LPT;         // lane group within a token's HP x 256 bytes
  const int hl = cg >> 4;               // head within the group
  const int c16 = cg & 15;              // channels 8 c16 .. 8 c16 + 7
  const int tg = tid / CF::LPT;         // token within an instruction round
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const uint32_t ROW = (uint32_t)G.heads * D * ES;
  const uint32_t pair_off = (uint32_t)h0 * D * ES;
  auto tile_rsrc = [&](const void* p, long t0) {
    const long left = cend - t0;
    const uint32_t rows = left <= 0 ? 0u : (left >= TILE ? (uint32_t)TILE : (uint32_t)left);
    const uint32_t bytes = rows == 0 ? 0u : rows * ROW - pair_off;   // the last row ends at this pair's channels
    return make_rsrc(reinterpret_cast<const char*>(p) + (size_t)t0 * ROW + pair_off, bytes);
  };
  uint32_t voff[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) voff[i] = (uint32_t)(i * TPI + tg) * ROW + (uint32_t)hl * D * ES + 8u * ES * c16;

  // this wave's head and its two 32-row tiles of S as A-fragments
  const int hw = wave >> 1;
  const float* Sw = states + ((size_t)seg * G.heads + h0 + hw) * SZ;
  typename M::frag sfrag[2][KSTEPS];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const float* srow = Sw + (size_t)(32 * (2 * (wave & 1) + v) + l32) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(srow + 16 * ks + 8 * hi);
      const f32x4 b = *reinterpret_cast<const f32x4*>(srow + 16 * ks + 8 * hi + 4);
      const float tmp[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      sfrag[v][ks] = M::from_f32(tmp);
    }
  }
  const float* zrow = states + ((size_t)seg * G.heads + h0 + hl) * SZ + D * D;
  float zc[8], wc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    zc[c] = zrow[8 * c16 + c];
    wc[c] = rms_w[8 * c16 + c];
  }

  const typename R::View rv = rope_view<D, true>(reinterpret_cast<float2*>(smem + RQ_BYTES + NUM_BYTES), rope, G,
                                                 cbeg, cend);
  const int t_last = cbeg < cend ? (int)((cend - 1) / (G.H * G.W)) : 0;
  const int p0 = 4 * c16;   // this thread's 4 pairs share one axis
  const int axis = (p0 < R::PT) ? 0 : ((p0 < R::PT + R::PY) ? 1 : 2);
  const int rbase = axis == 0 ? p0 - rv.t_lo * R::PT
                  : (axis == 1 ? rv.nt * R::PT + (p0 - R::PT) : rv.nt * R::PT + rv.H * R::PY + (p0 - R::PT - R::PY));
  const int rstride = axis == 0 ? R::PT : (axis == 1 ? R::PY : R::PX);
  // grid position of token tg of the current tile; tokens of a thread are TPI apart
  const int HW = G.H * G.W;
  GridPos pos;
  pos.set((int)(cbeg + tg), G.H, G.W);
  const int i_dt = TPI / HW, i_dy = (TPI % HW) / G.W, i_dx = (TPI % HW) % G.W;
  const int t_dt = TILE / HW, t_dy = (TILE % HW) / G.W, t_dx = (TILE % HW) % G.W;

  typedef typename IO::Raw Raw;
  Raw qr[DEPTH][TPT], gr[DEPTH][TPT];
  auto issue_q = [&](Raw (&r)[TPT], long t0) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(q, t0);
#pragma unroll
    for (int i = 0; i < TPT; ++i) r[i] = IO::load(rs, voff[i]);
  };
  auto issue_g = [&](Raw (&r)[TPT], long t0) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(g, t0);
#pragma unroll
    for (int i = 0; i < TPT; ++i) r[i] = IO::load(rs, voff[i]);
  };
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    issue_q(qr[d], cbeg + d * TILE);
    issue_g(gr[d], cbeg + d * TILE);
  }
  lds_barrier();   // RoPE rows staged

  // One tile.  Every path issues the same memory operations (rows past the
  // chunk read as zero, their stores are dropped), so the compiler's waits
  // cover exactly the rows in use.
  auto tile = [&](Raw (&qt)[TPT], Raw (&gt)[TPT], long t0) {
    float den[TPT];
    GridPos pp = pos;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int tc = pp.t < t_last ? pp.t : t_last;
      const int ps = axis == 0 ? tc : (axis == 1 ? pp.y : pp.x);
      const f32x4* e = reinterpret_cast<const f32x4*>(rv.tab + rbase + ps * rstride);
      const f32x4 ca = e[0], cb = e[1];
      typename R::CS cs;
      cs.c[0] = ca.x; cs.s[0] = ca.y; cs.c[1] = ca.z; cs.s[1] = ca.w;
      cs.c[2] = cb.x; cs.s[2] = cb.y; cs.c[3] = cb.z; cs.s[3] = cb.w;
      pp.advance(i_dt, i_dy, i_dx, G.H, G.W);

      const u32x4 u = IO::bf16x8(qt[i]);
      float ss = dot2sq(u.x, 0.f);
      ss = dot2sq(u.y, ss); ss = dot2sq(u.z, ss); ss = dot2sq(u.w, ss);
      const u32x4 rl = {relu2(u.x), relu2(u.y), relu2(u.z), relu2(u.w)};
      float ph[8];
      Elem<bf16_t>::unpack(rl, ph);
      float dp = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) dp += ph[c] * zc[c];
      ss = group_sum<16>(ss);
      dp = group_sum<16>(dp);
      const float ms = ss * (1.0f / D) + G.eps;
      const float r = ms * __builtin_amdgcn_rsqf(ms);   // sqrt(ms) without the IEEE sqrt sequence
      den[i] = dp + G.eps * r;
      R::apply(ph, cs);
      *reinterpret_cast<u32x4*>(rqs + ((i * TPI + tg) * HP + hl) * RQ_PITCH + 8 * c16) = Elem<bf16_t>::pack(ph);
    }
    pos.advance(t_dt, t_dy, t_dx, G.H, G.W);
    issue_q(qt, t0 + DEPTH * TILE);   // q rows consumed: refill DEPTH tiles ahead
    // rq tile complete; every wave has also finished reading the previous
    // tile's nums, so they may be overwritten below
    lds_barrier();

#pragma unroll
    for (int v = 0; v < 2; ++v) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const typename M::frag b = M::lds_frag(rqs + (l32 * HP + hw) * RQ_PITCH + ks * 16 + 8 * hi);
        acc = M::mma(sfrag[v][ks], b, acc);
      }
      // C[m = v channel 8(r/4) + 4 hi + r%4 of the tile][n = token l32]
      float* row = nums + (l32 * HP + hw) * NUM_PITCH + 32 * (2 * (wave & 1) + v) + 4 * hi;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        *reinterpret_cast<f32x4*>(row + 8 * rb) = (f32x4){acc[4 * rb], acc[4 * rb + 1], acc[4 * rb + 2], acc[4 * rb + 3]};
    }
    // nums complete; every wave has also finished reading rq
    lds_barrier();

    const __amdgpu_buffer_rsrc_t ors = tile_rsrc(out, t0);
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const float* src = nums + ((i * TPI + tg) * HP + hl) * NUM_PITCH + 8 * c16;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
      float y[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      float gv[8];
      Elem<bf16_t>::unpack(IO::bf16x8(gt[i]), gv);
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        y[c] *= __builtin_amdgcn_rcpf(1.0f + __expf(-gv[c]));   // sigmoid(g) * num
        ss += y[c] * y[c];
      }
      ss = group_sum<16>(ss);
      const float scale = out_scale(ss * (1.0f / D), den[i], G.eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = wc[c] * y[c] * scale;
      IO::store(ors, voff[i], y);   // rows past the chunk are dropped
    }
    issue_g(gt, t0 + DEPTH * TILE);   // g rows consumed: refill DEPTH tiles ahead
  };

  for (long t0 = cbeg; t0 < cend; t0 += DEPTH * TILE) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) tile(qr[d], gr[d], t0 + d * TILE);
  }
}

// ===========================================================================
// Fused output for bf16, d = 128, four heads per workgroup, with the work split
// by wave role.
//
// Four heads make each token's row segment 1 KB, so every wave instruction of
// the row streams reads or writes one whole contiguous kilobyte (a copy with
// this shape runs ~10% faster than with the 512-byte segments of head pairs).
// The 16 waves of the workgroup (one workgroup per CU) take two roles:
//   - 8 MFMA waves, two per head: wave w holds v rows 64 (w % 2) .. + 63 of
//     head w / 2's state as bf16 16x16x32 A-fragments (64 VGPRs, read as the
//     bf16 copy the reduce kernel writes), multiplies them by the tile's
//     rotated queries from LDS and writes the numerators to LDS; they also
//     load the g rows and write sigmoid(g) to LDS as fp16;
//   - 8 stream waves: wave w takes token w of every 8-token round (lane l:
//     head l / 16, channels 8 (l % 16) .. + 7), loads the q rows, builds
//     R phi(q) and the denominator, and in the epilogue forms
//     y = sigmoid(g) * num, the output RMSNorm and the store.
// Tiles are 16 tokens; the rotated queries, the numerators and the gates are
// double-buffered in LDS, so in one step the MFMA waves work on tile i while
// the stream waves finish tile i - 1 and prepare tile i + 1, with one barrier
// per step.  Since different waves carry the MFMAs and the vector work, the
// two overlap on every SIMD instead of alternating in lockstep phases.  The
// per-token LDS strides are odd multiples of 16 bytes, so the MFMA waves'
// 16-token accesses hit distinct banks.  The gate goes through LDS as fp16
// (relative rounding <= 2^-11, far below the output's bf16 rounding).
// The per-token math is output_kernel's.
// ===========================================================================
namespace quad2 {
constexpr int D = 128, HP = 4, TILE = 16;
constexpr int NMW = 8, NSW = 8;                        // MFMA waves (two per head), stream waves
constexpr int THREADS = 64 * (NMW + NSW);
constexpr int TPI = NSW;                               // tokens per round: one stream wave per token row
constexpr int TPT = TILE / TPI;                        // tokens per stream thread per tile
constexpr int QDEPTH = 2, GDEPTH = 2;                  // tiles of q / g rows in flight
constexpr int RQ_PITCH = D + 8;                        // 16-bit elements per (token, head) row of rq and sig
constexpr int NUM_PITCH = D + 4;                       // floats per (token, head) row of nums
constexpr int TOKQ = HP * RQ_PITCH + 8;                // 16-bit elements per token (69 x 16 bytes)
constexpr int TOKN = HP * NUM_PITCH + 4;               // floats per token (133 x 16 bytes)
constexpr int RQ_BYTES = TILE * TOKQ * 2;              // one buffer
constexpr int NUM_BYTES = TILE * TOKN * 4;
constexpr int SMEM = 2 * RQ_BYTES + 2 * NUM_BYTES + 2 * RQ_BYTES + kRopeLdsEntries * 8;
static_assert(SMEM <= 160 * 1024, "LDS budget");
}  // namespace quad2

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// The feature work of the four-head kernel for the waves that do it: R phi(q)
// of this thread's 8 channels of token rw + TPI i (i < TPT) of each tile into
// the rq buffer, and the denominators.  Row layout: wave w % 8 takes token w %
// 8 of each round; lane -> head lane / 16, channels 8 (lane % 16) .. + 7.
template <typename E>
struct QuadFeatures {
  using R = Rope<quad2::D>;
  typedef typename BufRow<E>::Raw Raw;
  float zc[8];               // key sums of this thread's channels
  int axis, rbase, rstride, t_last, rw, hl, c16;
  GridPos pos;               // of token rw of the next tile to prepare
  int i_dt, i_dy, i_dx, t_dt, t_dy, t_dx;
  const float2* tab;
  __device__ __forceinline__ QuadFeatures(const float* zrow, int rw_, int hl_, int c16_, const typename R::View& rv,
                                          long cbeg, long cend, const Geometry& G)
      : rw(rw_), hl(hl_), c16(c16_), tab(rv.tab) {
    using namespace quad2;
#pragma unroll
    for (int c = 0; c < 8; ++c) zc[c] = zrow[8 * c16 + c];
    t_last = cbeg < cend ? (int)((cend - 1) / (G.H * G.W)) : 0;
    const int p0 = 4 * c16;   // this thread's 4 pairs share one axis
    axis = (p0 < R::PT) ? 0 : ((p0 < R::PT + R::PY) ? 1 : 2);
    rbase = axis == 0 ? p0 - rv.t_lo * R::PT
          : (axis == 1 ? rv.nt * R::PT + (p0 - R::PT) : rv.nt * R::PT + rv.H * R::PY + (p0 - R::PT - R::PY));
    rstride = axis == 0 ? R::PT : (axis == 1 ? R::PY : R::PX);
    const int HW = G.H * G.W;
    pos.set((int)min(cbeg + rw, (long)G.N - 1), G.H, G.W);
    i_dt = TPI / HW; i_dy = (TPI % HW) / G.W; i_dx = (TPI % HW) % G.W;
    t_dt = TILE / HW; t_dy = (TILE % HW) / G.W; t_dx = (TILE % HW) % G.W;
  }
  // R phi(q) of the next tile (rows qt) into rq buffer rqb (bf16); its
  // denominators phi(q) . z + eps r into den
  __device__ __forceinline__ void run(const Raw (&qt)[quad2::TPT], bf16_t* rqb, const Geometry& G,
                                      float (&den)[quad2::TPT]) {
    using namespace quad2;
    GridPos pp = pos;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int tc = pp.t < t_last ? pp.t : t_last;
      const int ps = axis == 0 ? tc : (axis == 1 ? pp.y : pp.x);
      const f32x4* e = reinterpret_cast<const f32x4*>(tab + rbase + ps * rstride);
      const f32x4 ca = e[0], cb = e[1];
      typename R::CS cs;
      cs.c[0] = ca.x; cs.s[0] = ca.y; cs.c[1] = ca.z; cs.s[1] = ca.w;
      cs.c[2] = cb.x; cs.s[2] = cb.y; cs.c[3] = cb.z; cs.s[3] = cb.w;
      pp.advance(i_dt, i_dy, i_dx, G.H, G.W);
      u32x4 u;   // 8 channels as bf16 pairs (fp8 widens exactly)
      if constexpr (Elem<E>::is_f8) {
        u = (u32x4){Elem<E>::template bf16_pair<false>(qt[i].x), Elem<E>::template bf16_pair<true>(qt[i].x),
                    Elem<E>::template bf16_pair<false>(qt[i].y), Elem<E>::template bf16_pair<true>(qt[i].y)};
      } else {
        u = qt[i];
      }
      float ss = dot2sq(u.x, 0.f);
      ss = dot2sq(u.y, ss); ss = dot2sq(u.z, ss); ss = dot2sq(u.w, ss);
      const u32x4 rl = {relu2(u.x), relu2(u.y), relu2(u.z), relu2(u.w)};
      float ph[8];
      Elem<bf16_t>::unpack(rl, ph);
      float dp = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) dp += ph[c] * zc[c];
      ss = group_sum<16>(ss);
      dp = group_sum<16>(dp);
      const float ms = ss * (1.0f / D) + G.eps;
      const float r = ms * __builtin_amdgcn_rsqf(ms);   // sqrt(ms) without the IEEE sqrt sequence
      den[i] = dp + G.eps * r;
      R::apply(ph, cs);
      *reinterpret_cast<u32x4*>(rqb + (i * TPI + rw) * TOKQ + hl * RQ_PITCH + 8 * c16) = Elem<bf16_t>::pack(ph);
    }
    pos.advance(t_dt, t_dy, t_dx, G.H, G.W);
  }
};

// The four-head output kernel for bf16 rows (16 bytes per lane and 8
// channels): the MFMA waves compute sigmoid(g) and hand it to the stream waves
// through LDS as fp16; the stream waves compute the features of the next tile
// and the epilogue of the previous one.
template <typename E>
__global__ __launch_bounds__(quad2::THREADS) __attribute__((amdgpu_waves_per_eu(4, 4))) void output_quad_kernel(
    const E* __restrict__ q, const E* __restrict__ g, const float* __restrict__ states,
    const bf16_t* __restrict__ states_bf16, const float* __restrict__ rms_w, const float2* __restrict__ rope,
    E* __restrict__ out, Geometry G) {
  using namespace quad2;
  using BR = BufRow<E>;
  typedef typename BR::Raw Raw;
  constexpr uint32_t ES = sizeof(E);
  using R = Rope<D>;
  constexpr int SZ = D * D + D;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  bf16_t* rqs = reinterpret_cast<bf16_t*>(smem);                                    // [2][TILE][TOKQ]
  float* nums = reinterpret_cast<float*>(smem + 2 * RQ_BYTES);                      // [2][TILE][TOKN]
  uint16_t* sigs = reinterpret_cast<uint16_t*>(smem + 2 * RQ_BYTES + 2 * NUM_BYTES);  // [2][TILE][TOKQ] fp16
  float2* ropel = reinterpret_cast<float2*>(smem + 4 * RQ_BYTES + 2 * NUM_BYTES);

  // chunk-major over head quads: consecutive ids take the same token range
  const int nquads = G.heads / HP;
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x);
  const int ci = lin / nquads;
  const int quad = lin - ci * nquads;
  const int seg = ci / G.cps2;
  long s0, s1;
  seg_bounds(G, seg, s0, s1);
  const long cbeg = min(s0 + (long)(ci - seg * G.cps2) * G.chunk2, s1);
  const long cend = min(cbeg + (long)G.chunk2, s1);
  const int h0 = HP * quad;
  const int ntiles = (int)((cend - cbeg + TILE - 1) / TILE);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // row layout (both roles): wave w % 8 takes token w % 8 of each round; lane -> head lane / 16,
  // channels 8 (lane % 16) .. + 7
  const int rw = wave & 7;
  const int hl = lane >> 4;
  const int c16 = lane & 15;
  // Tile loads and stores go through buffer resources based at the tile's first
  // row and this quad, ending at the chunk's last row: rows past it read as zero
  // and stores to them are dropped.
  const uint32_t ROW = (uint32_t)G.heads * D * ES;
  const uint32_t quad_off = (uint32_t)h0 * D * ES;
  auto tile_rsrc = [&](const void* p, long t0) {
    const long left = cend - t0;
    const uint32_t rows = left <= 0 ? 0u : (left >= TILE ? (uint32_t)TILE : (uint32_t)left);
    const uint32_t bytes = rows == 0 ? 0u : rows * ROW - quad_off;   // the last row ends at this quad's channels
    return make_rsrc(reinterpret_cast<const char*>(p) + (size_t)t0 * ROW + quad_off, bytes);
  };
  uint32_t voff[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) voff[i] = (uint32_t)(i * TPI + rw) * ROW + (uint32_t)hl * D * ES + 8u * ES * c16;

  const typename R::View rv = rope_view<D, true>(ropel, rope, G, cbeg, cend);

  if (wave < NMW) {
    // ------------------------------ MFMA waves ------------------------------
    const int m = wave >> 1;            // head within the quad
    const int vh = 64 * (wave & 1);     // first v row of this wave
    const int r16 = lane & 15, k8 = lane >> 4;
    Raw gr[GDEPTH][TPT];
    auto issue_g = [&](Raw (&r)[TPT], long t0) {
      const __amdgpu_buffer_rsrc_t rs = tile_rsrc(g, t0);
#pragma unroll
      for (int i = 0; i < TPT; ++i) r[i] = BR::load(rs, voff[i], 0);
    };
#pragma unroll
    for (int d = 0; d < GDEPTH; ++d) issue_g(gr[d], cbeg + d * TILE);
    // A[i = v row vh + 16 mt + r16][k = 32 ks + 8 k8 + j] of the 16x16x32 MFMA
    const bf16_t* Sb = states_bf16 + ((size_t)seg * G.heads + h0 + m) * (D * D);
    bf16x8_t sf[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sf[mt][ks] = __builtin_bit_cast(bf16x8_t,
                                        *reinterpret_cast<const u32x4*>(Sb + (size_t)(vh + 16 * mt + r16) * D + 32 * ks + 8 * k8));
    lds_barrier();   // RoPE rows staged
    lds_barrier();   // rq of tile 0 written
    for (int i0 = 0; i0 < ntiles; i0 += GDEPTH) {
#pragma unroll
      for (int d = 0; d < GDEPTH; ++d) {
        const int i = i0 + d;
        if (i >= ntiles) break;   // uniform over the workgroup
        const long t0 = cbeg + (long)i * TILE;
        // numerators of tile i: num^T = S RQ^T, D[v = vh + 16 mt + 4 k8 + r][token r16]
        const bf16_t* rqb = rqs + (size_t)(i & 1) * (TILE * TOKQ);
        float* nb = nums + (size_t)(i & 1) * (TILE * TOKN);
        bf16x8_t bfr[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          bfr[ks] = __builtin_bit_cast(bf16x8_t,
                                       *reinterpret_cast<const u32x4*>(rqb + r16 * TOKQ + m * RQ_PITCH + 32 * ks + 8 * k8));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[mt][ks], bfr[ks], acc, 0, 0, 0);
          *reinterpret_cast<f32x4*>(nb + r16 * TOKN + m * NUM_PITCH + vh + 16 * mt + 4 * k8) = acc;
        }
        // sigmoid(g) of tile i, row layout, fp16
        uint16_t* sb = sigs + (size_t)(i & 1) * (TILE * TOKQ);
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
          float gv[8];
          Elem<E>::unpack(gr[d][j], gv);
          uint32_t w[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float s0 = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[2 * c]));
            const float s1 = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[2 * c + 1]));
            w[c] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){s0, s1}, f16x2_t));
          }
          *reinterpret_cast<u32x4*>(sb + (j * TPI + rw) * TOKQ + hl * RQ_PITCH + 8 * c16) = (u32x4){w[0], w[1], w[2], w[3]};
        }
        issue_g(gr[d], t0 + GDEPTH * TILE);
        lds_barrier();
      }
    }
    return;
  }

  // ------------------------------ stream waves ------------------------------
  const float* zrow = states + ((size_t)seg * G.heads + h0 + hl) * SZ + D * D;
  float zc[8], wc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    zc[c] = zrow[8 * c16 + c];
    wc[c] = rms_w[8 * c16 + c];
  }
  const int t_last = cbeg < cend ? (int)((cend - 1) / (G.H * G.W)) : 0;
  const int p0 = 4 * c16;   // this thread's 4 pairs share one axis
  const int axis = (p0 < R::PT) ? 0 : ((p0 < R::PT + R::PY) ? 1 : 2);
  const int rbase = axis == 0 ? p0 - rv.t_lo * R::PT
                  : (axis == 1 ? rv.nt * R::PT + (p0 - R::PT) : rv.nt * R::PT + rv.H * R::PY + (p0 - R::PT - R::PY));
  const int rstride = axis == 0 ? R::PT : (axis == 1 ? R::PY : R::PX);
  const int HW = G.H * G.W;
  GridPos pos;   // of token rw of the next tile to prepare; a thread's tokens are TPI apart
  pos.set((int)min(cbeg + rw, (long)G.N - 1), G.H, G.W);
  const int i_dt = TPI / HW, i_dy = (TPI % HW) / G.W, i_dx = (TPI % HW) % G.W;
  const int t_dt = TILE / HW, t_dy = (TILE % HW) / G.W, t_dx = (TILE % HW) % G.W;

  Raw qr[QDEPTH][TPT];
  auto issue_q = [&](Raw (&r)[TPT], long t0) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(q, t0);
#pragma unroll
    for (int i = 0; i < TPT; ++i) r[i] = BR::load(rs, voff[i], 0);
  };
#pragma unroll
  for (int d = 0; d < QDEPTH; ++d) issue_q(qr[d], cbeg + d * TILE);

  float den[2][TPT];   // denominators of the tiles in flight, by parity
  // R phi(q) of a tile into rq buffer b (bf16) and its denominators
  auto features = [&](Raw (&qt)[TPT], int b) {
    GridPos pp = pos;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int tc = pp.t < t_last ? pp.t : t_last;
      const int ps = axis == 0 ? tc : (axis == 1 ? pp.y : pp.x);
      const f32x4* e = reinterpret_cast<const f32x4*>(rv.tab + rbase + ps * rstride);
      const f32x4 ca = e[0], cb = e[1];
      typename R::CS cs;
      cs.c[0] = ca.x; cs.s[0] = ca.y; cs.c[1] = ca.z; cs.s[1] = ca.w;
      cs.c[2] = cb.x; cs.s[2] = cb.y; cs.c[3] = cb.z; cs.s[3] = cb.w;
      pp.advance(i_dt, i_dy, i_dx, G.H, G.W);
      u32x4 u;   // 8 channels as bf16 pairs (fp8 widens exactly)
      if constexpr (Elem<E>::is_f8) {
        u = (u32x4){Elem<E>::template bf16_pair<false>(qt[i].x), Elem<E>::template bf16_pair<true>(qt[i].x),
                    Elem<E>::template bf16_pair<false>(qt[i].y), Elem<E>::template bf16_pair<true>(qt[i].y)};
      } else {
        u = qt[i];
      }
      float ss = dot2sq(u.x, 0.f);
      ss = dot2sq(u.y, ss); ss = dot2sq(u.z, ss); ss = dot2sq(u.w, ss);
      const u32x4 rl = {relu2(u.x), relu2(u.y), relu2(u.z), relu2(u.w)};
      float ph[8];
      Elem<bf16_t>::unpack(rl, ph);
      float dp = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) dp += ph[c] * zc[c];
      ss = group_sum<16>(ss);
      dp = group_sum<16>(dp);
      const float ms = ss * (1.0f / D) + G.eps;
      const float r = ms * __builtin_amdgcn_rsqf(ms);   // sqrt(ms) without the IEEE sqrt sequence
      den[b][i] = dp + G.eps * r;
      R::apply(ph, cs);
      *reinterpret_cast<u32x4*>(rqs + (size_t)b * (TILE * TOKQ) + (i * TPI + rw) * TOKQ + hl * RQ_PITCH + 8 * c16) =
          Elem<bf16_t>::pack(ph);
    }
    pos.advance(t_dt, t_dy, t_dx, G.H, G.W);
  };
  // gate, RMSNorm and store of the tile at t0 from buffers b
  auto epilogue = [&](int b, long t0) {
    const __amdgpu_buffer_rsrc_t ors = tile_rsrc(out, t0);
    const float* nb = nums + (size_t)b * (TILE * TOKN);
    const uint16_t* sb = sigs + (size_t)b * (TILE * TOKQ);
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int tok = i * TPI + rw;
      const float* src = nb + tok * TOKN + hl * NUM_PITCH + 8 * c16;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 bb = *reinterpret_cast<const f32x4*>(src + 4);
      const u32x4 sw = *reinterpret_cast<const u32x4*>(sb + tok * TOKQ + hl * RQ_PITCH + 8 * c16);
      const float nm[8] = {a.x, a.y, a.z, a.w, bb.x, bb.y, bb.z, bb.w};
      const uint32_t sv[4] = {sw.x, sw.y, sw.z, sw.w};
      float y[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {   // sigmoid(g) * num, one v_fma_mix_f32 each
        const f16x2_t h = __builtin_bit_cast(f16x2_t, sv[c]);
        y[2 * c] = fmaf((float)h.x, nm[2 * c], 0.0f);
        y[2 * c + 1] = fmaf((float)h.y, nm[2 * c + 1], 0.0f);
      }
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss += y[c] * y[c];
      ss = group_sum<16>(ss);
      const float scale = out_scale(ss * (1.0f / D), den[b][i], G.eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = wc[c] * y[c] * scale;
      BR::store(ors, voff[i], 0, Elem<E>::pack(y));   // rows past the chunk are dropped
    }
  };

  lds_barrier();   // RoPE rows staged
  features(qr[0], 0);
  issue_q(qr[0], cbeg + QDEPTH * TILE);
  lds_barrier();   // rq of tile 0 written
  // step i: the MFMA waves take tile i; the stream waves finish tile i - 1 and
  // prepare tile i + 1 (past the chunk its rows read as zero)
  for (int i0 = 0; i0 < ntiles; i0 += QDEPTH) {
#pragma unroll
    for (int d = 0; d < QDEPTH; ++d) {
      const int i = i0 + d;
      if (i >= ntiles) break;   // uniform over the workgroup
      const long t0 = cbeg + (long)i * TILE;
      if (i >= 1) epilogue((i - 1) & 1, t0 - TILE);
      features(qr[(d + 1) % QDEPTH], (i + 1) & 1);
      issue_q(qr[(d + 1) % QDEPTH], t0 + TILE + QDEPTH * TILE);
      lds_barrier();
    }
  }
  if (ntiles > 0) epilogue((ntiles - 1) & 1, cbeg + (long)(ntiles - 1) * TILE);
}

// The four-head output kernel for fp8 rows (e4m3 or e5m2: 8 bytes per lane and
// 8 channels, a token's four heads 512 contiguous bytes per wave instruction),
// widened to bf16 exactly for the features.  With one-byte gates sigmoid(g)
// is a lookup in an LDS table of the 256 codes, so the roles split the vector
// work the other way round from the bf16 kernel above: the MFMA waves compute
// the next tile's features (R phi(q) and the denominators, handed to the
// stream waves through LDS) besides the numerators, and the stream waves read
// the gates and run the epilogue.
template <typename E>
__global__ __launch_bounds__(quad2::THREADS) __attribute__((amdgpu_waves_per_eu(4, 4))) void output_quad_f8_kernel(
    const E* __restrict__ q, const E* __restrict__ g, const float* __restrict__ states,
    const bf16_t* __restrict__ states_bf16, const float* __restrict__ rms_w, const float2* __restrict__ rope,
    E* __restrict__ out, Geometry G) {
  using namespace quad2;
  static_assert(Elem<E>::is_f8, "one-byte rows");
  using BR = BufRow<E>;
  typedef typename BR::Raw Raw;
  constexpr uint32_t ES = sizeof(E);
  using R = Rope<D>;
  constexpr int SZ = D * D + D;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  bf16_t* rqs = reinterpret_cast<bf16_t*>(smem);                                    // [2][TILE][TOKQ]
  float* nums = reinterpret_cast<float*>(smem + 2 * RQ_BYTES);                      // [2][TILE][TOKN]
  float* sig_tab = reinterpret_cast<float*>(smem + 2 * RQ_BYTES + 2 * NUM_BYTES);   // [256]
  float* dens = sig_tab + 256;                             // [4][TILE][HP], tile j in slot j & 3
  float2* ropel = reinterpret_cast<float2*>(smem + 4 * RQ_BYTES + 2 * NUM_BYTES);
  static_assert((256 + 4 * TILE * HP) * 4 <= 2 * RQ_BYTES, "gate table and denominators");

  // chunk-major over head quads: consecutive ids take the same token range
  const int nquads = G.heads / HP;
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x);
  const int ci = lin / nquads;
  const int quad = lin - ci * nquads;
  const int seg = ci / G.cps2;
  long s0, s1;
  seg_bounds(G, seg, s0, s1);
  const long cbeg = min(s0 + (long)(ci - seg * G.cps2) * G.chunk2, s1);
  const long cend = min(cbeg + (long)G.chunk2, s1);
  const int h0 = HP * quad;
  const int ntiles = (int)((cend - cbeg + TILE - 1) / TILE);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // row layout (both roles): wave w % 8 takes token w % 8 of each round; lane -> head lane / 16,
  // channels 8 (lane % 16) .. + 7
  const int rw = wave & 7;
  const int hl = lane >> 4;
  const int c16 = lane & 15;
  // Tile loads and stores go through buffer resources based at the tile's first
  // row and this quad, ending at the chunk's last row: rows past it read as zero
  // and stores to them are dropped.
  const uint32_t ROW = (uint32_t)G.heads * D * ES;
  const uint32_t quad_off = (uint32_t)h0 * D * ES;
  auto tile_rsrc = [&](const void* p, long t0) {
    const long left = cend - t0;
    const uint32_t rows = left <= 0 ? 0u : (left >= TILE ? (uint32_t)TILE : (uint32_t)left);
    const uint32_t bytes = rows == 0 ? 0u : rows * ROW - quad_off;   // the last row ends at this quad's channels
    return make_rsrc(reinterpret_cast<const char*>(p) + (size_t)t0 * ROW + quad_off, bytes);
  };
  uint32_t voff[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) voff[i] = (uint32_t)(i * TPI + rw) * ROW + (uint32_t)hl * D * ES + 8u * ES * c16;
  // rows of tile t0 of tensor p
  auto issue = [&](const E* p, Raw (&r)[TPT], long t0) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(p, t0);
#pragma unroll
    for (int i = 0; i < TPT; ++i) r[i] = BR::load(rs, voff[i], 0);
  };

  const typename R::View rv = rope_view<D, true>(ropel, rope, G, cbeg, cend);
  fill_sigmoid_fp8<E>(sig_tab, tid, THREADS);   // read after the first barrier

  if (wave < NMW) {
    // ------------------------------ MFMA waves ------------------------------
    const int m = wave >> 1;            // head within the quad
    const int vh = 64 * (wave & 1);     // first v row of this wave
    const int r16 = lane & 15, k8 = lane >> 4;
    Raw qr[QDEPTH][TPT];
#pragma unroll
    for (int d = 0; d < QDEPTH; ++d) issue(q, qr[d], cbeg + d * TILE);
    QuadFeatures<E> feat(states + ((size_t)seg * G.heads + h0 + hl) * SZ + D * D, rw, hl, c16, rv, cbeg, cend, G);
    // R phi(q) of tile j into rq buffer j & 1, its denominators into LDS slot j & 3
    auto features = [&](Raw (&qt)[TPT], int j) {
      float dn[TPT];
      feat.run(qt, rqs + (size_t)(j & 1) * (TILE * TOKQ), G, dn);
      if (c16 == 0) {
#pragma unroll
        for (int i = 0; i < TPT; ++i) dens[((j & 3) * TILE + i * TPI + rw) * HP + hl] = dn[i];
      }
    };
    // A[i = v row vh + 16 mt + r16][k = 32 ks + 8 k8 + j] of the 16x16x32 MFMA
    const bf16_t* Sb = states_bf16 + ((size_t)seg * G.heads + h0 + m) * (D * D);
    bf16x8_t sf[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sf[mt][ks] = __builtin_bit_cast(bf16x8_t,
                                        *reinterpret_cast<const u32x4*>(Sb + (size_t)(vh + 16 * mt + r16) * D + 32 * ks + 8 * k8));
    lds_barrier();   // RoPE rows and the gate table staged
    features(qr[0], 0);
    issue(q, qr[0], cbeg + QDEPTH * TILE);
    lds_barrier();   // rq of tile 0 written
    for (int i0 = 0; i0 < ntiles; i0 += QDEPTH) {
#pragma unroll
      for (int d = 0; d < QDEPTH; ++d) {
        const int i = i0 + d;
        if (i >= ntiles) break;   // uniform over the workgroup
        const long t0 = cbeg + (long)i * TILE;
        // numerators of tile i: num^T = S RQ^T, D[v = vh + 16 mt + 4 k8 + r][token r16]
        const bf16_t* rqb = rqs + (size_t)(i & 1) * (TILE * TOKQ);
        float* nb = nums + (size_t)(i & 1) * (TILE * TOKN);
        bf16x8_t bfr[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          bfr[ks] = __builtin_bit_cast(bf16x8_t,
                                       *reinterpret_cast<const u32x4*>(rqb + r16 * TOKQ + m * RQ_PITCH + 32 * ks + 8 * k8));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sf[mt][ks], bfr[ks], acc, 0, 0, 0);
          *reinterpret_cast<f32x4*>(nb + r16 * TOKN + m * NUM_PITCH + vh + 16 * mt + 4 * k8) = acc;
        }
        // features of tile i + 1 (past the chunk its rows read as zero)
        features(qr[(d + 1) % QDEPTH], i + 1);
        issue(q, qr[(d + 1) % QDEPTH], t0 + TILE + QDEPTH * TILE);
        lds_barrier();
      }
    }
    return;
  }

  // ------------------------------ stream waves ------------------------------
  float wc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) wc[c] = rms_w[8 * c16 + c];
  // gates of the tiles whose epilogue is next: tile j in slot j & 1, read two
  // steps after it is requested (the step loop below is unrolled by two)
  static_assert(QDEPTH == 2, "gate slots follow the two-tile unroll");
  Raw gq[2][TPT];
  issue(g, gq[0], cbeg);
  issue(g, gq[1], cbeg + TILE);
  // gate, RMSNorm and store of tile j (gates gt)
  auto epilogue = [&](int j, const Raw (&gt)[TPT]) {
    const __amdgpu_buffer_rsrc_t ors = tile_rsrc(out, cbeg + (long)j * TILE);
    const float* nb = nums + (size_t)(j & 1) * (TILE * TOKN);
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int tok = i * TPI + rw;
      const float* src = nb + tok * TOKN + hl * NUM_PITCH + 8 * c16;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 bb = *reinterpret_cast<const f32x4*>(src + 4);
      const float nm[8] = {a.x, a.y, a.z, a.w, bb.x, bb.y, bb.z, bb.w};
      float y[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = nm[c] * sigmoid_fp8(sig_tab, c < 4 ? gt[i].x : gt[i].y, c & 3);
      const float dn = dens[((j & 3) * TILE + tok) * HP + hl];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss += y[c] * y[c];
      ss = group_sum<16>(ss);
      const float scale = out_scale(ss * (1.0f / D), dn, G.eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = wc[c] * y[c] * scale;
      BR::store(ors, voff[i], 0, Elem<E>::pack(y));   // rows past the chunk are dropped
    }
  };

  lds_barrier();   // RoPE rows and the gate table staged
  lds_barrier();   // rq of tile 0 written
  // step i: the MFMA waves take tile i and prepare tile i + 1; the stream waves finish tile i - 1
  for (int i0 = 0; i0 < ntiles; i0 += QDEPTH) {
#pragma unroll
    for (int d = 0; d < QDEPTH; ++d) {
      const int i = i0 + d;
      if (i >= ntiles) break;   // uniform over the workgroup
      const long t0 = cbeg + (long)i * TILE;
      if (i >= 1) {
        // tile i - 1 (gate slot (d + 1) & 1, as i0 is even); the slot then takes tile i + 1
        epilogue(i - 1, gq[(d + 1) & 1]);
        issue(g, gq[(d + 1) & 1], t0 + TILE);
      }
      lds_barrier();
    }
  }
  if (ntiles > 0) {
    if ((ntiles - 1) & 1) epilogue(ntiles - 1, gq[1]);
    else epilogue(ntiles - 1, gq[0]);
  }
}

template <int D, typename E>
hipError_t launch_output(const LaunchArgs& a) {
  const Geometry& G = a.geo;
  if constexpr (D == 128 && sizeof(E) <= 2) {
    // the planner sets pass2_pair to 4 (bf16 or fp8) only for a head count divisible by 4
    // (and gives states_bf16), to 2 (bf16) only for an even one, both with the RoPE rows in LDS
    if (G.pass2_pair == 4) {
      const dim3 grid((G.heads / 4) * G.nseg * G.cps2);
      if constexpr (Elem<E>::is_f8)
        hipLaunchKernelGGL((output_quad_f8_kernel<E>), grid, dim3(quad2::THREADS), 0, a.stream, (const E*)a.q,
                           (const E*)a.g, (const float*)a.states, a.states_bf16, a.rms_w, (const float2*)a.rope,
                           (E*)a.out, G);
      else
        hipLaunchKernelGGL((output_quad_kernel<E>), grid, dim3(quad2::THREADS), 0, a.stream, (const E*)a.q,
                           (const E*)a.g, (const float*)a.states, a.states_bf16, a.rms_w, (const float2*)a.rope,
                           (E*)a.out, G);
      return hipGetLastError();
    }
  }
  if constexpr (D == 128 && Elem<E>::is_bf16) {
    if (G.pass2_pair == 2) {
      hipLaunchKernelGGL((output_pair_kernel<E, 2>), dim3((G.heads / 2) * G.nseg * G.cps2),
                         dim3(pair2::Cfg<2>::THREADS), 0, a.stream, (const E*)a.q, (const E*)a.g,
                         (const float*)a.states, a.rms_w, (const float2*)a.rope, (E*)a.out, G);
      return hipGetLastError();
    }
  }
  const int blocks = G.heads * G.nseg * G.cps2;
  if (G.rope_lds2)
    hipLaunchKernelGGL((output_kernel<D, E, true>), dim3(blocks), dim3(kThreads), 0, a.stream, (const E*)a.q,
                       (const E*)a.g, (const float*)a.states, a.rms_w, (const float2*)a.rope, (E*)a.out, G);
  else
    hipLaunchKernelGGL((output_kernel<D, E, false>), dim3(blocks), dim3(kThreads), 0, a.stream, (const E*)a.q,
                       (const E*)a.g, (const float*)a.states, a.rms_w, (const float2*)a.rope, (E*)a.out, G);
  return hipGetLastError();
}

template hipError_t launch_output<32, float>(const LaunchArgs&);
template hipError_t launch_output<64, float>(const LaunchArgs&);
template hipError_t launch_output<128, float>(const LaunchArgs&);
template hipError_t launch_output<32, bf16_t>(const LaunchArgs&);
template hipError_t launch_output<64, bf16_t>(const LaunchArgs&);
template hipError_t launch_output<128, bf16_t>(const LaunchArgs&);
template hipError_t launch_output<32, fp8_t>(const LaunchArgs&);
template hipError_t launch_output<64, fp8_t>(const LaunchArgs&);
template hipError_t launch_output<128, fp8_t>(const LaunchArgs&);
template hipError_t launch_output<32, bf8_t>(const LaunchArgs&);
template hipError_t launch_output<64, bf8_t>(const LaunchArgs&);
template hipError_t launch_output<128, bf8_t>(const LaunchArgs&);

}  // namespace gla
