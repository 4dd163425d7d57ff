// Pass 2 of the token-level causal form (SANA-Video notes, key design 2:
// causal linear attention as running sums of the per-token states and key
// sums).  Token i of a head reads
//   S_i = S_seg + sum_{j in seg, j <= i} beta_j v_j (R_j phi k^_j)^T
//   z_i = z_seg + sum_{j in seg, j <= i} phi k^_j
// (j < i when the own token is excluded), where (S_seg, z_seg) is the state
// exclusive of the token's segment that the reduce kernel wrote.
#include "gla_common.h"

namespace gla {

// Four waves per (head, segment) walk the segment in 32-token tiles (a
// workgroup takes one head or a head pair) and keep the running state
// transposed, S^T (k channel x v channel), in MFMA accumulators: wave w of a
// head owns v-channel tile w and every k-channel tile.  Per
// tile, with rq = R phi(q) (raw q; the RMS scale cancels, as in the
// bidirectional output kernel) and rk = beta R phi(k^):
//   num^T = S^T-as-A-operand x RQ^T      inter-tile part (state before the tile)
//         + V^T x AM^T                   intra-tile part, AM_ij = M_ij rk_j . rq_i
//   S^T  += RK^T x V                     state after the tile
//   den_i = phi(q_i) . z_i + eps r_i     z_i = running key sum up to token i
// For head pairs (bf16 operands) the denominator is split as the numerator is:
// phi(q_i) . z_run (the sums before the tile, fp32, in the feature phase) plus
// the masked row sums of phi(K^) phi(Q)^T (MFMA), and z_run grows by the
// tile's column sums of phi(K^) (an MFMA against ones); with fp32 operands the
// key sums are otherwise scanned in fp32.  The accumulator layout of S^T gives lane half
// h, register r the k channel 8(r/4) + 4h + r%4 of the lane's v column, so the
// state enters the numerator MFMA straight from registers, with the query
// operand read in that same channel order.
template <int D, typename E, int HP>
struct CausalCfg {
  typedef typename Elem<E>::Lds L;
  static constexpr int THREADS = kThreads * HP;              // four waves per head
  static constexpr int TT = 32;                              // tokens per tile
  static constexpr int CG = D / 8;                           // 8-channel groups per token and head
  static constexpr int TG = kThreads / CG;                   // token groups
  static constexpr int TPT = TG >= TT ? 1 : TT / TG;         // tokens per thread
  static constexpr int ACT = TT / TPT;                       // token groups with rows (d = 32 idles the rest)
  static constexpr int MT = D / 32;                          // 32-channel tiles
  static constexpr int PADL = Elem<L>::is_bf16 ? 8 : 4;      // elements
  // bf16 operands: token-major MFMA fragments come from the row-major rk and
  // v tiles through the LDS transpose read; fp32 operands keep transposed copies
  static constexpr bool TR = Elem<L>::is_bf16;
  // Row pitches (elements).  A 16-byte row read by 16 lanes (16 rows) is free
  // of bank conflicts when the pitch is 4 (mod 8) dwords; a transpose read (32
  // lanes: 4 rows x 64 bytes) when it is 16 (mod 64) dwords.  rq takes the
  // first; v (transpose reads only) the second; rk, read both ways, 20 (mod 64)
  // dwords, which keeps the row reads free and overlaps one transposed row pair.
  static constexpr int RP = D + PADL;                        // rqs: [token][channel]
  static constexpr int RPK = TR ? D + 40 : D + PADL;         // rks
  static constexpr int RPV = TR ? D + 32 : D + PADL;         // vs (bf16)
  static constexpr int CP = TT + PADL;                       // rkT, vT: [channel][token]; am: [i][j]
  static constexpr int FP = D + 4;                           // zk, nums: [token][channel] fp32
  static constexpr int RQ_OFF = 0;
  static constexpr int RK_OFF = RQ_OFF + TT * RP * (int)sizeof(L);
  static constexpr int KT_OFF = RK_OFF + TT * RPK * (int)sizeof(L);                 // rkT [D][CP] (fp32 only)
  static constexpr int VT_OFF = KT_OFF + (TR ? 0 : D * CP * (int)sizeof(L));         // vs [TT][RPV] or vT [D][CP]
  static constexpr int AM_OFF = VT_OFF + (TR ? TT * RPV : D * CP) * (int)sizeof(L);
  // Key sums.  Head pairs (bf16 operands) take the denominator's intra-tile
  // part and the tile's key sums on MFMA from bf16 rows of phi(q) ([TT][RP])
  // and phi(k) = relu(k) ([TT][RPK]; each token's RMS factor [TT] is applied
  // in those products), keeping the intra-tile denominators [TT] and the
  // tile's key sums [D] in fp32; otherwise phi(k^) is scanned in fp32
  // ([TT][FP]), which keeps a single head's LDS small enough for two
  // workgroups per CU.
  static constexpr bool MD = TR && HP == 2;
  static constexpr int ZK_OFF = AM_OFF + TT * CP * (int)sizeof(L);
  static constexpr int PHK_OFF = ZK_OFF + TT * RP * 2;
  static constexpr int DIN_OFF = PHK_OFF + TT * RPK * 2;
  static constexpr int ZS_OFF = DIN_OFF + TT * 4;
  static constexpr int INV_OFF = ZS_OFF + D * 4;
  static constexpr int ZK_BYTES = MD ? (TT * RP + TT * RPK) * 2 + (TT + D + TT) * 4 : TT * FP * 4;
  static constexpr int NUM_OFF = ZK_OFF + ZK_BYTES;
  static constexpr int SMEM = NUM_OFF + TT * FP * 4;        // per head
  static constexpr int ROPE = kRopeLdsEntriesCausal * 8;
  // waves per SIMD: a head pair's eight waves fill two; one head's four waves
  // reach two when two workgroups fit in LDS (with the RoPE rows)
  static constexpr int MIN_WAVES = HP == 2 ? 2 : (2 * (SMEM + ROPE) <= 160 * 1024 ? 2 : 1);
  static_assert(HP == 1 || (HP == 2 && HP * SMEM + ROPE <= 160 * 1024), "head pair must fit in LDS");
  static_assert(TPT * ACT == TT && TPT <= 2, "token split");
  static_assert(kThreads >= D, "scan threads");
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Operand fragment of 8 consecutive tokens of one channel from a row-major
// bf16 tile X[token][pitch] (ds_read_b64_tr_b16, two reads): lane l gets
// channel c0 + l % 32 at tokens tok0 + 8 (l / 32) + 0..7, the MFMA layout of
// a fragment whose K index is the token.  Within each 16-lane group, lane p
// addresses row (p / 4) and 4-channel block (p % 4) of a 4 x 16 block; the
// transpose hands lane i channel i of the block at the group's 4 rows.
__device__ __forceinline__ bf16x8 tr_frag(const bf16_t* X, int pitch, int tok0, int c0, int lane) {
  const int g = lane >> 4, p = lane & 15;
  const bf16_t* a = X + (tok0 + 8 * (g >> 1) + (p >> 2)) * pitch + c0 + 16 * (g & 1) + 4 * (p & 3);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 4 * pitch));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 r = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  return __builtin_bit_cast(bf16x8, r);
}

// The 8 channels of a raw row as 4 bf16 pairs (fp8 of either format widens exactly).
template <typename E>
__device__ __forceinline__ u32x4 bf16_words(const typename Elem<E>::Raw& r) {
  if constexpr (Elem<E>::is_f8) {
    return (u32x4){Elem<E>::template bf16_pair<false>(r.x), Elem<E>::template bf16_pair<true>(r.x),
                   Elem<E>::template bf16_pair<false>(r.y), Elem<E>::template bf16_pair<true>(r.y)};
  } else {
    return r;
  }
}

// LDS copy of the RoPE rows a segment needs (frames [t_lo, t_lo + nt), then
// the y and x blocks, laid out as the fp32 table) holding per pair the bf16
// words (cos, -sin) and (sin, cos): each rotated channel of a ReLU'd bf16
// pair is then one v_dot2_f32_bf16 with fp32 accumulation.
template <int D, int kMaxEntries, int THREADS>
__device__ __forceinline__ typename Rope<D>::View stage_rot_words(float2* lds, const float2* __restrict__ tab,
                                                                  const Geometry& G, long begin, long end) {
  using R = Rope<D>;
  const int HW = G.H * G.W;
  const int t_lo = begin < end ? (int)(begin / HW) : 0;
  const int nt = begin < end ? (int)((end - 1) / HW) - t_lo + 1 : 0;
  constexpr int PER = (kMaxEntries + THREADS - 1) / THREADS;
  const int n_t = nt * R::PT;
  const int total = n_t + G.H * R::PY + G.W * R::PX;
  float2 tmp[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = (int)threadIdx.x + j * THREADS;
    const int src = (i < n_t) ? t_lo * R::PT + i : G.T * R::PT + (i - n_t);
    tmp[j] = tab[i < total ? src : 0];
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = (int)threadIdx.x + j * THREADS;
    if (i < total)
      *reinterpret_cast<u32x2*>(lds + i) = (u32x2){pack2bf(tmp[j].x, -tmp[j].y), pack2bf(tmp[j].y, tmp[j].x)};
  }
  return typename R::View{lds, t_lo, nt, G.H};
}

// Operand fragments in the channel order of the accumulator layout.
template <typename L> struct PermFrag;
template <> struct PermFrag<bf16_t> {
  static constexpr int STEPS = 2;   // K = 16 steps per 32-channel block
  // slot j of lane half h in step s is channel 16s + 8(j/4) + 4h + j%4 of the block at p
  __device__ __forceinline__ static bf16x8 row(const bf16_t* p, int s, int h) {
    const uint2 a = *reinterpret_cast<const uint2*>(p + 16 * s + 4 * h);
    const uint2 b = *reinterpret_cast<const uint2*>(p + 16 * s + 8 + 4 * h);
    return __builtin_bit_cast(bf16x8, (uint4){a.x, a.y, b.x, b.y});
  }
  // accumulator registers 8s .. 8s+7 as an operand fragment (rounded to bf16)
  __device__ __forceinline__ static bf16x8 acc(const f32x16& c, int s) {
    uint4 u;
    u.x = pack2bf(c[8 * s + 0], c[8 * s + 1]);
    u.y = pack2bf(c[8 * s + 2], c[8 * s + 3]);
    u.z = pack2bf(c[8 * s + 4], c[8 * s + 5]);
    u.w = pack2bf(c[8 * s + 6], c[8 * s + 7]);
    return __builtin_bit_cast(bf16x8, u);
  }
};
template <> struct PermFrag<float> {
  static constexpr int STEPS = 16;  // K = 2 steps per 32-channel block
  __device__ __forceinline__ static float row(const float* p, int s, int h) { return p[8 * (s >> 2) + 4 * h + (s & 3)]; }
  __device__ __forceinline__ static float acc(const f32x16& c, int s) { return c[s]; }
};

// One beta per (token, head) through a buffer resource (rows past it read 0).
template <typename E> struct BetaLoad;
template <> struct BetaLoad<float> {
  typedef uint32_t Raw;
  __device__ __forceinline__ static Raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0);
  }
  __device__ __forceinline__ static float value(Raw x) { return __uint_as_float(x); }
};
template <> struct BetaLoad<bf16_t> {
  typedef unsigned short Raw;
  __device__ __forceinline__ static Raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, 0, 0);
  }
  __device__ __forceinline__ static float value(Raw x) { return __uint_as_float((uint32_t)x << 16); }
};
template <> struct BetaLoad<bf8_t> {
  typedef unsigned char Raw;
  __device__ __forceinline__ static Raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return (unsigned char)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, 0, 0);
  }
  __device__ __forceinline__ static float value(Raw x) { return __builtin_amdgcn_cvt_f32_bf8((int)x, 0); }
};
template <> struct BetaLoad<fp8_t> {
  typedef unsigned char Raw;
  __device__ __forceinline__ static Raw load(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return (unsigned char)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, 0, 0);
  }
  __device__ __forceinline__ static float value(Raw x) { return __builtin_amdgcn_cvt_f32_fp8((int)x, 0); }
};

// HP heads per workgroup (1, or 2 for bf16 operands at d = 128): with two,
// every row load and store covers the two heads' adjacent 2 x d elements of a
// token, which HBM serves faster than single-head segments; waves 4h..4h+3
// own head h of the pair.
template <int D, typename E, int HP, bool LDSR>
__global__ __launch_bounds__((CausalCfg<D, E, HP>::THREADS), (CausalCfg<D, E, HP>::MIN_WAVES)) void token_causal_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ beta,
    const E* __restrict__ g, const float* __restrict__ states, const float* __restrict__ rms_w,
    const float2* __restrict__ rope, E* __restrict__ out, Geometry G) {
  using C = CausalCfg<D, E, HP>;
  using L = typename C::L;
  using M = Mfma<L>;
  using PF = PermFrag<L>;
  using R = Rope<D>;
  using BR = BufRow<E>;
  using BL = BetaLoad<E>;
  typedef typename BR::Raw Raw;
  constexpr int TT = C::TT;
  constexpr int TPT = C::TPT;
  constexpr int SZ = D * D + D;
  constexpr int ROPE_BYTES = LDSR ? C::ROPE : 0;
  __shared__ __attribute__((aligned(16))) unsigned char smem[HP * C::SMEM + ROPE_BYTES];
  // per head h, from smem + h * SMEM:
  //   rqs  [TT][RP]   rq = R phi(q), raw q
  //   rks  [TT][RPK]  rk = beta R phi(k^)
  //   rkT  [D][CP]    rk transposed (fp32 operands only)
  //   vT   [TT][RPV]  v rows (bf16 operands) or [D][CP] v transposed
  //   am   [TT][CP]   masked rk_j . rq_i, row i
  //   zk   [TT][FP]   phi k^, then its running sums (fp32 scan), or
  //   phqs [TT][RP], phks [TT][RPK], dins [TT], zsum [D], invs [TT] (MFMA key sums; see CausalCfg)
  //   nums [TT][FP]   numerators (token, v channel), fp32
  auto rqs = [&](int h) { return reinterpret_cast<L*>(smem + h * C::SMEM + C::RQ_OFF); };
  auto rks = [&](int h) { return reinterpret_cast<L*>(smem + h * C::SMEM + C::RK_OFF); };
  auto rkT = [&](int h) { return reinterpret_cast<L*>(smem + h * C::SMEM + C::KT_OFF); };
  auto vT = [&](int h) { return reinterpret_cast<L*>(smem + h * C::SMEM + C::VT_OFF); };
  auto am = [&](int h) { return reinterpret_cast<L*>(smem + h * C::SMEM + C::AM_OFF); };
  auto zk = [&](int h) { return reinterpret_cast<float*>(smem + h * C::SMEM + C::ZK_OFF); };     // fp32 scan
  auto phqs = [&](int h) { return reinterpret_cast<bf16_t*>(smem + h * C::SMEM + C::ZK_OFF); };  // MFMA key sums
  auto phks = [&](int h) { return reinterpret_cast<bf16_t*>(smem + h * C::SMEM + C::PHK_OFF); };
  auto dins = [&](int h) { return reinterpret_cast<float*>(smem + h * C::SMEM + C::DIN_OFF); };
  auto zsum = [&](int h) { return reinterpret_cast<float*>(smem + h * C::SMEM + C::ZS_OFF); };
  auto invs = [&](int h) { return reinterpret_cast<float*>(smem + h * C::SMEM + C::INV_OFF); };
  auto nums = [&](int h) { return reinterpret_cast<float*>(smem + h * C::SMEM + C::NUM_OFF); };

  // workgroup -> (head group, segment), head groups of a segment consecutive
  const int lin = xcd_swizzle(blockIdx.x, gridDim.x);
  const int units = G.heads / HP;
  const int seg = lin / units;
  const int head0 = (lin - seg * units) * HP;
  long seg_begin, seg_end;
  seg_bounds(G, seg, seg_begin, seg_end);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // row work: thread = (token group, head of the pair, channel group), channels fastest
  const int cg = tid % C::CG;
  const int hl = (tid / C::CG) % HP;
  const int tg = tid / (C::CG * HP);
  // wave-uniform; true for every thread unless d = 32 (stated as a constant
  // then, so that the phases' row work and MFMAs share basic blocks)
  const bool rows = C::ACT * C::CG * HP == C::THREADS || tg < C::ACT;
  // MFMA and scan work: waves 4h..4h+3 serve head h
  const int hw = wave >> 2;
  const int ww = wave & 3;
  const bool mt_wave = C::MT >= 4 || ww < C::MT;   // this wave owns a 32-column tile of S^T
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool incl = G.include_self != 0;

  const uint32_t ROW = (uint32_t)G.heads * D * sizeof(E);
  const uint32_t head_off = (uint32_t)head0 * D * sizeof(E);
  const uint32_t BROW = (uint32_t)G.heads * sizeof(E);
  const uint32_t bhead_off = (uint32_t)head0 * sizeof(E);
  // rows [t0, min(t0 + TT, segment end)) of these heads: past them loads read 0
  // and stores are dropped
  auto tile_rows = [&](long t0) -> uint32_t {
    const long left = seg_end - t0;
    return left <= 0 ? 0u : (left >= TT ? (uint32_t)TT : (uint32_t)left);
  };
  auto tile_rsrc = [&](const void* p, long t0) {
    const uint32_t n = tile_rows(t0);
    return make_rsrc(reinterpret_cast<const char*>(p) + (size_t)t0 * ROW + head_off, n == 0 ? 0u : n * ROW - head_off);
  };
  auto beta_rsrc = [&](long t0) {
    const uint32_t n = tile_rows(t0);
    return make_rsrc(reinterpret_cast<const char*>(beta) + (size_t)t0 * BROW + bhead_off,
                     n == 0 ? 0u : n * BROW - bhead_off);
  };
  uint32_t voff[TPT], boff[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    voff[i] = (uint32_t)(tg * TPT + i) * ROW + (uint32_t)(hl * D + 8 * cg) * sizeof(E);
    boff[i] = (uint32_t)(tg * TPT + i) * BROW + (uint32_t)hl * sizeof(E);
  }

  // running state of head hw: S^T tiles of this wave's v columns, and (scan threads) z
  const float* Sst = states + ((size_t)seg * G.heads + head0 + hw) * SZ;
  f32x16 st[C::MT];
  if (mt_wave) {
#pragma unroll
    for (int ct = 0; ct < C::MT; ++ct)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(Sst + (size_t)(32 * ww + l32) * D + 32 * ct + 8 * rb + 4 * hi);
        st[ct][4 * rb] = s4.x; st[ct][4 * rb + 1] = s4.y; st[ct][4 * rb + 2] = s4.z; st[ct][4 * rb + 3] = s4.w;
      }
  }
  // key-sum scan: wave ww of the head takes channels 32 ww .. 32 ww + 31, lane
  // half hi the tile's tokens 16 hi .. 16 hi + 15; both halves hold the
  // running sum of their channel
  const bool scanner = !C::MD && 32 * ww < D;
  const int zc = 32 * ww + l32;
  float zrun = scanner ? Sst[D * D + zc] : 0.f;
  // MFMA key sums: the running key sums at this thread's 8 channels of head hl
  float zr[8];
  {
    const float* z0 = states + ((size_t)seg * G.heads + head0 + hl) * SZ + D * D + 8 * cg;
#pragma unroll
    for (int c = 0; c < 8; ++c) zr[c] = C::MD ? z0[c] : 0.f;
  }
  float wc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) wc[c] = rms_w[8 * cg + c];

  // bf16 operands with the rows in LDS: rotation words (see stage_rot_words);
  // otherwise fp32 (cos, sin) entries
  constexpr bool kWords = C::TR && LDSR;
  typename R::View rv;
  if constexpr (kWords)
    rv = stage_rot_words<D, kRopeLdsEntriesCausal, C::THREADS>(reinterpret_cast<float2*>(smem + HP * C::SMEM), rope,
                                                              G, seg_begin, seg_end);
  else
    rv = rope_view<D, LDSR, kRopeLdsEntriesCausal>(reinterpret_cast<float2*>(smem + HP * C::SMEM), rope, G, seg_begin,
                                                   seg_end);
  GridPos pos;
  pos.set((int)min(seg_begin + (long)tg * TPT, (long)G.N - 1), G.H, G.W);
  const int HW = G.H * G.W;
  const int adt = TT / HW, ady = (TT % HW) / G.W, adx = TT % G.W;

  Raw qr[TPT], kr[TPT], vr[TPT], gr[TPT];
  typename BL::Raw br[TPT];
  auto issue_qkvb = [&](long t0) {
    const __amdgpu_buffer_rsrc_t qs = tile_rsrc(q, t0), ks = tile_rsrc(k, t0), vs = tile_rsrc(v, t0);
    const __amdgpu_buffer_rsrc_t bs = beta_rsrc(t0);
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      qr[i] = BR::load(qs, voff[i], 0);
      kr[i] = BR::load(ks, voff[i], 0);
      vr[i] = BR::load(vs, voff[i], 0);
      br[i] = BL::load(bs, boff[i]);
    }
  };
  auto issue_g = [&](long t0) {
    const __amdgpu_buffer_rsrc_t gs = tile_rsrc(g, t0);
#pragma unroll
    for (int i = 0; i < TPT; ++i) gr[i] = BR::load(gs, voff[i], 0);
  };
  issue_qkvb(seg_begin);
  issue_g(seg_begin);
  if constexpr (LDSR) lds_barrier();

  // operand fragments of the previous tile's state update S^T += RK^T V, kept
  // in registers and issued during the next tile's feature work so that the
  // MFMAs run under vector instructions (zero before the first tile; the last
  // tile's update is not needed: the state after the segment comes from the
  // reduce kernel)
  typename M::frag vb[TT / M::KSTEP], fk[C::MT][TT / M::KSTEP];
#pragma unroll
  for (int ks = 0; ks < TT / M::KSTEP; ++ks) {
    vb[ks] = typename M::frag{};
#pragma unroll
    for (int ct = 0; ct < C::MT; ++ct) fk[ct][ks] = typename M::frag{};
  }

  for (long t0 = seg_begin; t0 < seg_end; t0 += TT) {
    if (mt_wave) {
#pragma unroll
      for (int ks = 0; ks < TT / M::KSTEP; ++ks)
#pragma unroll
        for (int ct = 0; ct < C::MT; ++ct) st[ct] = M::mma(fk[ct][ks], vb[ks], st[ct]);
    }
    // ---- A: token features (row layout), this tile's rows -> LDS ----------
    float phq[TPT][8], rq_scale[TPT], dpz[TPT];
    if (rows) {
      typename R::CS cs[TPT];
      GridPos pp = pos;
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        // rows past the segment end (zero k, v, beta; outputs dropped) take the
        // last staged frame's angles so that every factor stays finite
        cs[i] = R::fetch(rv, cg, min(pp.t, rv.t_lo + rv.nt - 1), pp.y, pp.x);
        pp.next(G.H, G.W);
      }
      if constexpr (C::TR) {
        // bf16 operands: RMS sums, ReLU and rotation on packed bf16 pairs
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
          const int tok = tg * TPT + i;
          uint32_t wa[4], wb[4];   // (cos, -sin), (sin, cos) of pairs 0..3
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if constexpr (kWords) {
              wa[j] = __float_as_uint(cs[i].c[j]);
              wb[j] = __float_as_uint(cs[i].s[j]);
            } else {
              wa[j] = pack2bf(cs[i].c[j], -cs[i].s[j]);
              wb[j] = pack2bf(cs[i].s[j], cs[i].c[j]);
            }
          }
          const u32x4 qw = bf16_words<E>(qr[i]), kw = bf16_words<E>(kr[i]);
          float ssq = dot2bf(qw.x, qw.x, dot2bf(qw.y, qw.y, dot2bf(qw.z, qw.z, dot2bf(qw.w, qw.w, 0.f))));
          float ssk = dot2bf(kw.x, kw.x, dot2bf(kw.y, kw.y, dot2bf(kw.z, kw.z, dot2bf(kw.w, kw.w, 0.f))));
          ssq = group_sum<C::CG>(ssq);
          ssk = group_sum<C::CG>(ssk);
          const float msq = ssq * (1.0f / D) + G.eps;
          rq_scale[i] = msq * __builtin_amdgcn_rsqf(msq);      // r = sqrt(mean(q^2) + eps)
          const float inv = rsqrtf(ssk * (1.0f / D) + G.eps);
          const float bi = BL::value(br[i]) * inv;
          const uint32_t ql[4] = {relu2(qw.x), relu2(qw.y), relu2(qw.z), relu2(qw.w)};
          const uint32_t kl[4] = {relu2(kw.x), relu2(kw.y), relu2(kw.z), relu2(kw.w)};
          float rq[8], rk[8], pk[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            rq[2 * j] = dot2bf(ql[j], wa[j], 0.f);
            rq[2 * j + 1] = dot2bf(ql[j], wb[j], 0.f);
            rk[2 * j] = bi * dot2bf(kl[j], wa[j], 0.f);
            rk[2 * j + 1] = bi * dot2bf(kl[j], wb[j], 0.f);
            phq[i][2 * j] = bf16lo(ql[j]);
            phq[i][2 * j + 1] = bf16hi(ql[j]);
            if constexpr (!C::MD) {
              pk[2 * j] = bf16lo(kl[j]) * inv;                // phi(k^)
              pk[2 * j + 1] = bf16hi(kl[j]) * inv;
            }
          }
          if constexpr (C::MD) {
            // the denominator's part from the key sums before this tile
            float dz = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) dz += phq[i][c] * zr[c];
            dpz[i] = group_sum<C::CG>(dz);
            *reinterpret_cast<u32x4*>(phqs(hl) + tok * C::RP + 8 * cg) = (u32x4){ql[0], ql[1], ql[2], ql[3]};
            // relu(k) as read; the RMS factor is applied in the key-sum products
            *reinterpret_cast<u32x4*>(phks(hl) + tok * C::RPK + 8 * cg) = (u32x4){kl[0], kl[1], kl[2], kl[3]};
            if (cg == 0) invs(hl)[tok] = inv;
          } else {
            float* zrow = zk(hl) + tok * C::FP + 8 * cg;
            *reinterpret_cast<f32x4*>(zrow) = (f32x4){pk[0], pk[1], pk[2], pk[3]};
            *reinterpret_cast<f32x4*>(zrow + 4) = (f32x4){pk[4], pk[5], pk[6], pk[7]};
          }
          *reinterpret_cast<u32x4*>(rqs(hl) + tok * C::RP + 8 * cg) = Elem<bf16_t>::pack(rq);
          *reinterpret_cast<u32x4*>(rks(hl) + tok * C::RPK + 8 * cg) = Elem<bf16_t>::pack(rk);
          *reinterpret_cast<u32x4*>(vT(hl) + tok * C::RPV + 8 * cg) = bf16_words<E>(vr[i]);
        }
      } else {
        // fp32 operands: fp32 features and transposed LDS copies of rk and v
        float kx[TPT][8], vx[TPT][8];
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
          const int tok = tg * TPT + i;
          float qx[8];
          Elem<E>::unpack(qr[i], qx);
          Elem<E>::unpack(kr[i], kx[i]);
          Elem<E>::unpack(vr[i], vx[i]);
          const float bt = BL::value(br[i]);
          float ssq = 0.f, ssk = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            ssq += qx[c] * qx[c];
            ssk += kx[i][c] * kx[i][c];
          }
          ssq = group_sum<C::CG>(ssq);
          ssk = group_sum<C::CG>(ssk);
          const float msq = ssq * (1.0f / D) + G.eps;
          rq_scale[i] = msq * __builtin_amdgcn_rsqf(msq);      // r = sqrt(mean(q^2) + eps)
          const float inv = rsqrtf(ssk * (1.0f / D) + G.eps);
          float rq[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            phq[i][c] = fmaxf(qx[c], 0.f);
            rq[c] = phq[i][c];
            kx[i][c] = fmaxf(kx[i][c] * inv, 0.f);           // phi(k^)
          }
          float* zrow = zk(hl) + tok * C::FP + 8 * cg;
          *reinterpret_cast<f32x4*>(zrow) = (f32x4){kx[i][0], kx[i][1], kx[i][2], kx[i][3]};
          *reinterpret_cast<f32x4*>(zrow + 4) = (f32x4){kx[i][4], kx[i][5], kx[i][6], kx[i][7]};
          R::apply(rq, cs[i]);
          R::apply(kx[i], cs[i]);
#pragma unroll
          for (int c = 0; c < 8; ++c) kx[i][c] *= bt;             // rk
          L* qd = rqs(hl) + tok * C::RP + 8 * cg;
          L* kd = rks(hl) + tok * C::RPK + 8 * cg;
          *reinterpret_cast<f32x4*>(qd) = (f32x4){rq[0], rq[1], rq[2], rq[3]};
          *reinterpret_cast<f32x4*>(qd + 4) = (f32x4){rq[4], rq[5], rq[6], rq[7]};
          *reinterpret_cast<f32x4*>(kd) = (f32x4){kx[i][0], kx[i][1], kx[i][2], kx[i][3]};
          *reinterpret_cast<f32x4*>(kd + 4) = (f32x4){kx[i][4], kx[i][5], kx[i][6], kx[i][7]};
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          store_tcol<L, TPT>(rkT(hl) + (8 * cg + c) * C::CP + tg * TPT, kx, c);
          store_tcol<L, TPT>(vT(hl) + (8 * cg + c) * C::CP + tg * TPT, vx, c);
        }
      }
    }
    pos.advance(adt, ady, adx, G.H, G.W);
    issue_qkvb(t0 + TT);   // the next tile's q, k, v, beta rows (zero past the segment)
    lds_barrier();

    // ---- B: masked intra-tile scores, key sums, inter-tile numerators -------
    if (ww == 0) {
      // AM^T[j][i] = rk_j . rq_i on MFMA (A = RK rows, B = RQ rows), masked, stored as am[i][j]
      f32x16 a = {};
#pragma unroll
      for (int ks = 0; ks < D / M::KSTEP; ++ks) {
        const typename M::frag fa = M::lds_frag(rks(hw) + l32 * C::RPK + ks * M::KSTEP + M::KPL * hi);
        const typename M::frag fb = M::lds_frag(rqs(hw) + l32 * C::RP + ks * M::KSTEP + M::KPL * hi);
        a = M::mma(fa, fb, a);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int j0 = 8 * rb + 4 * hi;
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + r;
          const bool keep = incl ? j <= l32 : j < l32;
          x[r] = keep ? a[4 * rb + r] : 0.f;
        }
        L* dst = am(hw) + l32 * C::CP + j0;
        if constexpr (Elem<L>::is_bf16)
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack2bf(x[0], x[1]), pack2bf(x[2], x[3]));
        else
          *reinterpret_cast<f32x4*>(dst) = (f32x4){x[0], x[1], x[2], x[3]};
      }
    }
    if constexpr (C::MD) {
      if (ww == 1) {
        // intra-tile denominators: P^T[j][i] = phi(k_j) . phi(q_i) on MFMA,
        // each row j times token j's RMS factor (phi(k^_j) = inv_j phi(k_j)),
        // masked like the scores and summed over j (16 registers, then the
        // other lane half through v_permlane32_swap)
        f32x16 a = {};
#pragma unroll
        for (int ks = 0; ks < D / M::KSTEP; ++ks) {
          const typename M::frag fa = M::lds_frag(phks(hw) + l32 * C::RPK + ks * M::KSTEP + M::KPL * hi);
          const typename M::frag fb = M::lds_frag(phqs(hw) + l32 * C::RP + ks * M::KSTEP + M::KPL * hi);
          a = M::mma(fa, fb, a);
        }
        float part = 0.f;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const f32x4 iv = *reinterpret_cast<const f32x4*>(invs(hw) + 8 * rb + 4 * hi);   // rows 8 rb + 4 hi + 0..3
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 8 * rb + 4 * hi + r;
            const bool keep = incl ? j <= l32 : j < l32;
            part += keep ? a[4 * rb + r] * iv[r] : 0.f;
          }
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
        if (hi == 0) dins(hw)[l32] = part + __uint_as_float(sw[1]);
      } else if (ww == 2) {
        // the tile's key sums per channel: (RMS factors) x phi(K) on MFMA,
        // sum over j of inv_j phi(k_j) = phi(k^_j) (every row of the product
        // holds the column sums)
        typename M::frag fi[TT / M::KSTEP];   // A[m][k = token 16 ks + 8 hi + e] = inv of that token, bf16
#pragma unroll
        for (int ks = 0; ks < TT / M::KSTEP; ++ks) {
          const f32x4 ia = *reinterpret_cast<const f32x4*>(invs(hw) + ks * M::KSTEP + M::KPL * hi);
          const f32x4 ib = *reinterpret_cast<const f32x4*>(invs(hw) + ks * M::KSTEP + M::KPL * hi + 4);
          const float iv[8] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
          fi[ks] = M::from_f32(iv);
        }
#pragma unroll
        for (int ct = 0; ct < C::MT; ++ct) {
          f32x16 a = {};
#pragma unroll
          for (int ks = 0; ks < TT / M::KSTEP; ++ks)
            a = M::mma(fi[ks], tr_frag(phks(hw), C::RPK, ks * M::KSTEP, 32 * ct, lane), a);
          if (hi == 0) zsum(hw)[32 * ct + l32] = a[0];
        }
      }
    }
    if (scanner) {
      // running key sums z_i of this tile's tokens (inclusive or exclusive of
      // token i): a 16-token prefix per lane half, the lower half's total
      // handed to the upper half with v_permlane32_swap
      constexpr int HT = TT / 2;
      float* zcol = zk(hw) + zc + HT * hi * C::FP;
      float p[HT];
#pragma unroll
      for (int j = 0; j < HT; ++j) p[j] = zcol[j * C::FP];
#pragma unroll
      for (int j = 1; j < HT; ++j) p[j] += p[j - 1];
      const float tot = p[HT - 1];
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tot), __float_as_uint(tot), false, false);
      const float lower = __uint_as_float(sw[0]);   // upper lanes: the lower half's total
      const float upper = __uint_as_float(sw[1]);   // lower lanes: the upper half's total
      const float base = hi ? zrun + lower : zrun;
      if (incl) {
#pragma unroll
        for (int j = 0; j < HT; ++j) zcol[j * C::FP] = base + p[j];
      } else {
        zcol[0] = base;
#pragma unroll
        for (int j = 1; j < HT; ++j) zcol[j * C::FP] = base + p[j - 1];
      }
      zrun += hi ? lower + tot : tot + upper;   // the same sum, in the same order, in both halves
    }
    f32x16 n = {};   // num^T of this wave's v tile
    if (mt_wave) {
      // inter-tile numerators: the state before this tile, as operand
      // fragments, times RQ^T (independent of the scores, so issued here)
#pragma unroll
      for (int ct = 0; ct < C::MT; ++ct)
#pragma unroll
        for (int s = 0; s < PF::STEPS; ++s)
          n = M::mma(PF::acc(st[ct], s), PF::row(rqs(hw) + l32 * C::RP + 32 * ct, s, hi), n);
      // this tile's S^T += RK^T V operands: A = rk^T[c][j], B = v[j][v] (this wave's v columns)
#pragma unroll
      for (int ks = 0; ks < TT / M::KSTEP; ++ks) {
        if constexpr (C::TR) vb[ks] = tr_frag(vT(hw), C::RPV, ks * M::KSTEP, 32 * ww, lane);
        else vb[ks] = M::lds_frag(vT(hw) + (32 * ww + l32) * C::CP + ks * M::KSTEP + M::KPL * hi);
#pragma unroll
        for (int ct = 0; ct < C::MT; ++ct) {
          if constexpr (C::TR) fk[ct][ks] = tr_frag(rks(hw), C::RPK, ks * M::KSTEP, 32 * ct, lane);
          else fk[ct][ks] = M::lds_frag(rkT(hw) + (32 * ct + l32) * C::CP + ks * M::KSTEP + M::KPL * hi);
        }
      }
    }
    // the gate sigmoid(g) of this tile's rows, computed here where the vector
    // unit would otherwise wait on the numerator MFMAs; the g registers are
    // then free for the next tile's rows
    float sig[TPT][8];
    if (rows) {
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        float gv[8];
        Elem<E>::unpack(gr[i], gv);
#pragma unroll
        for (int c = 0; c < 8; ++c) sig[i][c] = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[c]));
      }
    }
    issue_g(t0 + TT);
    lds_barrier();

    // ---- C: intra-tile numerators on MFMA, denominators ----------------------
    if (mt_wave) {
#pragma unroll
      for (int ks = 0; ks < TT / M::KSTEP; ++ks)
        n = M::mma(vb[ks], M::lds_frag(am(hw) + l32 * C::CP + ks * M::KSTEP + M::KPL * hi), n);
      float* row = nums(hw) + l32 * C::FP + 32 * ww + 4 * hi;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        *reinterpret_cast<f32x4*>(row + 8 * rb) = (f32x4){n[4 * rb], n[4 * rb + 1], n[4 * rb + 2], n[4 * rb + 3]};
    }
    float den[TPT];
    if (rows) {
      if constexpr (C::MD) {
#pragma unroll
        for (int i = 0; i < TPT; ++i)
          den[i] = dpz[i] + dins(hl)[tg * TPT + i] + G.eps * rq_scale[i];
        // running key sums after this tile
        const f32x4 za = *reinterpret_cast<const f32x4*>(zsum(hl) + 8 * cg);
        const f32x4 zb = *reinterpret_cast<const f32x4*>(zsum(hl) + 8 * cg + 4);
        zr[0] += za.x; zr[1] += za.y; zr[2] += za.z; zr[3] += za.w;
        zr[4] += zb.x; zr[5] += zb.y; zr[6] += zb.z; zr[7] += zb.w;
      } else {
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
          const float* zrow = zk(hl) + (tg * TPT + i) * C::FP + 8 * cg;
          const f32x4 za = *reinterpret_cast<const f32x4*>(zrow);
          const f32x4 zb = *reinterpret_cast<const f32x4*>(zrow + 4);
          float dp = phq[i][0] * za.x + phq[i][1] * za.y + phq[i][2] * za.z + phq[i][3] * za.w +
                     phq[i][4] * zb.x + phq[i][5] * zb.y + phq[i][6] * zb.z + phq[i][7] * zb.w;
          dp = group_sum<C::CG>(dp);
          den[i] = dp + G.eps * rq_scale[i];
        }
      }
    }
    lds_barrier();

    // ---- D: gate, RMSNorm, store --------------------------------------------
    if (rows) {
      const __amdgpu_buffer_rsrc_t ors = tile_rsrc(out, t0);
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const float* src = nums(hl) + (tg * TPT + i) * C::FP + 8 * cg;
        const f32x4 a = *reinterpret_cast<const f32x4*>(src);
        const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
        float y[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          y[c] *= sig[i][c];
          ss += y[c] * y[c];
        }
        ss = group_sum<C::CG>(ss);
        const float scale = out_scale(ss * (1.0f / D), den[i], G.eps);
#pragma unroll
        for (int c = 0; c < 8; ++c) y[c] = wc[c] * y[c] * scale;
        BR::store(ors, voff[i], 0, Elem<E>::pack(y));
      }
    }
  }
}

template <int D, typename E, int HP>
static void launch_token_causal_hp(const LaunchArgs& a) {
  const Geometry& G = a.geo;
  const int blocks = (G.heads / HP) * G.nseg;
  const int threads = CausalCfg<D, E, HP>::THREADS;
  if (G.rope_lds2)
    hipLaunchKernelGGL((token_causal_kernel<D, E, HP, true>), dim3(blocks), dim3(threads), 0, a.stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.beta, (const E*)a.g,
                       (const float*)a.states, a.rms_w, (const float2*)a.rope, (E*)a.out, G);
  else
    hipLaunchKernelGGL((token_causal_kernel<D, E, HP, false>), dim3(blocks), dim3(threads), 0, a.stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, (const E*)a.beta, (const E*)a.g,
                       (const float*)a.states, a.rms_w, (const float2*)a.rope, (E*)a.out, G);
}

template <int D, typename E>
hipError_t launch_token_causal(const LaunchArgs& a) {
  if constexpr (D == 128 && Elem<typename Elem<E>::Lds>::is_bf16) {
    if (a.geo.pass2_pair) {   // the planner sets it only for an even head count
      launch_token_causal_hp<D, E, 2>(a);
      return hipGetLastError();
    }
  }
  launch_token_causal_hp<D, E, 1>(a);
  return hipGetLastError();
}

template hipError_t launch_token_causal<32, float>(const LaunchArgs&);
template hipError_t launch_token_causal<64, float>(const LaunchArgs&);
template hipError_t launch_token_causal<128, float>(const LaunchArgs&);
template hipError_t launch_token_causal<32, bf16_t>(const LaunchArgs&);
template hipError_t launch_token_causal<64, bf16_t>(const LaunchArgs&);
template hipError_t launch_token_causal<128, bf16_t>(const LaunchArgs&);
template hipError_t launch_token_causal<32, fp8_t>(const LaunchArgs&);
template hipError_t launch_token_causal<64, fp8_t>(const LaunchArgs&);
template hipError_t launch_token_causal<128, fp8_t>(const LaunchArgs&);
template hipError_t launch_token_causal<32, bf8_t>(const LaunchArgs&);
template hipError_t launch_token_causal<64, bf8_t>(const LaunchArgs&);
template hipError_t launch_token_causal<128, bf8_t>(const LaunchArgs&);

}  // namespace gla
