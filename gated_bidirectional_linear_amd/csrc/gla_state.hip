// Pass 1: per-chunk partial states S_p = V_p^T (beta R phi K^)_p and key sums.
#include "gla_common.h"

namespace gla {

// ===========================================================================
// 2. State partials: S_p = V_p^T (beta R phi K^)_p and z_p = sum phi K^
// ===========================================================================
template <int D, typename E>
struct PartialCfg {
  static constexpr int CG = D / 8;                 // threads per token (8 channels each)
  static constexpr int TG = kThreads / CG;         // token groups
  static constexpr int TPT = kTile / TG;           // tokens per thread per tile
  static constexpr int MT = D / 32;                // 32-row MFMA tiles per dim
  static constexpr bool KSPLIT = MT * MT < 4;      // too few output tiles: waves split K
  static constexpr int TPW = KSPLIT ? 1 : MT * MT / 4;   // output tiles per wave
  static constexpr int PITCH = kTile + (Elem<E>::is_bf16 ? 8 : 2);  // LDS row pitch (elements)
  static constexpr int STAGE_BYTES = 2 * D * PITCH * (int)sizeof(E);
  static constexpr int ZRED_BYTES = TG * D * 4;
  static constexpr int KRED_BYTES = KSPLIT ? 4 * 64 * 16 * 4 : 0;
  static constexpr int SMEM = STAGE_BYTES > ZRED_BYTES ? (STAGE_BYTES > KRED_BYTES ? STAGE_BYTES : KRED_BYTES)
                                                       : (ZRED_BYTES > KRED_BYTES ? ZRED_BYTES : KRED_BYTES);
};

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

template <int D, typename E, bool LDSR>
__global__ __launch_bounds__(kThreads) void state_partial_kernel(
    const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ beta,
    const float2* __restrict__ rope, float* __restrict__ partial, Geometry G) {
  using C = PartialCfg<D, E>;
  using M = Mfma<E>;
  constexpr int ROPE_BYTES = LDSR ? kRopeLdsEntries * 8 : 0;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM + ROPE_BYTES];
  E* rkT = reinterpret_cast<E*>(smem);          // [D][PITCH]  (k channel, token)
  E* vT = rkT + D * C::PITCH;                   // [D][PITCH]  (v channel, token)

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
  const typename Rope<D>::View rv =
      rope_view<D, LDSR>(reinterpret_cast<float2*>(smem + C::SMEM), rope, G, ch.begin, ch.end);
  if (ch.begin < ch.end) issue(ch.begin);
  if constexpr (LDSR) lds_barrier();

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
      store_tcol<E, C::TPT>(rkT + (8 * cg + c) * C::PITCH + col, kx, c);
      store_tcol<E, C::TPT>(vT + (8 * cg + c) * C::PITCH + col, vx, c);
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
// Fragment-built pass 1 (bf16, d = 128).
//
// A workgroup of 4 waves walks its chunk in 64-token tiles; wave w loads and
// prepares the 16-token step w of every tile.  Lane l of a wave owns channels
// 4m..4m+3 (m = l % 32) of 8 tokens; lanes 0-31 and 32-63 (h = l / 32) take
// the two halves of the step.  Every row load is 8 bytes per lane and 32 lanes
// cover a whole 256-byte token row (two full rows per load instruction).
// Channel 4m + c is row/column m of MFMA tile c, so the 32x32x16 MFMA
// operand fragments are built in registers: the k-side fragment of tile c
// packs channel c of the lane's 8 tokens with v_cvt_pk_bf16_f32, the v-side
// fragment selects the same 16-bit halves from the raw rows with v_perm_b32.
// The 8 fragments of each step go to LDS in lane order (16-byte, conflict-free
// writes); after a barrier, wave w accumulates the 4 output tiles
// S[4m + w][4n + c] over the tile's 4 steps (16 MFMAs).  One fragment buffer
// (two barriers per tile) keeps LDS at 48 KB for three workgroups per CU.  Rows are read with raw buffer
// loads (wave-uniform token offset + one per-lane offset; tensors below
// 2 GiB, checked by the host); rows past the sequence read as zero, rows past
// the chunk are masked.
// ===========================================================================
namespace frag1 {
constexpr int kStep = 16;    // tokens per step (one MFMA K)
constexpr int kFragBytes = 64 * 16;            // one fragment for a wave
constexpr int kStepBytes = 8 * kFragBytes;     // 4 k-side + 4 v-side fragments
constexpr int kTileBytes = 4 * kStepBytes;     // the 4 steps of a tile

struct Rows {
  u32x2 k[8], v[8];
  uint32_t b;               // beta (bf16 bits) of token base + (lane & 15)
};

// bf16 pair (lo: token a, hi: token b) of channel c from two raw 4-channel rows
__device__ __forceinline__ uint32_t sel_channel(u32x2 ra, u32x2 rb, int c) {
  const uint32_t wa = (c < 2) ? ra.x : ra.y;
  const uint32_t wb = (c < 2) ? rb.x : rb.y;
  // v_perm_b32 dst = bytes of {wb:wa} picked by the selector (byte 0-3 = wa)
  return (c & 1) ? __builtin_amdgcn_perm(wb, wa, 0x07060302u) : __builtin_amdgcn_perm(wb, wa, 0x05040100u);
}

// Raw buffer resource over a whole tensor (gfx9 descriptor word 3): loads at
// offsets past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tensor_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}
}  // namespace frag1

template <bool LDSR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void state_partial_frag_kernel(
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const bf16_t* __restrict__ beta,
    const float2* __restrict__ rope, float* __restrict__ partial, Geometry G) {
  constexpr int D = 128;
  using namespace frag1;
  using R = Rope<D>;
  constexpr int ROPE_BYTES = LDSR ? kRopeLdsEntries * 8 : 0;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kTileBytes + ROPE_BYTES];

  const int lin = xcd_swizzle(blockIdx.x, gridDim.x);
  const Chunk ch = chunk_of(lin, G, G.cps1, G.chunk1);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int m = lane & 31;
  const int h = lane >> 5;
  const int HW = G.H * G.W;
  const uint32_t ROW = (uint32_t)G.heads * D * 2;          // bytes between tokens
  const __amdgpu_buffer_rsrc_t krs = tensor_rsrc(k, (uint32_t)G.N * ROW);
  const __amdgpu_buffer_rsrc_t vrs = tensor_rsrc(v, (uint32_t)G.N * ROW);
  const __amdgpu_buffer_rsrc_t brs = tensor_rsrc(beta, (uint32_t)G.N * G.heads * 2);
  const uint32_t lane_off = (uint32_t)(8 * h) * ROW + (uint32_t)ch.head * D * 2 + 8u * m;
  const uint32_t beta_off = ((uint32_t)(lane & 15) * (uint32_t)G.heads + (uint32_t)ch.head) * 2;

  // this lane's RoPE axis (pairs 2m and 2m+1 share it)
  const int axis = (2 * m < R::PT) ? 0 : ((2 * m < R::PT + R::PY) ? 1 : 2);
  const typename R::View rv = rope_view<D, LDSR>(reinterpret_cast<float2*>(smem + kTileBytes), rope, G,
                                                 ch.begin, ch.end);
  const int rbase = axis == 0 ? 2 * m - rv.t_lo * R::PT
                  : (axis == 1 ? rv.nt * R::PT + (2 * m - R::PT) : rv.nt * R::PT + rv.H * R::PY + (2 * m - R::PT - R::PY));
  const int rstride = axis == 0 ? R::PT : (axis == 1 ? R::PY : R::PX);

  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  float zacc[4] = {0.f, 0.f, 0.f, 0.f};

  auto issue = [&](Rows& r, long base) {
    const uint32_t b = (uint32_t)base;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      r.k[i] = ld8(krs, lane_off, (b + i) * ROW);
      r.v[i] = ld8(vrs, lane_off, (b + i) * ROW);
    }
    r.b = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(brs, (int)beta_off, (int)(b * (uint32_t)G.heads * 2), 0);
  };

  // Build this lane's 8 fragments of the step starting at `base` and store
  // them to LDS at `dst` (lane order).
  auto prepare = [&](const Rows& r, long base, unsigned char* dst) {
    const long n0 = base + 8 * h;
    const int bsrc = (int)(r.b << 16);
    const int nc = (int)min(n0, (long)G.N - 1);
    int tt = nc / HW;
    const int rem = nc - tt * HW;
    int yy = rem / G.W;
    int xx = rem - yy * G.W;
    const bool full = base + kStep <= ch.end;   // wave-uniform
    // The k-side RMS scale rides on the per-token factor: with
    // inv = 1/sqrt(mean(k^2) + eps), phi(k inv) = inv phi(k), so
    // rk = (beta inv) R phi(k) and the key sum adds inv phi(k).
    uint32_t kp[4][4];   // [channel slot c][token pair]
#pragma unroll
    for (int ip = 0; ip < 4; ++ip) {
      float rk2[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = 2 * ip + j;
        float ss = dot2sq(r.k[i].x, dot2sq(r.k[i].y, 0.f));
        ss = group_sum<16>(ss);
        ss += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(ss), 0x401F));  // lane ^ 16
        const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + G.eps);
        // beta of token base + 8h + i lives in lane 8h + i
        const float bt = __int_as_float(__builtin_amdgcn_ds_bpermute((8 * h + i) * 4, bsrc));
        const float keep = (full || n0 + i < ch.end) ? inv : 0.f;
        const uint32_t p01 = relu2(r.k[i].x), p23 = relu2(r.k[i].y);
        const float ph[4] = {bf16lo(p01), bf16hi(p01), bf16lo(p23), bf16hi(p23)};
#pragma unroll
        for (int c = 0; c < 4; ++c) zacc[c] += ph[c] * keep;
        const float sc = bt * keep;
        const int pos = axis == 0 ? tt : (axis == 1 ? yy : xx);
        const f32x4 cs = *reinterpret_cast<const f32x4*>(rv.tab + rbase + pos * rstride);
        rk2[j][0] = sc * (ph[0] * cs.x - ph[1] * cs.y);
        rk2[j][1] = sc * (ph[0] * cs.y + ph[1] * cs.x);
        rk2[j][2] = sc * (ph[2] * cs.z - ph[3] * cs.w);
        rk2[j][3] = sc * (ph[2] * cs.w + ph[3] * cs.z);
        ++xx;
        const bool wy = xx == G.W;
        xx = wy ? 0 : xx;
        yy += wy ? 1 : 0;
        const bool wt = yy == G.H;
        yy = wt ? 0 : yy;
        tt += wt ? 1 : 0;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) kp[c][ip] = pack2bf(rk2[0][c], rk2[1][c]);
    }
    // v rows past the chunk are zeroed so they cannot reach the state
    uint32_t vmask[4];
#pragma unroll
    for (int ip = 0; ip < 4; ++ip) {
      const bool v0 = full || n0 + 2 * ip < ch.end;
      const bool v1 = full || n0 + 2 * ip + 1 < ch.end;
      vmask[ip] = (v0 ? 0x0000ffffu : 0u) | (v1 ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 ku = {kp[c][0], kp[c][1], kp[c][2], kp[c][3]};
      const u32x4 vu = {sel_channel(r.v[0], r.v[1], c) & vmask[0], sel_channel(r.v[2], r.v[3], c) & vmask[1],
                        sel_channel(r.v[4], r.v[5], c) & vmask[2], sel_channel(r.v[6], r.v[7], c) & vmask[3]};
      *reinterpret_cast<u32x4*>(dst + c * kFragBytes + lane * 16) = ku;
      *reinterpret_cast<u32x4*>(dst + (4 + c) * kFragBytes + lane * 16) = vu;
    }
  };

  if constexpr (LDSR) lds_barrier();   // RoPE rows staged
  Rows rows;
  if (ch.begin < ch.end) issue(rows, ch.begin + wave * kStep);
  for (long t0 = ch.begin; t0 < ch.end; t0 += kTile) {
    unsigned char* tile = smem;
    if (t0 != ch.begin) lds_barrier();   // every wave is done with the previous tile's fragments
    const long base = t0 + wave * kStep;
    if (base < ch.end) {
      const Rows cur = rows;
      if (t0 + kTile < ch.end) issue(rows, base + kTile);   // prefetch this wave's next step
      prepare(cur, base, tile + wave * kStepBytes);
    } else {
      if (t0 + kTile < ch.end) issue(rows, base + kTile);
      // a step wholly past the chunk contributes nothing
#pragma unroll
      for (int f = 0; f < 8; ++f)
        *reinterpret_cast<u32x4*>(tile + wave * kStepBytes + f * kFragBytes + lane * 16) = (u32x4){0u, 0u, 0u, 0u};
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned char* st = tile + j * kStepBytes;
      const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + (4 + wave) * kFragBytes + lane * 16));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + c * kFragBytes + lane * 16));
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
      }
    }
  }

  // key sums: lanes m and m + 32 hold the same channels; then across waves
  float* zred = reinterpret_cast<float*>(smem);   // [4 waves][128]
  lds_barrier();
#pragma unroll
  for (int c = 0; c < 4; ++c) zacc[c] += __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) * 4, __float_as_int(zacc[c])));
  if (h == 0) *reinterpret_cast<f32x4*>(zred + wave * 128 + 4 * m) = (f32x4){zacc[0], zacc[1], zacc[2], zacc[3]};
  lds_barrier();
  float* dst = partial + ((size_t)ch.head * G.nseg * G.cps1 + ch.index) * (size_t)(D * D + D);
  if (wave == 0 && lane < 32) {
    f32x4 zz = *reinterpret_cast<const f32x4*>(zred + 4 * m);
#pragma unroll
    for (int wv = 1; wv < 4; ++wv) {
      const f32x4 o = *reinterpret_cast<const f32x4*>(zred + wv * 128 + 4 * m);
      zz.x += o.x; zz.y += o.y; zz.z += o.z; zz.w += o.w;
    }
    *reinterpret_cast<f32x4*>(dst + D * D + 4 * m) = zz;
  }
  // S[4 mr + wave][4 n + c] with mr = 8(r/4) + 4h + r%4, n = lane % 32
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int mr = 8 * (r >> 2) + 4 * h + (r & 3);
    *reinterpret_cast<f32x4*>(dst + (4 * mr + wave) * D + 4 * m) = (f32x4){acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
  }
}

template <int D, typename E>
hipError_t launch_state_partial(const LaunchArgs& a) {
  const Geometry& G = a.geo;
  const int blocks = G.heads * G.nseg * G.cps1;
  if constexpr (D == 128 && Elem<E>::is_bf16) {
    if (G.pass1_reg) {
      if (G.rope_lds1)
        hipLaunchKernelGGL((state_partial_frag_kernel<true>), dim3(blocks), dim3(kThreads), 0, a.stream,
                           (const bf16_t*)a.k, (const bf16_t*)a.v, (const bf16_t*)a.beta, (const float2*)a.rope,
                           a.partial, G);
      else
        hipLaunchKernelGGL((state_partial_frag_kernel<false>), dim3(blocks), dim3(kThreads), 0, a.stream,
                           (const bf16_t*)a.k, (const bf16_t*)a.v, (const bf16_t*)a.beta, (const float2*)a.rope,
                           a.partial, G);
      return hipGetLastError();
    }
  }
  if (G.rope_lds1)
    hipLaunchKernelGGL((state_partial_kernel<D, E, true>), dim3(blocks), dim3(kThreads), 0, a.stream,
                       (const E*)a.k, (const E*)a.v, (const E*)a.beta, (const float2*)a.rope, a.partial, G);
  else
    hipLaunchKernelGGL((state_partial_kernel<D, E, false>), dim3(blocks), dim3(kThreads), 0, a.stream,
                       (const E*)a.k, (const E*)a.v, (const E*)a.beta, (const float2*)a.rope, a.partial, G);
  return hipGetLastError();
}

template hipError_t launch_state_partial<32, float>(const LaunchArgs&);
template hipError_t launch_state_partial<64, float>(const LaunchArgs&);
template hipError_t launch_state_partial<128, float>(const LaunchArgs&);
template hipError_t launch_state_partial<32, bf16_t>(const LaunchArgs&);
template hipError_t launch_state_partial<64, bf16_t>(const LaunchArgs&);
template hipError_t launch_state_partial<128, bf16_t>(const LaunchArgs&);

}  // namespace gla
