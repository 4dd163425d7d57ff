// HIP kernels (gfx950) of the gated bidirectional ReLU linear-attention operator.
//
// Per head, with q^ = q/rms(q), k^ = k/rms(k), phi = ReLU, R_n the 3D RoPE
// rotation of token n (SANA-Video 2.0 digest, prelims "gated bilinear linear
// attention"; SANA-Video notes, key design 1 and 2):
//   S = sum_n beta_n v_n (R_n phi k^_n)^T,   z = sum_n phi k^_n
//   o_j = w * rmsnorm( sigmoid(g_j) * (S R_j phi q^_j) / (phi q^_j . z + eps) )
//
// The tokens are cut into "segments": one segment of N tokens for the
// bidirectional form, or one per block of latent frames for the block-causal
// form.  Four launches on the caller's stream:
//   1. rope_table_kernel   : per-axis cos/sin tables (angles in fp64).
//   2. state_partial_kernel: one workgroup per (head, chunk of a segment);
//      streams k, v, beta through LDS and builds the partial V^T (beta R phi K)
//      on MFMA (fp32 accumulation) plus the partial key sum.
//   3. state_reduce_kernel : fixed-shape pairwise tree over the chunk partials
//      of each segment, then an inclusive prefix over segments on top of the
//      carried state (block-causal) -> per-segment states.
//   4. output_kernel       : one workgroup per (head, chunk of tiles); holds
//      its slice of S as MFMA A-fragments in registers, streams q and g,
//      computes num^T = S RQ^T on MFMA, the denominator, gate and RMSNorm,
//      and writes the output once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_device.h"
#include "gla_launch.h"

namespace gla {

// ===========================================================================
// 1. RoPE tables
// ===========================================================================
template <int D>
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ tab, int T, int H, int W) {
  using R = Rope<D>;
  const long total = (long)T * R::PT + (long)H * R::PY + (long)W * R::PX;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  long pos, i;
  int da;
  if (idx < (long)T * R::PT) {
    pos = idx / R::PT; i = idx % R::PT; da = D / 4;
  } else if (idx < (long)T * R::PT + (long)H * R::PY) {
    const long r = idx - (long)T * R::PT;
    pos = r / R::PY; i = r % R::PY; da = 3 * D / 8;
  } else {
    const long r = idx - (long)T * R::PT - (long)H * R::PY;
    pos = r / R::PX; i = r % R::PX; da = 3 * D / 8;
  }
  const double ang = (double)pos * pow(10000.0, -2.0 * (double)i / (double)da);
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

// ===========================================================================
// Chunk geometry shared by the kernels (all integer arithmetic, no tables)
// ===========================================================================
struct Chunk {
  long begin, end;  // token range [begin, end)
  int head, seg, index;
};

__device__ __forceinline__ Chunk chunk_of(int lin, const Geometry& G, int cps, int chunk_len) {
  Chunk c;
  const int per_head = G.nseg * cps;
  c.head = lin / per_head;
  const int ci = lin - c.head * per_head;
  c.seg = ci / cps;
  c.index = ci;
  const int j = ci - c.seg * cps;
  const long s0 = (long)c.seg * G.seg_len;
  const long s1 = min(s0 + (long)G.seg_len, (long)G.N);
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

// Stage the RoPE rows of the frames a chunk spans (or use the global table).
template <int D, bool LDSR>
__device__ __forceinline__ typename Rope<D>::View rope_view(float2* lds, const float2* __restrict__ rope,
                                                            const Geometry& G, long begin, long end) {
  if constexpr (LDSR) {
    const int HW = G.H * G.W;
    const int t_lo = begin < end ? (int)(begin / HW) : 0;
    const int nt = begin < end ? (int)((end - 1) / HW) - t_lo + 1 : 0;
    return Rope<D>::template stage<kRopeLdsEntries>(lds, rope, G.T, G.H, G.W, t_lo, nt);
  } else {
    return typename Rope<D>::View{rope, 0, G.T, G.H};
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
// 3. Reduce chunk partials per segment (pairwise tree of fixed shape), then
//    inclusive prefix over segments on top of the carried state.
// ===========================================================================
template <int D>
__global__ __launch_bounds__(256) void state_reduce_kernel(const float* __restrict__ partial,
                                                           const float* S_in, const float* z_in,
                                                           float* __restrict__ states, float* S_out,
                                                           float* z_out, Geometry G) {
  constexpr int SZ = D * D + D;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int h = blockIdx.y;
  if (e >= SZ) return;
  float running = 0.f;
  if (S_in != nullptr) running = (e < D * D) ? S_in[(size_t)h * D * D + e] : z_in[(size_t)h * D + (e - D * D)];
  const float* src = partial + (size_t)h * G.nseg * G.cps1 * SZ + e;
  for (int s = 0; s < G.nseg; ++s) {
    float v[kMaxChunks];
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) v[i] = (i < G.cps1) ? src[(size_t)(s * G.cps1 + i) * SZ] : 0.f;
#pragma unroll
    for (int w = kMaxChunks / 2; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) v[i] += v[i + w];
    running += v[0];
    states[((size_t)s * G.heads + h) * SZ + e] = running;
  }
  if (S_out != nullptr) {
    if (e < D * D) S_out[(size_t)h * D * D + e] = running;
    else z_out[(size_t)h * D + (e - D * D)] = running;
  }
}

// ===========================================================================
// 4. Fused output
// ===========================================================================
template <int D, typename E>
struct OutputCfg {
  static constexpr int CG = D / 8;
  static constexpr int TG = kThreads / CG;
  static constexpr int TPT = kTile / TG;
  static constexpr int MT = D / 32;                 // v-channel tiles
  static constexpr int NTK = kTile / 32;            // token tiles
  static constexpr int PAIRS = MT * NTK;
  static constexpr int PPW = PAIRS >= 4 ? PAIRS / 4 : 1;   // (v tile, token tile) pairs per wave
  static constexpr int ACTIVE = PAIRS >= 4 ? 4 : PAIRS;    // waves with MFMA work
  static constexpr int RQ_PITCH = D + (Elem<E>::is_bf16 ? 8 : 4);  // elements
  static constexpr int NUM_PITCH = D + 4;                           // floats
  static constexpr int RQ_BYTES = kTile * RQ_PITCH * (int)sizeof(E);
  static constexpr int NUM_BYTES = kTile * NUM_PITCH * 4;
  static constexpr int SMEM = RQ_BYTES > NUM_BYTES ? RQ_BYTES : NUM_BYTES;
};

template <int D, typename E, bool LDSR>
__global__ __launch_bounds__(kThreads) void output_kernel(
    const E* __restrict__ q, const E* __restrict__ g, const float* __restrict__ states,
    const float* __restrict__ rms_w, const float2* __restrict__ rope, E* __restrict__ out, Geometry G) {
  using C = OutputCfg<D, E>;
  using M = Mfma<E>;
  constexpr int KSTEPS = D / M::KSTEP;
  constexpr int SZ = D * D + D;
  constexpr int ROPE_BYTES = LDSR ? kRopeLdsEntries * 8 : 0;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM + ROPE_BYTES];
  E* rqs = reinterpret_cast<E*>(smem);            // [kTile][RQ_PITCH]  (token, k channel)
  float* nums = reinterpret_cast<float*>(smem);   // [kTile][NUM_PITCH] (token, v channel)

  const int lin = xcd_swizzle(blockIdx.x, gridDim.x);
  const Chunk ch = chunk_of(lin, G, G.cps2, G.chunk2);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cg = tid % C::CG;
  const int tg = tid / C::CG;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int HW = G.H * G.W;

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

  typename Elem<E>::Raw qr[C::TPT], gr[C::TPT];
  auto issue = [&](long t0) {
    const long n0 = t0 + (long)tg * C::TPT;
    issue_rows<D, E, C::TPT>(q, n0, ch.end, G.heads, ch.head, cg, qr);
    issue_rows<D, E, C::TPT>(g, n0, ch.end, G.heads, ch.head, cg, gr);
  };
  const typename Rope<D>::View rv =
      rope_view<D, LDSR>(reinterpret_cast<float2*>(smem + C::SMEM), rope, G, ch.begin, ch.end);
  if (ch.begin < ch.end) issue(ch.begin);
  if constexpr (LDSR) lds_barrier();

  for (long t0 = ch.begin; t0 < ch.end; t0 += kTile) {
    const long n0 = t0 + (long)tg * C::TPT;
    float qx[C::TPT][8], gx[C::TPT][8];
    float rden[C::TPT];
    unpack_rows<E, C::TPT>(qr, n0, ch.end, qx);
    unpack_rows<E, C::TPT>(gr, n0, ch.end, gx);
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
      for (int c = 0; c < 8; ++c) ss += qx[i][c] * qx[i][c];
      ss = group_sum<C::CG>(ss);
      const float inv = rsqrtf(ss * (1.0f / D) + G.eps);
      float dp = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float p = fmaxf(qx[i][c] * inv, 0.f);
        qx[i][c] = p;
        dp += p * zc[c];
      }
      dp = group_sum<C::CG>(dp);
      rden[i] = 1.0f / (dp + G.eps);
      Rope<D>::apply(qx[i], cs[i]);
      E* dst = rqs + (tg * C::TPT + i) * C::RQ_PITCH + 8 * cg;
      if constexpr (Elem<E>::is_bf16) {
        uint4 u;
        u.x = pack2bf(qx[i][0], qx[i][1]); u.y = pack2bf(qx[i][2], qx[i][3]);
        u.z = pack2bf(qx[i][4], qx[i][5]); u.w = pack2bf(qx[i][6], qx[i][7]);
        *reinterpret_cast<uint4*>(dst) = u;
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(qx[i][0], qx[i][1], qx[i][2], qx[i][3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(qx[i][4], qx[i][5], qx[i][6], qx[i][7]);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) gx[i][c] = 1.0f / (1.0f + __expf(-gx[i][c]));
    }
    lds_barrier();

    f32x16 acc[C::PPW];
    if (wave < C::ACTIVE) {
#pragma unroll
      for (int u = 0; u < C::PPW; ++u) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;
        const int ntt = (wave * C::PPW + u) % C::NTK;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const typename M::frag b = M::lds_frag(rqs + (32 * ntt + l32) * C::RQ_PITCH + ks * M::KSTEP + M::KPL * hi);
          acc[u] = M::mma(sfrag[ks], b, acc[u]);
        }
      }
    }
    lds_barrier();
    if (wave < C::ACTIVE) {
#pragma unroll
      for (int u = 0; u < C::PPW; ++u) {
        const int ntt = (wave * C::PPW + u) % C::NTK;
        float* row = nums + (32 * ntt + l32) * C::NUM_PITCH + 32 * dvt + 4 * hi;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          *reinterpret_cast<float4*>(row + 8 * rb) =
              make_float4(acc[u][4 * rb], acc[u][4 * rb + 1], acc[u][4 * rb + 2], acc[u][4 * rb + 3]);
      }
    }
    lds_barrier();

#pragma unroll
    for (int i = 0; i < C::TPT; ++i) {
      const float* src = nums + (tg * C::TPT + i) * C::NUM_PITCH + 8 * cg;
      const float4 a = *reinterpret_cast<const float4*>(src);
      const float4 b = *reinterpret_cast<const float4*>(src + 4);
      float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        x[c] = gx[i][c] * x[c] * rden[i];
        ss += x[c] * x[c];
      }
      ss = group_sum<C::CG>(ss);
      const float inv = rsqrtf(ss * (1.0f / D) + G.eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) x[c] = wc[c] * x[c] * inv;
      const long n = n0 + i;
      if (n < ch.end) Elem<E>::store8(out + ((size_t)n * G.heads + ch.head) * D + 8 * cg, x);
    }
    lds_barrier();
  }
}

// ===========================================================================
// Host-side launchers
// ===========================================================================
template <int D, typename E>
static hipError_t launch_all(const LaunchArgs& a, Timer& tm) {
  const Geometry& G = a.geo;
  hipStream_t st = a.stream;
  {
    const long total = (long)G.T * (D / 8) + (long)G.H * (3 * D / 16) + (long)G.W * (3 * D / 16);
    const int blocks = (int)((total + 255) / 256);
    tm.begin(0, st);
    hipLaunchKernelGGL((rope_table_kernel<D>), dim3(blocks), dim3(256), 0, st, a.rope, G.T, G.H, G.W);
    tm.end(0, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int blocks = G.heads * G.nseg * G.cps1;
    tm.begin(1, st);
    if (G.rope_lds1)
      hipLaunchKernelGGL((state_partial_kernel<D, E, true>), dim3(blocks), dim3(kThreads), 0, st,
                         (const E*)a.k, (const E*)a.v, (const E*)a.beta, (const float2*)a.rope, a.partial, G);
    else
      hipLaunchKernelGGL((state_partial_kernel<D, E, false>), dim3(blocks), dim3(kThreads), 0, st,
                         (const E*)a.k, (const E*)a.v, (const E*)a.beta, (const float2*)a.rope, a.partial, G);
    tm.end(1, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    constexpr int SZ = D * D + D;
    dim3 grid((SZ + 255) / 256, G.heads);
    tm.begin(2, st);
    hipLaunchKernelGGL((state_reduce_kernel<D>), grid, dim3(256), 0, st, (const float*)a.partial, a.S_in, a.z_in,
                       a.states, a.S_out, a.z_out, G);
    tm.end(2, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int blocks = G.heads * G.nseg * G.cps2;
    tm.begin(3, st);
    if (G.rope_lds2)
      hipLaunchKernelGGL((output_kernel<D, E, true>), dim3(blocks), dim3(kThreads), 0, st, (const E*)a.q,
                         (const E*)a.g, (const float*)a.states, a.rms_w, (const float2*)a.rope, (E*)a.out, G);
    else
      hipLaunchKernelGGL((output_kernel<D, E, false>), dim3(blocks), dim3(kThreads), 0, st, (const E*)a.q,
                         (const E*)a.g, (const float*)a.states, a.rms_w, (const float2*)a.rope, (E*)a.out, G);
    tm.end(3, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_operator(const LaunchArgs& a, Timer& tm) {
  if (a.bf16) {
    switch (a.geo.d) {
      case 32: return launch_all<32, bf16_t>(a, tm);
      case 64: return launch_all<64, bf16_t>(a, tm);
      case 128: return launch_all<128, bf16_t>(a, tm);
    }
  } else {
    switch (a.geo.d) {
      case 32: return launch_all<32, float>(a, tm);
      case 64: return launch_all<64, float>(a, tm);
      case 128: return launch_all<128, float>(a, tm);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace gla
