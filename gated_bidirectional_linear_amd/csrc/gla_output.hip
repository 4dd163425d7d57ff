// Pass 2: the fused output kernel.
#include "gla_common.h"

namespace gla {

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

template <int D, typename E>
hipError_t launch_output(const LaunchArgs& a) {
  const Geometry& G = a.geo;
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

}  // namespace gla
