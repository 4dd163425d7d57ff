// Internal interface between the C ABI (gla_abi.cpp) and the kernel launchers.
//
// The operator (SANA-Video 2.0 digest, prelims "gated bilinear linear
// attention"; SANA-Video notes, key designs 1 and 2), per head, with
// q^ = q/rms(q), k^ = k/rms(k), phi = ReLU, R_n the 3D RoPE rotation of token n:
//   S = sum_n beta_n v_n (R_n phi k^_n)^T,   z = sum_n phi k^_n
//   o_j = w * rmsnorm( sigmoid(g_j) * (S R_j phi q^_j) / (phi q^_j . z + eps) )
//
// The tokens are cut into "segments": one segment of N tokens for the
// bidirectional form, one per block of latent frames for the block-causal
// form, or runs of 32-token tiles sized for parallelism in the token-causal
// form.  Up to four launches on the caller's stream:
//   1. rope_table_kernel    (gla_tables.hip): per-axis cos/sin tables, fp64 angles;
//      only when a pass-1 chunk's RoPE rows do not fit in LDS (otherwise pass 1
//      computes them and writes the table).
//   2. state_partial kernels (gla_state.hip): one workgroup per (head, chunk of
//      a segment) builds the partial V^T (beta R phi K^) on MFMA with fp32
//      accumulation, plus the partial key sum.
//   3. state_reduce_kernel  (gla_tables.hip): fixed-shape pairwise tree over the
//      chunk partials of each segment, then a prefix over segments on top of
//      the carried state -> per-segment states (inclusive of the segment, or
//      exclusive for the token-causal form) and the state after the call.
//   4. output_kernel        (gla_output.hip): one workgroup per (head or head
//      pair, chunk of tiles) holds its slice of S as MFMA A-fragments, streams
//      q and g, computes num^T = S RQ^T on MFMA, the denominator, gate and
//      RMSNorm, and writes the output once; or, in the token-causal form,
//      token_causal_kernel (gla_causal.hip), which walks each segment from its
//      exclusive state.
#pragma once
#include <hip/hip_runtime_api.h>

#include <cstddef>

namespace gla {

constexpr int kMaxChunks = 64;   // chunk partials per segment reduced by one tree
constexpr int kNumKernels = 4;   // rope table, state partials, reduce/prefix, output
// float2 entries of RoPE table a workgroup may stage in LDS (24 KB): at d = 128
// the y and x blocks of a 34 x 60 latent frame (1080p) and some 40 frames
constexpr int kRopeLdsEntries = 3072;
// Frames a chunk of the register-accumulating pass-1 kernel may span: its
// packed table row offsets give the frame rows 10 bits of 16-byte units.
constexpr int kRegRopeMaxFrames = 128;
// The token-causal kernel stages fewer (14 KB) so that two workgroups fit on a CU.
constexpr int kRopeLdsEntriesCausal = 1792;

// Token partition shared by all kernels of one call.  A segment is the unit of
// causality: the whole sequence (bidirectional) or one block of latent frames.
// A batch of independent sequences lies one item after another along the token
// axis; segments never straddle items.
struct Geometry {
  int T, H, W;  // T: frames of all items (batch * T_item), the RoPE table's frame rows
  int N;        // tokens of all items: batch * n_item
  int heads;
  int d;
  int batch;     // items
  int T_item;    // frames per item (RoPE positions restart at every item)
  int n_item;    // tokens per item, T_item * H * W
  int seg_len;   // tokens per segment (the last one of an item may be shorter)
  int segs_item; // segments per item
  int nseg;      // batch * segs_item
  int cps1;     // pass-1 chunks per segment (<= kMaxChunks)
  int chunk1;   // pass-1 tokens per chunk (multiple of the 64-token tile)
  int cps2;     // pass-2 chunks per segment
  int chunk2;   // pass-2 tokens per chunk
  int rope_lds1;  // pass 1 stages its RoPE table rows in LDS (else reads the global table)
  int rope_lds2;  // same for pass 2
  int pass1_reg;  // pass 1 uses the register-accumulating kernel (bf16, d = 128, RoPE rows in LDS)
  int pass2_pair; // heads per workgroup of the multi-head pass-2 kernels: 0 (one head), 2 (bf16,
                  // d = 128, even head count, RoPE rows in LDS; the token-causal walk takes pairs
                  // for bf16/fp8 operands at d = 128) or 4 (bf16, d = 128, head count divisible
                  // by 4, RoPE rows in LDS; reads the bf16 copy of the states)
  int t_offset;   // absolute frame of the call's frame 0 (RoPE positions only)
  int token_causal;   // token-level causal form: segments of seg_len tokens walked in order
  int include_self;   // token-causal: token i reads tokens j <= i (1) or j < i (0)
  int states_exclusive;  // per-segment states exclude their own segment (token-causal)
  float eps;
};

struct LaunchArgs {
  const void *q, *k, *v, *beta, *g;
  const float* rms_w;
  void* out;
  const float* S_in;  // carried state in (block-causal) or nullptr
  const float* z_in;
  float* S_out;       // carried state out (block-causal) or nullptr
  float* z_out;
  float2* rope;       // scratch: RoPE table
  float* partial;     // scratch: [heads][nseg*cps1][d*d + d]
  float* states;      // scratch: [nseg][heads][d*d + d]
  unsigned short* states_bf16;  // scratch: [nseg][heads][d*d], S of `states` rounded to bf16
                                // (written by the reduce kernel when pass2_pair == 4, else nullptr)
  int dtype;          // GLA_DTYPE_* of q, k, v, g, beta, out
  hipStream_t stream;
  Geometry geo;
};

// Optional per-kernel event timing (instrumentation only).
struct Timer {
  virtual void begin(int kernel, hipStream_t s) = 0;
  virtual void end(int kernel, hipStream_t s) = 0;
  virtual ~Timer() {}
};

hipError_t launch_operator(const LaunchArgs& a, Timer& tm);

// A scratch buffer that the caller holds for the whole process (the
// allocation-free entry point's static device array): its address on device
// `dev` (nullptr if it cannot be had) and its size in bytes.
struct FixedScratch {
  void* (*device_ptr)(int dev);
  size_t bytes;
};

// The bidirectional operator (gla_forward) with its scratch in `fixed`:
// GLA_ERR_TOO_LARGE, before anything is enqueued, when the call needs more.
int forward_fixed_scratch(const void* q, const void* k, const void* v, const void* beta, const void* g,
                          const float* rms_w, int T, int H, int W, int heads, int d, float eps, void* out,
                          void* stream, int dtype, const FixedScratch& fixed);

}  // namespace gla
