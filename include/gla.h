/*
 * gla.h -- C ABI of the MI355X (gfx950) gated bidirectional ReLU linear-attention
 * operator.
 *
 * The operation (SANA-Video 2.0 digest, prelims "gated bilinear linear
 * attention", output formula; SANA-Video notes, key design 1 "RoPE(ReLU(x))",
 * numerator-only RoPE; reader, appendix F.7 "gated RoPE-rotated linear state"):
 * for every head, with q^ = q/rms(q), k^ = k/rms(k), phi = ReLU and R_n the 3D
 * rotary rotation of token n on the (t, y, x) latent grid,
 *
 *     S   = sum_n beta_n v_n (R_n phi(k^_n))^T        (d x d, row = v channel)
 *     z   = sum_n phi(k^_n)                           (d)
 *     x_j = sigmoid(g_j) * (S R_j phi(q^_j)) / (phi(q^_j) . z + eps)
 *     out_j = rms_w * x_j / sqrt(mean(x_j^2) + eps)
 *
 * The block-causal form (SANA-Video notes, key design 2: cumulative state and
 * key sum as a constant-memory cache) visits blocks of `block_frames` latent
 * frames in order; tokens of block b read S and z summed over blocks <= b plus
 * the carried state passed in.  The token-causal form (same passage: running
 * sums per token) has token i read the sums over the tokens up to i.
 *
 * Conventions (the pages leave them open; one reading is fixed here):
 *   - token n = (t*H + y)*W + x, w fastest;
 *   - q, k, v, g, out: [N, heads, d] contiguous; beta: [N, heads];
 *     rms_w: [d] fp32 shared by all heads;
 *   - 3D RoPE: channels [0,d/4) follow t, [d/4,5d/8) follow y, [5d/8,d)
 *     follow x; pair i of an axis slice is channels (2i,2i+1) and turns by
 *     pos * 10000^(-2i/d_axis), (u,w) -> (u cos a - w sin a, u sin a + w cos a);
 *     row and column positions count from 0; the frame position of frame t
 *     of a call is t, plus t_offset in the calls that take one (streaming a
 *     video through successive calls);
 *   - one eps for the q/k RMS normalisation, the denominator and the output
 *     RMSNorm.
 *
 * Pointers: every tensor pointer is a DEVICE pointer, 16-byte aligned.  The
 * caller owns all buffers; the library keeps no pointer after a call returns.
 * `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 * are asynchronous: they validate on the host, enqueue kernels on `stream`
 * and return; the caller synchronises.  Results are bitwise reproducible for
 * identical inputs and shapes.  On a validation error (any status other than
 * GLA_ERR_HIP and GLA_ERR_ALLOC) nothing is enqueued and nothing is written;
 * GLA_ERR_ALLOC also enqueues nothing.  GLA_ERR_HIP means a kernel launch
 * failed after the call's earlier kernels were enqueued: the output is then
 * undefined, and in the causal forms the carried state may already hold the
 * state after the call.  Temporary device memory (RoPE tables, per-chunk
 * partial states) is taken stream-ordered from the device's default memory
 * pool and returned on the same stream; on its first call on a device the
 * library raises that pool's release threshold to the maximum, so that freed
 * scratch stays cached between calls (a setting of the process's default
 * pool, seen by its other users).  A call may be captured into a HIP graph (it
 * records kernels and stream-ordered allocations only, no memset nodes);
 * replays recompute it.
 */
#ifndef GLA_H
#define GLA_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GLA_OK = 0,
  GLA_ERR_NULL = -1,          /* a required pointer is NULL */
  GLA_ERR_SHAPE = -2,         /* T, H, W < 0, heads < 1, batch < 1, block_frames < 1, bad t_offset or include_self,
                                 eps not finite or below FLT_MIN, size overflow (N >= 2^31,
                                 N*heads*d >= 2^40, or a token row heads*d*elem_size >= 2^26 bytes) */
  GLA_ERR_DTYPE = -3,         /* dtype is not a gla_dtype value */
  GLA_ERR_ALIGN = -4,         /* a tensor pointer is not 16-byte aligned */
  GLA_ERR_HIP = -5,           /* no usable device, or a HIP runtime call or kernel launch failed */
  GLA_ERR_ALLOC = -6,         /* temporary device memory could not be obtained */
  GLA_ERR_UNSUPPORTED_D = -7, /* head dim not in {32, 64, 128} */
  GLA_ERR_ALIAS = -8,         /* out or the state overlaps another tensor */
  GLA_ERR_TOO_LARGE = -9      /* gla_forward_noalloc: the call needs more scratch than its static buffer */
} gla_status;

typedef enum {
  GLA_DTYPE_F32 = 0,      /* q, k, v, g, beta, out are float32 */
  GLA_DTYPE_BF16 = 1,     /* q, k, v, g, beta, out are bfloat16 (fp32 accumulation inside) */
  GLA_DTYPE_FP8_E4M3 = 2, /* q, k, v, g, beta, out are OCP FP8 E4M3 (e4m3fn: bias 7, max 448,
                             no infinities), one byte each; the state, the denominators and all
                             accumulation stay fp32 and the output is rounded to nearest even.
                             Low-precision operator I/O halves the bytes of a bandwidth-bound
                             op (SANA-Video 2.0 digest, weaknesses: the attention operator stays
                             BF16, so quantisation of the linear GEMMs alone saves only 5.8%). */
  GLA_DTYPE_FP8_E5M2 = 3  /* q, k, v, g, beta, out are OCP FP8 E5M2 (bias 15, max 57344, with
                             infinities and NaN; inputs must be finite), one byte each;
                             otherwise as GLA_DTYPE_FP8_E4M3:
                             fp32 state, denominators and accumulation, output rounded to nearest
                             even.  It trades one mantissa bit (2 against 3) for a range of 2^-16 to
                             57344, for inputs whose scale varies more than e4m3 holds. */
} gla_dtype;

/*
 * Bidirectional operator (SANA-Video 2.0 digest, prelims, output formula:
 * every token reads the state of all tokens).
 *
 *   q, k, v, g : [N, heads, d] in `dtype`, N = T*H*W        (read)
 *   beta       : [N, heads] in `dtype`, per-token write gate (read)
 *   rms_w      : [d] float32, output RMSNorm weight          (read)
 *   out        : [N, heads, d] in `dtype`                    (written; must not alias an input)
 *   T, H, W    : latent grid (frames, rows, columns), each >= 0; N = 0 is a no-op
 *   heads      : >= 1;  d : 32, 64 or 128;  eps : finite, >= FLT_MIN (a normal float); rows
 *                with phi(q^) = 0 (all-zero or all-negative q) give an all-zero output
 *                row for every such eps
 * When N == 0 the tensor pointers may be NULL.
 * Returns GLA_OK or a negative gla_status.
 */
int gla_forward(const void* q, const void* k, const void* v, const void* beta, const void* g,
                const float* rms_w, int T, int H, int W, int heads, int d, float eps,
                void* out, void* stream, int dtype);

/*
 * Block-causal operator with a constant-memory carried state (SANA-Video
 * notes, key design 2).
 *
 * Same tensors as gla_forward, plus
 *   state_S      : [heads, d, d] float32, row = v channel, column = k channel
 *   state_z      : [heads, d] float32
 *                  Both are read on entry (zeros = a fresh video) and
 *                  overwritten with the state after the last block.
 *   block_frames : latent frames per block, >= 1; the last block may be shorter.
 * Block b covers frames [b*block_frames, min((b+1)*block_frames, T)); its
 * tokens read the state inclusive of their own block.  When N == 0 the state
 * is left unchanged.
 */
int gla_block_causal_forward(const void* q, const void* k, const void* v, const void* beta,
                             const void* g, const float* rms_w, int T, int H, int W, int heads,
                             int d, float eps, void* out, void* stream, float* state_S,
                             float* state_z, int block_frames, int dtype);

/*
 * The block-causal operator for one piece of a longer video streamed through
 * successive calls: the carried state is the constant-memory cache that lets
 * generation go on block after block up to minute-long videos (SANA-Video
 * notes, overview and key design 2).
 *
 * Same arguments as gla_block_causal_forward, plus
 *   t_offset : absolute latent frame of this call's frame 0, >= 0 and a
 *              multiple of block_frames (a block cannot straddle two calls,
 *              since its tokens also read the block's later tokens);
 *              t_offset + T <= INT32_MAX.
 * The RoPE position of frame t is t_offset + t; rows and columns start at 0.
 * Calling with frames [0, T1) and then, on the returned state, with frames
 * [T1, T) and t_offset = T1 (T1 a multiple of block_frames) gives the output
 * and state of one call over [0, T).  gla_block_causal_forward is this call
 * with t_offset = 0.  A bad t_offset returns GLA_ERR_SHAPE.
 */
int gla_block_causal_forward_at(const void* q, const void* k, const void* v, const void* beta,
                                const void* g, const float* rms_w, int T, int H, int W, int heads,
                                int d, float eps, void* out, void* stream, float* state_S,
                                float* state_z, int block_frames, int t_offset, int dtype);

/*
 * Token-level causal operator (SANA-Video notes, key design 2: causal linear
 * attention written as running sums over the tokens up to the current one of
 * the per-token states and key sums).  Tokens are taken in the order
 * n = (t*H + y)*W + x.  Token i reads
 *     S_i = S_0 + sum_{j in J(i)} beta_j v_j (R_j phi(k^_j))^T
 *     z_i = z_0 + sum_{j in J(i)} phi(k^_j)
 * with J(i) = {j <= i} when include_self is 1 and {j < i} (strictly earlier
 * tokens, the notes' sums up to i - 1) when it is 0, and
 *     x_i = sigmoid(g_i) * (S_i R_i phi(q^_i)) / (phi(q^_i) . z_i + eps),
 *     out_i = rms_w * x_i / sqrt(mean(x_i^2) + eps).
 *
 * Same tensors as gla_forward, plus
 *   state_S, state_z : the carried state (S_0, z_0) as in
 *                      gla_block_causal_forward: read on entry, overwritten
 *                      with the state after the last token (which includes
 *                      every token of the call, whatever include_self is).
 *   include_self     : 0 or 1, as above.
 *   t_offset         : absolute latent frame of this call's frame 0, >= 0,
 *                      t_offset + T <= INT32_MAX.  Calling with frames [0, T1)
 *                      and then, on the returned state, with frames [T1, T)
 *                      and t_offset = T1 gives the output and state of one
 *                      call over [0, T).
 * A bad include_self or t_offset returns GLA_ERR_SHAPE.  When N == 0 the state
 * is left unchanged.
 */
int gla_token_causal_forward(const void* q, const void* k, const void* v, const void* beta, const void* g,
                             const float* rms_w, int T, int H, int W, int heads, int d, float eps, void* out,
                             void* stream, float* state_S, float* state_z, int include_self, int t_offset,
                             int dtype);

/*
 * Batches of independent sequences (the streaming design's constant-memory
 * state carried per video, SANA-Video notes, key design 2, for several videos
 * at once), in one launch sequence.  Each of `batch` items is a sequence of
 * the same (T, H, W) grid with its own state; the items do not interact.
 *
 *   q, k, v, g, out : [batch, N, heads, d] (item b's rows follow item b-1's)
 *   beta            : [batch, N, heads]
 *   state_S, state_z: [batch, heads, d, d] and [batch, heads, d] float32 (the
 *                     causal forms): item b's carried state, read on entry and
 *                     overwritten with the item's state after the call
 *   batch           : >= 1; batch * T < 2^31 and batch * N * heads * d < 2^40
 *                     (GLA_ERR_SHAPE otherwise)
 * Every other argument is the single-sequence call's and applies to every
 * item alike (t_offset included: all items are at the same frames of their
 * videos).  Item b's output and state equal the single-sequence call on item
 * b's tensors; the kernels cover all items at once, which fills the GPU where
 * one short item would not.  The single-sequence calls are these with
 * batch = 1.
 */
int gla_forward_batch(const void* q, const void* k, const void* v, const void* beta, const void* g,
                      const float* rms_w, int batch, int T, int H, int W, int heads, int d, float eps,
                      void* out, void* stream, int dtype);
int gla_block_causal_forward_batch(const void* q, const void* k, const void* v, const void* beta,
                                   const void* g, const float* rms_w, int batch, int T, int H, int W,
                                   int heads, int d, float eps, void* out, void* stream, float* state_S,
                                   float* state_z, int block_frames, int t_offset, int dtype);
int gla_token_causal_forward_batch(const void* q, const void* k, const void* v, const void* beta,
                                   const void* g, const float* rms_w, int batch, int T, int H, int W,
                                   int heads, int d, float eps, void* out, void* stream, float* state_S,
                                   float* state_z, int include_self, int t_offset, int dtype);

/*
 * gla_forward without any device-memory allocation, for callers that cannot
 * allocate: code under HIP graph capture that must not record allocation
 * nodes, tight serving loops, and harnesses that forbid hipMalloc.  Same
 * arguments, layout, ownership, results (bit for bit) and errors as
 * gla_forward.  Its scratch (RoPE table, chunk partial states, per-segment
 * states) lives in a static device array of 64 MiB that each device the
 * library runs on holds until the process ends; the call makes no hipMalloc,
 * hipMallocAsync or hipFree.
 *
 * Limit: a call needing more than 64 MiB of scratch returns GLA_ERR_TOO_LARGE
 * before anything is enqueued.  The need is about
 *     (T*d/8 + (H + W)*3d/16)*8 + (P + 1)*heads*(d*d + d)*4 bytes,
 * with P <= 64 chunk partials per head (about max(1, 256/heads) at d = 128 in
 * bf16 or fp8, max(1, 512/heads) otherwise), plus heads*d*d*2 bytes for the
 * bf16 copy of the states when the four-head output kernel runs (d = 128,
 * bf16 or fp8, heads divisible by 4): the 720p/60s workload (159,280 tokens,
 * 32 heads, d = 128) needs 20 MB.
 *
 * Concurrency: every call on one device uses that device's one array.  Calls
 * that can overlap on a device (on different streams, or from different
 * threads without ordering) race on it and give undefined results; calls on
 * one stream are ordered and safe.  Nothing in the array must start at zero:
 * each call writes every part of it that it reads.
 */
int gla_forward_noalloc(const void* q, const void* k, const void* v, const void* beta, const void* g,
                        const float* rms_w, int T, int H, int W, int heads, int d, float eps,
                        void* out, void* stream, int dtype);

/* Static text for a gla_status value (never NULL). */
const char* gla_status_string(int status);

/* Library ABI version: (major << 16) | minor.  Minor 6: GLA_DTYPE_FP8_E5M2. */
int gla_version(void);

/*
 * Kernel timing instrumentation.  While enabled (on != 0), every call records a
 * HIP event pair around each of its kernels on the call's stream.
 * gla_timing_read synchronises on those events, adds the elapsed milliseconds
 * of all calls made since the previous read into ms[i] and their launch counts
 * into launches[i] for kernel i < min(n, GLA_NUM_KERNELS), then clears the
 * record.  Kernel ids: 0 RoPE table, 1 state partials, 2 state reduce/prefix,
 * 3 fused output.  Timing is process-wide and not thread-safe; turning it on
 * adds event records to every call.  The events are timing-only (no
 * system-scope fence when they complete): waiting on them through
 * gla_timing_read does not make the calls' outputs visible to the host; the
 * caller still synchronises the stream for that.  Returns GLA_OK or GLA_ERR_HIP.
 */
#define GLA_NUM_KERNELS 4
int gla_timing_enable(int on);
int gla_timing_read(double* ms, long long* launches, int n);
const char* gla_kernel_name(int kernel_id);
/* Which kernels the timing records: bit i of mask selects kernel id i (all
 * by default).  Each timed kernel adds an event pair to the call's stream,
 * so timing fewer kernels disturbs the calls less.  Returns GLA_OK. */
int gla_timing_select(unsigned mask);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H */
