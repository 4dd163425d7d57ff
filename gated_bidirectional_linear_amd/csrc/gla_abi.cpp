// C ABI of the operator: argument validation, token partition, stream-ordered
// scratch, launch sequencing and optional per-kernel event timing.
#include <hip/hip_runtime_api.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/gla.h"
#include "../../include/gla_internal.h"
#include "gla_launch.h"

namespace {

using gla::Geometry;

constexpr int kTile = 64;
// Workgroups aimed for per launch: pass 1 writes one partial state per
// workgroup, so it stays near two per CU (256 CUs); pass 2 has no such cost
// and takes more for load balance.  gla_plan_override changes them for tests
// and tuning sweeps.
constexpr int kDefaultTargetWg1 = 512;
// The bf16, d = 128 pass-1 kernel keeps whole states in registers and runs
// one workgroup per CU.
constexpr int kDefaultTargetWgAcc1 = 256;
constexpr int kDefaultTargetWg2 = 2048;
// The paired-head output kernel (bf16, d = 128) runs two workgroups per CU
// (kPair2Slots at once).  Its launch is sized in whole rounds: one round, with
// chunks of at least kPair2MinTiles tiles (each workgroup first reads its two
// heads' 128 KB of state), or two rounds when one round's chunks would exceed
// kPair2LongChunk tokens.  Measured in the full step: 720p/60s 680 us at two
// rounds (1024 workgroups); 720p/5s with 32 heads 78 us at 512 workgroups
// against 91 us at 592; 480p 23 us with 192-token chunks against 30 us with
// 64-token ones.
constexpr int kPair2Slots = 512;
constexpr int kPair2MinTiles = 3;
constexpr int kPair2LongChunk = 2048;
// The four-head output kernel (bf16, d = 128, heads divisible by 4) runs one
// workgroup of 16 waves per CU: its launch aims for one round of 256
// workgroups, with chunks of whole 64-token tiles, at least kQuad2MinTiles of
// them (each workgroup first reads its four heads' 128 KB of bf16 state).
// Where that round would leave more than a quarter of the CUs idle (short
// sequences), the chunks are cut in the kernel's own 16-token tiles instead,
// at least kQuad2MinUnits of them.  Measured (whole call): 480p 51.2 us with
// 225 workgroups of 96 tokens against 52.3-53.8 us with 170 of 128;
// 720p/5s with 20 heads 93.3 us with 220 workgroups of 320 tokens against
// 96.6 us with 245 of 288.
constexpr int kQuad2Slots = 256;
constexpr int kQuad2MinTiles = 2;
constexpr int kQuadTile = 16;
constexpr int kQuad2MinUnits = 6;

// Launch-plan overrides (include/gla_internal.h): process-wide, 0 = the
// measured default.  Every call reads them once, into a Knobs snapshot, so a
// concurrent gla_plan_override cannot change a plan halfway through.
std::atomic<int> g_knobs[GLA_PLAN_NUM_KNOBS];

struct Knobs {
  int v[GLA_PLAN_NUM_KNOBS];
  static Knobs snapshot() {
    Knobs k;
    for (int i = 0; i < GLA_PLAN_NUM_KNOBS; ++i) k.v[i] = g_knobs[i].load(std::memory_order_relaxed);
    return k;
  }
  // the knob's value, or dflt where it is unset
  int get(int knob, int dflt) const { return v[knob] > 0 ? v[knob] : dflt; }
  bool on(int knob) const { return v[knob] > 0; }
};

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// (head, segment) units aimed for by the token-causal walk: each is walked in
// order by four waves; with head pairs two units share a workgroup.
constexpr int kDefaultTargetWgTokenCausal = 512;
constexpr int kTokenTile = 32;   // tokens per step of the token-causal kernel

enum class Form { bidirectional, block_causal, token_causal };

// Segment length: the whole sequence, one block of latent frames, or (token-
// causal form) a multiple of the 32-token tile chosen for parallelism.
// (Per batch item: segments never straddle items.)
int segment_length(Form form, int T, int H, int W, int heads, int block_frames, int batch, const Knobs& kn) {
  const long N = (long)T * H * W;
  if (form == Form::block_causal) {
    const int frames = (block_frames > 0 && block_frames < T) ? block_frames : T;
    return frames * H * W;
  }
  if (form == Form::token_causal) {
    const int want = ceil_div(kn.get(GLA_PLAN_TOKEN_CAUSAL_WORKGROUPS, kDefaultTargetWgTokenCausal), (long)heads * batch);
    const int nseg = want < 1 ? 1 : want;
    const long len = ((N + nseg - 1) / nseg + kTokenTile - 1) / kTokenTile * kTokenTile;
    return (int)(len < kTokenTile ? kTokenTile : len);
  }
  return (int)N;
}

// narrow: the I/O dtype is bf16 or fp8, whose rows the fast d = 128 pass-1 kernel takes as bf16
// words; bf16_io: the I/O dtype is bf16
Geometry plan(int T, int H, int W, int heads, int d, float eps, int seg_len, bool token_causal, bool narrow,
              bool bf16_io, int batch, const Knobs& kn) {
  Geometry G{};
  G.H = H; G.W = W; G.heads = heads; G.d = d; G.eps = eps;
  G.batch = batch;
  G.T_item = T;
  G.n_item = T * H * W;
  G.T = batch * T;
  G.N = batch * G.n_item;
  G.seg_len = seg_len;
  G.segs_item = ceil_div(G.n_item, G.seg_len);
  G.nseg = batch * G.segs_item;
  G.token_causal = token_causal ? 1 : 0;
  G.states_exclusive = token_causal ? 1 : 0;
  const int tiles_per_seg = ceil_div(G.seg_len, kTile);
  const int per_seg_heads = heads * G.nseg;

  // RoPE rows a chunk of L tokens needs in LDS: the y and x blocks plus the
  // frames it can span (at worst alignment).
  const int HW = H * W;
  const long yx = (long)H * (3 * d / 16) + (long)W * (3 * d / 16);
  auto rope_fits = [&](long L, int entries = gla::kRopeLdsEntries, long max_frames = 1L << 30) {
    long frames = (L + HW - 2) / HW + 1;
    if (frames > T) frames = T;
    return frames <= max_frames && yx + frames * (d / 8) <= entries;
  };

  // Whether any chunk's RoPE rows fit in LDS (the y and x blocks plus one
  // frame).  Where they cannot, every kernel reads the global table, and
  // smaller chunks would buy nothing.
  const bool lds_any = !kn.on(GLA_PLAN_ROPE_GLOBAL) && rope_fits(1);

  G.pass1_reg = (narrow && d == 128 && lds_any && !kn.on(GLA_PLAN_PASS1_GENERIC)) ? 1 : 0;
  const int target1 = G.pass1_reg ? kDefaultTargetWgAcc1 : kDefaultTargetWg1;
  // the register-accumulating kernel runs one workgroup per CU: rounding the
  // chunk count down keeps the launch to one round of workgroups (20 heads:
  // 240 workgroups, not 256 and then 4 more)
  const int want1 = G.pass1_reg ? kn.get(GLA_PLAN_PASS1_WORKGROUPS, target1) / per_seg_heads
                                : ceil_div(kn.get(GLA_PLAN_PASS1_WORKGROUPS, target1), per_seg_heads);
  int cps1 = want1 < 1 ? 1 : want1;
  if (cps1 > gla::kMaxChunks) cps1 = gla::kMaxChunks;
  if (cps1 > tiles_per_seg) cps1 = tiles_per_seg;
  // more (smaller) chunks when a chunk's RoPE rows would not fit in LDS
  const long frames1 = G.pass1_reg ? gla::kRegRopeMaxFrames : 1L << 30;
  while (lds_any && !rope_fits((long)ceil_div(tiles_per_seg, cps1) * kTile, gla::kRopeLdsEntries, frames1) &&
         cps1 < gla::kMaxChunks && cps1 < tiles_per_seg)
    ++cps1;
  G.chunk1 = ceil_div(tiles_per_seg, cps1) * kTile;
  G.cps1 = ceil_div(G.seg_len, G.chunk1);
  G.rope_lds1 = rope_fits(G.chunk1, gla::kRopeLdsEntries, frames1) ? 1 : 0;

  // Heads per workgroup of pass 2 at d = 128: four where the head count allows
  // (bf16: 1 KB token row segments; fp8: 512 bytes), else pairs for bf16 (the
  // pair kernel's fp8 instantiation spilled registers) and one head for fp8.
  // With fp8 rows the four-head kernel gives the feature work to its MFMA waves
  // (the gate is a table lookup there): at 720p/60s 453 us against 453-464 us
  // for the one-head kernel, and the whole call 825-836 us against 840-853 us.
  const int max_hp = kn.on(GLA_PLAN_PASS2_GENERIC) ? 1 : kn.get(GLA_PLAN_PASS2_HEADS, 4);
  G.pass2_pair = 0;
  if (narrow && d == 128 && !token_causal && lds_any) {   // bf16 or fp8 I/O
    if (heads % 4 == 0 && max_hp >= 4) G.pass2_pair = 4;
    else if (bf16_io && heads % 2 == 0 && max_hp >= 2) G.pass2_pair = 2;
  }
  const int per_seg_units2 = G.pass2_pair ? per_seg_heads / G.pass2_pair : per_seg_heads;
  // pass-2 chunks come in whole units of unit2 tokens
  int unit2 = kTile;
  int want2 = ceil_div(kn.get(GLA_PLAN_PASS2_WORKGROUPS, kDefaultTargetWg2), per_seg_units2);
  if (G.pass2_pair == 4 && !kn.on(GLA_PLAN_PASS2_WORKGROUPS)) {
    want2 = kQuad2Slots / per_seg_units2;   // chunks per segment in one round
    const int most = ceil_div(tiles_per_seg, kQuad2MinTiles);
    if (want2 > most) want2 = most;
    if (4L * per_seg_units2 * (want2 < 1 ? 1 : want2) < 3L * kQuad2Slots) {   // a quarter of the CUs idle
      unit2 = kQuadTile;
      want2 = kQuad2Slots / per_seg_units2;
      const int most_q = ceil_div(G.seg_len, kQuadTile * kQuad2MinUnits);
      if (want2 > most_q) want2 = most_q;
    }
  } else if (G.pass2_pair && !kn.on(GLA_PLAN_PASS2_WORKGROUPS)) {
    want2 = kPair2Slots / per_seg_units2;   // chunks per segment in one round
    if (want2 < 1) want2 = 1;
    if ((long)ceil_div(tiles_per_seg, want2) * kTile > kPair2LongChunk) want2 = 2 * kPair2Slots / per_seg_units2;
    const int most = ceil_div(tiles_per_seg, kPair2MinTiles);
    if (want2 > most) want2 = most;
  }
  const int units_per_seg2 = ceil_div(G.seg_len, unit2);
  int cps2 = want2 < 1 ? 1 : want2;
  if (cps2 > units_per_seg2) cps2 = units_per_seg2;
  while (lds_any && !rope_fits((long)ceil_div(units_per_seg2, cps2) * unit2) && cps2 < units_per_seg2) ++cps2;
  G.chunk2 = ceil_div(units_per_seg2, cps2) * unit2;
  G.cps2 = ceil_div(G.seg_len, G.chunk2);
  G.rope_lds2 = rope_fits(G.chunk2) ? 1 : 0;
  if (token_causal) {   // one workgroup walks a whole segment (of one head, or of a head pair)
    G.cps2 = 1;
    G.chunk2 = G.seg_len;
    G.rope_lds2 = rope_fits(G.seg_len, gla::kRopeLdsEntriesCausal) ? 1 : 0;
    // head pairs (bf16 operands, d = 128, even head count): 512-byte row segments
    const int walk_hp = kn.on(GLA_PLAN_PASS2_GENERIC) ? 1 : kn.get(GLA_PLAN_PASS2_HEADS, 2);
    G.pass2_pair = (narrow && d == 128 && heads % 2 == 0 && walk_hp >= 2) ? 2 : 0;
  }
  if (kn.on(GLA_PLAN_ROPE_GLOBAL)) G.rope_lds1 = G.rope_lds2 = 0;
  // the register-accumulating and paired-head kernels read their RoPE rows from LDS only
  if (!G.rope_lds1) G.pass1_reg = 0;
  if (!G.rope_lds2 && !token_causal) G.pass2_pair = 0;
  return G;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// timing instrumentation
// ---------------------------------------------------------------------------
// Timing-only events: no system-scope fence when they complete, so recording
// them does not write back and invalidate the caches between the kernels they
// bracket (the default fence added ~7 us per kernel boundary at 720p/60s).
// Events are taken from a free list and returned to it when read, so a timed
// call creates none once the list has grown to the calls' needs.
struct EventTimer final : gla::Timer {
  struct Rec { int id; hipEvent_t a, b; };
  bool on = false;
  unsigned mask = ~0u;            // kernel ids timed while on
  std::vector<Rec> recs;
  std::vector<hipEvent_t> open;   // per kernel id, start event awaiting its end
  std::vector<hipEvent_t> pool;   // created events not in use
  std::mutex mu;
  EventTimer() : open(gla::kNumKernels, nullptr) {}
  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
  }
  void begin(int id, hipStream_t s) override {
    if (!on || !((mask >> id) & 1u)) return;
    hipEvent_t e = take();
    if (e == nullptr) return;
    hipEventRecord(e, s);
    open[id] = e;
  }
  void end(int id, hipStream_t s) override {
    if (!on || open[id] == nullptr) return;
    hipEvent_t e = take();
    if (e == nullptr) return;
    hipEventRecord(e, s);
    recs.push_back({id, open[id], e});
    open[id] = nullptr;
  }
};

EventTimer& timer() {
  static EventTimer t;
  return t;
}

struct NullTimer final : gla::Timer {
  void begin(int, hipStream_t) override {}
  void end(int, hipStream_t) override {}
};

// ---------------------------------------------------------------------------
// memory pool: keep freed scratch cached in the pool between calls
// ---------------------------------------------------------------------------
std::mutex g_pool_mu;
bool g_pool_ready[256] = {false};

void prepare_pool() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return;
  std::lock_guard<std::mutex> lk(g_pool_mu);
  if (g_pool_ready[dev]) return;
  hipMemPool_t pool;
  if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
    uint64_t thr = UINT64_MAX;
    hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
  }
  g_pool_ready[dev] = true;
}

// ---------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------
// bytes per element of an I/O dtype (a known one)
int elem_size(int dtype) {
  return dtype == GLA_DTYPE_BF16 ? 2 : ((dtype == GLA_DTYPE_FP8_E4M3 || dtype == GLA_DTYPE_FP8_E5M2) ? 1 : 4);
}

struct Range { uintptr_t lo, hi; };

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

Range range_of(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + bytes};
}

int validate(const void* q, const void* k, const void* v, const void* beta, const void* g, const float* rms_w,
             int T, int H, int W, int heads, int d, float eps, const void* out, int dtype, bool causal,
             const float* S, const float* z, int block_frames, int batch) {
  if (dtype != GLA_DTYPE_F32 && dtype != GLA_DTYPE_BF16 && dtype != GLA_DTYPE_FP8_E4M3 && dtype != GLA_DTYPE_FP8_E5M2)
    return GLA_ERR_DTYPE;
  if (d != 32 && d != 64 && d != 128) return GLA_ERR_UNSUPPORTED_D;
  if (T < 0 || H < 0 || W < 0 || heads < 1 || batch < 1) return GLA_ERR_SHAPE;
  if (!(std::isfinite(eps) && eps >= FLT_MIN)) return GLA_ERR_SHAPE;
  if (causal && block_frames < 1) return GLA_ERR_SHAPE;
  // each product below stays under 2^62: every factor is < 2^31 and the
  // running product is checked against 2^31 before the next factor
  const long long BT = (long long)batch * T;
  if (BT >= (1LL << 31)) return GLA_ERR_SHAPE;
  const long long BTH = BT * H;
  if (BTH >= (1LL << 31) && W > 0) return GLA_ERR_SHAPE;
  const long long N = W > 0 ? BTH * W : 0;   // tokens of all items
  if (N >= (1LL << 31)) return GLA_ERR_SHAPE;
  if (heads > (1 << 20)) return GLA_ERR_SHAPE;
  if (N * heads * d >= (1LL << 40)) return GLA_ERR_SHAPE;
  // the kernels address up to 64 token rows of all heads through one 32-bit
  // buffer range: a token row (heads * d elements) must stay below 2^26 bytes
  const long long es_row = elem_size(dtype);
  if ((long long)heads * d * es_row >= (1LL << 26)) return GLA_ERR_SHAPE;
  if (N == 0) return GLA_OK;  // nothing is read or written
  const void* ptrs[] = {q, k, v, beta, g, rms_w, out, causal ? S : rms_w, causal ? z : rms_w};
  for (const void* p : ptrs)
    if (p == nullptr) return GLA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return GLA_ERR_ALIGN;
  const size_t es = (size_t)elem_size(dtype);
  const size_t big = (size_t)N * heads * d * es;
  const Range rin[] = {range_of(q, big), range_of(k, big), range_of(v, big), range_of(g, big),
                       range_of(beta, (size_t)N * heads * es), range_of(rms_w, (size_t)d * 4)};
  const Range rout = range_of(out, big);
  for (const Range& r : rin)
    if (overlap(rout, r)) return GLA_ERR_ALIAS;
  if (causal) {
    const Range rs = range_of(S, (size_t)batch * heads * d * d * 4);
    const Range rz = range_of(z, (size_t)batch * heads * d * 4);
    if (overlap(rs, rz) || overlap(rs, rout) || overlap(rz, rout)) return GLA_ERR_ALIAS;
    for (const Range& r : rin)
      if (overlap(rs, r) || overlap(rz, r)) return GLA_ERR_ALIAS;
  }
  return GLA_OK;
}

// fixed: when given, the call's scratch is that buffer (the allocation-free
// entry point) instead of a stream-ordered allocation.
int run(Form form, const void* q, const void* k, const void* v, const void* beta, const void* g, const float* rms_w,
        int batch, int T, int H, int W, int heads, int d, float eps, void* out, void* stream, int dtype, float* S,
        float* z, int block_frames, int t_offset, int include_self, const gla::FixedScratch* fixed = nullptr) {
  const bool causal = form != Form::bidirectional;
  const int st = validate(q, k, v, beta, g, rms_w, T, H, W, heads, d, eps, out, dtype, causal, S, z,
                          form == Form::block_causal ? block_frames : 1, batch);
  if (st != GLA_OK) return st;
  const long long N = (long long)batch * T * H * W;
  if (N == 0) return GLA_OK;

  const Knobs kn = Knobs::snapshot();
  const int seg_len = segment_length(form, T, H, W, heads, block_frames, batch, kn);
  Geometry G = plan(T, H, W, heads, d, eps, seg_len, form == Form::token_causal,
                    elem_size(dtype) <= 2, dtype == GLA_DTYPE_BF16, batch, kn);
  G.t_offset = t_offset;
  G.include_self = include_self;
  const size_t rope_bytes =
      align256(((size_t)G.T * (d / 8) + (size_t)H * (3 * d / 16) + (size_t)W * (3 * d / 16)) * 8);
  const size_t sz = (size_t)d * d + d;
  const size_t part_bytes = align256((size_t)heads * G.nseg * G.cps1 * sz * 4);
  const size_t state_bytes = align256((size_t)G.nseg * heads * sz * 4);
  const size_t sbf_bytes = G.pass2_pair == 4 ? align256((size_t)G.nseg * heads * d * d * 2) : 0;
  const size_t scratch_bytes = rope_bytes + part_bytes + state_bytes + sbf_bytes;
  if (fixed != nullptr && scratch_bytes > fixed->bytes) return GLA_ERR_TOO_LARGE;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  // no usable device (none present, or the runtime failed to start): report
  // it before any allocation or launch
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return GLA_ERR_HIP;
  }
  void* scratch = nullptr;
  if (fixed != nullptr) {
    scratch = fixed->device_ptr(dev);
    if (scratch == nullptr) return GLA_ERR_HIP;
  } else {
    prepare_pool();
    if (hipMallocAsync(&scratch, scratch_bytes, hs) != hipSuccess || scratch == nullptr) {
      (void)hipGetLastError();
      return GLA_ERR_ALLOC;
    }
  }
  char* base = static_cast<char*>(scratch);

  gla::LaunchArgs a{};
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g; a.rms_w = rms_w; a.out = out;
  a.S_in = S; a.z_in = z; a.S_out = S; a.z_out = z;
  a.rope = reinterpret_cast<float2*>(base);
  a.partial = reinterpret_cast<float*>(base + rope_bytes);
  a.states = reinterpret_cast<float*>(base + rope_bytes + part_bytes);
  a.states_bf16 = sbf_bytes ? reinterpret_cast<unsigned short*>(base + rope_bytes + part_bytes + state_bytes) : nullptr;
  a.dtype = dtype;
  a.stream = hs;
  a.geo = G;

  hipError_t e;
  EventTimer& tm = timer();
  if (tm.on) {
    std::lock_guard<std::mutex> lk(tm.mu);
    e = gla::launch_operator(a, tm);
  } else {
    NullTimer nt;
    e = gla::launch_operator(a, nt);
  }
  const hipError_t ef = fixed != nullptr ? hipSuccess : hipFreeAsync(scratch, hs);
  if (e != hipSuccess || ef != hipSuccess) {
    (void)hipGetLastError();
    return GLA_ERR_HIP;
  }
  return GLA_OK;
}

const char* const kKernelNames[gla::kNumKernels] = {"rope_table_kernel", "state_partial_kernel",
                                                     "state_reduce_kernel", "output_kernel"};

}  // namespace

namespace gla {
int forward_fixed_scratch(const void* q, const void* k, const void* v, const void* beta, const void* g,
                          const float* rms_w, int T, int H, int W, int heads, int d, float eps, void* out,
                          void* stream, int dtype, const FixedScratch& fixed) {
  return run(Form::bidirectional, q, k, v, beta, g, rms_w, 1, T, H, W, heads, d, eps, out, stream, dtype, nullptr,
             nullptr, 0, 0, 0, &fixed);
}
}  // namespace gla

extern "C" {

int gla_forward_batch(const void* q, const void* k, const void* v, const void* beta, const void* g,
                      const float* rms_w, int batch, int T, int H, int W, int heads, int d, float eps, void* out,
                      void* stream, int dtype) {
  return run(Form::bidirectional, q, k, v, beta, g, rms_w, batch, T, H, W, heads, d, eps, out, stream, dtype, nullptr,
             nullptr, 0, 0, 0);
}

int gla_forward(const void* q, const void* k, const void* v, const void* beta, const void* g, const float* rms_w,
                int T, int H, int W, int heads, int d, float eps, void* out, void* stream, int dtype) {
  return gla_forward_batch(q, k, v, beta, g, rms_w, 1, T, H, W, heads, d, eps, out, stream, dtype);
}

int gla_block_causal_forward_batch(const void* q, const void* k, const void* v, const void* beta, const void* g,
                                   const float* rms_w, int batch, int T, int H, int W, int heads, int d, float eps,
                                   void* out, void* stream, float* state_S, float* state_z, int block_frames,
                                   int t_offset, int dtype) {
  const bool frames_ok = block_frames >= 1 && t_offset >= 0 && t_offset % block_frames == 0 &&
                         (long long)t_offset + T <= INT32_MAX;
  if (!frames_ok) {
    // validate the rest first so dtype/d errors keep their precedence
    const int st =
        validate(q, k, v, beta, g, rms_w, T, H, W, heads, d, eps, out, dtype, true, state_S, state_z, 1, batch);
    return st != GLA_OK ? st : GLA_ERR_SHAPE;
  }
  return run(Form::block_causal, q, k, v, beta, g, rms_w, batch, T, H, W, heads, d, eps, out, stream, dtype, state_S,
             state_z, block_frames, t_offset, 0);
}

int gla_block_causal_forward_at(const void* q, const void* k, const void* v, const void* beta, const void* g,
                                const float* rms_w, int T, int H, int W, int heads, int d, float eps, void* out,
                                void* stream, float* state_S, float* state_z, int block_frames, int t_offset,
                                int dtype) {
  return gla_block_causal_forward_batch(q, k, v, beta, g, rms_w, 1, T, H, W, heads, d, eps, out, stream, state_S,
                                        state_z, block_frames, t_offset, dtype);
}

int gla_token_causal_forward_batch(const void* q, const void* k, const void* v, const void* beta, const void* g,
                                   const float* rms_w, int batch, int T, int H, int W, int heads, int d, float eps,
                                   void* out, void* stream, float* state_S, float* state_z, int include_self,
                                   int t_offset, int dtype) {
  const bool args_ok = (include_self == 0 || include_self == 1) && t_offset >= 0 && (long long)t_offset + T <= INT32_MAX;
  if (!args_ok) {
    // validate the rest first so dtype/d errors keep their precedence
    const int st =
        validate(q, k, v, beta, g, rms_w, T, H, W, heads, d, eps, out, dtype, true, state_S, state_z, 1, batch);
    return st != GLA_OK ? st : GLA_ERR_SHAPE;
  }
  return run(Form::token_causal, q, k, v, beta, g, rms_w, batch, T, H, W, heads, d, eps, out, stream, dtype, state_S,
             state_z, 0, t_offset, include_self);
}

int gla_token_causal_forward(const void* q, const void* k, const void* v, const void* beta, const void* g,
                             const float* rms_w, int T, int H, int W, int heads, int d, float eps, void* out,
                             void* stream, float* state_S, float* state_z, int include_self, int t_offset,
                             int dtype) {
  return gla_token_causal_forward_batch(q, k, v, beta, g, rms_w, 1, T, H, W, heads, d, eps, out, stream, state_S,
                                        state_z, include_self, t_offset, dtype);
}

int gla_block_causal_forward(const void* q, const void* k, const void* v, const void* beta, const void* g,
                             const float* rms_w, int T, int H, int W, int heads, int d, float eps, void* out,
                             void* stream, float* state_S, float* state_z, int block_frames, int dtype) {
  return gla_block_causal_forward_at(q, k, v, beta, g, rms_w, T, H, W, heads, d, eps, out, stream, state_S, state_z,
                                     block_frames, 0, dtype);
}

const char* gla_status_string(int status) {
  switch (status) {
    case GLA_OK: return "ok";
    case GLA_ERR_NULL: return "a required pointer is NULL";
    case GLA_ERR_SHAPE: return "invalid shape, block size, frame offset, causal mode flag, eps or size overflow";
    case GLA_ERR_DTYPE: return "unknown dtype";
    case GLA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case GLA_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case GLA_ERR_ALLOC: return "temporary device memory could not be obtained";
    case GLA_ERR_UNSUPPORTED_D: return "head dim must be 32, 64 or 128";
    case GLA_ERR_ALIAS: return "output or state buffer overlaps another tensor";
    case GLA_ERR_TOO_LARGE: return "the call needs more scratch than the allocation-free entry point's static buffer holds";
    default: return "unknown status";
  }
}

int gla_version(void) { return (1 << 16) | 6; }

int gla_timing_enable(int on) {
  EventTimer& tm = timer();
  std::lock_guard<std::mutex> lk(tm.mu);
  tm.on = on != 0;
  return GLA_OK;
}

int gla_timing_read(double* ms, long long* launches, int n) {
  EventTimer& tm = timer();
  std::lock_guard<std::mutex> lk(tm.mu);
  int st = GLA_OK;
  for (int i = 0; i < n && i < gla::kNumKernels; ++i) {
    if (ms) ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  for (auto& r : tm.recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) st = GLA_ERR_HIP;
    if (r.id < n) {
      if (ms) ms[r.id] += t;
      if (launches) launches[r.id] += 1;
    }
    tm.pool.push_back(r.a);
    tm.pool.push_back(r.b);
  }
  tm.recs.clear();
  return st;
}

int gla_timing_select(unsigned mask) {
  EventTimer& tm = timer();
  std::lock_guard<std::mutex> lk(tm.mu);
  tm.mask = mask;
  return GLA_OK;
}

int gla_plan_describe(int form, int batch, int T, int H, int W, int heads, int d, int dtype, int block_frames,
                      int* out, int n) {
  if (form < 0 || form > 2) return GLA_ERR_SHAPE;
  const Form f = form == 0 ? Form::bidirectional : (form == 1 ? Form::block_causal : Form::token_causal);
  // shape checks of the operator calls, without the tensors
  const int st = validate(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, T, H, W, heads, d, 1e-6f, nullptr,
                          dtype, f != Form::bidirectional, nullptr, nullptr,
                          f == Form::block_causal ? block_frames : 1, batch);
  if (st != GLA_OK && st != GLA_ERR_NULL) return st;
  if ((long long)T * H * W == 0) return GLA_ERR_SHAPE;   // an empty grid has no plan
  if (out == nullptr && n > 0) return GLA_ERR_NULL;
  const Knobs kn = Knobs::snapshot();
  const int seg_len = segment_length(f, T, H, W, heads, block_frames, batch, kn);
  const Geometry G = plan(T, H, W, heads, d, 1e-6f, seg_len, f == Form::token_causal, elem_size(dtype) <= 2,
                          dtype == GLA_DTYPE_BF16, batch, kn);
  const int v[] = {G.seg_len, G.segs_item, G.cps1, G.chunk1, G.cps2, G.chunk2,
                   G.pass1_reg, G.pass2_pair, G.rope_lds1, G.rope_lds2};
  for (int i = 0; i < n && i < (int)(sizeof(v) / sizeof(v[0])); ++i) out[i] = v[i];
  return GLA_OK;
}

int gla_plan_override(int knob, int value) {
  if (knob < 0 || knob >= GLA_PLAN_NUM_KNOBS || value < 0 || value > (1 << 24)) return GLA_ERR_SHAPE;
  g_knobs[knob].store(value, std::memory_order_relaxed);
  return GLA_OK;
}

const char* gla_kernel_name(int kernel_id) {
  if (kernel_id < 0 || kernel_id >= gla::kNumKernels) return "unknown";
  return kKernelNames[kernel_id];
}

}  // extern "C"
