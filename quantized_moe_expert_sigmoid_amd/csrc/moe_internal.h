// Internal declarations of libmoe (gfx950). Not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "moe.h"

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Device-side error flags, OR-ed by kernels into ctx->dev_err.
enum : uint32_t {
  ERRF_BAD_INDEX = 1u << 0,  // an expert index outside [0, E)
  ERRF_TIMEOUT = 1u << 1,    // a bounded wait gave up
  ERRF_RANGE = 1u << 2,      // an int32 accumulator bound was exceeded
};

struct moe_ctx {
  int device = 0;
  hipStream_t stream = nullptr;
  int n_cu = 256;
  // growable scratch (device)
  void *scratch = nullptr;
  size_t scratch_bytes = 0;
  // intermediates of the composed whole-layer path (kept apart from scratch,
  // which the per-step entry points reuse)
  void *io = nullptr;
  size_t io_bytes = 0;
  // buffers that scratch or io outgrew: freed only by moe_ctx_destroy, as
  // captured graphs and queued work may still address them
  std::vector<void *> retired;
  // while an allocation-free call runs: its io and scratch regions in the
  // library's static device array (moe_scratch / moe_io_scratch hand these
  // out instead of growing the context's buffers)
  char *fixed_io = nullptr, *fixed_scr = nullptr;
  size_t fixed_io_bytes = 0, fixed_scr_bytes = 0;
  // small persistent device block: error flags and counters
  uint32_t *dev_small = nullptr;  // kDevSmallBytes: [0] error flags; from word kBucketChunkWord, per-chunk counts
  int ffn_kernels = MOE_FFN_AUTO;
  // a second stream for work that may overlap the context stream's, forked
  // from and joined back into it with events (created on first use)
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  bool dbg_on = false;
  moe_debug_bufs dbg{};
  // per-kernel timing (measurement only)
  bool timing = false;
  struct TimedLaunch {
    hipEvent_t start, stop;
    int stage;
  };
  std::vector<TimedLaunch> timed;      // recorded, not yet read
  std::vector<hipEvent_t> event_pool;  // reusable events
};

// Bracket one kernel launch with timing events when ctx->timing is on.
struct MoeTimer {
  moe_ctx *ctx;
  int stage;
  hipEvent_t start = nullptr;
  MoeTimer(moe_ctx *c, int s);
  ~MoeTimer();
};

hipEvent_t moe_timing_event(moe_ctx *ctx);

// Launch a kernel on the context stream. With timing on, the dispatch itself
// carries the start/stop events (hipExtLaunchKernelGGL), so the recorded time
// is the kernel's own execution, not that of extra event packets around it.
template <typename K, typename... Args>
void moe_launch_on(moe_ctx *ctx, hipStream_t stream, int stage, K kernel, dim3 grid, dim3 block, Args... args) {
  hipEvent_t s = ctx->timing ? moe_timing_event(ctx) : nullptr;
  hipEvent_t e = s ? moe_timing_event(ctx) : nullptr;
  if (s && e) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, s, e, 0, args...);
    ctx->timed.push_back({s, e, stage});
    return;
  }
  if (s) ctx->event_pool.push_back(s);
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
}
template <typename K, typename... Args>
void moe_launch(moe_ctx *ctx, int stage, K kernel, dim3 grid, dim3 block, Args... args) {
  moe_launch_on(ctx, ctx->stream, stage, kernel, grid, block, args...);
}
// Fork: work enqueued on ctx->side after this call starts after everything
// enqueued on ctx->stream so far. Join: work enqueued on ctx->stream after
// this call starts after everything enqueued on ctx->side so far.
moe_status moe_side_fork(moe_ctx *ctx);
moe_status moe_side_join(moe_ctx *ctx);

moe_status moe_fail(moe_status st, const char *fmt, ...);
moe_status moe_hip_fail(hipError_t e, const char *what);
// Make the scratch at least `bytes` large; returns its pointer or nullptr.
moe_status moe_scratch(moe_ctx *ctx, size_t bytes, void **out);
moe_status moe_io_scratch(moe_ctx *ctx, size_t bytes, void **out);

#define MOE_HIP(expr)                                   \
  do {                                                  \
    hipError_t e__ = (expr);                            \
    if (e__ != hipSuccess) return moe_hip_fail(e__, #expr); \
  } while (0)

#define MOE_CHECK_LAUNCH(name)                       \
  do {                                               \
    hipError_t e__ = hipGetLastError();              \
    if (e__ != hipSuccess) return moe_hip_fail(e__, name); \
  } while (0)

static inline bool moe_aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static inline size_t moe_round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Parts of a scratch area laid out one after another, each on a 256-byte
// boundary; `size` is the area's total.
struct MoeLayout {
  size_t size = 0;
  size_t take(size_t bytes) {
    const size_t o = size;
    size = moe_round_up(size + bytes, 256);
    return o;
  }
};

// Launchers implemented in the .hip files
moe_status launch_quantize_rows(moe_ctx *ctx, int bits, const float *w, int64_t rows, int cols, uint8_t *packed,
                                float *scales);
moe_status launch_quantize_act(moe_ctx *ctx, const float *x, int T, int H, int8_t *xq, float *sx);
moe_status launch_router(moe_ctx *ctx, const moe_router_cfg *cfg, const float *x, const float *w_router,
                         const float *bias, int T, int H, int32_t *topk_idx, float *topk_w);
moe_status launch_bucket_public(moe_ctx *ctx, const int32_t *topk_idx, int T, int k, int E, int32_t *counts,
                                int32_t *offsets, int32_t *perm);
moe_status launch_expert_ffn(moe_ctx *ctx, int bits, const moe_expert_w *experts, const moe_expert_w *shared,
                             const uint8_t *expert_bits, const int8_t *xq, const float *sx, const int32_t *topk_idx,
                             int T, int H, int I, int E, int k, float *y_slots);
// The context's small device block (zeroed once, at creation): word 0 holds
// the error flags; from word kBucketChunkWord, the per-chunk expert counts of
// the chunked bucketing (at most kBucketChunks chunks of 1024 experts).
constexpr int kBucketChunks = 64;
constexpr int kBucketChunkWord = 1024;
constexpr size_t kDevSmallBytes = 4 * ((size_t)kBucketChunkWord + (size_t)kBucketChunks * 1024);

// Token tiles of the matrix-core expert FFN: up to kUnitM tokens of one
// expert per tile; a remainder of at most kUnitSmall tokens is a one-block tile
// (when experts average few tokens; otherwise every tile is full-size).
constexpr int kUnitM = 64;
constexpr int kUnitSmall = 16;
moe_status launch_bucket(moe_ctx *ctx, const int32_t *idx, int T, int k, int E, int32_t *counts, int32_t *offsets,
                         int32_t *perm, const uint8_t *expert_bits, int want_bits, int32_t *active,
                         int32_t *n_active, int2 *units, int32_t *n_units, int ubig_max, int has_shared,
                         int small_max);
bool expert_ffn_mfma_supported(int bits, int H, int I);
// Scratch bytes (moe_scratch) a launcher takes for these arguments: the same
// layouts the launchers use, so a caller can size a fixed area beforehand.
size_t router_scratch_bytes(const moe_ctx *ctx, const moe_router_cfg *cfg, int T, int H);
size_t expert_ffn_scratch_bytes(const moe_ctx *ctx, int bits, int has_shared, int T, int H, int I, int E, int k);
size_t expert_ffn_mfma_scratch_bytes(int bits, int has_shared, int T, int H, int I, int E, int k);
size_t layer_t1_scratch_bytes(const moe_ctx *ctx, const moe_router_cfg *cfg, int has_shared, int H, int I);
size_t ffn_t1_scratch_bytes(int I, int S);
moe_status launch_expert_ffn_mfma(moe_ctx *ctx, int bits, const moe_expert_w *experts, const moe_expert_w *shared,
                                  const uint8_t *expert_bits, const int8_t *xq, const float *sx,
                                  const int32_t *topk_idx, int T, int H, int I, int E, int k, float *y_slots);
moe_status launch_combine(moe_ctx *ctx, const float *y_slots, const float *topk_w, int T, int k, int H,
                          int has_shared, float *out);
bool decode_t1_supported(int bits, int H, int I, int k, int has_shared, int n_cu);
moe_status launch_layer_t1(moe_ctx *ctx, int bits, const moe_router_cfg *cfg, const float *x, const float *logits,
                           const float *w_router, const float *bias, const moe_expert_w *experts,
                           const moe_expert_w *shared, int H, int I, float *out, int32_t *topk_idx, float *topk_w,
                           int8_t *xq, float *sx, float *y_slots);
moe_status launch_ffn_t1(moe_ctx *ctx, int bits, const moe_expert_w *experts, const moe_expert_w *shared,
                         const uint8_t *expert_bits, const int8_t *xq, const float *sx, const int32_t *topk_idx,
                         int H, int I, int E, int k, float *y_slots);
// xf (nullable): the token's fp32 row, quantised inside the gate/up kernels
// (xq and sx are then unused)
moe_status launch_ffn_t1_mixed(moe_ctx *ctx, const int *widths, int n_widths, int shared_bits,
                               const moe_expert_w *experts, const moe_expert_w *shared, const uint8_t *expert_bits,
                               const int8_t *xq, const float *sx, const float *xf, const int32_t *topk_idx,
                               const float *topk_w, int H, int I, int E, int k, float *y_slots, float *out);

// ---------------------------------------------------------------------------
// Device side
// ---------------------------------------------------------------------------
#if defined(__HIPCC__)

#define MOE_WAVE 64

// float32 exp by Cody-Waite argument reduction: x = n*ln2 + r with
// n = rint(x*log2(e)), |r| <= ln2/2, ln2 split into a 16-fractional-bit head
// (45426/65536, exact) and an fp32 tail; e^r by its degree-7 Taylor
// polynomial in Horner form with fused multiply-adds; result = p * 2^n.
// Every step is a correctly rounded fp32 operation.
__device__ __forceinline__ float moe_exp_f32(float x) {
  constexpr double kLn2 = 0.69314718055994530941723212145818;
  constexpr float kLn2Hi = (float)(45426.0 / 65536.0);
  constexpr float kLn2Lo = (float)(kLn2 - 45426.0 / 65536.0);
  constexpr float kLog2e = (float)1.4426950408889634073599246810019;
  if (x != x) return x;
  if (x > 88.75f) return __builtin_inff();
  if (x < -104.0f) return 0.0f;
  const float n = __builtin_rintf(x * kLog2e);
  float r = __builtin_fmaf(-n, kLn2Hi, x);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float p = (float)(1.0 / 5040.0);
  p = __builtin_fmaf(p, r, (float)(1.0 / 720.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, (int)n);
}

// silu(g) = g / (1 + e^-g), correctly rounded fp32 add and divide.
__device__ __forceinline__ float moe_silu_f32(float g) {
  const float d = 1.0f + moe_exp_f32(-g);
  return g / d;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
  return v;
}

// signed 4 x int8 dot product accumulate (v_dot4_i32_i8)
__device__ __forceinline__ int sdot4(int a, int b, int c) { return __builtin_amdgcn_sdot4(a, b, c, false); }

// Per-width constants of the packed formats.
template <int BITS>
struct QFmt;
template <>
struct QFmt<8> {
  static constexpr int kOff = 0;     // code offset (two's complement)
  static constexpr int kEpc = 16;    // elements per 16-byte chunk
};
template <>
struct QFmt<4> {
  static constexpr int kOff = 8;     // nibble = q + 8
  static constexpr int kEpc = 32;
};
template <>
struct QFmt<2> {
  static constexpr int kOff = 2;     // field = q + 2
  static constexpr int kEpc = 64;
};

// Reorder the int8 activation bytes of one 16-byte chunk's worth of elements
// so that they line up with the unpacked weight fields:
//  - int4: a weight dword holds elements 8m..8m+7 as nibbles; (w & 0x0f0f0f0f)
//    yields elements {0,2,4,6} and ((w>>4) & 0x0f0f0f0f) yields {1,3,5,7}, so
//    the activation 8-byte group (x0..x7) is stored as (x0,x2,x4,x6 | x1,x3,x5,x7).
//  - int2: a weight dword holds elements 16m..16m+15 as 2-bit fields; field j
//    of every byte, (w >> 2j) & 0x03030303, yields elements {j,4+j,8+j,12+j},
//    so the 16-byte group is stored as 4 dwords (x_j, x_{4+j}, x_{8+j}, x_{12+j}).
//  - int8: natural order.
// perm_b32(hi, lo, sel): byte i of the result = byte sel_i of {hi:lo}
// (selectors 0-3 pick lo's bytes, 4-7 hi's).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// int4: 8 activation bytes (a = x0..x3, b = x4..x7) -> (even, odd)
__device__ __forceinline__ void act_order_q4(uint32_t a, uint32_t b, uint32_t &ev, uint32_t &od) {
  ev = perm_b32(b, a, 0x06040200u);  // x0, x2, x4, x6
  od = perm_b32(b, a, 0x07050301u);  // x1, x3, x5, x7
}
// int2: 16 activation bytes d0..d3 -> o0..o3 with oj = (x_j, x_{4+j}, x_{8+j}, x_{12+j})
__device__ __forceinline__ void act_order_q2(const uint32_t d[4], uint32_t o[4]) {
  // first gather byte j of d0,d1 and of d2,d3, then merge
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sel01 = (uint32_t)j | ((uint32_t)(4 + j) << 8);  // d0.byte j, d1.byte j in bytes 0,1
    const uint32_t lo = perm_b32(d[1], d[0], sel01 | 0x0c0c0000u);  // bytes 2,3 = 0
    const uint32_t hi = perm_b32(d[3], d[2], sel01 | 0x0c0c0000u);
    o[j] = perm_b32(hi, lo, 0x05040100u);                           // lo.b0, lo.b1, hi.b0, hi.b1
  }
}

#endif  // __HIPCC__
