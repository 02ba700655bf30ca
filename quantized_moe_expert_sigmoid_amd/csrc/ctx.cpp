// Context, error reporting, argument validation and the exported C ABI.
// Kernels live in the .hip files; every entry point here validates its
// arguments completely before anything is enqueued.
#include <algorithm>
#include <mutex>
#include <new>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "moe_internal.h"

static thread_local char g_err[512] = "";

moe_status moe_fail(moe_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

moe_status moe_hip_fail(hipError_t e, const char *what) {
  (void)hipGetLastError();  // clear the sticky launch error
  return moe_fail(e == hipErrorOutOfMemory ? MOE_ENOMEM : MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

extern "C" const char *moe_last_error(void) { return g_err; }
extern "C" int moe_abi_version(void) { return MOE_ABI_VERSION; }

// Scratch grows by allocating a larger buffer; the one it replaces is kept
// until moe_ctx_destroy, never freed earlier: a HIP graph captured from
// earlier calls holds its address, and so may work still queued on the
// stream, so freeing it would turn a later replay into a use of freed memory.
static moe_status grow(moe_ctx *ctx, void **buf, size_t *have, size_t bytes, void **out) {
  if (bytes > *have) {
    const size_t want = moe_round_up(bytes + bytes / 4, 1 << 20);
    void *p = nullptr;
    MOE_HIP(hipMalloc(&p, want));
    if (*buf) ctx->retired.push_back(*buf);
    *buf = p;
    *have = want;
  }
  *out = *buf;
  return MOE_OK;
}

moe_status moe_scratch(moe_ctx *ctx, size_t bytes, void **out) {
  if (ctx->fixed_scr) {  // an allocation-free call: its region of the static array
    if (bytes > ctx->fixed_scr_bytes)
      return moe_fail(MOE_EINVAL, "allocation-free call: %zu scratch bytes needed, %zu reserved", bytes,
                      ctx->fixed_scr_bytes);
    *out = ctx->fixed_scr;
    return MOE_OK;
  }
  return grow(ctx, &ctx->scratch, &ctx->scratch_bytes, bytes, out);
}

moe_status moe_io_scratch(moe_ctx *ctx, size_t bytes, void **out) {
  if (ctx->fixed_io) {
    if (bytes > ctx->fixed_io_bytes)
      return moe_fail(MOE_EINVAL, "allocation-free call: %zu io bytes needed, %zu reserved", bytes,
                      ctx->fixed_io_bytes);
    *out = ctx->fixed_io;
    return MOE_OK;
  }
  return grow(ctx, &ctx->io, &ctx->io_bytes, bytes, out);
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: one static device array per
// GPU (the code object's own global, resident until the process ends). Host
// code never uses the array's name as an address: moe_ctx_create takes the
// device address of each GPU's copy once, with that device current, and the
// allocation-free call hands that address to the launchers.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char noalloc_scratch[kNoAllocBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_noalloc_mu;
static void *g_noalloc_ptr[kMaxDevices];

// With `device` current: record the device address of its copy of the array.
static moe_status noalloc_bind(int device) {
  if (device < 0 || device >= kMaxDevices)
    return moe_fail(MOE_EUNSUPPORTED, "moe_ctx_create: device %d beyond the %d the library tracks", device,
                    kMaxDevices);
  std::lock_guard<std::mutex> g(g_noalloc_mu);
  if (g_noalloc_ptr[device]) return MOE_OK;
  void *p = nullptr;
  MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch)));
  if (!p) return moe_fail(MOE_EHIP, "hipGetSymbolAddress(noalloc_scratch) returned NULL");
  g_noalloc_ptr[device] = p;
  return MOE_OK;
}

static void *noalloc_ptr(int device) {
  std::lock_guard<std::mutex> g(g_noalloc_mu);
  return (device >= 0 && device < kMaxDevices) ? g_noalloc_ptr[device] : nullptr;
}

extern "C" moe_status moe_ctx_create(int device, void *hip_stream, moe_ctx **out) {
  if (!out) return moe_fail(MOE_EINVAL, "moe_ctx_create: out is NULL");
  *out = nullptr;
  int n = 0;
  MOE_HIP(hipGetDeviceCount(&n));
  if (device < 0 || device >= n) return moe_fail(MOE_EINVAL, "moe_ctx_create: device %d of %d", device, n);
  MOE_HIP(hipSetDevice(device));
  hipDeviceProp_t prop;
  MOE_HIP(hipGetDeviceProperties(&prop, device));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return moe_fail(MOE_EUNSUPPORTED, "moe_ctx_create: device %d is %s, this library is built for gfx950", device,
                    prop.gcnArchName);
  moe_status st = noalloc_bind(device);
  if (st) return st;
  moe_ctx *c = new (std::nothrow) moe_ctx();
  if (!c) return moe_fail(MOE_ENOMEM, "moe_ctx_create: host allocation");
  c->device = device;
  c->stream = (hipStream_t)hip_stream;
  c->n_cu = prop.multiProcessorCount;
  hipError_t e = hipMalloc(&c->dev_small, kDevSmallBytes);
  if (e != hipSuccess) {
    delete c;
    return moe_hip_fail(e, "hipMalloc(ctx counters)");
  }
  e = hipMemset(c->dev_small, 0, kDevSmallBytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  // the side stream and its events exist from the start, so no later call
  // (the allocation-free one included) creates them
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming);
  if (e != hipSuccess) {
    if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
    if (c->side) (void)hipStreamDestroy(c->side);
    (void)hipFree(c->dev_small);
    delete c;
    return moe_hip_fail(e, "moe_ctx_create: counters, side stream and events");
  }
  *out = c;
  return MOE_OK;
}

moe_status moe_side_fork(moe_ctx *ctx) {
  MOE_HIP(hipEventRecord(ctx->ev_fork, ctx->stream));
  MOE_HIP(hipStreamWaitEvent(ctx->side, ctx->ev_fork, 0));
  return MOE_OK;
}

moe_status moe_side_join(moe_ctx *ctx) {
  MOE_HIP(hipEventRecord(ctx->ev_join, ctx->side));
  MOE_HIP(hipStreamWaitEvent(ctx->stream, ctx->ev_join, 0));
  return MOE_OK;
}

hipEvent_t moe_timing_event(moe_ctx *ctx) {
  if (!ctx->event_pool.empty()) {
    hipEvent_t e = ctx->event_pool.back();
    ctx->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

MoeTimer::MoeTimer(moe_ctx *c, int s) : ctx(c), stage(s) {
  if (!ctx->timing) return;
  start = moe_timing_event(ctx);
  if (start && hipEventRecord(start, ctx->stream) != hipSuccess) {
    ctx->event_pool.push_back(start);
    start = nullptr;
  }
}

MoeTimer::~MoeTimer() {
  if (!start) return;
  hipEvent_t stop = moe_timing_event(ctx);
  if (stop && hipEventRecord(stop, ctx->stream) == hipSuccess) {
    ctx->timed.push_back({start, stop, stage});
  } else {
    ctx->event_pool.push_back(start);
    if (stop) ctx->event_pool.push_back(stop);
  }
}

extern "C" moe_status moe_ctx_set_ffn_kernels(moe_ctx *ctx, int which) {
  if (!ctx) return moe_fail(MOE_EINVAL, "moe_ctx_set_ffn_kernels: ctx is NULL");
  if (which != MOE_FFN_AUTO && which != MOE_FFN_DOT4 && which != MOE_FFN_MFMA)
    return moe_fail(MOE_EINVAL, "moe_ctx_set_ffn_kernels: %d is not MOE_FFN_AUTO, _DOT4 or _MFMA", which);
  ctx->ffn_kernels = which;
  return MOE_OK;
}

extern "C" moe_status moe_ctx_enable_timing(moe_ctx *ctx, int enable) {
  if (!ctx) return moe_fail(MOE_EINVAL, "moe_ctx_enable_timing: ctx is NULL");
  ctx->timing = enable != 0;
  return MOE_OK;
}

extern "C" moe_status moe_ctx_read_timing(moe_ctx *ctx, double *ms_host, int *n_host) {
  if (!ctx) return moe_fail(MOE_EINVAL, "moe_ctx_read_timing: ctx is NULL");
  MOE_HIP(hipSetDevice(ctx->device));
  double ms[MOE_N_STAGES] = {};
  int n[MOE_N_STAGES] = {};
  moe_status st = MOE_OK;
  for (auto &t : ctx->timed) {
    float v = 0.0f;
    hipError_t e = hipEventSynchronize(t.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&v, t.start, t.stop);
    if (e != hipSuccess && st == MOE_OK) st = moe_hip_fail(e, "hipEventElapsedTime");
    if (t.stage >= 0 && t.stage < MOE_N_STAGES) {
      ms[t.stage] += v;
      n[t.stage] += 1;
    }
    ctx->event_pool.push_back(t.start);
    ctx->event_pool.push_back(t.stop);
  }
  ctx->timed.clear();
  for (int i = 0; i < MOE_N_STAGES; ++i) {
    if (ms_host) ms_host[i] = ms[i];
    if (n_host) n_host[i] = n[i];
  }
  return st;
}

extern "C" void moe_ctx_destroy(moe_ctx *ctx) {
  if (!ctx) return;
  (void)hipSetDevice(ctx->device);
  (void)hipStreamSynchronize(ctx->stream);
  if (ctx->side) {
    (void)hipStreamSynchronize(ctx->side);
    (void)hipStreamDestroy(ctx->side);
    (void)hipEventDestroy(ctx->ev_fork);
    (void)hipEventDestroy(ctx->ev_join);
  }
  for (auto &t : ctx->timed) {
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  for (auto e : ctx->event_pool) (void)hipEventDestroy(e);
  if (ctx->scratch) (void)hipFree(ctx->scratch);
  if (ctx->io) (void)hipFree(ctx->io);
  for (void *p : ctx->retired) (void)hipFree(p);
  if (ctx->dev_small) (void)hipFree(ctx->dev_small);
  delete ctx;
}

extern "C" moe_status moe_ctx_set_stream(moe_ctx *ctx, void *hip_stream) {
  if (!ctx) return moe_fail(MOE_EINVAL, "moe_ctx_set_stream: ctx is NULL");
  ctx->stream = (hipStream_t)hip_stream;
  return MOE_OK;
}

extern "C" moe_status moe_ctx_check(moe_ctx *ctx) {
  if (!ctx) return moe_fail(MOE_EINVAL, "moe_ctx_check: ctx is NULL");
  MOE_HIP(hipSetDevice(ctx->device));
  MOE_HIP(hipStreamSynchronize(ctx->stream));
  uint32_t flags = 0;
  MOE_HIP(hipMemcpy(&flags, ctx->dev_small, sizeof flags, hipMemcpyDeviceToHost));
  if (flags) {
    uint32_t zero = 0;
    MOE_HIP(hipMemcpy(ctx->dev_small, &zero, sizeof zero, hipMemcpyHostToDevice));
    if (flags & ERRF_TIMEOUT) return moe_fail(MOE_ETIMEOUT, "device: a bounded wait gave up (flags 0x%x)", flags);
    if (flags & ERRF_BAD_INDEX) return moe_fail(MOE_EINVAL, "device: expert index out of range (flags 0x%x)", flags);
    return moe_fail(MOE_EINVAL, "device: error flags 0x%x", flags);
  }
  return MOE_OK;
}

extern "C" moe_status moe_ctx_set_debug(moe_ctx *ctx, const moe_debug_bufs *dbg) {
  if (!ctx) return moe_fail(MOE_EINVAL, "moe_ctx_set_debug: ctx is NULL");
  if (dbg) {
    ctx->dbg = *dbg;
    ctx->dbg_on = true;
  } else {
    ctx->dbg = moe_debug_bufs{};
    ctx->dbg_on = false;
  }
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Validation helpers
// ---------------------------------------------------------------------------

static bool dim_ok(int v) { return v > 0 && v % 64 == 0 && v <= 8192; }

#define REQUIRE(cond, ...)                                 \
  do {                                                     \
    if (!(cond)) return moe_fail(MOE_EINVAL, __VA_ARGS__); \
  } while (0)

static moe_status bind(moe_ctx *ctx, const char *fn) {
  if (!ctx) return moe_fail(MOE_EINVAL, "%s: ctx is NULL", fn);
  MOE_HIP(hipSetDevice(ctx->device));
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Exported entry points
// ---------------------------------------------------------------------------

extern "C" moe_status moe_quantize_rows(moe_ctx *ctx, int bits, const float *w, int64_t rows, int cols,
                                        uint8_t *packed, float *scales) {
  moe_status st = bind(ctx, "moe_quantize_rows");
  if (st) return st;
  REQUIRE(bits == 8 || bits == 4 || bits == 2, "moe_quantize_rows: bits %d not in {8,4,2}", bits);
  REQUIRE(cols > 0 && cols % 64 == 0 && cols <= (1 << 20), "moe_quantize_rows: cols %d", cols);
  REQUIRE(rows >= 0 && rows <= (int64_t)1 << 31, "moe_quantize_rows: rows %lld", (long long)rows);
  if (rows == 0) return MOE_OK;
  REQUIRE(w && packed && scales, "moe_quantize_rows: NULL pointer");
  REQUIRE(moe_aligned16(w) && moe_aligned16(packed), "moe_quantize_rows: pointers must be 16-byte aligned");
  return launch_quantize_rows(ctx, bits, w, rows, cols, packed, scales);
}

extern "C" moe_status moe_quantize_act_i8(moe_ctx *ctx, const float *x, int T, int H, int8_t *xq, float *sx) {
  moe_status st = bind(ctx, "moe_quantize_act_i8");
  if (st) return st;
  REQUIRE(T >= 0, "moe_quantize_act_i8: T %d", T);
  REQUIRE(dim_ok(H), "moe_quantize_act_i8: H %d must be a positive multiple of 64, <= 8192", H);
  if (T == 0) return MOE_OK;
  REQUIRE(x && xq && sx, "moe_quantize_act_i8: NULL pointer");
  REQUIRE(moe_aligned16(x) && moe_aligned16(xq), "moe_quantize_act_i8: pointers must be 16-byte aligned");
  return launch_quantize_act(ctx, x, T, H, xq, sx);
}

extern "C" moe_status moe_router_topk(moe_ctx *ctx, const moe_router_cfg *cfg, const float *x, const float *w_router,
                                      const float *bias, int T, int H, int32_t *topk_idx, float *topk_w) {
  moe_status st = bind(ctx, "moe_router_topk");
  if (st) return st;
  REQUIRE(cfg, "moe_router_topk: cfg is NULL");
  REQUIRE(cfg->n_experts >= 1 && cfg->n_experts <= 1024, "moe_router_topk: n_experts %d", cfg->n_experts);
  REQUIRE(cfg->top_p == cfg->top_p, "moe_router_topk: top_p is NaN");
  REQUIRE(cfg->top_k >= 1 && cfg->top_k <= 16 && cfg->top_k <= cfg->n_experts, "moe_router_topk: top_k %d",
          cfg->top_k);
  REQUIRE(T >= 0, "moe_router_topk: T %d", T);
  if (!cfg->logits_in) {
    REQUIRE(dim_ok(H), "moe_router_topk: H %d must be a positive multiple of 64, <= 8192", H);
    REQUIRE(w_router, "moe_router_topk: w_router is NULL");
    REQUIRE(moe_aligned16(w_router), "moe_router_topk: w_router must be 16-byte aligned");
  }
  if (T == 0) return MOE_OK;
  REQUIRE(x && topk_idx && topk_w, "moe_router_topk: NULL pointer");
  REQUIRE(moe_aligned16(x), "moe_router_topk: x must be 16-byte aligned");
  return launch_router(ctx, cfg, x, w_router, bias, T, H, topk_idx, topk_w);
}

extern "C" moe_status moe_bucket_tokens(moe_ctx *ctx, const int32_t *topk_idx, int T, int k, int E, int32_t *counts,
                                        int32_t *offsets, int32_t *perm) {
  moe_status st = bind(ctx, "moe_bucket_tokens");
  if (st) return st;
  REQUIRE(T >= 0 && k >= 1 && k <= 16 && E >= 1 && E <= 1024, "moe_bucket_tokens: T %d k %d E %d", T, k, E);
  REQUIRE((int64_t)T * k <= (1 << 24), "moe_bucket_tokens: T*k too large");
  REQUIRE(counts && offsets && (T == 0 || (topk_idx && perm)), "moe_bucket_tokens: NULL pointer");
  return launch_bucket_public(ctx, topk_idx, T, k, E, counts, offsets, perm);
}

// Argument checks of the expert FFN entry points (T == 0 passes: nothing to do).
static moe_status ffn_check(const char *fn, moe_ctx *ctx, const moe_expert_w *experts, const moe_expert_w *shared,
                            const int8_t *xq, const float *sx, const int32_t *topk_idx, int T, int H, int I, int E,
                            int k, float *y_slots) {
  moe_status st = bind(ctx, fn);
  if (st) return st;
  REQUIRE(T >= 0, "%s: T %d", fn, T);
  REQUIRE(dim_ok(H) && dim_ok(I), "%s: H %d and I %d must be positive multiples of 64, <= 8192", fn, H, I);
  REQUIRE(E >= 1 && E <= 1024 && k >= 1 && k <= 16 && k <= E, "%s: E %d k %d", fn, E, k);
  REQUIRE((int64_t)T * (k + 1) <= (1 << 22), "%s: T*(k+1) too large", fn);
  if (T == 0) return MOE_OK;
  REQUIRE(experts && xq && sx && topk_idx && y_slots, "%s: NULL pointer", fn);
  REQUIRE(moe_aligned16(xq) && moe_aligned16(y_slots), "%s: xq and y_slots must be 16-byte aligned", fn);
  if (shared) {
    REQUIRE(shared->gate && shared->up && shared->down && shared->s_gate && shared->s_up && shared->s_down,
            "%s: shared expert has a NULL member", fn);
    REQUIRE(moe_aligned16(shared->gate) && moe_aligned16(shared->up) && moe_aligned16(shared->down),
            "%s: shared expert weights must be 16-byte aligned", fn);
  }
  return MOE_OK;
}

static moe_status ffn_entry(const char *fn, int bits, moe_ctx *ctx, const moe_expert_w *experts,
                            const moe_expert_w *shared, const uint8_t *expert_bits, const int8_t *xq, const float *sx,
                            const int32_t *topk_idx, int T, int H, int I, int E, int k, float *y_slots) {
  moe_status st = ffn_check(fn, ctx, experts, shared, xq, sx, topk_idx, T, H, I, E, k, y_slots);
  if (st || T == 0) return st;
  return launch_expert_ffn(ctx, bits, experts, shared, expert_bits, xq, sx, topk_idx, T, H, I, E, k, y_slots);
}

// The mixed-width call on codes (xq, sx) or, with xf, on fp32 hidden states:
// a single token on the single-token kernels quantises inside its gate/up
// kernel; otherwise the rows are quantised into the context's io scratch first.
static moe_status ffn_mixed(const char *fn, moe_ctx *ctx, const moe_expert_w *experts, const moe_expert_w *shared,
                            int shared_bits, const uint8_t *expert_bits, int widths_mask, const int8_t *xq,
                            const float *sx, const float *xf, const int32_t *topk_idx, const float *topk_w, int T,
                            int H, int I, int E, int k, float *y_slots, float *out) {
  // ffn_check wants codes; with xf it checks xf in their place
  const void *xin = xf ? (const void *)xf : (const void *)xq;
  moe_status st = ffn_check(fn, ctx, experts, shared, static_cast<const int8_t *>(xin), xf ? xf : sx, topk_idx, T, H,
                            I, E, k, y_slots);
  if (st) return st;
  const int all = (1 << 8) | (1 << 4) | (1 << 2);
  REQUIRE(widths_mask != 0 && (widths_mask & ~all) == 0, "%s: widths_mask 0x%x (bits 8, 4 and 2 only)", fn,
          widths_mask);
  REQUIRE(!shared || shared_bits == 8 || shared_bits == 4 || shared_bits == 2, "%s: shared_bits %d", fn, shared_bits);
  REQUIRE(expert_bits, "%s: expert_bits is NULL", fn);
  if (T == 0) return MOE_OK;
  REQUIRE(!out || topk_w, "%s: out needs topk_w", fn);
  REQUIRE(!out || moe_aligned16(out), "%s: out must be 16-byte aligned", fn);
  int widths[3], n = 0;
  bool t1 = T == 1 && ctx->ffn_kernels == MOE_FFN_AUTO;
  for (int b : {8, 4, 2}) {
    const bool sh = shared && b == shared_bits;
    if (!(widths_mask & (1 << b)) && !sh) continue;
    widths[n++] = b;
    t1 = t1 && decode_t1_supported(b, H, I, k, sh ? 1 : 0, ctx->n_cu);
  }
  if (t1)
    return launch_ffn_t1_mixed(ctx, widths, n, shared_bits, experts, shared, expert_bits, xq, sx, xf, topk_idx,
                               topk_w, H, I, E, k, y_slots, out);
  if (xf) {  // codes of every row first, into the io scratch (the FFN launchers use the other scratch)
    void *io = nullptr;
    const size_t xq_bytes = moe_round_up((size_t)T * H, 256);
    if ((st = moe_io_scratch(ctx, xq_bytes + 4 * (size_t)T, &io))) return st;
    int8_t *xq_io = static_cast<int8_t *>(io);
    float *sx_io = reinterpret_cast<float *>(static_cast<char *>(io) + xq_bytes);
    if ((st = launch_quantize_act(ctx, xf, T, H, xq_io, sx_io))) return st;
    xq = xq_io;
    sx = sx_io;
  }
  for (int w = 0; w < n; ++w) {
    const moe_expert_w *sh = (shared && widths[w] == shared_bits) ? shared : nullptr;
    if ((st = launch_expert_ffn(ctx, widths[w], experts, sh, expert_bits, xq, sx, topk_idx, T, H, I, E, k, y_slots)))
      return st;
  }
  return out ? launch_combine(ctx, y_slots, topk_w, T, k, H, shared ? 1 : 0, out) : MOE_OK;
}

extern "C" moe_status moe_expert_ffn_mixed(moe_ctx *ctx, const moe_expert_w *experts, const moe_expert_w *shared,
                                           int shared_bits, const uint8_t *expert_bits, int widths_mask,
                                           const int8_t *xq, const float *sx, const int32_t *topk_idx,
                                           const float *topk_w, int T, int H, int I, int E, int k, float *y_slots,
                                           float *out) {
  return ffn_mixed("moe_expert_ffn_mixed", ctx, experts, shared, shared_bits, expert_bits, widths_mask, xq, sx,
                   nullptr, topk_idx, topk_w, T, H, I, E, k, y_slots, out);
}

extern "C" moe_status moe_expert_ffn_mixed_x(moe_ctx *ctx, const moe_expert_w *experts, const moe_expert_w *shared,
                                             int shared_bits, const uint8_t *expert_bits, int widths_mask,
                                             const float *x, const int32_t *topk_idx, const float *topk_w, int T,
                                             int H, int I, int E, int k, float *y_slots, float *out) {
  return ffn_mixed("moe_expert_ffn_mixed_x", ctx, experts, shared, shared_bits, expert_bits, widths_mask, nullptr,
                   nullptr, x, topk_idx, topk_w, T, H, I, E, k, y_slots, out);
}

extern "C" moe_status moe_expert_ffn_q4(moe_ctx *ctx, const moe_expert_w *experts, const moe_expert_w *shared,
                                        const uint8_t *expert_bits, const int8_t *xq, const float *sx,
                                        const int32_t *topk_idx, int T, int H, int I, int E, int k, float *y_slots) {
  return ffn_entry("moe_expert_ffn_q4", 4, ctx, experts, shared, expert_bits, xq, sx, topk_idx, T, H, I, E, k,
                   y_slots);
}
extern "C" moe_status moe_expert_ffn_q8(moe_ctx *ctx, const moe_expert_w *experts, const moe_expert_w *shared,
                                        const uint8_t *expert_bits, const int8_t *xq, const float *sx,
                                        const int32_t *topk_idx, int T, int H, int I, int E, int k, float *y_slots) {
  return ffn_entry("moe_expert_ffn_q8", 8, ctx, experts, shared, expert_bits, xq, sx, topk_idx, T, H, I, E, k,
                   y_slots);
}
extern "C" moe_status moe_expert_ffn_q2(moe_ctx *ctx, const moe_expert_w *experts, const moe_expert_w *shared,
                                        const uint8_t *expert_bits, const int8_t *xq, const float *sx,
                                        const int32_t *topk_idx, int T, int H, int I, int E, int k, float *y_slots) {
  return ffn_entry("moe_expert_ffn_q2", 2, ctx, experts, shared, expert_bits, xq, sx, topk_idx, T, H, I, E, k,
                   y_slots);
}

extern "C" moe_status moe_combine(moe_ctx *ctx, const float *y_slots, const float *topk_w, int T, int k, int H,
                                  int has_shared, float *out) {
  moe_status st = bind(ctx, "moe_combine");
  if (st) return st;
  REQUIRE(T >= 0 && k >= 1 && k <= 16, "moe_combine: T %d k %d", T, k);
  REQUIRE(dim_ok(H), "moe_combine: H %d must be a positive multiple of 64, <= 8192", H);
  if (T == 0) return MOE_OK;
  REQUIRE(y_slots && topk_w && out, "moe_combine: NULL pointer");
  REQUIRE(moe_aligned16(y_slots) && moe_aligned16(out), "moe_combine: pointers must be 16-byte aligned");
  return launch_combine(ctx, y_slots, topk_w, T, k, H, has_shared, out);
}

extern "C" size_t moe_expert_block_layout(int bits, int H, int I, size_t *offsets_host) {
  if (!(bits == 8 || bits == 4 || bits == 2) || H <= 0 || I <= 0 || H % 64 || I % 64) return 0;
  const size_t part[6] = {(size_t)I * H * bits / 8, (size_t)I * H * bits / 8, (size_t)H * I * bits / 8,
                          4 * (size_t)I, 4 * (size_t)I, 4 * (size_t)H};
  size_t off = 0;
  for (int i = 0; i < 6; ++i) {
    if (offsets_host) offsets_host[i] = off;
    off = moe_round_up(off + part[i], 256);
  }
  return off;
}

// Argument checks of the whole-layer entry points (T == 0 passes).
static moe_status layer_check(const char *fn, moe_ctx *ctx, int bits, const moe_router_cfg *cfg, const float *x,
                              const float *logits, const float *w_router, const moe_expert_w *experts,
                              const moe_expert_w *shared, int T, int H, int I, float *out, int8_t *xq,
                              float *y_slots) {
  moe_status st = bind(ctx, fn);
  if (st) return st;
  REQUIRE(bits == 8 || bits == 4 || bits == 2, "%s: bits %d not in {8,4,2}", fn, bits);
  REQUIRE(cfg, "%s: cfg is NULL", fn);
  REQUIRE(cfg->top_p == cfg->top_p, "%s: top_p is NaN", fn);
  const int E = cfg->n_experts, k = cfg->top_k;
  REQUIRE(E >= 1 && E <= 1024 && k >= 1 && k <= 16 && k <= E, "%s: E %d k %d", fn, E, k);
  REQUIRE(T >= 0 && (int64_t)T * (k + 1) <= (1 << 22), "%s: T %d", fn, T);
  REQUIRE(dim_ok(H) && dim_ok(I), "%s: H %d and I %d must be positive multiples of 64, <= 8192", fn, H, I);
  if (T == 0) return MOE_OK;
  REQUIRE(x && experts && out, "%s: NULL pointer", fn);
  REQUIRE(cfg->logits_in ? (logits != nullptr) : (w_router != nullptr),
          "%s: logits_in needs logits, otherwise w_router is required", fn);
  REQUIRE(moe_aligned16(x) && moe_aligned16(out) && (!xq || moe_aligned16(xq)) && (!y_slots || moe_aligned16(y_slots)),
          "%s: pointers must be 16-byte aligned", fn);
  REQUIRE(cfg->logits_in || moe_aligned16(w_router), "%s: w_router must be 16-byte aligned", fn);
  if (shared)
    REQUIRE(shared->gate && shared->up && shared->down && shared->s_gate && shared->s_up && shared->s_down,
            "%s: shared expert has a NULL member", fn);
  return MOE_OK;
}

static bool layer_is_t1(const moe_ctx *ctx, int bits, const moe_router_cfg *cfg, int T, int H, int I, int has_shared) {
  return T == 1 && decode_t1_supported(bits, H, I, cfg->top_k, has_shared, ctx->n_cu);
}

// io area of the composed path: the intermediates the caller did not ask for
struct LayerIo {
  size_t o_idx, o_w, o_xq, o_sx, o_y, size;
};
static LayerIo layer_io_layout(int T, int H, int k) {
  LayerIo l;
  MoeLayout m;
  l.o_idx = m.take(4 * (size_t)T * k);
  l.o_w = m.take(4 * (size_t)T * k);
  l.o_xq = m.take((size_t)T * H);
  l.o_sx = m.take(4 * (size_t)T);
  l.o_y = m.take(4 * (size_t)T * (k + 1) * H);
  l.size = m.size;
  return l;
}

// The layer's steps on the context stream (arguments already checked).
static moe_status layer_body(moe_ctx *ctx, int bits, const moe_router_cfg *cfg, const float *x, const float *logits,
                             const float *w_router, const float *bias, const moe_expert_w *experts,
                             const moe_expert_w *shared, int T, int H, int I, float *out, int32_t *topk_idx,
                             float *topk_w, int8_t *xq, float *sx, float *y_slots) {
  const int E = cfg->n_experts, k = cfg->top_k;
  const float *lg = cfg->logits_in ? logits : nullptr;
  if (layer_is_t1(ctx, bits, cfg, T, H, I, shared ? 1 : 0))
    return launch_layer_t1(ctx, bits, cfg, x, lg, w_router, bias, experts, shared, H, I, out, topk_idx, topk_w, xq, sx,
                           y_slots);
  const LayerIo l = layer_io_layout(T, H, k);
  void *io = nullptr;
  moe_status st = moe_io_scratch(ctx, l.size, &io);
  if (st) return st;
  char *b = static_cast<char *>(io);
  if (!topk_idx) topk_idx = reinterpret_cast<int32_t *>(b + l.o_idx);
  if (!topk_w) topk_w = reinterpret_cast<float *>(b + l.o_w);
  if (!xq) xq = reinterpret_cast<int8_t *>(b + l.o_xq);
  if (!sx) sx = reinterpret_cast<float *>(b + l.o_sx);
  if (!y_slots) y_slots = reinterpret_cast<float *>(b + l.o_y);
  if ((st = launch_quantize_act(ctx, x, T, H, xq, sx))) return st;
  if ((st = launch_router(ctx, cfg, lg ? lg : x, w_router, bias, T, H, topk_idx, topk_w))) return st;
  if ((st = launch_expert_ffn(ctx, bits, experts, shared, nullptr, xq, sx, topk_idx, T, H, I, E, k, y_slots)))
    return st;
  return launch_combine(ctx, y_slots, topk_w, T, k, H, shared ? 1 : 0, out);
}

extern "C" moe_status moe_layer_forward(moe_ctx *ctx, int bits, const moe_router_cfg *cfg, const float *x,
                                        const float *logits, const float *w_router, const float *bias,
                                        const moe_expert_w *experts, const moe_expert_w *shared, int T, int H, int I,
                                        float *out, int32_t *topk_idx, float *topk_w, int8_t *xq, float *sx,
                                        float *y_slots) {
  moe_status st = layer_check("moe_layer_forward", ctx, bits, cfg, x, logits, w_router, experts, shared, T, H, I, out,
                              xq, y_slots);
  if (st || T == 0) return st;
  return layer_body(ctx, bits, cfg, x, logits, w_router, bias, experts, shared, T, H, I, out, topk_idx, topk_w, xq,
                    sx, y_slots);
}

// Clears a context's fixed scratch regions when the allocation-free call returns.
struct FixedScratchScope {
  moe_ctx *c;
  ~FixedScratchScope() {
    c->fixed_io = c->fixed_scr = nullptr;
    c->fixed_io_bytes = c->fixed_scr_bytes = 0;
  }
};

extern "C" moe_status moe_layer_forward_noalloc(moe_ctx *ctx, int bits, const moe_router_cfg *cfg, const float *x,
                                                const float *logits, const float *w_router, const float *bias,
                                                const moe_expert_w *experts, const moe_expert_w *shared, int T,
                                                int H, int I, float *out, int32_t *topk_idx, float *topk_w,
                                                int8_t *xq, float *sx, float *y_slots) {
  const char *fn = "moe_layer_forward_noalloc";
  moe_status st = layer_check(fn, ctx, bits, cfg, x, logits, w_router, experts, shared, T, H, I, out, xq, y_slots);
  if (st || T == 0) return st;
  REQUIRE(!ctx->timing, "%s: per-kernel timing records events, which allocates; switch timing off", fn);
  const int has_shared = shared ? 1 : 0;
  size_t io = 0, scr = 0;
  if (layer_is_t1(ctx, bits, cfg, T, H, I, has_shared)) {
    scr = layer_t1_scratch_bytes(ctx, cfg, has_shared, H, I);
  } else {
    io = layer_io_layout(T, H, cfg->top_k).size;
    scr = std::max(router_scratch_bytes(ctx, cfg, T, H),
                   expert_ffn_scratch_bytes(ctx, bits, has_shared, T, H, I, cfg->n_experts, cfg->top_k));
  }
  REQUIRE(io + scr <= kNoAllocBytes,
          "%s: T %d, H %d, I %d, E %d, k %d needs %zu bytes of scratch; the static area holds %zu", fn, T, H, I,
          cfg->n_experts, cfg->top_k, io + scr, kNoAllocBytes);
  char *base = static_cast<char *>(noalloc_ptr(ctx->device));
  if (!base) return moe_fail(MOE_EHIP, "%s: no static scratch address for device %d", fn, ctx->device);
  FixedScratchScope scope{ctx};
  ctx->fixed_io = base;
  ctx->fixed_io_bytes = io;
  ctx->fixed_scr = base + io;
  ctx->fixed_scr_bytes = kNoAllocBytes - io;
  return layer_body(ctx, bits, cfg, x, logits, w_router, bias, experts, shared, T, H, I, out, topk_idx, topk_w, xq,
                    sx, y_slots);
}
