// Single-token (decode) layer path in three kernels: router logits and the
// activation quantisation; top-k fused with a streaming gate/up GEMV; the int8
// requantisation of the SwiGLU intermediate fused with the down GEMV and the
// combine.
//
// Pages: agentlenshq.com, "Colibri: running GLM-5.2 744B MoE on consumer
// hardware", section "Key features" (packed int4/int8/int2 with per-row
// scales, dequantisation on use, integer-dot matmuls) and section "Memory
// split" (always-on shared expert); tech.takumi3488.com, "Trying colibri"
// (DeepSeek-V3-family router, top-8 of 256); remio.ai, "Colibri shows how to
// run GLM-5.2 on a low-spec PC", section "How Colibri runs GLM-5.2" (a few
// experts per token, mixed into the output).
//
// One token per call means one (token, slot) pair per selected expert, so the
// kernels work on "slots": slot j < k is the j-th ranked expert, slot k the
// shared expert.
//  K1 router_gemv_t1_kernel: E/4 x KS workgroups compute K-slices of the
//     logits (one wave per expert and slice); KS more workgroups (the last
//     column) find max|x| over the token and quantise one slice of x each.
//  K2 gateup_t1_kernel (one 512-thread workgroup per CU): every wave first
//     issues the loads of its share of the shared expert's gate/up rows (known
//     before routing); meanwhile every workgroup sums the logit slices in fixed
//     order, applies the sigmoid and the bias, and one wave selects the top-k
//     (k rounds of a DPP wave max over order-preserving integer keys; equal
//     keys go to the lower id) and builds the slot table in LDS; workgroup 0
//     also publishes ids, weights and the slot table. Then the k*I routed
//     (gate row, up row) pairs, split into equal contiguous ranges over all
//     waves, stream through 16-byte loads two batches deep against the token's
//     int8 activations held in registers (field order); DPP reductions; one
//     store of a = silu(g)*u per row pair.
//  K3 down_combine_t1_kernel (one 512-thread workgroup per CU): the
//     workgroup loads every slot's a (the first down rows of every slot go
//     out right behind it) and requantises it while those rows are in
//     flight: max|a| per slot, the scale, the int8 codes (in the packed
//     weights' field order, into LDS) and their sums. Each wave then
//     multiplies its rows of every slot's down matrix (one row in flight
//     ahead), writes y per slot and the combined output
//     out[r] = y_shared + sum_j w_j y_j (the same fma order as moe_combine).
//     A CU keeps only some tens of KB of loads in flight and a wave that
//     queues more stalls at issue, so the kernels queue about that much at a
//     time.
// The per-step expert FFN of one token (routing given by the caller) runs K2
// and K3 without K1 and without the combine: K2 then builds the slot table
// from the given ids instead of the top-k, keeping only the slots whose expert
// has the call's width (the others, and ids of -1, are left to their own
// call), and K3 writes y of those slots and of the shared expert only.
// Kernel boundaries order the three steps: no atomics across workgroups, no
// cross-workgroup waits (contended device-scope atomics serialise at the
// memory side). Streaming loads are branch-free: a lane whose chunk index
// passes the row end reads a clamped in-bounds address and meets zero
// activation bytes.
#include <cstdlib>

#include "gemv_common.h"

namespace {

constexpr int kThreads = 256;                      // router kernel
constexpr int kFfnThreads = 512;                   // gate/up and down kernels
constexpr int kFfnWaves = kFfnThreads / MOE_WAVE;  // 8 waves: one workgroup per CU
constexpr int kMaxSlots = 9;                       // top-k <= 8 plus the shared expert
constexpr int kMaxSlices = 16;                     // K slices of the router logits
constexpr int kMaxE = 1024;
constexpr int kMaxX4 = 8;        // float4 of x per thread in the max pass: H <= 8192
constexpr int kMaxIDown = 4096;            // intermediate held in LDS by the down kernel
constexpr int kMaxPairsWg = kFfnThreads;  // routed row pairs per gate/up workgroup (one per thread)
constexpr int MOE_WAVE_HOST = 64;          // lanes per wave, for host-side shape choices

// One slot of the token: the expert's weights and its routing weight.
struct SlotEntry {
  moe_expert_w w;
  float weight;  // routing weight (1 for the shared expert)
  int expert;    // expert id (-1 for the shared expert and for slots dropped by top-p)
  int pad[2];
};
static_assert(sizeof(SlotEntry) == 64, "slot entries are 64 bytes");

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename P>
__device__ __forceinline__ P readlane_p(P p, int l) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return (P)(((uint64_t)hi << 32) | lo);
}
template <typename P>
__device__ __forceinline__ P uniform_p(P p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (P)(((uint64_t)hi << 32) | lo);
}

// The activation chunk a lane meets in a packed row of cpr chunks (zero past
// the row end), and its byte sum.
template <int BITS>
__device__ __forceinline__ void act_chunk_clamped(const int8_t *row, int c, int cpr, ActChunk<BITS> &o, int &bs) {
  const bool in = c < cpr;
  load_act_chunk<BITS>(row, in ? c : cpr - 1, o, bs);
  if (!in) {
    zero_chunk<BITS>(o);
    bs = 0;
  }
}

// ---------------------------------------------------------------------------
// K1: router logits slices and the activation quantisation
// ---------------------------------------------------------------------------
struct RouterT1Args {
  const float *x;       // [H]
  const float *logits;  // [E] or null
  const float *wr;      // [E][H]
  int H, E, kl, ks;
  float *partial;  // [ks][E]
  int8_t *xq;
  float *sx;
};

__global__ __launch_bounds__(kThreads) void router_gemv_t1_kernel(RouterT1Args a) {
  const int lane = threadIdx.x & (MOE_WAVE - 1);
  const int wave = threadIdx.x >> 6;
  const int ks = blockIdx.y;
  const int k0 = ks * a.kl;
  if (blockIdx.x + 1 < gridDim.x) {  // a logits workgroup
    const int e = blockIdx.x * (kThreads / MOE_WAVE) + wave;
    if (e < a.E) {
      const float *wrow = a.wr + (int64_t)e * a.H + k0;
      float acc = 0.0f;
      for (int c = lane * 4; c < a.kl; c += MOE_WAVE * 4) {
        const float4 wv = *reinterpret_cast<const float4 *>(wrow + c);
        const float4 xv = *reinterpret_cast<const float4 *>(a.x + k0 + c);
        acc = __builtin_fmaf(wv.x, xv.x, acc);
        acc = __builtin_fmaf(wv.y, xv.y, acc);
        acc = __builtin_fmaf(wv.z, xv.z, acc);
        acc = __builtin_fmaf(wv.w, xv.w, acc);
      }
      const float s = wave_sum_f32(acc);
      if (lane == 0) a.partial[(int64_t)ks * a.E + e] = s;
    }
    return;
  }
  // the last column: max|x| over the whole token, then quantise this slice
  __shared__ float red[kThreads / MOE_WAVE];
  float4 xv[kMaxX4];
#pragma unroll
  for (int q = 0; q < kMaxX4; ++q) {
    const int d = threadIdx.x + q * kThreads;
    xv[q] = (d < a.H / 4) ? reinterpret_cast<const float4 *>(a.x)[d] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float m = 0.0f;
#pragma unroll
  for (int q = 0; q < kMaxX4; ++q)
    m = fmaxf(m, fmaxf(fmaxf(fabsf(xv[q].x), fabsf(xv[q].y)), fmaxf(fabsf(xv[q].z), fabsf(xv[q].w))));
  m = wave_max_all(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sxv = (m == 0.0f) ? 0.0f : m / 127.0f;
  if (ks == 0 && threadIdx.x == 0) a.sx[0] = sxv;
  for (int d = k0 / 4 + threadIdx.x; d < (k0 + a.kl) / 4; d += kThreads) {
    const float4 v = reinterpret_cast<const float4 *>(a.x)[d];
    const float vv[4] = {v.x, v.y, v.z, v.w};
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int qq = 0;
      if (m != 0.0f) {
        float r = __builtin_rintf(vv[j] / sxv);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        qq = (int)r;
      }
      word |= (uint32_t)(uint8_t)(int8_t)qq << (8 * j);
    }
    reinterpret_cast<uint32_t *>(a.xq)[d] = word;
  }
}

// ---------------------------------------------------------------------------
// K2: top-k + gate/up stream
// ---------------------------------------------------------------------------
struct GateUpT1Args {
  // routing inputs
  const float *partial;  // [ks][E] logit slices (or null with logits)
  const float *logits;   // [E] or null
  const float *bias;     // [E] or null
  int E, k, ks;
  float routed_scale, top_p;
  const moe_expert_w *experts;
  moe_expert_w shared;
  int has_shared;
  // routing outputs (written by workgroup 0)
  int32_t *topk_idx;
  float *topk_w;
  SlotEntry *slots;
  // FFN
  const int8_t *xq;  // [H]
  const float *sx;   // [1]
  const float *xf;   // [H] fp32 hidden state, quantised in the kernel (template flag QX) instead of xq / sx
  int H, I, S;
  float *A;  // [S][I]
  moe_debug_bufs dbg;
  int dbg_on;
  // given routing (the per-step expert FFN): the slots' ids, and the width
  // filter (experts of another width are left to that width's call)
  const int32_t *given_idx;  // [k]
  const uint8_t *expert_bits;
  int want_bits;
  uint32_t *err;  // error flags: an id out of range or repeated
};

template <int BITS, int JG, int NB>
struct GuBatch {
  uint4 g[NB][JG], u[NB][JG];
};

// Row pointers of a wave's (at most two) routed slots.
struct WaveSlots {
  int s_first, I;
  const uint8_t *gate0, *up0, *gate1, *up1;
};

// Per-width kernel shapes: 16-byte chunks per lane of a gate/up row (JG) and
// of a down row (JD) the kernels are compiled for, row pairs per gate/up
// batch (NB) and down rows per batch (RB), two batches in flight each. A CU
// keeps some tens of KB of loads in flight; deeper queues only stall issue.
template <int BITS>
struct T1Shape;
template <>
struct T1Shape<4> {
  static constexpr int JG = 3, JD = 1, NB = 1, RB = 1;
};
template <>
struct T1Shape<8> {
  static constexpr int JG = 6, JD = 2, NB = 1, RB = 1;
};
template <>
struct T1Shape<2> {
  static constexpr int JG = 2, JD = 1, NB = 1, RB = 1;
};

// Load NB routed row pairs starting at routed pair qb; pairs past qlast (the
// wave's last pair, or pair 0 for a wave without routed pairs) re-read it
// (their results are dropped). The loads are unconditional, so the compiler
// can count them when it waits for older loads.
template <int BITS, int JG, int NB>
__device__ __forceinline__ void gu_load(const WaveSlots &ws, int qb, int qlast, int lane, int rowbytes, int cpr,
                                        GuBatch<BITS, JG, NB> &bt) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int q = (qb + b < qlast) ? qb + b : qlast;
    const int slot = uniform(q / ws.I);
    const int i = q - slot * ws.I;
    const bool first = slot == ws.s_first;
    const uint8_t *gate = (first ? ws.gate0 : ws.gate1) + (int64_t)i * rowbytes;
    const uint8_t *up = (first ? ws.up0 : ws.up1) + (int64_t)i * rowbytes;
#pragma unroll
    for (int j = 0; j < JG; ++j) {
      int c = lane + j * MOE_WAVE;
      c = c < cpr ? c : cpr - 1;
      bt.g[b][j] = ldg16_nt(gate, c);
      bt.u[b][j] = ldg16_nt(up, c);
    }
  }
}

// Load the wave's ns <= NB shared row pairs starting at row i0. Pair 0 is
// always loaded (a wave without shared pairs reads an in-bounds dummy row).
template <int BITS, int JG, int NB>
__device__ __forceinline__ void gu_load_shared(const uint8_t *gate, const uint8_t *up, int i0, int ns, int lane,
                                               int rowbytes, int cpr, GuBatch<BITS, JG, NB> &bt) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b == 0 || b < ns) {
      const int64_t o = (int64_t)(i0 + b) * rowbytes;
#pragma unroll
      for (int j = 0; j < JG; ++j) {
        int c = lane + j * MOE_WAVE;
        c = c < cpr ? c : cpr - 1;
        bt.g[b][j] = ldg16_nt(gate + o, c);
        bt.u[b][j] = ldg16_nt(up + o, c);
      }
    }
  }
}

// Dot products of the first n pairs of a batch; lane (lane0 + b) keeps pair
// b's sums.
template <int BITS, int JG, int NB>
__device__ __forceinline__ void gu_compute(int n, int lane0, int lane, const GuBatch<BITS, JG, NB> &bt,
                                           const ActChunk<BITS> (&xr)[JG], int &res_g, int &res_u) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b < n) {
      int ag = 0, au = 0;
#pragma unroll
      for (int j = 0; j < JG; ++j) {
        ag = dot_regs<BITS>(bt.g[b][j], xr[j], ag);
        au = dot_regs<BITS>(bt.u[b][j], xr[j], au);
      }
      ag = wave_sum_all(ag);
      au = wave_sum_all(au);
      if (lane == lane0 + b) {
        res_g = ag;
        res_u = au;
      }
    }
  }
}

// The gate/up work of workgroup vb of vn: the whole grid, or in the
// mixed-width kernel this width's part of it. has_sh: this part computes the
// shared expert; want_bits: the width whose slots it computes (given
// routing); write_table: it writes the global slot table and the error flag.
template <int BITS, int JG, int NB, bool GIVEN, bool QX = false>
__device__ __forceinline__ void gateup_t1_body(const GateUpT1Args &a, int vb, int vn, int has_sh, int want_bits,
                                               bool write_table) {
  static_assert(GIVEN || !QX, "in-kernel quantisation is for given routing");
  static_assert(NB == 1, "routed pairs are taken one at a time");
  constexpr int OFF = QFmt<BITS>::kOff;
  __shared__ float key_s[kMaxE], sig_s[kMaxE];
  __shared__ __align__(16) moe_expert_w exp_s[kMaxE];
  __shared__ SlotEntry slot_s[kMaxSlots];
  __shared__ int next_s;                   // the workgroup's routed-pair counter
  __shared__ int2 res_s[kMaxPairsWg];      // (gate, up) sums of the workgroup's routed pairs
  const int tid = threadIdx.x;
  const int lane = tid & (MOE_WAVE - 1);
  const int wave = tid >> 6;
  const int nw = vn * kFfnWaves;
  const int gw = vb * kFfnWaves + wave;
  const int rowbytes = a.H * BITS / 8;
  const int cpr = rowbytes / 16;
  // this wave's shared pairs [sh0, sh0 + ns); lanes [0, ns) keep their sums
  const int sh0 = has_sh ? uniform((int)((int64_t)gw * a.I / nw)) : 0;
  const int ns = has_sh ? uniform((int)((int64_t)(gw + 1) * a.I / nw)) - sh0 : 0;
  __shared__ int nkeep_s;  // routed slots kept (k, or fewer under top-p)
  if (tid == 0) next_s = 0;

  // ---- loads first: the routing inputs, the expert table, the token's int8
  // activations, all consumed only after the shared rows below are issued.
  // The loads are unconditional with clamped indices (slices past ks re-read
  // slice ks-1, experts past E re-read expert E-1): a load under a branch
  // makes the compiler wait for every older load at the branch's join. ----
  constexpr int kPer = kMaxE / kFfnThreads;
  const float *zsrc = a.logits ? a.logits : a.partial;
  const int nsum = a.logits ? 1 : a.ks;
  const float *bsrc = a.bias ? a.bias : zsrc;
  // (uniform branches cover the parts only large E or many slices need; at
  // most 63 loads can be outstanding, so the common case stays well below)
  float zs[kPer][kMaxSlices], bs[kPer];
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    if (!GIVEN && (m == 0 || a.E > m * kFfnThreads)) {
      const int e = min(tid + m * kFfnThreads, a.E - 1);
#pragma unroll
      for (int s = 0; s < kMaxSlices / 2; ++s) zs[m][s] = gptr(zsrc)[(int64_t)min(s, nsum - 1) * a.E + e];
      if (nsum > kMaxSlices / 2) {
#pragma unroll
        for (int s = kMaxSlices / 2; s < kMaxSlices; ++s) zs[m][s] = gptr(zsrc)[(int64_t)min(s, nsum - 1) * a.E + e];
      }
      bs[m] = gptr(bsrc)[e];
    }
  }
  constexpr int kExpPer = (3 * kMaxE + kFfnThreads - 1) / kFfnThreads;  // 16-byte pieces per thread
  uint4 exr[kExpPer];
#pragma unroll
  for (int i = 0; i < kExpPer; ++i)
    if (!GIVEN && (i < 2 || 3 * a.E > i * kFfnThreads))
      exr[i] = ldg16(a.experts, min(tid + i * kFfnThreads, 3 * a.E - 1));
  constexpr int EPC = QFmt<BITS>::kEpc;
  uint4 xraw[JG][EPC / 16];
  // QX: the token's fp32 row, this thread's float4s of it (H <= 8192)
  constexpr int kQx = QX ? kMaxX4 * kThreads / kFfnThreads : 1;
  __shared__ __align__(16) uint32_t xq_s[QX ? kMaxX4 * kThreads : 4];  // QX: the token's codes
  __shared__ float qred_s[kFfnWaves];
  float4 xv[kQx];
  float sxv = 0.0f;
  if constexpr (QX) {
#pragma unroll
    for (int q = 0; q < kQx; ++q) {
      const int d = tid + q * kFfnThreads;
      xv[q] = (d < a.H / 4) ? reinterpret_cast<const float4 *>(a.xf)[d] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  } else {
#pragma unroll
    for (int j = 0; j < JG; ++j) {
      const int c = min(lane + j * MOE_WAVE, cpr - 1);
#pragma unroll
      for (int u = 0; u < EPC / 16; ++u) xraw[j][u] = ldg16(a.xq + (int64_t)c * EPC, u);
    }
    sxv = a.sx[0];
  }
  asm volatile("" ::: "memory");

  // ---- the shared expert's rows: known before routing, so they stream while
  // the keys are formed and ranked (unconditional loads; without a shared
  // expert a dummy in-bounds row of xq is read and dropped) ----
  GuBatch<BITS, JG, NB> b0, b1;
  {
    // the dummy row: the token's codes (H bytes), or with QX its fp32 row (4 H
    // bytes; xq and sx are not passed then); a packed row is at most H bytes
    const uint8_t *dummy = QX ? reinterpret_cast<const uint8_t *>(a.xf) : reinterpret_cast<const uint8_t *>(a.xq);
    const uint8_t *sg_p = has_sh ? a.shared.gate : dummy;
    const uint8_t *su_p = has_sh ? a.shared.up : dummy;
    gu_load_shared<BITS, JG, NB>(sg_p, su_p, has_sh ? sh0 : 0, ns, lane, rowbytes, cpr, b0);
  }
  float sg_sh, su_sh;
  {
    const bool use = has_sh != 0;
    const int li = use ? sh0 + min(lane, max(ns - 1, 0)) : 0;
    const float *dummy_s = QX ? a.xf : a.sx;  // element 0 only
    sg_sh = gptr(use ? a.shared.s_gate : dummy_s)[li];
    su_sh = gptr(use ? a.shared.s_up : dummy_s)[li];
  }
  asm volatile("" ::: "memory");

  // QX: the activation rule on the row (the same arithmetic as the
  // quantisation kernel): sx = max|x| / 127, codes rint(x / sx) clamped to
  // [-127, 127] (all zero for an all-zero row), into LDS, then this lane's
  // chunks from there
  if constexpr (QX) {
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < kQx; ++q)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(xv[q].x), fabsf(xv[q].y)), fmaxf(fabsf(xv[q].z), fabsf(xv[q].w))));
    m = wave_max_all(m);
    if (lane == 0) qred_s[wave] = m;
    __syncthreads();
    m = qred_s[0];
#pragma unroll
    for (int w = 1; w < kFfnWaves; ++w) m = fmaxf(m, qred_s[w]);
    sxv = (m == 0.0f) ? 0.0f : m / 127.0f;
#pragma unroll
    for (int q = 0; q < kQx; ++q) {
      const int d = tid + q * kFfnThreads;
      const float vv[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int qq = 0;
        if (m != 0.0f) {
          float r = __builtin_rintf(vv[j] / sxv);
          r = fminf(fmaxf(r, -127.0f), 127.0f);
          qq = (int)r;
        }
        word |= (uint32_t)(uint8_t)(int8_t)qq << (8 * j);
      }
      if (d < a.H / 4) xq_s[d] = word;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < JG; ++j) {
      const int c = min(lane + j * MOE_WAVE, cpr - 1);
#pragma unroll
      for (int u = 0; u < EPC / 16; ++u) {
        const uint32_t *src = xq_s + (c * EPC + u * 16) / 4;
        xraw[j][u] = make_uint4(src[0], src[1], src[2], src[3]);
      }
    }
  }

  // ---- now consume: the expert table to LDS, the activations in field
  // order, the routing keys ----
#pragma unroll
  for (int i = 0; i < kExpPer; ++i) {
    const int idx = tid + i * kFfnThreads;
    if (!GIVEN && idx < 3 * a.E) reinterpret_cast<uint4 *>(exp_s)[idx] = exr[i];
  }
  ActChunk<BITS> xr[JG];
  int xs_lane = 0;
#pragma unroll
  for (int j = 0; j < JG; ++j) {
    int bs1 = 0;
    act_chunk_from<BITS>(xraw[j], xr[j], bs1);
    if (lane + j * MOE_WAVE >= cpr) {
      zero_chunk<BITS>(xr[j]);
      bs1 = 0;
    }
    xs_lane += bs1;
  }
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int e = tid + m * kFfnThreads;
    if (GIVEN || (m > 0 && a.E <= m * kFfnThreads)) break;
    float z = zs[m][0];  // slices in order
#pragma unroll
    for (int s = 1; s < kMaxSlices; ++s)
      if (s < nsum) z += zs[m][s];
    const float sg = 1.0f / (1.0f + moe_exp_f32(-z));
    float key = sg + (a.bias ? bs[m] : 0.0f);
    if (key != key) key = -__builtin_inff();  // a NaN key ranks last
    if (e < a.E) {
      key_s[e] = key + 0.0f;  // no -0 keys
      sig_s[e] = sg;
    }
  }
  __syncthreads();

  // ---- given routing: the slot table from the ids (wave 0). The global
  // table keeps the slots in their own order (a slot without work -- another
  // width, or -1 -- gets expert -1 and valid pointers of a slot with work);
  // in LDS the slots with work come first, each with its own index ----
  if constexpr (GIVEN) {
    if (wave == 0) {
      const int e = lane < a.k ? a.given_idx[lane] : -1;
      bool valid = e == -1 || (e >= 0 && e < a.E);
      bool act = e >= 0 && e < a.E;
      for (int j = 0; j < a.k; ++j) {  // a repeated id is an error, and computed for its first slot only
        const int ej = __builtin_amdgcn_readlane(e, j);
        if (j < lane && act && ej == e) {
          act = false;
          valid = false;
        }
      }
      const uint64_t bad = __ballot(!valid);
      if (bad && write_table && lane == 0) atomicOr(a.err, 1u);
      if (act && a.expert_bits) act = a.expert_bits[e] == want_bits;
      const uint64_t m = __ballot(act);
      const int na = __popcll(m);
      const int first = na ? __ffsll((unsigned long long)m) - 1 : 0;
      const int e_first = na ? __builtin_amdgcn_readlane(e, first) : -1;
      auto row_of = [&](int ex, uint4 (&row)[3]) {
        if (ex >= 0) {
#pragma unroll
          for (int q = 0; q < 3; ++q) row[q] = ldg16(a.experts + ex, q);
        } else if (has_sh) {
          const uint64_t pp[6] = {(uint64_t)a.shared.gate, (uint64_t)a.shared.up, (uint64_t)a.shared.down,
                                  (uint64_t)a.shared.s_gate, (uint64_t)a.shared.s_up, (uint64_t)a.shared.s_down};
#pragma unroll
          for (int q = 0; q < 3; ++q)
            row[q] = make_uint4((uint32_t)pp[2 * q], (uint32_t)(pp[2 * q] >> 32), (uint32_t)pp[2 * q + 1],
                                (uint32_t)(pp[2 * q + 1] >> 32));
        } else {
#pragma unroll
          for (int q = 0; q < 3; ++q) row[q] = make_uint4(0u, 0u, 0u, 0u);
        }
      };
      uint4 own[3], dummy[3];
      row_of(act ? e : e_first, own);
      row_of(e_first, dummy);
      if (lane < a.k) {
        const uint4 tag = make_uint4(0u, (uint32_t)(act ? e : -1), (uint32_t)lane, 0u);
        if (write_table) {
          uint4 *gdst = reinterpret_cast<uint4 *>(a.slots + lane);
#pragma unroll
          for (int q = 0; q < 3; ++q) gdst[q] = own[q];
          gdst[3] = tag;
        }
        if (act) {
          uint4 *dst = reinterpret_cast<uint4 *>(slot_s + __popcll(m & ((1ull << lane) - 1ull)));
#pragma unroll
          for (int q = 0; q < 3; ++q) dst[q] = own[q];
          dst[3] = tag;
        }
        if (lane >= na) {  // entries past the slots with work: valid pointers, never given pairs
          uint4 *dst = reinterpret_cast<uint4 *>(slot_s + lane);
#pragma unroll
          for (int q = 0; q < 3; ++q) dst[q] = dummy[q];
          dst[3] = make_uint4(0u, (uint32_t)-1, (uint32_t)lane, 0u);
        }
      } else if (lane == a.k && has_sh) {
        row_of(-1, own);
        const uint4 tag = make_uint4(__float_as_uint(1.0f), (uint32_t)-1, (uint32_t)a.k, 0u);
        uint4 *dst = reinterpret_cast<uint4 *>(slot_s + lane);
#pragma unroll
        for (int q = 0; q < 3; ++q) dst[q] = own[q];
        dst[3] = tag;
        if (write_table) {
          uint4 *gdst = reinterpret_cast<uint4 *>(a.slots + lane);
#pragma unroll
          for (int q = 0; q < 3; ++q) gdst[q] = own[q];
          gdst[3] = tag;
        }
      }
      if (lane == 0) nkeep_s = na;
    }
    __syncthreads();
    if (nkeep_s == 0 && !has_sh) return;  // nothing for this width
  }

  // ---- top-k and the slot table (wave 0) ----
  if (!GIVEN && wave == 0) {
    const int my_id = (a.E <= 4 * MOE_WAVE) ? wave_topk4(key_s, a.E, a.k, lane) : wave_topk16(key_s, a.E, a.k, lane);
    const float my_sig = lane < a.k ? sig_s[my_id] : 0.0f;
    float sum = 0.0f;  // in rank order
    for (int j = 0; j < a.k; ++j) sum += readlane_f(my_sig, j);
    float kept = sum;
    const int keep = a.top_p > 0.0f ? topp_keep(my_sig, sum, a.k, a.top_p, kept) : a.k;
    if (lane == 0) nkeep_s = keep;
    uint4 row[4];
    bool have = false;
    if (lane < a.k) {
      // a dropped slot keeps the first expert's pointers (valid rows for the
      // down kernel, whose result for it is zero), weight 0 and id -1
      const bool kp = lane < keep;
      const int id0 = __builtin_amdgcn_readlane(my_id, 0);
      const float wgt = kp ? a.routed_scale * (my_sig / kept) : 0.0f;
      const uint4 *src = reinterpret_cast<const uint4 *>(exp_s + (kp ? my_id : id0));
      row[0] = src[0];
      row[1] = src[1];
      row[2] = src[2];
      row[3] = make_uint4(__float_as_uint(wgt), (uint32_t)(kp ? my_id : -1), 0u, 0u);
      have = true;
      if (write_table) {
        a.topk_idx[lane] = kp ? my_id : -1;
        a.topk_w[lane] = wgt;
      }
    } else if (lane == a.k && has_sh) {
      const uint64_t p[6] = {(uint64_t)a.shared.gate, (uint64_t)a.shared.up, (uint64_t)a.shared.down,
                             (uint64_t)a.shared.s_gate, (uint64_t)a.shared.s_up, (uint64_t)a.shared.s_down};
#pragma unroll
      for (int q = 0; q < 3; ++q)
        row[q] = make_uint4((uint32_t)p[2 * q], (uint32_t)(p[2 * q] >> 32), (uint32_t)p[2 * q + 1],
                            (uint32_t)(p[2 * q + 1] >> 32));
      row[3] = make_uint4(__float_as_uint(1.0f), (uint32_t)-1, 0u, 0u);
      have = true;
    }
    if (have) {
      uint4 *dst = reinterpret_cast<uint4 *>(slot_s + lane);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = row[q];
      if (write_table) {
        uint4 *gdst = reinterpret_cast<uint4 *>(a.slots + lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) gdst[q] = row[q];
      }
    }
  }
  __syncthreads();

  // the workgroup's routed pairs [Q0, Q0 + np) of the kept slots' keep * I,
  // taken one at a time by its waves from an LDS counter: a wave whose loads
  // are served late takes fewer
  const int R = uniform(nkeep_s) * a.I;
  const int Q0 = uniform((int)((int64_t)vb * R / vn));
  const int np = uniform((int)((int64_t)(vb + 1) * R / vn)) - Q0;

  // ---- the workgroup's routed slots (a contiguous range spans at most two) ----
  WaveSlots ws;
  ws.I = a.I;
  const int qlast = np > 0 ? Q0 + np - 1 : 0;
  ws.s_first = uniform((np > 0 ? Q0 : 0) / a.I);
  const int s_last = uniform(qlast / a.I);
  ws.gate0 = uniform_p(slot_s[ws.s_first].w.gate);
  ws.up0 = uniform_p(slot_s[ws.s_first].w.up);
  ws.gate1 = uniform_p(slot_s[s_last].w.gate);
  ws.up1 = uniform_p(slot_s[s_last].w.up);
  // the global routed pair loaded for workgroup-local pair p: pairs past the
  // range re-read its last pair, and a workgroup without routed pairs reads
  // pair 0 (always valid; its results are never used)
  auto pair_at = [&](int p) { return np > 0 ? Q0 + min(p, np - 1) : 0; };
  // take the next routed pair (workgroup-local index; >= np when none is left)
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&next_s, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  int pa = grab();
  gu_load<BITS, JG, NB>(ws, pair_at(pa), qlast, lane, rowbytes, cpr, b1);

  // thread t < np: routed pair t's slot, row and scales (used after the loop)
  const bool rt_mine = tid < np;
  int rt_slot = 0, rt_i = 0;
  float rt_sg = 0.0f, rt_su = 0.0f;
  {
    const int q = Q0 + min(tid, max(np - 1, 0));
    rt_slot = q / a.I;
    rt_i = q - rt_slot * a.I;
    rt_sg = gptr(slot_s[rt_slot].w.s_gate)[rt_i];
    rt_su = gptr(slot_s[rt_slot].w.s_up)[rt_i];
  }
  const int xsum = wave_sum_all(xs_lane);

  // the wave's shared pairs (lanes [0, ns) keep their sums): the first batch
  // was issued before routing; more than one batch only when a width's part
  // of the mixed-width kernel has fewer waves than the shared expert has rows
  int res_g = 0, res_u = 0;
  if (ns > 0) gu_compute<BITS, JG, NB>(ns < NB ? ns : NB, 0, lane, b0, xr, res_g, res_u);
  for (int p = NB; p < ns; p += NB) {
    gu_load_shared<BITS, JG, NB>(a.shared.gate, a.shared.up, sh0 + p, ns - p, lane, rowbytes, cpr, b0);
    gu_compute<BITS, JG, NB>(ns - p < NB ? ns - p : NB, p, lane, b0, xr, res_g, res_u);
  }
  int pb = grab();
  gu_load<BITS, JG, NB>(ws, pair_at(pb), qlast, lane, rowbytes, cpr, b0);
  // routed pairs, two in flight (pairs past np re-read the last one; pa < pb)
  for (;;) {
    if (pa >= np) break;
    {
      int g0 = 0, u0 = 0;
      gu_compute<BITS, JG, NB>(1, 0, lane, b1, xr, g0, u0);
      if (lane == 0) res_s[pa] = make_int2(__builtin_amdgcn_readfirstlane(g0), __builtin_amdgcn_readfirstlane(u0));
    }
    pa = grab();
    gu_load<BITS, JG, NB>(ws, pair_at(pa), qlast, lane, rowbytes, cpr, b1);
    if (pb >= np) break;
    {
      int g0 = 0, u0 = 0;
      gu_compute<BITS, JG, NB>(1, 0, lane, b0, xr, g0, u0);
      if (lane == 0) res_s[pb] = make_int2(__builtin_amdgcn_readfirstlane(g0), __builtin_amdgcn_readfirstlane(u0));
    }
    pb = grab();
    gu_load<BITS, JG, NB>(ws, pair_at(pb), qlast, lane, rowbytes, cpr, b0);
  }

  // a = silu(g) * u: the wave's shared pairs, then the workgroup's routed pairs
  auto epilogue = [&](int gsum, int usum, float sg, float su, int slot, int i) {
    const int gi = gsum - OFF * xsum;
    const int ui = usum - OFF * xsum;
    const float g = (float)gi * sg * sxv;
    const float u = (float)ui * su * sxv;
    const float av = moe_silu_f32(g) * u;
    // with given routing the LDS slots with work come first: each keeps its own index
    const int own = (GIVEN && slot < a.k) ? slot_s[slot].pad[0] : slot;
    const int64_t o = (int64_t)own * a.I + i;
    a.A[o] = av;
    if (a.dbg_on) {
      if (a.dbg.accg) a.dbg.accg[o] = gi;
      if (a.dbg.accu) a.dbg.accu[o] = ui;
      if (a.dbg.a) a.dbg.a[o] = av;
    }
  };
  if (lane < ns) epilogue(res_g, res_u, sg_sh, su_sh, a.k, sh0 + lane);
  __syncthreads();
  if (rt_mine) {
    const int2 r = res_s[tid];
    epilogue(r.x, r.y, rt_sg, rt_su, rt_slot, rt_i);
  }
}

template <int BITS, int JG, int NB, bool GIVEN, bool QX = false>
__global__ __launch_bounds__(kFfnThreads) void gateup_t1_kernel(GateUpT1Args a) {
  gateup_t1_body<BITS, JG, NB, GIVEN, QX>(a, blockIdx.x, gridDim.x, a.has_shared, a.want_bits, blockIdx.x == 0);
}

// One token, every width of a mixed layer in one launch (routing given).
// Every workgroup reads the ids and the experts' widths and computes the same
// split of the grid between the widths present (8, 4, 2 in that order), in
// proportion to the bytes of their row pairs (the shared expert counted at
// its width); each part runs that width's gate/up over its share of the
// workgroups. Workgroup 0 writes the global slot table: each slot's expert
// with its width in pad[1], or expert -1 (no expert, a width outside the
// call's mask, a repeated id) with valid pointers for the down kernel's
// unconditional loads; it also raises the error flag for bad ids.
template <bool QX>
__global__ __launch_bounds__(kFfnThreads) void gateup_mixed_t1_kernel(GateUpT1Args a, int mask, int shared_bits) {
  const int lane = threadIdx.x & (MOE_WAVE - 1);
  const int wave = threadIdx.x >> 6;
  const int e = lane < a.k ? a.given_idx[lane] : -1;
  bool valid = e == -1 || (e >= 0 && e < a.E);
  bool act = e >= 0 && e < a.E;
  for (int j = 0; j < a.k; ++j) {  // a repeated id is an error, and computed for its first slot only
    const int ej = __builtin_amdgcn_readlane(e, j);
    if (j < lane && act && ej == e) {
      act = false;
      valid = false;
    }
  }
  const int sbits = a.has_shared ? shared_bits : 0;
  const int emask = mask | (sbits ? 1 << sbits : 0);  // the shared expert's width always runs
  int b = act ? (int)a.expert_bits[e] : 0;
  if (!((b == 8 || b == 4 || b == 2) && ((emask >> b) & 1))) b = 0;
  const int wb[3] = {8, 4, 2};
  int64_t bytes[3], tot = 0;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    const int n = __popcll(__ballot(b == wb[w])) + (sbits == wb[w] ? 1 : 0);
    bytes[w] = (int64_t)n * wb[w];
    tot += bytes[w];
  }
  if (blockIdx.x == 0 && wave == 0) {
    if (__ballot(!valid) && lane == 0) atomicOr(a.err, 1u);
    const uint64_t m = __ballot(b != 0);
    const int first = m ? __ffsll((unsigned long long)m) - 1 : 0;
    const int e_first = m ? __builtin_amdgcn_readlane(e, first) : -1;
    auto row_of = [&](int ex, uint4 (&row)[3]) {
      if (ex >= 0) {
#pragma unroll
        for (int q = 0; q < 3; ++q) row[q] = ldg16(a.experts + ex, q);
      } else if (a.has_shared) {
        const uint64_t pp[6] = {(uint64_t)a.shared.gate, (uint64_t)a.shared.up, (uint64_t)a.shared.down,
                                (uint64_t)a.shared.s_gate, (uint64_t)a.shared.s_up, (uint64_t)a.shared.s_down};
#pragma unroll
        for (int q = 0; q < 3; ++q)
          row[q] = make_uint4((uint32_t)pp[2 * q], (uint32_t)(pp[2 * q] >> 32), (uint32_t)pp[2 * q + 1],
                              (uint32_t)(pp[2 * q + 1] >> 32));
      } else {
#pragma unroll
        for (int q = 0; q < 3; ++q) row[q] = make_uint4(0u, 0u, 0u, 0u);
      }
    };
    uint4 row[3];
    if (lane < a.k) {
      row_of(b ? e : e_first, row);
      const uint4 tag = make_uint4(0u, (uint32_t)(b ? e : -1), (uint32_t)lane, (uint32_t)b);
      uint4 *gdst = reinterpret_cast<uint4 *>(a.slots + lane);
#pragma unroll
      for (int q = 0; q < 3; ++q) gdst[q] = row[q];
      gdst[3] = tag;
    } else if (lane == a.k && a.has_shared) {
      row_of(-1, row);
      const uint4 tag = make_uint4(__float_as_uint(1.0f), (uint32_t)-1, (uint32_t)a.k, (uint32_t)sbits);
      uint4 *gdst = reinterpret_cast<uint4 *>(a.slots + lane);
#pragma unroll
      for (int q = 0; q < 3; ++q) gdst[q] = row[q];
      gdst[3] = tag;
    }
  }
  if (tot == 0) return;
  // workgroups per width: first each width's minimum (enough that no
  // workgroup takes more than kMaxPairsWg routed pairs and no wave more than
  // one lane's worth of shared pairs; the launcher checks that the minimums
  // fit the grid), then the rest of the grid in proportion to the bytes of
  // the row pairs, its rounding remainder to the largest part
  const int nwg = gridDim.x;
  int cnt[3], big = 0, used = 0;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    const int routed = __popcll(__ballot(b == wb[w]));
    int mn = bytes[w] ? max(1, (routed * a.I + kMaxPairsWg - 1) / kMaxPairsWg) : 0;
    if (sbits == wb[w]) mn = max(mn, (a.I + kFfnWaves * MOE_WAVE - 1) / (kFfnWaves * MOE_WAVE));
    cnt[w] = mn;
    used += mn;
    if (bytes[w] > bytes[big]) big = w;
  }
  const int rest = max(nwg - used, 0);
  int given_out = 0;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    const int add = (int)(rest * bytes[w] / tot);
    cnt[w] += add;
    given_out += add;
  }
  cnt[big] += rest - given_out;
  const int vb0 = blockIdx.x;
  if (vb0 < cnt[0]) {
    gateup_t1_body<8, T1Shape<8>::JG, 1, true, QX>(a, vb0, cnt[0], sbits == 8, 8, false);
  } else if (vb0 < cnt[0] + cnt[1]) {
    gateup_t1_body<4, T1Shape<4>::JG, 1, true, QX>(a, vb0 - cnt[0], cnt[1], sbits == 4, 4, false);
  } else if (vb0 < cnt[0] + cnt[1] + cnt[2]) {
    gateup_t1_body<2, T1Shape<2>::JG, 1, true, QX>(a, vb0 - cnt[0] - cnt[1], cnt[2], sbits == 2, 2, false);
  }
}

// ---------------------------------------------------------------------------
// The requantisation arithmetic (the activation rule on a)
// ---------------------------------------------------------------------------
// int8 code of v under the scale sc = m/127 with inv = 1/sc (both correctly
// rounded): rint(v * inv) equals rint(v / sc) (the fp32 quotient) unless
// v * inv lies within 2^-15 of a half-integer. With |v| <= m the quotient is
// at most 127 in magnitude, where v * inv differs from the exact ratio by less
// than 2^-16 and the rounded quotient by less than 2^-15 (one rounding of 1/sc
// and one of the product, 2^-24 relative each), so outside that band both
// round to the same integer. `near` is raised for a value in the band; the
// caller then recomputes the code with the division.
__device__ __forceinline__ float code_fast(float v, float inv, bool &near) {
  const float t = v * inv;
  const float n = __builtin_rintf(t);
  near |= fabsf(t - n) > (0.5f - 0x1p-15f);  // t - n is exact (Sterbenz)
  return n;
}
__device__ __forceinline__ float code_exact(float v, float sc) {
  float r = __builtin_rintf(v / sc);
  return fminf(fmaxf(r, -127.0f), 127.0f);
}
// four codes (as floats in [-127, 127]) -> one dword of int8 codes
__device__ __forceinline__ uint32_t pack_codes(float c0, float c1, float c2, float c3) {
  uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(c0 + 128.0f, 0, 0u);
  w = __builtin_amdgcn_cvt_pk_u8_f32(c1 + 128.0f, 1, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(c2 + 128.0f, 2, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(c3 + 128.0f, 3, w);
  return w ^ 0x80808080u;
}
// A lane's natural-order code dword -> the dword at the same position in the
// weights' field order (int4: pairs of lanes hold the 8 elements of a group;
// int2: quads of lanes hold the 16 elements of a group).
template <int BITS>
__device__ __forceinline__ uint32_t field_order(uint32_t w, int lane) {
  if constexpr (BITS == 4) {
    const uint32_t o = (uint32_t)dpp_i<0xB1>((int)w);  // the neighbour's dword
    return (lane & 1) ? perm_b32(w, o, 0x07050301u) : perm_b32(o, w, 0x06040200u);
  } else if constexpr (BITS == 2) {
    const uint32_t d0 = (uint32_t)dpp_i<0x00>((int)w), d1 = (uint32_t)dpp_i<0x55>((int)w);
    const uint32_t d2 = (uint32_t)dpp_i<0xAA>((int)w), d3 = (uint32_t)dpp_i<0xFF>((int)w);
    const uint32_t j = (uint32_t)(lane & 3);
    const uint32_t sel = j | ((4u + j) << 8) | 0x0c0c0000u;
    const uint32_t lo = perm_b32(d1, d0, sel), hi = perm_b32(d3, d2, sel);
    return perm_b32(hi, lo, 0x05040100u);
  } else {
    return w;
  }
}

// ---------------------------------------------------------------------------
// K3: requantisation and down projection of every slot + combine
// ---------------------------------------------------------------------------
struct DownT1Args {
  const SlotEntry *slots;
  const float *A;  // [S][I] the SwiGLU intermediate (a slot without work here was never written: zero codes)
  int H, I, S, k, has_shared;
  float *y;    // [S][H] (the token's y_slots; slot stride H)
  float *out;  // [H]; given routing: nullable (no combine)
  moe_debug_bufs dbg;
  int dbg_on;
  // given routing with the combine: the slots' routing weights [k]; the
  // slots another width's call computed are read back from y
  const float *w_given;
};

// The requantisation of every slot's a, run by each down workgroup in
// its prologue: sa = max|a| / 127 and the codes rint(a / sa), clamped to
// [-127, 127] (the activation rule), in the field order of the slot's
// weights, with their per-slot sums. A slot dropped by top-p, or without work
// in a given-routing call, gets zero codes and scale (its a was never
// written). Every workgroup reads all S slots of a, RQ float4 of each per
// thread (RQ = ceil(I / 2048)); register group j holds slot (j + blockIdx.x)
// mod S, so the workgroups of one XCD do not all ask for the same lines at
// once. The loads go out behind the slot table and before the first down
// rows, so waiting for a never waits for a weight row (a wave's loads
// complete in order), and the arithmetic runs while those rows are in flight.
// This replaced a launch of its own (one workgroup per slot), which cost more
// than the 74 KB of a every down workgroup now reads from L2.
template <int RQ>
struct RqRegs {
  float4 v[kMaxSlots * RQ];
  int slot[kMaxSlots];  // the slot of register group j (uniform)
};

template <int RQ>
__device__ __forceinline__ void rq_load(const DownT1Args &a, RqRegs<RQ> &q) {
  const int S = a.S, n4 = a.I / 4;
  const int rot = blockIdx.x % S;
#pragma unroll
  for (int j = 0; j < kMaxSlots; ++j) {
    const int sj = j + rot >= S ? j + rot - S : j + rot;
    q.slot[j] = j < S ? sj : q.slot[0];  // groups past S re-read the first group's slot
    const float *As = a.A + (int64_t)q.slot[j] * a.I;
#pragma unroll
    for (int c = 0; c < RQ; ++c) {
      // past the slot's end: a re-read of its last float4, same maximum
      const uint4 u = ldg16(As, min((int)threadIdx.x + c * kFfnThreads, n4 - 1));
      q.v[j * RQ + c] =
          make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // issued before the wait for the slot table
}

// The codes of every slot into aq_s (slot s at byte s*I), from the registers
// rq_load filled. ex_l: lane s < S holds slot s's expert id (-1: no work);
// width(s): slot s's weight width (s uniform). Returns in lane s < S slot s's
// code sum and scale. Two barriers; every thread of the workgroup calls it.
template <int RQ, bool GIVEN, typename Width>
__device__ __forceinline__ void rq_codes(const DownT1Args &a, const RqRegs<RQ> &q, int ex_l, Width width,
                                         int8_t *aq_s, float (*red_m)[kFfnWaves], int (*red_c)[kFfnWaves],
                                         int &aqsum_l, float &sa_l) {
  const int tid = threadIdx.x, lane = tid & (MOE_WAVE - 1), wave = tid >> 6;
  const int S = a.S, n4 = a.I / 4;
  const int ls = lane < S ? lane : S - 1;
#pragma unroll
  for (int j = 0; j < kMaxSlots; ++j) {
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < RQ; ++c) {
      const float4 v = q.v[j * RQ + c];
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    m = wave_max_dpp(m);
    if (j < S && lane == 0) red_m[q.slot[j]][wave] = m;
  }
  __syncthreads();
  // lane s < S: slot s's scale, its reciprocal and the fast-path flag
  float m_l = red_m[ls][0];
#pragma unroll
  for (int w = 1; w < kFfnWaves; ++w) m_l = fmaxf(m_l, red_m[ls][w]);
  const bool zero_l = m_l == 0.0f || (ls < a.k && ex_l == -1);
  sa_l = zero_l ? 0.0f : m_l / 127.0f;
  const float inv_l = zero_l ? 0.0f : 1.0f / sa_l;
  const bool fast_l = sa_l >= 0x1p-126f && sa_l <= 0x1.fffffep127f;
#pragma unroll
  for (int j = 0; j < kMaxSlots; ++j) {
    if (j < S) {
      const int sj = q.slot[j];
      const float sc = readlane_f(sa_l, sj), inv = readlane_f(inv_l, sj);
      const bool zero = __builtin_amdgcn_readlane((int)zero_l, sj) != 0;
      const bool fast = __builtin_amdgcn_readlane((int)fast_l, sj) != 0;
      // given routing: a slot without work here (another width's, or -1)
      // belongs to another call, which writes its captured intermediates
      const bool mine = !GIVEN || !(sj < a.k && __builtin_amdgcn_readlane(ex_l, sj) == -1);
      const int wb = width(sj);
      int csum = 0;
#pragma unroll
      for (int c = 0; c < RQ; ++c) {
        const int f = tid + c * kFfnThreads;
        const float4 v = q.v[j * RQ + c];
        uint32_t word = 0;
        if (!zero) {
          bool near = !fast;
          float q0 = code_fast(v.x, inv, near), q1 = code_fast(v.y, inv, near);
          float q2 = code_fast(v.z, inv, near), q3 = code_fast(v.w, inv, near);
          if (near) {
            q0 = code_exact(v.x, sc);
            q1 = code_exact(v.y, sc);
            q2 = code_exact(v.z, sc);
            q3 = code_exact(v.w, sc);
          }
          word = pack_codes(q0, q1, q2, q3);
        }
        if (f >= n4) word = 0;
        csum = sdot4((int)word, 0x01010101, csum);
        // field groups are whole within lane pairs / quads (I is a multiple
        // of 64), so a lane's neighbours hold dwords of the same group
        const uint32_t fw = wb == 8 ? word : (wb == 4 ? field_order<4>(word, lane) : field_order<2>(word, lane));
        if (f < n4) {
          reinterpret_cast<uint32_t *>(aq_s + sj * a.I)[f] = fw;
          if (blockIdx.x == 0 && a.dbg_on && a.dbg.aq && mine)
            reinterpret_cast<uint32_t *>(a.dbg.aq + (int64_t)sj * a.I)[f] = word;
        }
      }
      csum = wave_sum_to63(csum);
      if (lane == 63) red_c[sj][wave] = csum;
      if (blockIdx.x == 0 && tid == 0 && a.dbg_on && a.dbg.sa && mine) a.dbg.sa[sj] = sc;
    }
  }
  __syncthreads();
  int cs = 0;
#pragma unroll
  for (int w = 0; w < kFfnWaves; ++w) cs += red_c[ls][w];
  aqsum_l = cs;
}

template <int BITS, int JD, int RB, bool GIVEN, int RQ>
__global__ __launch_bounds__(kFfnThreads) void down_combine_t1_kernel(DownT1Args a) {
  constexpr int OFF = QFmt<BITS>::kOff;
  constexpr int EPC = QFmt<BITS>::kEpc;
  __shared__ __align__(16) int8_t aq_s[kMaxSlots * kMaxIDown];
  __shared__ float rq_m[kMaxSlots][kFfnWaves];
  __shared__ int rq_c[kMaxSlots][kFfnWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (MOE_WAVE - 1);
  const int wave = tid >> 6;
  const int nw = gridDim.x * kFfnWaves;
  const int gw = blockIdx.x * kFfnWaves + wave;
  const int r0 = uniform((int)((int64_t)gw * a.H / nw)), r1 = uniform((int)((int64_t)(gw + 1) * a.H / nw));
  const int rowbytes = a.I * BITS / 8;
  const int cpr = rowbytes / 16;
  const int S = a.S;

  // ---- slot fields (lane s < S holds slot s's), then every slot's a ----
  const int ls = lane < S ? lane : S - 1;
  const uint8_t *down_l = a.slots[ls].w.down;
  const float *sdown_l = a.slots[ls].w.s_down;
  const float w_l = a.slots[ls].weight;
  const int ex_l = a.slots[ls].expert;
  // every slot's a, before anything waits for the slot table (the buffer is
  // always valid; in a call with no work here it is read and dropped)
  RqRegs<RQ> rq;
  rq_load<RQ>(a, rq);
  // given routing: only the slots with work here are written (a slot of
  // another width belongs to that width's call)
  const bool act_l = GIVEN ? (lane < S && (lane == a.k ? a.has_shared != 0 : ex_l != -1)) : lane < S;
  const bool comb = GIVEN && a.out != nullptr;
  const float wg_l = (comb && lane < a.k) ? a.w_given[lane] : 0.0f;
  if (GIVEN && __ballot(act_l) == 0) {
    if (!comb) return;
    // no slot has work here (and so no shared expert): the combine alone,
    // every slot read back; no weight row is read, as the slots' pointers
    // may be null in this case
    for (int r = r0; r < r1; ++r) {
      const float yall = (lane < a.k && wg_l != 0.0f) ? a.y[(int64_t)lane * a.H + r] : 0.0f;
      float acc = 0.0f;
#pragma unroll
      for (int s = 0; s < kMaxSlots - 1; ++s) {
        const float ws = readlane_f(wg_l, s);
        if (s < a.k && ws != 0.0f) acc = __builtin_fmaf(ws, readlane_f(yall, s), acc);
      }
      if (lane == 0) a.out[r] = acc;
    }
    return;
  }
  const uint8_t *dp[kMaxSlots];
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s) dp[s] = readlane_p(down_l, s < S ? s : S - 1);

  struct RowBatch {
    uint4 w[RB][kMaxSlots][JD];
    float sd[RB];
  };
  // rows past the wave's range re-read an in-bounds row, slots past S re-read
  // slot S-1 (unconditional loads; those results are dropped)
  auto load_rows = [&](int rb, RowBatch &bt) {
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int r = max((rb + b < r1) ? rb + b : r1 - 1, 0);
#pragma unroll
      for (int s = 0; s < kMaxSlots; ++s) {
#pragma unroll
        for (int j = 0; j < JD; ++j) {
          int c = lane + j * MOE_WAVE;
          c = c < cpr ? c : cpr - 1;
          bt.w[b][s][j] = ldg16_nt(dp[s] + (int64_t)r * rowbytes, c);
        }
      }
      bt.sd[b] = gptr(sdown_l)[r];
    }
  };
  RowBatch b0, b1;
  load_rows(r0, b0);  // the first down rows of every slot go out right behind a
  __builtin_amdgcn_sched_barrier(0);  // all of them before a is consumed
  // (the second batch goes out after the codes: issued here, it made the
  // kernel slower)
  int aqsum_l;
  float sa_l;
  rq_codes<RQ, GIVEN>(a, rq, ex_l, [](int) { return BITS; }, aq_s, rq_m, rq_c, aqsum_l, sa_l);

  if (r0 >= r1) return;
  load_rows(r0 + RB, b1);

  // every slot's codes, in registers in field order
  ActChunk<BITS> aqr[kMaxSlots][JD];
  int aqsum[kMaxSlots];
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s) {
    aqsum[s] = __builtin_amdgcn_readlane(aqsum_l, s < S ? s : S - 1);
#pragma unroll
    for (int j = 0; j < JD; ++j) {
      const int c = lane + j * MOE_WAVE;
      if (s < S && c < cpr) {
#pragma unroll
        for (int u = 0; u < EPC / 16; ++u) {
          const uint4 v = reinterpret_cast<const uint4 *>(aq_s + s * a.I + c * EPC)[u];
          aqr[s][j].d[4 * u + 0] = v.x;
          aqr[s][j].d[4 * u + 1] = v.y;
          aqr[s][j].d[4 * u + 2] = v.z;
          aqr[s][j].d[4 * u + 3] = v.w;
        }
      } else {
        zero_chunk<BITS>(aqr[s][j]);
      }
    }
  }
  auto compute_rows = [&](int rb, const RowBatch &bt) {
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int r = rb + b;
      if (r >= r1) break;
      int mine = 0;  // lane s keeps slot s's accumulator
#pragma unroll
      for (int s = 0; s < kMaxSlots; ++s) {
        if (s < S) {
          int acc = 0;
#pragma unroll
          for (int j = 0; j < JD; ++j) acc = dot_regs<BITS>(bt.w[b][s][j], aqr[s][j], acc);
          acc = wave_sum_all(acc) - OFF * aqsum[s];
          if (lane == s) mine = acc;
        }
      }
      const float yv = (float)mine * bt.sd[b] * sa_l;
      if (act_l) {
        a.y[(int64_t)lane * a.H + r] = yv;
        if (a.dbg_on && a.dbg.accd) a.dbg.accd[(int64_t)lane * a.H + r] = mine;
      }
      if constexpr (!GIVEN) {
        // combine in slot order: shared first, then j = 0..k-1
        float acc = a.has_shared ? readlane_f(yv, a.k) : 0.0f;
#pragma unroll
        for (int s = 0; s < kMaxSlots - 1; ++s)
          if (s < a.k) acc = __builtin_fmaf(readlane_f(w_l, s), readlane_f(yv, s), acc);
        if (lane == 0) a.out[r] = acc;
      } else if (comb) {
        // the combine over the whole of y_slots as the combine entry point
        // computes it: shared first, then the slots of nonzero weight in
        // order (a slot without work here holds what its own call wrote)
        float yall = yv;
        if (!act_l && lane < a.k && wg_l != 0.0f) yall = a.y[(int64_t)lane * a.H + r];
        float acc = a.has_shared ? readlane_f(yall, a.k) : 0.0f;
#pragma unroll
        for (int s = 0; s < kMaxSlots - 1; ++s) {
          const float ws = readlane_f(wg_l, s);
          if (s < a.k && ws != 0.0f) acc = __builtin_fmaf(ws, readlane_f(yall, s), acc);
        }
        if (lane == 0) a.out[r] = acc;
      }
    }
  };
  for (int rb = r0; rb < r1; rb += 2 * RB) {
    compute_rows(rb, b0);
    if (rb + RB >= r1) break;
    if (rb + 2 * RB < r1) load_rows(rb + 2 * RB, b0);
    compute_rows(rb + RB, b1);
    if (rb + 3 * RB < r1) load_rows(rb + 3 * RB, b1);
  }
}

// ---------------------------------------------------------------------------
// K3 of the mixed-width chain (routing given): the requantisation of every
// slot at its own width (pad[1] of its entry), the down projection of every
// slot at that width, then the combine. Lane l owns the 32-element units l,
// l + 64, ... of each slot's rows: a unit is 32 bytes of int8 codes, 16 of
// int4 and 8 of int2, and meets 32 codes of a in the field order of the
// slot's width (field groups at their natural positions, as rq_codes writes
// them), so a slot of any width keeps every lane
// busy. The loads are the same for every width -- one 16-byte piece per unit
// (two when the call has int8 slots) at a per-slot offset, an int2 unit's 8
// bytes being one half of its piece -- and only the dot product branches on
// the slot's width.
// ---------------------------------------------------------------------------
// 32 int2 fields (8 bytes) against 32 codes in int2 field order
__device__ __forceinline__ int dot_q2_half(uint32_t w0, uint32_t w1, const uint32_t *c, int acc) {
  constexpr uint32_t M = 0x03030303u;
  acc = sdot4((int)(w0 & M), (int)c[0], acc);
  acc = sdot4((int)((w0 >> 2) & M), (int)c[1], acc);
  acc = sdot4((int)((w0 >> 4) & M), (int)c[2], acc);
  acc = sdot4((int)((w0 >> 6) & M), (int)c[3], acc);
  acc = sdot4((int)(w1 & M), (int)c[4], acc);
  acc = sdot4((int)((w1 >> 2) & M), (int)c[5], acc);
  acc = sdot4((int)((w1 >> 4) & M), (int)c[6], acc);
  return sdot4((int)((w1 >> 6) & M), (int)c[7], acc);
}

template <int MAXB, int JU>
__global__ __launch_bounds__(kFfnThreads) void down_mixed_t1_kernel(DownT1Args a) {
  constexpr int NP = MAXB == 8 ? 2 : 1;  // 16-byte pieces loaded per unit
  __shared__ __align__(16) int8_t aq_s[kMaxSlots * kMaxIDown];
  __shared__ float rq_m[kMaxSlots][kFfnWaves];
  __shared__ int rq_c[kMaxSlots][kFfnWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (MOE_WAVE - 1);
  const int wave = tid >> 6;
  const int nw = gridDim.x * kFfnWaves;
  const int gw = blockIdx.x * kFfnWaves + wave;
  const int r0 = uniform((int)((int64_t)gw * a.H / nw)), r1 = uniform((int)((int64_t)(gw + 1) * a.H / nw));
  const int S = a.S;
  const int nu = a.I / 32;  // units per row

  // ---- slot fields (lane s < S holds slot s's), then every slot's a ----
  const int ls = lane < S ? lane : S - 1;
  const uint8_t *down_l = a.slots[ls].w.down;
  const float *sdown_l = a.slots[ls].w.s_down;
  const int bits_l = a.slots[ls].pad[1];
  const int ex_l = a.slots[ls].expert;
  // every slot's a, before anything waits for the slot table (the chain runs
  // for I <= 2048: one float4 of each slot per thread)
  RqRegs<1> rq;
  rq_load<1>(a, rq);
  const bool act_l = lane < S && (lane == a.k ? a.has_shared != 0 : ex_l != -1);
  const bool comb = a.out != nullptr;
  const float wg_l = (comb && lane < a.k) ? a.w_given[lane] : 0.0f;
  if (__ballot(act_l) == 0) {
    if (!comb) return;
    // no slot has work: the combine alone, every slot read back
    for (int r = r0; r < r1; ++r) {
      const float yall = (lane < a.k && wg_l != 0.0f) ? a.y[(int64_t)lane * a.H + r] : 0.0f;
      float acc = 0.0f;
#pragma unroll
      for (int s = 0; s < kMaxSlots - 1; ++s) {
        const float ws = readlane_f(wg_l, s);
        if (s < a.k && ws != 0.0f) acc = __builtin_fmaf(ws, readlane_f(yall, s), acc);
      }
      if (lane == 0) a.out[r] = acc;
    }
    return;
  }
  const uint8_t *dp[kMaxSlots];
  int bits[kMaxSlots], rowb[kMaxSlots];
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s) {
    const int sl = s < S ? s : S - 1;
    dp[s] = readlane_p(down_l, sl);
    // a slot without work reads (valid) rows as if int4 and drops them
    const int b = __builtin_amdgcn_readlane(bits_l, sl);
    bits[s] = (b == 8 || b == 2) ? b : 4;
    rowb[s] = a.I * bits[s] / 8;
  }
  // byte offset of this lane's unit u in a row of slot s: 16-byte aligned;
  // an int2 unit is 8 bytes, read as one half of the piece holding it
  auto unit_off = [&](int s, int u) {
    const int off = u * 4 * bits[s];
    return bits[s] == 2 ? min(off & ~15, rowb[s] - 16) : off;
  };

  struct RowBatch {
    uint4 w[kMaxSlots][JU][NP];
    float sd;
  };
  auto load_rows = [&](int r, RowBatch &bt) {
    r = max(min(r, r1 - 1), 0);
#pragma unroll
    for (int s = 0; s < kMaxSlots; ++s) {
      const uint8_t *row = dp[s] + (int64_t)r * rowb[s];
#pragma unroll
      for (int j = 0; j < JU; ++j) {
        const int u = min(lane + j * MOE_WAVE, nu - 1);
        const int o = unit_off(s, u);
        bt.w[s][j][0] = ldg16_nt(row + o, 0);
        if constexpr (NP == 2) bt.w[s][j][1] = ldg16_nt(row + (bits[s] == 8 ? o + 16 : o), 0);
      }
    }
    bt.sd = gptr(sdown_l)[r];
  };
  RowBatch b0, b1;
  load_rows(r0, b0);  // the first down rows of every slot go out right behind a
  __builtin_amdgcn_sched_barrier(0);  // all of them before a is consumed
  // every slot's codes at its own width (a slot without work: zero codes)
  int aqsum_l;
  float sa_l;
  rq_codes<1, true>(
      a, rq, ex_l,
      [&](int s) {
        const int b = __builtin_amdgcn_readlane(bits_l, s);
        return (b == 8 || b == 2) ? b : 4;
      },
      aq_s, rq_m, rq_c, aqsum_l, sa_l);
  if (r0 >= r1) return;
  load_rows(r0 + 1, b1);

  // every slot's 32 codes per unit, in registers
  uint32_t aqr[kMaxSlots][JU][8];
  int aqsum[kMaxSlots];
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s) {
    aqsum[s] = __builtin_amdgcn_readlane(aqsum_l, s < S ? s : S - 1);
#pragma unroll
    for (int j = 0; j < JU; ++j) {
      const int u = lane + j * MOE_WAVE;
      if (s < S && u < nu) {
        const uint4 v0 = reinterpret_cast<const uint4 *>(aq_s + s * a.I + u * 32)[0];
        const uint4 v1 = reinterpret_cast<const uint4 *>(aq_s + s * a.I + u * 32)[1];
        aqr[s][j][0] = v0.x; aqr[s][j][1] = v0.y; aqr[s][j][2] = v0.z; aqr[s][j][3] = v0.w;
        aqr[s][j][4] = v1.x; aqr[s][j][5] = v1.y; aqr[s][j][6] = v1.z; aqr[s][j][7] = v1.w;
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) aqr[s][j][q] = 0u;
      }
    }
  }
  auto compute_row = [&](int r, const RowBatch &bt) {
    int mine = 0;  // lane s keeps slot s's accumulator
#pragma unroll
    for (int s = 0; s < kMaxSlots; ++s) {
      if (s < S) {
        int acc = 0;
#pragma unroll
        for (int j = 0; j < JU; ++j) {
          const uint4 w = bt.w[s][j][0];
          if (bits[s] == 8) {
            const uint4 w1 = bt.w[s][j][NP - 1];
            const uint32_t wd[8] = {w.x, w.y, w.z, w.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int q = 0; q < 8; ++q) acc = sdot4((int)wd[q], (int)aqr[s][j][q], acc);
          } else if (bits[s] == 4) {
            constexpr uint32_t M = 0x0f0f0f0fu;
            const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              acc = sdot4((int)(wd[m] & M), (int)aqr[s][j][2 * m], acc);
              acc = sdot4((int)((wd[m] >> 4) & M), (int)aqr[s][j][2 * m + 1], acc);
            }
          } else {
            const int u = lane + j * MOE_WAVE;
            const bool hi = (u * 8) - unit_off(s, min(u, nu - 1)) == 8;
            acc = dot_q2_half(hi ? w.z : w.x, hi ? w.w : w.y, aqr[s][j], acc);
          }
        }
        const int off = bits[s] == 8 ? 0 : (bits[s] == 4 ? 8 : 2);
        acc = wave_sum_all(acc) - off * aqsum[s];
        if (lane == s) mine = acc;
      }
    }
    const float yv = (float)mine * bt.sd * sa_l;
    if (act_l) {
      a.y[(int64_t)lane * a.H + r] = yv;
      if (a.dbg_on && a.dbg.accd) a.dbg.accd[(int64_t)lane * a.H + r] = mine;
    }
    if (comb) {
      // the combine as the combine entry point computes it: shared first, then
      // the slots of nonzero weight in order (a slot without work here holds
      // what another call wrote)
      float yall = yv;
      if (!act_l && lane < a.k && wg_l != 0.0f) yall = a.y[(int64_t)lane * a.H + r];
      float acc = a.has_shared ? readlane_f(yall, a.k) : 0.0f;
#pragma unroll
      for (int s = 0; s < kMaxSlots - 1; ++s) {
        const float ws = readlane_f(wg_l, s);
        if (s < a.k && ws != 0.0f) acc = __builtin_fmaf(ws, readlane_f(yall, s), acc);
      }
      if (lane == 0) a.out[r] = acc;
    }
  };
  for (int r = r0; r < r1; r += 2) {
    compute_row(r, b0);
    if (r + 1 >= r1) break;
    if (r + 2 < r1) load_rows(r + 2, b0);
    compute_row(r + 1, b1);
    if (r + 3 < r1) load_rows(r + 3, b1);
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <int BITS, int JG, int NB, bool GIVEN = false>
moe_status launch_gu(moe_ctx *ctx, hipStream_t stream, const GateUpT1Args &g, int nwg) {
  if (GIVEN && g.xf)
    moe_launch_on(ctx, stream, MOE_STAGE_GATEUP, gateup_t1_kernel<BITS, JG, NB, GIVEN, GIVEN>, dim3(nwg),
                  dim3(kFfnThreads), g);
  else
    moe_launch_on(ctx, stream, MOE_STAGE_GATEUP, gateup_t1_kernel<BITS, JG, NB, GIVEN>, dim3(nwg), dim3(kFfnThreads),
                  g);
  MOE_CHECK_LAUNCH("gateup_t1_kernel");
  return MOE_OK;
}
// the down kernel with the requantisation of its launch: one float4 of each
// slot's a per thread up to I = 2048, two above (I <= 4096)
template <int BITS, int JD, int RB, bool GIVEN = false>
moe_status launch_dn(moe_ctx *ctx, hipStream_t stream, const DownT1Args &d, int nwg) {
  if (d.I / 4 <= kFfnThreads)
    moe_launch_on(ctx, stream, MOE_STAGE_DOWN, down_combine_t1_kernel<BITS, JD, RB, GIVEN, 1>, dim3(nwg),
                  dim3(kFfnThreads), d);
  else
    moe_launch_on(ctx, stream, MOE_STAGE_DOWN, down_combine_t1_kernel<BITS, JD, RB, GIVEN, 2>, dim3(nwg),
                  dim3(kFfnThreads), d);
  MOE_CHECK_LAUNCH("down_combine_t1_kernel");
  return MOE_OK;
}

}  // namespace

// Whether the single-token kernels handle this shape.
bool decode_t1_supported(int bits, int H, int I, int k, int has_shared, int n_cu) {
  if (k + has_shared > kMaxSlots || H / 4 > kMaxX4 * kThreads || I > kMaxIDown) return false;
  // a gate/up wave keeps its shared and routed row pairs one per lane, and
  // loads its shared pairs in one batch
  const int64_t waves = (int64_t)n_cu * kFfnWaves;
  const int64_t ns = has_shared ? (I + waves - 1) / waves : 0;
  if (ns > MOE_WAVE) return false;
  // a gate/up workgroup's routed pairs: one per thread in its epilogue
  if (((int64_t)k * I + n_cu - 1) / n_cu > kMaxPairsWg) return false;
  const int jg = moe_chunks_per_lane(H, bits), jd = moe_chunks_per_lane(I, bits);
  switch (bits) {
    case 4: return jg <= T1Shape<4>::JG && jd <= T1Shape<4>::JD && ns <= T1Shape<4>::NB;
    case 8: return jg <= T1Shape<8>::JG && jd <= T1Shape<8>::JD && ns <= T1Shape<8>::NB;
    default: return jg <= T1Shape<2>::JG && jd <= T1Shape<2>::JD && ns <= T1Shape<2>::NB;
  }
}

namespace {
// Scratch layout of the single-token layer: router K slices (the same slicing
// as moe_router_topk, so both paths add the same partial sums in the same
// order), the slot table, the intermediate and its codes, and the outputs a
// caller did not ask for.
struct T1LayerLayout {
  int ks;
  size_t o_part, o_slots, o_A, o_idx, o_w, o_xq, o_sx, o_y, size;
};
T1LayerLayout t1_layer_layout(const moe_ctx *ctx, int E, int k, int S, bool logits_in, int H, int I) {
  T1LayerLayout l;
  l.ks = 1;
  if (!logits_in) {
    const int groups = (E + 3) / 4;
    while (groups * l.ks < 2 * ctx->n_cu && H % (l.ks * 2 * 256) == 0 && l.ks < kMaxSlices) l.ks *= 2;
  } else {
    while (H % (l.ks * 2 * 256) == 0 && l.ks < 8) l.ks *= 2;
  }
  MoeLayout m;
  l.o_part = m.take(sizeof(float) * l.ks * E);
  l.o_slots = m.take(sizeof(SlotEntry) * kMaxSlots);
  l.o_A = m.take(sizeof(float) * S * I);
  l.o_idx = m.take(4 * k);
  l.o_w = m.take(4 * k);
  l.o_xq = m.take(H);
  l.o_sx = m.take(4);
  l.o_y = m.take(sizeof(float) * (k + 1) * H);
  l.size = m.size;
  return l;
}
}  // namespace

size_t layer_t1_scratch_bytes(const moe_ctx *ctx, const moe_router_cfg *cfg, int has_shared, int H, int I) {
  return t1_layer_layout(ctx, cfg->n_experts, cfg->top_k, cfg->top_k + has_shared, cfg->logits_in != 0, H, I).size;
}

moe_status launch_layer_t1(moe_ctx *ctx, int bits, const moe_router_cfg *cfg, const float *x, const float *logits,
                           const float *w_router, const float *bias, const moe_expert_w *experts,
                           const moe_expert_w *shared, int H, int I, float *out, int32_t *topk_idx, float *topk_w,
                           int8_t *xq, float *sx, float *y_slots) {
  const int E = cfg->n_experts, k = cfg->top_k;
  const int S = k + (shared ? 1 : 0);
  const T1LayerLayout l = t1_layer_layout(ctx, E, k, S, logits != nullptr, H, I);
  const int ks = l.ks;
  const int kl = H / ks;
  const size_t o_part = l.o_part, o_slots = l.o_slots, o_A = l.o_A,
               o_idx = l.o_idx, o_w = l.o_w, o_xq = l.o_xq, o_sx = l.o_sx, o_y = l.o_y;
  void *scr = nullptr;
  moe_status st = moe_scratch(ctx, l.size, &scr);
  if (st) return st;
  char *base = static_cast<char *>(scr);
  if (!topk_idx) topk_idx = reinterpret_cast<int32_t *>(base + o_idx);
  if (!topk_w) topk_w = reinterpret_cast<float *>(base + o_w);
  if (!xq) xq = reinterpret_cast<int8_t *>(base + o_xq);
  if (!sx) sx = reinterpret_cast<float *>(base + o_sx);
  if (!y_slots) y_slots = reinterpret_cast<float *>(base + o_y);
  SlotEntry *slots = reinterpret_cast<SlotEntry *>(base + o_slots);
  float *partial = reinterpret_cast<float *>(base + o_part);

  RouterT1Args r{};
  r.x = x;
  r.logits = logits;
  r.wr = w_router;
  r.H = H; r.E = E; r.kl = kl; r.ks = ks;
  r.partial = partial;
  r.xq = xq;
  r.sx = sx;
  // (E+3)/4 logits workgroups per slice plus one that quantises the slice
  moe_launch(ctx, MOE_STAGE_ROUTER, router_gemv_t1_kernel, dim3(logits ? 1 : (E + 3) / 4 + 1, ks), dim3(kThreads), r);
  MOE_CHECK_LAUNCH("router_gemv_t1_kernel");

  GateUpT1Args g{};
  g.partial = partial;
  g.logits = logits;
  g.bias = bias;
  g.E = E; g.k = k; g.ks = ks;
  g.routed_scale = cfg->routed_scale;
  g.top_p = cfg->top_p;
  g.experts = experts;
  if (shared) g.shared = *shared;
  g.has_shared = shared ? 1 : 0;
  g.topk_idx = topk_idx;
  g.topk_w = topk_w;
  g.slots = slots;
  g.xq = xq;
  g.sx = sx;
  g.H = H; g.I = I; g.S = S;
  g.A = reinterpret_cast<float *>(base + o_A);
  g.dbg = ctx->dbg;
  g.dbg_on = ctx->dbg_on ? 1 : 0;
  const int nwg = ctx->n_cu;  // one 8-wave workgroup per CU
  switch (bits) {
    case 4: st = launch_gu<4, T1Shape<4>::JG, T1Shape<4>::NB>(ctx, ctx->stream, g, nwg); break;
    case 8: st = launch_gu<8, T1Shape<8>::JG, T1Shape<8>::NB>(ctx, ctx->stream, g, nwg); break;
    default: st = launch_gu<2, T1Shape<2>::JG, T1Shape<2>::NB>(ctx, ctx->stream, g, nwg); break;
  }
  if (st) return st;

  DownT1Args d{};
  d.A = g.A;
  d.slots = slots;
  d.H = H; d.I = I; d.S = S; d.k = k;
  d.has_shared = shared ? 1 : 0;
  d.y = y_slots;
  d.out = out;
  d.dbg = ctx->dbg;
  d.dbg_on = ctx->dbg_on ? 1 : 0;
  switch (bits) {
    case 4: return launch_dn<4, T1Shape<4>::JD, T1Shape<4>::RB>(ctx, ctx->stream, d, nwg);
    case 8: return launch_dn<8, T1Shape<8>::JD, T1Shape<8>::RB>(ctx, ctx->stream, d, nwg);
    default: return launch_dn<2, T1Shape<2>::JD, T1Shape<2>::RB>(ctx, ctx->stream, d, nwg);
  }
}

namespace {

// The expert FFN of one token with its routing given (ids, activation codes
// and scale from the caller): the gate/up kernel and the requantisation with
// the down kernel above, without the router and the combine, enqueued on `stream` with its
// scratch at `base` (t1_chain_bytes). Slot j's output goes to y_slots row j
// for every valid id whose expert has this width (all of them without a
// width filter), the shared expert's to row k; the other rows are left as
// they were. An id outside [0, E), or one repeated within the token, raises
// the bad-index flag and gives no output (the later copy of a repeated id).
size_t t1_chain_bytes(int I, int S) {
  size_t off = 0;
  for (size_t b : {sizeof(SlotEntry) * kMaxSlots, sizeof(float) * S * I})
    off = moe_round_up(off + b, 256);
  return off;
}

moe_status t1_chain(moe_ctx *ctx, hipStream_t stream, char *base, int bits, const moe_expert_w *experts,
                    const moe_expert_w *shared, const uint8_t *expert_bits, const int8_t *xq, const float *sx,
                    const int32_t *topk_idx, int H, int I, int E, int k, float *y_slots, const float *topk_w = nullptr,
                    float *out = nullptr, const float *xf = nullptr) {
  const int S = k + (shared ? 1 : 0);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = moe_round_up(off + bytes, 256);
    return o;
  };
  const size_t o_slots = take(sizeof(SlotEntry) * kMaxSlots), o_A = take(sizeof(float) * S * I);
  SlotEntry *slots = reinterpret_cast<SlotEntry *>(base + o_slots);

  GateUpT1Args g{};
  g.E = E; g.k = k; g.ks = 1;
  g.experts = experts;
  if (shared) g.shared = *shared;
  g.has_shared = shared ? 1 : 0;
  g.slots = slots;
  g.xq = xq;
  g.sx = sx;
  g.xf = xf;
  g.H = H; g.I = I; g.S = S;
  g.A = reinterpret_cast<float *>(base + o_A);
  g.dbg = ctx->dbg;
  g.dbg_on = ctx->dbg_on ? 1 : 0;
  g.given_idx = topk_idx;
  g.expert_bits = expert_bits;
  g.want_bits = bits;
  g.err = ctx->dev_small;
  const int nwg = ctx->n_cu;
  moe_status st;
  switch (bits) {
    case 4: st = launch_gu<4, T1Shape<4>::JG, T1Shape<4>::NB, true>(ctx, stream, g, nwg); break;
    case 8: st = launch_gu<8, T1Shape<8>::JG, T1Shape<8>::NB, true>(ctx, stream, g, nwg); break;
    default: st = launch_gu<2, T1Shape<2>::JG, T1Shape<2>::NB, true>(ctx, stream, g, nwg); break;
  }
  if (st) return st;

  DownT1Args d{};
  d.A = g.A;
  d.slots = slots;
  d.H = H; d.I = I; d.S = S; d.k = k;
  d.has_shared = shared ? 1 : 0;
  d.y = y_slots;
  d.out = out;
  d.w_given = topk_w;
  d.dbg = ctx->dbg;
  d.dbg_on = ctx->dbg_on ? 1 : 0;
  switch (bits) {
    case 4: return launch_dn<4, T1Shape<4>::JD, T1Shape<4>::RB, true>(ctx, stream, d, nwg);
    case 8: return launch_dn<8, T1Shape<8>::JD, T1Shape<8>::RB, true>(ctx, stream, d, nwg);
    default: return launch_dn<2, T1Shape<2>::JD, T1Shape<2>::RB, true>(ctx, stream, d, nwg);
  }
}

}  // namespace

size_t ffn_t1_scratch_bytes(int I, int S) { return t1_chain_bytes(I, S); }

moe_status launch_ffn_t1(moe_ctx *ctx, int bits, const moe_expert_w *experts, const moe_expert_w *shared,
                         const uint8_t *expert_bits, const int8_t *xq, const float *sx, const int32_t *topk_idx,
                         int H, int I, int E, int k, float *y_slots) {
  void *scr = nullptr;
  moe_status st = moe_scratch(ctx, t1_chain_bytes(I, k + (shared ? 1 : 0)), &scr);
  if (st) return st;
  return t1_chain(ctx, ctx->stream, static_cast<char *>(scr), bits, experts, shared, expert_bits, xq, sx, topk_idx,
                  H, I, E, k, y_slots);
}

// Every width of a mixed layer for one token: the widths' chains one after
// the other on the context stream (each computes only its width's slots, so
// the chains write disjoint rows of y_slots and can share one scratch area),
// the shared expert's width last; with out, that last down kernel also does
// the combine, reading the earlier chains' slots back from y_slots. Running
// the narrower widths' chains on a second stream beside the first was
// slower: the fork and join cost more than the overlap gained.
namespace {
// Every width of a one-token mixed layer in one chain of two kernels: the
// width-split gate/up, then the requantisation and down projection of every
// slot at its width with the combine (when out).
moe_status t1_mixed_chain(moe_ctx *ctx, char *base, int mask, int shared_bits, const moe_expert_w *experts,
                          const moe_expert_w *shared, const uint8_t *expert_bits, const int8_t *xq, const float *sx,
                          const float *xf, const int32_t *topk_idx, const float *topk_w, int H, int I, int E, int k,
                          float *y_slots, float *out) {
  // the down kernel's requantisation holds one float4 of each slot's a per
  // thread (t1_mixed_chain_ok admits intermediates up to 2048 only)
  if (I / 4 > kFfnThreads) return moe_fail(MOE_EINVAL, "mixed single-token chain: intermediate %d above 2048", I);
  const int S = k + (shared ? 1 : 0);
  MoeLayout m;
  const size_t o_slots = m.take(sizeof(SlotEntry) * kMaxSlots), o_A = m.take(sizeof(float) * S * I);
  SlotEntry *slots = reinterpret_cast<SlotEntry *>(base + o_slots);
  GateUpT1Args g{};
  g.E = E; g.k = k; g.ks = 1;
  g.experts = experts;
  if (shared) g.shared = *shared;
  g.has_shared = shared ? 1 : 0;
  g.slots = slots;
  g.xq = xq;
  g.sx = sx;
  g.xf = xf;
  g.H = H; g.I = I; g.S = S;
  g.A = reinterpret_cast<float *>(base + o_A);
  g.dbg = ctx->dbg;
  g.dbg_on = ctx->dbg_on ? 1 : 0;
  g.given_idx = topk_idx;
  g.expert_bits = expert_bits;
  g.err = ctx->dev_small;
  const int nwg = ctx->n_cu;
  if (xf)
    moe_launch(ctx, MOE_STAGE_GATEUP, gateup_mixed_t1_kernel<true>, dim3(nwg), dim3(kFfnThreads), g, mask, shared_bits);
  else
    moe_launch(ctx, MOE_STAGE_GATEUP, gateup_mixed_t1_kernel<false>, dim3(nwg), dim3(kFfnThreads), g, mask,
               shared_bits);
  MOE_CHECK_LAUNCH("gateup_mixed_t1_kernel");
  DownT1Args d{};
  d.A = g.A;
  d.slots = slots;
  d.H = H; d.I = I; d.S = S; d.k = k;
  d.has_shared = shared ? 1 : 0;
  d.y = y_slots;
  d.out = out;
  d.w_given = topk_w;
  d.dbg = ctx->dbg;
  d.dbg_on = ctx->dbg_on ? 1 : 0;
  moe_launch(ctx, MOE_STAGE_DOWN, down_mixed_t1_kernel<4, 1>, dim3(nwg), dim3(kFfnThreads), d);
  MOE_CHECK_LAUNCH("down_mixed_t1_kernel");
  return MOE_OK;
}
}  // namespace

// Whether the one-chain mixed path takes a call: int4 and int2 experts (the
// shared one included) and at most 64 units of 32 intermediate elements per
// lane (with int8 slots, or a longer intermediate, its down kernel would hold
// twice the registers per slot and spill); other mixes run one chain per width.
static bool t1_mixed_chain_ok(const moe_ctx *ctx, int mask, int shared_bits, bool has_shared, int I, int k) {
  const int m = mask | (has_shared ? 1 << shared_bits : 0);
  if ((m & ~((1 << 4) | (1 << 2))) != 0 || I / 32 > MOE_WAVE_HOST) return false;
  // the gate/up kernel's per-width minimum workgroup counts, at their largest
  // (two widths, the routed slots split between them, the shared expert on
  // one of them), must fit its grid of one workgroup per CU
  const int64_t worst = ((int64_t)k * I + kMaxPairsWg - 1) / kMaxPairsWg + 2 +
                        (has_shared ? (I + kFfnWaves * MOE_WAVE_HOST - 1) / (kFfnWaves * MOE_WAVE_HOST) : 0);
  return worst <= ctx->n_cu;
}

moe_status launch_ffn_t1_mixed(moe_ctx *ctx, const int *widths, int n_widths, int shared_bits,
                               const moe_expert_w *experts, const moe_expert_w *shared, const uint8_t *expert_bits,
                               const int8_t *xq, const float *sx, const float *xf, const int32_t *topk_idx,
                               const float *topk_w, int H, int I, int E, int k, float *y_slots, float *out) {
  void *scr = nullptr;
  moe_status st = moe_scratch(ctx, t1_chain_bytes(I, k + (shared ? 1 : 0)), &scr);
  if (st) return st;
  int mask = 0;
  for (int w = 0; w < n_widths; ++w) mask |= 1 << widths[w];
  if (n_widths > 1 && t1_mixed_chain_ok(ctx, mask, shared_bits, shared != nullptr, I, k))
    return t1_mixed_chain(ctx, static_cast<char *>(scr), mask, shared_bits, experts, shared, expert_bits, xq, sx, xf,
                          topk_idx, topk_w, H, I, E, k, y_slots, out);
  const int last_bits = shared ? shared_bits : widths[n_widths - 1];
  int order[3], n = 0;
  for (int w = 0; w < n_widths; ++w)
    if (widths[w] != last_bits) order[n++] = widths[w];
  order[n++] = last_bits;
  for (int w = 0; w < n; ++w) {
    const bool last = w == n - 1;
    st = t1_chain(ctx, ctx->stream, static_cast<char *>(scr), order[w], experts, last ? shared : nullptr,
                  expert_bits, xq, sx, topk_idx, H, I, E, k, y_slots, last ? topk_w : nullptr, last ? out : nullptr, xf);
    if (st) return st;
  }
  return MOE_OK;
}
