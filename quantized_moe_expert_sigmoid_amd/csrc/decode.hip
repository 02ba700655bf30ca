// Single-token (decode) layer path in three kernels: router logits with the
// activation quantisation; top-k fused with a streaming gate/up GEMV; and the
// int8 requantisation fused with the down GEMV and the combine.
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
//     logits (one wave per expert and slice); the workgroups of column 0 also
//     find max|x| over the token and quantise their slice of x to int8.
//  K2 gateup_t1_kernel (one 512-thread workgroup per CU): every workgroup
//     sums the logit slices in fixed order, applies the sigmoid and the bias,
//     selects the top-k in one wave (k rounds of a DPP wave max; equal keys go
//     to the lower id) and builds the slot table in LDS; workgroup 0 also
//     publishes ids, weights and the slot table. Then the S*I (gate row, up
//     row) pairs, split into equal contiguous ranges over all waves, stream
//     through 16-byte loads two batches deep against the token's int8
//     activations held in registers (field order); DPP reductions; one store
//     of a = silu(g)*u per row pair.
//  K3 down_combine_t1_kernel (one 512-thread workgroup per CU): each wave
//     issues its first down-row loads, then the workgroup loads every slot's
//     a (an L2 hit), finds max|a| per slot and writes the int8 codes to LDS
//     while the weights are in flight; each wave then multiplies its H rows
//     of every slot's down matrix, writes y per slot and the combined output
//     out[r] = y_shared + sum_j w_j y_j (the same fma order as moe_combine).
// Kernel boundaries order the three steps: no atomics, no cross-workgroup
// waits (contended device-scope atomics serialise at the memory side).
// Streaming loads are branch-free: a lane whose chunk index passes the row
// end reads a clamped in-bounds address and meets zero activation bytes.
#include "gemv_common.h"

namespace {

constexpr int kThreads = 256;                      // router kernel
constexpr int kFfnThreads = 512;                   // gate/up and down kernels
constexpr int kFfnWaves = kFfnThreads / MOE_WAVE;  // 8 waves: one workgroup per CU
constexpr int kMaxSlots = 9;                       // top-k <= 8 plus the shared expert
constexpr int kMaxSlices = 16;                     // K slices of the router logits
constexpr int kMaxE = 1024;
constexpr int kMaxX4 = 8;       // float4 of x per thread in the max pass: H <= 8192
constexpr int kMaxIDown = 4096;  // intermediate held in LDS by the down kernel

// One slot of the token: the expert's weights and its routing weight.
struct SlotEntry {
  moe_expert_w w;
  float weight;  // routing weight (1 for the shared expert)
  int expert;    // expert id (-1 for the shared expert)
  int pad[2];
};
static_assert(sizeof(SlotEntry) == 64, "slot entries are 64 bytes");

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
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
  if (!a.logits) {
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
  }
  if (blockIdx.x != 0) return;
  // column 0: max|x| over the whole token, then quantise this slice of x
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
  float routed_scale;
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
  int H, I, S;
  float *A;  // [S][I]
  moe_debug_bufs dbg;
  int dbg_on;
};

// k rounds of (lane-local best, wave max of the keys, lowest id among the
// maxima) over keys in LDS: descending key, then ascending id.
__device__ __forceinline__ void wave_topk(const float *key_s, const float *sig_s, int E, int k, int lane,
                                          int *sel_id, float *sel_sig) {
  const int per = (E + MOE_WAVE - 1) / MOE_WAVE;
  unsigned taken = 0;
  for (int r = 0; r < k; ++r) {
    float lb = -__builtin_inff();
    int li = 0x7fffffff;
    for (int m = 0; m < per; ++m) {
      const int e = lane + m * MOE_WAVE;
      const bool ok = (e < E) & !((taken >> m) & 1u);
      const float kk = key_s[e < E ? e : E - 1];
      const bool better = ok & ((li == 0x7fffffff) | (kk > lb));
      lb = better ? kk : lb;
      li = better ? e : li;
    }
    const float wm = wave_max_dpp(lb);
    const int wid = wave_min_dpp((lb == wm) ? li : 0x7fffffff);
    if ((wid & (MOE_WAVE - 1)) == lane) taken |= 1u << (wid / MOE_WAVE);
    if (lane == 0) {
      sel_id[r] = wid;
      sel_sig[r] = sig_s[wid];
    }
  }
}

template <int BITS, int JG, int NB>
struct GuBatch {
  uint4 g[NB][JG], u[NB][JG];
};

// Row pointers of a wave's (at most two) slots.
struct WaveSlots {
  int s_first, I;
  const uint8_t *gate0, *up0, *gate1, *up1;
};

// Load NB row pairs starting at row pair qb; rows past the wave's range
// re-read its last row (their results are dropped).
template <int BITS, int JG, int NB>
__device__ __forceinline__ void gu_load(const WaveSlots &ws, int qb, int q1, int lane, int rowbytes, int cpr,
                                        GuBatch<BITS, JG, NB> &bt) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int q = (qb + b < q1) ? qb + b : q1 - 1;
    const int slot = uniform(q / ws.I);
    const int i = q - slot * ws.I;
    const bool first = slot == ws.s_first;
    const uint8_t *gate = (first ? ws.gate0 : ws.gate1) + (int64_t)i * rowbytes;
    const uint8_t *up = (first ? ws.up0 : ws.up1) + (int64_t)i * rowbytes;
#pragma unroll
    for (int j = 0; j < JG; ++j) {
      int c = lane + j * MOE_WAVE;
      c = c < cpr ? c : cpr - 1;
      bt.g[b][j] = ldg16(gate, c);
      bt.u[b][j] = ldg16(up, c);
    }
  }
}

// Dot products of one batch; lane (row pair - q0) keeps that pair's sums.
template <int BITS, int JG, int NB>
__device__ __forceinline__ void gu_compute(int qb, int q0, int q1, int lane, const GuBatch<BITS, JG, NB> &bt,
                                           const ActChunk<BITS> (&xr)[JG], int &res_g, int &res_u) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (qb + b < q1) {
      int ag = 0, au = 0;
#pragma unroll
      for (int j = 0; j < JG; ++j) {
        ag = dot_regs<BITS>(bt.g[b][j], xr[j], ag);
        au = dot_regs<BITS>(bt.u[b][j], xr[j], au);
      }
      ag = wave_sum_all(ag);
      au = wave_sum_all(au);
      if (lane == qb + b - q0) {
        res_g = ag;
        res_u = au;
      }
    }
  }
}

template <int BITS, int JG, int NB>
__global__ __launch_bounds__(kFfnThreads) void gateup_t1_kernel(GateUpT1Args a) {
  constexpr int OFF = QFmt<BITS>::kOff;
  __shared__ float key_s[kMaxE], sig_s[kMaxE];
  __shared__ __align__(16) moe_expert_w exp_s[kMaxE];
  __shared__ int sel_id[16];
  __shared__ float sel_sig[16];
  __shared__ SlotEntry slot_s[kMaxSlots];
  const int tid = threadIdx.x;
  const int lane = tid & (MOE_WAVE - 1);
  const int wave = tid >> 6;
  const int nw = gridDim.x * kFfnWaves;
  const int gw = blockIdx.x * kFfnWaves + wave;
  const int Q = a.S * a.I;
  const int q0 = uniform((int)((int64_t)gw * Q / nw)), q1 = uniform((int)((int64_t)(gw + 1) * Q / nw));
  const int rowbytes = a.H * BITS / 8;
  const int cpr = rowbytes / 16;

  // ---- routing keys (every thread, loads first) ----
  constexpr int kPer = kMaxE / kFfnThreads;
  float zs[kPer][kMaxSlices], bs[kPer];
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int e = tid + m * kFfnThreads;
    const bool ok = e < a.E;
#pragma unroll
    for (int s = 0; s < kMaxSlices; ++s) {
      zs[m][s] = 0.0f;
      if (ok && (a.logits ? s == 0 : s < a.ks))
        zs[m][s] = a.logits ? a.logits[e] : a.partial[(int64_t)s * a.E + e];
    }
    bs[m] = (ok && a.bias) ? a.bias[e] : 0.0f;
  }
  // the expert pointer table into LDS (48 bytes per expert, 16-byte pieces)
  {
    const uint4 *src = reinterpret_cast<const uint4 *>(a.experts);
    uint4 *dst = reinterpret_cast<uint4 *>(exp_s);
    for (int i = tid; i < 3 * a.E; i += kFfnThreads) dst[i] = ldg16(src, i);
  }
  // the token's activations in registers (the same for every slot)
  ActChunk<BITS> xr[JG];
  int xs_lane = 0;
#pragma unroll
  for (int j = 0; j < JG; ++j) {
    int bs1 = 0;
    act_chunk_clamped<BITS>(a.xq, lane + j * MOE_WAVE, cpr, xr[j], bs1);
    xs_lane += bs1;
  }
  const float sxv = a.sx[0];
  const int nsum = a.logits ? 1 : a.ks;
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int e = tid + m * kFfnThreads;
    float z = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxSlices; ++s)
      if (s < nsum) z += zs[m][s];
    const float sg = 1.0f / (1.0f + moe_exp_f32(-z));
    float key = sg + bs[m];
    if (key != key) key = -__builtin_inff();  // a NaN key ranks last
    if (e < a.E) {
      key_s[e] = key;
      sig_s[e] = sg;
    }
  }
  __syncthreads();

  // ---- top-k and the slot table (wave 0) ----
  if (wave == 0) {
    wave_topk(key_s, sig_s, a.E, a.k, lane, sel_id, sel_sig);
    float sum = 0.0f;
    for (int j = 0; j < a.k; ++j) sum += sel_sig[j];
    uint4 row[4];
    bool have = false;
    if (lane < a.k) {
      const int e = sel_id[lane];
      const float wgt = a.routed_scale * (sel_sig[lane] / sum);
      const uint4 *src = reinterpret_cast<const uint4 *>(exp_s + e);
      row[0] = src[0];
      row[1] = src[1];
      row[2] = src[2];
      row[3] = make_uint4(__float_as_uint(wgt), (uint32_t)e, 0u, 0u);
      have = true;
      if (blockIdx.x == 0) {
        a.topk_idx[lane] = e;
        a.topk_w[lane] = wgt;
      }
    } else if (lane == a.k && a.has_shared) {
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
      if (blockIdx.x == 0) {
        uint4 *gdst = reinterpret_cast<uint4 *>(a.slots + lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) gdst[q] = row[q];
      }
    }
  }
  __syncthreads();
  if (q0 >= q1) return;

  // ---- this wave's slots and row pairs ----
  WaveSlots ws;
  ws.I = a.I;
  ws.s_first = uniform(q0 / a.I);
  const int s_last = uniform((q1 - 1) / a.I);
  ws.gate0 = uniform_p(slot_s[ws.s_first].w.gate);
  ws.up0 = uniform_p(slot_s[ws.s_first].w.up);
  ws.gate1 = uniform_p(slot_s[s_last].w.gate);
  ws.up1 = uniform_p(slot_s[s_last].w.up);

  GuBatch<BITS, JG, NB> b0, b1;
  gu_load<BITS, JG, NB>(ws, q0, q1, lane, rowbytes, cpr, b0);

  const int my_q = q0 + lane;
  const bool mine = my_q < q1;
  const int my_slot = (mine ? my_q : q0) / a.I;
  const int my_i = (mine ? my_q : q0) - my_slot * a.I;
  const float sg = gptr(slot_s[my_slot].w.s_gate)[my_i];
  const float su = gptr(slot_s[my_slot].w.s_up)[my_i];
  const int xsum = wave_sum_all(xs_lane);

  int res_g = 0, res_u = 0;
  for (int qb = q0; qb < q1; qb += 2 * NB) {
    if (qb + NB < q1) gu_load<BITS, JG, NB>(ws, qb + NB, q1, lane, rowbytes, cpr, b1);
    gu_compute<BITS, JG, NB>(qb, q0, q1, lane, b0, xr, res_g, res_u);
    if (qb + NB >= q1) break;
    if (qb + 2 * NB < q1) gu_load<BITS, JG, NB>(ws, qb + 2 * NB, q1, lane, rowbytes, cpr, b0);
    gu_compute<BITS, JG, NB>(qb + NB, q0, q1, lane, b1, xr, res_g, res_u);
  }

  if (mine) {
    const int gi = res_g - OFF * xsum;
    const int ui = res_u - OFF * xsum;
    const float g = (float)gi * sg * sxv;
    const float u = (float)ui * su * sxv;
    const float av = moe_silu_f32(g) * u;
    const int64_t o = (int64_t)my_slot * a.I + my_i;
    a.A[o] = av;
    if (a.dbg_on) {
      if (a.dbg.accg) a.dbg.accg[o] = gi;
      if (a.dbg.accu) a.dbg.accu[o] = ui;
      if (a.dbg.a) a.dbg.a[o] = av;
    }
  }
}

// ---------------------------------------------------------------------------
// K3: requantisation + down projection of every slot + combine
// ---------------------------------------------------------------------------
struct DownT1Args {
  const SlotEntry *slots;
  const float *A;  // [S][I]
  int H, I, S, k, has_shared;
  float *y;    // [S][H] (the token's y_slots; slot stride H)
  float *out;  // [H]
  moe_debug_bufs dbg;
  int dbg_on;
};

constexpr int kRqF4 = kMaxIDown / 4 / kFfnThreads;  // float4 of one slot's a per thread (2)

template <int BITS, int JD, int RB>
__global__ __launch_bounds__(kFfnThreads) void down_combine_t1_kernel(DownT1Args a) {
  constexpr int OFF = QFmt<BITS>::kOff;
  __shared__ __align__(16) int8_t aq_s[kMaxSlots * kMaxIDown];
  __shared__ float red_s[kFfnWaves][kMaxSlots];
  const int tid = threadIdx.x;
  const int lane = tid & (MOE_WAVE - 1);
  const int wave = tid >> 6;
  const int nw = gridDim.x * kFfnWaves;
  const int gw = blockIdx.x * kFfnWaves + wave;
  const int r0 = uniform((int)((int64_t)gw * a.H / nw)), r1 = uniform((int)((int64_t)(gw + 1) * a.H / nw));
  const int rowbytes = a.I * BITS / 8;
  const int cpr = rowbytes / 16;
  const int S = a.S;

  // lane s < S holds slot s's fields; the down pointers become uniform
  const int ls = lane < S ? lane : S - 1;
  const uint8_t *down_l = a.slots[ls].w.down;
  const float *sdown_l = a.slots[ls].w.s_down;
  const float w_l = a.slots[ls].weight;
  const uint8_t *dp[kMaxSlots];
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s) dp[s] = readlane_p(down_l, s < S ? s : S - 1);

  // ---- every slot's a first (an L2 hit), then the first down rows ----
  const int n4 = a.I / 4;  // float4 per slot
  float4 av[kMaxSlots][kRqF4];
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s)
#pragma unroll
    for (int c = 0; c < kRqF4; ++c) {
      const int f = tid + c * kFfnThreads;
      av[s][c] = (s < S && f < n4) ? reinterpret_cast<const float4 *>(a.A + (int64_t)s * a.I)[f]
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  struct RowBatch {
    uint4 w[RB][kMaxSlots][JD];
    float sd[RB];
  };
  auto load_rows = [&](int rb, RowBatch &bt) {
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int r = (rb + b < r1) ? rb + b : r1 - 1;
#pragma unroll
      for (int s = 0; s < kMaxSlots; ++s) {
        if (s < S) {
#pragma unroll
          for (int j = 0; j < JD; ++j) {
            int c = lane + j * MOE_WAVE;
            c = c < cpr ? c : cpr - 1;
            bt.w[b][s][j] = ldg16(dp[s] + (int64_t)r * rowbytes, c);
          }
        }
      }
      bt.sd[b] = gptr(sdown_l)[r];
    }
  };
  RowBatch b0, b1;
  if (r0 < r1) load_rows(r0, b0);
  if (r0 + RB < r1) load_rows(r0 + RB, b1);

  // ---- requantise every slot's a into LDS (the workgroup together) ----
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s) {
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < kRqF4; ++c)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(av[s][c].x), fabsf(av[s][c].y)), fmaxf(fabsf(av[s][c].z), fabsf(av[s][c].w))));
    m = wave_max_dpp(m);
    if (lane == 0) red_s[wave][s] = m;
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s) {
    if (s < S) {
      float m = 0.0f;
#pragma unroll
      for (int w = 0; w < kFfnWaves; ++w) m = fmaxf(m, red_s[w][s]);
      const float sc = (m == 0.0f) ? 0.0f : m / 127.0f;
#pragma unroll
      for (int c = 0; c < kRqF4; ++c) {
        const int f = tid + c * kFfnThreads;
        if (f < n4) {
          const float vv[4] = {av[s][c].x, av[s][c].y, av[s][c].z, av[s][c].w};
          uint32_t word = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            int q = 0;
            if (m != 0.0f) {
              float r = __builtin_rintf(vv[j] / sc);
              r = fminf(fmaxf(r, -127.0f), 127.0f);
              q = (int)r;
            }
            word |= (uint32_t)(uint8_t)(int8_t)q << (8 * j);
          }
          reinterpret_cast<uint32_t *>(aq_s + s * a.I)[f] = word;
          if (blockIdx.x == 0 && a.dbg_on && a.dbg.aq) reinterpret_cast<uint32_t *>(a.dbg.aq + (int64_t)s * a.I)[f] = word;
        }
      }
      if (blockIdx.x == 0 && tid == 0 && a.dbg_on && a.dbg.sa) a.dbg.sa[s] = sc;
    }
  }
  float sa_l = 0.0f;  // lane s < S: slot s's scale
  {
    float m = 0.0f;
#pragma unroll
    for (int w = 0; w < kFfnWaves; ++w) m = fmaxf(m, red_s[w][ls]);
    sa_l = (m == 0.0f) ? 0.0f : m / 127.0f;
  }
  __syncthreads();
  if (r0 >= r1) return;

  // every slot's codes, in registers in field order
  ActChunk<BITS> aqr[kMaxSlots][JD];
  int aqsum[kMaxSlots];
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s) {
    int bs_lane = 0;
#pragma unroll
    for (int j = 0; j < JD; ++j) {
      const int c = lane + j * MOE_WAVE;
      if (s < S && c < cpr) {
        constexpr int EPC = QFmt<BITS>::kEpc;
        uint4 v[EPC / 16];
#pragma unroll
        for (int u = 0; u < EPC / 16; ++u) v[u] = reinterpret_cast<const uint4 *>(aq_s + s * a.I + c * EPC)[u];
        int bs = 0;
        act_chunk_from<BITS>(v, aqr[s][j], bs);
        bs_lane += bs;
      } else {
        zero_chunk<BITS>(aqr[s][j]);
      }
    }
    aqsum[s] = wave_sum_all(bs_lane);
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
      if (lane < S) {
        a.y[(int64_t)lane * a.H + r] = yv;
        if (a.dbg_on && a.dbg.accd) a.dbg.accd[(int64_t)lane * a.H + r] = mine;
      }
      // combine in slot order: shared first, then j = 0..k-1
      float acc = a.has_shared ? readlane_f(yv, a.k) : 0.0f;
#pragma unroll
      for (int s = 0; s < kMaxSlots - 1; ++s)
        if (s < a.k) acc = __builtin_fmaf(readlane_f(w_l, s), readlane_f(yv, s), acc);
      if (lane == 0) a.out[r] = acc;
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
// launch
// ---------------------------------------------------------------------------
template <int BITS, int JG, int NB>
moe_status launch_gu(moe_ctx *ctx, const GateUpT1Args &g, int nwg) {
  {
    MoeTimer tm_(ctx, MOE_STAGE_GATEUP);
    hipLaunchKernelGGL((gateup_t1_kernel<BITS, JG, NB>), dim3(nwg), dim3(kFfnThreads), 0, ctx->stream, g);
  }
  MOE_CHECK_LAUNCH("gateup_t1_kernel");
  return MOE_OK;
}
template <int BITS, int JD, int RB>
moe_status launch_dn(moe_ctx *ctx, const DownT1Args &d, int nwg) {
  {
    MoeTimer tm_(ctx, MOE_STAGE_DOWN);
    hipLaunchKernelGGL((down_combine_t1_kernel<BITS, JD, RB>), dim3(nwg), dim3(kFfnThreads), 0, ctx->stream, d);
  }
  MOE_CHECK_LAUNCH("down_combine_t1_kernel");
  return MOE_OK;
}

// Per-width kernel shapes: 16-byte chunks per lane of a gate/up row (JG) and
// of a down row (JD) the kernels are compiled for, row pairs per gate/up
// batch (NB), down rows per batch (RB).
template <int BITS>
struct T1Shape;
template <>
struct T1Shape<4> {
  static constexpr int JG = 3, JD = 1, NB = 3, RB = 1;
};
template <>
struct T1Shape<8> {
  static constexpr int JG = 6, JD = 2, NB = 2, RB = 1;
};
template <>
struct T1Shape<2> {
  static constexpr int JG = 2, JD = 1, NB = 4, RB = 1;
};

}  // namespace

// Whether the single-token kernels handle this shape.
bool decode_t1_supported(int bits, int H, int I, int k, int has_shared, int n_cu) {
  if (k + has_shared > kMaxSlots || H / 4 > kMaxX4 * kThreads || I > kMaxIDown) return false;
  // each gate/up wave owns at most 64 row pairs (one per lane)
  const int64_t waves = (int64_t)n_cu * kFfnWaves;
  if ((int64_t)(k + has_shared) * I > 64 * waves) return false;
  const int jg = moe_chunks_per_lane(H, bits), jd = moe_chunks_per_lane(I, bits);
  switch (bits) {
    case 4: return jg <= T1Shape<4>::JG && jd <= T1Shape<4>::JD;
    case 8: return jg <= T1Shape<8>::JG && jd <= T1Shape<8>::JD;
    default: return jg <= T1Shape<2>::JG && jd <= T1Shape<2>::JD;
  }
}

moe_status launch_layer_t1(moe_ctx *ctx, int bits, const moe_router_cfg *cfg, const float *x, const float *logits,
                           const float *w_router, const float *bias, const moe_expert_w *experts,
                           const moe_expert_w *shared, int H, int I, float *out, int32_t *topk_idx, float *topk_w,
                           int8_t *xq, float *sx, float *y_slots) {
  const int E = cfg->n_experts, k = cfg->top_k;
  const int S = k + (shared ? 1 : 0);
  // router K slices (the same slicing as moe_router_topk, so both paths add
  // the same partial sums in the same order)
  int ks = 1;
  if (!logits) {
    const int groups = (E + 3) / 4;
    while (groups * ks < 2 * ctx->n_cu && H % (ks * 2 * 256) == 0 && ks < kMaxSlices) ks *= 2;
  } else {
    while (H % (ks * 2 * 256) == 0 && ks < 8) ks *= 2;
  }
  const int kl = H / ks;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = moe_round_up(off + bytes, 256);
    return o;
  };
  const size_t o_part = take(sizeof(float) * ks * E), o_slots = take(sizeof(SlotEntry) * kMaxSlots),
               o_A = take(sizeof(float) * S * I), o_idx = take(4 * k), o_w = take(4 * k), o_xq = take(H),
               o_sx = take(4), o_y = take(sizeof(float) * (k + 1) * H);
  void *scr = nullptr;
  moe_status st = moe_scratch(ctx, off, &scr);
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
  {
    MoeTimer tm_(ctx, MOE_STAGE_ROUTER);
    hipLaunchKernelGGL(router_gemv_t1_kernel, dim3(logits ? 1 : (E + 3) / 4, ks), dim3(kThreads), 0, ctx->stream, r);
  }
  MOE_CHECK_LAUNCH("router_gemv_t1_kernel");

  GateUpT1Args g{};
  g.partial = partial;
  g.logits = logits;
  g.bias = bias;
  g.E = E; g.k = k; g.ks = ks;
  g.routed_scale = cfg->routed_scale;
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
    case 4: st = launch_gu<4, T1Shape<4>::JG, T1Shape<4>::NB>(ctx, g, nwg); break;
    case 8: st = launch_gu<8, T1Shape<8>::JG, T1Shape<8>::NB>(ctx, g, nwg); break;
    default: st = launch_gu<2, T1Shape<2>::JG, T1Shape<2>::NB>(ctx, g, nwg); break;
  }
  if (st) return st;

  DownT1Args d{};
  d.slots = slots;
  d.A = g.A;
  d.H = H; d.I = I; d.S = S; d.k = k;
  d.has_shared = shared ? 1 : 0;
  d.y = y_slots;
  d.out = out;
  d.dbg = ctx->dbg;
  d.dbg_on = ctx->dbg_on ? 1 : 0;
  switch (bits) {
    case 4: return launch_dn<4, T1Shape<4>::JD, T1Shape<4>::RB>(ctx, d, nwg);
    case 8: return launch_dn<8, T1Shape<8>::JD, T1Shape<8>::RB>(ctx, d, nwg);
    default: return launch_dn<2, T1Shape<2>::JD, T1Shape<2>::RB>(ctx, d, nwg);
  }
}
