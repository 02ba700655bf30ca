// SwiGLU expert FFN over packed int8 / int4 / int2 weights with int8
// activations and exact int32 integer dot products.
//
// agentlenshq.com, "Colibri: running GLM-5.2 744B MoE on consumer hardware",
// section "Key features": packed int4/int8/int2 kernels with per-row scales
// and dequantisation on use; int8 matmuls as integer dot products.
// Section "Memory split": the shared expert is resident and always applied.
// remio.ai, "Colibri shows how to run GLM-5.2 on a low-spec PC", section "The
// RAM wall became a storage problem": an expert needed by several batch
// positions is read once -- here every workgroup streams its weight rows once
// for all the tokens routed to that expert.
//
// Work decomposition (all on the context stream, no host round trip):
//  1. bucket_kernel: per-expert token lists and the active-expert list.
//  2. ffn_gateup_kernel: one workgroup per (active expert, tile of I rows);
//     4 waves x RW rows of gate and up. Each lane streams 16-byte chunks of
//     the packed rows, unpacks them in registers (offset-binary fields) and
//     runs v_dot4_i32_i8 against the activation bytes staged in LDS in the
//     matching field order. The offset (8 for int4, 2 for int2) is removed
//     once per row with the token's activation sum. Epilogue: scales, SiLU,
//     a = silu(g)*u to scratch, per-tile max|a|.
//  3. ffn_requant_kernel: per (token, slot) pair: sa = max|a|/127, aq.
//  4. ffn_down_kernel: one workgroup per (active expert, tile of H rows),
//     same inner loop against aq; y = acc * s_down * sa into y_slots.
#include <algorithm>

#include "moe_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;
constexpr int kTG = 4;          // tokens per group held in LDS / registers
constexpr int kMaxDim = 8192;   // max H and I

struct FfnArgs {
  const moe_expert_w *experts;
  moe_expert_w shared;
  int has_shared;
  const int8_t *xq;
  const float *sx;
  const int32_t *topk_idx;
  const uint8_t *expert_bits;
  int bits;
  int T, H, I, E, k;
  const int32_t *counts, *offsets, *perm, *active, *n_active;
  float *A;        // [P][I] SwiGLU intermediate
  float *tilemax;  // [P][tiles1] per-tile max|a|
  int8_t *aq;      // [P][I]
  float *sa;       // [P]
  float *y;        // [T][k+1][H]
  moe_debug_bufs dbg;
  int dbg_on;
  int tiles1, tiles2;
};

// Rows per wave and max 16-byte chunks per lane per row (dims <= 8192).
template <int BITS>
struct Shape {
  static constexpr int kJ = kMaxDim * BITS / 8 / 16 / MOE_WAVE;  // 8, 4, 2
  static constexpr int kRwGU = 8 / kJ;                           // 1, 2, 4 rows (x2 matrices)
  static constexpr int kRwD = 16 / kJ;                           // 2, 4, 8 rows
};

struct ExpertRef {
  moe_expert_w w;
  int ntok, tok_base, is_shared;
};

__device__ __forceinline__ bool resolve(const FfnArgs &a, int d, ExpertRef &r) {
  const int na = *a.n_active;
  if (d < na) {
    const int e = a.active[d];
    r.w = a.experts[e];
    r.ntok = a.counts[e];
    r.tok_base = a.offsets[e];
    r.is_shared = 0;
    return true;
  }
  if (a.has_shared && d == na) {
    r.w = a.shared;
    r.ntok = a.T;
    r.tok_base = 0;
    r.is_shared = 1;
    return true;
  }
  return false;
}

__device__ __forceinline__ void token_of(const FfnArgs &a, const ExpertRef &r, int g, int &t, int &slot) {
  if (r.is_shared) {
    t = g;
    slot = a.k;
  } else {
    const int ent = a.perm[r.tok_base + g];
    t = ent / a.k;
    slot = ent - t * a.k;
  }
}

// Reorder 16 activation bytes (elements 16u..16u+15) into the field order of
// the unpacked weights (see act_order_q4 / act_order_q2).
template <int BITS>
__device__ __forceinline__ uint4 act_order16(uint4 v) {
  if constexpr (BITS == 4) {
    uint4 o;
    act_order_q4(v.x, v.y, o.x, o.y);
    act_order_q4(v.z, v.w, o.z, o.w);
    return o;
  } else if constexpr (BITS == 2) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
    act_order_q2(d, o);
    return make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    return v;
  }
}

__device__ __forceinline__ int bytesum16(uint4 v) {
  const int ones = 0x01010101;
  int s = sdot4((int)v.x, ones, 0);
  s = sdot4((int)v.y, ones, s);
  s = sdot4((int)v.z, ones, s);
  return sdot4((int)v.w, ones, s);
}

// One 16-byte weight chunk against its activation bytes (LDS, field order).
template <int BITS>
__device__ __forceinline__ int dot_chunk(uint4 w, const int8_t *xc, int acc) {
  if constexpr (BITS == 8) {
    const uint4 x = *reinterpret_cast<const uint4 *>(xc);
    acc = sdot4((int)w.x, (int)x.x, acc);
    acc = sdot4((int)w.y, (int)x.y, acc);
    acc = sdot4((int)w.z, (int)x.z, acc);
    return sdot4((int)w.w, (int)x.w, acc);
  } else if constexpr (BITS == 4) {
    constexpr uint32_t M = 0x0f0f0f0fu;
    const uint4 x0 = *reinterpret_cast<const uint4 *>(xc);
    const uint4 x1 = *reinterpret_cast<const uint4 *>(xc + 16);
    acc = sdot4((int)(w.x & M), (int)x0.x, acc);
    acc = sdot4((int)((w.x >> 4) & M), (int)x0.y, acc);
    acc = sdot4((int)(w.y & M), (int)x0.z, acc);
    acc = sdot4((int)((w.y >> 4) & M), (int)x0.w, acc);
    acc = sdot4((int)(w.z & M), (int)x1.x, acc);
    acc = sdot4((int)((w.z >> 4) & M), (int)x1.y, acc);
    acc = sdot4((int)(w.w & M), (int)x1.z, acc);
    return sdot4((int)((w.w >> 4) & M), (int)x1.w, acc);
  } else {
    constexpr uint32_t M = 0x03030303u;
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 x = *reinterpret_cast<const uint4 *>(xc + 16 * m);
      acc = sdot4((int)(wd[m] & M), (int)x.x, acc);
      acc = sdot4((int)((wd[m] >> 2) & M), (int)x.y, acc);
      acc = sdot4((int)((wd[m] >> 4) & M), (int)x.z, acc);
      acc = sdot4((int)((wd[m] >> 6) & M), (int)x.w, acc);
    }
    return acc;
  }
}

// Stage nt rows of int8 activations (row length n, rows given by src_row(tt))
// into LDS in field order and accumulate their byte sums.
template <int BITS, typename RowPtr>
__device__ __forceinline__ void stage_rows(int8_t *xs, int *xsum, int nt, int n, RowPtr src_row) {
  const int upr = n / 16;
  for (int u = threadIdx.x; u < nt * upr; u += kThreads) {
    const int tt = u / upr;
    const int c16 = u - tt * upr;
    const uint4 v = *reinterpret_cast<const uint4 *>(src_row(tt) + c16 * 16);
    *reinterpret_cast<uint4 *>(xs + tt * n + c16 * 16) = act_order16<BITS>(v);
    atomicAdd(&xsum[tt], bytesum16(v));
  }
}

__device__ __forceinline__ const uint4 *chunk_ptr(const uint8_t *base, int64_t row, int rowbytes, int c) {
  return reinterpret_cast<const uint4 *>(base + row * (int64_t)rowbytes) + c;
}

// ---------------------------------------------------------------------------
// gate + up, SwiGLU epilogue
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(kThreads) void ffn_gateup_kernel(FfnArgs a) {
  constexpr int J = Shape<BITS>::kJ, RW = Shape<BITS>::kRwGU;
  constexpr int EPC = QFmt<BITS>::kEpc, OFF = QFmt<BITS>::kOff;
  __shared__ __align__(16) int8_t xs[kTG * kMaxDim];
  __shared__ int xsum[kTG];
  __shared__ int toks[kTG], slots[kTG];
  __shared__ unsigned tmax[kTG];

  const int d = blockIdx.x / a.tiles1;
  const int tile = blockIdx.x - d * a.tiles1;
  ExpertRef ex;
  if (!resolve(a, d, ex)) return;
  const int tid = threadIdx.x, lane = tid & (MOE_WAVE - 1), wave = tid >> 6;
  const int rowbytes = a.H * BITS / 8;
  const int cpr = rowbytes / 16;
  const int i0 = tile * (kWaves * RW) + wave * RW;

  for (int g0 = 0; g0 < ex.ntok; g0 += kTG) {
    const int nt = min(kTG, ex.ntok - g0);
    __syncthreads();
    if (tid < kTG) {
      xsum[tid] = 0;
      tmax[tid] = 0u;
      if (tid < nt) {
        int t, s;
        token_of(a, ex, g0 + tid, t, s);
        toks[tid] = t;
        slots[tid] = s;
      }
    }
    __syncthreads();
    stage_rows<BITS>(xs, xsum, nt, a.H, [&](int tt) { return a.xq + (int64_t)toks[tt] * a.H; });

    uint4 wg[RW][J], wu[RW][J];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = lane + j * MOE_WAVE;
        if (c < cpr) {
          wg[r][j] = *chunk_ptr(ex.w.gate, i0 + r, rowbytes, c);
          wu[r][j] = *chunk_ptr(ex.w.up, i0 + r, rowbytes, c);
        } else {
          wg[r][j] = make_uint4(0, 0, 0, 0);
          wu[r][j] = make_uint4(0, 0, 0, 0);
        }
      }
    __syncthreads();  // staged activations visible

    int accg[RW][kTG], accu[RW][kTG];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int tt = 0; tt < kTG; ++tt) accg[r][tt] = accu[r][tt] = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + j * MOE_WAVE;
      if (c < cpr) {
#pragma unroll
        for (int tt = 0; tt < kTG; ++tt) {
          if (tt < nt) {
            const int8_t *xc = xs + tt * a.H + c * EPC;
#pragma unroll
            for (int r = 0; r < RW; ++r) {
              accg[r][tt] = dot_chunk<BITS>(wg[r][j], xc, accg[r][tt]);
              accu[r][tt] = dot_chunk<BITS>(wu[r][j], xc, accu[r][tt]);
            }
          }
        }
      }
    }
    int my_g = 0, my_u = 0;
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int tt = 0; tt < kTG; ++tt) {
        if (tt < nt) {
          const int sg = wave_sum_i32(accg[r][tt]);
          const int su = wave_sum_i32(accu[r][tt]);
          if (lane == r * kTG + tt) {
            my_g = sg;
            my_u = su;
          }
        }
      }
    const int r = lane / kTG, tt = lane - (lane / kTG) * kTG;
    if (lane < RW * kTG && tt < nt) {
      const int i = i0 + r;
      const int t = toks[tt], slot = slots[tt];
      const int64_t p = (int64_t)t * (a.k + 1) + slot;
      const int gi = my_g - OFF * xsum[tt];
      const int ui = my_u - OFF * xsum[tt];
      const float g = (float)gi * ex.w.s_gate[i] * a.sx[t];
      const float u = (float)ui * ex.w.s_up[i] * a.sx[t];
      const float av = moe_silu_f32(g) * u;
      a.A[p * a.I + i] = av;
      if (a.dbg_on) {
        if (a.dbg.accg) a.dbg.accg[p * a.I + i] = gi;
        if (a.dbg.accu) a.dbg.accu[p * a.I + i] = ui;
        if (a.dbg.a) a.dbg.a[p * a.I + i] = av;
      }
      atomicMax(&tmax[tt], __float_as_uint(fabsf(av)));
    }
    __syncthreads();
    if (tid < nt) {
      const int64_t p = (int64_t)toks[tid] * (a.k + 1) + slots[tid];
      a.tilemax[p * a.tiles1 + tile] = __uint_as_float(tmax[tid]);
    }
  }
}

// ---------------------------------------------------------------------------
// requantisation of a: one workgroup per (token, slot) pair
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void ffn_requant_kernel(FfnArgs a) {
  const int64_t p = blockIdx.x;
  const int t = (int)(p / (a.k + 1));
  const int slot = (int)(p - (int64_t)t * (a.k + 1));
  if (slot < a.k) {
    const int e = a.topk_idx[(int64_t)t * a.k + slot];
    if (e < 0 || e >= a.E) return;
    if (a.expert_bits && a.expert_bits[e] != a.bits) return;
    for (int j = 0; j < slot; ++j)  // a repeated expert is computed for its first slot only
      if (a.topk_idx[(int64_t)t * a.k + j] == e) return;
  } else if (!a.has_shared) {
    return;
  }
  __shared__ float red[kWaves];
  float m = 0.0f;
  for (int i = threadIdx.x; i < a.tiles1; i += kThreads) m = fmaxf(m, a.tilemax[p * a.tiles1 + i]);
  m = wave_max_f32(m);
  if ((threadIdx.x & (MOE_WAVE - 1)) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = (m == 0.0f) ? 0.0f : m / 127.0f;
  for (int i = threadIdx.x; i < a.I; i += kThreads) {
    int q = 0;
    if (m != 0.0f) {
      float rr = __builtin_rintf(a.A[p * a.I + i] / s);
      rr = fminf(fmaxf(rr, -127.0f), 127.0f);
      q = (int)rr;
    }
    a.aq[p * a.I + i] = (int8_t)q;
    if (a.dbg_on && a.dbg.aq) a.dbg.aq[p * a.I + i] = (int8_t)q;
  }
  if (threadIdx.x == 0) {
    a.sa[p] = s;
    if (a.dbg_on && a.dbg.sa) a.dbg.sa[p] = s;
  }
}

// ---------------------------------------------------------------------------
// down projection
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(kThreads) void ffn_down_kernel(FfnArgs a) {
  constexpr int J = Shape<BITS>::kJ, RW = Shape<BITS>::kRwD;
  constexpr int EPC = QFmt<BITS>::kEpc, OFF = QFmt<BITS>::kOff;
  __shared__ __align__(16) int8_t xs[kTG * kMaxDim];
  __shared__ int xsum[kTG];
  __shared__ int toks[kTG], slots[kTG];
  __shared__ float sas[kTG];

  const int d = blockIdx.x / a.tiles2;
  const int tile = blockIdx.x - d * a.tiles2;
  ExpertRef ex;
  if (!resolve(a, d, ex)) return;
  const int tid = threadIdx.x, lane = tid & (MOE_WAVE - 1), wave = tid >> 6;
  const int rowbytes = a.I * BITS / 8;
  const int cpr = rowbytes / 16;
  const int r0 = tile * (kWaves * RW) + wave * RW;

  for (int g0 = 0; g0 < ex.ntok; g0 += kTG) {
    const int nt = min(kTG, ex.ntok - g0);
    __syncthreads();
    if (tid < kTG) {
      xsum[tid] = 0;
      if (tid < nt) {
        int t, s;
        token_of(a, ex, g0 + tid, t, s);
        toks[tid] = t;
        slots[tid] = s;
        sas[tid] = a.sa[(int64_t)t * (a.k + 1) + s];
      }
    }
    __syncthreads();
    stage_rows<BITS>(xs, xsum, nt, a.I,
                     [&](int tt) { return a.aq + ((int64_t)toks[tt] * (a.k + 1) + slots[tt]) * a.I; });

    uint4 wd[RW][J];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = lane + j * MOE_WAVE;
        wd[r][j] = (c < cpr) ? *chunk_ptr(ex.w.down, r0 + r, rowbytes, c) : make_uint4(0, 0, 0, 0);
      }
    __syncthreads();

    int acc[RW][kTG];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int tt = 0; tt < kTG; ++tt) acc[r][tt] = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + j * MOE_WAVE;
      if (c < cpr) {
#pragma unroll
        for (int tt = 0; tt < kTG; ++tt) {
          if (tt < nt) {
            const int8_t *xc = xs + tt * a.I + c * EPC;
#pragma unroll
            for (int r = 0; r < RW; ++r) acc[r][tt] = dot_chunk<BITS>(wd[r][j], xc, acc[r][tt]);
          }
        }
      }
    }
    int mine = 0;
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int tt = 0; tt < kTG; ++tt) {
        if (tt < nt) {
          const int s = wave_sum_i32(acc[r][tt]);
          if (lane == r * kTG + tt) mine = s;
        }
      }
    const int r = lane / kTG, tt = lane - (lane / kTG) * kTG;
    if (lane < RW * kTG && tt < nt) {
      const int row = r0 + r;
      const int t = toks[tt], slot = slots[tt];
      const int64_t p = (int64_t)t * (a.k + 1) + slot;
      const int di = mine - OFF * xsum[tt];
      a.y[p * a.H + row] = (float)di * ex.w.s_down[row] * sas[tt];
      if (a.dbg_on && a.dbg.accd) a.dbg.accd[p * a.H + row] = di;
    }
  }
}

template <int BITS>
moe_status launch_ffn_bits(moe_ctx *ctx, FfnArgs &a, int dmax) {
  {
    MoeTimer tm_(ctx, MOE_STAGE_GATEUP);
    hipLaunchKernelGGL(ffn_gateup_kernel<BITS>, dim3(dmax * a.tiles1), dim3(kThreads), 0, ctx->stream, a);
  }
  MOE_CHECK_LAUNCH("ffn_gateup_kernel");
  {
    MoeTimer tm_(ctx, MOE_STAGE_REQUANT);
    hipLaunchKernelGGL(ffn_requant_kernel, dim3(a.T * (a.k + 1)), dim3(kThreads), 0, ctx->stream, a);
  }
  MOE_CHECK_LAUNCH("ffn_requant_kernel");
  {
    MoeTimer tm_(ctx, MOE_STAGE_DOWN);
    hipLaunchKernelGGL(ffn_down_kernel<BITS>, dim3(dmax * a.tiles2), dim3(kThreads), 0, ctx->stream, a);
  }
  MOE_CHECK_LAUNCH("ffn_down_kernel");
  return MOE_OK;
}

int rows_per_wg_gu(int bits) { return kWaves * (bits == 8 ? Shape<8>::kRwGU : bits == 4 ? Shape<4>::kRwGU : Shape<2>::kRwGU); }
int rows_per_wg_d(int bits) { return kWaves * (bits == 8 ? Shape<8>::kRwD : bits == 4 ? Shape<4>::kRwD : Shape<2>::kRwD); }


// Which kernel family computes a call's expert FFN. MOE_FFN_AUTO follows
// the measured crossover at the GLM shape (int4, hidden 6144, intermediate
// 2048, top-8 + shared): up to kT1MaxTokens tokens the single-token kernels
// run once per token (2 tokens: 78 us against 101 for the vector kernels
// and 110 for the matrix cores; 3 tokens: 116 against 135 and 135); from 4
// tokens on the matrix cores win (4: 156 against 156 and 163 with
// hidden-state routing, 148 against 155 and 156 with Zipf routing; 8: 221
// against 310 and 277), their per-expert tiles reading each expert once for
// all its tokens.
constexpr int kT1MaxTokens = 3;
enum FfnRoute { kRouteMfma, kRouteT1, kRouteDot4, kRouteUnsupported };
FfnRoute ffn_route(const moe_ctx *ctx, int bits, int has_shared, int T, int H, int I, int k) {
  const bool mfma_ok = expert_ffn_mfma_supported(bits, H, I);
  if (ctx->ffn_kernels == MOE_FFN_MFMA && !mfma_ok) return kRouteUnsupported;
  if (ctx->ffn_kernels == MOE_FFN_AUTO && T <= kT1MaxTokens &&
      decode_t1_supported(bits, H, I, k, has_shared, ctx->n_cu))
    return kRouteT1;
  if (mfma_ok && (ctx->ffn_kernels == MOE_FFN_MFMA || (ctx->ffn_kernels == MOE_FFN_AUTO && T >= 2))) return kRouteMfma;
  return kRouteDot4;
}

// Scratch layout of the vector FFN.
struct Dot4Layout {
  int tiles1, tiles2;
  size_t o_counts, o_offsets, o_perm, o_active, o_nact, o_tmax, o_A, o_aq, o_sa, size;
};
Dot4Layout dot4_layout(int bits, int T, int H, int I, int E, int k) {
  Dot4Layout l;
  const int64_t P = (int64_t)T * (k + 1);
  l.tiles1 = I / rows_per_wg_gu(bits);
  l.tiles2 = H / rows_per_wg_d(bits);
  MoeLayout m;
  l.o_counts = m.take(4 * (size_t)E);
  l.o_offsets = m.take(4 * (size_t)(E + 1));
  l.o_perm = m.take(4 * (size_t)T * k);
  l.o_active = m.take(4 * (size_t)E);
  l.o_nact = m.take(4);
  l.o_tmax = m.take(4 * (size_t)P * l.tiles1);
  l.o_A = m.take(4 * (size_t)P * I);
  l.o_aq = m.take((size_t)P * I);
  l.o_sa = m.take(4 * (size_t)P);
  l.size = m.size;
  return l;
}

}  // namespace

size_t expert_ffn_scratch_bytes(const moe_ctx *ctx, int bits, int has_shared, int T, int H, int I, int E, int k) {
  switch (ffn_route(ctx, bits, has_shared, T, H, I, k)) {
    case kRouteMfma: return expert_ffn_mfma_scratch_bytes(bits, has_shared, T, H, I, E, k);
    case kRouteT1: return ffn_t1_scratch_bytes(I, k + has_shared);
    case kRouteDot4: return dot4_layout(bits, T, H, I, E, k).size;
    default: return 0;
  }
}

moe_status launch_expert_ffn(moe_ctx *ctx, int bits, const moe_expert_w *experts, const moe_expert_w *shared,
                             const uint8_t *expert_bits, const int8_t *xq, const float *sx, const int32_t *topk_idx,
                             int T, int H, int I, int E, int k, float *y_slots) {
  switch (ffn_route(ctx, bits, shared ? 1 : 0, T, H, I, k)) {
    case kRouteUnsupported:
      return moe_fail(MOE_EUNSUPPORTED, "expert FFN: the matrix-core kernels do not take H %d, I %d at %d bits", H, I,
                      bits);
    case kRouteMfma:
      return launch_expert_ffn_mfma(ctx, bits, experts, shared, expert_bits, xq, sx, topk_idx, T, H, I, E, k,
                                    y_slots);
    case kRouteT1: {
      // one single-token chain per token, in token order on the stream (the
      // chains share the scratch; each starts after the previous has ended).
      // Captured intermediates go to each token's rows.
      const moe_debug_bufs dbg = ctx->dbg;
      moe_status st = MOE_OK;
      for (int t = 0; t < T && st == MOE_OK; ++t) {
        if (ctx->dbg_on) {
          const int64_t p0 = (int64_t)t * (k + 1);
          ctx->dbg.accg = dbg.accg ? dbg.accg + p0 * I : nullptr;
          ctx->dbg.accu = dbg.accu ? dbg.accu + p0 * I : nullptr;
          ctx->dbg.a = dbg.a ? dbg.a + p0 * I : nullptr;
          ctx->dbg.aq = dbg.aq ? dbg.aq + p0 * I : nullptr;
          ctx->dbg.sa = dbg.sa ? dbg.sa + p0 : nullptr;
          ctx->dbg.accd = dbg.accd ? dbg.accd + p0 * H : nullptr;
        }
        st = launch_ffn_t1(ctx, bits, experts, shared, expert_bits, xq + (int64_t)t * H, sx + t,
                           topk_idx + (int64_t)t * k, H, I, E, k, y_slots + (int64_t)t * (k + 1) * H);
      }
      ctx->dbg = dbg;
      return st;
    }
    default:
      break;
  }
  const Dot4Layout l = dot4_layout(bits, T, H, I, E, k);
  FfnArgs a{};
  a.tiles1 = l.tiles1;
  a.tiles2 = l.tiles2;
  const size_t o_counts = l.o_counts, o_offsets = l.o_offsets, o_perm = l.o_perm, o_active = l.o_active,
               o_nact = l.o_nact, o_tmax = l.o_tmax, o_A = l.o_A, o_aq = l.o_aq, o_sa = l.o_sa;
  void *scr = nullptr;
  moe_status st = moe_scratch(ctx, l.size, &scr);
  if (st) return st;
  char *base = static_cast<char *>(scr);
  a.experts = experts;
  a.has_shared = shared ? 1 : 0;
  if (shared) a.shared = *shared;
  a.xq = xq;
  a.sx = sx;
  a.topk_idx = topk_idx;
  a.expert_bits = expert_bits;
  a.bits = bits;
  a.T = T; a.H = H; a.I = I; a.E = E; a.k = k;
  a.counts = reinterpret_cast<int32_t *>(base + o_counts);
  a.offsets = reinterpret_cast<int32_t *>(base + o_offsets);
  a.perm = reinterpret_cast<int32_t *>(base + o_perm);
  a.active = reinterpret_cast<int32_t *>(base + o_active);
  a.n_active = reinterpret_cast<int32_t *>(base + o_nact);
  a.tilemax = reinterpret_cast<float *>(base + o_tmax);
  a.A = reinterpret_cast<float *>(base + o_A);
  a.aq = reinterpret_cast<int8_t *>(base + o_aq);
  a.sa = reinterpret_cast<float *>(base + o_sa);
  a.y = y_slots;
  a.dbg = ctx->dbg;
  a.dbg_on = ctx->dbg_on ? 1 : 0;
  st = launch_bucket(ctx, topk_idx, T, k, E, const_cast<int32_t *>(a.counts), const_cast<int32_t *>(a.offsets),
                     const_cast<int32_t *>(a.perm), expert_bits, bits, const_cast<int32_t *>(a.active),
                     const_cast<int32_t *>(a.n_active), nullptr, nullptr, 0, 0, kUnitSmall);
  if (st) return st;
  const int dmax = (int)std::min<int64_t>(E, (int64_t)T * k) + a.has_shared;
  switch (bits) {
    case 8: return launch_ffn_bits<8>(ctx, a, dmax);
    case 4: return launch_ffn_bits<4>(ctx, a, dmax);
    default: return launch_ffn_bits<2>(ctx, a, dmax);
  }
}
