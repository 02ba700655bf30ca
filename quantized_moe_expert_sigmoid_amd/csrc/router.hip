// Sigmoid top-k router with a selection bias, and per-expert bucketing.
//
// tech.takumi3488.com, "Trying colibri": a DeepSeek-V3-family router
// (self-test section); 256 experts per layer, top-8 (section on the real
// 744B model). remio.ai, "How Colibri runs GLM-5.2": the router picks a few
// experts per token; "The RAM wall became a storage problem": requests for
// one expert from several batch positions are served by one read, which is
// what the per-expert buckets give the FFN.
//
// Logits are fp32 dot products, split over K into fixed slices whose partial
// sums are added in slice order (deterministic). Top-k runs one wave per
// token: sigmoid via the library's fp32 exp, key = sigmoid + bias, k rounds
// of a wave-wide (key desc, id asc) arg-max, weights = sigmoid / sum.
#include <algorithm>

#include "gemv_common.h"

namespace {

constexpr int kSmallT = 8;      // GEMV path up to this many tokens
constexpr int kTile = 64;       // GEMM tile (tokens x experts)
constexpr int kTileK = 16;      // GEMM K step through LDS

// --- logits, T <= kSmallT: one wave per (expert, K slice), all tokens -------
__global__ __launch_bounds__(256) void router_gemv_kernel(const float *__restrict__ x, const float *__restrict__ wr,
                                                          int T, int H, int E, int kl,
                                                          float *__restrict__ partial) {
  const int lane = threadIdx.x & (MOE_WAVE - 1);
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int ks = blockIdx.y;
  if (e >= E) return;
  const int k0 = ks * kl;
  const float *wrow = wr + (int64_t)e * H + k0;
  float acc[kSmallT];
#pragma unroll
  for (int t = 0; t < kSmallT; ++t) acc[t] = 0.0f;
  for (int c = lane * 4; c < kl; c += MOE_WAVE * 4) {
    const float4 wv = *reinterpret_cast<const float4 *>(wrow + c);
#pragma unroll
    for (int t = 0; t < kSmallT; ++t) {
      if (t < T) {
        const float4 xv = *reinterpret_cast<const float4 *>(x + (int64_t)t * H + k0 + c);
        acc[t] = __builtin_fmaf(wv.x, xv.x, acc[t]);
        acc[t] = __builtin_fmaf(wv.y, xv.y, acc[t]);
        acc[t] = __builtin_fmaf(wv.z, xv.z, acc[t]);
        acc[t] = __builtin_fmaf(wv.w, xv.w, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kSmallT; ++t) {
    if (t < T) {
      const float s = wave_sum_f32(acc[t]);
      if (lane == 0) partial[((int64_t)ks * T + t) * E + e] = s;
    }
  }
}

// --- logits, general T: 64x64 register-tiled GEMM over one K slice ----------
__global__ __launch_bounds__(256) void router_gemm_kernel(const float *__restrict__ x, const float *__restrict__ wr,
                                                          int T, int H, int E, int kl,
                                                          float *__restrict__ partial) {
  __shared__ float xs[kTileK][kTile + 4];
  __shared__ float ws[kTileK][kTile + 4];
  const int t0 = blockIdx.x * kTile;
  const int e0 = blockIdx.y * kTile;
  const int ks = blockIdx.z;
  const int k0 = ks * kl;
  const int tx = threadIdx.x & 15;  // expert sub-tile
  const int ty = threadIdx.x >> 4;  // token sub-tile
  float acc[4][4] = {};
  for (int kk = 0; kk < kl; kk += kTileK) {
    // each thread loads 4 floats of x and 4 of w: 64 rows x 16 k each
    const int r = threadIdx.x >> 2, c4 = (threadIdx.x & 3) * 4;
    {
      const int t = t0 + r;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < T) v = *reinterpret_cast<const float4 *>(x + (int64_t)t * H + k0 + kk + c4);
      xs[c4 + 0][r] = v.x; xs[c4 + 1][r] = v.y; xs[c4 + 2][r] = v.z; xs[c4 + 3][r] = v.w;
      const int e = e0 + r;
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < E) u = *reinterpret_cast<const float4 *>(wr + (int64_t)e * H + k0 + kk + c4);
      ws[c4 + 0][r] = u.x; ws[c4 + 1][r] = u.y; ws[c4 + 2][r] = u.z; ws[c4 + 3][r] = u.w;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kTileK; ++q) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[q][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[q][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) partial[((int64_t)ks * T + t) * E + e] = acc[i][j];
    }
  }
}

// --- logits, general T, on the fp32 matrix cores ----------------------------
// The same 64x64 tile as router_gemm_kernel; each wave owns a 32 x 32
// quarter as 2 x 2 blocks of v_mfma_f32_16x16x4f32 (lane l holds one x and
// one w value of token / expert l % 16 per product, at K position l / 16 of
// its step, and the results of tokens 4 (l / 16) .. +3 of expert l % 16).
// K steps of kMfmaK floats go through LDS row-major (a token's or expert's
// floats contiguous, rows padded by one 16-byte unit so the 16 rows a read
// spans hit distinct banks). Per 16 floats of K a lane reads one 16-byte
// unit of each of its rows, unit l / 16, and feeds its four floats to four
// consecutive products: product s of the 16 takes K positions 4q + s
// (q = 0..3, one per lane group), so the four products cover all 16 and x
// and w agree on every position. kl % kMfmaK == 0.
constexpr int kMfmaK = 32;
constexpr int kMfmaU = kMfmaK / 4 + 1;  // 16-byte units per LDS row (one of padding)
typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void router_gemm_mfma_kernel(const float *__restrict__ x,
                                                               const float *__restrict__ wr, int T, int H, int E,
                                                               int kl, float *__restrict__ partial) {
  __shared__ float4 xs[kTile][kMfmaU];
  __shared__ float4 ws[kTile][kMfmaU];
  const int t0 = blockIdx.x * kTile;
  const int e0 = blockIdx.y * kTile;
  const int ks = blockIdx.z;
  const int k0 = ks * kl;
  const int tid = threadIdx.x, lane = tid & (MOE_WAVE - 1), wave = tid >> 6;
  const int wt = (wave >> 1) * 32, we = (wave & 1) * 32;  // the wave's quarter of the tile
  const int l16 = lane & 15, kq = lane >> 4;
  // staging: thread tid moves 8 consecutive floats (units c2, c2 + 1) of row tid / 4 (x and w)
  const int r = tid >> 2, c2 = (tid & 3) * 2;
  const int t = t0 + r, e = e0 + r;
  const float *xrow = x + (int64_t)min(t, T - 1) * H + k0 + 4 * c2;
  const float *wrow = wr + (int64_t)min(e, E - 1) * H + k0 + 4 * c2;
  v4f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  float4 xa, xb, wa, wb;
  auto load = [&](int kk) {  // rows past T or E read a valid row; their products are never stored
    xa = *reinterpret_cast<const float4 *>(xrow + kk);
    xb = *reinterpret_cast<const float4 *>(xrow + kk + 4);
    wa = *reinterpret_cast<const float4 *>(wrow + kk);
    wb = *reinterpret_cast<const float4 *>(wrow + kk + 4);
  };
  load(0);
  for (int kk = 0; kk < kl; kk += kMfmaK) {
    __syncthreads();  // the previous step's reads are done
    xs[r][c2] = xa;
    xs[r][c2 + 1] = xb;
    ws[r][c2] = wa;
    ws[r][c2 + 1] = wb;
    __syncthreads();
    if (kk + kMfmaK < kl) load(kk + kMfmaK);  // the next step's loads fly under this step's products
#pragma unroll
    for (int k16 = 0; k16 < kMfmaK / 16; ++k16) {
      const int u = 4 * k16 + kq;
      const float4 a0 = xs[wt + l16][u], a1 = xs[wt + 16 + l16][u];
      const float4 b0 = ws[we + l16][u], b1 = ws[we + 16 + l16][u];
      const float av[2][4] = {{a0.x, a0.y, a0.z, a0.w}, {a1.x, a1.y, a1.z, a1.w}};
      const float bv[2][4] = {{b0.x, b0.y, b0.z, b0.w}, {b1.x, b1.y, b1.z, b1.w}};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i][q], bv[j][q], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ee = e0 + we + j * 16 + l16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int tt = t0 + wt + i * 16 + 4 * kq + q;
        if (tt < T && ee < E) partial[((int64_t)ks * T + tt) * E + ee] = acc[i][j][q];
      }
    }
}

// --- top-k: one wave per token ---------------------------------------------
// Each lane sums its experts' logit slices in slice order, forms sigmoid and
// key (a NaN key ranks last, -0 becomes +0) into the wave's LDS rows; the
// wave then selects the k best (descending key, ties to the lower id) with
// the DPP selection of the single-token path, and the weights are
// routed_scale * sigmoid / (sum of the selected sigmoids, in rank order).
// With top_p > 0 only the prefix topp_keep returns is kept (renormalised);
// the other slots get id -1 and weight 0.
constexpr int kTopkWaves = 4;

template <int NSL>  // logit slices
__global__ __launch_bounds__(kTopkWaves * MOE_WAVE) void router_topk_kernel(
    const float *__restrict__ partial, int T, int E, int k, const float *__restrict__ bias,
    float routed_scale, float top_p, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w) {
  __shared__ float key_s[kTopkWaves][1024], sig_s[kTopkWaves][1024];
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kTopkWaves + wave;
  if (t >= T) return;  // whole waves; no workgroup barrier below
  for (int e0 = 0; e0 < E; e0 += MOE_WAVE) {
    const int e = min(e0 + lane, E - 1);
    float zs[NSL];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) zs[sl] = partial[((int64_t)sl * T + t) * E + e];  // all issued, then summed
    float z = zs[0];
#pragma unroll
    for (int sl = 1; sl < NSL; ++sl) z += zs[sl];
    const float sg = 1.0f / (1.0f + moe_exp_f32(-z));
    float key = sg + (bias ? bias[e] : 0.0f);
    if (key != key) key = -__builtin_inff();
    if (e0 + lane < E) {
      key_s[wave][e] = key + 0.0f;
      sig_s[wave][e] = sg;
    }
  }
  const int my_id = E <= 4 * MOE_WAVE ? wave_topk4(key_s[wave], E, k, lane) : wave_topk16(key_s[wave], E, k, lane);
  const float my_sig = lane < k ? sig_s[wave][my_id] : 0.0f;
  float sum = 0.0f;  // in rank order
  for (int j = 0; j < k; ++j) sum += readlane_f(my_sig, j);
  float kept = sum;
  const int keep = top_p > 0.0f ? topp_keep(my_sig, sum, k, top_p, kept) : k;
  if (lane < k) {
    topk_idx[(int64_t)t * k + lane] = lane < keep ? my_id : -1;
    topk_w[(int64_t)t * k + lane] = lane < keep ? routed_scale * (my_sig / kept) : 0.0f;
  }
}

// --- bucketing: one workgroup, stable per-expert lists ----------------------
constexpr int kBThreads = 1024;
constexpr int kBitmapWords = 8192;

struct BucketArgs {
  const int32_t *idx;
  int T, k, E;
  int32_t *counts, *offsets, *perm;
  const uint8_t *expert_bits;  // nullable filter for the active list
  int want_bits;
  int32_t *active;    // nullable: experts with count > 0 passing the filter
  int32_t *n_active;  // nullable
  uint32_t *err;
  // nullable: token tiles of the active experts (and of the shared expert,
  // active position n_active, when has_shared) for the matrix-core FFN:
  // units[0 .. n_units[0]) are (active position, first token) of tiles of up
  // to kUnitM tokens holding more than small_max of them; units[ubig_max +
  // 0 .. n_units[1]) the remainders of 1..small_max tokens (small_max 0: none)
  int2 *units;
  int32_t *n_units;
  int ubig_max, has_shared;
  int small_max;
};

// Exclusive prefix sum over the workgroup's threads (in thread order): an
// inclusive scan inside each wave (shuffles), the wave totals scanned by
// wave 0 through LDS, two barriers. tmp holds at least one int per wave.
__device__ int block_exclusive_scan(int v, int *tmp) {
  constexpr int kW = kBThreads / MOE_WAVE;
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < MOE_WAVE; o <<= 1) {
    const int u = __shfl_up(incl, o, MOE_WAVE);
    if (lane >= o) incl += u;
  }
  if (lane == MOE_WAVE - 1) tmp[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kW ? tmp[lane] : 0;
#pragma unroll
    for (int o = 1; o < kW; o <<= 1) {
      const int u = __shfl_up(w, o, MOE_WAVE);
      if (lane >= o) w += u;
    }
    if (lane < kW) tmp[kW + lane] = w - (lane < kW ? tmp[lane] : 0);  // exclusive wave offsets
  }
  __syncthreads();
  const int r = tmp[kW + wave] + incl - v;
  __syncthreads();  // tmp is reused by the next scan
  return r;
}

// ids of token t with repeats dropped (a repeated id counts once, at its
// first slot) and -1 (a slot dropped by top-p) skipped; returns false when an
// id is otherwise out of range or repeated
__device__ __forceinline__ bool token_ids(const BucketArgs &a, int64_t t, int ids[16]) {
  bool ok = true;
  for (int j = 0; j < a.k; ++j) ids[j] = a.idx[t * a.k + j];
  for (int j = 0; j < a.k; ++j) {
    if (ids[j] == -1) continue;
    bool dup = false;
    for (int i = 0; i < j; ++i) dup |= ids[i] == ids[j];
    if (ids[j] < 0 || ids[j] >= a.E || dup) {
      ok = false;
      ids[j] = -1;
    }
  }
  return ok;
}

// Per-expert metadata from the counts, thread tid for expert tid < E (c: its
// count, eb: its width): counts and offsets (also into off[0 .. E] in LDS),
// the active list and the tiles of the matrix-core FFN. Every thread of the
// workgroup takes part (block-wide scans).
__device__ void bucket_meta(const BucketArgs &a, int c, int eb, int *tmp, int *off) {
  const int tid = threadIdx.x;
  const int E = a.E, T = a.T;
  const int ex = block_exclusive_scan(c, tmp);
  if (tid < E) {
    off[tid] = ex;
    a.counts[tid] = c;
    a.offsets[tid] = ex;
  }
  if (tid == E - 1) {
    off[E] = ex + c;
    a.offsets[E] = ex + c;
  }
  const int act = (tid < E && c > 0 && (!a.expert_bits || eb == a.want_bits)) ? 1 : 0;
  const int apos = block_exclusive_scan(act, tmp);
  if (a.active && act) a.active[apos] = tid;
  if (a.n_active && tid == E - 1) *a.n_active = apos + act;
  __syncthreads();
  if (a.units) {
    const int rem = c % kUnitM;
    const int nb = act ? c / kUnitM + (rem > a.small_max ? 1 : 0) : 0;
    const int ns = (act && rem > 0 && rem <= a.small_max) ? 1 : 0;
    const int bb = block_exclusive_scan(nb, tmp);
    const int sb = block_exclusive_scan(ns, tmp);
    for (int j = 0; j < nb; ++j) a.units[bb + j] = make_int2(apos, j * kUnitM);
    if (ns) a.units[a.ubig_max + sb] = make_int2(apos, (c / kUnitM) * kUnitM);
    __shared__ int tot[3];
    if (tid == kBThreads - 1) {
      tot[0] = bb + nb;
      tot[1] = sb + ns;
      tot[2] = apos + act;  // threads past E add nothing: the active count
    }
    __syncthreads();
    int nbig = tot[0], nsmall = tot[1];
    if (a.has_shared) {  // the shared expert takes every token
      const int sr = T % kUnitM;
      const int snb = T / kUnitM + (sr > a.small_max ? 1 : 0);
      for (int j = tid; j < snb; j += kBThreads) a.units[nbig + j] = make_int2(tot[2], j * kUnitM);
      if (tid == 0 && sr > 0 && sr <= a.small_max) a.units[a.ubig_max + nsmall] = make_int2(tot[2], (T / kUnitM) * kUnitM);
      nbig += snb;
      nsmall += (sr > 0 && sr <= a.small_max) ? 1 : 0;
    }
    if (tid == 0) {
      a.n_units[0] = nbig;
      a.n_units[1] = nsmall;
    }
  }
}

constexpr int kIdsCache = 4096;  // (token, slot) ids kept in LDS after the first read

__global__ __launch_bounds__(kBThreads) void bucket_kernel(BucketArgs a) {
  __shared__ int ids_s[kIdsCache];
  __shared__ int cnt[1024];
  __shared__ int off[1025];
  __shared__ int cursor[1024];
  __shared__ int tmp[kBThreads];
  __shared__ uint32_t bitmap[kBitmapWords];
  __shared__ int before[kBitmapWords];  // entries of the expert in earlier words of the chunk
  const int tid = threadIdx.x;
  const int E = a.E, k = a.k, T = a.T;
  // the width filter is read now, so its latency overlaps the counting
  const int eb = (a.expert_bits && tid < E) ? a.expert_bits[tid] : 0;
  // small calls keep the validated ids in LDS for the later passes
  const bool cached = (int64_t)T * k <= kIdsCache;
  auto ids_of = [&](int t, int (&ids)[16]) {
    if (cached) {
      for (int j = 0; j < k; ++j) ids[j] = ids_s[t * k + j];
    } else {
      token_ids(a, t, ids);
    }
  };

  for (int e = tid; e < 1024; e += kBThreads) {
    cnt[e] = 0;
    cursor[e] = 0;
  }
  __syncthreads();
  bool bad = false;
  for (int t = tid; t < T; t += kBThreads) {
    int ids[16];
    bad |= !token_ids(a, t, ids);
    for (int j = 0; j < k; ++j) {
      if (ids[j] >= 0) atomicAdd(&cnt[ids[j]], 1);
      if (cached) ids_s[t * k + j] = ids[j];
    }
  }
  if (bad) atomicOr(a.err, (uint32_t)ERRF_BAD_INDEX);
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  bucket_meta(a, c, eb, tmp, off);
  if (T == 0) return;

  // stable placement, tokens in chunks of 32 W (one bit per token and expert
  // in LDS): an entry's rank in its expert's list is the expert's count from
  // earlier chunks, plus its set bits in earlier words, plus those below it
  int W = kBitmapWords / E;  // words per expert: as many as the LDS holds, at most 64,
  if (W > 64) W = 64;
  if (W > (T + 31) / 32) W = (T + 31) / 32;  // and no more than the tokens need
  const int TC = 32 * W;
  for (int c0 = 0; c0 < T; c0 += TC) {
    const int nt = min(TC, T - c0);
    for (int i = tid; i < E * W; i += kBThreads) bitmap[i] = 0u;
    __syncthreads();
    for (int tl = tid; tl < nt; tl += kBThreads) {
      int ids[16];
      ids_of(c0 + tl, ids);
      for (int j = 0; j < k; ++j)
        if (ids[j] >= 0) atomicOr(&bitmap[ids[j] * W + (tl >> 5)], 1u << (tl & 31));
    }
    __syncthreads();
    for (int e = tid; e < E; e += kBThreads) {
      int run = cursor[e];
      for (int w = 0; w < W; ++w) {
        before[e * W + w] = run;
        run += __popc(bitmap[e * W + w]);
      }
      cursor[e] = run;
    }
    __syncthreads();
    for (int tl = tid; tl < nt; tl += kBThreads) {
      int ids[16];
      ids_of(c0 + tl, ids);
      const int w = tl >> 5;
      const uint32_t below = (1u << (tl & 31)) - 1u;
      for (int j = 0; j < k; ++j) {
        const int e = ids[j];
        if (e < 0) continue;
        const int r = before[e * W + w] + __popc(bitmap[e * W + w] & below);
        a.perm[off[e] + r] = (c0 + tl) * k + j;
      }
    }
    __syncthreads();
  }
}

// --- bucketing of many tokens: chunks of tokens, one workgroup each --------
// Stage 1 counts each chunk's entries per expert (one bit per (expert, token)
// in LDS) into the context's chunk-count table. Stage 2, on the same chunks,
// gives every expert its offset from all chunks' counts and each chunk its
// first rank per expert from the chunks before it, then places the chunk's
// entries by the same bits: every list ends in token order, exactly as the
// one-workgroup kernel leaves it. Workgroup 0 of stage 2 also writes the
// per-expert metadata (bucket_meta).
struct ChunkGeom {
  int C, TC, W;  // chunks, tokens per chunk (a multiple of 32), bitmap words per expert
};
inline ChunkGeom chunk_geom(int T, int E) {
  ChunkGeom g;
  g.C = std::min(kBucketChunks, (T + 31) / 32);
  g.TC = ((T + g.C - 1) / g.C + 31) / 32 * 32;
  g.W = g.TC / 32;
  if (g.W * E > kBitmapWords) g.C = 0;  // too many tokens per chunk for the LDS: the one-workgroup kernel
  return g;
}

__global__ __launch_bounds__(256) void bucket_count_kernel(BucketArgs a, int TC, int W, int32_t *cc) {
  __shared__ uint32_t bitmap[kBitmapWords];
  const int tid = threadIdx.x, E = a.E, k = a.k;
  const int c = blockIdx.x, c0 = c * TC, nt = min(TC, a.T - c0);
  for (int i = tid; i < E * W; i += 256) bitmap[i] = 0u;
  __syncthreads();
  bool bad = false;
  for (int tl = tid; tl < nt; tl += 256) {
    int ids[16];
    bad |= !token_ids(a, c0 + tl, ids);
    for (int j = 0; j < k; ++j)
      if (ids[j] >= 0) atomicOr(&bitmap[ids[j] * W + (tl >> 5)], 1u << (tl & 31));
  }
  if (bad) atomicOr(a.err, (uint32_t)ERRF_BAD_INDEX);
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int n = 0;
    for (int w = 0; w < W; ++w) n += __popc(bitmap[e * W + w]);
    cc[(int64_t)c * E + e] = n;
  }
}

__global__ __launch_bounds__(kBThreads) void bucket_place_kernel(BucketArgs a, int C, int TC, int W,
                                                                 const int32_t *cc) {
  __shared__ int off[1025];
  __shared__ int tmp[kBThreads];
  __shared__ uint32_t bitmap[kBitmapWords];
  __shared__ int before[kBitmapWords];  // the rank of the expert's first entry in each word of the chunk
  const int tid = threadIdx.x, E = a.E, k = a.k;
  const int c = blockIdx.x, c0 = c * TC, nt = min(TC, a.T - c0);
  const int eb = (a.expert_bits && tid < E) ? a.expert_bits[tid] : 0;
  int tot = 0, pre = 0;  // the expert's entries in all chunks, and in the chunks before this one
  if (tid < E)
    for (int c2 = 0; c2 < C; ++c2) {
      const int v = cc[(int64_t)c2 * E + tid];
      tot += v;
      pre += c2 < c ? v : 0;
    }
  if (c == 0) {
    bucket_meta(a, tot, eb, tmp, off);  // off[] as well
  } else {
    const int ex = block_exclusive_scan(tot, tmp);
    if (tid < E) off[tid] = ex;
  }
  for (int i = tid; i < E * W; i += kBThreads) bitmap[i] = 0u;
  __syncthreads();
  for (int tl = tid; tl < nt; tl += kBThreads) {
    int ids[16];
    token_ids(a, c0 + tl, ids);
    for (int j = 0; j < k; ++j)
      if (ids[j] >= 0) atomicOr(&bitmap[ids[j] * W + (tl >> 5)], 1u << (tl & 31));
  }
  __syncthreads();
  if (tid < E) {
    int run = off[tid] + pre;
    for (int w = 0; w < W; ++w) {
      before[tid * W + w] = run;
      run += __popc(bitmap[tid * W + w]);
    }
  }
  __syncthreads();
  for (int tl = tid; tl < nt; tl += kBThreads) {
    int ids[16];
    token_ids(a, c0 + tl, ids);
    const int w = tl >> 5;
    const uint32_t below = (1u << (tl & 31)) - 1u;
    for (int j = 0; j < k; ++j) {
      const int e = ids[j];
      if (e < 0) continue;
      a.perm[before[e * W + w] + __popc(bitmap[e * W + w] & below)] = (c0 + tl) * k + j;
    }
  }
}

}  // namespace

moe_status launch_bucket(moe_ctx *ctx, const int32_t *idx, int T, int k, int E, int32_t *counts, int32_t *offsets,
                         int32_t *perm, const uint8_t *expert_bits, int want_bits, int32_t *active,
                         int32_t *n_active, int2 *units, int32_t *n_units, int ubig_max, int has_shared,
                         int small_max) {
  BucketArgs a{idx,    T,        k,         E,         counts,     offsets,   perm,
               expert_bits, want_bits, active, n_active, ctx->dev_small, units, n_units,
               ubig_max, has_shared, small_max};
  // many entries: the chunked kernels (the one-workgroup kernel keeps small
  // calls' ids in LDS and needs no second launch)
#ifndef MOE_BUCKET_CHUNKED
#define MOE_BUCKET_CHUNKED 1
#endif
  const ChunkGeom g = (MOE_BUCKET_CHUNKED && (int64_t)T * k > kIdsCache) ? chunk_geom(T, E) : ChunkGeom{0, 0, 0};
  MoeTimer tm_(ctx, MOE_STAGE_BUCKET);
  if (g.C > 0) {
    int32_t *cc = reinterpret_cast<int32_t *>(ctx->dev_small) + kBucketChunkWord;
    hipLaunchKernelGGL(bucket_count_kernel, dim3(g.C), dim3(256), 0, ctx->stream, a, g.TC, g.W, cc);
    MOE_CHECK_LAUNCH("bucket_count_kernel");
    hipLaunchKernelGGL(bucket_place_kernel, dim3(g.C), dim3(kBThreads), 0, ctx->stream, a, g.C, g.TC, g.W, cc);
    MOE_CHECK_LAUNCH("bucket_place_kernel");
    return MOE_OK;
  }
  hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(kBThreads), 0, ctx->stream, a);
  MOE_CHECK_LAUNCH("bucket_kernel");
  return MOE_OK;
}

moe_status launch_bucket_public(moe_ctx *ctx, const int32_t *topk_idx, int T, int k, int E, int32_t *counts,
                                int32_t *offsets, int32_t *perm) {
  return launch_bucket(ctx, topk_idx, T, k, E, counts, offsets, perm, nullptr, 0, nullptr, nullptr, nullptr, nullptr,
                       0, 0, kUnitSmall);
}

namespace {
// K slices of the router logits (1 when the caller passes logits)
int router_slices(const moe_ctx *ctx, const moe_router_cfg *cfg, int T, int H) {
  if (cfg->logits_in) return 1;
  const int E = cfg->n_experts;
  int ks = 1;
  if (T <= kSmallT) {
    // enough waves to stream w_router with the whole chip: ~4 waves per CU
    const int groups = (E + 3) / 4;
    while (groups * ks < 2 * ctx->n_cu && H % (ks * 2 * 256) == 0 && ks < 16) ks *= 2;
  } else {
    const int tiles = ((T + kTile - 1) / kTile) * ((E + kTile - 1) / kTile);
    while (tiles * ks < 2 * ctx->n_cu && H % (ks * 2 * kTileK) == 0 && H / (ks * 2) >= 256 && ks < 16) ks *= 2;
  }
  return ks;
}
}  // namespace

size_t router_scratch_bytes(const moe_ctx *ctx, const moe_router_cfg *cfg, int T, int H) {
  if (cfg->logits_in) return 0;
  return sizeof(float) * (size_t)router_slices(ctx, cfg, T, H) * T * cfg->n_experts;
}

moe_status launch_router(moe_ctx *ctx, const moe_router_cfg *cfg, const float *x, const float *w_router,
                         const float *bias, int T, int H, int32_t *topk_idx, float *topk_w) {
  const int E = cfg->n_experts, k = cfg->top_k;
  const float *partial = x;
  int nslices = 1;
  if (!cfg->logits_in) {
    const int ks = router_slices(ctx, cfg, T, H);
    const int kl = H / ks;
    void *scr = nullptr;
    moe_status st = moe_scratch(ctx, sizeof(float) * (size_t)ks * T * E, &scr);
    if (st) return st;
    float *part = static_cast<float *>(scr);
    if (T <= kSmallT) {
      {
        MoeTimer tm_(ctx, MOE_STAGE_ROUTER);
        hipLaunchKernelGGL(router_gemv_kernel, dim3((E + 3) / 4, ks), dim3(256), 0, ctx->stream, x, w_router, T, H, E,
                           kl, part);
      }
    } else {
      {
        MoeTimer tm_(ctx, MOE_STAGE_ROUTER);
        const dim3 grid((T + kTile - 1) / kTile, (E + kTile - 1) / kTile, ks);
#ifndef MOE_ROUTER_MFMA
#define MOE_ROUTER_MFMA 1
#endif
        if (MOE_ROUTER_MFMA && kl % kMfmaK == 0)
          hipLaunchKernelGGL(router_gemm_mfma_kernel, grid, dim3(256), 0, ctx->stream, x, w_router, T, H, E, kl,
                             part);
        else
          hipLaunchKernelGGL(router_gemm_kernel, grid, dim3(256), 0, ctx->stream, x, w_router, T, H, E, kl, part);
      }
    }
    MOE_CHECK_LAUNCH("router logits kernel");
    partial = part;
    nslices = ks;
  }
  {
    MoeTimer tm_(ctx, MOE_STAGE_ROUTER);
    const dim3 g((T + kTopkWaves - 1) / kTopkWaves), b(kTopkWaves * MOE_WAVE);
    switch (nslices) {
      case 1: hipLaunchKernelGGL(router_topk_kernel<1>, g, b, 0, ctx->stream, partial, T, E, k, bias, cfg->routed_scale, cfg->top_p, topk_idx, topk_w); break;
      case 2: hipLaunchKernelGGL(router_topk_kernel<2>, g, b, 0, ctx->stream, partial, T, E, k, bias, cfg->routed_scale, cfg->top_p, topk_idx, topk_w); break;
      case 4: hipLaunchKernelGGL(router_topk_kernel<4>, g, b, 0, ctx->stream, partial, T, E, k, bias, cfg->routed_scale, cfg->top_p, topk_idx, topk_w); break;
      case 8: hipLaunchKernelGGL(router_topk_kernel<8>, g, b, 0, ctx->stream, partial, T, E, k, bias, cfg->routed_scale, cfg->top_p, topk_idx, topk_w); break;
      default: hipLaunchKernelGGL(router_topk_kernel<16>, g, b, 0, ctx->stream, partial, T, E, k, bias, cfg->routed_scale, cfg->top_p, topk_idx, topk_w); break;
    }
  }
  MOE_CHECK_LAUNCH("router_topk_kernel");
  return MOE_OK;
}
