// Multi-token SwiGLU expert FFN on the int8 matrix cores
// (v_mfma_i32_16x16x64_i8: 16 x 16 int32 results over 64 int8 products).
//
// agentlenshq.com, "Colibri: running GLM-5.2 744B MoE on consumer hardware",
// section "Key features": packed int4/int8/int2 weights with per-row scales,
// dequantised on use, and int8 matmuls as integer dot products (here the
// matrix cores' exact int32 accumulation). remio.ai, "Colibri shows how to run
// GLM-5.2 on a low-spec PC", section "The RAM wall became a storage problem":
// an expert needed by several batch positions is read once -- here once per
// tile of up to 64 of them.
//
// After bucket_kernel has built the per-expert token lists and their tiles:
//  1. act_field_kernel (int4 and int2 only): every token's int8 codes
//     reordered into the packed weights' field order -- per 32 elements the 16
//     even ones then the 16 odd ones (int4), per 64 elements the four 2-bit
//     fields of 16 elements each (int2), each such 16-byte step stored next
//     to the same step of the three neighbouring pieces (field_pos) -- and
//     the sum of the codes.
//  2. gu_mfma_kernel: one workgroup per (token tile, 64 rows of gate and of
//     up); wave w owns rows 16w..16w+15 of both. A row is read as 16-byte
//     pieces; per step lane l takes piece 4c + l/16 of row l%16 and splits it
//     into its 1, 2 or 4 fields (int8 bytes, or offset-binary values 0..15 /
//     0..3 held as int8). The matrix core pairs byte j of lane l's activation
//     operand with byte j of its weight operand, so the field order of the
//     activations makes each weight field meet its own element. The offset is
//     removed once per token with its code sum. Epilogue: the scales, SiLU,
//     a = silu(g) * u into the (token, slot) row of the intermediate.
//  3. requant_mfma_kernel: per (token, slot) pair: sa = max|a| / 127 and the
//     codes rint(a / sa), written in field order, and their sum.
//  4. dn_mfma_kernel: one workgroup per (token tile, 128 down rows), each wave
//     32 rows; y = acc * s_down * sa into the slot buffer.
// A tile holds up to 64 tokens of one expert, run as 4 blocks of 16 through
// the matrix core (rows past the expert's last token repeat it and are not
// stored); an expert's remainder of 1..16 tokens is a one-block tile (when
// experts average 32 or more tokens, a remainder is a full-size tile too).
// Each kind has its own launch: the one-block kernel needs fewer registers
// and runs more workgroups per CU, both keeping two weight steps in flight.
// Weight rows stream from HBM once per tile; the activation rows are re-read
// from L2.
#include <algorithm>

#include "gemv_common.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMaxI = 8192;

struct MArgs {
  const moe_expert_w *experts;
  moe_expert_w shared;
  int has_shared;
  const int8_t *xa;      // [T][xstride] token codes in field order (xq itself for int8)
  int xstride, astride;  // row strides of xa and aq: whole groups of four pieces
  const int32_t *xsum;   // [T] code sums (int4, int2)
  const float *sx;       // [T]
  const int32_t *topk_idx;
  const uint8_t *expert_bits;
  int bits, T, H, I, E, k;
  const int32_t *counts, *offsets, *perm, *active, *n_active;
  const int2 *units;      // tiles: [ubig_max] of up to 64 tokens, then the one-block tiles
  const int32_t *n_units;  // [2] tiles of each kind
  int ubig_max;
  int small_max;           // remainders of up to this many tokens are one-block tiles
  float *A;      // [P][I] SwiGLU intermediate, P = T (k + 1)
  int8_t *aq;    // [P][astride] its codes, field order
  int32_t *aqs;  // [P] code sums
  float *sa;     // [P]
  float *y;      // [T][k+1][H]
  moe_debug_bufs dbg;
  int dbg_on;
};

struct Ex {
  moe_expert_w w;
  int ntok, base, is_shared;
};

__device__ __forceinline__ bool resolve_ex(const MArgs &a, int d, Ex &r) {
  const int na = *a.n_active;
  if (d < na) {
    const int e = a.active[d];
    r.w = a.experts[e];
    r.ntok = a.counts[e];
    r.base = a.offsets[e];
    r.is_shared = 0;
    return true;
  }
  if (a.has_shared && d == na) {
    r.w = a.shared;
    r.ntok = a.T;
    r.base = 0;
    r.is_shared = 1;
    return true;
  }
  return false;
}

// token and (token, slot) row of the expert's g-th entry
__device__ __forceinline__ void pair_of(const MArgs &a, const Ex &ex, int g, int &t, int &p) {
  if (ex.is_shared) {
    t = g;
    p = g * (a.k + 1) + a.k;
  } else {
    const int ent = a.perm[ex.base + g];
    t = ent / a.k;
    p = t * (a.k + 1) + (ent - t * a.k);
  }
}

// field S of a 16-byte piece of packed weights as an int8 operand
template <int BITS, int S>
__device__ __forceinline__ v4i wfield(uint4 w) {
  if constexpr (BITS == 8) {
    return v4i{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
  } else if constexpr (BITS == 4) {
    constexpr uint32_t M = 0x0f0f0f0fu;
    return v4i{(int)((w.x >> (4 * S)) & M), (int)((w.y >> (4 * S)) & M), (int)((w.z >> (4 * S)) & M),
               (int)((w.w >> (4 * S)) & M)};
  } else {
    constexpr uint32_t M = 0x03030303u;
    return v4i{(int)((w.x >> (2 * S)) & M), (int)((w.y >> (2 * S)) & M), (int)((w.z >> (2 * S)) & M),
               (int)((w.w >> (2 * S)) & M)};
  }
}

__device__ __forceinline__ v4i mfma(v4i x, v4i w, v4i acc) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(x, w, acc, 0, 0, 0);
}

// Byte offset, in a row of field-ordered codes, of step s (16 bytes) of the
// lane-group piece b (EPC elements): pieces go in groups of four (one per
// lane group of a load), and within a group step s of the four pieces is 64
// contiguous bytes, so one load instruction reads a token's 64 bytes.
template <int BITS>
__device__ __forceinline__ int field_pos(int b, int s) {
  return (b >> 2) * 4 * QFmt<BITS>::kEpc + s * 64 + (b & 3) * 16;
}

struct TileTokens {
  int tok[64], pair[64], osum[64];
  float scale[64];
};

// ---------------------------------------------------------------------------
// token codes in field order
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(kThreads) void act_field_kernel(const int8_t *xq, int H, int8_t *xa, int xstride,
                                                              int32_t *xsum) {
  constexpr int EPC = QFmt<BITS>::kEpc, ND = EPC / 4;
  __shared__ int red[kThreads / MOE_WAVE];
  const int t = blockIdx.x;
  const uint32_t *src = reinterpret_cast<const uint32_t *>(xq + (int64_t)t * H);
  uint8_t *dst = reinterpret_cast<uint8_t *>(xa + (int64_t)t * xstride);
  int sum = 0;
  for (int blk = threadIdx.x; blk < H / EPC; blk += kThreads) {
    uint32_t d[ND], o[ND];
#pragma unroll
    for (int q = 0; q < ND / 4; ++q) {
      const uint4 v = reinterpret_cast<const uint4 *>(src + blk * ND)[q];
      d[4 * q] = v.x;
      d[4 * q + 1] = v.y;
      d[4 * q + 2] = v.z;
      d[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int q = 0; q < ND; ++q) sum = sdot4((int)d[q], 0x01010101, sum);
    if constexpr (BITS == 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) act_order_q4(d[2 * j], d[2 * j + 1], o[j], o[4 + j]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t f[4];
        act_order_q2(d + 4 * j, f);
#pragma unroll
        for (int s = 0; s < 4; ++s) o[4 * s + j] = f[s];
      }
    }
#pragma unroll
    for (int q = 0; q < ND / 4; ++q)
      *reinterpret_cast<uint4 *>(dst + field_pos<BITS>(blk, q)) =
          make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
  }
  sum = wave_sum_i32(sum);
  if ((threadIdx.x & (MOE_WAVE - 1)) == 0) red[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x == 0) xsum[t] = red[0] + red[1] + red[2] + red[3];
}

// ---------------------------------------------------------------------------
// acc[m][mat][nb] += the tokens of block m (16 each) times rows of block nb
// (16 each) of matrix mat, over whole rows of rowbytes packed bytes. wrow:
// this lane's row (l%16 of the block) of each matrix and block. Per step lane
// l takes piece 4c + l/16 of its row. The tokens' field-ordered codes (rows
// abase + ids[t] * astride) are staged in LDS once per workgroup: slices of
// 512 bytes per token, double-buffered, loaded one slice ahead into registers
// and written to LDS after the current slice is consumed, one barrier per
// slice. In LDS the 16-byte unit u of token t sits at unit u ^ (t & 15) of the
// token's row (t & (units - 1) for rows of fewer than 16 units), so the 16
// tokens a read instruction spans hit distinct banks.
// The weight pieces stream through registers D steps ahead.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ void lds_st16(lds_u8 *p, uint4 v) {
  *reinterpret_cast<__attribute__((address_space(3))) moe_u32x4 *>(p) = moe_u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ uint4 lds_ld16(const lds_u8 *p) {
  const moe_u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) moe_u32x4 *>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Weight pieces are loaded four lanes to a 64-byte piece group (lane l: row
// l / 4 of the 16-row block, piece l % 4 of the step), so a load instruction
// touches one cache line segment per four lanes, then regrouped across lanes
// into the matrix-core operand layout (lane m: row m % 16, piece m / 16)
// with four LDS-crossbar permutes per 16 bytes.
#ifndef MOE_MFMA_WPERM
#define MOE_MFMA_WPERM 1
#endif
constexpr bool kWPerm = MOE_MFMA_WPERM != 0;
// skip the staging of a tile's padding tokens
#ifndef MOE_MFMA_SKIP_PAD
#define MOE_MFMA_SKIP_PAD 1
#endif
constexpr bool kSkipPad = MOE_MFMA_SKIP_PAD != 0;

// the 16 bytes lane src holds, for every lane
__device__ __forceinline__ uint4 lane_gather16(uint4 v, int src) {
  const int a = src << 2;
  return make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.x), (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.y),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.z), (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.w));
}

// a wave-uniform pointer, held in scalar registers
template <typename P>
__device__ __forceinline__ P sgpr_p(P p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (P)(((uint64_t)hi << 32) | lo);
}

template <int BITS, int MB, int NM, int NB, int D0, int SL>
__device__ __forceinline__ void tile_mma_lds(const uint8_t *const (&wbase)[NM], const uint32_t (&woff)[NB],
                                             const int8_t *abase, int astride, const int *ids, int nt,
                                             int rowbytes, lds_u8 *lds, v4i (&acc)[MB][NM][NB]) {
  constexpr int EPC = QFmt<BITS>::kEpc, NS = EPC / 16;
  constexpr int SC = SL / (4 * EPC);      // steps per slice
  constexpr int D = D0 < SC ? D0 : SC;    // weight steps in flight (a divisor of SC)
  constexpr int UPT = SL / 16;            // 16-byte units per token and slice
  constexpr int TPI = kThreads / UPT;     // tokens one staging round covers
  constexpr int NI = MB * 16 / TPI;       // staged units per thread and slice
  constexpr int BUF = MB * 16 * SL;       // bytes per slice buffer
  static_assert(NI >= 1 && NI * TPI == MB * 16, "whole tokens per staging round");
  static_assert(SC % D == 0, "the weight buffers rotate within a slice");
  constexpr int SW = UPT < 16 ? UPT - 1 : 15;  // the LDS swizzle: unit u of token t at u ^ (t & SW)
  const int tid = threadIdx.x, grp = (tid & (MOE_WAVE - 1)) >> 4, r16 = tid & 15;
  const int nq = rowbytes / 16;
  const int nch = (nq + 3) / 4;
  const int nsl = (nch + SC - 1) / SC;
  // staging: this thread moves unit su of tokens tid / UPT + TPI i
  const int su = tid % UPT;
  const int8_t *srow[NI];
  int sdst[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int t = tid / UPT + TPI * i;
    srow[i] = abase + (int64_t)ids[t] * astride;
    sdst[i] = t * SL + ((su ^ (t & SW)) << 4);
  }
  // A staged unit whose piece lies past the row end (the last chunk's, or any
  // past the last chunk) is stored as zeros, so the weight pieces loaded for it
  // (clamped re-reads of the row's last piece) add nothing.
  uint4 st[NI];
  bool sv = true;      // the unit this thread stages in the slice in flight lies in the row
  bool sfull = true;   // every unit of that slice does (uniform)
  const int fullb = (nq / 4) * 4 * EPC;  // bytes of the row's complete chunks
  // Tokens past the tile's nt (the repeats of its last token) are neither
  // loaded nor stored: their LDS rows hold whatever they held, and the
  // products of those rows are never stored.
  bool sreal[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) sreal[i] = !kSkipPad || tid / UPT + TPI * i < nt;
  auto aload = [&](int sl) {
    const int o = sl * SL + su * 16;
    sv = (o / (4 * EPC)) * 4 + ((o >> 4) & 3) < nq;
    sfull = (sl + 1) * SL <= fullb;
    const int oc = min(o, astride - 16);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (sreal[i]) st[i] = ldg16(srow[i] + oc, 0);
  };
  auto astore = [&](int b) {
    if (sfull) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (sreal[i]) lds_st16(lds + b * BUF + sdst[i], st[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (sreal[i]) lds_st16(lds + b * BUF + sdst[i], sv ? st[i] : make_uint4(0u, 0u, 0u, 0u));
    }
  };
  uint4 wv[D][NM][NB];
  const int lpiece = kWPerm ? (tid & 3) : grp;  // the piece of the step this lane loads
  const int gsrc = 4 * r16 + grp;               // kWPerm: the lane that loaded this lane's operand
  auto bload = [&](int c, int b) {
    const uint32_t qo = (uint32_t)min(c * 4 + lpiece, nq - 1) << 4;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wv[b][m][nb] = ldg16(wbase[m] + (woff[nb] + qo), 0);
    __builtin_amdgcn_sched_barrier(0);  // issue here, D steps ahead of the use
  };
#pragma unroll
  for (int b = 0; b < D; ++b) bload(b, b);
  aload(0);
  astore(0);
  aload(1);
  __syncthreads();
  for (int sl = 0; sl < nsl; ++sl) {
    const lds_u8 *cur = lds + (sl & 1) * BUF;
#pragma unroll
    for (int cc = 0; cc < SC; ++cc) {
      const int c = sl * SC + cc, b = cc % D;
      if constexpr (kWPerm) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) wv[b][m][nb] = lane_gather16(wv[b][m][nb], gsrc);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        v4i x[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int t = mb * 16 + r16, u = cc * NS * 4 + s * 4 + grp;
          const uint4 v = lds_ld16(cur + t * SL + ((u ^ (t & SW)) << 4));
          x[mb] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        }
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            v4i w;
            if (s == 0) w = wfield<BITS, 0>(wv[b][m][nb]);
            else if (s == 1) w = wfield<BITS, 1>(wv[b][m][nb]);
            else if (s == 2) w = wfield<BITS, 2>(wv[b][m][nb]);
            else w = wfield<BITS, 3>(wv[b][m][nb]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb][m][nb] = mfma(x[mb], w, acc[mb][m][nb]);
          }
      }
      bload(c + D, b);
    }
    astore((sl + 1) & 1);  // the buffer read in the previous slice; every wave has passed the barrier after it
    aload(sl + 2);
    __syncthreads();
  }
}

// the tile's tokens (entries past the expert's last token repeat it)
template <int MB>
__device__ __forceinline__ int stage_tokens(const MArgs &a, const Ex &ex, int m0, bool down, int off,
                                            TileTokens &tt_s) {
  const int nt = min(MB * 16, ex.ntok - m0);  // >= 1 for a listed tile
  const int tid = threadIdx.x;
  if (tid < MB * 16) {
    int t, p;
    pair_of(a, ex, m0 + min(tid, nt - 1), t, p);
    tt_s.tok[tid] = t;
    tt_s.pair[tid] = p;
    tt_s.scale[tid] = down ? a.sa[p] : a.sx[t];
    if (off != 0) tt_s.osum[tid] = off * (down ? a.aqs[p] : a.xsum[t]);
  }
  return nt;
}

// MB = 4: the tiles of more than 16 tokens; MB = 1: the one-block tiles
// (SL: bytes of codes per token and staged slice). When experts average 32
// or more tokens (every remainder a full-size tile), the 64-token tiles stage
// 256-byte slices: half the LDS, so more workgroups per CU (T = 2048: 1.80
// against 1.86 ms per call); with fewer tokens 512-byte slices do better.
template <int MB>
struct GuShape {
  static constexpr int NB = MB == 4 ? 2 : 1, D = 2, SL = 512;
};
template <int MB>
struct DnShape {
  static constexpr int NB = 2, D = 2, SL = 512;
};
constexpr int kSlWide = 256;  // the 64-token tiles' slice when experts average 32 or more tokens

// ---------------------------------------------------------------------------
// gate + up: a workgroup takes 64 NB rows of each, a wave 16 NB
// ---------------------------------------------------------------------------
template <int BITS, int MB, int NB, int D, int SL>
__device__ __forceinline__ void gu_tile(const MArgs &a, TileTokens &tt_s, lds_u8 *lds, int d, int m0, int ntile) {
  constexpr int OFF = QFmt<BITS>::kOff;
  Ex ex;
  if (!resolve_ex(a, d, ex)) return;
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x >> 6;
  const int grp = lane >> 4, r16 = lane & 15;
  const int nt = stage_tokens<MB>(a, ex, m0, false, OFF, tt_s);
  const int rowbytes = a.H * BITS / 8;
  int row[NB];
  const uint8_t *const wbase[2] = {sgpr_p(ex.w.gate), sgpr_p(ex.w.up)};
  uint32_t woff[NB];
  float sg[NB], su[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    row[nb] = ntile * (64 * NB) + wave * (16 * NB) + nb * 16 + r16;
    const int rc = min(row[nb], a.I - 1);  // rows past I: re-read, not stored
    const int rl = min(kWPerm ? row[nb] - r16 + (lane >> 2) : row[nb], a.I - 1);  // the row this lane loads
    woff[nb] = (uint32_t)rl * (uint32_t)rowbytes;
    // global-space loads: a pending flat load would make every wait in the
    // K loop below a wait for all loads
    sg[nb] = gptr(ex.w.s_gate)[rc];
    su[nb] = gptr(ex.w.s_up)[rc];
  }
  __syncthreads();
  v4i acc[MB][2][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][0][nb] = acc[mb][1][nb] = v4i{0, 0, 0, 0};
  tile_mma_lds<BITS, MB, 2, NB, D, SL>(wbase, woff, a.xa, a.xstride, tt_s.tok, nt, rowbytes, lds, acc);
  // lane holds tokens 4*grp + r of each block, row row[nb]
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = mb * 16 + grp * 4 + r;
      if (tt >= nt) continue;
      const int64_t p = tt_s.pair[tt];
      const float sxt = tt_s.scale[tt];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (row[nb] >= a.I) continue;
        int gi = acc[mb][0][nb][r], ui = acc[mb][1][nb][r];
        if constexpr (OFF != 0) {
          gi -= tt_s.osum[tt];
          ui -= tt_s.osum[tt];
        }
        const float g = (float)gi * sg[nb] * sxt;
        const float u = (float)ui * su[nb] * sxt;
        const float av = moe_silu_f32(g) * u;
        const int64_t o = p * a.I + row[nb];
        a.A[o] = av;
        if (a.dbg_on) {
          if (a.dbg.accg) a.dbg.accg[o] = gi;
          if (a.dbg.accu) a.dbg.accu[o] = ui;
          if (a.dbg.a) a.dbg.a[o] = av;
        }
      }
    }
}

// Workgroup -> (tile, row tile). Workgroups go to the 8 XCDs in turn (id mod
// 8), each XCD with its own L2; the mapping gives every XCD a contiguous range
// of the (tile, row tile) order, row tiles fastest, so the workgroups that
// read one tile's activations run together on one XCD and find them in its L2
// (and those of an expert's next tile share its weight rows there).
__device__ __forceinline__ bool xcd_work(int n_units, int ntiles, int &unit, int &ntile) {
  const int total = n_units * ntiles;
  const int b = blockIdx.x;
  if (b >= total) return false;
  const int x = b & 7, slot = b >> 3, q = total >> 3, r = total & 7;
  const int L = x * q + min(x, r) + slot;  // a bijection of [0, total)
  unit = L / ntiles;
  ntile = L - unit * ntiles;
  return true;
}

// Full-size tiles: within one expert's block of (tile, row tile) work, the
// tiles vary fastest, so the workgroups that multiply the same weight rows
// against the expert's different token tiles are dispatched one after another
// on one XCD and read those rows from its L2 at about the same time. An
// expert's tiles are consecutive in the tile list; unit u of the plain order
// finds its expert's first tile (u minus its own index j) and the expert's
// tile count (from its token count, as the bucketing formed them).
__device__ __forceinline__ void expert_major(const MArgs &a, int ntiles, int &u, int &nt) {
  const int L = u * ntiles + nt;
  const int2 un = a.units[u];
  const int j = un.y / kUnitM;
  const int u0 = u - j;
  const int na = *a.n_active;
  const int c = un.x < na ? a.counts[a.active[un.x]] : a.T;  // past the active list: the shared expert
  const int rem = c % kUnitM;
  const int n = c / kUnitM + (rem > a.small_max ? 1 : 0);
  const int local = L - u0 * ntiles;
  nt = local / n;
  u = u0 + (local - nt * n);
}

template <int BITS, int MB, int SL = GuShape<MB>::SL>
__global__ __launch_bounds__(kThreads) void gu_mfma_kernel(MArgs a, int ntiles) {
  __shared__ TileTokens tt_s;
  __shared__ __align__(16) uint8_t abuf_s[2 * MB * 16 * SL];
  lds_u8 *abuf = (lds_u8 *)abuf_s;
  int u, nt;
  if (!xcd_work(a.n_units[MB == 4 ? 0 : 1], ntiles, u, nt)) return;
  if constexpr (MB == 4) expert_major(a, ntiles, u, nt);
  const int2 un = a.units[MB == 4 ? u : a.ubig_max + u];
  gu_tile<BITS, MB, GuShape<MB>::NB, GuShape<MB>::D, SL>(a, tt_s, abuf, un.x, un.y, nt);
}

// ---------------------------------------------------------------------------
// requantisation of a, one workgroup per (token, slot) pair
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(kThreads) void requant_mfma_kernel(MArgs a) {
  constexpr int G = (BITS == 8) ? 4 : (BITS == 4 ? 8 : 16);  // consecutive elements per thread and group
  constexpr int GD = G / 4;
  constexpr int kIt = (kMaxI / G + kThreads - 1) / kThreads;
  __shared__ float red_m[kThreads / MOE_WAVE];
  __shared__ int red_s[kThreads / MOE_WAVE];
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
  const int tid = threadIdx.x, lane = tid & (MOE_WAVE - 1), wave = tid >> 6;
  const int ng = a.I / G;
  const float4 *src = reinterpret_cast<const float4 *>(a.A + p * a.I);
  float4 v[kIt][GD];
  float m = 0.0f;
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int g = min(tid + it * kThreads, ng - 1);  // past the end: a re-read group, same maximum
#pragma unroll
    for (int q = 0; q < GD; ++q) {
      v[it][q] = src[g * GD + q];
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[it][q].x), fabsf(v[it][q].y)), fmaxf(fabsf(v[it][q].z), fabsf(v[it][q].w))));
    }
  }
  m = wave_max_f32(m);
  if (lane == 0) red_m[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  const float sc = (m == 0.0f) ? 0.0f : m / 127.0f;
  int csum = 0;
  uint8_t *dst = reinterpret_cast<uint8_t *>(a.aq + p * a.astride);
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int g = tid + it * kThreads;
    if (g >= ng) break;
    uint32_t nat[GD];
#pragma unroll
    for (int q = 0; q < GD; ++q) {
      const float e4[4] = {v[it][q].x, v[it][q].y, v[it][q].z, v[it][q].w};
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int c = 0;
        if (m != 0.0f) c = (int)fminf(fmaxf(__builtin_rintf(e4[j] / sc), -127.0f), 127.0f);
        w |= (uint32_t)(uint8_t)(int8_t)c << (8 * j);
      }
      nat[q] = w;
      csum = sdot4((int)w, 0x01010101, csum);
    }
    if (a.dbg_on && a.dbg.aq) {
#pragma unroll
      for (int q = 0; q < GD; ++q) reinterpret_cast<uint32_t *>(a.dbg.aq + p * a.I + g * G)[q] = nat[q];
    }
    if constexpr (BITS == 8) {
      *reinterpret_cast<uint32_t *>(dst + g * 4) = nat[0];
    } else if constexpr (BITS == 4) {
      uint32_t ev, od;
      act_order_q4(nat[0], nat[1], ev, od);
      *reinterpret_cast<uint32_t *>(dst + field_pos<4>(g >> 2, 0) + (g & 3) * 4) = ev;
      *reinterpret_cast<uint32_t *>(dst + field_pos<4>(g >> 2, 1) + (g & 3) * 4) = od;
    } else {
      uint32_t f[4];
      act_order_q2(nat, f);
#pragma unroll
      for (int s = 0; s < 4; ++s) *reinterpret_cast<uint32_t *>(dst + field_pos<2>(g >> 2, s) + (g & 3) * 4) = f[s];
    }
  }
  csum = wave_sum_i32(csum);
  if (lane == 0) red_s[wave] = csum;
  __syncthreads();
  if (tid == 0) {
    a.aqs[p] = red_s[0] + red_s[1] + red_s[2] + red_s[3];
    a.sa[p] = sc;
    if (a.dbg_on && a.dbg.sa) a.dbg.sa[p] = sc;
  }
}

// ---------------------------------------------------------------------------
// down: a workgroup takes 64 NB rows, a wave 16 NB
// ---------------------------------------------------------------------------
template <int BITS, int MB, int NB, int D, int SL>
__device__ __forceinline__ void dn_tile(const MArgs &a, TileTokens &tt_s, lds_u8 *lds, int d, int m0, int ntile) {
  constexpr int OFF = QFmt<BITS>::kOff;
  Ex ex;
  if (!resolve_ex(a, d, ex)) return;
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x >> 6;
  const int grp = lane >> 4, r16 = lane & 15;
  const int nt = stage_tokens<MB>(a, ex, m0, true, OFF, tt_s);
  const int rowbytes = a.I * BITS / 8;
  int row[NB];
  const uint8_t *const wbase[1] = {sgpr_p(ex.w.down)};
  uint32_t woff[NB];
  float sd[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    row[nb] = ntile * (64 * NB) + wave * (16 * NB) + nb * 16 + r16;
    const int rc = min(row[nb], a.H - 1);
    const int rl = min(kWPerm ? row[nb] - r16 + (lane >> 2) : row[nb], a.H - 1);  // the row this lane loads
    woff[nb] = (uint32_t)rl * (uint32_t)rowbytes;
    sd[nb] = gptr(ex.w.s_down)[rc];
  }
  __syncthreads();
  v4i acc[MB][1][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][0][nb] = v4i{0, 0, 0, 0};
  tile_mma_lds<BITS, MB, 1, NB, D, SL>(wbase, woff, a.aq, a.astride, tt_s.pair, nt, rowbytes, lds, acc);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = mb * 16 + grp * 4 + r;
      if (tt >= nt) continue;
      const int64_t p = tt_s.pair[tt];
      const float sat = tt_s.scale[tt];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (row[nb] >= a.H) continue;
        int di = acc[mb][0][nb][r];
        if constexpr (OFF != 0) di -= tt_s.osum[tt];
        a.y[p * a.H + row[nb]] = (float)di * sd[nb] * sat;
        if (a.dbg_on && a.dbg.accd) a.dbg.accd[p * a.H + row[nb]] = di;
      }
    }
}

template <int BITS, int MB, int SL = DnShape<MB>::SL>
__global__ __launch_bounds__(kThreads) void dn_mfma_kernel(MArgs a, int ntiles) {
  __shared__ TileTokens tt_s;
  __shared__ __align__(16) uint8_t abuf_s[2 * MB * 16 * SL];
  lds_u8 *abuf = (lds_u8 *)abuf_s;
  int u, nt;
  if (!xcd_work(a.n_units[MB == 4 ? 0 : 1], ntiles, u, nt)) return;
  if constexpr (MB == 4) expert_major(a, ntiles, u, nt);
  const int2 un = a.units[MB == 4 ? u : a.ubig_max + u];
  dn_tile<BITS, MB, DnShape<MB>::NB, DnShape<MB>::D, SL>(a, tt_s, abuf, un.x, un.y, nt);
}

template <int BITS>
moe_status launch_bits(moe_ctx *ctx, const MArgs &a, const int8_t *xq, int8_t *xa, int32_t *xsum, int usmall) {
  if constexpr (BITS != 8) {
    moe_launch(ctx, MOE_STAGE_BUCKET, act_field_kernel<BITS>, dim3(a.T), dim3(kThreads), xq, a.H, xa, a.xstride,
               xsum);
    MOE_CHECK_LAUNCH("act_field_kernel");
  }
  auto tiles = [](int n, int rows) { return (n + rows - 1) / rows; };
  const int g4 = tiles(a.I, 64 * GuShape<4>::NB), g1 = tiles(a.I, 64 * GuShape<1>::NB);
  const int d4 = tiles(a.H, 64 * DnShape<4>::NB), d1 = tiles(a.H, 64 * DnShape<1>::NB);
  // 1-D grids sized for the most tiles the bucket can list; the surplus
  // workgroups return at once. The two tile kinds write disjoint rows: the
  // 64-token tiles run on the side stream, overlapping the one-block tiles.
  moe_status st;
  if (a.small_max == 0) {
    // Experts average 32 or more tokens: every remainder is a full-size
    // tile, the bucketing lists no one-block tile, and the 64-token launches
    // run alone on the context stream with 256-byte slices.
    moe_launch(ctx, MOE_STAGE_GATEUP, gu_mfma_kernel<BITS, 4, kSlWide>, dim3(a.ubig_max * g4), dim3(kThreads), a,
               g4);
    MOE_CHECK_LAUNCH("gu_mfma_kernel");
    moe_launch(ctx, MOE_STAGE_REQUANT, requant_mfma_kernel<BITS>, dim3(a.T * (a.k + 1)), dim3(kThreads), a);
    MOE_CHECK_LAUNCH("requant_mfma_kernel");
    moe_launch(ctx, MOE_STAGE_DOWN, dn_mfma_kernel<BITS, 4, kSlWide>, dim3(a.ubig_max * d4), dim3(kThreads), a, d4);
    MOE_CHECK_LAUNCH("dn_mfma_kernel");
    return MOE_OK;
  }
  if ((st = moe_side_fork(ctx))) return st;
  moe_launch_on(ctx, ctx->side, MOE_STAGE_GATEUP, gu_mfma_kernel<BITS, 4>, dim3(a.ubig_max * g4), dim3(kThreads), a,
                g4);
  MOE_CHECK_LAUNCH("gu_mfma_kernel");
  moe_launch(ctx, MOE_STAGE_GATEUP, gu_mfma_kernel<BITS, 1>, dim3(usmall * g1), dim3(kThreads), a, g1);
  MOE_CHECK_LAUNCH("gu_mfma_kernel");
  if ((st = moe_side_join(ctx))) return st;
  moe_launch(ctx, MOE_STAGE_REQUANT, requant_mfma_kernel<BITS>, dim3(a.T * (a.k + 1)), dim3(kThreads), a);
  MOE_CHECK_LAUNCH("requant_mfma_kernel");
  if ((st = moe_side_fork(ctx))) return st;
  moe_launch_on(ctx, ctx->side, MOE_STAGE_DOWN, dn_mfma_kernel<BITS, 4>, dim3(a.ubig_max * d4), dim3(kThreads), a,
                d4);
  MOE_CHECK_LAUNCH("dn_mfma_kernel");
  moe_launch(ctx, MOE_STAGE_DOWN, dn_mfma_kernel<BITS, 1>, dim3(usmall * d1), dim3(kThreads), a, d1);
  MOE_CHECK_LAUNCH("dn_mfma_kernel");
  return moe_side_join(ctx);
}

}  // namespace

bool expert_ffn_mfma_supported(int bits, int H, int I) {
  return H % 16 == 0 && I % 16 == 0 && I <= kMaxI && (H * bits / 8) % 16 == 0 && (I * bits / 8) % 16 == 0;
}

namespace {
// Scratch layout of one matrix-core FFN call.
struct MfmaLayout {
  int dact, ubig, usmall, xstride, astride;
  size_t o_counts, o_offsets, o_perm, o_active, o_nact, o_units, o_nunits, o_xa, o_xsum, o_A, o_aq, o_aqs, o_sa;
  size_t size;
};

MfmaLayout mfma_layout(int bits, int has_shared, int T, int H, int I, int E, int k) {
  MfmaLayout l;
  const int64_t P = (int64_t)T * (k + 1);
  l.dact = (int)std::min<int64_t>(E, (int64_t)T * k);
  // sum over experts of ceil(n_e / 64) <= T k / 64 + (active experts), plus the shared expert's tiles
  l.ubig = (int)(((int64_t)T * k) / kUnitM + l.dact + 1 + (has_shared ? (T + kUnitM - 1) / kUnitM : 0));
  l.usmall = l.dact + 1;
  // rows of field-ordered codes hold whole groups of four lane pieces
  const int grp_bytes = 4 * (128 / bits);
  l.xstride = bits == 8 ? H : (int)moe_round_up(H, grp_bytes);
  l.astride = (int)moe_round_up(I, grp_bytes);
  MoeLayout m;
  l.o_counts = m.take(4 * (size_t)E);
  l.o_offsets = m.take(4 * (size_t)(E + 1));
  l.o_perm = m.take(4 * (size_t)T * k);
  l.o_active = m.take(4 * (size_t)E);
  l.o_nact = m.take(4);
  l.o_units = m.take(8 * (size_t)(l.ubig + l.usmall));
  l.o_nunits = m.take(8);
  l.o_xa = m.take(bits == 8 ? 0 : (size_t)T * l.xstride);
  l.o_xsum = m.take(4 * (size_t)T);
  l.o_A = m.take(4 * (size_t)P * I);
  l.o_aq = m.take((size_t)P * l.astride);
  l.o_aqs = m.take(4 * (size_t)P);
  l.o_sa = m.take(4 * (size_t)P);
  l.size = m.size;
  return l;
}
}  // namespace

size_t expert_ffn_mfma_scratch_bytes(int bits, int has_shared, int T, int H, int I, int E, int k) {
  return mfma_layout(bits, has_shared, T, H, I, E, k).size;
}

moe_status launch_expert_ffn_mfma(moe_ctx *ctx, int bits, const moe_expert_w *experts, const moe_expert_w *shared,
                                  const uint8_t *expert_bits, const int8_t *xq, const float *sx,
                                  const int32_t *topk_idx, int T, int H, int I, int E, int k, float *y_slots) {
  const int has_shared = shared ? 1 : 0;
  const MfmaLayout l = mfma_layout(bits, has_shared, T, H, I, E, k);
  const int ubig = l.ubig, usmall = l.usmall;
  void *scr = nullptr;
  moe_status st = moe_scratch(ctx, l.size, &scr);
  if (st) return st;
  char *base = static_cast<char *>(scr);
  MArgs a{};
  a.experts = experts;
  a.has_shared = has_shared;
  if (shared) a.shared = *shared;
  int8_t *xa = bits == 8 ? const_cast<int8_t *>(xq) : reinterpret_cast<int8_t *>(base + l.o_xa);
  int32_t *xsum = reinterpret_cast<int32_t *>(base + l.o_xsum);
  a.xa = xa;
  a.xstride = l.xstride;
  a.astride = l.astride;
  a.xsum = xsum;
  a.sx = sx;
  a.topk_idx = topk_idx;
  a.expert_bits = expert_bits;
  a.bits = bits;
  a.T = T; a.H = H; a.I = I; a.E = E; a.k = k;
  int32_t *counts = reinterpret_cast<int32_t *>(base + l.o_counts);
  int32_t *offsets = reinterpret_cast<int32_t *>(base + l.o_offsets);
  int32_t *perm = reinterpret_cast<int32_t *>(base + l.o_perm);
  int32_t *active = reinterpret_cast<int32_t *>(base + l.o_active);
  int32_t *nact = reinterpret_cast<int32_t *>(base + l.o_nact);
  int2 *units = reinterpret_cast<int2 *>(base + l.o_units);
  int32_t *nunits = reinterpret_cast<int32_t *>(base + l.o_nunits);
  a.counts = counts; a.offsets = offsets; a.perm = perm; a.active = active; a.n_active = nact;
  a.units = units;
  a.n_units = nunits;
  a.ubig_max = ubig;
  a.A = reinterpret_cast<float *>(base + l.o_A);
  a.aq = reinterpret_cast<int8_t *>(base + l.o_aq);
  a.aqs = reinterpret_cast<int32_t *>(base + l.o_aqs);
  a.sa = reinterpret_cast<float *>(base + l.o_sa);
  a.y = y_slots;
  a.dbg = ctx->dbg;
  a.dbg_on = ctx->dbg_on ? 1 : 0;
  // when experts average many tokens (k T / E >= 32), a remainder becomes a
  // full-size tile too: it then runs beside the expert's other tiles and
  // shares their weight rows through L2 instead of streaming them again
  a.small_max = (int64_t)T * k >= 32 * (int64_t)E ? 0 : kUnitSmall;
  st = launch_bucket(ctx, topk_idx, T, k, E, counts, offsets, perm, expert_bits, bits, active, nact, units, nunits,
                     ubig, has_shared, a.small_max);
  if (st) return st;
  if (T == 0) return MOE_OK;
  switch (bits) {
    case 8: return launch_bits<8>(ctx, a, xq, xa, xsum, usmall);
    case 4: return launch_bits<4>(ctx, a, xq, xa, xsum, usmall);
    default: return launch_bits<2>(ctx, a, xq, xa, xsum, usmall);
  }
}
