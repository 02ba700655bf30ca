// Device helpers shared by the streaming GEMV kernels: DPP wave reductions,
// activation chunks held in registers in the packed weights' field order,
// and the integer dot product of one 16-byte weight chunk.
#pragma once

#include "moe_internal.h"

// Pointers read from memory are generic (flat) to the compiler; flat loads
// also count against the scalar-load counter, so a wait for a scalar load
// would stall on them. Weight and activation reads go through this cast to
// the global address space instead.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T *gptr(const T *p) {
  return (const __attribute__((address_space(1))) T *)p;
}
typedef unsigned int moe_u32x4 __attribute__((ext_vector_type(4)));
// 16-byte global load of p[idx]
__device__ __forceinline__ uint4 ldg16(const void *p, int idx) {
  const moe_u32x4 v = gptr(reinterpret_cast<const moe_u32x4 *>(p))[idx];
  return make_uint4(v.x, v.y, v.z, v.w);
}
// The same with the non-temporal hint: for weight bytes read once per call,
// which need not stay in the caches (measured: a plain streaming read of
// 57 MB to 1 GiB runs 7-13% faster with it on this device).
__device__ __forceinline__ uint4 ldg16_nt(const void *p, int idx) {
  const moe_u32x4 v = __builtin_nontemporal_load(gptr(reinterpret_cast<const moe_u32x4 *>(p)) + idx);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// wave reductions with DPP (sum lands in lane 63)
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ int wave_sum_to63(int v) {
  v += dpp_i<0xB1>(v);        // quad_perm [1,0,3,2]
  v += dpp_i<0x4E>(v);        // quad_perm [2,3,0,1]
  v += dpp_i<0x141>(v);       // row_half_mirror
  v += dpp_i<0x140>(v);       // row_mirror
  v += dpp_i<0x142, 0xa>(v);  // row_bcast:15 -> rows 1, 3
  v += dpp_i<0x143, 0xc>(v);  // row_bcast:31 -> rows 2, 3
  return v;
}
// wave-uniform total
__device__ __forceinline__ int wave_sum_all(int v) { return __builtin_amdgcn_readlane(wave_sum_to63(v), 63); }

// max / min reductions: lanes of masked rows keep their own value
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_keep(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ float fmax_dpp_step(float v, int d) { return fmaxf(v, __int_as_float(d)); }
// wave-uniform maximum (no NaN inputs)
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmax_dpp_step(v, dpp_keep<0xB1>(__float_as_int(v)));
  v = fmax_dpp_step(v, dpp_keep<0x4E>(__float_as_int(v)));
  v = fmax_dpp_step(v, dpp_keep<0x141>(__float_as_int(v)));
  v = fmax_dpp_step(v, dpp_keep<0x140>(__float_as_int(v)));
  v = fmax_dpp_step(v, dpp_keep<0x142, 0xa>(__float_as_int(v)));
  v = fmax_dpp_step(v, dpp_keep<0x143, 0xc>(__float_as_int(v)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// wave-uniform minimum
__device__ __forceinline__ int wave_min_dpp(int v) {
  v = min(v, dpp_keep<0xB1>(v));
  v = min(v, dpp_keep<0x4E>(v));
  v = min(v, dpp_keep<0x141>(v));
  v = min(v, dpp_keep<0x140>(v));
  v = min(v, dpp_keep<0x142, 0xa>(v));
  v = min(v, dpp_keep<0x143, 0xc>(v));
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float wave_max_all(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
  return v;
}

// ---------------------------------------------------------------------------
// activation bytes met by one 16-byte chunk of a packed row, in field order
// (8-bit weights: 16 bytes, 4-bit: 32, 2-bit: 64)
// ---------------------------------------------------------------------------
template <int BITS>
struct ActChunk {
  static constexpr int kDw = QFmt<BITS>::kEpc / 4;
  uint32_t d[kDw];
};

template <int BITS>
__device__ __forceinline__ void act_chunk_from(const uint4 *v, ActChunk<BITS> &o, int &bytesum) {
  constexpr int EPC = QFmt<BITS>::kEpc;
  bytesum = 0;
#pragma unroll
  for (int u = 0; u < EPC / 16; ++u) {
    const uint4 x = v[u];
    const int ones = 0x01010101;
    bytesum = sdot4((int)x.x, ones, bytesum);
    bytesum = sdot4((int)x.y, ones, bytesum);
    bytesum = sdot4((int)x.z, ones, bytesum);
    bytesum = sdot4((int)x.w, ones, bytesum);
    if constexpr (BITS == 4) {
      act_order_q4(x.x, x.y, o.d[4 * u + 0], o.d[4 * u + 1]);
      act_order_q4(x.z, x.w, o.d[4 * u + 2], o.d[4 * u + 3]);
    } else if constexpr (BITS == 2) {
      const uint32_t in[4] = {x.x, x.y, x.z, x.w};
      uint32_t out[4];
      act_order_q2(in, out);
#pragma unroll
      for (int j = 0; j < 4; ++j) o.d[4 * u + j] = out[j];
    } else {
      o.d[0] = x.x;
      o.d[1] = x.y;
      o.d[2] = x.z;
      o.d[3] = x.w;
    }
  }
}

// Load the chunk's activation bytes (row of int8, chunk index c) and order them.
template <int BITS>
__device__ __forceinline__ void load_act_chunk(const int8_t *row, int c, ActChunk<BITS> &o, int &bytesum) {
  constexpr int EPC = QFmt<BITS>::kEpc;
  uint4 v[EPC / 16];
  const int8_t *p = row + (int64_t)c * EPC;
#pragma unroll
  for (int u = 0; u < EPC / 16; ++u) v[u] = ldg16(p, u);
  act_chunk_from<BITS>(v, o, bytesum);
}

template <int BITS>
__device__ __forceinline__ void zero_chunk(ActChunk<BITS> &o) {
#pragma unroll
  for (int q = 0; q < ActChunk<BITS>::kDw; ++q) o.d[q] = 0;
}

// sum over the chunk of code(w) * x, codes still offset (q + kOff)
template <int BITS>
__device__ __forceinline__ int dot_regs(uint4 w, const ActChunk<BITS> &x, int acc) {
  if constexpr (BITS == 8) {
    acc = sdot4((int)w.x, (int)x.d[0], acc);
    acc = sdot4((int)w.y, (int)x.d[1], acc);
    acc = sdot4((int)w.z, (int)x.d[2], acc);
    return sdot4((int)w.w, (int)x.d[3], acc);
  } else if constexpr (BITS == 4) {
    constexpr uint32_t M = 0x0f0f0f0fu;
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc = sdot4((int)(wd[m] & M), (int)x.d[2 * m], acc);
      acc = sdot4((int)((wd[m] >> 4) & M), (int)x.d[2 * m + 1], acc);
    }
    return acc;
  } else {
    constexpr uint32_t M = 0x03030303u;
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc = sdot4((int)(wd[m] & M), (int)x.d[4 * m + 0], acc);
      acc = sdot4((int)((wd[m] >> 2) & M), (int)x.d[4 * m + 1], acc);
      acc = sdot4((int)((wd[m] >> 4) & M), (int)x.d[4 * m + 2], acc);
      acc = sdot4((int)((wd[m] >> 6) & M), (int)x.d[4 * m + 3], acc);
    }
    return acc;
  }
}

// chunks per lane (ceil) of a packed row of n elements
__host__ __device__ constexpr int moe_chunks_per_lane(int n, int bits) {
  return (n * bits / 8 / 16 + MOE_WAVE - 1) / MOE_WAVE;
}

// ---------------------------------------------------------------------------
// top-k selection by one wave (router)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Order-preserving integer image of a float: a > b as floats (no NaN, no -0)
// if and only if key_bits(a) > key_bits(b) as signed integers.
__device__ __forceinline__ int key_bits(float f) {
  const int i = __float_as_int(f);
  return i ^ ((i >> 31) & 0x7fffffff);
}
// wave-uniform maximum of an int (DPP; lanes of masked rows keep their value)
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, dpp_keep<0xB1>(v));
  v = max(v, dpp_keep<0x4E>(v));
  v = max(v, dpp_keep<0x141>(v));
  v = max(v, dpp_keep<0x140>(v));
  v = max(v, dpp_keep<0x142, 0xa>(v));
  v = max(v, dpp_keep<0x143, 0xc>(v));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int64_t cat_key(int kb, int id) {
  return (int64_t)(((uint64_t)(uint32_t)kb << 32) | (uint32_t)~id);
}
__device__ __forceinline__ void cex(int64_t &a, int64_t &b) {  // (a, b) <- (max, min)
  const bool sw = b > a;
  const int64_t t = a;
  a = sw ? b : a;
  b = sw ? t : b;
}

// Top-k over the keys in LDS (descending key, then ascending id), run by one
// wave; lane r < k returns the id of rank r. Lane l holds keys l*4 .. l*4+3
// (E <= 256) as 64-bit (key, ~id) entries sorted in descending order, so
// every lane's head is its best and, since lanes hold ascending id ranges,
// the lowest lane whose head equals the wave maximum holds the lowest id among
// equal keys. Each round takes that head and shifts the winner's list.
__device__ __forceinline__ int wave_topk4(const float *key_s, int E, int k, int lane) {
  constexpr int64_t kNone = INT64_MIN;
  int64_t h[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane * 4 + m;
    h[m] = e < E ? cat_key(key_bits(key_s[e]), e) : kNone;
  }
  cex(h[0], h[1]);
  cex(h[2], h[3]);
  cex(h[0], h[2]);
  cex(h[1], h[3]);
  cex(h[1], h[2]);
  int my_id = 0;
  for (int r = 0; r < k; ++r) {
    const int hk = (int)(h[0] >> 32);
    const int wm = wave_max_i32(hk);
    const uint64_t mask = __ballot(hk == wm);
    const int wl = (int)__builtin_ctzll(mask);
    const int id = ~__builtin_amdgcn_readlane((int)(uint32_t)h[0], wl);
    if (lane == r) my_id = id;
    if (lane == wl) {
      h[0] = h[1];
      h[1] = h[2];
      h[2] = h[3];
      h[3] = kNone;
    }
  }
  return my_id;
}
// The same for E <= 1024: 16 keys per lane, each round recomputes the lane's
// best among the keys not yet taken.
__device__ __forceinline__ int wave_topk16(const float *key_s, int E, int k, int lane) {
  constexpr int64_t kNone = INT64_MIN;
  int64_t h[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int e = lane * 16 + m;
    h[m] = e < E ? cat_key(key_bits(key_s[e]), e) : kNone;
  }
  int my_id = 0;
  for (int r = 0; r < k; ++r) {
    int64_t best = h[0];
#pragma unroll
    for (int m = 1; m < 16; ++m) best = h[m] > best ? h[m] : best;
    const int hk = (int)(best >> 32);
    const int wm = wave_max_i32(hk);
    const uint64_t mask = __ballot(hk == wm);
    const int wl = (int)__builtin_ctzll(mask);
    const int id = ~__builtin_amdgcn_readlane((int)(uint32_t)best, wl);
    if (lane == r) my_id = id;
    if (lane == wl) {
#pragma unroll
      for (int m = 0; m < 16; ++m) h[m] = h[m] == best ? kNone : h[m];
    }
  }
  return my_id;
}

// Top-p truncation (agentlenshq.com, "Colibri: running GLM-5.2 744B MoE on
// consumer hardware", the --topp setting): lane j < k holds the sigmoid of the
// rank-j expert, sum their total. In rank order the normalised weights
// sig_j / sum accumulate in fp32; returns the length of the shortest prefix
// whose cumulative weight reaches top_p (k if none does, or top_p <= 0) and
// sets kept to the sum of the kept sigmoids in rank order. Wave-uniform.
__device__ __forceinline__ int topp_keep(float my_sig, float sum, int k, float top_p, float &kept) {
  int keep = k;
  if (top_p > 0.0f) {
    float cum = 0.0f;
    for (int j = 0; j < k; ++j) {
      cum += readlane_f(my_sig, j) / sum;
      if (cum >= top_p) {
        keep = j + 1;
        break;
      }
    }
  }
  kept = 0.0f;
  for (int j = 0; j < keep; ++j) kept += readlane_f(my_sig, j);
  return keep;
}
