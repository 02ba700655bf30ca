// Per-row symmetric quantisation and packing (int8 / int4 / int2) and the
// per-token int8 activation quantisation.
//
// agentlenshq.com, "Colibri: running GLM-5.2 744B MoE on consumer hardware",
// section "Key features": int8, packed int4 and packed int2 kernels with
// per-row scales; int8 matmuls as integer dot products (int8 operands).
//
// One workgroup per row: a float4 pass for max|w|, then a pass that writes
// one packed dword per thread and step. Divisions are IEEE fp32 divisions
// (the library is compiled without fast-math), rint rounds half to even.
#include "moe_internal.h"

namespace {

constexpr int kQThreads = 256;

template <int BITS>
__global__ __launch_bounds__(kQThreads) void quantize_rows_kernel(const float *__restrict__ w, int cols,
                                                                  uint8_t *__restrict__ packed,
                                                                  float *__restrict__ scales) {
  constexpr int kQmax = (1 << (BITS - 1)) - 1;
  constexpr int kEpd = 32 / BITS;  // elements per packed dword
  const int64_t row = blockIdx.x;
  const float *wr = w + row * (int64_t)cols;
  __shared__ float red[kQThreads / MOE_WAVE];

  float m = 0.0f;
  for (int c = threadIdx.x * 4; c < cols; c += kQThreads * 4) {
    const float4 v = *reinterpret_cast<const float4 *>(wr + c);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  m = wave_max_f32(m);
  if ((threadIdx.x & (MOE_WAVE - 1)) == 0) red[threadIdx.x / MOE_WAVE] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < kQThreads / MOE_WAVE; ++i) m = fmaxf(m, red[i]);

  const float qmax = (float)kQmax;
  const float s = (m == 0.0f) ? 0.0f : m / qmax;
  if (threadIdx.x == 0) scales[row] = s;

  const int ndw = cols / kEpd;
  uint32_t *dst = reinterpret_cast<uint32_t *>(packed + row * (int64_t)(cols * BITS / 8));
  for (int d = threadIdx.x; d < ndw; d += kQThreads) {
    uint32_t word = 0;
#pragma unroll
    for (int j4 = 0; j4 < kEpd; j4 += 4) {
      const float4 v4 = *reinterpret_cast<const float4 *>(wr + (int64_t)d * kEpd + j4);
      const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        int q = 0;
        if (m != 0.0f) {
          float r = __builtin_rintf(vv[jj] / s);
          r = fminf(fmaxf(r, -qmax), qmax);
          q = (int)r;
        }
        const uint32_t field = (BITS == 8) ? (uint32_t)(uint8_t)(int8_t)q : (uint32_t)(q + kQmax + 1);
        word |= field << ((j4 + jj) * BITS);
      }
    }
    dst[d] = word;
  }
}

template <int BITS>
moe_status launch_q(moe_ctx *ctx, const float *w, int64_t rows, int cols, uint8_t *packed, float *scales) {
  hipLaunchKernelGGL(quantize_rows_kernel<BITS>, dim3((unsigned)rows), dim3(kQThreads), 0, ctx->stream, w, cols,
                     packed, scales);
  MOE_CHECK_LAUNCH("quantize_rows_kernel");
  return MOE_OK;
}

// The activation rule on one token per workgroup, with the whole row held in
// registers: every load is issued before the first is used (the generic
// kernel above walks the row twice, one dependent load after another), then
// the same max, scale and per-element rounding. H <= kActMaxH, H % 4 == 0.
constexpr int kActMaxH = 8192;
constexpr int kActSteps = kActMaxH / (4 * kQThreads);

__global__ __launch_bounds__(kQThreads) void quantize_act_kernel(const float *__restrict__ x, int H,
                                                                 int8_t *__restrict__ xq, float *__restrict__ sx) {
  const int64_t t = blockIdx.x;
  const float4 *xr = reinterpret_cast<const float4 *>(x + t * (int64_t)H);
  const int n4 = H / 4;
  __shared__ float red[kQThreads / MOE_WAVE];
  float4 v[kActSteps];
#pragma unroll
  for (int i = 0; i < kActSteps; ++i) {
    const int c = threadIdx.x + i * kQThreads;
    v[i] = c < n4 ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < kActSteps; ++i)
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
  m = wave_max_f32(m);
  if ((threadIdx.x & (MOE_WAVE - 1)) == 0) red[threadIdx.x / MOE_WAVE] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < kQThreads / MOE_WAVE; ++i) m = fmaxf(m, red[i]);
  const float s = (m == 0.0f) ? 0.0f : m / 127.0f;
  if (threadIdx.x == 0) sx[t] = s;
  uint32_t *dst = reinterpret_cast<uint32_t *>(xq + t * (int64_t)H);
#pragma unroll
  for (int i = 0; i < kActSteps; ++i) {
    const int c = threadIdx.x + i * kQThreads;
    if (c >= n4) break;
    const float vv[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int q = 0;
      if (m != 0.0f) {
        float r = __builtin_rintf(vv[j] / s);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        q = (int)r;
      }
      word |= (uint32_t)(uint8_t)(int8_t)q << (8 * j);
    }
    dst[c] = word;
  }
}

}  // namespace

moe_status launch_quantize_rows(moe_ctx *ctx, int bits, const float *w, int64_t rows, int cols, uint8_t *packed,
                                float *scales) {
  switch (bits) {
    case 8: return launch_q<8>(ctx, w, rows, cols, packed, scales);
    case 4: return launch_q<4>(ctx, w, rows, cols, packed, scales);
    default: return launch_q<2>(ctx, w, rows, cols, packed, scales);
  }
}

// The activation rule is the 8-bit row rule applied per token.
moe_status launch_quantize_act(moe_ctx *ctx, const float *x, int T, int H, int8_t *xq, float *sx) {
  MoeTimer tm_(ctx, MOE_STAGE_ROUTER);
  if (H > kActMaxH || H % 4) return launch_q<8>(ctx, x, T, H, reinterpret_cast<uint8_t *>(xq), sx);
  hipLaunchKernelGGL(quantize_act_kernel, dim3((unsigned)T), dim3(kQThreads), 0, ctx->stream, x, H, xq, sx);
  MOE_CHECK_LAUNCH("quantize_act_kernel");
  return MOE_OK;
}
