// Weighted combine of the routed experts' outputs with the shared expert.
//
// remio.ai, "Colibri shows how to run GLM-5.2 on a low-spec PC", section "How
// Colibri runs GLM-5.2" (the layer output mixes the few experts the router
// chose); agentlenshq.com "Colibri ...", section "Memory split" (the shared
// expert is always applied). out[t] = y_shared[t] + sum_j w[t,j] * y_j[t],
// fp32 fused multiply-adds in slot order; one float4 per thread.
#include "moe_internal.h"

namespace {

constexpr int kMaxK = 16;  // the largest top-k the entry points accept

// Every slot's float4 is loaded before the first multiply-add (a loop bounded
// by the runtime k would issue them one at a time); the multiply-adds then
// run in slot order. A slot of weight 0 (dropped by top-p) is loaded but not
// used: its y may never have been written.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y, const float *__restrict__ w, int T,
                                                      int k, int H, int has_shared, float *__restrict__ out) {
  const int h4 = H / 4;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int t = (int)(q / h4);
  if (t >= T) return;
  const int hh = (int)(q - (int64_t)t * h4) * 4;
  const float *ys = y + (int64_t)t * (k + 1) * H;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (has_shared) acc = *reinterpret_cast<const float4 *>(ys + (int64_t)k * H + hh);
  float wv[kMaxK];
  float4 v[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) {
      wv[j] = w[(int64_t)t * k + j];
      v[j] = *reinterpret_cast<const float4 *>(ys + (int64_t)j * H + hh);
    }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    // fma(0, y, acc) = acc for finite y; a dropped slot's y is not used
    if (j >= k || wv[j] == 0.0f) continue;
    acc.x = __builtin_fmaf(wv[j], v[j].x, acc.x);
    acc.y = __builtin_fmaf(wv[j], v[j].y, acc.y);
    acc.z = __builtin_fmaf(wv[j], v[j].z, acc.z);
    acc.w = __builtin_fmaf(wv[j], v[j].w, acc.w);
  }
  *reinterpret_cast<float4 *>(out + (int64_t)t * H + hh) = acc;
}

}  // namespace

moe_status launch_combine(moe_ctx *ctx, const float *y_slots, const float *topk_w, int T, int k, int H,
                          int has_shared, float *out) {
  const int64_t n4 = (int64_t)T * (H / 4);
  {
    MoeTimer tm_(ctx, MOE_STAGE_COMBINE);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, ctx->stream, y_slots, topk_w,
                       T, k, H, has_shared, out);
  }
  MOE_CHECK_LAUNCH("combine_kernel");
  return MOE_OK;
}
