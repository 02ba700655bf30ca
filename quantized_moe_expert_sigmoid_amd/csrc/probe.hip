// Streaming-read probe: the HBM read bandwidth a plain, well-formed kernel
// reaches on this device when it reads a given number of bytes in one launch.
// It is the measured ceiling the weight-streaming kernels are compared with
// (beside the data-sheet peak): a launch of a few tens of MB pays the same
// ramp-up and drain as they do.
//
// Each launch reads one window of the caller's buffer; successive launches
// take successive windows, so with a buffer larger than the last-level cache
// every launch reads cold data. Each thread XORs the dwords it reads (16-byte
// loads, four in flight, grid-stride over the window); each workgroup writes
// one dword, and the host folds them, so a test can check that every byte of
// the window was read. The loads carry the non-temporal hint, as the weight
// streams do (a plain load reads 7-13% slower here).
#include <vector>

#include "gemv_common.h"

namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint8_t *base, int64_t n16, uint32_t *sink) {
  const moe_u32x4 *p = reinterpret_cast<const moe_u32x4 *>(base);
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const moe_u32x4 a = __builtin_nontemporal_load(gptr(p) + i);
    const moe_u32x4 b = __builtin_nontemporal_load(gptr(p) + i + stride);
    const moe_u32x4 c = __builtin_nontemporal_load(gptr(p) + i + 2 * stride);
    const moe_u32x4 d = __builtin_nontemporal_load(gptr(p) + i + 3 * stride);
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const moe_u32x4 a = __builtin_nontemporal_load(gptr(p) + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, MOE_WAVE);
  __shared__ uint32_t red[kProbeThreads / MOE_WAVE];
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x / MOE_WAVE;
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / MOE_WAVE; ++w) v ^= red[w];
    sink[blockIdx.x] = v;
  }
}

}  // namespace

extern "C" moe_status moe_probe_stream_read(moe_ctx *ctx, const void *buf, size_t buf_bytes, size_t bytes_per_launch,
                                            int wg_per_cu, int reps, uint32_t *xor_host, double *us_host) {
  if (!ctx || !buf) return moe_fail(MOE_EINVAL, "moe_probe_stream_read: NULL argument");
  if (!moe_aligned16(buf) || bytes_per_launch == 0 || bytes_per_launch % 16 || bytes_per_launch > buf_bytes ||
      bytes_per_launch / 16 > (size_t)INT64_MAX / 4)
    return moe_fail(MOE_EINVAL, "moe_probe_stream_read: buffer %p of %zu bytes, %zu bytes per launch (a positive "
                    "multiple of 16, at most the buffer, 16-byte aligned)", buf, buf_bytes, bytes_per_launch);
  if (wg_per_cu < 1 || wg_per_cu > 64 || reps < 1 || reps > 100000)
    return moe_fail(MOE_EINVAL, "moe_probe_stream_read: wg_per_cu %d reps %d", wg_per_cu, reps);
  MOE_HIP(hipSetDevice(ctx->device));
  const int nwg = ctx->n_cu * wg_per_cu;
  void *scr = nullptr;
  moe_status st = moe_scratch(ctx, sizeof(uint32_t) * (size_t)nwg, &scr);
  if (st) return st;
  uint32_t *sink = static_cast<uint32_t *>(scr);
  const size_t n_windows = buf_bytes / bytes_per_launch;
  std::vector<hipEvent_t> ev(2 * (size_t)reps, nullptr);
  auto cleanup = [&]() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
  };
  for (auto &e : ev) {
    const hipError_t he = hipEventCreate(&e);
    if (he != hipSuccess) {
      cleanup();
      return moe_hip_fail(he, "hipEventCreate");
    }
  }
  for (int r = 0; r < reps; ++r) {
    const uint8_t *w = static_cast<const uint8_t *>(buf) + (size_t)(r % n_windows) * bytes_per_launch;
    hipExtLaunchKernelGGL(stream_read_kernel, dim3(nwg), dim3(kProbeThreads), 0, ctx->stream, ev[2 * r],
                          ev[2 * r + 1], 0, w, (int64_t)(bytes_per_launch / 16), sink);
    const hipError_t he = hipGetLastError();
    if (he != hipSuccess) {
      cleanup();
      return moe_hip_fail(he, "stream_read_kernel");
    }
  }
  std::vector<uint32_t> h((size_t)nwg);
  hipError_t he = hipMemcpyAsync(h.data(), sink, sizeof(uint32_t) * (size_t)nwg, hipMemcpyDeviceToHost, ctx->stream);
  if (he == hipSuccess) he = hipStreamSynchronize(ctx->stream);
  double total_ms = 0.0;
  for (int r = 0; r < reps && he == hipSuccess; ++r) {
    float ms = 0.0f;
    he = hipEventElapsedTime(&ms, ev[2 * r], ev[2 * r + 1]);
    total_ms += ms;
  }
  cleanup();
  if (he != hipSuccess) return moe_hip_fail(he, "moe_probe_stream_read");
  uint32_t x = 0;
  for (uint32_t v : h) x ^= v;
  if (xor_host) *xor_host = x;
  if (us_host) *us_host = total_ms * 1e3 / reps;
  return MOE_OK;
}
