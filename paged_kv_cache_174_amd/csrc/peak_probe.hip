// Measured peaks of this GPU, for stating the attention kernels' fractions
// against what the chip sustains as well as against the vendor figures:
//   * the bf16 matrix-core rate: every SIMD issuing independent
//     v_mfma_f32_32x32x16_bf16 back to back (four accumulator chains per wave,
//     so no product waits for the one before it);
//   * the HBM read rate: a read of a large buffer, each workgroup its own
//     contiguous chunk, 16 bytes per lane and eight loads in flight.
// Neither is part of the attention path; bench.py times them with events.
#include "mfma_util.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

using namespace mx;

__global__ __launch_bounds__(256) void mfma_probe_kernel(int64_t iters, float* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(1e-3f * static_cast<float>((threadIdx.x + i) & 7));
    b[i] = static_cast<__bf16>(1e-3f * static_cast<float>((threadIdx.x * 3 + i) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t i = 0; i < iters; ++i) {
    c0 = mfma(a, b, c0);
    c1 = mfma(a, b, c1);
    c2 = mfma(a, b, c2);
    c3 = mfma(a, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void stream_probe_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                           u32x4* __restrict__ sink) {
  // Each workgroup reads its own contiguous chunk, eight 16-byte loads in
  // flight per lane.
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t hi = min(lo + per, n16);
  u32x4 acc = {0u, 0u, 0u, 0u};
  constexpr int kUnroll = 8;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256 * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = i + 256 * u < hi ? src[i + 256 * u] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  // (a store that depends on every loaded value keeps the loads)
  if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u) sink[threadIdx.x] = acc;
}

}  // namespace

}  // namespace pkv

extern "C" {

int pkv_probe_mfma(int64_t iters, void* sink, int64_t sink_floats, int64_t* out_flop, void* stream) {
  using namespace pkv;
  if (iters <= 0 || !sink || !out_flop) return fail(PKV_EINVAL, "pkv_probe_mfma: need iters > 0, sink and out_flop");
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(PKV_EHIP, "pkv_probe_mfma: no device");
  const int64_t blocks = 2 * static_cast<int64_t>(cus);  // two waves per SIMD
  if (sink_floats < blocks * 256) return fail(PKV_EINVAL, "pkv_probe_mfma: sink needs %lld floats", static_cast<long long>(blocks * 256));
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, static_cast<float*>(sink));
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return fail(PKV_EHIP, "pkv_probe_mfma: %s", hipGetErrorString(e));
  *out_flop = blocks * 4 /* waves */ * iters * 4 /* chains */ * (32LL * 32 * 16 * 2);
  return PKV_OK;
}

int pkv_probe_stream(const void* src, int64_t bytes, void* sink, void* stream) {
  using namespace pkv;
  if (!src || !sink || bytes < 16 || bytes % 16) return fail(PKV_EINVAL, "pkv_probe_stream: need src, sink and a multiple of 16 bytes");
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(PKV_EHIP, "pkv_probe_stream: no device");
  hipLaunchKernelGGL(stream_probe_kernel, dim3(static_cast<unsigned>(8 * cus)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const mx::u32x4*>(src), bytes / 16,
                     static_cast<mx::u32x4*>(sink));
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return fail(PKV_EHIP, "pkv_probe_stream: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // extern "C"
