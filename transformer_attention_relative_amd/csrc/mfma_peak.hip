// Measured peak of v_mfma_f32_32x32x16_bf16 on this device: the benchmark
// reports the fused kernels' rate against it as well as against the
// published dense peak.  Built as its own small library (libmfma_peak.so);
// not part of the relative-attention boundary.
//
// Every wave keeps eight independent accumulators, so the matrix cores
// never wait on a dependency; two four-wave workgroups per CU give each
// SIMD two waves, as in the attention kernels.
#include <hip/hip_runtime.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256, 2) void mfma_peak_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(e - lane));
  }
  f32x16 acc[8];
  for (int c = 0; c < 8; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
  for (int c = 0; c < 8; ++c)
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// Runs the probe on the current device and returns the sustained bf16 rate
// in TFLOP/s (dense, 2 flops per multiply-add), or a negative value on a HIP
// error.  `workgroups` workgroups of 256 threads, `iters` loop trips of 8
// MFMAs per wave.  Allocates and frees its own 4-byte-per-thread output.
extern "C" double mfma_peak_bf16_tflops(int workgroups, int iters) {
  if (workgroups < 1 || iters < 1) return -1.0;
  float* out = nullptr;
  const size_t n = (size_t)workgroups * 256;
  if (hipMalloc(&out, n * sizeof(float)) != hipSuccess) return -1.0;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  double result = -1.0;
  if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(workgroups), dim3(256), 0, 0, out, iters);  // warm-up
    hipEventRecord(e0, 0);
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(workgroups), dim3(256), 0, 0, out, iters);
    hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) == hipSuccess && hipGetLastError() == hipSuccess) {
      float ms = 0.f;
      hipEventElapsedTime(&ms, e0, e1);
      const double flops = (double)workgroups * 4 * iters * 8 * (32.0 * 32 * 16 * 2);
      if (ms > 0.f) result = flops / (ms * 1e-3) / 1e12;
    }
  }
  if (e0) hipEventDestroy(e0);
  if (e1) hipEventDestroy(e1);
  hipFree(out);
  return result;
}
