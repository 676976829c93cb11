// MFMA throughput probe (gfx950): the bf16 MFMA rate the chip sustains with
// no memory traffic, and the shader clock it runs at meanwhile.  A measuring
// instrument for the benchmark's roofline, not part of the attention library.
//
// Every wave issues `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 (the instruction the attention kernels use) on
// register operands; two workgroups of four waves per compute unit keep each
// SIMD's matrix pipe fed.  Wave 0 of each workgroup reads the shader clock
// counter (clock64) and the constant-rate wall clock (wall_clock64) around its
// loop, so the clock the chip ran at follows from their ratio.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* sink,
                                                        long long* clocks) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(lane + i));
    b[i] = (__bf16)(1e-3f * (float)(lane - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  long long t0 = 0, w0 = 0;
  if (threadIdx.x == 0) {
    t0 = clock64();
    w0 = wall_clock64();
  }
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + 0] = clock64() - t0;
    clocks[4 * blockIdx.x + 1] = wall_clock64() - w0;
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[blockIdx.x * 256 + threadIdx.x] = s;  // keeps the products alive
}

}  // namespace

extern "C" {

// Runs the probe on the current device: `iters` rounds per wave, 2 workgroups
// per compute unit.  Outputs: dense bf16 MFMA TFLOP/s achieved, the mean
// shader clock in MHz over the loop, the kernel time in ms (HIP events).
// Returns 0 on success, else the HIP error code.
int nomas_probe_mfma(int iters, double* tflops, double* clock_mhz, double* ms) {
  int dev = 0, cus = 0, wall_khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return (int)e;
  const int blocks = 2 * cus;
  float* sink = nullptr;
  long long* clocks = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if ((e = hipMalloc(&sink, sizeof(float) * 256 * blocks)) != hipSuccess) return (int)e;
  if ((e = hipMalloc(&clocks, sizeof(long long) * 4 * blocks)) != hipSuccess) {
    (void)hipFree(sink);
    return (int)e;
  }
  long long* host = new long long[4 * blocks];
  float t = 0.f;
  e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, 0, iters / 8, sink, clocks);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e0, 0);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, 0, iters, sink, clocks);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, 0);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(&t, e0, e1);
  if (e == hipSuccess)
    e = hipMemcpy(host, clocks, sizeof(long long) * 4 * blocks, hipMemcpyDeviceToHost);
  if (e == hipSuccess) {
    double cyc = 0, wall = 0;
    for (int b = 0; b < blocks; ++b) {
      cyc += (double)host[4 * b];
      wall += (double)host[4 * b + 1];
    }
    const double flops = (double)blocks * 4 /*waves*/ * iters * 4 /*MFMAs*/ * 32.0 * 32.0 * 16.0 * 2.0;
    *ms = t;
    *tflops = flops / (t * 1e-3) / 1e12;
    *clock_mhz = wall > 0 ? cyc / wall * (wall_khz * 1e-3) : 0.0;
  }
  delete[] host;
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(sink);
  (void)hipFree(clocks);
  return (int)e;
}

}  // extern "C"
