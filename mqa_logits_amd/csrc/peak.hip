// Matrix-core peak microbenchmark (measurement aid for bench.py, not part of
// the logits path): one wave per SIMD issues chains of the fp8
// v_mfma_scale_f32_16x16x128_f8f6f4 the logits kernels use, with 16
// independent accumulators per wave, and records its shader-clock cycles and
// real time so the caller gets both the achieved rate and the clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void mfma_peak_kernel(float* out, unsigned long long* clk, int iters) {
  const int l = threadIdx.x;
  v8i a[4], b;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 8; ++i) a[m][i] = 0x38383838 ^ (l << (i & 3)) ^ (m << 3);
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = 0x30303030 + i;
  v4f acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
  const long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(b));
#pragma unroll
    for (int m = 0; m < 16; ++m)
      acc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[m & 3], b, acc[m], 0, 0, 0,
                                                                112 + m, 0, 127);
  }
  const long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 16; ++m) s += acc[m][0] + acc[m][1] + acc[m][2] + acc[m][3];
  out[blockIdx.x * 64 + l] = s;
  if (l == 0) {
    clk[2 * blockIdx.x] = (unsigned long long)(c1 - c0);
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// Runs `waves` one-wave blocks of `iters` x 16 MFMAs on the current device and
// returns the achieved dense fp8 TFLOP/s (2 * 16 * 16 * 128 flops per MFMA over
// the event-timed kernel) and the mean shader clock in MHz (cycles over the
// 100 MHz real-time counter).  Returns 0, or a hipError_t value.
int mqa_measure_mfma_peak(int32_t waves, int32_t iters, double* tflops, double* sclk_mhz) {
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc(&out, (size_t)waves * 64 * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&clk, (size_t)waves * 2 * sizeof(unsigned long long));
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(waves), dim3(64), 0, 0, out, clk, iters);  // warm
    e = hipEventRecord(e0, 0);
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(waves), dim3(64), 0, 0, out, clk, iters);
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
  }
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e == hipSuccess) {
    unsigned long long* h = new unsigned long long[(size_t)waves * 2];
    e = hipMemcpy(h, clk, (size_t)waves * 2 * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    double cyc = 0, rt = 0;
    for (int i = 0; i < waves; ++i) { cyc += (double)h[2 * i]; rt += (double)h[2 * i + 1]; }
    delete[] h;
    const double flops = 2.0 * 16 * 16 * 128 * 16.0 * (double)iters * waves;
    *tflops = flops / (ms * 1e-3) / 1e12;
    *sclk_mhz = rt > 0 ? cyc / (rt * 10e-3) : 0.0;   // real-time ticks are 10 ns
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  if (clk) (void)hipFree(clk);
  return (int)e;
}

}  // extern "C"
