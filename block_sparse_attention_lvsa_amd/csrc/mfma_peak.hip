// Measured bf16 matrix-core peak of the GPU the benchmark runs on: a second
// denominator for the attention kernel's MFMA rate, next to the vendor's
// 2.5 PFLOP/s (which assumes the 2.4 GHz top engine clock).
//
// Every wave runs independent chains of v_mfma_f32_32x32x16_bf16 (the
// attention kernel's instruction) on register operands, no memory traffic,
// at the attention kernel's occupancy (3 waves per SIMD on every CU).  The
// rate is taken over launches after a warm-up, so the engine clock has
// settled to what this load alone draws; the clock is read from the shader
// cycle counter against the fixed 100 MHz real-time counter.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;          // independent accumulators per wave
constexpr int kWavesPerWg = 4;
constexpr int kWgPerCu = 3;         // 3 waves per SIMD, as the attention kernel

__global__ __launch_bounds__(kWavesPerWg * 64) void mfma_chains(int iters, float *sink, uint64_t *clocks) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(lane - e));
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16_t{};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = t1 - t0;
    clocks[1] = r1 - r0;
  }
}

}  // namespace

// Runs the chains for about `seconds` (after a warm-up of the same length)
// and reports the sustained dense bf16 MFMA rate in TFLOP/s and the mean
// engine clock in MHz over the timed launches.  Allocates and frees its own
// small device buffers (a benchmark helper, not part of the attention ABI).
// Returns 0, or a negative value on a HIP error.
extern "C" int lvsa_probe_mfma_peak(double seconds, double *tflops, double *mhz) {
  hipDeviceProp_t prop;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
  const int grid = prop.multiProcessorCount * kWgPerCu;
  float *sink = nullptr;
  uint64_t *clocks = nullptr;
  if (hipMalloc(&sink, sizeof(float) * grid * kWavesPerWg * 64) != hipSuccess) return -2;
  if (hipMalloc(&clocks, 2 * sizeof(uint64_t)) != hipSuccess) {
    (void)hipFree(sink);
    return -2;
  }
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  int rc = 0;
  // Calibrate the per-launch length on a short launch, then run ~20 ms
  // launches: a warm-up of `seconds`, then the timed ones.
  int iters = 2000;
  float ms = 0.f;
  hipLaunchKernelGGL(mfma_chains, dim3(grid), dim3(kWavesPerWg * 64), 0, 0, iters, sink, clocks);
  (void)hipEventRecord(e0, 0);
  hipLaunchKernelGGL(mfma_chains, dim3(grid), dim3(kWavesPerWg * 64), 0, 0, iters, sink, clocks);
  (void)hipEventRecord(e1, 0);
  if (hipEventSynchronize(e1) != hipSuccess) rc = -3;
  (void)hipEventElapsedTime(&ms, e0, e1);
  if (rc == 0 && ms > 0.f) {
    const double want = iters * 20.0 / ms;
    iters = want < 2000.0 ? 2000 : (want > 5e7 ? 50000000 : (int)want);
  }
  const int launches = seconds > 0 ? (int)(seconds * 1000.0 / 20.0) + 1 : 10;
  for (int i = 0; rc == 0 && i < launches; ++i)
    hipLaunchKernelGGL(mfma_chains, dim3(grid), dim3(kWavesPerWg * 64), 0, 0, iters, sink, clocks);
  double flops = 0.0, total_ms = 0.0, cycles = 0.0, real = 0.0;
  for (int i = 0; rc == 0 && i < launches; ++i) {
    (void)hipEventRecord(e0, 0);
    hipLaunchKernelGGL(mfma_chains, dim3(grid), dim3(kWavesPerWg * 64), 0, 0, iters, sink, clocks);
    (void)hipEventRecord(e1, 0);
    if (hipEventSynchronize(e1) != hipSuccess) {
      rc = -3;
      break;
    }
    (void)hipEventElapsedTime(&ms, e0, e1);
    uint64_t c[2] = {0, 0};
    if (hipMemcpy(c, clocks, sizeof c, hipMemcpyDeviceToHost) != hipSuccess) {
      rc = -3;
      break;
    }
    total_ms += ms;
    flops += (double)grid * kWavesPerWg * iters * kChains * (2.0 * 32 * 32 * 16);
    cycles += (double)c[0];
    real += (double)c[1];
  }
  if (rc == 0 && hipGetLastError() != hipSuccess) rc = -3;
  if (rc == 0) {
    *tflops = flops / (total_ms * 1e-3) / 1e12;
    *mhz = real > 0 ? cycles / (real / 100.0) : 0.0;  // memrealtime counts at 100 MHz
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipFree(sink);
  (void)hipFree(clocks);
  return rc;
}
