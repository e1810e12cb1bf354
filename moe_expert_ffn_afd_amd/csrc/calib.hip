// calib.hip -- measurement helper: the MFMA rate this GPU sustains with no
// memory traffic at all, and the shader clock it runs at meanwhile.  That is
// the ceiling the grouped GEMMs' MFMA fractions are read against (the spec
// peaks assume the full 2.4 GHz; under sustained MFMA load the clock drops).
//
// Every wave keeps NC independent accumulator chains of one MFMA kind busy for
// `iters` rounds: 8 waves per CU (two per SIMD), operands in registers, no
// loads or stores in the loop.  Thread 0 of each workgroup reads the shader
// clock counter (s_memtime) and the constant 100 MHz counter (s_memrealtime)
// around the loop, so their ratio gives the clock the loop ran at.
#include <vector>

#include "afd_device.h"

namespace afd {

using namespace dev;

template <int KIND>  // 0: bf16 32x32x16, 1: e4m3 16x16x128 (block-scaled kind), 2: int8 16x16x64
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* sink, unsigned long long* clocks) {
  const int lane = threadIdx.x & 63;
  unsigned long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  float s = 0.0f;
  if constexpr (KIND == 0) {
    constexpr int NC = 4;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.001f * (lane + i));
      b[i] = (__bf16)(0.002f * (lane - i));
    }
    f32x16 c[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) c[j][r] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < NC; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += c[j][r];
  } else if constexpr (KIND == 1) {
    constexpr int NC = 8;
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x38383838 + lane;  // small e4m3 codes
      b[i] = 0x30303030 + i;
    }
    f32x4 c[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) c[j][r] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < NC; ++j)
        c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[j], 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) s += c[j][r];
  } else {
    constexpr int NC = 8;
    i32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = 0x01010101 * ((lane + i) & 7);
      b[i] = 0x01010101 * (i + 1);
    }
    i32x4 c[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) c[j][r] = 0;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < NC; ++j) c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) s += (float)c[j][r];
  }
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - t0;
    clocks[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
  if (s == 1234.5f) sink[0] = s;  // keeps every product live
}

// flops of one wave's round of the loop
static double round_flops(int kind) {
  return kind == 0 ? 4.0 * 32 * 32 * 16 * 2 : kind == 1 ? 8.0 * 16 * 16 * 128 * 2 : 8.0 * 16 * 16 * 64 * 2;
}

hipError_t mfma_peak(int kind, int num_cus, int iters, double* tflops, double* clock_ghz) {
  const int blocks = 2 * num_cus;  // 8 waves per CU
  float* sink = nullptr;
  unsigned long long* clk = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc((void**)&sink, 4);
  if (e == hipSuccess) e = hipMalloc((void**)&clk, sizeof(unsigned long long) * 2 * blocks);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  std::vector<unsigned long long> host(2 * blocks);
  float ms = 0.0f;
  if (e == hipSuccess) {
    auto launch = [&](int n) {
      if (kind == 0)
        hipLaunchKernelGGL(mfma_peak_kernel<0>, dim3(blocks), dim3(256), 0, 0, n, sink, clk);
      else if (kind == 1)
        hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(blocks), dim3(256), 0, 0, n, sink, clk);
      else
        hipLaunchKernelGGL(mfma_peak_kernel<2>, dim3(blocks), dim3(256), 0, 0, n, sink, clk);
    };
    launch(iters / 8 + 1);  // warm-up (clocks ramp up)
    e = hipEventRecord(e0, 0);
    if (e == hipSuccess) launch(iters);
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess) e = hipMemcpy(host.data(), clk, host.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost);
  }
  if (e == hipSuccess) {
    const double waves = 4.0 * blocks;
    *tflops = waves * iters * round_flops(kind) / (ms * 1e-3) / 1e12;
    double ratio = 0.0;
    for (int b = 0; b < blocks; ++b) ratio += host[2 * b + 1] ? (double)host[2 * b] / (double)host[2 * b + 1] : 0.0;
    *clock_ghz = ratio / blocks * 0.1;  // s_memrealtime ticks at 100 MHz
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (sink) (void)hipFree(sink);
  if (clk) (void)hipFree(clk);
  return e;
}

}  // namespace afd
