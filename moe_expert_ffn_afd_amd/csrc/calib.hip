// calib.hip -- measurement helper: the MFMA rate this GPU sustains with no
// memory traffic at all, and the shader clock it runs at meanwhile.  That is
// the ceiling the grouped GEMMs' MFMA fractions are read against (the spec
// peaks assume the full 2.4 GHz; under sustained MFMA load the clock drops).
// A second loop adds the LDS fragment reads of the LDS-tiled bf16 GEMM, for
// the ceiling of that kernel's own instruction mix.
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

// The LDS-tiled bf16 GEMM's inner loop (gemm_tiled.h) without its copies,
// barriers or epilogue: per step each wave reads six 16-byte fragments from
// LDS (two 32-row activation fragments and four weight-panel fragments, the
// share of one 16-deep k slice of a 64-row x 4-panel wave tile) and issues
// the eight 32x32x16 MFMAs they feed.  The next step's fragments are read
// before this step's MFMAs, into the third of three fragment buffers, so no
// read waits on an MFMA that uses its registers.  READS false: the same MFMAs
// on fragments read once before the loop.  The LDS holds bf16 values of
// random sign and mantissa bits (finite, the operand bits toggle as a GEMM's
// do), 256 threads and 32 KiB per workgroup, two workgroups per CU.
template <bool READS>
__global__ __launch_bounds__(256, 2) void mfma_lds_kernel(int iters, float* sink, unsigned long long* clocks) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[32768];
  for (int i = threadIdx.x; i < 8192; i += 256)
    reinterpret_cast<uint32_t*>(lds)[i] = (((uint32_t)i * 2654435761u) & 0x807f807fu) | 0x3c003c00u;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  f32x16 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[j][r] = 0.0f;
  bf16x8 f0[6], f1[6], f2[6];
  auto rd = [&](bf16x8 (&f)[6], int step) {
    const int o = step * 6144 + wave * 512 + lane * 16;
#pragma unroll
    for (int k = 0; k < 6; ++k) f[k] = *reinterpret_cast<const bf16x8*>(lds + ((o + k * 1024) & 32767));
  };
  auto mm = [&](const bf16x8 (&f)[6]) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) c[4 * a + b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[2 + b], f[a], c[4 * a + b], 0, 0, 0);
  };
  rd(f0, 0);
  if (!READS) {
    rd(f1, 1);
    rd(f2, 2);
  }
  for (int it = 0; it < iters; it += 3) {
    if (READS) rd(f1, it + 1);
    __builtin_amdgcn_sched_barrier(0);
    mm(f0);
    __builtin_amdgcn_sched_barrier(0);
    if (READS) rd(f2, it + 2);
    __builtin_amdgcn_sched_barrier(0);
    mm(f1);
    __builtin_amdgcn_sched_barrier(0);
    if (READS) rd(f0, it + 3);
    __builtin_amdgcn_sched_barrier(0);
    mm(f2);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - t0;
    clocks[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
  if (s == 1234.5f) sink[0] = s;
}

// flops of one wave's round of the loop
static double round_flops(int kind) {
  return kind == 0 ? 4.0 * 32 * 32 * 16 * 2
       : kind == 1 ? 8.0 * 16 * 16 * 128 * 2
       : kind == 2 ? 8.0 * 16 * 16 * 64 * 2
                   : 8.0 * 32 * 32 * 16 * 2;  // kinds 3 and 4: one step of mfma_lds_kernel
}

// kind 0 bf16, 1 e4m3, 2 int8 register chains; 3 and 4 mfma_lds_kernel
// without and with its LDS fragment reads
hipError_t mfma_peak(int kind, int num_cus, int iters, double* tflops, double* clock_ghz) {
  if (kind >= 3) iters -= iters % 3;  // mfma_lds_kernel runs steps in threes
  if (iters <= 0) return hipErrorInvalidValue;
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
      else if (kind == 2)
        hipLaunchKernelGGL(mfma_peak_kernel<2>, dim3(blocks), dim3(256), 0, 0, n, sink, clk);
      else if (kind == 3)
        hipLaunchKernelGGL(mfma_lds_kernel<false>, dim3(blocks), dim3(256), 0, 0, n, sink, clk);
      else
        hipLaunchKernelGGL(mfma_lds_kernel<true>, dim3(blocks), dim3(256), 0, 0, n, sink, clk);
    };
    launch(kind >= 3 ? (iters / 24 + 1) * 3 : iters / 8 + 1);  // warm-up (clocks ramp up)
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
