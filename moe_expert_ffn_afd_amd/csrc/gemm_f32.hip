// gemm_f32.hip -- grouped expert GEMMs in plain fp32 (the fp32 layer variant).
//
// Same two GEMMs and m-tile list as the MFMA path (gate/up with SwiGLU, then
// down), computed with fp32 FMAs for full single precision: a workgroup task
// is one m-tile (<= 32 rows of one expert) times 256 output columns, one
// column per thread, with the tile's activation rows staged through LDS in
// 128-deep slices.  Weights stay in their original [K, N] row-major layout,
// so a warp's weight reads are coalesced along N.
#include "afd_internal.h"

namespace afd {

template <bool GATEUP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(F32Params p) {
  constexpr int BM = 32, KC = 128;
  __shared__ float as[BM][KC];
  const int tid = threadIdx.x;
  const int num_mt = __builtin_amdgcn_readfirstlane(p.num_mtiles[0]);
  const int ngrp = (p.ndim + 255) / 256;
  const int num_tasks = num_mt * ngrp;
  for (int task = blockIdx.x; task < num_tasks; task += gridDim.x) {
    const int mt = task % num_mt;
    const int q = task / num_mt;
    const int4 tile = p.mtiles[mt];
    const int e = tile.x, row0 = tile.y, rows = tile.z;
    const int n = q * 256 + tid;
    const bool ok = n < p.ndim;
    const float* w0 = p.w0 + (int64_t)e * p.kdim * p.ndim;
    const float* w1 = GATEUP ? p.w1 + (int64_t)e * p.kdim * p.ndim : nullptr;
    float acc0[BM], acc1[BM];
#pragma unroll
    for (int r = 0; r < BM; ++r) acc0[r] = acc1[r] = 0.0f;
    for (int k0 = 0; k0 < p.kdim; k0 += KC) {
      __syncthreads();
      for (int i = tid; i < BM * KC; i += 256) {
        const int r = i / KC, kk = i % KC;
        float v = 0.0f;
        if (r < rows && k0 + kk < p.kdim) {
          const int row = row0 + r;
          int64_t src = row;
          if (p.gather) src = row >= p.shared_row0 ? (row - p.shared_row0) : (p.sorted_assign[row] / p.top_k);
          v = p.a[src * p.kdim + k0 + kk];
        }
        as[r][kk] = v;
      }
      __syncthreads();
      if (ok) {
        const int kend = min(KC, p.kdim - k0);
        for (int kk = 0; kk < kend; ++kk) {
          const float b0 = w0[(int64_t)(k0 + kk) * p.ndim + n];
          const float b1 = GATEUP ? w1[(int64_t)(k0 + kk) * p.ndim + n] : 0.0f;
#pragma unroll
          for (int r = 0; r < BM; ++r) {
            acc0[r] = fmaf(as[r][kk], b0, acc0[r]);
            if (GATEUP) acc1[r] = fmaf(as[r][kk], b1, acc1[r]);
          }
        }
      }
    }
    if (ok) {
#pragma unroll
      for (int r = 0; r < BM; ++r) {
        if (r < rows) {
          float v = acc0[r];
          if (GATEUP) v = v / (1.0f + expf(-v)) * acc1[r];
          p.c[(int64_t)(row0 + r) * p.ndim + n] = v;
        }
      }
    }
  }
}

hipError_t launch_gemm_f32(bool gate_up, const F32Params& p, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (gate_up)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace afd
