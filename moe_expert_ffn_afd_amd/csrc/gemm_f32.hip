// gemm_f32.hip -- grouped expert GEMMs in plain fp32 (the fp32 layer variant).
//
// Same two GEMMs and m-tile list as the MFMA path (gate/up with SwiGLU, then
// down), computed with fp32 FMAs for full single precision.  A workgroup task
// is one m-tile (<= 32 rows of one expert) times 64 output columns; its four
// waves split each 64-deep slice of the reduction into four 16-deep parts
// (lane = column, so a wave's weight reads are coalesced along N in the
// original [K, N] row-major layout), with the tile's activation rows staged
// through LDS.  The four partial sums are added in a fixed order at the end,
// so the result does not depend on scheduling.
#include "afd_internal.h"

namespace afd {

template <bool GATEUP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(F32Params p) {
  constexpr int BM = 32, KC = 64, NC = 64, KS = 4;  // rows, slice depth, columns, reduction parts
  constexpr int NACC = GATEUP ? 2 : 1;
  __shared__ float as[BM][KC];
  __shared__ float red[NACC][KS - 1][BM][NC];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int ks = __builtin_amdgcn_readfirstlane(tid >> 6);  // reduction part of this wave
  const int num_mt = __builtin_amdgcn_readfirstlane(p.num_mtiles[0]);
  const int ngrp = (p.ndim + NC - 1) / NC;
  const int num_tasks = num_mt * ngrp;
  for (int task = blockIdx.x; task < num_tasks; task += gridDim.x) {
    const int mt = task % num_mt;
    const int q = task / num_mt;
    const int4 tile = p.mtiles[mt];
    const int e = tile.x, row0 = tile.y, rows = tile.z;
    const int n = q * NC + lane;
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
          if (p.gather) src = row >= p.shared_row0 ? (row - p.shared_row0) % p.shared_tokens : (p.sorted_assign[row] / p.top_k);
          v = p.a[src * p.kdim + k0 + kk];
        }
        as[r][kk] = v;
      }
      __syncthreads();
      if (ok) {
        const int kb = ks * (KC / KS);
        const int kend = min(kb + KC / KS, p.kdim - k0);
        float b0[KC / KS], b1[KC / KS];
#pragma unroll
        for (int i = 0; i < KC / KS; ++i) {  // the part's weight loads first
          const int kk = kb + i;
          b0[i] = kk < kend ? w0[(int64_t)(k0 + kk) * p.ndim + n] : 0.0f;
          b1[i] = GATEUP && kk < kend ? w1[(int64_t)(k0 + kk) * p.ndim + n] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < KC / KS; ++i) {
          const int kk = kb + i;
          if (kk >= kend) break;
#pragma unroll
          for (int r = 0; r < BM; ++r) {
            acc0[r] = fmaf(as[r][kk], b0[i], acc0[r]);
            if (GATEUP) acc1[r] = fmaf(as[r][kk], b1[i], acc1[r]);
          }
        }
      }
    }
    // fixed-order sum of the four parts: part 0 + part 1 + part 2 + part 3
    if (ks > 0) {
#pragma unroll
      for (int r = 0; r < BM; ++r) {
        red[0][ks - 1][r][lane] = acc0[r];
        if (GATEUP) red[NACC - 1][ks - 1][r][lane] = acc1[r];
      }
    }
    __syncthreads();
    if (ks == 0 && ok) {
#pragma unroll
      for (int r = 0; r < BM; ++r) {
        if (r < rows) {
          float v = acc0[r];
          float u = acc1[r];
#pragma unroll
          for (int j = 0; j < KS - 1; ++j) {
            v += red[0][j][r][lane];
            if (GATEUP) u += red[NACC - 1][j][r][lane];
          }
          if (GATEUP) v = v / (1.0f + expf(-v)) * u;
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
