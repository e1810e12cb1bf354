// gemm_f32.hip -- grouped expert GEMMs in fp32 (the fp32 layer variant).
//
// Same two GEMMs and m-tile list as the bf16 and 8-bit paths (gate/up with
// SwiGLU, then down), on the fp32 matrix cores: MFMA 16x16x4 f32 takes fp32
// operands and accumulates in fp32, so nothing is rounded to a narrower type
// (a bf16 or tf32 downcast would show errors of 1e-3 and more).
//
// A workgroup task is one m-tile (<= 32 rows of one expert, two 16-row
// blocks) times 16 output columns.  Its four waves split the reduction into
// four contiguous quarters and each runs the MFMAs of its quarter for both row
// blocks (and, for gate/up, both the gate and the up columns); the quarters'
// partial sums meet in LDS and are added in a fixed order (quarter 0 + 1 + 2
// + 3), so the result does not depend on scheduling.
//
// MFMA operands: the weight fragment first, the token fragment second, so
// lane l = i + 16 j holds token i and output columns 4 j .. 4 j + 3 of the
// task's 16 (one 16-byte store per row).  The reduction index of a fragment
// is permuted (slot j of MFMA s takes k = 4 j + s of a 16-deep chunk): the
// sum over k does not care about its order, and the permutation lets each
// lane read its token's 4 consecutive k values with one 16-byte load, while
// the weight loads stay 64-byte runs along the output columns of the original
// [K, N] row-major layout.
#include "afd_device.h"

namespace afd {

using namespace dev;

template <bool GATEUP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(F32Params p) {
  constexpr int NC = 16, KW = 4;  // columns per task (of 32 rows), waves over the reduction
  constexpr int NACC = GATEUP ? 2 : 1;
  __shared__ f32x4 red[KW - 1][NACC][2][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, i16 = lane & 15, j4 = lane >> 4;
  const int wq = uniform(tid >> 6);  // this wave's quarter of the reduction
  const int num_mt = uniform(p.num_mtiles[0]);
  const int num_tasks = num_mt * (p.ndim / NC);
  const int kq = p.kdim / KW;  // a multiple of 32 (kdim is a multiple of 128)
  for (int task = blockIdx.x; task < num_tasks; task += gridDim.x) {
    const int mt = task % num_mt;
    const int n0 = (task / num_mt) * NC;
    const int4 tile = p.mtiles[mt];
    const int e = tile.x, row0 = tile.y, rows = tile.z;
    // this lane's token in each row block, and where its row starts
    const float* arow[2];
    bool aok[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = rb * 16 + i16;
      aok[rb] = r < rows;
      int64_t src = row0 + r;
      if (p.gather && aok[rb]) {
        const int row = row0 + r;
        src = row >= p.shared_row0 ? (row - p.shared_row0) % p.shared_tokens : p.sorted_assign[row] / p.top_k;
      }
      arow[rb] = p.a + (aok[rb] ? src : 0) * p.kdim;
    }
    const int64_t woff = (int64_t)e * p.kdim * p.ndim + n0 + i16;  // this lane's weight column
    const float* w0 = p.w0 + woff;
    const float* w1 = GATEUP ? p.w1 + woff : nullptr;
    f32x4 acc[NACC][2];
#pragma unroll
    for (int m = 0; m < NACC; ++m) acc[m][0] = acc[m][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int kb = wq * kq;
    for (int k = kb; k < kb + kq; k += 32) {  // two 16-deep chunks per round
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int kk = k + 16 * c + 4 * j4;
        f32x4 a[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          a[rb] = aok[rb] ? *reinterpret_cast<const f32x4*>(arow[rb] + kk) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        float b[NACC][4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          b[0][s] = w0[(int64_t)(kk + s) * p.ndim];
          if (GATEUP) b[NACC - 1][s] = w1[(int64_t)(kk + s) * p.ndim];
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int m = 0; m < NACC; ++m)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
              acc[m][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(b[m][s], a[rb][s], acc[m][rb], 0, 0, 0);
      }
    }
    // fixed-order sum of the quarters, then SwiGLU (gate/up) and the stores
    if (wq > 0) {
#pragma unroll
      for (int m = 0; m < NACC; ++m)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) red[wq - 1][m][rb][lane] = acc[m][rb];
    }
    __syncthreads();
    if (wq == 0) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x4 v = acc[0][rb], u = acc[NACC - 1][rb];
#pragma unroll
        for (int j = 0; j < KW - 1; ++j) {
          v += red[j][0][rb][lane];
          if (GATEUP) u += red[j][NACC - 1][rb][lane];
        }
        if (GATEUP) {
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = v[c] / (1.0f + expf(-v[c])) * u[c];
        }
        const int r = rb * 16 + i16;
        if (r < rows) *reinterpret_cast<f32x4*>(p.c + (int64_t)(row0 + r) * p.ndim + n0 + 4 * j4) = v;
      }
    }
    __syncthreads();  // red is rewritten by the next task
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
