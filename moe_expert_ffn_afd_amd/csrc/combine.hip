// combine.hip -- top-k weighted combine of the expert outputs: one workgroup
// per token (the per-token body and its design are in combine.h).
#include "combine.h"

namespace afd {

template <int DT>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  __shared__ int rows[kMaxRowsPerToken];
  __shared__ float ws[kMaxRowsPerToken];
  __shared__ int nrows;
  combine_rows<DT>(p, blockIdx.x, true, threadIdx.x, blockDim.x, rows, ws, &nrows);
}

hipError_t launch_combine(int dtype, const CombineParams& p, int tokens, hipStream_t s) {
  if (tokens <= 0) return hipSuccess;
  if (dtype == kF32)
    hipLaunchKernelGGL(combine_kernel<kF32>, dim3(tokens), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(combine_kernel<kBF16>, dim3(tokens), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace afd
