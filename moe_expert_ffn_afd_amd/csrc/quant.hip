// quant.hip -- W8A8 layers: the per-row int8 re-quantisation of h, one wave per
// row (the row body and its reading are in quant.h).
#include "quant.h"

namespace afd {

__global__ __launch_bounds__(256) void quant_rows_kernel(QuantParams p) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  int r;
  if (blockIdx.y == 0) {  // routed rows (sorted order)
    if (i >= p.offsets[p.num_experts]) return;
    r = i;
  } else {                // the shared expert's rows
    if (i >= p.shared_rows) return;
    r = p.shared_row0 + i;
  }
  quant_row(p, r, lane);
}

hipError_t launch_quant_rows(const QuantParams& p, hipStream_t s) {
  const int n = p.routed_max > p.shared_rows ? p.routed_max : p.shared_rows;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((n + 3) / 4, p.shared_row0 >= 0 ? 2 : 1), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace afd
