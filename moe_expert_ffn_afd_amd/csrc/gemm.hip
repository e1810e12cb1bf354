// gemm.hip -- the light-list kernel of the streaming grouped expert GEMMs
// (bf16; the workgroup body and its design are in gemm_stream.h): used when a
// batch has light experts only, four waves per workgroup, several workgroups
// per CU.
#include <algorithm>

#include "gemm_stream.h"

namespace afd {

template <bool GATEUP, int MR>
__global__ __launch_bounds__(256) void gemm_grouped_kernel(GemmParams p) {
  if (p.only_launch && uniform(p.num_mtiles[3]) != p.only_launch) return;
  stream_body<GATEUP, MR, 1>(p, blockIdx.x, gridDim.x);
}

template <bool GATEUP, int MR>
static hipError_t launch_one(const GemmParams& p, int64_t max_tasks, int num_cus, hipStream_t s) {
  // persistent grid: never more workgroups than can be resident at once
  static int per_cu = 0;
  if (per_cu == 0) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_grouped_kernel<GATEUP, MR>, 256, kArowBytes<MR>) !=
            hipSuccess ||
        occ <= 0)
      occ = 1;
    per_cu = occ;
  }
  const int64_t grid = std::min<int64_t>(max_tasks, (int64_t)num_cus * per_cu);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_grouped_kernel<GATEUP, MR>), dim3((unsigned)grid), dim3(256), kArowBytes<MR>, s, p);
  return hipGetLastError();
}

int down_panels_per_task(int mr) { return kWaves * (mr == 1 ? AFD_DOWN_NPW : 2); }

hipError_t launch_gemm(int dtype, bool gate_up, int mr, const GemmParams& p, int64_t max_tasks, int num_cus,
                       hipStream_t s) {
  if (dtype != kBF16) return hipErrorInvalidValue;
  if (mr == 1) return gate_up ? launch_one<true, 1>(p, max_tasks, num_cus, s) : launch_one<false, 1>(p, max_tasks, num_cus, s);
  if (mr == 2) return gate_up ? launch_one<true, 2>(p, max_tasks, num_cus, s) : launch_one<false, 2>(p, max_tasks, num_cus, s);
  return hipErrorInvalidValue;
}

}  // namespace afd
