// gemm_tiled.hip -- the mixed bf16 GEMM kernel: the heavy m-tiles on the
// LDS-tiled body (gemm_tiled.h) and the light ones on the streaming body
// (gemm_stream.h), side by side on disjoint CUs of one launch.
#include <algorithm>

#include "gemm_stream.h"
#include "gemm_tiled.h"

namespace afd {

// One launch per GEMM of a bf16 layer with heavy experts: one workgroup of 8
// waves per CU, the first L of them (L from the dispatch, a multiple of 8
// where the grid is, so every XCD gets L/8) stream the light list as two
// 4-wave halves, the others run the heavy tiles.  The light tasks are bound
// by HBM and the heavy ones by MFMA and LDS, so running both at once overlaps
// the two limits instead of paying them one after the other.
template <bool GATEUP, int MR>
__global__ __launch_bounds__(kNW * 64, 1) void gemm_mixed_kernel(GemmParams heavy, GemmParams light) {
  static_assert(kNW == 2 * kWaves, "the light role runs two 4-wave halves");
  static_assert(2 * kArowBytes<MR> <= kLds, "the light role's row slots fit the tiled ring");
  if (light.only_launch && uniform(light.num_mtiles[3]) != light.only_launch) return;
  const int n = gridDim.x;
  const int L = min(max(uniform(light.num_mtiles[2]), 0), n);
  if ((int)blockIdx.x < L) {
    stream_body<GATEUP, MR, 2>(light, blockIdx.x, L);
    tiled_pool<GATEUP>(heavy, n - L);  // then the heavy list's tail, with the heavy workgroups
    return;
  }
  tiled_body<GATEUP>(heavy, blockIdx.x - L, n - L);
  // No light workgroups (no light tiles, or a grid of one workgroup, too
  // small to split): the heavy workgroups run the light list afterwards.
  if (L == 0) stream_body<GATEUP, MR, 2>(light, blockIdx.x, n);
}

template <bool GATEUP, int MR>
static hipError_t launch_mixed_one(const GemmParams& heavy, const GemmParams& light, int num_cus, hipStream_t s) {
  static bool ready = false;
  if (!ready) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_mixed_kernel<GATEUP, MR>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    ready = true;
  }
  if (num_cus <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_mixed_kernel<GATEUP, MR>), dim3((unsigned)num_cus), dim3(kNW * 64), kLds, s, heavy, light);
  return hipGetLastError();
}

int tiled_rows(int dtype) { return dtype == kBF16 ? kBM : 0; }
int tiled_panels() { return kBNP; }

hipError_t launch_gemm_mixed(bool gate_up, int mr, const GemmParams& heavy, const GemmParams& light, int num_cus,
                             hipStream_t s) {
  if (mr == 1)
    return gate_up ? launch_mixed_one<true, 1>(heavy, light, num_cus, s) : launch_mixed_one<false, 1>(heavy, light, num_cus, s);
  if (mr == 2)
    return gate_up ? launch_mixed_one<true, 2>(heavy, light, num_cus, s) : launch_mixed_one<false, 2>(heavy, light, num_cus, s);
  return hipErrorInvalidValue;
}

}  // namespace afd
