// gemm_ring.hip -- the block-FP8 and W8A8 ring GEMM kernels: one persistent
// launch per GEMM stage over both tile lists (the workgroup body and its design
// are in gemm_ring.h).
#include "gemm_ring.h"

namespace afd {

template <bool GATEUP, bool WNT, bool I8>
__global__ __launch_bounds__(kRingWaves * 64, 1) void gemm_ring_kernel(GemmParams p) {
  ring_stage<GATEUP, WNT, I8, false>(p, blockIdx.x, gridDim.x);
}

// 8-bit experts of many rows (the tiled list, gemm_tiled8.h), launched before
// the ring kernel of the same stage
template <bool GATEUP, bool I8>
__global__ __launch_bounds__(kT8Waves * 64, 1) void gemm_tiled8_kernel(GemmParams p) {
  const int G = gridDim.x, b = blockIdx.x;
  const int rank = (AFD_RING_XCD_REMAP && G % kXcds == 0) ? (b % kXcds) * (G / kXcds) + b / kXcds : b;
  tiled8_list<GATEUP, I8>(p, p.mtiles3, uniform(p.num_mtiles3[0]), rank, G);
}

template <bool GATEUP, bool I8>
static hipError_t launch_tiled8_one(const GemmParams& p, int64_t max_tasks, int num_cus, hipStream_t s) {
  constexpr int lds = kT8LdsBytes;
  static bool ready = false;
  if (!ready) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tiled8_kernel<GATEUP, I8>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    ready = true;
  }
  const int64_t grid = std::min<int64_t>(max_tasks, num_cus);  // one workgroup per CU (LDS)
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_tiled8_kernel<GATEUP, I8>), dim3((unsigned)grid), dim3(kT8Waves * 64), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm_tiled8(bool gate_up, bool int8, const GemmParams& p, int64_t max_tasks, int num_cus,
                              hipStream_t s) {
  if (int8)
    return gate_up ? launch_tiled8_one<true, true>(p, max_tasks, num_cus, s)
                   : launch_tiled8_one<false, true>(p, max_tasks, num_cus, s);
  return gate_up ? launch_tiled8_one<true, false>(p, max_tasks, num_cus, s)
                 : launch_tiled8_one<false, false>(p, max_tasks, num_cus, s);
}

template <bool GATEUP, bool WNT, bool I8>
static hipError_t launch_ring_one(const GemmParams& p, int64_t max_tasks, int num_cus, hipStream_t s) {
  constexpr int lds = kRingLdsBytes;
  static int per_cu = 0;
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_ring_kernel<GATEUP, WNT, I8>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_ring_kernel<GATEUP, WNT, I8>, kRingWaves * 64,
                                                     lds) != hipSuccess ||
        occ <= 0)
      occ = 1;
    per_cu = occ;
  }
  const int64_t grid = std::min<int64_t>(max_tasks, (int64_t)num_cus * per_cu);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_ring_kernel<GATEUP, WNT, I8>), dim3((unsigned)grid), dim3(kRingWaves * 64), lds, s, p);
  return hipGetLastError();
}

int ring_rows(bool heavy) { return heavy ? 128 : 64; }

template <bool I8>
static hipError_t launch_ring_fmt(bool gate_up, bool stream_weights, const GemmParams& p, int64_t max_tasks,
                                  int num_cus, hipStream_t s) {
  if (stream_weights)
    return gate_up ? launch_ring_one<true, true, I8>(p, max_tasks, num_cus, s)
                   : launch_ring_one<false, true, I8>(p, max_tasks, num_cus, s);
  return gate_up ? launch_ring_one<true, false, I8>(p, max_tasks, num_cus, s)
                 : launch_ring_one<false, false, I8>(p, max_tasks, num_cus, s);
}

hipError_t launch_gemm_ring(bool gate_up, bool stream_weights, bool int8, const GemmParams& p, int64_t max_tasks,
                            int num_cus, hipStream_t s) {
  return int8 ? launch_ring_fmt<true>(gate_up, stream_weights, p, max_tasks, num_cus, s)
              : launch_ring_fmt<false>(gate_up, stream_weights, p, max_tasks, num_cus, s);
}

}  // namespace afd
