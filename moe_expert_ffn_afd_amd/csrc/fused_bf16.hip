// fused_bf16.hip -- the whole FFN-side layer of a bf16 layer in one persistent
// launch: the dispatch phases and the combine of fused.h, and between them the
// two GEMM stages run as the separate launches run them:
//   G1  gate/up + SwiGLU: the light list alone on every workgroup (the
//       streaming body of gemm_stream.h, two 4-wave halves per workgroup)
//       where the dispatch kept every expert light, else the mixed split (the
//       dispatch's share of the workgroups streams the light list, the others
//       run the heavy tiles on the LDS-tiled body of gemm_tiled.h);
//   G2  down, the same way;
// separated by grid barriers.
#include "fused.h"
#include "gemm_stream.h"
#include "gemm_tiled.h"

namespace afd {

static_assert(kFusedWaves == kNW, "the fused kernel runs the LDS-tiled GEMM's workgroup");

namespace {

// One GEMM stage as workgroup b of G (the mixed kernel's roles; lo: the
// light-only launch's parameters, used when the dispatch chose it).
template <bool GATEUP, int MR_LO, int MR>
__device__ __forceinline__ void bf16_stage(const FusedParams& f, const GemmParams& lo, const GemmParams& light,
                                           const GemmParams& heavy, const int b, const int G) {
  if (f.auto_launch && uniform(light.num_mtiles[3]) == kLaunchLight) {
    stream_body<GATEUP, MR_LO, 2>(lo, b, G);
    return;
  }
  const int L = min(max(uniform(light.num_mtiles[2]), 0), G);
  if (b < L) {
    stream_body<GATEUP, MR, 2>(light, b, L);
    tiled_pool<GATEUP>(heavy, G - L);
    return;
  }
  tiled_body<GATEUP>(heavy, b - L, G - L);
  // no light workgroups (no light tiles, or a grid too small to split): the
  // heavy workgroups run the light list afterwards
  if (L == 0) stream_body<GATEUP, MR, 2>(light, b, G);
}

}  // namespace

template <int MR_LO, int MR>
__global__ __launch_bounds__(kFusedThreads, 1) void fused_bf16_kernel(FusedParams f) {
  extern __shared__ __attribute__((aligned(16))) uint8_t fused_lds[];
  int* const lds = reinterpret_cast<int*>(fused_lds);  // the dispatch phases use the GEMMs' LDS
  const int G = gridDim.x, b = blockIdx.x;
  int target = 0;

  fused_dispatch(f, b, G, lds, target);

  // ---- G1: gate/up + SwiGLU
  bf16_stage<true, MR_LO, MR>(f, f.gu_lo, f.gu, f.gu_heavy, b, G);
  grid_sync(f.bar, target, G, f.spin_limit);

  // ---- G2: down
  bf16_stage<false, MR_LO, MR>(f, f.dn_lo, f.dn, f.dn_heavy, b, G);
  grid_sync(f.bar, target, G, f.spin_limit);

  fused_combine(f, b, G);
}

template <int MR_LO, int MR>
static hipError_t launch_fused_bf16_one(const FusedParams& f, int num_cus, hipStream_t s) {
  static_assert(2 * kArowBytes<MR_LO> <= kLds && 2 * kArowBytes<MR> <= kLds, "light rows fit the tiled LDS");
  constexpr int lds = kLds;
  static int per_cu = 0;
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_bf16_kernel<MR_LO, MR>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fused_bf16_kernel<MR_LO, MR>, kFusedThreads, lds);
    if (e != hipSuccess) return e;
    if (occ < 1) return hipErrorInvalidConfiguration;  // a workgroup does not fit a CU
    per_cu = occ;
  }
  // one workgroup per CU of this call's share: every one is resident at once,
  // which the grid barriers need (at most 512: one chunk count per thread)
  const int grid = std::min(num_cus, kFusedMaxGrid);
  if (grid <= 0) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fused_bf16_kernel<MR_LO, MR>), dim3((unsigned)grid), dim3(kFusedThreads), lds, s, f);
  return hipGetLastError();
}

hipError_t launch_fused_bf16(int mr_lo, int mr, const FusedParams& f, int num_cus, hipStream_t s) {
  if (mr == 1) {
    if (mr_lo == 1) return launch_fused_bf16_one<1, 1>(f, num_cus, s);
    if (mr_lo == 2) return launch_fused_bf16_one<2, 1>(f, num_cus, s);
  } else if (mr == 2 && mr_lo == 2) {
    return launch_fused_bf16_one<2, 2>(f, num_cus, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace afd
