// fused.hip -- the whole FFN-side layer of a block-FP8 or W8A8 layer in one
// persistent launch: the dispatch phases and the combine of fused.h, and
//   D4  the activation scales gathered into sorted-row order (coalesced
//       stores; inside D3 they were 56 scattered stores per slot, which made
//       D3 the slowest phase after the GEMMs);
//   G1  gate/up + SwiGLU over both tile lists (gemm_ring.h);
//   Q   W8A8 only: h re-quantised to int8 per row (quant.h);
//   G2  down;
// between grid barriers.
#include "fused.h"
#include "gemm_ring.h"
#include "quant.h"

namespace afd {

static_assert(kFusedWaves == kRingWaves, "the fused kernel runs the ring GEMM's workgroup");

template <bool WNT, bool I8>
__global__ __launch_bounds__(kFusedThreads, 1) void fused_kernel(FusedParams f) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  int* const lds = reinterpret_cast<int*>(ring);  // the dispatch phases use the ring's LDS
  const DispatchParams& d = f.d;
  const int G = gridDim.x, b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int E = d.num_experts, K = f.top_k;
  int target = 0;

  fused_dispatch(f, b, G, lds, target);

  // ---- D4: the activation scales in sorted-row order (step-major), for the
  // routed rows and the shared expert's; consecutive threads write
  // consecutive rows of a step, 8 items per thread in flight
  {
    const int N = d.offsets[E];
    const int R = N + d.shared_parts * d.shared_rows;
    const int64_t total = (int64_t)f.ks * R, stride = (int64_t)G * kFusedThreads;
    constexpr int kU = 8;
    for (int64_t i0 = (int64_t)b * kFusedThreads + tid; i0 < total; i0 += kU * stride) {
      int tok[kU];
      int64_t dst[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = i0 + u * stride;
        dst[u] = -1;
        tok[u] = 0;
        if (i < total) {
          const int c = (int)(i / R), rr = (int)(i - (int64_t)c * R);
          const int row = rr < N ? rr : d.shared_row0 + (rr - N);
          tok[u] = rr < N ? d.sorted_assign[rr] / K : (rr - N) % d.shared_rows;
          tok[u] = tok[u] * f.ks + c;  // source index
          dst[u] = (int64_t)c * f.ld + row;
        }
      }
      float v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = dst[u] >= 0 ? f.x_src[tok[u]] : 0.0f;
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (dst[u] >= 0) f.x_dst[dst[u]] = v[u];
    }
  }
  grid_sync(f.bar, target, G, f.spin_limit);

  // ---- G1: gate/up + SwiGLU
  ring_stage<true, WNT, I8, true>(f.gu, b, G);
  grid_sync(f.bar, target, G, f.spin_limit);

  // ---- Q (W8A8): h to int8, one wave per row
  if constexpr (I8) {
    const int routed = f.qp.offsets[f.qp.num_experts];
    for (int i = b * kRingWaves + wave; i < routed; i += G * kRingWaves) quant_row(f.qp, i, lane);
    for (int i = b * kRingWaves + wave; i < f.qp.shared_rows; i += G * kRingWaves)
      quant_row(f.qp, f.qp.shared_row0 + i, lane);
    grid_sync(f.bar, target, G, f.spin_limit);
  }

  // ---- G2: down
  ring_stage<false, WNT, I8, true>(f.dn, b, G);
  grid_sync(f.bar, target, G, f.spin_limit);

  fused_combine(f, b, G);
}

template <bool WNT, bool I8>
static hipError_t launch_fused_one(const FusedParams& f, int num_cus, hipStream_t s) {
  constexpr int lds = kRingLdsBytes;
  static int per_cu = 0;
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_kernel<WNT, I8>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fused_kernel<WNT, I8>, kFusedThreads, lds);
    if (e != hipSuccess) return e;
    if (occ < 1) return hipErrorInvalidConfiguration;  // a workgroup does not fit a CU
    per_cu = occ;
  }
  // one workgroup per CU of this call's share: every one is resident at once,
  // which the grid barriers need (at most 512: one chunk count per thread)
  const int grid = std::min(num_cus, kFusedMaxGrid);
  if (grid <= 0) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fused_kernel<WNT, I8>), dim3((unsigned)grid), dim3(kFusedThreads), lds, s, f);
  return hipGetLastError();
}

hipError_t launch_fused(bool stream_weights, bool int8, const FusedParams& f, int num_cus, hipStream_t s) {
  if (int8)
    return stream_weights ? launch_fused_one<true, true>(f, num_cus, s) : launch_fused_one<false, true>(f, num_cus, s);
  return stream_weights ? launch_fused_one<true, false>(f, num_cus, s) : launch_fused_one<false, false>(f, num_cus, s);
}

}  // namespace afd
