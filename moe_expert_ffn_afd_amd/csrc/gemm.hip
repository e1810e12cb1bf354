// gemm.hip -- grouped expert GEMMs on MFMA (bf16 and block-FP8), gfx950.
//
// The FFN stage time is dominated by expert-weight reads and the grouped GEMM
// over the routed tokens ("FastAFD" structured summary, legend of Eq. (3));
// FastAFD's expert GPUs run block-FP8 grouped GEMMs with the activation fused
// (System Design item 3).  Two GEMMs per expert e with n_e routed rows:
//   gate/up:  h = silu(X_e Wg_e) * (X_e Wu_e)      [n_e, H] x [H, I]
//   down:     y = h_e Wd_e                          [n_e, I] x [I, H]
//
// Work decomposition.  The m-tile list (built on the device by the dispatch)
// holds runs of at most 32*MR rows of one expert.  A workgroup task is one
// m-tile times one group of 4 "units" along N, one unit per wave: for gate/up
// a unit is gate panel p plus up panel p (32 h columns, so a task covers 128
// h columns -- one FP8 requantisation group); for down a unit is two adjacent
// 32-column panels of H.  Every wave streams its own panels over the whole
// reduction straight from HBM into MFMA operand registers (the packed layout
// makes each 16-byte lane load one contiguous KiB per wave), with the next
// super-step's loads in flight while the current one is multiplied.  The
// activation rows are small, shared by the 4 waves and served from cache.
//
// MFMA orientation: the weight fragment is the first operand and the
// activation fragment the second, so the 32x32 accumulator holds out^T: lane l
// owns token column m = l % 32 and 16 output columns n = 8(r/4) + 4(l/32) + r%4
// (r = register).  Gate and up of the same (m, n) sit in the same register of
// two accumulators, so SwiGLU is elementwise, and a token's activation scale
// (FP8) is one value per lane.
//
// Block-FP8: a super-step is one 128-deep scale block; its two e4m3 MFMAs
// accumulate into a scratch accumulator that is then added with the product
// of the token's 1x128 scale and the weight's 128x128 block scale.  The
// gate/up epilogue requantises h to e4m3 with one fp32 scale per token and
// 128 h columns (amax / 448), the plain reading of running both expert GEMMs
// in block-FP8.  The rows outside an m-tile's count are computed on a
// duplicate of its first row and never stored.
#include <algorithm>

#include "afd_device.h"

namespace afd {

using namespace dev;

#ifndef AFD_XCD_REMAP
#define AFD_XCD_REMAP 0
#endif
#ifndef AFD_STAGES
#define AFD_STAGES 2
#endif
// cache policy of weight loads: 2 = non-temporal (streamed once; bf16),
// 0 = default (FP8 tiles of one expert re-read their panels from L2)
#ifndef AFD_B_AUX_BF16
#define AFD_B_AUX_BF16 2
#endif
#ifndef AFD_B_AUX_FP8
#define AFD_B_AUX_FP8 0
#endif
#ifndef AFD_PIPE_SCHED
#define AFD_PIPE_SCHED 1
#endif
#if AFD_PIPE_SCHED
#define AFD_PIPE_FENCE() __builtin_amdgcn_sched_barrier(0)
#else
#define AFD_PIPE_FENCE() ((void)0)
#endif

namespace {

template <int DT, int MR>
struct Stage {
  uint4 a[MR][4];
  uint4 b[2][4];
  float sa[MR];
};

}  // namespace

template <int DT, bool GATEUP, int MR>
__global__ __launch_bounds__(256) void gemm_grouped_kernel(GemmParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 5;
  const int col = lane & 31;
  __shared__ float red[MR][kWaves][32];  // FP8 requantisation: per-wave row amax

  const int num_mt = uniform(p.num_mtiles[0]);
  const int num_tasks = num_mt * p.n_groups;
  const int ks = p.k_steps;

  // Optional XCD-aware schedule (AFD_XCD_REMAP): workgroups are dealt
  // round-robin to the 8 XCDs; renumbering them so each XCD owns a contiguous
  // block of ranks puts consecutive tasks (sibling m-tiles of one expert) under
  // one L2.  Measured: it does not remove the sibling re-reads (the streams
  // drift apart further than their share of L2) and slows skewed batches, so
  // it is off.
  const int G = gridDim.x;
  const int rank = (AFD_XCD_REMAP && G % kXcds == 0) ? (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds
                                                     : blockIdx.x;
  for (int task = rank; task < num_tasks; task += G) {
    const int mt = task % num_mt;
    const int q = task / num_mt;
    const int4 tile = p.mtiles[mt];
    const int expert = uniform(tile.x);
    const int row0 = uniform(tile.y);
    const int rows = uniform(tile.z);
    const int unit = q * kWaves + wave;
    const bool active = GATEUP ? (unit < p.n_panels) : (2 * unit < p.n_panels);

    // activation rows (rows past the tile's count repeat its first row): one
    // 32-bit buffer offset per lane and row fragment; weights: SGPR offsets only
    int aoff[MR], soffA[MR];
#pragma unroll
    for (int mr = 0; mr < MR; ++mr) {
      int m = mr * 32 + col;
      int r = row0 + (m < rows ? m : 0);
      int src = r;
      if (p.gather) src = r >= p.shared_row0 ? (r - p.shared_row0) : (p.sorted_assign[r] / p.top_k);
      aoff[mr] = (int)(src * p.a_row_bytes) + g * 64;
      soffA[mr] = src * p.a_scale_ld * 4;
    }
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.a_scales, p.a_scale_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + (int64_t)expert * p.b_expert_bytes, p.b_expert_bytes);
    const int boff = uniform((int)((int64_t)(2 * unit) * p.b_panel_bytes));
    const int bpanel = (int)p.b_panel_bytes;
    const int voffB = lane * 16;
    // FP8 weight block scales of this wave's two panels, one per super-step:
    // lane l holds those of super-steps l and l + 64, read in the loop with
    // readlane (no memory operation inside the load pipeline)
    BlockScales sbs;
    if (DT == kFP8) {
      const int64_t eoff = (int64_t)expert * p.b_scale_rows * p.b_scale_cols;
      const int nb = GATEUP ? unit / 4 : unit / 2;
      sbs.load(p.b_scales0 + eoff + nb, (GATEUP ? p.b_scales1 : p.b_scales0) + eoff + nb, p.b_scale_cols, ks, lane);
    }

    f32x16 acc[MR][2];
#pragma unroll
    for (int mr = 0; mr < MR; ++mr)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mr][pp][r] = 0.0f;

    if (active) {
      // Loads of step c >= ks use an offset past the end of the buffer, which
      // the buffer unit returns as zeros: the loop body stays branch-free (so
      // the compiler's waits only cover the stage being multiplied) and the
      // phantom step adds exact zeros.
      const int oobA = (int)(p.a_bytes > 0x7fffffff ? 0x7fffffff : p.a_bytes);
      const int oobS = (int)(p.a_scale_bytes > 0x7fffffff ? 0x7fffffff : p.a_scale_bytes);
      const int oobB = (int)p.b_expert_bytes;
      auto load = [&](Stage<DT, MR>& s, int c) {
        const bool in = c < ks;
        const int sb = in ? boff + c * kStepPanelBytes : oobB;
        const int sa = in ? c * kStepBytes : oobA;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int j = 0; j < 4; ++j) s.b[pp][j] = bload16<DT == kBF16 ? AFD_B_AUX_BF16 : AFD_B_AUX_FP8>(rb, voffB, sb + pp * bpanel + j * 1024);
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) {
#pragma unroll
          for (int j = 0; j < 4; ++j) s.a[mr][j] = bload16(ra, aoff[mr], sa + j * 16);
          if (DT == kFP8)
            s.sa[mr] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rsa, soffA[mr], in ? c * 4 : oobS, 0));
        }
      };
      auto compute = [&](const Stage<DT, MR>& s, int c) {
        if (DT == kBF16) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mr = 0; mr < MR; ++mr)
#pragma unroll
              for (int pp = 0; pp < 2; ++pp)
                acc[mr][pp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(s.b[pp][j]), as_bf16x8(s.a[mr][j]), acc[mr][pp], 0, 0, 0);
        } else {
          const int cs = c < ks ? c : ks - 1;
          const float b0 = sbs.get0(cs), b1 = sbs.get1(cs);
#pragma unroll
          for (int mr = 0; mr < MR; ++mr) {
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              f32x16 t;
#pragma unroll
              for (int r = 0; r < 16; ++r) t[r] = 0.0f;
              t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  cat32(s.b[pp][0], s.b[pp][1]), cat32(s.a[mr][0], s.a[mr][1]), t, 0, 0, 0, 0, 0, 0);
              t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  cat32(s.b[pp][2], s.b[pp][3]), cat32(s.a[mr][2], s.a[mr][3]), t, 0, 0, 0, 0, 0, 0);
              const float sc = s.sa[mr] * (pp == 0 ? b0 : b1);
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[mr][pp][r] += t[r] * sc;
            }
          }
        }
      };

      // AFD_STAGES register stages: the loads of step c + AFD_STAGES - 1 are
      // issued, kept together by scheduling fences, ahead of step c's
      // multiplies, so AFD_STAGES - 1 super-steps stay in flight per wave.
      Stage<DT, MR> st[AFD_STAGES];
#pragma unroll
      for (int i = 0; i + 1 < AFD_STAGES; ++i) load(st[i], i);
      for (int c0 = 0; c0 < ks; c0 += AFD_STAGES) {
#pragma unroll
        for (int i = 0; i < AFD_STAGES; ++i) {
          load(st[(i + AFD_STAGES - 1) % AFD_STAGES], c0 + i + AFD_STAGES - 1);
          AFD_PIPE_FENCE();
          compute(st[i], c0 + i);
          AFD_PIPE_FENCE();
        }
      }
    }

    // ---------------------------------------------------------------- epilogue
    if (GATEUP) {
      float h[MR][16];
#pragma unroll
      for (int mr = 0; mr < MR; ++mr)
#pragma unroll
        for (int r = 0; r < 16; ++r) h[mr][r] = silu_mul(acc[mr][0][r], acc[mr][1][r]);

      if (DT == kBF16) {
        if (active) {
#pragma unroll
          for (int mr = 0; mr < MR; ++mr) {
            const int m = mr * 32 + col;
            if (m < rows) {
              uint8_t* out = p.c + (int64_t)(row0 + m) * p.c_row_bytes + (int64_t)(32 * unit) * 2;
#pragma unroll
              for (int r4 = 0; r4 < 4; ++r4) {
                const int n = 8 * r4 + 4 * g;
                uint2 v;
                v.x = pack_bf16x2(h[mr][4 * r4 + 0], h[mr][4 * r4 + 1]);
                v.y = pack_bf16x2(h[mr][4 * r4 + 2], h[mr][4 * r4 + 3]);
                *reinterpret_cast<uint2*>(out + n * 2) = v;
              }
            }
          }
        }
      } else {
        // amax of |h| per token over this task's 128 h columns
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) {
          float a = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) a = fmaxf(a, fabsf(h[mr][r]));
          a = fmaxf(a, __shfl_xor(a, 32, 64));
          if (g == 0) red[mr][wave][col] = a;
        }
        __syncthreads();
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) {
          float amax = fmaxf(fmaxf(red[mr][0][col], red[mr][1][col]), fmaxf(red[mr][2][col], red[mr][3][col]));
          const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
          const float inv = amax > 0.0f ? 448.0f / amax : 1.0f;
          const int m = mr * 32 + col;
          if (m < rows && active) {
            uint8_t* out = p.c + (int64_t)(row0 + m) * p.c_row_bytes + 32 * unit;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int n = 8 * r4 + 4 * g;
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = fminf(fmaxf(h[mr][4 * r4 + e] * inv, -448.0f), 448.0f);
              *reinterpret_cast<uint32_t*>(out + n) = pack_fp8x4(v[0], v[1], v[2], v[3]);
            }
            if (wave == 0 && g == 0) p.c_scales[(int64_t)(row0 + m) * p.c_scale_ld + q] = scale;
          }
        }
        __syncthreads();  // red[] is rewritten by the next task
      }
    } else if (active) {
#pragma unroll
      for (int mr = 0; mr < MR; ++mr) {
        const int m = mr * 32 + col;
        if (m < rows) {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            uint8_t* out = p.c + (int64_t)(row0 + m) * p.c_row_bytes + (int64_t)(32 * (2 * unit + pp)) * 2;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int n = 8 * r4 + 4 * g;
              uint2 v;
              v.x = pack_bf16x2(acc[mr][pp][4 * r4 + 0], acc[mr][pp][4 * r4 + 1]);
              v.y = pack_bf16x2(acc[mr][pp][4 * r4 + 2], acc[mr][pp][4 * r4 + 3]);
              *reinterpret_cast<uint2*>(out + n * 2) = v;
            }
          }
        }
      }
    }
  }
}

template <int DT, bool GATEUP, int MR>
static hipError_t launch_one(const GemmParams& p, int64_t max_tasks, int num_cus, hipStream_t s) {
  // persistent grid: never more workgroups than can be resident at once
  static int per_cu = 0;
  if (per_cu == 0) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_grouped_kernel<DT, GATEUP, MR>, 256, 0) !=
            hipSuccess ||
        occ <= 0)
      occ = 1;
    per_cu = occ;
  }
  const int64_t grid = std::min<int64_t>(max_tasks, (int64_t)num_cus * per_cu);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_grouped_kernel<DT, GATEUP, MR>), dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, bool gate_up, int mr, const GemmParams& p, int64_t max_tasks, int num_cus,
                       hipStream_t s) {
#define AFD_CASE(DT, GU, MRV) \
  if (dtype == DT && gate_up == GU && mr == MRV) return launch_one<DT, GU, MRV>(p, max_tasks, num_cus, s);
  AFD_CASE(kBF16, true, 1) AFD_CASE(kBF16, true, 2) AFD_CASE(kBF16, false, 1) AFD_CASE(kBF16, false, 2)
  AFD_CASE(kFP8, true, 1) AFD_CASE(kFP8, true, 2) AFD_CASE(kFP8, false, 1) AFD_CASE(kFP8, false, 2)
#undef AFD_CASE
  return hipErrorInvalidValue;
}

}  // namespace afd
