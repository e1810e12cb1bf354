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
#include "afd_internal.h"

namespace afd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ inline uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline i32x8 cat32(uint4 a, uint4 b) {
  i32x8 r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
}

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)a);
  uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)b);
  return lo | (hi << 16);
}

// 4 floats -> 4 e4m3 codes (round to nearest even; inputs already within +-448)
__device__ inline uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

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

  for (int task = blockIdx.x; task < num_tasks; task += gridDim.x) {
    const int mt = task % num_mt;
    const int q = task / num_mt;
    const int4 tile = p.mtiles[mt];
    const int expert = uniform(tile.x);
    const int row0 = uniform(tile.y);
    const int rows = uniform(tile.z);
    const int unit = q * kWaves + wave;
    const bool active = GATEUP ? (unit < p.n_panels) : (2 * unit < p.n_panels);

    // activation row pointers (rows past the tile's count repeat its first row)
    const uint8_t* arow[MR];
    const float* srow[MR];
#pragma unroll
    for (int mr = 0; mr < MR; ++mr) {
      int m = mr * 32 + col;
      int r = row0 + (m < rows ? m : 0);
      int64_t src = r;
      if (p.gather) src = r >= p.shared_row0 ? (r - p.shared_row0) : (p.sorted_assign[r] / p.top_k);
      arow[mr] = p.a + src * p.a_row_bytes + g * 64;
      srow[mr] = DT == kFP8 ? p.a_scales + src * p.a_scale_ld : nullptr;
    }
    const uint8_t* bbase = p.b + (int64_t)expert * p.b_expert_bytes +
                           (int64_t)(2 * unit) * p.b_panel_bytes + lane * 16;
    // FP8 weight block scales of this wave's two panels
    const float* sb0 = nullptr;
    const float* sb1 = nullptr;
    if (DT == kFP8) {
      int64_t eoff = (int64_t)expert * p.b_scale_rows * p.b_scale_cols;
      if (GATEUP) {
        sb0 = p.b_scales0 + eoff + unit / 4;
        sb1 = p.b_scales1 + eoff + unit / 4;
      } else {
        sb0 = p.b_scales0 + eoff + unit / 2;
        sb1 = sb0;
      }
    }

    f32x16 acc[MR][2];
#pragma unroll
    for (int mr = 0; mr < MR; ++mr)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mr][pp][r] = 0.0f;

    if (active) {
      auto load = [&](Stage<DT, MR>& s, int c) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            s.b[pp][j] = ld16(bbase + (int64_t)pp * p.b_panel_bytes + (int64_t)c * kStepPanelBytes + j * 1024);
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) {
#pragma unroll
          for (int j = 0; j < 4; ++j) s.a[mr][j] = ld16(arow[mr] + (int64_t)c * kStepBytes + j * 16);
          if (DT == kFP8) s.sa[mr] = srow[mr][c];
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
          const float b0 = sb0[(int64_t)c * p.b_scale_cols];
          const float b1 = sb1[(int64_t)c * p.b_scale_cols];
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

      Stage<DT, MR> s0, s1;
      load(s0, 0);
      for (int c = 0; c < ks; c += 2) {
        if (c + 1 < ks) load(s1, c + 1);
        compute(s0, c);
        if (c + 2 < ks) load(s0, c + 2);
        if (c + 1 < ks) compute(s1, c + 1);
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
static hipError_t launch_one(const GemmParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_grouped_kernel<DT, GATEUP, MR>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, bool gate_up, int mr, const GemmParams& p, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
#define AFD_CASE(DT, GU, MRV) \
  if (dtype == DT && gate_up == GU && mr == MRV) return launch_one<DT, GU, MRV>(p, grid, s);
  AFD_CASE(kBF16, true, 1) AFD_CASE(kBF16, true, 2) AFD_CASE(kBF16, false, 1) AFD_CASE(kBF16, false, 2)
  AFD_CASE(kFP8, true, 1) AFD_CASE(kFP8, true, 2) AFD_CASE(kFP8, false, 1) AFD_CASE(kFP8, false, 2)
#undef AFD_CASE
  return hipErrorInvalidValue;
}

}  // namespace afd
