// gemm_tiled.hip -- LDS-tiled grouped expert GEMMs for experts with many rows.
//
// Same two GEMMs as gemm.hip (gate/up with SwiGLU and, for block-FP8, the
// 1x128 re-quantisation of h; then down), for the m-tiles of "heavy" experts
// (rows >= a threshold): aggregated AFD batches concentrate tokens on popular
// experts ("FastAFD" summary, speculative decoding multiplies routed expert
// work; design-space study: expert FFNs are compute-intensive), where each
// weight panel must feed many rows and the MFMA pipes, not HBM, set the pace.
//
// A workgroup task is one m-tile of BM rows times 8 weight panels (256 GEMM
// columns: 128 h columns of gate+up, or 256 output columns of down).  Each
// super-step (128 bytes of K) of the task's weight panels and activation rows
// is copied HBM -> LDS by the buffer unit directly (no registers), into a ring
// of NS stages; the waves then read their MFMA fragments from LDS, so a
// weight byte is fetched once per tile and shared by every row of it.  The
// copy engine's LDS writes are invisible to the compiler, so the kernel
// orders them itself: it waits until only the younger stages are outstanding
// (s_waitcnt vmcnt) and then barriers, before any wave reads the stage.
//
// LDS fragments are read as ext_vector types: reading them through HIP's
// struct uint4 makes the compiler drain every in-flight copy before the read.
//
// LDS layout of a stage: weight panels exactly as packed in HBM (fragment
// order: conflict-free 16-byte reads), then activation rows of 128 bytes with
// the eight 16-byte slots of row r permuted by slot ^ ((r >> 1) & 7) (so the
// rows of an MFMA fragment read spread over all banks), then (FP8) the per-row
// activation scale of the super-step.
//
// bf16: tile 256 x 256, 8 waves (two per SIMD) as 4 x 2 of 64 rows x 4
//       panels, MFMA 32x32x16, 128 fp32 accumulators per lane; ring of 4
//       half-super-step slots (128 KiB), three in flight while one is
//       multiplied.
// FP8:  tile 128 x 256, 8 waves (two per SIMD) as 2 x 4 of 64 rows x 2
//       panels, MFMA 16x16x128 -- one MFMA spans a whole 128-deep scale block,
//       so each product is added straight into the accumulators times (token
//       scale x block scale); ring of 3 super-step slots (150 KiB).
#include <algorithm>
#include <type_traits>

#include "afd_device.h"

namespace afd {

using namespace dev;

namespace {

// Tile configuration.  NW waves form a WM x WN grid over BM rows x 8 panels;
// SUB = ring slots per super-step (a slot holds 128/SUB bytes of K per row).
template <int DT>
struct Tiled;
#ifndef AFD_TILED_BF16_NW
#define AFD_TILED_BF16_NW 8
#endif
#ifndef AFD_TILED_BF16_WM
#define AFD_TILED_BF16_WM 4
#endif
#ifndef AFD_TILED_BF16_NS
#define AFD_TILED_BF16_NS 4
#endif
template <>
struct Tiled<kBF16> {
  static constexpr int NW = AFD_TILED_BF16_NW, WM = AFD_TILED_BF16_WM, WN = NW / WM, BM = 256,
                       NS = AFD_TILED_BF16_NS, SUB = 2;
};
template <>
struct Tiled<kFP8> {
  static constexpr int NW = 8, WM = 2, WN = 4, BM = 128, NS = 3, SUB = 1;
};

#ifndef AFD_TILED_B_NT
#define AFD_TILED_B_NT 0  // 1: bf16 weight copies non-temporal (panels are re-read by sibling m-tiles)
#endif
#ifndef AFD_TILED_XCD_REMAP
#define AFD_TILED_XCD_REMAP 1
#endif
#ifndef AFD_TILED_MB
#define AFD_TILED_MB 4  // m-tiles per rasterisation block
#endif

constexpr int kBNP = 8;  // panels per task
constexpr int kMB = AFD_TILED_MB;

template <int DT>
constexpr int stage_bytes() {
  return (kBNP * kStepPanelBytes + Tiled<DT>::BM * kStepBytes) / Tiled<DT>::SUB + (DT == kFP8 ? Tiled<DT>::BM * 16 : 0);
}
template <int DT>
constexpr int lds_bytes() {
  return Tiled<DT>::NS * stage_bytes<DT>() + (DT == kFP8 ? 1024 : 0);  // + sink of idle scale copies
}

__device__ inline int clamp31(int64_t v) { return v > 0x7fffffff ? 0x7fffffff : (int)v; }

// LDS slot permutation of activation row r (rows of RB bytes, RB/16 slots):
// 16 consecutive rows reading the same 16-byte part hit 16 distinct
// (row, slot) bank groups, i.e. all 64 banks.
template <int RB>
__device__ inline int swz(int r) {
  return RB == 128 ? (r >> 1) & 7 : (r >> 2) & 3;
}

}  // namespace

template <int DT, bool GATEUP>
__global__ __launch_bounds__(Tiled<DT>::NW * 64, 1) void gemm_tiled_kernel(GemmParams p) {
  using C = Tiled<DT>;
  constexpr int NW = C::NW, WM = C::WM, WN = C::WN, BM = C::BM, NS = C::NS, SUB = C::SUB;
  constexpr int RB = kStepBytes / SUB;        // activation bytes per row and slot
  constexpr int PB = kStepPanelBytes / SUB;   // weight bytes per panel and slot
  constexpr int JJ = 4 / SUB;                 // 1 KiB chunks per panel and slot
  constexpr int B_OFF = 0, A_OFF = kBNP * PB, S_OFF = A_OFF + BM * RB;
  constexpr int STAGE = stage_bytes<DT>();
  constexpr int SINK = NS * STAGE;
  constexpr int ROWS_PER_COPY = 1024 / RB;
  constexpr int SLOTS = RB / 16;
  constexpr int B_DMA = kBNP * JJ / NW;                 // copies per wave and slot
  constexpr int A_DMA = BM * RB / 1024 / NW;
  constexpr int S_DMA = DT == kFP8 ? 1 : 0;
  constexpr int S_COPIES = BM / 64;                     // waves holding real scale rows
  constexpr int PER_STAGE = B_DMA + A_DMA + S_DMA;
  constexpr int WR = BM / WM;                           // rows per wave
  constexpr int NPW = kBNP / WN;                        // panels per wave
  static_assert(B_DMA * NW == kBNP * JJ && A_DMA * NW * 1024 == BM * RB, "copy split");
  static_assert(DT != kFP8 || (NPW == 2 && S_COPIES <= NW), "FP8 wave holds one gate/up unit");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float red[WM][WN][64];  // FP8 epilogue: per-wave row amax

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);  // scalar: LDS copy targets must be wave-uniform
  const int wm = wave / WN, wn = wave % WN;
  const int num_mt = uniform(p.num_mtiles[0]);
  const int num_tasks = num_mt * p.n_groups;
  const int ks = p.k_steps;
  const int oobA = clamp31(p.a_bytes), oobS = clamp31(p.a_scale_bytes);
  const int oobB = (int)p.b_expert_bytes;
  const int bpanel = (int)p.b_panel_bytes;
  const auto ra = make_rsrc(p.a, p.a_bytes);
  const auto rsa = make_rsrc(p.a_scales, p.a_scale_bytes);

  // Task order: blocks of kMB m-tiles x all column groups, column group
  // outer within a block, and workgroup ranks renumbered so each XCD owns a
  // contiguous run of tasks.  The ~32 tiles an XCD runs at once then share a
  // few activation chunks and weight panels through its L2.
  const int G = gridDim.x;
  const int rank = (AFD_TILED_XCD_REMAP && G % kXcds == 0) ? (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds
                                                           : blockIdx.x;
  const int nq = p.n_groups;
  const int full = (num_mt / kMB) * kMB * nq;  // tasks in complete blocks
  const int rem = num_mt % kMB;
  for (int task = rank; task < num_tasks; task += G) {
    int mt, q;
    if (task < full) {
      const int blk = task / (kMB * nq), w = task % (kMB * nq);
      q = w / kMB;
      mt = blk * kMB + w % kMB;
    } else {
      const int t = task - full;
      q = t / rem;
      mt = (num_mt / kMB) * kMB + t % rem;
    }
    const int4 tile = p.mtiles[mt];
    const int expert = uniform(tile.x), row0 = uniform(tile.y), rows = uniform(tile.z);
    const auto rb = make_rsrc(p.b + (int64_t)expert * p.b_expert_bytes, p.b_expert_bytes);
    const int pbase = uniform((int)((int64_t)q * kBNP * p.b_panel_bytes));

    auto src_row = [&](int r) -> int {  // activation row of tile row r (valid r)
      const int rr = row0 + r;
      if (!p.gather) return rr;
      return rr >= p.shared_row0 ? rr - p.shared_row0 : p.sorted_assign[rr] / p.top_k;
    };
    // Activation copy k of a wave covers rows (wave*A_DMA + k)*ROWS_PER_COPY
    // + [0, ROWS_PER_COPY); lane i -> row +i/SLOTS, LDS slot i%SLOTS holding
    // 16-byte part index pi = slot ^ swz(row); with two slots per super-step,
    // index pi of slot h is part (pi&1) + 2h + 4(pi>>1) (+32h rides in soffset).
    int avoff[A_DMA];
#pragma unroll
    for (int k = 0; k < A_DMA; ++k) {
      const int r = (wave * A_DMA + k) * ROWS_PER_COPY + lane / SLOTS;
      const int pi = (lane % SLOTS) ^ swz<RB>(r);
      const int part = SUB == 1 ? pi : (pi & 1) + 4 * (pi >> 1);
      avoff[k] = r < rows ? (int)((int64_t)src_row(r) * p.a_row_bytes) + part * 16 : oobA;
    }
    // FP8 activation scales: waves below S_COPIES copy 64 rows each (16 bytes
    // = the scales of 4 super-steps per row, the first used); the others copy
    // zeros into a sink so every wave issues the same number of copies
    int svoff = oobS;
    if (DT == kFP8) {
      const int r = wave * 64 + lane;
      if (wave < S_COPIES && r < rows) svoff = src_row(r) * p.a_scale_ld * 4;
    }

    // copy ring step t (super-step t / SUB, part t % SUB) into slot t % NS;
    // `in` false (prologue of very short reductions only) copies zeros
    auto issue = [&](int t, bool in) {
      uint8_t* st = smem + (t % NS) * STAGE;
      const int c = t / SUB, h = t % SUB;
#pragma unroll
      for (int k = 0; k < B_DMA; ++k) {
        const int i = wave * B_DMA + k, panel = i / JJ, j = i % JJ;
        const int so = in ? pbase + panel * bpanel + c * kStepPanelBytes + (h * JJ + j) * 1024 : oobB;
        if (DT == kBF16 && AFD_TILED_B_NT)
          dma16_nt(rb, st + B_OFF + panel * PB + j * 1024, lane * 16, so);
        else
          dma16(rb, st + B_OFF + panel * PB + j * 1024, lane * 16, so);
      }
#pragma unroll
      for (int k = 0; k < A_DMA; ++k)
        dma16(ra, st + A_OFF + (wave * A_DMA + k) * 1024, avoff[k], in ? c * kStepBytes + 32 * h : oobA);
      // 16-byte copies: the compiler tracks 4-byte LDS copies and would drain
      // every in-flight load before the next LDS read
      if (DT == kFP8)
        dma16(rsa, wave < S_COPIES ? st + S_OFF + wave * 1024 : smem + SINK, svoff, in ? c * 4 : oobS);
    };

    // accumulators: bf16 [WR/32 row frags][NPW panels] of 32x32; FP8 [WR/16
    // token sub-tiles][2 panels x 2 halves] of 16x16
    constexpr int NA = DT == kBF16 ? WR / 32 : WR / 16;
    constexpr int NB = DT == kBF16 ? NPW : 2 * NPW;
    typedef typename std::conditional<DT == kBF16, f32x16, f32x4>::type acc_t;
    constexpr int NR = DT == kBF16 ? 16 : 4;
    acc_t acc[NA][NB];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[a][b][r] = 0.0f;

    // FP8 weight block scales, one per super-step (see BlockScales): gate/up
    // -> block q of gate (panel 2wn) and up (panel 2wn+1); down -> block
    // (8q + 2wn) / 4 for both panels
    BlockScales sbs;
    if (DT == kFP8) {
      const int64_t eoff = (int64_t)expert * p.b_scale_rows * p.b_scale_cols;
      if (GATEUP)
        sbs.load(p.b_scales0 + eoff + q, p.b_scales1 + eoff + q, p.b_scale_cols, ks, lane);
      else
        sbs.load(p.b_scales0 + eoff + (8 * q + 2 * wn) / 4, p.b_scales0 + eoff + (8 * q + 2 * wn) / 4,
                 p.b_scale_cols, ks, lane);
    }

    auto compute = [&](const uint8_t* st, int t) {
      const uint8_t* Bs = st + B_OFF;
      const uint8_t* As = st + A_OFF;
      if constexpr (DT == kBF16) {
        // slot t holds MFMAs j = JJ(t%SUB) + jj of its super-step
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
          bf16x8 af[NA], bfr[NPW];
#pragma unroll
          for (int mr = 0; mr < NA; ++mr) {
            const int r = wm * WR + mr * 32 + (lane & 31);
            const int pi = SUB == 1 ? (lane >> 5) * 4 + jj : jj + 2 * (lane >> 5);
            af[mr] = *reinterpret_cast<const bf16x8*>(As + r * RB + (pi ^ swz<RB>(r)) * 16);
          }
#pragma unroll
          for (int pp = 0; pp < NPW; ++pp)
            bfr[pp] = *reinterpret_cast<const bf16x8*>(Bs + (wn * NPW + pp) * PB + jj * 1024 + lane * 16);
#pragma unroll
          for (int mr = 0; mr < NA; ++mr)
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp)
              acc[mr][pp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[pp], af[mr], acc[mr][pp], 0, 0, 0);
        }
      } else {
        const float* S = reinterpret_cast<const float*>(st + S_OFF);
        const int c = t;  // one slot per super-step
        const int cs = c < ks ? c : ks - 1;
        const float sbv[2] = {sbs.get0(cs), sbs.get1(cs)};
        const int kg = lane >> 4;  // which 32 bytes of the 128-deep block this lane carries
        const int g = kg >> 1, j0 = (kg & 1) * 2;
        i32x8 w[2][2];
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const uint8_t* lo = Bs + (2 * wn + pl) * PB + j0 * 1024 + (16 * s + (lane & 15) + 32 * g) * 16;
            w[pl][s] = cat32v(*reinterpret_cast<const i32x4*>(lo), *reinterpret_cast<const i32x4*>(lo + 1024));
          }
#pragma unroll
        for (int ts = 0; ts < NA; ++ts) {
          const int r = wm * WR + ts * 16 + (lane & 15);
          const int s0 = (2 * kg) ^ swz<RB>(r), s1 = (2 * kg + 1) ^ swz<RB>(r);
          const i32x8 x = cat32v(*reinterpret_cast<const i32x4*>(As + r * RB + s0 * 16),
                                 *reinterpret_cast<const i32x4*>(As + r * RB + s1 * 16));
          const float sa = S[4 * r];
#pragma unroll
          for (int pl = 0; pl < 2; ++pl) {
            const float sc = sa * sbv[pl];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              f32x4 tt = {0.0f, 0.0f, 0.0f, 0.0f};
              tt = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[pl][s], x, tt, 0, 0, 0, 0, 0, 0);
#pragma unroll
              for (int r4 = 0; r4 < 4; ++r4) acc[ts][pl * 2 + s][r4] += tt[r4] * sc;
            }
          }
        }
      }
    };

    // Prologue fills NS-1 slots; the steady loop (branch-free, so the
    // accumulators stay put) waits for its slot, barriers, refills the slot
    // freed by the previous step and multiplies; the last NS-1 steps drain
    // with shrinking waits.
    const int nsteps = ks * SUB;
#pragma unroll
    for (int i = 0; i + 1 < NS; ++i) issue(i, i < nsteps);
    int t = 0;
    for (; t + NS - 1 < nsteps; ++t) {
      wait_vmcnt<(NS - 2) * PER_STAGE>();  // this wave's copies of step t have landed
      raw_barrier();                        // ... and every wave's; slot of t-1 is free
      issue(t + NS - 1, true);
      compute(smem + (t % NS) * STAGE, t);
    }
    for (; t < nsteps; ++t) {  // drain: steps t+1 .. nsteps-1 are still in flight
      const int younger = nsteps - 1 - t;
      if (NS > 3 && younger >= 2)
        wait_vmcnt<(NS > 3 ? 2 : 0) * PER_STAGE>();
      else if (younger == 1)
        wait_vmcnt<PER_STAGE>();
      else
        wait_vmcnt<0>();
      raw_barrier();
      compute(smem + (t % NS) * STAGE, t);
    }
    wait_vmcnt<0>();  // prologue copies past the end (very short reductions)
    raw_barrier();    // every wave is done with the ring before the next task refills it

    // ------------------------------------------------------------- epilogue
    if constexpr (DT == kBF16) {
#pragma unroll
      for (int mr = 0; mr < NA; ++mr) {
        const int m = wm * WR + mr * 32 + (lane & 31);
        if (m >= rows) continue;
        uint8_t* orow = p.c + (int64_t)(row0 + m) * p.c_row_bytes;
#pragma unroll
        for (int pp = 0; pp < NPW; pp += (GATEUP ? 2 : 1)) {
          const int P = q * kBNP + wn * NPW + pp;  // packed panel index (gate/up: 2 per unit)
          if (P >= (GATEUP ? 2 * p.n_panels : p.n_panels)) continue;
          const int col0 = GATEUP ? 32 * (P / 2) : 32 * P;
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int n = 8 * r4 + 4 * (lane >> 5);
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = GATEUP ? silu_mul(acc[mr][pp][4 * r4 + e], acc[mr][pp + 1][4 * r4 + e]) : acc[mr][pp][4 * r4 + e];
            uint2 o;
            o.x = pack_bf16x2(v[0], v[1]);
            o.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<uint2*>(orow + (int64_t)(col0 + n) * 2) = o;
          }
        }
      }
    } else if constexpr (GATEUP) {
      // h for unit u = 4q + wn: gate sub-panels 0,1 and up sub-panels 2,3;
      // row amax over the task's 128 h columns = over the WN waves of a row half
      const int kg = lane >> 4;
      float h[NA][2][4];
#pragma unroll
      for (int ts = 0; ts < NA; ++ts) {
        float a = 0.0f;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            h[ts][s][r4] = silu_mul(acc[ts][s][r4], acc[ts][2 + s][r4]);
            a = fmaxf(a, fabsf(h[ts][s][r4]));
          }
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        a = fmaxf(a, __shfl_xor(a, 32, 64));
        if (kg == 0) red[wm][wn][ts * 16 + (lane & 15)] = a;
      }
      __syncthreads();
      const int u = 4 * q + wn;
#pragma unroll
      for (int ts = 0; ts < NA; ++ts) {
        const int mi = ts * 16 + (lane & 15);
        const int m = wm * WR + mi;
        float amax = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < WN; ++w2) amax = fmaxf(amax, red[wm][w2][mi]);
        const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
        const float inv = amax > 0.0f ? 448.0f / amax : 1.0f;
        if (m < rows) {
          uint8_t* orow = p.c + (int64_t)(row0 + m) * p.c_row_bytes + 32 * u;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = fminf(fmaxf(h[ts][s][e] * inv, -448.0f), 448.0f);
            *reinterpret_cast<uint32_t*>(orow + 16 * s + 4 * kg) = pack_fp8x4(v[0], v[1], v[2], v[3]);
          }
          if (wn == 0 && kg == 0) p.c_scales[(int64_t)(row0 + m) * p.c_scale_ld + q] = scale;
        }
      }
      __syncthreads();  // red[] is rewritten by the next task
    } else {
      const int kg = lane >> 4;
#pragma unroll
      for (int ts = 0; ts < NA; ++ts) {
        const int m = wm * WR + ts * 16 + (lane & 15);
        if (m >= rows) continue;
        uint8_t* orow = p.c + (int64_t)(row0 + m) * p.c_row_bytes;
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
          const int P = q * kBNP + 2 * wn + pl;
          if (P >= p.n_panels) continue;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int col = 32 * P + 16 * s + 4 * kg;
            uint2 o;
            o.x = pack_bf16x2(acc[ts][pl * 2 + s][0], acc[ts][pl * 2 + s][1]);
            o.y = pack_bf16x2(acc[ts][pl * 2 + s][2], acc[ts][pl * 2 + s][3]);
            *reinterpret_cast<uint2*>(orow + (int64_t)col * 2) = o;
          }
        }
      }
    }
  }
}

template <int DT, bool GATEUP>
static hipError_t launch_tiled_one(const GemmParams& p, int64_t max_tasks, int num_cus, hipStream_t s) {
  constexpr int lds = lds_bytes<DT>();
  constexpr int threads = Tiled<DT>::NW * 64;
  static int per_cu = 0;
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tiled_kernel<DT, GATEUP>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_tiled_kernel<DT, GATEUP>, threads, lds) !=
            hipSuccess ||
        occ <= 0)
      occ = 1;
    per_cu = occ;
  }
  const int64_t grid = std::min<int64_t>(max_tasks, (int64_t)num_cus * per_cu);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_tiled_kernel<DT, GATEUP>), dim3((unsigned)grid), dim3(threads), lds, s, p);
  return hipGetLastError();
}

int tiled_rows(int dtype) { return dtype == kFP8 ? Tiled<kFP8>::BM : Tiled<kBF16>::BM; }

hipError_t launch_gemm_tiled(int dtype, bool gate_up, const GemmParams& p, int64_t max_tasks, int num_cus,
                             hipStream_t s) {
  if (dtype == kBF16) return gate_up ? launch_tiled_one<kBF16, true>(p, max_tasks, num_cus, s)
                                     : launch_tiled_one<kBF16, false>(p, max_tasks, num_cus, s);
  if (dtype == kFP8) return gate_up ? launch_tiled_one<kFP8, true>(p, max_tasks, num_cus, s)
                                    : launch_tiled_one<kFP8, false>(p, max_tasks, num_cus, s);
  return hipErrorInvalidValue;
}

}  // namespace afd
