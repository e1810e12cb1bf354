// gemm_ring.hip -- block-FP8 grouped expert GEMMs fed by a weight ring in LDS.
//
// Same two GEMMs as gemm.hip / gemm_tiled.hip (gate/up with SwiGLU and the
// 1x128 re-quantisation of h, then down), for block-FP8 layers.  On the
// FFN-side GPU of a decode batch the expert weights are read once per layer
// and each weight byte feeds only tens to a few hundred rows ("FastAFD" design
// space: expert FFN time is weight reads plus the grouped GEMM), so these GEMMs
// are bound by HBM, and HBM only delivers its bandwidth with enough bytes in
// flight: at a few microseconds of loaded latency, on the order of 100 KiB per
// CU.
//
// A workgroup task is one m-tile (at most BM rows of one expert) times 8
// weight panels (256 GEMM columns).  Only the weights pass through LDS: the
// buffer unit copies each 128-deep super-step of the 8 panels (32 KiB) straight
// into a ring of NS slots, so NS-1 super-steps (96 KiB at NS = 4) are in flight
// per CU without holding a register.  The activation rows are small and served
// from cache; each wave loads its own two 16-row token tiles straight into MFMA
// operand registers, NS-1 steps ahead as well.  Their 1x128 scales are stored
// step-major in sorted-row order (by the dispatch for the hidden rows, by the
// gate/up epilogue for h), so one step's scales of a tile are one contiguous
// run that a single copy brings into the ring slot.  (A scalar loaded into a
// rotating register stage would cost a register copy, and the wait before that
// copy would drain the younger steps; one 16-byte load per row and step would
// spend as many cache-line requests as the activation rows themselves.)
// The steady loop is unrolled by NS so every register stage has a static
// index, and is branch-free: steps past the end load at out-of-range offsets,
// which the buffer unit returns as zeros (exact zero products), so one wait
// count serves every step.
//
// The copy engine's LDS writes are invisible to the compiler, so the kernel
// orders them itself: s_waitcnt vmcnt(N), N = the loads of the younger steps
// still allowed in flight, then a barrier; the slot refilled after the barrier
// is the one every wave finished reading one step earlier.
//
// MFMA 16x16x128 e4m3 (one instruction spans a whole scale block): weight
// fragment first, token fragment second, so lane l holds token l % 16 and
// output columns 4(l / 16) + r of a 16-column half panel; the product is added
// into the accumulator times (token scale x block scale).  Eight waves, two per
// SIMD, as WM x WN = (BM / 32) x (8 / (BM / 32)): each wave owns 32 rows and
// 8 / WN panels.
#include <algorithm>

#include "afd_device.h"

namespace afd {

using namespace dev;

namespace {

#ifndef AFD_RING_NS
#define AFD_RING_NS 4
#endif
#ifndef AFD_RING_B_AUX
#define AFD_RING_B_AUX 0  // cache policy of the weight copies
#endif
#ifndef AFD_RING_XCD_REMAP
#define AFD_RING_XCD_REMAP 1
#endif

constexpr int kRingWaves = 8;
constexpr int kRingPanels = 8;
constexpr int kRingWeightBytes = kRingPanels * kStepPanelBytes;  // 32 KiB per step

constexpr int kRingSlotBytes = kRingWeightBytes + 1024;  // + the tile's row scales of the step
constexpr int kRingLdsBytes = AFD_RING_NS * kRingSlotBytes + 1024;  // + sink of idle scale copies
constexpr int kRingNS = AFD_RING_NS;
constexpr int kRingMB = 4;  // m-tiles per rasterisation block

__device__ inline int clamp31(int64_t v) { return v > 0x7fffffff ? 0x7fffffff : (int)v; }

}  // namespace

// One task: m-tile `tile` (at most BM rows) x column group q.  Every wave of
// the workgroup calls it with the same arguments.
template <bool GATEUP, int BM>
__device__ __forceinline__ void ring_task(const GemmParams& p, const int4 tile, const int q) {
  // declared here, not passed in: the copies need pointers known to be in LDS
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  __shared__ float red[kRingWaves * 32];  // gate/up: per-wave token amax
  constexpr int NS = kRingNS;
  constexpr int WM = BM / 32, WN = kRingWaves / WM, NPW = kRingPanels / WN;
  constexpr int RT = 2;                                   // 16-row token tiles per wave
  constexpr int B_DMA = kRingPanels * 4 / kRingWaves;     // 1 KiB weight copies per wave and step
  constexpr int PER_STAGE = B_DMA + 2 * RT + 1;           // + two 16-byte row loads per tile + scales
  constexpr int SLOT = kRingSlotBytes;
  constexpr int S_OFF = kRingWeightBytes;
  constexpr int SINK = NS * SLOT;
  static_assert(WM * WN == kRingWaves && NPW % 2 == 0 && NPW <= 4 && BM <= 256, "wave grid");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int kg = lane >> 4;  // which 32 bytes of the 128-deep block this lane carries
  const int tok = lane & 15;
  const int ks = p.k_steps;
  const int nsr = (ks + NS - 1) / NS * NS;  // steps run: whole unrolled rounds
  const int oobA = clamp31(p.a_bytes), oobS = clamp31(p.a_scale_bytes);
  const int oobB = (int)p.b_expert_bytes;
  const int bpanel = (int)p.b_panel_bytes;
  const auto ra = make_rsrc(p.a, p.a_bytes);
  const auto rsa = make_rsrc(p.a_scales, p.a_scale_bytes);

  {
    const int expert = uniform(tile.x), row0 = uniform(tile.y), rows = uniform(tile.z);
    const auto rb = make_rsrc(p.b + (int64_t)expert * p.b_expert_bytes, p.b_expert_bytes);
    const int pbase = uniform((int)((int64_t)q * kRingPanels * p.b_panel_bytes));

    // this lane's token of each tile (rows past the count repeat the tile's
    // first row: computed, never stored)
    auto src_row = [&](int r) -> int {  // activation row of sorted row r
      return !p.gather ? r : r >= p.shared_row0 ? r - p.shared_row0 : p.sorted_assign[r] / p.top_k;
    };
    int aoff[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int m = wm * 32 + rt * 16 + tok;
      aoff[rt] = (int)((int64_t)src_row(row0 + (m < rows ? m : 0)) * p.a_row_bytes) + 32 * kg;
    }
    // scales: wave 0 copies the step's run of the tile's rows (lane i: rows
    // 4i .. 4i+3); the others copy zeros into a sink so every wave counts the
    // same loads per step
    const int svoff = (wave == 0 && 4 * lane < BM) ? (row0 + 4 * lane) * 4 : oobS;
    const int sstep = p.a_scale_ld * 4;

    // weight block scales, one per super-step: gate/up -> block q of gate (even
    // panels) and up (odd panels); down -> the block of this wave's panels
    BlockScales sbs;
    {
      const int64_t eoff = (int64_t)expert * p.b_scale_rows * p.b_scale_cols;
      if (GATEUP)
        sbs.load(p.b_scales0 + eoff + q, p.b_scales1 + eoff + q, p.b_scale_cols, ks, lane);
      else
        sbs.load(p.b_scales0 + eoff + (kRingPanels * q + NPW * wn) / 4,
                 p.b_scales0 + eoff + (kRingPanels * q + NPW * wn) / 4, p.b_scale_cols, ks, lane);
    }

    f32x4 acc[RT][2 * NPW];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int b = 0; b < 2 * NPW; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[rt][b][r] = 0.0f;

    i32x4 areg[NS][RT][2];

    // step c into ring slot `slot` and register stage `slot`
    auto issue = [&](int c, int slot) {
      const bool in = c < ks;
      uint8_t* st = ring + slot * SLOT;
#pragma unroll
      for (int k = 0; k < B_DMA; ++k) {
        const int i = wave * B_DMA + k, panel = i / 4, j = i % 4;
        dma16_aux<AFD_RING_B_AUX>(rb, st + panel * kStepPanelBytes + j * 1024, lane * 16,
                                  in ? pbase + panel * bpanel + c * kStepPanelBytes + j * 1024 : oobB);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        areg[slot][rt][0] = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[rt], in ? c * kStepBytes : oobA, 0);
        areg[slot][rt][1] = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[rt], in ? c * kStepBytes + 16 : oobA, 0);
      }
      dma16(rsa, wave == 0 ? st + S_OFF : ring + SINK, svoff, in ? c * sstep : oobS);
    };

    auto compute = [&](int slot, int c) {
      const uint8_t* Bs = ring + slot * SLOT;
      const float* S = reinterpret_cast<const float*>(Bs + S_OFF);
      float sa[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sa[rt] = S[wm * 32 + rt * 16 + tok];
      const int cs = c < ks ? c : ks - 1;
      const float sb0 = sbs.get0(cs), sb1 = sbs.get1(cs);
      i32x8 x[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) x[rt] = cat32v(areg[slot][rt][0], areg[slot][rt][1]);
      // weight fragment of a 16-column half panel: K bytes 32 kg .. +32 are
      // 1 KiB chunks 2(kg & 1), +1 of the panel's lane half kg >> 1
      const int g = kg >> 1, j0 = (kg & 1) * 2;
#pragma unroll
      for (int pp = 0; pp < NPW; ++pp) {
        const float sb = (GATEUP && (pp & 1)) ? sb1 : sb0;
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          const uint8_t* lo = Bs + (wn * NPW + pp) * kStepPanelBytes + j0 * 1024 + (16 * sh + tok + 32 * g) * 16;
          const i32x8 w = cat32v(*reinterpret_cast<const i32x4*>(lo), *reinterpret_cast<const i32x4*>(lo + 1024));
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
            t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x[rt], t, 0, 0, 0, 0, 0, 0);
            const float sc = sa[rt] * sb;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) acc[rt][pp * 2 + sh][r4] += t[r4] * sc;
          }
        }
      }
    };

    // The loads of one step stay together (scheduling fences): the wait
    // counter retires loads in order, so a step's loads mixed into a younger
    // step's would make the register waits drain that younger step.
#pragma unroll
    for (int i = 0; i + 1 < NS; ++i) {
      issue(i, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int t0 = 0; t0 < nsr; t0 += NS) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        wait_vmcnt<(NS - 2) * PER_STAGE>();  // step t0 + i has landed (this wave's copies) ...
        lds_reads_done();
        raw_barrier();                       // ... and every wave's; slot of the previous step is free
        issue(t0 + i + NS - 1, (i + NS - 1) % NS);
        __builtin_amdgcn_sched_barrier(0);
        compute(i, t0 + i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_vmcnt<0>();  // the out-of-range steps issued past the end
    lds_reads_done();
    raw_barrier();    // every wave is done with the ring before the next task refills it

    // ------------------------------------------------------------- epilogue
    if constexpr (GATEUP) {
      // h of unit u = 4q + (wn NPW + pp) / 2 (pp even: gate, pp + 1: up), per
      // token amax over the task's 128 h columns: this wave's, then over WN
      float h[RT][NPW / 2][2][4];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float a = 0.0f;
#pragma unroll
        for (int u = 0; u < NPW / 2; ++u)
#pragma unroll
          for (int sh = 0; sh < 2; ++sh)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const float v = silu_mul(acc[rt][4 * u + sh][r4], acc[rt][4 * u + 2 + sh][r4]);
              h[rt][u][sh][r4] = v;
              a = fmaxf(a, fabsf(v));
            }
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        a = fmaxf(a, __shfl_xor(a, 32, 64));
        if (kg == 0) red[(wm * WN + wn) * 32 + rt * 16 + tok] = a;
      }
      __syncthreads();
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int mi = rt * 16 + tok;
        const int m = wm * 32 + mi;
        float amax = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < WN; ++w2) amax = fmaxf(amax, red[(wm * WN + w2) * 32 + mi]);
        const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
        const float inv = amax > 0.0f ? 448.0f / amax : 1.0f;
        if (m < rows) {
          uint8_t* orow = p.c + (int64_t)(row0 + m) * p.c_row_bytes;
#pragma unroll
          for (int u = 0; u < NPW / 2; ++u) {
            const int unit = 4 * q + (wn * NPW) / 2 + u;
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = fminf(fmaxf(h[rt][u][sh][e] * inv, -448.0f), 448.0f);
              *reinterpret_cast<uint32_t*>(orow + 32 * unit + 16 * sh + 4 * kg) = pack_fp8x4(v[0], v[1], v[2], v[3]);
            }
          }
          if (wn == 0 && kg == 0) p.c_scales[(int64_t)q * p.c_scale_ld + row0 + m] = scale;
        }
      }
      __syncthreads();  // red[] is rewritten by the next task
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int m = wm * 32 + rt * 16 + tok;
        if (m >= rows) continue;
        uint8_t* orow = p.c + (int64_t)(row0 + m) * p.c_row_bytes;
#pragma unroll
        for (int pp = 0; pp < NPW; ++pp) {
          const int P = q * kRingPanels + wn * NPW + pp;
          if (P >= p.n_panels) continue;
#pragma unroll
          for (int sh = 0; sh < 2; ++sh) {
            const int col = 32 * P + 16 * sh + 4 * kg;
            uint2 o;
            o.x = pack_bf16x2(acc[rt][pp * 2 + sh][0], acc[rt][pp * 2 + sh][1]);
            o.y = pack_bf16x2(acc[rt][pp * 2 + sh][2], acc[rt][pp * 2 + sh][3]);
            *reinterpret_cast<uint2*>(orow + (int64_t)col * 2) = o;
          }
        }
      }
    }
  }
}

// Both tile lists in one persistent launch: the heavy list's tasks (m-tiles
// of up to 128 rows), then the light list's (up to 64 rows), so a GEMM stage
// has one tail instead of two.  Tasks run in blocks of kRingMB m-tiles x all
// column groups; workgroup ranks are renumbered so that each XCD owns a
// contiguous run of tasks (shared rows stay in its L2).
template <bool GATEUP>
__global__ __launch_bounds__(kRingWaves * 64, 1) void gemm_ring_kernel(GemmParams p) {
  const int nq = p.n_groups;
  const int nh = uniform(p.num_mtiles2 ? p.num_mtiles2[0] : 0);
  const int nl = uniform(p.num_mtiles[0]);
  const int th = nh * nq, tl = nl * nq;
  const int G = gridDim.x;
  const int rank = (AFD_RING_XCD_REMAP && G % kXcds == 0) ? (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds
                                                          : blockIdx.x;
  // task t of a list of n m-tiles -> (m-tile, column group)
  auto decode = [&](int t, int n, int& mt, int& q) {
    const int full = (n / kRingMB) * kRingMB * nq;
    if (t < full) {
      const int blk = t / (kRingMB * nq), w = t % (kRingMB * nq);
      q = w / kRingMB;
      mt = blk * kRingMB + w % kRingMB;
    } else {
      const int rem = n % kRingMB, u = t - full;
      q = u / rem;
      mt = (n / kRingMB) * kRingMB + u % rem;
    }
  };
  for (int task = rank; task < th + tl; task += G) {
    int mt, q;
    if (task < th) {
      decode(task, nh, mt, q);
      ring_task<GATEUP, 128>(p, p.mtiles2[mt], q);
    } else {
      decode(task - th, nl, mt, q);
      ring_task<GATEUP, 64>(p, p.mtiles[mt], q);
    }
  }
}

template <bool GATEUP>
static hipError_t launch_ring_one(const GemmParams& p, int64_t max_tasks, int num_cus, hipStream_t s) {
  constexpr int lds = kRingLdsBytes;
  static int per_cu = 0;
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_ring_kernel<GATEUP>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_ring_kernel<GATEUP>, kRingWaves * 64, lds) !=
            hipSuccess ||
        occ <= 0)
      occ = 1;
    per_cu = occ;
  }
  const int64_t grid = std::min<int64_t>(max_tasks, (int64_t)num_cus * per_cu);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_ring_kernel<GATEUP>), dim3((unsigned)grid), dim3(kRingWaves * 64), lds, s, p);
  return hipGetLastError();
}

int ring_rows(bool heavy) { return heavy ? 128 : 64; }

hipError_t launch_gemm_ring(bool gate_up, const GemmParams& p, int64_t max_tasks, int num_cus, hipStream_t s) {
  return gate_up ? launch_ring_one<true>(p, max_tasks, num_cus, s) : launch_ring_one<false>(p, max_tasks, num_cus, s);
}

}  // namespace afd
