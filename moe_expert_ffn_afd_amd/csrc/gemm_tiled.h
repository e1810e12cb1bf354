#pragma once
// gemm_tiled.h -- LDS-tiled grouped expert GEMMs for experts with many rows:
// the workgroup body, shared by the mixed kernel (gemm_tiled.hip) and the
// fused bf16 layer kernel (fused_bf16.hip).
//
// Same two GEMMs as gemm.hip (gate/up with SwiGLU, then down), bf16, for the
// m-tiles of "heavy" experts (rows >= a threshold): aggregated AFD batches
// concentrate tokens on popular experts ("FastAFD" summary, speculative
// decoding multiplies routed expert work; design-space study: expert FFNs are
// compute-intensive), where each weight panel must feed many rows and the MFMA
// pipes, not HBM, set the pace.
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
// LDS layout of a slot: weight panels exactly as packed in HBM (fragment
// order: conflict-free 16-byte reads), then activation rows of 64 bytes (half
// a super-step) with the four 16-byte parts of row r permuted by
// part ^ ((r >> 2) & 3) (so the rows of an MFMA fragment read spread over all
// banks).
//
// Tile 256 x 256, 8 waves (two per SIMD) as 4 x 2 of 64 rows x 4 panels, MFMA
// 32x32x16, 128 fp32 accumulators per lane; two slots of a whole super-step
// (64 KiB each), one copied while the other is multiplied: one barrier per
// super-step (four slots of half a super-step, three in flight, were 1-2 %
// slower: twice the barriers, and the copies hit in L2 anyway).  (Block-FP8 layers run
// gemm_ring.hip.)
//
// The kernels launched are gemm_mixed_kernel and the fused layer kernel: one
// 8-wave workgroup per CU, of which the dispatch gives a share to the light
// list (the streaming body of gemm_stream.h, as two 4-wave halves) and the
// rest to the heavy tiles, so the HBM-bound light experts and the MFMA-bound
// heavy ones run at the same time on disjoint CUs.
#include <algorithm>

#include "afd_device.h"

namespace afd {

using namespace dev;

namespace {

#ifndef AFD_TILED_NW
#define AFD_TILED_NW 8
#endif
#ifndef AFD_TILED_WM
#define AFD_TILED_WM 4
#endif
#ifndef AFD_TILED_NS
#define AFD_TILED_NS 2
#endif
#ifndef AFD_TILED_B_NT
#define AFD_TILED_B_NT 0  // 1: weight copies non-temporal (panels are re-read by sibling m-tiles)
#endif
#ifndef AFD_TILED_XCD_REMAP
#define AFD_TILED_XCD_REMAP 1
#endif
#ifndef AFD_TILED_MB
#define AFD_TILED_MB 4  // m-tiles per rasterisation block
#endif
#ifndef AFD_TILED_POOL
#define AFD_TILED_POOL 1  // the heavy list's last tasks claimed by the workgroups done first
#endif

// NW waves form a WM x WN grid over BM rows x 8 panels; SUB ring slots per
// super-step (a slot holds 128/SUB bytes of K per row).
#ifndef AFD_TILED_SUB
#define AFD_TILED_SUB 1
#endif
constexpr int kNW = AFD_TILED_NW, kWM = AFD_TILED_WM, kWN = kNW / kWM, kBM = 256, kNS = AFD_TILED_NS,
              kSUB = AFD_TILED_SUB;
#ifndef AFD_TILED_BNP
#define AFD_TILED_BNP 8
#endif
constexpr int kBNP = AFD_TILED_BNP;  // panels per task
constexpr int kMB = AFD_TILED_MB;
constexpr int kStage = (kBNP * kStepPanelBytes + kBM * kStepBytes) / kSUB;
constexpr int kLds = kNS * kStage;

__device__ inline int clamp31(int64_t v) { return v > 0x7fffffff ? 0x7fffffff : (int)v; }

// LDS slot permutation of activation row r (rows of RB bytes, RB/16 parts):
// 16 consecutive rows reading the same 16-byte part hit 16 distinct
// (row, part) bank groups, i.e. all 64 banks.
template <int RB>
__device__ inline int swz(int r) {
  return RB == 128 ? (r >> 1) & 7 : (r >> 2) & 3;
}

}  // namespace

// The heavy tasks first, first + stride, ... below the pool, then pool tasks
// claimed one at a time until none is left.  The pool is the list's last
// min(tasks, Gh) tasks (Gh: the workgroups with a static share), claimed from
// the counter p.pool[stage] (zeroed by the dispatch) by every workgroup done
// with its own work, the light ones included: tasks take about 120 us
// (gate/up) and a static share of 8.4 tasks leaves some workgroups a whole
// task behind the others.  first past the static tasks: pool tasks only.
template <bool GATEUP>
__device__ __forceinline__ void tiled_tasks(const GemmParams& p, const int first, const int stride, const int Gh) {
  constexpr int NW = kNW, WM = kWM, WN = kWN, BM = kBM, NS = kNS, SUB = kSUB;
  constexpr int RB = kStepBytes / SUB;        // activation bytes per row and slot
  constexpr int PB = kStepPanelBytes / SUB;   // weight bytes per panel and slot
  constexpr int JJ = 4 / SUB;                 // 1 KiB chunks per panel and slot
  constexpr int B_OFF = 0, A_OFF = kBNP * PB;
  constexpr int STAGE = kStage;
  constexpr int ROWS_PER_COPY = 1024 / RB;
  constexpr int SLOTS = RB / 16;
  constexpr int B_DMA = kBNP * JJ / NW;                 // copies per wave and slot
  constexpr int A_DMA = BM * RB / 1024 / NW;
  constexpr int PER_STAGE = B_DMA + A_DMA;
  constexpr int WR = BM / WM;                           // rows per wave
  constexpr int NPW = kBNP / WN;                        // panels per wave
  constexpr int NA = WR / 32;                           // 32-row fragments per wave
  static_assert(B_DMA * NW == kBNP * JJ && A_DMA * NW * 1024 == BM * RB, "copy split");
  static_assert(NPW % 2 == 0, "a wave holds whole gate/up panel pairs");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);  // scalar: LDS copy targets must be wave-uniform
  const int wm = wave / WN, wn = wave % WN;
  const int num_mt = uniform(p.num_mtiles[0]);
  const int num_tasks = num_mt * p.n_groups;
  const int ks = p.k_steps;
  const int oobA = clamp31(p.a_bytes);
  const int oobB = (int)p.b_expert_bytes;
  const int bpanel = (int)p.b_panel_bytes;
  const auto ra = make_rsrc(p.a, p.a_bytes);

  const int nq = p.n_groups;
  const int full = (num_mt / kMB) * kMB * nq;  // tasks in complete blocks
  const int rem = num_mt % kMB;
  const int pool = (AFD_TILED_POOL && p.pool) ? min(num_tasks, Gh) : 0;
  const int limit = num_tasks - pool;  // static tasks below, pool tasks from here
  __shared__ int claim_slot;
  auto claim = [&]() -> int {  // every thread calls it
    if (pool == 0) return num_tasks;
    if (tid == 0)
      claim_slot = __hip_atomic_fetch_add(p.pool + (GATEUP ? 0 : 1), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int c = uniform(claim_slot);
    __syncthreads();  // claim_slot is rewritten by the next claim
    return c < pool ? limit + c : num_tasks;
  };
  int task = first < limit ? first : claim();
  while (task < num_tasks) {
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
      return rr >= p.shared_row0 ? (rr - p.shared_row0) % p.shared_tokens : p.sorted_assign[rr] / p.top_k;
    };
    // Activation copy k of a wave covers rows (wave*A_DMA + k)*ROWS_PER_COPY
    // + [0, ROWS_PER_COPY); lane i -> row +i/SLOTS, LDS part i%SLOTS holding
    // 16-byte part index pi = part ^ swz(row); with two slots per super-step,
    // index pi of slot h is part (pi&1) + 2h + 4(pi>>1) (+32h rides in soffset).
    int avoff[A_DMA];
#pragma unroll
    for (int k = 0; k < A_DMA; ++k) {
      const int r = (wave * A_DMA + k) * ROWS_PER_COPY + lane / SLOTS;
      const int pi = (lane % SLOTS) ^ swz<RB>(r);
      const int part = SUB == 1 ? pi : (pi & 1) + 4 * (pi >> 1);
      avoff[k] = r < rows ? (int)((int64_t)src_row(r) * p.a_row_bytes) + part * 16 : oobA;
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
        if (AFD_TILED_B_NT)
          dma16_nt(rb, st + B_OFF + panel * PB + j * 1024, lane * 16, so);
        else
          dma16(rb, st + B_OFF + panel * PB + j * 1024, lane * 16, so);
      }
#pragma unroll
      for (int k = 0; k < A_DMA; ++k)
        dma16(ra, st + A_OFF + (wave * A_DMA + k) * 1024, avoff[k], in ? c * kStepBytes + 32 * h : oobA);
    };

    // accumulators: [NA row fragments][NPW panels] of 32x32
    f32x16 acc[NA][NPW];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int b = 0; b < NPW; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    auto compute = [&](const uint8_t* st) {
      const uint8_t* Bs = st + B_OFF;
      const uint8_t* As = st + A_OFF;
      // slot t holds MFMAs j = JJ(t%SUB) + jj of its super-step; the
      // fragments of sub-step jj + 1 are read before the products of jj, so
      // their LDS latency hides behind those MFMAs
      bf16x8 af[2][NA], bfr[2][NPW];
      auto frags = [&](const int jj, const int b) {
#pragma unroll
        for (int mr = 0; mr < NA; ++mr) {
          const int r = wm * WR + mr * 32 + (lane & 31);
          const int pi = SUB == 1 ? (lane >> 5) * 4 + jj : jj + 2 * (lane >> 5);
          af[b][mr] = *reinterpret_cast<const bf16x8*>(As + r * RB + (pi ^ swz<RB>(r)) * 16);
        }
#pragma unroll
        for (int pp = 0; pp < NPW; ++pp)
          bfr[b][pp] = *reinterpret_cast<const bf16x8*>(Bs + (wn * NPW + pp) * PB + jj * 1024 + lane * 16);
      };
      frags(0, 0);
#pragma unroll
      for (int jj = 0; jj < JJ; ++jj) {
        if (jj + 1 < JJ) frags(jj + 1, (jj + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mr = 0; mr < NA; ++mr)
#pragma unroll
          for (int pp = 0; pp < NPW; ++pp)
            acc[mr][pp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[jj & 1][pp], af[jj & 1][mr], acc[mr][pp], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
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
      lds_reads_done();
      raw_barrier();                        // ... and every wave's; slot of t-1 is free
      issue(t + NS - 1, true);
      compute(smem + (t % NS) * STAGE);
    }
    for (; t < nsteps; ++t) {  // drain: steps t+1 .. nsteps-1 are still in flight
      const int younger = nsteps - 1 - t;
      if (NS > 3 && younger >= 2)
        wait_vmcnt<(NS > 3 ? 2 : 0) * PER_STAGE>();
      else if (younger == 1)
        wait_vmcnt<PER_STAGE>();
      else
        wait_vmcnt<0>();
      lds_reads_done();
      raw_barrier();
      compute(smem + (t % NS) * STAGE);
    }
    wait_vmcnt<0>();  // prologue copies past the end (very short reductions)
    lds_reads_done();
    raw_barrier();    // every wave is done with the ring before the next task refills it

    // ------------------------------------------------------------- epilogue
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
        // lanes l and l ^ 32 swap halves: 16-byte stores of 8 columns
        const bool hi = lane >= 32;
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          uint2 o[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int r4 = 2 * r2 + k;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = GATEUP ? silu_mul(acc[mr][pp][4 * r4 + e], acc[mr][pp + 1][4 * r4 + e]) : acc[mr][pp][4 * r4 + e];
            o[k].x = pack_bf16x2(v[0], v[1]);
            o[k].y = pack_bf16x2(v[2], v[3]);
          }
          // (default policy: non-temporal stores of y made this kernel's down
          // launch 14 % slower, unlike the streaming and ring GEMMs')
          store_pair16(orow + (int64_t)(col0 + 16 * r2 + (hi ? 8 : 0)) * 2, o[0], o[1], hi);
        }
      }
    }
    task = task + stride < limit ? task + stride : claim();
  }
}

// The heavy tasks as workgroup b of the G workgroups with a static share.
// Task order: blocks of kMB m-tiles x all column groups, column group outer
// within a block, and workgroup ranks renumbered so each XCD owns a
// contiguous run of tasks.  The ~32 tiles an XCD runs at once then share a few
// activation chunks and weight panels through its L2.
template <bool GATEUP>
__device__ __forceinline__ void tiled_body(const GemmParams& p, const int b, const int G) {
  const int rank = (AFD_TILED_XCD_REMAP && G % kXcds == 0) ? (b % kXcds) * (G / kXcds) + b / kXcds : b;
  tiled_tasks<GATEUP>(p, rank, G, G);
}

// A workgroup done with other work (a light one of the mixed split) helps
// with the heavy pool of the Gh heavy workgroups.  Its LDS use must be over.
template <bool GATEUP>
__device__ __forceinline__ void tiled_pool(const GemmParams& p, const int Gh) {
  if (!AFD_TILED_POOL || !p.pool || Gh <= 0) return;
  __syncthreads();
  tiled_tasks<GATEUP>(p, 0x7fffffff, 1, Gh);
}

}  // namespace afd
