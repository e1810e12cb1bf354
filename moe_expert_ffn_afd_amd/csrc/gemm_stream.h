// gemm_stream.h -- streaming grouped expert GEMMs on MFMA (bf16), gfx950: the
// workgroup body, shared by the light-list kernel (gemm.hip) and the mixed
// heavy + light kernel (gemm_tiled.hip).
//
// The FFN stage time is dominated by expert-weight reads and the grouped GEMM
// over the routed tokens ("FastAFD" structured summary, legend of Eq. (3));
// FastAFD's expert GPUs run grouped GEMMs with the activation fused (System
// Design item 3).  Two GEMMs per expert e with n_e routed rows:
//   gate/up:  h = silu(X_e Wg_e) * (X_e Wu_e)      [n_e, H] x [H, I]
//   down:     y = h_e Wd_e                          [n_e, I] x [I, H]
//
// This body serves the "light" experts of a bf16 layer (at most one tile of
// 32*MR rows): their weights are read once and feed few rows, so it is bound
// by HBM.  Block-FP8 layers run gemm_ring.hip; heavy bf16 experts gemm_tiled.hip.
//
// Work decomposition.  The m-tile list (built on the device by the dispatch)
// holds runs of at most 32*MR rows of one expert.  A workgroup task is one
// m-tile times one group of 4 "units" along N, one unit per wave: for gate/up
// a unit is gate panel p plus up panel p (32 h columns, so a task covers 128
// h columns); for down a unit is NPW adjacent 32-column panels of H (4 for
// single-fragment tiles, else 2).  Every wave streams its own panels over the
// whole reduction straight from HBM into MFMA operand registers (the packed layout
// makes each 16-byte lane load one contiguous KiB per wave), with the next
// super-step's loads in flight while the current one is multiplied.  The
// activation rows are small and shared by the 4 waves: each step's rows are
// copied once per workgroup into LDS (a whole 128-byte row per 8 lanes, so a
// copy costs one cache-line request per row instead of one per row and wave
// and fragment), and each wave reads its fragments from there.
//
// MFMA orientation: the weight fragment is the first operand and the
// activation fragment the second, so the 32x32 accumulator holds out^T: lane l
// owns token column m = l % 32 and 16 output columns n = 8(r/4) + 4(l/32) + r%4
// (r = register).  Gate and up of the same (m, n) sit in the same register of
// two accumulators, so SwiGLU is elementwise.  The rows outside an m-tile's
// count are computed on a duplicate of its first row and never stored.
#pragma once

#include "afd_device.h"

namespace afd {

using namespace dev;

#ifndef AFD_XCD_REMAP
#define AFD_XCD_REMAP 0
#endif
// register stages per wave, by row fragments per tile
#ifndef AFD_STAGES_MR1
#define AFD_STAGES_MR1 2
#endif
#ifndef AFD_STAGES_GU1
#define AFD_STAGES_GU1 3  // gate/up, single-fragment tiles
#endif
#ifndef AFD_STAGES_MR2
#define AFD_STAGES_MR2 2
#endif
#ifndef AFD_STAGES_MIX
#define AFD_STAGES_MIX 2  // beside heavy tiles (two halves per workgroup)
#endif
// cache policy of the weight loads: 2 = non-temporal (streamed once)
#ifndef AFD_B_AUX
#define AFD_B_AUX 2
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

template <int NPW>
struct StageB {
  uint4 b[NPW][4];
};

constexpr int kArowSlots = 4;  // LDS slots of activation rows (a power of 2)
template <int MR>
constexpr int kArowBytes = kArowSlots * MR * 32 * kStepBytes;

}  // namespace

#ifndef AFD_DOWN_NPW
#define AFD_DOWN_NPW 4  // panels per wave of the single-fragment down GEMM
#endif

// One workgroup of 4 * HALVES waves, as workgroup `rank` of G: half h (waves
// 4h .. 4h+3, its own row slots in LDS) runs task t0 + h of every round t0 =
// HALVES * (rank + k G).  Both halves run every round, a half without a task
// on out-of-range copies and loads, so their barriers pair up.
template <bool GATEUP, int MR, int HALVES>
__device__ __forceinline__ void stream_body(const GemmParams& p, const int rank, const int G) {
  // panels per wave: gate/up 2 (one gate + up pair), down AFD_DOWN_NPW for
  // single-fragment tiles (registers allow it there), else 2
  constexpr int NPW = (GATEUP || MR > 1) ? 2 : AFD_DOWN_NPW;

  const int lane = threadIdx.x & 63;
  const int wave = uniform((threadIdx.x >> 6) & 3);
  const int half = HALVES > 1 ? uniform(threadIdx.x >> 8) : 0;
  const int g = lane >> 5;
  const int col = lane & 31;

  const int num_mt = uniform(p.num_mtiles[0]);
  const int num_tasks = num_mt * p.n_groups;
  const int ks = p.k_steps;

  // Optional XCD-aware schedule (AFD_XCD_REMAP): workgroups are dealt
  // round-robin to the 8 XCDs; renumbering them so each XCD owns a contiguous
  // block of ranks puts consecutive tasks (sibling m-tiles of one expert) under
  // one L2.  Measured: it does not remove the sibling re-reads (the streams
  // drift apart further than their share of L2) and slows skewed batches, so
  // it is off.
  const int r = (AFD_XCD_REMAP && G % kXcds == 0) ? (rank % kXcds) * (G / kXcds) + rank / kXcds : rank;
  for (int t0 = r * HALVES; t0 < num_tasks; t0 += G * HALVES) {
    const int task = t0 + half;
    const bool have = task < num_tasks;
    const int tk = have ? task : t0;  // a half without a task shadows the round's first one
    const int mt = tk % num_mt;
    const int q = tk / num_mt;
    const int4 tile = load_tile(p.mtiles, mt);
    const int expert = uniform(tile.x);
    const int row0 = uniform(tile.y);
    const int rows = uniform(tile.z);
    const int unit = q * kWaves + wave;
    const bool active = have && (GATEUP ? (unit < p.n_panels) : (NPW * unit < p.n_panels));

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + (int64_t)expert * p.b_expert_bytes, p.b_expert_bytes);
    const int boff = uniform((int)((int64_t)(NPW * unit) * p.b_panel_bytes));
    const int bpanel = (int)p.b_panel_bytes;
    const int voffB = lane * 16;

    f32x16 acc[MR][NPW];
#pragma unroll
    for (int mr = 0; mr < MR; ++mr)
#pragma unroll
      for (int pp = 0; pp < NPW; ++pp)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mr][pp][r] = 0.0f;

    {
      // kArowSlots x MR x 32 rows x 128 bytes (declared here, inside the block:
      // see the ring GEMM for why the copies want a local declaration)
      extern __shared__ __attribute__((aligned(16))) uint8_t lds_rows[];
      uint8_t* const arow = lds_rows + half * kArowBytes<MR>;
      // The step's activation rows go through LDS once per workgroup: wave w
      // copies rows 8w .. 8w+7 of every fragment (8 whole 128-byte rows per
      // copy), and every wave reads its MFMA fragments from there.  Weights
      // stay in registers.  Every wave runs the loop (copies and barriers),
      // an inactive one on out-of-range weight offsets.
      const int oobA = (int)(p.a_bytes > 0x7fffffff ? 0x7fffffff : p.a_bytes);
      const int oobB = (int)p.b_expert_bytes;
      const int bbase = active ? boff : oobB;
      // copy lane L: row 8 wave + L / 8 of a fragment, 16-byte chunk
      // (L + L / 8) % 8 of it, landing at byte 16 L of the wave's KiB: each
      // row's chunks are rotated by the row, so a fragment read is
      // conflict-free
      int doff[MR];
#pragma unroll
      for (int mr = 0; mr < MR; ++mr) {
        const int r8 = lane >> 3;
        const int m = mr * 32 + 8 * wave + r8;
        const int r = row0 + (m < rows ? m : 0);
        int src = r;
        if (p.gather) src = r >= p.shared_row0 ? (r - p.shared_row0) % p.shared_tokens : (p.sorted_assign[r] / p.top_k);
        doff[mr] = (int)(src * p.a_row_bytes) + (((lane & 7) + r8) & 7) * 16;
      }
      // fragment read of lane (col, g), chunk 4g + j of row col
      const int rbase = (col >> 3) * 1024 + (col & 7) * 128;
      auto load = [&](StageB<NPW>& s, int c) {
        const bool in = c < ks;
        uint8_t* dst = arow + (c & (kArowSlots - 1)) * (MR * 32 * kStepBytes) + wave * 1024;
        const int sa = uniform(in && have ? c * kStepBytes : oobA);
        const int sb = uniform(in && active ? bbase + c * kStepPanelBytes : oobB);
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) dma16(ra, dst + mr * 4096, doff[mr], sa);
#pragma unroll
        for (int pp = 0; pp < NPW; ++pp)
#pragma unroll
          for (int j = 0; j < 4; ++j) s.b[pp][j] = bload16<AFD_B_AUX>(rb, voffB, sb + pp * bpanel + j * 1024);
      };
      auto compute = [&](const StageB<NPW>& s, int c) {
        const uint8_t* src = arow + (c & (kArowSlots - 1)) * (MR * 32 * kStepBytes) + rbase;
        // The fragment reads are one asm block that also waits for them: as
        // plain loads, the compiler would make them wait for the copies of
        // the next step too (they might write the same LDS), which drains the
        // pipeline; the slot protocol above already orders them.
        i32x4 af[MR][4];
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) {
          uint32_t ad[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            ad[j] = (uint32_t)(uintptr_t)(lds_ptr)(src + mr * 4096 + (((4 * g + j) - (col & 7)) & 7) * 16);
          lds_read4x16(af[mr], ad);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int mr = 0; mr < MR; ++mr)
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp)
              acc[mr][pp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  as_bf16x8(s.b[pp][j]), __builtin_bit_cast(bf16x8, af[mr][j]), acc[mr][pp], 0, 0, 0);
      };
      // NST register stages of weights, kArowSlots LDS slots of rows: the
      // copy of step c + NST - 1 refills the slot read at step c + NST - 1 -
      // kArowSlots, which every wave finished before the previous barrier
      // (beside heavy tiles, all but the 4-panel down waves, whose registers
      // hold two stages only, take AFD_STAGES_MIX)
      constexpr bool wide = MR == 1 && !GATEUP;
      constexpr int NST = HALVES > 1 && !wide ? AFD_STAGES_MIX
                          : MR == 1           ? (GATEUP ? AFD_STAGES_GU1 : AFD_STAGES_MR1)
                                              : AFD_STAGES_MR2;
      constexpr int PER = MR + 4 * NPW;  // copies + weight loads per step
      static_assert(NST + 1 <= kArowSlots, "row slots");
      StageB<NPW> st[NST];
#pragma unroll
      for (int i = 0; i + 1 < NST; ++i) {
        load(st[i], i);
        AFD_PIPE_FENCE();
      }
      for (int c0 = 0; c0 < ks; c0 += NST) {
#pragma unroll
        for (int i = 0; i < NST; ++i) {
          load(st[(i + NST - 1) % NST], c0 + i + NST - 1);
          AFD_PIPE_FENCE();
          wait_vmcnt<(NST - 1) * PER>();  // step c0 + i has landed (this wave's loads and copies) ...
          raw_barrier();                  // ... and every wave's copies
          compute(st[i], c0 + i);
          AFD_PIPE_FENCE();
        }
      }
      wait_vmcnt<0>();  // the copies of steps past the end
      raw_barrier();    // every wave is done with the row slots before the next task
    }
    // ---------------------------------------------------------------- epilogue
    if (!active) continue;
    if (GATEUP) {
#pragma unroll
      for (int mr = 0; mr < MR; ++mr) {
        const int m = mr * 32 + col;
        if (m >= rows) continue;
        uint8_t* out = p.c + (int64_t)(row0 + m) * p.c_row_bytes + (int64_t)(32 * unit) * 2;
        // lane l holds columns 8 r4 + 4 g + 0..3; lanes l and l ^ 32 swap one
        // of each pair of r4 so every lane stores 8 consecutive columns
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          uint2 o[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int r4 = 2 * r2 + k;
            float h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = silu_mul(acc[mr][0][4 * r4 + e], acc[mr][1][4 * r4 + e]);
            o[k].x = pack_bf16x2(h[0], h[1]);
            o[k].y = pack_bf16x2(h[2], h[3]);
          }
          store_pair16(out + (16 * r2 + 8 * g) * 2, o[0], o[1], g != 0);
        }
      }
    } else {
#pragma unroll
      for (int mr = 0; mr < MR; ++mr) {
        const int m = mr * 32 + col;
        if (m >= rows) continue;
#pragma unroll
        for (int pp = 0; pp < NPW; ++pp) {
          if (NPW * unit + pp >= p.n_panels) continue;
          uint8_t* out = p.c + (int64_t)(row0 + m) * p.c_row_bytes + (int64_t)(32 * (NPW * unit + pp)) * 2;
#pragma unroll
          for (int r2 = 0; r2 < 2; ++r2) {
            uint2 o[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              const int r4 = 2 * r2 + k;
              o[k].x = pack_bf16x2(acc[mr][pp][4 * r4 + 0], acc[mr][pp][4 * r4 + 1]);
              o[k].y = pack_bf16x2(acc[mr][pp][4 * r4 + 2], acc[mr][pp][4 * r4 + 3]);
            }
            store_pair16<true>(out + (16 * r2 + 8 * g) * 2, o[0], o[1], g != 0);
          }
        }
      }
    }
  }
}

}  // namespace afd
