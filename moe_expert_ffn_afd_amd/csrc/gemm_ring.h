#pragma once
// gemm_ring.h -- block-FP8 and W8A8 grouped expert GEMMs fed by a weight ring in LDS:
// the workgroup body, shared by the ring kernels (gemm_ring.hip) and the fused
// layer kernel (fused.hip).
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
// from cache; each wave loads its own 16-row token tile straight into MFMA
// operand registers, NS-1 steps ahead as well (one tile per wave rather than
// two halves the row loads, which share the CU's cache-line request budget
// with the weight copies; the extra LDS reads of the weights cost less).  Every scale a step needs rides
// in the same slot: the tile's 1x128 row scales (stored step-major in
// sorted-row order, by the dispatch for the hidden rows and by the gate/up
// epilogue for h, so one step's scales of a tile are one contiguous run) and
// the two 128x128 weight block scales of the step.
//
// The pipeline runs across task boundaries: while a task's last steps are
// multiplied, the first NS-1 steps of the workgroup's next task are already in
// flight, and the task's epilogue (SwiGLU, re-quantisation, stores) runs while
// they land.  So nothing a task needs may be fetched with a wait of its own:
// the next task's m-tile is read with scalar loads, and the source rows of its
// gathered activations are copied into LDS one task ahead, behind the same
// in-order wait counts as the weights.
//
// The steady loop is unrolled by NS so every register stage has a static
// index, and is branch-free: steps past the end load at out-of-range offsets,
// which the buffer unit returns as zeros (exact zero products), so one wait
// count serves every step.  The copy engine's LDS writes are invisible to the
// compiler, so the kernel orders them itself: s_waitcnt vmcnt(N), N = the
// loads of the younger steps still allowed in flight, then a barrier; the slot
// refilled after the barrier is the one every wave finished reading one step
// earlier.
//
// MFMA 16x16x128 e4m3 (one instruction spans a whole scale block): weight
// fragment first, token fragment second, so lane l holds token l % 16 and
// output columns 4(l / 16) + r of a 16-column half panel; the product is added
// into the accumulator times (token scale x block scale).  Eight waves, two per
// SIMD, as WM x WN = (BM / 16) x (8 / (BM / 16)): each wave owns 16 rows and
// 8 / WN panels (8 x 1 for 128-row tiles, 4 x 2 for 64-row tiles).
//
// W8A8 layers (I8) run the same ring on int8 codes: each lane's 32 bytes of a
// step feed two int8 MFMAs 16x16x64 (its first and its second 16 bytes, in
// both operands, so every product pairs the same k), accumulated exactly in
// int32 over the whole reduction.  The scales are per token and per output
// channel, so they are applied once, in the epilogue: the task's last step
// carries them in its slot (the tile's row scales, the task's column scales).
// The gate/up epilogue stores h in bf16 with its per-row amax over the task's
// 128 columns; quant.hip turns that into int8 h with one scale per row.
#include <algorithm>
#include <type_traits>

#include "afd_device.h"
#include "gemm_tiled8.h"

namespace afd {

using namespace dev;

namespace {

#ifndef AFD_RING_NS
#define AFD_RING_NS 4
#endif
// Cache policy of the weight copies (WNT = the kernel's template argument):
// non-temporal when the layer runs alone (fp8_shared 1.6 % faster), the
// default when other forwards run beside it (the ping-pong microbatches read
// the same experts at about the same time, and with non-temporal copies the
// verify shard was 2 % slower).
#ifndef AFD_RING_RT_HEAVY
#define AFD_RING_RT_HEAVY 1  // 16-row token tiles per wave, 128-row m-tiles
#endif
#ifndef AFD_RING_RT_LIGHT
#define AFD_RING_RT_LIGHT 1  // same, 64-row m-tiles
#endif
#ifndef AFD_RING_XCD_REMAP
#define AFD_RING_XCD_REMAP 1
#endif
#ifndef AFD_RING_POOL
#define AFD_RING_POOL 1  // the light list's tail as a pool claimed by the workgroups done first
#endif

constexpr int kRingWaves = 8;
constexpr int kRingPanels = 8;
constexpr int kRingWeightBytes = kRingPanels * kStepPanelBytes;  // 32 KiB per step
// Each slot: the step's weights, then one 1 KiB scale copy per wave 0..2:
// the tile's row scales (wave 0), weight block scales 0 and 1 (waves 1 and 2).
constexpr int kRingScaleCopies = 3;
constexpr int kRingSlotBytes = kRingWeightBytes + kRingScaleCopies * 1024;
constexpr int kRingNS = AFD_RING_NS;
constexpr int kRingSinkOff = kRingNS * kRingSlotBytes;      // the other waves' (empty) scale copies
constexpr int kRingMetaOff = kRingSinkOff + 1024;           // per wave: source rows of two tasks ahead
constexpr int kRingMetaBytes = 256;                         // 64 lanes x 4 bytes
constexpr int kRingLdsBytes = kRingMetaOff + kRingWaves * 2 * kRingMetaBytes;
#ifndef AFD_RING_MB
#define AFD_RING_MB 4
#endif
constexpr int kRingMB = AFD_RING_MB;  // m-tiles per rasterisation block
constexpr int kRingMinRounds = 1;  // unrolled rounds per task
static_assert(kRingLdsBytes <= 160 * 1024 - 4096, "ring exceeds LDS");
static_assert(kT8LdsBytes <= kRingLdsBytes, "the tiled FP8 body runs in the ring kernels' LDS");

__device__ inline int clamp31(int64_t v) { return v > 0x7fffffff ? 0x7fffffff : (int)v; }

// Task t of a list of n m-tiles -> (m-tile, column group): blocks of kRingMB
// m-tiles x all column groups, so consecutive tasks share their rows in L2.
__device__ inline void ring_decode(int t, int n, int nq, int& mt, int& q) {
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
}

// One task as a wave holds it while its steps are issued: the m-tile, the
// column group and the per-lane offsets (buffer descriptors are rebuilt per
// step from these, which is cheaper than holding two tasks' in registers).
struct RingDesc {
  int expert, row0, rows, q;
  int ks;       // steps with data (0: an empty task, every copy out of range)
  int svoff;    // per lane: scale copy offset (out of range where unused)
  int aoff[2];  // per lane: activation offsets of the two token tiles
};

}  // namespace

// Every task rank + k * stride (k = 0, 1, ...) below min(limit, n_tiles x
// n_groups) of one m-tile list, in one continuous pipeline.  Every wave of the
// workgroup calls it with the same arguments.
template <bool GATEUP, int BM, bool WNT, bool I8>
__device__ __forceinline__ void ring_list(const GemmParams& p, const int4* tiles, const int n_tiles,
                                          const int first, const int stride, const int limit) {
  // declared here, not passed in: the copies need pointers known to be in LDS
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  __shared__ float red[kRingWaves * 32];  // gate/up: per-wave token amax
  constexpr int NS = kRingNS;
  constexpr int WM = BM / (16 * (BM > 64 ? AFD_RING_RT_HEAVY : AFD_RING_RT_LIGHT)), WN = kRingWaves / WM,
                NPW = kRingPanels / WN;
  constexpr int RT = BM > 64 ? AFD_RING_RT_HEAVY : AFD_RING_RT_LIGHT;  // 16-row token tiles per wave
  constexpr int WR = 16 * RT;                             // rows per wave
  constexpr int B_DMA = kRingPanels * 4 / kRingWaves;     // 1 KiB weight copies per wave and step
  constexpr int PER_STAGE = B_DMA + 2 * RT + 1;           // + two 16-byte row loads per tile + scales
  constexpr int SLOT = kRingSlotBytes;
  constexpr int S_OFF = kRingWeightBytes;
  static_assert(WM * WN == kRingWaves && NPW % 2 == 0 && NPW <= 8 && RT <= 2 && BM <= 256, "wave grid");
  static_assert(NS >= 2 && (NS - 2) * PER_STAGE < 64, "wait count");

  const int nq = p.n_groups;
  const int count = min(n_tiles * nq, limit);
  if (first >= count) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int kg = lane >> 4;  // which 32 bytes of the 128-deep block this lane carries
  const int tok = lane & 15;
  const int ks = p.k_steps;
  const int nsr = max((ks + NS - 1) / NS, kRingMinRounds) * NS;  // steps run: whole unrolled rounds
  const int oobA = clamp31(p.a_bytes), oobS = clamp31(p.a_scale_bytes);
  const int oobB = (int)p.b_expert_bytes;
  const int bpanel = (int)p.b_panel_bytes;
  const int wsb = p.b_scale_rows * p.b_scale_cols;  // block scales per expert and matrix
  const auto ra = make_rsrc(p.a, p.a_bytes);
  const auto rsa = make_rsrc(p.a_scales, p.a_scale_bytes);
  // this wave's scale copy: 0 = the tile's row scales, 1 / 2 = weight block
  // scale 0 / 1 of the step, -1 = none (its empty copy goes to the sink)
  const int scopy = wave < kRingScaleCopies ? wave : -1;
  const auto rmeta = make_rsrc(p.sorted_assign, (int64_t)p.shared_row0 * 4);
  // the source of this wave's scale copy, its bytes per step and an
  // out-of-range offset (expert and block enter the per-lane offset)
  const auto rs = scopy <= 0 ? rsa : make_rsrc((GATEUP && scopy == 2) ? p.b_scales1 : p.b_scales0, p.b_scale_bytes);
  const int sstep = scopy <= 0 ? p.a_scale_ld * 4 : p.b_scale_cols * 4;
  const int soob = scopy <= 0 ? oobS : clamp31(p.b_scale_bytes);
  uint8_t* const meta = ring + kRingMetaOff + wave * 2 * kRingMetaBytes;  // two buffers
  // down: the block scale of this wave's panels

  // gate/up: copy the sorted-row -> flat-slot entries of this wave's 32 rows of
  // a tile (lanes 0..31) and of the tile's first row (lane 32) into meta
  // buffer `buf`
  auto meta_copy = [&](const int4 tile, const bool valid, const int buf) {
    const int row0 = uniform(tile.y);
    int v = 0x7fffffff;
    if (valid && lane < WR) v = (row0 + wm * WR + lane) * 4;
    if (valid && lane == 32) v = row0 * 4;
    dma4(rmeta, meta + buf * kRingMetaBytes, v, 0);
  };

  auto make_desc = [&](const int4 tile, const int q, const bool valid, const int buf) {
    RingDesc d;
    d.expert = uniform(tile.x);
    d.row0 = uniform(tile.y);
    d.rows = valid ? uniform(tile.z) : 0;
    d.q = q;
    d.ks = valid ? ks : 0;
    const int* mi = reinterpret_cast<const int*>(meta + buf * kRingMetaBytes);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      // rows past the tile's count repeat its first row (computed, never stored)
      const int m = wm * WR + rt * 16 + tok;
      const int r = d.row0 + (m < d.rows ? m : 0);
      int src = r;
      if (GATEUP && r < p.shared_row0) src = (m < d.rows ? mi[rt * 16 + tok] : mi[32]) / p.top_k;
      if (GATEUP && r >= p.shared_row0) src = (r - p.shared_row0) % p.shared_tokens;
      d.aoff[rt] = valid ? (int)((int64_t)src * p.a_row_bytes) + 32 * kg : 0;
    }
    if (scopy == 0)  // lane i: rows 4i .. 4i+3 of the tile's run in a step
      d.svoff = (valid && 4 * lane < BM) ? (d.row0 + 4 * lane) * 4 : soob;
    else if (!I8)    // lane 0: one block scale of the step (row c of the expert's block grid)
      d.svoff = (valid && scopy > 0 && lane == 0) ? (d.expert * wsb + (GATEUP ? q : 2 * q + (scopy - 1))) * 4 : soob;
    else if (GATEUP) // I8 gate/up: lane i < 32: gate (wave 1) or up (wave 2) scales of columns 128q + 4i ..
      d.svoff = (valid && scopy > 0 && lane < 32) ? (d.expert * p.b_scale_cols + 128 * q + 4 * lane) * 4 : soob;
    else             // I8 down: wave 1, lane i: scales of columns 256q + 4i .. (wave 2 copies nothing)
      d.svoff = (valid && scopy == 1) ? (d.expert * p.b_scale_cols + 256 * q + 4 * lane) * 4 : soob;
    return d;
  };

  i32x4 areg[NS][RT][2];
  // fp32 accumulators (block-FP8, scaled per step) or int32 (W8A8, exact)
  typedef typename std::conditional<I8, i32x4, f32x4>::type acc_t;
  acc_t acc[RT][2 * NPW];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int b = 0; b < 2 * NPW; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[rt][b][r] = 0;

  // step s of the current task into ring slot `slot` and register stage
  // `slot`; s >= nsr: step s - nsr of the next task
  auto issue = [&](const RingDesc& cur, const RingDesc& nxt, int s, int slot) {
    const bool nx = s >= nsr;
    const int c = nx ? s - nsr : s;
    const bool in = c < (nx ? nxt.ks : cur.ks);
    const int expert = nx ? nxt.expert : cur.expert;
    const int q = nx ? nxt.q : cur.q;
    uint8_t* st = ring + slot * SLOT;
    const auto rb = make_rsrc(p.b + (int64_t)expert * p.b_expert_bytes, p.b_expert_bytes);
    const int pbase = q * kRingPanels * bpanel;
#pragma unroll
    for (int k = 0; k < B_DMA; ++k) {
      const int i = wave * B_DMA + k, panel = i / 4, j = i % 4;
      dma16_aux<WNT ? 2 : 0>(rb, st + panel * kStepPanelBytes + j * 1024, lane * 16,
                                in ? pbase + panel * bpanel + c * kStepPanelBytes + j * 1024 : oobB);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int aoff = nx ? nxt.aoff[rt] : cur.aoff[rt];
      areg[slot][rt][0] = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff, in ? c * kStepBytes : oobA, 0);
      areg[slot][rt][1] = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff, in ? c * kStepBytes + 16 : oobA, 0);
    }
    // block-FP8: every step's scales; W8A8: the task's scales, with its last
    // step run (slot NS - 1, still intact when the epilogue reads it).  (The
    // block-FP8 offset stays inside the call: computed ahead as a variable, it
    // made the compiler spill that kernel's registers.)
    if constexpr (I8)
      dma16(rs, scopy >= 0 ? st + S_OFF + scopy * 1024 : ring + kRingSinkOff, nx ? nxt.svoff : cur.svoff,
            (!nx && c == nsr - 1) ? 0 : soob);
    else
      dma16(rs, scopy >= 0 ? st + S_OFF + scopy * 1024 : ring + kRingSinkOff, nx ? nxt.svoff : cur.svoff,
            in ? c * sstep : soob);
  };

  auto compute_fp8 = [&](int slot) {
    const uint8_t* Bs = ring + slot * SLOT;
    const float* S = reinterpret_cast<const float*>(Bs + S_OFF);
    float sa[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) sa[rt] = S[wm * WR + rt * 16 + tok];
    const float sw0 = *reinterpret_cast<const float*>(Bs + S_OFF + 1024);
    const float sw1 = *reinterpret_cast<const float*>(Bs + S_OFF + 2048);
    i32x8 x[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) x[rt] = cat32v(areg[slot][rt][0], areg[slot][rt][1]);
    // weight fragment of a 16-column half panel: K bytes 32 kg .. +32 are
    // 1 KiB chunks 2(kg & 1), +1 of the panel's lane half kg >> 1
    const int g = kg >> 1, j0 = (kg & 1) * 2;
    // the weight fragments of PG panels first, then their products (PG = all
    // of a wave's panels up to 4)
    constexpr int PG = NPW < 4 ? NPW : 4;
#pragma unroll
    for (int p0 = 0; p0 < NPW; p0 += PG) {
      i32x8 wf[PG][2];
#pragma unroll
      for (int dp = 0; dp < PG; ++dp)
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          const uint8_t* lo = Bs + (wn * NPW + p0 + dp) * kStepPanelBytes + j0 * 1024 + (16 * sh + tok + 32 * g) * 16;
          wf[dp][sh] = cat32v(*reinterpret_cast<const i32x4*>(lo), *reinterpret_cast<const i32x4*>(lo + 1024));
        }
#pragma unroll
      for (int dp = 0; dp < PG; ++dp) {
        const int pp = p0 + dp;
        // gate/up: even panels gate, odd up; down: the 128-column block of the panel
        const float sb = GATEUP ? ((pp & 1) ? sw1 : sw0) : ((wn * NPW + pp) >= 4 ? sw1 : sw0);
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
            t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[dp][sh], x[rt], t, 0, 0, 0, 0, 0, 0);
            const float sc = sa[rt] * sb;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) acc[rt][pp * 2 + sh][r4] += t[r4] * sc;
          }
        }
      }
    }
  };

  auto compute_i8 = [&](int slot) {
    const uint8_t* Bs = ring + slot * SLOT;
      // two int8 MFMAs per 32 bytes of k: the first and the second 16 bytes of
      // both operands
      const int g = kg >> 1, j0 = (kg & 1) * 2;
#pragma unroll
      for (int pp = 0; pp < NPW; ++pp) {
        i32x4 wlo[2], whi[2];
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          const uint8_t* lo = Bs + (wn * NPW + pp) * kStepPanelBytes + j0 * 1024 + (16 * sh + tok + 32 * g) * 16;
          wlo[sh] = *reinterpret_cast<const i32x4*>(lo);
          whi[sh] = *reinterpret_cast<const i32x4*>(lo + 1024);
        }
#pragma unroll
        for (int sh = 0; sh < 2; ++sh)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            acc[rt][pp * 2 + sh] =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo[sh], areg[slot][rt][0], acc[rt][pp * 2 + sh], 0, 0, 0);
            acc[rt][pp * 2 + sh] =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(whi[sh], areg[slot][rt][1], acc[rt][pp * 2 + sh], 0, 0, 0);
          }
      }
  };

  auto compute = [&](int slot) {
    if constexpr (I8)
      compute_i8(slot);
    else
      compute_fp8(slot);
  };

  // The task's outputs.  Its barriers are the ring's kind (LDS only): the
  // next task's copies stay in flight.
  auto epilogue_fp8 = [&](const RingDesc& d) {
    const int row0 = d.row0, rows = d.rows, q = d.q;
    if constexpr (GATEUP) {
      // h of unit u = 4q + (wn NPW + pp) / 2 (pp even: gate, pp + 1: up), per
      // token amax over the task's 128 h columns: this wave's, then over WN
      // (a wave of a WN = 1 grid holds all of them: no exchange, no barriers)
      float h[RT][NPW / 2][2][4];
      float am[RT];
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
        am[rt] = a;
        if (WN > 1 && kg == 0) red[(wm * WN + wn) * 32 + rt * 16 + tok] = a;
      }
      if constexpr (WN > 1) {
        lds_reads_done();
        raw_barrier();
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int mi = rt * 16 + tok;
        const int m = wm * WR + mi;
        float amax = am[rt];
        if constexpr (WN > 1) {
          amax = 0.0f;
#pragma unroll
          for (int w2 = 0; w2 < WN; ++w2) amax = fmaxf(amax, red[(wm * WN + w2) * 32 + mi]);
        }
        const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
        const float inv = amax > 0.0f ? 448.0f / amax : 1.0f;
        if (m < rows) {
          uint8_t* orow = p.c + (int64_t)(row0 + m) * p.c_row_bytes;
#pragma unroll
          for (int u = 0; u < NPW / 2; ++u) {
            const int unit = 4 * q + (wn * NPW) / 2 + u;
            uint32_t o[2];
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = fminf(fmaxf(h[rt][u][sh][e] * inv, -448.0f), 448.0f);
              o[sh] = pack_fp8x4(v[0], v[1], v[2], v[3]);
            }
            // lanes kg and kg ^ 1 swap one half each: 8 consecutive codes per lane
            const bool odd = (kg & 1) != 0;
            const uint32_t rcv = __shfl_xor(odd ? o[0] : o[1], 16, 64);
            const uint2 w = odd ? make_uint2(rcv, o[1]) : make_uint2(o[0], rcv);
            *reinterpret_cast<uint2*>(orow + 32 * unit + (odd ? 16 + 4 * (kg - 1) : 4 * kg)) = w;
          }
          if (wn == 0 && kg == 0) p.c_scales[(int64_t)q * p.c_scale_ld + row0 + m] = scale;
        }
      }
      if constexpr (WN > 1) {
        lds_reads_done();
        raw_barrier();  // red[] is rewritten by the next task
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int pp = 0; pp < NPW; pp += 2) {
          const int P = q * kRingPanels + wn * NPW + pp;
          if (P >= p.n_panels) continue;
          uint4 v[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int b = (pp + k) * 2;
            v[k] = pair16_cols(
                make_uint2(pack_bf16x2(acc[rt][b][0], acc[rt][b][1]), pack_bf16x2(acc[rt][b][2], acc[rt][b][3])),
                make_uint2(pack_bf16x2(acc[rt][b + 1][0], acc[rt][b + 1][1]), pack_bf16x2(acc[rt][b + 1][2], acc[rt][b + 1][3])),
                kg);
          }
          store_line_pair<true>(p.c, p.c_row_bytes, p.n_panels, row0, rows, wm * WR + rt * 16, P, v[0], v[1], tok, kg);
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int b = 0; b < 2 * NPW; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[rt][b][r] = 0.0f;
  };

  // W8A8: the task's outputs from exact int32 sums.  Its scales came with its
  // last step (slot NS - 1): row m at Sx[m]; gate/up: the gate and up scales
  // of the task's h column c at Sc0[c], Sc1[c]; down: output column c of the
  // task at Sc0[c].  Gate/up stores h in bf16 and each row's amax over the
  // task's 128 columns (quant.hip re-quantises h per row from those).
  auto epilogue_i8 = [&](const RingDesc& d) {
    const int row0 = d.row0, rows = d.rows, q = d.q;
    const float* Sx = reinterpret_cast<const float*>(ring + (NS - 1) * SLOT + S_OFF);
    const float* Sc0 = reinterpret_cast<const float*>(ring + (NS - 1) * SLOT + S_OFF + 1024);
    const float* Sc1 = reinterpret_cast<const float*>(ring + (NS - 1) * SLOT + S_OFF + 2048);
    const bool odd = (kg & 1) != 0;
    // lane pairs (kg, kg ^ 1) of a token swap one half each, so every lane
    // stores 8 consecutive bf16 columns (16 bytes) from column 32 * unit
    auto store_pair = [&](uint8_t* orow, const int unit, const float (&v)[2][4], const bool nt) {
      uint2 o0, o1;
      o0.x = pack_bf16x2(v[0][0], v[0][1]);
      o0.y = pack_bf16x2(v[0][2], v[0][3]);
      o1.x = pack_bf16x2(v[1][0], v[1][1]);
      o1.y = pack_bf16x2(v[1][2], v[1][3]);
      const uint2 snd = odd ? o0 : o1;
      uint2 rcv;
      rcv.x = __shfl_xor(snd.x, 16, 64);
      rcv.y = __shfl_xor(snd.y, 16, 64);
      const uint4 w = odd ? make_uint4(rcv.x, rcv.y, o1.x, o1.y) : make_uint4(o0.x, o0.y, rcv.x, rcv.y);
      uint8_t* dst = orow + (int64_t)(odd ? 32 * unit + 16 + 4 * (kg - 1) : 32 * unit + 4 * kg) * 2;
      if (nt)
        store16<true>(dst, w);
      else
        store16(dst, w);
    };
    if constexpr (GATEUP) {
      float h[RT][NPW / 2][2][4];
      float am[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float sx = Sx[wm * WR + rt * 16 + tok];
        float a = 0.0f;
#pragma unroll
        for (int u = 0; u < NPW / 2; ++u)
#pragma unroll
          for (int sh = 0; sh < 2; ++sh)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int c = 32 * ((wn * NPW) / 2 + u) + 16 * sh + 4 * kg + r4;
              const float v = silu_mul((float)acc[rt][4 * u + sh][r4] * sx * Sc0[c],
                                       (float)acc[rt][4 * u + 2 + sh][r4] * sx * Sc1[c]);
              h[rt][u][sh][r4] = v;
              a = fmaxf(a, fabsf(v));
            }
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        a = fmaxf(a, __shfl_xor(a, 32, 64));
        am[rt] = a;
        if (WN > 1 && kg == 0) red[(wm * WN + wn) * 32 + rt * 16 + tok] = a;
      }
      if constexpr (WN > 1) {
        lds_reads_done();
        raw_barrier();
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int mi = rt * 16 + tok;
        const int m = wm * WR + mi;
        float amax = am[rt];
        if constexpr (WN > 1) {
          amax = 0.0f;
#pragma unroll
          for (int w2 = 0; w2 < WN; ++w2) amax = fmaxf(amax, red[(wm * WN + w2) * 32 + mi]);
        }
        if (m >= rows) continue;
        uint8_t* orow = p.c + (int64_t)(row0 + m) * p.c_row_bytes;
#pragma unroll
        for (int u = 0; u < NPW / 2; ++u) store_pair(orow, 4 * q + (wn * NPW) / 2 + u, h[rt][u], false);
        if (wn == 0 && kg == 0) p.c_scales[(int64_t)q * p.c_scale_ld + row0 + m] = amax;
      }
      if constexpr (WN > 1) {
        lds_reads_done();
        raw_barrier();  // red[] is rewritten by the next task
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float sx = Sx[wm * WR + rt * 16 + tok];  // (of a row past the task's: never stored)
#pragma unroll
        for (int pp = 0; pp < NPW; pp += 2) {
          const int P = q * kRingPanels + wn * NPW + pp;
          if (P >= p.n_panels) continue;
          uint4 v[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            float f[2][4];
#pragma unroll
            for (int sh = 0; sh < 2; ++sh)
#pragma unroll
              for (int r4 = 0; r4 < 4; ++r4)
                f[sh][r4] = (float)acc[rt][(pp + k) * 2 + sh][r4] * sx * Sc0[32 * (wn * NPW + pp + k) + 16 * sh + 4 * kg + r4];
            v[k] = pair16_cols(make_uint2(pack_bf16x2(f[0][0], f[0][1]), pack_bf16x2(f[0][2], f[0][3])),
                               make_uint2(pack_bf16x2(f[1][0], f[1][1]), pack_bf16x2(f[1][2], f[1][3])), kg);
          }
          store_line_pair<true>(p.c, p.c_row_bytes, p.n_panels, row0, rows, wm * WR + rt * 16, P, v[0], v[1], tok, kg);
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int b = 0; b < 2 * NPW; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[rt][b][r] = 0;
  };

  auto epilogue = [&](const RingDesc& d) {
    if constexpr (I8)
      epilogue_i8(d);
    else
      epilogue_fp8(d);
  };

  // The row sources of a task are copied two tasks ahead into alternating
  // buffers, so the descriptor of the next task can be built when the current
  // one starts, from data that landed behind the previous task's waits.  The
  // two tasks ahead of the loop may be waited for: nothing is in flight yet.
  int t = first, mt = 0, q = 0;
  ring_decode(t, n_tiles, nq, mt, q);
  const int4 tile = load_tile(tiles, mt);
  int t1 = t + stride, mt1 = mt, q1 = q;
  if (t1 < count) ring_decode(t1, n_tiles, nq, mt1, q1);
  int4 tile1 = load_tile(tiles, mt1);
  if (GATEUP) {
    meta_copy(tile, true, 0);
    meta_copy(tile1, t1 < count, 1);
    wait_vmcnt<0>();
  }
  RingDesc cur = make_desc(tile, q, true, 0);
  // The loads of one step stay together (scheduling fences): the wait
  // counter retires loads in order, so a step's loads mixed into a younger
  // step's would make the register waits drain that younger step.
  lds_reads_done();
#pragma unroll
  for (int i = 0; i + 1 < NS; ++i) {
    issue(cur, cur, i, i);
    __builtin_amdgcn_sched_barrier(0);
  }
  int buf = 0;  // meta buffer of the current task
  while (true) {
    const bool has_next = t1 < count;
    // the next task, from the row sources copied one task ago
    const RingDesc nxt = make_desc(tile1, q1, has_next, buf ^ 1);
    // the task after it: its tile, and its row sources into the buffer the
    // current task's came from (read when it started, so free)
    const int t2 = t1 + stride;
    int mt2 = mt1, q2 = q1;
    if (t2 < count) ring_decode(t2, n_tiles, nq, mt2, q2);
    const int4 tile2 = load_tile(tiles, mt2);
    lds_reads_done();
    // This copy goes out behind the current task's first steps; it only ever
    // makes the wait counts below stricter (as do the previous task's
    // stores), never looser.
    if (GATEUP) meta_copy(tile2, t2 < count, buf);
    __builtin_amdgcn_sched_barrier(0);
    int t0 = 0;
    do {  // the last round issues the next task's first NS - 1 steps
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        wait_vmcnt<(NS - 2) * PER_STAGE>();  // step t0 + i has landed (this wave's copies) ...
        lds_reads_done();
        raw_barrier();                       // ... and every wave's; slot of the previous step is free
        issue(cur, nxt, t0 + i + NS - 1, (i + NS - 1) % NS);
        __builtin_amdgcn_sched_barrier(0);
        compute(i);
        __builtin_amdgcn_sched_barrier(0);
      }
      t0 += NS;
    } while (t0 < nsr);
    epilogue(cur);
    if (!has_next) break;
    cur = nxt;
    t1 = t2;
    tile1 = tile2;
    q1 = q2;
    mt1 = mt2;
    buf ^= 1;
  }
  wait_vmcnt<0>();  // the empty steps issued past the last task
  lds_reads_done();
  raw_barrier();    // every wave is done with the ring before another list refills it
}

// One GEMM stage as workgroup b of G: with TILED, the 8-bit layers' tiled list
// first (m-tiles of up to 256 rows, gemm_tiled8.h; the fused layer kernel),
// then the heavy list's tasks (up to 128 rows), then the light list's (up to
// 64 rows), so a GEMM stage has one tail instead of several.  (The separate
// ring launch leaves the tiled list to a launch of its own before it, which
// keeps the ring kernel's registers at what the ring alone needs.)  A workgroup runs tasks rank,
// rank + G, ... of the lists in a row; ranks are renumbered so that each XCD
// owns a contiguous run of tasks (shared rows stay in its L2).
//
// The light list's last tasks (up to one per workgroup) form a pool instead:
// a workgroup done with its own tasks claims them one at a time from a
// counter (p.pool[stage], zeroed by the dispatch), each in a pipeline of its
// own.  The static shares end within a task of each other, but CUs do not run
// equally fast (measured: the last workgroup of a gate/up launch ends about
// 5 % after the first), so the fast ones take the tail.
template <bool GATEUP, bool WNT, bool I8, bool TILED>
__device__ __forceinline__ void ring_stage(const GemmParams& p, const int b, const int G) {
  const int nq = p.n_groups;
  const int nt = (TILED && p.num_mtiles3) ? uniform(p.num_mtiles3[0]) : 0;
  const int nh = uniform(p.num_mtiles2 ? p.num_mtiles2[0] : 0);
  const int nl = uniform(p.num_mtiles[0]);
  const int tt = nt * nq, th = nh * nq, tl = nl * nq;
  const int rank = (AFD_RING_XCD_REMAP && G % kXcds == 0) ? (b % kXcds) * (G / kXcds) + b / kXcds : b;
  // this workgroup's first task at or past index `base` of the lists in a row
  auto next_from = [&](const int base) { return rank >= base ? rank : rank + (base - rank + G - 1) / G * G; };
  if constexpr (TILED)
    if (nt > 0) tiled8_list<GATEUP, I8>(p, p.mtiles3, nt, rank, G);
  if (nh > 0) ring_list<GATEUP, 128, WNT, I8>(p, p.mtiles2, nh, next_from(tt) - tt, G, th);
  // this workgroup's first task past the heavy list, as an index into the light list
  const int first_l = next_from(tt + th) - (tt + th);
  const int pool = (AFD_RING_POOL && p.pool) ? min(tl, G) : 0;
  int first = first_l, stride = G, limit = tl - pool;
  for (;;) {
    ring_list<GATEUP, 64, WNT, I8>(p, p.mtiles, nl, first, stride, limit);
    if (pool == 0) break;
    __shared__ int claim;
    if (threadIdx.x == 0)
      claim = __hip_atomic_fetch_add(p.pool + (GATEUP ? 0 : 1), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int c = uniform(claim);
    __syncthreads();  // claim is rewritten by the next round
    if (c >= pool) break;
    first = tl - pool + c;  // one pool task
    stride = tl;
    limit = first + 1;
  }
}

}  // namespace afd
