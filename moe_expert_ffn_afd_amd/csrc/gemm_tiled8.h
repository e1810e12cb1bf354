#pragma once
// gemm_tiled8.h -- LDS-tiled block-FP8 grouped GEMM for experts with many
// rows: the workgroup body the ring GEMM kernels (and the fused layer kernel)
// run over the "tiled" m-tile list before their heavy and light lists.
//
// The weight-ring GEMM (gemm_ring.h) streams each task's weights through LDS
// and loads the activation rows into registers, one 16-row tile per wave: a
// weight byte feeds at most 128 rows, which suits experts of tens of rows,
// where HBM sets the pace.  Large batches (speculative verification multiplies
// the routed rows, "FastAFD" summary, speculative-decoding results) give each
// expert hundreds of rows, and there the ring's 128 x 256 tasks copy 48 KiB
// per 128-deep step for 8.4 MFLOP, too few flops per byte moved into the CU.
// This body runs tasks of 256 rows x 8 weight panels (256 GEMM columns): every
// 128-deep super-step the buffer unit copies the step's 8 weight panels (32
// KiB, packed exactly as for the ring) and the 256 rows (32 KiB) straight into
// LDS, with the step's scales, and each wave multiplies 64 rows x 4 panels out
// of LDS: 64 KiB per step for 16.8 MFLOP.
//
// Data flow per step (two slots of one super-step each, one copied while the
// other is multiplied, as in the bf16 LDS-tiled GEMM, gemm_tiled.h):
//   - weights: 8 panels x 4 KiB at the slot's start;
//   - rows: 256 x 128 bytes, the eight 16-byte parts of row r permuted by
//     part ^ ((r >> 1) & 7), so the MFMA fragment reads (16 rows x 32 bytes
//     per 16 lanes) are free of bank conflicts;
//   - scales: the tile's 256 row scales (one contiguous step-major run of the
//     1x128 activation scales, wave 0) and the step's two 128x128 weight block
//     scales (waves 1 and 2); the other waves' copies go to a sink.
// MFMA 16x16x128 e4m3, weight fragment first and token fragment second, so
// lane l holds token l % 16 and output columns 4 (l / 16) + r of a 16-column
// half panel, exactly as in the ring GEMM; each product is added into the
// accumulators times (token scale x block scale).  Eight waves, two per SIMD,
// as 4 x 2 of 64 rows (4 token tiles) x 4 panels: 128 fp32 accumulators per
// lane.  The epilogues are the ring GEMM's: gate/up forms h = silu(g) u,
// re-quantises it to e4m3 per token and 128 columns (amax / 448, the two
// waves of a row group exchanging their amax through LDS) and writes the
// scales step-major; down writes the bf16 expert outputs.
//
// W8A8 layers (I8) run the same tiles on int8 codes, as the ring does: each
// lane's 32 bytes of a step feed two int8 MFMAs 16x16x64 (its first and its
// second 16 bytes in both operands), summed exactly in int32 straight in the
// accumulators; the per-token and per-channel scales are constant along k, so
// the task's scales are copied once, at its start, into slot 0's scale area
// (no step writes it in this mode) and applied in the epilogue, which writes
// h in bf16 with each row's amax over the task's 128 columns (gate/up) or the
// bf16 outputs (down).
#include <algorithm>
#include <type_traits>

#include "afd_device.h"

namespace afd {

using namespace dev;

namespace {

constexpr int kT8Waves = 8;
constexpr int kT8Rows = kTiled8Rows;                           // rows of a tiled m-tile
constexpr int kT8Panels = 8;                                   // weight panels of a task
constexpr int kT8ScaleOff = kT8Panels * kStepPanelBytes + kT8Rows * kStepBytes;  // 64 KiB
constexpr int kT8Slot = kT8ScaleOff + 3 * 1024;                // + row scales, two block scales
constexpr int kT8SinkOff = 2 * kT8Slot;                        // the other waves' (empty) scale copies
constexpr int kT8RedOff = kT8SinkOff + 1024;                   // [8 waves][64 rows] token amax
constexpr int kT8LdsBytes = kT8RedOff + kT8Waves * 64 * 4;
static_assert(kT8LdsBytes <= 160 * 1024 - 8 * 1024, "tiled FP8 GEMM exceeds LDS");

__device__ inline int t8_swz(int r) { return (r >> 1) & 7; }
__device__ inline int t8_clamp31(int64_t v) { return v > 0x7fffffff ? 0x7fffffff : (int)v; }

}  // namespace

// Tasks first, first + stride, ... below n_tiles x n_groups of the tiled list
// `tiles` (m-tiles of up to 256 rows).  Every wave of the workgroup calls it
// with the same arguments; it ends with every copy landed and every wave past
// its last LDS read (the caller may reuse the LDS).
template <bool GATEUP, bool I8>
__device__ __forceinline__ void tiled8_list(const GemmParams& p, const int4* tiles, const int n_tiles,
                                            const int first, const int stride) {
  extern __shared__ __attribute__((aligned(16))) uint8_t t8lds[];
  constexpr int WN = 2, NPW = kT8Panels / WN;   // 4 x 2 waves; 4 panels each
  constexpr int RT = 4, WR = 16 * RT;           // 4 token tiles of 16 rows: 64 rows per wave
  constexpr int A_OFF = kT8Panels * kStepPanelBytes;
  constexpr int B_DMA = kT8Panels * 4 / kT8Waves;            // 1 KiB weight copies per wave and step
  constexpr int A_DMA = kT8Rows * kStepBytes / 1024 / kT8Waves;  // 1 KiB row copies per wave and step
  static_assert(B_DMA * kT8Waves == kT8Panels * 4 && A_DMA * 8 * kT8Waves == kT8Rows, "copy split");
  static_assert(WR * (kT8Waves / WN) == kT8Rows, "wave grid");

  const int nq = p.n_groups;
  const int count = n_tiles * nq;
  if (first >= count) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int kg = lane >> 4;  // which 32 bytes of the 128-deep block this lane carries
  const int tok = lane & 15;
  const int ks = p.k_steps;
  const int oobA = t8_clamp31(p.a_bytes), oobS = t8_clamp31(p.a_scale_bytes);
  const int oobB = (int)p.b_expert_bytes;
  const int bpanel = (int)p.b_panel_bytes;
  const int wsb = p.b_scale_rows * p.b_scale_cols;  // block scales per expert and matrix
  const auto ra = make_rsrc(p.a, p.a_bytes);
  // this wave's scale copy: 0 = the tile's row scales, 1 / 2 = weight block
  // scale 0 / 1 of the step, -1 = none (its empty copy goes to the sink)
  const int scopy = wave < 3 ? wave : -1;
  const auto rs = scopy <= 0 ? make_rsrc(p.a_scales, p.a_scale_bytes)
                             : make_rsrc((GATEUP && scopy == 2) ? p.b_scales1 : p.b_scales0, p.b_scale_bytes);
  const int sstep = scopy <= 0 ? p.a_scale_ld * 4 : p.b_scale_cols * 4;
  const int soob = scopy <= 0 ? oobS : t8_clamp31(p.b_scale_bytes);
  float* const red = reinterpret_cast<float*>(t8lds + kT8RedOff);

  for (int task = first; task < count; task += stride) {
    // blocks of 4 m-tiles x all column groups, column group outer
    int mt, q;
    {
      const int full = (n_tiles / 4) * 4 * nq;
      if (task < full) {
        const int blk = task / (4 * nq), w = task % (4 * nq);
        q = w / 4;
        mt = blk * 4 + w % 4;
      } else {
        const int rem = n_tiles % 4, u = task - full;
        q = u / rem;
        mt = (n_tiles / 4) * 4 + u % rem;
      }
    }
    const int4 tile = load_tile(tiles, mt);
    const int expert = uniform(tile.x), row0 = uniform(tile.y), rows = uniform(tile.z);
    const auto rb = make_rsrc(p.b + (int64_t)expert * p.b_expert_bytes, p.b_expert_bytes);
    const int pbase = q * kT8Panels * bpanel;

    // Row copy k of a wave covers tile rows (wave A_DMA + k) 8 + [0, 8):
    // lane i -> row + i / 8, LDS part i % 8 holding the row's 16-byte part
    // (i % 8) ^ t8_swz(row); rows past the tile's count copy zeros
    int avoff[A_DMA];
#pragma unroll
    for (int k = 0; k < A_DMA; ++k) {
      const int r = (wave * A_DMA + k) * 8 + lane / 8;
      int off = oobA;
      if (r < rows) {
        const int rr = row0 + r;
        int src = rr;
        if (p.gather)
          src = rr >= p.shared_row0 ? (rr - p.shared_row0) % p.shared_tokens : p.sorted_assign[rr] / p.top_k;
        off = (int)((int64_t)src * p.a_row_bytes) + ((lane % 8) ^ t8_swz(r)) * 16;
      }
      avoff[k] = off;
    }
    // wave 0, lane i: the scales of rows 4i .. 4i+3 of the tile (block-FP8:
    // in a step); block-FP8 waves 1 and 2, lane 0: one block scale of the
    // step; W8A8 gate/up waves 1 and 2, lane i < 32: the gate / up scales of
    // columns 128q + 4i ..; W8A8 down wave 1, lane i: of columns 256q + 4i ..
    int svoff = soob;
    if (scopy == 0)
      svoff = (row0 + 4 * lane) * 4;
    else if (!I8 && scopy > 0 && lane == 0)
      svoff = (expert * wsb + (GATEUP ? q : 2 * q + (scopy - 1))) * 4;
    else if (I8 && GATEUP && scopy > 0 && lane < 32)
      svoff = (expert * p.b_scale_cols + 128 * q + 4 * lane) * 4;
    else if (I8 && !GATEUP && scopy == 1)
      svoff = (expert * p.b_scale_cols + 256 * q + 4 * lane) * 4;
    // W8A8: the task's scales, once (landed by the first step's wait)
    if constexpr (I8)
      if (scopy >= 0) dma16(rs, t8lds + kT8ScaleOff + scopy * 1024, svoff, 0);

    // step c into slot `slot`; `in` false copies zeros (steps past the end)
    auto issue = [&](const int c, const int slot, const bool in) {
      uint8_t* st = t8lds + slot * kT8Slot;
#pragma unroll
      for (int k = 0; k < B_DMA; ++k) {
        const int i = wave * B_DMA + k, panel = i / 4, j = i % 4;
        dma16(rb, st + panel * kStepPanelBytes + j * 1024, lane * 16,
              in ? pbase + panel * bpanel + c * kStepPanelBytes + j * 1024 : oobB);
      }
#pragma unroll
      for (int k = 0; k < A_DMA; ++k)
        dma16(ra, st + A_OFF + (wave * A_DMA + k) * 1024, avoff[k], in ? c * kStepBytes : oobA);
      if constexpr (!I8)
        dma16(rs, scopy >= 0 ? st + kT8ScaleOff + scopy * 1024 : t8lds + kT8SinkOff, svoff, in ? c * sstep : soob);
    };

    // fp32 accumulators (block-FP8, scaled per step) or int32 (W8A8, exact)
    typedef typename std::conditional<I8, i32x4, f32x4>::type acc_t;
    acc_t acc[RT][2 * NPW];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int b = 0; b < 2 * NPW; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[rt][b][r] = 0;

    // W8A8: per step, the token fragments as two 16-byte halves (the first
    // and the second 16 bytes of the lane's 32), then per half panel two
    // int8 MFMAs into the accumulator
    auto compute_i8 = [&](const uint8_t* st) {
      i32x4 xl[RT], xh[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = wm * WR + rt * 16 + tok;
        const uint8_t* rp = st + A_OFF + r * kStepBytes;
        const int sw = t8_swz(r);
        xl[rt] = *reinterpret_cast<const i32x4*>(rp + ((2 * kg) ^ sw) * 16);
        xh[rt] = *reinterpret_cast<const i32x4*>(rp + ((2 * kg + 1) ^ sw) * 16);
      }
      const int g = kg >> 1, j0 = (kg & 1) * 2;
#pragma unroll
      for (int pp = 0; pp < NPW; ++pp) {
        const int P = wn * NPW + pp;
        i32x4 wl[2], wh[2];
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          const uint8_t* lo = st + P * kStepPanelBytes + j0 * 1024 + (16 * sh + tok + 32 * g) * 16;
          wl[sh] = *reinterpret_cast<const i32x4*>(lo);
          wh[sh] = *reinterpret_cast<const i32x4*>(lo + 1024);
        }
#pragma unroll
        for (int sh = 0; sh < 2; ++sh)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            acc[rt][pp * 2 + sh] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wl[sh], xl[rt], acc[rt][pp * 2 + sh], 0, 0, 0);
            acc[rt][pp * 2 + sh] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wh[sh], xh[rt], acc[rt][pp * 2 + sh], 0, 0, 0);
          }
      }
    };

    auto compute = [&](const uint8_t* st) {
      const float* S = reinterpret_cast<const float*>(st + kT8ScaleOff);
      float sa[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sa[rt] = S[wm * WR + rt * 16 + tok];
      const float sw0 = S[256], sw1 = S[512];
      // the token fragments of the wave's 4 tiles: 32 bytes of row r per lane
      i32x8 x[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = wm * WR + rt * 16 + tok;
        const uint8_t* rp = st + A_OFF + r * kStepBytes;
        const int s = t8_swz(r);
        x[rt] = cat32v(*reinterpret_cast<const i32x4*>(rp + ((2 * kg) ^ s) * 16),
                       *reinterpret_cast<const i32x4*>(rp + ((2 * kg + 1) ^ s) * 16));
      }
      // weight fragment of a 16-column half panel: K bytes 32 kg .. +32 are
      // 1 KiB chunks 2(kg & 1), +1 of the panel's lane half kg >> 1
      const int g = kg >> 1, j0 = (kg & 1) * 2;
      i32x8 wf[2];
      auto read_wf = [&](const int pp) {
        const int P = wn * NPW + pp;
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          const uint8_t* lo = st + P * kStepPanelBytes + j0 * 1024 + (16 * sh + tok + 32 * g) * 16;
          wf[sh] = cat32v(*reinterpret_cast<const i32x4*>(lo), *reinterpret_cast<const i32x4*>(lo + 1024));
        }
      };
      // Groups (panel pp, half sh) of four MFMAs, one per token tile; each
      // group's products are scaled into the accumulators while the next
      // group's MFMAs run (scheduling fences keep that order: left alone, the
      // compiler reused one product register and waited on every MFMA), and a
      // panel's weight fragments are read right after its last MFMA issued.
      f32x4 t[2][RT];  // products of the groups of even / odd index
      read_wf(0);
#pragma unroll
      for (int grp = 0; grp <= 2 * NPW; ++grp) {
        if (grp < 2 * NPW) {
          const int pp = grp >> 1, sh = grp & 1;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            t[grp & 1][rt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[sh], x[rt], z, 0, 0, 0, 0, 0, 0);
          }
          if (sh == 1 && pp + 1 < NPW) read_wf(pp + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (grp > 0) {
          const int pg = grp - 1, pp = pg >> 1, sh = pg & 1;
          const int P = wn * NPW + pp;
          // gate/up: even panels gate, odd up; down: the 128-column block of the panel
          const float sb = GATEUP ? ((pp & 1) ? sw1 : sw0) : (P >= 4 ? sw1 : sw0);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const float sc = sa[rt] * sb;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) acc[rt][pp * 2 + sh][r4] += t[pg & 1][rt][r4] * sc;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // prologue, then per step: this wave's copies of the step have landed,
    // every wave's too after the barrier (and every wave is done with the
    // other slot), the next step goes into the other slot, the products
    issue(0, 0, true);
    for (int c = 0; c < ks; ++c) {
      wait_vmcnt<0>();
      lds_reads_done();
      raw_barrier();
      issue(c + 1, (c + 1) & 1, c + 1 < ks);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (I8)
        compute_i8(t8lds + (c & 1) * kT8Slot);
      else
        compute(t8lds + (c & 1) * kT8Slot);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();  // the empty copy past the end
    lds_reads_done();
    raw_barrier();    // every wave is done with the slots before the next task refills them

    // ------------------------------------------------------------- epilogue
    if constexpr (I8) {
      // W8A8: the task's scales from slot 0's scale area: row m at Sx[m];
      // gate/up: the gate and up scales of h column c at Sc0[c], Sc1[c];
      // down: output column c of the task at Sc0[c]
      const float* Sx = reinterpret_cast<const float*>(t8lds + kT8ScaleOff);
      const float* Sc0 = Sx + 256;
      const float* Sc1 = Sx + 512;
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
          if (kg == 0) red[wave * 64 + rt * 16 + tok] = a;
        }
        lds_reads_done();
        raw_barrier();
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int mi = rt * 16 + tok;
          const int m = wm * WR + mi;
          float amax = 0.0f;
#pragma unroll
          for (int w2 = 0; w2 < WN; ++w2) amax = fmaxf(amax, red[(wm * WN + w2) * 64 + mi]);
          if (m >= rows) continue;
          uint8_t* orow = p.c + (int64_t)(row0 + m) * p.c_row_bytes;
#pragma unroll
          for (int u = 0; u < NPW / 2; ++u) store_pair(orow, 4 * q + (wn * NPW) / 2 + u, h[rt][u], false);
          if (wn == 0 && kg == 0) p.c_scales[(int64_t)q * p.c_scale_ld + row0 + m] = amax;
        }
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float sx = Sx[wm * WR + rt * 16 + tok];  // (of a row past the task's: never stored)
#pragma unroll
          for (int pp = 0; pp < NPW; pp += 2) {
            const int P = q * kT8Panels + wn * NPW + pp;
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
      // the next task's scale copy rewrites the area (and red[])
      lds_reads_done();
      raw_barrier();
    } else {
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
          if (kg == 0) red[wave * 64 + rt * 16 + tok] = a;
        }
        lds_reads_done();
        raw_barrier();
  #pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int mi = rt * 16 + tok;
          const int m = wm * WR + mi;
          float amax = 0.0f;
  #pragma unroll
          for (int w2 = 0; w2 < WN; ++w2) amax = fmaxf(amax, red[(wm * WN + w2) * 64 + mi]);
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
        lds_reads_done();
        raw_barrier();  // red[] is rewritten by the next task
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int pp = 0; pp < NPW; pp += 2) {
            const int P = q * kT8Panels + wn * NPW + pp;
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
    }
  }
}

}  // namespace afd
