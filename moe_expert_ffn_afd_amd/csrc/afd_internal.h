// afd_internal.h -- shared definitions of the HIP kernels and the host API.
//
// Data layout in HBM (all owned by the library):
//
//  Packed expert weights, "panel-major fragment" order.  A panel is 32 output
//  columns of one weight matrix over its whole reduction length K, cut into
//  super-steps of 128 bytes of K (64 bf16 or 128 e4m3 elements).  One
//  super-step of one panel is 4 KiB laid out exactly as four 1 KiB MFMA
//  operand loads of a 64-lane wave: lane l holds column n = l % 32 and the
//  64 contiguous bytes of K that start at byte 64 * (l / 32) of the super-step.
//  Load j (0..3) of lane l is bytes [16 j, 16 j + 16) of that run, so each
//  load instruction of a wave reads 1 KiB of contiguous memory.
//    bf16: load j = MFMA 32x32x16 number j; element e of the load is
//          k = 64 c + 32 g + 8 j + e   (c = super-step, g = l / 32)
//    e4m3: loads (2i, 2i+1) = the 32-byte operand of MFMA 32x32x64 number i;
//          byte b of that operand is k = 128 c + 64 g + 32 i + b
//  Activation rows ([rows, K] row-major) are read with the same k mapping, so
//  A and B operands agree lane by lane (the MFMA sums over whatever k each
//  (lane group, element) pair carries, as long as both operands carry the same).
//
//  Gate/up weights of one expert are one buffer of 2 I / 32 panels with gate
//  panel p at index 2p and up panel p at 2p + 1 (a wave streams both with one
//  base pointer and finds gate and up of the same h column in the same
//  accumulator register).  Down weights of one expert are H / 32 panels.
//  The shared expert, if any, is stored as experts E .. E + S - 1: its
//  intermediate dimension cut into S parts of width I (the last zero-padded;
//  SwiGLU separates along it, and zero columns and rows add exactly nothing),
//  each run as an expert of its own over all T tokens.
//
//  Block-FP8 scales: gate [E+S][H/128][I/128], up likewise, down
//  [E+S][I/128][H/128] (fp32, copies of the caller's); one super-step is one
//  128-deep scale block and one panel lies inside one 128-column block.
//
//  Workspace (per handle, sized for max_tokens T_max; N_max = T_max * K):
//    counts[E], offsets[E+1], err[1], num_mtiles[4] (light tiles, heavy tiles,
//    light workgroups of a mixed bf16 launch, the launch the dispatch chose)
//    chunk_base[n_chunks][E]          first sorted row of each (chunk, expert)
//    sorted_assign[N_max], row_of[N_max]
//    mtiles[max_mtiles] (int4) x 2    light and heavy lists {expert, first row, rows, 0}
//    h   [N_max + S T_max, I]         routed rows in sorted order, then the
//                                     shared expert's parts' rows (part-major,
//                                     token order) from row N_max; bf16 | e4m3 | fp32
//    FP8 activation scales, step-major over the same rows (one 128-deep
//    block per "step", so a tile's scales of one step are contiguous):
//    xs  [H/128][N_max + T_max]       the caller's 1x128 hidden scales,
//                                     gathered into sorted-row order
//    hs  [I/128][N_max + T_max]       h's 1x128 scales
//    y   [N_max + T_max, H]           expert outputs (unweighted), same rows;
//                                     bf16 | fp32
//  W8A8 layers (one scale per token and per output channel): h is bf16 as
//  the gate/up GEMM writes it, then h8 [N_max + T_max, I] int8 codes with
//  hs [N_max + T_max] one scale per row (quant.hip), xs [N_max + T_max] the
//  caller's per-token hidden scales in sorted-row order, and
//  pamax [I/128][N_max + T_max] each row's amax per 128-column task.  Weight
//  scales are copied as gate, up [E+S][I] and down [E+S][H].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace afd {

enum Dtype : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kW8A8 = 3 };

constexpr int kPanelCols = 32;         // output columns per panel
constexpr int kStepBytes = 128;        // bytes of K per super-step and row
constexpr int kStepPanelBytes = 4096;  // one super-step of one panel
constexpr int kWaves = 4;              // waves per GEMM workgroup
constexpr int kXcds = 8;               // accelerator complex dies of an MI355X (one L2 each)
constexpr int kDispatchThreads = 1024;
constexpr int kDispatchLdsInts = 12288;  // chunk x expert counters held in LDS (48 KiB)
constexpr int kMaxExperts = 512;
constexpr int kDispatchFuseSlots = 4096;  // up to this many flat slots: one dispatch launch
constexpr int kMaxTopK = 32;
constexpr int kMaxSharedParts = 16;  // a shared expert of up to 16 times the routed experts' width
constexpr int kMaxRowsPerToken = kMaxTopK + kMaxSharedParts;  // rows the combine adds per token

struct DispatchParams {
  const int32_t* ids;      // [n_flat]
  int32_t n_flat;          // T * K
  int32_t num_experts;     // E
  int32_t chunk_shift;     // chunk = 1 << chunk_shift flat slots (>= 10)
  int32_t n_chunks;
  int32_t* counts;         // [E]
  int32_t* offsets;        // [E+1]
  int32_t* chunk_base;     // [n_chunks][E]
  int32_t* err;            // [1] ids outside [-1, E)
  int32_t* sorted_assign;  // [n_flat]
  int32_t* row_of;         // [n_flat]
  int32_t bm_light;        // rows per m-tile of light experts (streaming GEMM)
  int32_t bm_heavy;        // rows per m-tile of heavy experts (LDS-tiled GEMM)
  int32_t heavy_min_rows;  // experts with at least this many rows are heavy
  int32_t shared_rows;     // T when a shared expert exists, else 0
  int32_t shared_row0;     // first shared row (N_max)
  int32_t shared_parts;    // the shared expert's parts of width I (experts E .. E + parts - 1), rows
                           // shared_row0 + v T + t for part v and token t
  int4* mtiles;            // light tile list
  int4* mtiles_heavy;      // heavy tile list
  int4* mtiles_tiled;      // 8-bit layers: tiled list (experts of at least tiled_min_rows rows)
  int32_t bm_tiled;        // rows per m-tile of the tiled list
  int32_t tiled_min_rows;  // experts with at least this many rows take the tiled list (a huge
                           // value: no tiled list)
  int32_t* num_mtiles;     // [8]: light tiles, heavy tiles, light workgroups of the mixed
                           //      GEMM, launch the dispatch chose (kLaunchLight / kLaunchMixed),
                           //      tiled tiles, 3 spare
  int32_t fused;           // 1: count_scan also places the slots (n_flat <= kDispatchFuseSlots)
  int32_t mix_cus;         // > 0: workgroups of the mixed bf16 GEMM launches (one per CU)
  int32_t auto_heavy_rows; // > 0: heavy experts only when some expert has at least this many
                           //      rows; else every expert is light, in tiles of bm_light_only
                           //      rows; 0: heavy_min_rows alone
  int32_t bm_light_only;   // light tile rows when auto_heavy_rows keeps every expert light
  int32_t* pool;           // [2] the GEMMs' tail-pool counters, zeroed here (or nullptr)
};

// The launch the dispatch chose for a bf16 call whose routing the host cannot
// see (num_mtiles[3]): the streaming GEMM over the light list alone, or the
// mixed GEMM over both lists.  The host launches both kernels with gates; the
// one not chosen returns at once.
constexpr int32_t kLaunchLight = 1;
// rows of the 8-bit LDS-tiled GEMM's m-tiles, and the fewest routed rows per
// expert on average (and the fewest of an expert) that use it
constexpr int kTiled8Rows = 256;
// 8-bit batches of at least kTiled8MeanRows routed rows per expert on average
// put every expert of more rows than one 128-row ring tile in the tiled list
constexpr int kTiled8MeanRows = 128;
constexpr int kTiled8MinRows = 129;
constexpr int32_t kLaunchMixed = 2;

// Cost of one heavy bf16 m-tile (tiled_rows() rows, both GEMMs) in units of
// one light m-tile, each on one CU: a heavy tile's MFMA time against a light
// tile's weight stream at the rate one light workgroup sustains beside the
// heavy ones (about 37 GB/s).  Measured on the aggregated Zipf batch: a heavy
// tile takes about 2.2 ms of one CU, a light one about 1.0 ms, and of the
// ratios tried (1.8, 2.2, 2.8) 1.8-2.2 balance the two roles; the ratio does
// not depend on H or I (both costs scale with H*I).  The dispatch splits the
// mixed launch's workgroups in proportion to the two lists' costs.
#ifndef AFD_HEAVY_TILE_COST
#define AFD_HEAVY_TILE_COST 2.2f
#endif
constexpr float kHeavyTileCost = AFD_HEAVY_TILE_COST;

struct GemmParams {
  const int4* mtiles;
  const int32_t* num_mtiles;     // [0] tiles of mtiles; [3] the launch the dispatch chose
  const int4* mtiles2;           // block-FP8 ring GEMM: the heavy list, run before `mtiles`
  const int32_t* num_mtiles2;
  const int4* mtiles3;           // 8-bit layers: the tiled list (gemm_tiled8.h), run first;
  const int32_t* num_mtiles3;    // nullptr: none
  const int32_t* sorted_assign;  // row -> flat slot (gate/up gather)
  int32_t top_k;
  int32_t shared_row0;           // rows >= this are shared-expert rows: token (row - shared_row0) % shared_tokens
  int32_t shared_tokens;         // T (the shared expert's parts lie one after another)
  int32_t gather;                // 1: A row = hidden[token of row]; 0: A row = a[row]
  const uint8_t* a;              // activation rows
  int64_t a_bytes;               // size of the activation buffer (< 2^31)
  int64_t a_row_bytes;
  const float* a_scales;         // fp8: step-major [K/128][a_scale_ld], sorted-row order
  int64_t a_scale_bytes;
  int32_t a_scale_ld;            // rows per step of a_scales
  const uint8_t* b;              // packed weights
  int64_t b_expert_bytes;
  int64_t b_panel_bytes;
  const float* b_scales0;        // fp8: gate (gate/up) or down scales
  const float* b_scales1;        // fp8: up scales (gate/up only)
  int64_t b_scale_bytes;         // fp8: bytes of each block-scale array (all experts)
  int32_t b_scale_rows;          // K / 128
  int32_t b_scale_cols;          // N / 128 of one matrix
  int32_t k_steps;               // K / super-step
  int32_t n_groups;              // workgroup tasks per m-tile along N
  int32_t n_panels;              // panels of one output matrix (I/32 or H/32)
  int32_t only_launch;           // 0: always run; kLaunchLight / kLaunchMixed: return at once
                                 // unless the dispatch chose that launch (num_mtiles[3])
  int32_t* pool;                 // [2] tail-pool counters (gate/up, down), zeroed by the dispatch:
                                 // the ring GEMM's light list, the bf16 heavy tiles; nullptr: no pool
  uint8_t* c;                    // output rows
  int64_t c_row_bytes;
  float* c_scales;               // fp8 gate/up: h scales, step-major [I/128][c_scale_ld]
  int32_t c_scale_ld;
};

// W8A8: h (bf16) -> int8 codes with one scale per row (quant.hip)
struct QuantParams {
  const uint8_t* h;        // [ld rows][inter] bf16
  const float* pamax;      // [inter / 128][ld]: each row's amax over each 128-column group
  int32_t ld;              // rows of the buffers
  int32_t inter;           // I
  const int32_t* offsets;  // offsets[num_experts] = routed rows of this call
  int32_t num_experts;
  int32_t routed_max;      // T * K (upper bound of the routed rows)
  int32_t shared_row0;     // first shared-expert row, -1 if none
  int32_t shared_rows;     // T with a shared expert, else 0
  int8_t* h8;              // [ld rows][inter] codes
  float* hsc;              // [ld] per-row scales
};

struct ScaleGatherParams {
  const float* src;              // caller's hidden scales [T][ks]
  int32_t ks;                    // H / 128
  int32_t tokens;                // T
  int32_t top_k;
  const int32_t* sorted_assign;  // row -> flat slot
  const int32_t* offsets;        // offsets[E] = routed rows
  int32_t num_experts;
  int32_t routed_max;            // T * K of this call (upper bound of the routed rows)
  int32_t shared_row0;           // N_max with a shared expert, else -1
  int32_t shared_parts;          // the shared expert's parts (rows shared_row0 + v T + t)
  float* dst;                    // [ks][ld]
  int32_t ld;
};

struct CombineParams {
  const uint8_t* y;        // [rows, H] bf16 | f32
  int64_t y_bytes;         // size of y (< 2^31)
  const int32_t* row_of;   // [T, K]
  const float* weights;    // [T, K]
  int32_t top_k;
  int32_t hidden;
  int32_t shared_row0;     // -1 when no shared expert
  int32_t shared_parts;    // the shared expert's parts: rows shared_row0 + v shared_stride + t, v in order
  int32_t shared_stride;   // T
  uint8_t* out;            // [T, H]
};

struct F32Params {
  const int4* mtiles;
  const int32_t* num_mtiles;
  const int32_t* sorted_assign;
  int32_t top_k;
  int32_t shared_row0;
  int32_t shared_tokens;    // T: shared rows map to tokens (row - shared_row0) % T
  int32_t gather;
  const float* a;           // [*, K] rows
  const float* w0;          // gate (gate/up) or down: [E+S][K][N]
  const float* w1;          // up
  int32_t kdim, ndim;
  float* c;                 // [rows, N]
};

// The whole layer in one persistent launch (fused.hip: block-FP8 and W8A8;
// fused_bf16.hip: bf16): the dispatch's, the GEMM stages' and the combine's
// parameters plus the grid-barrier state, all in the handle's workspace.
constexpr int kFusedMaxGrid = 512;  // workgroups of one fused launch (one chunk count per thread)
struct FusedParams {
  DispatchParams d;       // ids, sizes, outputs and tile-list parameters of the dispatch
  const float* x_src;     // the caller's hidden scales [T][ks]
  int32_t ks;             // block-FP8: H / 128; W8A8: 1
  float* x_dst;           // [ks][ld] in sorted-row order
  int32_t ld;             // rows of the activation buffers
  int32_t tokens;         // T
  int32_t top_k;
  GemmParams gu, dn;      // the two GEMM stages (light list in mtiles; 8-bit: heavy in mtiles2)
  GemmParams gu_heavy, dn_heavy;  // bf16: the heavy list (LDS-tiled body)
  GemmParams gu_lo, dn_lo;        // bf16: the light list when the dispatch keeps every expert light
  int32_t auto_launch;            // bf16: the dispatch chooses light-only or mixed (num_mtiles[3])
  QuantParams qp;         // W8A8: h to int8
  CombineParams cp;
  int32_t* bar;           // [4]: arrivals, departures, timed-out spins, spare (zero between calls)
  int32_t* chunk_counts;  // [grid][E] per-chunk expert counts
  int32_t* chunk_bad;     // [grid] ids outside [-1, E) per chunk
  int32_t* local_base;    // [grid][E] exclusive prefix of the chunk counts per expert
  int32_t* totals;        // [E]
  int32_t spin_limit;     // rounds a barrier spin waits before it counts a timeout and goes on
};

// launchers (return hipError_t of the launch)
hipError_t launch_dispatch_count_scan(const DispatchParams& p, hipStream_t s);
hipError_t launch_dispatch_scatter(const DispatchParams& p, hipStream_t s);
hipError_t launch_gather_scales(const ScaleGatherParams& p, hipStream_t s);
// bf16 only: streaming (gemm.hip) and LDS-tiled (gemm_tiled.hip) GEMMs;
// down_panels_per_task(mr): H panels of one streaming down task
int down_panels_per_task(int mr);
hipError_t launch_gemm(int dtype, bool gate_up, int mr, const GemmParams& p, int64_t max_tasks,
                       int num_cus, hipStream_t s);
// bf16 layers with heavy experts (gemm_tiled.hip): one launch of num_cus
// workgroups runs the heavy list (LDS-tiled) and the light list (streaming)
// side by side, split as the dispatch decided (num_mtiles[2])
hipError_t launch_gemm_mixed(bool gate_up, int mr, const GemmParams& heavy, const GemmParams& light, int num_cus,
                             hipStream_t s);
int tiled_rows(int dtype);  // m-tile rows of the LDS-tiled GEMM
int tiled_panels();         // weight panels of one LDS-tiled task
// Block-FP8 GEMM with a weight ring in LDS (gemm_ring.hip): one launch over
// the heavy list (mtiles2, m-tiles of up to ring_rows(true) rows) and then the
// light list (mtiles, up to ring_rows(false) rows)
// stream_weights: weight copies non-temporal (no other forward runs beside this one)
// int8: W8A8 codes (int8 MFMA, int32 accumulation, per-token and per-channel
// scales in the epilogue; gate/up writes bf16 h and per-row amax per task)
hipError_t launch_gemm_ring(bool gate_up, bool stream_weights, bool int8, const GemmParams& p, int64_t max_tasks,
                            int num_cus, hipStream_t s);
int ring_rows(bool heavy);
// 8-bit experts of many rows (gemm_tiled8.h): the tiled list (mtiles3) of a
// stage, launched before that stage's ring kernel (which then skips it)
hipError_t launch_gemm_tiled8(bool gate_up, bool int8, const GemmParams& p, int64_t max_tasks, int num_cus,
                              hipStream_t s);
hipError_t launch_gemm_f32(bool gate_up, const F32Params& p, int grid, hipStream_t s);
hipError_t launch_quant_rows(const QuantParams& p, hipStream_t s);
// calib.hip: the MFMA rate sustained with no memory traffic (kind 0 bf16,
// 1 e4m3, 2 int8) on num_cus CUs, and the shader clock meanwhile; synchronous
hipError_t mfma_peak(int kind, int num_cus, int iters, double* tflops, double* clock_ghz);
// one workgroup per CU of num_cus (all resident at once); stream_weights and
// int8 as for launch_gemm_ring
hipError_t launch_fused(bool stream_weights, bool int8, const FusedParams& f, int num_cus, hipStream_t s);
// bf16: mr_lo / mr the row fragments of the light-only / mixed launches' light tiles
hipError_t launch_fused_bf16(int mr_lo, int mr, const FusedParams& f, int num_cus, hipStream_t s);
hipError_t launch_combine(int dtype, const CombineParams& p, int tokens, hipStream_t s);
hipError_t launch_pack(int dtype, bool gate_up, const void* w_first, const void* w_second,
                       int64_t expert_in_stride_elems, int experts, int kdim, int ndim,
                       uint8_t* dst, int64_t dst_expert_bytes, hipStream_t s);

}  // namespace afd
