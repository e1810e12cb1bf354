/*
 * afd_ffn.h -- C ABI of the expert (FFN) side of an attention-FFN
 * disaggregated mixture-of-experts layer, for one AMD MI355X (gfx950).
 *
 * The operation (sources: "FastAFD" structured summary, System Design items
 * 1-4 and the legend of Eq. (3); vLLM AFD plugin blog, "FFN service" and
 * "connector layer"): the attention side keeps norms, projections and top-k
 * routing and publishes, per layer, token hidden states (block-FP8 in FastAFD)
 * with the routing metadata; the FFN side runs the routed experts' FFNs as
 * grouped GEMMs with the activation and returns the combined output.  This
 * library is that FFN-side computation on one GPU, for one layer and one
 * batch of tokens:
 *
 *   out[t] = sum_{k: ids[t,k] >= 0} w[t,k] * FFN_{ids[t,k]}(x_t)  (+ FFN_S(x_t))
 *   FFN_e(x) = Wd_e^T ( silu(Wg_e^T x) * (Wu_e^T x) )
 *
 * computed as: per-expert histogram of the ids, exclusive prefix scan,
 * stable expert-major permutation of the (token, slot) assignments, grouped
 * GEMM gate/up with fused SwiGLU, grouped GEMM down, and the top-k weighted
 * combine.  The pages do not spell the expert FFN out; SwiGLU is the reading
 * taken here.
 *
 * Conventions shared by every entry point:
 *  - Pointers named "device" point to GPU memory of the handle's device; the
 *    library never copies them to the host.  Rows are row-major, contiguous.
 *  - Every call returns an afd_status; nothing is thrown across the ABI.
 *    Argument and shape errors are found on the host before any GPU work;
 *    afd_ffn_last_error() then holds a message for the calling thread.
 *  - Work is enqueued asynchronously on the `stream` argument (a hipStream_t
 *    passed as void*; NULL = the device's null stream) and never synchronised
 *    by the library, except where an entry point says otherwise.
 *  - A handle may be used by one stream at a time: its workspace is reused
 *    by every forward.  Use afd_ffn_clone for a second concurrent stream.
 *  - The library must be loaded into a process whose HIP runtime is the one
 *    the caller allocates with (e.g. after `import torch` on ROCm).
 */
#ifndef AFD_FFN_H
#define AFD_FFN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct afd_ffn afd_ffn_t; /* opaque handle */

typedef enum {
    AFD_OK = 0,
    AFD_ERR_INVALID_ARG = 1,   /* NULL pointer, bad size, T > max_tokens ...   */
    AFD_ERR_UNSUPPORTED = 2,   /* shape or dtype the library does not handle     */
    AFD_ERR_OUT_OF_MEMORY = 3, /* device allocation failed in create / clone     */
    AFD_ERR_HIP = 4,           /* a HIP runtime call failed (message has it)     */
    AFD_ERR_BAD_ROUTING = 5    /* ids outside [-1, E) were seen (error query)    */
} afd_status;

typedef enum {
    AFD_DTYPE_F32 = 0,       /* fp32 activations, weights and output            */
    AFD_DTYPE_BF16 = 1,      /* bf16 activations, weights and output            */
    AFD_DTYPE_FP8_BLOCK = 2, /* OCP E4M3FN codes with fp32 scales: activations
                                per 1x128 group along H, weights per 128x128
                                block; output bf16 ("block-FP8" experts and FP8
                                tokens, FastAFD System Design items 1-2)        */
    AFD_DTYPE_W8A8 = 3       /* symmetric int8 codes with fp32 scales:
                                activations one per token, weights one per output
                                channel; int32 accumulation, h re-quantised per
                                row, output bf16 (the "W8A8" experts of the vLLM
                                AFD plugin blog's decode benchmark)             */
} afd_dtype;

/*
 * Layer description for afd_ffn_create.  H = hidden, I = inter,
 * E = num_experts (experts on this GPU), K = top_k.
 *
 * Weights (device, read only during afd_ffn_create, which copies and
 * re-lays them out into library-owned memory; the caller may free them as
 * soon as create returns):
 *   w_gate, w_up  [E, H, I]   element type per dtype (fp32 | bf16 | e4m3 code | int8)
 *   w_down        [E, I, H]
 *   s_gate, s_up  [E, H/128, I/128] fp32 block scales (AFD_DTYPE_FP8_BLOCK),
 *                 [E, I] fp32 per-column scales (AFD_DTYPE_W8A8), else NULL
 *   s_down        [E, I/128, H/128] (AFD_DTYPE_FP8_BLOCK), [E, H] (AFD_DTYPE_W8A8),
 *                 else NULL
 * Optional shared expert (shared_inter > 0, a multiple of 128 of at most
 * 16 x inter; applied to every token with weight 1 after the routed sum; one of
 * another width than the routed experts runs as ceil(shared_inter / inter)
 * parts of width inter, the last zero-padded, whose outputs the combine adds
 * in order):
 *   sh_gate, sh_up [H, shared_inter], sh_down [shared_inter, H], and for FP8
 *   sh_s_gate, sh_s_up [H/128, shared_inter/128], sh_s_down [shared_inter/128, H/128]
 *   (W8A8: sh_s_gate, sh_s_up [shared_inter], sh_s_down [H]).
 *
 * Alignment: bf16 and e4m3 weights 16-byte aligned, fp32 weights and all
 * scale arrays 4-byte aligned (otherwise AFD_ERR_INVALID_ARG).
 *
 * Limits: 1 <= E <= 512, 1 <= K <= 32, 1 <= max_tokens, max_tokens*K < 2^26;
 * H and I multiples of 128 for every dtype (block-FP8 and W8A8: at most 16384); the
 * activation buffers (max_tokens*K (+ max_tokens with a shared expert) rows of
 * max(H, I) elements and of H bf16/fp32 outputs, and max_tokens rows of H)
 * below 2^31 - 2^24 bytes each.
 * A configuration outside these limits is rejected with AFD_ERR_UNSUPPORTED.
 */
typedef struct {
    int32_t hidden;        /* H                                                */
    int32_t inter;         /* I                                                */
    int32_t num_experts;   /* E                                                */
    int32_t top_k;         /* K                                                */
    int32_t max_tokens;    /* largest T any forward will pass                  */
    int32_t shared_inter;  /* 0 = no shared expert                             */
    int32_t dtype;         /* afd_dtype                                        */
    int32_t device;        /* HIP device ordinal the handle lives on           */
    const void *w_gate, *w_up, *w_down;
    const float *s_gate, *s_up, *s_down;
    const void *sh_gate, *sh_up, *sh_down;
    const float *sh_s_gate, *sh_s_up, *sh_s_down;
} afd_ffn_config;

/* Host-only check of a configuration: the same checks afd_ffn_create makes
 * before touching the GPU (no HIP call is made). */
afd_status afd_ffn_validate_config(const afd_ffn_config *cfg);

/* Create a handle: validates `cfg`, allocates library-owned device memory
 * for the re-laid-out weights and a workspace sized for max_tokens, and packs
 * the weights (synchronously, on the device's null stream).  On success
 * *out_handle owns all of it; on failure nothing is leaked and *out_handle is
 * set to NULL. */
afd_status afd_ffn_create(const afd_ffn_config *cfg, afd_ffn_t **out_handle);

/* A second handle sharing src's packed weights (reference counted) with a
 * workspace of its own, so two microbatches can run on two streams at once
 * (FastAFD System Design item 4: two ping-pong microbatches). */
afd_status afd_ffn_clone(const afd_ffn_t *src, afd_ffn_t **out_handle);

/* How many forwards the caller runs at once on different streams (the
 * handle and its clones), 1 <= streams <= the device's CU count; default 1,
 * and a clone starts with its source's value.  The GEMM kernels keep
 * persistent grids resident: with streams = N each call's grids take 1/N of
 * the CUs, so concurrent calls (FastAFD System Design item 4: two ping-pong
 * microbatches) run side by side instead of one queueing behind the other's
 * resident workgroups; with streams > 1 the block-FP8 weight copies also
 * stay cacheable, so microbatches reading the same experts at about the same
 * time can share them.  Affects scheduling only, never results.  Returns
 * AFD_ERR_INVALID_ARG (handle unchanged) for a NULL handle or a value out of
 * range. */
afd_status afd_ffn_set_concurrency(afd_ffn_t *handle, int32_t streams);

/*
 * Run each later forward of this handle as ONE persistent launch instead of
 * five to eight (enable = 1), or as separate launches (0, the default).
 * FastAFD's expert GPUs run the MoE layer as one persistent kernel (System
 * Design item 3; the "Ablation Results" credit that fusion with about half the
 * step latency of separate kernels).  Here the launch runs the dispatch (every
 * workgroup counting and placing a chunk of the slots), gate/up + SwiGLU, the
 * W8A8 re-quantisation of h, down and the combine, separated by grid barriers
 * (bf16: each GEMM stage as the light-only or the mixed light + heavy split
 * the dispatch chooses, as the separate launches do); results are
 * bit-identical to the separate launches.  One workgroup per CU of
 * the call's share (afd_ffn_set_concurrency), all resident at once: the
 * caller must not keep other kernels occupying those CUs for long (a barrier
 * wait gives up after about a second, counts a timeout and goes on, so the
 * GPU never hangs, but that call's results are wrong; see
 * afd_ffn_fused_errors).  bf16, block-FP8 and W8A8 handles (fp32:
 * AFD_ERR_UNSUPPORTED); a clone starts with its source's setting;
 * afd_ffn_forward_noalloc always uses separate launches.  With timing on, the
 * whole launch is reported as stage 2 and the other stages as about 0.
 */
afd_status afd_ffn_set_fused(afd_ffn_t *handle, int32_t enable);

/* Timed-out grid-barrier waits of the handle's fused forwards since the last
 * query (synchronises the stream; *count is host memory; resets the count).
 * Returns AFD_ERR_HIP if > 0. */
afd_status afd_ffn_fused_errors(afd_ffn_t *handle, int32_t *count, void *stream);

/*
 * One layer forward for T = num_tokens tokens (0 <= T <= max_tokens):
 *   hidden         device [T, H]: fp32 | bf16 | e4m3 codes | int8 codes (per dtype)
 *   hidden_scales  device fp32: [T, H/128] for AFD_DTYPE_FP8_BLOCK, [T] (one per
 *                  token) for AFD_DTYPE_W8A8, else NULL
 *   topk_ids       device [T, K] int32; each in [0, E) or -1 ("expert not on
 *                  this GPU": contributes nothing).  Duplicate ids in a row
 *                  are separate assignments.  Ids outside [-1, E) are treated
 *                  as -1 and counted (see afd_ffn_routing_errors).
 *   topk_weights   device [T, K] fp32, used exactly as given
 *   out            device [T, H]: fp32 for AFD_DTYPE_F32, else bf16; every
 *                  element is written (rows with no local expert and no shared
 *                  expert are 0).  Must not alias the inputs.
 * hidden and out must be 16-byte aligned; hidden_scales, topk_ids and
 * topk_weights 4-byte aligned (otherwise AFD_ERR_INVALID_ARG, checked on the
 * host).  Asynchronous on `stream`; inputs and out must stay valid until the
 * stream work completes.  The dispatch (counts, offsets, permutation) of this call
 * stays in the handle's workspace until the next forward on the handle.
 * With timing off, a forward allocates nothing, waits for nothing and records
 * no memset, so it may be captured into a HIP graph on `stream` and replayed;
 * a replay recomputes everything from the captured pointers, and the handle's
 * workspace is shared with any other forward on the handle (replays and eager
 * calls on one handle must not overlap).
 */
afd_status afd_ffn_forward(afd_ffn_t *handle, int32_t num_tokens, const void *hidden,
                           const float *hidden_scales, const int32_t *topk_ids,
                           const float *topk_weights, void *out, void *stream);

/*
 * For callers that cannot allocate device memory when they run a layer: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same forward as afd_ffn_forward (same arguments, kernels and
 * results, bit for bit), except that its workspace (dispatch arrays, tile
 * lists, h, y and the FP8 activation scales) lies in a static device array of
 * the library, AFD_FFN_NOALLOC_SCRATCH_BYTES bytes per device, instead of the
 * handle's workspace.  It calls no allocating routine; the array's device
 * address is looked up once per device, at the first such call there (a
 * device holds the array until the process ends).  0 <= T is limited by that size, not by max_tokens: a call
 * whose workspace would exceed it returns AFD_ERR_UNSUPPORTED before any GPU
 * work (about 23 MiB for 256 tokens of H = 4096, I = 1536, K = 8 bf16; about
 * 150 KiB per token of H = 7168, I = 2048, K = 8 block-FP8 with a shared
 * expert).  No part of the array needs clearing: every element a call reads is
 * written earlier by that call.  Every such call on a device shares that
 * device's array, so calls that overlap on one device (on two streams, or a
 * replay beside an eager call) race and give wrong results; calls on one
 * stream one after another are fine.  Timing (afd_ffn_set_timing) and
 * afd_ffn_debug_dispatch do not apply to these calls.
 */
#define AFD_FFN_NOALLOC_SCRATCH_BYTES (64u << 20)
afd_status afd_ffn_forward_noalloc(afd_ffn_t *handle, int32_t num_tokens, const void *hidden,
                                   const float *hidden_scales, const int32_t *topk_ids,
                                   const float *topk_weights, void *out, void *stream);

/* Release a handle (NULL is accepted).  Packed weights are freed when their
 * last sharer is destroyed.  Call only after the handle's stream work has
 * completed. */
afd_status afd_ffn_destroy(afd_ffn_t *handle);

/* Static text for a status code. */
const char *afd_ffn_status_string(afd_status status);

/* Message of the last failed call on the calling thread ("" if none). */
const char *afd_ffn_last_error(void);

/*
 * Copy the dispatch of the last forward into caller device buffers
 * (asynchronous on `stream`; any pointer may be NULL to skip it):
 *   counts        [E]      assignments per expert
 *   offsets       [E+1]    exclusive prefix sums, offsets[E] = N
 *   sorted_assign [N]      flat slot indices t*K+k, expert by expert, each
 *                          expert's in ascending flat order
 *   row_of        [T, K]   position of slot (t,k) in sorted_assign, -1 if none
 * N = number of slots with a valid id; the caller sizes sorted_assign for T*K.
 */
afd_status afd_ffn_debug_dispatch(afd_ffn_t *handle, int32_t *counts, int32_t *offsets,
                                  int32_t *sorted_assign, int32_t *row_of, void *stream);

/* Number of ids outside [-1, E) seen by the last forward (synchronises the
 * stream; *count is host memory).  Returns AFD_ERR_BAD_ROUTING if > 0. */
afd_status afd_ffn_routing_errors(afd_ffn_t *handle, int32_t *count, void *stream);

/*
 * Canary-guarded workspace, a memory-safety check for tests (GPU address
 * sanitizers are not available for these kernels): with guard_bytes > 0 (a
 * multiple of 256, at most 16 MiB) the handle's workspace is allocated again
 * with a band of guard_bytes bytes of the canary value 0xA5 before its first
 * buffer and right after the last byte of every buffer it holds (dispatch
 * arrays, tile lists, pool counters, h, its scales, y, the fused launch's
 * state); 0 removes the bands.  Synchronises the device and frees the old
 * workspace, so no forward of this handle may be in flight; the dispatch of
 * the last forward is forgotten.  Results of later forwards are unchanged.
 * A clone starts with its source's setting.  afd_ffn_forward_noalloc does
 * not use the handle's workspace and is not covered.  Returns
 * AFD_ERR_INVALID_ARG for a bad size, AFD_ERR_OUT_OF_MEMORY if the new
 * workspace does not fit (the old one is kept).
 */
afd_status afd_ffn_set_canaries(afd_ffn_t *handle, int64_t guard_bytes);

/* Check every guard band of the handle's workspace (synchronises the stream,
 * then copies the bands to the host; *damaged_bytes is host memory): the
 * number of band bytes that no longer hold the canary.  Returns
 * AFD_ERR_HIP if > 0 (afd_ffn_last_error names the buffers the damaged
 * bands follow), AFD_ERR_INVALID_ARG if the handle has no canaries. */
afd_status afd_ffn_check_canaries(afd_ffn_t *handle, int64_t *damaged_bytes, void *stream);

/* Test facility: overwrite byte `offset` of guard band `band` (0 = the band
 * before the first buffer, then one per non-empty buffer in workspace order)
 * with a value other than the canary, from the host (synchronises the
 * device), so a test can show that afd_ffn_check_canaries finds the damage
 * and names the buffer the band follows.  AFD_ERR_INVALID_ARG without
 * canaries or for a band or offset out of range. */
afd_status afd_ffn_debug_poke_canary(afd_ffn_t *handle, int32_t band, int64_t offset);

/*
 * Per-kernel timing of forwards, for measurement.  When enabled, forward
 * records HIP events on its stream around each timed stage; the query
 * synchronises on each forward's last event and returns, per stage, the
 * summed time in milliseconds (0 for stages not timed) and the number of
 * forwards since the last reset, then resets.  Stages: 0 dispatch
 * count+scan, 1 dispatch scatter, 2 grouped GEMM gate/up + SwiGLU, 3 grouped
 * GEMM down, 4 combine.  ms must hold AFD_NUM_STAGES floats.
 *
 * set_timing: every stage (enable != 0) or none.  set_timing_stages: the
 * stages whose bit is set in stage_mask (bit s = stage s; 0 = none); each
 * event costs the stream a few microseconds, so a measurement loop times
 * only the stages it needs.  AFD_ERR_INVALID_ARG for a NULL handle or a bit
 * at AFD_NUM_STAGES or above.  The setting applies to later forwards.
 */
/*
 * Measurement helper (not part of a forward): the MFMA rate this device
 * sustains with no memory traffic, the ceiling the grouped GEMMs' MFMA
 * fractions are read against.  8 waves per CU each keep independent MFMA
 * chains of the dtype's kind busy for `iters` rounds (AFD_DTYPE_BF16: 32x32x16
 * bf16; AFD_DTYPE_FP8_BLOCK: 16x16x128 e4m3, the block-scaled kind;
 * AFD_DTYPE_W8A8: 16x16x64 int8).  *tflops: flops (int8: operations) per
 * second over the launch; *clock_ghz: the shader clock the loop ran at (shader
 * clock counter against the constant 100 MHz counter).  Allocates a few bytes,
 * synchronises the device; AFD_ERR_UNSUPPORTED for fp32.
 */
afd_status afd_ffn_mfma_peak(int32_t dtype, int32_t device, int32_t iters, double *tflops, double *clock_ghz);

/*
 * Measurement helper (not part of a forward): the bf16 MFMA rate of the
 * LDS-tiled GEMM's inner loop without its memory traffic.  8 waves per CU each
 * issue, per step, the eight 32x32x16 bf16 MFMAs of a 64-row x 4-panel wave
 * tile's 16-deep k slice; with lds_reads = 6 they first read that step's six
 * 16-byte fragments from LDS (two activation, four weight fragments: the
 * GEMM's ratio of LDS reads to MFMAs), with lds_reads = 0 the fragments stay
 * in registers.  `iters` steps (rounded down to a multiple of 3, at least 3).
 * *tflops: flops per second over the launch; *clock_ghz as for
 * afd_ffn_mfma_peak.  AFD_ERR_INVALID_ARG for lds_reads other than 0 or 6.
 * Allocates a few bytes, synchronises the device.
 */
afd_status afd_ffn_mfma_lds_peak(int32_t device, int32_t iters, int32_t lds_reads, double *tflops, double *clock_ghz);

#define AFD_NUM_STAGES 5
afd_status afd_ffn_set_timing(afd_ffn_t *handle, int32_t enable);
afd_status afd_ffn_set_timing_stages(afd_ffn_t *handle, uint32_t stage_mask);
afd_status afd_ffn_get_timing(afd_ffn_t *handle, float *ms, int32_t *num_forwards);

#ifdef __cplusplus
}
#endif

#endif /* AFD_FFN_H */
