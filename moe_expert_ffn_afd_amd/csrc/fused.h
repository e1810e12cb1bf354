#pragma once
// fused.h -- the parts of the one-launch FFN-side layer that do not depend on
// the weight format (fused.hip: block-FP8 and W8A8; fused_bf16.hip: bf16):
// the grid barrier, the dispatch phases and the combine phase.
//
// FastAFD's expert GPUs run the MoE layer as one persistent kernel (structured
// summary, System Design item 3: the token pull, the block-FP8 grouped GEMMs,
// the activation and the push-back in one launch; its ablation credits that
// fusion with about half the step latency of separate communication and GEMM
// kernels).  On one GPU there is no transfer to fold in; what one launch saves
// here is the launch gaps and the per-kernel heads and tails between the
// stages, and the dispatch runs on every workgroup instead of one.
//
// One workgroup of 8 waves per CU (the GEMM bodies' LDS allows one), all of
// them resident at once, so phases can be separated by grid barriers:
//   D1  every workgroup counts its chunk of the flat slots per expert;
//   D2  per expert, the exclusive scan of the chunk counts (experts spread
//       over the workgroups) and the expert's total;
//   D3  every workgroup scans the totals into the offsets and places its
//       chunk's slots at their stable rows (ballot ranks, as in dispatch.hip);
//       workgroup 0 also writes the counts, offsets and both m-tile lists
//       (and, bf16, the light / mixed choice and the split of the mixed
//       GEMM's workgroups);
//   then the format's own phases (activation scales, the two GEMM stages,
//   the W8A8 re-quantisation), and
//   C   the combine, two tokens at a time per workgroup (combine.h).
// The results equal the separate launches' bit for bit: the same per-element
// arithmetic in the same order, only scheduled differently.
//
// Grid barrier: after a workgroup barrier, thread 0 adds one to an arrival
// counter with an agent-scope release, polls it with relaxed agent-scope loads
// until every workgroup of the phase has arrived, then issues one agent-scope
// acquire.  The release and the acquire carry the cache maintenance that makes
// one XCD's stores visible to another's loads (each XCD has its own L2).  A
// spin gives up after a bounded number of rounds, counts a timeout and goes
// on, so a missing workgroup can never hang the GPU (the results of such a
// call are wrong and the host can read the count).  The last workgroup to
// leave resets the counters for the next call.
#include "combine.h"

namespace afd {

namespace {

constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = kFusedWaves * 64;

// Exclusive scan of one value per thread of the 8-wave workgroup; *total is
// the sum.  tmp: 16 ints of LDS.  Every thread calls it.
__device__ inline int scan512(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kFusedWaves ? tmp[lane] : 0;
#pragma unroll
    for (int d = 1; d < kFusedWaves; d <<= 1) {
      const int y = __shfl_up(w, d, 64);
      if (lane >= d) w += y;
    }
    if (lane < kFusedWaves) tmp[kFusedWaves + lane] = w;  // inclusive wave sums
  }
  __syncthreads();
  const int base = wave > 0 ? tmp[kFusedWaves + wave - 1] : 0;
  *total = tmp[2 * kFusedWaves - 1];
  const int r = base + x - v;
  __syncthreads();  // tmp may be reused by the caller
  return r;
}

// Every workgroup of the grid reaches this point before any goes on (see the
// file comment).  bar[0]: arrivals, bar[2]: spins that gave up.
__device__ inline void grid_sync(int32_t* bar, int& target, const int G, const int spin_limit) {
  target += G;
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(bar, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    // relaxed polls, one acquire after them: an acquire invalidates the XCD's
    // L2, and polling with it would keep invalidating the lines the
    // workgroups still in the phase are reading
    int n = 0;
    while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (++n > spin_limit) {
        __hip_atomic_fetch_add(bar + 2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

}  // namespace

// D1 .. D3 as workgroup b of G; lds: at least (9 kMaxExperts + 17) ints of the
// kernel's LDS; target: the grid barriers passed so far times G.
__device__ __forceinline__ void fused_dispatch(const FusedParams& f, const int b, const int G, int* const lds,
                                               int& target) {
  const DispatchParams& d = f.d;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int E = d.num_experts, n = d.n_flat;
  // this workgroup's chunk of the flat slots
  const int L = (n + G - 1) / G;
  const int f0 = min(b * L, n), f1 = min(f0 + L, n);

  // ---- D1: per-expert counts of the chunk
  {
    int* cnt = lds;                    // [E]
    int* bad = lds + kMaxExperts;      // [1]
    for (int e = tid; e < E; e += kFusedThreads) cnt[e] = 0;
    if (tid == 0) *bad = 0;
    __syncthreads();
    for (int i = f0 + tid; i < f1; i += kFusedThreads) {
      const int e = d.ids[i];
      if (e >= 0 && e < E)
        atomicAdd(&cnt[e], 1);
      else if (e != -1)
        atomicAdd(bad, 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kFusedThreads) f.chunk_counts[(int64_t)b * E + e] = cnt[e];
    if (tid == 0) f.chunk_bad[b] = *bad;
  }
  grid_sync(f.bar, target, G, f.spin_limit);

  // ---- D2: per expert, the chunks' exclusive prefix and the total
  {
    int* tmp = lds;  // [16]
    for (int e = b; e < E; e += G) {
      const int v = tid < G ? f.chunk_counts[(int64_t)tid * E + e] : 0;
      int tot = 0;
      const int ex = scan512(v, tmp, &tot);
      if (tid < G) f.local_base[(int64_t)tid * E + e] = ex;
      if (tid == 0) f.totals[e] = tot;
    }
    if (b == 0) {
      int tot = 0;
      scan512(tid < G ? f.chunk_bad[tid] : 0, tmp, &tot);
      if (tid == 0) d.err[0] = tot;
    }
  }
  grid_sync(f.bar, target, G, f.spin_limit);

  // ---- D3: offsets, tile lists (workgroup 0), stable placement of the chunk
  {
    int* cursor = lds;                      // [E]
    int* wcnt = lds + kMaxExperts;          // [8][E]
    int* tmp = lds + 9 * kMaxExperts;       // [16]
    const int cnt_e = tid < E ? f.totals[tid] : 0;
    int N = 0;
    const int off_e = scan512(cnt_e, tmp, &N);
    if (tid < E) cursor[tid] = off_e + f.local_base[(int64_t)b * E + tid];
    if (b == 0) {
      if (tid < E) {
        d.counts[tid] = cnt_e;
        d.offsets[tid] = off_e;
      }
      if (tid == 0) {
        d.offsets[E] = N;
        if (d.pool) d.pool[0] = d.pool[1] = 0;
      }
      // m-tile lists, as the dispatch kernel builds them: experts with at
      // least heavy_min rows in heavy tiles of bm_heavy rows, the others in
      // light tiles of bm_light, block-FP8 experts of at least tiled_min_rows
      // rows in tiled tiles of bm_tiled; routed experts in expert order, then
      // the shared expert.  With auto_heavy_rows (bf16), a batch whose largest
      // expert stays below it keeps every expert light, in tiles of
      // bm_light_only rows.
      int* mx = tmp + 16;
      if (tid == 0) *mx = 0;
      __syncthreads();
      if (tid < E) atomicMax(mx, cnt_e);
      __syncthreads();
      const bool mixed = d.auto_heavy_rows <= 0 || *mx >= d.auto_heavy_rows;
      const int heavy_min = mixed ? d.heavy_min_rows : 0x7fffffff;
      const int bm_light = mixed ? d.bm_light : d.bm_light_only;
      const bool has_tiled = d.tiled_min_rows < 0x7fffffff;  // uniform
      const bool tiled = has_tiled && cnt_e >= d.tiled_min_rows;
      const bool heavy = !tiled && cnt_e >= heavy_min;
      const int vl = (heavy || tiled) ? 0 : (cnt_e + bm_light - 1) / bm_light;
      const int vh = heavy ? (cnt_e + d.bm_heavy - 1) / d.bm_heavy : 0;
      const int vt = tiled ? (cnt_e + d.bm_tiled - 1) / d.bm_tiled : 0;
      int n_light = 0, n_heavy = 0, n_tiled = 0;
      const int offl = scan512(vl, tmp, &n_light);
      const int offh = scan512(vh, tmp, &n_heavy);
      const int offt = has_tiled ? scan512(vt, tmp, &n_tiled) : 0;
      if (tid < E) {
        for (int j = 0; j < vt; ++j)
          d.mtiles_tiled[offt + j] =
              make_int4(tid, off_e + j * d.bm_tiled, min(d.bm_tiled, cnt_e - j * d.bm_tiled), 0);
        for (int j = 0; j < vl; ++j)
          d.mtiles[offl + j] = make_int4(tid, off_e + j * bm_light, min(bm_light, cnt_e - j * bm_light), 0);
        for (int j = 0; j < vh; ++j)
          d.mtiles_heavy[offh + j] =
              make_int4(tid, off_e + j * d.bm_heavy, min(d.bm_heavy, cnt_e - j * d.bm_heavy), 0);
      }
      const bool sh_tiled = has_tiled && d.shared_rows >= d.tiled_min_rows;
      const bool sh_heavy = !sh_tiled && d.shared_rows >= heavy_min;
      const int bms = sh_tiled ? d.bm_tiled : sh_heavy ? d.bm_heavy : bm_light;
      const int per_part = (d.shared_rows + bms - 1) / bms;
      const int n_shared = per_part * d.shared_parts;
      int4* list = sh_tiled ? d.mtiles_tiled : sh_heavy ? d.mtiles_heavy : d.mtiles;
      const int base = sh_tiled ? n_tiled : sh_heavy ? n_heavy : n_light;
      for (int j = tid; j < n_shared; j += kFusedThreads) {
        const int v = j / per_part, r0 = (j - v * per_part) * bms;
        list[base + j] = make_int4(E + v, d.shared_row0 + v * d.shared_rows + r0, min(bms, d.shared_rows - r0), 0);
      }
      if (tid == 0) {
        const int nl = n_light + (sh_heavy || sh_tiled ? 0 : n_shared), nh = n_heavy + (sh_heavy ? n_shared : 0);
        d.num_mtiles[0] = nl;
        d.num_mtiles[1] = nh;
        // bf16: the grid's workgroups that stream the light list beside the
        // heavy tiles (the ring GEMMs take no split)
        d.num_mtiles[2] = dev::mixed_light_workgroups(d.mix_cus > 0 ? G : 0, nl, nh);
        d.num_mtiles[3] = mixed ? kLaunchMixed : kLaunchLight;
        d.num_mtiles[4] = n_tiled + (sh_tiled ? n_shared : 0);
      }
    }
    for (int i = tid; i < kFusedWaves * E; i += kFusedThreads) wcnt[i] = 0;
    __syncthreads();
    // rounds of 512 slots in flat order: each wave ranks its slots among equal
    // ids with ballots over the id bits, waves are ordered through per-wave
    // counts, and the per-expert cursors advance round by round
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int base = f0; base < f1; base += kFusedThreads) {
      const int fi = base + tid;
      const int e = fi < f1 ? d.ids[fi] : -1;
      const bool valid = e >= 0 && e < E;
      uint64_t match = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool on = valid && ((e >> bit) & 1);
        const uint64_t m = __ballot(on);
        match &= on ? m : ~m;
      }
      const int rank = __popcll(match & lt_mask);
      if (valid && rank == 0) wcnt[wave * E + e] = __popcll(match);
      __syncthreads();
      if (valid) {
        int prefix = 0;
        for (int w = 0; w < wave; ++w) prefix += wcnt[w * E + e];
        const int pos = cursor[e] + prefix + rank;
        d.sorted_assign[pos] = fi;
        d.row_of[fi] = pos;
      } else if (fi < f1) {
        d.row_of[fi] = -1;
      }
      __syncthreads();
      for (int x = tid; x < E; x += kFusedThreads) {
        int s = 0;
        for (int w = 0; w < kFusedWaves; ++w) s += wcnt[w * E + x];
        cursor[x] += s;
      }
      __syncthreads();
      if (valid && rank == 0) wcnt[wave * E + e] = 0;
      __syncthreads();
    }
  }
  grid_sync(f.bar, target, G, f.spin_limit);
}

// C, then the barrier counters reset by the last workgroup out
__device__ __forceinline__ void fused_combine(const FusedParams& f, const int b, const int G) {
  const int tid = threadIdx.x;
  // ---- C: combine, two tokens at a time per workgroup (4 waves each)
  {
    __shared__ int c_rows[2][kMaxRowsPerToken];
    __shared__ float c_ws[2][kMaxRowsPerToken];
    __shared__ int c_n[2];
    const int grp = tid >> 8;
    for (int t0 = 2 * b; t0 < f.tokens; t0 += 2 * G)
      combine_rows<kBF16>(f.cp, t0 + grp, t0 + grp < f.tokens, tid & 255, 256, c_rows[grp], c_ws[grp], &c_n[grp]);
  }

  // the last workgroup out resets the barrier counters for the next call
  __syncthreads();
  if (tid == 0) {
    const int left = __hip_atomic_fetch_add(f.bar + 1, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (left == G - 1) {
      __hip_atomic_store(f.bar, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(f.bar + 1, 0, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace afd
