// dispatch.hip -- expert dispatch of the routed (token, slot) assignments.
//
// The FFN side receives tokens with their top-k expert ids and must group the
// assignments by expert for the grouped GEMMs ("FastAFD" structured summary,
// legend of Eq. (3): the FFN stage covers dispatch of the routed tokens and
// the grouped GEMM over them).  The grouping is the stable counting sort of
// the flat slots f = t*K + k by expert id:
//   counts[e]            = #{f : ids[f] == e}
//   offsets[e]           = sum_{e' < e} counts[e'],  offsets[E] = N
//   sorted_assign[r]     = the flat slots of expert 0, then expert 1, ...,
//                          each expert's in ascending f
//   row_of[f]            = r with sorted_assign[r] == f, or -1
// Being a pure function of the ids, it is reproduced bit for bit.
//
// Two kernels (one for batches of at most kDispatchFuseSlots slots, where
// count_scan also does the placement).  count_scan (one workgroup):
// per-(chunk, expert) counts with LDS atomics (counts do not depend on order),
// per-expert prefix over chunks, exclusive scan over experts, first sorted row
// of every (chunk, expert), the GEMM m-tile lists and, for a mixed bf16
// launch, how many of its workgroups take the light list.  scatter (one
// workgroup per chunk): each wave ranks its
// 64 slots among equal ids with ballots over the id bits (match mask, popcount
// of the lower lanes), waves are ordered through per-wave counts in LDS, and
// rounds of 1024 slots advance per-expert cursors, so every slot lands at its
// stable position with no order-dependent atomics.
#include <algorithm>

#include "afd_device.h"

namespace afd {

namespace {

__device__ inline int block_exclusive_scan_1024(int v, int* lds_waves, int* total) {
  // 1024 threads = 16 waves of 64.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds_waves[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? lds_waves[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      int y = __shfl_up(w, d, 64);
      if (lane >= d) w += y;
    }
    if (lane < 16) lds_waves[16 + lane] = w;  // inclusive wave sums
  }
  __syncthreads();
  int base = wave > 0 ? lds_waves[16 + wave - 1] : 0;
  *total = lds_waves[16 + 15];
  int r = base + x - v;
  __syncthreads();  // lds_waves may be reused by the caller
  return r;
}

}  // namespace

// Stable placement of the flat slots [f0, f_end) in rounds of 1024: cursor[e]
// holds the next sorted row of expert e and advances round by round; wcnt is
// [16][E] LDS, zero on entry and on return; ids[f] the id of slot f (the
// caller's array, or a copy in LDS).  Every thread of the 1024-thread
// workgroup calls it.
__device__ void scatter_rounds(const DispatchParams& p, const int* ids, int f0, int f_end, int* cursor, int* wcnt) {
  const int E = p.num_experts;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = f0; base < f_end; base += kDispatchThreads) {
    const int f = base + tid;
    const int e = f < f_end ? ids[f] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      match &= bit ? m : ~m;
    }
    const int rank = __popcll(match & lt_mask);
    if (valid && rank == 0) wcnt[wave * E + e] = __popcll(match);
    __syncthreads();
    if (valid) {
      int prefix = 0;
      for (int w = 0; w < wave; ++w) prefix += wcnt[w * E + e];
      const int pos = cursor[e] + prefix + rank;
      p.sorted_assign[pos] = f;
      p.row_of[f] = pos;
    } else if (f < f_end) {
      p.row_of[f] = -1;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kDispatchThreads) {
      int s = 0;
      for (int w = 0; w < 16; ++w) s += wcnt[w * E + x];
      cursor[x] += s;
    }
    __syncthreads();
    if (valid && rank == 0) wcnt[wave * E + e] = 0;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kDispatchThreads) void dispatch_count_scan_kernel(DispatchParams p) {
  extern __shared__ int cc[];  // [n_chunks][E] counts, then chunk-local prefixes
  __shared__ int total[kMaxExperts];
  __shared__ int excl[kMaxExperts];
  __shared__ int scan_tmp[32];
  __shared__ int bad;
  __shared__ int max_rows;
  const int E = p.num_experts;
  const int tid = threadIdx.x;
  const int ncc = p.n_chunks * E;
  // small batches keep their ids in LDS for the placement: [n_flat] after wcnt
  int* ids_lds = cc + ncc + 16 * E;

  for (int i = tid; i < ncc; i += kDispatchThreads) cc[i] = 0;
  if (tid == 0) {
    bad = 0;
    max_rows = 0;
  }
  __syncthreads();

  // 8 id loads in flight per thread, then their LDS increments
  constexpr int kU = 8;
  for (int f0 = 0; f0 < p.n_flat; f0 += kU * kDispatchThreads) {
    int ev[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int f = f0 + u * kDispatchThreads + tid;
      ev[u] = f < p.n_flat ? p.ids[f] : -1;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int f = f0 + u * kDispatchThreads + tid;
      const int e = ev[u];
      if (p.fused && f < p.n_flat) ids_lds[f] = e;
      if (e >= 0 && e < E)
        atomicAdd(&cc[(f >> p.chunk_shift) * E + e], 1);
      else if (e != -1)
        atomicAdd(&bad, 1);
    }
  }
  __syncthreads();

  // per expert: chunk-local exclusive prefix over chunks, total count
  for (int e = tid; e < E; e += kDispatchThreads) {
    int run = 0;
    for (int c = 0; c < p.n_chunks; ++c) {
      int v = cc[c * E + e];
      cc[c * E + e] = run;
      run += v;
    }
    total[e] = run;
    atomicMax(&max_rows, run);
  }
  __syncthreads();

  // exclusive scan over experts (E <= 1024: one expert per thread)
  int n_routed = 0;
  {
    int v = tid < E ? total[tid] : 0;
    int x = block_exclusive_scan_1024(v, scan_tmp, &n_routed);
    if (tid < E) {
      excl[tid] = x;
      p.counts[tid] = v;
      p.offsets[tid] = x;
    }
    if (tid == 0) {
      p.offsets[E] = n_routed;
      p.err[0] = bad;
      if (p.pool) p.pool[0] = p.pool[1] = 0;
    }
  }
  __syncthreads();

  if (!p.fused)
    for (int i = tid; i < ncc; i += kDispatchThreads) p.chunk_base[i] = excl[i % E] + cc[i];

  // m-tile lists: experts with at least heavy_min_rows rows go to the heavy
  // list (tiles of bm_heavy rows), the others to the light list (bm_light);
  // block-FP8 experts with at least tiled_min_rows rows to the tiled list
  // (bm_tiled); routed experts in expert order, then the shared expert.  With
  // auto_heavy_rows, a batch whose largest expert stays below it keeps every
  // expert light, in tiles of bm_light_only rows (one launch of the streaming
  // GEMM); a larger one takes the mixed launch.
  {
    const bool mixed = p.auto_heavy_rows <= 0 || max_rows >= p.auto_heavy_rows;
    const int heavy_min = mixed ? p.heavy_min_rows : 0x7fffffff;
    const int bm_light = mixed ? p.bm_light : p.bm_light_only;
    const int n = tid < E ? total[tid] : 0;
    const bool has_tiled = p.tiled_min_rows < 0x7fffffff;  // uniform
    const bool tiled = has_tiled && n >= p.tiled_min_rows;
    const bool heavy = !tiled && n >= heavy_min;
    const int vl = (heavy || tiled) ? 0 : (n + bm_light - 1) / bm_light;
    const int vh = heavy ? (n + p.bm_heavy - 1) / p.bm_heavy : 0;
    const int vt = tiled ? (n + p.bm_tiled - 1) / p.bm_tiled : 0;
    int n_light = 0, n_heavy = 0, n_tiled = 0;
    const int offl = block_exclusive_scan_1024(vl, scan_tmp, &n_light);
    const int offh = block_exclusive_scan_1024(vh, scan_tmp, &n_heavy);
    const int offt = has_tiled ? block_exclusive_scan_1024(vt, scan_tmp, &n_tiled) : 0;
    if (tid < E) {
      for (int j = 0; j < vt; ++j) {
        const int r0 = j * p.bm_tiled;
        p.mtiles_tiled[offt + j] = make_int4(tid, excl[tid] + r0, min(p.bm_tiled, n - r0), 0);
      }
      for (int j = 0; j < vl; ++j) {
        const int r0 = j * bm_light;
        p.mtiles[offl + j] = make_int4(tid, excl[tid] + r0, min(bm_light, n - r0), 0);
      }
      for (int j = 0; j < vh; ++j) {
        const int r0 = j * p.bm_heavy;
        p.mtiles_heavy[offh + j] = make_int4(tid, excl[tid] + r0, min(p.bm_heavy, n - r0), 0);
      }
    }
    const bool sh_tiled = has_tiled && p.shared_rows >= p.tiled_min_rows;
    const bool sh_heavy = !sh_tiled && p.shared_rows >= heavy_min;
    const int bms = sh_tiled ? p.bm_tiled : sh_heavy ? p.bm_heavy : bm_light;
    const int per_part = (p.shared_rows + bms - 1) / bms;
    const int n_shared = per_part * p.shared_parts;
    int4* list = sh_tiled ? p.mtiles_tiled : sh_heavy ? p.mtiles_heavy : p.mtiles;
    const int base = sh_tiled ? n_tiled : sh_heavy ? n_heavy : n_light;
    for (int j = tid; j < n_shared; j += kDispatchThreads) {
      const int v = j / per_part, r0 = (j - v * per_part) * bms;
      list[base + j] = make_int4(E + v, p.shared_row0 + v * p.shared_rows + r0, min(bms, p.shared_rows - r0), 0);
    }
    if (tid == 0) {
      const int nl = n_light + (sh_heavy || sh_tiled ? 0 : n_shared), nh = n_heavy + (sh_heavy ? n_shared : 0);
      p.num_mtiles[0] = nl;
      p.num_mtiles[1] = nh;
      p.num_mtiles[2] = dev::mixed_light_workgroups(p.mix_cus, nl, nh);
      p.num_mtiles[3] = mixed ? kLaunchMixed : kLaunchLight;
      p.num_mtiles[4] = n_tiled + (sh_tiled ? n_shared : 0);
    }
  }

  // small batches: the placement too, all slots in order in this workgroup
  // (cursors start at the experts' first rows), instead of a second launch
  if (p.fused) {
    int* wcnt = cc + ncc;  // [16][E]
    for (int i = tid; i < 16 * E; i += kDispatchThreads) wcnt[i] = 0;
    __syncthreads();  // every read of total[] above is done: it becomes the cursors
    for (int e = tid; e < E; e += kDispatchThreads) total[e] = excl[e];
    __syncthreads();
    scatter_rounds(p, ids_lds, 0, p.n_flat, total, wcnt);
  }
}

__global__ __launch_bounds__(kDispatchThreads) void dispatch_scatter_kernel(DispatchParams p) {
  extern __shared__ int lds[];
  const int E = p.num_experts;
  int* cursor = lds;          // [E]
  int* wcnt = lds + E;        // [16][E] per-wave counts of the current round
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x;
  const int chunk_len = 1 << p.chunk_shift;
  const int f0 = chunk * chunk_len;
  const int f_end = min(f0 + chunk_len, p.n_flat);
  for (int e = tid; e < E; e += kDispatchThreads) cursor[e] = p.chunk_base[chunk * E + e];
  for (int i = tid; i < 16 * E; i += kDispatchThreads) wcnt[i] = 0;
  __syncthreads();
  scatter_rounds(p, p.ids, f0, f_end, cursor, wcnt);
}

// Block-FP8 only: the caller's 1x128 activation scales [T][H/128], gathered
// into the sorted rows of the gate/up GEMM and stored step-major
// (dst[c][row]), so that one GEMM step reads a tile's scales as one contiguous
// run.  One thread per (row, step c = blockIdx.y): coalesced stores, reads
// from the small, cache-resident source.  blockIdx.z = 0: routed rows (token
// of row r = sorted_assign[r] / K); 1 + v: part v of the shared expert's rows
// (token order).
__global__ __launch_bounds__(256) void gather_scales_kernel(ScaleGatherParams p) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  int row, token;
  if (blockIdx.z == 0) {
    if (i >= p.offsets[p.num_experts]) return;
    row = i;
    token = p.sorted_assign[i] / p.top_k;
  } else {
    if (i >= p.tokens) return;
    row = p.shared_row0 + (int)(blockIdx.z - 1) * p.tokens + i;
    token = i;
  }
  p.dst[(int64_t)c * p.ld + row] = p.src[(int64_t)token * p.ks + c];
}

hipError_t launch_gather_scales(const ScaleGatherParams& p, hipStream_t s) {
  const int n = std::max(p.routed_max, p.shared_row0 >= 0 ? p.tokens : 0);
  if (n <= 0 || p.ks <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_scales_kernel, dim3((n + 255) / 256, p.ks, p.shared_row0 >= 0 ? 1 + p.shared_parts : 1),
                     dim3(256), 0, s,
                     p);
  return hipGetLastError();
}

hipError_t launch_dispatch_count_scan(const DispatchParams& p, hipStream_t s) {
  // counters; with the placement fused: per-wave counts and the ids too
  // (at most 4 * 512 + 16 * 512 + 4096 ints = 56 KiB)
  size_t lds = sizeof(int) * ((size_t)p.n_chunks * p.num_experts + (p.fused ? 16 * (size_t)p.num_experts + p.n_flat : 0));
  hipLaunchKernelGGL(dispatch_count_scan_kernel, dim3(1), dim3(kDispatchThreads), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_dispatch_scatter(const DispatchParams& p, hipStream_t s) {
  if (p.n_chunks == 0 || p.fused) return hipSuccess;
  size_t lds = sizeof(int) * (size_t)17 * p.num_experts;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(p.n_chunks), dim3(kDispatchThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace afd
