// api.hip -- host side of the C ABI declared in include/afd_ffn.h.
//
// create: validate on the host, allocate library-owned packed weights and a
// workspace, pack.  forward: validate on the host, then enqueue on the
// caller's stream, with no host synchronisation and no device-to-host copy:
//   dispatch count+scan -> dispatch scatter -> grouped GEMM gate/up + SwiGLU
//   -> grouped GEMM down -> weighted combine.
// All sizes that depend on the routing (expert counts, m-tile list) live on
// the device; the GEMMs are persistent grids that read the tile count there.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <string>
#include <vector>

#include "../../include/afd_ffn.h"
#include "afd_internal.h"

using namespace afd;

namespace {

thread_local std::string g_last_error;

afd_status fail(afd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

#define AFD_HIP(expr)                                                                       \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess) return fail(AFD_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

struct WeightStore {
  std::atomic<int> refs{1};
  int device = 0;
  // bf16 / fp8: packed gate+up and down; f32: plain gate, up, down
  uint8_t* gu = nullptr;
  uint8_t* up = nullptr;  // f32 only
  uint8_t* dn = nullptr;
  float* sg = nullptr;
  float* su = nullptr;
  float* sd = nullptr;
  int64_t gu_expert_bytes = 0, dn_expert_bytes = 0;
  int64_t gu_panel_bytes = 0, dn_panel_bytes = 0;
  int64_t scale_bytes = 0;  // fp8: bytes of each of sg, su, sd
  ~WeightStore() {
    for (void* p : {(void*)gu, (void*)up, (void*)dn, (void*)sg, (void*)su, (void*)sd})
      if (p) (void)hipFree(p);
  }
};

int esize_of(int dtype) { return dtype == kF32 ? 4 : dtype == kBF16 ? 2 : 1; }

}  // namespace

struct afd_ffn {
  int H = 0, I = 0, E = 0, K = 0, Tmax = 0, S = 0, dtype = 0, device = 0;
  int num_cus = 256;
  int concurrency = 1;  // forwards the caller runs at once on other streams (afd_ffn_set_concurrency)
  WeightStore* w = nullptr;
  // workspace
  uint8_t* ws = nullptr;
  int32_t *counts = nullptr, *offsets = nullptr, *err = nullptr, *num_mtiles = nullptr;
  int32_t *chunk_base = nullptr, *sorted_assign = nullptr, *row_of = nullptr;
  int4* mtiles = nullptr;
  int4* mtiles_heavy = nullptr;
  uint8_t* h = nullptr;
  float* h_scales = nullptr;   // FP8: [I/128][h_rows] step-major
  float* x_scales = nullptr;   // FP8: [H/128][h_rows] hidden scales in sorted-row order
  int64_t h_rows = 0;
  uint8_t* y = nullptr;
  int max_chunks = 0, max_mtiles = 0;
  int last_T = 0;
  // per-stage timing: bit s of the mask times stage s (boundaries s and s + 1)
  uint32_t timing_mask = 0;
  std::vector<hipEvent_t> ev_free;
  std::vector<std::array<hipEvent_t, AFD_NUM_STAGES + 1>> ev_pending;  // per forward, per boundary (or null)
};

namespace {

int chunk_shift_for(int64_t n_flat, int E) {
  int shift = 10;
  while (((n_flat + (1ll << shift) - 1) >> shift) * E > kDispatchLdsInts) ++shift;
  return shift;
}

afd_status check_config(const afd_ffn_config* c) {
  if (!c) return fail(AFD_ERR_INVALID_ARG, "config is NULL");
  if (c->dtype < 0 || c->dtype > 2) return fail(AFD_ERR_UNSUPPORTED, "unknown dtype %d", c->dtype);
  if (c->hidden <= 0 || c->inter <= 0 || c->num_experts <= 0 || c->top_k <= 0 || c->max_tokens <= 0)
    return fail(AFD_ERR_INVALID_ARG, "hidden, inter, num_experts, top_k and max_tokens must be positive");
  if (c->hidden % 128 || c->inter % 128)
    return fail(AFD_ERR_UNSUPPORTED, "hidden (%d) and inter (%d) must be multiples of 128", c->hidden, c->inter);
  if (c->dtype == kFP8 && (c->hidden > 16384 || c->inter > 16384))
    return fail(AFD_ERR_UNSUPPORTED, "block-FP8 reductions are limited to 128 blocks (hidden, inter <= 16384)");
  if (c->num_experts > kMaxExperts) return fail(AFD_ERR_UNSUPPORTED, "num_experts %d > %d", c->num_experts, kMaxExperts);
  if (c->top_k > kMaxTopK) return fail(AFD_ERR_UNSUPPORTED, "top_k %d > %d", c->top_k, kMaxTopK);
  if ((int64_t)c->max_tokens * c->top_k >= (1ll << 26))
    return fail(AFD_ERR_UNSUPPORTED, "max_tokens * top_k must stay below 2^26");
  if (c->shared_inter < 0 || (c->shared_inter > 0 && c->shared_inter != c->inter))
    return fail(AFD_ERR_UNSUPPORTED, "shared_inter must be 0 or equal to inter");
  {
    // the GEMMs and the combine address rows (hidden, h, y) with 32-bit buffer offsets
    const int64_t es = c->dtype == kF32 ? 4 : c->dtype == kBF16 ? 2 : 1;
    const int64_t rows = (int64_t)c->max_tokens * c->top_k + (c->shared_inter > 0 ? c->max_tokens : 0);
    const int64_t lim = (1ll << 31) - (1ll << 24);
    const int64_t ys = c->dtype == kF32 ? 4 : 2;  // expert outputs y are bf16 | fp32
    if (rows * std::max(c->hidden, c->inter) * es > lim || (int64_t)c->max_tokens * c->hidden * es > lim ||
        rows * c->hidden * ys > lim)
      return fail(AFD_ERR_UNSUPPORTED, "activation buffers of max_tokens=%d exceed 2 GiB", c->max_tokens);
  }
  if (c->device < 0) return fail(AFD_ERR_INVALID_ARG, "device must be >= 0");
  if (!c->w_gate || !c->w_up || !c->w_down) return fail(AFD_ERR_INVALID_ARG, "weight pointer is NULL");
  const bool fp8 = c->dtype == kFP8;
  if (fp8 && (!c->s_gate || !c->s_up || !c->s_down))
    return fail(AFD_ERR_INVALID_ARG, "block-FP8 weights need s_gate, s_up and s_down");
  if (!fp8 && (c->s_gate || c->s_up || c->s_down))
    return fail(AFD_ERR_INVALID_ARG, "weight scales are only used with AFD_DTYPE_FP8_BLOCK");
  auto mis = [](const void* q, uintptr_t a) { return q && (reinterpret_cast<uintptr_t>(q) & (a - 1)); };
  {
    // bf16 / e4m3 weights are packed with 16-byte vector loads; fp32 ones are copied
    const uintptr_t wa = c->dtype == kF32 ? 4 : 16;
    if (mis(c->w_gate, wa) || mis(c->w_up, wa) || mis(c->w_down, wa) || mis(c->sh_gate, wa) ||
        mis(c->sh_up, wa) || mis(c->sh_down, wa))
      return fail(AFD_ERR_INVALID_ARG, "weights must be %d-byte aligned", (int)wa);
  }
  if (mis(c->s_gate, 4) || mis(c->s_up, 4) || mis(c->s_down, 4) || mis(c->sh_s_gate, 4) || mis(c->sh_s_up, 4) ||
      mis(c->sh_s_down, 4))
    return fail(AFD_ERR_INVALID_ARG, "weight scales must be 4-byte aligned");
  if (c->shared_inter > 0) {
    if (!c->sh_gate || !c->sh_up || !c->sh_down) return fail(AFD_ERR_INVALID_ARG, "shared expert weight is NULL");
    if (fp8 && (!c->sh_s_gate || !c->sh_s_up || !c->sh_s_down))
      return fail(AFD_ERR_INVALID_ARG, "shared expert scales are NULL");
  }
  return AFD_OK;
}

afd_status alloc_workspace(afd_ffn* a) {
  const int64_t nmax = (int64_t)a->Tmax * a->K;
  const int64_t rows = nmax + (a->S ? a->Tmax : 0);
  a->max_chunks = (int)((nmax + 1023) / 1024);
  a->max_mtiles = (int)(nmax / 32 + a->E + (a->S ? (a->Tmax + 31) / 32 : 0) + 1);
  const int es = esize_of(a->dtype);
  const int ys = a->dtype == kF32 ? 4 : 2;
  int64_t off = 0;
  auto take = [&](int64_t bytes) { int64_t o = off; off = align_up(off + bytes, 256); return o; };
  const int64_t o_counts = take(4ll * a->E), o_offsets = take(4ll * (a->E + 1)), o_err = take(4),
                o_nmt = take(16), o_cb = take(4ll * a->max_chunks * a->E), o_sa = take(4 * nmax),
                o_ro = take(4 * nmax), o_mt = take(16ll * a->max_mtiles), o_mth = take(16ll * a->max_mtiles),
                o_h = take(rows * a->I * es),
                o_hs = take(a->dtype == kFP8 ? rows * (a->I / 128) * 4 : 0),
                o_xs = take(a->dtype == kFP8 ? rows * (a->H / 128) * 4 : 0), o_y = take(rows * a->H * ys);
  if (hipMalloc((void**)&a->ws, off) != hipSuccess) {
    (void)hipGetLastError();
    a->ws = nullptr;
    return fail(AFD_ERR_OUT_OF_MEMORY, "workspace of %lld bytes", (long long)off);
  }
  a->counts = (int32_t*)(a->ws + o_counts);
  a->offsets = (int32_t*)(a->ws + o_offsets);
  a->err = (int32_t*)(a->ws + o_err);
  a->num_mtiles = (int32_t*)(a->ws + o_nmt);
  a->chunk_base = (int32_t*)(a->ws + o_cb);
  a->sorted_assign = (int32_t*)(a->ws + o_sa);
  a->row_of = (int32_t*)(a->ws + o_ro);
  a->mtiles = (int4*)(a->ws + o_mt);
  a->mtiles_heavy = (int4*)(a->ws + o_mth);
  a->h = a->ws + o_h;
  a->h_scales = a->dtype == kFP8 ? (float*)(a->ws + o_hs) : nullptr;
  a->x_scales = a->dtype == kFP8 ? (float*)(a->ws + o_xs) : nullptr;
  a->h_rows = rows;
  a->y = a->ws + o_y;
  AFD_HIP(hipMemset(a->ws, 0, off));
  return AFD_OK;
}

afd_status pack_weights(const afd_ffn_config* c, afd_ffn* a) {
  WeightStore* w = a->w;
  const int E = a->E, ES = a->E + a->S, H = a->H, I = a->I, dt = a->dtype;
  const int es = esize_of(dt);
  auto mal = [&](uint8_t** p, int64_t bytes) -> afd_status {
    if (hipMalloc((void**)p, bytes) != hipSuccess) {
      (void)hipGetLastError();
      *p = nullptr;
      return fail(AFD_ERR_OUT_OF_MEMORY, "weight buffer of %lld bytes", (long long)bytes);
    }
    return AFD_OK;
  };
  afd_status st;
  AFD_HIP(hipDeviceSynchronize());  // the caller's weight writes are complete
  if (dt == kF32) {
    const int64_t mat = (int64_t)H * I * 4;
    if ((st = mal(&w->gu, mat * ES)) || (st = mal(&w->up, mat * ES)) || (st = mal(&w->dn, mat * ES))) return st;
    AFD_HIP(hipMemcpy(w->gu, c->w_gate, mat * E, hipMemcpyDeviceToDevice));
    AFD_HIP(hipMemcpy(w->up, c->w_up, mat * E, hipMemcpyDeviceToDevice));
    AFD_HIP(hipMemcpy(w->dn, c->w_down, mat * E, hipMemcpyDeviceToDevice));
    if (a->S) {
      AFD_HIP(hipMemcpy(w->gu + mat * E, c->sh_gate, mat, hipMemcpyDeviceToDevice));
      AFD_HIP(hipMemcpy(w->up + mat * E, c->sh_up, mat, hipMemcpyDeviceToDevice));
      AFD_HIP(hipMemcpy(w->dn + mat * E, c->sh_down, mat, hipMemcpyDeviceToDevice));
    }
    w->gu_expert_bytes = w->dn_expert_bytes = mat;
    return AFD_OK;
  }
  w->gu_panel_bytes = (int64_t)H * 32 * es;
  w->dn_panel_bytes = (int64_t)I * 32 * es;
  w->gu_expert_bytes = 2ll * H * I * es;
  w->dn_expert_bytes = (int64_t)I * H * es;
  if ((st = mal(&w->gu, w->gu_expert_bytes * ES)) || (st = mal(&w->dn, w->dn_expert_bytes * ES))) return st;
  AFD_HIP(launch_pack(dt, true, c->w_gate, c->w_up, (int64_t)H * I, E, H, I, w->gu, w->gu_expert_bytes, 0));
  AFD_HIP(launch_pack(dt, false, c->w_down, nullptr, (int64_t)I * H, E, I, H, w->dn, w->dn_expert_bytes, 0));
  if (a->S) {
    AFD_HIP(launch_pack(dt, true, c->sh_gate, c->sh_up, (int64_t)H * I, 1, H, I, w->gu + w->gu_expert_bytes * E,
                        w->gu_expert_bytes, 0));
    AFD_HIP(launch_pack(dt, false, c->sh_down, nullptr, (int64_t)I * H, 1, I, H, w->dn + w->dn_expert_bytes * E,
                        w->dn_expert_bytes, 0));
  }
  if (dt == kFP8) {
    const int64_t sblk = (int64_t)(H / 128) * (I / 128) * 4;
    if ((st = mal((uint8_t**)&w->sg, sblk * ES)) || (st = mal((uint8_t**)&w->su, sblk * ES)) ||
        (st = mal((uint8_t**)&w->sd, sblk * ES)))
      return st;
    w->scale_bytes = sblk * ES;
    AFD_HIP(hipMemcpy(w->sg, c->s_gate, sblk * E, hipMemcpyDeviceToDevice));
    AFD_HIP(hipMemcpy(w->su, c->s_up, sblk * E, hipMemcpyDeviceToDevice));
    AFD_HIP(hipMemcpy(w->sd, c->s_down, sblk * E, hipMemcpyDeviceToDevice));
    if (a->S) {
      AFD_HIP(hipMemcpy((uint8_t*)w->sg + sblk * E, c->sh_s_gate, sblk, hipMemcpyDeviceToDevice));
      AFD_HIP(hipMemcpy((uint8_t*)w->su + sblk * E, c->sh_s_up, sblk, hipMemcpyDeviceToDevice));
      AFD_HIP(hipMemcpy((uint8_t*)w->sd + sblk * E, c->sh_s_down, sblk, hipMemcpyDeviceToDevice));
    }
  }
  AFD_HIP(hipDeviceSynchronize());
  return AFD_OK;
}

void free_handle(afd_ffn* a) {
  if (!a) return;
  for (auto& v : a->ev_pending)
    for (hipEvent_t e : v)
      if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : a->ev_free) (void)hipEventDestroy(e);
  if (a->ws) (void)hipFree(a->ws);
  if (a->w && a->w->refs.fetch_sub(1) == 1) delete a->w;
  delete a;
}

hipEvent_t take_event(afd_ffn* a) {
  if (!a->ev_free.empty()) {
    hipEvent_t e = a->ev_free.back();
    a->ev_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

extern "C" {

const char* afd_ffn_status_string(afd_status s) {
  switch (s) {
    case AFD_OK: return "ok";
    case AFD_ERR_INVALID_ARG: return "invalid argument";
    case AFD_ERR_UNSUPPORTED: return "unsupported";
    case AFD_ERR_OUT_OF_MEMORY: return "out of device memory";
    case AFD_ERR_HIP: return "HIP runtime error";
    case AFD_ERR_BAD_ROUTING: return "expert ids outside [-1, E)";
  }
  return "unknown status";
}

const char* afd_ffn_last_error(void) { return g_last_error.c_str(); }

afd_status afd_ffn_validate_config(const afd_ffn_config* cfg) {
  g_last_error.clear();
  return check_config(cfg);
}

afd_status afd_ffn_create(const afd_ffn_config* cfg, afd_ffn_t** out_handle) {
  g_last_error.clear();
  if (!out_handle) return fail(AFD_ERR_INVALID_ARG, "out_handle is NULL");
  *out_handle = nullptr;
  afd_status st = check_config(cfg);
  if (st) return st;
  DeviceGuard dg(cfg->device);
  if (!dg.ok) return fail(AFD_ERR_HIP, "cannot select device %d", cfg->device);
  afd_ffn* a = new afd_ffn();
  a->H = cfg->hidden;
  a->I = cfg->inter;
  a->E = cfg->num_experts;
  a->K = cfg->top_k;
  a->Tmax = cfg->max_tokens;
  a->S = cfg->shared_inter > 0 ? 1 : 0;
  a->dtype = cfg->dtype;
  a->device = cfg->device;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, cfg->device) == hipSuccess && cus > 0)
    a->num_cus = cus;
  a->w = new WeightStore();
  a->w->device = cfg->device;
  if ((st = pack_weights(cfg, a)) != AFD_OK || (st = alloc_workspace(a)) != AFD_OK) {
    std::string msg = g_last_error;
    free_handle(a);
    g_last_error = msg;
    return st;
  }
  *out_handle = a;
  return AFD_OK;
}

afd_status afd_ffn_clone(const afd_ffn_t* src, afd_ffn_t** out_handle) {
  g_last_error.clear();
  if (!src || !out_handle) return fail(AFD_ERR_INVALID_ARG, "NULL handle");
  *out_handle = nullptr;
  DeviceGuard dg(src->device);
  if (!dg.ok) return fail(AFD_ERR_HIP, "cannot select device %d", src->device);
  afd_ffn* a = new afd_ffn();
  a->H = src->H;
  a->I = src->I;
  a->E = src->E;
  a->K = src->K;
  a->Tmax = src->Tmax;
  a->S = src->S;
  a->dtype = src->dtype;
  a->device = src->device;
  a->num_cus = src->num_cus;
  a->concurrency = src->concurrency;
  a->w = src->w;
  a->w->refs.fetch_add(1);
  afd_status st = alloc_workspace(a);
  if (st) {
    std::string msg = g_last_error;
    free_handle(a);
    g_last_error = msg;
    return st;
  }
  *out_handle = a;
  return AFD_OK;
}

afd_status afd_ffn_destroy(afd_ffn_t* h) {
  g_last_error.clear();
  if (!h) return AFD_OK;
  DeviceGuard dg(h->device);
  free_handle(h);
  return AFD_OK;
}

afd_status afd_ffn_forward(afd_ffn_t* a, int32_t T, const void* hidden, const float* hidden_scales,
                           const int32_t* topk_ids, const float* topk_weights, void* out, void* stream) {
  g_last_error.clear();
  if (!a) return fail(AFD_ERR_INVALID_ARG, "handle is NULL");
  if (T < 0 || T > a->Tmax) return fail(AFD_ERR_INVALID_ARG, "num_tokens %d outside [0, %d]", T, a->Tmax);
  if (T > 0 && (!hidden || !topk_ids || !topk_weights || !out))
    return fail(AFD_ERR_INVALID_ARG, "hidden, topk_ids, topk_weights and out must be non-NULL");
  if (a->dtype == kFP8 && T > 0 && !hidden_scales)
    return fail(AFD_ERR_INVALID_ARG, "block-FP8 input needs hidden_scales");
  if (a->dtype != kFP8 && hidden_scales)
    return fail(AFD_ERR_INVALID_ARG, "hidden_scales is only used with AFD_DTYPE_FP8_BLOCK");
  {
    auto mis = [](const void* q, uintptr_t al) { return q && (reinterpret_cast<uintptr_t>(q) & (al - 1)); };
    if (mis(hidden, 16) || mis(out, 16))
      return fail(AFD_ERR_INVALID_ARG, "hidden and out must be 16-byte aligned");
    if (mis(hidden_scales, 4) || mis(topk_ids, 4) || mis(topk_weights, 4))
      return fail(AFD_ERR_INVALID_ARG, "hidden_scales, topk_ids and topk_weights must be 4-byte aligned");
  }
  DeviceGuard dg(a->device);
  if (!dg.ok) return fail(AFD_ERR_HIP, "cannot select device %d", a->device);
  hipStream_t s = (hipStream_t)stream;

  const int E = a->E, K = a->K, H = a->H, I = a->I, dt = a->dtype;
  const int64_t n_flat = (int64_t)T * K;
  const int64_t nmax = (int64_t)a->Tmax * K;
  // Light experts (rows <= bm_light, one m-tile) and heavier ones (and the
  // shared expert) go to two tile lists.  bf16: light experts stream their
  // weights through registers (gemm_stream.h), heavy ones take the LDS-tiled
  // GEMM (gemm_tiled.hip), which fetches each weight panel once per tile of
  // tiled_rows() rows; one mixed launch runs both, on disjoint CUs.
  // Block-FP8: both lists run the weight-ring GEMM (gemm_ring.hip), light
  // tiles (<= 64 rows) and heavy tiles of ring_rows(true) rows.  fp32 uses
  // light tiles of 32 rows only.
  const int mr = dt == kF32 ? 1 : (n_flat <= 32ll * E ? 1 : 2);
  const int bm = 32 * mr;
  const bool fp8 = dt == kFP8;
  const int bm_heavy = dt == kF32 ? bm : fp8 ? ring_rows(true) : tiled_rows(dt);
  // fp32 runs the light list only.  bf16 batches (no shared expert) of at
  // most 32 rows per expert on average usually need no heavy list either:
  // the streaming kernel runs alone (several workgroups per CU) over light
  // tiles of 32 * mr_lo rows.  But skewed routing can put hundreds of rows on
  // one expert of such a batch, and each of its light tiles would stream its
  // weights again.  The host does not see the routing, so the dispatch
  // chooses: every expert light while the largest has at most two light
  // tiles of rows, else the mixed launch.  Both kernels are launched; the
  // other returns at once.
  const bool light_only = dt == kF32;
  const bool auto_launch = dt == kBF16 && !a->S && n_flat <= 32ll * E;
  const int heavy_min = light_only ? 0x7fffffff : bm + 1;
  // light tiles when the dispatch keeps every expert light: 32 rows up to 16
  // rows per expert on average, else 64 (one tile for most experts of a
  // uniform batch); the mixed launch keeps 32-row light tiles
  const int mr_lo = n_flat <= 16ll * E ? 1 : 2;
  // CUs this call's persistent grids spread over: all of them, or an equal
  // share when the caller runs several forwards at once on other streams
  const int cus = std::max(1, a->num_cus / a->concurrency);
  // boundary b lies before stage b (b = AFD_NUM_STAGES: after the last)
  std::array<hipEvent_t, AFD_NUM_STAGES + 1> ev{};
  const uint32_t tmask = a->timing_mask;
  auto mark = [&](int b) -> afd_status {
    const bool need = ((tmask >> b) & 1u) || (b > 0 && ((tmask >> (b - 1)) & 1u));
    if (!need) return AFD_OK;
    hipEvent_t e = take_event(a);
    if (!e) return fail(AFD_ERR_HIP, "hipEventCreate failed");
    AFD_HIP(hipEventRecord(e, s));
    ev[b] = e;
    return AFD_OK;
  };
  afd_status st;

  DispatchParams d{};
  d.ids = topk_ids;
  d.n_flat = (int32_t)n_flat;
  d.num_experts = E;
  d.chunk_shift = chunk_shift_for(n_flat, E);
  d.n_chunks = (int32_t)((n_flat + (1ll << d.chunk_shift) - 1) >> d.chunk_shift);
  d.fused = n_flat <= kDispatchFuseSlots ? 1 : 0;
  d.mix_cus = dt == kBF16 ? cus : 0;
  d.auto_heavy_rows = auto_launch ? 2 * 32 * mr_lo + 1 : 0;
  d.bm_light_only = 32 * mr_lo;
  d.counts = a->counts;
  d.offsets = a->offsets;
  d.chunk_base = a->chunk_base;
  d.err = a->err;
  d.sorted_assign = a->sorted_assign;
  d.row_of = a->row_of;
  d.bm_light = bm;
  d.bm_heavy = bm_heavy;
  d.heavy_min_rows = heavy_min;
  d.shared_rows = a->S ? T : 0;
  d.shared_row0 = (int32_t)nmax;
  d.mtiles = a->mtiles;
  d.mtiles_heavy = a->mtiles_heavy;
  d.num_mtiles = a->num_mtiles;
  a->last_T = T;

  if ((st = mark(0))) return st;
  AFD_HIP(launch_dispatch_count_scan(d, s));
  if ((st = mark(1))) return st;
  if (T == 0) {
    // nothing else to do (the later stages count as not timed)
    if (tmask) a->ev_pending.push_back(ev);
    return AFD_OK;
  }
  AFD_HIP(launch_dispatch_scatter(d, s));
  if (dt == kFP8) {
    ScaleGatherParams sg{};
    sg.src = hidden_scales;
    sg.ks = H / 128;
    sg.tokens = T;
    sg.top_k = K;
    sg.sorted_assign = a->sorted_assign;
    sg.offsets = a->offsets;
    sg.num_experts = E;
    sg.routed_max = (int32_t)n_flat;
    sg.shared_row0 = a->S ? (int32_t)nmax : -1;
    sg.dst = a->x_scales;
    sg.ld = (int32_t)a->h_rows;
    AFD_HIP(launch_gather_scales(sg, s));
  }
  if ((st = mark(2))) return st;

  // upper bounds of the routed + shared m-tiles of this call, per list
  const int64_t mt_bound = n_flat / bm + std::min<int64_t>(E, n_flat) + (a->S ? (T + bm - 1) / bm : 0) + 1;
  const int64_t mth_bound = light_only ? 0 : n_flat / heavy_min + (a->S ? (T + bm_heavy - 1) / bm_heavy : 0) + 1;
  const int64_t rows_ld_h = (int64_t)I * esize_of(dt);
  const int64_t h_rows = nmax + (a->S ? a->Tmax : 0);
  const int occupancy_wgs = 4;  // resident workgroups per CU the persistent grids aim for

  if (dt == kF32) {
    F32Params g{};
    g.mtiles = a->mtiles;
    g.num_mtiles = a->num_mtiles;
    g.sorted_assign = a->sorted_assign;
    g.top_k = K;
    g.shared_row0 = (int32_t)nmax;
    g.gather = 1;
    g.a = (const float*)hidden;
    g.w0 = (const float*)a->w->gu;
    g.w1 = (const float*)a->w->up;
    g.kdim = H;
    g.ndim = I;
    g.c = (float*)a->h;
    int grid = (int)std::min<int64_t>(mt_bound * ((I + 63) / 64), (int64_t)cus * occupancy_wgs);
    AFD_HIP(launch_gemm_f32(true, g, grid, s));
    if ((st = mark(3))) return st;
    g.gather = 0;
    g.a = (const float*)a->h;
    g.w0 = (const float*)a->w->dn;
    g.w1 = nullptr;
    g.kdim = I;
    g.ndim = H;
    g.c = (float*)a->y;
    grid = (int)std::min<int64_t>(mt_bound * ((H + 63) / 64), (int64_t)cus * occupancy_wgs);
    AFD_HIP(launch_gemm_f32(false, g, grid, s));
    if ((st = mark(4))) return st;
  } else {
    const int es = esize_of(dt);
    GemmParams g{};
    g.mtiles = a->mtiles;
    g.num_mtiles = a->num_mtiles;
    g.sorted_assign = a->sorted_assign;
    g.top_k = K;
    g.shared_row0 = (int32_t)nmax;
    // gate/up: A = hidden rows gathered by token
    g.gather = 1;
    g.a = (const uint8_t*)hidden;
    g.a_bytes = (int64_t)T * H * es;
    g.a_row_bytes = (int64_t)H * es;
    g.a_scales = a->x_scales;  // gathered by gather_scales_kernel
    g.a_scale_bytes = fp8 ? (int64_t)(H / 128) * a->h_rows * 4 : 0;
    g.a_scale_ld = (int32_t)a->h_rows;
    g.b = a->w->gu;
    g.b_expert_bytes = a->w->gu_expert_bytes;
    g.b_panel_bytes = a->w->gu_panel_bytes;
    g.b_scales0 = a->w->sg;
    g.b_scale_bytes = a->w->scale_bytes;
    g.b_scales1 = a->w->su;
    g.b_scale_rows = H / 128;
    g.b_scale_cols = I / 128;
    g.k_steps = (int32_t)((int64_t)H * es / kStepBytes);
    g.n_panels = I / 32;
    g.n_groups = I / 128;
    g.c = a->h;
    g.c_row_bytes = rows_ld_h;
    g.c_scales = a->h_scales;
    g.c_scale_ld = (int32_t)a->h_rows;
    GemmParams gu_light = g;
    GemmParams gu_heavy = g;
    gu_heavy.mtiles = a->mtiles_heavy;
    gu_heavy.num_mtiles = a->num_mtiles + 1;
    gu_heavy.n_groups = (2 * I / 32 + tiled_panels() - 1) / tiled_panels();  // bf16 only
    // down: A = h rows in sorted order
    g.gather = 0;
    g.a = a->h;
    g.a_bytes = h_rows * rows_ld_h;
    g.a_row_bytes = rows_ld_h;
    g.a_scales = a->h_scales;
    g.a_scale_bytes = fp8 ? h_rows * (I / 128) * 4 : 0;
    g.a_scale_ld = (int32_t)a->h_rows;
    g.b = a->w->dn;
    g.b_expert_bytes = a->w->dn_expert_bytes;
    g.b_panel_bytes = a->w->dn_panel_bytes;
    g.b_scales0 = a->w->sd;
    g.b_scales1 = a->w->sd;
    g.b_scale_rows = I / 128;
    g.b_scale_cols = H / 128;
    g.k_steps = (int32_t)((int64_t)I * es / kStepBytes);
    g.n_panels = H / 32;
    // light tasks of the down GEMM: down_panels_per_task(mr) H panels (bf16
    // streaming GEMM) or 8 (block-FP8 ring GEMM, both lists)
    const int dn_panels = fp8 ? 8 : down_panels_per_task(mr);
    g.n_groups = (H / 32 + dn_panels - 1) / dn_panels;
    g.c = a->y;
    g.c_row_bytes = (int64_t)H * 2;
    g.c_scales = nullptr;
    g.c_scale_ld = 0;
    GemmParams dn_light = g;
    GemmParams dn_heavy = g;
    dn_heavy.mtiles = a->mtiles_heavy;
    dn_heavy.num_mtiles = a->num_mtiles + 1;
    dn_heavy.n_groups = (H / 32 + tiled_panels() - 1) / tiled_panels();  // bf16 only

    // One launch per GEMM (two gated ones where the dispatch chooses).  bf16:
    // the light list alone (streaming kernel, several workgroups per CU) or,
    // once heavy experts occur, the mixed kernel:
    // one workgroup per CU, the dispatch's share of them streaming the light
    // list while the rest run the heavy tiles (HBM-bound and MFMA-bound work
    // side by side; a heavy workgroup leaves no room for a light one on its
    // CU, so the split is by CU).  Block-FP8 runs both lists in one launch of
    // the ring GEMM.
    auto stage = [&](bool gate_up, const GemmParams& light, const GemmParams& heavy) -> hipError_t {
      if (fp8) {
        GemmParams both = light;
        both.mtiles2 = heavy.mtiles;
        both.num_mtiles2 = heavy.num_mtiles;
        return launch_gemm_ring(gate_up, a->concurrency == 1, both, (mt_bound + mth_bound) * light.n_groups, cus, s);
      }
      if (auto_launch) {
        GemmParams lo = light, mx = light;
        lo.only_launch = kLaunchLight;
        mx.only_launch = kLaunchMixed;
        if (!gate_up) lo.n_groups = (H / 32 + down_panels_per_task(mr_lo) - 1) / down_panels_per_task(mr_lo);
        const hipError_t e = launch_gemm(dt, gate_up, mr_lo, lo, mt_bound * lo.n_groups, cus, s);
        if (e != hipSuccess) return e;
        return launch_gemm_mixed(gate_up, mr, heavy, mx, cus, s);
      }
      return launch_gemm_mixed(gate_up, mr, heavy, light, cus, s);
    };
    AFD_HIP(stage(true, gu_light, gu_heavy));
    if ((st = mark(3))) return st;
    AFD_HIP(stage(false, dn_light, dn_heavy));
    if ((st = mark(4))) return st;
  }

  CombineParams cp{};
  cp.y = a->y;
  cp.y_bytes = (nmax + (a->S ? a->Tmax : 0)) * (int64_t)H * (dt == kF32 ? 4 : 2);
  cp.row_of = a->row_of;
  cp.weights = topk_weights;
  cp.top_k = K;
  cp.hidden = H;
  cp.shared_row0 = a->S ? (int32_t)nmax : -1;
  cp.out = (uint8_t*)out;
  AFD_HIP(launch_combine(dt == kF32 ? kF32 : kBF16, cp, T, s));
  if ((st = mark(5))) return st;
  if (tmask) a->ev_pending.push_back(ev);
  return AFD_OK;
}

afd_status afd_ffn_debug_dispatch(afd_ffn_t* a, int32_t* counts, int32_t* offsets, int32_t* sorted_assign,
                                  int32_t* row_of, void* stream) {
  g_last_error.clear();
  if (!a) return fail(AFD_ERR_INVALID_ARG, "handle is NULL");
  DeviceGuard dg(a->device);
  hipStream_t s = (hipStream_t)stream;
  const int64_t n = (int64_t)a->last_T * a->K;
  if (counts) AFD_HIP(hipMemcpyAsync(counts, a->counts, 4ll * a->E, hipMemcpyDeviceToDevice, s));
  if (offsets) AFD_HIP(hipMemcpyAsync(offsets, a->offsets, 4ll * (a->E + 1), hipMemcpyDeviceToDevice, s));
  if (sorted_assign && n) AFD_HIP(hipMemcpyAsync(sorted_assign, a->sorted_assign, 4 * n, hipMemcpyDeviceToDevice, s));
  if (row_of && n) AFD_HIP(hipMemcpyAsync(row_of, a->row_of, 4 * n, hipMemcpyDeviceToDevice, s));
  return AFD_OK;
}

afd_status afd_ffn_routing_errors(afd_ffn_t* a, int32_t* count, void* stream) {
  g_last_error.clear();
  if (!a || !count) return fail(AFD_ERR_INVALID_ARG, "NULL argument");
  DeviceGuard dg(a->device);
  hipStream_t s = (hipStream_t)stream;
  AFD_HIP(hipMemcpyAsync(count, a->err, 4, hipMemcpyDeviceToHost, s));
  AFD_HIP(hipStreamSynchronize(s));
  return *count > 0 ? fail(AFD_ERR_BAD_ROUTING, "%d ids outside [-1, %d)", *count, a->E) : AFD_OK;
}

afd_status afd_ffn_set_concurrency(afd_ffn_t* a, int32_t streams) {
  g_last_error.clear();
  if (!a) return fail(AFD_ERR_INVALID_ARG, "handle is NULL");
  if (streams < 1 || streams > a->num_cus)
    return fail(AFD_ERR_INVALID_ARG, "concurrency %d outside [1, %d]", streams, a->num_cus);
  a->concurrency = streams;
  return AFD_OK;
}

afd_status afd_ffn_set_timing(afd_ffn_t* a, int32_t enable) {
  g_last_error.clear();
  if (!a) return fail(AFD_ERR_INVALID_ARG, "handle is NULL");
  a->timing_mask = enable ? (1u << AFD_NUM_STAGES) - 1 : 0u;
  return AFD_OK;
}

afd_status afd_ffn_set_timing_stages(afd_ffn_t* a, uint32_t stage_mask) {
  g_last_error.clear();
  if (!a) return fail(AFD_ERR_INVALID_ARG, "handle is NULL");
  if (stage_mask >> AFD_NUM_STAGES)
    return fail(AFD_ERR_INVALID_ARG, "stage mask 0x%x has bits past stage %d", stage_mask, AFD_NUM_STAGES - 1);
  a->timing_mask = stage_mask;
  return AFD_OK;
}

afd_status afd_ffn_get_timing(afd_ffn_t* a, float* ms, int32_t* num_forwards) {
  g_last_error.clear();
  if (!a || !ms) return fail(AFD_ERR_INVALID_ARG, "NULL argument");
  DeviceGuard dg(a->device);
  for (int i = 0; i < AFD_NUM_STAGES; ++i) ms[i] = 0.0f;
  int n = 0;
  for (auto& v : a->ev_pending) {
    hipEvent_t last = nullptr;
    for (hipEvent_t e : v)
      if (e) last = e;
    if (last) AFD_HIP(hipEventSynchronize(last));
    for (int i = 0; i < AFD_NUM_STAGES; ++i) {
      if (!v[i] || !v[i + 1]) continue;
      float t = 0.0f;
      AFD_HIP(hipEventElapsedTime(&t, v[i], v[i + 1]));
      ms[i] += t;
    }
    for (hipEvent_t e : v)
      if (e) a->ev_free.push_back(e);
    ++n;
  }
  a->ev_pending.clear();
  if (num_forwards) *num_forwards = n;
  return AFD_OK;
}

}  // extern "C"
