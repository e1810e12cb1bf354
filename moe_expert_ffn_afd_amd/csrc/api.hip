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
#include <mutex>
#include <string>
#include <vector>

#include "../../include/afd_ffn.h"
#include "afd_internal.h"

using namespace afd;

// Device scratch of afd_ffn_forward_noalloc: the workspace of such a forward is
// carved out of this array instead of the handle's allocation.  Host code
// never passes the name itself to a kernel or a copy (on the host it is only a
// stand-in for the symbol): it uses the device address hipGetSymbolAddress
// returns, one per device (each device holds its own copy of the array).
// The array has external linkage: a `static` one stays a local symbol of the
// code object (this library is compiled without relocatable device code),
// which the runtime's lookup by name does not find.
__device__ __attribute__((used)) __align__(256) uint8_t afd_ffn_noalloc_scratch[AFD_FFN_NOALLOC_SCRATCH_BYTES];

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
  // bf16 / fp8 / w8a8: packed gate+up and down; f32: plain gate, up, down
  uint8_t* gu = nullptr;
  uint8_t* up = nullptr;  // f32 only
  uint8_t* dn = nullptr;
  float* sg = nullptr;
  float* su = nullptr;
  float* sd = nullptr;
  int64_t gu_expert_bytes = 0, dn_expert_bytes = 0;
  int64_t gu_panel_bytes = 0, dn_panel_bytes = 0;
  int64_t scale_bytes = 0;     // block-FP8: bytes of each of sg, su, sd; W8A8: of sg and su
  int64_t dn_scale_bytes = 0;  // bytes of sd
  ~WeightStore() {
    for (void* p : {(void*)gu, (void*)up, (void*)dn, (void*)sg, (void*)su, (void*)sd})
      if (p) (void)hipFree(p);
  }
};

int esize_of(int dtype) { return dtype == kF32 ? 4 : dtype == kBF16 ? 2 : 1; }

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_addr[kMaxScratchDevices];  // device address of the scratch array, per device ordinal

// Device address of the scratch array on `device`, which must be the current
// device; looked up once per device, at the first allocation-free forward there
// (the library's code object is loaded by then: handle creation ran its
// packing kernel on the device).
afd_status scratch_address(int device, uint8_t** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxScratchDevices)
    return fail(AFD_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", device,
                kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(afd_ffn_noalloc_scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(AFD_ERR_HIP, "hipGetSymbolAddress(afd_ffn_noalloc_scratch) on device %d failed: %s", device,
                  hipGetErrorString(e));
    }
    g_scratch_addr[device] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_addr[device];
  return AFD_OK;
}

}  // namespace

namespace {

// A canary guard band of a workspace: `off` bytes into the allocation, after
// the region `after` (the first band, before every region: "start").
struct GuardBand {
  int64_t off;
  const char* after;
};
constexpr uint8_t kCanaryByte = 0xA5;
constexpr int64_t kMaxGuardBytes = 16ll << 20;

// Per-forward device buffers (section "Workspace" of afd_internal.h), carved
// out of one allocation for a token capacity `tcap`.
struct Workspace {
  int32_t *counts = nullptr, *offsets = nullptr, *err = nullptr, *num_mtiles = nullptr;
  int32_t *chunk_base = nullptr, *sorted_assign = nullptr, *row_of = nullptr;
  int4* mtiles = nullptr;
  int4* mtiles_heavy = nullptr;
  int4* mtiles_tiled = nullptr;  // 8-bit layers: experts with many rows (gemm_tiled8.h)
  int32_t* pool = nullptr;    // [2] the ring GEMMs' tail-pool counters
  uint8_t* h = nullptr;       // bf16 | e4m3 | fp32 (W8A8: bf16, before re-quantisation)
  float* h_scales = nullptr;  // FP8: [I/128][h_rows] step-major; W8A8: [h_rows]
  float* x_scales = nullptr;  // FP8: [H/128][h_rows] hidden scales in sorted-row order; W8A8: [h_rows]
  uint8_t* h8 = nullptr;      // W8A8: [h_rows, I] int8 codes of h
  float* pamax = nullptr;     // W8A8: [I/128][h_rows] per-row amax of each gate/up task's columns
  uint8_t* y = nullptr;
  // the fused launch (8-bit layers): grid-barrier state and the dispatch's chunk sums
  int32_t *bar = nullptr, *chunk_counts = nullptr, *chunk_bad = nullptr, *local_base = nullptr, *totals = nullptr;
  int fused_grid = 0;  // workgroups the chunk arrays are sized for
  int64_t nmax = 0;    // routed-row capacity tcap * K; the shared expert's rows start here
  int64_t h_rows = 0;  // rows of h and y: nmax (+ tcap with a shared expert)
  int tcap = 0;
};

}  // namespace

struct afd_ffn {
  int H = 0, I = 0, E = 0, K = 0, Tmax = 0, S = 0, dtype = 0, device = 0;
  int num_cus = 256;
  int concurrency = 1;  // forwards the caller runs at once on other streams (afd_ffn_set_concurrency)
  int fused = 0;        // 1: the whole layer in one persistent launch (afd_ffn_set_fused)
  WeightStore* w = nullptr;
  uint8_t* ws_mem = nullptr;  // the handle's workspace allocation (sized for Tmax)
  Workspace ws;
  // canary guard bands of ws_mem (afd_ffn_set_canaries): band bytes (0: none)
  // and, per band, its offset and the region before it
  int64_t guard = 0;
  std::vector<GuardBand> bands;
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
  if (c->dtype < 0 || c->dtype > 3) return fail(AFD_ERR_UNSUPPORTED, "unknown dtype %d", c->dtype);
  if (c->hidden <= 0 || c->inter <= 0 || c->num_experts <= 0 || c->top_k <= 0 || c->max_tokens <= 0)
    return fail(AFD_ERR_INVALID_ARG, "hidden, inter, num_experts, top_k and max_tokens must be positive");
  if (c->hidden % 128 || c->inter % 128)
    return fail(AFD_ERR_UNSUPPORTED, "hidden (%d) and inter (%d) must be multiples of 128", c->hidden, c->inter);
  if (c->dtype == kFP8 && (c->hidden > 16384 || c->inter > 16384))
    return fail(AFD_ERR_UNSUPPORTED, "block-FP8 reductions are limited to 128 blocks (hidden, inter <= 16384)");
  if (c->dtype == kW8A8 && (c->hidden > 16384 || c->inter > 16384))
    return fail(AFD_ERR_UNSUPPORTED, "W8A8 reductions are limited to 16384 (int32 accumulation)");
  if (c->num_experts > kMaxExperts) return fail(AFD_ERR_UNSUPPORTED, "num_experts %d > %d", c->num_experts, kMaxExperts);
  if (c->top_k > kMaxTopK) return fail(AFD_ERR_UNSUPPORTED, "top_k %d > %d", c->top_k, kMaxTopK);
  if ((int64_t)c->max_tokens * c->top_k >= (1ll << 26))
    return fail(AFD_ERR_UNSUPPORTED, "max_tokens * top_k must stay below 2^26");
  if (c->shared_inter < 0 || c->shared_inter % 128 ||
      (int64_t)c->shared_inter > (int64_t)kMaxSharedParts * c->inter)
    return fail(AFD_ERR_UNSUPPORTED, "shared_inter (%d) must be 0 or a multiple of 128 of at most %d x inter",
                c->shared_inter, kMaxSharedParts);
  {
    // the GEMMs and the combine address rows (hidden, h, y) with 32-bit buffer offsets
    const int64_t es = c->dtype == kF32 ? 4 : c->dtype == kBF16 ? 2 : 1;
    const int64_t parts = (c->shared_inter + c->inter - 1) / c->inter;  // the shared expert's parts of width I
    const int64_t rows = (int64_t)c->max_tokens * c->top_k + parts * c->max_tokens;
    const int64_t lim = (1ll << 31) - (1ll << 24);
    const int64_t ys = c->dtype == kF32 ? 4 : 2;  // expert outputs y are bf16 | fp32
    const int64_t hs = c->dtype == kW8A8 ? 2 : es;  // W8A8 keeps h in bf16 before re-quantising it
    if (rows * std::max(c->hidden, c->inter) * es > lim || (int64_t)c->max_tokens * c->hidden * es > lim ||
        rows * c->hidden * ys > lim || rows * c->inter * hs > lim)
      return fail(AFD_ERR_UNSUPPORTED, "activation buffers of max_tokens=%d exceed 2 GiB", c->max_tokens);
  }
  if (c->device < 0) return fail(AFD_ERR_INVALID_ARG, "device must be >= 0");
  if (!c->w_gate || !c->w_up || !c->w_down) return fail(AFD_ERR_INVALID_ARG, "weight pointer is NULL");
  const bool fp8 = c->dtype == kFP8 || c->dtype == kW8A8;  // 8-bit codes with fp32 scales
  if (fp8 && (!c->s_gate || !c->s_up || !c->s_down))
    return fail(AFD_ERR_INVALID_ARG, "block-FP8 and W8A8 weights need s_gate, s_up and s_down");
  if (!fp8 && (c->s_gate || c->s_up || c->s_down))
    return fail(AFD_ERR_INVALID_ARG, "weight scales are only used with AFD_DTYPE_FP8_BLOCK and AFD_DTYPE_W8A8");
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

// Lay the workspace of a token capacity `tcap` out from `base` (which may be
// null: sizes only) and return its size in bytes.  guard > 0 puts a band of
// that many bytes (a multiple of 256) before the first region and right after
// the last byte of every region, listed in `bands` when given.
int64_t layout_workspace(const afd_ffn* a, int tcap, uint8_t* base, Workspace* w, int64_t guard = 0,
                         std::vector<GuardBand>* bands = nullptr) {
  const int64_t nmax = (int64_t)tcap * a->K;
  const int64_t rows = nmax + (int64_t)a->S * tcap;  // routed rows, then the shared expert's parts
  const int64_t max_chunks = (nmax + 1023) / 1024;
  const int64_t max_mtiles = nmax / 32 + a->E + (int64_t)a->S * ((tcap + 31) / 32) + 1;
  const int es = esize_of(a->dtype);
  const int ys = a->dtype == kF32 ? 4 : 2;
  const bool w8 = a->dtype == kW8A8;
  int64_t off = 0;
  if (bands) bands->clear();
  if (guard > 0) {  // the band before every region
    if (bands) bands->push_back({0, "start"});
    off = guard;
  }
  auto take = [&](int64_t bytes, const char* name) {  // a region, then its band from its exact end
    const int64_t o = off;
    if (guard > 0 && bytes > 0) {
      if (bands) bands->push_back({o + bytes, name});
      off = align_up(o + bytes + guard, 256);
    } else {
      off = align_up(o + bytes, 256);
    }
    return o;
  };
  const int64_t o_counts = take(4ll * a->E, "counts"), o_offsets = take(4ll * (a->E + 1), "offsets"),
                o_err = take(4, "err"), o_nmt = take(32, "num_mtiles"),
                o_cb = take(4ll * max_chunks * a->E, "chunk_base"), o_sa = take(4 * nmax, "sorted_assign"),
                o_ro = take(4 * nmax, "row_of"), o_mt = take(16ll * max_mtiles, "mtiles"),
                o_mth = take(16ll * max_mtiles, "mtiles_heavy"),
                o_mtt = take(a->dtype == kFP8 || w8 ? 16ll * max_mtiles : 0, "mtiles_tiled"),
                o_pool = take(16, "pool"),
                o_h = take(rows * a->I * (w8 ? 2 : es), "h"),
                o_hs = take(a->dtype == kFP8 ? rows * (a->I / 128) * 4 : w8 ? rows * 4 : 0, "h_scales"),
                o_xs = take(a->dtype == kFP8 ? rows * (a->H / 128) * 4 : w8 ? rows * 4 : 0, "x_scales"),
                o_h8 = take(w8 ? rows * a->I : 0, "h8"), o_pm = take(w8 ? rows * (a->I / 128) * 4 : 0, "pamax"),
                o_y = take(rows * a->H * ys, "y");
  const bool fz = a->dtype != kF32;  // the fused launch's state
  const int64_t fg = fz ? std::min(a->num_cus, kFusedMaxGrid) : 0;
  const int64_t o_bar = take(fz ? 16 : 0, "bar"), o_fcc = take(4 * fg * a->E, "chunk_counts"),
                o_fcb = take(4 * fg, "chunk_bad"), o_flb = take(4 * fg * a->E, "local_base"),
                o_ftot = take(fz ? 4ll * a->E : 0, "totals");
  if (base && w) {
    w->counts = (int32_t*)(base + o_counts);
    w->offsets = (int32_t*)(base + o_offsets);
    w->err = (int32_t*)(base + o_err);
    w->num_mtiles = (int32_t*)(base + o_nmt);
    w->chunk_base = (int32_t*)(base + o_cb);
    w->sorted_assign = (int32_t*)(base + o_sa);
    w->row_of = (int32_t*)(base + o_ro);
    w->mtiles = (int4*)(base + o_mt);
    w->mtiles_heavy = (int4*)(base + o_mth);
    w->mtiles_tiled = a->dtype == kFP8 || w8 ? (int4*)(base + o_mtt) : nullptr;
    w->pool = (int32_t*)(base + o_pool);
    w->h = base + o_h;
    const bool sc = a->dtype == kFP8 || w8;
    w->h_scales = sc ? (float*)(base + o_hs) : nullptr;
    w->x_scales = sc ? (float*)(base + o_xs) : nullptr;
    w->h8 = w8 ? base + o_h8 : nullptr;
    w->pamax = w8 ? (float*)(base + o_pm) : nullptr;
    w->bar = fz ? (int32_t*)(base + o_bar) : nullptr;
    w->chunk_counts = fz ? (int32_t*)(base + o_fcc) : nullptr;
    w->chunk_bad = fz ? (int32_t*)(base + o_fcb) : nullptr;
    w->local_base = fz ? (int32_t*)(base + o_flb) : nullptr;
    w->totals = fz ? (int32_t*)(base + o_ftot) : nullptr;
    w->fused_grid = (int)fg;
    w->y = base + o_y;
    w->nmax = nmax;
    w->h_rows = rows;
    w->tcap = tcap;
  }
  return off;
}

afd_status alloc_workspace(afd_ffn* a) {
  const int64_t bytes = layout_workspace(a, a->Tmax, nullptr, nullptr, a->guard);
  if (hipMalloc((void**)&a->ws_mem, bytes) != hipSuccess) {
    (void)hipGetLastError();
    a->ws_mem = nullptr;
    return fail(AFD_ERR_OUT_OF_MEMORY, "workspace of %lld bytes", (long long)bytes);
  }
  layout_workspace(a, a->Tmax, a->ws_mem, &a->ws, a->guard, &a->bands);
  AFD_HIP(hipMemset(a->ws_mem, 0, bytes));
  for (const GuardBand& b : a->bands) AFD_HIP(hipMemset(a->ws_mem + b.off, kCanaryByte, a->guard));
  if (a->guard > 0) AFD_HIP(hipDeviceSynchronize());  // the bands are filled before any forward runs
  return AFD_OK;
}

// Part v of the shared expert (its intermediate columns [v I, v I + I), the
// last part zero-padded to width I) as one expert's matrices: gate and up
// [H, I] from sh_gate, sh_up [H, shared_inter], down [I, H] from the rows of
// sh_down [shared_inter, H]; es bytes per element.  SwiGLU separates along the
// intermediate dimension, and zero columns and rows add exactly nothing.
afd_status copy_shared_part(const afd_ffn_config* c, const afd_ffn* a, int v, int es, uint8_t* g, uint8_t* u,
                            uint8_t* d) {
  const int H = a->H, I = a->I, Is = c->shared_inter;
  const int wv = std::min(I, Is - v * I);
  const int64_t mat = (int64_t)H * I * es;
  if (wv < I)
    for (uint8_t* q : {g, u, d}) AFD_HIP(hipMemset(q, 0, mat));
  AFD_HIP(hipMemcpy2D(g, (size_t)I * es, (const uint8_t*)c->sh_gate + (int64_t)v * I * es, (size_t)Is * es,
                      (size_t)wv * es, H, hipMemcpyDeviceToDevice));
  AFD_HIP(hipMemcpy2D(u, (size_t)I * es, (const uint8_t*)c->sh_up + (int64_t)v * I * es, (size_t)Is * es,
                      (size_t)wv * es, H, hipMemcpyDeviceToDevice));
  AFD_HIP(hipMemcpy(d, (const uint8_t*)c->sh_down + (int64_t)v * I * H * es, (int64_t)wv * H * es,
                    hipMemcpyDeviceToDevice));
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
    for (int v = 0; v < a->S; ++v)
      if ((st = copy_shared_part(c, a, v, 4, w->gu + mat * (E + v), w->up + mat * (E + v), w->dn + mat * (E + v))))
        return st;
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
    // each part of the shared expert, zero-padded to width I in a staging
    // buffer, then packed as expert E + v
    const int64_t mat = (int64_t)H * I * es;
    uint8_t* stg = nullptr;
    if ((st = mal(&stg, 3 * mat))) return st;
    for (int v = 0; v < a->S && st == AFD_OK; ++v) {
      st = copy_shared_part(c, a, v, es, stg, stg + mat, stg + 2 * mat);
      if (st == AFD_OK &&
          (launch_pack(dt, true, stg, stg + mat, (int64_t)H * I, 1, H, I, w->gu + w->gu_expert_bytes * (E + v),
                       w->gu_expert_bytes, 0) != hipSuccess ||
           launch_pack(dt, false, stg + 2 * mat, nullptr, (int64_t)I * H, 1, I, H,
                       w->dn + w->dn_expert_bytes * (E + v), w->dn_expert_bytes, 0) != hipSuccess ||
           hipDeviceSynchronize() != hipSuccess))
        st = fail(AFD_ERR_HIP, "packing part %d of the shared expert failed", v);
    }
    (void)hipFree(stg);
    if (st) return st;
  }
  if (dt == kW8A8) {
    // per output channel: gate, up [E+S][I], down [E+S][H]
    const int64_t sgu = (int64_t)I * 4, sdn = (int64_t)H * 4;
    if ((st = mal((uint8_t**)&w->sg, sgu * ES)) || (st = mal((uint8_t**)&w->su, sgu * ES)) ||
        (st = mal((uint8_t**)&w->sd, sdn * ES)))
      return st;
    w->scale_bytes = sgu * ES;
    w->dn_scale_bytes = sdn * ES;
    AFD_HIP(hipMemcpy(w->sg, c->s_gate, sgu * E, hipMemcpyDeviceToDevice));
    AFD_HIP(hipMemcpy(w->su, c->s_up, sgu * E, hipMemcpyDeviceToDevice));
    AFD_HIP(hipMemcpy(w->sd, c->s_down, sdn * E, hipMemcpyDeviceToDevice));
    for (int v = 0; v < a->S; ++v) {
      // part v: the gate and up scales of its columns (1 for the padding, whose
      // codes are 0), the down scales (per output column) unchanged
      const int wv = std::min(I, c->shared_inter - v * I);
      float* g = (float*)((uint8_t*)w->sg + sgu * (E + v));
      float* u = (float*)((uint8_t*)w->su + sgu * (E + v));
      AFD_HIP(hipMemsetD32((hipDeviceptr_t)g, 0x3f800000, I));
      AFD_HIP(hipMemsetD32((hipDeviceptr_t)u, 0x3f800000, I));
      AFD_HIP(hipMemcpy(g, c->sh_s_gate + (int64_t)v * I, 4ll * wv, hipMemcpyDeviceToDevice));
      AFD_HIP(hipMemcpy(u, c->sh_s_up + (int64_t)v * I, 4ll * wv, hipMemcpyDeviceToDevice));
      AFD_HIP(hipMemcpy((uint8_t*)w->sd + sdn * (E + v), c->sh_s_down, sdn, hipMemcpyDeviceToDevice));
    }
  }
  if (dt == kFP8) {
    const int64_t sblk = (int64_t)(H / 128) * (I / 128) * 4;
    if ((st = mal((uint8_t**)&w->sg, sblk * ES)) || (st = mal((uint8_t**)&w->su, sblk * ES)) ||
        (st = mal((uint8_t**)&w->sd, sblk * ES)))
      return st;
    w->scale_bytes = w->dn_scale_bytes = sblk * ES;
    AFD_HIP(hipMemcpy(w->sg, c->s_gate, sblk * E, hipMemcpyDeviceToDevice));
    AFD_HIP(hipMemcpy(w->su, c->s_up, sblk * E, hipMemcpyDeviceToDevice));
    AFD_HIP(hipMemcpy(w->sd, c->s_down, sblk * E, hipMemcpyDeviceToDevice));
    for (int v = 0; v < a->S; ++v) {
      // part v: its columns' blocks of the gate and up grids [H/128][Is/128]
      // and its rows' blocks of the down grid [Is/128][H/128] (1 for the
      // padding blocks, whose codes are 0)
      const int wb = std::min(I, c->shared_inter - v * I) / 128, ib = I / 128, isb = c->shared_inter / 128;
      float* g = (float*)((uint8_t*)w->sg + sblk * (E + v));
      float* u = (float*)((uint8_t*)w->su + sblk * (E + v));
      float* dd = (float*)((uint8_t*)w->sd + sblk * (E + v));
      for (float* q : {g, u, dd}) AFD_HIP(hipMemsetD32((hipDeviceptr_t)q, 0x3f800000, (H / 128) * ib));
      AFD_HIP(hipMemcpy2D(g, 4ll * ib, c->sh_s_gate + (int64_t)v * ib, 4ll * isb, 4ll * wb, H / 128,
                          hipMemcpyDeviceToDevice));
      AFD_HIP(hipMemcpy2D(u, 4ll * ib, c->sh_s_up + (int64_t)v * ib, 4ll * isb, 4ll * wb, H / 128,
                          hipMemcpyDeviceToDevice));
      AFD_HIP(hipMemcpy(dd, c->sh_s_down + (int64_t)v * ib * (H / 128), 4ll * wb * (H / 128),
                        hipMemcpyDeviceToDevice));
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
  if (a->ws_mem) (void)hipFree(a->ws_mem);
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

// Host checks of a forward's arguments (T at most `tcap`).
afd_status check_forward_args(const afd_ffn* a, int32_t T, int64_t tcap, const void* hidden,
                              const float* hidden_scales, const int32_t* topk_ids, const float* topk_weights,
                              const void* out) {
  if (!a) return fail(AFD_ERR_INVALID_ARG, "handle is NULL");
  if (T < 0 || T > tcap) return fail(AFD_ERR_INVALID_ARG, "num_tokens %d outside [0, %lld]", T, (long long)tcap);
  if (T > 0 && (!hidden || !topk_ids || !topk_weights || !out))
    return fail(AFD_ERR_INVALID_ARG, "hidden, topk_ids, topk_weights and out must be non-NULL");
  const bool scaled = a->dtype == kFP8 || a->dtype == kW8A8;
  if (scaled && T > 0 && !hidden_scales)
    return fail(AFD_ERR_INVALID_ARG, "block-FP8 and W8A8 input needs hidden_scales");
  if (!scaled && hidden_scales)
    return fail(AFD_ERR_INVALID_ARG, "hidden_scales is only used with AFD_DTYPE_FP8_BLOCK and AFD_DTYPE_W8A8");
  auto mis = [](const void* q, uintptr_t al) { return q && (reinterpret_cast<uintptr_t>(q) & (al - 1)); };
  if (mis(hidden, 16) || mis(out, 16)) return fail(AFD_ERR_INVALID_ARG, "hidden and out must be 16-byte aligned");
  if (mis(hidden_scales, 4) || mis(topk_ids, 4) || mis(topk_weights, 4))
    return fail(AFD_ERR_INVALID_ARG, "hidden_scales, topk_ids and topk_weights must be 4-byte aligned");
  return AFD_OK;
}

// Enqueue one forward on `stream` with the buffers of `w` (capacity w.tcap >= T).
// `timed`: record the handle's timing events (the handle's own workspace only).
// `own_ws`: w is the handle's workspace (the fused launch keeps its barrier
// state there, zero between calls).
afd_status forward_impl(afd_ffn* a, const Workspace& w, bool timed, bool own_ws, int32_t T, const void* hidden,
                        const float* hidden_scales, const int32_t* topk_ids, const float* topk_weights, void* out,
                        void* stream) {
  DeviceGuard dg(a->device);
  if (!dg.ok) return fail(AFD_ERR_HIP, "cannot select device %d", a->device);
  hipStream_t s = (hipStream_t)stream;

  const int E = a->E, K = a->K, H = a->H, I = a->I, dt = a->dtype;
  const int64_t n_flat = (int64_t)T * K;
  const int64_t nmax = w.nmax;
  // Light experts (rows <= bm_light, one m-tile) and heavier ones (and the
  // shared expert) go to two tile lists.  bf16: light experts stream their
  // weights through registers (gemm_stream.h), heavy ones take the LDS-tiled
  // GEMM (gemm_tiled.hip), which fetches each weight panel once per tile of
  // tiled_rows() rows; one mixed launch runs both, on disjoint CUs.
  // Block-FP8 and W8A8: both lists run the weight-ring GEMM (gemm_ring.hip),
  // light tiles (<= 64 rows) and heavy tiles of ring_rows(true) rows.  fp32
  // uses light tiles of 32 rows only.
  const int mr = dt == kF32 ? 1 : (n_flat <= 32ll * E ? 1 : 2);
  const int bm = 32 * mr;
  const bool w8 = dt == kW8A8;
  const bool fp8 = dt == kFP8 || w8;  // 8-bit codes: the ring GEMM
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
  const uint32_t tmask = timed ? a->timing_mask : 0u;
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
  d.counts = w.counts;
  d.offsets = w.offsets;
  d.chunk_base = w.chunk_base;
  d.err = w.err;
  d.sorted_assign = w.sorted_assign;
  d.row_of = w.row_of;
  d.bm_light = bm;
  d.bm_heavy = bm_heavy;
  d.heavy_min_rows = heavy_min;
  d.shared_rows = a->S ? T : 0;
  d.shared_parts = a->S;
  d.shared_row0 = (int32_t)nmax;
  d.mtiles = w.mtiles;
  d.mtiles_heavy = w.mtiles_heavy;
  // 8-bit batches of at least 128 routed rows per expert on average: the
  // experts of more rows than one 128-row ring tile take the LDS-tiled 8-bit
  // body (256-row tiles, gemm_tiled8.h) instead of two or more ring tiles,
  // each of which would stream the expert's weights again
  const bool tiled8 = fp8 && n_flat >= (int64_t)kTiled8MeanRows * E;
  d.mtiles_tiled = w.mtiles_tiled;
  d.bm_tiled = kTiled8Rows;
  d.tiled_min_rows = tiled8 ? kTiled8MinRows : 0x7fffffff;
  d.num_mtiles = w.num_mtiles;
  d.pool = dt != kF32 ? w.pool : nullptr;  // the tail pools of the ring and the bf16 tiled GEMMs

  // the whole layer in one persistent launch (afd_ffn_set_fused; not fp32)
  const bool use_fused = own_ws && a->fused && dt != kF32 && T > 0;
  if ((st = mark(0))) return st;
  if (!use_fused) AFD_HIP(launch_dispatch_count_scan(d, s));
  if ((st = mark(1))) return st;
  if (T == 0) {
    // nothing else to do (the later stages count as not timed)
    if (tmask) a->ev_pending.push_back(ev);
    return AFD_OK;
  }
  if (!use_fused) AFD_HIP(launch_dispatch_scatter(d, s));
  if (fp8 && !use_fused) {
    // the hidden rows' scales in sorted-row order: block-FP8 one per 128
    // columns (step-major), W8A8 one per token
    ScaleGatherParams sg{};
    sg.src = hidden_scales;
    sg.ks = w8 ? 1 : H / 128;
    sg.tokens = T;
    sg.top_k = K;
    sg.sorted_assign = w.sorted_assign;
    sg.offsets = w.offsets;
    sg.num_experts = E;
    sg.routed_max = (int32_t)n_flat;
    sg.shared_row0 = a->S ? (int32_t)nmax : -1;
    sg.shared_parts = a->S;
    sg.dst = w.x_scales;
    sg.ld = (int32_t)w.h_rows;
    AFD_HIP(launch_gather_scales(sg, s));
  }
  if ((st = mark(2))) return st;  // (fused: the boundary before its one launch)

  // upper bounds of the routed + shared m-tiles of this call, per list
  const int64_t mt_bound = n_flat / bm + std::min<int64_t>(E, n_flat) + (int64_t)a->S * ((T + bm - 1) / bm) + 1;
  const int64_t mtt_bound =
      tiled8 ? n_flat / kTiled8Rows + std::min<int64_t>(E, n_flat / kTiled8MinRows) +
                   (int64_t)a->S * ((T + kTiled8Rows - 1) / kTiled8Rows) + 1
             : 0;
  const int64_t mth_bound =
      light_only ? 0 : n_flat / heavy_min + (int64_t)a->S * ((T + bm_heavy - 1) / bm_heavy) + 1;
  const int64_t rows_ld_h = (int64_t)I * (w8 ? 2 : esize_of(dt));  // W8A8: bf16 h before re-quantisation
  const int64_t h_rows = w.h_rows;
  const int occupancy_wgs = 4;  // resident workgroups per CU the persistent grids aim for

  CombineParams cp{};
  cp.y = w.y;
  cp.y_bytes = w.h_rows * (int64_t)H * (dt == kF32 ? 4 : 2);
  cp.row_of = w.row_of;
  cp.weights = topk_weights;
  cp.top_k = K;
  cp.hidden = H;
  cp.shared_row0 = a->S ? (int32_t)nmax : -1;
  cp.shared_parts = a->S;
  cp.shared_stride = T;
  cp.out = (uint8_t*)out;
  QuantParams qp{};  // W8A8: h -> int8 codes with one scale per row, for the down GEMM
  qp.h = w.h;
  qp.pamax = w.pamax;
  qp.ld = (int32_t)w.h_rows;
  qp.inter = I;
  qp.offsets = w.offsets;
  qp.num_experts = E;
  qp.routed_max = (int32_t)n_flat;
  qp.shared_row0 = a->S ? (int32_t)nmax : -1;
  qp.shared_rows = a->S * T;  // every part's rows, one after another
  qp.h8 = (int8_t*)w.h8;
  qp.hsc = w.h_scales;

  if (dt == kF32) {
    F32Params g{};
    g.mtiles = w.mtiles;
    g.num_mtiles = w.num_mtiles;
    g.sorted_assign = w.sorted_assign;
    g.top_k = K;
    g.shared_row0 = (int32_t)nmax;
    g.shared_tokens = T;
    g.gather = 1;
    g.a = (const float*)hidden;
    g.w0 = (const float*)a->w->gu;
    g.w1 = (const float*)a->w->up;
    g.kdim = H;
    g.ndim = I;
    g.c = (float*)w.h;
    int grid = (int)std::min<int64_t>(mt_bound * (I / 16), (int64_t)cus * occupancy_wgs);
    AFD_HIP(launch_gemm_f32(true, g, grid, s));
    if ((st = mark(3))) return st;
    g.gather = 0;
    g.a = (const float*)w.h;
    g.w0 = (const float*)a->w->dn;
    g.w1 = nullptr;
    g.kdim = I;
    g.ndim = H;
    g.c = (float*)w.y;
    grid = (int)std::min<int64_t>(mt_bound * (H / 16), (int64_t)cus * occupancy_wgs);
    AFD_HIP(launch_gemm_f32(false, g, grid, s));
    if ((st = mark(4))) return st;
  } else {
    const int es = esize_of(dt);
    GemmParams g{};
    g.mtiles = w.mtiles;
    g.num_mtiles = w.num_mtiles;
    g.sorted_assign = w.sorted_assign;
    g.top_k = K;
    g.shared_row0 = (int32_t)nmax;
    g.shared_tokens = T;
    // gate/up: A = hidden rows gathered by token
    g.gather = 1;
    g.a = (const uint8_t*)hidden;
    g.a_bytes = (int64_t)T * H * es;
    g.a_row_bytes = (int64_t)H * es;
    g.a_scales = w.x_scales;  // gathered by gather_scales_kernel
    g.a_scale_bytes = fp8 ? (int64_t)(w8 ? 1 : H / 128) * w.h_rows * 4 : 0;
    g.a_scale_ld = (int32_t)w.h_rows;
    g.b = a->w->gu;
    g.b_expert_bytes = a->w->gu_expert_bytes;
    g.b_panel_bytes = a->w->gu_panel_bytes;
    g.b_scales0 = a->w->sg;
    g.b_scale_bytes = a->w->scale_bytes;
    g.b_scales1 = a->w->su;
    g.b_scale_rows = H / 128;
    g.b_scale_cols = w8 ? I : I / 128;  // W8A8: per output channel
    g.k_steps = (int32_t)((int64_t)H * es / kStepBytes);
    g.n_panels = I / 32;
    g.n_groups = I / 128;
    g.c = w.h;
    g.c_row_bytes = rows_ld_h;
    g.c_scales = w8 ? w.pamax : w.h_scales;  // W8A8: each row's amax per task, for quant.hip
    g.c_scale_ld = (int32_t)w.h_rows;
    g.pool = dt != kF32 ? w.pool : nullptr;  // the ring GEMMs' and the bf16 heavy tiles' tail pools
    g.mtiles3 = tiled8 ? w.mtiles_tiled : nullptr;  // block-FP8: the tiled list, run first
    g.num_mtiles3 = w.num_mtiles + 4;
    GemmParams gu_light = g;
    GemmParams gu_heavy = g;
    gu_heavy.mtiles = w.mtiles_heavy;
    gu_heavy.num_mtiles = w.num_mtiles + 1;
    gu_heavy.n_groups = (2 * I / 32 + tiled_panels() - 1) / tiled_panels();  // bf16 only
    // down: A = h rows in sorted order (W8A8: their int8 codes)
    g.gather = 0;
    g.a = w8 ? w.h8 : w.h;
    g.a_bytes = h_rows * (w8 ? I : rows_ld_h);
    g.a_row_bytes = w8 ? I : rows_ld_h;
    g.a_scales = w.h_scales;
    g.a_scale_bytes = fp8 ? h_rows * (w8 ? 1 : I / 128) * 4 : 0;
    g.a_scale_ld = (int32_t)w.h_rows;
    g.b = a->w->dn;
    g.b_expert_bytes = a->w->dn_expert_bytes;
    g.b_panel_bytes = a->w->dn_panel_bytes;
    g.b_scales0 = a->w->sd;
    g.b_scales1 = a->w->sd;
    g.b_scale_bytes = a->w->dn_scale_bytes;
    g.b_scale_rows = I / 128;
    g.b_scale_cols = w8 ? H : H / 128;
    g.k_steps = (int32_t)((int64_t)I * es / kStepBytes);
    g.n_panels = H / 32;
    // light tasks of the down GEMM: down_panels_per_task(mr) H panels (bf16
    // streaming GEMM) or 8 (block-FP8 ring GEMM, both lists)
    const int dn_panels = fp8 ? 8 : down_panels_per_task(mr);
    g.n_groups = (H / 32 + dn_panels - 1) / dn_panels;
    g.c = w.y;
    g.c_row_bytes = (int64_t)H * 2;
    g.c_scales = nullptr;
    g.c_scale_ld = 0;
    GemmParams dn_light = g;
    GemmParams dn_heavy = g;
    dn_heavy.mtiles = w.mtiles_heavy;
    dn_heavy.num_mtiles = w.num_mtiles + 1;
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
        if (tiled8) {
          const hipError_t e = launch_gemm_tiled8(gate_up, w8, both, mtt_bound * light.n_groups, cus, s);
          if (e != hipSuccess) return e;
        }
        return launch_gemm_ring(gate_up, a->concurrency == 1, w8, both, (mt_bound + mth_bound) * light.n_groups,
                                cus, s);
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
    if (use_fused) {
      // one launch: dispatch, both GEMM stages (and the W8A8 re-quantisation)
      // and the combine, timed as the gate/up stage
      FusedParams fp{};
      fp.d = d;
      fp.x_src = hidden_scales;
      fp.ks = w8 ? 1 : H / 128;
      fp.x_dst = w.x_scales;
      fp.ld = (int32_t)w.h_rows;
      fp.tokens = T;
      fp.top_k = K;
      fp.gu = gu_light;
      fp.gu.mtiles2 = gu_heavy.mtiles;
      fp.gu.num_mtiles2 = gu_heavy.num_mtiles;
      fp.dn = dn_light;
      fp.dn.mtiles2 = dn_heavy.mtiles;
      fp.dn.num_mtiles2 = dn_heavy.num_mtiles;
      fp.qp = qp;
      fp.cp = cp;
      fp.bar = w.bar;
      fp.chunk_counts = w.chunk_counts;
      fp.chunk_bad = w.chunk_bad;
      fp.local_base = w.local_base;
      fp.totals = w.totals;
      fp.spin_limit = 1 << 20;
      if (fp8) {
        AFD_HIP(launch_fused(a->concurrency == 1, w8, fp, std::min(cus, w.fused_grid), s));
      } else {
        // bf16: the mixed GEMM's parameters (the light list in gu / dn) and,
        // where the dispatch chooses, the light-only ones
        fp.gu = gu_light;
        fp.dn = dn_light;
        fp.gu_heavy = gu_heavy;
        fp.dn_heavy = dn_heavy;
        fp.gu_lo = gu_light;
        fp.dn_lo = dn_light;
        fp.dn_lo.n_groups = (H / 32 + down_panels_per_task(mr_lo) - 1) / down_panels_per_task(mr_lo);
        fp.auto_launch = auto_launch ? 1 : 0;
        AFD_HIP(launch_fused_bf16(auto_launch ? mr_lo : mr, mr, fp, std::min(cus, w.fused_grid), s));
      }
      for (int b = 3; b <= AFD_NUM_STAGES; ++b)
        if ((st = mark(b))) return st;
      if (tmask) a->ev_pending.push_back(ev);
      return AFD_OK;
    }
    AFD_HIP(stage(true, gu_light, gu_heavy));
    if (w8) AFD_HIP(launch_quant_rows(qp, s));
    if ((st = mark(3))) return st;
    AFD_HIP(stage(false, dn_light, dn_heavy));
    if ((st = mark(4))) return st;
  }

  AFD_HIP(launch_combine(dt == kF32 ? kF32 : kBF16, cp, T, s));
  if ((st = mark(5))) return st;
  if (tmask) a->ev_pending.push_back(ev);
  return AFD_OK;
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
  a->S = (cfg->shared_inter + cfg->inter - 1) / cfg->inter;  // the shared expert's parts of width I
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
  a->fused = src->fused;
  a->guard = src->guard;
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
  afd_status st = check_forward_args(a, T, a ? a->Tmax : 0, hidden, hidden_scales, topk_ids, topk_weights, out);
  if (st) return st;
  st = forward_impl(a, a->ws, true, true, T, hidden, hidden_scales, topk_ids, topk_weights, out, stream);
  if (st == AFD_OK) a->last_T = T;
  return st;
}

afd_status afd_ffn_forward_noalloc(afd_ffn_t* a, int32_t T, const void* hidden, const float* hidden_scales,
                                   const int32_t* topk_ids, const float* topk_weights, void* out, void* stream) {
  g_last_error.clear();
  afd_status st = check_forward_args(a, T, 0x7fffffff, hidden, hidden_scales, topk_ids, topk_weights, out);
  if (st) return st;
  const int64_t need = layout_workspace(a, T, nullptr, nullptr);
  if (need > (int64_t)AFD_FFN_NOALLOC_SCRATCH_BYTES)
    return fail(AFD_ERR_UNSUPPORTED, "a forward of %d tokens needs %lld bytes of workspace; the static scratch holds %lld",
                T, (long long)need, (long long)AFD_FFN_NOALLOC_SCRATCH_BYTES);
  DeviceGuard dg(a->device);
  if (!dg.ok) return fail(AFD_ERR_HIP, "cannot select device %d", a->device);
  uint8_t* base = nullptr;
  if ((st = scratch_address(a->device, &base))) return st;
  Workspace w;
  layout_workspace(a, T, base, &w);
  return forward_impl(a, w, false, false, T, hidden, hidden_scales, topk_ids, topk_weights, out, stream);
}

afd_status afd_ffn_debug_dispatch(afd_ffn_t* a, int32_t* counts, int32_t* offsets, int32_t* sorted_assign,
                                  int32_t* row_of, void* stream) {
  g_last_error.clear();
  if (!a) return fail(AFD_ERR_INVALID_ARG, "handle is NULL");
  DeviceGuard dg(a->device);
  hipStream_t s = (hipStream_t)stream;
  const int64_t n = (int64_t)a->last_T * a->K;
  const Workspace& w = a->ws;
  if (counts) AFD_HIP(hipMemcpyAsync(counts, w.counts, 4ll * a->E, hipMemcpyDeviceToDevice, s));
  if (offsets) AFD_HIP(hipMemcpyAsync(offsets, w.offsets, 4ll * (a->E + 1), hipMemcpyDeviceToDevice, s));
  if (sorted_assign && n) AFD_HIP(hipMemcpyAsync(sorted_assign, w.sorted_assign, 4 * n, hipMemcpyDeviceToDevice, s));
  if (row_of && n) AFD_HIP(hipMemcpyAsync(row_of, w.row_of, 4 * n, hipMemcpyDeviceToDevice, s));
  return AFD_OK;
}

afd_status afd_ffn_routing_errors(afd_ffn_t* a, int32_t* count, void* stream) {
  g_last_error.clear();
  if (!a || !count) return fail(AFD_ERR_INVALID_ARG, "NULL argument");
  DeviceGuard dg(a->device);
  hipStream_t s = (hipStream_t)stream;
  AFD_HIP(hipMemcpyAsync(count, a->ws.err, 4, hipMemcpyDeviceToHost, s));
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

afd_status afd_ffn_set_canaries(afd_ffn_t* a, int64_t guard_bytes) {
  g_last_error.clear();
  if (!a) return fail(AFD_ERR_INVALID_ARG, "handle is NULL");
  if (guard_bytes < 0 || guard_bytes > kMaxGuardBytes || guard_bytes % 256)
    return fail(AFD_ERR_INVALID_ARG, "guard_bytes %lld: a multiple of 256 in [0, %lld]", (long long)guard_bytes,
                (long long)kMaxGuardBytes);
  DeviceGuard dg(a->device);
  if (!dg.ok) return fail(AFD_ERR_HIP, "cannot select device %d", a->device);
  AFD_HIP(hipDeviceSynchronize());  // no forward of the handle may still use the old workspace
  uint8_t* old_mem = a->ws_mem;
  const Workspace old_ws = a->ws;
  const int64_t old_guard = a->guard;
  std::vector<GuardBand> old_bands = a->bands;
  a->guard = guard_bytes;
  a->ws_mem = nullptr;
  afd_status st = alloc_workspace(a);
  if (st) {  // keep the old workspace
    if (a->ws_mem) (void)hipFree(a->ws_mem);
    a->ws_mem = old_mem;
    a->ws = old_ws;
    a->guard = old_guard;
    a->bands = old_bands;
    return st;
  }
  AFD_HIP(hipFree(old_mem));
  a->last_T = 0;
  return AFD_OK;
}

afd_status afd_ffn_check_canaries(afd_ffn_t* a, int64_t* damaged_bytes, void* stream) {
  g_last_error.clear();
  if (!a || !damaged_bytes) return fail(AFD_ERR_INVALID_ARG, "NULL argument");
  *damaged_bytes = 0;
  if (a->guard <= 0) return fail(AFD_ERR_INVALID_ARG, "the handle has no canaries (afd_ffn_set_canaries)");
  DeviceGuard dg(a->device);
  if (!dg.ok) return fail(AFD_ERR_HIP, "cannot select device %d", a->device);
  AFD_HIP(hipStreamSynchronize((hipStream_t)stream));
  std::vector<uint8_t> host(a->guard);
  std::string where;
  int64_t bad = 0;
  for (const GuardBand& b : a->bands) {
    AFD_HIP(hipMemcpy(host.data(), a->ws_mem + b.off, a->guard, hipMemcpyDeviceToHost));
    int64_t n = 0, first = -1;
    for (int64_t i = 0; i < a->guard; ++i)
      if (host[i] != kCanaryByte) {
        if (first < 0) first = i;
        ++n;
      }
    if (n) {
      char buf[128];
      snprintf(buf, sizeof buf, "%s%lld bytes after %s (first at +%lld)", where.empty() ? "" : "; ", (long long)n,
               b.after, (long long)first);
      where += buf;
    }
    bad += n;
  }
  *damaged_bytes = bad;
  return bad ? fail(AFD_ERR_HIP, "canaries overwritten: %s", where.c_str()) : AFD_OK;
}

afd_status afd_ffn_debug_poke_canary(afd_ffn_t* a, int32_t band, int64_t offset) {
  g_last_error.clear();
  if (!a) return fail(AFD_ERR_INVALID_ARG, "handle is NULL");
  if (a->guard <= 0) return fail(AFD_ERR_INVALID_ARG, "the handle has no canaries (afd_ffn_set_canaries)");
  if (band < 0 || band >= (int32_t)a->bands.size() || offset < 0 || offset >= a->guard)
    return fail(AFD_ERR_INVALID_ARG, "band %d, offset %lld outside %d bands of %lld bytes", band, (long long)offset,
                (int)a->bands.size(), (long long)a->guard);
  DeviceGuard dg(a->device);
  if (!dg.ok) return fail(AFD_ERR_HIP, "cannot select device %d", a->device);
  AFD_HIP(hipDeviceSynchronize());
  AFD_HIP(hipMemset(a->ws_mem + a->bands[band].off + offset, (int)(uint8_t)~kCanaryByte, 1));
  AFD_HIP(hipDeviceSynchronize());
  return AFD_OK;
}

afd_status afd_ffn_mfma_peak(int32_t dtype, int32_t device, int32_t iters, double* tflops, double* clock_ghz) {
  g_last_error.clear();
  if (!tflops || !clock_ghz || iters <= 0) return fail(AFD_ERR_INVALID_ARG, "NULL output or iters <= 0");
  const int kind = dtype == kBF16 ? 0 : dtype == kFP8 ? 1 : dtype == kW8A8 ? 2 : -1;
  if (kind < 0) return fail(AFD_ERR_UNSUPPORTED, "dtype %d has no MFMA peak measurement", dtype);
  DeviceGuard dg(device);
  if (!dg.ok) return fail(AFD_ERR_HIP, "cannot select device %d", device);
  int cus = 0;
  AFD_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device));
  AFD_HIP(mfma_peak(kind, cus, iters, tflops, clock_ghz));
  return AFD_OK;
}

afd_status afd_ffn_mfma_lds_peak(int32_t device, int32_t iters, int32_t lds_reads, double* tflops, double* clock_ghz) {
  g_last_error.clear();
  if (!tflops || !clock_ghz || iters < 3) return fail(AFD_ERR_INVALID_ARG, "NULL output or iters < 3");
  if (lds_reads != 0 && lds_reads != 6) return fail(AFD_ERR_INVALID_ARG, "lds_reads must be 0 or 6, not %d", lds_reads);
  DeviceGuard dg(device);
  if (!dg.ok) return fail(AFD_ERR_HIP, "cannot select device %d", device);
  int cus = 0;
  AFD_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device));
  AFD_HIP(mfma_peak(lds_reads ? 4 : 3, cus, iters, tflops, clock_ghz));
  return AFD_OK;
}

afd_status afd_ffn_set_fused(afd_ffn_t* a, int32_t enable) {
  g_last_error.clear();
  if (!a) return fail(AFD_ERR_INVALID_ARG, "handle is NULL");
  if (enable != 0 && enable != 1) return fail(AFD_ERR_INVALID_ARG, "enable must be 0 or 1, not %d", enable);
  if (enable && a->dtype == kF32)
    return fail(AFD_ERR_UNSUPPORTED, "the fused launch serves bf16, block-FP8 and W8A8 layers");
  a->fused = enable;
  return AFD_OK;
}

afd_status afd_ffn_fused_errors(afd_ffn_t* a, int32_t* count, void* stream) {
  g_last_error.clear();
  if (!a || !count) return fail(AFD_ERR_INVALID_ARG, "NULL argument");
  *count = 0;
  if (!a->ws.bar) return AFD_OK;
  DeviceGuard dg(a->device);
  hipStream_t s = (hipStream_t)stream;
  AFD_HIP(hipMemcpyAsync(count, a->ws.bar + 2, 4, hipMemcpyDeviceToHost, s));
  AFD_HIP(hipStreamSynchronize(s));
  if (*count) AFD_HIP(hipMemsetAsync(a->ws.bar + 2, 0, 4, s));
  return *count > 0 ? fail(AFD_ERR_HIP, "%d grid-barrier waits of fused forwards timed out", *count) : AFD_OK;
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
