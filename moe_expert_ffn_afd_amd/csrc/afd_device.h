// afd_device.h -- device helpers shared by the GEMM kernels (gfx950).
#pragma once

#include "afd_internal.h"

namespace afd {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline i32x8 cat32(uint4 a, uint4 b) {
  i32x8 r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
}

__device__ inline i32x8 cat32v(i32x4 a, i32x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)a);
  uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)b);
  return lo | (hi << 16);
}

// 4 floats -> 4 e4m3 codes (round to nearest even; inputs already within +-448)
__device__ inline uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// A 16-byte store; NT: non-temporal (the expert outputs y of the streaming
// and ring GEMMs, read once by the combine much later: their down launches
// ran 2-3 % faster with it).
template <bool NT = false>
__device__ inline void store16(uint8_t* dst, uint4 v) {
  if (NT) {
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4v*>(dst));
  } else {
    *reinterpret_cast<uint4*>(dst) = v;
  }
}

// 32x32 MFMA output rows: lane l holds 4 columns of a row for each of two
// r4 values (columns 8 r4 + 4 (l >> 5) + 0..3, lo = the even r4, hi_v = the
// odd one).  Lanes l and l ^ 32 swap halves so each stores 8 consecutive
// columns (16 bytes) at dst: the lower lane columns 16 r2 + 0..7, the upper
// lane 16 r2 + 8..15.  Both lanes of a pair must be active.
template <bool NT = false>
__device__ inline void store_pair16(uint8_t* dst, uint2 lo, uint2 hi_v, bool upper) {
  const uint2 snd = upper ? lo : hi_v;
  uint2 rcv;
  rcv.x = __shfl_xor(snd.x, 32, 64);
  rcv.y = __shfl_xor(snd.y, 32, 64);
  store16<NT>(dst, upper ? make_uint4(rcv.x, rcv.y, hi_v.x, hi_v.y) : make_uint4(lo.x, lo.y, rcv.x, rcv.y));
}

// 16x16 MFMA outputs of the down GEMMs (ring and tiled 8-bit): lane l =
// tok + 16 kg holds 4 columns of each 16-column half of a 32-column panel for
// token tok (o0: columns 4 kg + 0..3, o1: 16 + 4 kg + 0..3).  Lane pairs
// (kg, kg ^ 1) swap one half each, so every lane holds 8 consecutive bf16
// columns (16 bytes); lanes kg = 0, 2, 1, 3 hold the panel's parts 0 .. 3.
// Both lanes of a pair must be active.
__device__ inline uint4 pair16_cols(uint2 o0, uint2 o1, int kg) {
  const bool odd = (kg & 1) != 0;
  const uint2 snd = odd ? o0 : o1;
  uint2 rcv;
  rcv.x = __shfl_xor(snd.x, 16, 64);
  rcv.y = __shfl_xor(snd.y, 16, 64);
  return odd ? make_uint4(rcv.x, rcv.y, o1.x, o1.y) : make_uint4(o0.x, o0.y, rcv.x, rcv.y);
}

// Stores one 16-token tile's outputs of panels P and P + 1 (P even: one
// 128-byte line of each row) as whole lines.  a, b: this lane's 16 bytes of
// panel P and P + 1, as pair16_cols leaves them.  Tokens tok and tok ^ 8
// swap their b (a DPP rotation by 8 within each 16-lane row), so store h
// covers the 8 tokens 8h .. 8h + 7 whole, each lane writing its own a or the
// swapped-in b.  Half-line stores (one panel of 16 tokens each) leave every
// line's other half to another store, and with non-temporal stores the down
// launches wrote about 1.45x the bytes of y back.  Token t of the tile is
// output row row0 + mb + t at c + row * row_bytes; rows mb + t >= rows and
// panels >= n_panels are not stored.  Every lane calls it.
template <bool NT>
__device__ inline void store_line_pair(uint8_t* c, int64_t row_bytes, int n_panels, int row0, int rows, int mb, int P,
                                       uint4 a, uint4 b, int tok, int kg) {
  const uint4 bx = make_uint4((uint32_t)__builtin_amdgcn_update_dpp(0, (int)b.x, 0x128, 0xf, 0xf, false),
                              (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b.y, 0x128, 0xf, 0xf, false),
                              (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b.z, 0x128, 0xf, 0xf, false),
                              (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b.w, 0x128, 0xf, 0xf, false));
  const int part = ((kg & 1) << 1) | (kg >> 1);  // this lane's 16-byte part of a panel
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bool own = (tok >> 3) == h;
    const int m = mb + (own ? tok : tok ^ 8);
    const int pn = own ? P : P + 1;
    if (m < rows && pn < n_panels) store16<NT>(c + (int64_t)(row0 + m) * row_bytes + (int64_t)(32 * pn + 8 * part) * 2, own ? a : bx);
  }
}

// Four 16-byte LDS reads at the given byte addresses, waited for inside the
// same asm block (the outputs are complete when it ends).  For reads the
// compiler must not order against in-flight copies into LDS.
__device__ inline void lds_read4x16(i32x4 (&d)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

// m-tile mt of a device-built tile list.  The lists are not written by the
// GEMM kernels, so the read goes through the constant address space and
// becomes a scalar load (a vector load would need a wait of its own in the
// middle of a load pipeline).
__device__ inline int4 load_tile(const int4* tiles, int mt) {
  typedef const __attribute__((address_space(4))) int* cptr;
  const cptr c = (cptr)(const void*)tiles;
  const int i = 4 * uniform(mt);
  return make_int4(c[i], c[i + 1], c[i + 2], c[i + 3]);
}

// Raw buffer resource: stride 0, byte-addressed; reads at offsets >= the
// record count return zero without touching memory.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

template <int AUX = 0>
__device__ inline uint4 bload16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}

// Buffer loads straight into LDS: lane i's 16 (or 4) bytes land at
// lds + 16 i (or 4 i); the LDS base must be wave-uniform.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, soff, 0, 0);
}
__device__ inline void dma16_nt(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, soff, 0, 2);
}
template <int AUX>
__device__ inline void dma16_aux(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, soff, 0, AUX);
}
__device__ inline void dma4(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 4, voff, soff, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until this wave's LDS reads have returned (lgkmcnt(0); vmcnt and
// expcnt left at their no-wait maxima): a slot may be refilled by another
// wave's copy once every wave has passed the next barrier.
__device__ inline void lds_reads_done() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Workgroup barrier without the memory-model fence __syncthreads adds (which
// would wait for every in-flight load); the empty asm keeps the compiler from
// moving memory operations across it.
__device__ inline void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroups of the mixed bf16 GEMM launch (cus of them) that take the light
// list: in proportion to the light list's share of the cost, a multiple of 8
// where cus is (the same number on every XCD), at least one for a nonempty
// list of either kind when cus allows two.
__device__ inline int mixed_light_workgroups(int cus, int nl, int nh) {
  if (cus <= 0 || nl == 0) return 0;
  if (nh == 0) return cus;
  if (cus < 2) return 0;  // one workgroup runs both lists, heavy first
  const float share = (float)nl / ((float)nl + kHeavyTileCost * (float)nh);
  int l = (int)(share * (float)cus + 0.5f);
  if (cus % kXcds == 0 && cus >= 2 * kXcds) {
    l = (l + kXcds / 2) / kXcds * kXcds;
    return min(max(l, kXcds), cus - kXcds);
  }
  return min(max(l, 1), cus - 1);
}

}  // namespace dev
}  // namespace afd
