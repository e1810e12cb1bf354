// quant.h -- W8A8 layers: the per-row int8 re-quantisation of h between the
// two grouped expert GEMMs (quant.hip's kernel and the fused layer kernel).
//
// In a W8A8 layer both expert GEMMs take 8-bit activations (vLLM AFD plugin
// blog, decode benchmark: DeepSeek-V3.2 in W8A8): the tokens arrive as int8
// with one scale per token, and h = silu(X Wg) * (X Wu) is brought to int8
// with one scale per row before h Wd.  The gate/up GEMM (gemm_ring.h) writes
// h in bf16 plus each row's amax over every 128-column task; a row's scale is
// amax / 127 over those (1 for an all-zero row), its codes
// round-half-even(h / scale) clamped to +-127.  One wave per row: coalesced
// 16-byte loads of 8 bf16, 8-byte stores of codes.
#pragma once

#include "afd_internal.h"

namespace afd {

// Row r of h, by one wave (lane = the thread's lane): amax over the row's
// task maxima, then the codes and the scale.
__device__ __forceinline__ void quant_row(const QuantParams& p, const int r, const int lane) {
  const int groups = p.inter / 128;
  float amax = 0.0f;
  for (int g = lane; g < groups; g += 64) amax = fmaxf(amax, p.pamax[(int64_t)g * p.ld + r]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
  const float scale = amax > 0.0f ? amax / 127.0f : 1.0f;
  const float inv = amax > 0.0f ? 127.0f / amax : 1.0f;
  const uint8_t* src = p.h + (int64_t)r * p.inter * 2;
  int8_t* dst = p.h8 + (int64_t)r * p.inter;
  for (int c = 8 * lane; c < p.inter; c += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t)c * 2);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t bits = (k & 1) ? (u[k >> 1] & 0xffff0000u) : (u[k >> 1] << 16);
      const float q = fminf(fmaxf(rintf(__uint_as_float(bits) * inv), -127.0f), 127.0f);
      o[k >> 2] |= ((uint32_t)(int)q & 0xffu) << (8 * (k & 3));
    }
    *reinterpret_cast<uint2*>(dst + c) = make_uint2(o[0], o[1]);
  }
  if (lane == 0) p.hsc[r] = scale;
}


}  // namespace afd
