// combine.h -- the top-k weighted combine of one token (combine.hip's kernel
// and the fused layer kernel run it).
//
// The FFN side returns, per token, the routing-weighted sum of its experts'
// outputs ("FastAFD" structured summary, System Design item 3: push-back of
// the MoE result; vLLM AFD blog, FFN service returns the computed output):
//   out[t] = sum_k w[t,k] * y[row_of[t,k]]   (k in order, slots with row -1
//            skipped)  + sum_v y[shared_row0 + v T + t]  (the shared expert's
//            parts, weight 1)
// accumulated in fp32 in a fixed order, so the result does not depend on
// scheduling.  The token's rows are compacted first (dropped slots cost
// nothing), then read with 16-byte coalesced loads, up to 8 rows in flight per
// thread before the ordered sums.
#pragma once

#include "afd_device.h"

namespace afd {

// Token t of the combine by a group of `nthr` threads (a multiple of 64; this
// thread is number `tid` of it) with its own LDS lists rows[kMaxRowsPerToken],
// ws[kMaxRowsPerToken] and nrows[1].  Every thread of the workgroup calls it the
// same number of times (it holds two workgroup barriers); a thread whose group
// has no token this round passes active = false.  Ends with every thread past
// the reads of its group's lists.
template <int DT>
__device__ __forceinline__ void combine_rows(const CombineParams& p, const int t, const bool active, const int tid,
                                             const int nthr, int* rows, float* ws, int* nrows) {
  // the token's rows to add, in order: routed slots with a row (k order), then
  // the shared expert's row; compacted so dropped slots cost nothing
  if (active && tid < 64) {
    const int r = tid < p.top_k ? p.row_of[(int64_t)t * p.top_k + tid] : -1;
    const bool valid = r >= 0;
    const uint64_t mask = __ballot(valid);
    const int pos = __popcll(mask & ((1ull << tid) - 1));
    if (valid) {
      rows[pos] = r;
      ws[pos] = p.weights[(int64_t)t * p.top_k + tid];
    }
    const int n = __popcll(mask);
    if (tid == 0) {
      const int parts = p.shared_row0 >= 0 ? p.shared_parts : 0;
      for (int v = 0; v < parts; ++v) {  // the shared expert's parts, in order
        rows[n + v] = p.shared_row0 + v * p.shared_stride + t;
        ws[n + v] = 1.0f;
      }
      *nrows = n + parts;
    }
  }
  __syncthreads();
  constexpr int kVec = DT == kF32 ? 4 : 8;  // elements per 16-byte vector
  constexpr int kEsz = DT == kF32 ? 4 : 2;
  constexpr int kBatch = 8;                 // row loads in flight per thread
  const int nvec = p.hidden / kVec;
  const int row_bytes = p.hidden * kEsz;
  const auto ry = dev::make_rsrc(p.y, p.y_bytes);
  const int nr = active ? dev::uniform(*nrows) : 0;
  for (int v = tid; active && v < nvec; v += nthr) {
    float acc[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) acc[i] = 0.0f;
    for (int k0 = 0; k0 < nr; k0 += kBatch) {
      // the batch's loads first, then the sums in order (the row is the same
      // for the whole workgroup: scalar offset; the lane's 16 bytes: vector)
      uint4 d[kBatch];
#pragma unroll
      for (int kk = 0; kk < kBatch; ++kk)
        if (k0 + kk < nr) d[kk] = dev::bload16(ry, v * 16, dev::uniform(rows[k0 + kk]) * row_bytes);
#pragma unroll
      for (int kk = 0; kk < kBatch; ++kk) {
        if (k0 + kk >= nr) break;
        const float w = ws[k0 + kk];
        if (DT == kF32) {
          const float f[4] = {__uint_as_float(d[kk].x), __uint_as_float(d[kk].y), __uint_as_float(d[kk].z),
                              __uint_as_float(d[kk].w)};
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] += w * f[i];
        } else {
          const uint32_t u[4] = {d[kk].x, d[kk].y, d[kk].z, d[kk].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += w * __uint_as_float(u[i] << 16);
            acc[2 * i + 1] += w * __uint_as_float(u[i] & 0xffff0000u);
          }
        }
      }
    }
    uint8_t* o = p.out + ((int64_t)t * p.hidden + (int64_t)v * kVec) * kEsz;
    if (DT == kF32) {
      *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    } else {
      uint4 d;
      uint32_t* u = reinterpret_cast<uint32_t*>(&d);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)acc[2 * i]);
        uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)acc[2 * i + 1]);
        u[i] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(o) = d;
    }
  }
  __syncthreads();  // rows[] and ws[] are rewritten by the next token
}

}  // namespace afd
