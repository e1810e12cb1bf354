// pack.hip -- one-time re-layout of expert weights into the panel-major
// fragment order the grouped GEMMs stream (layout described in
// afd_internal.h).  Runs at handle creation only.
//
// One workgroup moves one super-step (128 bytes of K) of four adjacent
// 32-column panels of one matrix of one expert: it reads the [KS x 128]
// block of the row-major source (KS = 64 bf16 or 128 e4m3 rows, 16 KiB) with
// coalesced 16-byte loads into LDS, then writes the four 4 KiB panel steps,
// each thread assembling 16-byte lane operands from LDS columns.
#include "afd_internal.h"

namespace afd {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
                                                   int64_t in_expert_elems, int kdim, int ndim, int esize,
                                                   int gate_up, uint8_t* __restrict__ dst, int64_t dst_expert_bytes) {
  __shared__ uint4 tile[1024];  // [KS rows][128 * esize bytes]
  const int tid = threadIdx.x;
  const int n_groups = ndim / 128;
  const int c = blockIdx.x / n_groups;   // super-step
  const int pg = blockIdx.x % n_groups;  // group of 4 panels
  const int e = blockIdx.y;
  const int slot = blockIdx.z;           // gate/up: 0 gate, 1 up; down: 0
  const uint8_t* src = (slot == 0 ? w0 : w1) + (int64_t)e * in_expert_elems * esize;
  const int ks = kStepBytes / esize;     // rows of K in one super-step
  const int row_bytes = 128 * esize;     // 128 columns
  const int chunks_per_row = row_bytes / 16;
  uint8_t* lds = reinterpret_cast<uint8_t*>(tile);

  for (int ch = tid; ch < 1024; ch += 256) {
    const int r = ch / chunks_per_row;
    const int cb = (ch % chunks_per_row) * 16;
    const int64_t k = (int64_t)c * ks + r;
    tile[ch] = *reinterpret_cast<const uint4*>(src + (k * ndim + (int64_t)pg * 128) * esize + cb);
  }
  __syncthreads();

  const int64_t panel_bytes = (int64_t)kdim * 32 * esize;
  for (int ch = tid; ch < 1024; ch += 256) {
    const int pl = ch >> 8;         // panel within the group
    const int j = (ch >> 6) & 3;    // load index within the super-step
    const int l = ch & 63;          // lane
    const int g = l >> 5, n = 32 * pl + (l & 31);
    uint8_t bytes[16];
    for (int b = 0; b < 16; b += esize) {
      const int kb = 64 * g + 16 * j + b;  // byte offset of k within the super-step
      const int kl = kb / esize;           // k row within the block
      for (int x = 0; x < esize; ++x) bytes[b + x] = lds[kl * row_bytes + n * esize + x];
    }
    const int panel = 4 * pg + pl;
    const int64_t pidx = gate_up ? (2 * panel + slot) : panel;
    uint8_t* out = dst + (int64_t)e * dst_expert_bytes + pidx * panel_bytes + (int64_t)c * kStepPanelBytes +
                   j * 1024 + l * 16;
    uint4 v;
    __builtin_memcpy(&v, bytes, 16);
    *reinterpret_cast<uint4*>(out) = v;
  }
}

hipError_t launch_pack(int dtype, bool gate_up, const void* w_first, const void* w_second,
                       int64_t expert_in_stride_elems, int experts, int kdim, int ndim, uint8_t* dst,
                       int64_t dst_expert_bytes, hipStream_t s) {
  const int esize = dtype == kBF16 ? 2 : 1;
  const int steps = kdim * esize / kStepBytes;
  dim3 grid(steps * (ndim / 128), experts, gate_up ? 2 : 1);
  hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, s, (const uint8_t*)w_first,
                     (const uint8_t*)(gate_up ? w_second : w_first), expert_in_stride_elems, kdim, ndim, esize,
                     gate_up ? 1 : 0, dst, dst_expert_bytes);
  return hipGetLastError();
}

}  // namespace afd
