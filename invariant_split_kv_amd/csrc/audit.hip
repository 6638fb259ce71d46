// Value-range audit of the latent cache (desc.check_inputs, 128-head MLA).
//
// The 128-head MLA kernels take V (the first 512 latent dims) into their PV
// product as fp16: bf16 values of magnitude up to 65280 and down to 2^-14
// convert exactly, smaller ones become fp16 subnormals (absolute error below
// 2^-24) and larger ones (65536 and up, infinities, NaN) do not fit.  This
// kernel looks at every attended latent row of a batch -- positions [0, len)
// of dense rows, the first topk_len listed positions of sparse rows -- and
// records one row, position and dim whose V value is 65536 or more in
// magnitude (or not finite).  It runs only after the table audit has checked
// every page and position it reads.

#include "device.hpp"
#include "isk_internal.hpp"

namespace isk {
namespace {

constexpr int kAuditWaves = 4;
constexpr int kAuditBlocksPerRow = 32;

__global__ void __launch_bounds__(64 * kAuditWaves) v_range_kernel(VRangeAudit a) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kAuditWaves + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * kAuditWaves;
  const int len = min(max(a.lens[b], 0), a.max_pages * a.page_size);
  const int units = a.topk_idx != nullptr ? min(max(a.topk_len[b], 0), a.topk_width) : len;
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
  for (int u = wave; u < units; u += nwaves) {
    const int pos = a.topk_idx != nullptr ? a.topk_idx[(size_t)b * a.topk_width + u] : u;
    if (pos < 0 || pos >= len) continue;
    const int pg = bt[pos / a.page_size];
    if (pg < 0 || pg >= a.num_pages) continue;
    const size_t slot = (size_t)pg * a.page_size + pos % a.page_size;
    const uint4 x = *(const uint4*)(a.kv + slot * kMlaDqk + 8 * lane);   // dims 8 lane .. 8 lane + 7
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    int bad_dim = -1;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t h = (w[k >> 1] >> (16 * (k & 1))) & 0x7fffu;
      if (h >= 0x4780u && bad_dim < 0) bad_dim = 8 * lane + k;   // |v| >= 2^16, inf or NaN
    }
    if (bad_dim >= 0 && atomicCAS(&a.found[0], 0, 1) == 0) {
      a.found[1] = b;
      a.found[2] = pos;
      a.found[3] = bad_dim;
    }
  }
}

}  // namespace

hipError_t launch_v_range_audit(const VRangeAudit& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(v_range_kernel, dim3(kAuditBlocksPerRow, a.batch), dim3(64 * kAuditWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace isk
