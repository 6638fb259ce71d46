// Streaming-read and row-gather microbenchmarks (gfx950): the achievable HBM
// read rates of this part for the decode paths' two access patterns, the
// second roofline denominators next to the 8 TB/s published figure.
//
// Every thread reads 16-byte pieces of the buffer in a grid-stride loop
// (piece (block x 256 + thread) + k x (grid x 256)), four loads in flight per
// iteration, and folds them with XOR so that no load can be dropped; each
// workgroup writes one word of the fold, so the XOR of all the words is the
// XOR of every 32-bit word of the buffer.  Each load instruction of a wave
// covers 1 KiB of contiguous memory and each pass of the grid one contiguous
// stretch; the caller sizes the grid to cover every compute unit several
// times.

#include "device.hpp"
#include "isk_internal.hpp"

namespace isk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

__global__ void __launch_bounds__(kProbeThreads) hbm_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                 uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  // Full rounds of kProbeUnroll strided loads.
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d, 64);
  __shared__ uint32_t wsum[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = wsum[0] ^ wsum[1] ^ wsum[2] ^ wsum[3];
}

// Row gather: rows[r] names a row of `row_bytes` bytes in src (a multiple of
// 16); piece j of the flattened list is piece j % P of row rows[j / P], P =
// row_bytes / 16, read in the same grid-stride order, so each load
// instruction of a wave covers 1 KiB of consecutive pieces (one or two rows).
// This is the access pattern of a sparse top-k tile load.
__global__ void __launch_bounds__(kProbeThreads) hbm_gather_kernel(const unsigned char* __restrict__ src,
                                                                   const int32_t* __restrict__ rows, size_t n16,
                                                                   uint32_t pieces, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  auto at = [&](size_t j) {
    const uint32_t r = (uint32_t)(j / pieces), c = (uint32_t)(j - (size_t)r * pieces);
    return (const u32x4*)(src + ((size_t)(uint32_t)rows[r] * pieces + c) * 16);
  };
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    const u32x4* a[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) a[u] = at(i + u * stride);
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(a[u]);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(at(i));
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d, 64);
  __shared__ uint32_t wsum[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = wsum[0] ^ wsum[1] ^ wsum[2] ^ wsum[3];
}

}  // namespace

hipError_t launch_hbm_gather(const void* src, const int32_t* rows, int n_rows, int row_bytes, uint32_t* sink,
                             int blocks, hipStream_t s) {
  const uint32_t pieces = (uint32_t)row_bytes / 16;
  hipLaunchKernelGGL(hbm_gather_kernel, dim3(blocks), dim3(kProbeThreads), 0, s, (const unsigned char*)src, rows,
                     (size_t)n_rows * pieces, pieces, sink);
  return hipGetLastError();
}

hipError_t launch_hbm_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(blocks), dim3(kProbeThreads), 0, s, (const u32x4*)src, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace isk
