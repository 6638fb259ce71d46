// Batch-invariant RMSNorm for gfx950.
//
// The inference-research gotcha "batch-invariance-is-not-universal-across-
// kernel-paths" (section "Root cause") lists small-batch split reductions in
// RMSNorm among the strategies that make a row's result depend on how many
// rows share the call.  Here every row is reduced by exactly one workgroup,
// with one fixed summation order, whatever the number of rows:
//   * thread t of the 256 owns the 8-element vectors t, t + 256, ... of the
//     row; it loads them once (16-byte loads, kept in registers) and sums
//     their squares in fp32, vector by vector and element by element;
//   * a wave-wide xor butterfly (every lane ends with the same bits) and
//     then the four wave sums in wave order give the row's sum of squares;
//   * r = 1 / sqrt(sum / dim + eps) (correctly rounded fp32 square root and
//     division), y = (x * r) * w, rounded to bf16 to nearest even.
// A row's output bits therefore depend only on the row, its weight and eps.

#include "device.hpp"
#include "isk_internal.hpp"

namespace isk {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxVecs = kRmsNormMaxDim / 8 / kThreads;   // 16-byte vectors per thread at most

__global__ void __launch_bounds__(kThreads) rmsnorm_kernel(RmsNormLaunch a) {
  const int row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nvec = a.dim / 8;
  const uint4* xr = (const uint4*)(a.x + (size_t)row * a.dim);
  const uint4* wr = (const uint4*)a.w;
  __shared__ float wsum[kThreads / 64];

  uint4 xv[kMaxVecs];
#pragma unroll
  for (int k = 0; k < kMaxVecs; ++k) {
    const int v = t + k * kThreads;
    xv[k] = v < nvec ? xr[v] : uint4{0u, 0u, 0u, 0u};
  }
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxVecs; ++k) {
    const uint32_t e[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_lo(e[j]), hi = bf16_hi(e[j]);
      acc = fmaf(lo, lo, acc);
      acc = fmaf(hi, hi, acc);
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  float total = wsum[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) total += wsum[w];
  const float r = 1.0f / sqrtf(total / (float)a.dim + a.eps);

  uint4* yr = (uint4*)(a.y + (size_t)row * a.dim);
#pragma unroll
  for (int k = 0; k < kMaxVecs; ++k) {
    const int v = t + k * kThreads;
    if (v < nvec) {
      const uint4 wv = wr[v];
      const uint32_t e[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
      const uint32_t g[4] = {wv.x, wv.y, wv.z, wv.w};
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = pack_bf16x2((bf16_lo(e[j]) * r) * bf16_lo(g[j]), (bf16_hi(e[j]) * r) * bf16_hi(g[j]));
      yr[v] = uint4{o[0], o[1], o[2], o[3]};
    }
  }
}

}  // namespace

hipError_t launch_rmsnorm(const RmsNormLaunch& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(a.rows), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace isk
