// Batch-invariant bf16 linear layer, y = x w^T with fp32 accumulation, for
// gfx950.
//
// The gllm issue "Greedy outputs depend on batch composition (NVFP4
// GEMV/GEMM switch at 32 rows is a candidate)" (section "Candidate cause")
// describes a matmul that picks its kernel by row count, and whose two
// kernels round the activations differently, so a row's result depends on
// how many rows share the call; its section "Next steps" proposes that both
// kernels use the same activation precision, so that the switch changes
// speed only.  This library's two tile shapes follow that rule and go
// further: they compute every output element with the same instructions.
//   * Rows <= 32 (decode-sized, weight-bandwidth bound): 16-row tiles.
//     Rows > 32: 64-row tiles, which reuse each weight fragment for four
//     row tiles.
//   * Both take bf16 activations.  The four waves of a workgroup each own a
//     quarter of K and run v_mfma_f32_16x16x32_bf16 over it in ascending k
//     from zero; the partial sums are added in wave order,
//     ((c0 + c1) + c2) + c3.  Rows of a tile past M contribute nothing to
//     other rows (their operand is zero and their outputs are not stored).
// An element's bits therefore depend only on its row of x, its row of w and
// K: never on M, on the other rows, or on which tile shape ran.

#include "device.hpp"
#include "isk_internal.hpp"

namespace isk {
namespace {

template <int TM>
__global__ void __launch_bounds__(256) linear_kernel(LinearLaunch a) {
  constexpr int T = TM / 16;   // 16-row MFMA tiles per workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g16 = lane >> 4;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * TM;
  const int kq = a.k / 4;      // K range of this wave: [wave * kq, (wave + 1) * kq)
  const size_t kb = (size_t)wave * kq + 8 * g16;

  // Operand fragments: lane (i16, g16) holds 8 consecutive k of one row.
  // A = x rows m0 + 16t + i16, B = w row n0 + i16 (the output column).
  const bf16x8* wp = (const bf16x8*)(a.w + (size_t)(n0 + i16) * a.k + kb);
  const bf16x8* xp[T];
  bool xok[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int m = m0 + 16 * t + i16;
    xok[t] = m < a.m;
    xp[t] = (const bf16x8*)(a.x + (size_t)(xok[t] ? m : 0) * a.k + kb);
  }
  const bf16x8 zero = {};
  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // k-steps of 32, the next step's fragments loaded before this step's MFMAs.
  const int steps = kq / 32;
  bf16x8 bcur = wp[0], acur[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acur[t] = xok[t] ? xp[t][0] : zero;
  for (int s = 0; s < steps; ++s) {
    bf16x8 bnext = bcur, anext[T];
#pragma unroll
    for (int t = 0; t < T; ++t) anext[t] = acur[t];
    if (s + 1 < steps) {
      bnext = wp[4 * (s + 1)];
#pragma unroll
      for (int t = 0; t < T; ++t) anext[t] = xok[t] ? xp[t][4 * (s + 1)] : zero;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(acur[t], bcur, acc[t], 0, 0, 0);
    bcur = bnext;
#pragma unroll
    for (int t = 0; t < T; ++t) acur[t] = anext[t];
  }

  // Partial sums of waves 1..3 through LDS; wave 0 adds them in wave order.
  __shared__ f32x4 part[3][T][64];
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) part[wave - 1][t][lane] = acc[t];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    f32x4 sum = acc[t];
    sum = sum + part[0][t][lane];
    sum = sum + part[1][t][lane];
    sum = sum + part[2][t][lane];
    // lane (i16, g16) holds rows m0 + 16t + 4*g16 + r, column n0 + i16
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * t + 4 * g16 + r;
      if (m < a.m) a.y[(size_t)m * a.n + n0 + i16] = sum[r];
    }
  }
}

}  // namespace

hipError_t launch_linear(const LinearLaunch& a, hipStream_t s) {
  if (a.m == 0) return hipSuccess;
  if (a.m <= kLinearSmallRows) {
    hipLaunchKernelGGL(linear_kernel<16>, dim3(a.n / 16, (a.m + 15) / 16), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(linear_kernel<64>, dim3(a.n / 16, (a.m + 63) / 64), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace isk
