// Fixed-order combine of split partials (gfx950).
//
// The merge step of the split-KV scheme on the FlashMLA issue page "Sparse
// MLA decode is not batch-invariant ..." (section "Where it comes from"): the
// partial outputs o_i of a row's splits are weighted by their log-sum-exp
// scales and summed.  That page traces the batch dependence to how many
// splits there are and where they fall, not to the loop itself; here the
// splits of a row are fixed by its own length, and this kernel merges them in
// ascending split order with one fixed arithmetic sequence for every split
// count (no per-count code variants, no atomics):
//   m = max_i lse_i;  e_i = 2^((lse_i - m) * log2 e);  S = sum_i e_i;
//   lse = m + ln S;   out = sum_i (e_i / S) * o_i   (fp32 FMA chain, i ascending)
// One wave handles one (row, head); lane l owns Dv/64 consecutive dims.
// Rows with one split were written by the split kernel and are skipped; rows
// with none get out = 0 and lse = -inf.

#include "device.hpp"
#include "isk_internal.hpp"

namespace isk {
namespace {

template <int DPL>
__global__ void __launch_bounds__(256) combine_kernel(CombineLaunch a) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= a.batch * a.hq) return;
  const int b = pair / a.hq, h = pair - b * a.hq;
  const RowInfo ri = a.rows[b];
  if (ri.n_parts == 1) return;

  float o[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) o[j] = 0.f;
  float lse_out = -INFINITY;

  if (ri.n_parts > 1) {
    const float* lse_p = a.part_lse + (size_t)ri.part_off * a.hq + h;
    float m = -INFINITY;
    for (int i = 0; i < ri.n_parts; ++i) m = fmaxf(m, lse_p[(size_t)i * a.hq]);
    if (m != -INFINITY) {
      float ssum = 0.f;
      for (int i = 0; i < ri.n_parts; ++i) ssum += fast_exp2((lse_p[(size_t)i * a.hq] - m) * kLog2e);
      const float inv = 1.f / ssum;
      lse_out = m + fast_log2(ssum) * kLn2;
      const float* op = a.part_o + ((size_t)ri.part_off * a.hq + h) * a.dv + DPL * lane;
      const size_t stride = (size_t)a.hq * a.dv;
      auto load = [&](int i, float (&v)[DPL]) {
        const float* src = op + (size_t)i * stride;
        if constexpr (DPL % 4 == 0) {
#pragma unroll
          for (int j = 0; j < DPL; j += 4) {
            const f32x4 x = *(const f32x4*)(src + j);
            v[j] = x[0]; v[j + 1] = x[1]; v[j + 2] = x[2]; v[j + 3] = x[3];
          }
        } else if constexpr (DPL == 2) {
          const f32x2 x = *(const f32x2*)src;
          v[0] = x[0]; v[1] = x[1];
        } else {
          v[0] = src[0];
        }
      };
      auto accumulate = [&](int i, const float (&v)[DPL]) {
        const float w = fast_exp2((lse_p[(size_t)i * a.hq] - m) * kLog2e) * inv;
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[j] = fmaf(w, v[j], o[j]);
      };
      // Four partials' loads in flight at a time; the accumulation order is
      // still i = 0, 1, 2, ... for every split count.
      int i = 0;
      for (; i + 4 <= ri.n_parts; i += 4) {
        float v0[DPL], v1[DPL], v2[DPL], v3[DPL];
        load(i, v0); load(i + 1, v1); load(i + 2, v2); load(i + 3, v3);
        accumulate(i, v0); accumulate(i + 1, v1); accumulate(i + 2, v2); accumulate(i + 3, v3);
      }
      for (; i < ri.n_parts; ++i) {
        float v0[DPL];
        load(i, v0);
        accumulate(i, v0);
      }
    }
  }

  const size_t ob = ((size_t)b * a.hq + h) * a.dv + DPL * lane;
  if (a.out_f32) {
    float* dst = (float*)a.out + ob;
#pragma unroll
    for (int j = 0; j < DPL; ++j) dst[j] = o[j];
  } else {
    uint16_t* dst = (uint16_t*)a.out + ob;
    if constexpr (DPL % 2 == 0) {
#pragma unroll
      for (int j = 0; j < DPL; j += 2) *(uint32_t*)(dst + j) = pack_bf16x2(o[j], o[j + 1]);
    } else {
      dst[0] = (uint16_t)(pack_bf16x2(o[0], 0.f) & 0xffffu);
    }
  }
  if (a.lse != nullptr && lane == 0) a.lse[(size_t)b * a.hq + h] = lse_out;
}

}  // namespace

hipError_t launch_combine(const CombineLaunch& a, hipStream_t s) {
  const int pairs = a.batch * a.hq;
  if (pairs == 0) return hipSuccess;
  const dim3 grid((pairs + 3) / 4), block(256);
  switch (a.dv) {
    case 64: hipLaunchKernelGGL(combine_kernel<1>, grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(combine_kernel<2>, grid, block, 0, s, a); break;
    case 512: hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace isk
