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
// Partials are fp32, or fp16 for the 128-head MLA kernels with bf16 output
// (widened exactly to fp32 on load; the arithmetic is the same).
// One wave handles one (row, head); lane l owns Dv/64 consecutive dims.  The
// LSEs are loaded lane-parallel and the partials up to eight at a time, so a
// row costs a few memory round trips instead of one per split.
// Rows with one split were written by the split kernel and are skipped; rows
// with none get out = 0 and lse = -inf.

#include <utility>

#include "device.hpp"
#include "isk_internal.hpp"

namespace isk {
namespace {

template <int DPL>
__device__ __forceinline__ void load_part(const float* src, float (&v)[DPL]) {
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
}

// fp16 partials (exact widening to fp32).
template <int DPL>
__device__ __forceinline__ void load_part(const uint16_t* src, float (&v)[DPL]) {
  auto half = [](uint32_t bits) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits); };
  if constexpr (DPL % 8 == 0) {
#pragma unroll
    for (int j = 0; j < DPL; j += 8) {
      const uint4 x = *(const uint4*)(src + j);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[j + 2 * k] = half(w[k] & 0xffffu);
        v[j + 2 * k + 1] = half(w[k] >> 16);
      }
    }
  } else if constexpr (DPL == 2) {
    const uint32_t x = *(const uint32_t*)src;
    v[0] = half(x & 0xffffu); v[1] = half(x >> 16);
  } else {
#pragma unroll
    for (int j = 0; j < DPL; ++j) v[j] = half(src[j]);
  }
}

// Partials as loaded (the first splits' before the weights are known, later
// ones a group at a time): fp32 values, or fp16 kept packed (four VGPRs for
// eight values, widened at the FMA), which keeps the fp16 kernel at 70
// VGPRs (seven waves a SIMD).
template <int DPL, typename P>
struct Early;
template <int DPL>
struct Early<DPL, float> {
  float v[DPL];
  __device__ __forceinline__ void load(const float* src) { load_part<DPL>(src, v); }
  __device__ __forceinline__ void fma_into(float w, float (&o)[DPL]) const {
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[j] = fmaf(w, v[j], o[j]);
  }
};
template <int DPL>
struct Early<DPL, uint16_t> {
  static_assert(DPL % 8 == 0, "fp16 partials are loaded 8 values at a time");
  uint4 v[DPL / 8];
  __device__ __forceinline__ void load(const uint16_t* src) {
#pragma unroll
    for (int i = 0; i < DPL / 8; ++i) v[i] = *(const uint4*)(src + 8 * i);
  }
  __device__ __forceinline__ void fma_into(float w, float (&o)[DPL]) const {
    auto half = [](uint32_t bits) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits); };
#pragma unroll
    for (int i = 0; i < DPL / 8; ++i) {
      const uint32_t x[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[8 * i + 2 * k] = fmaf(w, half(x[k] & 0xffffu), o[8 * i + 2 * k]);
        o[8 * i + 2 * k + 1] = fmaf(w, half(x[k] >> 16), o[8 * i + 2 * k + 1]);
      }
    }
  }
};

// The partials' LSEs are loaded lane-parallel (lane l of chunk c holds split
// 64c + l); the sum of the weights and the output FMA chain still run over
// the splits one at a time in ascending order (v_readlane of the lane that
// holds split i), so every value is the one the sequential definition gives.
template <int DPL, typename P>
__global__ void __launch_bounds__(256) combine_kernel(CombineLaunch a) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= a.batch * a.hq) return;
  const int b = pair / a.hq, h = pair - b * a.hq;
  const RowInfo ri = a.inl.n_segs > 0 ? a.inl.rows[b] : a.rows[b];
  if (ri.n_parts == 1) return;

  float o[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) o[j] = 0.f;
  float lse_out = -INFINITY;

  if (ri.n_parts > 1) {
    const float* lse_p = a.part_lse + (size_t)ri.part_off * a.hq + h;
    const int n = ri.n_parts;
    // The LSEs of chunk c (splits 64c .. 64c+63, lane-parallel); with at most
    // 64 splits (every row up to 98304 tokens) the one chunk is loaded once.
    const float x0 = lane < n ? lse_p[(size_t)lane * a.hq] : -INFINITY;
    // Up to eight splits (most rows): the partials do not depend on the
    // weights, so their loads go out with the LSEs' and the row costs one
    // memory round trip.
    const P* op = (const P*)a.part_o + ((size_t)ri.part_off * a.hq + h) * a.dv + DPL * lane;
    const size_t stride = (size_t)a.hq * a.dv;
    constexpr int kEarly = 8;
    Early<DPL, P> ve[kEarly];
    if (n <= kEarly) {
#pragma unroll
      for (int k = 0; k < kEarly; ++k)
        if (k < n) ve[k].load(op + (size_t)k * stride);
    }
    auto lse_chunk = [&](int c) { return c == 0 ? x0 : (c + lane < n ? lse_p[(size_t)(c + lane) * a.hq] : -INFINITY); };
    // m = max_i lse_i (exact, any order).
    float m = -INFINITY;
    for (int c = 0; c < n; c += 64) {
      const float x = lse_chunk(c);
      float w = x;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) w = fmaxf(w, __shfl_xor(w, d, 64));
      m = fmaxf(m, w);
    }
    if (m != -INFINITY) {
      // S = sum_i 2^((lse_i - m) log2 e), i ascending.
      float ssum = 0.f;
      for (int c = 0; c < n; c += 64) {
        const float x = lse_chunk(c);
        const float e = fast_exp2((x - m) * kLog2e);
        const int cn = min(64, n - c);
        for (int i = 0; i < cn; ++i) ssum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), i));
      }
      const float inv = 1.f / ssum;
      lse_out = m + fast_log2(ssum) * kLn2;
      // out = sum_i (e_i / S) o_i, an FMA chain with i ascending; the
      // partials' loads go out eight (fp16: four) at a time, then the rest.
      if (n <= kEarly) {
        const float wl = fast_exp2((x0 - m) * kLog2e) * inv;
#pragma unroll
        for (int k = 0; k < kEarly; ++k) {
          if (k < n) {
            const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), k));
            ve[k].fma_into(w, o);
          }
        }
      }
      for (int c = 0; n > kEarly && c < n; c += 64) {
        const float x = lse_chunk(c);
        const float wl = fast_exp2((x - m) * kLog2e) * inv;
        const int cn = min(64, n - c);
        // Loads of a group go out together, then its FMAs in order.
        auto group = [&](int i0, auto kn) {
          constexpr int K = decltype(kn)::value;
          Early<DPL, P> v[K];
#pragma unroll
          for (int k = 0; k < K; ++k) v[k].load(op + (size_t)(c + i0 + k) * stride);
#pragma unroll
          for (int k = 0; k < K; ++k) {
            const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), i0 + k));
            v[k].fma_into(w, o);
          }
        };
        // (fp16 partials: groups of four, which keeps the kernel's register
        // count at the early path's)
        constexpr int kGroup = sizeof(P) == 2 ? 4 : 8;
        int i = 0;
        for (; i + kGroup <= cn; i += kGroup) group(i, std::integral_constant<int, kGroup>{});
        if (i + 4 <= cn) {
          group(i, std::integral_constant<int, 4>{});
          i += 4;
        }
        switch (cn - i) {
          case 3: group(i, std::integral_constant<int, 3>{}); break;
          case 2: group(i, std::integral_constant<int, 2>{}); break;
          case 1: group(i, std::integral_constant<int, 1>{}); break;
          default: break;
        }
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
  if (a.part_f16) {
    if (a.dv != 512) return hipErrorInvalidValue;
    hipLaunchKernelGGL((combine_kernel<8, uint16_t>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  switch (a.dv) {
    case 64: hipLaunchKernelGGL((combine_kernel<1, float>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((combine_kernel<2, float>), grid, block, 0, s, a); break;
    case 512: hipLaunchKernelGGL((combine_kernel<8, float>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace isk
