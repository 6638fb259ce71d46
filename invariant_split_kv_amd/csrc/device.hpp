// Device helpers for the gfx950 kernels (wave64, bf16, MFMA, LDS transfers).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace isk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define ISK_LDS __attribute__((address_space(3)))

// log2(e) and ln(2), correctly rounded to float.
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

// bf16 pair from a 32-bit word.  Takes the word by value: bit-casting an
// ext_vector element lvalue directly (e.g. v.y) reads element 0 with this
// compiler, so vector elements must be copied into a scalar first.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Hardware exp2 / log2 (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even fp32 -> bf16 pair (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_convertvector(v, bf16x2);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, to_bf16x2(a, b));
}

// Two floats to fp16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// Butterfly reductions inside a wave: every lane ends with the same bits
// (fp32 max is exact; the add tree pairs the same operands in every lane).
__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float wave_add_xor(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

// 16-byte direct global -> LDS load: lane l writes lds_chunk + 16 * l.
__device__ __forceinline__ void load_lds_16(const void* gsrc, ISK_LDS void* lds_chunk) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_chunk, 16, 0, 0);
}

// The same load with the nontemporal hint (cache-policy bit nt): for dense
// KV tiles, read once per call from pools larger than the Infinity Cache, so
// that they neither allocate there nor displace (and write back) other data.
__device__ __forceinline__ void load_lds_16_stream(const void* gsrc, ISK_LDS void* lds_chunk) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_chunk, 16, 0, 2);
}

// Transposing LDS read of four 16-bit values (ds_read_b64_tr_b16).  Within
// each group of 16 lanes, lane i receives element (i % 4) of the 8-byte rows
// addressed by lanes 4r + i / 4, r = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const ISK_LDS void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((ISK_LDS s16x4*)p);
}

__device__ __forceinline__ void wait_vmem_all() {
  // vmcnt = 0 (gfx9 encoding: vmcnt low bits [3:0], high bits [15:14];
  // expcnt [6:4] and lgkmcnt [11:8] left at their maxima).
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

}  // namespace isk
