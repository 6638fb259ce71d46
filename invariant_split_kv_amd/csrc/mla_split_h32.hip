// Absorbed-MLA split kernel for gfx950 with 32 query heads per wave (used
// when the head count is a multiple of 128; dense and sparse top-k).
//
// Same job as the 16-head kernel in mla_split.hip: the split stage of the
// split-KV scheme on the FlashMLA issue page "Sparse MLA decode is not
// batch-invariant ..." (section "Where it comes from"), with split boundaries
// from the host planner that depend only on the row's own length.
//   * One workgroup = four waves (one per SIMD) = 128 heads of one split, so
//     a KV tile is copied into LDS once per split.  For S^T, wave w owns
//     heads [32w, 32w + 32) and keeps their whole 576-dim query slice in
//     VGPRs (36 MFMA B operands); for PV it owns dims [128w, 128w + 128) of
//     all 128 heads.
//   * 32-token tiles (72 pieces of 16 B per token) are copied HBM -> LDS by
//     16-byte direct loads, four tiles in flight.  Piece c of tile row t sits
//     at LDS piece t*72 + (c ^ key(t)), key(t) = 4*((t>>1)&1) + ((t>>2)&3):
//     the 16 rows of one K operand read and the 4-row x 32-byte blocks of a
//     transposing V read land on distinct LDS banks.  Masked rows (past the
//     split end, invalid sparse slots, pages outside the pool) are copied
//     from a 16-byte zero block, so every tile issues the same number of
//     loads and the tile waits can count them.
//   * S^T (32 tokens x 32 heads) = K * Q^T with v_mfma_f32_32x32x16_bf16,
//     fp32 accumulation, one chain over the 36 k-steps.  Lane (n, h) ends up
//     with the 16 scores of head n for tokens 8*(e>>2) + 4h + (e&3).
//   * Online softmax in the log2 domain, p = 2^(s*scale*log2(e) - m + 7)
//     with one fused multiply-add per score, and a lazily moved reference
//     max (the accumulator is rescaled only when a head's max outgrows the
//     reference by more than 2^8).  p is rounded to fp16 for the PV product
//     (the 2^7 factor keeps p within fp16's normal range; it cancels in o =
//     acc / l and is taken out of the LSE); the normaliser sums the fp32 p.
//     Each wave's P and alphas go through LDS to the waves holding the dims.
//   * O^T (128 dims x 128 heads per wave) += V^T * P^T with
//     v_mfma_f32_32x32x16_f16.  Each wave converts the V^T fragments of its
//     own dims from bf16 to fp16 in registers, once per tile, in the shadows
//     of its MFMAs.  The output block of a wave is 256 fp32 values per lane
//     and lives in AGPRs a0..a255 for the whole split, written only by the
//     inline-asm MFMAs below; the compiler's own code uses VGPRs only (the
//     file is built with MFMA results in VGPRs and no VGPR spills to AGPRs).
//     The LDS operands of both products pass through a fixed register ring
//     (v232..v255) written and read only by inline asm, with explicit lgkmcnt
//     waits; v231 is the inline asm's own scratch register.
// Every reduction order above is fixed by the segment's own token range, so
// the bits of a segment's result do not depend on anything else in the batch.

#include <utility>

#include "device.hpp"
#include "isk_internal.hpp"

namespace isk {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kTok = 32;                                   // tokens per LDS tile
constexpr int kBufs = 4;                                   // LDS tile buffers (tiles in flight)
constexpr int kWaves = 4;
constexpr int kHeadsPerBlock = 32 * kWaves;                // 128
constexpr int kPieces = kMlaDqk / 8;                       // 72 pieces of 16 B per latent row
constexpr int kRowBytes = kMlaDqk * 2;                     // 1152
constexpr int kTileBytes = kTok * kRowBytes;               // 36864
constexpr int kLoadsPerWave = kTok * kPieces / 64 / kWaves;   // 9 wave-wide 16-byte loads per tile
constexpr int kKSteps = kMlaDqk / 16;                      // 36
constexpr int kKDepth = 4;                                 // K operand reads in flight (k-steps)
constexpr int kDvTiles = kMlaDv / 32;                      // 16
constexpr int kPvSteps = 2 * kDvTiles;                     // (k-step, dim tile) pairs per tile
constexpr float kRescaleThreshold = 8.0f;                  // log2 units
// p is computed as 2^(x - m + kPShift): at most 2^(8 + 7), well inside fp16,
// and fp16 subnormals only start 2^21 below the reference max.
constexpr float kPShift = 7.0f;

static_assert(kLoadsPerWave * 64 * kWaves == kTok * kPieces, "tile must split evenly over the waves");
static_assert(kKDepth - 1 <= 15 && kKDepth <= 6, "lgkmcnt field / ring slots");

__device__ __forceinline__ int key(int t) { return (((t >> 1) & 1) << 2) | ((t >> 2) & 3); }

// Source of the zero rows (masked tokens).
__device__ __attribute__((aligned(16))) uint32_t g_zero_piece[4];

// ---------------------------------------------------------------------------
// Output block in fixed AGPRs.  Only these asm statements touch AGPRs.

// Clobber list naming all 256 AGPRs (makes the kernel allocate them).
#define ISK_A10(p) "a" #p "0", "a" #p "1", "a" #p "2", "a" #p "3", "a" #p "4", \
                   "a" #p "5", "a" #p "6", "a" #p "7", "a" #p "8", "a" #p "9"
#define ISK_ALL_AGPRS                                                                               \
  ISK_A10(), ISK_A10(1), ISK_A10(2), ISK_A10(3), ISK_A10(4), ISK_A10(5), ISK_A10(6), ISK_A10(7),   \
      ISK_A10(8), ISK_A10(9), ISK_A10(10), ISK_A10(11), ISK_A10(12), ISK_A10(13), ISK_A10(14),      \
      ISK_A10(15), ISK_A10(16), ISK_A10(17), ISK_A10(18), ISK_A10(19), ISK_A10(20), ISK_A10(21),    \
      ISK_A10(22), ISK_A10(23), ISK_A10(24), "a250", "a251", "a252", "a253", "a254", "a255"

template <int DT>
__device__ __forceinline__ void acc_zero_tile() {
  asm volatile(
      "v_accvgpr_write_b32 a[%0*16+0], 0\n\tv_accvgpr_write_b32 a[%0*16+1], 0\n\t"
      "v_accvgpr_write_b32 a[%0*16+2], 0\n\tv_accvgpr_write_b32 a[%0*16+3], 0\n\t"
      "v_accvgpr_write_b32 a[%0*16+4], 0\n\tv_accvgpr_write_b32 a[%0*16+5], 0\n\t"
      "v_accvgpr_write_b32 a[%0*16+6], 0\n\tv_accvgpr_write_b32 a[%0*16+7], 0\n\t"
      "v_accvgpr_write_b32 a[%0*16+8], 0\n\tv_accvgpr_write_b32 a[%0*16+9], 0\n\t"
      "v_accvgpr_write_b32 a[%0*16+10], 0\n\tv_accvgpr_write_b32 a[%0*16+11], 0\n\t"
      "v_accvgpr_write_b32 a[%0*16+12], 0\n\tv_accvgpr_write_b32 a[%0*16+13], 0\n\t"
      "v_accvgpr_write_b32 a[%0*16+14], 0\n\tv_accvgpr_write_b32 a[%0*16+15], 0" ::"n"(DT));
}

template <int... DT>
__device__ __forceinline__ void acc_zero_all(std::integer_sequence<int, DT...>) {
  (acc_zero_tile<DT>(), ...);
}

__device__ __forceinline__ void acc_zero() {
  asm volatile("" ::: ISK_ALL_AGPRS);
  acc_zero_all(std::make_integer_sequence<int, kDvTiles>{});
  // vector-ALU write of an AGPR -> MFMA srcC read
  asm volatile("s_nop 4");
}

#define ISK_SCALE4(o)                                                                       \
  "v_accvgpr_read_b32 %0, a[%5*16+" #o "+0]\n\tv_accvgpr_read_b32 %1, a[%5*16+" #o "+1]\n\t"  \
  "v_accvgpr_read_b32 %2, a[%5*16+" #o "+2]\n\tv_accvgpr_read_b32 %3, a[%5*16+" #o "+3]\n\t"  \
  "v_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %4\n\tv_mul_f32 %2, %2, %4\n\tv_mul_f32 %3, %3, %4\n\t" \
  "v_accvgpr_write_b32 a[%5*16+" #o "+0], %0\n\tv_accvgpr_write_b32 a[%5*16+" #o "+1], %1\n\t" \
  "v_accvgpr_write_b32 a[%5*16+" #o "+2], %2\n\tv_accvgpr_write_b32 a[%5*16+" #o "+3], %3\n\t"

// acc[dt] *= alpha (per lane).
template <int DT>
__device__ __forceinline__ void acc_scale(float alpha) {
  float t0, t1, t2, t3;
  asm volatile(ISK_SCALE4(0) ISK_SCALE4(4) ISK_SCALE4(8) ISK_SCALE4(12)
               : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
               : "v"(alpha), "n"(DT));
}

// acc[T] *= al[T & 3] (head tile ht = T & 3).
template <int... T>
__device__ __forceinline__ void acc_scale_heads(const float (&al)[4], std::integer_sequence<int, T...>) {
  (acc_scale<T>(al[T & 3]), ...);
}

// Wait states between the last MFMA write of the accumulator and a
// vector-ALU access of it: 16 (the compiler puts 12 after a 32x32x16 MFMA
// of its own before a vector-ALU read or write of the result).  With one
// wave per SIMD every wait state costs four cycles, so no more are used.
__device__ __forceinline__ void acc_settle() {
  asm volatile("s_nop 7\n\ts_nop 7");
}

template <int DT>
__device__ __forceinline__ void acc_read(float (&o)[16]) {
  asm volatile(
      "v_accvgpr_read_b32 %0, a[%16*16+0]\n\tv_accvgpr_read_b32 %1, a[%16*16+1]\n\t"
      "v_accvgpr_read_b32 %2, a[%16*16+2]\n\tv_accvgpr_read_b32 %3, a[%16*16+3]\n\t"
      "v_accvgpr_read_b32 %4, a[%16*16+4]\n\tv_accvgpr_read_b32 %5, a[%16*16+5]\n\t"
      "v_accvgpr_read_b32 %6, a[%16*16+6]\n\tv_accvgpr_read_b32 %7, a[%16*16+7]\n\t"
      "v_accvgpr_read_b32 %8, a[%16*16+8]\n\tv_accvgpr_read_b32 %9, a[%16*16+9]\n\t"
      "v_accvgpr_read_b32 %10, a[%16*16+10]\n\tv_accvgpr_read_b32 %11, a[%16*16+11]\n\t"
      "v_accvgpr_read_b32 %12, a[%16*16+12]\n\tv_accvgpr_read_b32 %13, a[%16*16+13]\n\t"
      "v_accvgpr_read_b32 %14, a[%16*16+14]\n\tv_accvgpr_read_b32 %15, a[%16*16+15]"
      : "=v"(o[0]), "=v"(o[1]), "=v"(o[2]), "=v"(o[3]), "=v"(o[4]), "=v"(o[5]), "=v"(o[6]), "=v"(o[7]),
        "=v"(o[8]), "=v"(o[9]), "=v"(o[10]), "=v"(o[11]), "=v"(o[12]), "=v"(o[13]), "=v"(o[14]), "=v"(o[15])
      : "n"(DT));
}

// ---------------------------------------------------------------------------
// Operand ring.  LDS reads in flight land in v232..v255 (six 4-register
// slots; slot i = v[232+4i .. 235+4i]) and the MFMAs read them there by name:
// the compiler never sees these registers (the kernel caps its own
// allocation at 231 VGPRs), so it can neither copy an operand before its wait
// nor reuse the register while the read is outstanding.  v231, also outside
// the compiler's allocation, is scratch for single asm statements: no
// compiler-visible temporaries pass between consecutive statements, which
// would make the compiler put a wait state between them.  S^T uses slots
// 0..kKDepth-1 and, from hook 30 on, slots 4 and 5 for the first V^T
// fragments; PV uses slots 0..2 for P and 3..5 for V^T.
#define ISK_RING_VGPRS "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", \
                       "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", \
                       "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255"
constexpr int kRingSlots = 6;
static_assert(kKDepth <= 4, "S^T reads may only use ring slots 0..3");

__device__ __forceinline__ void ring_claim() { asm volatile("" ::: ISK_RING_VGPRS); }

// LDS reads complete in order, so waiting until at most N are outstanding
// waits for every read issued before the last N.
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}

// ---------------------------------------------------------------------------
// PV, split by dims.  Wave w computes O^T for dims [128w, 128w + 128) of all
// 128 heads of the block.  Accumulator tile T = 4*dt + ht (dt = local dim
// tile 0..3, ht = head tile 0..3) holds, for lane (n, h), O^T[128w + 32dt +
// 8q + 4h + e][32ht + n] at a[16T + 4q + e].  Step s = 8*dt + 4*j + ht:
//   acc[T] += V^T(dim tile 4w + dt, k-step j) * P^T(k-step j, head tile ht),
// v_mfma_f32_32x32x16_f16.  Lane (n, h) of either operand covers the eight
// tokens 16j + 8*(e>>2) + 4h + (e&3), e = 0..7, the order in which the
// softmax holds them.
//  * P^T(j, ht) is the fp16 P that wave ht computed for its own heads; it is
//    exchanged through LDS as pl[ht][j][lane] (16 bytes), written and read
//    back by the same lane index, so a wave-wide access is one contiguous
//    KiB.  P reads go to ring slot s % 3, three steps ahead of their MFMA.
//  * V^T fragment vf = 2*dt + j comes from the bf16 row tile by two
//    transposing reads: lane (i16, gp, h) gets four dims' worth of rows
//    16j + 8u + 4h + (i16 >> 2), dims 32*dt' + 16*gp + 4*(i16 & 3) (dt' the
//    tile's global dim tile), at vaddr[2*(dt'&1) + u] plus an immediate.
//    The four dwords (two bf16 each) are converted to fp16 pairs in place,
//    so each wave converts only the V it multiplies, once per tile.  bf16
//    values with magnitude in [2^-14, 65504] are exact in fp16; the
//    round-toward-zero conversion keeps larger ones finite (clamped to
//    65504) and truncates smaller ones to fp16 subnormals.  Fragment vf
//    lives in ring slot 5 - vf % 3.  Fragments 0 and 1 are read and
//    converted in the S^T stream; fragment vf >= 2 is read after step
//    4vf - 8 and converted one dword per step after steps 4vf-4 .. 4vf-1,
//    three vector-ALU instructions in each MFMA's shadow.
constexpr int kPBytes = kWaves * 2 * 1024;   // pl[4][2][64] x 16 B
constexpr int kXBytes = 32 * 16;             // per-head floats [n][ht]: alpha, later l
// Sparse segments: the pool rows of a window of kWinSlots top-k slots are
// resolved once per window (index, then block-table entry) into LDS, so a
// tile's loads need no dependent global reads (whose waits would also wait
// for the tile loads already in flight).
constexpr int kWinSlots = 1024;
constexpr int kWinBytes = kWinSlots * 4;
constexpr uint32_t kNoRow = 0xffffffffu;     // masked slot
static_assert(kWinSlots % 256 == 0 && kWinSlots % kTok == 0, "window fill and tile alignment");

template <int VF>
struct VFrag {
  static constexpr int dt = VF >> 1, j = VF & 1, slot = 5 - VF % 3;
  static constexpr int off0 = kRowBytes * 16 * j + 128 * (dt >> 1);
  static constexpr int off1 = kRowBytes * (16 * j + 8) + 128 * (dt >> 1);
  static constexpr int m = 2 * (dt & 1);
};

// LDS operations of one tile's PV stream, in issue order: the alpha read and
// the P reads of steps 0..2 before step 0; after the MFMA of step s the P
// read of step s+3 and, every fourth step, the two reads of fragment s/4+2.
constexpr int pv_ops_in_step(int s) { return (s + 3 < kPvSteps ? 1 : 0) + (s % 4 == 0 && s / 4 + 2 < 8 ? 2 : 0); }
constexpr int pv_issued_before(int s) {   // operations issued before the MFMA of step s
  int n = 4;
  for (int u = 0; u < s; ++u) n += pv_ops_in_step(u);
  return n;
}
constexpr int pv_idx_p(int t) { return t < 3 ? 1 + t : pv_issued_before(t - 3); }
constexpr int pv_idx_v(int vf) {   // index of the second read of fragment vf >= 2
  return pv_issued_before(4 * vf - 8) + (4 * vf - 8 + 3 < kPvSteps ? 1 : 0) + 1;
}
// Younger operations than the P read of step s when its MFMA waits.
constexpr int pv_wait_p(int s) { return pv_issued_before(s) - pv_idx_p(s) - 1; }
// Younger operations than fragment vf's reads when its conversion starts,
// after the operations of step 4vf - 4.
constexpr int pv_wait_v(int vf) { return pv_issued_before(4 * vf - 3) - pv_idx_v(vf) - 1; }

template <int VF>
__device__ __forceinline__ void v_issue(const uint32_t (&vaddr)[4]) {
  using V = VFrag<VF>;
  asm volatile("ds_read_b64_tr_b16 v[232+%2*4:233+%2*4], %0 offset:%3\n\t"
               "ds_read_b64_tr_b16 v[234+%2*4:235+%2*4], %1 offset:%4" ::"v"(vaddr[V::m]),
               "v"(vaddr[V::m + 1]), "n"(V::slot), "n"(V::off0), "n"(V::off1));
}

// bf16 pair -> fp16 pair in place: the high value as fp32 goes to the
// scratch register v231, the low one is shifted up in place.
#define ISK_CV_DWORD(i)                                                                       \
  "v_and_b32 v231, 0xffff0000, v[232+%0*4+" #i "]\n\t"                                       \
  "v_lshlrev_b32 v[232+%0*4+" #i "], 16, v[232+%0*4+" #i "]\n\t"                             \
  "v_cvt_pkrtz_f16_f32 v[232+%0*4+" #i "], v[232+%0*4+" #i "], v231\n\t"

// Dword I of fragment VF to fp16.  Dword 0 first waits until at most N LDS
// operations are outstanding (N < 0: no wait; N must cover only operations
// younger than the fragment's reads).  With kNext, dword 3 is followed by
// the MFMA of the next PV step, which reads the fragment: a vector-ALU write
// must be two wait states ahead of an MFMA read of the register, and that
// step's lgkmcnt wait is the second.
template <int VF, int I, int N, bool kNext = false>
__device__ __forceinline__ void v_convert_dword() {
  static_assert(N <= 15, "lgkmcnt field");
  if constexpr (N >= 0)
    asm volatile("s_waitcnt lgkmcnt(%1)\n\t" ISK_CV_DWORD(%2) ::"n"(VFrag<VF>::slot), "n"(N), "n"(I));
  else if constexpr (I == 3 && kNext)
    asm volatile(ISK_CV_DWORD(%2) "s_nop 0" ::"n"(VFrag<VF>::slot), "n"(N), "n"(I));
  else
    asm volatile(ISK_CV_DWORD(%2) ::"n"(VFrag<VF>::slot), "n"(N), "n"(I));
}

template <int S>
__device__ __forceinline__ void p_issue(uint32_t paddr) {
  constexpr int j = (S >> 2) & 1, ht = S & 3;
  asm volatile("ds_read_b128 v[232+%1*4:235+%1*4], %0 offset:%2" ::"v"(paddr), "n"(S % 3), "n"(2048 * ht + 1024 * j));
}

// One PV step: the MFMA of step S, then the P read of step S+3 and, every
// fourth step, the reads of fragment S/4+2; at odd steps 1..17, when the
// next tile is a full dense tile, also load S/2 of that tile (16 bytes per
// lane from `base`, into LDS at the wave's M0 base + 4096 * load).
#define ISK_PV_MFMA "v_mfma_f32_32x32x16_f16 a[%[T]*16:%[T]*16+15], v[232+%[VS]*4:235+%[VS]*4], v[232+%[PS]*4:235+%[PS]*4], a[%[T]*16:%[T]*16+15]\n\t"

template <int S>
__device__ __forceinline__ void pv_step() {
  constexpr int dt = S >> 3, ht = S & 3, vf = S >> 2;
  asm volatile(ISK_PV_MFMA ::[T] "n"(4 * dt + ht), [VS] "n"(VFrag<vf>::slot), [PS] "n"(S % 3));
}

// Next-tile loads placed in the PV stream.  The stream sets M0 freely: the
// caller saves the compiler's M0 before the stream and restores it after.
struct PvDma {
  const unsigned char* base;
  uint32_t m0;          // LDS address of this wave's load 0
  uint32_t p16, keys;   // LoadOffsets fields
};

// MFMA of step S and load PI.  The lane's source offset
// (p16 ^ (key_PI << 4)) + 4096*PI (key_PI in bits [3PI, 3PI+3) of `keys`;
// p16 < 4096, so this equals (p16 + 4096*PI) ^ (key_PI << 4)) is formed in
// the scratch register v231 after the M0 write, so that its vector-ALU
// instructions also cover the wait state the load needs after that write.
template <int S, int PI>
__device__ __forceinline__ void pv_step_dma(const PvDma& d) {
  constexpr int dt = S >> 3, ht = S & 3, vf = S >> 2;
  constexpr int sh = 3 * PI - 4;   // right shift taking key_PI to bits 4..6
#define ISK_PV_DMA_OPS                                                                                   \
  ::[T] "n"(4 * dt + ht), [VS] "n"(VFrag<vf>::slot), [PS] "n"(S % 3),                                  \
    [m0] "s"(d.m0 + (uint32_t)(kWaves * 1024 * PI)), [pio] "n"(4096 * PI), [sh] "n"(sh < 0 ? -sh : sh),  \
    [p16] "v"(d.p16), [keys] "v"(d.keys), [msk] "s"(0x70u), [base] "s"(d.base)
  // bitop3 0x6c: (src0 & src2) ^ src1.
  if constexpr (PI == 0)
    asm volatile(ISK_PV_MFMA
                 "s_mov_b32 m0, %[m0]\n\t"
                 "v_lshlrev_b32 v231, %[sh], %[keys]\n\t"
                 "v_bitop3_b32 v231, v231, %[p16], %[msk] bitop3:0x6c\n\t"
                 "global_load_lds_dwordx4 v231, %[base]" ISK_PV_DMA_OPS);
  else if constexpr (sh < 0)
    asm volatile(ISK_PV_MFMA
                 "s_mov_b32 m0, %[m0]\n\t"
                 "v_lshlrev_b32 v231, %[sh], %[keys]\n\t"
                 "v_bitop3_b32 v231, v231, %[p16], %[msk] bitop3:0x6c\n\t"
                 "v_add_u32 v231, %[pio], v231\n\t"
                 "global_load_lds_dwordx4 v231, %[base]" ISK_PV_DMA_OPS);
  else
    asm volatile(ISK_PV_MFMA
                 "s_mov_b32 m0, %[m0]\n\t"
                 "v_lshrrev_b32 v231, %[sh], %[keys]\n\t"
                 "v_bitop3_b32 v231, v231, %[p16], %[msk] bitop3:0x6c\n\t"
                 "v_add_u32 v231, %[pio], v231\n\t"
                 "global_load_lds_dwordx4 v231, %[base]" ISK_PV_DMA_OPS);
#undef ISK_PV_DMA_OPS
}

template <int S, bool kDmaOn>
__device__ __forceinline__ void pv_do(const uint32_t (&vaddr)[4], uint32_t paddr, const PvDma& dma) {
  constexpr int PI = S >> 1;
  constexpr bool dma_here = (S & 1) != 0 && PI < kLoadsPerWave;
  static_assert(pv_wait_p(S) >= 0 && pv_wait_p(S) <= 15, "lgkmcnt field");
  wait_lgkm<pv_wait_p(S)>();
  if constexpr (kDmaOn && dma_here)
    pv_step_dma<S, PI>(dma);
  else
    pv_step<S>();
  if constexpr (S + 3 < kPvSteps) p_issue<S + 3>(paddr);
  if constexpr (S % 4 == 0 && S / 4 + 2 < 8) v_issue<S / 4 + 2>(vaddr);
  constexpr int cvf = S / 4 + 1, ci = S % 4;   // fragment converted in steps 4cvf-4 .. 4cvf-1
  if constexpr (cvf >= 2 && cvf < 8) v_convert_dword<cvf, ci, ci == 0 ? pv_wait_v(cvf) : -1, true>();
}

template <bool kDmaOn, int... S>
__device__ __forceinline__ void pv_all(const uint32_t (&vaddr)[4], uint32_t paddr, const PvDma& dma,
                                       std::integer_sequence<int, S...>) {
  uint32_t saved_m0;
  if constexpr (kDmaOn) asm volatile("s_mov_b32 %0, m0" : "=s"(saved_m0));
  (pv_do<S, kDmaOn>(vaddr, paddr, dma), ...);
  if constexpr (kDmaOn) asm volatile("s_mov_b32 m0, %0" ::"s"(saved_m0));
}

// ---------------------------------------------------------------------------
// LDS operations the softmax hooks put into the S^T stream of the next tile:
// hook 4 writes this lane's alpha, hooks 12 and 13 read V^T fragments 0 and
// 1 of the current tile, hook 29 writes the lane's two P fragments.  Hooks
// 30..33 convert fragment 0 and hooks 32..35 fragment 1, a dword each.
constexpr int hook_ops(int kk) { return kk == 4 ? 1 : kk == 12 || kk == 13 || kk == 29 ? 2 : 0; }

// K operand reads of S^T (k-step kk): lane (n, h) reads piece 2*kk + h of
// tile row n, at kaddr[kk & 3] + 128*(kk >> 2).
template <int KK>
__device__ __forceinline__ void k_issue(const uint32_t (&kaddr)[4]) {
  asm volatile("ds_read_b128 v[232+%1*4:235+%1*4], %0 offset:%2" ::"v"(kaddr[KK & 3]), "n"(KK % kKDepth),
               "n"(128 * (KK >> 2)));
}

// LDS operations younger than the S^T read of step KK when its MFMA waits:
// the S^T reads issued after it and, with the conversion on, whatever the
// hooks of steps KK-4 .. KK-1 issued (the read of step KK goes out right
// before hook KK-4).
template <bool kConv>
constexpr int qk_younger(int kk) {
  int n = (kk + kKDepth < kKSteps ? kk + kKDepth : kKSteps) - kk - 1;
  if (kConv)
    for (int h = kk - kKDepth; h < kk; ++h) n += h >= 0 ? hook_ops(h) : 0;
  return n;
}

// s += K-slot * q[kk] (S^T in VGPRs, fp32).  The first step starts from 0.
// Without kConv (the S^T of a segment's first tile) the last step is followed
// by the wait states a vector-ALU read of its result needs, inside the same
// asm so nothing can be scheduled in between.  In the tile loop (kConv) the
// result is first read in the next loop step, after the whole PV stream, so
// no wait states are added there.
template <int KK, bool kConv, typename Hook>
__device__ __forceinline__ void qk_do(const uint32_t (&kaddr)[4], const bf16x8 (&qr)[kKSteps], f32x16& s,
                                      Hook& hook) {
  static_assert(qk_younger<kConv>(KK) <= 15, "lgkmcnt field");
  wait_lgkm<qk_younger<kConv>(KK)>();
  if constexpr (KK == 0) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, v[232+%2*4:235+%2*4], %1, 0"
                 : "=&v"(s) : "v"(qr[KK]), "n"(KK % kKDepth));
  } else if constexpr (KK + 1 < kKSteps) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, v[232+%2*4:235+%2*4], %1, %0"
                 : "+v"(s) : "v"(qr[KK]), "n"(KK % kKDepth));
  } else if constexpr (kConv) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, v[232+%2*4:235+%2*4], %1, %0"
                 : "+v"(s) : "v"(qr[KK]), "n"(KK % kKDepth));
  } else {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, v[232+%2*4:235+%2*4], %1, %0\n\t"
                 "s_nop 7\n\ts_nop 7"
                 : "+v"(s) : "v"(qr[KK]), "n"(KK % kKDepth));
  }
  if constexpr (KK + kKDepth < kKSteps) k_issue<KK + kKDepth>(kaddr);
  // Independent vector-ALU work placed in this MFMA's shadow.
  __builtin_amdgcn_sched_barrier(0);
  hook(std::integral_constant<int, KK>{});
  __builtin_amdgcn_sched_barrier(0);
}

template <int... KK>
__device__ __forceinline__ void qk_issue_first(const uint32_t (&kaddr)[4], std::integer_sequence<int, KK...>) {
  (k_issue<KK>(kaddr), ...);
}

template <bool kConv, typename Hook, int... KK>
__device__ __forceinline__ void qk_all(const uint32_t (&kaddr)[4], const bf16x8 (&qr)[kKSteps], f32x16& s,
                                       Hook& hook, std::integer_sequence<int, KK...>) {
  (qk_do<KK, kConv>(kaddr, qr, s, hook), ...);
}

// S^T of one tile (buffer at LDS address `tile`), with `hook` run in the
// MFMA shadows (kConv: the hook also issues the LDS operations counted by
// hook_ops).
template <bool kConv, typename Hook>
__device__ __forceinline__ void qk_tile(uint32_t tile, uint32_t k_lane0, const bf16x8 (&qr)[kKSteps], f32x16& s,
                                        Hook& hook) {
  uint32_t kaddr[4];
  kaddr[0] = tile + k_lane0;
#pragma unroll
  for (int m = 1; m < 4; ++m) kaddr[m] = kaddr[0] ^ (32u * m);
  __builtin_amdgcn_sched_barrier(0);
  qk_issue_first(kaddr, std::make_integer_sequence<int, kKDepth>{});
  qk_all<kConv>(kaddr, qr, s, hook, std::make_integer_sequence<int, kKSteps>{});
  __builtin_amdgcn_sched_barrier(0);
}

// The softmax slices of the last tile of a split, with no S^T to overlap.
template <typename Hook, int... KK>
__device__ __forceinline__ void softmax_only(Hook& hook, std::integer_sequence<int, KK...>) {
  (hook(std::integral_constant<int, KK>{}), ...);
}

// vmcnt(n) with expcnt and lgkmcnt left at their maxima (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------
// Tile staging: wave w issues the 9 wave-wide loads i = w + 4*jj; lane l of
// load i fills LDS piece slot p = 64*i + l, i.e. tile row t = p / 72 and
// latent piece (p % 72) ^ key(t).  Every tile costs exactly kLoadsPerWave
// vector-memory instructions per wave (after any index loads), whatever the
// mask, so "tile it has landed" is a fixed vmcnt.

// Scalar plan of a dense tile: first pool row of the tile and row-valid mask.
struct DenseTile {
  const unsigned char* base;
  uint32_t mask;
};

// Source offsets of a lane's tile loads.  Load jj of wave w fills LDS piece
// slot p = p0 + 256*jj (p0 = 64*w + lane) with latent piece (p % 72) ^ key(t)
// of tile row t = p / 72; since key(t) < 8 only flips bits of p % 72 inside
// its aligned group of 8, the source byte offset within the tile's rows is
// 16 * (p ^ key(t)).  The nine 3-bit keys are packed into one register.
struct LoadOffsets {
  uint32_t p16;    // 16 * p0
  uint32_t keys;   // key of load jj in bits [3jj, 3jj + 3)
  __device__ __forceinline__ void init(int wave, int lane) {
    const int p0 = 64 * wave + lane;
    p16 = 16u * (uint32_t)p0;
    keys = 0u;
#pragma unroll
    for (int jj = 0; jj < kLoadsPerWave; ++jj) keys |= (uint32_t)key((p0 + 256 * jj) / kPieces) << (3 * jj);
  }
  // jj may be a run-time (wave-uniform) value.
  __device__ __forceinline__ uint32_t operator()(int jj) const {
    return (p16 + 4096u * (uint32_t)jj) ^ (__builtin_amdgcn_ubfe(keys, 3 * jj, 3) << 4);
  }
};

template <bool kSparse>
struct Stager {
  const unsigned char* kv;
  const int32_t* bt_row;
  const int32_t* idx_row;
  int page_size, num_pages, len, seg_end;

  // Dense: tiles start at multiples of 32 and pages hold a multiple of 64
  // tokens, so a tile is one contiguous run of rows inside one page.  The
  // block-table entries of pages pbase .. pbase+63 sit in `pwin` (lane i
  // holds entry pbase + i); the caller keeps pi - pbase in [0, 64).
  // (pi, off) = (u0 / page_size, u0 % page_size).
  __device__ __forceinline__ DenseTile plan(int u0, int pi, int off, int pbase, int pwin) const {
    const int nvalid = min(kTok, seg_end - u0);
    const int pg = __builtin_amdgcn_readlane(pwin, pi - pbase);
    const bool page_ok = pg >= 0 && pg < num_pages;
    DenseTile t;
    t.mask = !page_ok ? 0u : (nvalid >= kTok ? ~0u : ((1u << nvalid) - 1u));
    t.base = kv + ((size_t)(page_ok ? pg : 0) * page_size + off) * (size_t)kRowBytes;
    return t;
  }

  // All 9 loads of a dense tile with masked rows read from the zero block.
  __device__ __forceinline__ void issue_masked(const DenseTile& t, ISK_LDS unsigned char* buf, int wave, int lane,
                                               const LoadOffsets& so) const {
    const unsigned char* zero = (const unsigned char*)g_zero_piece;
    int l = lane;
    asm volatile("" : "+v"(l));   // recomputed per call, not kept live across the tile loop
#pragma unroll
    for (int jj = 0; jj < kLoadsPerWave; ++jj) {
      const int i = wave + kWaves * jj;
      const int tr = (i * 64 + l) / kPieces;
      const unsigned char* src = ((t.mask >> tr) & 1u) ? t.base + (size_t)so(jj) : zero;
      load_lds_16(src, buf + i * 1024);
    }
  }

  // Sparse: pool rows of slots [w0, w0 + kWinSlots) into the LDS window
  // (kNoRow where the slot is past the segment, its position is outside
  // [0, len) or its page is outside the pool); kWinSlots / 256 slots per
  // thread of the workgroup.  The caller makes the writes visible (lgkmcnt
  // wait and barrier) before any issue_sparse reads them.  With kGroup =
  // kWinSlots / 256 all index reads go out together, then all table reads
  // (segment start); with kGroup = 1 one slot is resolved at a time, which
  // keeps few registers live (window moves inside the tile loop).
  template <int kGroup>
  __device__ __forceinline__ void fill_window(int w0, ISK_LDS uint32_t* win, int tid) const {
    static_assert((kWinSlots / 256) % kGroup == 0, "group size");
    // Opaque to the compiler here, so the division set-up below is not
    // hoisted out of the tile loop and kept live across it.
    int ps = page_size;
    asm volatile("" : "+s"(ps));
#pragma unroll
    for (int k0 = 0; k0 < kWinSlots / 256; k0 += kGroup) {
      int pos[kGroup];
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        const int slot = w0 + 256 * (k0 + k) + tid;
        pos[k] = slot < seg_end ? idx_row[slot] : -1;
      }
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        bool ok = pos[k] >= 0 && pos[k] < len;
        const int pg = ok ? bt_row[pos[k] / ps] : 0;
        ok = ok && pg >= 0 && pg < num_pages;
        win[256 * (k0 + k) + tid] = ok ? (uint32_t)pg * (uint32_t)ps + (uint32_t)(pos[k] % ps) : kNoRow;
      }
    }
  }

  // All 9 loads of a sparse tile (slots u0 .. u0+31 of the top-k list); the
  // slots' pool rows come from the LDS window that starts at slot wbase
  // (u0 - wbase is in [0, kWinSlots - kTok]).
  __device__ __forceinline__ uint32_t issue_sparse(int u0, ISK_LDS unsigned char* buf, int wave, int lane,
                                                   const ISK_LDS uint32_t* win, int wbase) const {
    const unsigned char* zero = (const unsigned char*)g_zero_piece;
    const uint32_t row = win[u0 - wbase + (lane & 31)];
    const bool ok = lane < 32 && row != kNoRow;
    const uint32_t my_row = ok ? row : 0u;
    const uint32_t mask = (uint32_t)__ballot(ok);
    int l = lane;
    asm volatile("" : "+v"(l));
#pragma unroll
    for (int jj = 0; jj < kLoadsPerWave; ++jj) {
      const int i = wave + kWaves * jj;
      const int p = i * 64 + l;
      const int t = p / kPieces;
      const int c = (p - t * kPieces) ^ key(t);
      const uint32_t r = (uint32_t)__shfl((int)my_row, t, 64);
      const unsigned char* src = ((mask >> t) & 1u) ? kv + (size_t)r * kRowBytes + c * 16 : zero;
      load_lds_16(src, buf + i * 1024);
    }
    return mask;
  }

  // Whole dense tile at once; returns the row-valid mask.
  __device__ __forceinline__ uint32_t operator()(int u0, ISK_LDS unsigned char* buf, int wave, int lane,
                                                 const LoadOffsets& so, int pbase, int pwin) const {
    const DenseTile t = plan(u0, u0 / page_size, u0 % page_size, pbase, pwin);
    if (t.mask == ~0u) {
#pragma unroll
      for (int jj = 0; jj < kLoadsPerWave; ++jj)
        load_lds_16(t.base + (size_t)so(jj), buf + (wave + kWaves * jj) * 1024);
    } else {
      issue_masked(t, buf, wave, lane, so);
    }
    return t.mask;
  }
};

template <bool kSparse>
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_num_vgpr(231)))
mla_split_h32_kernel(MlaLaunch a) {
  __shared__ __attribute__((aligned(1024))) unsigned char
      lds_raw[kBufs * kTileBytes + kPBytes + kXBytes + (kSparse ? kWinBytes : 0)];
  ISK_LDS unsigned char* tiles = (ISK_LDS unsigned char*)lds_raw;
  const uint32_t tiles_u32 = (uint32_t)(uintptr_t)tiles;
  const uint32_t pl_u32 = tiles_u32 + kBufs * kTileBytes;   // fp16 P of the current tile, all heads
  const uint32_t x_u32 = pl_u32 + kPBytes;                  // per-head alpha (per tile) or l (epilogue)
  // sparse: pool rows of the current window of top-k slots
  ISK_LDS uint32_t* const win = (ISK_LDS uint32_t*)(lds_raw + kBufs * kTileBytes + kPBytes + kXBytes);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n32 = lane & 31, hh = lane >> 5, i16 = lane & 15, gp = (lane >> 4) & 1;
  // block id -> (task, head block): head blocks of one task sit 8 ids apart
  // (same XCD under round-robin dealing of workgroups to the 8 XCDs).
  const int n_hb = a.hq / kHeadsPerBlock;
  const int bid = blockIdx.x;
  const int g = (bid / (8 * n_hb)) * 8 + (bid & 7);
  const int hb = (bid >> 3) % n_hb;
  if (g >= a.n_groups) return;
  ring_claim();
  // Wave index as a wave-uniform (scalar) value for address arithmetic.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int head = hb * kHeadsPerBlock + wave * 32 + n32;
  const bool inl = a.inl.n_segs > 0;   // segments by value: one per task
  const int seg_first = inl ? g : a.groups[g], seg_last = inl ? g + 1 : a.groups[g + 1];

  // Per-lane LDS byte offsets of the operand reads (compile-time parts at the use).
  //  K (A operand of S^T), k-step kk: tile row n32, piece 2*kk + hh
  //    -> k_lane[kk & 3] + 128*(kk >> 2).
  //  V^T fragment (transposing reads): v_lane[2*(dt&1) + u], see VFrag.
  // For m = 0..3 both offsets differ only in address bits 5-6 (the row
  // offsets are multiples of 128 and a tile buffer starts at a multiple of
  // 1024), so only m = 0 is kept: offset[m] = offset[0] ^ (32*m).
  uint32_t k_lane0, v_lane0;
  {
    const int kh = key(n32);
    k_lane0 = kRowBytes * n32 + 16 * (hh ^ kh);
    const int hp = (i16 & 3) >> 1;
    v_lane0 = kRowBytes * (4 * hh + (i16 >> 2)) + 64 * (i16 >> 3) + 32 * gp + 16 * (hp ^ hh) + 8 * (i16 & 1);
  }
  // Source offsets (within the tile's rows) of this lane's full-tile loads.
  LoadOffsets so;
  so.init(wave_u, lane);

  for (int si = seg_first; si < seg_last; ++si) {
    Seg sg = fetch_seg(a.inl, a.segs, a.topk_idx != nullptr ? a.topk_len : a.lens, si);
    const int b = sg.row;
    // A sparse segment past the main index width gathers from the extra KV
    // source, at its slots [begin - topk_width, end - topk_width).  The
    // extra lengths are device-only, so positions past the extra block
    // table's capacity are masked here.
    const bool from_extra = kSparse && sg.begin >= a.topk_width;
    if (from_extra) {
      sg.begin -= a.topk_width;
      sg.end -= a.topk_width;
    }
    const Stager<kSparse> stage =
        from_extra ? Stager<kSparse>{(const unsigned char*)a.xkv, a.xblock_table + (size_t)b * a.xmax_pages,
                                     a.xtopk_idx + (size_t)b * a.xtopk_width, a.xpage_size, a.xnum_pages,
                                     min(a.xlens[b], a.xmax_pages * a.xpage_size), sg.end}
                   : Stager<kSparse>{(const unsigned char*)a.kv, a.block_table + (size_t)b * a.max_pages,
                                     kSparse ? a.topk_idx + (size_t)b * a.topk_width : nullptr, a.page_size,
                                     a.num_pages, __builtin_amdgcn_readfirstlane(min(a.lens[b], a.max_pages * a.page_size)), sg.end};

    // Every wave is done reading the previous segment's tiles.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();

    // Block-table window of the segment (dense): lane i holds the entry of
    // page pbase + i (-1 past the segment's pages); moved on by 64 pages
    // when the next tile to plan leaves it.
    int pbase = sg.begin / a.page_size;
    int pwin = -1;
    auto load_window = [&]() {
      const int pl = pbase + lane;
      pwin = (long long)pl * a.page_size < (long long)sg.end ? stage.bt_row[pl] : -1;
    };
    if constexpr (!kSparse) load_window();
    // Query slice: lane (n32, hh) holds q[head][16*kk + 8*hh + 0..7].
    bf16x8 qr[kKSteps];
    {
      const bf16x8* qrow = (const bf16x8*)(a.q + ((size_t)b * a.hq + head) * kMlaDqk + 8 * hh);
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) qr[kk] = qrow[2 * kk];
    }
    // Sparse: the row window of the segment's first kWinSlots slots (its
    // index and table reads are waited for here, together with the query).
    int wbase = sg.begin;
    if constexpr (kSparse) {
      stage.template fill_window<kWinSlots / 256>(wbase, win, (int)threadIdx.x);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
    }
    // The window has landed once only the query loads are younger.
    wait_vmcnt<kKSteps>();

    float m_ref = -INFINITY, l_run = 0.f;
    acc_zero();

    const int n_tiles = (sg.end - sg.begin + kTok - 1) / kTok;
    // Prologue: tiles 0..2 in flight (loads for missing tiles come
    // from the zero block into unused buffers, so the count is always 27);
    // masks kept in a register ring.
    uint32_t mk[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      ISK_LDS unsigned char* tb = tiles + t * kTileBytes;
      if (t < n_tiles) {
        if constexpr (kSparse)
          mk[t] = stage.issue_sparse(sg.begin + t * kTok, tb, wave_u, lane, win, wbase);
        else
          mk[t] = stage(sg.begin + t * kTok, tb, wave_u, lane, so, pbase, pwin);
      } else {
        mk[t] = 0u;
        stage.issue_masked(DenseTile{(const unsigned char*)a.kv, 0u}, tb, wave_u, lane, so);
      }
    }
    uint32_t mk0 = mk[0], mk1 = mk[1], mk2 = mk[2];
    // Page and in-page offset of tile it+3, advanced by one tile per step.
    int pn = (sg.begin + 3 * kTok) / a.page_size, on = (sg.begin + 3 * kTok) % a.page_size;
    // The query has landed once only the 27 prologue loads are younger; the
    // compiler cannot prove this inside the tile loop and would otherwise
    // wait for every outstanding load at each tile.
    wait_vmcnt<3 * kLoadsPerWave>();
    // Pass the query through an empty asm: later uses read its outputs, so
    // the compiler has no load of these registers left to wait for in the
    // tile loop.
#pragma unroll
    for (int kk = 0; kk < kKSteps; kk += 4)
      asm volatile("" : "+v"(qr[kk]), "+v"(qr[kk + 1]), "+v"(qr[kk + 2]), "+v"(qr[kk + 3]));

    // S^T of tile 0 (tiles 1 and 2 -- or their zero stand-ins -- are the
    // 18 younger loads).
    wait_vmcnt<2 * kLoadsPerWave>();
    __builtin_amdgcn_s_barrier();
    f32x16 s_cur;
    {
      auto none = [](auto) {};
      qk_tile<false>(tiles_u32, k_lane0, qr, s_cur, none);
    }

    // Tile loop, software-pipelined by one tile: step `it` computes S^T of
    // tile it+1 and, in the shadows of those MFMAs, the softmax of tile it,
    // whose P (fp16) and alpha go to LDS for the other waves; after a barrier
    // every wave adds V^T * P^T of tile it for its 128 dims and all heads.
    // Buffers: it (PV), it+1 (S^T), it+2 and it+3 (loads in flight).
    const uint32_t pw = pl_u32 + 2048u * wave_u + 16u * lane;   // this lane's P fragments
    const uint32_t xw = x_u32 + 16u * n32 + 4u * wave_u;        // this head's alpha / l slot
    for (int it = 0; it < n_tiles; ++it) {
      const bool has_next = it + 1 < n_tiles;
      // Tile it+1 has landed once only the loads of tile it+2 (or of a zero
      // stand-in of the prologue) are younger; after the barrier every wave
      // is also done with tile it-1, whose buffer the loads of tile it+3
      // reuse, and with the P and alpha of tile it-1.
      if (it + 2 < max(n_tiles, 3))
        wait_vmcnt<kLoadsPerWave>();
      else
        wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      // Re-derive lane offsets inside the loop instead of keeping every
      // derived value live across it.
      asm volatile("" : "+v"(so.p16), "+v"(so.keys), "+v"(k_lane0), "+v"(v_lane0));
      const uint32_t mask = mk0;
      mk0 = mk1;
      mk1 = mk2;
      // Loads of tile it+3 (buffer free since the barrier).  Sparse tiles
      // are issued here.  A dense tile is planned in the hooks of S^T steps
      // 6..11 below (scalar work in MFMA shadows); a full one's 9 loads are
      // then spread over the PV MFMA stream, a partial or masked one's are
      // issued right after the S^T stream.
      ISK_LDS unsigned char* nbuf = tiles + ((it + 3) & 3) * kTileBytes;
      const bool stage_on = it + 3 < n_tiles;
      const int u0n = sg.begin + (it + 3) * kTok;
      if (stage_on) {
        if constexpr (kSparse) {
          if (u0n - wbase >= kWinSlots) {   // every 32 tiles: the next window
            // Every wave issued its last tile from the old window before
            // the barrier at the top of this step.
            wbase += kWinSlots;
            stage.template fill_window<1>(wbase, win, (int)threadIdx.x);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
          }
          mk2 = stage.issue_sparse(u0n, nbuf, wave_u, lane, win, wbase);
        } else if (pn - pbase >= 64) {   // every 64 pages: the next window
          pbase = pn;
          load_window();
          // Waited for here, so that no other path into the plan below
          // carries a wait for it (the compiler would otherwise wait for
          // every outstanding tile load at each step).
          asm volatile("" ::"v"(pwin));
        }
      }
      // Dense plan of tile it+3 (page entry, row mask, first pool row); the
      // page cursor (pn, on) advances by one tile every step.
      int pg_n = 0, row_n = 0;
      uint32_t mask_n = 0u;
      const unsigned char* base_n = nullptr;
      const int buf = it & 3;

      // ---- online softmax of tile it; lane holds head n32, tokens
      // 8*(e>>2) + 4*hh + (e&3).  Masked scores become -inf first.
      if (mask != ~0u) {   // partial or masked tile (wave-uniform test)
        const uint32_t mh = mask >> (4 * hh);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          s_cur[e] = __builtin_amdgcn_ubfe(mh, 8 * (e >> 2) + (e & 3), 1) ? s_cur[e] : -INFINITY;
      }
      float mx = -INFINITY, alpha = 1.f, m_sub = 0.f, psum = 0.f;
      f16x8 ph[2];
      // V^T fragments of tile it for this wave's dims (dim tiles 4w ..).
      uint32_t vaddr[4];
      vaddr[0] = tiles_u32 + buf * kTileBytes + 256u * wave_u + v_lane0;
#pragma unroll
      for (int m = 1; m < 4; ++m) vaddr[m] = vaddr[0] ^ (32u * m);
      // The softmax in slices, one per k-step of the next tile's S^T:
      //  0..3   max over the raw scores (with scale > 0, checked by the
      //         planner, the max of the scaled scores, rounding included)
      //  4      lane-pair max, lazy reference move, alpha (to LDS)
      //  5..20  p = 2^(s*scale - m + 7), one score per slice
      //  6..11  (dense) scalar plan of tile it+3
      //  12, 13 reads of V^T fragments 0 and 1
      //  21..28 p -> fp16, one pair per slice; sum of the fp32 p
      //  29     running normaliser; P to LDS
      //  30..35 conversion of fragments 0 (30..33) and 1 (32..35)
      auto softmax = [&](auto kc) {
        constexpr int KK = decltype(kc)::value;
        if constexpr (KK < 4) {
#pragma unroll
          for (int e = 4 * KK; e < 4 * KK + 4; ++e) mx = fmaxf(mx, s_cur[e]);
        } else if constexpr (KK == 4) {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
          const float m_old = m_ref;
          const bool move = mx > m_old + kRescaleThreshold || (m_old == -INFINITY && mx > -INFINITY);
          const float m_new = move ? mx : m_old;
          // acc is still 0 before the first move: no rescale then.
          alpha = move && m_old != -INFINITY ? fast_exp2(m_old - m_new) : 1.0f;
          m_ref = m_new;
          m_sub = m_new == -INFINITY ? 0.f : m_new - kPShift;
          // Both lanes of a head write the same value.
          asm volatile("ds_write_b32 %0, %1" ::"v"(xw), "v"(alpha));
        } else if constexpr (KK < 21) {
          constexpr int e = KK - 5;
          s_cur[e] = fast_exp2(__builtin_fmaf(s_cur[e], a.scale_log2, -m_sub));
        } else if constexpr (KK < 29) {
          constexpr int q = KK - 21, j = q >> 2, r = q & 3;
          const float p0 = s_cur[2 * q], p1 = s_cur[2 * q + 1];
          ph[j][2 * r] = (_Float16)p0;
          ph[j][2 * r + 1] = (_Float16)p1;
          psum += p0;
          psum += p1;
        } else if constexpr (KK == 29) {
          l_run = l_run * alpha + psum;
          asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:1024" ::"v"(pw), "v"(ph[0]), "v"(ph[1]));
        }
        if constexpr (!kSparse) {
          // Each piece is pinned to its hook by an empty asm use of its result.
          if constexpr (KK == 6) {
            pg_n = __builtin_amdgcn_readlane(pwin, pn - pbase);
            asm volatile("" ::"s"(pg_n));
          } else if constexpr (KK == 7) {
            // page entry outside the pool: the whole tile is masked
            pg_n = pg_n >= 0 && pg_n < a.num_pages ? pg_n : -1;
            asm volatile("" ::"s"(pg_n));
          } else if constexpr (KK == 8) {
            const int nvalid = min(kTok, sg.end - u0n);
            mask_n = pg_n < 0 ? 0u : (nvalid >= kTok ? ~0u : ((1u << nvalid) - 1u));
            asm volatile("" ::"s"(mask_n));
          } else if constexpr (KK == 9) {
            row_n = max(pg_n, 0) * a.page_size + on;
            asm volatile("" ::"s"(row_n));
          } else if constexpr (KK == 10) {
            base_n = (const unsigned char*)a.kv + (size_t)(uint32_t)row_n * kRowBytes;
            asm volatile("" ::"s"(base_n));
          } else if constexpr (KK == 11) {
            on += kTok;
            if (on >= a.page_size) {
              on -= a.page_size;
              ++pn;
            }
            asm volatile("" ::"s"(on), "s"(pn));
          }
        }
        if constexpr (KK == 12) v_issue<0>(vaddr);
        if constexpr (KK == 13) v_issue<1>(vaddr);
        // The reads of hooks 12 and 13 are complete once the MFMA of step 18
        // has waited; without an S^T stream (last tile) hook 30 waits itself.
        if constexpr (KK == 30)
          if (!has_next) wait_lgkm<0>();
        if constexpr (KK >= 30 && KK <= 33) v_convert_dword<0, KK - 30, -1>();
        if constexpr (KK >= 32 && KK <= 35) v_convert_dword<1, KK - 32, -1>();
      };
      f32x16 s_next;
      if (has_next)
        qk_tile<true>(tiles_u32 + ((it + 1) & 3) * kTileBytes, k_lane0, qr, s_next, softmax);
      else
        softmax_only(softmax, std::make_integer_sequence<int, kKSteps>{});
      bool defer = false;
      if constexpr (!kSparse) {
        if (stage_on) {
          mk2 = mask_n;
          defer = mask_n == ~0u;
          if (!defer) stage.issue_masked(DenseTile{base_n, mask_n}, nbuf, wave_u, lane, so);
        }
      }
      // Every wave's P and alpha of tile it are in LDS.
      wait_lgkm<0>();
      __builtin_amdgcn_s_barrier();

      // ---- O^T += V^T * P^T for this wave's dims and all heads.  The alpha
      // of the four heads this lane accumulates comes first; the accumulator
      // is rescaled when any of them moved (lanes that did not move have
      // alpha == 1 exactly).
      const uint32_t pr = pl_u32 + 16u * lane;
      float al[4];
      __builtin_amdgcn_sched_barrier(0);
      // The alphas land in ring slot 3 (V^T fragment 2 is read into it only
      // after the first MFMA), the first P reads in slots 0..2.
      static_assert(VFrag<2>::slot == 3, "alpha slot");
      asm volatile("ds_read_b128 v[244:247], %0" ::"v"(x_u32 + 16u * n32));
      p_issue<0>(pr);
      p_issue<1>(pr);
      p_issue<2>(pr);
      asm volatile("s_waitcnt lgkmcnt(3)\n\tv_mov_b32 %0, v244\n\tv_mov_b32 %1, v245\n\tv_mov_b32 %2, v246\n\tv_mov_b32 %3, v247"
                   : "=v"(al[0]), "=v"(al[1]), "=v"(al[2]), "=v"(al[3]));
      __builtin_amdgcn_sched_barrier(0);
      if (__ballot(al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f) != 0ull) {
        acc_settle();
        acc_scale_heads(al, std::make_integer_sequence<int, 16>{});
        asm volatile("s_nop 4");
      }
      // LDS address of this wave's first load of tile it+3 (wave-uniform).
      const PvDma dma{base_n, tiles_u32 + ((it + 3) & 3) * kTileBytes + wave_u * 1024, so.p16, so.keys};
      __builtin_amdgcn_sched_barrier(0);
      if (defer)
        pv_all<true>(vaddr, pr, dma, std::make_integer_sequence<int, kPvSteps>{});
      else
        pv_all<false>(vaddr, pr, dma, std::make_integer_sequence<int, kPvSteps>{});
      __builtin_amdgcn_sched_barrier(0);
      s_cur = s_next;
    }

    // ---- epilogue: o = acc / l, lse = ln 2 * (m_ref - kPShift + log2 l).
    // Each head's l goes through LDS to the waves holding its dims.
    float l_tot;
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
      l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const bool empty = !(l_tot > 0.f);
    const float lse_v = empty ? -INFINITY : (m_ref - kPShift + fast_log2(l_tot)) * kLn2;
    __builtin_amdgcn_s_barrier();   // every wave is done with the last alphas
    asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(xw), "v"(l_tot) : "memory");
    __builtin_amdgcn_s_barrier();
    float inv[4];
    {
      float l4[4];
      asm volatile("ds_read_b128 v[232:235], %4\n\ts_waitcnt lgkmcnt(0)\n\tv_mov_b32 %0, v232\n\tv_mov_b32 %1, v233\n\t"
                   "v_mov_b32 %2, v234\n\tv_mov_b32 %3, v235"
                   : "=v"(l4[0]), "=v"(l4[1]), "=v"(l4[2]), "=v"(l4[3])
                   : "v"(x_u32 + 16u * n32));
#pragma unroll
      for (int t = 0; t < 4; ++t) inv[t] = l4[t] > 0.f ? 1.f / l4[t] : 0.f;
    }
    acc_settle();
    // lane holds O^T[128w + 32*dt + 8*q + 4*hh + e][32*ht + n32] at
    // acc[4*dt + ht][4q + e] (row and wave re-read here so that their address
    // arithmetic is not hoisted out of the segment loop and kept live
    // across it).
    int head_e = head;
    asm volatile("" : "+v"(head_e));
    float* of32 = nullptr;
    uint16_t* obf = nullptr;   // bf16 output, or fp16 partials (f16out)
    bool f16out = false;
    {
      const size_t hb0 = (size_t)(hb * kHeadsPerBlock + n32);   // head of tile ht = 0
      const size_t base = (sg.part >= 0 ? (size_t)sg.part : (size_t)b) * a.hq + hb0;
      const size_t eo = base * kMlaDv + 128 * (size_t)wave_u + 4 * hh;
      if (sg.part >= 0) {
        if (a.part_f16) {
          obf = (uint16_t*)a.part_o + eo;
          f16out = true;
        } else {
          of32 = a.part_o + eo;
        }
        if (hh == 0) a.part_lse[(size_t)sg.part * a.hq + head_e] = lse_v;
      } else {
        if (a.out_f32)
          of32 = (float*)a.out + eo;
        else
          obf = (uint16_t*)a.out + eo;
        if (a.lse != nullptr && hh == 0) a.lse[(size_t)b * a.hq + head_e] = lse_v;
      }
    }
    auto store_tile = [&](int t, const float (&o)[16]) {
      const int dt = t >> 2, ht = t & 3;
      const size_t off = (size_t)ht * 32 * kMlaDv + 32 * dt;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 r = f32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]} * inv[ht];
        if (of32 != nullptr) {
          *(f32x4*)(of32 + off + 8 * q) = r;
        } else if (f16out) {
          uint2 w;
          w.x = pack_f16x2(r[0], r[1]);
          w.y = pack_f16x2(r[2], r[3]);
          *(uint2*)(obf + off + 8 * q) = w;
        } else {
          uint2 w;
          w.x = pack_bf16x2(r[0], r[1]);
          w.y = pack_bf16x2(r[2], r[3]);
          *(uint2*)(obf + off + 8 * q) = w;
        }
      }
    };
    {
      float o[16];
      acc_read<0>(o); store_tile(0, o);
      acc_read<1>(o); store_tile(1, o);
      acc_read<2>(o); store_tile(2, o);
      acc_read<3>(o); store_tile(3, o);
      acc_read<4>(o); store_tile(4, o);
      acc_read<5>(o); store_tile(5, o);
      acc_read<6>(o); store_tile(6, o);
      acc_read<7>(o); store_tile(7, o);
      acc_read<8>(o); store_tile(8, o);
      acc_read<9>(o); store_tile(9, o);
      acc_read<10>(o); store_tile(10, o);
      acc_read<11>(o); store_tile(11, o);
      acc_read<12>(o); store_tile(12, o);
      acc_read<13>(o); store_tile(13, o);
      acc_read<14>(o); store_tile(14, o);
      acc_read<15>(o); store_tile(15, o);
    }
  }
}

}  // namespace

hipError_t launch_mla_split_h32(const MlaLaunch& a, hipStream_t s, const LaunchEvents& ev) {
  if (a.n_groups == 0) return hipSuccess;
  if (a.hq % kHeadsPerBlock != 0) return hipErrorInvalidValue;
  const int n_hb = a.hq / kHeadsPerBlock;
  const int n_blocks = ((a.n_groups + 7) / 8) * 8 * n_hb;
  const dim3 grid(n_blocks), block(64 * kWaves);
  if (a.topk_idx != nullptr) return launch_one(mla_split_h32_kernel<true>, grid, block, s, a, ev);
  return launch_one(mla_split_h32_kernel<false>, grid, block, s, a, ev);
}

}  // namespace isk
