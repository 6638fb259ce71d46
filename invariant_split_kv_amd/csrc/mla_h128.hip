// Absorbed-MLA split kernel for gfx950, one workgroup per split and block of
// 128 query heads (used for MLA when the head count is a multiple of 128:
// dense rows, and sparse top-k rows whose splits hold at most 1024 slots of
// a latent pool under 4 GiB).
//
// The split stage of the split-KV scheme on the FlashMLA issue page "Sparse
// MLA decode is not batch-invariant ..." (section "Where it comes from"), with
// split boundaries from the host planner that depend only on the row's own
// length.  Four waves, one per SIMD: for S^T = K Q^T wave w owns heads
// [32w, 32w + 32) of the block (their 576-dim query slice in VGPRs), for
// O^T += V^T P^T it owns dims [128w, 128w + 128) of all 128 heads (the fp32
// output block in AGPRs).  The tile loop of a segment is one generated
// inline-asm block (gen_mla_h128.py, run by the build), which documents the
// schedule and the register plan; this file plans the segment, runs the block
// and writes the output from the accumulator.  The arithmetic is the one of
// mla_split_h32.hip (same operands, same orders), so both give the same bits.
//
// Sparse splits (the top-k gather of the same page): before the block, the
// workgroup resolves the split's slots into an LDS window -- per slot the
// value 1152 (r - t) mod 2^32, r the slot's pool row (0 for an invalid slot:
// a position outside [0, len), a page outside the pool, or past the split's
// end) and t its row in its 32-slot tile -- and one row-valid mask per tile.
// A tile load adds its lane's piece offset 16 (72 t + piece) to the window
// value, which gives the piece's byte offset 1152 r + 16 piece in the pool,
// so every load is one 32-bit offset from the pool base.

#include <utility>

#include "device.hpp"
#include "isk_internal.hpp"
#include "mla_h128_seg.inc"

namespace isk {
namespace {

constexpr int kWaves = 4;
constexpr int kHeadsPerBlock = 128;
constexpr int kTok = 32;
constexpr int kXOff = 4 * kTok * kMlaDqk * 2 + 8192;   // per-head floats after the tiles and the P exchange
constexpr float kPShift = 7.0f;                        // p carries a factor 2^7 (taken out of the LSE)
constexpr int kStageRow = 144;
constexpr int kFmtF32 = 0, kFmtBF16 = 1, kFmtF16 = 2;   // output row formats                         // bytes per head row of the output staging (128 + 16)
// global-memory pointer types (the stores use a scalar base)
typedef __attribute__((address_space(1))) unsigned char GU8;
typedef __attribute__((address_space(1))) f32x4 GF32x4;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) u32x2 GU32x2;
typedef __attribute__((address_space(4))) MlaLaunch KArg;   // the kernel arguments
static_assert(ISK_H128_LDS_BYTES == kXOff + 512, "LDS layout of the generated block");
static_assert(ISK_H128_WIN_OFF >= ISK_H128_LDS_BYTES && ISK_H128_MASK_OFF == ISK_H128_WIN_OFF + 4 * ISK_H128_WIN_SLOTS &&
                  ISK_H128_SPARSE_LDS_BYTES >= ISK_H128_MASK_OFF + 4 * (ISK_H128_WIN_SLOTS / kTok) &&
                  ISK_H128_SPARSE_LDS_BYTES <= 160 * 1024,
              "LDS layout of the sparse window");
static_assert(ISK_H128_WIN_SLOTS == kMlaH128MaxSparseSlots, "sparse split limit of the dispatch");
constexpr uint32_t kRowBytes = 2 * kMlaDqk;   // 1152

#define ISK_H128_A10(p) "a" #p "0", "a" #p "1", "a" #p "2", "a" #p "3", "a" #p "4", \
                        "a" #p "5", "a" #p "6", "a" #p "7", "a" #p "8", "a" #p "9"
#define ISK_H128_ALL_AGPRS                                                                                   \
  ISK_H128_A10(), ISK_H128_A10(1), ISK_H128_A10(2), ISK_H128_A10(3), ISK_H128_A10(4), ISK_H128_A10(5),      \
      ISK_H128_A10(6), ISK_H128_A10(7), ISK_H128_A10(8), ISK_H128_A10(9), ISK_H128_A10(10), ISK_H128_A10(11), \
      ISK_H128_A10(12), ISK_H128_A10(13), ISK_H128_A10(14), ISK_H128_A10(15), ISK_H128_A10(16),               \
      ISK_H128_A10(17), ISK_H128_A10(18), ISK_H128_A10(19), ISK_H128_A10(20), ISK_H128_A10(21),               \
      ISK_H128_A10(22), ISK_H128_A10(23), ISK_H128_A10(24), "a250", "a251", "a252", "a253", "a254", "a255"

// Accumulator tile T (16 fp32 per lane) out of AGPRs.  The last MFMA that
// wrote it must be at least 16 wait states back (acc_settle).
template <int T>
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
      : "n"(T));
}

// Sparse split: slots [0, n) of the segment's top-k list `idx` (1 <= n <=
// 1024) into the window (see the file comment).  The 256 threads take slots
// 256 k + tid; the index reads of all four rounds go out together (clamped
// to slot n - 1, so no read is predicated), then the table reads.  Wave w's
// ballot of round k is the mask of tiles 8 k + 2 w and 8 k + 2 w + 1.  The
// lane is derived here rather than kept across the segment's asm block.
__device__ __forceinline__ void resolve_window(unsigned char* lds_raw, const int32_t* idx, const int32_t* bt, int n,
                                               int len, int P, int npg, int wave) {
  ISK_LDS uint32_t* const win = (ISK_LDS uint32_t*)(lds_raw + ISK_H128_WIN_OFF);
  ISK_LDS uint32_t* const masks = (ISK_LDS uint32_t*)(lds_raw + ISK_H128_MASK_OFF);
  constexpr int kRounds = ISK_H128_WIN_SLOTS / 256;
  int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(lane));
  const int tid = 64 * wave + lane;
  int pos[kRounds];
#pragma unroll
  for (int k = 0; k < kRounds; ++k) pos[k] = idx[min(256 * k + tid, n - 1)];
  // page index and in-page offset of each valid position (table entry 0 is
  // read for the others, so the four table reads carry no predicate either)
  const uint32_t pu = (uint32_t)P;
  bool ok[kRounds];
  uint32_t pi[kRounds], po[kRounds];
#pragma unroll
  for (int k = 0; k < kRounds; ++k) {
    ok[k] = 256 * k + tid < n && pos[k] >= 0 && pos[k] < len;
    const uint32_t p = ok[k] ? (uint32_t)pos[k] : 0u;
    pi[k] = p / pu;
    po[k] = p - pi[k] * pu;
  }
  int pg[kRounds];
#pragma unroll
  for (int k = 0; k < kRounds; ++k) pg[k] = bt[pi[k]];
#pragma unroll
  for (int k = 0; k < kRounds; ++k) {
    const int u = 256 * k + tid;
    const bool valid = ok[k] && pg[k] >= 0 && pg[k] < npg;
    const uint32_t r = valid ? (uint32_t)pg[k] * pu + po[k] : 0u;
    win[u] = kRowBytes * (r - (uint32_t)(u & (kTok - 1)));
    const uint64_t bal = __ballot(valid);
    if (lane == 0) {
      masks[2 * (4 * k + wave)] = (uint32_t)bal;
      masks[2 * (4 * k + wave) + 1] = (uint32_t)(bal >> 32);
    }
  }
}

template <bool kSparse>
__global__ void __launch_bounds__(256, 1) mla_h128_kernel(MlaLaunch a) {
  __shared__ __attribute__((aligned(1024))) unsigned char
      lds_raw[kSparse ? ISK_H128_SPARSE_LDS_BYTES : ISK_H128_LDS_BYTES];
  asm volatile("" ::: ISK_H128_ALL_AGPRS);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // block id -> (task, head block): head blocks of one task sit 8 ids apart
  // (the same XCD under round-robin dealing of workgroups to the 8 XCDs).
  const int n_hb = a.hq / kHeadsPerBlock;
  const int bid = blockIdx.x;
  const int g = (bid / (8 * n_hb)) * 8 + (bid & 7);
  const int hb = (bid >> 3) % n_hb;
  if (g >= a.n_groups) return;
  const bool inl = a.inl.n_segs > 0;
  const int seg_first = inl ? g : a.groups[g], seg_last = inl ? g + 1 : a.groups[g + 1];
  const uint32_t lds = (uint32_t)(uintptr_t)lds_raw;
  ISK_LDS float* const xs = (ISK_LDS float*)(lds_raw + kXOff);   // [n32][ht]

  for (int si = seg_first; si < seg_last; ++si) {
    const Seg sg = fetch_seg(a.inl, a.segs, a.topk_idx != nullptr ? a.topk_len : a.lens, si);
    const int b = sg.row;
    // Every wave is done with the previous segment's LDS.
    __syncthreads();
    const int ntiles = (sg.end - sg.begin + kTok - 1) / kTok;
    float m_ref = -INFINITY, l_run = 0.f;
    if (kSparse && ntiles > 0) {
      const uint16_t* qw = a.q + ((size_t)b * a.hq + hb * kHeadsPerBlock + wave * 32) * kMlaDqk;
      // The source fields are read from the kernel arguments here, per
      // split, rather than held in SGPRs across the tile loop.
      // (constant address space: scalar loads).
      const KArg* sa = (const KArg*)__builtin_amdgcn_kernarg_segment_ptr();
      asm volatile("" : "+s"(sa));
      // A split past the main index width gathers from the extra KV source,
      // at its slots [begin - topk_width, end - topk_width).
      const bool from_extra = sg.begin >= sa->topk_width;
      const int u0 = from_extra ? sg.begin - sa->topk_width : sg.begin;
      const uintptr_t kv = (uintptr_t)(from_extra ? sa->xkv : sa->kv);
      const int P = from_extra ? sa->xpage_size : sa->page_size;
      const int cap = from_extra ? sa->xmax_pages * sa->xpage_size : sa->max_pages * sa->page_size;
      const int len = min(from_extra ? sa->xlens[b] : sa->lens[b], cap);
      const int32_t* idx = from_extra ? sa->xtopk_idx + (size_t)b * sa->xtopk_width + u0
                                      : sa->topk_idx + (size_t)b * sa->topk_width + u0;
      const int32_t* bt = from_extra ? sa->xblock_table + (size_t)b * sa->xmax_pages
                                     : sa->block_table + (size_t)b * sa->max_pages;
      resolve_window(lds_raw, idx, bt, sg.end - sg.begin, len, P, from_extra ? sa->xnum_pages : sa->num_pages, wave);
      __syncthreads();
      asm volatile(ISK_H128_SPARSE_SEG_ASM
                   : "={v224}"(m_ref), "={v225}"(l_run)
                   : [q] "s"(qw), [kv_lo] "s"((uint32_t)kv), [kv_hi] "s"((uint32_t)(kv >> 32)), [ntiles] "s"(ntiles),
                     [scale] "s"(a.scale_log2), [w] "s"(wave), [lds] "s"(lds)
                   : ISK_H128_SEG_CLOBBERS);
    } else if (!kSparse && ntiles > 0) {
      const uint16_t* qw = a.q + ((size_t)b * a.hq + hb * kHeadsPerBlock + wave * 32) * kMlaDqk;
      const uintptr_t kv = (uintptr_t)a.kv;
      const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
      const int P = a.page_size;
      const int pbase = sg.begin / P, on0 = sg.begin % P;
      const int pend = (sg.end + P - 1) / P;   // pages of the row holding tokens below the end
      asm volatile(ISK_H128_SEG_ASM
                   : "={v224}"(m_ref), "={v225}"(l_run)
                   : [q] "s"(qw), [kv_lo] "s"((uint32_t)kv), [kv_hi] "s"((uint32_t)(kv >> 32)), [bt] "s"(bt),
                     [ntiles] "s"(ntiles), [begin] "s"(sg.begin), [end] "s"(sg.end), [P] "s"(P),
                     [npg] "s"(a.num_pages), [pbase] "s"(pbase), [on0] "s"(on0), [pend] "s"(pend),
                     [scale] "s"(a.scale_log2), [w] "s"(wave), [lds] "s"(lds)
                   : ISK_H128_SEG_CLOBBERS);
    } else {
      asm volatile(
          ".irp i, 0,16,32,48,64,80,96,112,128,144,160,176,192,208,224,240\n\t"
          ".irp k, 0,1,2,3,4,5,6,7,8,9,10,11,12,13,14,15\n\t"
          "v_accvgpr_write_b32 a[\\i+\\k], 0\n\t.endr\n\t.endr\n\ts_nop 4" ::: ISK_H128_ALL_AGPRS);
    }

    // The launch arguments are read again here rather than kept in SGPRs
    // across the block.
    const MlaLaunch* ka = (const MlaLaunch*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ka));
    // Lane values are derived here, after the block (which owns every VGPR),
    // so that none has to be kept in memory across it.
    int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(lane));   // no lane-dependent value of the epilogue is computed earlier
    int part = __builtin_amdgcn_readfirstlane(sg.part), brow = __builtin_amdgcn_readfirstlane(b);
    asm volatile("" : "+s"(part), "+s"(brow));
    const int n32 = lane & 31, hh = lane >> 5;
    // ---- o = acc / l, lse = ln 2 (m_ref - 7 + log2 l); the lane pair of a
    // head adds its two halves of l in the same order in both lanes.
    float l_tot;
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
      l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const bool empty = !(l_tot > 0.f);
    const float lse_v = empty ? -INFINITY : (m_ref - kPShift + fast_log2(l_tot)) * kLn2;
    __syncthreads();   // every wave is done with the last alphas
    if (hh == 0) xs[4 * n32 + wave] = l_tot;
    __syncthreads();
    // inv of the head tile of accumulator group gg: (gg + wave) & 3
    float inv[4];
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const float l = xs[4 * n32 + ((gg + wave) & 3)];
      inv[gg] = l > 0.f ? 1.f / l : 0.f;
    }
    asm volatile("s_nop 7\n\ts_nop 7");
    const int head = hb * kHeadsPerBlock + wave * 32 + n32;
    const bool to_part = part >= 0;
    const size_t row0 = (to_part ? (size_t)part : (size_t)brow) * ka->hq + (size_t)hb * kHeadsPerBlock;   // head 0 of the block
    if (to_part) {
      if (hh == 0) ka->part_lse[(size_t)part * ka->hq + head] = lse_v;
    } else if (ka->lse != nullptr && hh == 0) {
      ka->lse[(size_t)brow * ka->hq + head] = lse_v;
    }
    // Output rows [row0, row0 + 128): fp32 (2 KB a row: fp32 output, or
    // partials of an fp32-output launch), bf16 output or fp16 partials (1 KB).
    const int fmt = to_part ? (ka->part_f16 ? kFmtF16 : kFmtF32) : (ka->out_f32 ? kFmtF32 : kFmtBF16);
    const size_t esz = fmt == kFmtF32 ? 4 : 2;
    // The launch arguments come from the kernarg segment, so the compiler
    // no longer knows the pointers are global memory: say so, and keep the
    // block base uniform (scalar base + 32-bit lane offset stores).
    const uintptr_t base = (uintptr_t)((unsigned char*)(to_part ? (void*)ka->part_o : ka->out) + row0 * kMlaDv * esz);
    GU8* const blk = (GU8*)(((uintptr_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base));
    // The output block goes through LDS (the tile buffers are free now) so
    // that every store instruction writes whole rows of the output: round dt
    // stages dims 32 dt .. 32 dt + 31 of the wave's 128 for all 128 heads
    // ([head][dim], rows padded to 144 bytes against bank conflicts), then
    // eight lanes write one head's 32 dims.
    ISK_LDS float* const stage = (ISK_LDS float*)(lds_raw + wave * (kHeadsPerBlock * kStageRow));
    const int sh = lane >> 3, sc = lane & 7;
    auto stage_tile = [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      constexpr int gg = t & 3;
      const int ht = (gg + wave) & 3;
      float o[16];
      acc_read<t>(o);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 r = f32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]} * inv[gg];
        *(ISK_LDS f32x4*)(stage + ((32 * ht + n32) * kStageRow + 32 * q + 16 * hh) / 4) = r;
      }
    };
    // One round: the 16 reads of the staged rows are all issued before the
    // first store; FMT is the row format.
    auto rounds = [&](auto fc) {
      constexpr int FMT = decltype(fc)::value;
      constexpr uint32_t esz = FMT == kFmtF32 ? 4 : 2;
      auto store_round = [&](int dt) {
        asm volatile("" ::: "memory");   // the round's staging writes come first (other lanes read them)
        f32x4 r[16];
#pragma unroll
        for (int s16 = 0; s16 < 16; ++s16)
          r[s16] = *(const ISK_LDS f32x4*)(stage + ((8 * s16 + sh) * kStageRow + 16 * sc) / 4);
        uint32_t voff = ((uint32_t)sh * kMlaDv + 128u * wave + 32u * dt + 4u * sc) * esz;
#pragma unroll
        for (int s16 = 0; s16 < 16; ++s16) {
          if constexpr (FMT == kFmtF32) {
            *(GF32x4*)(blk + voff) = r[s16];
          } else if constexpr (FMT == kFmtBF16) {
            *(GU32x2*)(blk + voff) = u32x2{pack_bf16x2(r[s16][0], r[s16][1]), pack_bf16x2(r[s16][2], r[s16][3])};
          } else {
            *(GU32x2*)(blk + voff) = u32x2{pack_f16x2(r[s16][0], r[s16][1]), pack_f16x2(r[s16][2], r[s16][3])};
          }
          voff += 8u * kMlaDv * esz;
          asm volatile("" : "+v"(voff));
        }
        asm volatile("" ::: "memory");   // the reads come before the next round's writes
      };
      stage_tile(std::integral_constant<int, 0>{}); stage_tile(std::integral_constant<int, 1>{});
      stage_tile(std::integral_constant<int, 2>{}); stage_tile(std::integral_constant<int, 3>{});
      store_round(0);
      stage_tile(std::integral_constant<int, 4>{}); stage_tile(std::integral_constant<int, 5>{});
      stage_tile(std::integral_constant<int, 6>{}); stage_tile(std::integral_constant<int, 7>{});
      store_round(1);
      stage_tile(std::integral_constant<int, 8>{}); stage_tile(std::integral_constant<int, 9>{});
      stage_tile(std::integral_constant<int, 10>{}); stage_tile(std::integral_constant<int, 11>{});
      store_round(2);
      stage_tile(std::integral_constant<int, 12>{}); stage_tile(std::integral_constant<int, 13>{});
      stage_tile(std::integral_constant<int, 14>{}); stage_tile(std::integral_constant<int, 15>{});
      store_round(3);
    };
    __syncthreads();   // every wave is done with the tile buffers
    if (fmt == kFmtF32)
      rounds(std::integral_constant<int, kFmtF32>{});
    else if (fmt == kFmtBF16)
      rounds(std::integral_constant<int, kFmtBF16>{});
    else
      rounds(std::integral_constant<int, kFmtF16>{});
  }
}

}  // namespace

hipError_t launch_mla_h128(const MlaLaunch& a, hipStream_t s, const LaunchEvents& ev) {
  if (a.n_groups == 0) return hipSuccess;
  if (a.hq % kHeadsPerBlock != 0) return hipErrorInvalidValue;
  const int n_hb = a.hq / kHeadsPerBlock;
  const int n_blocks = ((a.n_groups + 7) / 8) * 8 * n_hb;
  if (a.topk_idx == nullptr) return launch_one(mla_h128_kernel<false>, dim3(n_blocks), dim3(64 * kWaves), s, a, ev);
  // Sparse: every split fits the window and every pool the 32-bit offsets.
  if (a.max_seg_units > ISK_H128_WIN_SLOTS || !mla_h128_pool_fits(a.num_pages, a.page_size) ||
      (a.xtopk_idx != nullptr && !mla_h128_pool_fits(a.xnum_pages, a.xpage_size)))
    return hipErrorInvalidValue;
  return launch_one(mla_h128_kernel<true>, dim3(n_blocks), dim3(64 * kWaves), s, a, ev);
}

}  // namespace isk
