// Absorbed-MLA split kernel for gfx950 (dense and sparse top-k).
//
// One workgroup runs the splits ("segments") of one task; for each segment it
// computes, for all query heads of one batch row, softmax attention over the
// segment's tokens and writes either the partial (o_i, lse_i) or, for a row
// with a single split, the final output.  This is the split stage of the
// split-KV scheme on the FlashMLA issue page "Sparse MLA decode is not
// batch-invariant ..." (section "Where it comes from"); the split boundaries
// come from the host planner and depend only on the row's own length.
//
// Data flow per 64-token tile (kMlaTile):
//   * The tile's latent rows (576 bf16 = 72 pieces of 16 B each) are copied
//     straight from HBM into LDS with 16-byte global->LDS loads, double
//     buffered: tile t+1 streams in while tile t is computed.  Piece c of
//     tile row t sits at LDS piece (t*72 + (c ^ h(t))) with the XOR key
//     h(t) = 4*((t >> 1) & 1) + ((t >> 3) & 3): the 16 rows one MFMA operand
//     read touches (8 rows apart, see qk_token) get 8 distinct keys per row
//     parity, so a 16-lane phase of that read hits 16 distinct 16-byte bank
//     groups.
//     Masked rows (past the split end, sparse slots that are -1 or out of
//     range, pages outside the pool) are written as zeros instead of loaded.
//   * Each wave owns 16 query heads and keeps their query slice in
//     registers as the B operand of S^T = K * Q^T (v_mfma_f32_16x16x32_bf16,
//     fp32 accumulation).  The 16 token rows of each M-tile are permuted so
//     that the S^T result already sits in the lane layout of the PV operand.
//   * Online softmax in fp32 with exp2: per head, running max m (butterfly
//     max over the 4 lane groups), rescale alpha = 2^(m_old - m_new),
//     p = 2^(x - m_new).  For the bf16 MFMA, p is split into p_hi = bf16(p)
//     and p_lo = bf16(p - p_hi); the PV product runs on both, so the weights
//     carry ~16 significant bits; the normaliser l sums the fp32 p.
//   * O^T += V^T * P^T on MFMA with V^T read from the same LDS tile through
//     the transposing read ds_read_b64_tr_b16 (V is the first 512 columns of
//     the latent row).
// Every reduction order above is fixed by the segment's own token range, so
// the bits of a segment's result do not depend on anything else in the batch.

#include "device.hpp"
#include "isk_internal.hpp"

namespace isk {
namespace {

constexpr int kPieces = kMlaDqk / 8;                   // 72 pieces per latent row
constexpr int kRowBytes = kMlaDqk * 2;                 // 1152
constexpr int kTileBytes = kMlaTile * kRowBytes;       // 73728
constexpr int kTileInstr = kMlaTile * kPieces / 64;    // 72 wave-wide 16B loads per tile
constexpr int kKSteps = kMlaDqk / 32;                  // 18 MFMA k-steps for Q.K
constexpr int kDvTiles = kMlaDv / 16;                  // 32 output dim tiles

// Token (row of the tile) held by S^T row m of M-tile tau.  M-tiles 2k and
// 2k+1 together cover tokens [32k, 32k+32); lane group g (= m >> 2) gets
// tokens 32k + 8g + {0..3} from tile 2k and 32k + 8g + {4..7} from 2k+1,
// exactly the 8 consecutive tokens its PV operand needs.
__device__ __forceinline__ int qk_token(int tau, int m) {
  return 32 * (tau >> 1) + 8 * (m >> 2) + 4 * (tau & 1) + (m & 3);
}

// XOR key of tile row t (< 8, so c ^ key stays inside c's aligned block of 8
// pieces and inside the 72-piece row).
__device__ __forceinline__ int swz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 3) & 3); }

// Staging offsets of a four-wave workgroup: wave w issues the 18 wave-wide
// loads i = w + 4j of a tile; lane l of load i fills LDS piece slot
// p = 64*i + l, i.e. tile row t = p / 72, latent piece (p % 72) ^ swz(t).
// These byte offsets within the tile's source rows do not change from tile to
// tile, so they are computed once.
struct StageOffsets {
  int off[kTileInstr / 4];
  int row[kTileInstr / 4];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < kTileInstr / 4; ++j) {
      const int p = (wave + 4 * j) * 64 + lane;
      const int t = p / kPieces;
      const int c = (p - t * kPieces) ^ swz(t);
      off[j] = t * kRowBytes + c * 16;
      row[j] = t;
    }
  }
};

template <bool kSparse>
struct Stager {
  const unsigned char* kv;      // pool base (bytes)
  const int32_t* bt_row;        // block table row of the segment's batch row
  const int32_t* idx_row;       // sparse: top-k index row
  int page_size, num_pages, len, seg_begin, seg_end;

  // Issue the loads of tile `it` into `buf`; returns the tile's row-valid mask.
  __device__ __forceinline__ uint64_t operator()(int it, ISK_LDS unsigned char* buf, int wave, int nw,
                                                 int lane, const StageOffsets& so) const {
    // Partial tiles and the sparse path recompute their per-lane addresses
    // here rather than keep them live across the tile loop.
    asm volatile("" : "+v"(lane));
    const int u0 = seg_begin + it * kMlaTile;
    uint64_t mask;
    uint32_t my_row = 0;        // pool row index of tile row `lane` (sparse)
    const unsigned char* dense_base = kv;
    if constexpr (kSparse) {
      const int slot = u0 + lane;
      bool ok = slot < seg_end;
      const int pos = ok ? idx_row[slot] : -1;
      ok = ok && pos >= 0 && pos < len;
      const int pg = ok ? bt_row[pos / page_size] : 0;
      ok = ok && pg >= 0 && pg < num_pages;
      my_row = ok ? (uint32_t)pg * (uint32_t)page_size + (uint32_t)(pos % page_size) : 0u;
      mask = __ballot(ok);
    } else {
      // Tiles start at multiples of 64 and pages hold a multiple of 64 tokens,
      // so a tile is one contiguous run of rows inside one page.
      const int nvalid = min(kMlaTile, seg_end - u0);
      const int pg = bt_row[u0 / page_size];
      const bool page_ok = pg >= 0 && pg < num_pages;
      mask = !page_ok ? 0ull : (nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1ull));
      if (page_ok)
        dense_base = kv + ((size_t)pg * page_size + (u0 % page_size)) * (size_t)kRowBytes;
      if (nw == 4 && mask == ~0ull) {
        // Full tile of a four-wave workgroup: precomputed offsets, no checks.
#pragma unroll
        for (int j = 0; j < kTileInstr / 4; ++j) load_lds_16_stream(dense_base + so.off[j], buf + (wave + 4 * j) * 1024);
        return mask;
      }
    }
    for (int i = wave; i < kTileInstr; i += nw) {
      const int p = i * 64 + lane;             // LDS piece slot written by this lane
      const int t = p / kPieces;               // tile row
      const int c = (p - t * kPieces) ^ swz(t);    // latent piece stored there
      ISK_LDS unsigned char* chunk = buf + i * 1024;
      const bool valid = (mask >> t) & 1ull;
      const unsigned char* src;
      if constexpr (kSparse) {
        const uint32_t r = (uint32_t)__shfl((int)my_row, t, 64);
        src = kv + (size_t)r * kRowBytes + c * 16;
      } else {
        src = dense_base + (size_t)t * kRowBytes + c * 16;
      }
      if (valid) {
        if constexpr (kSparse)
          load_lds_16(src, chunk);
        else
          load_lds_16_stream(src, chunk);
      } else {
        *(ISK_LDS f32x4*)(buf + p * 16) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    return mask;
  }
};

// Lazy rescale threshold (log2 units): the softmax reference max of a head
// only moves when the head's running max exceeds it by more than this, so the
// accumulator rescale (3 instructions per AGPR) runs a handful of times per
// split instead of every tile.  p = 2^(x - m_ref) stays below 2^8.
constexpr float kRescaleThreshold = 8.0f;

// Prefetch distance (in MFMA steps) of the V^T operand reads.
constexpr int kVDepth = 4;

// Heads: each wave computes the scores and softmax of 16 query heads; a
// workgroup of up to four waves (one per SIMD) owns up to 64 heads.  With
// fewer than 64 heads (16 or 32) the four waves still run, KDS = 64 / Hq
// waves per head group: they compute the same scores and softmax (the same
// operations, so the same bits) and split the 32 output dim tiles between
// them, each doing 32 / KDS of the PV product.  With more than 64 heads the
// split runs as several workgroups ("head blocks") that read the same KV
// tiles; their block ids are g + 8*hb so that they land on the same XCD
// (workgroups are dealt to the 8 XCDs round-robin by id) one right after the
// other and the second read of a tile is served by that XCD's L2.
constexpr int kH2 = 1;

template <bool kSparse, int KDS>
__global__ void __launch_bounds__(256, 1) mla_split_kernel(MlaLaunch a) {
  constexpr int kNt = kDvTiles / KDS;   // output dim tiles of this wave
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[2 * kTileBytes];
  ISK_LDS unsigned char* lds = (ISK_LDS unsigned char*)lds_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int i16 = lane & 15, g16 = lane >> 4;
  // block id -> (task g, head block hb); see the comment above the kernel.
  const int n_groups16 = nw / KDS;   // head groups of 16 in this workgroup
  const int n_hb = a.hq / (n_groups16 * 16);
  const int bid = blockIdx.x;
  const int g = (bid / (8 * n_hb)) * 8 + (bid & 7);
  const int hb = (bid >> 3) % n_hb;
  if (g >= a.n_groups) return;
  const int hg = wave % n_groups16, dpart = wave / n_groups16;   // head group, part of the dims
  const int head0 = hb * n_groups16 * 16 + hg * 16 + i16;
  const bool inl = a.inl.n_segs > 0;   // segments by value: one per task
  const int seg_first = inl ? g : a.groups[g], seg_last = inl ? g + 1 : a.groups[g + 1];
  const unsigned char* kv = (const unsigned char*)a.kv;

  // Per-lane LDS byte offsets of the MFMA operand reads.  With the XOR key
  // swz(), each operand address splits into a per-lane part (below, one per
  // parity of the k-step or per dim tile modulo 4) and a compile-time part.
  //  K operand, M-tile tau, k-step kk, lane (a = i16>>2, b = i16&3, g = g16):
  //    row 32*(tau>>1) + 4*(tau&1) + 8a + b, piece 4kk + g, key 4*(b>>1) + a.
  //  V^T operand, k-step kap, read r, dim tile nt, lane (ts = i16>>2, q = i16&3):
  //    row 32*kap + 4r + 8*g16 + ts, piece 2nt + (q>>1), byte 8*(q&1), key 4*(ts>>1) + g16.
  int k_lane_off[2], v_lane_off[4];
  {
    const int a4 = i16 >> 2, b4 = i16 & 3;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      k_lane_off[par] = kRowBytes * (8 * a4 + b4) + 64 * (par ^ (b4 >> 1)) + 16 * (g16 ^ a4);
    const int ts = i16 >> 2, q = i16 & 3;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      v_lane_off[m] = kRowBytes * (8 * g16 + ts) + 64 * (((m >> 1) & 1) ^ (ts >> 1)) + 32 * ((m & 1) ^ (g16 >> 1)) +
                      16 * ((q >> 1) ^ (g16 & 1)) + 8 * (q & 1) + 128 * (kNt / 4) * dpart;
  }
  StageOffsets so;
  if (nw == 4) so.init(wave, lane);

  // Compile-time part of the operand addresses.
  auto k_tile_off = [](int tau, int kk) {
    return kRowBytes * (32 * (tau >> 1) + 4 * (tau & 1)) + 128 * (kk >> 1);
  };
  // step j: k-step kap = j / kNt, this wave's dim tile nt = j % kNt (dim
  // tile kNt*dpart + nt of the row; its part of the offset is in v_lane_off)
  auto v_read = [&](const ISK_LDS unsigned char* T, int j, s16x4* dst) {
    const int kap = j / kNt, nt = j % kNt;
    const ISK_LDS unsigned char* vb = T + v_lane_off[nt & 3];
    dst[0] = lds_read_tr16(vb + kRowBytes * 32 * kap + 128 * (nt >> 2));
    dst[1] = lds_read_tr16(vb + kRowBytes * (32 * kap + 4) + 128 * (nt >> 2));
  };

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
    Stager<kSparse> stage =
        from_extra ? Stager<kSparse>{(const unsigned char*)a.xkv, a.xblock_table + (size_t)b * a.xmax_pages,
                                     a.xtopk_idx + (size_t)b * a.xtopk_width, a.xpage_size, a.xnum_pages,
                                     min(a.xlens[b], a.xmax_pages * a.xpage_size), sg.begin, sg.end}
                   : Stager<kSparse>{kv, a.block_table + (size_t)b * a.max_pages,
                                     kSparse ? a.topk_idx + (size_t)b * a.topk_width : nullptr, a.page_size,
                                     a.num_pages, min(a.lens[b], a.max_pages * a.page_size), sg.begin, sg.end};

    __syncthreads();   // every wave is done with the LDS tiles of the previous segment

    // Query slices as MFMA B operands: lane (i16, g16) of half h2 holds
    // q[head0 + 16*h2][32*kk + 8*g16 + 0..7].
    bf16x8 qf[kH2][kKSteps];
#pragma unroll
    for (int h2 = 0; h2 < kH2; ++h2) {
      const bf16x8* qrow =
          (const bf16x8*)(a.q + ((size_t)b * a.hq + head0 + 16 * h2) * kMlaDqk + 8 * g16);
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) qf[h2][kk] = qrow[4 * kk];
    }

    float m_ref[kH2], l_run[kH2];
    f32x4 acc[kH2][kNt];
#pragma unroll
    for (int h2 = 0; h2 < kH2; ++h2) {
      m_ref[h2] = -INFINITY;
      l_run[h2] = 0.f;
#pragma unroll
      for (int nt = 0; nt < kNt; ++nt) acc[h2][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int n_tiles = (sg.end - sg.begin + kMlaTile - 1) / kMlaTile;
    uint64_t mask_next = n_tiles > 0 ? stage(0, lds, wave, nw, lane, so) : 0ull;

    for (int it = 0; it < n_tiles; ++it) {
      wait_vmem_all();
      __syncthreads();   // tile `it` has landed; tile it-1's buffer is free
      const uint64_t mask = mask_next;
      ISK_LDS unsigned char* T = lds + (it & 1) * kTileBytes;
      if (it + 1 < n_tiles) mask_next = stage(it + 1, lds + ((it + 1) & 1) * kTileBytes, wave, nw, lane, so);

      // ---- S^T = K * Q^T for 64 tokens x 16 heads per half (4 M-tiles)
      // Operand A of M-tile tau, k-step kk: lane (i16, g16) reads piece
      // (4*kk + g16) of tile row qk_token(tau, i16).  With the XOR swizzle
      // that address splits into a per-lane base plus a compile-time offset.
      f32x4 s[kH2][4];
#pragma unroll
      for (int h2 = 0; h2 < kH2; ++h2)
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) s[h2][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        // Software pipeline: the 4 operand reads of step kk+1 are issued before
        // the MFMAs of step kk; the scheduling fences keep the compiler from
        // hoisting further reads (which would cost registers, not time).
        bf16x8 kf[2][4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) kf[0][tau] = *(const ISK_LDS bf16x8*)(T + k_lane_off[0] + k_tile_off(tau, 0));
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
          const int cur = kk & 1;
          if (kk + 1 < kKSteps) {
#pragma unroll
            for (int tau = 0; tau < 4; ++tau)
              kf[cur ^ 1][tau] = *(const ISK_LDS bf16x8*)(T + k_lane_off[(kk + 1) & 1] + k_tile_off(tau, kk + 1));
          }
#pragma unroll
          for (int tau = 0; tau < 4; ++tau) {
#pragma unroll
            for (int h2 = 0; h2 < kH2; ++h2)
              s[h2][tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[cur][tau], qf[h2][kk], s[h2][tau], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- online softmax (log2 domain); lane holds head (head0 + 16*h2) and
      // tokens 32*(tau>>1) + 8*g16 + 4*(tau&1) + j, tau = 0..3, j = 0..3
      bf16x8 pb[kH2][2], pl[kH2][2];
      bool any_rescale = false;
      float alpha[kH2];
#pragma unroll
      for (int h2 = 0; h2 < kH2; ++h2) {
        float mx = -INFINITY;
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int tok = 32 * (tau >> 1) + 8 * g16 + 4 * (tau & 1) + j;
            const bool v = (mask >> tok) & 1ull;
            s[h2][tau][j] = v ? s[h2][tau][j] * a.scale_log2 : -INFINITY;
            mx = fmaxf(mx, s[h2][tau][j]);
          }
        }
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        // Move the reference only when the max outgrows it by the threshold.
        const float m_old = m_ref[h2];
        const bool move = mx > m_old + kRescaleThreshold || (m_old == -INFINITY && mx > -INFINITY);
        const float m_new = move ? mx : m_old;
        alpha[h2] = move ? fast_exp2(m_old - m_new) : 1.0f;   // m_old = -inf -> 0
        any_rescale |= move && m_old != -INFINITY;            // acc is still 0 before the first move
        m_ref[h2] = m_new;
        const float m_sub = m_new == -INFINITY ? 0.f : m_new;

        // p = 2^(x - m) in fp32 is split into bf16 p_hi + p_lo (p_lo = the
        // rounding residual, itself rounded); both feed the PV product, which
        // keeps the relative weight error near 2^-17 instead of bf16's 2^-9.
        // The normaliser sums the fp32 p.
        float psum = 0.f;
#pragma unroll
        for (int kap = 0; kap < 2; ++kap) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int tau = 2 * kap + h;
            float p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) p[j] = fast_exp2(s[h2][tau][j] - m_sub);
            const bf16x2 h01 = to_bf16x2(p[0], p[1]);
            const bf16x2 h23 = to_bf16x2(p[2], p[3]);
            const bf16x2 l01 = to_bf16x2(p[0] - (float)h01[0], p[1] - (float)h01[1]);
            const bf16x2 l23 = to_bf16x2(p[2] - (float)h23[0], p[3] - (float)h23[1]);
            pb[h2][kap][4 * h + 0] = h01[0];
            pb[h2][kap][4 * h + 1] = h01[1];
            pb[h2][kap][4 * h + 2] = h23[0];
            pb[h2][kap][4 * h + 3] = h23[1];
            pl[h2][kap][4 * h + 0] = l01[0];
            pl[h2][kap][4 * h + 1] = l01[1];
            pl[h2][kap][4 * h + 2] = l23[0];
            pl[h2][kap][4 * h + 3] = l23[1];
#pragma unroll
            for (int j = 0; j < 4; ++j) psum += p[j];
          }
        }
        l_run[h2] = l_run[h2] * alpha[h2] + psum;
      }
      // Wave-uniform skip: lanes that did not move have alpha == 1 exactly,
      // and multiplying by 1 would not change their bits.
      if (__ballot(any_rescale) != 0ull) {
#pragma unroll
        for (int h2 = 0; h2 < kH2; ++h2)
#pragma unroll
          for (int nt = 0; nt < kNt; ++nt) acc[h2][nt] *= alpha[h2];
      }

      // ---- O^T += V^T * P^T; V^T operand via transposing LDS reads.
      // For k-step kap and dim tile nt, lane (i16, g16) addresses 4 dims of
      // tile rows 32*kap + 8*g16 + (i16 >> 2) (+4 for the second read).
      {
        // 2 kNt steps (kap, nt); the two transposing reads of step j + kVDepth
        // are issued before the MFMAs of step j.
        constexpr int kSteps = 2 * kNt;
        s16x4 vr[kVDepth][2];
#pragma unroll
        for (int j = 0; j < kVDepth; ++j) v_read(T, j, vr[j]);
#pragma unroll
        for (int j = 0; j < kSteps; ++j) {
          const int kap = j / kNt, nt = j % kNt;
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(vr[j % kVDepth][0], vr[j % kVDepth][1], 0, 1, 2, 3, 4, 5, 6, 7));
          if (j + kVDepth < kSteps) v_read(T, j + kVDepth, vr[j % kVDepth]);
#pragma unroll
          for (int h2 = 0; h2 < kH2; ++h2) {
            acc[h2][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[h2][kap], acc[h2][nt], 0, 0, 0);
            acc[h2][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[h2][kap], acc[h2][nt], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // ---- epilogue: o = acc / l, lse = ln(2) * (m_ref + log2 l)
#pragma unroll
    for (int h2 = 0; h2 < kH2; ++h2) {
      const int head = head0 + 16 * h2;
      float l_tot = wave_add_xor(l_run[h2], 16);
      l_tot = wave_add_xor(l_tot, 32);
      const bool empty = !(l_tot > 0.f);
      const float inv = empty ? 0.f : 1.f / l_tot;
      const float lse_v = empty ? -INFINITY : (m_ref[h2] + fast_log2(l_tot)) * kLn2;
      // this wave's dims: dim tiles kNt*dpart .. ; the LSE from the first part
      const int d0 = 16 * kNt * dpart;
      if (sg.part >= 0) {
        float* po = a.part_o + ((size_t)sg.part * a.hq + head) * kMlaDv + d0 + 4 * g16;
#pragma unroll
        for (int nt = 0; nt < kNt; ++nt) *(f32x4*)(po + 16 * nt) = acc[h2][nt] * inv;
        if (g16 == 0 && dpart == 0) a.part_lse[(size_t)sg.part * a.hq + head] = lse_v;
      } else {
        const size_t ob = ((size_t)b * a.hq + head) * kMlaDv + d0 + 4 * g16;
        if (a.out_f32) {
          float* o = (float*)a.out + ob;
#pragma unroll
          for (int nt = 0; nt < kNt; ++nt) *(f32x4*)(o + 16 * nt) = acc[h2][nt] * inv;
        } else {
          uint16_t* o = (uint16_t*)a.out + ob;
#pragma unroll
          for (int nt = 0; nt < kNt; ++nt) {
            const f32x4 r = acc[h2][nt] * inv;
            uint2 w;
            w.x = pack_bf16x2(r[0], r[1]);
            w.y = pack_bf16x2(r[2], r[3]);
            *(uint2*)(o + 16 * nt) = w;
          }
        }
        if (a.lse != nullptr && g16 == 0 && dpart == 0) a.lse[(size_t)b * a.hq + head] = lse_v;
      }
    }
  }
}

}  // namespace

hipError_t launch_mla_split(const MlaLaunch& a, hipStream_t s, const LaunchEvents& ev) {
  if (a.n_groups == 0) return hipSuccess;
  // Heads per workgroup: all of them up to 64, else 64 (hq % 64 == 0 is
  // checked by the planner).  16 and 32 heads run four waves that split the
  // output dims; 48 heads run three waves.
  const int hw = a.hq <= 64 ? a.hq : 64;
  const int n_hb = a.hq / hw;
  const int n_blocks = ((a.n_groups + 7) / 8) * 8 * n_hb;
  const dim3 grid(n_blocks);
  const bool sp = a.topk_idx != nullptr;
  if (hw == 16)
    return sp ? launch_one(mla_split_kernel<true, 4>, grid, dim3(256), s, a, ev)
              : launch_one(mla_split_kernel<false, 4>, grid, dim3(256), s, a, ev);
  if (hw == 32)
    return sp ? launch_one(mla_split_kernel<true, 2>, grid, dim3(256), s, a, ev)
              : launch_one(mla_split_kernel<false, 2>, grid, dim3(256), s, a, ev);
  const dim3 block(hw * 4);
  return sp ? launch_one(mla_split_kernel<true, 1>, grid, block, s, a, ev)
            : launch_one(mla_split_kernel<false, 1>, grid, block, s, a, ev);
}

}  // namespace isk
