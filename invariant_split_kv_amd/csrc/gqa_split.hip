// Dense grouped-query split kernel for gfx950.
//
// One workgroup runs the splits of one task for one kv head: for each split
// ("segment") it computes softmax attention of the G query heads that share
// that kv head over the segment's tokens, then writes the partial
// (o_i, lse_i) of the split-KV scheme (FlashMLA issue page "Sparse MLA decode
// is not batch-invariant ...", section "Where it comes from"), or the final
// output when the row has a single split.
//
// The work per token is G*(2*D) multiply-adds against 4*D bytes of K and V,
// about 4 FLOP per byte for G = 4, so the kernel is bound by HBM, not by the
// matrix cores; it uses vector ALU arithmetic:
//   * 64-token K and V tiles of the kv head are copied HBM -> LDS with 16-byte
//     direct loads, double buffered.  Piece c (8 dims) of tile row t is stored
//     at piece (c ^ (t & 7)) of that row, so that 8 lanes reading the same
//     column of 8 consecutive rows hit distinct banks.
// Two layouts share that staging.  With G = 4, 8 or 16 the four waves split
// each tile by tokens (gqa_tok_kernel, described there).  With G < 4
// (gqa_split_kernel) 4/G waves take each head and split its output dims:
//   * Scores: lane t owns token t of the tile and accumulates the dot product
//     with packed bf16 pairs (v_dot2_f32_bf16, fp32 accumulate), in a fixed
//     dimension order.
//   * Softmax per head: wave-wide butterfly max, p = 2^(x - m) in fp32; each
//     lane keeps a partial normaliser for its token slot, summed by a fixed
//     butterfly at the end of the segment.
//   * PV: each lane owns one output dim and accumulates p_t * v_t[d] in
//     fp32 over the tile's tokens in order.

#include "device.hpp"
#include "isk_internal.hpp"

namespace isk {
namespace {

constexpr int kTile = kGqaTile;   // 64 tokens per tile, one per lane

template <int D>
struct GqaShape {
  static constexpr int kPieces = D / 8;                 // 16-byte pieces per row
  static constexpr int kTileBytes = kTile * D * 2;      // one of K or V
  static constexpr int kInstr = kTile * kPieces / 64;   // wave-wide 16B loads per tile
  static constexpr int kDimsPerLane = D / 64;
};

template <int D>
__device__ __forceinline__ uint64_t gqa_stage(const GqaLaunch& a, int b, int hk, int u0, int seg_end,
                                              ISK_LDS unsigned char* kbuf, ISK_LDS unsigned char* vbuf,
                                              int wave, int nw, int lane) {
  using S = GqaShape<D>;
  asm volatile("" : "+v"(lane));   // keep per-lane addresses out of the loop preheader
  const int P = a.page_size;
  // Token row `lane` of this tile: its pool offset (in elements) of K; V is
  // Hkv*P*D elements further.
  const int pos = u0 + lane;
  bool ok = pos < seg_end;
  const int pg = ok ? a.block_table[(size_t)b * a.max_pages + pos / P] : 0;
  ok = ok && pg >= 0 && pg < a.num_pages;
  const size_t my_off = ok ? ((((size_t)pg * 2) * a.hkv + hk) * P + pos % P) * (size_t)D : 0;
  const uint64_t mask = __ballot(ok);
  const size_t v_delta = (size_t)a.hkv * P * D;
  const unsigned char* kv = (const unsigned char*)a.kv;
  for (int i = wave; i < S::kInstr; i += nw) {
    const int p = i * 64 + lane;
    const int t = p / S::kPieces;
    const int c = (p % S::kPieces) ^ (t & 7);
    const bool valid = (mask >> t) & 1ull;
    const size_t off = (size_t)__shfl((long long)my_off, t, 64);
    if (valid) {
      const unsigned char* src = kv + (off + (size_t)c * 8) * 2;
      load_lds_16_stream(src, kbuf + i * 1024);
      load_lds_16_stream(src + v_delta * 2, vbuf + i * 1024);
    } else {
      *(ISK_LDS f32x4*)(kbuf + p * 16) = f32x4{0.f, 0.f, 0.f, 0.f};
      *(ISK_LDS f32x4*)(vbuf + p * 16) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  return mask;
}

// One or two query heads per kv head (G < 4): four waves, 4/G of them per
// head.  The waves of a head compute its scores and softmax with the same
// operations (so the same bits) and split its D output dims, D/(4/G) each,
// one dim per lane (lanes past the wave's dims compute a copy of one and do
// not store it).
template <int D, int G>
__global__ void __launch_bounds__(256) gqa_split_kernel(GqaLaunch a) {
  using S = GqaShape<D>;
  constexpr int kParts = 4 / G;        // waves per head
  constexpr int DW = D / kParts;       // dims of a wave
  static_assert(G == 1 || G == 2, "one or two heads per kv head");
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[4 * S::kTileBytes + 4 * kTile * 4];
  ISK_LDS unsigned char* lds = (ISK_LDS unsigned char*)lds_raw;
  ISK_LDS unsigned char* kbufs = lds;                               // [2][tile]
  ISK_LDS unsigned char* vbufs = lds + 2 * S::kTileBytes;           // [2][tile]
  ISK_LDS float* p_lds = (ISK_LDS float*)(lds + 4 * S::kTileBytes); // [wave][64]

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = wave % G, dp = wave / G;   // head of the wave, part of its dims
  const int hk = blockIdx.y;
  const int task = blockIdx.x;
  const bool inl = a.inl.n_segs > 0;   // segments by value: one per task
  const int seg_first = inl ? task : a.groups[task], seg_last = inl ? task + 1 : a.groups[task + 1];
  ISK_LDS float* my_p = p_lds + wave * kTile;
  // PV: lane owns dim d of the head (a copy of dim dp*DW for lanes >= DW)
  const bool owner = lane < DW;
  const int d = dp * DW + (owner ? lane : 0);
  const int vpiece = d / 8, vin = (d % 8) * 2;

  for (int si = seg_first; si < seg_last; ++si) {
    const Seg sg = fetch_seg(a.inl, a.segs, a.lens, si);
    const int b = sg.row;
    __syncthreads();   // LDS tiles of the previous segment are no longer read

    // q of head G hk + h as packed bf16 pairs
    const int head = hk * G + h;
    uint32_t qv[D / 2];
    {
      const uint4* qrow = (const uint4*)(a.q + ((size_t)b * a.hq + head) * D);
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const uint4 w = qrow[c];
        qv[4 * c + 0] = w.x; qv[4 * c + 1] = w.y;
        qv[4 * c + 2] = w.z; qv[4 * c + 3] = w.w;
      }
    }
    float m_run = -INFINITY, l_lane = 0.f, acc = 0.f;

    const int n_tiles = (sg.end - sg.begin + kTile - 1) / kTile;
    uint64_t mask_next = n_tiles > 0 ? gqa_stage<D>(a, b, hk, sg.begin, sg.end, kbufs, vbufs, wave, 4, lane) : 0ull;

    for (int it = 0; it < n_tiles; ++it) {
      wait_vmem_all();
      __syncthreads();
      const uint64_t mask = mask_next;
      const int cur = it & 1;
      ISK_LDS unsigned char* K = kbufs + cur * S::kTileBytes;
      ISK_LDS unsigned char* V = vbufs + cur * S::kTileBytes;
      if (it + 1 < n_tiles)
        mask_next = gqa_stage<D>(a, b, hk, sg.begin + (it + 1) * kTile, sg.end, kbufs + (cur ^ 1) * S::kTileBytes,
                                 vbufs + (cur ^ 1) * S::kTileBytes, wave, 4, lane);

      // ---- scores: lane = token
      float sc = 0.f;
      {
        const ISK_LDS unsigned char* krow = K + lane * (D * 2);
#pragma unroll
        for (int c = 0; c < S::kPieces; ++c) {
          const u32x4 kp = *(const ISK_LDS u32x4*)(krow + ((c ^ (lane & 7)) * 16));
          sc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[4 * c + 0]), as_bf16x2(kp[0]), sc, false);
          sc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[4 * c + 1]), as_bf16x2(kp[1]), sc, false);
          sc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[4 * c + 2]), as_bf16x2(kp[2]), sc, false);
          sc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[4 * c + 3]), as_bf16x2(kp[3]), sc, false);
        }
      }

      // ---- softmax of the head (log2 domain)
      const bool valid = (mask >> lane) & 1ull;
      const float x = valid ? sc * a.scale_log2 : -INFINITY;
      float mx = x;
#pragma unroll
      for (int sh = 1; sh < 64; sh <<= 1) mx = wave_max_xor(mx, sh);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      const float p = fast_exp2(x - m_use);
      l_lane = l_lane * alpha + p;
      acc *= alpha;
      my_p[lane] = p;
      // p of this wave is read back by the same wave only.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // ---- PV: dim d over the tile's tokens in order
#pragma unroll 4
      for (int t4 = 0; t4 < kTile; t4 += 4) {
        const f32x4 pw = *(const ISK_LDS f32x4*)(my_p + t4);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = t4 + u;
          const ISK_LDS unsigned char* vp = V + t * (D * 2) + ((vpiece ^ (t & 7)) * 16) + vin;
          const float v = __uint_as_float((uint32_t)(*(const ISK_LDS uint16_t*)vp) << 16);
          acc = fmaf(pw[u], v, acc);
        }
      }
    }

    // ---- epilogue
    float l_tot = l_lane;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) l_tot = wave_add_xor(l_tot, sh);
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_v = empty ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;
    const float o = acc * inv;
    if (sg.part >= 0) {
      if (owner) a.part_o[((size_t)sg.part * a.hq + head) * D + d] = o;
      if (lane == 0 && dp == 0) a.part_lse[(size_t)sg.part * a.hq + head] = lse_v;
    } else {
      const size_t ob = ((size_t)b * a.hq + head) * D + d;
      if (owner) {
        if (a.out_f32) ((float*)a.out)[ob] = o;
        else ((uint16_t*)a.out)[ob] = (uint16_t)(pack_bf16x2(o, 0.f) & 0xffffu);
      }
      if (a.lse != nullptr && lane == 0 && dp == 0) a.lse[(size_t)b * a.hq + head] = lse_v;
    }
  }
}

// Four, eight or sixteen query heads per kv head (G = 4, 8, 16): the four
// waves split each 64-token tile by tokens instead of by heads.  Wave w takes tile rows
// 16w..16w+15 for all G heads, so a tile's K and V rows are each read and
// converted by one wave only, and every wave keeps its own online-softmax
// state:
//   * scores: lane (h, t) = (lane / (64/G), lane % (64/G)) scores rows
//     16w + (64/G) r + t, r < G/4, against head h (the G lanes of a row read
//     the same K bytes, which LDS broadcasts);
//   * softmax: the max of a head over the wave's 16 rows is the max of the
//     lane's rows, then a butterfly over the head's 64/G lanes; p = 2^(x - m)
//     in fp32; each lane keeps the normaliser of its head over its rows
//     (rows in ascending order) across tiles;
//   * PV: lane l owns D/64 dims of all G heads and accumulates p_t * v_t[d]
//     over the wave's rows in order;
//   * end of the split: the four waves' (m, l, acc) are merged in wave order
//     w = 0..3, o = sum_w 2^(m_w - m) acc_w / sum_w 2^(m_w - m) l_w; wave w
//     finishes heads w, w + 4, ...
// Every order is fixed by the split's own token range.
template <int D, int G>
__global__ void __launch_bounds__(256) gqa_tok_kernel(GqaLaunch a) {
  using S = GqaShape<D>;
  constexpr int DPL = S::kDimsPerLane;
  constexpr int kRowsPerWave = kTile / 4;
  constexpr int kSlots = 64 / G;                    // lanes (row slots) per head
  constexpr int kRowsPerLane = kRowsPerWave / kSlots;
  static_assert(kRowsPerWave == 16 && (G == 4 || G == 8 || G == 16), "16 rows of a 64-token tile per wave; G = 4, 8, 16");
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[4 * S::kTileBytes + 4 * kRowsPerWave * G * 4];
  ISK_LDS unsigned char* lds = (ISK_LDS unsigned char*)lds_raw;
  ISK_LDS unsigned char* kbufs = lds;                               // [2][tile]
  ISK_LDS unsigned char* vbufs = lds + 2 * S::kTileBytes;           // [2][tile]
  ISK_LDS float* p_lds = (ISK_LDS float*)(lds + 4 * S::kTileBytes); // [wave][row][head]
  // merge area at the end of a split (the tile buffers are free then)
  ISK_LDS float* mg_acc = (ISK_LDS float*)lds;                      // [wave][head][D]
  ISK_LDS float* mg_ml = mg_acc + 4 * G * D;                        // [m | l][wave][head]
  static_assert(4 * G * D * 4 + 8 * G * 4 <= 4 * S::kTileBytes, "merge area within the tile buffers");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane / kSlots, tr = lane % kSlots;   // score lane: head, row slot
  const int hk = blockIdx.y;
  const int task = blockIdx.x;
  const bool inl = a.inl.n_segs > 0;
  const int seg_first = inl ? task : a.groups[task], seg_last = inl ? task + 1 : a.groups[task + 1];
  ISK_LDS float* my_p = p_lds + wave * kRowsPerWave * G;

  for (int si = seg_first; si < seg_last; ++si) {
    const Seg sg = fetch_seg(a.inl, a.segs, a.lens, si);
    const int b = sg.row;
    __syncthreads();   // LDS of the previous segment is no longer read

    // q of head G hk + hh as packed bf16 pairs (the lanes of a head load the
    // same row)
    uint32_t qv[D / 2];
    {
      const uint4* qrow = (const uint4*)(a.q + ((size_t)b * a.hq + G * hk + hh) * D);
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const uint4 w = qrow[c];
        qv[4 * c + 0] = w.x; qv[4 * c + 1] = w.y; qv[4 * c + 2] = w.z; qv[4 * c + 3] = w.w;
      }
    }
    float m_mine = -INFINITY, l_lane = 0.f;   // running max and normaliser of head hh (this lane's rows)
    float acc[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < DPL; ++j) acc[h][j] = 0.f;

    const int n_tiles = (sg.end - sg.begin + kTile - 1) / kTile;
    uint64_t mask_next = n_tiles > 0 ? gqa_stage<D>(a, b, hk, sg.begin, sg.end, kbufs, vbufs, wave, 4, lane) : 0ull;

    for (int it = 0; it < n_tiles; ++it) {
      wait_vmem_all();
      __syncthreads();
      const uint64_t mask = mask_next;
      const int cur = it & 1;
      ISK_LDS unsigned char* K = kbufs + cur * S::kTileBytes;
      ISK_LDS unsigned char* V = vbufs + cur * S::kTileBytes;
      if (it + 1 < n_tiles)
        mask_next = gqa_stage<D>(a, b, hk, sg.begin + (it + 1) * kTile, sg.end, kbufs + (cur ^ 1) * S::kTileBytes,
                                 vbufs + (cur ^ 1) * S::kTileBytes, wave, 4, lane);

      // ---- scores of (rows of this lane, head hh), log2 domain
      float x[kRowsPerLane];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < kRowsPerLane; ++r) {
        const int row = kRowsPerWave * wave + kSlots * r + tr;
        const ISK_LDS unsigned char* krow = K + row * (D * 2);
        float sc = 0.f;
#pragma unroll
        for (int c = 0; c < S::kPieces; ++c) {
          const u32x4 kp = *(const ISK_LDS u32x4*)(krow + ((c ^ (row & 7)) * 16));
          sc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[4 * c + 0]), as_bf16x2(kp[0]), sc, false);
          sc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[4 * c + 1]), as_bf16x2(kp[1]), sc, false);
          sc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[4 * c + 2]), as_bf16x2(kp[2]), sc, false);
          sc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[4 * c + 3]), as_bf16x2(kp[3]), sc, false);
        }
        x[r] = (mask >> row) & 1ull ? sc * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[r]);
      }
      // ---- softmax of head hh over the wave's rows
#pragma unroll
      for (int sh = 1; sh < kSlots; sh <<= 1) mx = wave_max_xor(mx, sh);
      const float m_new = fmaxf(m_mine, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_mine - m_use);
      m_mine = m_new;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < kRowsPerLane; ++r) {
        const float p = fast_exp2(x[r] - m_use);
        psum += p;
        my_p[(kSlots * r + tr) * G + hh] = p;
      }
      l_lane = l_lane * alpha + psum;
      // every head's alpha, from its first lane (uniform within the head's lanes)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float al = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), kSlots * h));
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[h][j] *= al;
      }
      // p of this wave's rows is read back by the same wave only.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // ---- PV over the wave's 16 rows, in order
      {
        const int vpiece = (DPL * lane) / 8;
        const int vin = (DPL * lane * 2) % 16;
#pragma unroll
        for (int u = 0; u < kRowsPerWave; ++u) {
          const int t = kRowsPerWave * wave + u;
          f32x4 pw[G / 4];
#pragma unroll
          for (int c = 0; c < G / 4; ++c) pw[c] = *(const ISK_LDS f32x4*)(my_p + u * G + 4 * c);
          const ISK_LDS unsigned char* vp = V + t * (D * 2) + ((vpiece ^ (t & 7)) * 16) + vin;
          if constexpr (DPL == 2) {
            const uint32_t w = *(const ISK_LDS uint32_t*)vp;
            const float v0 = bf16_lo(w), v1 = bf16_hi(w);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              acc[h][0] = fmaf(pw[h >> 2][h & 3], v0, acc[h][0]);
              acc[h][1] = fmaf(pw[h >> 2][h & 3], v1, acc[h][1]);
            }
          } else {
            const float v0 = __uint_as_float((uint32_t)(*(const ISK_LDS uint16_t*)vp) << 16);
#pragma unroll
            for (int h = 0; h < G; ++h) acc[h][0] = fmaf(pw[h >> 2][h & 3], v0, acc[h][0]);
          }
        }
      }
    }

    // ---- merge of the four waves' states; wave w finishes heads w, w + 4, ...
    float l_h = l_lane;
#pragma unroll
    for (int sh = 1; sh < kSlots; sh <<= 1) l_h = wave_add_xor(l_h, sh);
    __syncthreads();   // every wave is done with the tile buffers
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < DPL; ++j) mg_acc[(wave * G + h) * D + DPL * lane + j] = acc[h][j];
    if (tr == 0) {
      mg_ml[wave * G + hh] = m_mine;
      mg_ml[4 * G + wave * G + hh] = l_h;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < G / 4; ++c) {
      const int h = wave + 4 * c, head = G * hk + h;
      float m = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) m = fmaxf(m, mg_ml[w * G + h]);
      float l_tot = 0.f, o[DPL];
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[j] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = mg_ml[w * G + h];
        const float sw = mw == -INFINITY ? 0.f : fast_exp2(mw - m);
        l_tot = fmaf(sw, mg_ml[4 * G + w * G + h], l_tot);
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[j] = fmaf(sw, mg_acc[(w * G + h) * D + DPL * lane + j], o[j]);
      }
      const bool empty = !(l_tot > 0.f);
      const float inv = empty ? 0.f : 1.f / l_tot;
      const float lse_v = empty ? -INFINITY : (m + fast_log2(l_tot)) * kLn2;
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[j] *= inv;
      if (sg.part >= 0) {
        float* po = a.part_o + ((size_t)sg.part * a.hq + head) * D + DPL * lane;
        if constexpr (DPL == 2) *(f32x2*)po = f32x2{o[0], o[1]};
        else po[0] = o[0];
        if (lane == 0) a.part_lse[(size_t)sg.part * a.hq + head] = lse_v;
      } else {
        const size_t ob = ((size_t)b * a.hq + head) * D + DPL * lane;
        if (a.out_f32) {
          float* op = (float*)a.out + ob;
          if constexpr (DPL == 2) *(f32x2*)op = f32x2{o[0], o[1]};
          else op[0] = o[0];
        } else {
          uint16_t* op = (uint16_t*)a.out + ob;
          if constexpr (DPL == 2) {
            *(uint32_t*)op = pack_bf16x2(o[0], o[1]);
          } else {
            op[0] = (uint16_t)(pack_bf16x2(o[0], 0.f) & 0xffffu);
          }
        }
        if (a.lse != nullptr && lane == 0) a.lse[(size_t)b * a.hq + head] = lse_v;
      }
    }
  }
}

template <int D>
hipError_t launch_d(const GqaLaunch& a, hipStream_t s, const LaunchEvents& ev) {
  const int g = a.hq / a.hkv;
  const dim3 grid(a.n_groups, a.hkv);
  switch (g) {
    case 1: return launch_one(gqa_split_kernel<D, 1>, grid, dim3(256), s, a, ev);
    case 2: return launch_one(gqa_split_kernel<D, 2>, grid, dim3(256), s, a, ev);
    case 4: return launch_one(gqa_tok_kernel<D, 4>, grid, dim3(256), s, a, ev);
    case 8: return launch_one(gqa_tok_kernel<D, 8>, grid, dim3(256), s, a, ev);
    case 16: return launch_one(gqa_tok_kernel<D, 16>, grid, dim3(256), s, a, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gqa_split(const GqaLaunch& a, hipStream_t s, const LaunchEvents& ev) {
  if (a.n_groups == 0) return hipSuccess;
  if (a.d == 128) return launch_d<128>(a, s, ev);
  if (a.d == 64) return launch_d<64>(a, s, ev);
  return hipErrorInvalidValue;
}

}  // namespace isk
