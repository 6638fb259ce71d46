// Batch-invariant bf16 linear layer, y = x w^T with fp32 accumulation, for
// gfx950.
//
// The gllm issue "Greedy outputs depend on batch composition (NVFP4
// GEMV/GEMM switch at 32 rows is a candidate)" (section "Candidate cause")
// describes a matmul that picks its kernel by row count, and whose two
// kernels round the activations differently, so a row's result depends on
// how many rows share the call; its section "Next steps" proposes that both
// kernels use the same activation precision, so that the switch changes
// speed only.  This library's tile shapes follow that rule and go further:
// they compute every output element with the same instructions.
//   * Rows <= 32 (decode-sized, weight-bandwidth bound): one 16- or 32-row
//     tile, so the weights are read once.  Rows <= 64: one 64-row tile,
//     which reuses each weight fragment for four row tiles.  In these
//     shapes a wave covers two 16-column fragments, so each activation
//     fragment feeds two MFMAs.  More rows: tiles staged through LDS --
//     with K a multiple of 256, the smallest of 128 x 64, 128 x 128 and
//     256 x 128 whose count fits one round on the CUs, 64-wide K stages;
//     other K, 128 x 128 tiles with 32-wide K stages (below).  (Every
//     workgroup of the row-tile kernels re-reads all of its activation rows
//     from L2 for only 32 output columns, so from 65 rows on the LDS-tiled
//     kernels are faster even with a single, partly empty block of rows.)
//   * All take bf16 activations.  The four waves of a workgroup each own a
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

template <int TM, int NB>
__global__ void __launch_bounds__(256) linear_kernel(LinearLaunch a) {
  constexpr int T = TM / 16;   // 16-row MFMA tiles per workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g16 = lane >> 4;
  const int n0 = blockIdx.x * 16 * NB, m0 = blockIdx.y * TM;
  const int kq = a.k / 4;      // K range of this wave: [wave * kq, (wave + 1) * kq)
  const size_t kb = (size_t)wave * kq + 8 * g16;

  // Operand fragments: lane (i16, g16) holds 8 consecutive k of one row.
  // A = x rows m0 + 16t + i16, B = w rows n0 + 16u + i16 (the output
  // columns; NB of them per lane, so each x fragment feeds NB MFMAs).
  // Columns past n read the last row of w and are not stored.
  const bf16x8* wp[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) wp[u] = (const bf16x8*)(a.w + (size_t)min(n0 + 16 * u + i16, a.n - 1) * a.k + kb);
  const bf16x8* xp[T];
  bool xok[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int m = m0 + 16 * t + i16;
    xok[t] = m < a.m;
    xp[t] = (const bf16x8*)(a.x + (size_t)(xok[t] ? m : 0) * a.k + kb);
  }
  const bf16x8 zero = {};
  f32x4 acc[T][NB];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int u = 0; u < NB; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // k-steps of 32 through a register ring of D steps: step s's fragments are
  // loaded D steps ahead, so D loads per operand fragment are in flight per
  // wave.  Each MFMA chain still runs over s in ascending order.
  constexpr int D = T == 1 ? 8 : (T == 2 ? 4 : 2);
  const int steps = kq / 32;
  bf16x8 bq[NB][D], aq[T][D];
  // Prologue in the main loop's load order, unconditional (slots past the
  // last step reload it and are never used).
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int st = min(j, steps - 1);
#pragma unroll
    for (int u = 0; u < NB; ++u) bq[u][j] = wp[u][4 * st];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const bf16x8 v = xp[t][4 * st];
      aq[t][j] = xok[t] ? v : zero;
    }
  }
  auto mfmas = [&](int j) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int u = 0; u < NB; ++u) acc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[t][j], bq[u][j], acc[t][u], 0, 0, 0);
  };
  auto refill = [&](int j, int st) {
#pragma unroll
    for (int u = 0; u < NB; ++u) bq[u][j] = wp[u][4 * st];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const bf16x8 v = xp[t][4 * st];
      aq[t][j] = xok[t] ? v : zero;
    }
  };
  // Main loop: every refill is in range, so the body is straight-line code and
  // the loads of one pass stay in flight while the next pass's MFMAs run.
  // (Rows past m read row 0 and are replaced by zeros.)
  int s0 = 0;
  for (; s0 + 2 * D <= steps; s0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      mfmas(j);
      refill(j, s0 + j + D);
    }
  }
  // Tail: the last (fewer than 2 D) steps, refilling only in range.
  for (; s0 < steps; s0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int st = s0 + j;
      if (st < steps) {
        mfmas(j);
        if (st + D < steps) refill(j, st + D);
      }
    }
  }

  // Partial sums of waves 1..3 through LDS; wave 0 adds them in wave order.
  __shared__ f32x4 part[3][T][NB][64];
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int u = 0; u < NB; ++u) part[wave - 1][t][u][lane] = acc[t][u];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      f32x4 sum = acc[t][u];
      sum = sum + part[0][t][u][lane];
      sum = sum + part[1][t][u][lane];
      sum = sum + part[2][t][u][lane];
      // lane (i16, g16) holds rows m0 + 16t + 4*g16 + r, column n0 + 16u + i16
      const int n = n0 + 16 * u + i16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * t + 4 * g16 + r;
        if (m < a.m && n < a.n) a.y[(size_t)m * a.n + n] = sum[r];
      }
    }
}

// Large row counts: 128 x 128 output tiles staged through LDS.  Wave
// (wm, wn) computes rows 64*wm .. +63 and columns 64*wn .. +63 as 4 x 4
// MFMA tiles.  K is walked in 32-wide stages, quarter by quarter: within a
// quarter the MFMA chain starts from zero and runs in ascending k; at the end
// of quarter q its sums are added to the running total (total = c0, then
// total + c1, + c2, + c3) -- the same arithmetic per element as the
// 16/64-row kernel above, only computed by one wave instead of four.
constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kStageBytes = (kBM + kBN) * kBK * 2;   // A then B, 64 B per row

__global__ void __launch_bounds__(256) linear_tiled_kernel(LinearLaunch a) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kStageBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g16 = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;

  // Staging: 16 wave-wide 16-byte loads per stage (8 for A, 8 for B), four
  // per wave.  Load i covers LDS bytes [1024 i, 1024 i + 1024) of the stage:
  // tile row (1024 i + 16 lane) / 64, 8-element chunk lane % 4.  Rows past
  // m or n read the last valid row (their results are never stored).
  const unsigned char* src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = wave + 4 * j;            // 0..7: A rows, 8..15: B rows
    const int r = (1024 * (i & 7) + 16 * lane) / 64, c = lane & 3;
    if (i < 8) {
      const int m = min(m0 + r, a.m - 1);
      src[j] = (const unsigned char*)(a.x + (size_t)m * a.k + 8 * c);
    } else {
      const int n = min(n0 + r, a.n - 1);
      src[j] = (const unsigned char*)(a.w + (size_t)n * a.k + 8 * c);
    }
  }
  auto stage = [&](int s, int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = wave + 4 * j;
      load_lds_16(src[j] + (size_t)s * kBK * 2, (ISK_LDS unsigned char*)lds + buf * kStageBytes + 1024 * i);
    }
  };

  f32x4 acc[4][4], total[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = total[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_stages = a.k / kBK, per_quarter = n_stages / 4;
  stage(0, 0);
  for (int s = 0; s < n_stages; ++s) {
    __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0) expcnt(0) lgkmcnt(0): this wave's loads of stage s landed
    __syncthreads();                 // ... and every wave's; every wave is done with buffer (s+1) & 1
    if (s + 1 < n_stages) stage(s + 1, (s + 1) & 1);
    const ISK_LDS unsigned char* A = (const ISK_LDS unsigned char*)lds + (s & 1) * kStageBytes;
    const ISK_LDS unsigned char* B = A + kBM * kBK * 2;
    bf16x8 af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = *(const ISK_LDS bf16x8*)(A + (64 * wm + 16 * i + i16) * 64 + 16 * g16);
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = *(const ISK_LDS bf16x8*)(B + (64 * wn + 16 * j + i16) * 64 + 16 * g16);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    if ((s + 1) % per_quarter == 0) {   // end of a K quarter
      const bool first = s + 1 == per_quarter;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          total[i][j] = first ? acc[i][j] : total[i][j] + acc[i][j];
          acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 64 * wn + 16 * j + i16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 64 * wm + 16 * i + 4 * g16 + r;
        if (m < a.m && n < a.n) a.y[(size_t)m * a.n + n] = total[i][j][r];
      }
    }
}


// Large row counts with K a multiple of 256: kGM x kTN output tiles, 256 x
// 128, 128 x 128 or 128 x 64.  Wave (wm, wn) computes rows kGM/2*wm ..
// +kGM/2-1 and columns kTN/2*wn .. +kTN/2-1 as 8 x 4, 4 x 4 or 4 x 2 MFMA
// tiles; with 256-row tiles each
// 16-byte fragment read from LDS feeds four or eight MFMAs (the 128 x 128
// tiles above feed four), a third fewer LDS reads per MFMA.  K is staged 64 wide through a ring of three 48 KB (32 KB)
// buffers, two stages in flight while one is consumed.  A staged row
// is 128 bytes; its eight 16-byte chunks are stored XOR-permuted by the row
// index (chunk c of row r at slot c ^ (r mod 8)), so the 16 rows that one
// fragment read touches spread over all banks.  The per-element arithmetic
// (quarters of K, each a fresh chain in ascending k, added in order) is the
// same as in the kernels above.
constexpr int kGN = 128, kGK = 64;
constexpr int kGRowBytes = kGK * 2;                          // 128

// A 16-byte-per-lane global -> LDS load written as inline assembly: issued
// through the builtin, the compiler's wait insertion falls back to waiting
// for every LDS read before each use, which would stall the MFMA stream.  It
// has no vector register outputs (the kernel's own vmcnt waits cover its
// data) and puts M0, which holds the LDS address, back as it found it.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_off) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(gsrc), "s"(lds_off) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | 0x0F70);
}

template <int kGM, int kTN>
__global__ void __launch_bounds__(256) linear_big_kernel(LinearLaunch a) {
  constexpr int kGBufBytes = (kGM + kTN) * kGRowBytes;       // 48, 32 or 24 KB
  constexpr int kGLoads = kGBufBytes / (256 * 16);           // 12, 8 or 6 per thread per stage
  constexpr int kAT = kGM / 32;                              // A fragments per wave: 8 or 4
  constexpr int kBT = kTN / 32;                              // B fragments per wave: 4 or 2
  constexpr int kB1 = kBT == 4 ? 3 : kBT;                    // of which read in the first pre-read group
  static_assert(kGLoads % 2 == 0 && kGLoads / 2 <= kAT && kAT >= 4, "group schedule");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[3 * kGBufBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g16 = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = blockIdx.y * kGM, n0 = blockIdx.x * kTN;

  // Staging: 4 kGLoads wave-wide 16-byte loads per stage, kGLoads per wave.  Load
  // i = wave + 4 j fills LDS bytes [1024 i, 1024 i + 1024) of the buffer,
  // staged rows 8 i .. 8 i + 7 (rows 0..255: x, 256..383: w); lane L writes
  // slot L mod 8 of row 8 i + L / 8 and so fetches chunk (L mod 8) ^ (L / 8).
  // Rows past m or n read the last valid row (their results are not stored).
  const unsigned char* src[kGLoads];
  const int chunk = (lane & 7) ^ (lane >> 3);
#pragma unroll
  for (int j = 0; j < kGLoads; ++j) {
    const int r = 8 * (wave + 4 * j) + (lane >> 3);
    if (j < kGM / 32) {
      const int m = min(m0 + r, a.m - 1);
      src[j] = (const unsigned char*)(a.x + (size_t)m * a.k) + 16 * chunk;
    } else {
      const int n = min(n0 + r - kGM, a.n - 1);
      src[j] = (const unsigned char*)(a.w + (size_t)n * a.k) + 16 * chunk;
    }
  }
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds_base = (uint32_t)(size_t)(ISK_LDS unsigned char*)lds;
  auto stage = [&](int s, int buf) {
#pragma unroll
    for (int j = 0; j < kGLoads; ++j)
      dma16(src[j] + (size_t)s * kGRowBytes, lds_base + buf * kGBufBytes + 1024 * (wave_s + 4 * j));
  };
  // Fragment reads: row 16 t + i16 of a 16-row tile, k chunk 4 h + g16 of
  // substep h, found at slot (4 h + g16) ^ (i16 mod 8).
  const int slot0 = 16 * (g16 ^ (i16 & 7)), slot1 = 16 * ((4 + g16) ^ (i16 & 7));
  const int a_row = (kGM / 2 * wm + i16) * kGRowBytes, b_row = (kGM + kTN / 2 * wn + i16) * kGRowBytes;

  f32x4 acc[kAT][kBT], total[kAT][kBT];
#pragma unroll
  for (int i = 0; i < kAT; ++i)
#pragma unroll
    for (int j = 0; j < kBT; ++j) acc[i][j] = total[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Each k32 half of a stage is eight groups of four MFMAs (one A fragment
  // against four B fragments), each group its own scheduling region that
  // also reads the A fragment two groups ahead.  The first half's groups
  // issue the next-but-one stage's loads, two per group; its last two groups
  // read the second half's B fragments and first A fragments.  In the
  // second half, once every read of the stage has landed (after group 5),
  // the waves barrier -- the next stage is in LDS, this one's buffer is free
  // -- and its last two groups read the next stage's first fragments, so a
  // stage starts with no barrier and no read latency.
  const int n_stages = a.k / kGK, per_quarter = n_stages / 4;
  bf16x8 af[2][kAT], bf[2][kBT];
  auto read_b = [&](const ISK_LDS unsigned char* base, int h, int j) {
    bf[h][j] = *(const ISK_LDS bf16x8*)(base + b_row + 16 * j * kGRowBytes + (h == 0 ? slot0 : slot1));
  };
  auto read_a = [&](const ISK_LDS unsigned char* base, int h, int i) {
    af[h][i] = *(const ISK_LDS bf16x8*)(base + a_row + 16 * i * kGRowBytes + (h == 0 ? slot0 : slot1));
  };
  stage(0, 0);
  stage(1, 1);
  wait_vmem_le<kGLoads>();
  asm volatile("s_barrier" ::: "memory");
  {
    const ISK_LDS unsigned char* base = (const ISK_LDS unsigned char*)lds;
    for (int j = 0; j < kBT; ++j) read_b(base, 0, j);
    read_a(base, 0, 0);
    read_a(base, 0, 1);
  }
  int buf = 0, s = 0;
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int i = 0; i < kAT; ++i)
#pragma unroll
      for (int j = 0; j < kBT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < per_quarter; ++t, ++s) {
      // Stage s + 2 goes to the buffer read in stage s - 1.  The last two
      // stages load stage n - 1 again into a buffer that is not read again,
      // so the loop has no branch; the wait after the loop drains them.
      const int fill = min(s + 2, n_stages - 1);
      const int fill_buf = buf == 0 ? 2 : buf - 1;
      const int next_buf = buf == 2 ? 0 : buf + 1;
      const ISK_LDS unsigned char* base = (const ISK_LDS unsigned char*)lds + buf * kGBufBytes;
      const ISK_LDS unsigned char* next = (const ISK_LDS unsigned char*)lds + next_buf * kGBufBytes;
#pragma unroll
      for (int i = 0; i < kAT; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + 2 < kAT) read_a(base, 0, i + 2);
        if (i < kGLoads / 2) {   // stage s + 2, two loads per MFMA group
          dma16(src[2 * i] + (size_t)fill * kGRowBytes, lds_base + fill_buf * kGBufBytes + 1024 * (wave_s + 8 * i));
          dma16(src[2 * i + 1] + (size_t)fill * kGRowBytes, lds_base + fill_buf * kGBufBytes + 1024 * (wave_s + 8 * i + 4));
        }
        if (i == kAT - 2) {
          for (int j = 0; j < kB1; ++j) read_b(base, 1, j);
        } else if (i == kAT - 1) {
          for (int j = kB1; j < kBT; ++j) read_b(base, 1, j);
          read_a(base, 1, 0); read_a(base, 1, 1);
        }
#pragma unroll
        for (int j = 0; j < kBT; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0][i], bf[0][j], acc[i][j], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kAT; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + 2 < kAT) read_a(base, 1, i + 2);
        if (i == kAT - 2) {
          // Every read of stage s landed (lgkmcnt 0) and this wave's loads of
          // stage s + 1 too (vmcnt: stage s + 2's may still be in flight).
          __builtin_amdgcn_s_waitcnt(kGLoads | 0x70);
          asm volatile("s_barrier" ::: "memory");
          for (int j = 0; j < kB1; ++j) read_b(next, 0, j);
        } else if (i == kAT - 1) {
          for (int j = kB1; j < kBT; ++j) read_b(next, 0, j);
          read_a(next, 0, 0); read_a(next, 0, 1);
        }
#pragma unroll
        for (int j = 0; j < kBT; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1][i], bf[1][j], acc[i][j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      buf = next_buf;
    }
    // End of quarter q: total = c0, then total + c1, + c2, + c3.
#pragma unroll
    for (int i = 0; i < kAT; ++i)
#pragma unroll
      for (int j = 0; j < kBT; ++j) total[i][j] = q == 0 ? acc[i][j] : total[i][j] + acc[i][j];
  }
  wait_vmem_le<0>();   // no load into this workgroup's LDS outlives it
#pragma unroll
  for (int i = 0; i < kAT; ++i)
#pragma unroll
    for (int j = 0; j < kBT; ++j) {
      const int n = n0 + kTN / 2 * wn + 16 * j + i16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + kGM / 2 * wm + 16 * i + 4 * g16 + r;
        if (m < a.m && n < a.n) a.y[(size_t)m * a.n + n] = total[i][j][r];
      }
    }
}

}  // namespace

// Output-column fragments per wave in the row-tile kernels: two, so each
// activation fragment feeds two MFMAs per row tile and a workgroup covers 32
// columns.  (One: 32 rows took 39 us at n = k = 7168, bound by the
// activation re-reads from L2; two: 27 us; four: 40 us, too few
// workgroups to keep the weight stream busy.)
constexpr int kNB = 2;
hipError_t launch_linear(const LinearLaunch& a, hipStream_t s) {
  if (a.m == 0) return hipSuccess;
  if (a.m <= 16) {
    hipLaunchKernelGGL((linear_kernel<16, kNB>), dim3((a.n + 16 * kNB - 1) / (16 * kNB), 1), dim3(256), 0, s, a);
  } else if (a.m <= kLinearSmallRows) {
    hipLaunchKernelGGL((linear_kernel<32, kNB>), dim3((a.n + 16 * kNB - 1) / (16 * kNB), 1), dim3(256), 0, s, a);
  } else if (a.m <= kLinearTiledRows) {
    hipLaunchKernelGGL((linear_kernel<64, kNB>), dim3((a.n + 16 * kNB - 1) / (16 * kNB), (a.m + 63) / 64), dim3(256), 0, s, a);
  } else if (a.k % 256 == 0) {
    // The smallest tile whose count fits one round on the CUs: 128 x 64,
    // then 128 x 128 (half and a quarter of a 256 x 128 tile's work); else
    // 256 x 128 tiles, the best LDS ratio at full load.
    static int cus = 0;
    if (cus == 0) {
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    }
    const long nb = (a.n + kGN - 1) / kGN, nb64 = (a.n + 63) / 64, mb128 = (a.m + 127) / 128;
    if (mb128 * nb64 <= cus)
      hipLaunchKernelGGL((linear_big_kernel<128, 64>), dim3(nb64, mb128), dim3(256), 0, s, a);
    else if (mb128 * nb <= cus)
      hipLaunchKernelGGL((linear_big_kernel<128, 128>), dim3(nb, mb128), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((linear_big_kernel<256, 128>), dim3(nb, (a.m + 255) / 256), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(linear_tiled_kernel, dim3((a.n + kBN - 1) / kBN, (a.m + kBM - 1) / kBM), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace isk
