// Internal declarations shared by the host runtime (api.cpp, plan.cpp) and
// the kernel launchers (*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "isk.h"

namespace isk {

// Frozen numerics constants.  A row's split boundaries are multiples of the
// split length, and tile boundaries inside a split are multiples of the tile,
// so both are functions of the row's own length and these constants only.
constexpr int kGqaTile = 64;          // tokens per GQA wave step
constexpr int kMlaTile = 64;          // tokens per LDS tile of the 16-head MLA kernel
constexpr int kGqaSplitDefault = 512;
constexpr int kMlaSplitDefault = 1536;
constexpr int kSparseSplitDefault = 512;
constexpr int kMlaDqk = 576;
constexpr float kLog2eHost = 1.44269504088896340736f;   // log2(e), rounded to float

// Split partials are fp16 (2 bytes a value) for the 128-head MLA kernels with
// bf16 output (their PV operand is fp16, so every partial is in fp16 range);
// fp32 everywhere else.
inline bool partials_fp16(const isk_desc& d) {
  return d.kind == ISK_KIND_MLA && d.num_q_heads % 128 == 0 && d.out_dtype != ISK_OUT_F32;
}
constexpr int kMlaDv = 512;
// Batch-balanced comparison mode: block granularity, parts and per-row
// overhead charge of the batch-wide scheduler it reproduces.
constexpr int kBalancedBlock = 64;
constexpr int kBalancedParts = 256;
constexpr int kBalancedOverhead = 1;

// One split of one row: units [begin, end) of row `row`; `part` is the
// workspace partial slot, or -1 when the row has a single split and writes
// the final output directly.
struct Seg {
  int32_t row, begin, end, part;
};

struct RowInfo {
  int32_t part_off;   // first partial slot of the row
  int32_t n_parts;    // 0: empty row; 1: written directly; >1: combined
};

// Per-row plans small enough for the kernel arguments travel there instead
// of through the workspace, so a decode call enqueues no upload copy before
// its kernels.  Segment j (one per workgroup task, launch order) is stored as
// row << 16 | split index i, and its range is rebuilt from the row's units:
// [i*S, min((i+1)*S, min(units[row], cap))), units being the device lengths
// (dense; cap = max_pages_per_row * page_size) or the device top-k counts
// (sparse; cap = topk_width); its partial slot is rows[row].part_off + i
// when the row has more than one split, else -1.
constexpr int kInlineSegs = 640;
constexpr int kInlineRows = 128;
struct InlinePlan {
  int32_t n_segs;        // 0: the plan is read from the workspace
  int32_t split_units;   // S
  int32_t cap;           // max_pages_per_row * page_size (dense), topk_width (sparse)
  int32_t reserved;
  uint32_t seg[kInlineSegs];
  RowInfo rows[kInlineRows];
};

// Segment si of a launch; `units` is the device copy of the row lengths
// (dense) or of the top-k counts (sparse).
__device__ __forceinline__ Seg fetch_seg(const InlinePlan& p, const Seg* segs, const int32_t* units, int si) {
  if (p.n_segs == 0) return segs[si];
  const uint32_t e = p.seg[si];
  const int row = (int)(e >> 16), i = (int)(e & 0xffffu);
  const int L = min(max(units[row], 0), p.cap);
  const RowInfo ri = p.rows[row];
  return Seg{row, i * p.split_units, min((i + 1) * p.split_units, L), ri.n_parts > 1 ? ri.part_off + i : -1};
}

struct PlanData {
  isk_desc desc{};
  int32_t batch = 0;
  int32_t split_units = 0;
  std::vector<int32_t> units;       // per-row units (tokens or top-k slots)
  std::vector<Seg> segs;            // launch order
  std::vector<int32_t> seg_group;   // group of each segment (for inspection)
  std::vector<int32_t> groups;      // CSR offsets into segs, size n_groups + 1
  std::vector<RowInfo> rows;
  int32_t n_partials = 0;
  bool any_combine = false;         // some row has 0 or >1 splits
  // Extra KV source (sparse MLA): its segments cover units
  // [desc.topk_width + j0, desc.topk_width + j1) of the row.
  bool has_extra = false;
  isk_extra_desc extra{};
  std::vector<int32_t> extra_units; // per-row valid extra top-k counts
  // Length bands (empty: one split length S for every row).
  std::vector<isk_split_band> bands;
  int32_t max_seg_units = 0;        // longest segment (units)
};

constexpr int kMaxBands = 16;
// Launch-order blocks of the per-row planner: kXcdBlock tasks, of which XCD
// x (task % kXcds under round-robin dealing) takes kXcdBlock / kXcds
// consecutive sorted ones.
constexpr int kXcds = 8;
constexpr int kXcdBlock = 32;

// Byte layout of the per-call metadata at the head of the workspace.
struct MetaLayout {
  size_t segs_off, groups_off, rows_off, bytes;        // meta block
  size_t part_o_off, part_lse_off, audit_off, total;    // whole workspace
};
MetaLayout meta_layout(const PlanData& p);

// Planner (host only; no HIP calls).  Returns an empty string on success,
// otherwise the error message; *status receives the isk_status.
// With `extra` non-NULL the plan also covers an extra KV source
// (extra_topk_len_host gives its per-row valid counts).
// With `bands` non-NULL each row's split length comes from the band table
// (n_bands entries) instead of one S.
std::string plan_build(PlanData& p, const isk_desc& d, int32_t batch, const int32_t* lens_host,
                       const int32_t* topk_len_host, int* status, const isk_extra_desc* extra = nullptr,
                       const int32_t* extra_topk_len_host = nullptr, const isk_split_band* bands = nullptr,
                       int32_t n_bands = 0);

// ---------------------------------------------------------------- launchers
// Optional profiling events of a split-kernel launch.  When set, the kernel
// goes through hipExtLaunchKernel, which stamps the events with the kernel's
// own start and end (not the time the stream reached a marker).
struct LaunchEvents {
  hipEvent_t begin = nullptr, end = nullptr;
};

// Launch a kernel whose only argument is the struct `a`.
template <typename Arg>
inline hipError_t launch_one(void (*kernel)(Arg), dim3 grid, dim3 block, hipStream_t s, const Arg& a,
                             const LaunchEvents& ev) {
  if (ev.begin == nullptr && ev.end == nullptr) {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, a);
    return hipGetLastError();
  }
  Arg copy = a;
  void* args[] = {&copy};
  return hipExtLaunchKernel((const void*)kernel, grid, block, args, 0, s, ev.begin, ev.end, 0);
}

struct GqaLaunch {
  const uint16_t* q; const uint16_t* kv;
  const int32_t* block_table; const int32_t* lens;
  const Seg* segs; const int32_t* groups;
  float* part_o; float* part_lse; void* out; float* lse;
  int32_t n_groups, hq, hkv, d, page_size, num_pages, max_pages, out_f32;
  float scale_log2;
  InlinePlan inl;   // n_segs > 0: segments by value (groups are one segment each)
};
hipError_t launch_gqa_split(const GqaLaunch& a, hipStream_t s, const LaunchEvents& ev = {});

struct MlaLaunch {
  const uint16_t* q; const uint16_t* kv;
  const int32_t* block_table; const int32_t* lens;
  const int32_t* topk_idx; const int32_t* topk_len;   // sparse rows (NULL when dense)
  const Seg* segs; const int32_t* groups;
  float* part_o; float* part_lse; void* out; float* lse;
  int32_t n_groups, hq, page_size, num_pages, max_pages, topk_width, out_f32;
  float scale_log2;
  // Partials in fp16 (2 bytes a value) instead of fp32; only the 128-head
  // kernels, whose PV operand is fp16 already, take it.
  int32_t part_f16;
  // Extra KV source (sparse only; xtopk_idx NULL when absent).  A segment
  // whose begin is >= topk_width gathers from it, at extra slots
  // [begin - topk_width, end - topk_width).
  const uint16_t* xkv; const int32_t* xblock_table; const int32_t* xlens; const int32_t* xtopk_idx;
  int32_t xpage_size, xnum_pages, xmax_pages, xtopk_width;
  int32_t max_seg_units;   // longest segment of the launch (units)
  InlinePlan inl;   // n_segs > 0: segments by value (groups are one segment each; no extra source)
};
hipError_t launch_mla_split(const MlaLaunch& a, hipStream_t s, const LaunchEvents& ev = {});       // 16 heads per wave
hipError_t launch_mla_split_h32(const MlaLaunch& a, hipStream_t s, const LaunchEvents& ev = {});   // 32 heads per wave, hq % 128 == 0
// 128-head kernel: dense, or sparse when every segment holds at most
// kMlaH128MaxSparseSlots slots and each latent pool the kernel gathers from
// spans at most 4 GiB (its tile loads take 32-bit offsets from the pool base).
constexpr int kMlaH128MaxSparseSlots = 1024;
inline bool mla_h128_pool_fits(int64_t num_pages, int64_t page_size) {
  return num_pages * page_size * (int64_t)(2 * kMlaDqk) <= ((int64_t)1 << 32);
}
hipError_t launch_mla_h128(const MlaLaunch& a, hipStream_t s, const LaunchEvents& ev = {});        // hq % 128 == 0

struct CombineLaunch {
  const RowInfo* rows; const float* part_o; const float* part_lse;
  void* out; float* lse;
  int32_t batch, hq, dv, out_f32;
  int32_t part_f16;   // partials stored as fp16 (part_o then holds 2-byte values)
  InlinePlan inl;   // n_segs > 0: per-row partial slots by value
};
hipError_t launch_combine(const CombineLaunch& a, hipStream_t s);

// Batch-invariant RMSNorm: one workgroup per row.
constexpr int kRmsNormMaxDim = 16384;
struct RmsNormLaunch {
  const uint16_t* x; const uint16_t* w; uint16_t* y;
  int32_t rows, dim;
  float eps;
};
hipError_t launch_rmsnorm(const RmsNormLaunch& a, hipStream_t s);

// Value-range audit of the latent cache for the 128-head MLA kernels
// (check_inputs): found[0] becomes 1 and found[1..3] = (row, position, dim)
// of one V value of magnitude >= 65536 (or not finite).
struct VRangeAudit {
  const uint16_t* kv; const int32_t* block_table; const int32_t* lens;
  const int32_t* topk_idx; const int32_t* topk_len;   // topk_idx NULL: dense rows
  int32_t batch, max_pages, page_size, num_pages, topk_width;
  int32_t* found;
};
hipError_t launch_v_range_audit(const VRangeAudit& a, hipStream_t s);

// Fixed device workspace of isk_attn_decode_static (noalloc.hip).
size_t static_workspace_bytes();
hipError_t static_workspace(void** ptr);   // device address on the current device

// Streaming-read microbenchmark (isk_hbm_read_probe).
hipError_t launch_hbm_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t s);
// Row-gather microbenchmark (isk_hbm_gather_probe).
hipError_t launch_hbm_gather(const void* src, const int32_t* rows, int n_rows, int row_bytes, uint32_t* sink,
                             int blocks, hipStream_t s);

// Batch-invariant linear layer: tile shape chosen by row count, same bits.
constexpr int kLinearSmallRows = 32;    // up to here: 16-row tiles
constexpr int kLinearTiledRows = 64;    // up to here: one 64-row tile; above: 256 x 128 (K % 256 == 0) or 128 x 128 LDS tiles
struct LinearLaunch {
  const uint16_t* x; const uint16_t* w; float* y;
  int32_t m, n, k;
};
hipError_t launch_linear(const LinearLaunch& a, hipStream_t s);

// Each launch struct is one kernel argument; HIP takes up to 4 KB of them.
static_assert(sizeof(GqaLaunch) <= 4096 && sizeof(MlaLaunch) <= 4096 && sizeof(CombineLaunch) <= 4096,
              "kernel arguments exceed 4 KB");

}  // namespace isk
