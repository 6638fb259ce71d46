// Host split planner (no HIP calls; usable without a GPU).
//
// Per-row mode follows the request on the FlashMLA issue page "Sparse MLA
// decode is not batch-invariant ..." (section "Question"): a row's split
// count comes only from its own length and fixed constants:
//   n_b = ceil(U_b / S),  split i = [i*S, min((i+1)*S, U_b)),
// where U_b is the row's length in tokens (dense) or its valid top-k count
// (sparse) and S the frozen split length of the kind.  An exclusive scan over
// rows assigns workspace slots to the partials; it decides where partials
// live, never what is computed.  Splits are dispatched longest first, which
// changes only which compute unit runs a split and when (within each block of
// 32 tasks the order is permuted so that a row's consecutive splits share an
// XCD).  A sparse row with
// an extra KV source gets the same rule applied to its extra top-k count;
// those splits follow the main set's in the row's partial order.
//
// With a length-band table the split length is chosen per row, again from
// the row's own units only: the first band whose bound covers U_b (the last
// band covers everything longer) gives S_band, and a band with a split cap
// n_max stretches its splits when ceil(U_b / S_band) > n_max:
//   S_b = 64 * ceil(ceil(U_b / n_max) / 64),  n_b = ceil(U_b / S_b) <= n_max.
// This is the piecewise n = f(L) with per-band S and N_max that the FlashMLA
// issue page leaves open (section "Question") as the way to trade occupancy
// against partial traffic without making a row depend on its batch.
//
// Batch-balanced mode exists for comparison only.  It reproduces the
// scheduler that page describes (same section: a block quota per part derived
// from the total over the whole batch, then greedy packing that cuts rows at
// part boundaries), so a row's splits depend on its batchmates.

#include <algorithm>
#include <cmath>
#include <sstream>

#include "isk_internal.hpp"

namespace isk {
namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

std::string fail(int* status, int code, const std::string& msg) {
  *status = code;
  return msg;
}

}  // namespace

MetaLayout meta_layout(const PlanData& p) {
  MetaLayout m{};
  m.segs_off = 0;
  m.groups_off = align256(m.segs_off + p.segs.size() * sizeof(Seg));
  m.rows_off = align256(m.groups_off + p.groups.size() * sizeof(int32_t));
  m.bytes = align256(m.rows_off + p.rows.size() * sizeof(RowInfo));
  const int dv = p.desc.head_dim_v;
  m.part_o_off = m.bytes;
  const size_t part_elem = partials_fp16(p.desc) ? 2 : sizeof(float);
  m.part_lse_off = align256(m.part_o_off + (size_t)p.n_partials * p.desc.num_q_heads * dv * part_elem);
  m.audit_off = align256(m.part_lse_off + (size_t)p.n_partials * p.desc.num_q_heads * sizeof(float));
  m.total = m.audit_off + 256;   // four ints of the value-range audit (check_inputs)
  return m;
}

static std::string check_desc(const isk_desc& d, int* status) {
  std::ostringstream e;
  if (d.kind != ISK_KIND_GQA && d.kind != ISK_KIND_MLA) return fail(status, ISK_ERR_INVALID_ARG, "desc.kind must be ISK_KIND_GQA or ISK_KIND_MLA");
  if (d.num_q_heads <= 0 || d.num_kv_heads <= 0) return fail(status, ISK_ERR_INVALID_ARG, "head counts must be positive");
  if (d.page_size <= 0 || d.num_pages <= 0 || d.max_pages_per_row <= 0)
    return fail(status, ISK_ERR_INVALID_ARG, "page_size, num_pages and max_pages_per_row must be positive");
  if (d.split_mode != ISK_SPLIT_PER_ROW && d.split_mode != ISK_SPLIT_BATCH_BALANCED)
    return fail(status, ISK_ERR_INVALID_ARG, "desc.split_mode is not a valid isk_split_mode");
  if (d.out_dtype != ISK_OUT_BF16 && d.out_dtype != ISK_OUT_F32)
    return fail(status, ISK_ERR_INVALID_ARG, "desc.out_dtype is not a valid isk_out_dtype");
  if (d.split_tokens < 0 || d.split_tokens % 64 != 0)
    return fail(status, ISK_ERR_INVALID_ARG, "desc.split_tokens must be 0 or a positive multiple of 64");
  if (!std::isfinite(d.scale) || !(d.scale > 0.f))
    return fail(status, ISK_ERR_INVALID_ARG, "desc.scale must be finite and positive");
  if (d.topk_width < 0) return fail(status, ISK_ERR_INVALID_ARG, "desc.topk_width must be >= 0");
  // Row lengths and token positions are 32-bit in the kernels.
  if ((long long)d.max_pages_per_row * d.page_size > 0x7fffffffLL)
    return fail(status, ISK_ERR_UNSUPPORTED, "max_pages_per_row * page_size must fit in int32");
  if (d.kind == ISK_KIND_GQA) {
    if (d.num_q_heads % d.num_kv_heads != 0) return fail(status, ISK_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
    const int g = d.num_q_heads / d.num_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16)
      return fail(status, ISK_ERR_UNSUPPORTED, "GQA group size Hq/Hkv must be 1, 2, 4, 8 or 16");
    if (d.head_dim_qk != 64 && d.head_dim_qk != 128) return fail(status, ISK_ERR_UNSUPPORTED, "GQA head_dim_qk must be 64 or 128");
    if (d.head_dim_v != d.head_dim_qk) return fail(status, ISK_ERR_INVALID_ARG, "GQA head_dim_v must equal head_dim_qk");
    if (d.topk_width != 0) return fail(status, ISK_ERR_UNSUPPORTED, "top-k gather is supported for MLA only");
  } else {
    if (d.num_kv_heads != 1) return fail(status, ISK_ERR_INVALID_ARG, "MLA has one latent kv head (num_kv_heads = 1)");
    if (d.head_dim_qk != kMlaDqk || d.head_dim_v != kMlaDv) return fail(status, ISK_ERR_UNSUPPORTED, "MLA needs head_dim_qk 576 and head_dim_v 512");
    if (d.num_q_heads % 16 != 0 || (d.num_q_heads > 64 && d.num_q_heads % 64 != 0))
      return fail(status, ISK_ERR_UNSUPPORTED, "MLA num_q_heads must be a multiple of 16 (and of 64 above 64)");
    if (d.topk_width == 0 && d.page_size % 64 != 0) return fail(status, ISK_ERR_UNSUPPORTED, "dense MLA needs page_size a multiple of 64");
    // The MLA kernels index pool rows (token slots) with 32-bit arithmetic.
    if ((long long)d.num_pages * d.page_size > 0x7fffffffLL)
      return fail(status, ISK_ERR_UNSUPPORTED, "MLA pools are limited to 2^31 - 1 token rows (num_pages * page_size)");
  }
  *status = ISK_OK;
  return "";
}

// Split length of a row with `U` units under a band table.
static int32_t band_split(const std::vector<isk_split_band>& bands, int32_t U) {
  size_t k = 0;
  while (k + 1 < bands.size() && U > bands[k].max_units) ++k;
  const isk_split_band& bd = bands[k];
  const int32_t n = (int32_t)(((long long)U + bd.split_units - 1) / bd.split_units);
  if (bd.max_splits <= 0 || n <= bd.max_splits) return bd.split_units;
  const long long per = ((long long)U + bd.max_splits - 1) / bd.max_splits;
  return (int32_t)((per + 63) / 64 * 64);
}

std::string plan_build(PlanData& p, const isk_desc& d, int32_t batch, const int32_t* lens_host,
                       const int32_t* topk_len_host, int* status, const isk_extra_desc* extra,
                       const int32_t* extra_topk_len_host, const isk_split_band* bands, int32_t n_bands) {
  std::string err = check_desc(d, status);
  if (*status != ISK_OK) return err;
  if (bands != nullptr) {
    if (n_bands < 1 || n_bands > kMaxBands)
      return fail(status, ISK_ERR_INVALID_ARG, "n_bands must be in [1, 16]");
    if (d.split_mode != ISK_SPLIT_PER_ROW)
      return fail(status, ISK_ERR_INVALID_ARG, "a band table needs split_mode ISK_SPLIT_PER_ROW");
    if (d.split_tokens != 0)
      return fail(status, ISK_ERR_INVALID_ARG, "desc.split_tokens must be 0 with a band table (the bands give S)");
    if (extra != nullptr) return fail(status, ISK_ERR_UNSUPPORTED, "band tables are not combined with an extra KV source");
    for (int32_t k = 0; k < n_bands; ++k) {
      const isk_split_band& bd = bands[k];
      std::ostringstream e;
      e << "bands[" << k << "]: ";
      if (bd.split_units <= 0 || bd.split_units % 64 != 0)
        return fail(status, ISK_ERR_INVALID_ARG, e.str() + "split_units must be a positive multiple of 64");
      if (bd.max_splits < 0) return fail(status, ISK_ERR_INVALID_ARG, e.str() + "max_splits must be >= 0");
      if (bd.reserved != 0) return fail(status, ISK_ERR_INVALID_ARG, e.str() + "reserved must be 0");
      if (bd.max_units < 0 || (k > 0 && bd.max_units <= bands[k - 1].max_units))
        return fail(status, ISK_ERR_INVALID_ARG, e.str() + "max_units must be >= 0 and strictly increasing");
    }
  }
  if (extra != nullptr) {
    if (d.kind != ISK_KIND_MLA || d.topk_width <= 0)
      return fail(status, ISK_ERR_UNSUPPORTED, "an extra KV source needs a sparse MLA descriptor (topk_width > 0)");
    if (d.split_mode != ISK_SPLIT_PER_ROW)
      return fail(status, ISK_ERR_UNSUPPORTED, "an extra KV source is planned in per-row split mode only");
    if (extra->page_size <= 0 || extra->num_pages <= 0 || extra->max_pages_per_row <= 0 || extra->topk_width <= 0)
      return fail(status, ISK_ERR_INVALID_ARG,
                  "extra page_size, num_pages, max_pages_per_row and topk_width must be positive");
    if ((long long)extra->num_pages * extra->page_size > 0x7fffffffLL)
      return fail(status, ISK_ERR_UNSUPPORTED, "extra pools are limited to 2^31 - 1 token rows");
    if ((long long)extra->max_pages_per_row * extra->page_size > 0x7fffffffLL)
      return fail(status, ISK_ERR_UNSUPPORTED, "extra max_pages_per_row * page_size must fit in int32");
    if ((long long)d.topk_width + extra->topk_width > 0x7fffffffLL)
      return fail(status, ISK_ERR_UNSUPPORTED, "topk_width + extra topk_width must fit in int32");
    if (extra_topk_len_host == nullptr) return fail(status, ISK_ERR_INVALID_ARG, "extra_topk_len_host is NULL");
  }
  if (batch <= 0) return fail(status, ISK_ERR_INVALID_ARG, "batch must be >= 1");
  if (lens_host == nullptr) return fail(status, ISK_ERR_INVALID_ARG, "lens_host is NULL");
  const bool sparse = d.topk_width > 0;
  if (sparse && topk_len_host == nullptr) return fail(status, ISK_ERR_INVALID_ARG, "topk_len_host is NULL for a sparse plan");
  if (!sparse && topk_len_host != nullptr) return fail(status, ISK_ERR_INVALID_ARG, "topk_len_host must be NULL for a dense plan");

  const long long cap = (long long)d.max_pages_per_row * d.page_size;
  std::vector<int32_t> units(batch);
  for (int b = 0; b < batch; ++b) {
    const int32_t L = lens_host[b];
    if (L < 0 || L > cap) {
      std::ostringstream e;
      e << "lens_host[" << b << "] = " << L << " is outside [0, max_pages_per_row * page_size = " << cap << "]";
      return fail(status, ISK_ERR_INVALID_ARG, e.str());
    }
    units[b] = sparse ? std::min(std::max(topk_len_host[b], 0), d.topk_width) : L;
  }

  int32_t S = d.split_tokens;
  if (S == 0) S = d.kind == ISK_KIND_GQA ? kGqaSplitDefault : (sparse ? kSparseSplitDefault : kMlaSplitDefault);

  p.desc = d;
  p.batch = batch;
  p.split_units = S;
  p.bands.assign(bands, bands != nullptr ? bands + n_bands : bands);
  p.units = units;
  p.segs.clear();
  p.seg_group.clear();
  p.groups.clear();
  p.rows.assign(batch, RowInfo{0, 0});
  p.n_partials = 0;
  p.has_extra = extra != nullptr;
  p.extra = extra != nullptr ? *extra : isk_extra_desc{};
  p.extra_units.assign(extra != nullptr ? batch : 0, 0);
  for (int b = 0; b < (int)p.extra_units.size(); ++b)
    p.extra_units[b] = std::min(std::max(extra_topk_len_host[b], 0), extra->topk_width);

  std::vector<std::vector<Seg>> row_segs(batch);
  std::vector<int32_t> seg_part_of;   // group index per segment (balanced)

  if (d.split_mode == ISK_SPLIT_PER_ROW) {
    if (!p.bands.empty()) p.split_units = 0;
    for (int b = 0; b < batch; ++b) {
      const int32_t U = units[b];
      const int32_t S = p.bands.empty() ? p.split_units : band_split(p.bands, U);
      if (!p.bands.empty() && U > 0) p.split_units = std::max(p.split_units, S);
      const int32_t n = (int32_t)(((long long)U + S - 1) / S);
      for (int32_t i = 0; i < n; ++i) row_segs[b].push_back(Seg{b, i * S, (int32_t)std::min<long long>((long long)(i + 1) * S, U), 0});
      if (p.has_extra) {
        // The extra set's splits follow the main set's, by the same rule;
        // their units are offset by the main index width.
        const int32_t W = d.topk_width, X = p.extra_units[b];
        const int32_t nx = (int32_t)(((long long)X + S - 1) / S);
        for (int32_t i = 0; i < nx; ++i) row_segs[b].push_back(Seg{b, W + i * S, W + (int32_t)std::min<long long>((long long)(i + 1) * S, X), 0});
      }
    }
  } else {
    // Batch-wide quota: total blocks plus a fixed overhead charge per row,
    // divided over the parts; each part takes up to `payload` blocks, paying
    // the overhead for every row piece it starts.
    const int blk = kBalancedBlock;
    long long total = 0;
    for (int b = 0; b < batch; ++b) total += (units[b] + blk - 1) / blk + kBalancedOverhead;
    const long long payload = (total + kBalancedParts - 1) / kBalancedParts + kBalancedOverhead;
    int part = 0;
    long long used = 0;
    for (int b = 0; b < batch; ++b) {
      const long long blocks = (units[b] + blk - 1) / blk;
      long long pos = 0;
      while (pos < blocks) {
        const long long avail = payload - used - kBalancedOverhead;
        if (avail <= 0) { ++part; used = 0; continue; }
        const long long take = std::min(avail, blocks - pos);
        Seg s{b, (int32_t)(pos * blk), (int32_t)std::min<long long>((pos + take) * blk, units[b]), 0};
        row_segs[b].push_back(s);
        seg_part_of.push_back(part);
        used += take + kBalancedOverhead;
        pos += take;
        if (used >= payload) { ++part; used = 0; }
      }
    }
  }

  // Partial slots: rows in batch order, a row's splits in order.
  for (int b = 0; b < batch; ++b) {
    const int32_t n = (int32_t)row_segs[b].size();
    p.rows[b] = RowInfo{p.n_partials, n};
    if (n > 1) {
      for (int32_t i = 0; i < n; ++i) row_segs[b][i].part = p.n_partials + i;
      p.n_partials += n;
    } else if (n == 1) {
      row_segs[b][0].part = -1;
    }
  }
  p.any_combine = false;
  for (int b = 0; b < batch; ++b) p.any_combine |= p.rows[b].n_parts != 1;

  if (d.split_mode == ISK_SPLIT_PER_ROW) {
    // One split per workgroup task, longest first (ties: batch order, split
    // order), at the granularity of blocks of kXcdBlock tasks.
    for (int b = 0; b < batch; ++b)
      for (const Seg& s : row_segs[b]) p.segs.push_back(s);
    std::stable_sort(p.segs.begin(), p.segs.end(),
                     [](const Seg& x, const Seg& y) { return (x.end - x.begin) > (y.end - y.begin); });
    // Task t runs on XCD t % 8 (the kernels' block-to-task mapping under
    // round-robin dealing of workgroups to the 8 XCDs).  In each full block
    // of 32 tasks, XCD x takes sorted tasks 4x .. 4x+3: consecutive splits
    // of one row, which read the same query, then share an L2, while the
    // blocks stay in longest-first order.
    for (size_t b0 = 0; b0 + kXcdBlock <= p.segs.size(); b0 += kXcdBlock) {
      Seg blk[kXcdBlock];
      for (int k = 0; k < kXcdBlock; ++k) blk[k] = p.segs[b0 + k];
      for (int x = 0; x < kXcds; ++x)
        for (int j = 0; j < kXcdBlock / kXcds; ++j) p.segs[b0 + kXcds * j + x] = blk[(kXcdBlock / kXcds) * x + j];
    }
    p.groups.resize(p.segs.size() + 1);
    for (size_t i = 0; i <= p.segs.size(); ++i) p.groups[i] = (int32_t)i;
    p.seg_group.resize(p.segs.size());
    for (size_t i = 0; i < p.segs.size(); ++i) p.seg_group[i] = (int32_t)i;
  } else {
    // One part per workgroup task; a part's pieces run in row order.
    size_t k = 0;
    for (int b = 0; b < batch; ++b)
      for (const Seg& s : row_segs[b]) { p.segs.push_back(s); p.seg_group.push_back(seg_part_of[k++]); }
    // seg order is already grouped by part (parts increase monotonically).
    const int n_groups = p.seg_group.empty() ? 0 : p.seg_group.back() + 1;
    p.groups.assign(n_groups + 1, 0);
    for (int32_t g : p.seg_group) p.groups[g + 1]++;
    for (int g = 0; g < n_groups; ++g) p.groups[g + 1] += p.groups[g];
  }
  p.max_seg_units = 0;
  for (const Seg& s : p.segs) p.max_seg_units = std::max(p.max_seg_units, s.end - s.begin);
  *status = ISK_OK;
  return "";
}

}  // namespace isk
