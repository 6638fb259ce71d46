// C ABI of libisk: argument checks, plan objects, per-call metadata upload and
// kernel launches.  Every entry point returns an isk_status and records a
// thread-local message on failure; nothing throws across the boundary.

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <sstream>
#include <string>
#include <vector>

#include "isk_internal.hpp"

using isk::MetaLayout;
using isk::PlanData;

namespace {

thread_local std::string g_err;

int set_err(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_err(hipError_t e, const char* what) {
  std::ostringstream s;
  s << what << ": " << hipGetErrorString(e);
  return set_err(ISK_ERR_HIP, s.str());
}

// Pinned staging ring for the per-call metadata: a decode may be enqueued
// while up to kRing earlier uploads of the same plan are still pending.
constexpr int kRing = 4;

}  // namespace

struct isk_plan {
  PlanData data;
  MetaLayout layout{};
  std::vector<unsigned char> meta_host;   // serialised metadata
  // Staging ring of an uploaded plan, sized at plan time (prepare_staging):
  // isk_attn_decode itself allocates nothing.  ring_mu serialises decode
  // calls of several threads on the slot cursor and the slots.
  void* staging[kRing] = {};
  size_t staging_bytes[kRing] = {};
  hipEvent_t staged[kRing] = {};
  int ring_next = 0;
  hipError_t staging_error = hipSuccess;  // why the ring could not be prepared
  std::mutex ring_mu;
  hipEvent_t t_split_begin = nullptr, t_split_end = nullptr, t_combine_end = nullptr;   // profiling hook
  isk::InlinePlan inl{};                  // n_segs > 0: passed by value, no upload
};

namespace {

// Diagnostic switch: ISK_DENSE_MLA_KERNEL=h32 routes dense 128-head MLA
// through the gather kernel (mla_split_h32) instead of the generated tile
// loop, so tests can compare the two on the same inputs.  Read once.
bool dense_h128_off() {
  static const bool off = [] {
    const char* v = std::getenv("ISK_DENSE_MLA_KERNEL");
    return v != nullptr && std::strcmp(v, "h32") == 0;
  }();
  return off;
}

// Diagnostic switch: ISK_SPARSE_MLA_KERNEL=h32 routes sparse 128-head MLA
// through the gather kernel even where the generated tile loop takes it.
// Read once.
bool sparse_h128_off() {
  static const bool off = [] {
    const char* v = std::getenv("ISK_SPARSE_MLA_KERNEL");
    return v != nullptr && std::strcmp(v, "h32") == 0;
  }();
  return off;
}

// Sparse plans the generated tile loop takes: every split within its slot
// window, every latent pool within its 32-bit tile offsets.
bool sparse_h128_fits(const PlanData& pd) {
  const isk_desc& d = pd.desc;
  return pd.max_seg_units <= isk::kMlaH128MaxSparseSlots && isk::mla_h128_pool_fits(d.num_pages, d.page_size) &&
         (!pd.has_extra || isk::mla_h128_pool_fits(pd.extra.num_pages, pd.extra.page_size));
}

// Split-kernel family of a plan's decode (ISK_KERNEL_*).
int split_kernel_of(const PlanData& pd) {
  const isk_desc& d = pd.desc;
  if (d.kind == ISK_KIND_GQA) return ISK_KERNEL_GQA;
  if (d.num_q_heads % 128 != 0) return ISK_KERNEL_MLA_H16;
  const bool sparse = d.topk_width > 0;
  if (!sparse) return dense_h128_off() ? ISK_KERNEL_MLA_H32 : ISK_KERNEL_MLA_H128;
  return sparse_h128_fits(pd) && !sparse_h128_off() ? ISK_KERNEL_MLA_H128 : ISK_KERNEL_MLA_H32;
}

// Per-row plans (dense, or sparse without an extra source) that fit go to
// the kernels by value (see InlinePlan).
void build_inline(isk_plan* p) {
  const PlanData& d = p->data;
  isk::InlinePlan& inl = p->inl;
  inl = isk::InlinePlan{};
  const bool fits = d.desc.split_mode == ISK_SPLIT_PER_ROW && !d.has_extra &&
                    !d.segs.empty() && d.segs.size() <= (size_t)isk::kInlineSegs && d.batch <= isk::kInlineRows &&
                    d.groups.size() == d.segs.size() + 1;
  if (!fits) return;
  for (size_t j = 0; j < d.segs.size(); ++j) {
    const isk::Seg& sg = d.segs[j];
    const int32_t i = sg.begin / d.split_units;
    // The kernels rebuild exactly this segment from (row, i) and the row's length.
    if (d.groups[j] != (int32_t)j || i > 0xffff || sg.begin != i * d.split_units ||
        sg.end != std::min((i + 1) * d.split_units, d.units[sg.row]))
      return;
    inl.seg[j] = ((uint32_t)sg.row << 16) | (uint32_t)i;
  }
  for (int b = 0; b < d.batch; ++b) inl.rows[b] = d.rows[b];
  inl.split_units = d.split_units;
  inl.cap = d.desc.topk_width > 0 ? d.desc.topk_width
                                  : (int32_t)std::min<long long>((long long)d.desc.max_pages_per_row * d.desc.page_size,
                                                                 0x7fffffffLL);
  inl.n_segs = (int32_t)d.segs.size();
}

void serialise(isk_plan* p) {
  build_inline(p);
  p->layout = isk::meta_layout(p->data);
  p->meta_host.assign(p->layout.bytes, 0);
  std::memcpy(p->meta_host.data() + p->layout.segs_off, p->data.segs.data(), p->data.segs.size() * sizeof(isk::Seg));
  std::memcpy(p->meta_host.data() + p->layout.groups_off, p->data.groups.data(), p->data.groups.size() * sizeof(int32_t));
  std::memcpy(p->meta_host.data() + p->layout.rows_off, p->data.rows.data(), p->data.rows.size() * sizeof(isk::RowInfo));
}

// The pinned staging ring of a plan whose metadata is uploaded (not passed
// by value) is created and sized here, at plan time, so that the decode path
// allocates nothing: kRing slots of at least the metadata size (with half
// again of headroom, so that a growing batch re-allocates rarely) and one
// event each.  A slot is only freed after its last upload has completed.
// Without a usable GPU the ring stays unprepared and staging_error says why;
// a decode of such a plan then fails with ISK_ERR_HIP.
void prepare_staging(isk_plan* p) {
  p->staging_error = hipSuccess;
  if (p->inl.n_segs > 0) return;
  const size_t need = std::max<size_t>(p->layout.bytes, 256);
  for (int i = 0; i < kRing; ++i) {
    if (p->staged[i] == nullptr) {
      const hipError_t e = hipEventCreateWithFlags(&p->staged[i], hipEventDisableTiming);
      if (e != hipSuccess) {
        p->staged[i] = nullptr;
        p->staging_error = e;
        return;
      }
    }
    if (p->staging_bytes[i] < need) {
      if (p->staging[i] != nullptr) {
        (void)hipEventSynchronize(p->staged[i]);
        (void)hipHostFree(p->staging[i]);
      }
      p->staging[i] = nullptr;
      p->staging_bytes[i] = 0;
      const size_t cap = need + need / 2;
      const hipError_t e = hipHostMalloc(&p->staging[i], cap, hipHostMallocDefault);
      if (e != hipSuccess) {
        p->staging[i] = nullptr;
        p->staging_error = e;
        return;
      }
      p->staging_bytes[i] = cap;
    }
  }
}

void release_staging(isk_plan* p) {
  for (int i = 0; i < kRing; ++i) {
    if (p->staged[i] != nullptr) {
      (void)hipEventSynchronize(p->staged[i]);
      (void)hipEventDestroy(p->staged[i]);
      p->staged[i] = nullptr;
    }
    if (p->staging[i] != nullptr) {
      (void)hipHostFree(p->staging[i]);
      p->staging[i] = nullptr;
      p->staging_bytes[i] = 0;
    }
  }
}

// Audit of the tables against the plan (desc.check_inputs).  Copies the
// device tables to the host (synchronising the stream).
int audit_extra(const isk_plan* p, const isk_extra_kv& x, hipStream_t stream);

// The value-range audit (128-head MLA): V of every attended row must fit the
// fp16 PV operand.  `found` is four ints of device workspace.
int audit_v_range(const isk_plan* p, const void* kv_pages, const int32_t* block_table, const int32_t* lens,
                  const int32_t* topk_idx, const int32_t* topk_len, const isk_extra_kv* extra, int32_t* found,
                  hipStream_t stream) {
  const isk_desc& d = p->data.desc;
  int32_t h[4] = {0, 0, 0, 0};
  for (int set = 0; set < (extra != nullptr ? 2 : 1); ++set) {
    const bool x = set == 1;
    isk::VRangeAudit a{};
    a.kv = (const uint16_t*)(x ? extra->kv_pages : kv_pages);
    a.block_table = x ? extra->block_table : block_table;
    a.lens = x ? extra->lens : lens;
    a.topk_idx = x ? extra->topk_idx : (d.topk_width > 0 ? topk_idx : nullptr);
    a.topk_len = x ? extra->topk_len : topk_len;
    a.batch = p->data.batch;
    a.max_pages = x ? p->data.extra.max_pages_per_row : d.max_pages_per_row;
    a.page_size = x ? p->data.extra.page_size : d.page_size;
    a.num_pages = x ? p->data.extra.num_pages : d.num_pages;
    a.topk_width = x ? p->data.extra.topk_width : d.topk_width;
    a.found = found;
    hipError_t e = hipMemsetAsync(found, 0, 4 * sizeof(int32_t), stream);
    if (e == hipSuccess) e = isk::launch_v_range_audit(a, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(h, found, sizeof(h), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_err(e, "check_inputs: value-range audit");
    if (h[0] != 0) {
      std::ostringstream s;
      s << "check_inputs: " << (x ? "extra " : "") << "row " << h[1] << " position " << h[2] << " has V[" << h[3]
        << "] of magnitude 65536 or more (or not finite), outside the fp16 PV operand of the 128-head MLA kernels";
      return set_err(ISK_ERR_RANGE, s.str());
    }
  }
  return ISK_OK;
}

int audit_inputs(const isk_plan* p, const int32_t* block_table, const int32_t* lens, const int32_t* topk_idx,
                 const int32_t* topk_len, const isk_extra_kv* extra, hipStream_t stream) {
  const isk_desc& d = p->data.desc;
  const int B = p->data.batch;
  std::vector<int32_t> h_lens(B), h_bt((size_t)B * d.max_pages_per_row), h_tl, h_idx;
  hipError_t e = hipMemcpyAsync(h_lens.data(), lens, B * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h_bt.data(), block_table, h_bt.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  const bool sparse = d.topk_width > 0;
  if (sparse && e == hipSuccess) {
    h_tl.resize(B);
    h_idx.resize((size_t)B * d.topk_width);
    e = hipMemcpyAsync(h_tl.data(), topk_len, B * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess)
      e = hipMemcpyAsync(h_idx.data(), topk_idx, h_idx.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_err(e, "check_inputs: copying tables to the host");

  auto page_ok = [&](int b, int pos) {
    const int32_t pg = h_bt[(size_t)b * d.max_pages_per_row + pos / d.page_size];
    return pg >= 0 && pg < d.num_pages;
  };
  for (int b = 0; b < B; ++b) {
    const int32_t L = h_lens[b];
    if (!sparse && L != p->data.units[b]) {
      std::ostringstream s;
      s << "check_inputs: lens[" << b << "] = " << L << " differs from the planned length " << p->data.units[b];
      return set_err(ISK_ERR_INVALID_ARG, s.str());
    }
    if (L < 0 || (long long)L > (long long)d.max_pages_per_row * d.page_size) {
      std::ostringstream s;
      s << "check_inputs: lens[" << b << "] = " << L << " out of range";
      return set_err(ISK_ERR_INDEX, s.str());
    }
    if (!sparse) {
      for (int j = 0; j < L; j += d.page_size)
        if (!page_ok(b, j)) {
          std::ostringstream s;
          s << "check_inputs: block_table[" << b << "][" << j / d.page_size << "] is not a page of the pool";
          return set_err(ISK_ERR_INDEX, s.str());
        }
    } else {
      const int32_t n = std::min(std::max(h_tl[b], 0), d.topk_width);
      if (n != p->data.units[b]) {
        std::ostringstream s;
        s << "check_inputs: topk_len[" << b << "] differs from the planned count";
        return set_err(ISK_ERR_INVALID_ARG, s.str());
      }
      for (int j = 0; j < n; ++j) {
        const int32_t pos = h_idx[(size_t)b * d.topk_width + j];
        if (pos < 0 || pos >= L) {
          std::ostringstream s;
          s << "check_inputs: topk_idx[" << b << "][" << j << "] = " << pos << " is not a position in [0, " << L
            << ") although the slot is below topk_len";
          return set_err(ISK_ERR_INDEX, s.str());
        }
        if (!page_ok(b, pos)) {
          std::ostringstream s;
          s << "check_inputs: the page of topk_idx[" << b << "][" << j << "] is not a page of the pool";
          return set_err(ISK_ERR_INDEX, s.str());
        }
      }
    }
  }
  return extra != nullptr ? audit_extra(p, *extra, stream) : ISK_OK;
}

// The same audit for the extra KV source.
int audit_extra(const isk_plan* p, const isk_extra_kv& x, hipStream_t stream) {
  const isk_extra_desc& d = p->data.extra;
  const int B = p->data.batch;
  std::vector<int32_t> h_lens(B), h_bt((size_t)B * d.max_pages_per_row), h_tl(B), h_idx((size_t)B * d.topk_width);
  hipError_t e = hipMemcpyAsync(h_lens.data(), x.lens, B * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h_bt.data(), x.block_table, h_bt.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(h_tl.data(), x.topk_len, B * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h_idx.data(), x.topk_idx, h_idx.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_err(e, "check_inputs: copying the extra tables to the host");
  for (int b = 0; b < B; ++b) {
    const int32_t L = h_lens[b];
    if (L < 0 || (long long)L > (long long)d.max_pages_per_row * d.page_size) {
      std::ostringstream s;
      s << "check_inputs: extra lens[" << b << "] = " << L << " out of range";
      return set_err(ISK_ERR_INDEX, s.str());
    }
    const int32_t n = std::min(std::max(h_tl[b], 0), d.topk_width);
    if (n != p->data.extra_units[b]) {
      std::ostringstream s;
      s << "check_inputs: extra topk_len[" << b << "] differs from the planned count";
      return set_err(ISK_ERR_INVALID_ARG, s.str());
    }
    for (int j = 0; j < n; ++j) {
      const int32_t pos = h_idx[(size_t)b * d.topk_width + j];
      if (pos < 0 || pos >= L) {
        std::ostringstream s;
        s << "check_inputs: extra topk_idx[" << b << "][" << j << "] = " << pos << " is not a position in [0, " << L
          << ") although the slot is below the extra topk_len";
        return set_err(ISK_ERR_INDEX, s.str());
      }
      const int32_t pg = h_bt[(size_t)b * d.max_pages_per_row + pos / d.page_size];
      if (pg < 0 || pg >= d.num_pages) {
        std::ostringstream s;
        s << "check_inputs: the page of extra topk_idx[" << b << "][" << j << "] is not a page of the extra pool";
        return set_err(ISK_ERR_INDEX, s.str());
      }
    }
  }
  return ISK_OK;
}

}  // namespace

extern "C" {

const char* isk_last_error(void) { return g_err.c_str(); }

const char* isk_numerics_id(void) {
  static const std::string id = [] {
    std::ostringstream s;
    s << "isk-2 arch=gfx950"
      << " gqa_tile=" << isk::kGqaTile
      << " split_gqa=" << isk::kGqaSplitDefault << " split_mla=" << isk::kMlaSplitDefault
      << " split_topk=" << isk::kSparseSplitDefault
      << " gqa=vdot2-bf16/fp32-pv(g>=4:4-wave-token-split,wave-order-merge)"
      << " mla(hq%128=0)=qk:mfma32x32x16-bf16/pv:mfma32x32x16-f16(p-fp16-rne-x2^7,v-bf16-to-fp16-rtz)/tile32/rescale-thr8"
      << "/partials-fp16-rne(bf16-out)"
      << " mla(other)=mfma16x16x32-bf16/tile64/p-hi+lo-bf16/rescale-thr8 combine=fixed-order-fp32"
      << " balanced=blk" << isk::kBalancedBlock << "-parts" << isk::kBalancedParts << "-ovh" << isk::kBalancedOverhead;
    return s.str();
  }();
  return id.c_str();
}

int isk_plan_create(const isk_desc* desc, int32_t batch, const int32_t* lens_host, const int32_t* topk_len_host,
                    isk_plan** plan_out) {
  if (plan_out == nullptr) return set_err(ISK_ERR_INVALID_ARG, "plan_out is NULL");
  *plan_out = nullptr;
  if (desc == nullptr) return set_err(ISK_ERR_INVALID_ARG, "desc is NULL");
  isk_plan* p = new (std::nothrow) isk_plan();
  if (p == nullptr) return set_err(ISK_ERR_INVALID_ARG, "out of host memory");
  int status = ISK_OK;
  std::string msg = isk::plan_build(p->data, *desc, batch, lens_host, topk_len_host, &status);
  if (status != ISK_OK) {
    delete p;
    return set_err(status, msg);
  }
  serialise(p);
  prepare_staging(p);
  *plan_out = p;
  return ISK_OK;
}

int isk_plan_create_extra(const isk_desc* desc, const isk_extra_desc* extra, int32_t batch, const int32_t* lens_host,
                          const int32_t* topk_len_host, const int32_t* extra_topk_len_host, isk_plan** plan_out) {
  if (plan_out == nullptr) return set_err(ISK_ERR_INVALID_ARG, "plan_out is NULL");
  *plan_out = nullptr;
  if (desc == nullptr || extra == nullptr) return set_err(ISK_ERR_INVALID_ARG, "desc or extra is NULL");
  isk_plan* p = new (std::nothrow) isk_plan();
  if (p == nullptr) return set_err(ISK_ERR_INVALID_ARG, "out of host memory");
  int status = ISK_OK;
  std::string msg =
      isk::plan_build(p->data, *desc, batch, lens_host, topk_len_host, &status, extra, extra_topk_len_host);
  if (status != ISK_OK) {
    delete p;
    return set_err(status, msg);
  }
  serialise(p);
  prepare_staging(p);
  *plan_out = p;
  return ISK_OK;
}

int isk_plan_create_banded(const isk_desc* desc, const isk_split_band* bands, int32_t n_bands, int32_t batch,
                           const int32_t* lens_host, const int32_t* topk_len_host, isk_plan** plan_out) {
  if (plan_out == nullptr) return set_err(ISK_ERR_INVALID_ARG, "plan_out is NULL");
  *plan_out = nullptr;
  if (desc == nullptr || bands == nullptr) return set_err(ISK_ERR_INVALID_ARG, "desc or bands is NULL");
  isk_plan* p = new (std::nothrow) isk_plan();
  if (p == nullptr) return set_err(ISK_ERR_INVALID_ARG, "out of host memory");
  int status = ISK_OK;
  std::string msg = isk::plan_build(p->data, *desc, batch, lens_host, topk_len_host, &status, nullptr, nullptr,
                                    bands, n_bands);
  if (status != ISK_OK) {
    delete p;
    return set_err(status, msg);
  }
  serialise(p);
  prepare_staging(p);
  *plan_out = p;
  return ISK_OK;
}

int isk_plan_update(isk_plan* plan, int32_t batch, const int32_t* lens_host, const int32_t* topk_len_host) {
  if (plan == nullptr) return set_err(ISK_ERR_INVALID_ARG, "plan is NULL");
  if (plan->data.has_extra)
    return set_err(ISK_ERR_INVALID_ARG, "a plan with an extra KV source is re-planned with isk_plan_create_extra");
  PlanData fresh;
  int status = ISK_OK;
  const std::vector<isk_split_band>& bands = plan->data.bands;
  std::string msg = isk::plan_build(fresh, plan->data.desc, batch, lens_host, topk_len_host, &status, nullptr,
                                    nullptr, bands.empty() ? nullptr : bands.data(), (int32_t)bands.size());
  if (status != ISK_OK) return set_err(status, msg);
  plan->data = std::move(fresh);
  serialise(plan);
  prepare_staging(plan);
  return ISK_OK;
}

int isk_plan_destroy(isk_plan* plan) {
  if (plan == nullptr) return ISK_OK;
  release_staging(plan);
  delete plan;
  return ISK_OK;
}

int isk_plan_query(const isk_plan* plan, isk_plan_info* info) {
  if (plan == nullptr || info == nullptr) return set_err(ISK_ERR_INVALID_ARG, "plan or info_out is NULL");
  info->batch = plan->data.batch;
  info->split_tokens = plan->data.split_units;
  info->num_segments = (int32_t)plan->data.segs.size();
  info->num_groups = (int32_t)plan->data.groups.size() - 1;
  info->num_partials = plan->data.n_partials;
  info->split_kernel = split_kernel_of(plan->data);
  info->workspace_bytes = plan->layout.total;
  return ISK_OK;
}

size_t isk_plan_workspace_bytes(const isk_plan* plan) { return plan == nullptr ? 0 : plan->layout.total; }

int isk_plan_segments(const isk_plan* plan, int32_t* records, int32_t capacity) {
  if (plan == nullptr) return set_err(ISK_ERR_INVALID_ARG, "plan is NULL");
  const int32_t n = (int32_t)plan->data.segs.size();
  if (records != nullptr) {
    for (int32_t i = 0; i < n && i < capacity; ++i) {
      const isk::Seg& s = plan->data.segs[i];
      int32_t* r = records + 5 * (size_t)i;
      r[0] = s.row; r[1] = s.begin; r[2] = s.end; r[3] = s.part; r[4] = plan->data.seg_group[i];
    }
  }
  return n;
}

namespace {

// Pointer checks of a decode call (everything but the workspace).
int check_decode_args(const isk_desc& d, const void* q, const void* kv_pages, const int32_t* block_table,
                      const int32_t* lens, const int32_t* topk_idx, const int32_t* topk_len, const void* out,
                      const float* lse) {
  const bool sparse = d.topk_width > 0;
  if (q == nullptr || kv_pages == nullptr || block_table == nullptr || lens == nullptr || out == nullptr)
    return set_err(ISK_ERR_INVALID_ARG, "q, kv_pages, block_table, lens and out must be non-NULL");
  if (sparse && (topk_idx == nullptr || topk_len == nullptr))
    return set_err(ISK_ERR_INVALID_ARG, "sparse plan: topk_idx and topk_len must be non-NULL");
  if (!sparse && (topk_idx != nullptr || topk_len != nullptr))
    return set_err(ISK_ERR_INVALID_ARG, "dense plan: topk_idx and topk_len must be NULL");
  auto aligned = [](const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; };
  if (!aligned(q, 16) || !aligned(kv_pages, 16) || !aligned(out, 16) || !aligned(block_table, 4) || !aligned(lens, 4) ||
      (lse != nullptr && !aligned(lse, 4)) || (sparse && !aligned(topk_idx, 4)))
    return set_err(ISK_ERR_INVALID_ARG, "q, kv_pages and out must be 16-byte aligned, tables 4-byte aligned");
  return ISK_OK;
}

}  // namespace

static int decode_impl(const isk_plan* plan_c, const void* q, const void* kv_pages, const int32_t* block_table,
                       const int32_t* lens, const int32_t* topk_idx, const int32_t* topk_len,
                       const isk_extra_kv* extra, void* out, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream_v) {
  if (plan_c == nullptr) return set_err(ISK_ERR_INVALID_ARG, "plan is NULL");
  isk_plan* plan = const_cast<isk_plan*>(plan_c);   // staging ring only (under ring_mu); the plan itself is not changed
  const PlanData& pd = plan->data;
  const isk_desc& d = pd.desc;
  const bool sparse = d.topk_width > 0;
  hipStream_t stream = (hipStream_t)stream_v;
  {
    const int rc = check_decode_args(d, q, kv_pages, block_table, lens, topk_idx, topk_len, out, lse);
    if (rc != ISK_OK) return rc;
  }
  if (pd.has_extra && extra == nullptr)
    return set_err(ISK_ERR_INVALID_ARG, "the plan has an extra KV source: call isk_attn_decode_extra");
  if (!pd.has_extra && extra != nullptr)
    return set_err(ISK_ERR_INVALID_ARG, "the plan has no extra KV source (create it with isk_plan_create_extra)");
  if (extra != nullptr) {
    if (extra->kv_pages == nullptr || extra->block_table == nullptr || extra->lens == nullptr ||
        extra->topk_idx == nullptr || extra->topk_len == nullptr)
      return set_err(ISK_ERR_INVALID_ARG, "every pointer of the extra KV source must be non-NULL");
    if ((uintptr_t)extra->kv_pages % 16 != 0 || (uintptr_t)extra->block_table % 4 != 0 ||
        (uintptr_t)extra->lens % 4 != 0 || (uintptr_t)extra->topk_idx % 4 != 0 || (uintptr_t)extra->topk_len % 4 != 0)
      return set_err(ISK_ERR_INVALID_ARG, "extra kv_pages must be 16-byte aligned, extra tables 4-byte aligned");
  }
  if (workspace == nullptr || workspace_bytes < plan->layout.total) {
    std::ostringstream s;
    s << "workspace of " << workspace_bytes << " bytes is smaller than the " << plan->layout.total << " the plan needs";
    return set_err(ISK_ERR_WORKSPACE, s.str());
  }
  if (((uintptr_t)workspace & 255u) != 0) return set_err(ISK_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  if (d.check_inputs) {
    int rc = audit_inputs(plan, block_table, lens, topk_idx, topk_len, extra, stream);
    if (rc == ISK_OK && d.kind == ISK_KIND_MLA && d.num_q_heads % 128 == 0)
      rc = audit_v_range(plan, kv_pages, block_table, lens, topk_idx, topk_len, extra,
                         (int32_t*)((unsigned char*)workspace + plan->layout.audit_off), stream);
    if (rc != ISK_OK) return rc;
  }

  // Upload the metadata through a pinned staging slot (plans passed by value
  // in the kernel arguments need none).
  hipError_t e;
  const bool by_value = plan->inl.n_segs > 0;
  unsigned char* ws = (unsigned char*)workspace;
  if (!by_value) {
    std::lock_guard<std::mutex> lock(plan->ring_mu);
    const int slot = plan->ring_next;
    const size_t mbytes = plan->layout.bytes;
    if (plan->staged[slot] == nullptr || plan->staging_bytes[slot] < mbytes)
      return hip_err(plan->staging_error != hipSuccess ? plan->staging_error : hipErrorNotInitialized,
                     "the plan's metadata staging (prepared when the plan was made) is missing");
    plan->ring_next = (slot + 1) % kRing;
    e = hipEventSynchronize(plan->staged[slot]);
    if (e != hipSuccess) return hip_err(e, "waiting for an earlier metadata upload");
    std::memcpy(plan->staging[slot], plan->meta_host.data(), mbytes);
    e = hipMemcpyAsync(ws, plan->staging[slot], mbytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_err(e, "hipMemcpyAsync (metadata upload)");
    e = hipEventRecord(plan->staged[slot], stream);
    if (e != hipSuccess) return hip_err(e, "hipEventRecord");
  }

  const isk::Seg* segs = (const isk::Seg*)(ws + plan->layout.segs_off);
  const int32_t* groups = (const int32_t*)(ws + plan->layout.groups_off);
  const isk::RowInfo* rows = (const isk::RowInfo*)(ws + plan->layout.rows_off);
  float* part_o = (float*)(ws + plan->layout.part_o_off);
  float* part_lse = (float*)(ws + plan->layout.part_lse_off);
  const int32_t n_groups = (int32_t)pd.groups.size() - 1;
  const float scale_log2 = d.scale * isk::kLog2eHost;

  // Partials of the 128-head MLA kernels (fp16 PV operand) are fp16 when the
  // output is bf16; every other kernel, and fp32 output, keeps fp32 partials.
  const int32_t part_f16 = isk::partials_fp16(d);
  isk::LaunchEvents ev;
  ev.begin = plan->t_split_begin;
  ev.end = plan->t_split_end;
  if (d.kind == ISK_KIND_GQA) {
    isk::GqaLaunch a{(const uint16_t*)q, (const uint16_t*)kv_pages, block_table, lens, segs, groups, part_o, part_lse,
                     out, lse, n_groups, d.num_q_heads, d.num_kv_heads, d.head_dim_qk, d.page_size, d.num_pages,
                     d.max_pages_per_row, d.out_dtype == ISK_OUT_F32, scale_log2, plan->inl};
    e = isk::launch_gqa_split(a, stream, ev);
    if (e != hipSuccess) return hip_err(e, "launching the GQA split kernel");
  } else {
    isk::MlaLaunch a{(const uint16_t*)q, (const uint16_t*)kv_pages, block_table, lens, sparse ? topk_idx : nullptr,
                     sparse ? topk_len : nullptr, segs, groups, part_o, part_lse, out, lse, n_groups, d.num_q_heads,
                     d.page_size, d.num_pages, d.max_pages_per_row, d.topk_width, d.out_dtype == ISK_OUT_F32, scale_log2, part_f16,
                     nullptr, nullptr, nullptr, nullptr, 0, 0, 0, 0, pd.max_seg_units, plan->inl};
    if (extra != nullptr) {
      a.xkv = (const uint16_t*)extra->kv_pages;
      a.xblock_table = extra->block_table;
      a.xlens = extra->lens;
      a.xtopk_idx = extra->topk_idx;
      a.xpage_size = pd.extra.page_size;
      a.xnum_pages = pd.extra.num_pages;
      a.xmax_pages = pd.extra.max_pages_per_row;
      a.xtopk_width = pd.extra.topk_width;
    }
    // 128-head blocks (32 heads per wave) when the head count allows it:
    // the generated tile loop for dense rows, and for sparse rows whose
    // splits fit its slot window (pools within its 32-bit offsets); the
    // gather kernel (same bits) otherwise.
    switch (split_kernel_of(pd)) {
      case ISK_KERNEL_MLA_H16: e = isk::launch_mla_split(a, stream, ev); break;
      case ISK_KERNEL_MLA_H128: e = isk::launch_mla_h128(a, stream, ev); break;
      default: e = isk::launch_mla_split_h32(a, stream, ev); break;
    }
    if (e != hipSuccess) return hip_err(e, "launching the MLA split kernel");
  }
  if (pd.any_combine) {
    isk::CombineLaunch c{rows, part_o, part_lse, out, lse, pd.batch, d.num_q_heads, d.head_dim_v,
                         d.out_dtype == ISK_OUT_F32, part_f16, plan->inl};
    e = isk::launch_combine(c, stream);
    if (e != hipSuccess) return hip_err(e, "launching the combine kernel");
  }
  if (plan->t_combine_end != nullptr) {
    e = hipEventRecord(plan->t_combine_end, stream);
    if (e != hipSuccess) return hip_err(e, "hipEventRecord (timing)");
  }
  return ISK_OK;
}

int isk_attn_decode(const isk_plan* plan, const void* q, const void* kv_pages, const int32_t* block_table,
                    const int32_t* lens, const int32_t* topk_idx, const int32_t* topk_len, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(plan, q, kv_pages, block_table, lens, topk_idx, topk_len, nullptr, out, lse, workspace,
                     workspace_bytes, stream);
}

int isk_attn_decode_extra(const isk_plan* plan, const void* q, const void* kv_pages, const int32_t* block_table,
                          const int32_t* lens, const int32_t* topk_idx, const int32_t* topk_len,
                          const isk_extra_kv* extra, void* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (extra == nullptr) return set_err(ISK_ERR_INVALID_ARG, "extra is NULL");
  return decode_impl(plan, q, kv_pages, block_table, lens, topk_idx, topk_len, extra, out, lse, workspace,
                     workspace_bytes, stream);
}

int isk_attn_decode_static(const isk_plan* plan, const void* q, const void* kv_pages, const int32_t* block_table,
                           const int32_t* lens, const int32_t* topk_idx, const int32_t* topk_len, void* out,
                           float* lse, void* stream) {
  if (plan == nullptr) return set_err(ISK_ERR_INVALID_ARG, "plan is NULL");
  const size_t cap = isk::static_workspace_bytes();
  if (plan->layout.total > cap) {
    std::ostringstream s;
    s << "the plan needs a workspace of " << plan->layout.total << " bytes; the static workspace holds " << cap
      << " (use isk_attn_decode with a workspace of its own)";
    return set_err(ISK_ERR_WORKSPACE, s.str());
  }
  void* ws = nullptr;
  const hipError_t e = isk::static_workspace(&ws);
  if (e != hipSuccess) return hip_err(e, "hipGetSymbolAddress (static workspace)");
  return decode_impl(plan, q, kv_pages, block_table, lens, topk_idx, topk_len, nullptr, out, lse, ws, cap, stream);
}

int isk_attn_decode_oneshot(const isk_desc* desc, int32_t batch, const int32_t* lens_host,
                            const int32_t* topk_len_host, const void* q, const void* kv_pages,
                            const int32_t* block_table, const int32_t* lens, const int32_t* topk_idx,
                            const int32_t* topk_len, void* out, float* lse, void* stream_v) {
  isk_plan* plan = nullptr;
  int rc = isk_plan_create(desc, batch, lens_host, topk_len_host, &plan);
  if (rc != ISK_OK) return rc;
  rc = check_decode_args(*desc, q, kv_pages, block_table, lens, topk_idx, topk_len, out, lse);
  if (rc != ISK_OK) {
    const std::string msg = isk_last_error();
    (void)isk_plan_destroy(plan);
    return set_err(rc, msg);
  }
  hipStream_t stream = (hipStream_t)stream_v;
  const size_t bytes = plan->layout.total;
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, bytes, stream);
  if (e != hipSuccess) {
    (void)isk_plan_destroy(plan);
    return hip_err(e, "hipMallocAsync (workspace)");
  }
  if (((uintptr_t)ws & 255u) != 0) {
    (void)hipFreeAsync(ws, stream);
    (void)isk_plan_destroy(plan);
    return set_err(ISK_ERR_WORKSPACE, "hipMallocAsync returned a workspace that is not 256-byte aligned");
  }
  rc = isk_attn_decode(plan, q, kv_pages, block_table, lens, topk_idx, topk_len, out, lse, ws, bytes, stream_v);
  const std::string msg = rc != ISK_OK ? std::string(isk_last_error()) : std::string();
  e = hipFreeAsync(ws, stream);
  // Waits until the split-list upload has executed (the kernels read the
  // device copy in the workspace, not the plan's staging memory).
  (void)isk_plan_destroy(plan);
  if (rc != ISK_OK) return set_err(rc, msg);
  if (e != hipSuccess) return hip_err(e, "hipFreeAsync (workspace)");
  return ISK_OK;
}

int isk_rmsnorm(const void* x, const void* w, void* y, int32_t rows, int32_t dim, float eps, void* stream) {
  if (rows < 0) return set_err(ISK_ERR_INVALID_ARG, "rows must be >= 0");
  if (dim < 8 || dim > isk::kRmsNormMaxDim || dim % 8 != 0) {
    std::ostringstream s;
    s << "dim must be a multiple of 8 in [8, " << isk::kRmsNormMaxDim << "]";
    return set_err(ISK_ERR_UNSUPPORTED, s.str());
  }
  if (!std::isfinite(eps) || eps < 0.f) return set_err(ISK_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (rows == 0) return ISK_OK;
  if (x == nullptr || w == nullptr || y == nullptr) return set_err(ISK_ERR_INVALID_ARG, "x, w and y must be non-NULL");
  if ((uintptr_t)x % 16 != 0 || (uintptr_t)w % 16 != 0 || (uintptr_t)y % 16 != 0)
    return set_err(ISK_ERR_INVALID_ARG, "x, w and y must be 16-byte aligned");
  isk::RmsNormLaunch a{(const uint16_t*)x, (const uint16_t*)w, (uint16_t*)y, rows, dim, eps};
  const hipError_t e = isk::launch_rmsnorm(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_err(e, "launching the RMSNorm kernel");
  return ISK_OK;
}

int isk_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
  if (src == nullptr || sink == nullptr) return set_err(ISK_ERR_INVALID_ARG, "src and sink must be non-NULL");
  if (bytes == 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0)
    return set_err(ISK_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 and src 16-byte aligned");
  if (blocks < 1 || blocks > 65536) return set_err(ISK_ERR_INVALID_ARG, "blocks must be in [1, 65536]");
  const hipError_t e = isk::launch_hbm_read(src, bytes, sink, blocks, (hipStream_t)stream);
  if (e != hipSuccess) return hip_err(e, "launching the HBM read probe");
  return ISK_OK;
}

int isk_hbm_gather_probe(const void* src, size_t src_bytes, const int32_t* rows, int32_t n_rows, int32_t row_bytes,
                         uint32_t* sink, int32_t blocks, void* stream) {
  if (src == nullptr || rows == nullptr || sink == nullptr)
    return set_err(ISK_ERR_INVALID_ARG, "src, rows and sink must be non-NULL");
  if (row_bytes <= 0 || row_bytes % 16 != 0 || (uintptr_t)src % 16 != 0 || (uintptr_t)rows % 4 != 0)
    return set_err(ISK_ERR_INVALID_ARG, "row_bytes must be a positive multiple of 16, src 16-byte and rows 4-byte aligned");
  if (n_rows < 1) return set_err(ISK_ERR_INVALID_ARG, "n_rows must be >= 1");
  if (src_bytes < (size_t)row_bytes) return set_err(ISK_ERR_INVALID_ARG, "src_bytes is smaller than one row");
  if (blocks < 1 || blocks > 65536) return set_err(ISK_ERR_INVALID_ARG, "blocks must be in [1, 65536]");
  const hipError_t e = isk::launch_hbm_gather(src, rows, n_rows, row_bytes, sink, blocks, (hipStream_t)stream);
  if (e != hipSuccess) return hip_err(e, "launching the HBM gather probe");
  return ISK_OK;
}

int isk_linear_bf16(const void* x, const void* w, float* y, int32_t m, int32_t n, int32_t k, void* stream) {
  if (m < 0) return set_err(ISK_ERR_INVALID_ARG, "m must be >= 0");
  if (n <= 0 || n % 16 != 0) return set_err(ISK_ERR_UNSUPPORTED, "n must be a positive multiple of 16");
  if (k <= 0 || k % 128 != 0) return set_err(ISK_ERR_UNSUPPORTED, "k must be a positive multiple of 128");
  if (m == 0) return ISK_OK;
  if (x == nullptr || w == nullptr || y == nullptr) return set_err(ISK_ERR_INVALID_ARG, "x, w and y must be non-NULL");
  if ((uintptr_t)x % 16 != 0 || (uintptr_t)w % 16 != 0 || (uintptr_t)y % 4 != 0)
    return set_err(ISK_ERR_INVALID_ARG, "x and w must be 16-byte aligned, y 4-byte aligned");
  isk::LinearLaunch a{(const uint16_t*)x, (const uint16_t*)w, y, m, n, k};
  const hipError_t e = isk::launch_linear(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_err(e, "launching the linear kernel");
  return ISK_OK;
}

int isk_plan_set_timing_events(isk_plan* plan, void* split_begin, void* split_end, void* combine_end) {
  if (plan == nullptr) return set_err(ISK_ERR_INVALID_ARG, "plan is NULL");
  plan->t_split_begin = (hipEvent_t)split_begin;
  plan->t_split_end = (hipEvent_t)split_end;
  plan->t_combine_end = (hipEvent_t)combine_end;
  return ISK_OK;
}

}  // extern "C"
