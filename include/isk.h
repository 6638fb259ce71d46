/*
 * isk.h - C ABI of the batch-invariant split-KV decode-attention library
 * (libisk.so, built for AMD Instinct MI355X / gfx950).
 *
 * What the library computes.  For every batch row b and query head h it
 * returns softmax attention of the row's query over the row's own keys and
 * values, plus the natural-log log-sum-exp of the scaled scores:
 *     s_t = scale * <q[b,h,:], k_t>,  lse = ln sum_t exp(s_t),
 *     out[b,h,:] = sum_t exp(s_t - lse) * v_t.
 * It computes this the split-KV way described on the FlashMLA issue page
 * "Sparse MLA decode is not batch-invariant ..." (section "Where it comes
 * from"): each row's keys are cut into splits, every split yields a partial
 * output and its log-sum-exp, and a combine step merges the partials with
 * log-sum-exp weights.  Unlike the scheduler that page describes, the
 * default split rule here follows the request in that page's section
 * "Question": a row's split count and split boundaries are a function of
 * that row's own length (or top-k count) and fixed library constants only,
 * never of batch-wide totals, and the combine runs in a fixed order.  A
 * row's output bits therefore do not depend on its batchmates or its
 * position in the batch.
 *
 * Kinds:
 *   ISK_KIND_GQA  dense grouped-query attention; query head h reads kv head
 *                 h / (Hq / Hkv).
 *   ISK_KIND_MLA  absorbed multi-head latent attention: one shared latent
 *                 row of head_dim_qk (576) values per token is the key, its
 *                 first head_dim_v (512) values are the value.  With
 *                 topk_width > 0 each row attends only the positions listed
 *                 in its top-k index array (the sparse call of the page's
 *                 section "Measurement": indices plus a per-row valid count).
 *
 * Conventions for every entry point:
 *   - Return value: ISK_OK (0) or a negative isk_status.  Nothing throws or
 *     aborts across the ABI; on failure isk_last_error() gives a message.
 *   - Tensors are dense, row-major, and device pointers unless the name ends
 *     in _host.  The caller owns all tensors and the workspace; the library
 *     owns only plans.  bf16 means IEEE binary32 truncated to its top 16
 *     bits (the usual bfloat16 layout).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     isk_attn_decode only enqueues work on it and returns.
 */
#ifndef ISK_H
#define ISK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define ISK_API __attribute__((visibility("default")))
#else
#define ISK_API
#endif

typedef enum isk_status {
  ISK_OK = 0,
  ISK_ERR_INVALID_ARG = -1,   /* bad pointer, size, shape or enum value          */
  ISK_ERR_UNSUPPORTED = -2,   /* valid request this build has no kernel for      */
  ISK_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required      */
  ISK_ERR_INDEX = -4,         /* check_inputs found a table/index entry invalid   */
  ISK_ERR_HIP = -5,           /* a HIP runtime call failed (message has detail)  */
  ISK_ERR_RANGE = -6          /* check_inputs found a value the kernel cannot take */
} isk_status;

typedef enum isk_kind { ISK_KIND_GQA = 0, ISK_KIND_MLA = 1 } isk_kind;

/* ISK_SPLIT_PER_ROW: split count ceil(units_b / split_tokens) from the row's
 * own units only (tokens, or top-k slots for sparse rows); batch-invariant.
 * ISK_SPLIT_BATCH_BALANCED: comparison mode reproducing the batch-wide
 * scheduler that the FlashMLA issue page describes (section "Where it comes
 * from"): a per-part block quota computed from the sum over the whole batch,
 * then greedy packing that cuts rows at part boundaries.  Deterministic for
 * a fixed batch, but a row's bits depend on its batchmates. */
typedef enum isk_split_mode { ISK_SPLIT_PER_ROW = 0, ISK_SPLIT_BATCH_BALANCED = 1 } isk_split_mode;

typedef enum isk_out_dtype { ISK_OUT_BF16 = 0, ISK_OUT_F32 = 1 } isk_out_dtype;

typedef struct isk_desc {
  int32_t kind;              /* isk_kind                                              */
  int32_t num_q_heads;       /* Hq.  GQA: Hkv * {1,2,4,8,16}.  MLA: multiple of 16,
                                and of 64 above 64                                    */
  int32_t num_kv_heads;      /* Hkv.  MLA: must be 1                                  */
  int32_t head_dim_qk;       /* GQA: 64 or 128.  MLA: 576                             */
  int32_t head_dim_v;        /* GQA: equal to head_dim_qk.  MLA: 512                  */
  int32_t page_size;         /* tokens per KV page (dense MLA: a multiple of 64)      */
  int32_t num_pages;         /* pages in the pool; block-table entries must be below  */
                             /* it.  MLA: num_pages * page_size below 2^31            */
  int32_t max_pages_per_row; /* row stride of block_table                             */
  int32_t topk_width;        /* 0: dense.  >0 (MLA only): row stride of topk_idx      */
  int32_t split_mode;        /* isk_split_mode                                        */
  int32_t split_tokens;      /* 0: library constant for the kind; else a multiple of
                                the kind's tile (GQA 64, MLA 64)                      */
  int32_t out_dtype;         /* isk_out_dtype                                         */
  int32_t check_inputs;      /* 1: copy tables to the host and validate them first    */
  float scale;               /* score scale (finite, > 0), applied in fp32 after the dot product */
} isk_desc;

typedef struct isk_plan isk_plan;   /* opaque, host-owned */

typedef struct isk_plan_info {
  int32_t batch;
  int32_t split_tokens;      /* resolved split length in units (tokens or slots);
                                with a band table, the longest one any row uses   */
  int32_t num_segments;      /* splits (one partial output each, or a direct write)  */
  int32_t num_groups;        /* workgroup tasks the split kernel is launched with    */
  int32_t num_partials;      /* partial (o, lse) slots in the workspace              */
  int32_t split_kernel;      /* ISK_KERNEL_* family the plan's decode launches       */
  uint64_t workspace_bytes;  /* minimum workspace size for isk_attn_decode           */
} isk_plan_info;

/*
 * Split-kernel families (isk_plan_info.split_kernel).  Every family computes
 * the same arithmetic for a given kind and head count, so which one runs
 * changes speed, never bits:
 *   ISK_KERNEL_GQA       GQA split kernel.
 *   ISK_KERNEL_MLA_H16   MLA, 16 query heads per wave (head counts that are
 *                        not a multiple of 128).
 *   ISK_KERNEL_MLA_H32   MLA, blocks of 128 heads, 32 heads per wave, tiles
 *                        gathered by compiled code (sparse plans the
 *                        generated loop does not take: a split of more than
 *                        1024 slots, or a latent pool above 4 GiB).
 *   ISK_KERNEL_MLA_H128  MLA, blocks of 128 heads, the generated tile loop
 *                        (dense rows; sparse rows within the limits above).
 */
#define ISK_KERNEL_GQA 1
#define ISK_KERNEL_MLA_H16 2
#define ISK_KERNEL_MLA_H32 3
#define ISK_KERNEL_MLA_H128 4

/*
 * isk_plan_create - plan the splits of one decode batch on the host.
 *
 * desc           problem description (copied; the caller may free it).
 * batch          number of rows B (>= 1).
 * lens_host      [B] host int32 KV lengths L_b >= 0, L_b <= max_pages_per_row
 *                * page_size.  Must equal the device `lens` later passed to
 *                isk_attn_decode.
 * topk_len_host  [B] host int32 valid top-k counts for sparse MLA (clamped to
 *                [0, topk_width]), NULL when dense.
 * plan_out       receives the new plan.
 *
 * Per-row mode implements the per-row split rule requested in the FlashMLA
 * issue page, section "Question".  The planning is host work.  A plan whose
 * split list is uploaded to the device (extra source, balanced mode, or more
 * than 640 splits or 128 rows) also gets its pinned staging ring
 * here: four host buffers of the split-list size with half again of
 * headroom, and four events, so that isk_attn_decode allocates nothing.  On
 * a machine without a usable GPU the plan is still made (for host-side use:
 * query, segments) but cannot be decoded with (ISK_ERR_HIP).  Errors:
 * ISK_ERR_INVALID_ARG, ISK_ERR_UNSUPPORTED (no kernel for the shape).
 */
ISK_API int isk_plan_create(const isk_desc* desc, int32_t batch, const int32_t* lens_host,
                    const int32_t* topk_len_host, isk_plan** plan_out);

/*
 * Length band of a per-row split table.  The FlashMLA issue page (section
 * "Question") asks for split counts that depend only on a row's own length
 * and fixed constants; a band table is such a function, piecewise in the
 * length: each band has its own split length and an optional split cap.
 *   max_units    rows with units U <= max_units belong to the first such band
 *                (bounds strictly increasing; the last band also takes every
 *                longer row).
 *   split_units  S of the band: a positive multiple of 64.
 *   max_splits   0: no cap.  Else, when ceil(U / S) > max_splits, the row's
 *                split length becomes 64 * ceil(ceil(U / max_splits) / 64),
 *                so it gets at most max_splits longer splits.
 *   reserved     must be 0.
 */
typedef struct isk_split_band {
  int32_t max_units;
  int32_t split_units;
  int32_t max_splits;
  int32_t reserved;
} isk_split_band;

/*
 * isk_plan_create_banded - isk_plan_create with a per-row split length taken
 * from a band table instead of one constant.  Row b (units U_b: tokens, or
 * valid top-k slots when sparse) gets n_b = ceil(U_b / S_b) splits
 * [i*S_b, min((i+1)*S_b, U_b)), S_b the band rule above, so its splits, and
 * its output bits, still depend on U_b and the table only.  A table whose
 * first band covers every length with split_units S and no cap plans exactly
 * as isk_plan_create with split_tokens S.
 *
 * bands      [n_bands] host array (copied), 1 <= n_bands <= 16.
 * desc       as for isk_plan_create, with split_mode ISK_SPLIT_PER_ROW and
 *            split_tokens 0.  Other arguments as for isk_plan_create.
 * isk_plan_update re-plans with the same table.  Plans of this kind are not
 * combined with an extra KV source.  Host only.
 * Errors: ISK_ERR_INVALID_ARG (table or descriptor), ISK_ERR_UNSUPPORTED.
 */
ISK_API int isk_plan_create_banded(const isk_desc* desc, const isk_split_band* bands, int32_t n_bands,
                                   int32_t batch, const int32_t* lens_host, const int32_t* topk_len_host,
                                   isk_plan** plan_out);

/*
 * isk_plan_update - re-plan an existing plan in place for new lengths (the
 * next decode step), keeping its descriptor, its band table (if any) and its
 * pinned staging ring.  When the new split list outgrows the ring's buffers
 * they are re-allocated here (each after its last upload has executed);
 * otherwise no allocation.  Same arguments and errors as isk_plan_create.
 * Decode calls already enqueued keep the split list they uploaded.  Must not
 * run while another thread decodes with the same plan.
 */
ISK_API int isk_plan_update(isk_plan* plan, int32_t batch, const int32_t* lens_host,
                    const int32_t* topk_len_host);

/* isk_plan_destroy - free a plan (NULL is accepted).  Waits until the plan's
 * pending split-list uploads have executed, then frees its pinned staging
 * memory.  The caller must not destroy a plan while another thread uses it. */
ISK_API int isk_plan_destroy(isk_plan* plan);

/* isk_plan_query - sizes of a plan.  Host only. */
ISK_API int isk_plan_query(const isk_plan* plan, isk_plan_info* info_out);

/* isk_plan_workspace_bytes - minimum workspace bytes (0 if plan is NULL). */
ISK_API size_t isk_plan_workspace_bytes(const isk_plan* plan);

/*
 * isk_plan_segments - host copy of the plan's split list, for inspection and
 * tests.  Writes up to `capacity` records of 5 int32 each:
 *   {row, begin, end, partial_slot, group}
 * where [begin, end) is the split's range in the row's units (token
 * positions, or top-k slots for sparse rows), partial_slot is the workspace
 * slot the split writes (-1: the row has one split and writes the output
 * directly), and group is the workgroup task that runs it.  Records are in
 * launch order.  Returns the number of segments (or a negative status).
 */
ISK_API int isk_plan_segments(const isk_plan* plan, int32_t* records_out, int32_t capacity);

/*
 * isk_attn_decode - run split kernels and the fixed-order combine.
 *
 * plan        from isk_plan_create/update.  Its split list is not changed;
 *             an uploaded one goes through the plan's staging ring, whose
 *             slot cursor a lock guards, so threads may decode with one
 *             plan at the same time (each with its own workspace).  The
 *             call allocates no memory and creates no HIP object.
 * q           [B, Hq, head_dim_qk] bf16.
 * kv_pages    GQA: [num_pages, 2, Hkv, page_size, head_dim] bf16 (index 0 = K,
 *             1 = V).  MLA: [num_pages, page_size, 576] bf16; with Hq a
 *             multiple of 128 the V part enters the PV product as fp16 (see
 *             "Value range" below).
 * block_table [B, max_pages_per_row] int32; entry j of row b is the page
 *             holding the row's tokens [j*page_size, (j+1)*page_size).
 * lens        [B] int32 device copy of lens_host.
 * topk_idx    sparse MLA: [B, topk_width] int32 row-local token positions;
 *             a slot below topk_len[b] whose value lies outside [0, L_b)
 *             (e.g. -1) is skipped.  NULL when dense.
 * topk_len    sparse MLA: [B] int32 device copy of topk_len_host (a plan
 *             passed by value rebuilds its split ranges from it, as a dense
 *             one does from lens).  NULL when dense.
 * out         [B, Hq, head_dim_v] bf16 or fp32 (desc.out_dtype); rows with
 *             nothing to attend get 0.
 * lse         [B, Hq] fp32 natural-log LSE of the scaled scores (-inf for
 *             rows with nothing to attend).  May be NULL.
 * workspace   device memory of at least isk_plan_workspace_bytes(plan) bytes,
 *             256-byte aligned; holds the split partials (fp32, or fp16 on
 *             the 128-head MLA path with bf16 output) and the uploaded
 *             split list (a per-row plan of at most 640 splits and 128 rows,
 *             dense or sparse without an extra source, goes to the kernels in
 *             their arguments instead, with no upload).  Must not be shared by calls in flight at the same time.
 * stream      hipStream_t (as void*).
 *
 * Out-of-range block-table entries and top-k positions are masked in the
 * kernels (never dereferenced); with desc.check_inputs = 1 they are instead
 * reported as ISK_ERR_INDEX before any kernel runs (this synchronises the
 * stream and copies the tables to the host).
 *
 * Value range: with Hq a multiple of 128 the MLA kernels take V (the first
 * 512 latent dims of the attended rows) into their PV product as fp16.
 * Every bf16 value of magnitude in [2^-14, 65280] converts exactly; smaller
 * ones become fp16 subnormals (rounded toward zero, absolute error below
 * 2^-24); 65536 and above, infinities and NaN do not fit (a finite one is
 * taken as 65504).  The 16-head path (other head counts) and GQA take any
 * finite bf16 value.  With desc.check_inputs = 1 on the 128-head path, an
 * attended V value of magnitude 65536 or more (or not finite) is reported
 * as ISK_ERR_RANGE, naming its row, position and dim, before any attention
 * kernel runs.  Errors: ISK_ERR_INVALID_ARG, ISK_ERR_WORKSPACE,
 * ISK_ERR_INDEX, ISK_ERR_RANGE, ISK_ERR_HIP.
 */
ISK_API int isk_attn_decode(const isk_plan* plan, const void* q, const void* kv_pages,
                    const int32_t* block_table, const int32_t* lens,
                    const int32_t* topk_idx, const int32_t* topk_len,
                    void* out, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * isk_attn_decode_oneshot - plan, allocate the workspace and decode in one
 * call, for callers that decode a batch once (the signature the pages give
 * for the decode entry: q, KV pages, block table, lengths and optional top-k
 * indices in, out and lse out; FlashMLA issue "Sparse MLA decode is not
 * batch-invariant ...", section "Where it comes from").
 *
 * desc, batch, lens_host, topk_len_host: as for isk_plan_create (host).
 * q .. lse, stream: as for isk_attn_decode.
 *
 * The workspace comes from hipMallocAsync on `stream` and is released with
 * hipFreeAsync on the same stream after the kernels, so the call allocates
 * stream-ordered device memory (unlike isk_attn_decode).  The plan is built
 * and destroyed inside the call; the call returns once the split list has
 * been uploaded, with the kernels still in flight on `stream`.  Output bits
 * equal those of isk_plan_create + isk_attn_decode on the same inputs.
 * Errors: those of isk_plan_create and isk_attn_decode; ISK_ERR_HIP when the
 * stream-ordered allocation fails.
 */
ISK_API int isk_attn_decode_oneshot(const isk_desc* desc, int32_t batch, const int32_t* lens_host,
                            const int32_t* topk_len_host, const void* q, const void* kv_pages,
                            const int32_t* block_table, const int32_t* lens, const int32_t* topk_idx,
                            const int32_t* topk_len, void* out, float* lse, void* stream);

/*
 * Extra KV source of sparse MLA decode.  The sparse FlashMLA call on the
 * FlashMLA issue page "Sparse MLA decode is not batch-invariant ..." also
 * takes extra_indices_in_kvcache / extra_topk_length into a second cache,
 * extra_k_cache (sections "Measurement" and "Environment").  The page names
 * these arguments without defining them; this library reads them as a second
 * gathered key set per row, from its own paged latent cache, attended in the
 * same softmax as the main set: row b attends the valid main positions and
 * the valid extra positions (each checked against its own cache length).
 * The extra set's splits follow the main set's in the row's fixed combine
 * order and are cut by the same per-row rule (the extra top-k count and the
 * sparse split length only), so the output bits stay batch-invariant.
 */
typedef struct isk_extra_desc {
  int32_t page_size;          /* tokens per page of the extra pool (>= 1)          */
  int32_t num_pages;          /* pages in the extra pool                             */
  int32_t max_pages_per_row;  /* columns of the extra block table                    */
  int32_t topk_width;         /* columns of the extra index array (>= 1)             */
} isk_extra_desc;

typedef struct isk_extra_kv {  /* device pointers, owned by the caller */
  const void* kv_pages;          /* [num_pages, page_size, 576] bf16                  */
  const int32_t* block_table;    /* [B, max_pages_per_row] int32                      */
  const int32_t* lens;           /* [B] int32 extra cache length of each row          */
  const int32_t* topk_idx;       /* [B, topk_width] int32 row-local positions         */
  const int32_t* topk_len;       /* [B] int32 device copy of extra_topk_len_host      */
} isk_extra_kv;

/*
 * isk_plan_create_extra - plan a sparse MLA batch with an extra KV source.
 *
 * desc                 as for isk_plan_create; must be ISK_KIND_MLA with
 *                      topk_width > 0 and split_mode ISK_SPLIT_PER_ROW.
 * extra                the extra source's shape (copied).
 * lens_host,
 * topk_len_host        as for isk_plan_create (main set).
 * extra_topk_len_host  [B] host int32 valid extra top-k counts (clamped to
 *                      [0, extra->topk_width]).
 *
 * Row b gets ceil(topk_len_b / S) main splits followed by
 * ceil(extra_topk_len_b / S) extra splits, S the sparse split length; in
 * isk_plan_segments records an extra split's range is reported shifted by
 * desc->topk_width (slot j of the extra set is unit topk_width + j).  Plans
 * with an extra source are used with isk_attn_decode_extra only and are not
 * re-planned by isk_plan_update (create a new plan).  Host only.  Errors:
 * ISK_ERR_INVALID_ARG, ISK_ERR_UNSUPPORTED.
 */
ISK_API int isk_plan_create_extra(const isk_desc* desc, const isk_extra_desc* extra, int32_t batch,
                                  const int32_t* lens_host, const int32_t* topk_len_host,
                                  const int32_t* extra_topk_len_host, isk_plan** plan_out);

/*
 * isk_attn_decode_extra - isk_attn_decode for a plan from
 * isk_plan_create_extra: the same arguments plus `extra`, a host struct of
 * the extra source's device tensors (all non-NULL).  Extra positions outside
 * [0, extra lens[b]) and extra block-table entries outside the extra pool
 * are masked; with desc.check_inputs = 1 they are reported as ISK_ERR_INDEX
 * instead.  Errors: those of isk_attn_decode.
 */
ISK_API int isk_attn_decode_extra(const isk_plan* plan, const void* q, const void* kv_pages,
                                  const int32_t* block_table, const int32_t* lens,
                                  const int32_t* topk_idx, const int32_t* topk_len,
                                  const isk_extra_kv* extra, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * isk_attn_decode_static - isk_attn_decode without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace is a
 * fixed 64 MiB device array inside the library (one per GPU the library
 * runs on, held until the process ends); the call allocates nothing.  Same
 * kernels, bits and arguments as isk_attn_decode otherwise (no extra KV
 * source).  A plan that needs more than 64 MiB of workspace
 * (isk_plan_workspace_bytes) is rejected with ISK_ERR_WORKSPACE.  Every
 * call on a GPU uses the same array, which keeps the last call's contents:
 * calls that overlap on one GPU (other streams, other threads) race.
 * Errors: those of isk_attn_decode.
 */
ISK_API int isk_attn_decode_static(const isk_plan* plan, const void* q, const void* kv_pages,
                                   const int32_t* block_table, const int32_t* lens, const int32_t* topk_idx,
                                   const int32_t* topk_len, void* out, float* lse, void* stream);

/*
 * isk_rmsnorm - batch-invariant RMS normalisation of `rows` rows:
 *     y[r, i] = x[r, i] / sqrt(mean_j x[r, j]^2 + eps) * w[i].
 * The inference-research gotcha "batch-invariance-is-not-universal-across-
 * kernel-paths" (section "Root cause") names small-batch split reductions in
 * RMSNorm as a batch-invariance breaker; here one workgroup reduces each row
 * in one fixed fp32 order whatever `rows` is, so a row's output bits do not
 * depend on the other rows.
 *
 * x      [rows, dim] bf16, 16-byte aligned (device).
 * w      [dim] bf16, 16-byte aligned (device).
 * y      [rows, dim] bf16 (device), rounded to nearest even; may equal x.
 * rows   >= 0 (0 is a no-op).
 * dim    a multiple of 8 in [8, 16384].
 * eps    finite, >= 0.
 * stream hipStream_t (as void*); the call only enqueues the kernel.
 * Errors: ISK_ERR_INVALID_ARG, ISK_ERR_UNSUPPORTED (dim), ISK_ERR_HIP.
 */
ISK_API int isk_rmsnorm(const void* x, const void* w, void* y, int32_t rows, int32_t dim, float eps, void* stream);

/*
 * isk_linear_bf16 - batch-invariant linear layer y = x w^T:
 *     y[r, j] = sum_k x[r, k] * w[j, k]   (bf16 inputs, fp32 accumulation).
 * The gllm issue "Greedy outputs depend on batch composition (NVFP4
 * GEMV/GEMM switch at 32 rows is a candidate)" (sections "Candidate cause"
 * and "Next steps") traces batch dependence to a kernel switch by row count
 * whose two sides round activations differently.  This entry point also
 * switches tile shapes by row count (one 16- or 32-row tile up to 32 rows,
 * one 64-row tile up to 64, LDS-staged tiles above: 128 x 64, 128 x 128 or
 * 256 x 128 by tile count when k is a multiple of 256, else 128 x 128), but
 * every shape takes
 * bf16 activations and computes each element with the same arithmetic (K
 * split in four fixed quarters, each an MFMA chain in ascending k from
 * zero, the quarters added in order), so the switch changes speed only: a
 * row's outputs do not depend on m.
 *
 * x  [m, k] bf16, 16-byte aligned (device).
 * w  [n, k] bf16 (one row per output feature), 16-byte aligned (device).
 * y  [m, n] fp32 (device); must not overlap x or w.
 * m >= 0 (0 is a no-op); n a positive multiple of 16; k a positive multiple
 * of 128.  stream: hipStream_t (as void*); the call only enqueues the kernel.
 * Errors: ISK_ERR_INVALID_ARG, ISK_ERR_UNSUPPORTED (n, k), ISK_ERR_HIP.
 */
ISK_API int isk_linear_bf16(const void* x, const void* w, float* y, int32_t m, int32_t n, int32_t k, void* stream);

/*
 * isk_hbm_read_probe - measurement utility: one streaming read of `bytes`
 * bytes at `src` (16-byte pieces, grid-stride, nontemporal loads, four in
 * flight per thread), folded with XOR into one 32-bit word per workgroup at
 * sink[0 .. blocks).  Timed with HIP events over a buffer larger than the
 * 256 MB last-level cache, it gives this part's achievable HBM read rate:
 * the second roofline denominator next to the 8 TB/s published figure (the
 * FlashMLA issue page "Sparse MLA decode is not batch-invariant ..." quotes
 * its bandwidth figures against the hardware's memory roofline, section
 * "Measurement / Environment").
 *
 * src    device buffer, 16-byte aligned; bytes a positive multiple of 16.
 * sink   device array of at least `blocks` uint32 (written).
 * blocks workgroups of 256 threads, in [1, 65536].
 * stream hipStream_t (as void*); the call only enqueues the kernel.
 * Errors: ISK_ERR_INVALID_ARG, ISK_ERR_HIP.
 */
ISK_API int isk_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, void* stream);

/*
 * isk_hbm_gather_probe - measurement utility: one read of the `n_rows` rows
 * of `row_bytes` bytes at src + rows[r] * row_bytes (r = 0 .. n_rows-1), in
 * 16-byte pieces in list order (each wave's load instruction covers 1 KiB of
 * consecutive pieces, the same pattern as a sparse top-k tile load), folded
 * with XOR into one 32-bit word per workgroup at sink[0 .. blocks).  With the
 * rows a sparse batch gathers (the FlashMLA issue page "Sparse MLA decode is
 * not batch-invariant ...", section "Where it comes from", top-k attention)
 * it gives the achievable rate of that gather, the sparse path's roofline
 * next to the streaming rate of isk_hbm_read_probe.
 *
 * src        device buffer of src_bytes bytes, 16-byte aligned.
 * rows       [n_rows] device int32 row indices; the caller keeps every
 *            (rows[r] + 1) * row_bytes <= src_bytes (not checked on the device).
 * row_bytes  a positive multiple of 16; n_rows >= 1.
 * sink       device array of at least `blocks` uint32 (written).
 * blocks     workgroups of 256 threads, in [1, 65536].
 * stream     hipStream_t (as void*); the call only enqueues the kernel.
 * Errors: ISK_ERR_INVALID_ARG, ISK_ERR_HIP.
 */
ISK_API int isk_hbm_gather_probe(const void* src, size_t src_bytes, const int32_t* rows, int32_t n_rows,
                                 int32_t row_bytes, uint32_t* sink, int32_t blocks, void* stream);

/*
 * isk_plan_set_timing_events - profiling hook.  Subsequent isk_attn_decode
 * calls with this plan launch the split kernel through hipExtLaunchKernel
 * with `split_begin` and `split_end` as its start and stop events, so they
 * carry the split kernel's own start and end times, and record
 * `combine_end` on the call's stream after the combine kernel (or right
 * after the split kernel when no row needs combining).  Each argument is a
 * hipEvent_t passed as void*; NULL disables that event (with both split
 * events NULL the split kernel is launched the ordinary way).  Meant for
 * timing the kernels with hipEventElapsedTime; the caller owns the events
 * and may swap them between calls.  Host only; never fails for a non-NULL
 * plan.
 */
ISK_API int isk_plan_set_timing_events(isk_plan* plan, void* split_begin, void* split_end, void* combine_end);

/* isk_last_error - message for the last failing call on this thread
 * ("" if none).  The pointer stays valid until the thread's next call. */
ISK_API const char* isk_last_error(void);

/* isk_numerics_id - the build's numerics identity: target architecture, the
 * frozen split and tile constants, the operand precisions and the kernel
 * versions.  Output bits are claimed batch-invariant for a fixed value of
 * this string (and GPU model) only: the page "batch-invariance-is-not-
 * universal-across-kernel-paths" (section "Workaround") says invariance has
 * to be measured on the exact configuration that ships, since another kernel
 * path or precision changes the arithmetic.  Never NULL; owned by the
 * library. */
ISK_API const char* isk_numerics_id(void);

#ifdef __cplusplus
}
#endif

#endif /* ISK_H */
