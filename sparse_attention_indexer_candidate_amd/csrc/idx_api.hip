// C-ABI entry points of libidx (declared in include/idx.h): host-side validation,
// then launches on the caller's stream.  Every check runs before the first HIP call,
// so the error paths need no GPU.
#include "idx.h"
#include "idx_internal.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

namespace {

// Scratch of idx_sparse_mqa_logits_topk_noalloc (the split path's logits, fewer rows
// than CUs), so that entry point needs no workspace and allocates nothing.  Each GPU the
// library runs on holds its own copy for the life of the process.  Host code never uses
// this name as an address (on the host it is a stand-in symbol): scratch_device_ptr()
// looks up each device's copy once with hipGetSymbolAddress and that pointer is what
// the kernels receive.
static_assert(IDX_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte granules");
static __device__ __align__(256) uint8_t scratch[IDX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

thread_local char g_err[512] = "";
thread_local idx::Timing g_timing = {nullptr, nullptr};

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return IDX_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The engine-start checks of the sparse indexer backend builder, restated for
// the gfx950 kernels.  Does not modify cfg.
int check(const idx_config *cfg, int32_t *sbk_out) {
    if (!cfg) return fail(IDX_EINVAL, "config is NULL");
    if (cfg->num_heads != idx::kHeads || cfg->head_dim != idx::kHeadDim)
        return fail(IDX_EUNSUPPORTED, "kernels are built for num_heads=%d head_dim=%d (got %d, %d)",
                    idx::kHeads, idx::kHeadDim, cfg->num_heads, cfg->head_dim);
    if (cfg->q_format != IDX_Q_MXFP4 && cfg->q_format != IDX_Q_FP8_E4M3_ROWSCALE)
        return fail(IDX_EINVAL, "unknown q_format %d", cfg->q_format);
    if (cfg->score_format != IDX_SCORE_FP32 && cfg->score_format != IDX_SCORE_BF16)
        return fail(IDX_EINVAL, "unknown score_format %d", cfg->score_format);
    if (cfg->candidate_block_size <= 0 || cfg->num_candidate_blocks <= 0)
        return fail(IDX_EINVAL, "candidate_block_size (%d) and num_candidate_blocks (%d) must be > 0",
                    cfg->candidate_block_size, cfg->num_candidate_blocks);
    const int32_t cbs = cfg->candidate_block_size;
    int32_t sbk = cfg->sparse_block_kv;
    if (sbk == 0) {
        if (cbs % 64 == 0) sbk = 64;
        else if (cbs == 16 || cbs == 32) sbk = cbs;
        else return fail(IDX_EUNSUPPORTED, "no sparse block size for candidate_block_size %d "
                         "(need a multiple of 64, or 16 or 32)", cbs);
    } else if (!(sbk == 16 || sbk == 32 || sbk == 64) || cbs % sbk != 0) {
        return fail(IDX_EUNSUPPORTED, "sparse_block_kv %d must be 16, 32 or 64 and divide "
                    "candidate_block_size %d", sbk, cbs);
    }
    if (cfg->page_size <= 0 || cfg->page_size % sbk != 0)
        return fail(IDX_EINVAL, "page_size %d must be a positive multiple of sparse_block_kv %d",
                    cfg->page_size, sbk);
    const int64_t cols = (int64_t)cfg->num_candidate_blocks * cbs;
    if (cols > IDX_MAX_ROW_COLS)
        return fail(IDX_EUNSUPPORTED, "num_candidate_blocks * candidate_block_size = %lld exceeds %d",
                    (long long)cols, IDX_MAX_ROW_COLS);
    if (cfg->topk < 1 || cfg->topk > cols || cfg->topk > IDX_MAX_TOPK)
        return fail(IDX_EINVAL, "topk %d must be in [1, min(%lld, %d)]", cfg->topk,
                    (long long)cols, IDX_MAX_TOPK);
    if (sbk_out) *sbk_out = sbk;
    return IDX_OK;
}

int check_filled(const idx_config *cfg, int32_t *sbk) {
    int rc = check(cfg, sbk);
    if (rc) return rc;
    if (cfg->sparse_block_kv == 0)
        return fail(IDX_EINVAL, "config not checked: call idx_check_config first");
    return IDX_OK;
}

int check_rows(const idx_rows *rows) {
    if (!rows) return fail(IDX_EINVAL, "rows is NULL");
    if (rows->num_rows < 0) return fail(IDX_EINVAL, "num_rows %d < 0", rows->num_rows);
    if (rows->num_rows > 0 && !rows->row_ke) return fail(IDX_EINVAL, "row_ke is NULL");
    if (rows->rows_per_request < 0)
        return fail(IDX_EINVAL, "rows_per_request %d < 0", rows->rows_per_request);
    return IDX_OK;
}

int check_kcache(const idx_config *cfg, const idx_kcache *k) {
    if (!k) return fail(IDX_EINVAL, "k cache is NULL");
    if (!k->values || !k->scales || !k->block_table)
        return fail(IDX_EINVAL, "k cache values, scales and block_table must be non-NULL");
    if (k->num_pages <= 0 || k->num_tables <= 0 || k->pages_per_table <= 0)
        return fail(IDX_EINVAL, "num_pages, num_tables and pages_per_table must be > 0");
    if (k->block_table_stride < k->pages_per_table)
        return fail(IDX_EINVAL, "block_table_stride %lld < pages_per_table %d",
                    (long long)k->block_table_stride, k->pages_per_table);
    const int64_t vrow = (int64_t)cfg->page_size * (idx::kHeadDim / 2);
    const int64_t srow = (int64_t)cfg->page_size * (idx::kHeadDim / 32);
    if (k->values_page_stride < vrow || k->scales_page_stride < srow)
        return fail(IDX_EINVAL, "page strides (%lld, %lld) smaller than a page's values / scales "
                    "(%lld, %lld bytes)", (long long)k->values_page_stride,
                    (long long)k->scales_page_stride, (long long)vrow, (long long)srow);
    if (!aligned(k->values, 16) || k->values_page_stride % 16 != 0)
        return fail(IDX_EINVAL, "k values base and page stride must be 16-byte aligned");
    if (!aligned(k->block_table, 4)) return fail(IDX_EINVAL, "block_table must be 4-byte aligned");
    return IDX_OK;
}

int check_schedule(const idx_config *cfg, const idx_rows *rows, const idx_schedule *sched) {
    if (!sched) return fail(IDX_EINVAL, "schedule is NULL");
    if (!sched->sparse_indices || !sched->end || !sched->work)
        return fail(IDX_EINVAL, "schedule sparse_indices, end and work must be non-NULL");
    int32_t sbk = 0;
    check(cfg, &sbk);
    const int32_t nsb = cfg->num_candidate_blocks * (cfg->candidate_block_size / sbk);
    const size_t need = idx::schedule_work_bytes(rows->num_rows, nsb);
    if (sched->work_bytes < need)
        return fail(IDX_EWORKSPACE, "schedule work has %zu bytes, needs %zu", sched->work_bytes,
                    need);
    if (!aligned(sched->sparse_indices, 4) || !aligned(sched->end, 4) || !aligned(sched->work, 4))
        return fail(IDX_EINVAL, "schedule buffers must be 4-byte aligned");
    return IDX_OK;
}

int check_q(const idx_config *cfg, const void *qv, const void *qs, const void *w) {
    if (!qv || !qs || !w) return fail(IDX_EINVAL, "q_values, q_scales and weights must be non-NULL");
    if (!aligned(qv, 16)) return fail(IDX_EINVAL, "q_values must be 16-byte aligned");
    if (cfg->score_format == IDX_SCORE_BF16 ? !aligned(w, 8) : !aligned(w, 4))
        return fail(IDX_EINVAL, "weights must be %d-byte aligned",
                    cfg->score_format == IDX_SCORE_BF16 ? 8 : 4);
    if (cfg->q_format == IDX_Q_FP8_E4M3_ROWSCALE && !aligned(qs, 4))
        return fail(IDX_EINVAL, "fp8 row scales must be 4-byte aligned");
    return IDX_OK;
}

idx::KCache to_kcache(const idx_config *cfg, const idx_kcache *k) {
    return idx::KCache{k->values, k->values_page_stride, k->scales, k->scales_page_stride,
                       k->num_pages, k->block_table, k->block_table_stride, k->num_tables,
                       k->pages_per_table, cfg->page_size};
}

idx::Rows to_rows(const idx_rows *r) {
    return idx::Rows{r->num_rows, r->row_ks, r->row_ke, r->row_table, r->rows_per_request};
}

idx::Schedule to_schedule(const idx_config *cfg, int32_t sbk, const idx_schedule *s) {
    const int32_t nsb = cfg->num_candidate_blocks * (cfg->candidate_block_size / sbk);
    // capacity in rows of the work buffer; its layout depends only on work_bytes and
    // nsb, so every call that passes the same schedule agrees on it
    const size_t cap = s->work_bytes / ((1 + (size_t)nsb) * sizeof(int32_t));
    int32_t *kept = (int32_t *)s->work;
    const int32_t lsbk = sbk == 16 ? 4 : sbk == 32 ? 5 : 6;
    return idx::Schedule{s->sparse_indices, s->end, kept, kept + cap, nsb, sbk, lsbk};
}

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(IDX_EHIP, "%s: %s", what, hipGetErrorString(e));
    return IDX_OK;
}

// The current device's copy of `scratch`, looked up on the first call on that device
// (with that device current) and kept.  Returns IDX_OK and sets *out, or an error.
int scratch_device_ptr(void **out) {
    int dev = 0;
    int rc;
    if ((rc = hip_status(hipGetDevice(&dev), "hipGetDevice"))) return rc;
    if (dev < 0 || dev >= kMaxDevices)
        return fail(IDX_EUNSUPPORTED, "device %d: the scratch table holds %d devices", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if ((rc = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                             "hipGetSymbolAddress(scratch)")))
            return rc;
        if (!p) return fail(IDX_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return IDX_OK;
}

}  // namespace

extern "C" {

int idx_check_config(idx_config *cfg) {
    int32_t sbk = 0;
    int rc = check(cfg, &sbk);
    if (rc) return rc;
    cfg->sparse_block_kv = sbk;
    return ok();
}

int32_t idx_num_sparse_blocks(const idx_config *cfg) {
    int32_t sbk = 0;
    int rc = check(cfg, &sbk);
    if (rc) return rc;
    ok();
    return cfg->num_candidate_blocks * (cfg->candidate_block_size / sbk);
}

size_t idx_schedule_work_bytes(const idx_config *cfg, int32_t max_rows) {
    int32_t sbk = 0;
    if (check(cfg, &sbk)) return 0;
    ok();
    return idx::schedule_work_bytes(max_rows,
                                    cfg->num_candidate_blocks * (cfg->candidate_block_size / sbk));
}

size_t idx_workspace_bytes(const idx_config *cfg, int32_t max_rows, int32_t max_ctx) {
    if (check(cfg, nullptr)) return 0;
    if (max_rows < 0 || max_ctx < 0) {
        fail(IDX_EINVAL, "max_rows and max_ctx must be >= 0");
        return 0;
    }
    ok();
    const size_t sparse = (size_t)max_rows * cfg->num_candidate_blocks * cfg->candidate_block_size;
    const size_t dense = (size_t)max_rows * (((size_t)max_ctx + 63) / 64 * 64);
    return (sparse > dense ? sparse : dense) * sizeof(float);
}

const char *idx_last_error(void) { return g_err; }

int idx_sparse_plan(const idx_config *cfg, int32_t num_rows, int32_t num_layers,
                    int32_t logits_home, idx_plan_info *out) {
    int32_t sbk = 0;
    int rc;
    if ((rc = check(cfg, &sbk))) return rc;
    if (!out) return fail(IDX_EINVAL, "out is NULL");
    if (num_rows < 0) return fail(IDX_EINVAL, "num_rows %d < 0", num_rows);
    if (num_layers < 1 || num_layers > IDX_MAX_LAYERS)
        return fail(IDX_EINVAL, "num_layers %d must be in [1, %d]", num_layers, IDX_MAX_LAYERS);
    const int32_t ncols = cfg->num_candidate_blocks * cfg->candidate_block_size;
    const idx::Plan p = idx::plan_sparse(cfg->q_format, sbk, ncols, num_rows, num_layers,
                                         idx::device_cus(), logits_home != 0);
    static_assert(IDX_PLAN_ROW_GROUP_LAYERS == idx::kPlanRowGroupLayers &&
                  IDX_PLAN_SPLIT == idx::kPlanSplit, "one numbering of the plans");
    idx_plan_info info = {p, 1, 0, "", "", 0, ""};
    switch (p) {
    case idx::kPlanNone: break;
    case idx::kPlanSplit:
        info.scoring_kernel = "score_split_kernel";
        info.selection_kernel = "topk_split_kernel";
        break;
    case idx::kPlanOneRow:
        info.scoring_kernel = "fused_row_kernel";
        info.selects_in_scoring_kernel = 1;
        break;
    case idx::kPlanRowGroup:
        info.scoring_kernel = "row_group_kernel";
        info.selects_in_scoring_kernel = 1;
        break;
    case idx::kPlanSplitLayers:
        info.scoring_kernel = "score_split_layers_kernel";
        info.selection_kernel = "topk_split_layers_kernel";
        info.layers_per_scoring_launch = num_layers;
        break;
    case idx::kPlanOneRowLayers:
        info.scoring_kernel = "fused_layers_kernel";
        info.selects_in_scoring_kernel = 1;
        info.layers_per_scoring_launch = num_layers;
        break;
    case idx::kPlanRowGroupLayers:
        info.scoring_kernel = "row_group_layers_kernel";
        info.selects_in_scoring_kernel = 1;
        info.layers_per_scoring_launch = num_layers;
        break;
    }
    if (p == idx::kPlanNone) info.layers_per_scoring_launch = 0;
    info.expand_and_score_kernel = info.scoring_kernel;
    switch (idx::expansion_place(cfg->q_format, sbk, cfg->num_candidate_blocks, ncols, num_rows,
                                 num_layers, idx::device_cus(), logits_home != 0)) {
    case idx::kExpandLaunch: break;
    case idx::kExpandOneRow:
        info.expansion_in_scoring_kernel = 1;
        info.expand_and_score_kernel =
            p == idx::kPlanOneRow ? "expand_fused_row_kernel" : "expand_fused_layers_kernel";
        break;
    case idx::kExpandSplit:
        info.expansion_in_scoring_kernel = 1;
        info.expand_and_score_kernel = p == idx::kPlanSplit ? "score_split_expand_kernel"
                                                            : "score_split_expand_layers_kernel";
        break;
    }
    *out = info;
    return ok();
}

int idx_set_timing_events(void *start_event, void *stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr))
        return fail(IDX_EINVAL, "timing events must be both set or both NULL");
    g_timing = idx::Timing{(hipEvent_t)start_event, (hipEvent_t)stop_event};
    return ok();
}

int idx_expand_candidates(const idx_config *cfg, const idx_rows *rows, const idx_kcache *k,
                          const int32_t *candidate_blocks, int64_t cand_stride,
                          const idx_schedule *sched, void *stream) {
    int32_t sbk = 0;
    int rc;
    if ((rc = check_filled(cfg, &sbk)) || (rc = check_rows(rows)) || (rc = check_kcache(cfg, k)) ||
        (rc = check_schedule(cfg, rows, sched)))
        return rc;
    if (rows->num_rows > 0 && !candidate_blocks) return fail(IDX_EINVAL, "candidate_blocks is NULL");
    if (cand_stride < cfg->num_candidate_blocks)
        return fail(IDX_EINVAL, "cand_stride %lld < num_candidate_blocks %d",
                    (long long)cand_stride, cfg->num_candidate_blocks);
    const idx::Schedule s = to_schedule(cfg, sbk, sched);
    if ((rc = hip_status(idx::launch_expand(to_rows(rows), to_kcache(cfg, k), candidate_blocks,
                                            cand_stride, cfg->num_candidate_blocks,
                                            cfg->candidate_block_size, s, (hipStream_t)stream),
                         "expand launch")))
        return rc;
    return ok();
}

int idx_sparse_mqa_logits_topk(const idx_config *cfg, const idx_rows *rows, const void *q_values,
                               const void *q_scales, const void *weights, const idx_kcache *k,
                               const idx_schedule *sched, int32_t *topk_indices,
                               int64_t out_stride, float *logits_out, void *workspace,
                               size_t workspace_bytes, void *stream) {
    int32_t sbk = 0;
    int rc;
    if ((rc = check_filled(cfg, &sbk)) || (rc = check_rows(rows)) || (rc = check_kcache(cfg, k)) ||
        (rc = check_schedule(cfg, rows, sched)) || (rc = check_q(cfg, q_values, q_scales, weights)))
        return rc;
    if (!topk_indices || !aligned(topk_indices, 4))
        return fail(IDX_EINVAL, "topk_indices must be non-NULL and 4-byte aligned");
    if (out_stride < cfg->topk)
        return fail(IDX_EINVAL, "out_stride %lld < topk %d", (long long)out_stride, cfg->topk);
    const idx::Schedule s = to_schedule(cfg, sbk, sched);
    const int32_t ncols = s.nsb * s.sbk;
    if (!logits_out) {
        const size_t need = (size_t)rows->num_rows * ncols * sizeof(float);
        if (!workspace && need) return fail(IDX_EWORKSPACE, "workspace is NULL (needs %zu bytes)", need);
        if (workspace_bytes < need)
            return fail(IDX_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
        if (!aligned(workspace, 16)) return fail(IDX_EINVAL, "workspace must be 16-byte aligned");
    } else if (!aligned(logits_out, 16)) {
        return fail(IDX_EINVAL, "logits_out must be 16-byte aligned");
    }
    const idx::Rows r = to_rows(rows);
    const idx::KCache kc = to_kcache(cfg, k);
    hipStream_t st = (hipStream_t)stream;
    if ((rc = hip_status(idx::launch_sparse(cfg->q_format, cfg->score_format, r, q_values,
                                            q_scales, weights, kc, s, logits_out,
                                            (float *)workspace, cfg->topk, topk_indices,
                                            out_stride, g_timing, st),
                         "sparse launch")))
        return rc;
    return ok();
}

int idx_sparse_mqa_logits_topk_noalloc(const idx_config *cfg, const idx_rows *rows,
                                       const void *q_values, const void *q_scales,
                                       const void *weights, const idx_kcache *k,
                                       const idx_schedule *sched, int32_t *topk_indices,
                                       int64_t out_stride, float *logits_out, void *stream) {
    int32_t sbk = 0;
    int rc;
    if ((rc = check_filled(cfg, &sbk)) || (rc = check_rows(rows)) || (rc = check_kcache(cfg, k)) ||
        (rc = check_schedule(cfg, rows, sched)) || (rc = check_q(cfg, q_values, q_scales, weights)))
        return rc;
    if (!topk_indices || !aligned(topk_indices, 4))
        return fail(IDX_EINVAL, "topk_indices must be non-NULL and 4-byte aligned");
    if (out_stride < cfg->topk)
        return fail(IDX_EINVAL, "out_stride %lld < topk %d", (long long)out_stride, cfg->topk);
    if (logits_out && !aligned(logits_out, 16))
        return fail(IDX_EINVAL, "logits_out must be 16-byte aligned");
    if (rows->num_rows == 0) return ok();   // nothing to launch, nothing to look up
    const idx::Schedule s = to_schedule(cfg, sbk, sched);
    const int32_t ncols = s.nsb * s.sbk;
    // Only the split plan (fewer rows than CUs) keeps logits outside the scoring kernel;
    // without logits_out they go to this device's static scratch.
    float *scratch_logits = nullptr;
    if (!logits_out && idx::plan_sparse(cfg->q_format, sbk, ncols, rows->num_rows, 1,
                                        idx::device_cus(), true) == idx::kPlanSplit) {
        const size_t need = (size_t)rows->num_rows * ncols * sizeof(float);
        if (need > IDX_NOALLOC_SCRATCH_BYTES)
            return fail(IDX_EWORKSPACE, "the call needs %zu bytes of logits scratch, more than "
                        "the %u bytes of static scratch (use idx_sparse_mqa_logits_topk with a "
                        "workspace)", need, (unsigned)IDX_NOALLOC_SCRATCH_BYTES);
        void *p = nullptr;
        if ((rc = scratch_device_ptr(&p))) return rc;
        scratch_logits = (float *)p;
    }
    if ((rc = hip_status(idx::launch_sparse(cfg->q_format, cfg->score_format, to_rows(rows),
                                            q_values, q_scales, weights, to_kcache(cfg, k), s,
                                            logits_out,
                                            scratch_logits, cfg->topk, topk_indices, out_stride,
                                            g_timing, (hipStream_t)stream),
                         "sparse launch")))
        return rc;
    return ok();
}

// The checks of a multi-layer call after those of its config, rows and schedule: the
// layer count, every layer's pool, query and outputs (one cache geometry: only values
// and scales may differ from layer 0's), and the workspace when some layer has no
// logits_out.  Fills ls.
static int check_layers(const idx_config *cfg, const idx_rows *rows, int32_t num_layers,
                        const idx_layer *layers, int64_t out_stride, const idx::Schedule &s,
                        void *workspace, size_t workspace_bytes, idx::LayerSet &ls) {
    int rc;
    if (num_layers < 1 || num_layers > IDX_MAX_LAYERS)
        return fail(IDX_EINVAL, "num_layers %d must be in [1, %d]", num_layers, IDX_MAX_LAYERS);
    if (!layers) return fail(IDX_EINVAL, "layers is NULL");
    if (out_stride < cfg->topk)
        return fail(IDX_EINVAL, "out_stride %lld < topk %d", (long long)out_stride, cfg->topk);
    const idx_kcache &k0 = layers[0].k;
    bool need_ws = false;
    ls = {};
    for (int l = 0; l < num_layers; ++l) {
        const idx_layer &L = layers[l];
        if ((rc = check_kcache(cfg, &L.k)) || (rc = check_q(cfg, L.q_values, L.q_scales, L.weights))) {
            char why[sizeof g_err];
            memcpy(why, g_err, sizeof why);
            return fail(rc, "layer %d: %s", l, why);
        }
        const idx_kcache &k = L.k;
        if (k.values_page_stride != k0.values_page_stride ||
            k.scales_page_stride != k0.scales_page_stride || k.num_pages != k0.num_pages ||
            k.block_table != k0.block_table || k.block_table_stride != k0.block_table_stride ||
            k.num_tables != k0.num_tables || k.pages_per_table != k0.pages_per_table)
            return fail(IDX_EINVAL, "layer %d: k cache geometry differs from layer 0's (only "
                        "values and scales may differ)", l);
        if (!L.topk_indices || !aligned(L.topk_indices, 4))
            return fail(IDX_EINVAL, "layer %d: topk_indices must be non-NULL and 4-byte aligned", l);
        if (L.logits_out && !aligned(L.logits_out, 16))
            return fail(IDX_EINVAL, "layer %d: logits_out must be 16-byte aligned", l);
        need_ws = need_ws || !L.logits_out;
        ls.q_values[l] = L.q_values;
        ls.q_scales[l] = L.q_scales;
        ls.weights[l] = L.weights;
        ls.k_values[l] = k.values;
        ls.k_scales[l] = k.scales;
        ls.logits_out[l] = L.logits_out;
        ls.out[l] = L.topk_indices;
    }
    if (need_ws) {
        const size_t need = (size_t)rows->num_rows * s.nsb * s.sbk * sizeof(float);
        if (!workspace && need) return fail(IDX_EWORKSPACE, "workspace is NULL (needs %zu bytes)", need);
        if (workspace_bytes < need)
            return fail(IDX_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
        if (!aligned(workspace, 16)) return fail(IDX_EINVAL, "workspace must be 16-byte aligned");
    }
    return IDX_OK;
}

static_assert(idx::kMaxLayers == IDX_MAX_LAYERS, "one layer limit for the launch and the ABI");

int idx_sparse_mqa_logits_topk_layers(const idx_config *cfg, const idx_rows *rows,
                                      const idx_schedule *sched, int32_t num_layers,
                                      const idx_layer *layers, int64_t out_stride,
                                      void *workspace, size_t workspace_bytes, void *stream) {
    int32_t sbk = 0;
    int rc;
    if ((rc = check_filled(cfg, &sbk)) || (rc = check_rows(rows)) ||
        (rc = check_schedule(cfg, rows, sched)))
        return rc;
    const idx::Schedule s = to_schedule(cfg, sbk, sched);
    idx::LayerSet ls;
    if ((rc = check_layers(cfg, rows, num_layers, layers, out_stride, s, workspace,
                           workspace_bytes, ls)))
        return rc;
    if ((rc = hip_status(idx::launch_sparse_layers(cfg->q_format, cfg->score_format,
                                                   to_rows(rows), num_layers, ls,
                                                   to_kcache(cfg, &layers[0].k), s,
                                                   (float *)workspace,
                                                   workspace ? workspace_bytes : 0, cfg->topk,
                                                   out_stride, g_timing,
                                                   (hipStream_t)stream),
                         "sparse layers launch")))
        return rc;
    return ok();
}

int idx_expand_and_score_layers(const idx_config *cfg, const idx_rows *rows,
                                const int32_t *candidate_blocks, int64_t cand_stride,
                                const idx_schedule *sched, int32_t num_layers,
                                const idx_layer *layers, int64_t out_stride, void *workspace,
                                size_t workspace_bytes, void *stream) {
    int32_t sbk = 0;
    int rc;
    if ((rc = check_filled(cfg, &sbk)) || (rc = check_rows(rows)) ||
        (rc = check_schedule(cfg, rows, sched)))
        return rc;
    if (rows->num_rows > 0 && !candidate_blocks) return fail(IDX_EINVAL, "candidate_blocks is NULL");
    if (cand_stride < cfg->num_candidate_blocks)
        return fail(IDX_EINVAL, "cand_stride %lld < num_candidate_blocks %d",
                    (long long)cand_stride, cfg->num_candidate_blocks);
    const idx::Schedule s = to_schedule(cfg, sbk, sched);
    idx::LayerSet ls;
    if ((rc = check_layers(cfg, rows, num_layers, layers, out_stride, s, workspace,
                           workspace_bytes, ls)))
        return rc;
    if ((rc = hip_status(idx::launch_expand_sparse_layers(
                             cfg->q_format, cfg->score_format, to_rows(rows), num_layers, ls,
                             to_kcache(cfg, &layers[0].k), s, candidate_blocks, cand_stride,
                             cfg->num_candidate_blocks, cfg->candidate_block_size,
                             (float *)workspace, workspace ? workspace_bytes : 0, cfg->topk,
                             out_stride, g_timing, (hipStream_t)stream),
                         "expand and score launch")))
        return rc;
    return ok();
}

int idx_dense_masked_logits_topk(const idx_config *cfg, const idx_rows *rows, int32_t max_ctx,
                                 const void *q_values, const void *q_scales,
                                 const void *weights, const idx_kcache *k,
                                 const idx_schedule *sched, int32_t *topk_indices,
                                 int64_t out_stride, float *logits_out, int64_t logits_stride,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    int32_t sbk = 0;
    int rc;
    if ((rc = check_filled(cfg, &sbk)) || (rc = check_rows(rows)) || (rc = check_kcache(cfg, k)) ||
        (rc = check_schedule(cfg, rows, sched)) || (rc = check_q(cfg, q_values, q_scales, weights)))
        return rc;
    if (max_ctx <= 0 || max_ctx > IDX_MAX_DENSE_COLS)
        return fail(IDX_EUNSUPPORTED, "max_ctx %d must be in [1, %d]", max_ctx, IDX_MAX_DENSE_COLS);
    if (!topk_indices || !aligned(topk_indices, 4))
        return fail(IDX_EINVAL, "topk_indices must be non-NULL and 4-byte aligned");
    if (out_stride < cfg->topk)
        return fail(IDX_EINVAL, "out_stride %lld < topk %d", (long long)out_stride, cfg->topk);
    const int32_t ncols = (max_ctx + 63) / 64 * 64;
    float *logits = logits_out;
    int64_t lstride = logits_stride;
    if (logits) {
        if (lstride < ncols || lstride % 4 != 0)
            return fail(IDX_EINVAL, "logits_stride %lld must be a multiple of 4 and >= %d",
                        (long long)lstride, ncols);
    } else {
        lstride = ncols;
        const size_t need = (size_t)rows->num_rows * ncols * sizeof(float);
        if (!workspace && need) return fail(IDX_EWORKSPACE, "workspace is NULL (needs %zu bytes)", need);
        if (workspace_bytes < need)
            return fail(IDX_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
        logits = (float *)workspace;
    }
    if (!aligned(logits, 16)) return fail(IDX_EINVAL, "logits buffer must be 16-byte aligned");
    const idx::Rows r = to_rows(rows);
    const idx::KCache kc = to_kcache(cfg, k);
    const idx::Schedule s = to_schedule(cfg, sbk, sched);
    hipStream_t st = (hipStream_t)stream;
    if ((rc = hip_status(idx::launch_score_dense(cfg->q_format, cfg->score_format, r, max_ctx,
                                                 q_values, q_scales, weights, kc, logits,
                                                 lstride, g_timing, st),
                         "dense score launch")))
        return rc;
    if ((rc = hip_status(idx::launch_dense_topk(r, kc, s, logits, lstride, ncols, cfg->topk,
                                                topk_indices, out_stride, st),
                         "dense top-k launch")))
        return rc;
    return ok();
}

size_t idx_publish_workspace_bytes(const idx_config *cfg, int32_t max_rows, int32_t max_ctx) {
    if (check(cfg, nullptr)) return 0;
    if (max_rows < 0 || max_ctx < 0) {
        fail(IDX_EINVAL, "max_rows and max_ctx must be >= 0");
        return 0;
    }
    ok();
    return (size_t)max_rows * idx::publish_parts_per_row(max_ctx, cfg->candidate_block_size) *
           sizeof(uint32_t);
}

int idx_publish_candidates(const idx_config *cfg, const idx_rows *rows, int32_t max_ctx,
                           const void *q_values, const void *q_scales, const void *weights,
                           const idx_kcache *k, int32_t *candidate_blocks, int64_t cand_stride,
                           float *logits_out, int64_t logits_stride, void *workspace,
                           size_t workspace_bytes, void *stream) {
    int rc;
    if ((rc = check_filled(cfg, nullptr)) || (rc = check_rows(rows)) ||
        (rc = check_kcache(cfg, k)) || (rc = check_q(cfg, q_values, q_scales, weights)))
        return rc;
    const int32_t cbs = cfg->candidate_block_size, nb = cfg->num_candidate_blocks;
    if (max_ctx <= 0 || ((int64_t)max_ctx + cbs - 1) / cbs > idx::kMaxPublishBlocks)
        return fail(IDX_EUNSUPPORTED, "max_ctx %d must be in [1, %lld] (%d blocks of %d tokens)",
                    max_ctx, (long long)idx::kMaxPublishBlocks * cbs, idx::kMaxPublishBlocks, cbs);
    if (!candidate_blocks || !aligned(candidate_blocks, 4))
        return fail(IDX_EINVAL, "candidate_blocks must be non-NULL and 4-byte aligned");
    if (cand_stride < nb)
        return fail(IDX_EINVAL, "cand_stride %lld < num_candidate_blocks %d",
                    (long long)cand_stride, nb);
    const int64_t ncols = ((int64_t)max_ctx + 63) / 64 * 64;
    if (logits_out && (logits_stride < ncols || !aligned(logits_out, 4)))
        return fail(IDX_EINVAL, "logits_stride %lld must be >= %lld and logits_out 4-byte aligned",
                    (long long)logits_stride, (long long)ncols);
    const size_t need = (size_t)rows->num_rows *
                        idx::publish_parts_per_row(max_ctx, cbs) * sizeof(uint32_t);
    if (need && !workspace) return fail(IDX_EWORKSPACE, "workspace is NULL (needs %zu bytes)", need);
    if (workspace_bytes < need)
        return fail(IDX_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if (!aligned(workspace, 4)) return fail(IDX_EINVAL, "workspace must be 4-byte aligned");
    if ((rc = hip_status(idx::launch_publish(cfg->q_format, cfg->score_format, to_rows(rows),
                                             max_ctx, q_values, q_scales, weights,
                                             to_kcache(cfg, k), cbs, nb, candidate_blocks,
                                             cand_stride, logits_out, logits_stride,
                                             (uint32_t *)workspace, g_timing,
                                             (hipStream_t)stream),
                         "publish launch")))
        return rc;
    return ok();
}

int idx_gather_k_workspace(const idx_config *cfg, const idx_kcache *k, int32_t num_reqs,
                           const int32_t *cu_seq_lens, const int32_t *req_table,
                           int32_t max_seq_len, int32_t max_tokens, uint8_t *values_out,
                           uint8_t *scales_out, void *stream) {
    int rc;
    if ((rc = check_filled(cfg, nullptr)) || (rc = check_kcache(cfg, k))) return rc;
    if (num_reqs < 0 || max_seq_len < 0 || max_tokens < 0)
        return fail(IDX_EINVAL, "num_reqs, max_seq_len and max_tokens must be >= 0");
    if (num_reqs > 65535) return fail(IDX_EUNSUPPORTED, "num_reqs %d > 65535", num_reqs);
    if (num_reqs > 0 && !cu_seq_lens) return fail(IDX_EINVAL, "cu_seq_lens is NULL");
    if (max_tokens > 0 && (!values_out || !scales_out))
        return fail(IDX_EINVAL, "values_out and scales_out must be non-NULL");
    if (!aligned(values_out, 16) || !aligned(scales_out, 4))
        return fail(IDX_EINVAL, "values_out must be 16-byte and scales_out 4-byte aligned");
    if (!aligned(k->scales, 4) || k->scales_page_stride % 4 != 0)
        return fail(IDX_EINVAL, "k scales base and page stride must be 4-byte aligned");
    if ((rc = hip_status(idx::launch_gather_k(to_kcache(cfg, k), num_reqs, cu_seq_lens, req_table,
                                              max_seq_len, max_tokens, values_out, scales_out,
                                              g_timing, (hipStream_t)stream),
                         "gather launch")))
        return rc;
    return ok();
}

int idx_measure_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    if (!src || !sink) return fail(IDX_EINVAL, "src and sink must be non-NULL");
    if (!aligned(src, 16) || bytes % 16 != 0 || bytes == 0)
        return fail(IDX_EINVAL, "src must be 16-byte aligned and bytes a nonzero multiple of 16");
    if (!aligned(sink, 4)) return fail(IDX_EINVAL, "sink must be 4-byte aligned");
    int rc;
    if ((rc = hip_status(idx::launch_measure_read(src, bytes, sink, (hipStream_t)stream),
                         "read launch")))
        return rc;
    return ok();
}

int idx_measure_mfma(int32_t iters, float *sink, void *stream) {
    if (iters < 1) return fail(IDX_EINVAL, "iters %d must be >= 1", iters);
    if (!sink || !aligned(sink, 4)) return fail(IDX_EINVAL, "sink must be non-NULL and 4-byte aligned");
    int rc;
    if ((rc = hip_status(idx::launch_measure_mfma(iters, sink, (hipStream_t)stream), "mfma launch")))
        return rc;
    return ok();
}

int idx_measure_mfma_relu(int32_t iters, float *sink, void *stream) {
    if (iters < 1) return fail(IDX_EINVAL, "iters %d must be >= 1", iters);
    if (!sink || !aligned(sink, 4)) return fail(IDX_EINVAL, "sink must be non-NULL and 4-byte aligned");
    int rc;
    if ((rc = hip_status(idx::launch_measure_mfma_relu(iters, sink, (hipStream_t)stream),
                         "mfma relu launch")))
        return rc;
    return ok();
}

int idx_measure_fp8_dot(const uint8_t *q_e4m3, const uint8_t *k_e2m1, const uint8_t *k_scales,
                        int32_t mode, float *out, void *stream) {
    if (!q_e4m3 || !k_e2m1 || !k_scales || !out)
        return fail(IDX_EINVAL, "q_e4m3, k_e2m1, k_scales and out must be non-NULL");
    if (!aligned(q_e4m3, 16) || !aligned(k_e2m1, 16) || !aligned(out, 4))
        return fail(IDX_EINVAL, "q_e4m3 and k_e2m1 must be 16-byte aligned, out 4-byte aligned");
    if (mode < 0 || mode > 2) return fail(IDX_EINVAL, "mode %d must be 0, 1 or 2", mode);
    int rc;
    if ((rc = hip_status(idx::launch_measure_fp8_dot(q_e4m3, k_e2m1, k_scales, mode, out,
                                                     (hipStream_t)stream),
                         "fp8 dot launch")))
        return rc;
    return ok();
}

static_assert(idx::kMeasureWgs == IDX_MEASURE_WGS, "one workgroup count for the launch and the ABI");

int64_t idx_measure_mfma_flops(int32_t iters) {
    // waves x rounds x 8 chains x (16 x 16 x 128 multiply-adds x 2)
    return (int64_t)IDX_MEASURE_WGS * 4 * (iters > 0 ? iters : 0) * 8 * (16 * 16 * 128 * 2);
}

}  // extern "C"
