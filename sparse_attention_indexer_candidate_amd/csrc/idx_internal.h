// Internal interface between the C-ABI entry points (idx_api.hip) and the kernel
// launchers (idx_expand.hip, idx_sparse.hip, idx_row_groups.hip, idx_dense.hip,
// idx_gather.hip, idx_measure.hip; their shared device code is idx_device.h).  Not
// installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace idx {

constexpr int kHeads = 64;
constexpr int kHeadDim = 128;

// Layout of idx_schedule.work for a capacity of R rows: int32 kept[R] (sparse blocks
// listed per row), then int32 pages[R][nsb] (the page holding each listed sparse
// block, resolved through the block table once per step).
inline size_t schedule_work_bytes(int32_t max_rows, int32_t nsb) {
    return (size_t)(max_rows > 0 ? max_rows : 0) * (1 + (size_t)nsb) * sizeof(int32_t);
}

struct KCache {
    const uint8_t *values;
    int64_t values_page_stride;
    const uint8_t *scales;
    int64_t scales_page_stride;
    int64_t num_pages;
    const int32_t *block_table;
    int64_t block_table_stride;
    int32_t num_tables;
    int32_t pages_per_table;
    int32_t page_size;
};

struct Rows {
    int32_t num_rows;
    const int32_t *ks;     // may be null (all 0)
    const int32_t *ke;
    const int32_t *table;  // may be null (row r -> r)
    int32_t rows_per_request;   // > 1: consecutive rows share K (placement hint)
};

struct Schedule {
    int32_t *sparse_indices;  // [rows][nsb]
    int32_t *end;             // [rows]
    int32_t *kept;            // [rows]
    int32_t *pages;           // [rows][nsb]
    int32_t nsb;              // sparse blocks per row
    int32_t sbk;              // tokens per sparse block (16, 32 or 64)
    int32_t lsbk;             // log2(sbk)
};

hipError_t launch_expand(const Rows &rows, const KCache &k, const int32_t *cand, int64_t cand_stride,
                         int32_t nb, int32_t cbs, const Schedule &s, hipStream_t stream);

// The sparse path: scores every sparse column of every row and writes each row's
// top-k into out.  With at least as many rows as CUs one launch does both per row
// (logits in LDS; copied to logits_out if given); otherwise a split scoring launch
// writes logits [rows][nsb*sbk] to logits_out or workspace and a second launch
// selects.
// Events attached to the scoring kernel's dispatch, which timestamps its start and end
// (null: none).
struct Timing {
    hipEvent_t start, stop;
};

// Launch plans of the sparse path (the C ABI's IDX_PLAN_* values).  One rule picks the
// plan for the launchers below and for idx_sparse_plan, so callers that account for a
// call's kernels (a benchmark) read the same choice the launch makes.
enum Plan : int {
    kPlanNone = 0,            // no rows or no layers: nothing is launched
    kPlanSplit = 1,           // per layer: score_split_kernel, then topk_split_kernel
    kPlanOneRow = 2,          // per layer: fused_row_kernel (one workgroup scores and selects a row)
    kPlanRowGroup = 3,        // per layer: row_group_kernel (2-row groups share K tiles)
    kPlanSplitLayers = 4,     // all layers: score_split_layers_kernel, then topk_split_layers_kernel
    kPlanOneRowLayers = 5,    // all layers in one fused_layers_kernel launch
    kPlanRowGroupLayers = 6,  // all layers in one row_group_layers_kernel launch
};

// CUs of the calling thread's current device (256 if the query fails).
int device_cus();

// The plan of a sparse call: q_format, sparse block size, candidate columns a row
// (NB*cbs), rows, layers, the device's CUs, and whether every layer's logits have a
// home for a batched split launch (each layer's logits_out, or a workspace of
// num_layers * num_rows * ncols floats).
Plan plan_sparse(int q_format, int32_t sbk, int32_t ncols, int32_t num_rows, int32_t num_layers,
                 int cus, bool logits_home);

// score_format: 0 = fp32 weights [rows][64] and fp32 logits; 1 = bf16 weights (codes,
// 8-byte aligned rows) and every logit rounded to bf16 before the selection.
hipError_t launch_sparse(int q_format, int score_format, const Rows &rows, const void *q_values,
                         const void *q_scales, const void *weights, const KCache &k,
                         const Schedule &s, float *logits_out, float *workspace, int32_t topk,
                         int32_t *out, int64_t out_stride, const Timing &timing,
                         hipStream_t stream);

// Per-layer pointers of a multi-layer sparse call (layers [0, num_layers) used).  The
// layers share the rows, the schedule and every KCache field but the two pools.
constexpr int kMaxLayers = 8;
struct LayerSet {
    const void *q_values[kMaxLayers];
    const void *q_scales[kMaxLayers];
    const void *weights[kMaxLayers];
    const uint8_t *k_values[kMaxLayers];
    const uint8_t *k_scales[kMaxLayers];
    float *logits_out[kMaxLayers];   // entries may be null
    int32_t *out[kMaxLayers];
};

// The sparse path for num_layers layers.  With two or more layers: rows that take the
// one-row kernel run every layer in one launch, two rows a CU; fewer rows than CUs run
// every layer in one split scoring launch and one selection launch (grid z / y = layer)
// when each layer's logits have a home (its logits_out, or its slice of a workspace of
// num_layers * rows * NB*cbs floats).  The timing events ride on the (scoring) launch.
// Otherwise each layer is launched as launch_sparse does, in layer order, reusing the
// workspace (the events ride on every layer's scoring launch, so they time the last).
hipError_t launch_sparse_layers(int q_format, int score_format, const Rows &rows,
                                int32_t num_layers, const LayerSet &layers, const KCache &k,
                                const Schedule &s, float *workspace, size_t workspace_bytes,
                                int32_t topk, int64_t out_stride, const Timing &timing,
                                hipStream_t stream);

// launch_expand then launch_sparse_layers, with the expansion inside the scoring launch
// where expansion_place says so (nb <= 128): the one-row kernels in one round (plan
// kPlanOneRow / kPlanOneRowLayers, sbk = 64, rows x layers <= 2 x CUs for MXFP4 queries,
// < 2 x CUs for fp8: their 8-wave shapes), or
// the split scoring launch in one round (plan kPlanSplit with one layer, kPlanSplitLayers;
// fp8 queries only with sbk = 64).  Each workgroup
// expands its row in LDS and one workgroup a row writes the schedule, the same values
// launch_expand writes.  Otherwise the expansion launch, then launch_sparse_layers.
enum ExpandPlace : int {
    kExpandLaunch = 0,   // launch_expand, then the scoring launches
    kExpandOneRow = 1,   // expand_fused_row_kernel / expand_fused_layers_kernel
    kExpandSplit = 2,    // score_split_expand_kernel / score_split_expand_layers_kernel
};
ExpandPlace expansion_place(int q_format, int32_t sbk, int32_t nb, int32_t ncols,
                            int32_t num_rows, int32_t num_layers, int cus, bool logits_home);
hipError_t launch_expand_sparse_layers(int q_format, int score_format, const Rows &rows,
                                       int32_t num_layers, const LayerSet &layers,
                                       const KCache &k, const Schedule &s, const int32_t *cand,
                                       int64_t cand_stride, int32_t nb, int32_t cbs,
                                       float *workspace, size_t workspace_bytes, int32_t topk,
                                       int64_t out_stride, const Timing &timing,
                                       hipStream_t stream);

// Row groups (plan kPlanRowGroup / kPlanRowGroupLayers; MXFP4 queries, sbk = 64, NB*cbs <=
// 8192): two rows a workgroup share K tiles, logits in LDS, selected in turn.  Called by
// launch_sparse / launch_sparse_layers when their plan says so; the events ride on the
// launch.
hipError_t launch_row_groups(const Rows &rows, const void *q_values, const void *q_scales,
                             const void *weights, int sf, const KCache &k, const Schedule &s,
                             float *logits_out, int32_t topk, int32_t *out, int64_t out_stride,
                             const Timing &timing, hipStream_t stream);
hipError_t launch_row_groups_layers(const Rows &rows, int32_t num_layers, const LayerSet &layers,
                                    int sf, const KCache &k, const Schedule &s, int32_t topk,
                                    int64_t out_stride, const Timing &timing, hipStream_t stream);

// Scores every token t < max_ctx of every row into logits [rows][logits_stride]
// (-inf outside [ks, ke)).
hipError_t launch_score_dense(int q_format, int score_format, const Rows &rows, int32_t max_ctx,
                              const void *q_values, const void *q_scales, const void *weights,
                              const KCache &k, float *logits, int64_t logits_stride,
                              const Timing &timing, hipStream_t stream);

// The candidate-source layer's publication: every token of [ks, ke) of each row scored
// (logits optional: null, or [rows][logits_stride] with -inf outside [ks, ke)), blocks of
// cbs tokens scored by their largest logit, the nb best blocks written to cand [rows]
// [cand_stride] ascending, then -1.  parts: scratch of rows * publish_parts_per_row
// uint32.  Requires ceil(max_ctx / cbs) <= kMaxPublishBlocks and nb <= 512.
constexpr int kMaxPublishBlocks = 4096;
inline int64_t publish_parts_per_row(int32_t max_ctx, int32_t cbs) {
    const int64_t p = cbs >= 64 ? 64 : cbs;
    return ((int64_t)max_ctx + 63) / 64 * (64 / p);
}
hipError_t launch_publish(int q_format, int score_format, const Rows &rows, int32_t max_ctx,
                          const void *q_values, const void *q_scales, const void *weights,
                          const KCache &k, int32_t cbs, int32_t nb, int32_t *cand,
                          int64_t cand_stride, float *logits, int64_t logits_stride,
                          uint32_t *parts, const Timing &timing, hipStream_t stream);

// Per-row top-k over the dense logits (tokens masked to the schedule's blocks).
hipError_t launch_dense_topk(const Rows &rows, const KCache &k, const Schedule &s,
                             const float *logits, int64_t logits_stride, int32_t ncols,
                             int32_t topk, int32_t *out, int64_t out_stride, hipStream_t stream);

// Packs requests' paged K into a contiguous workspace (see gather_k_kernel).
hipError_t launch_gather_k(const KCache &k, int32_t num_reqs, const int32_t *cu_seq_lens,
                           const int32_t *req_table, int32_t max_seq_len, int32_t max_tokens,
                           uint8_t *values_out, uint8_t *scales_out, const Timing &timing,
                           hipStream_t stream);

// Reference kernels for the rates that bound the indexer (measurement only).
constexpr int kMeasureWgs = 4096;   // workgroups of 256 threads
hipError_t launch_measure_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);
hipError_t launch_measure_mfma(int32_t iters, float *sink, hipStream_t stream);
hipError_t launch_measure_mfma_relu(int32_t iters, float *sink, hipStream_t stream);
hipError_t launch_measure_fp8_dot(const uint8_t *q, const uint8_t *kv, const uint8_t *ks,
                                  int32_t mode, float *out, hipStream_t stream);

}  // namespace idx
