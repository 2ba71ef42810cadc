/*
 * idx.h — C ABI of the candidate-consuming sparse MQA-logits indexer for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (vLLM DeepSeek-V4.1 two-level selection; pages
 * vllm.model_executor.layers.sparse_mqa_indexer, the DeepSeek-V4.1 sparse
 * indexer backend source, and vllm.model_executor.layers.rocm_paged_mxfp4_indexer):
 * a candidate-source layer publishes candidate blocks per query row; a consuming
 * layer scores only the tokens inside those blocks, reading a paged MXFP4 K cache
 * in place, and returns the row's top-k token indices.  For a row with query
 * heads q_h (h < H), per-head weights w_h and candidate token set T:
 *
 *     logit[t] = sum_h w_h * max(q_h . k_t, 0)            (fp32 result)
 *     out      = the min(topk, |T|) tokens of T with the largest logits,
 *                ties toward the lower token, in ascending token order,
 *                followed by -1 up to topk.
 *
 * Conventions shared by every entry point:
 *  - Pointers named in the structs and arguments are DEVICE pointers owned by
 *    the caller unless a comment says "host".  Nothing is allocated per call.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously on it; the call returns once the launches are queued.
 *  - Every argument check runs on the host before any launch.  On error the call
 *    returns a negative idx_status, launches nothing, and idx_last_error() gives a
 *    message (per calling thread).
 *  - Device data is trusted as far as the stated preconditions go; page ids
 *    outside [0, num_pages), table rows outside [0, num_tables) and logical pages
 *    outside [0, pages_per_table) are never dereferenced: the affected sparse
 *    blocks are dropped from the schedule instead (so a result computed from such
 *    input is unspecified, but no read leaves the caller's buffers).
 *  - Calls on one stream are ordered; concurrent calls that share a schedule or
 *    workspace on different streams race.
 */
#ifndef IDX_H
#define IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    IDX_OK = 0,
    IDX_EINVAL = -1,         /* a null pointer, a negative size, an inconsistent shape */
    IDX_EUNSUPPORTED = -2,   /* a configuration the kernels are not built for */
    IDX_EWORKSPACE = -3,     /* a schedule or workspace buffer that is too small */
    IDX_EHIP = -4            /* a HIP launch or runtime error */
} idx_status;

/* Query formats.  MXFP4: e2m1 values packed two per byte (element 2i in the low
 * nibble) with one UE8M0 scale byte per 32 elements.  FP8: OCP e4m3fn codes with
 * one fp32 scale per row applied to every dot product before the ReLU (the pages
 * name the fp8 x fp4 kernel variant on the backend source page). */
enum { IDX_Q_MXFP4 = 0, IDX_Q_FP8_E4M3_ROWSCALE = 1 };

/* Scoring formats.  FP32: fp32 head weights and fp32 logits, the gfx950 layer's
 * (rocm_paged_mxfp4_indexer page, RocmSparseMQAIndexer.weights_dtype: the head reduce
 * costs the same in either dtype there, so weights and logits stay fp32).  BF16: the
 * SM100 layer's semantics (sparse_mqa_indexer page, SparseMQAIndexer.weights_dtype =
 * bfloat16; backend source page, DeepseekV41SparseIndexerMetadataBuilder.__init__: the
 * top-k runs on the kernels' bf16 logits with no fp32 fallback): bf16 head weights
 * (codes, widened exactly) and every logit rounded to the nearest bf16 (ties to even)
 * before the selection, whose rule is unchanged (ties toward the lower token).  Use it
 * where indices must match that path; with 8 significant bits ties are common. */
enum { IDX_SCORE_FP32 = 0, IDX_SCORE_BF16 = 1 };

/* Per-model configuration, checked once (the backend builder's engine-start
 * checks on the sparse indexer backend page).  Host struct. */
typedef struct {
    int32_t num_heads;             /* H; the kernels are built for 64 */
    int32_t head_dim;              /* D; the kernels are built for 128 */
    int32_t q_format;              /* IDX_Q_* */
    int32_t page_size;             /* tokens per cache page; a multiple of sparse_block_kv */
    int32_t candidate_block_size;  /* cbs: tokens per candidate block, > 0 */
    int32_t sparse_block_kv;       /* sbk: tokens per sparse block; 0 = choose (filled in) */
    int32_t num_candidate_blocks;  /* NB: candidate ids per row, > 0 */
    int32_t topk;                  /* 1 <= topk <= NB * cbs, and <= IDX_MAX_TOPK */
    int32_t score_format;          /* IDX_SCORE_* */
} idx_config;

/* Kernel limits (sizes of the on-chip top-k working set). */
#define IDX_MAX_ROW_COLS 8192      /* NB * cbs for the sparse path */
#define IDX_MAX_DENSE_COLS 65536   /* max_ctx for the dense comparator */
#define IDX_MAX_TOPK 8192

/* Paged MXFP4 K cache of one layer.  A page holds page_size tokens; token slot j
 * of page p has D/2 bytes of packed e2m1 values at values + p*values_page_stride
 * + j*(D/2) and D/32 UE8M0 scale bytes at scales + p*scales_page_stride +
 * j*(D/32), scale byte i covering elements [32i, 32i+32).  Logical page n of
 * table row b is block_table[b*block_table_stride + n].  (The pages state only
 * that the model writes the cache in the order the gfx950 kernel reads it; this
 * two-pointer form covers both an interleaved and a split pool.) */
typedef struct {
    const uint8_t *values;
    int64_t values_page_stride;    /* bytes between consecutive pages */
    const uint8_t *scales;
    int64_t scales_page_stride;    /* bytes between consecutive pages */
    int64_t num_pages;             /* pages in the pool */
    const int32_t *block_table;    /* int32 [num_tables][block_table_stride] */
    int64_t block_table_stride;    /* int32 elements between table rows */
    int32_t num_tables;
    int32_t pages_per_table;       /* logical pages readable per table row */
} idx_kcache;

/* The rows of one call (SparseMQARowsMetadata on the backend page): decode rows
 * (ks = 0, ke = the compressed context length, one table row each) or one prefill
 * chunk (per-row [ks, ke), all rows on the request's table row).
 * rows_per_request: how many consecutive rows belong to one request and share its
 * table row, as the next_n query rows of a request do in SparseMQAIndexer.forward
 * (sparse_mqa_indexer page: q of shape [batch, next_n, H, D]; MTP / speculative
 * rows); 0 or 1: independent rows.  A placement hint, nothing more: with a value
 * above 1 the decode scoring kernels run each aligned group of 8 consecutive rows on
 * one XCD, so the K blocks those rows share cross the fabric once (through that XCD's
 * L2).  Results never depend on it; negative values are IDX_EINVAL. */
typedef struct {
    int32_t num_rows;              /* >= 0; 0 launches nothing */
    const int32_t *row_ks;         /* [num_rows] K-range start, or NULL for all 0 */
    const int32_t *row_ke;         /* [num_rows] exclusive K-range end */
    const int32_t *row_table;      /* [num_rows] row -> table row, or NULL for row r -> r */
    int32_t rows_per_request;      /* >= 0; placement hint (above) */
} idx_rows;

/* The shared sparse-column schedule of one step (built by idx_expand_candidates,
 * read by every consuming layer of the step; the backend page's per-row
 * sparse_indices / end scratch that the first consumer fills and later ones
 * reuse).  Caller-owned device memory. */
typedef struct {
    int32_t *sparse_indices;       /* [num_rows][NSB] ascending sparse block ids, then -1 */
    int32_t *end;                  /* [num_rows] valid token count |T| */
    void *work;                    /* idx_schedule_work_bytes() bytes, opaque */
    size_t work_bytes;
} idx_schedule;

/* Validate a configuration once, before any step, and fill in sparse_block_kv when it
 * is 0: 64 if cbs % 64 == 0, else cbs when cbs is 16 or 32.  Restates the engine-start
 * checks of DeepseekV41SparseIndexerMetadataBuilder.__init__ (DeepSeek-V4.1 sparse
 * indexer backend source page): a two-level model needs candidate_block_size > 0 and
 * candidate_topk_blocks > 0, the page size must be a multiple of the sparse block size
 * that pick_sparse_block_kv chooses (its body is not shown; the rule above is this
 * library's reading), and the top-k must fit the sparse columns
 * (check_deep_select_layout, body not shown either: 1 <= topk <= NB*cbs here, with the
 * kernels' limits IDX_MAX_ROW_COLS and IDX_MAX_TOPK).  Like the builder, which raises at
 * engine start instead of falling back per step, an unsupported configuration is an
 * error (IDX_EUNSUPPORTED / IDX_EINVAL), never a slower path.  cfg: host struct, read,
 * and sparse_block_kv written on success.  Host only. */
int idx_check_config(idx_config *cfg);

/* NSB = NB * (cbs / sbk) sparse blocks a row: the builder's num_sparse_blocks
 * (candidate_topk_blocks * (candidate_block_size // sparse_block_kv), backend source
 * page), which sizes the per-row sparse_indices.  Returns NSB, or a negative
 * idx_status for a bad config.  Host. */
int32_t idx_num_sparse_blocks(const idx_config *cfg);

/* Bytes of idx_schedule.work for up to max_rows rows.  The builder owns the per-row
 * scratch of the sparse schedule (sparse_indices, end and the column buffers, sized by
 * its maximum row count at construction, backend source page) so that the layer op
 * allocates nothing per step; here the caller allocates it once from this size.  Host;
 * 0 on a bad config or max_rows < 0. */
size_t idx_schedule_work_bytes(const idx_config *cfg, int32_t max_rows);

/* Bytes of scratch for up to max_rows rows: the sparse path needs
 * max_rows * NB * cbs fp32 logits; the dense comparator max_rows * max_ctx
 * (pass max_ctx = 0 when it is not used).  The pages size the logits scratch the same
 * way, rows x candidate columns for the sparse kernels (the builder's prefill budget) and
 * rows x context for the dense indexer (its profiling-run reservation on the
 * sparse_mqa_indexer page); the caller allocates it once.  Host; 0 on a bad config. */
size_t idx_workspace_bytes(const idx_config *cfg, int32_t max_rows, int32_t max_ctx);

/* Message of the last failing call on this thread ("" if none): the text the pages'
 * builder puts in its ValueError / NotImplementedError (engine start) and the layer
 * its per-step asserts, as a C status (the return value) plus this message.  The
 * string is thread-local and owned by the library; it stays valid until the thread's
 * next call.  Host. */
const char *idx_last_error(void);

/* Launch plan of a sparse call: which kernels idx_sparse_mqa_logits_topk (num_layers = 1)
 * or idx_sparse_mqa_logits_topk_layers launches for these sizes on the calling thread's
 * current device (the choice depends on its CU count).  Not a step of the method (the
 * pages fix what is computed, not how it is launched); it lets a caller that accounts
 * for a call's kernels, such as a benchmark, read the choice the launch makes. */
enum {
    IDX_PLAN_NONE = 0,             /* no rows or no layers: nothing launched */
    IDX_PLAN_SPLIT = 1,            /* per layer: split scoring kernel, then a selection kernel */
    IDX_PLAN_ONE_ROW = 2,          /* per layer: one workgroup scores and selects a row */
    IDX_PLAN_ROW_GROUP = 3,        /* per layer: 2-row groups share K tiles, score and select */
    IDX_PLAN_SPLIT_LAYERS = 4,     /* all layers: one split scoring and one selection launch */
    IDX_PLAN_ONE_ROW_LAYERS = 5,   /* all layers in one launch of one-row workgroups */
    IDX_PLAN_ROW_GROUP_LAYERS = 6  /* all layers in one launch of row groups */
};
typedef struct {
    int32_t plan;                       /* IDX_PLAN_* */
    int32_t layers_per_scoring_launch;  /* layers one launch of the scoring kernel covers */
    int32_t selects_in_scoring_kernel;  /* 1: no logits leave the scoring kernel */
    const char *scoring_kernel;         /* the kernel that streams K (static string) */
    const char *selection_kernel;       /* the separate selection kernel, or "" */
    int32_t expansion_in_scoring_kernel; /* 1: idx_expand_and_score_layers expands each row
                                            inside its scoring kernel (no expansion launch) */
    const char *expand_and_score_kernel; /* the kernel that streams K in that call */
} idx_plan_info;

/* Fills *out for a call on num_rows rows and num_layers layers (1..IDX_MAX_LAYERS).
 * logits_home: nonzero when every layer's logits have a home for the batched split
 * launches (each layer's logits_out is set, or the workspace holds num_layers * num_rows *
 * NB*cbs floats); it matters only with fewer rows than CUs.  Returns IDX_OK or a
 * negative idx_status (bad config, negative rows, layers out of range, out NULL).  Host;
 * queries the current device's CU count once. */
int idx_sparse_plan(const idx_config *cfg, int32_t num_rows, int32_t num_layers,
                    int32_t logits_home, idx_plan_info *out);

/* Optional timing hook for benchmarks (not a step of the method: the pages publish no
 * timings).  While set, every idx_sparse_mqa_logits_topk,
 * idx_sparse_mqa_logits_topk_layers, idx_expand_and_score_layers,
 * idx_dense_masked_logits_topk and
 * idx_gather_k_workspace call made on this thread launches its scoring kernel (the one
 * that streams the K cache; for the gather, its one kernel) with start_event and
 * stop_event attached
 * to the dispatch (hipExtLaunchKernel): they take the kernel's own start and end
 * timestamps, so hipEventElapsedTime gives its duration without queueing gaps.  Both
 * are hipEvent_t handles owned by the caller; pass NULL, NULL to clear.  Host;
 * returns IDX_EINVAL if exactly one of them is NULL. */
int idx_set_timing_events(void *start_event, void *stop_event);

/* Step a1: candidate expansion.  For each row, drop negative ids, count repeated
 * ids once, sort ascending, split each candidate block into cbs/sbk sparse blocks,
 * keep those holding a token of [ks, ke), pad with -1; end = number of valid
 * tokens.  candidate_blocks is int32 [num_rows][cand_stride] (first NB used).
 * Runs once per step; the schedule then serves every consuming layer whose K
 * cache uses the same block table and pool size.  The pages: the first consuming layer
 * of a step builds the candidate expansion and schedule that all later ones reuse
 * (backend source page, module docstring and SparseMQARowsMetadata: sparse_indices
 * [rows, num_sparse_blocks] and end [rows]); each candidate block of cbs tokens splits
 * into cbs / sparse_block_kv sparse blocks (the builder's num_sparse_blocks).  k: its
 * block table resolves each listed sparse block's page once per step (stored in the
 * schedule's work buffer).  Errors: IDX_EINVAL / IDX_EWORKSPACE on the host before any
 * launch (null pointers, a cand_stride below NB, a work buffer too small). */
int idx_expand_candidates(const idx_config *cfg, const idx_rows *rows, const idx_kcache *k,
                          const int32_t *candidate_blocks, int64_t cand_stride,
                          const idx_schedule *sched, void *stream);

/* Steps a2-a6 (and a8 with the fp8 format): paged gather, MX-scaled MFMA,
 * ReLU + fp32 weighted head reduce, masking, per-row top-k.  The consuming layer's call
 * of SparseMQAIndexer.forward (sparse_mqa_indexer page), which fills the index buffer
 * with -1 and calls sparse_mqa_logits_paged_decode for the decode rows (one query per
 * row, row_ks = 0, row_ke = the compressed context length, a block-table row each) and
 * sparse_mqa_logits_prefill_chunk per prefill chunk (row_ks / row_ke = the chunk's
 * cu_seqlen_ks / cu_seqlen_ke); and of RocmSparseMQAIndexer.forward
 * (rocm_paged_mxfp4_indexer page), which scores the same candidate pool straight from the
 * paged MXFP4 cache with fp32 weights and fp32 logits.  One entry point serves both row
 * kinds (the backend page's SparseMQARowsMetadata covers both).
 *   q_values: MXFP4 u8 [num_rows][H][D/2]; FP8 u8 [num_rows][H][D]
 *   q_scales: MXFP4 u8 [num_rows][H][D/32]; FP8 float [num_rows] (s_r > 0)
 *   weights:  IDX_SCORE_FP32: float [num_rows][H], 4-byte aligned;
 *             IDX_SCORE_BF16: bf16 codes uint16 [num_rows][H], 8-byte aligned
 *   topk_indices: int32 rows of out_stride elements; slots [0, topk) written
 *   logits_out: NULL, or float [num_rows][NB*cbs]: the logit of sparse column c
 *     (token sparse_indices[c / sbk] * sbk + c % sbk), -inf where invalid
 *   workspace: idx_workspace_bytes(cfg, num_rows, 0) bytes unless logits_out
 *     is given (then it may be NULL).
 * Serves decode rows and a prefill chunk alike; the schedule must come from
 * idx_expand_candidates on the same rows. */
int idx_sparse_mqa_logits_topk(const idx_config *cfg, const idx_rows *rows, const void *q_values,
                               const void *q_scales, const void *weights, const idx_kcache *k,
                               const idx_schedule *sched, int32_t *topk_indices,
                               int64_t out_stride, float *logits_out, void *workspace,
                               size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): idx_sparse_mqa_logits_topk without
 * the workspace argument.  When the call needs a logits scratch (logits_out NULL and
 * fewer rows than the device's CUs, so rows are split over workgroups and a second
 * kernel selects: idx_sparse_plan's IDX_PLAN_SPLIT), the logits go to a static scratch
 * array of IDX_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; num_rows * NB * cbs * 4 bytes must fit in it (always true for the split
 * plan on a 256-CU MI355X: at most 255 rows of 8192 columns), else IDX_EWORKSPACE and
 * nothing is launched.  Every other argument, the results and the errors are those of
 * idx_sparse_mqa_logits_topk.  The call allocates nothing (no hipMalloc, no allocating
 * library routine); its first call on a device looks up that device's scratch address.
 * The scratch keeps the last call's contents, and every logit a call reads it has
 * written first.  Calls that overlap on one GPU (on different streams, or from several
 * threads at once) share that GPU's scratch and race: order them on one stream. */
#define IDX_NOALLOC_SCRATCH_BYTES (8u << 20)
int idx_sparse_mqa_logits_topk_noalloc(const idx_config *cfg, const idx_rows *rows,
                                       const void *q_values, const void *q_scales,
                                       const void *weights, const idx_kcache *k,
                                       const idx_schedule *sched, int32_t *topk_indices,
                                       int64_t out_stride, float *logits_out, void *stream);

/* Steps a2-a6 for several consuming layers of one step (the DeepSeek-V4.1 sparse
 * indexer backend source: the per-row schedule scratch that the first consuming
 * layer fills is reused by the later ones, each with its own K cache, query and
 * weights).  Same result, layer by layer, as
 * calling idx_sparse_mqa_logits_topk once per layer in layer order.  With two or
 * more layers whose row-layers take the one-row-per-workgroup kernel (num_rows *
 * num_layers >= the device's CUs, and not the prefill row-group case) all layers run in
 * one launch with two row-layers on a CU at a time, so one's selection overlaps
 * another's K stream.  With two or more layers and fewer row-layers than CUs, every
 * layer runs in one split scoring launch and one selection launch when each layer's
 * logits have a home:
 * its logits_out, or its slice of a workspace of idx_workspace_bytes(cfg, num_layers *
 * num_rows, 0) bytes (layer l at l * num_rows * NB*cbs floats); with a smaller
 * workspace the layers run one after another.  A prefill chunk's rows (the row-group
 * case) run every layer in one launch as well.  layers is a HOST array of num_layers
 * (1..IDX_MAX_LAYERS) entries.  Every layer's k must equal layers[0].k in every field
 * but values and scales (one page geometry and block table for the step, as the
 * schedule requires).  workspace: as for idx_sparse_mqa_logits_topk when some
 * layer's logits_out is NULL; it is reused layer after layer.  The timing events
 * (idx_set_timing_events), if set, time the one launch, or else the last layer's
 * scoring kernel. */
#define IDX_MAX_LAYERS 8
typedef struct {
    const void *q_values;          /* as in idx_sparse_mqa_logits_topk */
    const void *q_scales;
    const void *weights;
    idx_kcache k;                  /* this layer's pool */
    int32_t *topk_indices;         /* int32 rows of out_stride elements */
    float *logits_out;             /* NULL or float [num_rows][NB*cbs] */
} idx_layer;

int idx_sparse_mqa_logits_topk_layers(const idx_config *cfg, const idx_rows *rows,
                                      const idx_schedule *sched, int32_t num_layers,
                                      const idx_layer *layers, int64_t out_stride,
                                      void *workspace, size_t workspace_bytes, void *stream);

/* Step a1 and steps a2-a6 for the consuming layers of one step in one call: the same
 * results (every layer's topk_indices and logits_out) and the same schedule in sched as
 * idx_expand_candidates(cfg, rows, &layers[0].k, candidate_blocks, cand_stride, sched)
 * followed by idx_sparse_mqa_logits_topk_layers(cfg, rows, sched, num_layers, layers,
 * ...), so a later call of the step can still reuse the schedule (the backend source
 * page: the step's first consuming layer builds the expansion and schedule that later
 * ones reuse).  With NB <= 128 the expansion runs inside the scoring launch: each
 * scoring workgroup expands its row in LDS and one workgroup a row writes the schedule,
 * so there is no expansion launch and no schedule round trip through memory before the K
 * stream starts.  That holds where the rows take the one-row-per-workgroup kernel
 * (num_rows >= the device's CUs, or num_rows * num_layers >= CUs with two or more layers;
 * not the prefill row-group case) in one round (num_rows * num_layers <= 2 x CUs; fp8
 * queries: fewer than 2 x CUs) with sparse_block_kv 64, and where they take the split
 * scoring launch (fewer rows, or row-layers, than CUs: one layer, or every layer in one
 * launch pair; fp8 queries with sparse_block_kv 64 only) when all its workgroups (rows x
 * layers x one per 512 columns) are resident at once (MXFP4: 6 x CUs, fp8: 3 x CUs).
 * idx_sparse_plan's expansion_in_scoring_kernel says which.  Otherwise the two calls'
 * launches.  Arguments and errors: those of the two calls (candidate_blocks
 * and cand_stride as in idx_expand_candidates; the workspace rule as in
 * idx_sparse_mqa_logits_topk_layers, also when the one launch needs none).  The timing
 * events time the scoring launch as in idx_sparse_mqa_logits_topk_layers. */
int idx_expand_and_score_layers(const idx_config *cfg, const idx_rows *rows,
                                const int32_t *candidate_blocks, int64_t cand_stride,
                                const idx_schedule *sched, int32_t num_layers,
                                const idx_layer *layers, int64_t out_stride, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Step a9, the comparator the sparse path replaces (the dense indexer scores the
 * whole context and masks to the candidates: module summary of the
 * sparse_mqa_indexer page): scores every token of [ks, ke) with the same
 * per-column arithmetic as the sparse path, keeps the tokens whose sparse block is
 * in the schedule, and selects the top-k with the same rule, so both return
 * identical indices.  Needs the block table to map every page of [0, ke).
 *   logits_out: NULL or float [num_rows][logits_stride] (token t at column t,
 *     -inf outside [ks, ke)); workspace: idx_workspace_bytes(cfg, rows, max_ctx)
 *     bytes when logits_out is NULL.  max_ctx bounds every ke. */
int idx_dense_masked_logits_topk(const idx_config *cfg, const idx_rows *rows, int32_t max_ctx,
                                 const void *q_values, const void *q_scales,
                                 const void *weights, const idx_kcache *k,
                                 const idx_schedule *sched, int32_t *topk_indices,
                                 int64_t out_stride, float *logits_out, int64_t logits_stride,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* The candidate-source layer: publishes the candidate pool that the consuming layers read
 * (rocm_paged_mxfp4_indexer page: RocmSparseAttnIndexer, a two-level indexer's source
 * layer, hands candidate_blocks and candidate_write to the dense indexer's HIP path;
 * sparse_mqa_indexer page, module summary: the candidate-source indexer publishes the top
 * candidate blocks and later indexers pick their top-k tokens inside them).  The pages
 * give no pooling rule; this library's reading: every token t of a row's [ks, ke) is
 * scored with the same per-token logit as the consuming path (and the dense comparator),
 * a block b of cbs = candidate_block_size tokens scores the largest logit among its tokens
 * in [ks, ke) (blocks holding none are not eligible), and the row publishes the NB =
 * num_candidate_blocks eligible blocks with the largest scores, ties toward the lower
 * block id, in ascending block order, then -1 (fewer eligible blocks than NB).  The result
 * is the consuming layers' candidate_blocks input (idx_expand_candidates).
 *   candidate_blocks: int32 [num_rows][cand_stride], the first NB slots written
 *   max_ctx: bounds every ke (like the dense comparator); ceil(max_ctx / cbs) <= 4096
 *   logits_out: NULL, or float [num_rows][logits_stride] (logits_stride >=
 *     round_up(max_ctx, 64)): token t at column t, -inf outside [ks, ke)
 *   workspace: idx_publish_workspace_bytes(cfg, num_rows, max_ctx) bytes (per-part
 *     maxima of the scoring pass), 4-byte aligned
 * Needs the block table to map every page of [0, ke).  Two launches (scoring with the
 * block maxima reduced in the same pass, then the block selection); the timing events, if
 * set, ride on the scoring launch.  Errors as for the other calls, on the host before any
 * launch. */
size_t idx_publish_workspace_bytes(const idx_config *cfg, int32_t max_rows, int32_t max_ctx);
int idx_publish_candidates(const idx_config *cfg, const idx_rows *rows, int32_t max_ctx,
                           const void *q_values, const void *q_scales, const void *weights,
                           const idx_kcache *k, int32_t *candidate_blocks, int64_t cand_stride,
                           float *logits_out, int64_t logits_stride, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Packed K workspace (the gather of a prefill chunk's paged K into one contiguous
 * buffer that the pages' backend performs before scoring a chunk, the
 * cp_gather_indexer_k_quant_cache call on the sparse_mqa_indexer page): request r's
 * positions p in [0, cu_seq_lens[r+1] - cu_seq_lens[r]) are copied from the paged
 * cache (table row req_table[r], or r when req_table is NULL) to workspace row
 * cu_seq_lens[r] + p:
 *   values_out: u8 [max_tokens][D/2] (16-byte aligned), the row's packed e2m1 values;
 *   scales_out: u8 [max_tokens][D/32] (4-byte aligned), its UE8M0 scale bytes (one
 *     int32 a row when D = 128).
 * cu_seq_lens: int32 [num_reqs + 1] device array, non-decreasing from >= 0.  Rows at
 * or past max_tokens, and positions at or past max_seq_len (host; bounds every
 * request's length), are not written; a position whose table row, logical page or
 * page id is out of range is written as zeros.  k's scales base and page stride must be
 * 4-byte aligned.  The workspace then serves idx_expand_candidates and the scoring calls
 * as a one-page cache (page_size >= the chunk's rows, values/scales page strides
 * max_tokens * D/2 and max_tokens * D/32, a one-entry block table), in workspace
 * coordinates.  The timing events, if set, ride on the gather launch. */
int idx_gather_k_workspace(const idx_config *cfg, const idx_kcache *k, int32_t num_reqs,
                           const int32_t *cu_seq_lens, const int32_t *req_table,
                           int32_t max_seq_len, int32_t max_tokens, uint8_t *values_out,
                           uint8_t *scales_out, void *stream);

/* ---- Measurement (not a step of the indexer) ----
 * Reference kernels for the two rates that bound the indexer, for a benchmark to time
 * with events on `stream` next to the indexer's own kernels: the measured read
 * bandwidth (the K gather streams pages of the cache) and the measured MX-FP4 MFMA
 * rate (the scoring contraction), beside the published peaks.  Both launch
 * IDX_MEASURE_WGS workgroups of 256 threads and return IDX_EINVAL (launching nothing)
 * on a bad argument.
 *
 * idx_measure_read: reads every 16-byte word of [src, src + bytes) once (device
 *   memory; src 16-byte aligned, bytes a nonzero multiple of 16) and writes one
 *   checksum word per workgroup to sink (device, IDX_MEASURE_WGS uint32).
 * idx_measure_mfma: every wave runs `iters` (>= 1) rounds of 8 independent
 *   v_mfma_scale_f32_16x16x128_f8f6f4 on e2m1 operands held in registers and writes
 *   one float per wave to sink (device, IDX_MEASURE_WGS * 4 floats);
 *   idx_measure_mfma_flops(iters) is the number of floating-point operations one
 *   call performs (host).
 * idx_measure_mfma_relu: the same MFMA count as idx_measure_mfma, each product fresh
 *   and folded through the ReLU-weight epilogue of the indexer score (an integer max
 *   and an fp32 FMA per accumulator, 9 VALU operations per MFMA); it measures the MFMA
 *   rate left once the vector ALUs issue that epilogue on the same SIMDs, the ceiling
 *   of a scoring loop whose K tiles come from cache.  Same sink and flop count as
 *   idx_measure_mfma. */
#define IDX_MEASURE_WGS 4096
int idx_measure_read(const void *src, size_t bytes, uint32_t *sink, void *stream);
/* idx_measure_fp8_dot: the two ways to form the fp8-query dot products, for the record
 *   of why the fp8 path converts to bf16 (an accuracy check, not a rate): 16 query rows
 *   of e4m3 codes (q_e4m3 u8 [16][128], device) against 16 tokens of e2m1 codes with UE8M0
 *   block scales (k_e2m1 u8 [16][64] packed, k_scales u8 [16][4], device) -> out fp32
 *   [16 rows][16 tokens] (device).  mode 0: the MX-scaled fp8 x fp4 MFMA on the codes;
 *   mode 1: both operands converted exactly to bf16 and the bf16 MFMA, as the fp8-query
 *   scoring kernels do; mode 2: the MX-scaled fp8 x fp8 MFMA with K's e2m1 values
 *   converted exactly to e4m3.  One wave; IDX_EINVAL on a bad argument. */
int idx_measure_fp8_dot(const uint8_t *q_e4m3, const uint8_t *k_e2m1, const uint8_t *k_scales,
                        int32_t mode, float *out, void *stream);
int idx_measure_mfma(int32_t iters, float *sink, void *stream);
int idx_measure_mfma_relu(int32_t iters, float *sink, void *stream);
int64_t idx_measure_mfma_flops(int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* IDX_H */
