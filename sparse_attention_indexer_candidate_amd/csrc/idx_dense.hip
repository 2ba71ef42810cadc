// Scoring of every token of a row's range:
//
//  score_dense_kernel + topk_split_kernel<dense>
//                       the comparator: every token of [ks, ke) with the same
//                       per-tile code, then the candidates' keys gathered from the
//                       dense row in schedule order and the same selection
//  score_pool_kernel + pool_select_kernel
//                       the candidate-source layer: block maxima of the same logits,
//                       then the published top blocks

#include "idx_device.h"

namespace idx {
namespace {

// Dense scoring (the comparator): column t is token t, every token < max_ctx.  G64: pages
// hold a multiple of 64 tokens.
template <int QF, bool G64>
__global__ __launch_bounds__(kScoreThreads) void score_dense_kernel(
    Rows rows, int32_t max_ctx, const void *qv, const void *qs, const void *weights, KCache k,
    float *logits, int64_t lstride, int groups_per_wg, int32_t sf) {
    const int row = blockIdx.x;
    const int wave = uniform(threadIdx.x / kWave);
    const int ngroups = (max_ctx + 63) / 64;
    constexpr int PW = 4;  // groups per wave (groups_per_wg = 16)
    const int g0 = min(blockIdx.y * groups_per_wg + wave * PW, ngroups);
    const int g1 = min(g0 + PW, ngroups);
    const int ks = rows.ks ? rows.ks[row] : 0;
    const int ke = min(rows.ke[row], max_ctx);
    const int tbl = rows.table ? rows.table[row] : row;
    const bool tbl_ok = tbl >= 0 && tbl < k.num_tables;
    const int32_t *bt = k.block_table + (int64_t)(tbl_ok ? tbl : 0) * k.block_table_stride;
    float *lrow = logits + (int64_t)row * lstride;
    QFrag<QF> f;
    if (g0 * 64 < ke && g1 * 64 > ks && tbl_ok)
        load_q<QF>(f, qv, qs, weights, sf, row, threadIdx.x & (kWave - 1));
    score_groups<QF, 4, 2, G64>(k, f, ks, ke, g0, g1, sf,
                                DenseDesc{bt, ks, tbl_ok ? ke : 0, k.page_size, k.pages_per_table},
                                [&](int t, float v, bool ok) {    // t < ngroups*64 <= lstride
                                    lrow[t] = ok ? v : -INFINITY;
                                });
}

// ------------------------------------------------------- candidate source -------
//
// The candidate-source layer's publication (the pool a two-level indexer's source layer
// writes for the consuming layers): every token of a row's [ks, ke) is scored as the
// dense comparator scores it; block b (cbs tokens) scores the largest logit among its
// tokens in range; the row's NB best blocks (ties toward the lower id) are published,
// ascending, then -1.  Two kernels: the scoring kernel reduces each part of p = min(cbs,
// 64) consecutive tokens to one key (the order-preserving key of its largest logit, 0 when
// it holds no token in range) in the same pass, so no logit needs to leave it; the
// selection kernel combines a block's cbs/p parts and selects the blocks.

// Scoring with part keys: as score_dense_kernel (same per-column arithmetic), the logits
// optional (logits may be null), parts [rows][pstride] (pstride = ngroups * 64 / p) with
// p = 1 << lp (16, 32 or 64).
template <int QF, bool G64>
__global__ __launch_bounds__(kScoreThreads) void score_pool_kernel(
    Rows rows, int32_t max_ctx, const void *qv, const void *qs, const void *weights, KCache k,
    float *logits, int64_t lstride, uint32_t *parts, int64_t pstride, int32_t lp,
    int groups_per_wg, int32_t sf) {
    const int row = blockIdx.x;
    const int wave = uniform(threadIdx.x / kWave);
    const int lane = threadIdx.x & (kWave - 1);
    const int ngroups = (max_ctx + 63) / 64;
    constexpr int PW = 4;  // groups per wave (groups_per_wg = 16)
    const int g0 = min(blockIdx.y * groups_per_wg + wave * PW, ngroups);
    const int g1 = min(g0 + PW, ngroups);
    const int ks = rows.ks ? rows.ks[row] : 0;
    const int ke = min(rows.ke[row], max_ctx);
    const int tbl = rows.table ? rows.table[row] : row;
    const bool tbl_ok = tbl >= 0 && tbl < k.num_tables;
    const int32_t *bt = k.block_table + (int64_t)(tbl_ok ? tbl : 0) * k.block_table_stride;
    float *lrow = logits ? logits + (int64_t)row * lstride : nullptr;
    uint32_t *prow = parts + (int64_t)row * pstride;
    const int p = 1 << lp;
    QFrag<QF> f;
    if (g0 * 64 < ke && g1 * 64 > ks && tbl_ok)
        load_q<QF>(f, qv, qs, weights, sf, row, lane);
    score_groups<QF, 4, 2, G64>(k, f, ks, ke, g0, g1, sf,
                           DenseDesc{bt, ks, tbl_ok ? ke : 0, k.page_size, k.pages_per_table},
                           [&](int t, float v, bool ok) {   // t < ngroups*64 <= lstride
                               if (lrow) lrow[t] = ok ? v : -INFINITY;
                               uint32_t key = ok ? bits_key(__float_as_uint(v)) : 0u;
#pragma unroll
                               for (int j = 1; j < kWave; j <<= 1)
                                   if (j < p) key = max(key, (uint32_t)lane_xor((int)key, j));
                               if ((lane & (p - 1)) == 0) prow[t >> lp] = key;
                           });
}

// Selection of the published blocks, one workgroup a row: thread i owns blocks
// [i*KPT, (i+1)*KPT) of the row's ceil(ke / cbs) blocks, each block's key the largest of
// its q = cbs / p part keys (0: no token of the block in range, the block is not
// eligible); the NB largest keys win, ties toward the lower block.
struct PoolLds {
    alignas(16) int32_t stage[kMaxNB];
    SelectLds<kTopkThreads> sel;
};

template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void pool_select_kernel(
    const uint32_t *parts, int64_t pstride, const int32_t *p_ks, const int32_t *p_ke,
    int32_t max_ctx, int32_t cbs, int32_t lp, int32_t nb, int32_t *cand, int64_t cand_stride) {
    __shared__ PoolLds L;
    const int row = blockIdx.x, tid = threadIdx.x;
    const int ke = max(0, min(p_ke[row], max_ctx));
    const int nblk = (ke + cbs - 1) / cbs;
    const int q = cbs >> lp;
    const uint32_t *prow = parts + (int64_t)row * pstride;
    (void)p_ks;   // blocks below ks hold no token in range: their part keys are 0
    select_clear(L.sel);
    uint32_t key[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int b = tid * KPT + i;
        uint32_t m = 0u;
        if (b < nblk)
            for (int j = 0; j < q; ++j) {
                const int64_t pi = (int64_t)b * q + j;
                m = max(m, pi < pstride ? prow[pi] : 0u);
            }
        key[i] = m;
    }
    int count;
    uint32_t kmin, kmax;
    block_key_stats<kTopkThreads>(key, keys_live(key), L.sel, count, kmin, kmax);
    select_topk<kTopkThreads, KPT>(key, keys_live(key), count, kmin, kmax, nb,
                                   cand + (int64_t)row * cand_stride, L.sel, L.stage,
                                   [&](int c0, int (&tok)[KPT]) {
#pragma unroll
                                       for (int i = 0; i < KPT; ++i) tok[i] = c0 + i;
                                   });
}

}  // namespace

hipError_t launch_score_dense(int q_format, int score_format, const Rows &rows, int32_t max_ctx,
                              const void *q_values, const void *q_scales, const void *weights,
                              const KCache &k, float *logits, int64_t logits_stride,
                              const Timing &timing, hipStream_t stream) {
    if (rows.num_rows == 0) return hipSuccess;
    const int ngroups = (max_ctx + 63) / 64;
    const int gpw = 16;
    const dim3 grid(rows.num_rows, (ngroups + gpw - 1) / gpw);
#define IDX_LAUNCH_DENSE(QF_, G64_)                                                                \
    hipExtLaunchKernelGGL((score_dense_kernel<QF_, G64_>), grid, dim3(kScoreThreads), 0, stream,   \
                          timing.start, timing.stop, 0, rows, max_ctx, q_values, q_scales,         \
                          weights, k, logits, logits_stride, gpw, score_format)
    const bool g64 = k.page_size % 64 == 0;
    if (q_format == 0) {
        if (g64) IDX_LAUNCH_DENSE(0, true);
        else IDX_LAUNCH_DENSE(0, false);
    } else {
        if (g64) IDX_LAUNCH_DENSE(1, true);
        else IDX_LAUNCH_DENSE(1, false);
    }
#undef IDX_LAUNCH_DENSE
    return hipGetLastError();
}

hipError_t launch_publish(int q_format, int score_format, const Rows &rows, int32_t max_ctx,
                          const void *q_values, const void *q_scales, const void *weights,
                          const KCache &k, int32_t cbs, int32_t nb, int32_t *cand,
                          int64_t cand_stride, float *logits, int64_t logits_stride,
                          uint32_t *parts, const Timing &timing, hipStream_t stream) {
    if (rows.num_rows == 0) return hipSuccess;
    const int ngroups = (max_ctx + 63) / 64;
    const int lp = cbs >= 64 ? 6 : cbs == 32 ? 5 : 4;
    const int64_t pstride = publish_parts_per_row(max_ctx, cbs);
    const int gpw = 16;
    const dim3 grid(rows.num_rows, (ngroups + gpw - 1) / gpw);
#define IDX_LAUNCH_POOL(QF_, G64_)                                                                 \
    hipExtLaunchKernelGGL((score_pool_kernel<QF_, G64_>), grid, dim3(kScoreThreads), 0, stream,    \
                          timing.start, timing.stop, 0, rows, max_ctx, q_values, q_scales,         \
                          weights, k, logits, logits_stride, parts, pstride, lp, gpw, score_format)
    const bool g64 = k.page_size % 64 == 0;
    if (q_format == 0) {
        if (g64) IDX_LAUNCH_POOL(0, true);
        else IDX_LAUNCH_POOL(0, false);
    } else {
        if (g64) IDX_LAUNCH_POOL(1, true);
        else IDX_LAUNCH_POOL(1, false);
    }
#undef IDX_LAUNCH_POOL
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    static_assert(8 * kTopkThreads == kMaxPublishBlocks, "one thread's 8 blocks in registers");
    hipLaunchKernelGGL(pool_select_kernel<8>, dim3(rows.num_rows), dim3(kTopkThreads), 0, stream,
                       parts, pstride, rows.ks, rows.ke, max_ctx, cbs, lp, nb, cand, cand_stride);
    return hipGetLastError();
}

hipError_t launch_dense_topk(const Rows &rows, const KCache &k, const Schedule &s,
                             const float *logits, int64_t logits_stride, int32_t ncols,
                             int32_t topk, int32_t *out, int64_t out_stride, hipStream_t stream) {
    if (rows.num_rows == 0) return hipSuccess;
    const int nsbcols = s.nsb * s.sbk;   // candidate columns a row
    if (nsbcols <= 8 * kTopkThreads)
        hipLaunchKernelGGL((topk_split_kernel<true, 8>), dim3(rows.num_rows), dim3(kTopkThreads), 0,
                           stream, logits, s.sparse_indices, rows.ks, rows.ke, s.kept, s.nsb, s.lsbk,
                           logits_stride, ncols, topk, out, out_stride);
    else
        hipLaunchKernelGGL((topk_split_kernel<true, 16>), dim3(rows.num_rows), dim3(kTopkThreads), 0,
                           stream, logits, s.sparse_indices, rows.ks, rows.ke, s.kept, s.nsb, s.lsbk,
                           logits_stride, ncols, topk, out, out_stride);
    return hipGetLastError();
}

}  // namespace idx
