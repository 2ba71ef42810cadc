// Sparse scoring and selection over the step's schedule, and the choice among the
// launch shapes (plan_sparse):
//
//  fused_row_kernel     rows >= CUs: one workgroup scores a whole row into LDS
//                       and selects from LDS (no global round trip, no cross-workgroup
//                       sync); with >= 2 rows a CU two rows share a CU (MXFP4: 8-wave
//                       rows, fp8: 4-wave rows)
//  fused_layers_kernel  the one-row kernel for several layers sharing a schedule, one
//                       launch (grid.y = layer); two row-layers a CU, so one row's
//                       selection overlaps another's K stream
//  score_split_kernel + topk_split_kernel
//                       fewer rows than CUs: rows split over workgroups, logits in
//                       global scratch, selection in a second launch (and the
//                       multi-layer pair, grid.z / grid.y = layer)
//  row groups           >= 8 rows a CU with MXFP4 queries: idx_row_groups.hip
//
// and, for the call that also expands the candidates (launch_expand_sparse_layers), the
// same scoring with each row's expansion inside: expand_fused_row_kernel,
// expand_fused_layers_kernel, score_split_expand_kernel, score_split_expand_layers_kernel.

#include "idx_device.h"

namespace idx {
namespace {

// Rows of one request (speculative / MTP rows: consecutive rows on one table row) read
// mostly the same K blocks.  Workgroups go to the 8 XCDs round-robin by linear id, and
// each XCD has its own L2, so when the caller declares such rows (rows_per_request > 1)
// blockIdx.x is mapped to rows such that the 8 consecutive rows of every aligned group
// of 8 run on one XCD (their blockIdx.x values lie 8 apart, so they are also dispatched
// close together) and a block that several of them read crosses the fabric once.
// group_rows: the row count with that placement, 0 for none (identity); rows past the
// last whole 64-row block keep their index.  Measured on 64 requests of two decode rows
// (split kernels): 18.2-18.5 vs 19.2-19.9 us a step, the scoring kernel's fetches down
// from 35.6 MB to the 22.5 MB of distinct blocks; on 256 requests of two rows and 128 of
// four (one-row kernel): 33.6-35.4 vs 37.3-38.3 and 32.3-33.0 vs 38.7-39.4 us.  Rows that
// share nothing lose ~2 % with it in the one-row kernel, hence the hint.  (A
// one-dimensional grid with the same placement was ~3 us slower on every workload.)
__device__ __forceinline__ int xcd_grouped_row(int x, int group_rows) {
    const int full = group_rows & ~63;
    return x < full ? (x & ~63) + 8 * (x & 7) + ((x >> 3) & 7) : x;
}

// Rows split over workgroups: grid = (rows, chunks of groups_per_wg 64-column groups);
// each wave scores a contiguous quarter of its workgroup's groups into logits.  The
// leading scalar arguments are what the first loads need (the row's schedule entries
// and query, and the row count that places the row): the hardware preloads them into
// SGPRs at wave launch, so those loads issue at once; ks / ke (only the validity of the
// scored columns needs them) and the cache geometry arrive while they fly.
template <int QF, int PW, bool G64>
__device__ __forceinline__ void score_split_row(
    const int32_t *si_base, const int32_t *pg_base, const void *qv, const void *qs,
    const void *weights, int32_t nsb, int32_t sbk, int32_t groups_per_wg, int32_t group_rows,
    const Rows &rows, const KCache &k, float *logits, int sf) {
    const int row = xcd_grouped_row(blockIdx.x, group_rows);
    const int wave = uniform(threadIdx.x / kWave);
    const int ncols = nsb * sbk;
    const int ngroups = (ncols + 63) / 64;
    const int g0 = min(blockIdx.y * groups_per_wg + wave * PW, ngroups);
    const int g1 = min(g0 + PW, ngroups);
    QFrag<QF> f;
    load_q<QF>(f, qv, qs, weights, sf, row, threadIdx.x & (kWave - 1));
    const int32_t *si = si_base + (int64_t)row * nsb, *pg = pg_base + (int64_t)row * nsb;
    const int32_t ks_raw = (rows.ks ? rows.ks : rows.ke)[row];   // no load behind a branch
    const int ks = rows.ks ? ks_raw : 0, ke = rows.ke[row];
    float *lrow = logits + (int64_t)row * ncols;
    score_groups<QF, PW, PW, G64>(k, f, ks, ke, g0, g1, sf, SparseDesc{si, pg, nsb, sbk},
                             [&](int c, float v, bool ok) {
                                 if (c < ncols) lrow[c] = ok ? v : -INFINITY;
                             });
}

// Split grid: 8 groups a workgroup, two a wave (two groups a wave hide the schedule-to-K
// load chain better than one: measured 3-7 % faster steps on 64- and 128-row decode
// batches).  The split plan takes fewer rows than CUs, so the grid (rows x up to 16
// chunks of a row's 128 groups) stays within a few thousand workgroups and covers the CUs
// several times over.
constexpr int kSplitGroupsPerWave = 2;
constexpr int kSplitGroupsPerWg = (kScoreThreads / kWave) * kSplitGroupsPerWave;

// fp8 queries: at most 168 VGPRs, so three workgroups share a CU (the compiler's own
// choice, 170, fits two: measured 5 % slower steps on 128-row decode batches and on rows
// in requests of two).
template <int QF>
constexpr int split_waves_per_simd() {
    return QF == 1 ? 3 : 1;
}

template <int QF, int PW, bool G64>
__global__ __launch_bounds__(kScoreThreads, (split_waves_per_simd<QF>())) void score_split_kernel(
    const int32_t *si_base, const int32_t *pg_base, const void *qv, const void *qs,
    const void *weights, int32_t nsb, int32_t sbk, int32_t groups_per_wg, int32_t group_rows,
    Rows rows, KCache k, float *logits, int32_t sf) {
    score_split_row<QF, PW, G64>(si_base, pg_base, qv, qs, weights, nsb, sbk, groups_per_wg,
                                 group_rows, rows, k, logits, sf);
}

// Logits of layer l of a multi-layer split launch: the layer's logits_out, else its slice
// of the workspace.
__device__ __forceinline__ float *layer_logits(const LayerSet &ls, int l, float *ws,
                                               int64_t ws_layer) {
    return ls.logits_out[l] ? ls.logits_out[l] : ws + (int64_t)l * ws_layer;
}

// Several layers sharing a schedule, fewer rows than CUs: grid.z = layer.
template <int QF, int PW, bool G64>
__global__ __launch_bounds__(kScoreThreads, (split_waves_per_simd<QF>())) void score_split_layers_kernel(
    const int32_t *si_base, const int32_t *pg_base, int32_t nsb, int32_t sbk,
    int32_t groups_per_wg, int32_t group_rows, Rows rows, KCache k, LayerSet ls, float *ws,
    int64_t ws_layer, int32_t sf) {
    const int l = blockIdx.z;
    KCache kl = k;
    kl.values = ls.k_values[l];
    kl.scales = ls.k_scales[l];
    score_split_row<QF, PW, G64>(si_base, pg_base, ls.q_values[l], ls.q_scales[l],
                                 ls.weights[l], nsb, sbk, groups_per_wg, group_rows, rows, kl,
                                 layer_logits(ls, l, ws, ws_layer), sf);
}

// A row's candidate expansion inside a scoring kernel: the published candidate blocks,
// and the schedule arrays that the workgroup writes when kept is set (one workgroup a
// row), so the schedule is the expansion launch's.
struct FusedExpand {
    const int32_t *cand;
    int64_t cand_stride;
    int32_t nb;
    int32_t cbs;
    int32_t *si;
    int32_t *pg;
    int32_t *end;
    int32_t *kept;   // null: this workgroup writes no schedule
};

// Candidate ids a lane of the expansions inside the scoring kernels: up to 128
// candidate blocks a row.
constexpr int kFusedExpandIds = 2;

struct SplitExpandLds {
    int32_t stage[kFusedExpandIds * kWave];
    int32_t si[kMaxNSB];
    int32_t pg[kMaxNSB];
};

// score_split_row with the row's expansion inside: wave 0 loads the row's metadata and
// candidate ids and lists its kept sparse blocks and pages in LDS while the other waves
// load the query; then the workgroup scores its chunk from the LDS schedule.  Every chunk
// of a row expands the row again (a candidate load, a sort in registers and a block-table
// load, all on-chip after the first); the workgroup with ex.kept set also writes the
// row's schedule, which the selection launch reads.
template <int QF, int PW, bool G64>
__device__ __forceinline__ void score_split_row_expand(
    SplitExpandLds &L, const FusedExpand &ex, const void *qv, const void *qs,
    const void *weights, int32_t nsb, int32_t sbk, int32_t groups_per_wg, int32_t group_rows,
    const Rows &rows, const KCache &k, float *logits, int sf) {
    const int row = xcd_grouped_row(blockIdx.x, group_rows);
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = uniform(tid / kWave);
    const int ncols = nsb * sbk;
    const int ngroups = (ncols + 63) / 64;
    const int g0 = min(blockIdx.y * groups_per_wg + wave * PW, ngroups);
    const int g1 = min(g0 + PW, ngroups);
    // the row's metadata and candidate ids, then the query: one round trip (a null ks or
    // table pointer reads ke's slot, then the value is replaced)
    const int32_t ks_raw = (rows.ks ? rows.ks : rows.ke)[row];
    const int32_t ke_raw = rows.ke[row];
    const int32_t tbl_raw = (rows.table ? rows.table : rows.ke)[row];
    int craw[kFusedExpandIds];
    if (wave == 0) {
#pragma unroll
        for (int e = 0; e < kFusedExpandIds; ++e) {
            const int i = e * kWave + lane;
            craw[e] = ex.cand[(int64_t)row * ex.cand_stride + min(i, ex.nb - 1)];
            if (i >= ex.nb) craw[e] = -1;
        }
    }
    // MXFP4 queries load while wave 0 expands; fp8 queries (bf16 fragments, held to 168
    // VGPRs) load after it, so their registers are not live across the sort (they still
    // fly with the first K loads)
    QFrag<QF> f;
    if constexpr (QF == 0) load_q<QF>(f, qv, qs, weights, sf, row, lane);
    const int ks = rows.ks ? ks_raw : 0, ke = ke_raw;
    if (wave == 0) {
        const int tbl = rows.table ? tbl_raw : row;
        int ntok;
        const int nlist = expand_row<kFusedExpandIds>(craw, ks, ke, tbl >= 0 && tbl < k.num_tables,
                                                      tbl, ex.cbs, sbk, nsb, k, L.stage, L.si,
                                                      L.pg, ntok);
        if (lane == 0 && ex.kept) {
            ex.end[row] = ntok;
            ex.kept[row] = nlist;
        }
    }
    __syncthreads();
    if constexpr (QF == 1) load_q<QF>(f, qv, qs, weights, sf, row, lane);
    if (ex.kept)
        for (int i = tid; i < nsb; i += kScoreThreads) {
            ex.si[(int64_t)row * nsb + i] = L.si[i];
            ex.pg[(int64_t)row * nsb + i] = L.pg[i];
        }
    float *lrow = logits + (int64_t)row * ncols;
    score_groups<QF, PW, PW, G64>(k, f, ks, ke, g0, g1, sf, SparseDesc{L.si, L.pg, nsb, sbk},
                             [&](int c, float v, bool ok) {
                                 if (c < ncols) lrow[c] = ok ? v : -INFINITY;
                             });
}

// The split scoring launches with the expansion inside (both query formats, fp8 held to
// the same 168 VGPRs as score_split_kernel); chunk 0 of each row (of layer 0) writes the
// schedule.  The leading scalar arguments are the candidate row's address terms (kernarg
// preload).
template <int QF, bool G64>
__global__ __launch_bounds__(kScoreThreads, (split_waves_per_simd<QF>())) void score_split_expand_kernel(
    const int32_t *cand, int64_t cand_stride, const void *qv, const void *qs,
    const void *weights, int32_t nb, int32_t cbs, int32_t nsb, int32_t sbk,
    int32_t groups_per_wg, int32_t group_rows, Rows rows, KCache k, Schedule s, float *logits,
    int32_t sf) {
    __shared__ SplitExpandLds lds;
    const FusedExpand ex = {cand, cand_stride, nb, cbs, s.sparse_indices, s.pages, s.end,
                            blockIdx.y == 0 ? s.kept : nullptr};
    score_split_row_expand<QF, kSplitGroupsPerWave, G64>(lds, ex, qv, qs, weights, nsb, sbk,
                                                         groups_per_wg, group_rows, rows, k,
                                                         logits, sf);
}

template <int QF, bool G64>
__global__ __launch_bounds__(kScoreThreads, (split_waves_per_simd<QF>())) void score_split_expand_layers_kernel(
    const int32_t *cand, int64_t cand_stride, int32_t nb, int32_t cbs, int32_t nsb,
    int32_t sbk, int32_t groups_per_wg, int32_t group_rows, Rows rows, KCache k, LayerSet ls,
    Schedule s, float *ws, int64_t ws_layer, int32_t sf) {
    __shared__ SplitExpandLds lds;
    const int l = blockIdx.z;
    KCache kl = k;
    kl.values = ls.k_values[l];
    kl.scales = ls.k_scales[l];
    const FusedExpand ex = {cand, cand_stride, nb, cbs, s.sparse_indices, s.pages, s.end,
                            blockIdx.y == 0 && l == 0 ? s.kept : nullptr};
    score_split_row_expand<QF, kSplitGroupsPerWave, G64>(
        lds, ex, ls.q_values[l], ls.q_scales[l], ls.weights[l], nsb, sbk, groups_per_wg,
        group_rows, rows, kl, layer_logits(ls, l, ws, ws_layer), sf);
}

// The selection of a multi-layer split launch: grid.y = layer.
template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void topk_split_layers_kernel(
    const int32_t *si_base, const int32_t *p_ks, const int32_t *p_ke, const int32_t *p_kept,
    int32_t nsb, int32_t lsbk, int32_t topk, LayerSet ls, float *ws, int64_t ws_layer,
    int64_t ostride) {
    __shared__ TopkLds lds;
    const int l = blockIdx.y;
    topk_split_row<false, KPT>(lds, layer_logits(ls, l, ws, ws_layer), si_base, p_ks, p_ke, p_kept,
                               nsb, lsbk, (int64_t)0, 0, topk, ls.out[l], ostride);
}

// Rows >= CUs: one workgroup per row; waves take units of the row's valid 64-column
// groups from a shared counter, logits stay in LDS, then the same workgroup selects.
// logits_out (optional) gets a copy of every column.  The table row is not checked
// here: the expansion lists nothing for a row whose table row is invalid (kept = 0),
// and the schedule comes from the expansion of the same rows.
template <int NT>
struct FusedLds {
    alignas(16) uint32_t word[kMaxRowCols];   // column words (bits_key), then the stage
    int32_t si[kMaxNSB];
    int32_t pg[kMaxNSB];
    int unit;
    int kept;                                 // the row's kept count when expanded here
    SelectLds<NT, 5> sel;
};

// U: 64-column groups a wave takes per unit (two units in flight).  E = 0: the row's
// schedule comes from the expansion launch (si_base, pg_base, p_kept); E > 0: wave 0
// expands the row's candidates (ex, E ids a lane, nb <= 64 E) into LDS while the other
// waves load the query, and si_base, pg_base and p_kept are not read.
template <int QF, int NT, int KPT, int U, bool G64, int E = 0>
__device__ __forceinline__ void fused_row(
    FusedLds<NT> &L, int row, const int32_t *si_base, const int32_t *pg_base, const void *qv,
    const void *qs, const void *weights, const int32_t *p_kept, int32_t nsb, int32_t lsbk,
    const Rows &rows, const KCache &k, float *logits_out, int32_t topk, int32_t *out,
    int64_t ostride, int sf, const FusedExpand &ex = {}) {
    uint32_t *s_word = L.word;
    int32_t *s_si = L.si;
    int32_t *s_pg = L.pg;
    int &s_unit = L.unit;
    SelectLds<NT, 5> &s_sel = L.sel;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int sbk = 1 << lsbk;
    RowInfo ri;
    ri.ncols = nsb * sbk;
    ri.tbl_ok = true;
    QFrag<QF> f;
    if constexpr (E == 0) {
        ri.si = si_base + (int64_t)row * nsb;
        ri.pg = pg_base + (int64_t)row * nsb;
        ri.kept = max(0, min(uniform(p_kept[row]), nsb));
        load_q<QF>(f, qv, qs, weights, sf, row, lane);   // overlaps the schedule copy
        // Every slot [0, nsb) is written by the expansion (-1 past the kept count), so
        // the copy is not bound by the kept load: the schedule, the kept count and the
        // query are one memory round trip, not two.
        for (int i = tid; i < nsb; i += NT) {
            s_si[i] = ri.si[i];
            s_pg[i] = ri.pg[i];
        }
        // ks / ke (their pointers are not preloaded) are needed only for the validity of
        // the scored columns; loaded after the first loads so no wait for them comes first
        const int vrow = row + opaque_zero();
        const int32_t ks_raw = (rows.ks ? rows.ks : rows.ke)[vrow];   // no load behind a branch
        ri.ks = rows.ks ? ks_raw : 0;
        ri.ke = rows.ke[vrow];
    } else {
        // the row's metadata and candidate ids, then the query: one round trip (a null
        // ks or table pointer reads ke's slot, then the value is replaced)
        const int vrow = row + opaque_zero();
        const int32_t ks_raw = (rows.ks ? rows.ks : rows.ke)[vrow];
        const int32_t ke_raw = rows.ke[vrow];
        const int32_t tbl_raw = (rows.table ? rows.table : rows.ke)[vrow];
        int craw[E];
        if (tid < kWave) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int i = e * kWave + lane;
                craw[e] = ex.cand[(int64_t)row * ex.cand_stride + min(i, ex.nb - 1)];
                if (i >= ex.nb) craw[e] = -1;
            }
        }
        // fp8 queries (bf16 fragments) load after the expansion, so their registers are not
        // live across its sort
        if constexpr (QF == 0) load_q<QF>(f, qv, qs, weights, sf, row, lane);
        ri.ks = rows.ks ? ks_raw : 0;
        ri.ke = ke_raw;
        if (tid < kWave) {
            const int tbl = rows.table ? tbl_raw : row;
            int ntok;
            const int nlist = expand_row<E>(craw, ri.ks, ri.ke, tbl >= 0 && tbl < k.num_tables,
                                            tbl, ex.cbs, sbk, nsb, k,
                                            reinterpret_cast<int32_t *>(s_word), s_si, s_pg,
                                            ntok);
            if (lane == 0) {
                L.kept = nlist;
                if (ex.kept) {
                    ex.end[row] = ntok;
                    ex.kept[row] = nlist;
                }
            }
        }
    }
    if (tid == 0) s_unit = 0;
    select_clear(s_sel);
    __syncthreads();
    if constexpr (E > 0) {
        if constexpr (QF == 1) load_q<QF>(f, qv, qs, weights, sf, row, lane);
        ri.kept = uniform(L.kept);
        if (ex.kept)
            for (int i = tid; i < nsb; i += NT) {
                ex.si[(int64_t)row * nsb + i] = s_si[i];
                ex.pg[(int64_t)row * nsb + i] = s_pg[i];
            }
    }
    ri.valid_cols = ri.kept * sbk;
    // The selection's first digit is counted while scoring (the scoring waits on
    // memory, so the extra instructions are free): valid keys per key >> 23.
    int nv = 0;
    int *hist0 = &s_sel.hist[0][0];
    const int vgroups = (ri.valid_cols + 63) / 64;
    const int nunits = (vgroups + U - 1) / U;
    const int valid_cols = ri.valid_cols;
    float *lout = logits_out ? logits_out + (int64_t)row * ri.ncols : nullptr;
    score_units<QF, U, G64>(
        k, f, ri.ks, ri.ke, sf,
        [&](int tile, int &page, int &tok) {
            const int c = tile * 16;
            if (c < valid_cols) {
                const int slot = c / sbk;
                page = s_pg[slot];
                tok = s_si[slot] * sbk + c % sbk;
            }
        },
        [&]() {
            int u = 0;
            if (lane == 0) u = atomicAdd(&s_unit, 1);
            u = uniform(u);
            return u < nunits ? u : -1;
        },
        [&](int c, float lg, bool valid) {
            if (c < ri.ncols) {
                const uint32_t w = valid ? __float_as_uint(lg) : kNoColumn;
                s_word[c] = w;
                if (lout) lout[c] = valid ? lg : -INFINITY;
                if (valid) {
                    ++nv;
                    atomicAdd(hist0 + (bits_key(w) >> 23), 1);
                }
            }
        });
    if (lout)
        for (int c = vgroups * 64 + tid; c < ri.ncols; c += NT) lout[c] = -INFINITY;
    int nvalid;
    uint32_t kmin, kmax;   // not needed with the first digit counted
    block_stats_combine<NT>(wave_scan((uint32_t)nv, 0u, OpAdd{}), 0u, 0u, s_sel, nvalid, kmin,
                            kmax);   // also publishes s_word, s_si and the first digit
    uint32_t key[KPT];
#pragma unroll
    for (int i = 0; i < KPT; i += 4) {
        const int c = tid * KPT + i;   // columns past valid_cols: stale LDS, read but not used
        const uint4 x = *reinterpret_cast<const uint4 *>(&s_word[c]);
        key[i] = c < ri.valid_cols ? bits_key(x.x) : 0u;
        key[i + 1] = c + 1 < ri.valid_cols ? bits_key(x.y) : 0u;
        key[i + 2] = c + 2 < ri.valid_cols ? bits_key(x.z) : 0u;
        key[i + 3] = c + 3 < ri.valid_cols ? bits_key(x.w) : 0u;
    }
    select_topk<NT, KPT, true>(key, keys_live(key), nvalid, kmin, kmax, topk, out + (int64_t)row * ostride, s_sel,
                         reinterpret_cast<int32_t *>(s_word), SparseTokens<KPT>{s_si, lsbk});
}

// One layer.  The leading scalar arguments are what the first loads need (the row's
// schedule entries and kept count, its query): preloaded into SGPRs at wave launch, so
// those loads are one round trip.  MXFP4 queries: 16 waves of one-group units a row (one
// row a CU), or, with at least two rows per CU, 8 waves held to 128 VGPRs (WPE = 4
// waves a SIMD) so that two rows share a CU and one selects while the other streams
// K; fp8 queries: 8 waves of 2-group units, or with at least two rows per CU 4 waves,
// two rows a CU (the keys a thread in one sparse block: 32 keys need sbk >= 32).
template <int QF, int NT, int KPT, int U, int WPE, bool G64>
__global__ __launch_bounds__(NT, WPE) void fused_row_kernel(
    const int32_t *si_base, const int32_t *pg_base, const void *qv, const void *qs,
    const void *weights, const int32_t *p_kept, int32_t nsb, int32_t lsbk, int32_t group_rows,
    Rows rows, KCache k, float *logits_out, int32_t topk, int32_t *out, int64_t ostride,
    int32_t sf) {
    __shared__ FusedLds<NT> lds;
    fused_row<QF, NT, KPT, U, G64>(lds, xcd_grouped_row(blockIdx.x, group_rows), si_base,
                                   pg_base, qv, qs, weights, p_kept, nsb, lsbk, rows, k,
                                   logits_out, topk, out, ostride, sf);
}

// Several consuming layers of one step in one launch (grid.y = layer): the layers share
// the rows, the schedule and the cache geometry, and differ in their query, weights, K
// pool and outputs.  A CU that finishes a row of one layer starts a row of the next at
// once, so the layers' launch costs and their start and end skews are paid once.  With
// MXFP4 queries a row takes 8 waves of one-group units held to 128 VGPRs (WPE = 4 waves
// a SIMD), so two rows share a CU: one selects while the other streams K.  fp8 queries
// (208-238 VGPRs, two waves a SIMD) with at least two row-layers a CU: 4 waves a row, two
// rows a CU, so the CUs take the row-layers in half as many rounds, each ending in a
// selection (measured 4 % faster launches on the four-layer long decode than one 8-wave
// row a CU); the keys a thread then lie in one sparse block (KPT <= sbk), which with 32
// keys needs sbk >= 32, else the 8-wave form.
template <int QF, int NT, int KPT, int U, int WPE, bool G64>
__global__ __launch_bounds__(NT, WPE) void fused_layers_kernel(
    const int32_t *si_base, const int32_t *pg_base, const int32_t *p_kept, int32_t nsb,
    int32_t lsbk, int32_t topk, int32_t group_rows, Rows rows, KCache k, LayerSet ls,
    int64_t ostride, int32_t sf) {
    __shared__ FusedLds<NT> lds;
    const int layer = blockIdx.y;
    KCache kl = k;
    kl.values = ls.k_values[layer];
    kl.scales = ls.k_scales[layer];
    fused_row<QF, NT, KPT, U, G64>(lds, xcd_grouped_row(blockIdx.x, group_rows), si_base,
                                   pg_base, ls.q_values[layer], ls.q_scales[layer],
                                   ls.weights[layer], p_kept, nsb, lsbk, rows, kl,
                                   ls.logits_out[layer], topk, ls.out[layer], ostride, sf);
}

// The one-row kernels with each row's candidate expansion inside (64-token sparse blocks,
// up to 128 candidate blocks a row: two ids a lane; MXFP4 queries, or fp8 in the 8-wave
// shapes): wave 0 expands the row into LDS while the other waves load an MXFP4 query, and the workgroups of layer 0 also
// write the schedule, so a later call can reuse it.  The expansion launch and the
// schedule round trip between it and the scoring launch are gone; every workgroup of a
// row (one a layer) expands it again, which costs a candidate load, a sort in registers
// and a block-table load.  The leading scalar arguments are the candidate row's address
// terms (kernarg preload).
template <int QF, int NT, int KPT, int U, int WPE>
__global__ __launch_bounds__(NT, WPE) void expand_fused_row_kernel(
    const int32_t *cand, int64_t cand_stride, const void *qv, const void *qs,
    const void *weights, int32_t nb, int32_t cbs, int32_t nsb, int32_t lsbk, int32_t group_rows,
    Rows rows, KCache k, Schedule s, float *logits_out, int32_t topk, int32_t *out,
    int64_t ostride, int32_t sf) {
    __shared__ FusedLds<NT> lds;
    const FusedExpand ex = {cand, cand_stride, nb, cbs, s.sparse_indices, s.pages, s.end, s.kept};
    fused_row<QF, NT, KPT, U, true, kFusedExpandIds>(
        lds, xcd_grouped_row(blockIdx.x, group_rows), nullptr, nullptr, qv, qs, weights,
        nullptr, nsb, lsbk, rows, k, logits_out, topk, out, ostride, sf, ex);
}

template <int QF, int KPT, int U, int WPE>
__global__ __launch_bounds__(512, WPE) void expand_fused_layers_kernel(
    const int32_t *cand, int64_t cand_stride, int32_t nb, int32_t cbs, int32_t nsb,
    int32_t lsbk, int32_t topk, int32_t group_rows, Rows rows, KCache k, LayerSet ls,
    Schedule s, int64_t ostride, int32_t sf) {
    __shared__ FusedLds<512> lds;
    const int layer = blockIdx.y;
    KCache kl = k;
    kl.values = ls.k_values[layer];
    kl.scales = ls.k_scales[layer];
    const FusedExpand ex = {cand, cand_stride, nb, cbs, s.sparse_indices, s.pages, s.end,
                            layer == 0 ? s.kept : nullptr};
    fused_row<QF, 512, KPT, U, true, kFusedExpandIds>(
        lds, xcd_grouped_row(blockIdx.x, group_rows), nullptr, nullptr, ls.q_values[layer],
        ls.q_scales[layer], ls.weights[layer], nullptr, nsb, lsbk, rows, kl,
        ls.logits_out[layer], topk, ls.out[layer], ostride, sf, ex);
}

}  // namespace

// group_rows argument of the decode scoring kernels (see xcd_grouped_row).
static int32_t grouped_rows(const Rows &rows) {
    return rows.rows_per_request > 1 ? rows.num_rows : 0;
}

int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}


Plan plan_sparse(int q_format, int32_t sbk, int32_t ncols, int32_t num_rows, int32_t num_layers,
                 int cus, bool logits_home) {
    if (num_rows <= 0 || num_layers <= 0) return kPlanNone;
    // At least 8 rows per CU with MXFP4 queries and 64-token sparse blocks: row groups
    // (K tiles shared across the rows of a table).
    const bool groups = q_format == 0 && sbk == 64 && ncols <= 8192 && num_rows >= 8 * cus;
    if (groups) return num_layers >= 2 ? kPlanRowGroupLayers : kPlanRowGroup;
    if (num_rows >= cus) return num_layers >= 2 ? kPlanOneRowLayers : kPlanOneRow;
    // Fewer rows than CUs but at least as many row-layers: one workgroup a row-layer, all
    // layers in one launch (measured 14-25 % faster steps than the split launch pair on
    // 64- and 128-row decode batches with 2 to 8 layers, both query formats: the
    // selection runs in the scoring launch and no logits leave it).
    if (num_layers >= 2 && (int64_t)num_rows * num_layers >= cus) return kPlanOneRowLayers;
    // otherwise every layer in one split launch pair when each layer's logits have a
    // home, else layer by layer
    return num_layers >= 2 && logits_home ? kPlanSplitLayers : kPlanSplit;
}

template <int QF>
static hipError_t launch_sparse_q(const Rows &rows, const void *q_values, const void *q_scales,
                                  const void *weights, int sf, const KCache &k, const Schedule &s,
                                  float *logits_out, float *workspace, int32_t topk, int32_t *out,
                                  int64_t out_stride, const Timing &timing, hipStream_t stream) {
    hipError_t e;
    const int ncols = s.nsb * s.sbk;
    const int ngroups = (ncols + 63) / 64;
    const Plan plan = plan_sparse(QF, s.sbk, ncols, rows.num_rows, 1, device_cus(), true);
    if constexpr (QF == 0) {
        if (plan == kPlanRowGroup)
            return launch_row_groups(rows, q_values, q_scales, weights, sf, k, s, logits_out,
                                     topk, out, out_stride, timing, stream);
    }
    if (plan == kPlanOneRow) {
        // MXFP4, one row a CU: 16 waves with 1-group units (measured 10 % faster 4-layer
        // steps than 8 waves with 4-group units: the row's last unit, and so the wait
        // before the selection, is shorter).  MXFP4 with two or more rows a CU: 8 waves
        // with 1-group units, two rows a CU (measured 23 % faster on 512-2000 rows of 4096
        // columns).  fp8 queries need more registers: 2-group units, 8 waves a row, or 4
        // waves and two rows a CU when there are two or more rows a CU.
#define IDX_LAUNCH_FUSED_G(NT_, KPT_, U_, WPE_, G64_)                                           \
    hipExtLaunchKernelGGL((fused_row_kernel<QF, NT_, KPT_, U_, WPE_, G64_>), dim3(rows.num_rows), \
                          dim3(NT_), 0, stream, timing.start, timing.stop, 0, s.sparse_indices,   \
                          s.pages, q_values, q_scales, weights, s.kept, s.nsb, s.lsbk,            \
                          grouped_rows(rows), rows, k, logits_out, topk, out, out_stride, sf)
#define IDX_LAUNCH_FUSED(NT_, KPT_, U_, WPE_)                                                    \
    do {                                                                                           \
        if (s.sbk == 64) IDX_LAUNCH_FUSED_G(NT_, KPT_, U_, WPE_, true);                            \
        else IDX_LAUNCH_FUSED_G(NT_, KPT_, U_, WPE_, false);                                       \
    } while (0)
        if constexpr (QF == 0) {
            if (rows.num_rows < 2 * device_cus()) {
                if (ncols <= 1024 * 4) IDX_LAUNCH_FUSED(1024, 4, 1, 1);
                else IDX_LAUNCH_FUSED(1024, 8, 1, 1);
                return hipGetLastError();
            }
        }
        if constexpr (QF == 1) {
            // fp8 with two or more rows a CU: 4-wave rows, two a CU (as fused_layers_kernel;
            // measured 7-8 % faster steps on 512 and 1024 rows of 4096 columns)
            if (rows.num_rows >= 2 * device_cus() && (ncols <= 256 * 16 || s.sbk >= 32)) {
                if (ncols <= 256 * 4) IDX_LAUNCH_FUSED(256, 4, 2, 2);
                else if (ncols <= 256 * 8) IDX_LAUNCH_FUSED(256, 8, 2, 2);
                else if (ncols <= 256 * 16) IDX_LAUNCH_FUSED(256, 16, 2, 2);
                else IDX_LAUNCH_FUSED(256, 32, 2, 2);
                return hipGetLastError();
            }
        }
        constexpr int U = QF == 0 ? 1 : 2;
        constexpr int WPE = QF == 0 ? 4 : 1;
        if (ncols <= 512 * 4) IDX_LAUNCH_FUSED(512, 4, U, WPE);
        else if (ncols <= 512 * 8) IDX_LAUNCH_FUSED(512, 8, U, WPE);
        else IDX_LAUNCH_FUSED(512, 16, U, WPE);
#undef IDX_LAUNCH_FUSED
#undef IDX_LAUNCH_FUSED_G
        return hipGetLastError();
    }
    float *logits = logits_out ? logits_out : workspace;
    const int gpw = kSplitGroupsPerWg;
    const dim3 sgrid(rows.num_rows, (ngroups + gpw - 1) / gpw);
#define IDX_LAUNCH_SPLIT_G(G64_)                                                                   \
    hipExtLaunchKernelGGL((score_split_kernel<QF, kSplitGroupsPerWave, G64_>), sgrid,              \
                          dim3(kScoreThreads), 0, stream, timing.start, timing.stop, 0,            \
                          s.sparse_indices, s.pages, q_values, q_scales, weights, s.nsb, s.sbk,    \
                          gpw, grouped_rows(rows), rows, k, logits, sf)
    if (s.sbk == 64)
        IDX_LAUNCH_SPLIT_G(true);
    else
        IDX_LAUNCH_SPLIT_G(false);
#undef IDX_LAUNCH_SPLIT_G
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ncols <= 8 * kTopkThreads)
        hipLaunchKernelGGL((topk_split_kernel<false, 8>), dim3(rows.num_rows), dim3(kTopkThreads), 0,
                           stream, logits, s.sparse_indices, rows.ks, rows.ke, s.kept, s.nsb, s.lsbk,
                           (int64_t)0, 0, topk, out, out_stride);
    else
        hipLaunchKernelGGL((topk_split_kernel<false, 16>), dim3(rows.num_rows), dim3(kTopkThreads), 0,
                           stream, logits, s.sparse_indices, rows.ks, rows.ke, s.kept, s.nsb, s.lsbk,
                           (int64_t)0, 0, topk, out, out_stride);
    return hipGetLastError();
}

hipError_t launch_sparse(int q_format, int score_format, const Rows &rows, const void *q_values,
                         const void *q_scales, const void *weights, const KCache &k,
                         const Schedule &s, float *logits_out, float *workspace, int32_t topk,
                         int32_t *out, int64_t out_stride, const Timing &timing,
                         hipStream_t stream) {
    if (rows.num_rows == 0) return hipSuccess;
    if (q_format == 0)
        return launch_sparse_q<0>(rows, q_values, q_scales, weights, score_format, k, s,
                                  logits_out, workspace, topk, out, out_stride, timing, stream);
    return launch_sparse_q<1>(rows, q_values, q_scales, weights, score_format, k, s, logits_out,
                              workspace, topk, out, out_stride, timing, stream);
}

template <int QF>
static hipError_t launch_split_layers(const Rows &rows, int32_t num_layers, const LayerSet &layers,
                                      int sf, const KCache &k, const Schedule &s, float *workspace,
                                      int32_t topk, int64_t out_stride, const Timing &timing,
                                      hipStream_t stream) {
    const int ncols = s.nsb * s.sbk;
    const int ngroups = (ncols + 63) / 64;
    const int64_t ws_layer = (int64_t)rows.num_rows * ncols;
    const int gpw = kSplitGroupsPerWg;   // as for one layer (launch_sparse_q)
    const dim3 sgrid(rows.num_rows, (ngroups + gpw - 1) / gpw, num_layers);
#define IDX_LAUNCH_SPLIT_LAYERS_G(G64_)                                                            \
    hipExtLaunchKernelGGL((score_split_layers_kernel<QF, kSplitGroupsPerWave, G64_>), sgrid,       \
                          dim3(kScoreThreads), 0, stream, timing.start, timing.stop, 0,            \
                          s.sparse_indices, s.pages, s.nsb, s.sbk, gpw, grouped_rows(rows), rows,  \
                          k, layers, workspace, ws_layer, sf)
    if (s.sbk == 64)
        IDX_LAUNCH_SPLIT_LAYERS_G(true);
    else
        IDX_LAUNCH_SPLIT_LAYERS_G(false);
#undef IDX_LAUNCH_SPLIT_LAYERS_G
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 tgrid(rows.num_rows, num_layers);
    if (ncols <= 8 * kTopkThreads)
        hipLaunchKernelGGL((topk_split_layers_kernel<8>), tgrid, dim3(kTopkThreads), 0, stream,
                           s.sparse_indices, rows.ks, rows.ke, s.kept, s.nsb, s.lsbk, topk, layers,
                           workspace, ws_layer, out_stride);
    else
        hipLaunchKernelGGL((topk_split_layers_kernel<16>), tgrid, dim3(kTopkThreads), 0, stream,
                           s.sparse_indices, rows.ks, rows.ke, s.kept, s.nsb, s.lsbk, topk, layers,
                           workspace, ws_layer, out_stride);
    return hipGetLastError();
}

hipError_t launch_sparse_layers(int q_format, int score_format, const Rows &rows,
                                int32_t num_layers, const LayerSet &layers, const KCache &k,
                                const Schedule &s, float *workspace, size_t workspace_bytes,
                                int32_t topk, int64_t out_stride, const Timing &timing,
                                hipStream_t stream) {
    const int sf = score_format;
    if (rows.num_rows == 0 || num_layers == 0) return hipSuccess;
    const int ncols = s.nsb * s.sbk;
    // every layer's logits must have a home for the batched split launches: its
    // logits_out or its slice of the workspace
    bool all_out = true;
    for (int l = 0; l < num_layers; ++l) all_out = all_out && layers.logits_out[l];
    const size_t need = (size_t)num_layers * rows.num_rows * ncols * sizeof(float);
    const bool home = all_out || (workspace && workspace_bytes >= need);
    const Plan plan = plan_sparse(q_format, s.sbk, ncols, rows.num_rows, num_layers, device_cus(),
                                  home);
    if (plan == kPlanRowGroupLayers)
        return launch_row_groups_layers(rows, num_layers, layers, sf, k, s, topk, out_stride,
                                        timing, stream);
    if (plan == kPlanSplitLayers) {
        if (q_format == 0)
            return launch_split_layers<0>(rows, num_layers, layers, sf, k, s, workspace, topk,
                                          out_stride, timing, stream);
        return launch_split_layers<1>(rows, num_layers, layers, sf, k, s, workspace, topk,
                                      out_stride, timing, stream);
    }
    if (plan == kPlanOneRowLayers) {
        const dim3 grid(rows.num_rows, num_layers);
#define IDX_LAUNCH_LAYERS_G(QF_, NT_, KPT_, U_, WPE_, G64_)                                      \
    hipExtLaunchKernelGGL((fused_layers_kernel<QF_, NT_, KPT_, U_, WPE_, G64_>), grid, dim3(NT_),  \
                          0, stream, timing.start, timing.stop, 0, s.sparse_indices, s.pages,      \
                          s.kept, s.nsb, s.lsbk, topk, grouped_rows(rows), rows, k, layers,        \
                          out_stride, sf)
#define IDX_LAUNCH_LAYERS(QF_, NT_, KPT_, U_, WPE_)                                              \
    do {                                                                                           \
        if (s.sbk == 64) IDX_LAUNCH_LAYERS_G(QF_, NT_, KPT_, U_, WPE_, true);                      \
        else IDX_LAUNCH_LAYERS_G(QF_, NT_, KPT_, U_, WPE_, false);                                 \
    } while (0)
        if (q_format == 0) {
            if (ncols <= 512 * 4) IDX_LAUNCH_LAYERS(0, 512, 4, 1, 4);
            else if (ncols <= 512 * 8) IDX_LAUNCH_LAYERS(0, 512, 8, 1, 4);
            else IDX_LAUNCH_LAYERS(0, 512, 16, 1, 4);
        } else if ((int64_t)rows.num_rows * num_layers >= 2 * device_cus() &&
                   (ncols <= 256 * 16 || s.sbk >= 32)) {
            if (ncols <= 256 * 4) IDX_LAUNCH_LAYERS(1, 256, 4, 2, 2);
            else if (ncols <= 256 * 8) IDX_LAUNCH_LAYERS(1, 256, 8, 2, 2);
            else if (ncols <= 256 * 16) IDX_LAUNCH_LAYERS(1, 256, 16, 2, 2);
            else IDX_LAUNCH_LAYERS(1, 256, 32, 2, 2);
        } else {
            if (ncols <= 512 * 4) IDX_LAUNCH_LAYERS(1, 512, 4, 2, 1);
            else if (ncols <= 512 * 8) IDX_LAUNCH_LAYERS(1, 512, 8, 2, 1);
            else IDX_LAUNCH_LAYERS(1, 512, 16, 2, 1);
        }
#undef IDX_LAUNCH_LAYERS
#undef IDX_LAUNCH_LAYERS_G
        return hipGetLastError();
    }
    for (int l = 0; l < num_layers; ++l) {
        KCache kl = k;
        kl.values = layers.k_values[l];
        kl.scales = layers.k_scales[l];
        const hipError_t e = launch_sparse(q_format, sf, rows, layers.q_values[l],
                                           layers.q_scales[l], layers.weights[l], kl, s,
                                           layers.logits_out[l], workspace, topk, layers.out[l],
                                           out_stride, timing, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

ExpandPlace expansion_place(int q_format, int32_t sbk, int32_t nb, int32_t ncols,
                            int32_t num_rows, int32_t num_layers, int cus, bool logits_home) {
    const Plan plan = plan_sparse(q_format, sbk, ncols, num_rows, num_layers, cus, logits_home);
    if (nb > kFusedExpandIds * kWave) return kExpandLaunch;
    // One-row kernels: only when every row-layer's workgroup is resident at once (at most
    // two a CU): then the expansion overlaps the other workgroups' K streams and the
    // expansion launch is saved (measured 4-6 % faster steps on the 64-row, 4-layer decode
    // batch, 10 % on 256 rows of one layer).  With more rounds each workgroup's expansion, repeated for every layer,
    // delays its own K stream by what the expansion launch costs (256 rows, 4 layers, 8192
    // columns: steps within noise of the two launches, the scoring launch ~3 us longer).
    // fp8 queries: the 8-wave one-row shapes only (fewer than 2 x CUs row-layers; at 2 x CUs
    // their launches take 4-wave rows)
    const int64_t row_layers = (int64_t)num_rows * num_layers;
    if (sbk == 64 && (plan == kPlanOneRow || plan == kPlanOneRowLayers) &&
        (q_format == 0 ? row_layers <= 2 * (int64_t)cus : row_layers < 2 * (int64_t)cus))
        return kExpandOneRow;
    // Split launches (fewer rows, or row-layers, than CUs; short workgroups bound by
    // latency) whose workgroups are all resident at once (MXFP4: 80 VGPRs, six a CU; fp8:
    // 168, three a CU): the expansion launch and its schedule round trip are saved
    // (measured 7-11 % faster steps on 64- and 128-row decode batches).  A second round
    // waits on its own expansions (fp8 on 128 rows, 1024 workgroups: 1.6 % slower steps).
    // fp8 queries only with 64-token sparse blocks: the generic tile path does not fit
    // their 168 VGPRs with the expansion's state.
    const int64_t wgs = (int64_t)num_rows * num_layers *
                        ((((ncols + 63) / 64) + kSplitGroupsPerWg - 1) / kSplitGroupsPerWg);
    if ((q_format == 0 || sbk == 64) && wgs <= (q_format == 0 ? 6 : 3) * (int64_t)cus &&
        ((plan == kPlanSplit && num_layers == 1) || plan == kPlanSplitLayers))
        return kExpandSplit;
    return kExpandLaunch;
}

// The split pair with the expansion inside the scoring launch (one layer, or every layer
// in one launch pair): the selection launch as in launch_sparse_q / launch_split_layers.
template <int QF>
static hipError_t launch_split_expand(const Rows &rows, int32_t num_layers,
                                      const LayerSet &layers, int sf, const KCache &k,
                                      const Schedule &s, const int32_t *cand,
                                      int64_t cand_stride, int32_t nb, int32_t cbs,
                                      float *workspace, int32_t topk, int64_t out_stride,
                                      const Timing &timing, hipStream_t stream) {
    const int ncols = s.nsb * s.sbk;
    const int ngroups = (ncols + 63) / 64;
    const int gpw = kSplitGroupsPerWg;
    hipError_t e;
    if (num_layers == 1) {
        float *logits = layers.logits_out[0] ? layers.logits_out[0] : workspace;
        const dim3 sgrid(rows.num_rows, (ngroups + gpw - 1) / gpw);
#define IDX_LAUNCH_SPLIT_EXPAND_G(G64_)                                                            \
    hipExtLaunchKernelGGL((score_split_expand_kernel<QF, G64_>), sgrid, dim3(kScoreThreads), 0,    \
                          stream, timing.start, timing.stop, 0, cand, cand_stride,                 \
                          layers.q_values[0], layers.q_scales[0], layers.weights[0], nb, cbs,      \
                          s.nsb, s.sbk, gpw, grouped_rows(rows), rows, k, s, logits, sf)
        if (s.sbk == 64)
            IDX_LAUNCH_SPLIT_EXPAND_G(true);
        else if constexpr (QF == 0)
            IDX_LAUNCH_SPLIT_EXPAND_G(false);
        else
            return hipErrorInvalidValue;   // fp8 with sbk < 64: not placed here
#undef IDX_LAUNCH_SPLIT_EXPAND_G
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (ncols <= 8 * kTopkThreads)
            hipLaunchKernelGGL((topk_split_kernel<false, 8>), dim3(rows.num_rows),
                               dim3(kTopkThreads), 0, stream, logits, s.sparse_indices, rows.ks,
                               rows.ke, s.kept, s.nsb, s.lsbk, (int64_t)0, 0, topk,
                               layers.out[0], out_stride);
        else
            hipLaunchKernelGGL((topk_split_kernel<false, 16>), dim3(rows.num_rows),
                               dim3(kTopkThreads), 0, stream, logits, s.sparse_indices, rows.ks,
                               rows.ke, s.kept, s.nsb, s.lsbk, (int64_t)0, 0, topk,
                               layers.out[0], out_stride);
        return hipGetLastError();
    }
    const int64_t ws_layer = (int64_t)rows.num_rows * ncols;
    const dim3 sgrid(rows.num_rows, (ngroups + gpw - 1) / gpw, num_layers);
#define IDX_LAUNCH_SPLIT_EXPAND_LAYERS_G(G64_)                                                     \
    hipExtLaunchKernelGGL((score_split_expand_layers_kernel<QF, G64_>), sgrid,                     \
                          dim3(kScoreThreads), 0,                                                  \
                          stream, timing.start, timing.stop, 0, cand, cand_stride, nb, cbs, s.nsb, \
                          s.sbk, gpw, grouped_rows(rows), rows, k, layers, s, workspace, ws_layer, \
                          sf)
    if (s.sbk == 64)
        IDX_LAUNCH_SPLIT_EXPAND_LAYERS_G(true);
    else if constexpr (QF == 0)
        IDX_LAUNCH_SPLIT_EXPAND_LAYERS_G(false);
    else
        return hipErrorInvalidValue;   // fp8 with sbk < 64: not placed here
#undef IDX_LAUNCH_SPLIT_EXPAND_LAYERS_G
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 tgrid(rows.num_rows, num_layers);
    if (ncols <= 8 * kTopkThreads)
        hipLaunchKernelGGL((topk_split_layers_kernel<8>), tgrid, dim3(kTopkThreads), 0, stream,
                           s.sparse_indices, rows.ks, rows.ke, s.kept, s.nsb, s.lsbk, topk, layers,
                           workspace, ws_layer, out_stride);
    else
        hipLaunchKernelGGL((topk_split_layers_kernel<16>), tgrid, dim3(kTopkThreads), 0, stream,
                           s.sparse_indices, rows.ks, rows.ke, s.kept, s.nsb, s.lsbk, topk, layers,
                           workspace, ws_layer, out_stride);
    return hipGetLastError();
}

hipError_t launch_expand_sparse_layers(int q_format, int score_format, const Rows &rows,
                                       int32_t num_layers, const LayerSet &layers,
                                       const KCache &k, const Schedule &s, const int32_t *cand,
                                       int64_t cand_stride, int32_t nb, int32_t cbs,
                                       float *workspace, size_t workspace_bytes, int32_t topk,
                                       int64_t out_stride, const Timing &timing,
                                       hipStream_t stream) {
    if (rows.num_rows == 0 || num_layers == 0) return hipSuccess;
    const int ncols = s.nsb * s.sbk;
    const int sf = score_format;
    const int cus = device_cus();
    // as launch_sparse_layers: every layer's logits need a home for the batched split pair
    bool all_out = true;
    for (int l = 0; l < num_layers; ++l) all_out = all_out && layers.logits_out[l];
    const size_t need = (size_t)num_layers * rows.num_rows * ncols * sizeof(float);
    const bool home = all_out || (workspace && workspace_bytes >= need);
    const ExpandPlace place = expansion_place(q_format, s.sbk, nb, ncols, rows.num_rows,
                                              num_layers, cus, home);
    if (place == kExpandLaunch) {
        const hipError_t e = launch_expand(rows, k, cand, cand_stride, nb, cbs, s, stream);
        if (e != hipSuccess) return e;
        return launch_sparse_layers(q_format, score_format, rows, num_layers, layers, k, s,
                                    workspace, workspace_bytes, topk, out_stride, timing, stream);
    }
    if (place == kExpandSplit) {
        if (q_format == 0)
            return launch_split_expand<0>(rows, num_layers, layers, sf, k, s, cand, cand_stride,
                                          nb, cbs, workspace, topk, out_stride, timing, stream);
        return launch_split_expand<1>(rows, num_layers, layers, sf, k, s, cand, cand_stride, nb,
                                      cbs, workspace, topk, out_stride, timing, stream);
    }
    if (num_layers == 1) {
        // the launch shapes of launch_sparse_q's one-row plan
#define IDX_LAUNCH_EXPAND_ROW(QF_, NT_, KPT_, U_, WPE_)                                           \
    hipExtLaunchKernelGGL((expand_fused_row_kernel<QF_, NT_, KPT_, U_, WPE_>), dim3(rows.num_rows), \
                          dim3(NT_), 0, stream, timing.start, timing.stop, 0, cand, cand_stride,   \
                          layers.q_values[0], layers.q_scales[0], layers.weights[0], nb, cbs,      \
                          s.nsb, s.lsbk, grouped_rows(rows), rows, k, s, layers.logits_out[0],     \
                          topk, layers.out[0], out_stride, sf)
        if (q_format == 1) {   // fewer than 2 x CUs rows (expansion_place): 8-wave rows
            if (ncols <= 512 * 4) IDX_LAUNCH_EXPAND_ROW(1, 512, 4, 2, 1);
            else if (ncols <= 512 * 8) IDX_LAUNCH_EXPAND_ROW(1, 512, 8, 2, 1);
            else IDX_LAUNCH_EXPAND_ROW(1, 512, 16, 2, 1);
        } else if (rows.num_rows < 2 * cus) {
            if (ncols <= 1024 * 4) IDX_LAUNCH_EXPAND_ROW(0, 1024, 4, 1, 1);
            else IDX_LAUNCH_EXPAND_ROW(0, 1024, 8, 1, 1);
        } else if (ncols <= 512 * 4) IDX_LAUNCH_EXPAND_ROW(0, 512, 4, 1, 4);   // 2 x CUs rows
        else if (ncols <= 512 * 8) IDX_LAUNCH_EXPAND_ROW(0, 512, 8, 1, 4);
        else IDX_LAUNCH_EXPAND_ROW(0, 512, 16, 1, 4);
#undef IDX_LAUNCH_EXPAND_ROW
        return hipGetLastError();
    }
    const dim3 grid(rows.num_rows, num_layers);
#define IDX_LAUNCH_EXPAND_LAYERS(QF_, KPT_, U_, WPE_)                                             \
    hipExtLaunchKernelGGL((expand_fused_layers_kernel<QF_, KPT_, U_, WPE_>), grid, dim3(512), 0,   \
                          stream, timing.start, timing.stop, 0, cand, cand_stride, nb, cbs, s.nsb,  \
                          s.lsbk, topk, grouped_rows(rows), rows, k, layers, s, out_stride, sf)
    if (q_format == 1) {   // fewer than 2 x CUs row-layers (expansion_place): 8-wave rows
        if (ncols <= 512 * 4) IDX_LAUNCH_EXPAND_LAYERS(1, 4, 2, 1);
        else if (ncols <= 512 * 8) IDX_LAUNCH_EXPAND_LAYERS(1, 8, 2, 1);
        else IDX_LAUNCH_EXPAND_LAYERS(1, 16, 2, 1);
    } else if (ncols <= 512 * 4) IDX_LAUNCH_EXPAND_LAYERS(0, 4, 1, 4);
    else if (ncols <= 512 * 8) IDX_LAUNCH_EXPAND_LAYERS(0, 8, 1, 4);
    else IDX_LAUNCH_EXPAND_LAYERS(0, 16, 1, 4);
#undef IDX_LAUNCH_EXPAND_LAYERS
    return hipGetLastError();
}

}  // namespace idx
