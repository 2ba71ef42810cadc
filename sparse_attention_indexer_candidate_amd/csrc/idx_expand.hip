// Candidate expansion: a row's published candidate blocks -> the step's sparse-column
// schedule (sorted distinct kept sparse blocks with their pages, the valid-token count),
// one wave per row.  Every consuming layer of the step reads the same schedule.

#include "idx_device.h"

namespace idx {
namespace {

// ---------------------------------------------------------------- expansion ----

constexpr int kExpandThreads = 256;
constexpr int kExpandRows = kExpandThreads / kWave;

// One wave per row (expand_row: sort, dedupe, list the kept sparse blocks with their
// pages), four rows a workgroup.
//
// The leading scalar arguments are what the first loads need; they come first so the
// hardware preloads them into SGPRs at wave launch (kernarg preload), and the row's
// metadata and candidate ids are one round trip: no load sits behind a branch or
// behind another load (a null ks or table pointer reads ke's slot, then the value is
// replaced).
template <int E>
__global__ __launch_bounds__(kExpandThreads) void expand_kernel(
    int32_t num_rows, const int32_t *p_ks, const int32_t *p_ke, const int32_t *p_tbl,
    const int32_t *cand, int64_t cand_stride, int32_t nb, int32_t cbs, KCache k, Schedule s) {
    __shared__ int32_t s_blk[kExpandRows][kMaxNB];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int r = blockIdx.x * kExpandRows + wave;
    if (r >= num_rows) return;  // whole wave; no workgroup barriers below
    const int32_t ks_raw = (p_ks ? p_ks : p_ke)[r];
    const int32_t ke_raw = p_ke[r];
    const int32_t tbl_raw = (p_tbl ? p_tbl : p_ke)[r];
    int craw[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = e * kWave + lane;
        craw[e] = cand[(int64_t)r * cand_stride + min(i, nb - 1)];
        if (i >= nb) craw[e] = -1;
    }
    const int64_t ks = p_ks ? ks_raw : 0;
    const int64_t ke = ke_raw;
    const int tbl = p_tbl ? tbl_raw : r;
    const bool tbl_ok = tbl >= 0 && tbl < k.num_tables;
    int ntok;
    const int nlist = expand_row<E>(craw, ks, ke, tbl_ok, tbl, cbs, s.sbk, s.nsb, k, s_blk[wave],
                                    s.sparse_indices + (int64_t)r * s.nsb,
                                    s.pages + (int64_t)r * s.nsb, ntok);
    if (lane == 0) {
        s.end[r] = ntok;
        s.kept[r] = nlist;
    }
}

}  // namespace

hipError_t launch_expand(const Rows &rows, const KCache &k, const int32_t *cand, int64_t cand_stride,
                         int32_t nb, int32_t cbs, const Schedule &s, hipStream_t stream) {
    if (rows.num_rows == 0) return hipSuccess;
    const dim3 grid((rows.num_rows + kExpandRows - 1) / kExpandRows);
#define IDX_LAUNCH_EXPAND(E_)                                                                    \
    hipLaunchKernelGGL(expand_kernel<E_>, grid, dim3(kExpandThreads), 0, stream, rows.num_rows,   \
                       rows.ks, rows.ke, rows.table, cand, cand_stride, nb, cbs, k, s)
    if (nb <= 64) IDX_LAUNCH_EXPAND(1);
    else if (nb <= 128) IDX_LAUNCH_EXPAND(2);
    else if (nb <= 256) IDX_LAUNCH_EXPAND(4);
    else IDX_LAUNCH_EXPAND(8);
#undef IDX_LAUNCH_EXPAND
    return hipGetLastError();
}

}  // namespace idx
