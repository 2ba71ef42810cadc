// Candidate expansion: a row's published candidate blocks -> the step's sparse-column
// schedule (sorted distinct kept sparse blocks with their pages, the valid-token count),
// one wave per row.  Every consuming layer of the step reads the same schedule.

#include "idx_device.h"

namespace idx {
namespace {

// ---------------------------------------------------------------- expansion ----

constexpr int kExpandThreads = 256;
constexpr int kExpandRows = kExpandThreads / kWave;

// One wave per row; lane l holds candidate ids l, l + 64, ... (E per lane).  Ids that
// are negative or hold no token of [ks, ke) become INT_MAX; a bitonic sort over the
// 64*E register slots (shuffles across lanes, swaps within a lane) orders them; an id
// is kept if it differs from its predecessor (so repeats count once); kept blocks
// split into cbs/sbk sparse blocks, of which those holding a token of [ks, ke) and
// mapped by the block table inside the pool are listed in order with their page.
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
    const int sbk = s.sbk, nsb = s.nsb, per = cbs / sbk;

    int v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int b = craw[e];
        const bool ok = b >= 0 && (int64_t)b * cbs < ke && ((int64_t)b + 1) * cbs > ks;
        v[e] = ok ? b : INT_MAX;
    }
#pragma unroll
    for (int kk = 2; kk <= kWave * E; kk <<= 1) {
#pragma unroll
        for (int j = kk >> 1; j > 0; j >>= 1) {
            if (j >= kWave) {
                const int je = j / kWave;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (e & je) continue;
                    const int e2 = e | je;
                    const bool asc = ((e * kWave + lane) & kk) == 0;
                    const int a = v[e], b = v[e2];
                    const bool sw = asc ? (a > b) : (a < b);
                    v[e] = sw ? b : a;
                    v[e2] = sw ? a : b;
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int x = e * kWave + lane;
                    const int p = lane_xor(v[e], j);
                    const bool lower = (x & j) == 0, asc = (x & kk) == 0;
                    v[e] = (lower == asc) ? min(v[e], p) : max(v[e], p);
                }
            }
        }
    }
    int nkept = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        int prev = __builtin_amdgcn_update_dpp(0, v[e], 0x138, 0xF, 0xF, false);   // wave_shr:1
        if (lane == 0) prev = (e == 0) ? -1 : __builtin_amdgcn_readlane(v[e > 0 ? e - 1 : 0], kWave - 1);
        const bool keep = v[e] != INT_MAX && v[e] != prev;
        const uint64_t m = __ballot(keep);
        if (keep) s_blk[wave][nkept + __popcll(m & lanemask_lt())] = v[e];
        nkept += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();

    int32_t *out_si = s.sparse_indices + (int64_t)r * nsb;
    int32_t *out_pg = s.pages + (int64_t)r * nsb;
    const int total = nkept * per;
    int nlist = 0, ntok = 0;
    for (int base = 0; base < total; base += kWave) {
        const int i = base + lane;
        bool ok = false;
        int32_t sb = 0, page = -1;
        if (i < total) {
            const int64_t sb64 = (int64_t)s_blk[wave][i / per] * per + i % per;
            const int64_t lo = max(sb64 * sbk, ks), hi = min(sb64 * sbk + sbk, ke);
            const int64_t lp = sb64 * sbk / k.page_size;
            if (hi > lo && tbl_ok && lp < k.pages_per_table) {
                page = k.block_table[(int64_t)tbl * k.block_table_stride + lp];
                ok = page >= 0 && page < k.num_pages;
                if (ok) ntok += (int)(hi - lo);
            }
            sb = (int32_t)sb64;
        }
        const uint64_t m = __ballot(ok);
        if (ok) {
            const int pos = nlist + __popcll(m & lanemask_lt());
            out_si[pos] = sb;
            out_pg[pos] = page;
        }
        nlist += __popcll(m);
    }
    for (int i = nlist + lane; i < nsb; i += kWave) {
        out_si[i] = -1;
        out_pg[i] = -1;
    }
    ntok = wave_sum(ntok);
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
