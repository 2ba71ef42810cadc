// gfx950 kernels of the candidate-consuming sparse MQA-logits indexer.
//
//  expand_kernel       candidate expansion -> sparse-column schedule (one workgroup per row)
//  score_*_kernel      paged gather of e2m1 K + UE8M0 scales, MX-scaled MFMA
//                      [64 heads x 128] . [128 x 16 columns], ReLU, fp32 weighted
//                      head reduce; one wave per 64-column group
//  topk_kernel         per-row radix select on the fp32 logits with ties toward the
//                      lower column, ascending output, -1 fill (one workgroup per row)
//
// The operation follows the vLLM DeepSeek-V4.1 pages (sparse_mqa_indexer,
// the sparse indexer backend source, rocm_paged_mxfp4_indexer): logits over the
// candidate blocks only, fp32 weights and logits on gfx950, top-k token ids with
// -1 past the valid count.
//
// MFMA operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 (measured on gfx950):
//   A (16 x 128), e2m1: lane l holds row l%16, k = 32*(l/16) + j (j < 32), element
//     j in nibble j of the lane's first 4 dwords (low nibble first);
//   A, e4m3: lane l holds row l%16, bytes j < 16 -> k = 16*(l/16) + j and bytes
//     j >= 16 -> k = 64 + 16*(l/16) + j - 16;
//   B (128 x 16) mirrors A with column l%16;
//   the lane's scale byte (op_sel 0) scales row/column l%16, k-block l/16 (32 k);
//   C: lane l holds column l%16, rows 4*(l/16) + v in its 4 accumulators.
// With A = 16 query heads of one row and B = 16 tokens of K, one 16-byte load per
// lane delivers a token's packed values straight into the B operand, and the head
// reduce is 16 in-register FMAs per lane plus a 4-way cross-lane exchange.
#include "idx_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxNB = 512;    // NB * cbs <= 8192 with cbs >= 16
constexpr int kMaxNSB = 512;   // NSB * sbk <= 8192 with sbk >= 16
constexpr int kMaxDenseBlocks = 65536 / 16;

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ---------------------------------------------------------------- block scans --

__device__ __forceinline__ int wave_incl_scan(int x) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    return x;
}

// Exclusive prefix sum over the workgroup (NT threads); *total gets the sum.
// smem holds NT/64 + 1 ints.  Contains barriers: call from every thread.
template <int NT>
__device__ int block_excl_scan(int x, int *total, int *smem) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    int incl = wave_incl_scan(x);
    if (lane == kWave - 1) smem[wid] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int w = 0; w < NT / kWave; ++w) {
            int t = smem[w];
            smem[w] = acc;
            acc += t;
        }
        smem[NT / kWave] = acc;
    }
    __syncthreads();
    int res = smem[wid] + incl - x;
    *total = smem[NT / kWave];
    __syncthreads();
    return res;
}

// ---------------------------------------------------------------- expansion ----

constexpr int kExpandThreads = 256;

// One workgroup per row.  kept[i] marks candidate ids that are >= 0, hold a token
// of [ks, ke) and are the first occurrence of their id; a kept id's rank among
// kept ids gives its sorted position; each kept block splits into cbs/sbk sparse
// blocks at positions rank*per + j, of which those holding a token of [ks, ke)
// (and whose page the table maps inside the pool) are compacted in order.
__global__ __launch_bounds__(kExpandThreads) void expand_kernel(Rows rows, KCache k,
                                                                const int32_t *cand,
                                                                int64_t cand_stride, int32_t nb,
                                                                int32_t cbs, Schedule s) {
    __shared__ int32_t s_id[kMaxNB];
    __shared__ int32_t s_keep[kMaxNB];
    __shared__ int32_t s_sb[kMaxNSB];
    __shared__ int32_t s_cnt[kMaxNSB];
    __shared__ int s_scan[kExpandThreads / kWave + 1];
    constexpr int NT = kExpandThreads;
    const int r = blockIdx.x, tid = threadIdx.x;
    const int64_t ks = rows.ks ? rows.ks[r] : 0;
    const int64_t ke = rows.ke[r];
    const int tbl = rows.table ? rows.table[r] : r;
    const bool tbl_ok = tbl >= 0 && tbl < k.num_tables;
    const int sbk = s.sbk, nsb = s.nsb, per = cbs / sbk;

    for (int i = tid; i < nb; i += NT) s_id[i] = cand[(int64_t)r * cand_stride + i];
    for (int i = tid; i < nsb; i += NT) {
        s_sb[i] = -1;
        s_cnt[i] = 0;
    }
    __syncthreads();
    for (int i = tid; i < nb; i += NT) {
        const int b = s_id[i];
        bool keep = b >= 0 && (int64_t)b * cbs < ke && ((int64_t)b + 1) * cbs > ks;
        for (int j = 0; j < i && keep; ++j) keep = s_id[j] != b;
        s_keep[i] = keep;
    }
    __syncthreads();
    for (int i = tid; i < nb; i += NT) {
        if (!s_keep[i]) continue;
        const int b = s_id[i];
        int rank = 0;
        for (int j = 0; j < nb; ++j) rank += (s_keep[j] && s_id[j] < b);
        for (int j = 0; j < per; ++j) {
            const int64_t sb = (int64_t)b * per + j;
            const int64_t lo = max(sb * sbk, ks), hi = min(sb * sbk + sbk, ke);
            if (hi <= lo) continue;
            const int64_t lp = sb * sbk / k.page_size;
            if (!tbl_ok || lp >= k.pages_per_table) continue;
            const int32_t page = k.block_table[(int64_t)tbl * k.block_table_stride + lp];
            if (page < 0 || page >= k.num_pages) continue;
            s_sb[rank * per + j] = (int32_t)sb;
            s_cnt[rank * per + j] = (int32_t)(hi - lo);
        }
    }
    __syncthreads();
    const int chunk = (nsb + NT - 1) / NT;
    const int c0 = min(tid * chunk, nsb), c1 = min(c0 + chunk, nsb);
    int mine = 0, toks = 0;
    for (int i = c0; i < c1; ++i) {
        mine += s_sb[i] >= 0;
        toks += s_cnt[i];
    }
    int total = 0, tok_total = 0;
    int pos = block_excl_scan<NT>(mine, &total, s_scan);
    block_excl_scan<NT>(toks, &tok_total, s_scan);
    int32_t *out = s.sparse_indices + (int64_t)r * nsb;
    for (int i = c0; i < c1; ++i)
        if (s_sb[i] >= 0) out[pos++] = s_sb[i];
    for (int i = total + tid; i < nsb; i += NT) out[i] = -1;
    if (tid == 0) {
        s.end[r] = tok_total;
        s.kept[r] = total;
    }
}

// ---------------------------------------------------------------- scoring ------

constexpr int kScoreThreads = 256;

// Per-lane query state of one row: the A operands of the four 16-head tiles, their
// scale operands, and the weights of the heads whose accumulators the lane holds
// (heads 16*ht + 4*(lane/16) + v).
template <int QF>
struct QFrag {
    v8i a[4];
    int sc[4];
    float w[4][4];
};

template <int QF>
__device__ __forceinline__ void load_q(QFrag<QF> &f, const void *qv, const void *qs,
                                       const float *weights, int row, int lane) {
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        const int64_t h = (int64_t)row * kHeads + 16 * ht + n;
        if (QF == 0) {
            const uint4 x = *(const uint4 *)((const uint8_t *)qv + h * (kHeadDim / 2) + 16 * g);
            f.a[ht] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
            f.sc[ht] = ((const uint8_t *)qs)[h * (kHeadDim / 32) + g];
        } else {
            const uint8_t *p = (const uint8_t *)qv + h * kHeadDim;
            const uint4 x = *(const uint4 *)(p + 16 * g);
            const uint4 y = *(const uint4 *)(p + 64 + 16 * g);
            f.a[ht] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                          (int)y.x, (int)y.y, (int)y.z, (int)y.w};
            f.sc[ht] = 127;  // 2^0: the fp8 row scale is folded into the weights
        }
    }
    const float rs = (QF == 1) ? ((const float *)qs)[row] : 1.0f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            f.w[ht][v] = weights[(int64_t)row * kHeads + 16 * ht + 4 * g + v] * rs;
}

// Partial weighted ReLU head sum of the lane's 16 heads for its column of one
// 16-token tile.  The same code serves the sparse and the dense kernels, so a
// token's logit does not depend on which path scored it.
template <int QF>
__device__ __forceinline__ float tile_partial(const QFrag<QF> &f, const v8i &kb, int ksc) {
    float p = 0.0f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.a[ht], kb, acc, QF == 0 ? 4 : 0, 4,
                                                               0, f.sc[ht], 0, ksc);
#pragma unroll
        for (int v = 0; v < 4; ++v) p = __builtin_fmaf(f.w[ht][v], fmaxf(acc[v], 0.0f), p);
    }
    return p;
}

// Lanes of group g = lane/16 hold partial sums p[t] (their 16 heads) of column
// lane%16 of tiles t = 0..3.  Returns, in lane l, the full sum of tile l/16's
// column l%16, i.e. of column l of the 64-column group.  Every tile's sum is
// ((p(g0) + p(g0^2)) + (p(g0^1) + p(g0^3))) up to the order of operands of each
// addition, so the result does not depend on the column's position in the group.
__device__ __forceinline__ float reduce_transpose4(float p0, float p1, float p2, float p3,
                                                   int lane) {
    const int g = lane >> 4;
    const bool b1 = (g & 2) != 0, b0 = (g & 1) != 0;
    const float a0 = b1 ? p2 : p0, a1 = b1 ? p3 : p1;
    const float s0 = b1 ? p0 : p2, s1 = b1 ? p1 : p3;
    const float q0 = a0 + __shfl_xor(s0, 32, kWave);
    const float q1 = a1 + __shfl_xor(s1, 32, kWave);
    const float keep = b0 ? q1 : q0, send = b0 ? q0 : q1;
    return keep + __shfl_xor(send, 16, kWave);
}

// Tile of 16 consecutive tokens starting at tok0 (inside one page): the lane's
// B operand (16 bytes of token tok0 + lane%16, k-block lane/16) and scale byte.
__device__ __forceinline__ void load_k_tile(const KCache &k, int32_t page, int32_t j0, int lane,
                                            v8i &kb, int &ksc) {
    const int n = lane & 15, g = lane >> 4;
    const int64_t slot = (int64_t)j0 + n;
    const uint4 x = *(const uint4 *)(k.values + (int64_t)page * k.values_page_stride +
                                     slot * (kHeadDim / 2) + 16 * g);
    kb = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
    ksc = k.scales[(int64_t)page * k.scales_page_stride + slot * (kHeadDim / 32) + g];
}

// Sparse scoring.  grid = (rows, column chunks); each wave takes 64-column groups of
// the row's sparse-column space round robin.  Column c maps to token
// sparse_indices[c / sbk] * sbk + c % sbk; a 16-column tile never crosses a sparse
// block (sbk is a multiple of 16) nor a page (page_size is a multiple of sbk).
template <int QF>
__global__ __launch_bounds__(kScoreThreads) void score_sparse_kernel(
    Rows rows, const void *qv, const void *qs, const float *weights, KCache k, Schedule s,
    float *logits, int groups_per_wg) {
    const int row = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int ncols = s.nsb * s.sbk;
    const int ngroups = (ncols + 63) / 64;
    const int gb = blockIdx.y * groups_per_wg;
    const int ge = min(gb + groups_per_wg, ngroups);
    const int kept = max(0, min(uniform(s.kept[row]), s.nsb));
    const int valid_cols = kept * s.sbk;
    const int ks = rows.ks ? rows.ks[row] : 0;
    const int ke = rows.ke[row];
    const int tbl = rows.table ? rows.table[row] : row;
    const bool tbl_ok = tbl >= 0 && tbl < k.num_tables;
    const int32_t *si = s.sparse_indices + (int64_t)row * s.nsb;
    const int32_t *bt = k.block_table + (int64_t)(tbl_ok ? tbl : 0) * k.block_table_stride;
    float *lrow = logits + (int64_t)row * ncols;

    QFrag<QF> f;
    if (gb * 64 < valid_cols && tbl_ok) load_q<QF>(f, qv, qs, weights, row, lane);

    for (int grp = gb + wave; grp < ge; grp += kScoreThreads / kWave) {
        const int c0 = grp * 64;
        v8i kb[4];
        int ksc[4];
        bool tv[4];
        int tok0[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int tc = c0 + 16 * t;
            tv[t] = false;
            tok0[t] = 0;
            if (tc < valid_cols && tbl_ok) {
                const int sb = uniform(si[tc / s.sbk]);
                const int64_t tok = (int64_t)sb * s.sbk + tc % s.sbk;
                const int64_t lp = tok / k.page_size;
                const int32_t page =
                    (sb >= 0 && lp < k.pages_per_table) ? uniform(bt[lp]) : -1;
                if (page >= 0 && page < k.num_pages) {
                    tv[t] = true;
                    tok0[t] = (int)tok;
                    load_k_tile(k, page, (int)(tok % k.page_size), lane, kb[t], ksc[t]);
                }
            }
        }
        float p[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) p[t] = tv[t] ? tile_partial<QF>(f, kb[t], ksc[t]) : 0.0f;
        const float lg = reduce_transpose4(p[0], p[1], p[2], p[3], lane);
        const int g = lane >> 4;
        const bool mine = g == 0 ? tv[0] : g == 1 ? tv[1] : g == 2 ? tv[2] : tv[3];
        const int tk = (g == 0 ? tok0[0] : g == 1 ? tok0[1] : g == 2 ? tok0[2] : tok0[3]) + (lane & 15);
        const int c = c0 + lane;
        if (c < ncols) lrow[c] = (mine && tk >= ks && tk < ke) ? lg : -INFINITY;
    }
}

// Dense scoring (the comparator): column t is token t, every token < max_ctx.
template <int QF>
__global__ __launch_bounds__(kScoreThreads) void score_dense_kernel(
    Rows rows, int32_t max_ctx, const void *qv, const void *qs, const float *weights, KCache k,
    float *logits, int64_t lstride, int groups_per_wg) {
    const int row = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int ngroups = (max_ctx + 63) / 64;
    const int gb = blockIdx.y * groups_per_wg;
    const int ge = min(gb + groups_per_wg, ngroups);
    const int ks = rows.ks ? rows.ks[row] : 0;
    const int ke = min(rows.ke[row], max_ctx);
    const int tbl = rows.table ? rows.table[row] : row;
    const bool tbl_ok = tbl >= 0 && tbl < k.num_tables;
    const int32_t *bt = k.block_table + (int64_t)(tbl_ok ? tbl : 0) * k.block_table_stride;
    float *lrow = logits + (int64_t)row * lstride;

    QFrag<QF> f;
    if (gb * 64 < ke && (gb + groups_per_wg) * 64 > ks && tbl_ok)
        load_q<QF>(f, qv, qs, weights, row, lane);

    for (int grp = gb + wave; grp < ge; grp += kScoreThreads / kWave) {
        const int c0 = grp * 64;
        v8i kb[4];
        int ksc[4];
        bool tv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int tok = c0 + 16 * t;
            tv[t] = false;
            if (tok < ke && tok + 16 > ks && tbl_ok) {
                const int lp = tok / k.page_size;
                const int32_t page = lp < k.pages_per_table ? uniform(bt[lp]) : -1;
                if (page >= 0 && page < k.num_pages) {
                    tv[t] = true;
                    load_k_tile(k, page, tok % k.page_size, lane, kb[t], ksc[t]);
                }
            }
        }
        float p[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) p[t] = tv[t] ? tile_partial<QF>(f, kb[t], ksc[t]) : 0.0f;
        const float lg = reduce_transpose4(p[0], p[1], p[2], p[3], lane);
        const int g = lane >> 4;
        const bool mine = g == 0 ? tv[0] : g == 1 ? tv[1] : g == 2 ? tv[2] : tv[3];
        const int t = c0 + lane;  // < ngroups * 64 <= lstride
        lrow[t] = (mine && t >= ks && t < ke) ? lg : -INFINITY;
    }
}

// ---------------------------------------------------------------- top-k --------

constexpr int kTopkThreads = 1024;

// Order-preserving map of an fp32 logit to uint32 (larger float -> larger key);
// -0 is first made +0 so the two compare equal.  Finite logits map above 0x007FFFFF,
// so key 0 is free to mark an invalid column.
__device__ __forceinline__ uint32_t ordered_key(float x) {
    const uint32_t u = __float_as_uint(x + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup per row.  Thread i owns columns [i*KPT, (i+1)*KPT), so column order
// (= ascending token order) is thread order then register order.  The count-th
// largest key is found MSB-first with 8-bit digits; a pass stops early once the
// chosen digit's bucket is taken whole.  Selected: keys above the prefix, plus the
// first k_rem keys equal to it in column order (ties toward the lower token).
template <int KPT, bool DENSE>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(Rows rows, Schedule s,
                                                            const float *logits, int64_t lstride,
                                                            int32_t ncols, int32_t topk,
                                                            int32_t *out, int64_t ostride) {
    __shared__ int32_t s_si[DENSE ? 1 : kMaxNSB];
    __shared__ uint32_t s_bits[DENSE ? kMaxDenseBlocks / 32 : 1];
    __shared__ int s_hist[256];
    __shared__ int s_scan[kTopkThreads / kWave + 1];
    __shared__ int s_w[4];
    __shared__ int s_sel[3];
    constexpr int NT = kTopkThreads;
    const int row = blockIdx.x, tid = threadIdx.x;
    const int ks = rows.ks ? rows.ks[row] : 0;
    const int ke = rows.ke[row];
    const int kept = max(0, min(s.kept[row], s.nsb));
    const int sbk = s.sbk;
    const int32_t *si = s.sparse_indices + (int64_t)row * s.nsb;
    int32_t *orow = out + (int64_t)row * ostride;

    if (!DENSE) {
        for (int i = tid; i < kept; i += NT) s_si[i] = si[i];
    } else {
        const int nwords = (ncols / sbk + 31) / 32;
        for (int i = tid; i < nwords; i += NT) s_bits[i] = 0u;
        __syncthreads();
        for (int i = tid; i < kept; i += NT) {
            const int b = si[i];
            if (b >= 0 && b < ncols / sbk) atomicOr(&s_bits[b >> 5], 1u << (b & 31));
        }
    }
    __syncthreads();

    auto token_of = [&](int c) -> int {
        return DENSE ? c : s_si[c / sbk] * sbk + c % sbk;
    };
    auto valid_col = [&](int c) -> bool {
        if (DENSE) {
            if (c < ks || c >= ke || c >= ncols) return false;
            const int b = c / sbk;
            return (s_bits[b >> 5] >> (b & 31)) & 1u;
        }
        if (c >= kept * sbk) return false;
        const int t = token_of(c);
        return t >= ks && t < ke;
    };

    uint32_t key[KPT];
    int nvalid = 0;
    const int cbase = tid * KPT;
    const float *lrow = logits + (int64_t)row * lstride;
#pragma unroll
    for (int i = 0; i < KPT; i += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (cbase + i < ncols) x = *(const float4 *)(lrow + cbase + i);
        const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool v = valid_col(cbase + i + j);
            key[i + j] = v ? ordered_key(xs[j]) : 0u;
            nvalid += v;
        }
    }
    int total_valid = 0;
    block_excl_scan<NT>(nvalid, &total_valid, s_scan);
    const int count = min(topk, total_valid);

    // Radix select of the count-th largest key (skipped when every valid key is taken).
    const bool take_all = count == total_valid;
    uint32_t prefix = 0;
    int depth = 0, k_rem = count;
    if (!take_all) {
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            if (tid < 256) s_hist[tid] = 0;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const uint32_t kk = key[i];
                if (kk != 0u && (pass == 0 || (kk >> (shift + 8)) == prefix))
                    atomicAdd(&s_hist[(kk >> shift) & 255u], 1);
            }
            __syncthreads();
            int c = 0, incl = 0;
            if (tid < 256) {
                c = s_hist[255 - tid];
                incl = wave_incl_scan(c);
                if ((tid & 63) == 63) s_w[tid >> 6] = incl;
            }
            __syncthreads();
            if (tid < 256) {
                for (int w = 0; w < (tid >> 6); ++w) incl += s_w[w];
                const int before = incl - c;
                if (before < k_rem && incl >= k_rem) {
                    s_sel[0] = 255 - tid;
                    s_sel[1] = k_rem - before;
                    s_sel[2] = c;
                }
            }
            __syncthreads();
            prefix = (prefix << 8) | (uint32_t)s_sel[0];
            k_rem = s_sel[1];
            depth += 8;
            const bool whole = s_sel[2] == k_rem;
            __syncthreads();
            if (whole) break;
        }
    }

    // Compaction in column order.
    int ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const uint32_t kk = key[i];
        if (kk == 0u) continue;
        if (take_all) {
            ++ngt;
        } else {
            const uint32_t top = kk >> (32 - depth);
            ngt += top > prefix;
            neq += top == prefix;
        }
    }
    int tot_gt = 0, tot_eq = 0;
    int gpos = block_excl_scan<NT>(ngt, &tot_gt, s_scan);
    int epos = block_excl_scan<NT>(neq, &tot_eq, s_scan);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const uint32_t kk = key[i];
        if (kk == 0u) continue;
        const int c = cbase + i;
        if (take_all) {
            if (gpos < count) orow[gpos] = token_of(c);
            ++gpos;
            continue;
        }
        const uint32_t top = kk >> (32 - depth);
        if (top > prefix) {
            const int pos = gpos + min(epos, k_rem);
            if (pos < count) orow[pos] = token_of(c);
            ++gpos;
        } else if (top == prefix) {
            if (epos < k_rem && gpos + epos < count) orow[gpos + epos] = token_of(c);
            ++epos;
        }
    }
    for (int i = count + tid; i < topk; i += NT) orow[i] = -1;
}

}  // namespace

// ---------------------------------------------------------------- launchers ----

hipError_t launch_expand(const Rows &rows, const KCache &k, const int32_t *cand, int64_t cand_stride,
                         int32_t nb, int32_t cbs, const Schedule &s, hipStream_t stream) {
    if (rows.num_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(expand_kernel, dim3(rows.num_rows), dim3(kExpandThreads), 0, stream, rows,
                       k, cand, cand_stride, nb, cbs, s);
    return hipGetLastError();
}

static int sparse_groups_per_wg(int32_t num_rows, int ngroups) {
    // Enough workgroups to cover 256 CUs several times over, each wave at least
    // one 64-column group.
    int gpw = 4;
    while (gpw < 16 && (int64_t)num_rows * ((ngroups + gpw - 1) / gpw) > 4096) gpw *= 2;
    return gpw;
}

hipError_t launch_score_sparse(int q_format, const Rows &rows, const void *q_values,
                               const void *q_scales, const float *weights, const KCache &k,
                               const Schedule &s, float *logits, hipStream_t stream) {
    if (rows.num_rows == 0) return hipSuccess;
    const int ngroups = (s.nsb * s.sbk + 63) / 64;
    const int gpw = sparse_groups_per_wg(rows.num_rows, ngroups);
    dim3 grid(rows.num_rows, (ngroups + gpw - 1) / gpw);
    if (q_format == 0)
        hipLaunchKernelGGL(score_sparse_kernel<0>, grid, dim3(kScoreThreads), 0, stream, rows,
                           q_values, q_scales, weights, k, s, logits, gpw);
    else
        hipLaunchKernelGGL(score_sparse_kernel<1>, grid, dim3(kScoreThreads), 0, stream, rows,
                           q_values, q_scales, weights, k, s, logits, gpw);
    return hipGetLastError();
}

hipError_t launch_score_dense(int q_format, const Rows &rows, int32_t max_ctx, const void *q_values,
                              const void *q_scales, const float *weights, const KCache &k,
                              float *logits, int64_t logits_stride, hipStream_t stream) {
    if (rows.num_rows == 0) return hipSuccess;
    const int ngroups = (max_ctx + 63) / 64;
    const int gpw = 16;
    dim3 grid(rows.num_rows, (ngroups + gpw - 1) / gpw);
    if (q_format == 0)
        hipLaunchKernelGGL(score_dense_kernel<0>, grid, dim3(kScoreThreads), 0, stream, rows,
                           max_ctx, q_values, q_scales, weights, k, logits, logits_stride, gpw);
    else
        hipLaunchKernelGGL(score_dense_kernel<1>, grid, dim3(kScoreThreads), 0, stream, rows,
                           max_ctx, q_values, q_scales, weights, k, logits, logits_stride, gpw);
    return hipGetLastError();
}

hipError_t launch_topk(bool dense, const Rows &rows, const Schedule &s, const float *logits,
                       int64_t logits_stride, int32_t ncols, int32_t topk, int32_t *out,
                       int64_t out_stride, hipStream_t stream) {
    if (rows.num_rows == 0) return hipSuccess;
    if (dense)
        hipLaunchKernelGGL((topk_kernel<64, true>), dim3(rows.num_rows), dim3(kTopkThreads), 0,
                           stream, rows, s, logits, logits_stride, ncols, topk, out, out_stride);
    else
        hipLaunchKernelGGL((topk_kernel<8, false>), dim3(rows.num_rows), dim3(kTopkThreads), 0,
                           stream, rows, s, logits, logits_stride, ncols, topk, out, out_stride);
    return hipGetLastError();
}

}  // namespace idx
