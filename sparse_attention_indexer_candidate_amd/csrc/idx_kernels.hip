// gfx950 kernels of the candidate-consuming sparse MQA-logits indexer.
//
//  expand_kernel        candidate expansion -> sparse-column schedule, one wave per row:
//                       register/shuffle bitonic sort of the candidate ids, ballot
//                       compaction, block-table lookups (page ids kept in the schedule)
//  score core           paged gather of e2m1 K + UE8M0 scales, MX-scaled MFMA
//                       [64 heads x 128] . [128 x 16 tokens], ReLU, fp32 weighted head
//                       reduce; one wave per 64-column group, K loads batched
//  select_topk          per-row radix select on fp32 logits, ties toward the lower
//                       column, ascending output, -1 fill (one workgroup per row);
//                       validity comes from the tokens, never from a logit's value
//  row_group_kernel     >= 8 rows per CU with MXFP4 queries (prefill chunks): 2 rows
//                       per workgroup share K tiles; logits in LDS, selected in turn
//  fused_row_kernel     rows >= CUs otherwise: one workgroup scores a whole row into LDS
//                       and selects from LDS (no global round trip, no cross-workgroup
//                       sync); MXFP4 with >= 2 rows a CU: 8-wave rows, two a CU
//  fused_layers_kernel  the one-row kernel for several layers sharing a schedule, one
//                       launch (grid.y = layer); MXFP4: 8-wave rows, two a CU, so one
//                       row's selection overlaps another's K stream
//  score_split_kernel + topk_split_kernel
//                       fewer rows than CUs: rows split over workgroups, logits in
//                       global scratch, selection in a second launch
//  score_dense_kernel + topk_split_kernel<dense>
//                       the comparator: every token of [ks, ke) with the same
//                       per-tile code, then the candidates' keys gathered from the
//                       dense row in schedule order and the same selection
//  measure_read_kernel, measure_mfma_kernel, measure_mfma_relu_kernel
//                       reference rates for the roofline (read stream, MFMA-only loop,
//                       MFMA loop with the ReLU-weight epilogue)
//
// Kernel arguments: the expansion, split and one-row kernels take the pointers their
// first loads need as leading scalar arguments, which gfx950 preloads into SGPRs at
// wave launch (the build passes -amdgpu-kernarg-preload-count), and issue those loads
// before any is used, with no load behind a branch: a kernel's first memory round trip
// is then its first data, not its own arguments.
//
// The operation follows the vLLM DeepSeek-V4.1 pages (sparse_mqa_indexer, the
// sparse indexer backend source, rocm_paged_mxfp4_indexer): logits over the
// candidate blocks only, fp32 weights and logits on gfx950, top-k token ids with -1
// past the valid count.
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
//
// fp8 (e4m3) queries use v_mfma_f32_16x16x32_bf16 instead: the MX fp8 x fp4 MFMA
// adds each aligned group of 8 products in a narrow adder (measured: 448 + 2^-9
// in one group returns 448), which misses the fp32 tolerance on real data, while
// the bf16 MFMA keeps fp32-level sums.  e4m3 codes and scaled e2m1 values are
// exact in bf16 (converted with v_cvt_scalef32_pk_bf16_fp8 / _fp4).  The bf16
// MFMA's k slot (step s, lane group g, element j) carries dimension
// 32*g + 8*s + j for both operands, so lane g again reads the 32 dimensions of
// its scale block: the same 16-byte K load and scale byte as the fp4 path.
//
// No kernel here synchronises workgroups through memory: an agent-scope release /
// acquire pair costs an L2 writeback and invalidate on this multi-XCD part
// (measured: +29 us on a 64-row decode batch), so cross-workgroup hand-offs go
// through kernel boundaries instead.
#include "idx_internal.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

namespace idx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxNB = 512;          // NB * cbs <= 8192 with cbs >= 16
constexpr int kMaxNSB = 512;         // NSB * sbk <= 8192 with sbk >= 16
constexpr int kMaxRowCols = 8192;    // NB * cbs

// Pointers rebuilt from integers (per-tile bases read back from lanes) are tagged
// with the global address space so loads use the global (not flat) path.
#define kGlobal __attribute__((address_space(1)))

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// A zero the compiler cannot see through: added to a uniform index it makes the load a
// vector load, which issues in program order beside the kernel's other first loads
// (a scalar load of a uniform address may be scheduled after a later wait).
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

// 64-bit value from two 32-bit halves as returned by v_readlane (a signed int): both
// halves are zero-extended, never sign-extended.
__device__ __forceinline__ uint64_t join64(int hi, int lo) {
    return ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo;
}

// Slot of token t (>= 0) within its page: a mask when the page size is a power of two
// (the usual case; the test is uniform), a division otherwise.
__device__ __forceinline__ int page_slot(int t, int page_size) {
    return (page_size & (page_size - 1)) == 0 ? (t & (page_size - 1)) : t % page_size;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & (kWave - 1);
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---------------------------------------------------------------- reductions ---

// Lane scans use DPP (data-parallel primitives: an operand read from another lane of
// the same instruction, no LDS traffic).  Four row_shr steps scan each 16-lane row;
// row_bcast:15 then adds the last lane of rows 0 and 2 into rows 1 and 3, and
// row_bcast:31 adds lane 31 (the total of rows 0-1) into rows 2 and 3.  A lane whose
// source does not exist, or whose row the step leaves out, reads the identity.  Call
// with every lane of the wave active.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_from(uint32_t identity, uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)x, CTRL, ROWS, 0xF, false);
}

struct OpAdd {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct OpMin {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); }
};
struct OpMax {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); }
};

// Inclusive scan over the wave's lanes in lane order.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x, uint32_t identity, Op op) {
    x = op(x, dpp_from<0x111, 0xF>(identity, x));   // row_shr:1
    x = op(x, dpp_from<0x112, 0xF>(identity, x));   // row_shr:2
    x = op(x, dpp_from<0x114, 0xF>(identity, x));   // row_shr:4
    x = op(x, dpp_from<0x118, 0xF>(identity, x));   // row_shr:8
    x = op(x, dpp_from<0x142, 0xA>(identity, x));   // row_bcast:15 into rows 1, 3
    x = op(x, dpp_from<0x143, 0xC>(identity, x));   // row_bcast:31 into rows 2, 3
    return x;
}

// x from lane (lane ^ j), j a power of two below 64 (a constant after unrolling), from
// registers only: quad permutes for 1 and 2, a half-row mirror then a quad reverse for
// 4, a row rotate by 8 for 8, and the 16- / 32-lane swaps for 16 and 32.
__device__ __forceinline__ int lane_xor(int x, int j) {
    const int lane = threadIdx.x & (kWave - 1);
    switch (j) {
    case 1: return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    case 2: return __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    case 4: {
        const int y = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
        return __builtin_amdgcn_update_dpp(0, y, 0x1B, 0xF, 0xF, false);        // quad_perm 3,2,1,0
    }
    case 8: return __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);  // row_ror:8
    case 16: {
        // rows (0,1,2,3) of the results: first = (x0, x0, x2, x2), second = (x1, x1, x3, x3)
        const auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
        return (int)((lane & 16) ? r[0] : r[1]);
    }
    default: {
        // halves of the results: first = (lo, lo), second = (hi, hi)
        const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
        return (int)((lane & 32) ? r[0] : r[1]);
    }
    }
}

__device__ __forceinline__ int wave_incl_scan(int x) { return (int)wave_scan((uint32_t)x, 0u, OpAdd{}); }

__device__ __forceinline__ int wave_sum(int x) {
    return __builtin_amdgcn_readlane(wave_incl_scan(x), kWave - 1);
}

// Exclusive prefix sum over the workgroup (NT threads); *total gets the sum.  wsum
// holds NT/64 ints.  One barrier; wsum must not be written again before the next one.
template <int NT>
__device__ int block_excl_scan(int x, int *total, int *wsum) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int incl = wave_incl_scan(x);
    if (lane == kWave - 1) wsum[wid] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        const int t = wsum[w];
        before += w < wid ? t : 0;
        all += t;
    }
    *total = all;
    return before + incl - x;
}

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

// ---------------------------------------------------------------- scoring ------

// Raw K data of one lane for a 16-token tile: 16 bytes of packed e2m1 (dimensions
// [32g, 32g+32) of token tok0 + lane%16) and the UE8M0 byte scaling them.
struct KTile {
    uint4 v;
    int sc;
};

// Per-lane query state of one row.  MXFP4: the A operands of the four 16-head tiles
// and their scale operands.  FP8: the same data converted to bf16, per head tile and
// k step.  Both: the weights of the heads whose accumulators the lane holds (heads
// 16*ht + 4*(lane/16) + v), times the row scale for fp8.
template <int QF>
struct QFrag;

template <>
struct QFrag<0> {
    v8i a[4];
    int sc[4];
    float w[4][4];
};

template <>
struct QFrag<1> {
    v8bf a[4][4];
    float w[4][4];
};

__device__ __forceinline__ v8bf cat4(v2bf a, v2bf b, v2bf c, v2bf d) {
    return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ void load_q(QFrag<0> &f, const void *qv, const void *qs, int row,
                                       int lane) {
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        const int64_t h = (int64_t)row * kHeads + 16 * ht + n;
        const uint4 x = *(const uint4 *)((const uint8_t *)qv + h * (kHeadDim / 2) + 16 * g);
        f.a[ht] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
        f.sc[ht] = ((const uint8_t *)qs)[h * (kHeadDim / 32) + g];
    }
}

__device__ __forceinline__ void load_q(QFrag<1> &f, const void *qv, const void *qs, int row,
                                       int lane) {
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        const int64_t h = (int64_t)row * kHeads + 16 * ht + n;
        const uint8_t *p = (const uint8_t *)qv + h * kHeadDim + 32 * g;
        const uint4 x = *(const uint4 *)p, y = *(const uint4 *)(p + 16);
        const uint32_t d[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
        for (int st = 0; st < 4; ++st)
            f.a[ht][st] = cat4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[2 * st], 1.0f, false),
                               __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[2 * st], 1.0f, true),
                               __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[2 * st + 1], 1.0f, false),
                               __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[2 * st + 1], 1.0f, true));
    }
}

// bf16 code(s) in a 32-bit word -> fp32: the low half, the high half (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// fp32 -> the nearest bf16 value (ties to the even significand), kept as the fp32 it
// widens to: the bf16 scoring format rounds every logit so before the selection.
__device__ __forceinline__ float round_bf16(float x) {
    const uint32_t u = __float_as_uint(x);
    return __uint_as_float((u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u);
}

// The logit the selection sees: fp32 (sf = 0) or rounded to bf16 (sf = 1); a NaN (a NaN
// or infinite weight) becomes -inf, the lowest rank.  So every logit that reaches a
// selection is a number, and the column word kNoColumn (a NaN pattern) can only mean
// "no column".
__device__ __forceinline__ float score_out(int sf, float x) {
    x = __builtin_isnan(x) ? -INFINITY : x;
    return sf ? round_bf16(x) : x;
}

// Weights of the lane's 16 heads: fp32 (sf = 0) or bf16 codes (sf = 1), each lane's 4
// consecutive heads read as two 8-byte loads issued whatever the format (no load behind
// a branch: fp32 takes bytes [0, 16) of its run, bf16 bytes [0, 8) twice; both stay inside
// the row's weights, which are 8-byte aligned).
template <int QF>
__device__ __forceinline__ void load_q_weights(QFrag<QF> &f, const void *qs, const void *weights,
                                               int sf, int row, int lane) {
    const int g = lane >> 4;
    const float rs = (QF == 1) ? ((const float *)qs)[row] : 1.0f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        const int64_t i = (int64_t)row * kHeads + 16 * ht + 4 * g;
        const uint8_t *p = (const uint8_t *)weights + (i << (2 - sf));
        const uint2 a = *(const uint2 *)p, b = *(const uint2 *)(p + (sf ? 0 : 8));
        f.w[ht][0] = (sf ? bf16_lo(a.x) : __uint_as_float(a.x)) * rs;
        f.w[ht][1] = (sf ? bf16_hi(a.x) : __uint_as_float(a.y)) * rs;
        f.w[ht][2] = (sf ? bf16_lo(a.y) : __uint_as_float(b.x)) * rs;
        f.w[ht][3] = (sf ? bf16_hi(a.y) : __uint_as_float(b.y)) * rs;
    }
}

template <int QF>
__device__ __forceinline__ void load_q(QFrag<QF> &f, const void *qv, const void *qs,
                                       const void *weights, int sf, int row, int lane) {
    load_q(f, qv, qs, row, lane);
    load_q_weights(f, qs, weights, sf, row, lane);
}

// ReLU as one integer max on the float's bits: negative values (and -0) have the
// sign bit set, so they become +0; non-negative values pass unchanged.  (fmaxf would
// cost a second instruction to quiet NaN inputs.)  A NaN dot product (a NaN scale byte
// or e4m3 code among its inputs) comes out of the matrix cores with the sign bit set
// (measured on both the MX-FP4 and the bf16 MFMA), so it becomes 0, the ReLU(NaN) = 0
// rule of the oracle.
__device__ __forceinline__ float relu(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// Weighted ReLU of one head tile's accumulators into the lane's partial sum.
__device__ __forceinline__ float relu_weighted(const float (&w)[4], v4f acc, float p) {
#pragma unroll
    for (int v = 0; v < 4; ++v) p = __builtin_fmaf(w[v], relu(acc[v]), p);
    return p;
}

// Partial weighted ReLU head sum of the lane's 16 heads for its column of one
// 16-token tile.  The same code serves the sparse and the dense kernels, so a
// token's logit does not depend on which path scored it.
// (weights passed apart from the query operands: the row-group kernel keeps them in LDS)
__device__ __forceinline__ float tile_partial(const QFrag<0> &f, const float (&w)[4][4],
                                              const KTile &k) {
    const v8i kb = v8i{(int)k.v.x, (int)k.v.y, (int)k.v.z, (int)k.v.w, 0, 0, 0, 0};
    float p = 0.0f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.a[ht], kb, acc, 4, 4, 0, f.sc[ht],
                                                               0, k.sc);
        p = relu_weighted(w[ht], acc, p);
    }
    return p;
}

__device__ __forceinline__ float tile_partial(const QFrag<0> &f, const KTile &k) {
    return tile_partial(f, f.w, k);
}

__device__ __forceinline__ float tile_partial(const QFrag<1> &f, const KTile &k) {
    // 2^(sc - 127) as fp32 (sc = 0 is the subnormal 2^-127; 0xFF is NaN in UE8M0, as the
    // MX-scaled MFMA of the MXFP4 path reads it)
    const float scale = __uint_as_float(k.sc == 0 ? 0x00400000u
                                        : k.sc == 0xFF ? 0x7FC00000u : (uint32_t)k.sc << 23);
    const uint32_t d[4] = {k.v.x, k.v.y, k.v.z, k.v.w};
    v8bf b[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
        b[st] = cat4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[st], scale, 0),
                     __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[st], scale, 1),
                     __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[st], scale, 2),
                     __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[st], scale, 3));
    float p = 0.0f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < 4; ++st)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[ht][st], b[st], acc, 0, 0, 0);
        p = relu_weighted(f.w[ht], acc, p);
    }
    return p;
}

// Lanes of row g = lane/16 hold partial sums p[t] (their 16 heads) of column
// lane%16 of tiles t = 0..3.  Returns, in lane l, the full sum of tile l/16's column
// l%16, i.e. of column l of the 64-column group.  v_permlane32_swap(a, b) moves b's
// lanes 0-31 into a's lanes 32-63 and a's lanes 32-63 into b's lanes 0-31; the sum
// of the two results therefore pairs rows (0,2) and (1,3); v_permlane16_swap then
// pairs rows (0,1) and (2,3).  Every tile's column sum comes out as
// (p(row0) + p(row2)) + (p(row1) + p(row3)) with the same operand order, so the
// result does not depend on the column's position in the group.
__device__ __forceinline__ float reduce_transpose4(float p0, float p1, float p2, float p3) {
    const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2),
                                                    false, false);
    const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3),
                                                    false, false);
    const float q0 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    const float q1 = __uint_as_float(y[0]) + __uint_as_float(y[1]);
    const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(q0), __float_as_uint(q1),
                                                    false, false);
    return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}



// Scores the 64-column groups [g0, g1) of one row, in rounds of RG <= 16 groups.  Lane t
// first resolves tile t of the round: desc gives its page (-1: nothing to score) and
// first token, from which the lane forms the tile's value and scale base addresses,
// so all descriptor loads and address arithmetic of a round cost one memory latency
// and one pass of vector instructions.  A tile then costs scalar reads of those
// addresses and two loads at a per-lane offset (token lane%16, scale block lane/16)
// that never changes.
//
// The round runs as RG/U units of U groups, fully unrolled, loading unit u+1 while
// unit u computes (two U-group buffers, 2*U*4 KB in flight per wave).  Loads are
// never under a branch: a tile with nothing to score, or beyond the round's groups,
// reads the pool's first bytes (in bounds, and an L2 hit after the first time) and
// its result is dropped by a select.  Branch-free loads keep the compiler's
// memory-counter waits exact (a load under an if makes it wait for everything).
// K loads carry the non-temporal hint: a decode row reads each K byte once, and the
// streaming policy measured 4-9 % faster steps than the default one (the row-group
// kernel, whose rows share K tiles through the caches, keeps the default).
// sink(c, logit, valid) receives every column of the groups; valid says whether the
// column is a token of [ks, ke) (the logit is meaningless otherwise).  Every lane of the
// wave calls it together.
//
// G64 (every 64-column group is one 64-token run of one page: 64-token sparse blocks, or
// the dense comparator on pages of a multiple of 64 tokens): lane q resolves group q of
// the round (desc.group), the four tiles of a group load from one base with immediate
// offsets, and a group is scored or dropped whole (4 lane reads a group instead of 16,
// no per-tile selects).
template <int QF, int RG, int U, bool G64, class Desc, class Sink>
__device__ __forceinline__ void score_groups(const KCache &k, const QFrag<QF> &f, int ks, int ke,
                                             int g0, int g1, int sf, Desc desc, Sink sink) {
    static_assert(RG <= 16 && RG % U == 0, "units must tile a round of at most 16 groups");
    constexpr int NU = RG / U;
    const int lane = threadIdx.x & (kWave - 1);
    const int n = lane & 15, g = lane >> 4;
    const uint32_t voff = n * (kHeadDim / 2) + 16 * g;
    const uint32_t soff = n * (kHeadDim / 32) + g;
    if constexpr (G64) {
        for (int r0 = g0; r0 < g1; r0 += RG) {
            const int ng = min(RG, g1 - r0);
            int page = -1, ttok = 0;
            if (lane < ng) desc.group(r0 + lane, page, ttok);
            const bool ok = page >= 0 && page < k.num_pages && ttok >= 0;
            uint64_t vb = (uint64_t)k.values, sb = (uint64_t)k.scales;  // safe, never scored
            if (ok) {
                const int64_t j0 = page_slot(ttok, k.page_size);
                vb += (uint64_t)((int64_t)page * k.values_page_stride + j0 * (kHeadDim / 2));
                sb += (uint64_t)((int64_t)page * k.scales_page_stride + j0 * (kHeadDim / 32));
            }
            const uint32_t vlo = (uint32_t)vb, vhi = (uint32_t)(vb >> 32);
            const uint32_t slo = (uint32_t)sb, shi = (uint32_t)(sb >> 32);
            const uint64_t okmask = __ballot(ok);  // bit q: group q has something to score
            KTile kt[2][U][4];
            auto load_unit = [&](int u, KTile(&b)[U][4]) {
#pragma unroll
                for (int q = 0; q < U; ++q) {
                    const int src = u * U + q;
                    const kGlobal uint8_t *vp = (const kGlobal uint8_t *)join64(
                        __builtin_amdgcn_readlane(vhi, src), __builtin_amdgcn_readlane(vlo, src));
                    const kGlobal uint8_t *sp = (const kGlobal uint8_t *)join64(
                        __builtin_amdgcn_readlane(shi, src), __builtin_amdgcn_readlane(slo, src));
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const v4u x = __builtin_nontemporal_load(
                            (const kGlobal v4u *)(vp + t * 16 * (kHeadDim / 2) + voff));
                        b[q][t].v = make_uint4(x[0], x[1], x[2], x[3]);
                        b[q][t].sc =
                            __builtin_nontemporal_load(sp + t * 16 * (kHeadDim / 32) + soff);
                    }
                }
            };
            auto finish_unit = [&](int u, const KTile(&b)[U][4]) {
#pragma unroll
                for (int q = 0; q < U; ++q) {
                    const int grp = u * U + q;
                    if (grp >= ng) break;
                    const float lg = score_out(
                        sf, reduce_transpose4(tile_partial(f, b[q][0]), tile_partial(f, b[q][1]),
                                              tile_partial(f, b[q][2]), tile_partial(f, b[q][3])));
                    const int tok = __builtin_amdgcn_readlane(ttok, grp) + lane;
                    const bool valid = ((okmask >> grp) & 1) && tok >= ks && tok < ke;
                    sink((r0 + grp) * 64 + lane, lg, valid);
                }
            };
            load_unit(0, kt[0]);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if (u + 1 < NU) load_unit(u + 1, kt[(u + 1) & 1]);
                if (u * U < ng) finish_unit(u, kt[u & 1]);
            }
        }
        return;
    }
    for (int r0 = g0; r0 < g1; r0 += RG) {
        const int ng = min(RG, g1 - r0);
        int page = -1, ttok = 0;
        if (lane < ng * 4) desc(r0 * 4 + lane, page, ttok);
        const bool ok = page >= 0 && page < k.num_pages && ttok >= 0;
        uint64_t vb = (uint64_t)k.values, sb = (uint64_t)k.scales;  // safe, never scored
        if (ok) {
            const int64_t j0 = page_slot(ttok, k.page_size);
            vb += (uint64_t)((int64_t)page * k.values_page_stride + j0 * (kHeadDim / 2));
            sb += (uint64_t)((int64_t)page * k.scales_page_stride + j0 * (kHeadDim / 32));
        }
        const uint32_t vlo = (uint32_t)vb, vhi = (uint32_t)(vb >> 32);
        const uint32_t slo = (uint32_t)sb, shi = (uint32_t)(sb >> 32);
        const uint64_t okmask = __ballot(ok);  // bit t: tile t has something to score
        KTile kt[2][U][4];
        auto load_unit = [&](int u, KTile(&b)[U][4]) {
#pragma unroll
            for (int q = 0; q < U; ++q)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int src = (u * U + q) * 4 + t;
                    const kGlobal uint8_t *vp = (const kGlobal uint8_t *)join64(
                        __builtin_amdgcn_readlane(vhi, src), __builtin_amdgcn_readlane(vlo, src));
                    const kGlobal uint8_t *sp = (const kGlobal uint8_t *)join64(
                        __builtin_amdgcn_readlane(shi, src), __builtin_amdgcn_readlane(slo, src));
                    const v4u x = __builtin_nontemporal_load((const kGlobal v4u *)(vp + voff));
                    b[q][t].v = make_uint4(x[0], x[1], x[2], x[3]);
                    b[q][t].sc = __builtin_nontemporal_load(sp + soff);
                }
        };
        auto finish_unit = [&](int u, const KTile(&b)[U][4]) {
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const int grp = u * U + q;
                if (grp >= ng) break;
                float p[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float v = tile_partial(f, b[q][t]);
                    p[t] = ((okmask >> (grp * 4 + t)) & 1) ? v : 0.0f;
                }
                const float lg = score_out(sf, reduce_transpose4(p[0], p[1], p[2], p[3]));
                const int tok = __shfl(ttok, grp * 4 + g, kWave) + n;
                const bool valid = ((okmask >> (grp * 4 + g)) & 1) && tok >= ks && tok < ke;
                sink((r0 + grp) * 64 + lane, lg, valid);
            }
        };
        load_unit(0, kt[0]);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            if (u + 1 < NU) load_unit(u + 1, kt[(u + 1) & 1]);
            if (u * U < ng) finish_unit(u, kt[u & 1]);
        }
    }
}

// Scores units of U 64-column groups that grab() hands out (unit u covers groups
// [uU, uU+U); grab returns -1 once the row is done), so the waves of a workgroup share
// a row dynamically and finish together.  Two units are in flight per wave: the next
// unit's K loads are issued before the current one computes.  Tile descriptors come
// from desc (read from LDS by the caller); loads are branch-free as in score_groups (a
// tile with nothing to score, or a unit past the end, reads the pool's first bytes and
// its result is dropped).  sink(c, logit, valid) receives every column of the units
// scored; valid says whether the column is a token of [ks, ke) (logit is meaningless
// otherwise).
//
// G64 (64-token sparse blocks, so every page holds whole 64-token runs): a group is one
// run of one page, its four tiles are consecutive 1 KB value runs and 64-byte scale runs.
// One uniform descriptor then serves the whole group; the loads use a scalar base with
// immediate offsets, and a group is scored or dropped whole.  Per group that saves the
// per-tile descriptor lanes, 16 lane reads, the 64-bit address arithmetic per tile, the
// per-tile drop selects and the token shuffle (vector ALU time the epilogue shares).
template <int QF, int U, bool G64, class Desc, class Grab, class Sink>
__device__ __forceinline__ void score_units(const KCache &k, const QFrag<QF> &f, int ks, int ke,
                                            int sf, Desc desc, Grab grab, Sink sink) {
    static_assert(4 * U <= kWave, "one lane per tile of a unit");
    const int lane = threadIdx.x & (kWave - 1);
    const int n = lane & 15, g = lane >> 4;
    const uint32_t voff = n * (kHeadDim / 2) + 16 * g;
    const uint32_t soff = n * (kHeadDim / 32) + g;
    if constexpr (G64) {
        auto issue = [&](int u, KTile (&b)[U][4], int (&t0)[U], uint32_t &okm) {
            okm = 0u;
#pragma unroll
            for (int q = 0; q < U; ++q) {
                int page = -1, tt = 0;
                if (u >= 0) desc((u * U + q) * 4, page, tt);   // every lane: one LDS word
                page = uniform(page);
                tt = uniform(tt);
                const bool ok = page >= 0 && page < k.num_pages && tt >= 0;
                int64_t ov = 0, os = 0;   // a dropped group reads the pool's first bytes
                if (ok) {
                    const int64_t j0 = page_slot(tt, k.page_size);
                    ov = (int64_t)page * k.values_page_stride + j0 * (kHeadDim / 2);
                    os = (int64_t)page * k.scales_page_stride + j0 * (kHeadDim / 32);
                }
                const kGlobal uint8_t *vp = (const kGlobal uint8_t *)k.values + ov;
                const kGlobal uint8_t *sp = (const kGlobal uint8_t *)k.scales + os;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const v4u x = __builtin_nontemporal_load(
                        (const kGlobal v4u *)(vp + t * 16 * (kHeadDim / 2) + voff));
                    b[q][t].v = make_uint4(x[0], x[1], x[2], x[3]);
                    b[q][t].sc = __builtin_nontemporal_load(sp + t * 16 * (kHeadDim / 32) + soff);
                }
                t0[q] = tt;
                okm |= (uint32_t)ok << q;
            }
        };
        auto finish = [&](int u, const KTile (&b)[U][4], const int (&t0)[U], uint32_t okm) {
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const float lg = score_out(
                    sf, reduce_transpose4(tile_partial(f, b[q][0]), tile_partial(f, b[q][1]),
                                          tile_partial(f, b[q][2]), tile_partial(f, b[q][3])));
                const int tok = t0[q] + lane;
                const bool full = t0[q] >= ks && t0[q] + 64 <= ke;   // uniform
                const bool valid = ((okm >> q) & 1u) && (full || (tok >= ks && tok < ke));
                sink((u * U + q) * 64 + lane, lg, valid);
            }
        };
        KTile ka[U][4], kb[U][4];
        int ta[U], tb[U];
        uint32_t ma = 0u, mb = 0u;
        int ua = grab();
        issue(ua, ka, ta, ma);
        int ub = grab();
        issue(ub, kb, tb, mb);
        while (true) {
            if (ua < 0) break;
            finish(ua, ka, ta, ma);
            ua = grab();
            issue(ua, ka, ta, ma);
            if (ub < 0) break;
            finish(ub, kb, tb, mb);
            ub = grab();
            issue(ub, kb, tb, mb);
        }
        return;
    }
    auto issue = [&](int u, KTile (&b)[U][4], int &ttok, uint64_t &okmask) {
        int page = -1, tt = 0;
        if (u >= 0 && lane < 4 * U) desc(u * 4 * U + lane, page, tt);
        const bool ok = page >= 0 && page < k.num_pages && tt >= 0;
        uint64_t vb = (uint64_t)k.values, sb = (uint64_t)k.scales;
        if (ok) {
            const int64_t j0 = page_slot(tt, k.page_size);
            vb += (uint64_t)((int64_t)page * k.values_page_stride + j0 * (kHeadDim / 2));
            sb += (uint64_t)((int64_t)page * k.scales_page_stride + j0 * (kHeadDim / 32));
        }
        const uint32_t vlo = (uint32_t)vb, vhi = (uint32_t)(vb >> 32);
        const uint32_t slo = (uint32_t)sb, shi = (uint32_t)(sb >> 32);
        okmask = __ballot(ok);
        ttok = tt;
#pragma unroll
        for (int q = 0; q < U; ++q)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int src = q * 4 + t;
                const kGlobal uint8_t *vp = (const kGlobal uint8_t *)join64(
                    __builtin_amdgcn_readlane(vhi, src), __builtin_amdgcn_readlane(vlo, src));
                const kGlobal uint8_t *sp = (const kGlobal uint8_t *)join64(
                    __builtin_amdgcn_readlane(shi, src), __builtin_amdgcn_readlane(slo, src));
                const v4u x = __builtin_nontemporal_load((const kGlobal v4u *)(vp + voff));
                b[q][t].v = make_uint4(x[0], x[1], x[2], x[3]);
                b[q][t].sc = __builtin_nontemporal_load(sp + soff);
            }
    };
    auto finish = [&](int u, const KTile (&b)[U][4], int ttok, uint64_t okmask) {
#pragma unroll
        for (int q = 0; q < U; ++q) {
            float p[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float v = tile_partial(f, b[q][t]);
                p[t] = ((okmask >> (q * 4 + t)) & 1) ? v : 0.0f;
            }
            const float lg = score_out(sf, reduce_transpose4(p[0], p[1], p[2], p[3]));
            const int tok = __shfl(ttok, q * 4 + g, kWave) + n;
            const bool valid = ((okmask >> (q * 4 + g)) & 1) && tok >= ks && tok < ke;
            sink((u * U + q) * 64 + lane, lg, valid);
        }
    };
    KTile ka[U][4], kb[U][4];
    int ta = 0, tb = 0;
    uint64_t ma = 0, mb = 0;
    int ua = grab();
    issue(ua, ka, ta, ma);
    int ub = grab();
    issue(ub, kb, tb, mb);
    while (true) {
        if (ua < 0) break;
        finish(ua, ka, ta, ma);
        ua = grab();
        issue(ua, ka, ta, ma);
        if (ub < 0) break;
        finish(ub, kb, tb, mb);
        ub = grab();
        issue(ub, kb, tb, mb);
    }
}

// Tile descriptor of a row's sparse column space: tile t covers columns [16t, 16t+16)
// of sparse block slot 16t / sbk, tokens sparse_indices[slot] * sbk + 16t % sbk + i,
// on the page the schedule resolved for that slot.  Slots past the row's kept count
// hold page -1 (the expansion pads them), so the loads need not wait for that count.
struct SparseDesc {
    const int32_t *si, *pg;
    int nsb, sbk;
    __device__ __forceinline__ void operator()(int tile, int &page, int &tok) const {
        const int slot = tile * 16 / sbk;
        if (slot < nsb) {
            page = pg[slot];
            tok = si[slot] * sbk + tile * 16 % sbk;
        }
    }
    // 64-column group grp when sbk = 64: its one sparse block
    __device__ __forceinline__ void group(int grp, int &page, int &tok) const {
        (*this)(grp * 4, page, tok);
    }
};

// Tile descriptor of the dense comparator: tile t is tokens [16t, 16t+16).
struct DenseDesc {
    const int32_t *bt;
    int ks, ke, page_size, pages_per_table;
    __device__ __forceinline__ void operator()(int tile, int &page, int &tok) const {
        const int t0 = tile * 16;
        if (t0 < ke && t0 + 16 > ks) {
            const int lp = t0 / page_size;
            if (lp < pages_per_table) page = bt[lp];
            tok = t0;
        }
    }
    // tokens [64 grp, 64 grp + 64) when page_size is a multiple of 64: one page
    __device__ __forceinline__ void group(int grp, int &page, int &tok) const {
        const int t0 = grp * 64;
        if (t0 < ke && t0 + 64 > ks) {
            const int lp = t0 / page_size;
            if (lp < pages_per_table) page = bt[lp];
            tok = t0;
        }
    }
};

struct RowInfo {
    int ks, ke, kept, valid_cols, ncols;
    bool tbl_ok;
    const int32_t *si, *pg;
};

__device__ __forceinline__ RowInfo row_info(const Rows &rows, const KCache &k, const Schedule &s,
                                            int row) {
    RowInfo ri;
    ri.ks = rows.ks ? rows.ks[row] : 0;
    ri.ke = rows.ke[row];
    const int tbl = rows.table ? rows.table[row] : row;
    const int kept = uniform(s.kept[row]);   // not behind the table check: both loads fly
    ri.tbl_ok = tbl >= 0 && tbl < k.num_tables;
    ri.kept = ri.tbl_ok ? max(0, min(kept, s.nsb)) : 0;
    ri.valid_cols = ri.kept * s.sbk;
    ri.ncols = s.nsb * s.sbk;
    ri.si = s.sparse_indices + (int64_t)row * s.nsb;
    ri.pg = s.pages + (int64_t)row * s.nsb;
    return ri;
}

// ---------------------------------------------------------------- top-k --------

// Keys: an order-preserving map of an fp32 logit to uint32 (larger float -> larger
// key): a negative logit's bits are inverted, a non-negative one gets the sign bit
// set.  Finite logits map above 0x007FFFFF, so key 0 is free to mark an invalid column.
// Column words in LDS (the one-row and row-group kernels): a valid column holds its
// logit's bits, any other kNoColumn (a NaN pattern, taken to mean "no logit").  The map
// needs no -0 step (a scored logit is never -0: each head sum starts from +0 and adds
// w * ReLU terms, and a round-to-nearest sum is -0 only when both operands are); it
// takes kNoColumn to the invalid key 0 by itself, and -inf, a valid logit, to
// 0x007FFFFF.
constexpr uint32_t kNoColumn = 0xFFFFFFFFu;
__device__ __forceinline__ uint32_t bits_key(uint32_t u) {
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Workgroup LDS of the row selection: one 256-bucket histogram per radix pass (at
// most four: each pass narrows the key range by 8 bits or more; NH = 5 when the first
// digit is a 512-bucket histogram built while scoring, see select_topk), the per-wave
// partial statistics and the per-wave totals of the compaction scan.
template <int NT, int NH = 4>
struct SelectLds {
    alignas(16) int hist[NH][256];
    uint32_t part[3][NT / kWave];
    int wsum[NT / kWave];
};

// Zeroes the histograms.  Call before the barrier of block_key_stats.
template <int NT, int NH>
__device__ __forceinline__ void select_clear(SelectLds<NT, NH> &L) {
    for (int i = threadIdx.x; i < NH * 256; i += NT) L.hist[i >> 8][i & 255] = 0;
}

// Per-thread partial statistics of keys (key 0: invalid column, not counted).
struct KeyStats {
    int n = 0;
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    __device__ __forceinline__ void add(uint32_t k) {
        if (k != 0u) {
            ++n;
            mn = min(mn, k);
            mx = max(mx, k);
        }
    }
};

// Lane kWave-1 of each wave holds its wave's count of valid keys, smallest and largest
// valid key; combines them over the workgroup.  Contains one barrier (which also
// publishes whatever the threads wrote to LDS before the call).
template <int NT, int NH>
__device__ __forceinline__ void block_stats_combine(uint32_t n, uint32_t mn, uint32_t mx,
                                                    SelectLds<NT, NH> &L, int &count,
                                                    uint32_t &kmin, uint32_t &kmax) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    if (lane == kWave - 1) {
        L.part[0][wid] = n;
        L.part[1][wid] = mn;
        L.part[2][wid] = mx;
    }
    __syncthreads();
    int c = 0;
    uint32_t a = 0xFFFFFFFFu, b = 0u;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        c += (int)L.part[0][w];
        a = min(a, L.part[1][w]);
        b = max(b, L.part[2][w]);
    }
    count = c;
    kmin = a;
    kmax = b;
}

// Combines per-thread partials over the workgroup: count of valid keys, smallest and
// largest valid key (one barrier, see block_stats_combine).
template <int NT, int NH>
__device__ void block_key_stats(KeyStats p, SelectLds<NT, NH> &L, int &count, uint32_t &kmin,
                                uint32_t &kmax) {
    block_stats_combine<NT>(wave_scan((uint32_t)p.n, 0u, OpAdd{}),
                            wave_scan(p.mn, 0xFFFFFFFFu, OpMin{}), wave_scan(p.mx, 0u, OpMax{}),
                            L, count, kmin, kmax);
}

// True when one of the thread's keys is valid (nonzero).
template <int KPT>
__device__ __forceinline__ bool keys_live(const uint32_t (&key)[KPT]) {
    uint32_t a = 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i) a |= key[i];
    return a != 0u;
}

// The same statistics straight from the keys in registers (live: keys_live(key), or
// false only where every key is 0): the count from wave ballots, and the minimum as
// 1 + min(key - 1), in which the invalid key 0 wraps to the largest value and drops
// out without a test.  A wave with no live thread skips the keys.
template <int NT, int KPT, int NH>
__device__ void block_key_stats(const uint32_t (&key)[KPT], bool live, SelectLds<NT, NH> &L,
                                int &count, uint32_t &kmin, uint32_t &kmax) {
    uint32_t n = 0, mnm1 = 0xFFFFFFFFu, mx = 0u;
    if (__ballot(live) != 0ull) {   // uniform: the whole wave takes it or skips it
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            n += (uint32_t)__popcll(__ballot(key[i] != 0u));
            mnm1 = min(mnm1, key[i] - 1u);
            mx = max(mx, key[i]);
        }
    }
    block_stats_combine<NT>(n, wave_scan(mnm1, 0xFFFFFFFFu, OpMin{}), wave_scan(mx, 0u, OpMax{}),
                            L, count, kmin, kmax);
    kmin += 1u;   // no valid key: 0
}

// Bucket of h[0, 64*B) that holds the k_rem-th largest key counted in it, scanned from
// the top by one wave (every wave finds the same answer, so no barrier follows): lane
// l owns buckets 64B-1-Bl down to 64B-B-Bl.  d is the bucket, before the count above
// it, c its own count.  h is 16-byte aligned.
template <int B>
__device__ __forceinline__ void find_bucket(const int *h, int k_rem, int &d, int &before, int &c) {
    static_assert(B % 4 == 0, "whole 16-byte reads");
    const int lane = threadIdx.x & (kWave - 1);
    const int top = 64 * B - 1 - B * lane;
    int cnt[B];   // cnt[j]: bucket top - j
#pragma unroll
    for (int j = 0; j < B; j += 4) {
        const int4 x = *reinterpret_cast<const int4 *>(h + top - j - 3);
        cnt[j] = x.w;
        cnt[j + 1] = x.z;
        cnt[j + 2] = x.y;
        cnt[j + 3] = x.x;
    }
    int sum = 0;
#pragma unroll
    for (int j = 0; j < B; ++j) sum += cnt[j];
    const int incl = wave_incl_scan(sum);
    // exactly one lane's buckets hold the k_rem-th largest key (if any lane's do)
    int bf = incl - sum, dd = top, cc = cnt[0];
    bool down = true;
#pragma unroll
    for (int j = 1; j < B; ++j) {
        down = down && bf + cc < k_rem;
        if (down) {
            bf += cc;
            --dd;
            cc = cnt[j];
        }
    }
    const uint64_t m = __ballot(incl - sum < k_rem && incl >= k_rem);
    const int src = (int)__builtin_ctzll(m);
    d = __builtin_amdgcn_readlane(dd, src);
    before = __builtin_amdgcn_readlane(bf, src);
    c = __builtin_amdgcn_readlane(cc, src);
}

// Top-k of one row by one workgroup of NT threads.  Thread i holds the keys of columns
// [i*KPT, (i+1)*KPT) (key 0: invalid column); column order is ascending token order.
// live may be false only where all of the thread's keys are 0 (keys_live(key), or a
// coarser test); such threads skip the per-key work.
// count_valid, kmin and kmax come from block_key_stats; count = min(topk, count_valid).
// The count-th largest key is found by radix passes over key - lo, where [lo, hi] is
// the key range still holding it (first [kmin, kmax]): a pass histograms the top 8
// bits of the range's width, and every wave scans the 256 buckets from the top, so all
// waves take the same bucket with no second barrier.  The search stops once the chosen
// bucket is taken whole or is a single key value.  With PRE the caller has already
// counted the valid keys per key >> 23 into hist[0..1] (kmin and kmax unused): that
// first digit needs no pass over the keys, and three 8-, 8- and 7-bit passes remain.
// Selected: keys above hi, plus the
// first k_rem keys in [lo, hi] in column order (ties toward the lower token).
// tokens(c0, tok) fills the tokens of columns c0 .. c0+KPT-1.  The chosen tokens are
// placed in column order into stage (LDS, 16-byte aligned, a multiple of 4 ints and at
// least count_valid of them, free once the keys are in registers) and copied out with
// coalesced stores: orow[0, topk) gets the chosen tokens ascending, then -1.
template <int NT, int KPT, bool PRE = false, int NH = 4, class Tokens>
__device__ void select_topk(const uint32_t (&key)[KPT], bool live, int count_valid, uint32_t kmin,
                            uint32_t kmax, int32_t topk, int32_t *orow, SelectLds<NT, NH> &L,
                            int32_t *stage, Tokens tokens) {
    static_assert(NT <= NH * 256, "the histograms double as spare slots, one per thread");
    static_assert(!PRE || NH == 5, "a prebuilt first digit takes hist[0..1] and 3 more passes");
    const int tid = threadIdx.x;
    const int count = min(topk, count_valid);
    uint32_t lo = 1u, hi = 0u;   // every valid key taken
    int k_rem = 0;
    bool whole = true;           // the chosen keys are exactly those >= lo
    if (count < count_valid) {
        k_rem = count;
        whole = false;
        int first = 0;           // histogram of the next pass
        if constexpr (PRE) {
            // hist[0..1] holds the count of valid keys per key >> 23 (sign and
            // exponent: one bucket per binade); the range then has 23 bits left
            int d, before, c;
            find_bucket<8>(&L.hist[0][0], k_rem, d, before, c);
            lo = max((uint32_t)d << 23, 1u);   // the invalid key 0 stays out
            hi = ((uint32_t)d << 23) | 0x7FFFFFu;
            k_rem -= before;
            whole = c == k_rem;
            first = 2;
        } else {
            lo = kmin;
            hi = kmax;
        }
        for (int pass = first; pass < NH && !whole; ++pass) {
            const uint32_t span = hi - lo;
            const int s = max(0, 24 - __clz((int)span));   // (span >> s) < 256
            int *h = L.hist[pass];
            if (!PRE && pass == 0) {
                // No range test: every valid key lies in [kmin, kmax], and the
                // invalid key 0 saturates into bucket 0.  That can only raise bucket
                // 0's count: the bucket holding the count-th largest valid key is
                // still the one found below (count < count_valid), and a raised count
                // there can only turn `whole` false, never true wrongly.  Threads
                // holding no valid key (columns past the row's end) add nothing, so
                // few invalid keys meet on bucket 0 (same-address atomics serialize).
                if (live) {
#pragma unroll
                    for (int i = 0; i < KPT; ++i)
                        atomicAdd(&h[__builtin_elementwise_sub_sat(key[i], lo) >> s], 1);
                }
            } else if (live) {
#pragma unroll
                for (int i = 0; i < KPT; ++i) {
                    const uint32_t d = key[i] - lo;
                    if (d <= span) atomicAdd(&h[d >> s], 1);
                }
            }
            __syncthreads();
            int d, before, c;
            find_bucket<4>(h, k_rem, d, before, c);
            const uint32_t w = s ? (1u << s) - 1u : 0u;
            lo += (uint32_t)d << s;
            hi = (hi - lo <= w) ? hi : lo + w;
            k_rem -= before;
            whole = c == k_rem;
            if (s == 0) break;
        }
    }

    int tok[KPT];
    // after the scan's barrier every key is in registers and the histograms are read,
    // so the stage and the spare slots (unchosen columns write there) are free
    int *spare = &L.hist[0][0] + tid;
    if (whole) {
        // exactly count keys are >= lo (all valid keys when lo = 1; otherwise the
        // keys above the final bucket plus that whole bucket)
        int nsel = 0;
        if (live) {
#pragma unroll
            for (int i = 0; i < KPT; ++i) nsel += key[i] >= lo;
        }
        int tot = 0;
        int pos = block_excl_scan<NT>(nsel, &tot, L.wsum);
        if (live) {
            tokens(tid * KPT, tok);
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const bool sel = key[i] >= lo;
                *(sel ? &stage[pos] : spare) = tok[i];
                pos += sel;
            }
        }
    } else {
        // Ties at the threshold: compaction in column order; gt and eq counts share
        // one scan (each < 2^16).
        int ngt = 0, neq = 0;
        if (live) {
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                ngt += key[i] > hi;
                neq += key[i] >= lo && key[i] <= hi;
            }
        }
        int tot = 0;
        const int excl = block_excl_scan<NT>(ngt | (neq << 16), &tot, L.wsum);
        int gpos = excl & 0xFFFF, epos = excl >> 16;
        if (live) {
            tokens(tid * KPT, tok);
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const bool gt = key[i] > hi, eq = key[i] >= lo && key[i] <= hi;
                const int pos = gpos + min(epos, k_rem);
                const bool sel = (gt || (eq && epos < k_rem)) && pos < count;
                *(sel ? &stage[pos] : spare) = tok[i];
                gpos += gt;
                epos += eq;
            }
        }
    }
    __syncthreads();
    if ((topk & 3) == 0 && (reinterpret_cast<uintptr_t>(orow) & 15) == 0) {
        // 16-byte stores; stage is read only below count (rounded up to 4, which
        // stays inside it: its size is a multiple of 4 and at least count_valid)
        for (int i = 4 * tid; i < topk; i += 4 * NT) {
            int4 v = make_int4(-1, -1, -1, -1);
            if (i < count) {
                const int4 x = *reinterpret_cast<const int4 *>(stage + i);
                v = make_int4(x.x, i + 1 < count ? x.y : -1, i + 2 < count ? x.z : -1,
                              i + 3 < count ? x.w : -1);
            }
            *reinterpret_cast<int4 *>(orow + i) = v;
        }
    } else {
        for (int i = tid; i < topk; i += NT) orow[i] = i < count ? stage[i] : -1;
    }
}

// ---------------------------------------------------------------- kernels ------

constexpr int kScoreThreads = 256;
constexpr int kTopkThreads = 512;

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

template <int QF, int PW, bool G64>
__global__ __launch_bounds__(kScoreThreads) void score_split_kernel(
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
__global__ __launch_bounds__(kScoreThreads) void score_split_layers_kernel(
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

// Tokens of the KPT sparse columns c0 .. c0+KPT-1 (KPT divides sbk = 1 << lsbk, and c0
// is a multiple of KPT, so they share one sparse block: token = block * sbk + offset).
template <int KPT>
struct SparseTokens {
    const int32_t *si_lds;
    int lsbk;
    __device__ __forceinline__ void operator()(int c0, int (&tok)[KPT]) const {
        const int base = (si_lds[c0 >> lsbk] << lsbk) + (c0 & ((1 << lsbk) - 1));
#pragma unroll
        for (int i = 0; i < KPT; ++i) tok[i] = base + i;
    }
};

// Selection for rows whose logits a separate scoring kernel wrote to global memory.
// Sparse (DENSE = false): the row's logits in sparse column order (score_split_kernel).
// Dense (DENSE = true): logits by token, lstride floats apart, lcols tokens a row (a
// multiple of 16; score_dense_kernel).  The candidate tokens in ascending order are
// the schedule's sparse blocks in order, so the dense keys are gathered from the row
// at those tokens and the selection is the sparse one: identical logits give
// identical indices.  A column is valid when it lies in a kept block and its token in
// [ks, ke) (dense: and below lcols); the logit's value plays no part (a valid -inf
// logit is selectable, the lowest of all).
// KPT keys a thread (8 for rows of up to 4096 columns, so every thread holds keys; 16
// up to 8192).
//
// The leading scalar arguments are what the first loads need (the row's logits, its
// schedule entries, ks / ke / kept): preloaded into SGPRs at wave launch, so those
// loads are one round trip with no load of their addresses before them.  The table
// row is not checked here: the expansion lists nothing for a row whose table row is
// invalid (kept = 0), and the schedule comes from the expansion of the same rows.
struct TopkLds {
    int32_t si[kMaxNSB];
    alignas(16) int32_t stage[kMaxRowCols];
    SelectLds<kTopkThreads> sel;
};

template <bool DENSE, int KPT>
__device__ __forceinline__ void topk_split_row(
    TopkLds &L, const float *logits, const int32_t *si_base, const int32_t *p_ks,
    const int32_t *p_ke, const int32_t *p_kept, int32_t nsb, int32_t lsbk, int64_t lstride,
    int32_t lcols, int32_t topk, int32_t *out, int64_t ostride) {
    static_assert(KPT == 8 || KPT == 16, "a run of 8 or 16 columns: whole float4s, inside one "
                  "sparse block (sbk >= 16), and a dense run starting at a multiple of KPT, which "
                  "divides the row length lcols (a multiple of 64)");
    static_assert(KPT * kTopkThreads <= kMaxRowCols, "the stage holds every column");
    int32_t *s_si = L.si;
    int32_t *s_stage = L.stage;
    SelectLds<kTopkThreads> &s_sel = L.sel;
    const int row = blockIdx.x, tid = threadIdx.x;
    const int sbk = 1 << lsbk, ncols = nsb << lsbk;
    const int32_t *si = si_base + (int64_t)row * nsb;
    const int vrow = row + opaque_zero();                  // vector loads, issued first
    const int32_t ks_raw = (p_ks ? p_ks : p_ke)[vrow];     // no load behind a branch
    const int ks = p_ks ? ks_raw : 0, ke = p_ke[vrow];
    const int valid_cols = max(0, min(p_kept[vrow], nsb)) * sbk;
    const float *lrow = logits + (int64_t)row * (DENSE ? lstride : (int64_t)ncols);
    const int c0 = tid * KPT;   // the thread's KPT columns lie in one sparse block
    const bool has = c0 < ncols;
    // Every load of the prologue is issued before any is used, and none sits behind a
    // branch (a branch around a load makes the compiler wait for it there): addresses
    // are clamped into the buffers and the values masked afterwards.  Sparse logits are
    // columns c0.. (every column was written); dense ones are tokens tok0.., read once
    // the schedule entry is in (tok0 is a multiple of KPT, lcols of 64, so the run lies
    // wholly inside or outside the row; -1 entries past the kept count give tok0 < 0).
    static_assert(kMaxNSB <= kTopkThreads, "one schedule entry a thread for the LDS copy");
    const int32_t si_c0 = si[min(c0 >> lsbk, nsb - 1)];
    const int32_t si_cp = si[min(tid, nsb - 1)];
    float x[KPT];
    auto load_run = [&](int at, bool rd) {
#pragma unroll
        for (int i = 0; i < KPT; i += 4) {
            float4 v = *(const float4 *)(lrow + (rd ? at : 0) + i);
            if (!rd) v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            x[i] = v.x;
            x[i + 1] = v.y;
            x[i + 2] = v.z;
            x[i + 3] = v.w;
        }
    };
    if constexpr (!DENSE) load_run(c0, has);
    const int tok0 = has ? (si_c0 << lsbk) + (c0 & (sbk - 1)) : 0;   // token of column c0
    if constexpr (DENSE) load_run(tok0, has && tok0 >= 0 && tok0 < lcols);
    if (tid < nsb) s_si[tid] = si_cp;
    select_clear(s_sel);
    // The valid columns of the thread (in a kept block, token in [ks, ke)) are one run
    // [c0 + lo, c0 + hi): a bit mask, so no key needs a branch.  The scoring never
    // writes -0 (see bits_key).
    static_assert(KPT < 32, "one mask bit per key");
    const int lo = min(KPT, max(0, ks - tok0));
    const int hi = max(0, min(min(KPT, valid_cols - c0),
                              min(ke, DENSE ? lcols : INT_MAX) - tok0));
    const uint32_t vmask = ((1u << hi) - 1u) & ~((1u << lo) - 1u);
    uint32_t key[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i)
        key[i] = bits_key(__float_as_uint(x[i])) & (0u - ((vmask >> i) & 1u));
    const bool live = vmask != 0u;
    int nvalid;
    uint32_t kmin, kmax;
    block_key_stats<kTopkThreads>(key, live, s_sel, nvalid, kmin, kmax);
    select_topk<kTopkThreads, KPT>(key, live, nvalid, kmin, kmax, topk,
                                   out + (int64_t)row * ostride, s_sel, s_stage,
                                   SparseTokens<KPT>{s_si, lsbk});
}

template <bool DENSE, int KPT>
__global__ __launch_bounds__(kTopkThreads) void topk_split_kernel(
    const float *logits, const int32_t *si_base, const int32_t *p_ks, const int32_t *p_ke,
    const int32_t *p_kept, int32_t nsb, int32_t lsbk, int64_t lstride, int32_t lcols,
    int32_t topk, int32_t *out, int64_t ostride) {
    __shared__ TopkLds lds;
    topk_split_row<DENSE, KPT>(lds, logits, si_base, p_ks, p_ke, p_kept, nsb, lsbk, lstride, lcols,
                               topk, out, ostride);
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
    SelectLds<NT, 5> sel;
};

// U: 64-column groups a wave takes per unit (two units in flight).
template <int QF, int NT, int KPT, int U, bool G64>
__device__ __forceinline__ void fused_row(
    FusedLds<NT> &L, int row, const int32_t *si_base, const int32_t *pg_base, const void *qv,
    const void *qs, const void *weights, const int32_t *p_kept, int32_t nsb, int32_t lsbk,
    const Rows &rows, const KCache &k, float *logits_out, int32_t topk, int32_t *out,
    int64_t ostride, int sf) {
    uint32_t *s_word = L.word;
    int32_t *s_si = L.si;
    int32_t *s_pg = L.pg;
    int &s_unit = L.unit;
    SelectLds<NT, 5> &s_sel = L.sel;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int sbk = 1 << lsbk;
    RowInfo ri;
    ri.si = si_base + (int64_t)row * nsb;
    ri.pg = pg_base + (int64_t)row * nsb;
    ri.kept = max(0, min(uniform(p_kept[row]), nsb));
    ri.valid_cols = ri.kept * sbk;
    ri.ncols = nsb * sbk;
    ri.tbl_ok = true;
    QFrag<QF> f;
    load_q<QF>(f, qv, qs, weights, sf, row, lane);   // overlaps the schedule copy
    // Every slot [0, nsb) is written by the expansion (-1 past the kept count), so the
    // copy is not bound by the kept load: the schedule, the kept count and the query
    // are one memory round trip, not two.
    for (int i = tid; i < nsb; i += NT) {
        s_si[i] = ri.si[i];
        s_pg[i] = ri.pg[i];
    }
    // ks / ke (their pointers are not preloaded) are needed only for the validity of the
    // scored columns; loaded after the first loads so no wait for them comes first
    const int vrow = row + opaque_zero();
    const int32_t ks_raw = (rows.ks ? rows.ks : rows.ke)[vrow];   // no load behind a branch
    ri.ks = rows.ks ? ks_raw : 0;
    ri.ke = rows.ke[vrow];
    if (tid == 0) s_unit = 0;
    select_clear(s_sel);
    __syncthreads();
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
// K; fp8 queries: 8 waves of 2-group units.
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
// a SIMD), so two rows share a CU: one selects while the other streams K.
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

// ---------------------------------------------------------------- row groups ---
//
// Many rows on one table (a prefill chunk): a workgroup of kGroupWaves waves takes GR
// consecutive rows.  When they share a table row, a block id means the same K tokens
// for all of them, so the workgroup first merges the rows' schedule lists into one list
// of distinct sparse blocks, each with its page and its slot in every row.  Every wave
// then scores all GR rows for the union entries it owns (entries w, w+4, ...): one K
// tile load feeds GR x 4 MFMAs instead of 4.  Logits stay in LDS; the whole workgroup
// then selects the rows in turn (select_topk, 16 keys a thread: a quarter of the steps
// one wave would take).  Rows on different table rows are merged one row at a time (no
// sharing).  GR = 2 with the weights in LDS keeps a wave under 128 VGPRs and the LDS
// near 38 KB, so four workgroups share a CU.

constexpr int kGroupWaves = 4;
constexpr int kGroupThreads = kGroupWaves * kWave;

template <int NCMAX, int GR>
struct GroupLds {
    static constexpr int NSB = NCMAX / 64;       // sparse blocks per row (sbk = 64)
    struct alignas(16) Entry {                   // a distinct block of the group
        int32_t block, page;
        uint32_t slots;                          // slot byte per row, 0xFF: row lacks it
        int32_t pad;
    };
    uint32_t logit[GR][NCMAX];                   // column words (bits_key), then the stage
    int32_t si[GR][NSB];
    union {                                      // the merge's outputs, then the selection
        struct {
            int32_t pg[GR][NSB];
            Entry uent[GR * NSB];
        } m;
        SelectLds<kGroupThreads> sel;
    } u;
    float w[GR][kHeads];                         // head weights (not held in registers)
    int wsum[kGroupWaves];
};

// Number of entries of the ascending list a[0, n) below x (n <= N, a power of two).
template <int N>
__device__ __forceinline__ int lower_bound_lds(const int32_t *a, int n, int32_t x) {
    int pos = 0;
#pragma unroll
    for (int step = N; step > 0; step >>= 1)
        if (pos + step <= n && a[pos + step - 1] < x) pos += step;
    return pos;
}

// a[i] for a runtime i without spilling the register array to scratch memory.
template <int N>
__device__ __forceinline__ int pick(const int (&a)[N], int i) {
    int v = a[0];
#pragma unroll
    for (int q = 1; q < N; ++q) v = (i == q) ? a[q] : v;
    return v;
}

// SF: the scoring format (0 fp32, 1 bf16), a template parameter here because this kernel
// is bound by its vector ALU work (the fp32 form carries no rounding instructions).
template <int NCMAX, int GR, int SF>
__device__ __forceinline__ void row_group_rows(
    GroupLds<NCMAX, GR> &lds, const Rows &rows, const void *qv, const void *qs,
    const void *weights, const KCache &k, const Schedule &s, float *logits_out, int32_t topk,
    int32_t *out, int64_t ostride) {
    constexpr int sf = SF;
    static_assert(GR >= 1 && GR <= kGroupWaves, "a wave selects each row");
    static_assert(64 % (NCMAX / kGroupThreads) == 0, "a thread's keys lie in one sparse block");
    using L = GroupLds<NCMAX, GR>;
    constexpr int NSB = L::NSB;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = uniform(tid / kWave);
    // Last group first: in a causal chunk later rows hold more columns, so the longest
    // workgroups start first and the short ones fill the tail.
    const int row0 = (gridDim.x - 1 - blockIdx.x) * GR;
    const int ncols = s.nsb * 64;

    // Query operands first: their loads overlap the schedule merge below.  The head
    // weights go to LDS (16 VGPRs a row less, so more waves share each SIMD).
    QFrag<0> f[GR];
#pragma unroll
    for (int r = 0; r < GR; ++r)
        if (row0 + r < rows.num_rows) load_q(f[r], qv, qs, row0 + r, lane);
    for (int i = tid; i < GR * kHeads; i += kGroupThreads) {
        // fp32, or a bf16 code read as the aligned 32-bit word holding it (the weights
        // are 8-byte aligned, so that word lies inside them); no load behind a branch
        const int r = i / kHeads;
        const int64_t e = (int64_t)row0 * kHeads + min(i, (rows.num_rows - row0) * kHeads - 1);
        const uint32_t x = *(const uint32_t *)((const uint8_t *)weights +
                                               (sf ? (e * 2) & ~(int64_t)3 : e * 4));
        const float wv = sf ? ((e & 1) ? bf16_hi(x) : bf16_lo(x)) : __uint_as_float(x);
        lds.w[r][i % kHeads] = row0 + r < rows.num_rows ? wv : 0.0f;
    }

    // Row metadata (uniform: every thread reads the same words).
    int ks[GR], ke[GR], kept[GR], tbl[GR];
#pragma unroll
    for (int r = 0; r < GR; ++r) {
        const int row = row0 + r;
        if (row < rows.num_rows) {
            const RowInfo ri = row_info(rows, k, s, row);
            ks[r] = ri.ks;
            ke[r] = ri.ke;
            kept[r] = min(ri.kept, NSB);
            tbl[r] = rows.table ? rows.table[row] : row;
        } else {
            ks[r] = ke[r] = kept[r] = 0;
            tbl[r] = -1 - r;
        }
    }
    bool share = true;
#pragma unroll
    for (int r = 1; r < GR; ++r) share = share && (kept[r] == 0 || tbl[r] == tbl[0]);

    for (int i = tid; i < GR * NSB; i += kGroupThreads) {
        const int r = i / NSB, j = i % NSB;
        // loaded without waiting for kept (in bounds: j < nsb), then masked
        int32_t b = INT_MAX, p = -1;
        if (row0 + r < rows.num_rows && j < s.nsb) {
            b = s.sparse_indices[(int64_t)(row0 + r) * s.nsb + j];
            p = s.pages[(int64_t)(row0 + r) * s.nsb + j];
        }
        if (j >= pick(kept, r)) {
            b = INT_MAX;
            p = -1;
        }
        lds.si[r][j] = b;
        lds.u.m.pg[r][j] = p;
    }
    __syncthreads();

    // Union entries: entry (r, j) represents block b unless an earlier row of the
    // shared group lists it too; slots of b in the other rows come from binary search.
    constexpr int EPT = (GR * NSB + kGroupThreads - 1) / kGroupThreads;
    typename L::Entry ent[EPT];
    bool rep[EPT];
    int nrep = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = tid + e * kGroupThreads;
        const int r = i / NSB, j = i % NSB;
        rep[e] = false;
        if (i < GR * NSB && j < pick(kept, r)) {
            const int32_t b = lds.si[r][j];
            uint32_t slots = 0xFFFFFFFFu;
            bool first = true;
#pragma unroll
            for (int q = 0; q < GR; ++q) {
                int slot = -1;
                if (q == r) {
                    slot = j;
                } else if (share) {
                    const int pos = lower_bound_lds<NSB>(lds.si[q], kept[q], b);
                    if (pos < kept[q] && lds.si[q][pos] == b) slot = pos;
                }
                if (slot >= 0) {
                    slots &= ~(0xFFu << (8 * q));
                    slots |= (uint32_t)slot << (8 * q);
                    if (q < r) first = false;
                }
            }
            rep[e] = first;
            ent[e] = typename L::Entry{b, lds.u.m.pg[r][j], slots, 0};
        }
        nrep += rep[e];
    }
    int ucount = 0;
    int upos = block_excl_scan<kGroupThreads>(nrep, &ucount, lds.wsum);
#pragma unroll
    for (int e = 0; e < EPT; ++e)
        if (rep[e]) lds.u.m.uent[upos++] = ent[e];
    __syncthreads();

    // Scoring: wave w takes entries w, w + kGroupWaves, ...; the next entry's K tiles
    // load while the current one computes.
    const int n = lane & 15, g = lane >> 4;
    const uint32_t voff = n * (kHeadDim / 2) + 16 * g;
    const uint32_t soff = n * (kHeadDim / 32) + g;
    auto load_entry = [&](int u, KTile (&kt)[4], int4 &e) {
        e = make_int4(0, -1, -1, 0);
        if (u < ucount) {
            const typename L::Entry &x = lds.u.m.uent[u];
            e = make_int4(x.block, x.page, (int)x.slots, 0);
        }
        e.x = uniform(e.x);
        e.y = uniform(e.y);
        e.z = uniform(e.z);
        const bool ok = e.y >= 0 && e.y < k.num_pages;
        const int64_t j0 = ok ? page_slot(e.x * 64, k.page_size) : 0;
        const kGlobal uint8_t *vb = (const kGlobal uint8_t *)k.values +
                                    (ok ? (int64_t)e.y * k.values_page_stride + j0 * 64 : 0);
        const kGlobal uint8_t *sb = (const kGlobal uint8_t *)k.scales +
                                    (ok ? (int64_t)e.y * k.scales_page_stride + j0 * 4 : 0);
        if (!ok) e.z = -1;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const v4u x = *(const kGlobal v4u *)(vb + t * 1024 + voff);
            kt[t].v = make_uint4(x[0], x[1], x[2], x[3]);
            kt[t].sc = sb[t * 64 + soff];
        }
    };
    auto score_entry = [&](const KTile (&kt)[4], int4 e) {
        const uint32_t slots = (uint32_t)e.z;   // 0xFF bytes (or e.z = -1): row absent
        const int tok = e.x * 64 + lane;
#pragma unroll
        for (int r = 0; r < GR; ++r) {
            const uint32_t slot = (slots >> (8 * r)) & 0xFFu;
            if (slot == 0xFFu) continue;
            float w[4][4];
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
                const float4 x = *(const float4 *)&lds.w[r][16 * ht + 4 * g];
                w[ht][0] = x.x;
                w[ht][1] = x.y;
                w[ht][2] = x.z;
                w[ht][3] = x.w;
            }
            const float lg = score_out(sf, reduce_transpose4(
                tile_partial(f[r], w, kt[0]), tile_partial(f[r], w, kt[1]),
                tile_partial(f[r], w, kt[2]), tile_partial(f[r], w, kt[3])));
            // Keep two MFMAs ahead of the ReLU-weight epilogue (8 VALU ops per MFMA):
            // the epilogue of MFMA i runs while MFMA i+1 and i+2 execute.
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
#pragma unroll
            for (int i = 0; i < 14; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            // the block's 64 tokens all lie in [ks, ke) except in a row's first and last
            // kept blocks (uniform test), so the per-column test is mostly skipped
            const bool full = e.x * 64 >= ks[r] && e.x * 64 + 64 <= ke[r];
            const bool valid = full || (tok >= ks[r] && tok < ke[r]);
            const int c = (int)slot * 64 + lane;
            lds.logit[r][c] = valid ? __float_as_uint(lg) : kNoColumn;
            if (logits_out) logits_out[(int64_t)(row0 + r) * ncols + c] = valid ? lg : -INFINITY;
        }
    };
    KTile ka[4], kb[4];
    int4 ea, eb;
    load_entry(wave, ka, ea);
    for (int u = wave; u < ucount; u += 2 * kGroupWaves) {
        load_entry(u + kGroupWaves, kb, eb);
        score_entry(ka, ea);
        load_entry(u + 2 * kGroupWaves, ka, ea);
        score_entry(kb, eb);   // past the last entry eb names no row
    }
    if (logits_out)
        for (int r = 0; r < GR; ++r)
            if (row0 + r < rows.num_rows)
                for (int c = kept[r] * 64 + tid; c < ncols; c += kGroupThreads)
                    logits_out[(int64_t)(row0 + r) * ncols + c] = -INFINITY;
    __syncthreads();

    // Selection: the whole workgroup takes the group's rows in turn (the merge's LDS is
    // free now and holds the selection's histograms).
    constexpr int KPT = NCMAX / kGroupThreads;
#pragma unroll 1
    for (int r = 0; r < GR; ++r) {
        const int row = row0 + r;
        if (row >= rows.num_rows) break;
        // The row's valid tokens are its kept blocks' tokens in column order (ascending),
        // less those of the first block below ks and of the last block at or past ke (the
        // kept blocks are ascending and each meets [ks, ke)).  When they number at most
        // topk every one is chosen whatever its logit: write them straight out.
        const int kr = pick(kept, r), ksr = pick(ks, r), ker = pick(ke, r);
        const int lead = kr ? max(0, ksr - 64 * lds.si[r][0]) : 0;
        const int trail = kr ? max(0, 64 * lds.si[r][kr - 1] + 64 - ker) : 0;
        const int nvalid = kr * 64 - lead - trail;
        if (nvalid <= topk) {
            int32_t *orow = out + (int64_t)row * ostride;
            for (int c = lead + tid; c < kr * 64 - trail; c += kGroupThreads)
                orow[c - lead] = lds.si[r][c >> 6] * 64 + (c & 63);
            for (int i = max(nvalid, 0) + tid; i < topk; i += kGroupThreads) orow[i] = -1;
            continue;
        }
        select_clear(lds.u.sel);
        // KPT divides 64, so a thread's columns are all below the row's scored columns
        // (kept blocks of 64) or all above them (stale LDS, read but not used)
        const bool mine = tid * KPT < pick(kept, r) * 64;
        uint32_t key[KPT];
#pragma unroll
        for (int i = 0; i < KPT; ++i) key[i] = 0u;
        if (mine) {
#pragma unroll
            for (int i = 0; i < KPT; i += 4) {
                const uint4 x = *reinterpret_cast<const uint4 *>(&lds.logit[r][tid * KPT + i]);
                key[i] = bits_key(x.x);
                key[i + 1] = bits_key(x.y);
                key[i + 2] = bits_key(x.z);
                key[i + 3] = bits_key(x.w);
            }
        }
        int cnt;
        uint32_t kmin, kmax;
        block_key_stats<kGroupThreads>(key, mine, lds.u.sel, cnt, kmin, kmax);   // also publishes the clear
        select_topk<kGroupThreads, KPT>(key, mine, cnt, kmin, kmax, topk, out + (int64_t)row * ostride,
                                        lds.u.sel, reinterpret_cast<int32_t *>(lds.logit[r]),
                                        SparseTokens<KPT>{lds.si[r], 6});
    }
}

template <int NCMAX, int GR, int SF>
__global__ __launch_bounds__(kGroupThreads) void row_group_kernel(
    Rows rows, const void *qv, const void *qs, const void *weights, KCache k, Schedule s,
    float *logits_out, int32_t topk, int32_t *out, int64_t ostride) {
    __shared__ GroupLds<NCMAX, GR> lds;
    row_group_rows<NCMAX, GR, SF>(lds, rows, qv, qs, weights, k, s, logits_out, topk, out,
                                  ostride);
}

// Several layers of a prefill chunk sharing one schedule, one launch (grid.y = layer):
// each layer's groups go heaviest first, and the next layer's heavy groups fill the CUs
// that the previous layer's light ones leave.
template <int NCMAX, int GR, int SF>
__global__ __launch_bounds__(kGroupThreads) void row_group_layers_kernel(
    Rows rows, KCache k, Schedule s, LayerSet ls, int32_t topk, int64_t ostride) {
    __shared__ GroupLds<NCMAX, GR> lds;
    const int l = blockIdx.y;
    KCache kl = k;
    kl.values = ls.k_values[l];
    kl.scales = ls.k_scales[l];
    row_group_rows<NCMAX, GR, SF>(lds, rows, ls.q_values[l], ls.q_scales[l], ls.weights[l], kl,
                                  s, ls.logits_out[l], topk, ls.out[l], ostride);
}


// ---------------------------------------------------------------- measurement --
//
// Reference rates for the roofline, run on the same chip as the indexer: a plain
// read stream (what the K gather can at best reach) and an MFMA-only loop on the
// MX-FP4 instruction the scoring uses (what the contraction can at best reach).

constexpr int kMeasureThreads = 256;

// Every 16-byte word of src[0, n16) read once: thread g reads words g + j*T (T = all
// threads), eight non-temporal loads in flight (the fastest of the shapes measured:
// 6.3-6.5 TB/s), contiguous across the wave; an XOR of everything read goes to
// sink[workgroup] so the loads are live.
__global__ __launch_bounds__(kMeasureThreads) void measure_read_kernel(const uint4 *src, int64_t n16,
                                                                       uint32_t *sink) {
    const int64_t nthr = (int64_t)gridDim.x * kMeasureThreads;
    int64_t i = (int64_t)blockIdx.x * kMeasureThreads + threadIdx.x;
    uint32_t acc = 0;
    const v4u *s4 = reinterpret_cast<const v4u *>(src);
    for (; i + 7 * nthr < n16; i += 8 * nthr) {
        v4u v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(s4 + i + j * nthr);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
    for (; i < n16; i += nthr) {
        const v4u a = __builtin_nontemporal_load(s4 + i);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    for (int o = kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
    __shared__ uint32_t w[kMeasureThreads / kWave];
    if ((threadIdx.x & (kWave - 1)) == 0) w[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int j = 0; j < kMeasureThreads / kWave; ++j) x ^= w[j];
        sink[blockIdx.x] = x;
    }
}

// ---------------------------------------------------------- K workspace gather ---
//
// Packs a prefill chunk's paged K into a contiguous workspace: request r's positions
// [0, cu[r+1] - cu[r]) go to workspace rows cu[r] + p, D/2 value bytes and D/32 scale
// bytes a row.  grid = (tiles of kGatherTokens positions, requests); four threads copy a
// position's 64 value bytes, 16 each, and the first of them its 4 scale bytes.  A
// position whose table row, logical page or page id is out of range gets zeros; rows at
// or past max_tokens are not written.  A plain stream: HBM-bound, read once.
constexpr int kGatherTokens = 64;
constexpr int kGatherThreads = kGatherTokens * 4;

__global__ __launch_bounds__(kGatherThreads) void gather_k_kernel(
    const int32_t *cu, const int32_t *req_table, int32_t max_tokens, KCache k,
    uint8_t *values_out, uint8_t *scales_out) {
    const int r = blockIdx.y, tid = threadIdx.x, part = tid & 3;
    const int p = blockIdx.x * kGatherTokens + (tid >> 2);
    const int c0 = cu[r], len = cu[r + 1] - c0;
    const int tbl = req_table ? req_table[r] : r;
    if (c0 < 0 || p >= len || (int64_t)c0 + p >= max_tokens) return;
    const int64_t dst = (int64_t)c0 + p;
    const int lp = p / k.page_size;
    int page = -1;
    if (tbl >= 0 && tbl < k.num_tables && lp < k.pages_per_table)
        page = k.block_table[(int64_t)tbl * k.block_table_stride + lp];
    const bool ok = page >= 0 && page < k.num_pages;
    const int64_t slot = page_slot(p, k.page_size);
    v4u v = {0u, 0u, 0u, 0u};
    uint32_t sc = 0u;
    if (ok) {
        v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(
            k.values + (int64_t)page * k.values_page_stride + slot * (kHeadDim / 2) + 16 * part));
        if (part == 0)
            sc = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(
                k.scales + (int64_t)page * k.scales_page_stride + slot * (kHeadDim / 32)));
    }
    *reinterpret_cast<v4u *>(values_out + dst * (kHeadDim / 2) + 16 * part) = v;
    if (part == 0) *reinterpret_cast<uint32_t *>(scales_out + dst * (kHeadDim / 32)) = sc;
}

// The two ways of forming e4m3 x (e2m1 with UE8M0 block scales) dot products over 128
// dimensions, for 16 query rows against 16 tokens, one wave: (mode 0) the MX-scaled
// v_mfma_scale_f32_16x16x128_f8f6f4 on the raw codes (query scale bytes 127), and (mode 1)
// the fp8-query kernels' route: both operands converted exactly to bf16 (the token's
// scale applied in the conversion) and v_mfma_f32_16x16x32_bf16.  q: e4m3 [16][128];
// kv: packed e2m1 [16][64]; ks: UE8M0 [16][4]; out: fp32 [16 rows][16 tokens].
__global__ __launch_bounds__(kWave) void measure_fp8_dot_kernel(const uint8_t *q,
                                                                const uint8_t *kv,
                                                                const uint8_t *ks, int32_t mode,
                                                                float *out) {
    const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;
    // B: token n, dimensions [32g, 32g + 32) as 16 bytes, and their scale byte
    const uint4 kb = *(const uint4 *)(kv + n * 64 + 16 * g);
    const int ksc = ks[n * 4 + g];
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (mode == 0 || mode == 2) {
        // A: row n, bytes j < 16 -> dimension 16g + j, bytes j >= 16 -> 64 + 16g + j - 16
        const uint4 a0 = *(const uint4 *)(q + n * 128 + 16 * g);
        const uint4 a1 = *(const uint4 *)(q + n * 128 + 64 + 16 * g);
        const v8i a = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                          (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        if (mode == 0) {
            const v8i b = v8i{(int)kb.x, (int)kb.y, (int)kb.z, (int)kb.w, 0, 0, 0, 0};
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 4, 0, 127, 0,
                                                                   ksc);
        } else {
            // B as e4m3 in A's layout: token n's e2m1 values of dimensions [16g, 16g+16)
            // (packed bytes [8g, 8g+8)) and [64+16g, 64+16g+16) (bytes [32+8g, 32+8g+8)),
            // each converted exactly (every e2m1 value is an e4m3 value)
            const uint2 k0 = *(const uint2 *)(kv + n * 64 + 8 * g);
            const uint2 k1 = *(const uint2 *)(kv + n * 64 + 32 + 8 * g);
            const uint32_t src[4] = {k0.x, k0.y, k1.x, k1.y};
            int b8[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t lo = 0u, hi = 0u;   // nibbles 0-3 and 4-7 of src[w], low first
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t c = (src[w] >> (4 * j)) & 15u, m = c & 7u;
                    const uint32_t e = (m == 0u ? 0u : m == 1u ? 0x30u : 0x38u + 4u * (m - 2u)) |
                                       ((c & 8u) << 4);
                    if (j < 4) lo |= e << (8 * j);
                    else hi |= e << (8 * (j - 4));
                }
                b8[2 * w] = (int)lo;
                b8[2 * w + 1] = (int)hi;
            }
            const v8i b = v8i{b8[0], b8[1], b8[2], b8[3], b8[4], b8[5], b8[6], b8[7]};
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0,
                                                                   ksc);
        }
    } else {
        // A: row n, dimensions [32g, 32g + 32) as bf16 (the bf16 MFMA's k slot of step s,
        // lane group g, element j carries dimension 32g + 8s + j, as in load_q)
        const uint8_t *pq = q + n * 128 + 32 * g;
        const uint4 x = *(const uint4 *)pq, y = *(const uint4 *)(pq + 16);
        const uint32_t dq[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
        v8bf qa[4];
#pragma unroll
        for (int st = 0; st < 4; ++st)
            qa[st] = cat4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dq[2 * st], 1.0f, false),
                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dq[2 * st], 1.0f, true),
                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dq[2 * st + 1], 1.0f, false),
                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dq[2 * st + 1], 1.0f, true));
        KTile kt{kb, ksc};
        const float scale = __uint_as_float(ksc == 0 ? 0x00400000u
                                            : ksc == 0xFF ? 0x7FC00000u : (uint32_t)ksc << 23);
        const uint32_t d[4] = {kt.v.x, kt.v.y, kt.v.z, kt.v.w};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const v8bf b = cat4(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[st], scale, 0),
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[st], scale, 1),
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[st], scale, 2),
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[st], scale, 3));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[st], b, acc, 0, 0, 0);
        }
    }
    // C: lane holds token n, rows 4g + v
#pragma unroll
    for (int v = 0; v < 4; ++v) out[(4 * g + v) * 16 + n] = acc[v];
}

// Each wave: iters rounds of 8 independent v_mfma_scale_f32_16x16x128_f8f6f4 chains on
// e2m1 operands held in registers (nonzero codes that differ by lane; scale bytes
// 127), no memory traffic until one float per wave goes to sink.
__global__ __launch_bounds__(kMeasureThreads) void measure_mfma_kernel(int32_t iters, float *sink) {
    const int lane = threadIdx.x & (kWave - 1);
    const int x = 0x3A5C1E72 ^ (lane * 0x01030507) ^ iters;
    const v8i a = v8i{x | 0x11111111, (x >> 3) | 0x22222222, (x << 5) | 0x11111111,
                      x ^ 0x7F3E1D2C, 0, 0, 0, 0};
    const v8i b = v8i{(x * 7) | 0x11111111, x ^ 0x5A5A5A5A, (x >> 7) | 0x33333333,
                      (x * 13) | 0x21212121, 0, 0, 0, 0};
    v4f acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 4, 4, 0, 127, 0,
                                                                      127);
    }
    float t = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) t += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    if (lane == 0) sink[blockIdx.x * (kMeasureThreads / kWave) + threadIdx.x / kWave] = t;
}

// The MFMA rate that the scoring epilogue leaves: the same 8 MX-FP4 MFMAs a round as
// measure_mfma_kernel, each a fresh product (C = 0, the B operand bumped by one VALU add),
// and every product's 4 accumulators folded through the ReLU-weight epilogue (an integer
// max and an fp32 FMA each), 9 VALU operations per MFMA, as the prefill scoring loop
// issues them.  Registers only; one float per wave goes to sink.
__global__ __launch_bounds__(kMeasureThreads) void measure_mfma_relu_kernel(int32_t iters,
                                                                           float *sink) {
    const int lane = threadIdx.x & (kWave - 1);
    const int x = 0x3A5C1E72 ^ (lane * 0x01030507) ^ iters;
    const v8i a = v8i{x | 0x11111111, (x >> 3) | 0x22222222, (x << 5) | 0x11111111,
                      x ^ 0x7F3E1D2C, 0, 0, 0, 0};
    v8i b = v8i{(x * 7) | 0x11111111, x ^ 0x5A5A5A5A, (x >> 7) | 0x33333333,
                (x * 13) | 0x21212121, 0, 0, 0, 0};
    const float w[4] = {0.125f + lane * 1e-3f, 0.25f, -0.5f, 0.375f};
    float p = 0.0f;
    for (int it = 0; it < iters; ++it) {
        v4f r[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            b[0] += 0x10;
            r[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a, b, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 4, 4, 0, 127, 0, 127);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) p = relu_weighted(w, r[c], p);
    }
    if (lane == 0) sink[blockIdx.x * (kMeasureThreads / kWave) + threadIdx.x / kWave] = p;
}

}  // namespace

// ---------------------------------------------------------------- launchers ----

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
        constexpr int GR = 2;
        if (plan == kPlanRowGroup) {
            const dim3 grid((rows.num_rows + GR - 1) / GR);
#define IDX_LAUNCH_GROUP(NC_, SF_)                                                                  \
    hipExtLaunchKernelGGL((row_group_kernel<NC_, GR, SF_>), grid, dim3(kGroupThreads), 0, stream,   \
                          timing.start, timing.stop, 0, rows, q_values, q_scales, weights, k, s,   \
                          logits_out, topk, out, out_stride)
            if (ncols <= 4096) {
                if (sf) IDX_LAUNCH_GROUP(4096, 1);
                else IDX_LAUNCH_GROUP(4096, 0);
            } else {
                if (sf) IDX_LAUNCH_GROUP(8192, 1);
                else IDX_LAUNCH_GROUP(8192, 0);
            }
#undef IDX_LAUNCH_GROUP
            return hipGetLastError();
        }
    }
    if (plan == kPlanOneRow) {
        // MXFP4, one row a CU: 16 waves with 1-group units (measured 10 % faster 4-layer
        // steps than 8 waves with 4-group units: the row's last unit, and so the wait
        // before the selection, is shorter).  MXFP4 with two or more rows a CU: 8 waves
        // with 1-group units, two rows a CU (measured 23 % faster on 512-2000 rows of 4096
        // columns).  fp8 queries need more registers: 8 waves, 2-group units.
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
    // Enough workgroups to cover the CUs several times over; 4 waves each with two or
    // more 64-column groups (two groups a wave hide the schedule-to-K load chain better
    // than one: measured 3-7 % faster steps on 64- and 128-row decode batches).
    int gpw = 8;
    while (gpw < 16 && (int64_t)rows.num_rows * ((ngroups + gpw - 1) / gpw) > 4096) gpw *= 2;
    const dim3 sgrid(rows.num_rows, (ngroups + gpw - 1) / gpw);
#define IDX_LAUNCH_SPLIT_G(PW_, G64_)                                                              \
    hipExtLaunchKernelGGL((score_split_kernel<QF, PW_, G64_>), sgrid, dim3(kScoreThreads), 0,      \
                          stream, timing.start, timing.stop, 0, s.sparse_indices, s.pages,         \
                          q_values, q_scales, weights, s.nsb, s.sbk, gpw, grouped_rows(rows),      \
                          rows, k, logits, sf)
#define IDX_LAUNCH_SPLIT(PW_)                                                                      \
    do {                                                                                           \
        if (s.sbk == 64) IDX_LAUNCH_SPLIT_G(PW_, true);                                            \
        else IDX_LAUNCH_SPLIT_G(PW_, false);                                                       \
    } while (0)
    if (gpw == 8)
        IDX_LAUNCH_SPLIT(2);
    else
        IDX_LAUNCH_SPLIT(4);
#undef IDX_LAUNCH_SPLIT
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
    int gpw = 8;   // as for one layer (launch_sparse_q)
    while (gpw < 16 && (int64_t)rows.num_rows * ((ngroups + gpw - 1) / gpw) > 4096) gpw *= 2;
    const dim3 sgrid(rows.num_rows, (ngroups + gpw - 1) / gpw, num_layers);
#define IDX_LAUNCH_SPLIT_LAYERS_G(PW_, G64_)                                                       \
    hipExtLaunchKernelGGL((score_split_layers_kernel<QF, PW_, G64_>), sgrid, dim3(kScoreThreads),  \
                          0, stream, timing.start, timing.stop, 0, s.sparse_indices, s.pages,      \
                          s.nsb, s.sbk, gpw, grouped_rows(rows), rows, k, layers, workspace,       \
                          ws_layer, sf)
#define IDX_LAUNCH_SPLIT_LAYERS(PW_)                                                               \
    do {                                                                                           \
        if (s.sbk == 64) IDX_LAUNCH_SPLIT_LAYERS_G(PW_, true);                                     \
        else IDX_LAUNCH_SPLIT_LAYERS_G(PW_, false);                                                \
    } while (0)
    if (gpw == 8)
        IDX_LAUNCH_SPLIT_LAYERS(2);
    else
        IDX_LAUNCH_SPLIT_LAYERS(4);
#undef IDX_LAUNCH_SPLIT_LAYERS
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
    if (plan == kPlanRowGroupLayers) {
        constexpr int GR = 2;
        const dim3 grid((rows.num_rows + GR - 1) / GR, num_layers);
#define IDX_LAUNCH_GROUP_LAYERS(NC_, SF_)                                                          \
    hipExtLaunchKernelGGL((row_group_layers_kernel<NC_, GR, SF_>), grid, dim3(kGroupThreads), 0,     \
                          stream, timing.start, timing.stop, 0, rows, k, s, layers, topk, out_stride)
        if (ncols <= 4096) {
            if (sf) IDX_LAUNCH_GROUP_LAYERS(4096, 1);
            else IDX_LAUNCH_GROUP_LAYERS(4096, 0);
        } else {
            if (sf) IDX_LAUNCH_GROUP_LAYERS(8192, 1);
            else IDX_LAUNCH_GROUP_LAYERS(8192, 0);
        }
#undef IDX_LAUNCH_GROUP_LAYERS
        return hipGetLastError();
    }
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

hipError_t launch_gather_k(const KCache &k, int32_t num_reqs, const int32_t *cu_seq_lens,
                           const int32_t *req_table, int32_t max_seq_len, int32_t max_tokens,
                           uint8_t *values_out, uint8_t *scales_out, const Timing &timing,
                           hipStream_t stream) {
    if (num_reqs == 0 || max_seq_len == 0 || max_tokens == 0) return hipSuccess;
    const dim3 grid((max_seq_len + kGatherTokens - 1) / kGatherTokens, num_reqs);
    hipExtLaunchKernelGGL(gather_k_kernel, grid, dim3(kGatherThreads), 0, stream, timing.start,
                          timing.stop, 0, cu_seq_lens, req_table, max_tokens, k, values_out,
                          scales_out);
    return hipGetLastError();
}

hipError_t launch_measure_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
    hipLaunchKernelGGL(measure_read_kernel, dim3(kMeasureWgs), dim3(kMeasureThreads), 0, stream,
                       (const uint4 *)src, (int64_t)(bytes / 16), sink);
    return hipGetLastError();
}

hipError_t launch_measure_fp8_dot(const uint8_t *q, const uint8_t *kv, const uint8_t *ks,
                                  int32_t mode, float *out, hipStream_t stream) {
    hipLaunchKernelGGL(measure_fp8_dot_kernel, dim3(1), dim3(kWave), 0, stream, q, kv, ks, mode,
                       out);
    return hipGetLastError();
}

hipError_t launch_measure_mfma(int32_t iters, float *sink, hipStream_t stream) {
    hipLaunchKernelGGL(measure_mfma_kernel, dim3(kMeasureWgs), dim3(kMeasureThreads), 0, stream, iters,
                       sink);
    return hipGetLastError();
}

hipError_t launch_measure_mfma_relu(int32_t iters, float *sink, hipStream_t stream) {
    hipLaunchKernelGGL(measure_mfma_relu_kernel, dim3(kMeasureWgs), dim3(kMeasureThreads), 0, stream,
                       iters, sink);
    return hipGetLastError();
}

}  // namespace idx
