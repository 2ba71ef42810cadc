// Device code shared by the gfx950 kernels of the candidate-consuming sparse MQA-logits
// indexer, included by every kernel source (all of it inline device code, so each kernel
// is compiled with its whole path in view):
//
//  helpers, reductions  wave-uniform values, DPP / permlane scans, workgroup scans
//  score core           paged gather of e2m1 K + UE8M0 scales, MX-scaled MFMA
//                       [64 heads x 128] . [128 x 16 tokens], ReLU, fp32 weighted head
//                       reduce; one wave per 64-column group, K loads batched
//                       (score_groups, score_units over a SparseDesc or DenseDesc)
//  select_topk          per-row radix select on fp32 logits, ties toward the lower
//                       column, ascending output, -1 fill (one workgroup per row);
//                       validity comes from the tokens, never from a logit's value
//  topk_split_kernel    the selection over logits a separate scoring launch wrote to
//                       global memory (split rows, and the dense comparator)
//
// Kernel sources: idx_expand.hip (candidate expansion), idx_sparse.hip (split, one-row
// and multi-layer launches, the plan), idx_row_groups.hip (prefill chunks),
// idx_dense.hip (dense comparator, candidate source), idx_gather.hip (K workspace
// gather), idx_measure.hip (reference kernels for the measured ceilings).
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
#pragma once

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

// Candidate expansion of one row by one wave.  craw: the row's candidate ids, lane l
// holding ids l, l + 64, ... (E a lane; -1 past NB).  Ids that are negative or hold no
// token of [ks, ke) become INT_MAX; a bitonic sort over the 64*E register slots
// (shuffles across lanes, swaps within a lane) orders them; an id is kept if it differs
// from its predecessor (so repeats count once); kept blocks split into cbs/sbk sparse
// blocks, of which those holding a token of [ks, ke) and mapped by the block table
// inside the pool are listed in order with their page: out_si / out_pg [0, nlist), then
// -1 up to nsb (global or LDS memory).  stage: the wave's scratch of 64*E ints (LDS).
// Returns nlist; ntok gets the row's valid token count (the same in every lane).
template <int E>
__device__ __forceinline__ int expand_row(const int (&craw)[E], int64_t ks, int64_t ke,
                                          bool tbl_ok, int tbl, int32_t cbs, int32_t sbk,
                                          int32_t nsb, const KCache &k, int32_t *stage,
                                          int32_t *out_si, int32_t *out_pg, int &ntok) {
    const int lane = threadIdx.x & (kWave - 1);
    const int per = cbs / sbk;
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
        if (keep) stage[nkept + __popcll(m & lanemask_lt())] = v[e];
        nkept += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();

    // E sparse blocks a lane per pass, every block-table load of the pass issued before
    // the first is used: one memory round trip per pass (one in all when each candidate
    // block is one sparse block).
    const int total = nkept * per;
    int nlist = 0;
    ntok = 0;
    for (int base = 0; base < total; base += E * kWave) {
        int32_t sb[E], page[E], cnt[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = base + e * kWave + lane;
            sb[e] = 0;
            page[e] = -1;
            cnt[e] = 0;
            if (i < total) {
                const int64_t sb64 = (int64_t)stage[i / per] * per + i % per;
                const int64_t lo = max(sb64 * sbk, ks), hi = min(sb64 * sbk + sbk, ke);
                const int64_t lp = sb64 * sbk / k.page_size;
                if (hi > lo && tbl_ok && lp < k.pages_per_table) {
                    page[e] = k.block_table[(int64_t)tbl * k.block_table_stride + lp];
                    cnt[e] = (int)(hi - lo);
                }
                sb[e] = (int32_t)sb64;
            }
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool ok = page[e] >= 0 && page[e] < k.num_pages;
            if (ok) ntok += cnt[e];
            const uint64_t m = __ballot(ok);
            if (ok) {
                const int pos = nlist + __popcll(m & lanemask_lt());
                out_si[pos] = sb[e];
                out_pg[pos] = page[e];
            }
            nlist += __popcll(m);
        }
    }
    for (int i = nlist + lane; i < nsb; i += kWave) {
        out_si[i] = -1;
        out_pg[i] = -1;
    }
    ntok = wave_sum(ntok);
    return nlist;
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

// ---------------------------------------------------------------- shared kernels --

constexpr int kScoreThreads = 256;
constexpr int kTopkThreads = 512;

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

}  // namespace
}  // namespace idx
