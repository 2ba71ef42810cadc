// Row groups: >= 8 rows a CU with MXFP4 queries and 64-token sparse blocks (prefill
// chunks).  Two rows a workgroup share K tiles; logits stay in LDS and are selected
// in turn.

#include "idx_device.h"

namespace idx {
namespace {

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

}  // namespace

hipError_t launch_row_groups(const Rows &rows, const void *q_values, const void *q_scales,
                             const void *weights, int sf, const KCache &k, const Schedule &s,
                             float *logits_out, int32_t topk, int32_t *out, int64_t out_stride,
                             const Timing &timing, hipStream_t stream) {
    constexpr int GR = 2;
    const int ncols = s.nsb * s.sbk;
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

hipError_t launch_row_groups_layers(const Rows &rows, int32_t num_layers, const LayerSet &layers,
                                    int sf, const KCache &k, const Schedule &s, int32_t topk,
                                    int64_t out_stride, const Timing &timing, hipStream_t stream) {
    constexpr int GR = 2;
    const int ncols = s.nsb * s.sbk;
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

}  // namespace idx
