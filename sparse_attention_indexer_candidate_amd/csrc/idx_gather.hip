#include "idx_device.h"

namespace idx {
namespace {

// ---------------------------------------------------------- K workspace gather ---
//
// Packs a prefill chunk's paged K into a contiguous workspace: request r's positions
// [0, cu[r+1] - cu[r]) go to workspace rows cu[r] + p, D/2 value bytes and D/32 scale
// bytes a row.  grid = (tiles of kGatherTokens positions, requests); four threads copy a
// position's 64 value bytes, 16 each, and the first of them its 4 scale bytes.  A
// position whose table row, logical page or page id is out of range gets zeros; positions
// at or past max_seq_len and rows at or past max_tokens are not written.  A plain stream:
// HBM-bound, read once.
constexpr int kGatherTokens = 64;
constexpr int kGatherThreads = kGatherTokens * 4;

__global__ __launch_bounds__(kGatherThreads) void gather_k_kernel(
    const int32_t *cu, const int32_t *req_table, int32_t max_seq_len, int32_t max_tokens,
    KCache k, uint8_t *values_out, uint8_t *scales_out) {
    const int r = blockIdx.y, tid = threadIdx.x, part = tid & 3;
    const int p = blockIdx.x * kGatherTokens + (tid >> 2);
    // the grid covers max_seq_len rounded up to whole tiles: the tail is cut here
    const int c0 = cu[r], len = min(cu[r + 1] - c0, max_seq_len);
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

}  // namespace

hipError_t launch_gather_k(const KCache &k, int32_t num_reqs, const int32_t *cu_seq_lens,
                           const int32_t *req_table, int32_t max_seq_len, int32_t max_tokens,
                           uint8_t *values_out, uint8_t *scales_out, const Timing &timing,
                           hipStream_t stream) {
    if (num_reqs == 0 || max_seq_len == 0 || max_tokens == 0) return hipSuccess;
    const dim3 grid((max_seq_len + kGatherTokens - 1) / kGatherTokens, num_reqs);
    hipExtLaunchKernelGGL(gather_k_kernel, grid, dim3(kGatherThreads), 0, stream, timing.start,
                          timing.stop, 0, cu_seq_lens, req_table, max_seq_len, max_tokens, k,
                          values_out, scales_out);
    return hipGetLastError();
}

}  // namespace idx
